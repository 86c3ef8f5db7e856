// Wide-wave bf16 forward of the dense coupling on gfx950 (project page
// "Spatial-Spectral Coupling as Attention", section "How it works": the
// product softmax(F_N F_M^T / sqrt(d)) Phi_M; section "The bottleneck": the
// map itself is never stored).
//
// One workgroup = 4 waves over 256 target rows, one wave per SIMD; a wave
// owns 64 rows as two 32-row blocks.  Every K fragment read from LDS feeds
// the score MFMAs of both row blocks and every V^T fragment the value MFMAs
// of both, so the LDS reads, and the global->LDS loads, per MFMA are half
// those of a 32-row wave: the chip runs at a power-limited clock here, and
// moving less data per product is what buys time.
//
// Per 64-key tile t a wave forms the scores S^T = K Q^T of both row blocks
// (K rows read in the sigma_row order, so each lane's C-layout elements are
// consecutive keys), the probabilities P = exp2(S c2 - m) against the row's
// bounded reference m = c2 |q| max_j |k_j| (no running maximum), and
// O^T += V^T P^T with V^T from the grouped-transposed copy.  Step t runs the
// scores of tile t + 1 (32 MFMAs at d = 128), then the value products of
// tile t (56 MFMAs at kp = 224) with the softmax of tile t + 1 spread between
// them.  K and V^T tiles are triple-buffered: step t loads K(t + 3) and
// V(t + 2), and the wait at its end covers only the previous step's loads.
// Past the last tile the K windows are empty (zero scores whose
// probabilities meet zero V^T columns and a zero ones row), so every step
// has the same shape.
//
// Column k of V^T is 1 on every source row: column k of the accumulator is
// the row sum of the same bf16 probabilities.  A row sum below 2^-60 marks
// the workgroup's two 128-row blocks in the fallback array; fwd_bf16 then
// redoes them with a running reference.
#include "tile_bf16.hpp"

namespace ssc {
namespace tb {

typedef unsigned short u16x8v __attribute__((ext_vector_type(8)));

template <int D, int KP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_wide(FwdArgs a) {
  constexpr int NW = 4;
  using SK = TileSrc<D, NW>;
  using SV = TileSrcG<KP, NW>;
  constexpr int NIK = SK::NI, NIV = SV::NI, KB = NIK * 1024, VB = NIV * 1024;
  constexpr int NCB = KP / 32, NS = D / 16;
  __shared__ __attribute__((aligned(1024))) char sK0[KB];
  __shared__ __attribute__((aligned(1024))) char sK1[KB];
  __shared__ __attribute__((aligned(1024))) char sK2[KB];
  __shared__ __attribute__((aligned(1024))) char sV0[VB];
  __shared__ __attribute__((aligned(1024))) char sV1[VB];
  __shared__ __attribute__((aligned(1024))) char sV2[VB];
  __shared__ int s_under;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int row0 = blockIdx.x * 256 + wave * 64 + l32;  // row of block rb: row0 + 32 rb
  const int nt = (a.n_M + kTile - 1) / kTile;

  SK sK;
  sK.init(a.Kp, a.n_M);
  SV sV;
  sV.init(a.Vt, a.groupsVt);
  constexpr int NJK = SK::NJ, NJV = SV::NJ, NL = NJK + NJV;
  static_assert(NL < 16, "vmcnt field");
  // load j of a wave is tile instruction wave + j NW, clamped to the tile's
  // last (a repeat writes the same bytes to the same place): NL loads per
  // wave and step, no branch
  int lidx[NL], loff[NL];
  static_for<NL>([&](auto j) {
    if (j < NJK) {
      lidx[j] = min(wave + j * NW, NIK - 1);
      loff[j] = SK::dense_offset(lidx[j], lane, 0);
    } else {
      lidx[j] = min(wave + (j - NJK) * NW, NIV - 1);
      loff[j] = (int)SV::dense_offset(lidx[j], lane, 0);
    }
  });
  auto load_k = [&](const int tile, char* dst, const int j) __attribute__((always_inline)) {
    sK.load_dense_at(dst, sK.window(tile * kTile), loff[j], lidx[j], 0);
  };
  auto load_v = [&](const int tile, char* dst, const int j) __attribute__((always_inline)) {
    sV.load_at(dst, sV.window(tile * kGroupsPerTile), (unsigned)loff[NJK + j], lidx[NJK + j], 0);
  };

  // Q fragments of both row blocks and their bounded references (a negative
  // scale is folded into Q by an exact sign flip)
  const bool neg = a.c2 < 0.f;
  const float c2 = neg ? -a.c2 : a.c2;
  bf16x8 qf[2][NS];
  float m_bound[2];
  {
    float km2 = 0.f;
    for (int j = lane; j < kNormParts; j += 64) km2 = fmaxf(km2, a.knorm2[j]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) km2 = fmaxf(km2, __shfl_xor(km2, m, 64));
    const bf16* Q = reinterpret_cast<const bf16*>(a.Q);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = row0 + 32 * rb;
      const bool ok = row < a.n_N;
      float qn2 = 0.f;
#pragma unroll
      for (int dc = 0; dc < NS; ++dc) {
        bf16x8 v = ok ? *reinterpret_cast<const bf16x8*>(Q + (size_t)row * D + dc * 16 + h * 8) : bf16x8{};
        if (neg) v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u16x8v, v) ^ (unsigned short)0x8000);
        qf[rb][dc] = v;
#pragma unroll
        for (int e = 0; e < 8; ++e) qn2 = fmaf((float)v[e], (float)v[e], qn2);
      }
      qn2 += xor32(qn2);
      m_bound[rb] = c2 * sqrtf(qn2 * km2);
    }
  }
  RowReaderP<D> rk;
  rk.init(l32, h);
  GroupReader gv;
  gv.init(l32, h);

  f32x16 acc[2][NCB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = f32x16{};
  if (tid == 0) s_under = 0;

  // element pair 2m, 2m + 1 of the scores of row block rb, key half kh, into
  // the probability operand of key chunk 2 kh + m / 4
  auto slice = [&](const f32x16& s_, bf16x8* pn_, const int rb, const int m) __attribute__((always_inline)) {
    const float p0 = fexp2(fmaf(s_[2 * m], c2, -m_bound[rb]));
    const float p1 = fexp2(fmaf(s_[2 * m + 1], c2, -m_bound[rb]));
    put_pair(pn_[m >> 2], m & 3, p0, p1);
  };
  constexpr int AH = 4, UA = 2 * NS, UB = 4 * NCB;
  // scores of one tile for both row blocks: UA operand reads, 2 UA MFMAs
  auto scores = [&](const char* Kt, f32x16 (&s_)[2][2]) __attribute__((always_inline)) {
    bf16x8 ring[AH];
    static_for<AH>([&](auto u) { ring[u] = rk.read(Kt, u / NS, u % NS); });
    static_for<UA>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 cur = ring[u % AH];
      if (u + AH < UA) ring[u % AH] = rk.read(Kt, (u + AH) / NS, (u + AH) % NS);
      constexpr int kh = u / NS, cc = u % NS;
      s_[0][kh] = mma(cur, qf[0][cc], s_[0][kh]);
      s_[1][kh] = mma(cur, qf[1][cc], s_[1][kh]);
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  // softmax of a tile's scores into its probability operands (both blocks)
  auto softmax_all = [&](const f32x16 (&s_)[2][2], bf16x8 (&p_)[2][4]) __attribute__((always_inline)) {
    static_for<2>([&](auto rb) {
      static_for<2>([&](auto kh) {
        static_for<8>([&](auto m) { slice(s_[rb][kh], &p_[rb][2 * kh], rb, m); });
      });
    });
  };

  // prologue: K(0..2), V(0..1); scores and softmax of tile 0
  static_for<NJK>([&](auto j) {
    load_k(0, sK0, j);
    load_k(1, sK1, j);
    load_k(2, sK2, j);
  });
  static_for<NJV>([&](auto j) {
    load_v(0, sV0, j);
    load_v(1, sV1, j);
  });
  wait_loads();
  __syncthreads();
  bf16x8 pc[2][4];  // probabilities of the tile whose value products run next
  {
    f32x16 s0[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) s0[rb][0] = s0[rb][1] = f32x16{};
    scores(sK0, s0);
    softmax_all(s0, pc);
  }
  __syncthreads();  // every wave is done with K(0) before step 0 refills its buffer

  // Step t: scores of tile t + 1 from Kr, value products of tile t from Vr
  // (against pc) with the softmax of tile t + 1 spread between them; loads
  // K(t + 3) into Kw and V(t + 2) into Vw (their previous tiles were read in
  // step t - 1).
  constexpr int LSTRIDE = (UA + UB) / NL > 1 ? (UA + UB) / NL : 1;
  bf16x8 pn_half[2][2];  // probabilities of the next tile's current key half
  auto load_j = [&](const int t, char* Kw, char* Vw, const int j) __attribute__((always_inline)) {
    if (j < NJK) load_k(t + 3, Kw, j);
    else load_v(t + 2, Vw, j - NJK);
  };
  // A step runs as two halves, one per key half kh of the tiles: the scores
  // of tile t + 1's key half kh for both row blocks (NS x 2 MFMAs), then the
  // value products of tile t's key chunks 2 kh, 2 kh + 1 (NCB x 2 x 2 MFMAs)
  // with the softmax of those scores between them; only one half's scores
  // are live at a time.
  constexpr int UAH = NS, UBH = 2 * NCB, UH = UAH + UBH;
  auto step = [&](const int t, const char* Kr, char* Kw, const char* Vr, char* Vw) __attribute__((always_inline)) {
    static_for<2>([&](auto kh) {
      f32x16 sn[2] = {f32x16{}, f32x16{}};
      bf16x8 ring[AH];
      // operand u of the half: K fragments first, then V^T fragments
      auto operand = [&](const int u) -> bf16x8 {
        if (u < UAH) return rk.read(Kr, kh, u);
        const int v = u - UAH;
        return gv.read(Vr, v / 2, 2 * kh + v % 2);
      };
      static_for<AH>([&](auto u) { ring[u] = operand(u); });
      static_for<UH>([&](auto u) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 cur = ring[u % AH];
        if (u + AH < UH) ring[u % AH] = operand(u + AH);
        if (u < UAH) {
          sn[0] = mma(cur, qf[0][u], sn[0]);
          sn[1] = mma(cur, qf[1][u], sn[1]);
        } else {
          constexpr int v = u - UAH, cb = v / 2, kc = 2 * kh + v % 2;
          acc[0][cb] = mma(cur, pc[0][kc], acc[0][cb]);
          acc[1][cb] = mma(cur, pc[1][kc], acc[1][cb]);
          // 16 slices (rb, m) of this half's scores over the value steps;
          // they overwrite the probability chunks 2 kh, 2 kh + 1 of pc only
          // after the last value product that reads them
          static_for<16>([&](auto q) {
            if (q * UBH / 16 == v) slice(sn[q / 8], &pn_half[q / 8][0], q / 8, q % 8);
          });
        }
        constexpr int w = kh * UH + u;
        if (w % LSTRIDE == 0 && w / LSTRIDE < NL) load_j(t, Kw, Vw, w / LSTRIDE);
      });
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        pc[rb][2 * kh] = pn_half[rb][0];
        pc[rb][2 * kh + 1] = pn_half[rb][1];
      }
    });
    static_for<NL>([&](auto j) {
      if (j >= (2 * UH + LSTRIDE - 1) / LSTRIDE) load_j(t, Kw, Vw, j);
    });
    // this wave's loads of the previous step have landed (in-order counter)
    // and after the barrier every wave's have; the wait as a builtin so the
    // compiler's own wait insertion counts it, the barrier plain because the
    // fence of __syncthreads would also wait for this step's loads.  Every
    // LDS read of the step has fed its MFMA.
    __builtin_amdgcn_s_waitcnt(0x0F70 | NL);  // vmcnt(NL)
    asm volatile("s_barrier" ::: "memory");
  };

  int t = 0;
  for (; t + 2 < nt; t += 3) {
    step(t, sK1, sK0, sV0, sV2);
    step(t + 1, sK2, sK1, sV1, sV0);
    step(t + 2, sK0, sK2, sV2, sV1);
  }
  if (t < nt) {
    step(t, sK1, sK0, sV0, sV2);
    ++t;
  }
  if (t < nt) step(t, sK2, sK1, sV1, sV0);
  wait_loads();

  // ---- row sums from the ones column, the underflow check, the stores
  const int kk = a.k & 31, hk = (kk >> 2) & 1, ik = 4 * (kk >> 3) + (kk & 3), ck = a.k >> 5;
  float l_tot[2];
  bool low = false;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float l_part = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (cb == ck && i == ik && h == hk) l_part = acc[rb][cb][i];
    l_tot[rb] = l_part + xor32(l_part);
    if (row0 + 32 * rb < a.n_N && !(l_tot[rb] >= 0x1p-60f)) low = true;
  }
  if (low) atomicOr(&s_under, 1);
  __syncthreads();
  const bool under = s_under != 0;
  if (tid < 2) {
    const int b = 2 * blockIdx.x + tid, nb = (a.n_N + 127) / 128;
    if (b < nb) a.fallback_out[b] = under ? 1 : 0;
  }
  if (under) return;
  const bool vec = (a.k & 3) == 0;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = row0 + 32 * rb;
    if (row >= a.n_N) continue;
    const float inv = 1.f / l_tot[rb];
    float* Orow = a.O + (size_t)row * a.k;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = cb * 32 + 8 * g + 4 * h;
        if (vec) {
          if (c < a.k)
            *reinterpret_cast<f32x4*>(Orow + c) = f32x4{acc[rb][cb][4 * g] * inv, acc[rb][cb][4 * g + 1] * inv,
                                                         acc[rb][cb][4 * g + 2] * inv, acc[rb][cb][4 * g + 3] * inv};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < a.k) Orow[c + e] = acc[rb][cb][4 * g + e] * inv;
        }
      }
    if (h == 0) a.lse[row] = (m_bound[rb] + log2f(l_tot[rb])) * kLn2;
  }
}

}  // namespace tb

// The wide forward needs a spare padded column for the row sums (k < KP).
hipError_t launch_fwd_wide(int D, int KP, const FwdArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                          \
  if (D == DD && KP == KK) {                                                                   \
    hipLaunchKernelGGL((tb::fwd_wide<DD, KK>), dim3(grid), dim3(256), 0, st, a);               \
    return hipGetLastError();                                                                  \
  }
  SSC_L(128, 224)
  SSC_L(128, 128)
  SSC_L(128, 64)
  SSC_L(128, 32)
  SSC_L(64, 224)
  SSC_L(64, 128)
  SSC_L(64, 64)
  SSC_L(64, 32)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
