// Paired-wave bf16 forward of the dense coupling on gfx950 (project page
// "Spatial-Spectral Coupling as Attention", section "How it works": the
// product softmax(F_N F_M^T / sqrt(d)) Phi_M; section "The bottleneck": the
// map itself is never stored).
//
// One workgroup = 8 waves over 128 target rows, two waves per SIMD.  Waves w
// and w + 4 own the same 32 rows and split every tile of 64 source rows:
// wave w takes keys 0-31, wave w + 4 keys 32-63.  Each wave forms its 32 x 32
// scores S^T = K Q^T (D / 16 MFMAs, K rows read in the sigma_row order), the
// probabilities P = exp2(S c2 - m) against the row's bounded reference
// m = c2 |q| max_j |k_j| (no probability exceeds 1 and no running maximum is
// needed, so partial sums of the two waves simply add), and its share of
// O^T += V^T P^T (KP / 32 x 2 MFMAs, V from its grouped-transposed copy).
// A single wave per SIMD cannot keep the matrix core busy (its MFMAs issue
// one after another with the softmax, reads and waits in between); two
// waves of the same work on one SIMD fill each other's gaps.
//
// Pipeline: step t issues, as one chain of MFMAs, the scores of tile t + 1
// and the value products of tile t - 1, with the softmax of tile t spread
// between them, so every step of every wave has the same mix of matrix and
// vector work.  K and V tiles are triple-buffered and loaded two steps
// before their use (K(t + 3) and V(t + 1) during step t): the wait at the
// end of a step is for the loads of the step before, which have had a whole
// step to land.
//
// Column k of the transposed V is 1 on every source row, so column k of the
// accumulator is the row sum of the same bf16 probabilities.  At the end the
// pair adds its accumulators through LDS.  A row whose sum falls below
// 2^-60 (the bound sat far above its scores) marks its workgroup in a flag
// array; fwd_bf16 then redoes the marked workgroups with a running
// reference (exact in every case).
#include "tile_bf16.hpp"

namespace ssc {
namespace tb {

typedef unsigned short u16x8w __attribute__((ext_vector_type(8)));

template <int D, int KP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_pair(FwdArgs a) {
  constexpr int NW = 8;  // waves, all of them load
  using SK = TileSrc<D, NW>;
  using SV = TileSrcG<KP, NW>;
  // a tile buffer holds exactly the tile's slots: the loads of a wave's last
  // round that fall past the tile are skipped
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
  const int rb = wave & 3, kh = wave >> 2;  // row block; key half of every tile
  const int h = lane >> 5, l32 = lane & 31;
  const int row = blockIdx.x * 128 + rb * 32 + l32;
  const bool row_ok = row < a.n_N;
  const int nt = (a.n_M + kTile - 1) / kTile;

  SK sK;
  sK.init(a.Kp, a.n_M);
  SV sV;
  sV.init(a.Vt, a.groupsVt);
  constexpr int NJK = SK::NJ, NJV = SV::NJ, NL = NJK + NJV;
  // Load j of a wave is tile instruction wave + j NW.  Past the tile's last
  // instruction a wave repeats that last one (the same bytes to the same LDS
  // address as its owner, so the duplicate is harmless): every wave then
  // issues NL loads per step, with no branch, and the compiler's wait
  // bookkeeping and the wait at the end of a step see the same count.
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

  // Q fragments and the bounded reference (a negative scale is folded into
  // Q by an exact sign flip, so the reference is always a maximum)
  const bool neg = a.c2 < 0.f;
  const float c2 = neg ? -a.c2 : a.c2;
  bf16x8 qf[NS];
  {
    const bf16* Q = reinterpret_cast<const bf16*>(a.Q);
#pragma unroll
    for (int dc = 0; dc < NS; ++dc) {
      qf[dc] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + (size_t)row * D + dc * 16 + h * 8) : bf16x8{};
      if (neg) qf[dc] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u16x8w, qf[dc]) ^ (unsigned short)0x8000);
    }
  }
  float m_bound;
  {
    float qn2 = 0.f;
#pragma unroll
    for (int dc = 0; dc < NS; ++dc)
#pragma unroll
      for (int e = 0; e < 8; ++e) qn2 = fmaf((float)qf[dc][e], (float)qf[dc][e], qn2);
    qn2 += xor32(qn2);
    float km2 = 0.f;
    for (int j = lane; j < kNormParts; j += 64) km2 = fmaxf(km2, a.knorm2[j]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) km2 = fmaxf(km2, __shfl_xor(km2, m, 64));
    m_bound = c2 * sqrtf(qn2 * km2);
  }
  RowReaderP<D> rk;
  rk.init(l32, h, kh);  // the rows of this wave's key half
  GroupReaderHalf rv;
  rv.init(l32, h, kh);

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  if (tid == 0) s_under = 0;

  constexpr int AH = 4, UV = 2 * NCB, U = NS + UV;
  // element pair 2m, 2m + 1 of the scores s_ into the probability operand pn_
  auto slice = [&](const f32x16& s_, bf16x8* pn_, const int m) __attribute__((always_inline)) {
    const float p0 = fexp2(fmaf(s_[2 * m], c2, -m_bound));
    const float p1 = fexp2(fmaf(s_[2 * m + 1], c2, -m_bound));
    put_pair(pn_[m >> 2], m & 3, p0, p1);
  };
  // scores of this wave's key half of a tile: NS MFMAs into s_, operand
  // reads AH steps ahead, f(u) between them
  auto scores = [&](const char* Kt, f32x16& s_, auto f) __attribute__((always_inline)) {
    bf16x8 ring[AH];
    static_for<AH>([&](auto u) { ring[u] = rk.read(Kt, 0, u); });
    static_for<NS>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 cur = ring[u % AH];
      if (u + AH < NS) ring[u % AH] = rk.read(Kt, 0, u + AH);
      s_ = mma(cur, qf[u], s_);
      f(u);
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  // value products of one tile: its chunks 2 kh, 2 kh + 1 against pp_
  auto values = [&](const char* Vr, const bf16x8* pp_) __attribute__((always_inline)) {
    bf16x8 ring[AH];
    static_for<AH>([&](auto u) { ring[u] = rv.read(Vr, u % NCB, u / NCB); });
    static_for<UV>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 cur = ring[u % AH];
      if (u + AH < UV) ring[u % AH] = rv.read(Vr, (u + AH) % NCB, (u + AH) / NCB);
      acc[u % NCB] = mma(cur, pp_[u / NCB], acc[u % NCB]);
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: K(0), K(1), K(2) and V(0); the scores of tile 0
  static_for<NJK>([&](auto j) {
    load_k(0, sK0, j);
    load_k(1, sK1, j);
    load_k(2, sK2, j);
  });
  static_for<NJV>([&](auto j) { load_v(0, sV0, j); });
  wait_loads();
  __syncthreads();
  f32x16 sc = f32x16{};  // scores of the tile whose softmax runs in the next step
  bf16x8 pp[2] = {bf16x8{}, bf16x8{}};  // probabilities of the tile whose value products run next
  scores(sK0, sc, [](auto) {});
  __syncthreads();  // every wave is done with K(0) before step 0 refills its buffer

  // Step t reads K(t + 1) from K[(t + 1) % 3] and V(t - 1) from V[(t - 1) % 3]
  // and loads K(t + 3) into K[t % 3] and V(t + 1) into V[(t + 1) % 3], whose
  // previous tiles were read in step t - 1.  Past the end the windows are
  // empty and the loads write zeros into buffers nobody reads.
  constexpr int LSTRIDE = U / NL > 1 ? U / NL : 1;
  auto load_j = [&](const int t, char* Kw, char* Vw, const int j) __attribute__((always_inline)) {
    if (j < NJK) load_k(t + 3, Kw, j);
    else load_v(t + 1, Vw, j - NJK);
  };
  auto end_step = [&]() __attribute__((always_inline)) {
    // this wave's loads of the step before have landed (in-order counter);
    // after the barrier every wave's have.  A plain barrier: the fence of
    // __syncthreads would wait for this step's loads too.  Every LDS read
    // of the step has fed its MFMA before the barrier, so no read is still
    // pending when another wave's load overwrites its buffer.
    // (the wait as a builtin, so that the compiler's own wait insertion knows
    // of it)
    static_assert(NL < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | NL);  // vmcnt(NL), expcnt and lgkmcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
  };
  auto full_step = [&](const int t, const char* Kr, char* Kw, const char* Vr, char* Vw) __attribute__((always_inline)) {
    bf16x8 pn[2];
    f32x16 sn = f32x16{};
    auto operand = [&](const int u) -> bf16x8 {
      if (u < NS) return rk.read(Kr, 0, u);
      const int v = u - NS;
      return rv.read(Vr, v % NCB, v / NCB);
    };
    bf16x8 ring[AH];
    static_for<AH>([&](auto u) { ring[u] = operand(u); });
    static_for<U>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 cur = ring[u % AH];
      if (u + AH < U) ring[u % AH] = operand(u + AH);
      if (u < NS) {
        sn = mma(cur, qf[u], sn);
      } else {
        constexpr int v = u - NS;
        acc[v % NCB] = mma(cur, pp[v / NCB], acc[v % NCB]);
      }
      static_for<8>([&](auto m) {
        if (m * U / 8 == u) slice(sc, pn, m);
      });
      if (u % LSTRIDE == 0 && u / LSTRIDE < NL) load_j(t, Kw, Vw, u / LSTRIDE);
    });
    __builtin_amdgcn_sched_barrier(0);
    static_for<NL>([&](auto j) {
      if (j >= (U + LSTRIDE - 1) / LSTRIDE) load_j(t, Kw, Vw, j);
    });
    sc = sn;
    pp[0] = pn[0];
    pp[1] = pn[1];
    end_step();
  };

  // step 0: scores of tile 1 (if any) with the softmax of tile 0; loads K(3), V(1)
  {
    static_for<NL>([&](auto j) { load_j(0, sK0, sV1, j); });
    bf16x8 pn[2];
    if (nt > 1) {
      f32x16 sn = f32x16{};
      scores(sK1, sn, [&](auto u) {
        static_for<8>([&](auto m) {
          if (m * NS / 8 == u) slice(sc, pn, m);
        });
      });
      sc = sn;
    } else {
      static_for<8>([&](auto m) { slice(sc, pn, m); });
    }
    pp[0] = pn[0];
    pp[1] = pn[1];
    end_step();
  }
  // steady steps 1 .. nt - 2, three at a time (the buffer rotation)
  int t = 1;
  for (; t + 2 < nt - 1; t += 3) {
    full_step(t, sK2, sK1, sV0, sV2);
    full_step(t + 1, sK0, sK2, sV1, sV0);
    full_step(t + 2, sK1, sK0, sV2, sV1);
  }
  if (t < nt - 1) {
    full_step(t, sK2, sK1, sV0, sV2);
    ++t;
  }
  if (t < nt - 1) {
    full_step(t, sK0, sK2, sV1, sV0);
    ++t;
  }
  // step nt - 1 (if it is not step 0): softmax of tile nt - 1, value products
  // of tile nt - 2; step nt: value products of tile nt - 1, which was loaded
  // in the step before.  These run once, so their buffers are picked at run
  // time.
  auto vbuf = [&](const int tile) -> const char* {
    const int r = tile % 3;
    return r == 0 ? sV0 : r == 1 ? sV1 : sV2;
  };
  wait_loads();
  __syncthreads();
  if (t == nt - 1 && t >= 1) {
    bf16x8 pn[2];
    static_for<8>([&](auto m) { slice(sc, pn, m); });
    values(vbuf(nt - 2), pp);
    pp[0] = pn[0];
    pp[1] = pn[1];
  }
  values(vbuf(nt - 1), pp);

  // ---- the pair adds its accumulators through LDS (the tile buffers are free
  // now): first the row sums, then each 32-column block in rounds of F
  // fields; the key-half-0 wave of each pair normalises and stores
  __syncthreads();
  constexpr int RBYTES = KB > VB ? KB : VB;
  constexpr int F = RBYTES >= 16384 ? 16 : RBYTES >= 8192 ? 8 : 4;
  static_assert(4 * F * 64 * 4 <= RBYTES, "reduction buffer");
  float* red = reinterpret_cast<float*>(KB > VB ? sK0 : sV0);  // [4 row blocks][F fields][64 lanes]
  float* lred = reinterpret_cast<float*>(KB > VB ? sV1 : sK1);
  const int kk = a.k & 31, hk = (kk >> 2) & 1, ik = 4 * (kk >> 3) + (kk & 3), ck = a.k >> 5;
  float l_part = 0.f;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (cb == ck && i == ik && h == hk) l_part = acc[cb][i];
  if (kh == 1) lred[rb * 64 + lane] = l_part;
  __syncthreads();
  if (kh == 0) l_part += lred[rb * 64 + lane];
  const float l_tot = l_part + xor32(l_part);
  if (kh == 0 && row_ok && !(l_tot >= 0x1p-60f)) atomicOr(&s_under, 1);
  __syncthreads();
  const bool under = s_under != 0;
  if (tid == 0) a.fallback_out[blockIdx.x] = under ? 1 : 0;
  if (under) return;
  const float inv = 1.f / l_tot;
  float* Orow = a.O + (size_t)row * a.k;
  const bool vec = (a.k & 3) == 0;
  static_for<NCB>([&](auto cb) {
    static_for<16 / F>([&](auto fg) {
      if (kh == 1) {
#pragma unroll
        for (int i = 0; i < F; ++i) red[(rb * F + i) * 64 + lane] = acc[cb][fg * F + i];
      }
      __syncthreads();
      if (kh == 0) {
#pragma unroll
        for (int i = 0; i < F; ++i) acc[cb][fg * F + i] += red[(rb * F + i) * 64 + lane];
      }
      __syncthreads();
    });
    if (kh == 0 && row_ok) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = cb * 32 + 8 * g + 4 * h;
        if (vec) {
          if (c < a.k)
            *reinterpret_cast<f32x4*>(Orow + c) = f32x4{acc[cb][4 * g] * inv, acc[cb][4 * g + 1] * inv,
                                                         acc[cb][4 * g + 2] * inv, acc[cb][4 * g + 3] * inv};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < a.k) Orow[c + e] = acc[cb][4 * g + e] * inv;
        }
      }
    }
  });
  if (kh == 0 && row_ok && h == 0) a.lse[row] = (m_bound + log2f(l_tot)) * kLn2;
}

}  // namespace tb

// The paired forward needs a spare padded column for the row sums (k < KP);
// KP = 256 with k = 256 uses fwd_bf16 directly.
hipError_t launch_fwd_pair(int D, int KP, const FwdArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                          \
  if (D == DD && KP == KK) {                                                                   \
    hipLaunchKernelGGL((tb::fwd_pair<DD, KK>), dim3(grid), dim3(512), 0, st, a);               \
    return hipGetLastError();                                                                  \
  }
  SSC_L(128, 224)
  SSC_L(128, 256)
  SSC_L(128, 128)
  SSC_L(128, 64)
  SSC_L(128, 32)
  SSC_L(64, 224)
  SSC_L(64, 256)
  SSC_L(64, 128)
  SSC_L(64, 64)
  SSC_L(64, 32)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
