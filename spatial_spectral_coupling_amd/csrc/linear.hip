// Linear-attention (ELU feature map) coupling on gfx950: the pages'
// linearized baseline, which replaces the softmax by the feature map
// phi(x) = elu(x) + 1 (ai4snews digest, "Interpretation"; project page,
// "Runtime and memory", Table 1 row "Linear attention (ELU)"):
//
//   KV = phi(K)^T V,  z = phi(K)^T 1,  den_i = phi(q_i).z,
//   O_i = phi(q_i) KV / den_i.
//
// Both products with the d x k matrices are done on bf16 MFMA with the
// normaliser folded in: the source rows are extended by a constant column
// (V_ext = [V | 1] at column kp-1), so one Gram product gives KV and z
// together, and one row product gives phi(q_i) KV and den_i together.  The
// backward uses the same folding:
//   g_i = dO_i / den_i, s_i = (dO_i . O_i) / den_i, G_ext = [g | -s],
//   dA = G_ext KVz_ext^T (gradient w.r.t. phi(Q)), dQ = phi'(Q) * dA,
//   dKVz_ext = phi(Q)^T G_ext = [dKV | dz],
//   dK = phi'(K) * (V_ext dKVz_ext^T), dV = phi(K) dKV.
// Everything is O(n (d + k)) memory traffic: the kernels are HBM / latency
// bound; the Gram sums are split over row blocks and reduced in a fixed
// order (deterministic).  The forward is three launches (Gram sums,
// reduction, rows); so is the backward, whose two Gram sums (the second one
// also forming s), two reductions and three row passes (dQ, dK, dV) each
// share a launch, as none reads what the others of its launch write.
// With FEAT = 1 the kernels take precomputed feature rows in place of Q and
// K (identity map, phi' = 1: the "dQ" / "dK" outputs are then the gradients
// w.r.t. the features); the Performer coupling runs on them.
#include "tile_bf16.hpp"

namespace ssc {
namespace lin {

using tb::Geo;
using tb::put_pair;
using tb::RowReader;
using tb::static_for;
using tb::TrReader;

constexpr int kGramTile = 128;  // rows per LDS tile of the Gram kernel
constexpr int kGramWaves = 8;   // waves per workgroup of the Gram kernel (two per SIMD)
constexpr int kApplyRows = 128; // rows per workgroup of the row kernels (4 waves x 32)

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __builtin_amdgcn_exp2f(x * kLog2e); }
template <int FEAT>
__device__ __forceinline__ float feat(float x) { return FEAT ? x : phi(x); }

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Eight consecutive elements c0 .. c0+7 of a row of width w (elements past w
// read as 0); vector load when the row stride allows it.
__device__ __forceinline__ void row8(const bf16* row, int c0, int w, bool vec, float* out) {
  if (vec && c0 + 8 <= w) {
    const bf16x8 v = ld8(row + c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = c0 + e < w ? (float)row[c0 + e] : 0.f;
  }
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) put_pair(r, m, v[2 * m], v[2 * m + 1]);
  return r;
}

// Copy a row-major bf16 matrix [ROWS x W] (global, unpadded) into an LDS
// tile with the padded pitch of Geo<W>; loads are issued in batches of
// eight before their stores, so they are in flight together.
template <int W, int ROWS>
__device__ __forceinline__ void stage_matrix(char* lds, const bf16* g, int tid) {
  constexpr int CW = W / 8, N = ROWS * CW, B = 8;
  for (int base = 0; base < N; base += B * 256) {
    bf16x8 v[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int ch = base + j * 256 + tid;
      if (ch < N) v[j] = ld8(g + (size_t)ch * 8);
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int ch = base + j * 256 + tid;
      if (ch < N) {
        const int r = ch / CW, c = ch - r * CW;
        *reinterpret_cast<bf16x8*>(lds + r * Geo<W>::PITCH + c * 16) = v[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gram sums over a block of rows:  part[b] = A^T B  ([D x KP], fp32)
//   MODE 0 (forward):  A = phi(K),  B = V_ext = [V | 1 at column KP-1]
//   MODE 1 (backward): A = phi(Q),  B = G_ext = [dO / den | -s at KP-1]
// Rows past the end contribute 0.  In MODE 1 the row terms rden = 1 / den
// and s = (dO . O) / den are formed here too: each thread adds the products
// of its 8-column chunk of dO and O, the chunk sums of a row are added in
// column order, and -s is then written into the last column of the tile
// (rden and s also go out for the dQ rows).
// ---------------------------------------------------------------------------
template <int D, int KP, int MODE, int FEAT>
struct GramCfg {
  static constexpr int AP = Geo<D>::PITCH, BP = Geo<KP>::PITCH;
  // identity features, backward: G_ext as a bf16 high + low pair
  static constexpr bool BLO = FEAT == 1 && MODE == 1;
  static constexpr int PS = KP / 8 + 1;  // row stride of the chunk dot products
  static constexpr int bytes(int tr) { return tr * AP + tr * BP * (BLO ? 2 : 1) + (MODE == 1 ? tr * PS * 4 : 0); }
  // rows per LDS tile: halved for the backward (its tile loads of dO and O
  // stay in flight in registers during the MFMAs) and where the tile would
  // not fit the LDS
  static constexpr int TR = MODE == 1 || bytes(kGramTile) > 160 * 1024 ? kGramTile / 2 : kGramTile;
  static constexpr int LDS = bytes(TR);
};

template <int D, int KP, int MODE, int FEAT>
__device__ __forceinline__ void gram_body(const LinArgs& a, int blk, char* smem, float* part_out) {
  using C = GramCfg<D, KP, MODE, FEAT>;
  constexpr int AP = C::AP, BP = C::BP, TR = C::TR, PS = C::PS;
  constexpr bool BLO = C::BLO;
  char* As = smem;
  char* Bs = As + TR * AP;
  char* Bl = Bs + TR * BP;
  float* pdot = reinterpret_cast<float*>(Bs + TR * BP * (BLO ? 2 : 1));
  // kGramWaves waves: wave w owns the 32-row block mb = w % NMB of the
  // output and its column blocks nb = w / NMB + t * (kGramWaves / NMB), so
  // its A operand fragment is read once per k step
  constexpr int NMB = D / 32, NNB = KP / 32, WPM = kGramWaves / NMB, NBW = (NNB + WPM - 1) / WPM;
  constexpr int NT = kGramWaves * 64;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mb = wave % NMB, nb0 = wave / NMB;
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  TrReader<D> ta;
  ta.init(tr_r, tr_c);
  TrReader<KP> tbr;
  tbr.init(tr_r, tr_c);

  const int n = MODE == 0 ? a.n_M : a.n_N;
  const int r_begin = blk * a.gram_rows;
  const int r_end = min(n, r_begin + a.gram_rows);
  const bf16* X = reinterpret_cast<const bf16*>(MODE == 0 ? a.K : a.Q);
  const bf16* Y = reinterpret_cast<const bf16*>(MODE == 0 ? a.V : a.dO);
  const bool vec = (a.k & 7) == 0;
  const bool vec4 = (a.k & 3) == 0;
  const int nch = (a.k + 7) / 8;  // chunks of a row that hold data

  f32x16 acc[NBW];
#pragma unroll
  for (int t = 0; t < NBW; ++t) acc[t] = f32x16{};

  // The global loads of a tile go into registers; those of the next tile are
  // issued as soon as the current one is in LDS, so they are in flight
  // during its MFMAs.
  // 16-byte chunks of a tile and per thread (the last round may be partial)
  constexpr int CA = TR * (D / 8), CB = TR * (KP / 8);
  constexpr int NXA = (CA + NT - 1) / NT, NYB = (CB + NT - 1) / NT;
  bf16x8 xa[NXA], yb[NYB];
  f32x4 ob[MODE == 1 ? 2 * NYB : 1];
  float dv[MODE == 1 ? NYB : 1];
  auto load_tile = [&](int r0) {
#pragma unroll
    for (int j = 0; j < NXA; ++j) {
      const int ch = tid + NT * j, r = ch / (D / 8), c8 = ch - r * (D / 8), gr = r0 + r;
      xa[j] = (CA % NT == 0 || ch < CA) && gr < r_end ? ld8(X + (size_t)gr * D + c8 * 8) : bf16x8{};
    }
#pragma unroll
    for (int j = 0; j < NYB; ++j) {
      const int ch = tid + NT * j, r = ch / (KP / 8), c8 = ch - r * (KP / 8), gr = r0 + r;
      const bool in = (CB % NT == 0 || ch < CB) && gr < r_end && c8 * 8 < a.k;
      if (in && vec && c8 * 8 + 8 <= a.k) {
        yb[j] = ld8(Y + (size_t)gr * a.k + c8 * 8);
      } else if (in) {
        float v[8];
        row8(Y + (size_t)gr * a.k, c8 * 8, a.k, false, v);
        yb[j] = pack8(v);
      } else {
        yb[j] = bf16x8{};
      }
      if (MODE == 1) {
        const int jj = MODE == 1 ? j : 0;
        dv[jj] = gr < r_end ? a.den[gr] : 1.f;
        const float* Or = a.O + (size_t)(gr < r_end ? gr : 0) * a.k + c8 * 8;
        if (in && vec4 && c8 * 8 + 8 <= a.k) {
          ob[2 * jj] = *reinterpret_cast<const f32x4*>(Or);
          ob[2 * jj + 1] = *reinterpret_cast<const f32x4*>(Or + 4);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float o = in && c8 * 8 + e < a.k ? Or[e] : 0.f;
            if (e < 4) ob[2 * jj][e] = o;
            else ob[2 * jj + 1][e - 4] = o;
          }
        }
      }
    }
  };
  if (r_begin < r_end) load_tile(r_begin);

  for (int r0 = r_begin; r0 < r_end; r0 += TR) {
#pragma unroll
    for (int j = 0; j < NXA; ++j) {
      const int ch = tid + NT * j, r = ch / (D / 8), c8 = ch - r * (D / 8);
      if (CA % NT != 0 && ch >= CA) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = r0 + r < r_end ? feat<FEAT>((float)xa[j][e]) : 0.f;
      *reinterpret_cast<bf16x8*>(As + r * AP + c8 * 16) = pack8(v);
    }
#pragma unroll
    for (int j = 0; j < NYB; ++j) {
      const int ch = tid + NT * j, r = ch / (KP / 8), c8 = ch - r * (KP / 8), gr = r0 + r;
      if (CB % NT != 0 && ch >= CB) continue;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)yb[j][e];
      if (MODE == 1) {
        const int jj = MODE == 1 ? j : 0;
        float pd = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) pd += v[e] * (e < 4 ? ob[2 * jj][e] : ob[2 * jj + 1][e - 4]);
        if (gr < r_end && c8 < nch) pdot[r * PS + c8] = pd;
        const float rd = 1.f / dv[jj];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= rd;
      }
      if (MODE == 0 && gr < r_end && c8 == KP / 8 - 1) v[7] = 1.f;
      const bf16x8 hv = pack8(v);
      *reinterpret_cast<bf16x8*>(Bs + r * BP + c8 * 16) = hv;
      if (BLO) {
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = v[e] - (float)hv[e];
        *reinterpret_cast<bf16x8*>(Bl + r * BP + c8 * 16) = pack8(lo);
      }
    }
    if (r0 + TR < r_end) load_tile(r0 + TR);
    __syncthreads();
    if (MODE == 1) {
      // s of each row of the tile: its chunk sums in column order; -s goes
      // into column KP-1 (past k, so far a zero)
      const int gr = r0 + tid;
      if (tid < TR && gr < r_end) {
        float sum = 0.f;
        for (int c = 0; c < nch; ++c) sum += pdot[tid * PS + c];
        const float rd = 1.f / a.den[gr];
        const float sv = sum * rd;
        const bf16 hs = (bf16)(-sv);
        *reinterpret_cast<bf16*>(Bs + tid * BP + (KP - 1) * 2) = hs;
        if (BLO) *reinterpret_cast<bf16*>(Bl + tid * BP + (KP - 1) * 2) = (bf16)(-sv - (float)hs);
        a.rden[gr] = rd;
        a.s[gr] = sv;
      }
      __syncthreads();
    }
#pragma unroll
    for (int kc = 0; kc < TR / 16; ++kc) {
      const bf16x8 af = ta.frag(As, mb, kc);
#pragma unroll
      for (int t = 0; t < NBW; ++t) {
        const int nb = nb0 + WPM * t;
        if (NNB % WPM == 0 || nb < NNB) {
          acc[t] = mma(af, tbr.frag(Bs, nb, kc), acc[t]);
          if (BLO) acc[t] = mma(af, tbr.frag(Bl, nb, kc), acc[t]);
        }
      }
    }
    __syncthreads();
  }
  float* part = part_out + (size_t)blk * D * KP;
#pragma unroll
  for (int t = 0; t < NBW; ++t) {
    const int nb = nb0 + WPM * t;
    if (NNB % WPM == 0 || nb < NNB) {
#pragma unroll
      for (int i = 0; i < 16; ++i) part[(size_t)(mb * 32 + c_row(i, h)) * KP + nb * 32 + l32] = acc[t][i];
    }
  }
}

// Forward: the Gram sums of the key side alone.
template <int D, int KP, int FEAT>
__global__ __launch_bounds__(kGramWaves * 64) void lin_gram(LinArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GramCfg<D, KP, 0, FEAT>::LDS];
  gram_body<D, KP, 0, FEAT>(a, blockIdx.x, smem, a.part);
}

// Backward: both Gram sums in one launch (they read only inputs): workgroups
// [0, gM) sum phi(K)^T V_ext into part, the others phi(Q)^T G_ext into partN.
template <int D, int KP, int FEAT>
__global__ __launch_bounds__(kGramWaves * 64) void lin_gram_bwd(LinArgs a, int gM) {
  constexpr int L0 = GramCfg<D, KP, 0, FEAT>::LDS, L1 = GramCfg<D, KP, 1, FEAT>::LDS;
  __shared__ __attribute__((aligned(16))) char smem[L0 > L1 ? L0 : L1];
  if ((int)blockIdx.x < gM) gram_body<D, KP, 0, FEAT>(a, blockIdx.x, smem, a.part);
  else gram_body<D, KP, 1, FEAT>(a, (int)blockIdx.x - gM, smem, a.partN);
}

// Fixed-order sum of the Gram partials, written as bf16 in both layouts:
// M [D x KP] and MT [KP x D]; with Mlo / MTlo also the bf16 rounding of the
// remainder (the pair carries the sum to about 2^-17).
struct RedJob {
  const float* part;
  int nparts;
  bf16 *M, *MT, *Mlo, *MTlo;
};

template <int D, int KP>
__device__ __forceinline__ void reduce_body(const RedJob& j, int blk) {
  // eight threads per output element: thread u sums the partials u, u + 8,
  // ... (one of eight independent partial sums), then the eight sums are
  // combined in a fixed order (deterministic)
  __shared__ float s8[8][32];
  const int u = threadIdx.x >> 5, e = threadIdx.x & 31;
  const int idx = blk * 32 + e;
  const int nparts = j.nparts;
  float acc = 0.f;
  if (idx < D * KP) {
    // eight partials loaded together, added in the same order as one at a time
    const float* src = j.part + idx;
    constexpr size_t ST = (size_t)D * KP;
    int b = u;
    for (; b + 56 < nparts; b += 64) {
      float v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) v[m] = __builtin_nontemporal_load(src + (size_t)(b + 8 * m) * ST);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc += v[m];
    }
    for (; b < nparts; b += 8) acc += src[(size_t)b * ST];
  }
  s8[u][e] = acc;
  __syncthreads();
  if (u != 0 || idx >= D * KP) return;
  const float s = ((s8[0][e] + s8[1][e]) + (s8[2][e] + s8[3][e])) + ((s8[4][e] + s8[5][e]) + (s8[6][e] + s8[7][e]));
  const int d = idx / KP, c = idx - d * KP;
  const bf16 v = (bf16)s;
  j.M[idx] = v;
  j.MT[(size_t)c * D + d] = v;
  if (j.Mlo != nullptr) {
    const bf16 lo = (bf16)(s - (float)v);
    j.Mlo[idx] = lo;
    j.MTlo[(size_t)c * D + d] = lo;
  }
}

template <int D, int KP>
__global__ __launch_bounds__(256) void lin_reduce(RedJob j) {
  reduce_body<D, KP>(j, blockIdx.x);
}

// The backward's two reductions in one launch (G workgroups each).
template <int D, int KP>
__global__ __launch_bounds__(256) void lin_reduce2(RedJob j0, RedJob j1) {
  constexpr int G = (D * KP + 31) / 32;
  if ((int)blockIdx.x < G) reduce_body<D, KP>(j0, blockIdx.x);
  else reduce_body<D, KP>(j1, (int)blockIdx.x - G);
}

// ---------------------------------------------------------------------------
// Row kernels (a wave owns 32 rows; lane l32 owns row l32 of the wave's block)
//   MODE 0: O = phi(Q) KV / den, den = phi(Q) z        (LDS: KVz^T [KP x D])
//   MODE 1: dQ = phi'(Q) * (G_ext KVz_ext^T)            (LDS: KVz_ext [D x KP])
//   MODE 2: dK = phi'(K) * (V_ext dKVz_ext^T)            (LDS: dKVz_ext [D x KP])
//   MODE 3: dV = phi(K) dKV                              (LDS: dKVz_ext^T [KP x D])
// (one layout each, so two workgroups fit a CU).  With FEAT = 1 the matrix of
// modes 0, 1, 2 runs as a bf16 high + low pair (both in LDS, two MFMAs per
// step), and so does G_ext in mode 1.
// A lane loads the operand fragments of its own row into registers.  Modes
// 1 and 2 take them as the A operand (C[row][col]: a lane holds 32
// consecutive columns of 16 rows, so the dQ / dK stores are whole lines, and
// reads the phi' factor of those entries from Q or K); modes 0 and 3 take
// them as the B operand (C[col][row]: the lane holds its own row).
// ---------------------------------------------------------------------------
template <int D, int KP, int MODE, int FEAT>
struct ApplyCfg {
  // which layouts this mode reads, and whether with a low part
  static constexpr bool USE_T = MODE == 0 || MODE == 3;
  static constexpr bool USE_M = MODE == 1 || MODE == 2;
  static constexpr bool LO_T = FEAT && MODE == 0, LO_M = FEAT && USE_M;
  static constexpr int SZ_T = USE_T ? KP * Geo<D>::PITCH : 0;  // [KP x D] layout
  static constexpr int SZ_M = USE_M ? D * Geo<KP>::PITCH : 0;  // [D x KP] layout
  static constexpr int LDS = SZ_T * (LO_T ? 2 : 1) + SZ_M * (LO_M ? 2 : 1) + 16;
};

template <int D, int KP, int MODE, int FEAT>
__device__ __forceinline__ void apply_body(const LinArgs& a, int blk, char* lds) {
  using C = ApplyCfg<D, KP, MODE, FEAT>;
  constexpr bool USE_T = C::USE_T, USE_M = C::USE_M, LO_T = C::LO_T, LO_M = C::LO_M;
  constexpr int SZ_T = C::SZ_T, SZ_M = C::SZ_M;
  char* LT = lds;
  char* LTlo = lds + SZ_T;
  char* LM = lds + SZ_T * (LO_T ? 2 : 1);
  char* LMlo = LM + SZ_M;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int n = MODE >= 2 ? a.n_M : a.n_N;
  const int row = blk * kApplyRows + wave * 32 + l32;
  const bool row_ok = row < n;
  const bool vec = (a.k & 7) == 0;

  if (USE_T) stage_matrix<D, KP>(LT, reinterpret_cast<const bf16*>(MODE == 0 ? a.MT : a.dMT), tid);
  if (LO_T) stage_matrix<D, KP>(LTlo, reinterpret_cast<const bf16*>(a.MTlo), tid);
  if (USE_M) stage_matrix<KP, D>(LM, reinterpret_cast<const bf16*>(MODE == 1 ? a.M : a.dM), tid);
  if (LO_M) stage_matrix<KP, D>(LMlo, reinterpret_cast<const bf16*>(MODE == 1 ? a.Mlo : a.dMlo), tid);
  __syncthreads();

  RowReader<D> rT;
  rT.init(l32, h);
  RowReader<KP> rM;
  rM.init(l32, h);

  // this lane's row of phi(X) (MODE 0: Q, MODE 3: K) as bf16 fragments
  const bf16* X = reinterpret_cast<const bf16*>(MODE >= 2 ? a.K : a.Q) + (size_t)(row_ok ? row : 0) * D;
  bf16x8 xf[D / 16];
  if (MODE == 0 || MODE == 3) {
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      float v[8];
      row8(X, cc * 16 + 8 * h, D, true, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = row_ok ? feat<FEAT>(v[e]) : 0.f;
      xf[cc] = pack8(v);
    }
  }

  if (MODE == 0) {
    f32x16 acc[KP / 32];
#pragma unroll
    for (int mb = 0; mb < KP / 32; ++mb) {
      acc[mb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        acc[mb] = mma(rT.read(LT, mb, cc), xf[cc], acc[mb]);
        if (LO_T) acc[mb] = mma(rT.read(LTlo, mb, cc), xf[cc], acc[mb]);
      }
    }
    // den = C[KP-1][row]: element 15 of the last block, held by the h = 1 lanes
    const float own = acc[KP / 32 - 1][15], other = xor32(own);
    const float den = h ? own : other;
    if (row_ok) {
      const float rd = 1.f / den;
      float* Orow = a.O + (size_t)row * a.k;
#pragma unroll
      for (int mb = 0; mb < KP / 32; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = mb * 32 + 8 * g + 4 * h;
          if ((a.k & 3) == 0 && c + 4 <= a.k) {
            *reinterpret_cast<f32x4*>(Orow + c) =
                f32x4{acc[mb][4 * g] * rd, acc[mb][4 * g + 1] * rd, acc[mb][4 * g + 2] * rd, acc[mb][4 * g + 3] * rd};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (c + e < a.k) Orow[c + e] = acc[mb][4 * g + e] * rd;
          }
        }
      }
      if (h == 0) a.den[row] = FEAT ? __logf(den) + a.rowoff[row] : den;
    }
    return;
  }

  if (MODE == 1) {
    // G_ext row fragments: c < k: dO / den; c = KP-1: -s; else 0
    const bf16* dOr = reinterpret_cast<const bf16*>(a.dO) + (size_t)(row_ok ? row : 0) * a.k;
    const float rd = row_ok ? a.rden[row] : 0.f, sv = row_ok ? a.s[row] : 0.f;
    // identity features: G_ext as a bf16 high + low pair too (the product
    // takes hi.hi + lo.hi + hi.lo)
    bf16x8 gf[KP / 16], gl[FEAT ? KP / 16 : 1];
#pragma unroll
    for (int cc = 0; cc < KP / 16; ++cc) {
      float v[8];
      row8(dOr, cc * 16 + 8 * h, a.k, vec, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= rd;
      if (cc == KP / 16 - 1 && h == 1) v[7] = -sv;
      gf[cc] = pack8(v);
      if (FEAT) {
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = v[e] - (float)gf[cc][e];
        gl[FEAT ? cc : 0] = pack8(lo);
      }
    }
    // dQ as C[row][col] (the lane's G_ext fragments as the A operand): lane
    // (l32, h) holds rows base + c_row(i, h) at columns mb * 32 + l32, so a
    // store writes 32 consecutive columns of a row
    f32x16 acc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      acc[mb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < KP / 16; ++cc) {
        const bf16x8 mh = rM.read(LM, mb, cc);
        acc[mb] = mma(gf[cc], mh, acc[mb]);
        if (LO_M) acc[mb] = mma(gf[cc], rM.read(LMlo, mb, cc), acc[mb]);
        if (FEAT) acc[mb] = mma(gl[FEAT ? cc : 0], mh, acc[mb]);
      }
    }
    const int base = blk * kApplyRows + wave * 32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = base + c_row(i, h);
      if (r >= n) continue;
      const bf16* Qr = reinterpret_cast<const bf16*>(a.Q) + (size_t)r * D;
      float* out = a.dQ + (size_t)r * D;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
        const int d = mb * 32 + l32;
        out[d] = FEAT ? acc[mb][i] : dphi((float)Qr[d]) * acc[mb][i];
      }
    }
    return;
  }

  if (MODE == 2 || MODE == 3) {
  // MODE 2: V_ext row fragments (c < k: V; c = KP-1: 1; else 0)
  const bf16* Vr = reinterpret_cast<const bf16*>(a.V) + (size_t)(row_ok ? row : 0) * a.k;
  bf16x8 vf[KP / 16];
#pragma unroll
  for (int cc = 0; cc < KP / 16; ++cc) {
    float v[8];
    row8(Vr, cc * 16 + 8 * h, a.k, vec, v);
    if (cc == KP / 16 - 1 && h == 1) v[7] = 1.f;
    vf[cc] = pack8(v);
  }
  if (MODE == 2) {
  // dK as C[row][col], as dQ in mode 1
  f32x16 c1[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    c1[mb] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < KP / 16; ++cc) {
      c1[mb] = mma(vf[cc], rM.read(LM, mb, cc), c1[mb]);
      if (LO_M) c1[mb] = mma(vf[cc], rM.read(LMlo, mb, cc), c1[mb]);
    }
  }
  const int base = blk * kApplyRows + wave * 32;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = base + c_row(i, h);
    if (r >= n) continue;
    const bf16* Kr = reinterpret_cast<const bf16*>(a.K) + (size_t)r * D;
    float* out = a.dK + (size_t)r * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const int d = mb * 32 + l32;
      out[d] = FEAT ? c1[mb][i] : dphi((float)Kr[d]) * c1[mb][i];
    }
  }
  }
  if (MODE == 3) {
  f32x16 c2[KP / 32];
#pragma unroll
  for (int nb = 0; nb < KP / 32; ++nb) {
    c2[nb] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) c2[nb] = mma(rT.read(LT, nb, cc), xf[cc], c2[nb]);
  }
  if (row_ok) {
    float* out = a.dV + (size_t)row * a.k;
#pragma unroll
    for (int nb = 0; nb < KP / 32; ++nb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = nb * 32 + 8 * g + 4 * h;
        if ((a.k & 3) == 0 && c + 4 <= a.k) {
          *reinterpret_cast<f32x4*>(out + c) = f32x4{c2[nb][4 * g], c2[nb][4 * g + 1], c2[nb][4 * g + 2], c2[nb][4 * g + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < a.k) out[c + e] = c2[nb][4 * g + e];
        }
      }
    }
  }
  }
  }
}

// Forward rows (mode 0).
template <int D, int KP, int FEAT>
__global__ __launch_bounds__(256) void lin_apply(LinArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[ApplyCfg<D, KP, 0, FEAT>::LDS];
  apply_body<D, KP, 0, FEAT>(a, blockIdx.x, lds);
}

// Backward rows in one launch (all three read only the reduced matrices and
// inputs): workgroups [0, g1) the dQ rows (mode 1), [g1, g1 + g2) the dK rows
// (mode 2), the rest the dV rows (mode 3).
template <int D, int KP, int FEAT>
__global__ __launch_bounds__(256) void lin_apply_bwd(LinArgs a, int g1, int g2) {
  constexpr int L1 = ApplyCfg<D, KP, 1, FEAT>::LDS, L2 = ApplyCfg<D, KP, 2, FEAT>::LDS,
                L3 = ApplyCfg<D, KP, 3, FEAT>::LDS;
  constexpr int L12 = L1 > L2 ? L1 : L2;
  __shared__ __attribute__((aligned(16))) char lds[L12 > L3 ? L12 : L3];
  const int b = blockIdx.x;
  if (b < g1) apply_body<D, KP, 1, FEAT>(a, b, lds);
  else if (b < g1 + g2) apply_body<D, KP, 2, FEAT>(a, b - g1, lds);
  else apply_body<D, KP, 3, FEAT>(a, b - g1 - g2, lds);
}

}  // namespace lin

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define SSC_LIN_INSTANCES(X) \
  X(128, 224)                \
  X(128, 256)                \
  X(128, 128)                \
  X(128, 64)                 \
  X(128, 32)                 \
  X(64, 224)                 \
  X(64, 256)                 \
  X(64, 128)                 \
  X(64, 64)                  \
  X(64, 32)

hipError_t launch_lin_gram(int D, int KP, bool ident, const LinArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                              \
  if (D == DD && KP == KK) {                                                                       \
    if (ident) hipLaunchKernelGGL((lin::lin_gram<DD, KK, 1>), dim3(grid), dim3(lin::kGramWaves * 64), 0, st, a); \
    else hipLaunchKernelGGL((lin::lin_gram<DD, KK, 0>), dim3(grid), dim3(lin::kGramWaves * 64), 0, st, a);       \
    return hipGetLastError();                                                                      \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_lin_gram_bwd(int D, int KP, bool ident, const LinArgs& a, int gM, int gN, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                      \
  if (D == DD && KP == KK) {                                                                               \
    if (ident) hipLaunchKernelGGL((lin::lin_gram_bwd<DD, KK, 1>), dim3(gM + gN), dim3(lin::kGramWaves * 64), 0, st, a, gM); \
    else hipLaunchKernelGGL((lin::lin_gram_bwd<DD, KK, 0>), dim3(gM + gN), dim3(lin::kGramWaves * 64), 0, st, a, gM);       \
    return hipGetLastError();                                                                              \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

static lin::RedJob red_job(const float* part, int nparts, void* M, void* MT, void* Mlo, void* MTlo) {
  return lin::RedJob{part, nparts, reinterpret_cast<bf16*>(M), reinterpret_cast<bf16*>(MT),
                     reinterpret_cast<bf16*>(Mlo), reinterpret_cast<bf16*>(MTlo)};
}

hipError_t launch_lin_reduce(int D, int KP, const float* part, int nparts, void* M, void* MT, void* Mlo, void* MTlo,
                             hipStream_t st) {
  const lin::RedJob j = red_job(part, nparts, M, MT, Mlo, MTlo);
#define SSC_L(DD, KK)                                                                                    \
  if (D == DD && KP == KK) {                                                                             \
    hipLaunchKernelGGL((lin::lin_reduce<DD, KK>), dim3((DD * KK + 31) / 32), dim3(256), 0, st, j);       \
    return hipGetLastError();                                                                            \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_lin_reduce2(int D, int KP, const float* part0, int nparts0, void* M0, void* MT0, void* Mlo0,
                              void* MTlo0, const float* part1, int nparts1, void* M1, void* MT1, void* Mlo1,
                              void* MTlo1, hipStream_t st) {
  const lin::RedJob j0 = red_job(part0, nparts0, M0, MT0, Mlo0, MTlo0);
  const lin::RedJob j1 = red_job(part1, nparts1, M1, MT1, Mlo1, MTlo1);
#define SSC_L(DD, KK)                                                                                     \
  if (D == DD && KP == KK) {                                                                              \
    hipLaunchKernelGGL((lin::lin_reduce2<DD, KK>), dim3(2 * ((DD * KK + 31) / 32)), dim3(256), 0, st, j0, j1); \
    return hipGetLastError();                                                                             \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_lin_apply(int D, int KP, bool ident, const LinArgs& a, hipStream_t st) {
  const int grid = (a.n_N + lin::kApplyRows - 1) / lin::kApplyRows;
#define SSC_L(DD, KK)                                                                         \
  if (D == DD && KP == KK) {                                                                  \
    if (ident) hipLaunchKernelGGL((lin::lin_apply<DD, KK, 1>), dim3(grid), dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((lin::lin_apply<DD, KK, 0>), dim3(grid), dim3(256), 0, st, a);       \
    return hipGetLastError();                                                                 \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_lin_apply_bwd(int D, int KP, bool ident, const LinArgs& a, hipStream_t st) {
  const int g1 = (a.n_N + lin::kApplyRows - 1) / lin::kApplyRows;
  const int g2 = (a.n_M + lin::kApplyRows - 1) / lin::kApplyRows;
#define SSC_L(DD, KK)                                                                                             \
  if (D == DD && KP == KK) {                                                                                      \
    if (ident) hipLaunchKernelGGL((lin::lin_apply_bwd<DD, KK, 1>), dim3(g1 + 2 * g2), dim3(256), 0, st, a, g1, g2); \
    else hipLaunchKernelGGL((lin::lin_apply_bwd<DD, KK, 0>), dim3(g1 + 2 * g2), dim3(256), 0, st, a, g1, g2);       \
    return hipGetLastError();                                                                                     \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
