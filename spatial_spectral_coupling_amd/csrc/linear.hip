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
// order (deterministic).
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
// Rows past the end contribute 0.
// ---------------------------------------------------------------------------
template <int D, int KP, int MODE, int FEAT>
__global__ __launch_bounds__(256) void lin_gram(LinArgs a) {
  constexpr int AP = Geo<D>::PITCH, BP = Geo<KP>::PITCH;
  // identity features, backward: G_ext as a bf16 high + low pair
  constexpr bool BLO = FEAT == 1 && MODE == 1;
  // rows per LDS tile (halved where the low part would not fit)
  constexpr int TR = BLO && (kGramTile * (AP + 2 * BP) > 160 * 1024) ? kGramTile / 2 : kGramTile;
  __shared__ __attribute__((aligned(16))) char As[TR * AP];
  __shared__ __attribute__((aligned(16))) char Bs[TR * BP];
  __shared__ __attribute__((aligned(16))) char Bl[BLO ? TR * BP : 16];
  constexpr int NMB = D / 32, NNB = KP / 32, NB = NMB * NNB, NBW = (NB + 3) / 4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  TrReader<D> ta;
  ta.init(tr_r, tr_c);
  TrReader<KP> tbr;
  tbr.init(tr_r, tr_c);

  const int n = MODE == 0 ? a.n_M : a.n_N;
  const int r_begin = blockIdx.x * kLinGramRows;
  const int r_end = min(n, r_begin + kLinGramRows);
  const bf16* X = reinterpret_cast<const bf16*>(MODE == 0 ? a.K : a.Q);
  const bf16* Y = reinterpret_cast<const bf16*>(MODE == 0 ? a.V : a.dO);
  const bool vec = (a.k & 7) == 0;

  f32x16 acc[NBW];
#pragma unroll
  for (int t = 0; t < NBW; ++t) acc[t] = f32x16{};

  for (int r0 = r_begin; r0 < r_end; r0 += TR) {
    // every load of the tile first (in flight together), then the feature
    // map / scaling and the LDS stores
    constexpr int NXA = TR * (D / 8) / 256, NYB = TR * (KP / 8) / 256;
    static_assert(NXA * 256 == TR * (D / 8) && NYB * 256 == TR * (KP / 8), "gram tile split");
    bf16x8 xa[NXA], yb[NYB];
    float rdv[MODE == 1 ? NYB : 1], sv[MODE == 1 ? NYB : 1];
#pragma unroll
    for (int j = 0; j < NXA; ++j) {
      const int ch = tid + 256 * j, r = ch / (D / 8), c8 = ch - r * (D / 8), gr = r0 + r;
      xa[j] = gr < r_end ? ld8(X + (size_t)gr * D + c8 * 8) : bf16x8{};
    }
#pragma unroll
    for (int j = 0; j < NYB; ++j) {
      const int ch = tid + 256 * j, r = ch / (KP / 8), c8 = ch - r * (KP / 8), gr = r0 + r;
      const bool in = gr < r_end && c8 * 8 < a.k;
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
        rdv[MODE == 1 ? j : 0] = gr < r_end ? a.rden[gr] : 0.f;
        sv[MODE == 1 ? j : 0] = gr < r_end && c8 == KP / 8 - 1 ? a.s[gr] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < NXA; ++j) {
      const int ch = tid + 256 * j, r = ch / (D / 8), c8 = ch - r * (D / 8);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = r0 + r < r_end ? feat<FEAT>((float)xa[j][e]) : 0.f;
      *reinterpret_cast<bf16x8*>(As + r * AP + c8 * 16) = pack8(v);
    }
#pragma unroll
    for (int j = 0; j < NYB; ++j) {
      const int ch = tid + 256 * j, r = ch / (KP / 8), c8 = ch - r * (KP / 8), gr = r0 + r;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)yb[j][e];
      if (MODE == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= rdv[MODE == 1 ? j : 0];
      }
      if (gr < r_end && c8 == KP / 8 - 1) v[7] = MODE == 0 ? 1.f : -sv[MODE == 1 ? j : 0];
      const bf16x8 hv = pack8(v);
      *reinterpret_cast<bf16x8*>(Bs + r * BP + c8 * 16) = hv;
      if (BLO) {
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = v[e] - (float)hv[e];
        *reinterpret_cast<bf16x8*>(Bl + r * BP + c8 * 16) = pack8(lo);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < TR / 16; ++kc) {
#pragma unroll
      for (int t = 0; t < NBW; ++t) {
        const int bi = wave + 4 * t;
        if (NB % 4 == 0 || bi < NB) {
          const bf16x8 af = ta.frag(As, bi / NNB, kc);
          acc[t] = mma(af, tbr.frag(Bs, bi % NNB, kc), acc[t]);
          if (BLO) acc[t] = mma(af, tbr.frag(Bl, bi % NNB, kc), acc[t]);
        }
      }
    }
    __syncthreads();
  }
  float* part = a.part + (size_t)blockIdx.x * D * KP;
#pragma unroll
  for (int t = 0; t < NBW; ++t) {
    const int bi = wave + 4 * t;
    if (NB % 4 == 0 || bi < NB) {
      const int mb = bi / NNB, nb = bi % NNB;
#pragma unroll
      for (int i = 0; i < 16; ++i) part[(size_t)(mb * 32 + c_row(i, h)) * KP + nb * 32 + l32] = acc[t][i];
    }
  }
}

// Fixed-order sum of the Gram partials, written as bf16 in both layouts:
// M [D x KP] and MT [KP x D]; with Mlo / MTlo also the bf16 rounding of the
// remainder (the pair carries the sum to about 2^-17).
template <int D, int KP>
__global__ __launch_bounds__(256) void lin_reduce(const float* part, int nparts, bf16* M, bf16* MT, bf16* Mlo,
                                                  bf16* MTlo) {
  // eight threads per output element: thread u sums the partials u, u + 8,
  // ... (one of eight independent partial sums), then the eight sums are
  // combined in a fixed order (deterministic)
  __shared__ float s8[8][32];
  const int u = threadIdx.x >> 5, e = threadIdx.x & 31;
  const int idx = blockIdx.x * 32 + e;
  float acc = 0.f;
  if (idx < D * KP)
    for (int b = u; b < nparts; b += 8) acc += part[(size_t)b * D * KP + idx];
  s8[u][e] = acc;
  __syncthreads();
  if (u != 0 || idx >= D * KP) return;
  const float s = ((s8[0][e] + s8[1][e]) + (s8[2][e] + s8[3][e])) + ((s8[4][e] + s8[5][e]) + (s8[6][e] + s8[7][e]));
  const int d = idx / KP, c = idx - d * KP;
  const bf16 v = (bf16)s;
  M[idx] = v;
  MT[(size_t)c * D + d] = v;
  if (Mlo != nullptr) {
    const bf16 lo = (bf16)(s - (float)v);
    Mlo[idx] = lo;
    MTlo[(size_t)c * D + d] = lo;
  }
}

// Per target row of the backward: rden = 1 / den, s = (dO . O) / den
// (16 lanes per row, 16 rows per workgroup; the 16 partial dot products are
// added in a fixed butterfly order).
__global__ __launch_bounds__(256) void lin_rowprep(LinArgs a) {
  const int sub = threadIdx.x & 15;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool ok = row < a.n_N;
  const bf16* dO = reinterpret_cast<const bf16*>(a.dO) + (size_t)(ok ? row : 0) * a.k;
  const float* O = a.O + (size_t)(ok ? row : 0) * a.k;
  float acc = 0.f;
  if (ok) {
    if ((a.k & 3) == 0) {
      for (int c = 4 * sub; c < a.k; c += 64) {
        const bf16x4 g = *reinterpret_cast<const bf16x4*>(dO + c);
        const f32x4 o = *reinterpret_cast<const f32x4*>(O + c);
        acc += ((float)g[0] * o[0] + (float)g[1] * o[1]) + ((float)g[2] * o[2] + (float)g[3] * o[3]);
      }
    } else {
      for (int c = sub; c < a.k; c += 16) acc += (float)dO[c] * O[c];
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (ok && sub == 0) {
    const float rd = 1.f / a.den[row];
    a.rden[row] = rd;
    a.s[row] = acc * rd;
  }
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
// Scores are computed transposed (C[col][row]) so that a lane holds its own
// row and the operand fragments of that row come from its own registers.
// ---------------------------------------------------------------------------
template <int D, int KP, int MODE, int FEAT>
__global__ __launch_bounds__(256) void lin_apply(LinArgs a) {
  // which layouts this mode reads, and whether with a low part
  constexpr bool USE_T = MODE == 0 || MODE == 3;
  constexpr bool USE_M = MODE == 1 || MODE == 2;
  constexpr bool LO_T = FEAT && MODE == 0, LO_M = FEAT && USE_M;
  constexpr int SZ_T = USE_T ? KP * Geo<D>::PITCH : 0;  // [KP x D] layout
  constexpr int SZ_M = USE_M ? D * Geo<KP>::PITCH : 0;  // [D x KP] layout
  __shared__ __attribute__((aligned(16))) char lds[SZ_T * (LO_T ? 2 : 1) + SZ_M * (LO_M ? 2 : 1) + 16];
  char* LT = lds;
  char* LTlo = lds + SZ_T;
  char* LM = lds + SZ_T * (LO_T ? 2 : 1);
  char* LMlo = LM + SZ_M;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int n = MODE >= 2 ? a.n_M : a.n_N;
  const int row = blockIdx.x * kApplyRows + wave * 32 + l32;
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
    f32x16 acc[D / 32];
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      acc[mb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < KP / 16; ++cc) {
        const bf16x8 mh = rM.read(LM, mb, cc);
        acc[mb] = mma(mh, gf[cc], acc[mb]);
        if (LO_M) acc[mb] = mma(rM.read(LMlo, mb, cc), gf[cc], acc[mb]);
        if (FEAT) acc[mb] = mma(mh, gl[FEAT ? cc : 0], acc[mb]);
      }
    }
    if (row_ok) {
      const bf16* Qr = reinterpret_cast<const bf16*>(a.Q) + (size_t)row * D;
      float* out = a.dQ + (size_t)row * D;
#pragma unroll
      for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = mb * 32 + 8 * g + 4 * h;
          if (FEAT) {
            *reinterpret_cast<f32x4*>(out + d0) =
                f32x4{acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]};
          } else {
            const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(Qr + d0);
            *reinterpret_cast<f32x4*>(out + d0) =
                f32x4{dphi((float)q4[0]) * acc[mb][4 * g], dphi((float)q4[1]) * acc[mb][4 * g + 1],
                      dphi((float)q4[2]) * acc[mb][4 * g + 2], dphi((float)q4[3]) * acc[mb][4 * g + 3]};
          }
        }
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
  f32x16 c1[D / 32];
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb) {
    c1[mb] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < KP / 16; ++cc) {
      c1[mb] = mma(rM.read(LM, mb, cc), vf[cc], c1[mb]);
      if (LO_M) c1[mb] = mma(rM.read(LMlo, mb, cc), vf[cc], c1[mb]);
    }
  }
  if (row_ok) {
    const bf16* Kr = reinterpret_cast<const bf16*>(a.K) + (size_t)row * D;
    float* out = a.dK + (size_t)row * D;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = mb * 32 + 8 * g + 4 * h;
        if (FEAT) {
          *reinterpret_cast<f32x4*>(out + d0) = f32x4{c1[mb][4 * g], c1[mb][4 * g + 1], c1[mb][4 * g + 2], c1[mb][4 * g + 3]};
        } else {
          const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(Kr + d0);
          *reinterpret_cast<f32x4*>(out + d0) =
              f32x4{dphi((float)k4[0]) * c1[mb][4 * g], dphi((float)k4[1]) * c1[mb][4 * g + 1],
                    dphi((float)k4[2]) * c1[mb][4 * g + 2], dphi((float)k4[3]) * c1[mb][4 * g + 3]};
        }
      }
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

hipError_t launch_lin_gram(int D, int KP, int mode, bool ident, const LinArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                         \
  if (D == DD && KP == KK) {                                                                                  \
    if (ident) {                                                                                              \
      if (mode == 0) hipLaunchKernelGGL((lin::lin_gram<DD, KK, 0, 1>), dim3(grid), dim3(256), 0, st, a);      \
      else hipLaunchKernelGGL((lin::lin_gram<DD, KK, 1, 1>), dim3(grid), dim3(256), 0, st, a);                \
    } else {                                                                                                  \
      if (mode == 0) hipLaunchKernelGGL((lin::lin_gram<DD, KK, 0, 0>), dim3(grid), dim3(256), 0, st, a);      \
      else hipLaunchKernelGGL((lin::lin_gram<DD, KK, 1, 0>), dim3(grid), dim3(256), 0, st, a);                \
    }                                                                                                         \
    return hipGetLastError();                                                                                 \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_lin_reduce(int D, int KP, const float* part, int nparts, void* M, void* MT, void* Mlo, void* MTlo,
                             hipStream_t st) {
#define SSC_L(DD, KK)                                                                                    \
  if (D == DD && KP == KK) {                                                                             \
    hipLaunchKernelGGL((lin::lin_reduce<DD, KK>), dim3((DD * KK + 31) / 32), dim3(256), 0, st, part, nparts,   \
                       reinterpret_cast<bf16*>(M), reinterpret_cast<bf16*>(MT), reinterpret_cast<bf16*>(Mlo),  \
                       reinterpret_cast<bf16*>(MTlo));                                                   \
    return hipGetLastError();                                                                            \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_lin_rowprep(const LinArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(lin::lin_rowprep, dim3((a.n_N + 15) / 16), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, int KP, int FEAT>
void launch_lin_apply_t(int mode, const LinArgs& a, int grid, hipStream_t st) {
  if (mode == 0) hipLaunchKernelGGL((lin::lin_apply<D, KP, 0, FEAT>), dim3(grid), dim3(256), 0, st, a);
  else if (mode == 1) hipLaunchKernelGGL((lin::lin_apply<D, KP, 1, FEAT>), dim3(grid), dim3(256), 0, st, a);
  else if (mode == 2) hipLaunchKernelGGL((lin::lin_apply<D, KP, 2, FEAT>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((lin::lin_apply<D, KP, 3, FEAT>), dim3(grid), dim3(256), 0, st, a);
}

hipError_t launch_lin_apply(int D, int KP, int mode, bool ident, const LinArgs& a, hipStream_t st) {
  const int n = mode >= 2 ? a.n_M : a.n_N;
  const int grid = (n + lin::kApplyRows - 1) / lin::kApplyRows;
#define SSC_L(DD, KK)                                                                 \
  if (D == DD && KP == KK) {                                                          \
    if (ident) launch_lin_apply_t<DD, KK, 1>(mode, a, grid, st);                      \
    else launch_lin_apply_t<DD, KK, 0>(mode, a, grid, st);                            \
    return hipGetLastError();                                                         \
  }
  SSC_LIN_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
