// Functional-map solve after the coupling on gfx950.  The coupled
// functional-map pipelines consume only the product Pi_NM Phi_M (project
// page "Spatial-Spectral Coupling as Attention", section "How it works"); the
// least-squares map between the two spectral bases is
//
//     C = argmin_C || Phi_N C - O ||_F = (Phi_N^T Phi_N)^{-1} Phi_N^T O,
//
// with O = Pi_NM Phi_M, and its backward for an upstream gradient dC is
// dO = Phi_N (Phi_N^T Phi_N)^{-1} dC (the basis is held fixed).
//
//   fm_gram   -- partial sums of G = Phi^T Phi (lower 32-blocks only) and
//                R = Phi^T O with bf16 MFMAs, one workgroup per (row block,
//                32-column block); O enters as a bf16 high part plus the
//                bf16 rounding of the remainder (together O to about 2^-17),
//                both products accumulated in one fp32 accumulator;
//   fm_reduce -- fixed-order sums of the partials (deterministic);
//   fm_chol   -- Cholesky factor of G in one workgroup, the matrix held in
//                registers (16 x 16 cyclic ownership), one barrier per
//                column; L is written packed by rows and by columns;
//   fm_solve  -- one wave per right-hand side column: right-looking forward
//                and backward substitution, the solved entry broadcast with
//                readlane, the L columns / rows of four steps read one
//                group ahead from LDS
//                (C = G^-1 R, or X = G^-1 dC);
//   fm_apply  -- backward rows dO = Phi X (bf16 MFMA, X in LDS).
// G must be positive definite (Phi_N of full column rank); otherwise the
// factor has a non-positive pivot and C / dO come out as NaN.
#include "tile_bf16.hpp"

namespace ssc {
namespace fm {

using tb::Geo;
using tb::put_pair;
using tb::TrReader;

constexpr int kTileRows = 64;

__device__ __forceinline__ int tri(int i) { return i * (i + 1) / 2; }
// Start of column c in the column-packed lower triangle of a k x k matrix.
__device__ __forceinline__ int colstart(int c, int k) { return c * k - c * (c - 1) / 2; }

// Eight consecutive bf16 elements c0 .. c0+7 of a row of width w as floats
// (past w: 0), element by element (rows that are not 16-byte aligned).
__device__ __forceinline__ void rowb8_slow(const bf16* row, int c0, int w, float* out) {
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = c0 + e < w ? (float)row[c0 + e] : 0.f;
}

// Four consecutive elements c0 .. c0+3 (past w: 0); one 8-byte load when
// the row allows it.
__device__ __forceinline__ void rowb4(const bf16* row, int c0, int w, bool vec, float* out) {
  if (vec && c0 + 4 <= w) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(row + c0);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (float)v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = c0 + e < w ? (float)row[c0 + e] : 0.f;
  }
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) put_pair(r, m, v[2 * m], v[2 * m + 1]);
  return r;
}

// ---------------------------------------------------------------------------
// Gram partials.  Workgroup (block b, column block nb) sums over its rows
//   G[:, nb] for the row blocks mb >= nb:  Phi[:, mb]^T Phi[:, nb]
//   R[:, nb] for every row block mb:      Phi[:, mb]^T (O_hi + O_lo)[:, nb]
// into part[b][0] and part[b][1] ([KP x KP] each; only those blocks are
// written).  The next 64-row tile is loaded into registers while the
// current one is multiplied.
// ---------------------------------------------------------------------------
template <int KP, bool FWD>
struct GramTile {
  static constexpr int CH = KP / 32;  // 16-byte Phi chunks per thread per tile
  bf16x8 p[CH];
  f32x4 o[2];                         // O: 64 rows x 32 columns, 2 float4 per thread

  __device__ __forceinline__ void load(const FmArgs& a, int r0, int r_end, int nb, int tid, bool vec, bool vec4) {
    const bf16* Phi = reinterpret_cast<const bf16*>(a.Phi);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int ch = tid + 256 * j, r = ch / (KP / 8), c8 = ch - r * (KP / 8), gr = r0 + r;
      const bool ok = gr < r_end && c8 * 8 < a.k;
      if (vec) {
        p[j] = ok ? *reinterpret_cast<const bf16x8*>(Phi + (size_t)gr * a.k + c8 * 8) : bf16x8{};
      } else {
        float v[8];
        if (ok) rowb8_slow(Phi + (size_t)gr * a.k, c8 * 8, a.k, v);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
        p[j] = pack8(v);
      }
    }
    if (FWD) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ch = tid + 256 * j, r = ch >> 3, col = nb * 32 + (ch & 7) * 4, gr = r0 + r;
        const float* orow = a.O + (size_t)gr * a.k;
        if (vec4) {
          o[j] = gr < r_end && col < a.k ? *reinterpret_cast<const f32x4*>(orow + col) : f32x4{};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[j][e] = gr < r_end && col + e < a.k ? orow[col + e] : 0.f;
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* As, char* Bh, char* Bl, int tid) const {
    constexpr int P = Geo<KP>::PITCH, PB = Geo<32>::PITCH;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int ch = tid + 256 * j, r = ch / (KP / 8), c8 = ch - r * (KP / 8);
      *reinterpret_cast<bf16x8*>(As + r * P + c8 * 16) = p[j];
    }
    if (FWD) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int ch = tid + 256 * j, r = ch >> 3, c4 = ch & 7;
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = (bf16)o[j][e];
          lo[e] = (bf16)(o[j][e] - (float)hi[e]);
        }
        *reinterpret_cast<bf16x4*>(Bh + r * PB + c4 * 8) = hi;
        *reinterpret_cast<bf16x4*>(Bl + r * PB + c4 * 8) = lo;
      }
    }
  }
};

template <int KP, bool FWD>
__global__ __launch_bounds__(256) void fm_gram(FmArgs a) {
  constexpr int P = Geo<KP>::PITCH, PB = Geo<32>::PITCH;
  constexpr int NNB = KP / 32;
  constexpr int NT = FWD ? (2 * NNB + 3) / 4 : (NNB + 3) / 4;  // output blocks per wave
  constexpr int NPROD = FWD ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char As[kTileRows * P];
  __shared__ __attribute__((aligned(16))) char Bh[FWD ? kTileRows * PB : 16];
  __shared__ __attribute__((aligned(16))) char Bl[FWD ? kTileRows * PB : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  TrReader<KP> tr;
  tr.init(tr_r, tr_c);
  TrReader<32> trb;
  trb.init(tr_r, tr_c);

  const int nb = blockIdx.y, nG = NNB - nb;
  const int r_begin = blockIdx.x * a.rows, r_end = min(a.n, r_begin + a.rows);
  const bool vec = (a.k & 7) == 0, vec4 = (a.k & 3) == 0;

  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};

  GramTile<KP, FWD> cur;
  cur.load(a, r_begin, r_end, nb, tid, vec, vec4);
  const int nt = (r_end - r_begin + kTileRows - 1) / kTileRows;
  for (int it = 0; it < nt; ++it) {
    cur.store(As, Bh, Bl, tid);
    __syncthreads();
    if (it + 1 < nt) cur.load(a, r_begin + (it + 1) * kTileRows, r_end, nb, tid, vec, vec4);
#pragma unroll
    for (int kc = 0; kc < kTileRows / 16; ++kc) {
      const bf16x8 bphi = tr.frag(As, nb, kc);
      bf16x8 bh{}, bl{};
      if (FWD) {
        bh = trb.frag(Bh, 0, kc);
        bl = trb.frag(Bl, 0, kc);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int bi = wave + 4 * t;
        if (bi < nG) {
          acc[t] = mma(tr.frag(As, nb + bi, kc), bphi, acc[t]);
        } else if (FWD && bi < nG + NNB) {
          const bf16x8 am = tr.frag(As, bi - nG, kc);
          acc[t] = mma(am, bh, acc[t]);
          acc[t] = mma(am, bl, acc[t]);
        }
      }
    }
    __syncthreads();
  }
  float* pG = a.part + (size_t)blockIdx.x * NPROD * KP * KP;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int bi = wave + 4 * t;
    float* dst = nullptr;
    int mb = 0;
    if (bi < nG) {
      dst = pG;
      mb = nb + bi;
    } else if (FWD && bi < nG + NNB) {
      dst = pG + (size_t)KP * KP;
      mb = bi - nG;
    }
    if (dst != nullptr) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[(size_t)(mb * 32 + c_row(i, h)) * KP + nb * 32 + l32] = acc[t][i];
    }
  }
}

// Fixed-order sums over the row blocks: G (lower 32-blocks; the others are
// set to 0 and never read) and, with two products, R.
__global__ __launch_bounds__(256) void fm_reduce(FmArgs a, int nblk, int nprod, int KP) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= KP * KP) return;
  const size_t stride = (size_t)KP * KP;
  const int r = idx / KP, c = idx - r * KP;
  for (int w = 0; w < nprod; ++w) {
    if (w == 0 && (r >> 5) < (c >> 5)) {
      a.G[idx] = 0.f;
      continue;
    }
    const float* src = a.part + w * stride + idx;
    float s = 0.f;
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + (size_t)(b + u) * nprod * stride);
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < nblk; ++b) s += src[(size_t)b * nprod * stride];
    (w == 0 ? a.G : a.R)[idx] = s;
  }
}

// ---------------------------------------------------------------------------
// Cholesky factor G = L L^T, one workgroup of 256 threads.  Thread
// (ti, tc) = (tid / 16, tid % 16) holds the entries (ti + 16x, tc + 16y),
// y <= x, in registers.  Step j: the owners of column j publish it to LDS
// (double buffered), every thread forms l_ij = a_ij / sqrt(a_jj) for its rows
// and columns and subtracts l_i l_c from its trailing entries.  Padded rows
// (i >= k) start as zero rows and stay so.
// ---------------------------------------------------------------------------
template <int KP>
__global__ __launch_bounds__(256) void fm_chol(FmArgs a) {
  constexpr int NR = KP / 16;
  // column j, entries i > j (0 elsewhere), and its pivot; double buffered
  __shared__ float col[2][KP];
  __shared__ float piv[2];
  const int tid = threadIdx.x, ti = tid >> 4, tc = tid & 15, k = a.k;
  float A[NR * (NR + 1) / 2];
#pragma unroll
  for (int x = 0; x < NR; ++x)
#pragma unroll
    for (int y = 0; y <= x; ++y) {
      const int i = ti + 16 * x, c = tc + 16 * y;
      A[x * (x + 1) / 2 + y] = i < k && c < k ? a.G[(size_t)i * KP + c] : 0.f;
    }
#pragma unroll
  for (int JB = 0; JB < NR; ++JB) {
    const int jend = min(16, k - 16 * JB);
    for (int jt = 0; jt < jend; ++jt) {
      const int j = 16 * JB + jt;
      float* cb = col[j & 1];
      if (tc == jt) {
#pragma unroll
        for (int x = JB; x < NR; ++x) {
          const int i = ti + 16 * x;
          const float v = A[x * (x + 1) / 2 + JB];
          cb[i] = i > j ? v : 0.f;
          if (i == j) piv[j & 1] = v;
        }
      }
      __syncthreads();
      const float p = piv[j & 1];
      const float rd = __builtin_amdgcn_rsqf(p), d = p * rd;
      float li[NR], lc[NR];
#pragma unroll
      for (int x = JB; x < NR; ++x) {
        li[x] = cb[ti + 16 * x] * rd;
        lc[x] = cb[tc + 16 * x] * rd;
      }
#pragma unroll
      for (int x = JB; x < NR; ++x)
#pragma unroll
        for (int y = JB; y <= x; ++y) A[x * (x + 1) / 2 + y] = fmaf(-li[x], lc[y], A[x * (x + 1) / 2 + y]);
      if (tc == jt) {
#pragma unroll
        for (int x = JB; x < NR; ++x) {
          const int i = ti + 16 * x;
          float& e = A[x * (x + 1) / 2 + JB];
          e = i > j ? li[x] : (i == j ? d : e);
        }
      }
    }
  }
#pragma unroll
  for (int x = 0; x < NR; ++x)
#pragma unroll
    for (int y = 0; y <= x; ++y) {
      const int i = ti + 16 * x, c = tc + 16 * y;
      if (i < k && c <= i) {
        const float v = A[x * (x + 1) / 2 + y];
        a.Lrow[tri(i) + c] = v;
        a.Lcol[colstart(c, k) + (i - c)] = v;
        if (i == c) a.rdiag[i] = 1.f / v;
      }
    }
}

// ---------------------------------------------------------------------------
// x = L^-T L^-1 b for right-hand side column c = blockIdx.x (one wave).
// Lane l holds x_p for p = l + 64 s.  Forward step i: x_i /= l_ii, broadcast
// with readlane, x_p -= l_pi x_i for p > i (column i of L from LDS, packed by
// columns); backward step i (descending): x_i /= l_ii, x_p -= l_ip x_i for
// p < i (row i, packed by rows).  The L values of step i + 1 are read during
// step i.  MODE 0: b = column c of R (KP x KP), x -> column c of C (k x k
// fp32, row-major).  MODE 1: b = column c of dC (k x k), x -> column c of X
// (KP x KP bf16, zero padded).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bcast(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// One packing of L (at most tri(256) floats) in whole 1 KB rounds, plus the
// 256 floats that masked reads past the end may touch.
constexpr int kSolveLds = 33280;
static_assert(kSolveLds * 4 >= ((kFmMaxK * (kFmMaxK + 1) / 2 * 4 + 1023) / 1024) * 1024 &&
                  kSolveLds >= kFmMaxK * (kFmMaxK + 1) / 2 + 256,
              "solve LDS size");

// tri(k) floats of a packed factor into T with direct loads (16 bytes per
// lane, 1 KB per instruction; past the end: zeros).
__device__ __forceinline__ void stage_factor(float* T, const float* src, int nt, int lane) {
  const tb::i32x4 rs = tb::make_rsrc(src, (unsigned)nt * 4u);
  const int rounds = (nt * 4 + 1023) / 1024;
  for (int r = 0; r < rounds; ++r)
    tb::ssc_raw_buffer_load_lds(rs, (tb::lds_void_t*)(T + r * 256), 16, r * 1024 + lane * 16, 0, 0, 0);
  tb::wait_loads();
}

template <int KP, int MODE>
__global__ __launch_bounds__(64) void fm_solve(FmArgs a) {
  constexpr int NS = (KP + 63) / 64;
  __shared__ __attribute__((aligned(16))) float T[kSolveLds];
  __shared__ float rdl[kFmMaxK];
  const int lane = threadIdx.x, c = blockIdx.x, k = a.k;
  if (c >= k) {  // MODE 1: zero padding columns of X
    if (MODE == 1)
      for (int i = lane; i < KP; i += 64) a.X[(size_t)i * KP + c] = (bf16)0.f;
    return;
  }
  const int nt = tri(k);
  for (int i = lane; i < k; i += 64) rdl[i] = a.rdiag[i];
  float x[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int p = lane + 64 * s;
    x[s] = p < k ? (MODE == 0 ? a.R[(size_t)p * KP + c] : a.dC[(size_t)p * k + c]) : 0.f;
  }
  stage_factor(T, a.Lcol, nt, lane);
  __syncthreads();

  // The L values and 1 / l_ii of four steps are read one group ahead.
  float cur[4][NS], nxt[4][NS], rc[4], rn[4];
  // forward substitution, L by columns: l_pi at colstart(i) + p - i
  auto fetch_f = [&](int i0, float (&L)[4][NS], float (&r)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ic = min(i0 + u, k - 1), base = colstart(ic, k) - ic;
#pragma unroll
      for (int s = 0; s < NS; ++s) L[u][s] = T[base + lane + 64 * s];
      r[u] = rdl[ic];
    }
  };
#pragma unroll
  for (int S = 0; S < NS; ++S) {
    const int ibeg = 64 * S, iend = min(64 * S + 64, k);
    if (ibeg < iend) fetch_f(ibeg, cur, rc);
    for (int i0 = ibeg; i0 < iend; i0 += 4) {
      fetch_f(i0 + 4, nxt, rn);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u;
        if (i < iend) {
          const float xi = bcast(x[S], i - ibeg) * rc[u];
          x[S] = lane == i - ibeg ? xi : x[S];
          // slot S: only rows p > i change; slots above S lie wholly
          // below row i (rows past k take junk and are never read)
          x[S] = lane > i - ibeg ? fmaf(-cur[u][S], xi, x[S]) : x[S];
#pragma unroll
          for (int s = S + 1; s < NS; ++s) x[s] = fmaf(-cur[u][s], xi, x[s]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        rc[u] = rn[u];
#pragma unroll
        for (int s = 0; s < NS; ++s) cur[u][s] = nxt[u][s];
      }
    }
  }
  __syncthreads();
  stage_factor(T, a.Lrow, nt, lane);
  __syncthreads();

  // backward substitution, L by rows: l_ip at tri(i) + p
  auto fetch_b = [&](int i0, float (&L)[4][NS], float (&r)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ic = max(i0 - u, 0), base = tri(ic);
#pragma unroll
      for (int s = 0; s < NS; ++s) L[u][s] = T[base + lane + 64 * s];
      r[u] = rdl[ic];
    }
  };
#pragma unroll
  for (int S = NS - 1; S >= 0; --S) {
    const int ibeg = 64 * S, ihi = min(64 * S + 63, k - 1);
    if (ibeg <= ihi) fetch_b(ihi, cur, rc);
    for (int i0 = ihi; i0 >= ibeg; i0 -= 4) {
      fetch_b(i0 - 4, nxt, rn);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 - u;
        if (i >= ibeg) {
          const float xi = bcast(x[S], i - ibeg) * rc[u];
          x[S] = lane == i - ibeg ? xi : x[S];
          // slot S: only rows p < i change; slots below S lie wholly above
          x[S] = lane < i - ibeg ? fmaf(-cur[u][S], xi, x[S]) : x[S];
#pragma unroll
          for (int s = 0; s < S; ++s) x[s] = fmaf(-cur[u][s], xi, x[s]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        rc[u] = rn[u];
#pragma unroll
        for (int s = 0; s < NS; ++s) cur[u][s] = nxt[u][s];
      }
    }
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int p = lane + 64 * s;
    if (MODE == 0) {
      if (p < k) a.C[(size_t)p * k + c] = x[s];
    } else {
      if (p < KP) a.X[(size_t)p * KP + c] = (bf16)(p < k ? x[s] : 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// Backward rows: dO = Phi X.  A wave owns 32 rows (their Phi fragments in
// registers, the MFMA column operand); X (KP x KP bf16) sits in LDS and
// enters as transposed reads, so the accumulators hold dO^T for the wave's
// rows (rows of dO^T = columns of dO).
// ---------------------------------------------------------------------------
template <int KP>
__global__ __launch_bounds__(256) void fm_apply(FmArgs a) {
  constexpr int P = Geo<KP>::PITCH;
  __shared__ __attribute__((aligned(16))) char Xs[KP * P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  TrReader<KP> tr;
  tr.init(tr_r, tr_c);
  for (int ch = tid; ch < KP * (KP / 8); ch += 256) {
    const int r = ch / (KP / 8), c8 = ch - r * (KP / 8);
    *reinterpret_cast<bf16x8*>(Xs + r * P + c8 * 16) = *reinterpret_cast<const bf16x8*>(a.X + (size_t)r * KP + c8 * 8);
  }
  const int row = blockIdx.x * 128 + wave * 32 + l32;
  const bool row_ok = row < a.n;
  const bf16* Phi = reinterpret_cast<const bf16*>(a.Phi) + (size_t)row * a.k;
  const bool vec = (a.k & 3) == 0;
  // The transposed X reads carry the k rows kc*16 + {4h..4h+3, 8+4h..8+4h+3}
  // in a lane's eight elements; the Phi fragment takes the same columns.
  bf16x8 pf[KP / 16];
#pragma unroll
  for (int kc = 0; kc < KP / 16; ++kc) {
    float v[8];
    if (row_ok) {
      rowb4(Phi, kc * 16 + 4 * h, a.k, vec, v);
      rowb4(Phi, kc * 16 + 8 + 4 * h, a.k, vec, v + 4);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    pf[kc] = pack8(v);
  }
  __syncthreads();
  f32x16 acc[KP / 32];
#pragma unroll
  for (int cb = 0; cb < KP / 32; ++cb) acc[cb] = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KP / 16; ++kc)
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) acc[cb] = mma(tr.frag(Xs, cb, kc), pf[kc], acc[cb]);
  if (!row_ok) return;
  float* out = a.dO + (size_t)row * a.k;
#pragma unroll
  for (int cb = 0; cb < KP / 32; ++cb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // accumulator elements 4q .. 4q+3 are the columns c0 .. c0+3
      const int c0 = cb * 32 + 8 * q + 4 * h;
      if (vec && c0 + 4 <= a.k) {
        *reinterpret_cast<f32x4*>(out + c0) =
            f32x4{acc[cb][4 * q], acc[cb][4 * q + 1], acc[cb][4 * q + 2], acc[cb][4 * q + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c0 + e < a.k) out[c0 + e] = acc[cb][4 * q + e];
      }
    }
}

}  // namespace fm

#define SSC_FM_INSTANCES(X) X(224) X(256) X(128) X(64) X(32)

void fm_blocks(int n, int KP, int* rows, int* nblk) {
  // about 512 Gram workgroups: (row blocks) x (KP / 32 column blocks)
  const int want = (512 + KP / 32 - 1) / (KP / 32);
  const int r = (n + want - 1) / want;
  *rows = ((r + fm::kTileRows - 1) / fm::kTileRows) * fm::kTileRows;
  *nblk = (n + *rows - 1) / *rows;
}

hipError_t launch_fm_gram(int KP, bool fwd, const FmArgs& a, int nblk, hipStream_t st) {
#define SSC_L(KK)                                                                                 \
  if (KP == KK) {                                                                                 \
    if (fwd) hipLaunchKernelGGL((fm::fm_gram<KK, true>), dim3(nblk, KK / 32), dim3(256), 0, st, a); \
    else hipLaunchKernelGGL((fm::fm_gram<KK, false>), dim3(nblk, KK / 32), dim3(256), 0, st, a);   \
    return hipGetLastError();                                                                     \
  }
  SSC_FM_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_fm_reduce(int KP, bool fwd, const FmArgs& a, int nblk, hipStream_t st) {
  hipLaunchKernelGGL(fm::fm_reduce, dim3((KP * KP + 255) / 256), dim3(256), 0, st, a, nblk, fwd ? 2 : 1, KP);
  return hipGetLastError();
}

hipError_t launch_fm_chol(int KP, const FmArgs& a, hipStream_t st) {
#define SSC_L(KK)                                                                \
  if (KP == KK) {                                                                \
    hipLaunchKernelGGL((fm::fm_chol<KK>), dim3(1), dim3(256), 0, st, a);        \
    return hipGetLastError();                                                    \
  }
  SSC_FM_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_fm_solve(int KP, int mode, const FmArgs& a, hipStream_t st) {
#define SSC_L(KK)                                                                       \
  if (KP == KK) {                                                                       \
    if (mode == 0) hipLaunchKernelGGL((fm::fm_solve<KK, 0>), dim3(a.k), dim3(64), 0, st, a); \
    else hipLaunchKernelGGL((fm::fm_solve<KK, 1>), dim3(KK), dim3(64), 0, st, a);       \
    return hipGetLastError();                                                           \
  }
  SSC_FM_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_fm_apply(int KP, const FmArgs& a, hipStream_t st) {
#define SSC_L(KK)                                                                            \
  if (KP == KK) {                                                                            \
    hipLaunchKernelGGL((fm::fm_apply<KK>), dim3((a.n + 127) / 128), dim3(256), 0, st, a);     \
    return hipGetLastError();                                                                \
  }
  SSC_FM_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
