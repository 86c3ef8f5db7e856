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
//   fm_gram   -- Gram partials over blocks of 2048 rows with bf16 MFMA:
//                G = Phi^T Phi and R = Phi^T O, O split into a bf16 high and
//                low part (their sum is O to about 2^-17), fp32 accumulation;
//   fm_reduce -- fixed-order sums of the partials (deterministic);
//   fm_chol   -- Cholesky factor L of G, one workgroup, G's lower triangle
//                in LDS (right-looking, one column per step);
//   fm_solve  -- one single-wave workgroup per right-hand side column:
//                x = L^-T L^-1 b with L in LDS (C = G^-1 R, or X = G^-1 dC);
//   fm_apply  -- backward rows dO = Phi X (bf16 MFMA, X in LDS).
// G must be positive definite (Phi_N of full column rank); otherwise the
// factor has a non-positive pivot and C / dO come out as NaN.
#include "tile_bf16.hpp"

namespace ssc {
namespace fm {

using tb::Geo;
using tb::put_pair;
using tb::static_for;
using tb::TrReader;

constexpr int kTileRows = 64;

__device__ __forceinline__ int tri(int i) { return i * (i + 1) / 2; }

// Eight consecutive bf16 elements c0 .. c0+7 of a row of width w as floats
// (past w: 0); one vector load when the row allows it.
__device__ __forceinline__ void rowb8(const bf16* row, int c0, int w, bool vec, float* out) {
  if (vec && c0 + 8 <= w) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(row + c0);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = c0 + e < w ? (float)row[c0 + e] : 0.f;
  }
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
// Gram partials: part[which][block] = Phi_block^T B_block ([KP x KP]),
// which 0: B = Phi, 1: B = high part of O, 2: B = low part of O.
// ---------------------------------------------------------------------------
template <int KP>
__global__ __launch_bounds__(256) void fm_gram(FmArgs a) {
  constexpr int P = Geo<KP>::PITCH;
  __shared__ __attribute__((aligned(16))) char As[kTileRows * P];
  __shared__ __attribute__((aligned(16))) char Bs[kTileRows * P];
  constexpr int NNB = KP / 32, NB = NNB * NNB, NBW = (NB + 3) / 4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  TrReader<KP> tr;
  tr.init(tr_r, tr_c);

  const int which = blockIdx.y;
  const int r_begin = blockIdx.x * kFmRows, r_end = min(a.n, r_begin + kFmRows);
  const bf16* Phi = reinterpret_cast<const bf16*>(a.Phi);
  const bool vec = (a.k & 7) == 0;
  const bool vec4 = (a.k & 3) == 0;
  const char* Bt = which == 0 ? As : Bs;

  f32x16 acc[NBW];
#pragma unroll
  for (int t = 0; t < NBW; ++t) acc[t] = f32x16{};

  for (int r0 = r_begin; r0 < r_end; r0 += kTileRows) {
    for (int ch = tid; ch < kTileRows * (KP / 8); ch += 256) {
      const int r = ch / (KP / 8), c8 = ch - r * (KP / 8), gr = r0 + r;
      float v[8];
      if (gr < r_end) {
        rowb8(Phi + (size_t)gr * a.k, c8 * 8, a.k, vec, v);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
      }
      *reinterpret_cast<bf16x8*>(As + r * P + c8 * 16) = pack8(v);
      if (which > 0) {
        float o[8];
        const float* orow = a.O + (size_t)gr * a.k;
        if (gr < r_end && vec4 && c8 * 8 + 8 <= a.k) {
          const f32x4 o0 = *reinterpret_cast<const f32x4*>(orow + c8 * 8);
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(orow + c8 * 8 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = o0[e];
            o[e + 4] = o1[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = gr < r_end && c8 * 8 + e < a.k ? orow[c8 * 8 + e] : 0.f;
        }
        if (which == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = o[e] - (float)(bf16)o[e];
        }
        *reinterpret_cast<bf16x8*>(Bs + r * P + c8 * 16) = pack8(o);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kc = 0; kc < kTileRows / 16; ++kc) {
#pragma unroll
      for (int t = 0; t < NBW; ++t) {
        const int bi = wave + 4 * t;
        if (NB % 4 == 0 || bi < NB) acc[t] = mma(tr.frag(As, bi / NNB, kc), tr.frag(Bt, bi % NNB, kc), acc[t]);
      }
    }
    __syncthreads();
  }
  float* part = a.part + ((size_t)which * gridDim.x + blockIdx.x) * KP * KP;
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

// Fixed-order sums: G = sum_b part[0][b]; R = sum_b part[1][b] + sum_b
// part[2][b] (with two products: only G).
__global__ __launch_bounds__(256) void fm_reduce(FmArgs a, int nblk, int nprod, int KP) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= KP * KP) return;
  const size_t stride = (size_t)KP * KP;
  float s[3] = {0.f, 0.f, 0.f};
  for (int w = 0; w < nprod; ++w)
    for (int b = 0; b < nblk; ++b) s[w] += a.part[((size_t)w * nblk + b) * stride + idx];
  a.G[idx] = s[0];
  if (nprod == 3) a.R[idx] = s[1] + s[2];
}

// ---------------------------------------------------------------------------
// Cholesky factor of G (k x k), one workgroup of 1024 threads: the lower
// triangle, packed by rows, in LDS; step j scales column j by the square
// root of the pivot and subtracts its outer product from the trailing
// triangle.  L is written packed to global memory.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void fm_chol(FmArgs a, int KP) {
  __shared__ float T[kFmMaxK * (kFmMaxK + 1) / 2];
  const int tid = threadIdx.x, k = a.k;
  for (int t = tid; t < k * k; t += 1024) {
    const int i = t / k, j = t - i * k;
    if (j <= i) T[tri(i) + j] = a.G[(size_t)i * KP + j];
  }
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    const float pivot = T[tri(j) + j];
    __syncthreads();  // every thread has read the pivot before it changes
    const float d = sqrtf(pivot);
    if (tid == 0) T[tri(j) + j] = d;
    const float rd = 1.f / d;
    for (int i = j + 1 + tid; i < k; i += 1024) T[tri(i) + j] *= rd;
    __syncthreads();
    // trailing triangle: rows i > j, columns j < c <= i, 32 row groups x 32
    for (int i = j + 1 + (tid >> 5); i < k; i += 32) {
      const float lij = T[tri(i) + j];
      for (int c = j + 1 + (tid & 31); c <= i; c += 32) T[tri(i) + c] -= lij * T[tri(c) + j];
    }
    __syncthreads();
  }
  for (int t = tid; t < tri(k); t += 1024) a.L[t] = T[t];
}

// ---------------------------------------------------------------------------
// x = L^-T L^-1 b for right-hand side column c = blockIdx.x (one wave):
// forward then backward substitution, the dot products spread over the 64
// lanes and reduced with shuffles.  MODE 0: b = column c of R (KP x KP),
// x -> column c of C (k x k fp32, row-major).  MODE 1: b = column c of dC
// (k x k), x -> column c of X (KP x KP bf16, zero padded).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(64) void fm_solve(FmArgs a, int KP) {
  __shared__ float T[kFmMaxK * (kFmMaxK + 1) / 2];
  __shared__ float x[kFmMaxK];
  const int lane = threadIdx.x, c = blockIdx.x, k = a.k;
  if (c >= k) {  // MODE 1: zero padding columns of X
    if (MODE == 1)
      for (int i = lane; i < KP; i += 64) a.X[(size_t)i * KP + c] = (bf16)0.f;
    return;
  }
  for (int t = lane; t < tri(k); t += 64) T[t] = a.L[t];
  for (int i = lane; i < k; i += 64) x[i] = MODE == 0 ? a.R[(size_t)i * KP + c] : a.dC[(size_t)i * k + c];
  __syncthreads();
  for (int i = 0; i < k; ++i) {
    float s = 0.f;
    for (int p = lane; p < i; p += 64) s += T[tri(i) + p] * x[p];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (lane == 0) x[i] = (x[i] - s) / T[tri(i) + i];
    __syncthreads();
  }
  for (int i = k - 1; i >= 0; --i) {
    float s = 0.f;
    for (int p = i + 1 + lane; p < k; p += 64) s += T[tri(p) + i] * x[p];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (lane == 0) x[i] = (x[i] - s) / T[tri(i) + i];
    __syncthreads();
  }
  if (MODE == 0) {
    for (int i = lane; i < k; i += 64) a.C[(size_t)i * k + c] = x[i];
  } else {
    for (int i = lane; i < KP; i += 64) a.X[(size_t)i * KP + c] = (bf16)(i < k ? x[i] : 0.f);
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
    for (int i = 0; i < 16; ++i) {
      const int c = cb * 32 + c_row(i, h);
      if (c < a.k) out[c] = acc[cb][i];
    }
}

}  // namespace fm

#define SSC_FM_INSTANCES(X) X(224) X(256) X(128) X(64) X(32)

hipError_t launch_fm_gram(int KP, const FmArgs& a, int nblk, int nprod, hipStream_t st) {
#define SSC_L(KK)                                                                            \
  if (KP == KK) {                                                                            \
    hipLaunchKernelGGL((fm::fm_gram<KK>), dim3(nblk, nprod), dim3(256), 0, st, a);            \
    return hipGetLastError();                                                                \
  }
  SSC_FM_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_fm_reduce(int KP, const FmArgs& a, int nblk, int nprod, hipStream_t st) {
  hipLaunchKernelGGL(fm::fm_reduce, dim3((KP * KP + 255) / 256), dim3(256), 0, st, a, nblk, nprod, KP);
  return hipGetLastError();
}

hipError_t launch_fm_chol(int KP, const FmArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(fm::fm_chol, dim3(1), dim3(1024), 0, st, a, KP);
  return hipGetLastError();
}

hipError_t launch_fm_solve(int KP, int mode, const FmArgs& a, hipStream_t st) {
  if (mode == 0) hipLaunchKernelGGL((fm::fm_solve<0>), dim3(a.k), dim3(64), 0, st, a, KP);
  else hipLaunchKernelGGL((fm::fm_solve<1>), dim3(KP), dim3(64), 0, st, a, KP);
  return hipGetLastError();
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
