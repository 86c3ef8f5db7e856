// Performer (FAVOR+) coupling on gfx950: the pages' second linearized
// baseline (ai4snews digest, "Synopsis"; project page, "Abstract"), read as
// the FAVOR+ estimator of the softmax kernel with positive random features:
//
//     phi(x)_i = exp(sqrt(c) w_i . x - c |x|^2 / 2) / sqrt(m),
//     O_q = phi(q) (sum_j phi(k_j) v_j^T) / (phi(q) . sum_j phi(k_j)),
//
// with c the softmax scale and m directions w_i (rows of W [m x d], an
// input; m, d in {64, 128}).
// The ratio is unchanged when phi_i(k) is multiplied by e^{-M_i} for every
// key and phi_i(q) by e^{M_i - M_q}: the kernels use M_i = max_j of key j's
// exponent for feature i and M_q = the largest shifted query exponent of
// row q, so every stored feature lies in (0, 1] and the largest query
// feature of a row is 1 (no overflow; no row underflows entirely).  The
// |q|^2 term and 1/sqrt(m) are row constants and cancel as well.  The
// linear-attention kernels (identity feature map) then form the products;
// ln den is reported for the true features: ln(den of the shifted features)
// + M_q - c|q|^2/2 - ln m.
//
//   pf_feat      -- the features of 128 rows per workgroup: S = X W^T on bf16
//                   MFMA (transposed: a lane owns a row, the features of that
//                   row sit in its accumulators), then
//                   mode 0: per-block maxima of the key exponents,
//                   mode 1: key features exp2(s - M_i),
//                   mode 2/3: query features exp2(u - M_q), u = s + M_i, and
//                   the row offset (forward) or the shifted den recovered
//                   from ln den (backward);
//                   (modes 1 and 2/3 share one launch, pf_feat_kq: both read
//                   only the key maxima);
//   pf_maxreduce -- M_i = max over the blocks (exact, order-free);
//   pf_dx2       -- dX = sqrt(c) (dF o F) W - c x rowsum(dF o F) (keys; for
//                   queries the row sum vanishes: dO.O - dO.O), dF o F as a
//                   bf16 high + low pair on MFMA; query and key rows in one
//                   launch.
#include "tile_bf16.hpp"

namespace ssc {
namespace pf {

using tb::Geo;
using tb::put_pair;
using tb::RowReader;
using tb::TrReader;

constexpr int kRows = 128;  // rows per workgroup (4 waves x 32)
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) put_pair(r, m, v[2 * m], v[2 * m + 1]);
  return r;
}

// W [M x D] bf16 (row-major, global) into LDS with the padded pitch.
template <int D, int M>
__device__ __forceinline__ void stage_w(char* lds, const bf16* W, int tid) {
  constexpr int CW = D / 8;
  for (int ch = tid; ch < M * CW; ch += 256) {
    const int r = ch / CW, c = ch - r * CW;
    *reinterpret_cast<bf16x8*>(lds + r * Geo<D>::PITCH + c * 16) =
        *reinterpret_cast<const bf16x8*>(W + (size_t)r * D + c * 8);
  }
}

// D: row width d; M: feature count m.
// blk: this workgroup's row block; LDS: Ws [M x D] (padded pitch), sred
// (4 M floats for mode 0, else M), s_sq (kRows floats, mode 0).
template <int D, int M, int MODE>
__device__ __forceinline__ void feat_body(const PfArgs& a, int blk, char* Ws, float* sred, float* s_sq) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  stage_w<D, M>(Ws, reinterpret_cast<const bf16*>(a.W), tid);
  if (MODE != 0)
    for (int f = tid; f < M; f += 256) sred[f] = a.M2[f];
  const int row = blk * kRows + wave * 32 + l32;
  const bool row_ok = row < a.n;
  const bf16* X = reinterpret_cast<const bf16*>(a.X) + (size_t)(row_ok ? row : 0) * D;
  bf16x8 xf[D / 16];
  float ss = 0.f;
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(X + cc * 16 + 8 * h);
    if (!row_ok) v = bf16x8{};
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += (float)v[e] * (float)v[e];
    xf[cc] = v;
  }
  ss += __shfl_xor(ss, 32, 64);
  const float sig2 = sqrtf(a.scale) * kLog2e;
  const float sq2 = 0.5f * a.scale * ss * kLog2e;
  RowReader<D> rw;
  rw.init(l32, h);

  if (MODE == 0) {
    // Key maxima: the product with the operands swapped, C[row][feature],
    // so a lane holds 16 rows of one feature and the maximum over the rows
    // is mostly in-lane.  The row terms come through LDS (-inf for rows past
    // the end).
    s_sq[wave * 32 + l32] = row_ok ? sq2 : INFINITY;
    __syncthreads();
#pragma unroll
    for (int fb = 0; fb < M / 32; ++fb) {
      f32x16 c = f32x16{};
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) c = mma(xf[cc], rw.read(Ws, fb, cc), c);
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, sig2 * c[i] - s_sq[wave * 32 + c_row(i, h)]);
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (h == 0) sred[wave * M + fb * 32 + l32] = m;
    }
    __syncthreads();
    for (int f = tid; f < M; f += 256)
      a.part[(size_t)blk * M + f] =
          fmaxf(fmaxf(sred[f], sred[M + f]), fmaxf(sred[2 * M + f], sred[3 * M + f]));
    return;
  }

  __syncthreads();
  f32x16 acc[M / 32];
#pragma unroll
  for (int fb = 0; fb < M / 32; ++fb) {
    acc[fb] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) acc[fb] = mma(rw.read(Ws, fb, cc), xf[cc], acc[fb]);
  }
  // feature fb*32 + c_row(i, h) of row l32 is acc[fb][i]; exponents in log2 units

  float mq = 0.f;
  if (MODE >= 2) {
    // u = s + M_i; M_q = max over the row's features (both lane halves)
    float m = -INFINITY;
#pragma unroll
    for (int fb = 0; fb < M / 32; ++fb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[fb][i] = sig2 * acc[fb][i] + sred[fb * 32 + c_row(i, h)];
        m = fmaxf(m, acc[fb][i]);
      }
    mq = fmaxf(m, __shfl_xor(m, 32, 64));
  } else {
#pragma unroll
    for (int fb = 0; fb < M / 32; ++fb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[fb][i] = sig2 * acc[fb][i] - sq2 - sred[fb * 32 + c_row(i, h)];
  }
  if (!row_ok) return;
  bf16* F = a.F + (size_t)row * M;
#pragma unroll
  for (int fb = 0; fb < M / 32; ++fb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (bf16)__builtin_amdgcn_exp2f(acc[fb][4 * q + e] - mq);
      *reinterpret_cast<bf16x4*>(F + fb * 32 + 8 * q + 4 * h) = o;
    }
  if (MODE >= 2 && h == 0) {
    const float off = (mq - sq2) * kLn2 - __logf((float)M);
    if (MODE == 2) a.rowoff[row] = off;
    else a.den[row] = __expf(a.lnden[row] - off);
  }
}

// The per-block key maxima (mode 0).
template <int D, int M, int MODE>
__global__ __launch_bounds__(256) void pf_feat(PfArgs a) {
  static_assert(MODE == 0, "the feature modes run in pf_feat_kq");
  __shared__ __attribute__((aligned(16))) char Ws[M * Geo<D>::PITCH];
  __shared__ float sred[4 * M];
  __shared__ float s_sq[kRows];
  feat_body<D, M, MODE>(a, blockIdx.x, Ws, sred, s_sq);
}

// The key features (mode 1, workgroups [0, gK)) and the query features (mode
// QMODE, the rest) in one launch: both read only the key maxima.
template <int D, int M, int QMODE>
__global__ __launch_bounds__(256) void pf_feat_kq(PfArgs ak, PfArgs aq, int gK) {
  __shared__ __attribute__((aligned(16))) char Ws[M * Geo<D>::PITCH];
  __shared__ float sred[M];
  if ((int)blockIdx.x < gK) feat_body<D, M, 1>(ak, blockIdx.x, Ws, sred, nullptr);
  else feat_body<D, M, QMODE>(aq, (int)blockIdx.x - gK, Ws, sred, nullptr);
}

// One workgroup per feature (M of them): the block maxima in parallel, then a tree.
__global__ __launch_bounds__(256) void pf_maxreduce(PfArgs a, int M) {
  __shared__ float sm[4];
  const int f = blockIdx.x, tid = threadIdx.x;
  float m = -INFINITY;
  for (int b = tid; b < a.nblk; b += 256) m = fmaxf(m, a.part[(size_t)b * M + f]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((tid & 63) == 0) sm[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) a.M2[f] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
}

// dX = sqrt(c) (dF o F) W  -  [keys] c x rowsum(dF o F).  A wave owns 32 rows;
// W^T enters as transposed LDS reads (A operand: output dimension x feature),
// so a lane's G fragment takes the features kc*16 + {4h..4h+3, 8+4h..8+4h+3}.
template <int D, int M, int MODE>
__device__ __forceinline__ void dx_body(const PfArgs& a, int blk, char* Ws) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  stage_w<D, M>(Ws, reinterpret_cast<const bf16*>(a.W), tid);
  const int row = blk * kRows + wave * 32 + l32;
  const bool row_ok = row < a.n;
  const size_t r = (size_t)(row_ok ? row : 0) * D, rf = (size_t)(row_ok ? row : 0) * M;
  bf16x8 gh[M / 16], gl[M / 16];
  float rs = 0.f;
#pragma unroll
  for (int kc = 0; kc < M / 16; ++kc) {
    float hi[8], lo[8];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int f0 = kc * 16 + 8 * p + 4 * h;
      const f32x4 df = *reinterpret_cast<const f32x4*>(a.dF + rf + f0);
      const bf16x4 fv = *reinterpret_cast<const bf16x4*>(a.F + rf + f0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g = row_ok ? df[e] * (float)fv[e] : 0.f;
        rs += g;
        const float gh1 = (float)(bf16)g;
        hi[4 * p + e] = gh1;
        lo[4 * p + e] = g - gh1;
      }
    }
    gh[kc] = pack8(hi);
    gl[kc] = pack8(lo);
  }
  rs += __shfl_xor(rs, 32, 64);
  __syncthreads();
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  TrReader<D> tw;
  tw.init(tr_r, tr_c);
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    acc[db] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < M / 16; ++kc) {
      const bf16x8 w = tw.frag(Ws, db, kc);
      acc[db] = mma(w, gh[kc], acc[db]);
      acc[db] = mma(w, gl[kc], acc[db]);
    }
  }
  if (!row_ok) return;
  const float sig = sqrtf(a.scale), c = a.scale;
  const bf16* X = reinterpret_cast<const bf16*>(a.X) + r;
  float* out = a.dX + r;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d0 = db * 32 + 8 * q + 4 * h;
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = sig * acc[db][4 * q + e];
      if (MODE == 1) {
        const bf16x4 xv = *reinterpret_cast<const bf16x4*>(X + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] -= c * (float)xv[e] * rs;
      }
      *reinterpret_cast<f32x4*>(out + d0) = o;
    }
}

// The query rows (mode 0, workgroups [0, gQ)) and the key rows (mode 1, the
// rest) in one launch.
template <int D, int M>
__global__ __launch_bounds__(256) void pf_dx2(PfArgs aq, PfArgs ak, int gQ) {
  __shared__ __attribute__((aligned(16))) char Ws[M * Geo<D>::PITCH];
  if ((int)blockIdx.x < gQ) dx_body<D, M, 0>(aq, blockIdx.x, Ws);
  else dx_body<D, M, 1>(ak, (int)blockIdx.x - gQ, Ws);
}

}  // namespace pf

#define SSC_PF_INSTANCES(X) X(128, 128) X(128, 64) X(64, 64) X(64, 128)

hipError_t launch_pf_keymax(int D, int M, const PfArgs& a, hipStream_t st) {
  const int grid = (a.n + pf::kRows - 1) / pf::kRows;
  if (grid == 0) return hipSuccess;  // no rows
#define SSC_L(DD, MM)                                                                         \
  if (D == DD && M == MM) {                                                                   \
    hipLaunchKernelGGL((pf::pf_feat<DD, MM, 0>), dim3(grid), dim3(256), 0, st, a);            \
    return hipGetLastError();                                                                 \
  }
  SSC_PF_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_pf_feat_kq(int D, int M, int qmode, const PfArgs& ak, const PfArgs& aq, hipStream_t st) {
  const int gK = (ak.n + pf::kRows - 1) / pf::kRows, gQ = (aq.n + pf::kRows - 1) / pf::kRows;
  if (gK + gQ == 0) return hipSuccess;
#define SSC_L(DD, MM)                                                                                          \
  if (D == DD && M == MM) {                                                                                    \
    if (qmode == 2) hipLaunchKernelGGL((pf::pf_feat_kq<DD, MM, 2>), dim3(gK + gQ), dim3(256), 0, st, ak, aq, gK); \
    else hipLaunchKernelGGL((pf::pf_feat_kq<DD, MM, 3>), dim3(gK + gQ), dim3(256), 0, st, ak, aq, gK);            \
    return hipGetLastError();                                                                                  \
  }
  SSC_PF_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_pf_maxreduce(int M, const PfArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pf::pf_maxreduce, dim3(M), dim3(256), 0, st, a, M);
  return hipGetLastError();
}

hipError_t launch_pf_dx2(int D, int M, const PfArgs& aq, const PfArgs& ak, hipStream_t st) {
  const int gQ = (aq.n + pf::kRows - 1) / pf::kRows, gK = (ak.n + pf::kRows - 1) / pf::kRows;
  if (gQ + gK == 0) return hipSuccess;
#define SSC_L(DD, MM)                                                                              \
  if (D == DD && M == MM) {                                                                        \
    hipLaunchKernelGGL((pf::pf_dx2<DD, MM>), dim3(gQ + gK), dim3(256), 0, st, aq, ak, gQ);         \
    return hipGetLastError();                                                                      \
  }
  SSC_PF_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
