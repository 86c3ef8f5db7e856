// Block kernels of the spatial-spectral coupling on gfx950:
//   fwd_kernel  O = softmax(Q K^T scale) V and lse, online softmax over tiles;
//   dq_kernel   dQ = scale * (P * (dO V^T - D)) K, P recomputed from lse;
//   dkv_kernel  dV = P^T dO, dK = scale * dS^T Q, per block of source rows.
// (Coupling as attention with Q = F_N, K = F_M, V = Phi_M: project page
// "Spatial-Spectral Coupling as Attention", section "How it works"; the
// restricted support of the geo variant: section "Geo-FlashAttention".)
//
// A workgroup is 4 waves and owns 128 rows (32 per wave) of one side; it
// streams the other side in tiles of 64 positions (4 groups of 16) through
// LDS.  Scores are computed with the owned rows as the MFMA column operand,
// so every lane holds one owned row and 16 streamed positions per 32 x 32
// block: the softmax statistics of a row live in one lane pair (l, l ^ 32)
// and the probabilities feed the second product directly from registers
// (see common.hpp).  The streamed positions come from a RunStream: one run
// for the dense coupling, or the selected source patches (forward, dQ) /
// the selecting target patches (dK/dV) of the geo coupling.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace ssc {

template <typename T>
struct Elems {
  static constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
};

template <typename T>
__device__ __forceinline__ typename FragT<T>::type load_frag_global(const T* p);
template <>
__device__ __forceinline__ bf16x8 load_frag_global<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ f32x8 load_frag_global<float>(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <typename T>
__device__ __forceinline__ typename FragT<T>::type lds_frag_row(const T* p);
template <>
__device__ __forceinline__ bf16x8 lds_frag_row<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <>
__device__ __forceinline__ f32x8 lds_frag_row<float>(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Row-layout tile: 64 positions x W elements from X [npos x W].
template <typename T, int W>
__device__ __forceinline__ void stage_rows(T* __restrict__ lds, const T* __restrict__ X,
                                           const int (&gbase)[kGroupsPerTile], int tid) {
  constexpr int E = Elems<T>::E;
  constexpr int CPR = W / E;
  constexpr int PITCH = W + E;
#pragma unroll
  for (int slot = 0; slot < kGroupsPerTile; ++slot) {
    const int b = gbase[slot];
    for (int e = tid; e < kGroup * CPR; e += kThreads) {
      const int w = e / CPR, cc = e - w * CPR;
      Chunk v = b >= 0 ? ld_chunk(X + (size_t)(b + w) * W + cc * E) : zero_chunk();
      st_chunk(lds + (slot * kGroup + w) * PITCH + cc * E, v);
    }
  }
}

// Transposed tile [W][64 (+pad)] from the grouped layout Xg [npos/16][W][16].
template <typename T, int W>
__device__ __forceinline__ void stage_tr(T* __restrict__ lds, const T* __restrict__ Xg,
                                         const int (&gbase)[kGroupsPerTile], int tid) {
  constexpr int E = Elems<T>::E;
  constexpr int CPG = kGroup / E;
  constexpr int PITCH = kTile + E;
#pragma unroll
  for (int slot = 0; slot < kGroupsPerTile; ++slot) {
    const int b = gbase[slot];
    const T* blk = Xg + (size_t)(b >= 0 ? b / kGroup : 0) * W * kGroup;
    for (int e = tid; e < W * CPG; e += kThreads) {
      const int c = e / CPG, part = e - c * CPG;
      Chunk v = b >= 0 ? ld_chunk(blk + c * kGroup + part * E) : zero_chunk();
      st_chunk(lds + c * PITCH + slot * kGroup + part * E, v);
    }
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, int D, int KP>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdArgs a) {
  typedef typename FragT<T>::type Frag;
  constexpr int E = Elems<T>::E;
  constexpr int KPITCH = D + E;
  constexpr int VPITCH = kTile + E;
  __shared__ __attribute__((aligned(16))) T Ks[kTile * KPITCH];
  __shared__ __attribute__((aligned(16))) T Vt[KP * VPITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;

  int q_begin, q_end;
  RunStream ks;
  if (a.items == nullptr) {
    q_begin = blockIdx.x * kRowsPerWG;
    q_end = a.n_N;
    ks = RunStream{nullptr, 1, nullptr, nullptr, a.npadM, a.n_M};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    const Item it = a.items[blockIdx.x];
    q_begin = a.offN[it.patch] + it.row0;
    q_end = a.offN[it.patch + 1];
    ks = RunStream{a.idx + (size_t)it.patch * a.s, a.s, a.poffM, a.offM, 0, 0};
  }
  const int row = q_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;

  const T* Q = reinterpret_cast<const T*>(a.Q);
  const T* Kp = reinterpret_cast<const T*>(a.Kp);
  const T* Vg = reinterpret_cast<const T*>(a.Vg);

  Frag qf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    if (row_ok) qf[dc] = load_frag_global<T>(Q + (size_t)row * D + dc * 16 + h * 8);
    else qf[dc] = Frag{};
  }

  f32x16 acc[KP / 32];
#pragma unroll
  for (int cb = 0; cb < KP / 32; ++cb) acc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.c2;

  const int ntiles = (total_groups(ks) + kGroupsPerTile - 1) / kGroupsPerTile;
  GroupCursor cur;
  cur.start(ks);
  for (int t = 0; t < ntiles; ++t) {
    int gbase[kGroupsPerTile], gval[kGroupsPerTile];
#pragma unroll
    for (int sl = 0; sl < kGroupsPerTile; ++sl) cur.next(ks, gbase[sl], gval[sl]);
    __syncthreads();
    stage_rows<T, D>(Ks, Kp, gbase, tid);
    stage_tr<T, KP>(Vt, Vg, gbase, tid);
    __syncthreads();

    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
        sc[kb] = mma(lds_frag_row<T>(Ks + (kb * 32 + l32) * KPITCH + dc * 16 + h * 8), qf[dc], sc[kb]);
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = kb * 2 + (i >> 3);
        const int w = 8 * ((i >> 2) & 1) + 4 * h + (i & 3);
        const float x = (w < gval[slot]) ? sc[kb][i] * c2 : -INFINITY;
        sc[kb][i] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = fmaxf(mloc, xor32(mloc));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(sc[kb][i] - m_use);
        sc[kb][i] = p;
        lsum += p;
      }
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) acc[cb] *= alpha;

#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const Frag av = lds_tr8(Vt + (cb * 32 + l32) * VPITCH + kc * 16 + 4 * h);
        const Frag bv = c_to_frag<T>(sc[kc >> 1], (kc & 1) * 8);
        acc[cb] = mma(av, bv, acc[cb]);
      }
    }
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    float* Orow = a.O + (size_t)row * a.k;
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = cb * 32 + c_row(i, h);
        if (c < a.k) Orow[c] = acc[cb][i] * inv;
      }
    }
    if (h == 0) a.lse[row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <typename T, int D, int KP>
__global__ __launch_bounds__(kThreads) void dq_kernel(DqArgs a) {
  typedef typename FragT<T>::type Frag;
  constexpr int E = Elems<T>::E;
  constexpr int KPITCH = D + E;
  constexpr int VPITCH = KP + E;
  constexpr int TPITCH = kTile + E;
  __shared__ __attribute__((aligned(16))) T Ks[kTile * KPITCH];
  __shared__ __attribute__((aligned(16))) T Vs[kTile * VPITCH];
  __shared__ __attribute__((aligned(16))) T Kt[D * TPITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;

  int q_begin, q_end, pos_begin;
  RunStream ks;
  if (a.items == nullptr) {
    q_begin = blockIdx.x * kRowsPerWG;
    q_end = a.n_N;
    pos_begin = q_begin;
    ks = RunStream{nullptr, 1, nullptr, nullptr, a.npadM, a.n_M};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    const Item it = a.items[blockIdx.x];
    q_begin = a.offN[it.patch] + it.row0;
    q_end = a.offN[it.patch + 1];
    pos_begin = a.poffN[it.patch] + it.row0;
    ks = RunStream{a.idx + (size_t)it.patch * a.s, a.s, a.poffM, a.offM, 0, 0};
  }
  const int row = q_begin + wave * 32 + l32;
  const int pos = pos_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;

  const T* Qp = reinterpret_cast<const T*>(a.Qp);
  const T* dOp = reinterpret_cast<const T*>(a.dOp);
  const T* Kp = reinterpret_cast<const T*>(a.Kp);
  const T* Vp = reinterpret_cast<const T*>(a.Vp);
  const T* Kg = reinterpret_cast<const T*>(a.Kg);

  Frag qf[D / 16], of[KP / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    qf[dc] = row_ok ? load_frag_global<T>(Qp + (size_t)pos * D + dc * 16 + h * 8) : Frag{};
#pragma unroll
  for (int kc = 0; kc < KP / 16; ++kc)
    of[kc] = row_ok ? load_frag_global<T>(dOp + (size_t)pos * KP + kc * 16 + h * 8) : Frag{};
  const float lse2 = row_ok ? a.lse2p[pos] : INFINITY;
  const float Dq = row_ok ? a.Dp[pos] : 0.f;
  const float c2 = a.c2;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  const int ntiles = (total_groups(ks) + kGroupsPerTile - 1) / kGroupsPerTile;
  GroupCursor cur;
  cur.start(ks);
  for (int t = 0; t < ntiles; ++t) {
    int gbase[kGroupsPerTile], gval[kGroupsPerTile];
#pragma unroll
    for (int sl = 0; sl < kGroupsPerTile; ++sl) cur.next(ks, gbase[sl], gval[sl]);
    __syncthreads();
    stage_rows<T, D>(Ks, Kp, gbase, tid);
    stage_rows<T, KP>(Vs, Vp, gbase, tid);
    stage_tr<T, D>(Kt, Kg, gbase, tid);
    __syncthreads();

    f32x16 ds[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
        s = mma(lds_frag_row<T>(Ks + (kb * 32 + l32) * KPITCH + dc * 16 + h * 8), qf[dc], s);
#pragma unroll
      for (int kc = 0; kc < KP / 16; ++kc)
        dp = mma(lds_frag_row<T>(Vs + (kb * 32 + l32) * VPITCH + kc * 16 + h * 8), of[kc], dp);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int slot = kb * 2 + (i >> 3);
        const int w = 8 * ((i >> 2) & 1) + 4 * h + (i & 3);
        const float p = (w < gval[slot]) ? fast_exp2(s[i] * c2 - lse2) : 0.f;
        ds[kb][i] = p * (dp[i] - Dq);
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const Frag av = lds_tr8(Kt + (db * 32 + l32) * TPITCH + kc * 16 + 4 * h);
        const Frag bv = c_to_frag<T>(ds[kc >> 1], (kc & 1) * 8);
        dq[db] = mma(av, bv, dq[db]);
      }
    }
  }

  if (row_ok) {
    float* out = a.dQ + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[db * 32 + c_row(i, h)] = a.scale * dq[db][i];
    }
  }
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <typename T, int D, int KP>
__global__ __launch_bounds__(kThreads) void dkv_kernel(DkvArgs a) {
  typedef typename FragT<T>::type Frag;
  constexpr int E = Elems<T>::E;
  constexpr int QPITCH = D + E;
  constexpr int OPITCH = KP + E;
  constexpr int TPITCH = kTile + E;
  __shared__ __attribute__((aligned(16))) T Qs[kTile * QPITCH];
  __shared__ __attribute__((aligned(16))) T dOs[kTile * OPITCH];
  __shared__ __attribute__((aligned(16))) T Qt[D * TPITCH];
  __shared__ __attribute__((aligned(16))) T dOt[KP * TPITCH];
  __shared__ __attribute__((aligned(16))) float lse2s[kTile];
  __shared__ __attribute__((aligned(16))) float Ds[kTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;

  int k_begin, k_end, kpos_begin;
  RunStream qs;
  if (a.items == nullptr) {
    k_begin = blockIdx.x * kRowsPerWG;
    k_end = a.n_M;
    kpos_begin = k_begin;
    qs = RunStream{nullptr, 1, nullptr, nullptr, a.npadN, a.n_N};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    const Item it = a.items[blockIdx.x];
    k_begin = a.offM[it.patch] + it.row0;
    k_end = a.offM[it.patch + 1];
    kpos_begin = a.poffM[it.patch] + it.row0;
    const int i0 = a.inv_off[it.patch];
    qs = RunStream{a.inv_idx + i0, a.inv_off[it.patch + 1] - i0, a.poffN, a.offN, 0, 0};
  }
  const int krow = k_begin + wave * 32 + l32;
  const int kpos = kpos_begin + wave * 32 + l32;
  const bool key_ok = krow < k_end;

  const T* Kp = reinterpret_cast<const T*>(a.Kp);
  const T* Vp = reinterpret_cast<const T*>(a.Vp);
  const T* Qp = reinterpret_cast<const T*>(a.Qp);
  const T* dOp = reinterpret_cast<const T*>(a.dOp);
  const T* Qg = reinterpret_cast<const T*>(a.Qg);
  const T* dOg = reinterpret_cast<const T*>(a.dOg);

  Frag kf[D / 16], vf[KP / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    kf[dc] = key_ok ? load_frag_global<T>(Kp + (size_t)kpos * D + dc * 16 + h * 8) : Frag{};
#pragma unroll
  for (int kc = 0; kc < KP / 16; ++kc)
    vf[kc] = key_ok ? load_frag_global<T>(Vp + (size_t)kpos * KP + kc * 16 + h * 8) : Frag{};
  const float c2 = a.c2;

  f32x16 dv[KP / 32], dk[D / 32];
#pragma unroll
  for (int cb = 0; cb < KP / 32; ++cb) dv[cb] = f32x16{};
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = f32x16{};

  const int ntiles = (total_groups(qs) + kGroupsPerTile - 1) / kGroupsPerTile;
  GroupCursor cur;
  cur.start(qs);
  for (int t = 0; t < ntiles; ++t) {
    int gbase[kGroupsPerTile], gval[kGroupsPerTile];
#pragma unroll
    for (int sl = 0; sl < kGroupsPerTile; ++sl) cur.next(qs, gbase[sl], gval[sl]);
    __syncthreads();
    stage_rows<T, D>(Qs, Qp, gbase, tid);
    stage_rows<T, KP>(dOs, dOp, gbase, tid);
    stage_tr<T, D>(Qt, Qg, gbase, tid);
    stage_tr<T, KP>(dOt, dOg, gbase, tid);
    if (tid < kTile) {
      const int sl = tid / kGroup, w = tid % kGroup;
      int b = -1, v = 0;
#pragma unroll
      for (int j = 0; j < kGroupsPerTile; ++j)
        if (j == sl) {
          b = gbase[j];
          v = gval[j];
        }
      const bool ok = b >= 0 && w < v;
      lse2s[tid] = ok ? a.lse2p[b + w] : INFINITY;
      Ds[tid] = ok ? a.Dp[b + w] : 0.f;
    }
    __syncthreads();

    f32x16 pb[2], ds[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int dc = 0; dc < D / 16; ++dc)
        s = mma(lds_frag_row<T>(Qs + (qb * 32 + l32) * QPITCH + dc * 16 + h * 8), kf[dc], s);
#pragma unroll
      for (int kc = 0; kc < KP / 16; ++kc)
        dp = mma(lds_frag_row<T>(dOs + (qb * 32 + l32) * OPITCH + kc * 16 + h * 8), vf[kc], dp);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = qb * 32 + c_row(i, h);
        const float p = fast_exp2(s[i] * c2 - lse2s[qr]);
        pb[qb][i] = p;
        ds[qb][i] = p * (dp[i] - Ds[qr]);
      }
    }
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const Frag av = lds_tr8(dOt + (cb * 32 + l32) * TPITCH + kc * 16 + 4 * h);
        dv[cb] = mma(av, c_to_frag<T>(pb[kc >> 1], (kc & 1) * 8), dv[cb]);
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const Frag av = lds_tr8(Qt + (db * 32 + l32) * TPITCH + kc * 16 + 4 * h);
        dk[db] = mma(av, c_to_frag<T>(ds[kc >> 1], (kc & 1) * 8), dk[db]);
      }
    }
  }

  if (key_ok) {
    float* okr = a.dK + (size_t)krow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) okr[db * 32 + c_row(i, h)] = a.scale * dk[db][i];
    }
    if (a.dV == nullptr) return;  // dK only
    float* ovr = a.dV + (size_t)krow * a.k;
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = cb * 32 + c_row(i, h);
        if (c < a.k) ovr[c] = dv[cb][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// instances and launchers
// ---------------------------------------------------------------------------
// fp32 instances of the generic kernels (bf16 runs the tb:: kernels of
// attn_bf16_q.hip / attn_bf16_kv.hip)
#define SSC_FOR_EACH_INSTANCE(X) \
  X(float, 64, 32)               \
  X(float, 64, 64)               \
  X(float, 64, 128)              \
  X(float, 128, 32)              \
  X(float, 128, 64)              \
  X(float, 128, 128)

template <typename T> constexpr DType dtype_of();
template <> constexpr DType dtype_of<bf16>() { return DType::BF16; }
template <> constexpr DType dtype_of<float>() { return DType::F32; }

// Compiled shapes: bf16 d in {64, 128} with every padded width (the tb::
// kernels), fp32 d in {64, 128} with padded widths up to 128.
bool supported(DType t, int D, int KP) {
  if (D != 64 && D != 128) return false;
  if (t == DType::BF16) return KP == 32 || KP == 64 || KP == 128 || KP == 224 || KP == 256;
  return KP == 32 || KP == 64 || KP == 128;
}

hipError_t launch_fwd(DType t, int D, int KP, const FwdArgs& a, int grid, hipStream_t st) {
#define SSC_L(TT, DD, KK)                                                                   \
  if (t == dtype_of<TT>() && D == DD && KP == KK) {                                         \
    hipLaunchKernelGGL((fwd_kernel<TT, DD, KK>), dim3(grid), dim3(kThreads), 0, st, a);   \
    return hipGetLastError();                                                               \
  }
  SSC_FOR_EACH_INSTANCE(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_dq(DType t, int D, int KP, const DqArgs& a, int grid, hipStream_t st) {
#define SSC_L(TT, DD, KK)                                                                   \
  if (t == dtype_of<TT>() && D == DD && KP == KK) {                                         \
    hipLaunchKernelGGL((dq_kernel<TT, DD, KK>), dim3(grid), dim3(kThreads), 0, st, a);    \
    return hipGetLastError();                                                               \
  }
  SSC_FOR_EACH_INSTANCE(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_dkv(DType t, int D, int KP, const DkvArgs& a, int grid, hipStream_t st) {
#define SSC_L(TT, DD, KK)                                                                   \
  if (t == dtype_of<TT>() && D == DD && KP == KK) {                                         \
    hipLaunchKernelGGL((dkv_kernel<TT, DD, KK>), dim3(grid), dim3(kThreads), 0, st, a);   \
    return hipGetLastError();                                                               \
  }
  SSC_FOR_EACH_INSTANCE(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
