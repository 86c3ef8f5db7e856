// bf16 block kernels of the spatial-spectral coupling on gfx950.
//
// Same mathematics as attn.hip (forward with online softmax; dQ pass; dK/dV
// pass; project page "Spatial-Spectral Coupling as Attention", sections
// "How it works" and "Geo-FlashAttention"), with a data movement built for
// CDNA4:
//  * tiles of 64 streamed rows are copied global -> LDS with direct loads
//    (global_load_lds, 16 bytes per lane) into a double buffer, so the next
//    tile is in flight while the current one is multiplied;
//  * only row-layout tiles are staged.  Operands whose contraction runs along
//    the tile's rows (V^T in the forward, K^T in dQ, Q^T and dO^T in dK/dV)
//    are read with ds_read_b64_tr_b16: in a 16-lane group, lane j addresses
//    row r0 + j/4, columns c0 + 4(j%4) .. +3, and lane i receives rows
//    r0..r0+3 of column c0 + i -- four k-elements of an MFMA operand;
//  * rows are gathered one by one from the caller's arrays, so the geo
//    support (concatenated source patches) needs no padding: a tile may span
//    several patches and only the stream's last tile is partial;
//  * LDS rows are XOR-swizzled at 16-byte granularity (slot = chunk ^ f(row))
//    so that row-fragment reads (32 rows, one chunk) and transposed reads
//    (4 rows x 32 bytes per 16 lanes) spread over the banks.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace ssc {
namespace tb {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// Geometry of a row tile of W bf16 columns: CW data chunks of 16 bytes per
// row, padded to P slots (a power of two).
template <int W>
struct Geo {
  static constexpr int CW = W / 8;
  static constexpr int P = CW <= 4 ? 4 : (CW <= 8 ? 8 : (CW <= 16 ? 16 : 32));
  static constexpr int MASK = (P < 16 ? P : 16) - 1;
  static constexpr int BYTES = kTile * P * 16;
};

__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 2) & 1); }

template <int W>
__device__ __forceinline__ int slot(int r, int c) {
  return c ^ (swz(r) & Geo<W>::MASK);
}

// 8 consecutive columns [8c, 8c+8) of tile row r.
template <int W>
__device__ __forceinline__ bf16x8 rd_row(const char* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + (r * Geo<W>::P + slot<W>(r, c)) * 16);
}

// Transposed read: this lane addresses 4 columns starting at C (C % 4 == 0)
// of row r.
template <int W>
__device__ __forceinline__ bf16x4 rd_tr(const char* tile, int r, int C) {
  const char* p = tile + (r * Geo<W>::P + slot<W>(r, C >> 3)) * 16 + ((C >> 2) & 1) * 8;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Operand of an MFMA whose contraction runs over tile rows: rows
// kc*16 + {4h..4h+3, 8+4h..8+4h+3}, column block cb (32 columns); tr_r and
// tr_c are this lane's row / column offsets (4h + (i>>2), 16(G&1) + 4(i&3)).
template <int W>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int cb, int kc, int tr_r, int tr_c) {
  const bf16x4 lo = rd_tr<W>(tile, kc * 16 + tr_r, cb * 32 + tr_c);
  const bf16x4 hi = rd_tr<W>(tile, kc * 16 + 8 + tr_r, cb * 32 + tr_c);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Issue the direct loads of one row tile (64 rows) into LDS.  `rows` holds
// the 64 global row indices (negative = no row: any valid row is loaded and
// masked later).  X has row stride ldx elements and at least CW chunks per
// row; slots beyond CW receive a duplicate of chunk 0 (never read).
template <int W, int NW>
__device__ __forceinline__ void load_tile(char* tile, const bf16* __restrict__ X, int ldx, const int* rows,
                                          int wave, int lane) {
  constexpr int P = Geo<W>::P, CW = Geo<W>::CW, NI = kTile * P / 64;
  for (int inst = wave; inst < NI; inst += NW) {
    const int s = inst * 64 + lane;
    const int r = s / P, p = s % P;
    int c = p ^ (swz(r) & Geo<W>::MASK);
    if (c >= CW) c = 0;
    int row = rows[r];
    row = row < 0 ? 0 : row;
    const bf16* src = X + (size_t)row * ldx + c * 8;
    __builtin_amdgcn_global_load_lds((void*)src, (lds_void_t*)(tile + inst * 1024), 16, 0, 0);
  }
}

// 64 fp32 values gathered by row index (negative -> index `sentinel`).
__device__ __forceinline__ void load_vec64(float* dst, const float* __restrict__ src, const int* rows, int sentinel,
                                           int lane) {
  int row = rows[lane];
  row = row < 0 ? sentinel : row;
  __builtin_amdgcn_global_load_lds((void*)(src + row), (lds_void_t*)dst, 4, 0, 0);
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position -> row cursor over a run stream (one per thread; positions of a
// thread only grow).  Run r covers positions [pf[r], pf[r+1]) and starts at
// global row start(r).  Dense: one run of `total` rows starting at row 0.
struct RowCursor {
  const int* pf;       // nullptr = dense
  const int* list;     // run r -> patch
  const int* off;      // patch -> first row
  int nruns, total;
  int r, next, base;   // current run, its end position, row - position

  __device__ __forceinline__ void init() {
    r = 0;
    if (pf == nullptr) {
      next = total;
      base = 0;
      return;
    }
    next = nruns > 0 ? pf[1] : 0;
    base = nruns > 0 ? off[list[0]] - pf[0] : 0;
  }
  __device__ __forceinline__ int row(int x) {
    if (x >= total) return -1;
    if (pf != nullptr) {
      while (x >= next) {
        ++r;
        next = pf[r + 1];
        base = off[list[r]] - pf[r];
      }
    }
    return base + x;
  }
};

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int D, int KP, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_bf16(FwdArgs a) {
  constexpr int KB = Geo<D>::BYTES, VB = Geo<KP>::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * (KB + VB)];
  __shared__ int rowtab[2][kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int q_begin, q_end;
  RowCursor rc;
  if (a.items == nullptr) {
    q_begin = blockIdx.x * (NW * 32);
    q_end = a.n_N;
    rc = RowCursor{nullptr, nullptr, nullptr, 1, a.n_M, 0, 0, 0};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    const Item it = a.items[blockIdx.x];
    q_begin = a.offN[it.patch] + it.row0;
    q_end = a.offN[it.patch + 1];
    const int* pf = a.run_pf + (size_t)it.patch * (a.s + 1);
    rc = RowCursor{pf, a.idx + (size_t)it.patch * a.s, a.offM, a.s, pf[a.s], 0, 0, 0};
  }
  const int total = rc.total;
  const int ntiles = (total + kTile - 1) / kTile;
  const int row = q_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;
  const bool wave_on = q_begin + wave * 32 < q_end;

  const bf16* Q = reinterpret_cast<const bf16*>(a.Q);
  const bf16* K = reinterpret_cast<const bf16*>(a.Kp);
  const bf16* Vp = reinterpret_cast<const bf16*>(a.Vp);

  bf16x8 qf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    qf[dc] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + (size_t)row * D + dc * 16 + h * 8) : bf16x8{};

  f32x16 acc[KP / 32];
#pragma unroll
  for (int cb = 0; cb < KP / 32; ++cb) acc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.c2;

  if (tid < kTile) {
    rc.init();
    rowtab[0][tid] = rc.row(tid);
    rowtab[1][tid] = rc.row(kTile + tid);
  }
  __syncthreads();
  if (ntiles > 0) {
    load_tile<D, NW>(smem, K, D, rowtab[0], wave, lane);
    load_tile<KP, NW>(smem + KB, Vp, KP, rowtab[0], wave, lane);
  }
  wait_loads();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    char* Kt = smem + b * (KB + VB);
    char* Vt = Kt + KB;
    if (t + 1 < ntiles) {
      char* Kn = smem + (b ^ 1) * (KB + VB);
      load_tile<D, NW>(Kn, K, D, rowtab[b ^ 1], wave, lane);
      load_tile<KP, NW>(Kn + KB, Vp, KP, rowtab[b ^ 1], wave, lane);
    }
    if (wave_on) {
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc)
          sc[kb] = mma(rd_row<D>(Kt, kb * 32 + l32, 2 * dc + h), qf[dc], sc[kb]);
      }
      const int nvalid = total - t * kTile;  // keys >= nvalid are masked
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = (kb * 32 + c_row(i, h) < nvalid) ? sc[kb][i] * c2 : -INFINITY;
          sc[kb][i] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, xor32(mloc));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fexp2(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fexp2(sc[kb][i] - m_use);
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
        for (int kc = 0; kc < 4; ++kc)
          acc[cb] = mma(tr_frag<KP>(Vt, cb, kc, tr_r, tr_c), c_to_frag<bf16>(sc[kc >> 1], (kc & 1) * 8), acc[cb]);
      }
    }
    if (tid < kTile && t + 2 < ntiles) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
    wait_loads();
    __syncthreads();
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    float* Orow = a.O + (size_t)row * a.k;
    const bool vec = (a.k & 3) == 0;
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = cb * 32 + 8 * g + 4 * h;
        if (vec) {
          if (c < a.k)
            *reinterpret_cast<f32x4*>(Orow + c) =
                f32x4{acc[cb][4 * g] * inv, acc[cb][4 * g + 1] * inv, acc[cb][4 * g + 2] * inv, acc[cb][4 * g + 3] * inv};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < a.k) Orow[c + e] = acc[cb][4 * g + e] * inv;
        }
      }
    }
    if (h == 0) a.lse[row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
template <int D, int KP, int NW>
__global__ __launch_bounds__(NW * 64) void dq_bf16(DqArgs a) {
  constexpr int KB = Geo<D>::BYTES, VB = Geo<KP>::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * (KB + VB)];
  __shared__ int rowtab[2][kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int q_begin, q_end;
  RowCursor rc;
  if (a.items == nullptr) {
    q_begin = blockIdx.x * (NW * 32);
    q_end = a.n_N;
    rc = RowCursor{nullptr, nullptr, nullptr, 1, a.n_M, 0, 0, 0};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    const Item it = a.items[blockIdx.x];
    q_begin = a.offN[it.patch] + it.row0;
    q_end = a.offN[it.patch + 1];
    const int* pf = a.run_pf + (size_t)it.patch * (a.s + 1);
    rc = RowCursor{pf, a.idx + (size_t)it.patch * a.s, a.offM, a.s, pf[a.s], 0, 0, 0};
  }
  const int total = rc.total;
  const int ntiles = (total + kTile - 1) / kTile;
  const int row = q_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;
  const bool wave_on = q_begin + wave * 32 < q_end;

  const bf16* Q = reinterpret_cast<const bf16*>(a.Qp);
  const bf16* dOp = reinterpret_cast<const bf16*>(a.dOp);
  const bf16* K = reinterpret_cast<const bf16*>(a.Kp);
  const bf16* Vp = reinterpret_cast<const bf16*>(a.Vp);

  bf16x8 qf[D / 16], of[KP / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    qf[dc] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + (size_t)row * D + dc * 16 + h * 8) : bf16x8{};
#pragma unroll
  for (int kc = 0; kc < KP / 16; ++kc)
    of[kc] = row_ok ? *reinterpret_cast<const bf16x8*>(dOp + (size_t)row * KP + kc * 16 + h * 8) : bf16x8{};
  const float lse2 = row_ok ? a.lse2p[row] : INFINITY;
  const float Dq = row_ok ? a.Dp[row] : 0.f;
  const float c2 = a.c2;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  if (tid < kTile) {
    rc.init();
    rowtab[0][tid] = rc.row(tid);
    rowtab[1][tid] = rc.row(kTile + tid);
  }
  __syncthreads();
  if (ntiles > 0) {
    load_tile<D, NW>(smem, K, D, rowtab[0], wave, lane);
    load_tile<KP, NW>(smem + KB, Vp, KP, rowtab[0], wave, lane);
  }
  wait_loads();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    char* Kt = smem + b * (KB + VB);
    char* Vt = Kt + KB;
    if (t + 1 < ntiles) {
      char* Kn = smem + (b ^ 1) * (KB + VB);
      load_tile<D, NW>(Kn, K, D, rowtab[b ^ 1], wave, lane);
      load_tile<KP, NW>(Kn + KB, Vp, KP, rowtab[b ^ 1], wave, lane);
    }
    if (wave_on) {
      const int nvalid = total - t * kTile;
      f32x16 ds[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) s = mma(rd_row<D>(Kt, kb * 32 + l32, 2 * dc + h), qf[dc], s);
#pragma unroll
        for (int kc = 0; kc < KP / 16; ++kc) dp = mma(rd_row<KP>(Vt, kb * 32 + l32, 2 * kc + h), of[kc], dp);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = (kb * 32 + c_row(i, h) < nvalid) ? fexp2(s[i] * c2 - lse2) : 0.f;
          ds[kb][i] = p * (dp[i] - Dq);
        }
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          dq[db] = mma(tr_frag<D>(Kt, db, kc, tr_r, tr_c), c_to_frag<bf16>(ds[kc >> 1], (kc & 1) * 8), dq[db]);
      }
    }
    if (tid < kTile && t + 2 < ntiles) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
    wait_loads();
    __syncthreads();
  }

  if (row_ok) {
    float* out = a.dQ + (size_t)row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = db * 32 + 8 * g + 4 * h;
        *reinterpret_cast<f32x4*>(out + c) = f32x4{a.scale * dq[db][4 * g], a.scale * dq[db][4 * g + 1],
                                                   a.scale * dq[db][4 * g + 2], a.scale * dq[db][4 * g + 3]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <int D, int KP, int NW>
__global__ __launch_bounds__(NW * 64) void dkv_bf16(DkvArgs a) {
  constexpr int QB = Geo<D>::BYTES, OB = Geo<KP>::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[2 * (QB + OB)];
  __shared__ __attribute__((aligned(16))) float lse2s[2][kTile];
  __shared__ __attribute__((aligned(16))) float Ds[2][kTile];
  __shared__ int rowtab[2][kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int k_begin, k_end;
  RowCursor rc;
  if (a.items == nullptr) {
    k_begin = blockIdx.x * (NW * 32);
    k_end = a.n_M;
    rc = RowCursor{nullptr, nullptr, nullptr, 1, a.n_N, 0, 0, 0};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    const Item it = a.items[blockIdx.x];
    k_begin = a.offM[it.patch] + it.row0;
    k_end = a.offM[it.patch + 1];
    const int i0 = a.inv_off[it.patch];
    const int nr = a.inv_off[it.patch + 1] - i0;
    const int* pf = a.inv_pf + i0 + it.patch;
    rc = RowCursor{pf, a.inv_idx + i0, a.offN, nr, pf[nr], 0, 0, 0};
  }
  const int total = rc.total;
  const int ntiles = (total + kTile - 1) / kTile;
  const int krow = k_begin + wave * 32 + l32;
  const bool key_ok = krow < k_end;
  const bool wave_on = k_begin + wave * 32 < k_end;

  const bf16* K = reinterpret_cast<const bf16*>(a.Kp);
  const bf16* Vp = reinterpret_cast<const bf16*>(a.Vp);
  const bf16* Q = reinterpret_cast<const bf16*>(a.Qp);
  const bf16* dOp = reinterpret_cast<const bf16*>(a.dOp);
  const int sentinel = a.n_N;  // lse2p[n_N] = +inf, Dp[n_N] = 0

  bf16x8 kf[D / 16], vf[KP / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    kf[dc] = key_ok ? *reinterpret_cast<const bf16x8*>(K + (size_t)krow * D + dc * 16 + h * 8) : bf16x8{};
#pragma unroll
  for (int kc = 0; kc < KP / 16; ++kc)
    vf[kc] = key_ok ? *reinterpret_cast<const bf16x8*>(Vp + (size_t)krow * KP + kc * 16 + h * 8) : bf16x8{};
  const float c2 = a.c2;

  f32x16 dv[KP / 32], dk[D / 32];
#pragma unroll
  for (int cb = 0; cb < KP / 32; ++cb) dv[cb] = f32x16{};
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = f32x16{};

  if (tid < kTile) {
    rc.init();
    rowtab[0][tid] = rc.row(tid);
    rowtab[1][tid] = rc.row(kTile + tid);
  }
  __syncthreads();
  if (ntiles > 0) {
    load_tile<D, NW>(smem, Q, D, rowtab[0], wave, lane);
    load_tile<KP, NW>(smem + QB, dOp, KP, rowtab[0], wave, lane);
    if (wave == 0) load_vec64(lse2s[0], a.lse2p, rowtab[0], sentinel, lane);
    if (wave == NW - 1) load_vec64(Ds[0], a.Dp, rowtab[0], sentinel, lane);
  }
  wait_loads();
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int b = t & 1;
    char* Qt = smem + b * (QB + OB);
    char* Ot = Qt + QB;
    if (t + 1 < ntiles) {
      char* Qn = smem + (b ^ 1) * (QB + OB);
      load_tile<D, NW>(Qn, Q, D, rowtab[b ^ 1], wave, lane);
      load_tile<KP, NW>(Qn + QB, dOp, KP, rowtab[b ^ 1], wave, lane);
      if (wave == 0) load_vec64(lse2s[b ^ 1], a.lse2p, rowtab[b ^ 1], sentinel, lane);
      if (wave == NW - 1) load_vec64(Ds[b ^ 1], a.Dp, rowtab[b ^ 1], sentinel, lane);
    }
    if (wave_on) {
      f32x16 pb[2], ds[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int dc = 0; dc < D / 16; ++dc) s = mma(rd_row<D>(Qt, qb * 32 + l32, 2 * dc + h), kf[dc], s);
#pragma unroll
        for (int kc = 0; kc < KP / 16; ++kc) dp = mma(rd_row<KP>(Ot, qb * 32 + l32, 2 * kc + h), vf[kc], dp);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = qb * 32 + c_row(i, h);
          const float p = fexp2(s[i] * c2 - lse2s[b][qr]);
          pb[qb][i] = p;
          ds[qb][i] = p * (dp[i] - Ds[b][qr]);
        }
      }
#pragma unroll
      for (int cb = 0; cb < KP / 32; ++cb) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          dv[cb] = mma(tr_frag<KP>(Ot, cb, kc, tr_r, tr_c), c_to_frag<bf16>(pb[kc >> 1], (kc & 1) * 8), dv[cb]);
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          dk[db] = mma(tr_frag<D>(Qt, db, kc, tr_r, tr_c), c_to_frag<bf16>(ds[kc >> 1], (kc & 1) * 8), dk[db]);
      }
    }
    if (tid < kTile && t + 2 < ntiles) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
    wait_loads();
    __syncthreads();
  }

  if (key_ok) {
    float* okr = a.dK + (size_t)krow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = db * 32 + 8 * g + 4 * h;
        *reinterpret_cast<f32x4*>(okr + c) = f32x4{a.scale * dk[db][4 * g], a.scale * dk[db][4 * g + 1],
                                                   a.scale * dk[db][4 * g + 2], a.scale * dk[db][4 * g + 3]};
      }
    }
    float* ovr = a.dV + (size_t)krow * a.k;
    const bool vec = (a.k & 3) == 0;
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = cb * 32 + 8 * g + 4 * h;
        if (vec) {
          if (c < a.k)
            *reinterpret_cast<f32x4*>(ovr + c) = f32x4{dv[cb][4 * g], dv[cb][4 * g + 1], dv[cb][4 * g + 2], dv[cb][4 * g + 3]};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < a.k) ovr[c + e] = dv[cb][4 * g + e];
        }
      }
    }
  }
}

}  // namespace tb

// ---------------------------------------------------------------------------
// instances and launchers
// ---------------------------------------------------------------------------
#define SSC_BF16_INSTANCES(X) \
  X(128, 224)                 \
  X(128, 256)                 \
  X(128, 128)                 \
  X(128, 64)                  \
  X(128, 32)                  \
  X(64, 224)                  \
  X(64, 256)                  \
  X(64, 128)                  \
  X(64, 64)                   \
  X(64, 32)

hipError_t launch_fwd_bf16(int D, int KP, const FwdArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                       \
  if (D == DD && KP == KK) {                                                                                \
    hipLaunchKernelGGL((tb::fwd_bf16<DD, KK, kWavesQ>), dim3(grid), dim3(kWavesQ * 64), 0, st, a);          \
    return hipGetLastError();                                                                               \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_dq_bf16(int D, int KP, const DqArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                       \
  if (D == DD && KP == KK) {                                                                                \
    hipLaunchKernelGGL((tb::dq_bf16<DD, KK, kWavesQ>), dim3(grid), dim3(kWavesQ * 64), 0, st, a);           \
    return hipGetLastError();                                                                               \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_dkv_bf16(int D, int KP, const DkvArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                       \
  if (D == DD && KP == KK) {                                                                                \
    hipLaunchKernelGGL((tb::dkv_bf16<DD, KK, kWavesK>), dim3(grid), dim3(kWavesK * 64), 0, st, a);          \
    return hipGetLastError();                                                                               \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
