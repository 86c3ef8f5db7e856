// Preparation kernels of the coupling:
//   pack_kernel  -- rows of one tensor into the padded patch layout (row-major
//                   copy and grouped-transposed copy), plus D = rowdot(dO, O)
//                   and lse * log2(e) on the target side of the backward;
//   pad_bf16_kernel -- bf16 rows padded to the MFMA width (ones / -D columns),
//                   D and lse * log2(e) for the backward's target side;
//   plan_kernel  -- validates patch offsets and the selection, builds padded
//                   offsets, work items and the inverse selection lists;
//   plan_pad_kernel -- the plan and the bf16 padding of a geo call in one
//                   launch (the padding on the CUs the plan leaves idle);
//   pool_kernel  -- patch-mean descriptors in fp64 ("pool source keys");
//   topk_kernel  -- patch scores <Qbar_p, Kbar_q> in fp64 and the top-s source
//                   patches per target patch, ties to the lower index
//                   ("score source patches", "keep the top R per target
//                   patch": project page, section "Geo-FlashAttention").
//
// Padded patch layout: patch p occupies padded positions
// [poff[p], poff[p+1]) with poff[p+1] - poff[p] = roundup(|p|, 16); its rows
// sit at the front in their patch-sorted order and the tail is zero.  The
// grouped-transposed copy stores every group of 16 positions as a [W][16]
// block, so a tile of 64 gathered positions is four contiguous blocks.
#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

namespace ssc {

// ---------------------------------------------------------------------------
// pack
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  constexpr int E = 16 / sizeof(T);
  constexpr int WMAX = 256;
  __shared__ __attribute__((aligned(16))) T tile[kGroup * (WMAX + E)];
  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int pos0 = g * kGroup;
  int row0, nrows;
  if (a.poff == nullptr) {
    row0 = pos0;
    nrows = min(max(a.n - pos0, 0), kGroup);
  } else {
    if (g >= *a.n_groups) return;
    // patch p: the last one with poff[p] <= pos0 (binary search, uniform)
    int lo = 0, hi = a.P - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.poff[mid] <= pos0) lo = mid;
      else hi = mid - 1;
    }
    const int local = pos0 - a.poff[lo];
    row0 = a.off[lo] + local;
    nrows = min(max(a.off[lo + 1] - a.off[lo] - local, 0), kGroup);
  }
  const int W = a.W, w = a.w, pitch = W + E;
  const T* X = reinterpret_cast<const T*>(a.X);
  for (int e = tid; e < kGroup * W; e += 256) {
    const int r = e / W, c = e - r * W;
    T v = T(0.f);
    if (r < nrows && c < w) v = X[(size_t)(row0 + r) * w + c];
    else if (r < nrows && c == w && a.ones) v = T(1.f);
    tile[r * pitch + c] = v;
  }
  __syncthreads();
  if (a.Xp != nullptr) {
    T* Xp = reinterpret_cast<T*>(a.Xp);
    const int cpr = W / E;
    for (int e = tid; e < kGroup * cpr; e += 256) {
      const int r = e / cpr, cc = e - r * cpr;
      st_chunk(Xp + (size_t)(pos0 + r) * W + cc * E, *reinterpret_cast<const Chunk*>(tile + r * pitch + cc * E));
    }
  }
  if (a.Xg != nullptr) {
    T* blk = reinterpret_cast<T*>(a.Xg) + (size_t)g * W * kGroup;
    constexpr int CPG = kGroup / E;
    for (int e = tid; e < W * CPG; e += 256) {
      const int c = e / CPG, part = e - c * CPG;
      T v[E];
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = tile[(part * E + j) * pitch + c];
      st_chunk(blk + c * kGroup + part * E, *reinterpret_cast<const Chunk*>(v));
    }
  }
  if (a.Dp != nullptr) {
    // 16 lanes per row: partial dot products, then a butterfly over the 16.
    const int r = tid >> 4, j = tid & 15;
    float part = 0.f;
    if (r < nrows) {
      const float* O = a.O + (size_t)(row0 + r) * w;
      for (int c = j; c < w; c += 16) part += to_f32(tile[r * pitch + c]) * O[c];
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 16);
    if (j == 0) {
      a.Dp[pos0 + r] = r < nrows ? part : 0.f;
      float l2 = INFINITY;
      if (r < nrows) {
        const float l = a.lse[row0 + r];
        l2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
      }
      a.lse2p[pos0 + r] = l2;
    }
  }
}

// bf16 rows padded to W <= 256 columns (position = row), plus the rowdot /
// lse extras: 16 lanes per row, each owning the 16-byte chunks j and j + 16
// of the padded row; VEC: w % 8 == 0 and 16-byte aligned rows (of X and O),
// so every chunk inside the row is one 16-byte load (two for O).  Present
// rows get `ones` columns of 1 from column w on; with dcol (and O), columns w
// and w + 1 hold -D split into a bf16 high part and a bf16 low part (their
// sum is -D to about 2^-17 relative), so a product with a ones column adds -D.
// Rows 16 blk .. 16 blk + 15 of one bf16 padding job, 16 threads a row
// (tid < 256; no barrier, no LDS).
template <bool VEC>
__device__ __forceinline__ void pad_rows(const PackArgs& a, int blk, int tid) {
  const int r = blk * 16 + (tid >> 4), j = tid & 15;
  const int w = a.w, cw = a.W / 8;
  const bool present = r < a.n;
  const bf16* X = reinterpret_cast<const bf16*>(a.X) + (size_t)r * w;
  bf16* Xp = reinterpret_cast<bf16*>(a.Xp) + (size_t)r * a.W;
  const float* O = a.O != nullptr ? a.O + (size_t)r * w : nullptr;
  float part = 0.f;
  bf16x8 v[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int c = j + 16 * m, c0 = 8 * c;
    if (c >= cw) continue;
    if (VEC && present && c0 + 8 <= w) {
      v[m] = *reinterpret_cast<const bf16x8*>(X + c0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = c0 + e;
        float x = 0.f;
        if (present && col < w) x = (float)X[col];
        else if (present && col < w + a.ones) x = 1.f;
        v[m][e] = (bf16)x;
      }
    }
    if (O != nullptr && present) {
      if (VEC && c0 + 8 <= w) {
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + c0), o1 = *reinterpret_cast<const f32x4*>(O + c0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) part += (float)v[m][e] * o0[e] + (float)v[m][e + 4] * o1[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < w) part += (float)v[m][e] * O[c0 + e];
      }
    }
  }
  if (a.Dp != nullptr) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 16);
  }
  if (a.dcol && present) {
    const bf16 hi = (bf16)(-part);
    const bf16 lo = (bf16)(-part - (float)hi);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = 8 * (j + 16 * m) + e;
        if (col == w) v[m][e] = hi;
        if (col == w + 1) v[m][e] = lo;
      }
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
    if (j + 16 * m < cw) *reinterpret_cast<bf16x8*>(Xp + 8 * (j + 16 * m)) = v[m];
  if (a.Dp != nullptr && j == 0) {
    a.Dp[r] = present ? part : 0.f;
    float l2 = INFINITY;
    if (present) {
      const float l = a.lse[r];
      l2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }
    a.lse2p[r] = l2;
  }
}

template <bool VEC>
__global__ __launch_bounds__(256) void pad_bf16_kernel(PackArgs a) {
  pad_rows<VEC>(a, blockIdx.x, threadIdx.x);
}

// Grouped-transposed copy of bf16 rows: one workgroup per 64 rows (4 groups
// of 16).  The rows' block X[j0 .. j0 + 64) is contiguous, so it is read with
// coalesced loads (16 bytes when w % 8 == 0) into LDS (pitch 257 halves, so
// reading a column hits distinct banks); the 4 groups' [W][16] blocks are
// one contiguous output range, written in 16-byte chunks of 8 positions.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const unsigned short* X, int n, int w, int W, int ones,
                                                             unsigned short* Xt, int npad) {
  constexpr int P = 257;
  __shared__ unsigned short t[64 * P];
  const int j0 = blockIdx.x * 64, tid = threadIdx.x;
  const int rows = min(64, n - j0);
  const int total = rows > 0 ? rows * w : 0;
  const unsigned short* src = X + (size_t)j0 * w;
  if ((w & 7) == 0) {
    for (int q = tid; q < total / 8; q += 256) {
      const Chunk v = ld_chunk(src + 8 * q);
      const int r = (8 * q) / w, c0 = 8 * q - r * w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t[r * P + c0 + 2 * e] = (unsigned short)(v.w[e] & 0xffffu);
        t[r * P + c0 + 2 * e + 1] = (unsigned short)(v.w[e] >> 16);
      }
    }
  } else {
    for (int i = tid; i < total; i += 256) t[(i / w) * P + i % w] = src[i];
  }
  __syncthreads();
  // chunk q of the block's 4 groups: group g = q / (2 W), row c, half h
  for (int q = tid; q < W * 8; q += 256) {
    const int g = q / (2 * W), rem = q - g * 2 * W, c = rem >> 1, jj = 16 * g + 8 * (rem & 1);
    unsigned short v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = jj + e;
      unsigned short x = 0;
      if (j < rows) {
        if (c < w) x = t[j * P + c];
        else if (c < w + ones) x = 0x3f80;  // bf16 1.0
      }
      v[e] = x;
    }
    Chunk o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o.w[e] = (uint32_t)v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
    st_chunk(Xt + ((size_t)(j0 / 16 + g) * W + c) * 16 + 8 * (rem & 1), o);
  }
}

hipError_t launch_transpose_bf16(const void* X, int n, int w, int W, int ones, void* Xt, int npad, hipStream_t st) {
  if (npad <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(npad / 64), dim3(256), 0, st,
                     reinterpret_cast<const unsigned short*>(X), n, w, W, ones, reinterpret_cast<unsigned short*>(Xt),
                     npad);
  return hipGetLastError();
}

// Squared norms of bf16 rows (d = 64 or 128, 16-byte aligned rows), their
// maximum per workgroup: one thread per 16-byte chunk, the d / 8 chunks of a
// row reduced over consecutive lanes, grid-stride over the rows.
__global__ __launch_bounds__(256) void keynorm_kernel(const bf16* K, int n, int d, float* part) {
  __shared__ float wmax[4];
  const int cpr = d / 8;                 // chunks per row: 8 or 16
  const int rows_per_block = 256 / cpr;
  const int tid = threadIdx.x, c = tid % cpr;
  float best = 0.f;
  for (int r0 = blockIdx.x * rows_per_block; r0 < n; r0 += gridDim.x * rows_per_block) {
    const int r = r0 + tid / cpr;
    float s2 = 0.f;
    if (r < n) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(K + (size_t)r * d + c * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) s2 = fmaf((float)v[e], (float)v[e], s2);
    }
    for (int m = cpr / 2; m >= 1; m >>= 1) s2 += __shfl_xor(s2, m, 64);
    best = fmaxf(best, s2);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) best = fmaxf(best, __shfl_xor(best, m, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) part[blockIdx.x] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

hipError_t launch_keynorm(const void* K, int n, int d, float* part, hipStream_t st) {
  hipLaunchKernelGGL(keynorm_kernel, dim3(kNormParts), dim3(256), 0, st, reinterpret_cast<const bf16*>(K), n, d,
                     part);
  return hipGetLastError();
}

bool pad_bf16_applies(DType t, const PackArgs& a) {
  return t == DType::BF16 && a.poff == nullptr && a.Xg == nullptr && a.Xp != nullptr && (a.W & 7) == 0 &&
         a.W <= 256;
}
bool pad_bf16_vec(const PackArgs& a) {
  return (a.w & 7) == 0 && (reinterpret_cast<uintptr_t>(a.X) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(a.O) & 15) == 0;
}

hipError_t launch_pack(DType t, const PackArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (pad_bf16_applies(t, a)) {
    // dense row padding: one block per group of 16 positions
    const bool vec = pad_bf16_vec(a);
    if (vec) hipLaunchKernelGGL(pad_bf16_kernel<true>, dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(pad_bf16_kernel<false>, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (t == DType::BF16) hipLaunchKernelGGL(pack_kernel<bf16>, dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(pack_kernel<float>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// plan (one workgroup of 1024 threads)
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanRows = 32;       // target patches per chunk of the selection pass
constexpr int kMaxPatches = 8192;   // per side

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Exclusive scan of f(i), i < n, written to out[0..n] (out[n] = total).
// Chunks of kPlanThreads with a running carry: wave scans, then a scan of
// the wave totals.  Returns the total.
template <typename F>
__device__ int block_scan_excl(int n, F f, int* out, int* lds /* kPlanWaves + 1 */) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += kPlanThreads) {
    const int i = base + tid;
    const int v = i < n ? f(i) : 0;
    const int inc = wave_incl_scan(v);
    if (lane == 63) lds[w] = inc;
    __syncthreads();
    if (w == 0) {
      const int t = lane < kPlanWaves ? lds[lane] : 0;
      const int ti = wave_incl_scan(t);
      if (lane < kPlanWaves) lds[lane] = ti - t;
      if (lane == kPlanWaves - 1) lds[kPlanWaves] = ti;
    }
    __syncthreads();
    if (i < n) out[i] = carry + lds[w] + inc - v;
    carry += lds[kPlanWaves];
    __syncthreads();
  }
  if (tid == 0) out[n] = carry;
  __syncthreads();
  return carry;
}

// Exclusive prefix of one value per thread over the workgroup; *total gets
// the sum.
__device__ int block_excl1(int v, int* lds /* kPlanWaves + 1 */, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) lds[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int t = lane < kPlanWaves ? lds[lane] : 0;
    const int ti = wave_incl_scan(t);
    if (lane < kPlanWaves) lds[lane] = ti - t;
    if (lane == kPlanWaves - 1) lds[kPlanWaves] = ti;
  }
  __syncthreads();
  const int r = lds[w] + inc - v;
  *total = lds[kPlanWaves];
  __syncthreads();
  return r;
}

constexpr int kCostBuckets = 4096;  // item costs (stream tiles), clamped, for the dispatch order

// Work items of one side: patch p has rows off[p] .. off[p+1] (items of
// `rows` rows) and a gathered stream of tiles(p) tiles.  Without `spl` the
// items come in patch order and cover whole streams.  With `spl`: N items
// fill N / kRoundCUs full rounds plus R = N mod kRoundCUs; the R cheapest
// items (cost ascending, then item order) are split into m = min(kMaxParts,
// kRoundCUs / R) parts of their stream, and the dispatch order is the whole
// items by decreasing cost, then the parts.  Which items are split and their
// slots depend only on the costs, so the results do not depend on the
// (atomic) order among equal-cost whole items.  Returns the number of units.
template <typename TilesF>
__device__ int make_items(int nP, const int* off, int rows, TilesF tiles, Item* items, SplitItem* spl, int* n_split,
                          int* tmp /* 3 (nP + 1) */, int* lds, int* hist /* kCostBuckets */, int* s_misc /* 2 */,
                          int* tl /* nP, LDS */, int* cn /* nP, LDS */) {
  const int tid = threadIdx.x;
  int* eqb = tmp + (nP + 1);
  int* spb = tmp + 2 * (nP + 1);
  // per patch: items and stream tiles, kept in LDS
  for (int p = tid; p < nP; p += kPlanThreads) {
    cn[p] = (off[p + 1] - off[p] + rows - 1) / rows;
    tl[p] = spl != nullptr ? tiles(p) : 0;
  }
  __syncthreads();
  const int N = block_scan_excl(nP, [=](int p) { return cn[p]; }, tmp, lds);
  int R = spl != nullptr ? N % kRoundCUs : 0;
  int m = R > 0 ? min(kMaxParts, kRoundCUs / R) : 1;
  if (m < 2) {
    R = 0;
    m = 1;
  }
  // the patch of item i (tmp[p] <= i < tmp[p + 1]): items are spread over the
  // threads one by one, so a patch with many items is not left to one thread
  auto patch_of = [&](int i) {
    int lo = 0, hi = nP - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tmp[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  };
  if (R == 0) {
    for (int i = tid; i < N; i += kPlanThreads) {
      const int p = patch_of(i);
      items[i] = Item{p, (i - tmp[p]) * rows, 0, 0x7fffffff, -1};
    }
    if (tid == 0 && n_split != nullptr) *n_split = 0;
    __syncthreads();
    return N;
  }
  auto cost = [&](int p) { return min(tl[p], kCostBuckets - 1); };
  for (int c = tid; c < kCostBuckets; c += kPlanThreads) hist[c] = 0;
  __syncthreads();
  for (int p = tid; p < nP; p += kPlanThreads) {
    const int nt = cn[p];
    if (nt > 0) atomicAdd(&hist[cost(p)], nt);
  }
  __syncthreads();
  // threshold bucket c*: the R-th cheapest item has cost c*
  constexpr int BPT = kCostBuckets / kPlanThreads;
  {
    int v = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) v += hist[BPT * tid + i];
    int tot;
    int cum = block_excl1(v, lds, &tot);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int h = hist[BPT * tid + i];
      if (cum < R && cum + h >= R) {
        s_misc[0] = BPT * tid + i;
        s_misc[1] = cum;
      }
      cum += h;
    }
  }
  __syncthreads();
  const int cstar = s_misc[0], need = R - s_misc[1];
  block_scan_excl(nP, [&](int p) { return cost(p) == cstar ? cn[p] : 0; }, eqb, lds);
  auto nsplit = [&](int p) {
    const int c = cost(p), nt = cn[p];
    return c < cstar ? nt : c == cstar ? min(max(need - eqb[p], 0), nt) : 0;
  };
  block_scan_excl(nP, nsplit, spb, lds);
  // whole items by decreasing cost: start of each bucket in the order
  {
    int v = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int c = kCostBuckets - 1 - (BPT * tid + i);
      v += c > cstar ? hist[c] : c == cstar ? hist[c] - need : 0;
    }
    int tot;
    int cum = block_excl1(v, lds, &tot);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int c = kCostBuckets - 1 - (BPT * tid + i);
      const int hu = c > cstar ? hist[c] : c == cstar ? hist[c] - need : 0;
      hist[c] = cum;
      cum += hu;
    }
  }
  __syncthreads();
  const int U = N - R;
  // item t of patch p: split (its parts after the U whole items) if t <
  // nsplit(p), else whole (placed in its cost bucket)
  for (int i = tid; i < N; i += kPlanThreads) {
    const int p = patch_of(i), t = i - tmp[p], ns = nsplit(p);
    if (t >= ns) {
      items[atomicAdd(&hist[cost(p)], 1)] = Item{p, t * rows, 0, 0x7fffffff, -1};
      continue;
    }
    const int T = tl[p], j = spb[p] + t;
    spl[j] = SplitItem{p, t * rows, m, j * m};
    for (int q = 0; q < m; ++q)
      items[U + j * m + q] = Item{p, t * rows, (int)((long long)q * T / m), (int)((long long)(q + 1) * T / m), j * m + q};
  }
  if (tid == 0) *n_split = R;
  __syncthreads();
  return U + R * m;
}

// Entries e0 .. e1 - 1 of the selection (one chunk of target patches): a
// thread takes e0 + tid + r kPlanThreads.  The first kChunkRegs of them are
// kept in registers across the phases of a chunk (every one when
// s <= kChunkRegs kPlanThreads / kPlanRows); the rest are read again.
constexpr int kChunkRegs = 2;

__device__ __forceinline__ void load_chunk(const int* idx, int e0, int e1, int* qc) {
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) {
    const int e = e0 + (int)threadIdx.x + r * kPlanThreads;
    qc[r] = e < e1 ? idx[e] : -1;
  }
}

template <typename F>
__device__ __forceinline__ void for_chunk(const int* idx, int e0, int e1, const int* qc, F f) {
#pragma unroll
  for (int r = 0; r < kChunkRegs; ++r) {
    const int e = e0 + (int)threadIdx.x + r * kPlanThreads;
    if (e < e1) f(e, qc[r]);
  }
  for (int e = e0 + (int)threadIdx.x + kChunkRegs * kPlanThreads; e < e1; e += kPlanThreads) f(e, idx[e]);
}

// The selection is read in chunks of kPlanRows target patches: every entry
// (p, q) of a chunk sets bit p - p0 of mask[q] (a bit already set is a
// repeated source patch within row p).  For the inverse lists, the rank of
// p among the chunk's patches selecting q is the number of mask bits below
// it, so list q is filled in ascending p, chunk after chunk, with no sort.
// Two mask arrays alternate between chunks, so the bits of one chunk are
// cleared while the next chunk sets its own.
__device__ __forceinline__ void plan_body(const PlanArgs& a, const int role_block) {
  __shared__ int lds[kPlanWaves + 1];
  __shared__ int s_offM[kMaxPatches + 1];  // source offsets; later the second mask array
  __shared__ unsigned s_mask[kMaxPatches];
  __shared__ int s_cur[kMaxPatches];   // counts, then the next free slot of list q
  __shared__ int s_acc[kMaxPatches];   // target rows in list q so far
  __shared__ int s_szN[2][kPlanRows], s_offN[2][kPlanRows];
  const int tid = threadIdx.x;
  const int P_N = a.P_N, P_M = a.P_M, S = a.s;
  const bool inverse = a.inv_off != nullptr && a.idx != nullptr;
  // With inverse lists the plan runs as two workgroups: role 0 builds the
  // target side (selection check, padded offsets, run tables, target items),
  // role 1 the source side (list lengths, inverse lists, source items).  Both
  // check the same conditions on the same inputs (offsets, entry range,
  // repeats within a row), so they reach the same verdict; each writes only
  // its own outputs and counters.  Without inverse lists one workgroup (role
  // 0) does everything.
  const int role = inverse ? role_block : 0;
  const int* offN = a.offN;
  const int* offM = a.offM;
  // ---- offsets: validation, source offsets into LDS
  int bad = 0;
  if (tid == 0) {
    bad |= a.offN[0] != 0 || a.offN[P_N] != a.n_N;
    bad |= a.offM[0] != 0 || a.offM[P_M] != a.n_M;
  }
  for (int p = tid; p < P_N; p += kPlanThreads) bad |= a.offN[p] > a.offN[p + 1];
  for (int q = tid; q <= P_M; q += kPlanThreads) {
    const int o = a.offM[q];
    s_offM[q] = o;
    if (q < P_M) {
      bad |= o > a.offM[q + 1];
      s_mask[q] = 0u;
      s_cur[q] = 0;
      s_acc[q] = 0;
    }
  }
  bad = __syncthreads_or(bad);
  const int nC = (P_N + kPlanRows - 1) / kPlanRows;  // selection chunks
  auto chunk_end = [&](int c) { return min((c + 1) * kPlanRows, P_N) * S; };
  // ---- selection: range (both roles), list lengths (role 1) and repeats
  // within a row: role 0 here by the chunk masks, role 1 in its inverse
  // pass (which builds the same masks) before anything is published.
  if (!bad && a.idx != nullptr) {
    if (role == 1) {
      const int nE = P_N * S;
      for (int e = tid; e < nE; e += 4 * kPlanThreads) {
        int qv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) qv[r] = e + r * kPlanThreads < nE ? a.idx[e + r * kPlanThreads] : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = qv[r];
          if (e + r * kPlanThreads >= nE) continue;
          if (q < 0 || q >= P_M) bad = 1;
          else atomicAdd(&s_cur[q], 1);
        }
      }
    } else {
      // s_cur is not needed on the target side: the second mask array
      unsigned* const buf0 = s_mask;
      unsigned* const buf1 = reinterpret_cast<unsigned*>(s_cur);
      int qc[kChunkRegs], qp[kChunkRegs], qn[kChunkRegs];
      load_chunk(a.idx, 0, chunk_end(0), qc);
      for (int c = 0; c < nC; ++c) {
        const int p0 = c * kPlanRows, e0 = p0 * S, e1 = chunk_end(c);
        if (c + 1 < nC) load_chunk(a.idx, e1, chunk_end(c + 1), qn);
        unsigned* cur = (c & 1) ? buf1 : buf0;
        for_chunk(a.idx, e0, e1, qc, [&](int e, int q) {
          if (q < 0 || q >= P_M) {
            bad = 1;
            return;
          }
          const unsigned bit = 1u << (e / S - p0);
          if (atomicOr(&cur[q], bit) & bit) bad = 1;
        });
        if (c > 0) {
          unsigned* prev = (c & 1) ? buf0 : buf1;
          for_chunk(a.idx, e0 - kPlanRows * S, e0, qp, [&](int, int q) {
            if (q >= 0 && q < P_M) prev[q] = 0u;
          });
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kChunkRegs; ++r) {
          qp[r] = qc[r];
          qc[r] = qn[r];
        }
      }
    }
  }
  auto fail = [&]() {
    if (tid == 0) {
      a.counters[0] = a.counters[1] = a.counters[2] = a.counters[3] = 0;
      a.counters[5] = a.counters[6] = 0;  // no split items either: the merge passes idle
      a.counters[4] = 1;
    }
  };
  bad = __syncthreads_or(bad);
  if (bad) {
    fail();
    return;
  }
  // ---- padded offsets
  int gN = 0, gM = 0;
  if (role == 0) {
    gN = block_scan_excl(P_N, [=](int p) { return (offN[p + 1] - offN[p] + kGroup - 1) & ~(kGroup - 1); }, a.poffN,
                         lds);
    gM = block_scan_excl(P_M, [&](int q) { return (s_offM[q + 1] - s_offM[q] + kGroup - 1) & ~(kGroup - 1); },
                         a.poffM, lds);
  }
  // ---- per target patch: the run table of its key stream (the selected
  // source patches in selection order)
  if (role == 0 && a.run_tab != nullptr && a.idx != nullptr) {
    for (int p = tid; p < P_N; p += kPlanThreads) {
      int acc = 0;
      const int* row = a.idx + (size_t)p * S;
      RunEntry* tab = a.run_tab + (size_t)p * S;
#pragma unroll 8
      for (int r = 0; r < S; ++r) {
        const int q = row[r];
        const int o = s_offM[q], n = s_offM[q + 1] - o;
        tab[r] = RunEntry{acc + n, o - acc};
        acc += n;
      }
    }
    __syncthreads();
  }
  // ---- inverse selection lists: inv[q] = target patches p with q in idx[p],
  // ascending, and their run tables
  if (role == 1) {
    block_scan_excl(P_M, [&](int q) { return s_cur[q]; }, a.inv_off, lds);
    // a repeat within a row stops the pass before its chunk is placed (two
    // copies of an entry would advance their list twice)
    __shared__ int s_rep;
    if (tid == 0) s_rep = 0;
    for (int q = tid; q < P_M; q += kPlanThreads) {
      s_cur[q] = a.inv_off[q];
      s_offM[q] = 0;
    }
    __syncthreads();
    // Chunk c: phase A sets its bits in mask array c & 1 (a bit already set is a
    // repeat) and advances the lists by chunk c - 1; phase B places its
    // entries and clears the bits of chunk c - 1.
    unsigned* const buf0 = s_mask;
    unsigned* const buf1 = reinterpret_cast<unsigned*>(s_offM);
    int qc[kChunkRegs], qp[kChunkRegs], qn[kChunkRegs];
    load_chunk(a.idx, 0, chunk_end(0), qc);
    int o_lo = 0, o_hi = 0;  // offN[p0 + tid], offN[p0 + tid + 1] of the next chunk
    if (tid < kPlanRows && tid < P_N) {
      o_lo = offN[tid];
      o_hi = offN[tid + 1];
    }
    for (int c = 0; c < nC; ++c) {
      const int p0 = c * kPlanRows, e0 = p0 * S, e1 = chunk_end(c), cb = c & 1;
      const int* szN = s_szN[cb];
      const int* sofN = s_offN[cb];
      // phase A
      if (tid < kPlanRows) {
        s_offN[cb][tid] = o_lo;
        s_szN[cb][tid] = o_hi - o_lo;
      }
      if (c + 1 < nC) {
        load_chunk(a.idx, e1, chunk_end(c + 1), qn);
        if (tid < kPlanRows && p0 + kPlanRows + tid < P_N) {
          o_lo = offN[p0 + kPlanRows + tid];
          o_hi = offN[p0 + kPlanRows + tid + 1];
        }
      }
      if (c > 0) {
        // the last patch of chunk c - 1 selecting q advances list q
        const unsigned* prev = cb ? buf0 : buf1;
        const int* szP = s_szN[cb ^ 1];
        for_chunk(a.idx, e0 - kPlanRows * S, e0, qp, [&](int e, int q) {
          const int j = e / S - (p0 - kPlanRows);
          const unsigned m = prev[q];
          if (31 - __clz(m) == j) {
            int add = 0;
            for (unsigned b = m; b; b &= b - 1u) add += szP[__ffs(b) - 1];
            s_cur[q] += __popc(m);
            s_acc[q] += add;
          }
        });
      }
      unsigned* cur = cb ? buf1 : buf0;
      for_chunk(a.idx, e0, e1, qc, [&](int e, int q) {
        const unsigned bit = 1u << (e / S - p0);
        if (atomicOr(&cur[q], bit) & bit) s_rep = 1;
      });
      __syncthreads();
      if (s_rep) break;
      // phase B
      for_chunk(a.idx, e0, e1, qc, [&](int e, int q) {
        const int j = e / S - p0;
        unsigned below = cur[q] & ((1u << j) - 1u);
        const int slot = s_cur[q] + __popc(below);
        int pre = s_acc[q];
        while (below) {
          pre += szN[__ffs(below) - 1];
          below &= below - 1u;
        }
        a.inv_idx[slot] = p0 + j;
        if (a.inv_tab != nullptr) a.inv_tab[slot] = RunEntry{pre + szN[j], sofN[j] - pre};
      });
      if (c > 0) {
        unsigned* prev = cb ? buf0 : buf1;
        for_chunk(a.idx, e0 - kPlanRows * S, e0, qp, [&](int, int q) { prev[q] = 0u; });
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kChunkRegs; ++r) {
        qp[r] = qc[r];
        qc[r] = qn[r];
      }
    }
    // a repeated entry: nothing is published
    if (s_rep) {
      fail();
      return;
    }
  }
  // ---- work items (row blocks of rowsQ / rowsK rows within a patch)
  __shared__ int s_misc[2];
  // [3 (max(P_N, P_M) + 1)] per role
  int* tmp = a.scratch + (size_t)role * 3 * ((P_N > P_M ? P_N : P_M) + 1);
  const RunEntry* rt = a.run_tab;
  const int* io = a.inv_off;
  const RunEntry* it = a.inv_tab;
  auto tilesQ = [=](int p) { return rt != nullptr ? (rt[(size_t)p * S + S - 1].end + kTile - 1) / kTile : 0; };
  int* s_tl = reinterpret_cast<int*>(s_mask);  // free after the selection passes
  const int nQ = role == 0 ? make_items(P_N, offN, a.rowsQ, tilesQ, a.itemsQ, rt != nullptr ? a.splitQ : nullptr,
                                        a.counters + 5, tmp, lds, s_acc, s_misc, s_tl, s_cur)
                           : 0;
  auto tilesK = [=](int q) {
    if (it == nullptr) return 0;
    const int b = io[q], e = io[q + 1];
    return e > b ? (it[e - 1].end + kTile - 1) / kTile : 0;
  };
  // source-side items drive only the dK/dV pass (a plan with inverse lists)
  const bool items_k = inverse ? role == 1 : io != nullptr || rt == nullptr;
  const int nK = items_k ? make_items(P_M, offM, a.rowsK, tilesK, a.itemsK, it != nullptr ? a.splitK : nullptr,
                                      a.counters + 6, tmp, lds, s_acc, s_misc, s_tl, s_cur)
                         : 0;
  if (!inverse && io == nullptr && rt != nullptr && tid == 0) a.counters[6] = 0;
  if (tid == 0) {
    if (role == 0) {
      a.counters[0] = nQ;
      a.counters[2] = gN / kGroup;
      a.counters[3] = gM / kGroup;
      a.counters[4] = 0;
    }
    if (role == 1 || !inverse) a.counters[1] = nK;
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) { plan_body(a, blockIdx.x); }

// The plan (workgroups 0 .. nplan - 1) and up to two bf16 row-padding jobs
// in one launch: the other workgroups take four 16-row blocks each (one per
// 256 threads), so the padding runs on the other CUs while the plan's
// workgroups run.  The jobs do not read what the plan writes.
__global__ __launch_bounds__(kPlanThreads) void plan_pad_kernel(PlanArgs a, int nplan, PackArgs p0, int g0, int vec0,
                                                               PackArgs p1, int g1, int vec1) {
  if ((int)blockIdx.x < nplan) {
    plan_body(a, blockIdx.x);
    return;
  }
  const int vb = ((int)blockIdx.x - nplan) * (kPlanThreads / 256) + (int)threadIdx.x / 256;
  const int vt = (int)threadIdx.x & 255;
  if (vb < g0) {
    if (vec0) pad_rows<true>(p0, vb, vt);
    else pad_rows<false>(p0, vb, vt);
  } else if (vb - g0 < g1) {
    if (vec1) pad_rows<true>(p1, vb - g0, vt);
    else pad_rows<false>(p1, vb - g0, vt);
  }
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  const bool inverse = a.inv_off != nullptr && a.idx != nullptr;
  hipLaunchKernelGGL(plan_kernel, dim3(inverse ? 2 : 1), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_plan_pad(const PlanArgs& a, const PackArgs* jobs, const int* grids, int njobs, hipStream_t st) {
  if (njobs < 0 || njobs > 2) return hipErrorInvalidValue;
  const bool inverse = a.inv_off != nullptr && a.idx != nullptr;
  const int nplan = inverse ? 2 : 1;
  PackArgs p[2]{};
  int g[2] = {0, 0}, vec[2] = {0, 0};
  for (int i = 0; i < njobs; ++i) {
    if (!pad_bf16_applies(DType::BF16, jobs[i])) return hipErrorInvalidValue;
    p[i] = jobs[i];
    g[i] = grids[i] > 0 ? grids[i] : 0;
    vec[i] = pad_bf16_vec(jobs[i]) ? 1 : 0;
  }
  const int per = kPlanThreads / 256;
  const int nb = nplan + (g[0] + g[1] + per - 1) / per;
  hipLaunchKernelGGL(plan_pad_kernel, dim3(nb), dim3(kPlanThreads), 0, st, a, nplan, p[0], g[0], vec[0], p[1], g[1],
                     vec[1]);
  return hipGetLastError();
}

// Offsets rule check for the debug build's patch scoring: workgroup 0 checks
// offN, workgroup 1 offM; either sets *flag on a violation.  The flag is
// cleared by a one-thread kernel launched before it on the same stream.
__global__ __launch_bounds__(256) void check_offsets_kernel(const int* offN, int P_N, int n_N, const int* offM,
                                                            int P_M, int n_M, int* flag) {
  const int* off = blockIdx.x == 0 ? offN : offM;
  const int P = blockIdx.x == 0 ? P_N : P_M, n = blockIdx.x == 0 ? n_N : n_M;
  int bad = 0;
  if (threadIdx.x == 0) bad = off[0] != 0 || off[P] != n;
  for (int p = threadIdx.x; p < P; p += blockDim.x) bad |= off[p] > off[p + 1];
  if (__syncthreads_or(bad) && threadIdx.x == 0) atomicOr(flag, 1);
}

__global__ void clear_flag_kernel(int* flag) { *flag = 0; }

// One patch per side selecting the other, each array 16-byte aligned:
// offN = p[0..1] = {0, n_N}, offM = p[4..5] = {0, n_M}, idx = p[8] = {0}
// (a dense coupling run through the geo kernels).
__global__ void one_patch_kernel(int* p, int n_N, int n_M) {
  const int t = threadIdx.x;
  if (t < 12) p[t] = t == 1 ? n_N : t == 5 ? n_M : 0;
}

hipError_t launch_one_patch(int* p, int n_N, int n_M, hipStream_t st) {
  hipLaunchKernelGGL(one_patch_kernel, dim3(1), dim3(64), 0, st, p, n_N, n_M);
  return hipGetLastError();
}

hipError_t launch_check_offsets(const int* offN, int P_N, int n_N, const int* offM, int P_M, int n_M, int* flag,
                                hipStream_t st) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, st, flag);
  hipLaunchKernelGGL(check_offsets_kernel, dim3(2), dim3(256), 0, st, offN, P_N, n_N, offM, P_M, n_M, flag);
  return hipGetLastError();
}

// Outputs of a rejected geo plan (fp32 path): quiet NaN, so that a result
// computed from invalid offsets or an invalid selection cannot pass for one.
__global__ __launch_bounds__(256) void invalid_fill_kernel(const int* status, float* x0, size_t n0, float* x1,
                                                           size_t n1, float* x2, size_t n2) {
  if (*status == 0) return;
  const size_t stride = (size_t)gridDim.x * blockDim.x, g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const float q = __builtin_nanf("");
  if (x0 != nullptr)
    for (size_t i = g; i < n0; i += stride) x0[i] = q;
  if (x1 != nullptr)
    for (size_t i = g; i < n1; i += stride) x1[i] = q;
  if (x2 != nullptr)
    for (size_t i = g; i < n2; i += stride) x2[i] = q;
}

hipError_t launch_invalid_fill(const int* status, float* x0, size_t n0, float* x1, size_t n1, float* x2, size_t n2,
                               hipStream_t st) {
  hipLaunchKernelGGL(invalid_fill_kernel, dim3(256), dim3(256), 0, st, status, x0, n0, x1, n1, x2, n2);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// patch pooling (fp64 sums, then the mean)
// ---------------------------------------------------------------------------
// One workgroup per patch.  Thread t owns the column pair t % (d/2) and the
// row phase t / (d/2): it sums rows begin + phase, begin + phase + NPH, ...
// in fp64, and the NPH phase sums are then added in phase order.  The order
// is fixed, so the result is deterministic.  Every partial sum is exact in
// fp64 (hence equal to the sum in any order, row order included) when it
// needs at most 53 significant bits: with p significant bits per entry (8
// for bf16, 24 for fp32), at most 2^12 rows and nonzero magnitudes within a
// factor 2^r of each other, a sum spans p + r + 12 bits, so r <= 33 (bf16)
// or r <= 17 (fp32) with rows <= 4096.
// bf16 rows (16-byte aligned, d in {64, 128}): thread t owns the 8-column
// chunk t % (d/8) and the row phase t / (d/8) (16 or 32 phases), one 16-byte
// load per row; same fixed phase order, same exactness.
__global__ __launch_bounds__(256) void pool_bf16_kernel(PoolArgs a) {
  __shared__ double part[256][8];
  const int b = blockIdx.x, tid = threadIdx.x;
  const bool tgt = b < a.P_N;
  const int p = tgt ? b : b - a.P_N;
  const int* off = tgt ? a.offN : a.offM;
  const int n = tgt ? a.n_N : a.n_M;
  const bf16* X = reinterpret_cast<const bf16*>(tgt ? a.Q : a.K);
  const int begin = min(max(off[p], 0), n);
  const int end = min(max(off[p + 1], begin), n);
  const int cnt = end - begin;
  const int nch = a.d / 8, nph = 256 / nch;
  const int ch = tid % nch, ph = tid / nch;
  double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int r = begin + ph; r < end; r += nph) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(X + (size_t)r * a.d + 8 * ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += (double)(float)v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[tid][e] = s[e];
  __syncthreads();
  if (tid < a.d) {
    const int c = tid, cc = c / 8, e = c % 8;
    double t = 0.0;
    for (int q = 0; q < nph; ++q) t += part[q * nch + cc][e];
    const double m = cnt > 0 ? t / (double)cnt : 0.0;
    if (tgt) a.Qbar[(size_t)p * a.d + c] = m;
    else a.KbarT[(size_t)c * a.P_M + p] = m;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(PoolArgs a) {
  __shared__ double part[256][2];
  const int b = blockIdx.x, tid = threadIdx.x;
  const bool tgt = b < a.P_N;
  const int p = tgt ? b : b - a.P_N;
  const int* off = tgt ? a.offN : a.offM;
  const int n = tgt ? a.n_N : a.n_M;
  const T* X = reinterpret_cast<const T*>(tgt ? a.Q : a.K);
  const int begin = min(max(off[p], 0), n);
  const int end = min(max(off[p + 1], begin), n);
  const int cnt = end - begin;
  const int npairs = a.d / 2, nph = 256 / npairs;  // d in {64, 128}: 4 or 8 phases
  const int cp = tid % npairs, ph = tid / npairs;
  double s0 = 0.0, s1 = 0.0;
  if (ph < nph) {
    for (int r = begin + ph; r < end; r += nph) {
      const T* x = X + (size_t)r * a.d + 2 * cp;
      s0 += (double)to_f32(x[0]);
      s1 += (double)to_f32(x[1]);
    }
  }
  part[tid][0] = s0;
  part[tid][1] = s1;
  __syncthreads();
  if (tid < npairs) {
    double t0 = 0.0, t1 = 0.0;
    for (int q = 0; q < nph; ++q) {
      t0 += part[q * npairs + tid][0];
      t1 += part[q * npairs + tid][1];
    }
    const double m0 = cnt > 0 ? t0 / (double)cnt : 0.0, m1 = cnt > 0 ? t1 / (double)cnt : 0.0;
    const int c = 2 * tid;
    if (tgt) {
      a.Qbar[(size_t)p * a.d + c] = m0;
      a.Qbar[(size_t)p * a.d + c + 1] = m1;
    } else {
      a.KbarT[(size_t)c * a.P_M + p] = m0;
      a.KbarT[(size_t)(c + 1) * a.P_M + p] = m1;
    }
  }
}

hipError_t launch_pool(DType t, const PoolArgs& a, hipStream_t st) {
  const int grid = a.P_N + a.P_M;
  if (t == DType::BF16 && (reinterpret_cast<uintptr_t>(a.Q) & 15) == 0 && (reinterpret_cast<uintptr_t>(a.K) & 15) == 0 &&
      (a.d == 64 || a.d == 128))
    hipLaunchKernelGGL(pool_bf16_kernel, dim3(grid), dim3(256), 0, st, a);
  else if (t == DType::BF16) hipLaunchKernelGGL(pool_kernel<bf16>, dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(pool_kernel<float>, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scores and top-s (one workgroup per target patch, the score row in LDS)
// ---------------------------------------------------------------------------
constexpr int kMaxD = 128;

// The score row lives in LDS: statically sized for the largest P_M, or
// (SMALL) for at most kSmallPatches, which leaves room for more workgroups
// per CU.
constexpr int kSmallPatches = 2048;

// s up to kGroupTop and at least kGroupMinCands candidates: the ranking first
// keeps each 64-candidate group's top s (measured: 112 -> 76 us for the 640
// patches of 160k vertices; slower for 256, which counts directly)
constexpr int kGroupTop = 32;
constexpr int kGroupMinCands = 512;

template <bool SMALL>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  constexpr int CAP = SMALL ? kSmallPatches : kMaxPatches;
  constexpr int WCAP = (CAP + 63) / 64 * kGroupTop;  // group winners
  __shared__ double qb[kMaxD];
  __shared__ double C[CAP];
  __shared__ double winv[WCAP];
  __shared__ int win[WCAP];
  __shared__ int nwin;
  const int p = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) nwin = 0;
  for (int c = tid; c < a.d; c += 256) qb[c] = a.Qbar[(size_t)p * a.d + c];
  __syncthreads();
  for (int q = tid; q < a.P_M; q += 256) {
    // d is a multiple of 16 (64 or 128): unrolled so that the independent
    // column loads are in flight together
    double acc = 0.0;
    const double* kt = a.KbarT + q;
    for (int c0 = 0; c0 < a.d; c0 += 16) {
      double kv[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) kv[c] = kt[(size_t)(c0 + c) * a.P_M];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = fma(qb[c0 + c], kv[c], acc);
    }
    C[q] = acc;
    if (a.scores != nullptr) a.scores[(size_t)p * a.P_M + q] = acc;
  }
  __syncthreads();
  // rank of q in the strict order (score desc, index asc)
  if (a.s <= kGroupTop && a.P_M >= kGroupMinCands) {
    // Two stages.  A candidate's rank within its group of 64 (the
    // candidates a wave holds in one pass) is at most its rank overall, so
    // the top s overall are among the groups' top s; and every candidate
    // ahead of a top-s candidate is itself in the top s, so ranking the
    // group winners against each other gives their exact overall ranks.
    for (int base = 0; base < a.P_M; base += 256) {
      const int q = base + tid, w0 = base + (tid & ~63);
      const int wn = min(64, a.P_M - w0);  // (wave-uniform)
      if (q < a.P_M) {
        const double v = C[q];
        int rank = 0;
#pragma unroll 8
        for (int j = 0; j < wn; ++j) {
          const double v2 = C[w0 + j];
          rank += (v2 > v) || (v2 == v && w0 + j < q);
        }
        if (rank < a.s) {
          const int slot = atomicAdd(&nwin, 1);
          win[slot] = q;
          winv[slot] = v;
        }
      }
    }
    __syncthreads();
    const int nw = nwin;
    for (int i = tid; i < nw; i += 256) {
      const int q = win[i];
      const double v = winv[i];
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < nw; ++j) {
        const double v2 = winv[j];
        rank += (v2 > v) || (v2 == v && win[j] < q);
      }
      if (rank < a.s) a.idx[(size_t)p * a.s + rank] = q;
    }
    return;
  }
  for (int q = tid; q < a.P_M; q += 256) {
    const double v = C[q];
    int rank = 0;
    for (int q2 = 0; q2 < a.P_M; ++q2) {
      const double v2 = C[q2];
      rank += (v2 > v) || (v2 == v && q2 < q);
    }
    if (rank < a.s) a.idx[(size_t)p * a.s + rank] = q;
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.P_M <= kSmallPatches) hipLaunchKernelGGL(topk_kernel<true>, dim3(a.P_N), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(topk_kernel<false>, dim3(a.P_N), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssc
