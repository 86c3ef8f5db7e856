// Geodesic farthest-point-sampling partition on gfx950.  Geo-FlashAttention
// partitions each surface into patches by geodesic farthest-point sampling
// (project page "Spatial-Spectral Coupling as Attention", sections
// "Abstract" and "Geo-FlashAttention"):
//
//   * geodesic distance: shortest path on the mesh's edge graph, an edge
//     weighing its Euclidean length sqrt((dx^2 + dy^2) + dz^2) in fp64;
//   * seed 0 is vertex 0; seed t is the vertex farthest from the seeds
//     chosen before it (ties to the lower vertex index);
//   * every vertex is labelled with its nearest seed (ties to the earlier
//     seed).
//
//   fps_prep  -- checks the adjacency (offsets and neighbour indices), edge
//                lengths with explicitly rounded fp64 operations (no fused
//                multiply-add), a padded copy of the adjacency (kFpsSlots
//                neighbours and lengths per vertex, used when no vertex has
//                more), and the initial state (distance +inf, label 0,
//                chunk maxima +inf);
//   fps_run   -- one workgroup of 1024 threads runs all P steps.  Step t
//                relaxes outward from seed t with a frontier worklist (the
//                first kLdsQueue entries of a round's queue sit in LDS; a
//                vertex is queued once per round, which an LDS bitmap per
//                round tracks up to kSeenBits vertices, per-vertex round
//                stamps in the workspace beyond): a
//                vertex's distance is lowered by a 64-bit atomic minimum on
//                its bit pattern (non-negative doubles order like their
//                bits) only when the path through seed t is strictly
//                shorter, which also relabels it t and queues it for the
//                next round; a vertex that seed t does not bring strictly
//                closer stops the wave there (its neighbours cannot gain
//                either: the distance field satisfies the triangle
//                inequality in fp64 because rounding is monotone).  The
//                converged field equals the shortest-path sums along the
//                paths, as a Dijkstra run would form them.  The next seed is
//                the argmax over per-chunk maxima (256 vertices a chunk,
//                recomputed only for chunks the step touched).
// dist is read only through device-coherent atomic loads, so no stale cache
// line is ever used after an atomic update made in L2.
#include "common.hpp"
#include "kernels.hpp"

namespace ssc {
namespace fps {

constexpr int kThreads = 1024;
constexpr int kChunk = 256;  // vertices per argmax chunk
constexpr int kGroup = 8;    // lanes per frontier vertex (one per neighbour)
static_assert(kGroup == kFpsSlots, "a lane per padded neighbour slot");
constexpr int kLdsQueue = 8192;  // queue entries of a round held in LDS (the rest in the workspace)
constexpr int kSeenWords = 8192;  // words of each of the two "queued this round" bitmaps
constexpr int kSeenBits = 32 * kSeenWords;
typedef unsigned long long u64;
constexpr u64 kInfBits = 0x7FF0000000000000ull;

__device__ __forceinline__ u64 umax(u64 a, u64 b) { return a > b ? a : b; }

__device__ __forceinline__ u64 load_bits(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Each operation rounded on its own (no fused multiply-add), as the
// definition sums the squares.
__device__ __forceinline__ double edge_len(const double* x, int u, int v) {
#pragma clang fp contract(off)
  const double dx = x[3 * u] - x[3 * v];
  const double dy = x[3 * u + 1] - x[3 * v + 1];
  const double dz = x[3 * u + 2] - x[3 * v + 2];
  const double xx = dx * dx, yy = dy * dy, zz = dz * dz;
  return sqrt((xx + yy) + zz);
}

// One thread per vertex: validation, edge lengths, padded adjacency,
// initial state.  Bit 0 of bad[b]: block b saw an invalid offset or
// neighbour; bit 1: a vertex of block b has more than kFpsSlots neighbours.
__global__ __launch_bounds__(256) void fps_prep(FpsArgs a) {
  const int u = blockIdx.x * 256 + threadIdx.x;
  int bad = 0;
  if (u < a.n) {
    const int o0 = a.off[u], o1 = a.off[u + 1];
    if ((u == 0 && o0 != 0) || (u == a.n - 1 && o1 != a.nnz) || o0 < 0 || o1 < o0 || o1 > a.nnz) {
      bad = 1;
    } else {
      if (o1 - o0 > kFpsSlots) bad = 2;
      for (int e = o0; e < o1; ++e) {
        const int v = a.adj[e];
        if (v < 0 || v >= a.n) {
          bad = 1;
        } else {
          const double len = edge_len(a.x, u, v);
          a.w[e] = len;
          if (e - o0 < kFpsSlots) a.wp[(size_t)u * kFpsSlots + (e - o0)] = len;
        }
      }
#pragma unroll
      for (int j = 0; j < kFpsSlots; ++j)
        a.adjp[(size_t)u * kFpsSlots + j] = j < o1 - o0 ? a.adj[o0 + j] : -1;
    }
    reinterpret_cast<u64*>(a.dist)[u] = kInfBits;
    a.labels[u] = 0;
    a.stamp[u] = -1;
  }
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < a.nchunk) {
    a.cmax[c] = kInfBits;
    a.cflag[c] = 0;
  }
  const int b0 = __syncthreads_or(bad & 1), b1 = __syncthreads_or(bad & 2);
  if (threadIdx.x == 0) a.bad[blockIdx.x] = (b0 ? 1 : 0) | (b1 ? 2 : 0);
}

// Maximum of (bits, index) pairs: larger bits, then lower index.
__device__ __forceinline__ void better(u64& b, int& i, u64 b2, int i2) {
  if (b2 > b || (b2 == b && i2 < i)) {
    b = b2;
    i = i2;
  }
}

__global__ __launch_bounds__(kThreads) void fps_run(FpsArgs a) {
  __shared__ int s_queue[2][kLdsQueue];  // entries i < kLdsQueue of the two rounds' queues
  // bit v of s_seen[b]: v sits in the queue of a round r with r & 1 == b
  // (meshes of at most kSeenBits vertices)
  __shared__ unsigned s_seen[2][kSeenWords];
  __shared__ int s_cnt[3];
  __shared__ int s_flag;
  __shared__ int s_seed;
  __shared__ u64 s_wb[kThreads / 64];
  __shared__ int s_wi[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n;
  u64* dbits = reinterpret_cast<u64*>(a.dist);

  if (tid == 0) {
    s_flag = 0;
    s_cnt[0] = s_cnt[1] = s_cnt[2] = 0;
  }
  const bool lds_seen = n <= kSeenBits;
  for (int i = tid; i < 2 * kSeenWords; i += kThreads) (&s_seen[0][0])[i] = 0u;
  __syncthreads();
  int wide = 0;  // some vertex has more than kFpsSlots neighbours
  for (int b = tid; b < a.nblk; b += kThreads) {
    const int f = a.bad[b];
    if (f & 1) s_flag = 1;
    wide |= f & 2;
  }
  const bool padded = !__syncthreads_or(wide);
  if (s_flag) {  // invalid adjacency: nothing is computed
    for (int t = tid; t < a.P; t += kThreads) a.seeds[t] = -1;
    for (int v = tid; v < n; v += kThreads) {
      a.labels[v] = -1;
      dbits[v] = 0x7FF8000000000000ull;  // NaN
    }
    return;
  }

  // A step needs at most n rounds: shortest paths are simple (weights are
  // non-negative and rounding is monotone), and after round h every vertex
  // whose best path has h edges is final.  A step past n + 1 rounds would be
  // a fault of this code; it ends the run with seeds[t] = -2.
  int r = 0;                       // rounds run so far (uniform)
  int seed = 0;
  for (int t = 0; t < a.P; ++t) {
    // seed t starts the queue of round r
    if (tid == 0) {
      a.seeds[t] = seed;
      int c0 = 0;
      if (load_bits(dbits + seed) > 0ull) {
        atomicMin(dbits + seed, 0ull);
        a.labels[seed] = t;
        a.cflag[seed / kChunk] = 1;
        a.stamp[seed] = r;
        s_queue[r & 1][0] = seed;
        c0 = 1;
      }
      s_seed = c0;
    }
    __syncthreads();
    int cnt = s_seed;
    int rstep = 0;
    while (cnt > 0 && rstep <= n) {
      // queue entry i of a round: LDS below kLdsQueue, the workspace above
      // (a round queues each vertex at most once, so i < n)
      const int* qin_l = s_queue[r & 1];
      int* qout_l = s_queue[(r + 1) & 1];
      const int* qin = a.queue + (size_t)(r & 1) * n;
      int* qout = a.queue + (size_t)((r + 1) & 1) * n;
      int* ctr = &s_cnt[r % 3];
      if (tid == 0) s_cnt[(r + 1) % 3] = 0;  // last read two rounds ago
      const int stamp_next = r + 1;
      for (int base = 0; base < cnt; base += kThreads / kGroup) {
        const int q = base + tid / kGroup, j = tid % kGroup;
        if (q < cnt) {
          const int u = q < kLdsQueue ? qin_l[q] : qin[q];
          // u leaves this round's bitmap (which the next round but one reuses)
          if (lds_seen && j == 0) atomicAnd(&s_seen[r & 1][u >> 5], ~(1u << (u & 31)));
          const double du = __longlong_as_double((long long)load_bits(dbits + u));
          // the padded adjacency: lane j takes neighbour slot j (kGroup ==
          // kFpsSlots), read together with du; else the CSR rows
          int e = 0, o1 = 0, v = -1;
          double wuv = 0.0;
          if (padded) {
            v = a.adjp[(size_t)u * kFpsSlots + j];
            wuv = a.wp[(size_t)u * kFpsSlots + j];
          } else {
            e = a.off[u] + j;
            o1 = a.off[u + 1];
          }
          for (;;) {
            if (!padded) {
              if (e >= o1) break;
              v = a.adj[e];
              wuv = a.w[e];
              e += kGroup;
            } else if (v < 0) {
              break;
            }
            const double cand = du + wuv;
            const u64 cb = (u64)__double_as_longlong(cand);
            const u64 old = atomicMin(dbits + v, cb);
            if (cb < old) {
              a.labels[v] = t;
              a.cflag[v / kChunk] = 1;
              bool first;
              if (lds_seen) {
                const unsigned bit = 1u << (v & 31);
                first = (atomicOr(&s_seen[(r + 1) & 1][v >> 5], bit) & bit) == 0u;
              } else {
                first = atomicExch(a.stamp + v, stamp_next) != stamp_next;
              }
              if (first) {
                const int i = atomicAdd(ctr, 1);
                if (i < kLdsQueue) qout_l[i] = v;
                else qout[i] = v;
              }
            }
            if (padded) break;
          }
        }
      }
      __syncthreads();
      cnt = *ctr;
      ++r;
      ++rstep;
    }
    if (cnt > 0) {
      if (tid == 0) a.seeds[t] = -2;
      return;
    }
    if (t + 1 == a.P) break;

    // chunk maxima of the chunks this step touched: wave w owns the chunks
    // c = w (mod 16); a lane reads the flag of one of them, so a wave finds
    // its flagged chunks with one load and a ballot per 64 of them
    constexpr int kWaves = kThreads / 64;
    for (int c0 = wave; c0 < a.nchunk; c0 += 64 * kWaves) {
      const int cl = c0 + kWaves * lane;
      unsigned long long fl = __ballot(cl < a.nchunk && a.cflag[cl] != 0);
      while (fl != 0ull) {
        const int b = __ffsll((long long)fl) - 1;
        fl &= fl - 1ull;
        const int c = c0 + kWaves * b;
        u64 m = 0;
#pragma unroll
        for (int j = 0; j < kChunk / 64; ++j) {
          const int v = c * kChunk + j * 64 + lane;
          if (v < n) m = umax(m, load_bits(dbits + v));
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = umax(m, (u64)__shfl_xor(m, o, 64));
        if (lane == 0) {
          a.cmax[c] = m;
          a.cflag[c] = 0;
        }
      }
    }
    __syncthreads();
    // the largest chunk maximum, lowest chunk on ties
    u64 bb = 0;
    int bi = 0x7fffffff;
    for (int c = tid; c < a.nchunk; c += kThreads) better(bb, bi, a.cmax[c], c);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const u64 b2 = __shfl_xor(bb, o, 64);
      const int i2 = __shfl_xor(bi, o, 64);
      better(bb, bi, b2, i2);
    }
    if (lane == 0) {
      s_wb[wave] = bb;
      s_wi[wave] = bi;
    }
    __syncthreads();
    if (wave == 0) {
      bb = lane < kThreads / 64 ? s_wb[lane] : 0;
      bi = lane < kThreads / 64 ? s_wi[lane] : 0x7fffffff;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const u64 b2 = __shfl_xor(bb, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        better(bb, bi, b2, i2);
      }
      // lowest vertex of that chunk holding the maximum
      int found = -1;
#pragma unroll
      for (int j = 0; j < kChunk / 64; ++j) {
        const int v = bi * kChunk + j * 64 + lane;
        const bool hit = v < n && load_bits(dbits + v) == bb;
        const unsigned long long mask = __ballot(hit);
        if (found < 0 && mask != 0ull) found = bi * kChunk + j * 64 + (__ffsll((long long)mask) - 1);
      }
      if (lane == 0) s_seed = found;
    }
    __syncthreads();
    seed = s_seed;
  }
}

}  // namespace fps

hipError_t launch_fps(const FpsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(fps::fps_prep, dim3(a.nblk), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fps::fps_run, dim3(1), dim3(fps::kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssc
