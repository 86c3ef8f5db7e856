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
//   fps_wide  -- (meshes of kFpsWideMin vertices or more with the padded
//                adjacency) the first steps, whose cells cover much of the
//                mesh, on a grid of resident workgroups: the same rounds,
//                separated by a grid barrier whose wait is bounded, until a
//                step's largest round queue stays below a threshold; a wait
//                that runs out sets an abort flag and the workgroups leave,
//                and fps_run then redoes every step from the initial state;
//   fps_run   -- one workgroup of 1024 threads runs the remaining steps (all
//                P steps when fps_wide did not run).  Step t
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
  if (blockIdx.x == 0 && threadIdx.x < (int)(sizeof(FpsCtl) / 4)) reinterpret_cast<int*>(a.ctl)[threadIdx.x] = 0;
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

// ---------------------------------------------------------------------------
// The first steps on many workgroups.

constexpr int kWideThreads = 1024;
constexpr int kWideGroups = kWideThreads / kGroup;  // frontier vertices a workgroup takes per pass

// Grid barrier over the workgroups of a cooperative launch.  Every wave
// waits for its own memory operations; then thread 0 alone publishes the
// workgroup's writes device-wide (the fence writes back the whole L2, so one
// per workgroup serves every wave), arrives, polls the arrival count (at
// most `spin` polls, fewer once another workgroup has given up; spin = 0
// gives up at once) and discards stale cache lines, which the workgroup's
// waves share.  Returns false when this workgroup gave up; it has set the
// abort flag then.
__device__ bool grid_sync(FpsCtl* ctl, unsigned long long& epoch, unsigned spin, int* s_ok) {
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all 0
  __syncthreads();
  epoch += 1;
  if (threadIdx.x == 0) {
    const unsigned long long target = epoch * gridDim.x;
    __threadfence();
    __hip_atomic_fetch_add(&ctl->bar, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = spin > 0 ? 1 : 0;
    unsigned polls = 0;
    while (ok && __hip_atomic_load(&ctl->bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(&ctl->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0 || ++polls > spin) ok = 0;
      else __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) __hip_atomic_store(&ctl->abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// Steps 0, 1, ... as in fps_run (at most a.wide_steps of them, ending after
// the first step whose largest round queue stays below a.wide_frontier), a
// round's queue spread over the workgroups (kWideGroups entries each per
// pass) and the rounds separated by grid_sync.  A vertex is queued once per round through its round stamp; a
// wave reserves the queue slots of its new entries with one atomic add.
// The first round of a step has the seed as its only entry, which
// workgroup 0 both places and takes, so a step needs no barrier of its own.
// After a step every workgroup recomputes its share of the touched chunks'
// maxima, and after one more barrier each finds the same next seed.
__global__ __launch_bounds__(kWideThreads) void fps_wide(FpsArgs a) {
  __shared__ int s_ok, s_seed;
  __shared__ u64 s_wb[kWideThreads / 64];
  __shared__ int s_wi[kWideThreads / 64];
  FpsCtl* ctl = a.ctl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.n;
  u64* dbits = reinterpret_cast<u64*>(a.dist);

  // every workgroup reads the same flags, so all leave here or none: an
  // invalid adjacency is left to fps_run, and so are meshes without the
  // padded adjacency
  int flags = 0;
  for (int b = tid; b < a.nblk; b += kWideThreads) flags |= a.bad[b];
  if (__syncthreads_or(flags) != 0) return;

  unsigned long long epoch = 0;
  int r = 0, done = 0;
  // the seed (known to workgroup 0 only) and its distance (known to all:
  // the largest chunk maximum, +inf for seed 0)
  int seed = 0;
  u64 seed_bits = kInfBits;
  for (int t = 0; t < a.wide_steps; ++t) {
    const int cnt0 = seed_bits > 0ull ? 1 : 0;
    if (blockIdx.x == 0 && tid == 0) {
      a.seeds[t] = seed;
      if (cnt0) {
        atomicMin(dbits + seed, 0ull);
        a.labels[seed] = t;
        a.cflag[seed / kChunk] = 1;
        a.stamp[seed] = r;
        a.queue[(size_t)(r & 1) * n] = seed;
      }
    }
    __syncthreads();
    int cnt = cnt0, peak = cnt0;
    int rstep = 0;
    while (cnt > 0 && rstep <= n) {
      const int* qin = a.queue + (size_t)(r & 1) * n;
      int* qout = a.queue + (size_t)((r + 1) & 1) * n;
      int* ctr = &ctl->cnt[r % 3];
      if (blockIdx.x == 0 && tid == 0) ctl->cnt[(r + 1) % 3] = 0;  // last read two rounds ago
      const int stamp_next = r + 1;
      for (int base = blockIdx.x * kWideGroups; base < cnt; base += gridDim.x * kWideGroups) {
        const int q = base + tid / kGroup, j = tid % kGroup;
        int push = -1;
        if (q < cnt) {
          const int u = qin[q];
          const double du = __longlong_as_double((long long)load_bits(dbits + u));
          const int v = a.adjp[(size_t)u * kFpsSlots + j];
          const double wuv = a.wp[(size_t)u * kFpsSlots + j];
          if (v >= 0) {
            const u64 cb = (u64)__double_as_longlong(du + wuv);
            const u64 old = atomicMin(dbits + v, cb);
            if (cb < old) {
              a.labels[v] = t;
              a.cflag[v / kChunk] = 1;
              if (atomicExch(a.stamp + v, stamp_next) != stamp_next) push = v;
            }
          }
        }
        const u64 m = __ballot(push >= 0);
        if (m != 0ull) {
          const int leader = __ffsll((long long)m) - 1;
          int wbase = 0;
          if (lane == leader) wbase = atomicAdd(ctr, __popcll(m));
          wbase = __shfl(wbase, leader, 64);
          if (push >= 0)
            qout[wbase + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u))] =
                push;
        }
      }
      if (!grid_sync(ctl, epoch, a.spin, &s_ok)) return;
      cnt = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      peak = max(peak, cnt);
      ++r;
      ++rstep;
    }
    if (cnt > 0) {  // the round bound: a fault of this code
      if (blockIdx.x == 0 && tid == 0) {
        a.seeds[t] = -2;
        ctl->status = 2;
      }
      return;
    }
    // later steps stay here while their frontiers keep many workgroups busy
    // (the counts, hence the decision, are the same in every workgroup)
    done = t + 1;
    if (done == a.wide_steps || peak < a.wide_frontier) break;

    // maxima of the touched chunks, one chunk a wave
    for (int c = blockIdx.x * (kWideThreads / 64) + wave; c < a.nchunk; c += gridDim.x * (kWideThreads / 64)) {
      if (a.cflag[c] == 0) continue;
      u64 mx = 0;
#pragma unroll
      for (int j = 0; j < kChunk / 64; ++j) {
        const int v = c * kChunk + j * 64 + lane;
        if (v < n) mx = umax(mx, load_bits(dbits + v));
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = umax(mx, (u64)__shfl_xor(mx, o, 64));
      if (lane == 0) {
        a.cmax[c] = mx;
        a.cflag[c] = 0;
      }
    }
    if (!grid_sync(ctl, epoch, a.spin, &s_ok)) return;
    // the next seed: the largest chunk maximum (lowest chunk on ties), which
    // every workgroup finds alike, then in workgroup 0 the lowest vertex of
    // that chunk holding it (the only workgroup that reads the seed, before
    // it changes the seed's distance)
    u64 bb = 0;
    int bi = 0x7fffffff;
    for (int c = tid; c < a.nchunk; c += kWideThreads) better(bb, bi, a.cmax[c], c);
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
      bb = lane < kWideThreads / 64 ? s_wb[lane] : 0;
      bi = lane < kWideThreads / 64 ? s_wi[lane] : 0x7fffffff;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const u64 b2 = __shfl_xor(bb, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        better(bb, bi, b2, i2);
      }
      int found = -1;
      if (blockIdx.x == 0) {
#pragma unroll
        for (int j = 0; j < kChunk / 64; ++j) {
          const int v = bi * kChunk + j * 64 + lane;
          const bool hit = v < n && load_bits(dbits + v) == bb;
          const unsigned long long mask = __ballot(hit);
          if (found < 0 && mask != 0ull) found = bi * kChunk + j * 64 + (__ffsll((long long)mask) - 1);
        }
      }
      if (lane == 0) {
        s_seed = found;
        s_wb[0] = bb;
      }
    }
    __syncthreads();
    seed = s_seed;
    seed_bits = s_wb[0];
    __syncthreads();  // s_wb is rewritten at the next step's end
  }
  if (blockIdx.x == 0 && tid == 0) {
    ctl->t_end = done;
    ctl->r_end = r;
    ctl->status = 3;
  }
}

// ---------------------------------------------------------------------------
// The remaining steps on one workgroup.

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

  // The next seed: chunk maxima of the chunks the last step touched, then
  // the largest of them (lowest chunk on ties) and the lowest vertex of that
  // chunk holding it.
  auto next_seed = [&]() -> int {
    // wave w owns the chunks c = w (mod 16); a lane reads the flag of one of
    // them, so a wave finds its flagged chunks with one load and a ballot per
    // 64 of them
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
    return s_seed;
  };

  // Continue after fps_wide: from its last step when it ran its steps, from
  // the initial state, restored here, when one of its barrier waits gave up.
  int t0 = 0, r = 0;  // first step here; rounds run so far (uniform)
  if (a.ctl->abort != 0) {
    for (int v = tid; v < n; v += kThreads) {
      dbits[v] = kInfBits;
      a.labels[v] = 0;
      a.stamp[v] = -1;
    }
    for (int c = tid; c < a.nchunk; c += kThreads) {
      a.cmax[c] = kInfBits;
      a.cflag[c] = 0;
    }
    __threadfence();
    __syncthreads();
  } else if (a.ctl->status == 2) {
    return;  // fps_wide ended the run (seeds[t] = -2)
  } else if (a.ctl->status == 3) {
    t0 = a.ctl->t_end;
    r = a.ctl->r_end;
  }
  if (t0 >= a.P) return;

  // A step needs at most n rounds: shortest paths are simple (weights are
  // non-negative and rounding is monotone), and after round h every vertex
  // whose best path has h edges is final.  A step past n + 1 rounds would be
  // a fault of this code; it ends the run with seeds[t] = -2.
  int seed = t0 > 0 ? next_seed() : 0;
  for (int t = t0; t < a.P; ++t) {
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

    seed = next_seed();
  }
}

}  // namespace fps

hipError_t launch_fps(const FpsArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(fps::fps_prep, dim3(a.nblk), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.wide_steps > 0) {
    // one workgroup per CU, all resident at once (a cooperative launch
    // guarantees it or fails); if it cannot run, fps_run takes every step
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) {
      FpsArgs aw = a;
      void* args[] = {&aw};
      const int grid = std::max(1, std::min(cus, a.wide_blocks));
      if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&fps::fps_wide), dim3(grid),
                                     dim3(fps::kWideThreads), args, 0, st) != hipSuccess)
        (void)hipGetLastError();
    }
  }
  hipLaunchKernelGGL(fps::fps_run, dim3(1), dim3(fps::kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ssc
