// C ABI of the coupling library: validation, workspace layout and launches.
// Entry points and their contracts are declared in include/ssc.h.
#include "ssc.h"

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"
#include "kernels.hpp"

using namespace ssc;

namespace {

thread_local int g_last_hip = 0;

const int kKPads[] = {32, 64, 128, 224, 256};

int kpad_for(int k) {
  for (int kp : kKPads)
    if (k >= 1 && k <= kp) return kp;
  return 0;
}

// bf16 forward: V padded with at least one spare column (the ones column
// that carries the softmax row sums) unless k is the largest padded width.
int kpad_fwd_bf16(int k) { return k < kKPads[4] ? kpad_for(k + 1) : kpad_for(k); }
// bf16 backward: two spare columns when they fit (V: ones, dO: -D as bf16
// high + low parts, so the dP products yield dP - D).
int kpad_bwd_bf16(int k) { return k + 2 <= kKPads[4] ? kpad_for(k + 2) : kpad_for(k); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Buf {
  const void* p;
  size_t bytes;
};

bool overlaps(const Buf& a, const Buf& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output must be disjoint from every input and from the other outputs.
bool disjoint(std::initializer_list<Buf> outs, std::initializer_list<Buf> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Buf& i : ins)
      if (overlaps(*o, i)) return false;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlaps(*o, *o2)) return false;
  }
  return true;
}

bool all_ok(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr || !aligned16(p)) return false;
  return true;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr size_t kNone = ~size_t(0);

struct Layout {
  size_t Kp = kNone, Kg = kNone, Vp = kNone, Vg = kNone;
  size_t Qp = kNone, Qg = kNone, dOp = kNone, dOg = kNone, lse2p = kNone, Dp = kNone;
  size_t poffN = kNone, poffM = kNone, itemsQ = kNone, itemsK = kNone, counters = kNone;
  size_t inv_off = kNone, inv_idx = kNone, scratch = kNone;
  size_t Qbar = kNone, KbarT = kNone;
  size_t run_tab = kNone, inv_tab = kNone;
  size_t knorm = kNone;  // bf16 forward: partial maxima of the key-row norms
  size_t splitQ = kNone, splitK = kNone, partQ = kNone, partK = kNone;  // bf16 geo: split items, partial sums
  size_t flag = kNone;   // patch scoring: offsets verdict (read by the debug build)
  size_t Vt = kNone;     // dense bf16 forward: V grouped-transposed, npadT / 16 groups of [KP][16]
  size_t fallback = kNone;  // dense bf16 forward: per-workgroup fallback marks
  int npadT = 0;         // positions of the transposed copies (a multiple of the 64-row tile)
  size_t total = 0;
  int npadN = 0, npadM = 0;  // padded positions (upper bound for geo)
};

// bf16: only k-padded row copies of V and dO (plus rowdot / lse by row with a
// sentinel entry at index n), the geo plan, run prefix sums and inverse lists.
Layout make_layout_bf16(ssc_op op, int n_N, int n_M, int d, int k, int P_N, int P_M, int s) {
  Layout L;
  const size_t KP = (size_t)kpad_for(k);
  const bool geo = op == SSC_OP_GEO_FWD || op == SSC_OP_GEO_BWD;
  L.npadN = (int)round_up((size_t)n_N + 1, kGroup);
  L.npadM = (int)round_up((size_t)n_M + 1, kGroup);
  const size_t nN = (size_t)L.npadN, nM = (size_t)L.npadM;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  L.npadT = (int)round_up((size_t)n_M, kTile);
  switch (op) {
    case SSC_OP_DENSE_FWD:
      L.Vt = take((size_t)kpad_fwd_bf16(k) * L.npadT * 2);
      L.knorm = take(kNormParts * 4);
      L.fallback = take(((size_t)n_N + kRowsFwd - 1) / kRowsFwd * 4);
      break;
    case SSC_OP_GEO_FWD:
      L.Vp = take(nM * (size_t)kpad_fwd_bf16(k) * 2);
      L.knorm = take(kNormParts * 4);
      break;
    case SSC_OP_DENSE_BWD:
    case SSC_OP_GEO_BWD:
      L.Vp = take(nM * (size_t)kpad_bwd_bf16(k) * 2);
      L.dOp = take(nN * (size_t)kpad_bwd_bf16(k) * 2);
      L.lse2p = take(nN * 4);
      L.Dp = take(nN * 4);
      break;
    case SSC_OP_PATCH_TOPK:
      L.Qbar = take((size_t)P_N * d * 8);
      L.KbarT = take((size_t)d * P_M * 8);
      L.flag = take(4);
      break;
    default:  // the other ops have layouts of their own
      break;
  }
  if (geo) {
    const int rQ = kRowsFwd < kRowsDq ? kRowsFwd : kRowsDq, rK = kRowsDkv;
    L.poffN = take(((size_t)P_N + 1) * 4);
    L.poffM = take(((size_t)P_M + 1) * 4);
    L.itemsQ = take(((size_t)(n_N + rQ - 1) / rQ + P_N + kRoundCUs) * sizeof(Item));
    L.itemsK = take(((size_t)(n_M + rK - 1) / rK + P_M + kRoundCUs) * sizeof(Item));
    L.counters = take(8 * 4);
    L.scratch = take((op == SSC_OP_GEO_BWD ? 6 : 3) * ((size_t)(P_N > P_M ? P_N : P_M) + 1) * 4);
    L.splitQ = take(kRoundCUs * sizeof(SplitItem));
    L.splitK = take(kRoundCUs * sizeof(SplitItem));
    // partial sums of split items: kRoundCUs parts x 256 threads x fields
    const size_t T = (size_t)kRoundCUs * 256 * 4;
    if (op == SSC_OP_GEO_FWD) L.partQ = take(T * ((size_t)(kpad_fwd_bf16(k) / 32) * 16 + 2));
    if (op == SSC_OP_GEO_BWD) {
      L.partQ = take(T * ((size_t)d / 32) * 16);
      L.partK = take(T * ((size_t)d / 32 + kpad_bwd_bf16(k) / 32) * 16);
    }
    L.run_tab = take((size_t)P_N * s * sizeof(RunEntry));
    if (op == SSC_OP_GEO_BWD) {
      L.inv_off = take(((size_t)P_M + 1) * 4);
      L.inv_idx = take((size_t)P_N * s * 4);
      L.inv_tab = take((size_t)P_N * s * sizeof(RunEntry));
    }
  }
  L.total = off;
  return L;
}

Layout make_layout(ssc_op op, ssc_dtype t, int n_N, int n_M, int d, int k, int P_N, int P_M, int s) {
  if (t == SSC_BF16) return make_layout_bf16(op, n_N, n_M, d, k, P_N, P_M, s);
  Layout L;
  const size_t es = t == SSC_BF16 ? 2 : 4;
  const size_t KP = (size_t)kpad_for(k);
  const bool geo = op == SSC_OP_GEO_FWD || op == SSC_OP_GEO_BWD;
  L.npadN = (int)round_up((size_t)n_N + (geo ? (size_t)kGroup * P_N : 0), kGroup);
  L.npadM = (int)round_up((size_t)n_M + (geo ? (size_t)kGroup * P_M : 0), kGroup);
  const size_t nN = (size_t)L.npadN, nM = (size_t)L.npadM;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = round_up(off + bytes, 256);
    return o;
  };
  switch (op) {
    case SSC_OP_DENSE_FWD:
    case SSC_OP_GEO_FWD:
      L.Kp = take(nM * d * es);
      L.Vg = take(nM * KP * es);
      break;
    case SSC_OP_DENSE_BWD:
    case SSC_OP_GEO_BWD:
      L.Kp = take(nM * d * es);
      L.Kg = take(nM * d * es);
      L.Vp = take(nM * KP * es);
      L.Qp = take(nN * d * es);
      L.Qg = take(nN * d * es);
      L.dOp = take(nN * KP * es);
      L.dOg = take(nN * KP * es);
      L.lse2p = take(nN * 4);
      L.Dp = take(nN * 4);
      break;
    case SSC_OP_PATCH_TOPK:
      L.Qbar = take((size_t)P_N * d * 8);
      L.KbarT = take((size_t)d * P_M * 8);
      break;
    default:  // the other ops have layouts of their own
      break;
  }
  if (geo) {
    L.poffN = take(((size_t)P_N + 1) * 4);
    L.poffM = take(((size_t)P_M + 1) * 4);
    L.itemsQ = take(((size_t)(n_N + kRowsPerWG - 1) / kRowsPerWG + P_N) * sizeof(Item));
    L.itemsK = take(((size_t)(n_M + kRowsPerWG - 1) / kRowsPerWG + P_M) * sizeof(Item));
    L.counters = take(8 * 4);
    L.scratch = take((op == SSC_OP_GEO_BWD ? 6 : 3) * ((size_t)(P_N > P_M ? P_N : P_M) + 1) * 4);
    if (op == SSC_OP_GEO_BWD) {
      L.inv_off = take(((size_t)P_M + 1) * 4);
      L.inv_idx = take((size_t)P_N * s * 4);
    }
  }
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

ssc_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SSC_OK;
  g_last_hip = (int)e;
  return SSC_ERR_HIP;
}

#define SSC_TRY(expr)                        \
  do {                                       \
    const hipError_t e_ = (expr);            \
    if (e_ != hipSuccess) return hip_status(e_); \
  } while (0)

#ifdef SSC_DEBUG
constexpr bool kDebug = true;
#else
constexpr bool kDebug = false;
#endif

// Debug build: wait for the stream and report a device-side verdict flag
// (nonzero: a precondition the host cannot see was violated).
ssc_status debug_verdict(const int* flag, hipStream_t s) {
  int v = 0;
  SSC_TRY(hipMemcpyAsync(&v, flag, sizeof(int), hipMemcpyDeviceToHost, s));
  SSC_TRY(hipStreamSynchronize(s));
  return v != 0 ? SSC_ERR_INVALID_ARG : SSC_OK;
}

DType dt(ssc_dtype t) { return t == SSC_BF16 ? DType::BF16 : DType::F32; }

// Kernel timer: when armed for a kernel family, every launch of that family
// on this thread is bracketed by a pair of HIP events recorded on the
// launch's own stream.  Pairs are created when the timer is armed, so timed
// loops create nothing.
struct KernelTimer {
  std::string family;
  std::vector<hipEvent_t> ev;  // start/stop interleaved
  size_t used = 0;             // pairs consumed
  bool overflow = false;
};
thread_local KernelTimer g_timer;

template <typename F>
hipError_t timed(const char* family, hipStream_t s, F&& launch) {
  KernelTimer& t = g_timer;
  if (t.family.empty() || t.family != family) return launch();
  if (2 * (t.used + 1) > t.ev.size()) {
    t.overflow = true;
    return launch();
  }
  hipEvent_t a = t.ev[2 * t.used], b = t.ev[2 * t.used + 1];
  ++t.used;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  return hipEventRecord(b, s);
}

// Shape checks shared by the coupling entry points.
// Rows per side: tiles address rows with 32-bit byte offsets (rows x up to
// 512 bytes), kept below 2^31.
constexpr int kMaxRows = 1 << 22;

ssc_status check_shape(ssc_dtype t, int n_N, int n_M, int d, int k) {
  if (t != SSC_F32 && t != SSC_BF16) return SSC_ERR_INVALID_ARG;
  if (n_N < 0 || n_M < 1 || d < 1 || k < 1) return SSC_ERR_INVALID_ARG;
  const int KP = kpad_for(k);
  if (KP == 0 || !supported(dt(t), d, KP)) return SSC_ERR_UNSUPPORTED;
  if (n_N > kMaxRows || n_M > kMaxRows) return SSC_ERR_UNSUPPORTED;
  return SSC_OK;
}

ssc_status check_patches(int n_N, int P_N, int n_M, int P_M, int s) {
  if (P_N < 1 || P_M < 1 || s < 1 || s > P_M) return SSC_ERR_INVALID_ARG;
  if (P_N > 8192 || P_M > 8192) return SSC_ERR_UNSUPPORTED;
  (void)n_N;
  (void)n_M;
  return SSC_OK;
}

// Linear coupling: bf16 only, one spare padded column for the normaliser.
int kpad_lin(int k) { return kpad_for(k + 1); }

ssc_status check_linear(ssc_dtype t, int n_N, int n_M, int d, int k) {
  if (t != SSC_F32 && t != SSC_BF16) return SSC_ERR_INVALID_ARG;
  if (n_N < 0 || n_M < 1 || d < 1 || k < 1) return SSC_ERR_INVALID_ARG;
  if (t != SSC_BF16 || (d != 64 && d != 128) || kpad_lin(k) == 0) return SSC_ERR_UNSUPPORTED;
  if (n_N > kMaxRows || n_M > kMaxRows) return SSC_ERR_UNSUPPORTED;
  return SSC_OK;
}

// Performer: the linear coupling's shapes, and m in {64, 128} features.
ssc_status check_performer(ssc_dtype t, int n_N, int n_M, int d, int k, int m) {
  const ssc_status st = check_linear(t, n_N, n_M, d, k);
  if (st != SSC_OK) return st;
  if (m < 1) return SSC_ERR_INVALID_ARG;
  if (m != 64 && m != 128) return SSC_ERR_UNSUPPORTED;
  return SSC_OK;
}

struct LinLayout {
  size_t part = kNone, M = kNone, MT = kNone, dM = kNone, dMT = kNone, rden = kNone, s = kNone;
  size_t total = 0;
  int parts_M = 0, parts_N = 0;
  int gram_rows = kLinGramRows;  // rows per workgroup of the Gram sums
};

LinLayout make_lin_layout(bool bwd, int n_N, int n_M, int d, int k) {
  LinLayout L;
  const size_t KP = (size_t)kpad_lin(k);
  // The Gram workgroups (one per CU: their tiles fill most of the LDS) run
  // in one round where possible: the rows per workgroup double until the
  // forward's key blocks, or the backward's key and query blocks together,
  // number at most kRoundCUs.  Fewer workgroups also mean fewer partials.
  auto nblk = [&](int n, int rows) { return (n + rows - 1) / rows; };
  auto blocks = [&](int rows) { return nblk(n_M, rows) + (bwd ? nblk(n_N, rows) : 0); };
  while (blocks(L.gram_rows) > kRoundCUs && L.gram_rows < (1 << 22)) L.gram_rows *= 2;
  L.parts_M = nblk(n_M, L.gram_rows);
  L.parts_N = nblk(n_N, L.gram_rows);
  // the backward keeps both Gram sums' partials (one launch forms both)
  const int parts = bwd ? L.parts_M + L.parts_N : L.parts_M;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = round_up(o + bytes, 256);
    return at_;
  };
  L.part = take((size_t)parts * d * KP * 4);
  L.M = take((size_t)d * KP * 2);
  L.MT = take((size_t)d * KP * 2);
  if (bwd) {
    L.dM = take((size_t)d * KP * 2);
    L.dMT = take((size_t)d * KP * 2);
    L.rden = take((size_t)n_N * 4 + 4);
    L.s = take((size_t)n_N * 4 + 4);
  }
  L.total = o;
  return L;
}

// Performer coupling: the linear layout plus the feature buffers.
struct PfLayout {
  LinLayout lin;
  size_t part = kNone, M2 = kNone, FQ = kNone, FK = kNone, rowoff = kNone, den = kNone, dFQ = kNone,
         dFK = kNone, Mlo = kNone, MTlo = kNone, dMlo = kNone, dMTlo = kNone;
  size_t total = 0;
  int nblk_M = 0;
};

// m features per row: the linear kernels run on feature rows of width m.
PfLayout make_pf_layout(bool bwd, int n_N, int n_M, int m, int k) {
  PfLayout L;
  L.lin = make_lin_layout(bwd, n_N, n_M, m, k);
  L.nblk_M = (n_M + 127) / 128;
  size_t o = L.lin.total;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = round_up(o + bytes, 256);
    return at_;
  };
  L.part = take((size_t)L.nblk_M * m * 4);
  L.M2 = take((size_t)m * 4);
  L.FQ = take((size_t)n_N * m * 2);
  L.FK = take((size_t)n_M * m * 2);
  const size_t mat = (size_t)m * kpad_lin(k) * 2;
  L.Mlo = take(mat);
  L.MTlo = take(mat);
  if (bwd) {
    L.dMlo = take(mat);
    L.dMTlo = take(mat);
  }
  if (!bwd) {
    L.rowoff = take((size_t)n_N * 4);
  } else {
    L.den = take((size_t)n_N * 4);
    L.dFQ = take((size_t)n_N * m * 4);
    L.dFK = take((size_t)n_M * m * 4);
  }
  L.total = o;
  return L;
}

// Functional-map solve: bf16 basis only; 1 <= k <= 256; n >= 1.
ssc_status check_fmap(ssc_dtype t, int n, int k) {
  if (n < 1 || k < 1) return SSC_ERR_INVALID_ARG;
  if (t != SSC_BF16 || k > kFmMaxK || kpad_for(k) == 0) return SSC_ERR_UNSUPPORTED;
  return SSC_OK;
}

// Farthest-point sampling: n >= 1 vertices, nnz >= 0 adjacency entries,
// 1 <= P <= n seeds.
ssc_status check_fps(int n, int nnz, int P) {
  if (n < 1 || nnz < 0 || P < 1 || P > n) return SSC_ERR_INVALID_ARG;
  return SSC_OK;
}

struct FpsLayout {
  size_t w = kNone, adjp = kNone, wp = kNone, stamp = kNone, queue = kNone, cmax = kNone, cflag = kNone, bad = kNone,
         ctl = kNone;
  size_t total = 0;
  int nchunk = 0, nblk = 0;
};

FpsLayout make_fps_layout(int n, int nnz) {
  FpsLayout L;
  L.nchunk = (n + 255) / 256;
  L.nblk = (n + 255) / 256;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = round_up(o + bytes, 256);
    return at_;
  };
  L.w = take((size_t)nnz * 8);
  L.adjp = take((size_t)n * kFpsSlots * 4);
  L.wp = take((size_t)n * kFpsSlots * 8);
  L.stamp = take((size_t)n * 4);
  L.queue = take((size_t)n * 8);
  L.cmax = take((size_t)L.nchunk * 8);
  L.cflag = take((size_t)L.nchunk * 4);
  L.bad = take((size_t)L.nblk * 4);
  L.ctl = take(sizeof(FpsCtl));
  L.total = o;
  return L;
}

struct FmLayout {
  size_t part = kNone, G = kNone, R = kNone, Lrow = kNone, Lcol = kNone, rdiag = kNone, X = kNone;
  size_t total = 0;
  int nblk = 0, rows = 0;
};

FmLayout make_fm_layout(bool bwd, int n, int k) {
  FmLayout L;
  const int kp = kpad_for(k);
  const size_t KP = (size_t)kp;
  fm_blocks(n, kp, &L.rows, &L.nblk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = o;
    o = round_up(o + bytes, 256);
    return at_;
  };
  L.part = take((size_t)(bwd ? 1 : 2) * L.nblk * KP * KP * 4);
  L.G = take(KP * KP * 4);
  if (!bwd) L.R = take(KP * KP * 4);
  L.Lrow = take((size_t)k * (k + 1) / 2 * 4);
  L.Lcol = take((size_t)k * (k + 1) / 2 * 4);
  L.rdiag = take((size_t)k * 4);
  if (bwd) L.X = take(KP * KP * 2);
  L.total = o;
  return L;
}

// Dense bf16 couplings with few row blocks (on a side) run as a geo coupling with one
// patch per side selecting the other (the same exact softmax over every
// key): the geo planner splits the items of a short item list along their
// key stream and merges the parts, so the call fills the chip where the
// dense kernels would launch a few dozen workgroups.  The one-patch offsets
// and selection sit in the first kOnePatchBytes of the workspace, the geo
// call's workspace after them.
constexpr size_t kOnePatchBytes = 256;
thread_local int g_dense_split = -1;  // -1: by size, 0: never, 1: always (bf16)

bool dense_split_route(ssc_dtype t, int n_N, int n_M, bool bwd) {
  if (t != SSC_BF16 || n_N <= 0 || g_dense_split == 0) return false;
  if (g_dense_split == 1) return true;
  // at most half a round of items on a side, so that each of its items is
  // split in two or more: the forward's rows; either side of the backward
  // (its dQ pass has n_N / 128 items, its dK/dV pass n_M / 128, and the
  // planner splits each side on its own, so a long side stays whole items)
  const int half = kRoundCUs / 2;
  const int iN = (n_N + kRowsFwd - 1) / kRowsFwd, iM = (n_M + kRowsDkv - 1) / kRowsDkv;
  return bwd ? iN <= half || iM <= half : iN <= half;
}

size_t one_patch_ws(ssc_op op, ssc_dtype t, int n_N, int n_M, int d, int k) {
  const ssc_op g = op == SSC_OP_DENSE_FWD ? SSC_OP_GEO_FWD : SSC_OP_GEO_BWD;
  return kOnePatchBytes + make_layout(g, t, n_N, n_M, d, k, 1, 1, 1).total;
}

ssc_status check_ws_bytes(size_t need, void* ws, size_t ws_bytes) {
  if (need == 0) return SSC_OK;
  if (ws == nullptr || ws_bytes < need) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  return SSC_OK;
}

ssc_status check_ws(const Layout& L, void* ws, size_t ws_bytes) { return check_ws_bytes(L.total, ws, ws_bytes); }

}  // namespace

extern "C" {

size_t ssc_workspace_bytes(ssc_op op, ssc_dtype dtype, int n_N, int n_M, int d, int k, int P_N, int P_M,
                           int s) {
  switch (op) {
    case SSC_OP_DENSE_FWD:
    case SSC_OP_DENSE_BWD: {
      if (check_shape(dtype, n_N, n_M, d, k) != SSC_OK) return 0;
      // enough for either route (the one-patch geo route is bf16 only)
      const size_t dn = make_layout(op, dtype, n_N, n_M, d, k, 0, 0, 0).total;
      if (dtype != SSC_BF16) return dn;
      const size_t gp = one_patch_ws(op, dtype, n_N, n_M, d, k);
      return dn > gp ? dn : gp;
    }
    case SSC_OP_GEO_FWD:
    case SSC_OP_GEO_BWD:
      if (check_shape(dtype, n_N, n_M, d, k) != SSC_OK) return 0;
      if (check_patches(n_N, P_N, n_M, P_M, s) != SSC_OK) return 0;
      break;
    case SSC_OP_PATCH_TOPK:
      if (d != 64 && d != 128) return 0;
      if (check_patches(n_N, P_N, n_M, P_M, s) != SSC_OK) return 0;
      break;
    case SSC_OP_LINEAR_FWD:
    case SSC_OP_LINEAR_BWD:
      if (check_linear(dtype, n_N, n_M, d, k) != SSC_OK) return 0;
      return make_lin_layout(op == SSC_OP_LINEAR_BWD, n_N, n_M, d, k).total;
    case SSC_OP_FMAP_FWD:
    case SSC_OP_FMAP_BWD:
      if (check_fmap(dtype, n_N, k) != SSC_OK) return 0;
      return make_fm_layout(op == SSC_OP_FMAP_BWD, n_N, k).total;
    case SSC_OP_PERFORMER_FWD:
    case SSC_OP_PERFORMER_BWD: {
      const int m = P_N == 0 ? d : P_N;  // P_N carries the feature count m
      if (check_performer(dtype, n_N, n_M, d, k, m) != SSC_OK) return 0;
      return make_pf_layout(op == SSC_OP_PERFORMER_BWD, n_N, n_M, m, k).total;
    }
    case SSC_OP_FPS:
      if (check_fps(n_N, n_M, P_N) != SSC_OK) return 0;
      return make_fps_layout(n_N, n_M).total;
    default:
      return 0;
  }
  return make_layout(op, dtype, n_N, n_M, d, k, P_N, P_M, s).total;
}

const char* ssc_status_string(ssc_status status) {
  switch (status) {
    case SSC_OK: return "ok";
    case SSC_ERR_INVALID_ARG: return "invalid argument";
    case SSC_ERR_UNSUPPORTED: return "unsupported shape";
    case SSC_ERR_WORKSPACE: return "workspace too small";
    case SSC_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int ssc_last_hip_error(void) { return g_last_hip; }

int ssc_debug_build(void) { return kDebug ? 1 : 0; }

int ssc_timer_arm(const char* family, int capacity) {
  KernelTimer& t = g_timer;
  for (hipEvent_t e : t.ev)
    if (e != nullptr) (void)hipEventDestroy(e);
  t.ev.clear();
  t.used = 0;
  t.overflow = false;
  t.family = family != nullptr ? family : "";
  if (t.family.empty() || capacity <= 0) {
    t.family.clear();
    return SSC_OK;
  }
  t.ev.resize(2 * (size_t)capacity, nullptr);
  for (hipEvent_t& e : t.ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      t.family.clear();
      return hip_status(r);
    }
  }
  return SSC_OK;
}

int ssc_timer_read(float* total_ms, int* count) {
  KernelTimer& t = g_timer;
  if (total_ms == nullptr || count == nullptr) return SSC_ERR_INVALID_ARG;
  float sum = 0.f;
  for (size_t i = 0; i < t.used; ++i) {
    hipError_t r = hipEventSynchronize(t.ev[2 * i + 1]);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]);
    if (r != hipSuccess) return hip_status(r);
    sum += ms;
  }
  *total_ms = sum;
  *count = t.overflow ? -(int)t.used : (int)t.used;
  t.used = 0;
  t.overflow = false;
  return SSC_OK;
}

int ssc_dense_split(int mode) {
  const int prev = g_dense_split;
  if (mode >= -1 && mode <= 1) g_dense_split = mode;
  return prev;
}

int ssc_query(int which, int arg) {
  if (which == 0) return kpad_for(arg);
  if (which == 1) return kGroup;
  return -1;
}

ssc_status coupling_dense_fwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, const void* Q, const void* K,
                              const void* V, float scale, float* O, float* lse, void* ws, size_t ws_bytes,
                              ssc_stream stream) {
  ssc_status st = check_shape(dtype, n_N, n_M, d, k);
  if (st != SSC_OK) return st;
  if (n_N == 0) return SSC_OK;
  if (!all_ok({Q, K, V, O, lse})) return SSC_ERR_INVALID_ARG;
  const size_t es = dtype == SSC_BF16 ? 2 : 4;
  const bool split = dense_split_route(dtype, n_N, n_M, false);
  const Layout L = make_layout(SSC_OP_DENSE_FWD, dtype, n_N, n_M, d, k, 0, 0, 0);
  if ((st = split ? check_ws_bytes(one_patch_ws(SSC_OP_DENSE_FWD, dtype, n_N, n_M, d, k), ws, ws_bytes)
                  : check_ws(L, ws, ws_bytes)) != SSC_OK)
    return st;
  const Buf bQ{Q, (size_t)n_N * d * es}, bK{K, (size_t)n_M * d * es}, bV{V, (size_t)n_M * k * es};
  const Buf bO{O, (size_t)n_N * k * 4}, bl{lse, (size_t)n_N * 4}, bw{ws, ws_bytes};
  if (!disjoint({bO, bl, bw}, {bQ, bK, bV})) return SSC_ERR_INVALID_ARG;
  if (split) {
    // every argument checked: the one-patch offsets, then the geo call
    int* p = static_cast<int*>(ws);
    SSC_TRY(launch_one_patch(p, n_N, n_M, reinterpret_cast<hipStream_t>(stream)));
    return coupling_geo_fwd(dtype, d, k, n_N, 1, p, n_M, 1, p + 4, 1, p + 8, Q, K, V, scale, O, lse,
                            static_cast<char*>(ws) + kOnePatchBytes, ws_bytes - kOnePatchBytes, stream);
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_for(k);
  if (dtype == SSC_BF16) {
    const int KPf = kpad_fwd_bf16(k);
    const bool ones = k < KPf;
    char* Vt = at<char>(ws, L.Vt);
    SSC_TRY(launch_transpose_bf16(V, n_M, k, KPf, ones ? 1 : 0, Vt, L.npadT, s));
    float* knorm = at<float>(ws, L.knorm);
    SSC_TRY(launch_keynorm(K, n_M, d, knorm, s));
    FwdArgs a{};
    a.Q = Q; a.Kp = K; a.Vt = Vt; a.groupsVt = L.npadT / kGroup; a.O = O; a.lse = lse;
    a.n_N = n_N; a.k = k; a.c2 = scale * kLog2e; a.n_M = n_M; a.knorm2 = knorm;
    const int rQ = kRowsFwd, grid = (n_N + rQ - 1) / rQ;
    if (!ones) {
      SSC_TRY(timed("fwd", s, [&] { return launch_fwd_bf16(d, KPf, ones, a, grid, s); }));
      return SSC_OK;
    }
    // a pass with the bounded reference, then the one-wave kernel on the
    // 128-row blocks whose row sums underflowed (none, normally: those
    // workgroups exit at once).  The wide-wave pass (256 rows a workgroup)
    // moves half the data per product; below 128 of its workgroups the
    // paired-wave pass (128 rows) fills more of the chip, and only it has
    // the kp = 256 instances.
    a.fallback_out = at<int>(ws, L.fallback);
    const int gw = (n_N + 255) / 256;
    if (KPf <= 224 && gw >= kWideMinWGs) {
      SSC_TRY(timed("fwd", s, [&] { return launch_fwd_wide(d, KPf, a, gw, s); }));
    } else {
      SSC_TRY(timed("fwd", s, [&] { return launch_fwd_pair(d, KPf, a, grid, s); }));
    }
    a.fallback = a.fallback_out;
    SSC_TRY(launch_fwd_bf16(d, KPf, ones, a, grid, s));
    return SSC_OK;
  }
  const int ngroups = L.npadM / kGroup;
  const void* Kp = K;
  if (n_M % kGroup != 0) {
    PackArgs pk{};
    pk.X = K; pk.Xp = at<char>(ws, L.Kp); pk.n = n_M; pk.w = d; pk.W = d;
    SSC_TRY(launch_pack(dt(dtype), pk, ngroups, s));
    Kp = pk.Xp;
  }
  PackArgs pv{};
  pv.X = V; pv.Xg = at<char>(ws, L.Vg); pv.n = n_M; pv.w = k; pv.W = KP;
  SSC_TRY(launch_pack(dt(dtype), pv, ngroups, s));

  FwdArgs a{};
  a.Q = Q; a.Kp = Kp; a.Vg = pv.Xg; a.O = O; a.lse = lse;
  a.n_N = n_N; a.k = k; a.c2 = scale * kLog2e;
  a.npadM = L.npadM; a.n_M = n_M;
  SSC_TRY(timed("fwd", s, [&] { return launch_fwd(dt(dtype), d, KP, a, (n_N + kRowsPerWG - 1) / kRowsPerWG, s); }));
  return SSC_OK;
}

ssc_status coupling_dense_bwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, const void* Q, const void* K,
                              const void* V, float scale, const float* O, const void* dO, const float* lse,
                              float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_shape(dtype, n_N, n_M, d, k);
  if (st != SSC_OK) return st;
  // no target rows: dK = dV = 0, nothing reads Q, O, dO, lse or writes dQ
  if (!all_ok({K, V, dK}) || !aligned16(dV)) return SSC_ERR_INVALID_ARG;
  if (n_N > 0 && !all_ok({Q, O, dO, lse, dQ})) return SSC_ERR_INVALID_ARG;
  const size_t es = dtype == SSC_BF16 ? 2 : 4;
  const bool split = dense_split_route(dtype, n_N, n_M, true);
  const Layout L = make_layout(SSC_OP_DENSE_BWD, dtype, n_N, n_M, d, k, 0, 0, 0);
  if ((st = split ? check_ws_bytes(one_patch_ws(SSC_OP_DENSE_BWD, dtype, n_N, n_M, d, k), ws, ws_bytes)
                  : check_ws(L, ws, ws_bytes)) != SSC_OK)
    return st;
  const Buf bQ{Q, (size_t)n_N * d * es}, bK{K, (size_t)n_M * d * es}, bV{V, (size_t)n_M * k * es};
  const Buf bO{O, (size_t)n_N * k * 4}, bdO{dO, (size_t)n_N * k * es}, bl{lse, (size_t)n_N * 4};
  const Buf bdQ{dQ, (size_t)n_N * d * 4}, bdK{dK, (size_t)n_M * d * 4}, bdV{dV, (size_t)n_M * k * 4};
  const Buf bw{ws, ws_bytes};
  if (!disjoint({bdQ, bdK, bdV, bw}, {bQ, bK, bV, bO, bdO, bl})) return SSC_ERR_INVALID_ARG;
  if (split) {
    int* p = static_cast<int*>(ws);
    SSC_TRY(launch_one_patch(p, n_N, n_M, reinterpret_cast<hipStream_t>(stream)));
    return coupling_geo_bwd(dtype, d, k, n_N, 1, p, n_M, 1, p + 4, 1, p + 8, Q, K, V, scale, O, dO, lse, dQ, dK,
                            dV, static_cast<char*>(ws) + kOnePatchBytes, ws_bytes - kOnePatchBytes, stream);
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_for(k);
  const DType T = dt(dtype);
  if (dtype == SSC_BF16) {
    const int KPb = kpad_bwd_bf16(k);
    const bool dcol = k + 2 <= KPb;
    PackArgs pv{};
    pv.X = V; pv.Xp = at<char>(ws, L.Vp); pv.n = n_M; pv.w = k; pv.W = KPb; pv.ones = dcol ? 2 : 0;
    SSC_TRY(launch_pack(T, pv, L.npadM / kGroup, s));
    PackArgs po{};
    po.X = dO; po.Xp = at<char>(ws, L.dOp); po.n = n_N; po.w = k; po.W = KPb; po.dcol = dcol;
    po.O = O; po.lse = lse; po.Dp = at<float>(ws, L.Dp); po.lse2p = at<float>(ws, L.lse2p);
    SSC_TRY(launch_pack(T, po, L.npadN / kGroup, s));
    const float c2 = scale * kLog2e;
    if (n_N > 0) {
      DqArgs q{};
      q.Qp = Q; q.dOp = po.Xp; q.lse2p = po.lse2p; q.Dp = po.Dp; q.Kp = K; q.Vp = pv.Xp; q.dQ = dQ;
      q.n_N = n_N; q.c2 = c2; q.scale = scale; q.n_M = n_M;
      const int rQ = kRowsDq;
      SSC_TRY(timed("dq", s, [&] { return launch_dq_bf16(d, KPb, dcol, q, (n_N + rQ - 1) / rQ, s); }));
    }
    DkvArgs b{};
    b.Kp = K; b.Vp = pv.Xp; b.Qp = Q; b.dOp = po.Xp; b.lse2p = po.lse2p; b.Dp = po.Dp; b.dK = dK; b.dV = dV;
    b.n_M = n_M; b.k = k; b.c2 = c2; b.scale = scale; b.n_N = n_N;
    const int rK = kRowsDkv;
    SSC_TRY(timed("dkv", s, [&] { return launch_dkv_bf16(d, KPb, dcol, dV != nullptr, b, (n_M + rK - 1) / rK, s); }));
    return SSC_OK;
  }

  PackArgs pk{};
  pk.X = K; pk.Xp = at<char>(ws, L.Kp); pk.Xg = at<char>(ws, L.Kg); pk.n = n_M; pk.w = d; pk.W = d;
  SSC_TRY(launch_pack(T, pk, L.npadM / kGroup, s));
  PackArgs pv{};
  pv.X = V; pv.Xp = at<char>(ws, L.Vp); pv.n = n_M; pv.w = k; pv.W = KP;
  SSC_TRY(launch_pack(T, pv, L.npadM / kGroup, s));
  PackArgs pq{};
  pq.X = Q; pq.Xp = at<char>(ws, L.Qp); pq.Xg = at<char>(ws, L.Qg); pq.n = n_N; pq.w = d; pq.W = d;
  SSC_TRY(launch_pack(T, pq, L.npadN / kGroup, s));
  PackArgs po{};
  po.X = dO; po.Xp = at<char>(ws, L.dOp); po.Xg = at<char>(ws, L.dOg); po.n = n_N; po.w = k; po.W = KP;
  po.O = O; po.lse = lse; po.Dp = at<float>(ws, L.Dp); po.lse2p = at<float>(ws, L.lse2p);
  SSC_TRY(launch_pack(T, po, L.npadN / kGroup, s));

  const float c2 = scale * kLog2e;
  if (n_N > 0) {
    DqArgs q{};
    q.Qp = pq.Xp; q.dOp = po.Xp; q.lse2p = po.lse2p; q.Dp = po.Dp;
    q.Kp = pk.Xp; q.Vp = pv.Xp; q.Kg = pk.Xg; q.dQ = dQ;
    q.n_N = n_N; q.c2 = c2; q.scale = scale; q.npadM = L.npadM; q.n_M = n_M;
    SSC_TRY(timed("dq", s, [&] { return launch_dq(T, d, KP, q, (n_N + kRowsPerWG - 1) / kRowsPerWG, s); }));
  }
  DkvArgs b{};
  b.Kp = pk.Xp; b.Vp = pv.Xp; b.Qp = pq.Xp; b.dOp = po.Xp; b.Qg = pq.Xg; b.dOg = po.Xg;
  b.lse2p = po.lse2p; b.Dp = po.Dp; b.dK = dK; b.dV = dV;
  b.n_M = n_M; b.k = k; b.c2 = c2; b.scale = scale; b.npadN = L.npadN; b.n_N = n_N;
  SSC_TRY(timed("dkv", s, [&] { return launch_dkv(T, d, KP, b, (n_M + kRowsPerWG - 1) / kRowsPerWG, s); }));
  return SSC_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free patch scoring: the same kernels with their scratch (the
// fp64 patch means and the debug verdict) in a file-scope device array.
// Its size bounds the patch counts; every GPU the library runs on holds its
// own copy until the process ends.  The kernels write every scratch entry
// they read (pooling writes each patch mean, the verdict flag is cleared by
// a kernel), so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
namespace {
constexpr int kNoAllocMaxPatches = 2048;  // P_N, P_M <= this, d <= 128
constexpr size_t kNoAllocScratchBytes = 2 * (size_t)kNoAllocMaxPatches * 128 * sizeof(double) + 256;
}  // namespace

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // address of `scratch` on each device (set on first use there)

// The device address of `scratch` on the device of `stream`: looked up once
// per device with that device current (host code must never pass the
// array's own name, which is a host-side stand-in, to a kernel).
ssc_status scratch_on(hipStream_t stream, void** out) {
  int dev = 0;
  if (stream != nullptr) {
    SSC_TRY(hipStreamGetDevice(stream, &dev));
  } else {
    SSC_TRY(hipGetDevice(&dev));
  }
  if (dev < 0 || dev >= kMaxDevices) return SSC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    SSC_TRY(hipGetDevice(&cur));
    if (cur != dev) SSC_TRY(hipSetDevice(dev));
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return hip_status(e2);
    }
    if (e != hipSuccess) return hip_status(e);
    if (ptr == nullptr) return SSC_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SSC_OK;
}
}  // namespace

extern "C" {

ssc_status patch_score_topk(ssc_dtype dtype, int d, int n_N, int P_N, const int* offN, const void* Q, int n_M,
                            int P_M, const int* offM, const void* K, int s, int* idx, double* scores, void* ws,
                            size_t ws_bytes, ssc_stream stream) {
  if (dtype != SSC_F32 && dtype != SSC_BF16) return SSC_ERR_INVALID_ARG;
  if (n_N < 0 || n_M < 0) return SSC_ERR_INVALID_ARG;
  ssc_status st = check_patches(n_N, P_N, n_M, P_M, s);
  if (st != SSC_OK) return st;
  if (d != 64 && d != 128) return SSC_ERR_UNSUPPORTED;
  if (!all_ok({offN, offM, idx})) return SSC_ERR_INVALID_ARG;
  if ((n_N > 0 && !all_ok({Q})) || (n_M > 0 && !all_ok({K}))) return SSC_ERR_INVALID_ARG;
  if (scores != nullptr && !aligned16(scores)) return SSC_ERR_INVALID_ARG;
  const size_t es = dtype == SSC_BF16 ? 2 : 4;
  const Layout L = make_layout(SSC_OP_PATCH_TOPK, dtype, n_N, n_M, d, 1, P_N, P_M, s);
  if ((st = check_ws(L, ws, ws_bytes)) != SSC_OK) return st;
  const Buf bQ{Q, (size_t)n_N * d * es}, bK{K, (size_t)n_M * d * es};
  const Buf boN{offN, ((size_t)P_N + 1) * 4}, boM{offM, ((size_t)P_M + 1) * 4};
  const Buf bi{idx, (size_t)P_N * s * 4}, bs{scores, (size_t)P_N * P_M * 8}, bw{ws, ws_bytes};
  if (!disjoint({bi, bs, bw}, {bQ, bK, boN, boM})) return SSC_ERR_INVALID_ARG;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  PoolArgs pa{};
  pa.Q = Q; pa.K = K; pa.offN = offN; pa.offM = offM;
  pa.n_N = n_N; pa.n_M = n_M; pa.P_N = P_N; pa.P_M = P_M; pa.d = d;
  pa.Qbar = at<double>(ws, L.Qbar); pa.KbarT = at<double>(ws, L.KbarT);
  SSC_TRY(launch_pool(dt(dtype), pa, hs));
  TopkArgs ta{};
  ta.Qbar = pa.Qbar; ta.KbarT = pa.KbarT; ta.P_N = P_N; ta.P_M = P_M; ta.d = d; ta.s = s;
  ta.idx = idx; ta.scores = scores;
  SSC_TRY(launch_topk(ta, hs));
  if (kDebug) {
    int* flag = at<int>(ws, L.flag);
    SSC_TRY(launch_check_offsets(offN, P_N, n_N, offM, P_M, n_M, flag, hs));
    return debug_verdict(flag, hs);
  }
  return SSC_OK;
}

ssc_status patch_score_topk_noalloc(ssc_dtype dtype, int d, int n_N, int P_N, const int* offN, const void* Q,
                                    int n_M, int P_M, const int* offM, const void* K, int s, int* idx,
                                    double* scores, ssc_stream stream) {
  if (dtype != SSC_F32 && dtype != SSC_BF16) return SSC_ERR_INVALID_ARG;
  if (n_N < 0 || n_M < 0) return SSC_ERR_INVALID_ARG;
  ssc_status st = check_patches(n_N, P_N, n_M, P_M, s);
  if (st != SSC_OK) return st;
  if (d != 64 && d != 128) return SSC_ERR_UNSUPPORTED;
  if (P_N > kNoAllocMaxPatches || P_M > kNoAllocMaxPatches) return SSC_ERR_WORKSPACE;
  const Layout L = make_layout(SSC_OP_PATCH_TOPK, dtype, n_N, n_M, d, 1, P_N, P_M, s);
  if (L.total > kNoAllocScratchBytes) return SSC_ERR_WORKSPACE;
  void* ptr = nullptr;
  if ((st = scratch_on(reinterpret_cast<hipStream_t>(stream), &ptr)) != SSC_OK) return st;
  return patch_score_topk(dtype, d, n_N, P_N, offN, Q, n_M, P_M, offM, K, s, idx, scores, ptr, L.total, stream);
}

namespace {

ssc_status geo_common_checks(ssc_dtype dtype, int d, int k, int n_N, int P_N, const int* offN, int n_M, int P_M,
                             const int* offM, int s, const int* idx) {
  ssc_status st = check_shape(dtype, n_N, n_M, d, k);
  if (st != SSC_OK) return st;
  if ((st = check_patches(n_N, P_N, n_M, P_M, s)) != SSC_OK) return st;
  if (!all_ok({offN, offM, idx})) return SSC_ERR_INVALID_ARG;
  return SSC_OK;
}

// pads / pad_grids: bf16 row-padding jobs (at most two) that run in the
// plan's launch, on the CUs the plan leaves idle
ssc_status launch_geo_plan(const Layout& L, void* ws, const int* offN, const int* offM, const int* idx, int n_N,
                           int n_M, int P_N, int P_M, int s, bool inverse, hipStream_t hs, bool bf16_path,
                           const PackArgs* pads = nullptr, const int* pad_grids = nullptr, int npads = 0) {
  PlanArgs pl{};
  pl.offN = offN; pl.offM = offM; pl.idx = idx;
  pl.n_N = n_N; pl.n_M = n_M; pl.P_N = P_N; pl.P_M = P_M; pl.s = s;
  // target rows per item: the forward call plans for the forward kernel, the
  // backward call for the dQ kernel
  pl.rowsQ = bf16_path ? (inverse ? kRowsDq : kRowsFwd) : kRowsPerWG;
  pl.rowsK = bf16_path ? kRowsDkv : kRowsPerWG;
  if (bf16_path) {
    pl.run_tab = at<RunEntry>(ws, L.run_tab);
    if (inverse) pl.inv_tab = at<RunEntry>(ws, L.inv_tab);
    pl.splitQ = at<SplitItem>(ws, L.splitQ);
    pl.splitK = at<SplitItem>(ws, L.splitK);
  }
  pl.poffN = at<int>(ws, L.poffN); pl.poffM = at<int>(ws, L.poffM);
  pl.itemsQ = at<Item>(ws, L.itemsQ); pl.itemsK = at<Item>(ws, L.itemsK);
  pl.counters = at<int>(ws, L.counters); pl.scratch = at<int>(ws, L.scratch);
  if (inverse) {
    pl.inv_off = at<int>(ws, L.inv_off);
    pl.inv_idx = at<int>(ws, L.inv_idx);
  }
  bool fuse = npads > 0;
  for (int i = 0; i < npads; ++i) fuse = fuse && pad_bf16_applies(DType::BF16, pads[i]);
  if (fuse) {
    SSC_TRY(launch_plan_pad(pl, pads, pad_grids, npads, hs));
  } else {
    SSC_TRY(launch_plan(pl, hs));
    for (int i = 0; i < npads; ++i) SSC_TRY(launch_pack(DType::BF16, pads[i], pad_grids[i], hs));
  }
  return SSC_OK;
}

}  // namespace

ssc_status coupling_geo_fwd(ssc_dtype dtype, int d, int k, int n_N, int P_N, const int* offN, int n_M, int P_M,
                            const int* offM, int s, const int* idx, const void* Q, const void* K, const void* V,
                            float scale, float* O, float* lse, void* ws, size_t ws_bytes, ssc_stream stream) {
  ssc_status st = geo_common_checks(dtype, d, k, n_N, P_N, offN, n_M, P_M, offM, s, idx);
  if (st != SSC_OK) return st;
  if (n_N == 0) return SSC_OK;
  if (!all_ok({Q, K, V, O, lse})) return SSC_ERR_INVALID_ARG;
  const size_t es = dtype == SSC_BF16 ? 2 : 4;
  const Layout L = make_layout(SSC_OP_GEO_FWD, dtype, n_N, n_M, d, k, P_N, P_M, s);
  if ((st = check_ws(L, ws, ws_bytes)) != SSC_OK) return st;
  const Buf bQ{Q, (size_t)n_N * d * es}, bK{K, (size_t)n_M * d * es}, bV{V, (size_t)n_M * k * es};
  const Buf boN{offN, ((size_t)P_N + 1) * 4}, boM{offM, ((size_t)P_M + 1) * 4}, bi{idx, (size_t)P_N * s * 4};
  const Buf bO{O, (size_t)n_N * k * 4}, bl{lse, (size_t)n_N * 4}, bw{ws, ws_bytes};
  if (!disjoint({bO, bl, bw}, {bQ, bK, bV, boN, boM, bi})) return SSC_ERR_INVALID_ARG;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_for(k);
  const DType T = dt(dtype);
  int* counters = at<int>(ws, L.counters);
  if (dtype == SSC_BF16) {
    const int KPf = kpad_fwd_bf16(k);
    const bool ones = k < KPf;
    PackArgs pv{};
    pv.X = V; pv.Xp = at<char>(ws, L.Vp); pv.n = n_M; pv.w = k; pv.W = KPf; pv.ones = ones;
    const int gv = L.npadM / kGroup;
    // the V padding runs in the plan's launch
    if ((st = launch_geo_plan(L, ws, offN, offM, idx, n_N, n_M, P_N, P_M, s, false, hs, true, &pv, &gv, 1)) != SSC_OK)
      return st;
    float* knorm = at<float>(ws, L.knorm);
    SSC_TRY(launch_keynorm(K, n_M, d, knorm, hs));
    FwdArgs a{};
    a.Q = Q; a.Kp = K; a.Vp = pv.Xp; a.O = O; a.lse = lse; a.knorm2 = knorm;
    a.n_N = n_N; a.k = k; a.c2 = scale * kLog2e;
    a.items = at<Item>(ws, L.itemsQ); a.n_items = counters + 0; a.offN = offN; a.n_M = n_M;
    a.idx = idx; a.s = s; a.offM = offM; a.run_tab = at<RunEntry>(ws, L.run_tab);
    a.part = at<float>(ws, L.partQ); a.split = at<SplitItem>(ws, L.splitQ); a.n_split = counters + 5;
    a.status = counters + 4;
    const int rQ = kRowsFwd;
    SSC_TRY(timed("geo_fwd", hs,
                  [&] { return launch_fwd_bf16(d, KPf, ones, a, (n_N + rQ - 1) / rQ + P_N + kRoundCUs, hs); }));
    SSC_TRY(launch_fwd_merge_bf16(d, KPf, ones, a, hs));
    return kDebug ? debug_verdict(counters + 4, hs) : SSC_OK;
  }
  if ((st = launch_geo_plan(L, ws, offN, offM, idx, n_N, n_M, P_N, P_M, s, false, hs, false)) != SSC_OK) return st;

  PackArgs pk{};
  pk.X = K; pk.Xp = at<char>(ws, L.Kp); pk.n = n_M; pk.w = d; pk.W = d;
  pk.poff = at<int>(ws, L.poffM); pk.off = offM; pk.P = P_M; pk.n_groups = counters + 3;
  SSC_TRY(launch_pack(T, pk, L.npadM / kGroup, hs));
  PackArgs pv = pk;
  pv.X = V; pv.Xp = nullptr; pv.Xg = at<char>(ws, L.Vg); pv.w = k; pv.W = KP;
  SSC_TRY(launch_pack(T, pv, L.npadM / kGroup, hs));

  FwdArgs a{};
  a.Q = Q; a.Kp = pk.Xp; a.Vg = pv.Xg; a.O = O; a.lse = lse;
  a.n_N = n_N; a.k = k; a.c2 = scale * kLog2e;
  a.items = at<Item>(ws, L.itemsQ); a.n_items = counters + 0; a.offN = offN;
  a.idx = idx; a.s = s; a.poffM = pk.poff; a.offM = offM;
  SSC_TRY(timed("geo_fwd", hs, [&] { return launch_fwd(T, d, KP, a, (n_N + kRowsPerWG - 1) / kRowsPerWG + P_N, hs); }));
  SSC_TRY(launch_invalid_fill(counters + 4, O, (size_t)n_N * k, lse, (size_t)n_N, nullptr, 0, hs));
  return kDebug ? debug_verdict(counters + 4, hs) : SSC_OK;
}

ssc_status coupling_geo_bwd(ssc_dtype dtype, int d, int k, int n_N, int P_N, const int* offN, int n_M, int P_M,
                            const int* offM, int s, const int* idx, const void* Q, const void* K, const void* V,
                            float scale, const float* O, const void* dO, const float* lse, float* dQ, float* dK,
                            float* dV, void* ws, size_t ws_bytes, ssc_stream stream) {
  ssc_status st = geo_common_checks(dtype, d, k, n_N, P_N, offN, n_M, P_M, offM, s, idx);
  if (st != SSC_OK) return st;
  // no target rows: dK = dV = 0, nothing reads Q, O, dO, lse or writes dQ
  if (!all_ok({K, V, dK}) || !aligned16(dV)) return SSC_ERR_INVALID_ARG;
  if (n_N > 0 && !all_ok({Q, O, dO, lse, dQ})) return SSC_ERR_INVALID_ARG;
  const size_t es = dtype == SSC_BF16 ? 2 : 4;
  const Layout L = make_layout(SSC_OP_GEO_BWD, dtype, n_N, n_M, d, k, P_N, P_M, s);
  if ((st = check_ws(L, ws, ws_bytes)) != SSC_OK) return st;
  const Buf bQ{Q, (size_t)n_N * d * es}, bK{K, (size_t)n_M * d * es}, bV{V, (size_t)n_M * k * es};
  const Buf bO{O, (size_t)n_N * k * 4}, bdO{dO, (size_t)n_N * k * es}, bl{lse, (size_t)n_N * 4};
  const Buf boN{offN, ((size_t)P_N + 1) * 4}, boM{offM, ((size_t)P_M + 1) * 4}, bi{idx, (size_t)P_N * s * 4};
  const Buf bdQ{dQ, (size_t)n_N * d * 4}, bdK{dK, (size_t)n_M * d * 4}, bdV{dV, (size_t)n_M * k * 4};
  const Buf bw{ws, ws_bytes};
  if (!disjoint({bdQ, bdK, bdV, bw}, {bQ, bK, bV, bO, bdO, bl, boN, boM, bi})) return SSC_ERR_INVALID_ARG;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_for(k);
  const DType T = dt(dtype);
  int* counters = at<int>(ws, L.counters);
  if (dtype == SSC_BF16) {
    const int KPb = kpad_bwd_bf16(k);
    const bool dcol = k + 2 <= KPb;
    PackArgs pads[2]{};
    PackArgs& pv = pads[0];
    pv.X = V; pv.Xp = at<char>(ws, L.Vp); pv.n = n_M; pv.w = k; pv.W = KPb; pv.ones = dcol ? 2 : 0;
    PackArgs& po = pads[1];
    po.X = dO; po.Xp = at<char>(ws, L.dOp); po.n = n_N; po.w = k; po.W = KPb; po.dcol = dcol;
    po.O = O; po.lse = lse; po.Dp = at<float>(ws, L.Dp); po.lse2p = at<float>(ws, L.lse2p);
    // the V and dO padding run in the plan's launch (no dO rows: V only)
    const int grids[2] = {L.npadM / kGroup, L.npadN / kGroup};
    if ((st = launch_geo_plan(L, ws, offN, offM, idx, n_N, n_M, P_N, P_M, s, true, hs, true, pads, grids,
                              n_N > 0 ? 2 : 1)) != SSC_OK)
      return st;
    const float c2 = scale * kLog2e;
    if (n_N > 0) {
      DqArgs q{};
      q.Qp = Q; q.dOp = po.Xp; q.lse2p = po.lse2p; q.Dp = po.Dp; q.Kp = K; q.Vp = pv.Xp; q.dQ = dQ;
      q.n_N = n_N; q.c2 = c2; q.scale = scale;
      q.items = at<Item>(ws, L.itemsQ); q.n_items = counters + 0; q.offN = offN; q.n_M = n_M;
      q.idx = idx; q.s = s; q.offM = offM; q.run_tab = at<RunEntry>(ws, L.run_tab);
      q.part = at<float>(ws, L.partQ); q.split = at<SplitItem>(ws, L.splitQ); q.n_split = counters + 5;
      q.status = counters + 4;
      const int rQ = kRowsDq;
      SSC_TRY(timed("geo_dq", hs,
                    [&] { return launch_dq_bf16(d, KPb, dcol, q, (n_N + rQ - 1) / rQ + P_N + kRoundCUs, hs); }));
      SSC_TRY(launch_dq_merge_bf16(d, q, hs));
    }
    DkvArgs b{};
    b.Kp = K; b.Vp = pv.Xp; b.Qp = Q; b.dOp = po.Xp; b.lse2p = po.lse2p; b.Dp = po.Dp; b.dK = dK; b.dV = dV;
    b.n_M = n_M; b.k = k; b.c2 = c2; b.scale = scale; b.n_N = n_N;
    b.items = at<Item>(ws, L.itemsK); b.n_items = counters + 1; b.offM = offM; b.offN = offN;
    b.inv_off = at<int>(ws, L.inv_off); b.inv_idx = at<int>(ws, L.inv_idx); b.inv_tab = at<RunEntry>(ws, L.inv_tab);
    b.part = at<float>(ws, L.partK); b.split = at<SplitItem>(ws, L.splitK); b.n_split = counters + 6;
    b.status = counters + 4;
    const int rK = kRowsDkv;
    const bool want_dv = dV != nullptr;
    SSC_TRY(timed("geo_dkv", hs, [&] {
      return launch_dkv_bf16(d, KPb, dcol, want_dv, b, (n_M + rK - 1) / rK + P_M + kRoundCUs, hs);
    }));
    SSC_TRY(launch_dkv_merge_bf16(d, KPb, want_dv, b, hs));
    return kDebug ? debug_verdict(counters + 4, hs) : SSC_OK;
  }
  if ((st = launch_geo_plan(L, ws, offN, offM, idx, n_N, n_M, P_N, P_M, s, true, hs, false)) != SSC_OK) return st;
  int* poffN = at<int>(ws, L.poffN);
  int* poffM = at<int>(ws, L.poffM);

  PackArgs pk{};
  pk.X = K; pk.Xp = at<char>(ws, L.Kp); pk.Xg = at<char>(ws, L.Kg); pk.n = n_M; pk.w = d; pk.W = d;
  pk.poff = poffM; pk.off = offM; pk.P = P_M; pk.n_groups = counters + 3;
  SSC_TRY(launch_pack(T, pk, L.npadM / kGroup, hs));
  PackArgs pv = pk;
  pv.X = V; pv.Xp = at<char>(ws, L.Vp); pv.Xg = nullptr; pv.w = k; pv.W = KP;
  SSC_TRY(launch_pack(T, pv, L.npadM / kGroup, hs));
  PackArgs pq{};
  pq.X = Q; pq.Xp = at<char>(ws, L.Qp); pq.Xg = at<char>(ws, L.Qg); pq.n = n_N; pq.w = d; pq.W = d;
  pq.poff = poffN; pq.off = offN; pq.P = P_N; pq.n_groups = counters + 2;
  SSC_TRY(launch_pack(T, pq, L.npadN / kGroup, hs));
  PackArgs po = pq;
  po.X = dO; po.Xp = at<char>(ws, L.dOp); po.Xg = at<char>(ws, L.dOg); po.w = k; po.W = KP;
  po.O = O; po.lse = lse; po.Dp = at<float>(ws, L.Dp); po.lse2p = at<float>(ws, L.lse2p);
  SSC_TRY(launch_pack(T, po, L.npadN / kGroup, hs));

  const float c2 = scale * kLog2e;
  if (n_N > 0) {
    DqArgs q{};
    q.Qp = pq.Xp; q.dOp = po.Xp; q.lse2p = po.lse2p; q.Dp = po.Dp;
    q.Kp = pk.Xp; q.Vp = pv.Xp; q.Kg = pk.Xg; q.dQ = dQ;
    q.n_N = n_N; q.c2 = c2; q.scale = scale;
    q.items = at<Item>(ws, L.itemsQ); q.n_items = counters + 0; q.offN = offN; q.poffN = poffN;
    q.idx = idx; q.s = s; q.poffM = poffM; q.offM = offM;
    SSC_TRY(timed("geo_dq", hs, [&] { return launch_dq(T, d, KP, q, (n_N + kRowsPerWG - 1) / kRowsPerWG + P_N, hs); }));
  }
  DkvArgs b{};
  b.Kp = pk.Xp; b.Vp = pv.Xp; b.Qp = pq.Xp; b.dOp = po.Xp; b.Qg = pq.Xg; b.dOg = po.Xg;
  b.lse2p = po.lse2p; b.Dp = po.Dp; b.dK = dK; b.dV = dV;
  b.n_M = n_M; b.k = k; b.c2 = c2; b.scale = scale;
  b.items = at<Item>(ws, L.itemsK); b.n_items = counters + 1; b.offM = offM; b.poffM = poffM;
  b.inv_off = at<int>(ws, L.inv_off); b.inv_idx = at<int>(ws, L.inv_idx); b.poffN = poffN; b.offN = offN;
  SSC_TRY(timed("geo_dkv", hs, [&] { return launch_dkv(T, d, KP, b, (n_M + kRowsPerWG - 1) / kRowsPerWG + P_M, hs); }));
  SSC_TRY(launch_invalid_fill(counters + 4, n_N > 0 ? dQ : nullptr, (size_t)n_N * d, dK, (size_t)n_M * d, dV,
                              (size_t)n_M * k, hs));
  return kDebug ? debug_verdict(counters + 4, hs) : SSC_OK;
}

ssc_status coupling_linear_fwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, const void* Q, const void* K,
                               const void* V, float* O, float* den, void* ws, size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_linear(dtype, n_N, n_M, d, k);
  if (st != SSC_OK) return st;
  if (n_N == 0) return SSC_OK;
  if (!all_ok({Q, K, V, O, den})) return SSC_ERR_INVALID_ARG;
  const LinLayout L = make_lin_layout(false, n_N, n_M, d, k);
  if (ws == nullptr || ws_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  const Buf bQ{Q, (size_t)n_N * d * 2}, bK{K, (size_t)n_M * d * 2}, bV{V, (size_t)n_M * k * 2};
  const Buf bO{O, (size_t)n_N * k * 4}, bd{den, (size_t)n_N * 4}, bw{ws, ws_bytes};
  if (!disjoint({bO, bd, bw}, {bQ, bK, bV})) return SSC_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_lin(k);
  LinArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.den = den;
  a.part = at<float>(ws, L.part); a.M = at<char>(ws, L.M); a.MT = at<char>(ws, L.MT);
  a.n_N = n_N; a.n_M = n_M; a.k = k; a.gram_rows = L.gram_rows;
  SSC_TRY(timed("lin_gram", s, [&] { return launch_lin_gram(d, KP, false, a, L.parts_M, s); }));
  SSC_TRY(launch_lin_reduce(d, KP, a.part, L.parts_M, at<char>(ws, L.M), at<char>(ws, L.MT), nullptr, nullptr, s));
  SSC_TRY(timed("lin_apply", s, [&] { return launch_lin_apply(d, KP, false, a, s); }));
  return SSC_OK;
}

ssc_status coupling_linear_bwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, const void* Q, const void* K,
                               const void* V, const float* O, const void* dO, const float* den, float* dQ,
                               float* dK, float* dV, void* ws, size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_linear(dtype, n_N, n_M, d, k);
  if (st != SSC_OK) return st;
  // no target rows: dK = dV = 0 (the query-side Gram sum is empty), nothing
  // reads Q, O, dO, den or writes dQ
  if (!all_ok({K, V, dK, dV})) return SSC_ERR_INVALID_ARG;
  if (n_N > 0 && !all_ok({Q, O, dO, den, dQ})) return SSC_ERR_INVALID_ARG;
  const LinLayout L = make_lin_layout(true, n_N, n_M, d, k);
  if (ws == nullptr || ws_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  const Buf bQ{Q, (size_t)n_N * d * 2}, bK{K, (size_t)n_M * d * 2}, bV{V, (size_t)n_M * k * 2};
  const Buf bO{O, (size_t)n_N * k * 4}, bdO{dO, (size_t)n_N * k * 2}, bd{den, (size_t)n_N * 4};
  const Buf bdQ{dQ, (size_t)n_N * d * 4}, bdK{dK, (size_t)n_M * d * 4}, bdV{dV, (size_t)n_M * k * 4};
  const Buf bw{ws, ws_bytes};
  if (!disjoint({bdQ, bdK, bdV, bw}, {bQ, bK, bV, bO, bdO, bd})) return SSC_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_lin(k);
  LinArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.O = const_cast<float*>(O); a.den = const_cast<float*>(den);
  a.rden = at<float>(ws, L.rden); a.s = at<float>(ws, L.s); a.part = at<float>(ws, L.part);
  a.M = at<char>(ws, L.M); a.MT = at<char>(ws, L.MT); a.dM = at<char>(ws, L.dM); a.dMT = at<char>(ws, L.dMT);
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.n_N = n_N; a.n_M = n_M; a.k = k; a.gram_rows = L.gram_rows;
  a.partN = a.part + (size_t)L.parts_M * d * KP;
  // both Gram sums (the second also forms rden and s), both reductions, then
  // the dQ, dK and dV rows: three launches
  SSC_TRY(launch_lin_gram_bwd(d, KP, false, a, L.parts_M, L.parts_N, s));
  SSC_TRY(launch_lin_reduce2(d, KP, a.part, L.parts_M, at<char>(ws, L.M), at<char>(ws, L.MT), nullptr, nullptr,
                             a.partN, L.parts_N, at<char>(ws, L.dM), at<char>(ws, L.dMT), nullptr, nullptr, s));
  SSC_TRY(launch_lin_apply_bwd(d, KP, false, a, s));
  return SSC_OK;
}

// The key maxima and the key / query features of the Performer coupling.
static ssc_status pf_features(int d, int m, const PfLayout& L, void* ws, int n_N, int n_M, const void* Q,
                              const void* K, const void* W, float scale, int qmode, float* rowoff,
                              const float* lnden, float* den, hipStream_t s) {
  PfArgs p{};
  p.W = W; p.scale = scale; p.part = at<float>(ws, L.part); p.M2 = at<float>(ws, L.M2);
  p.X = K; p.n = n_M; p.nblk = L.nblk_M; p.F = at<bf16>(ws, L.FK);
  SSC_TRY(launch_pf_keymax(d, m, p, s));
  SSC_TRY(launch_pf_maxreduce(m, p, s));
  // key and query features in one launch (both need only the key maxima)
  PfArgs pq = p;
  pq.X = Q; pq.n = n_N; pq.F = at<bf16>(ws, L.FQ); pq.rowoff = rowoff; pq.lnden = lnden; pq.den = den;
  SSC_TRY(timed("pf_feat", s, [&] { return launch_pf_feat_kq(d, m, qmode, p, pq, s); }));
  return SSC_OK;
}

ssc_status coupling_performer_fwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, int m, const void* Q,
                                  const void* K, const void* V, const void* W, float scale, float* O, float* lnden,
                                  void* ws, size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_performer(dtype, n_N, n_M, d, k, m);
  if (st != SSC_OK) return st;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SSC_ERR_INVALID_ARG;
  if (n_N == 0) return SSC_OK;
  if (!all_ok({Q, K, V, W, O, lnden})) return SSC_ERR_INVALID_ARG;
  const PfLayout L = make_pf_layout(false, n_N, n_M, m, k);
  if (ws == nullptr || ws_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  const Buf bQ{Q, (size_t)n_N * d * 2}, bK{K, (size_t)n_M * d * 2}, bV{V, (size_t)n_M * k * 2};
  const Buf bW{W, (size_t)m * d * 2};
  const Buf bO{O, (size_t)n_N * k * 4}, bd{lnden, (size_t)n_N * 4}, bw{ws, ws_bytes};
  if (!disjoint({bO, bd, bw}, {bQ, bK, bV, bW})) return SSC_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* rowoff = at<float>(ws, L.rowoff);
  st = pf_features(d, m, L, ws, n_N, n_M, Q, K, W, scale, 2, rowoff, nullptr, nullptr, s);
  if (st != SSC_OK) return st;
  // the linear coupling on the m-wide feature rows
  const int KP = kpad_lin(k);
  LinArgs a{};
  a.Q = at<bf16>(ws, L.FQ); a.K = at<bf16>(ws, L.FK); a.V = V; a.O = O; a.den = lnden; a.rowoff = rowoff;
  a.part = at<float>(ws, L.lin.part); a.M = at<char>(ws, L.lin.M); a.MT = at<char>(ws, L.lin.MT);
  a.Mlo = at<char>(ws, L.Mlo); a.MTlo = at<char>(ws, L.MTlo);
  a.n_N = n_N; a.n_M = n_M; a.k = k; a.gram_rows = L.lin.gram_rows;
  SSC_TRY(launch_lin_gram(m, KP, true, a, L.lin.parts_M, s));
  SSC_TRY(launch_lin_reduce(m, KP, a.part, L.lin.parts_M, at<char>(ws, L.lin.M), at<char>(ws, L.lin.MT),
                            at<char>(ws, L.Mlo), at<char>(ws, L.MTlo), s));
  SSC_TRY(launch_lin_apply(m, KP, true, a, s));
  return SSC_OK;
}

ssc_status coupling_performer_bwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, int m, const void* Q,
                                  const void* K, const void* V, const void* W, float scale, const float* O,
                                  const void* dO, const float* lnden, float* dQ, float* dK, float* dV, void* ws,
                                  size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_performer(dtype, n_N, n_M, d, k, m);
  if (st != SSC_OK) return st;
  if (!(scale > 0.f) || !(scale < 1e30f)) return SSC_ERR_INVALID_ARG;
  // no target rows: dK = dV = 0, as for the linear coupling
  if (!all_ok({K, V, W, dK, dV})) return SSC_ERR_INVALID_ARG;
  if (n_N > 0 && !all_ok({Q, O, dO, lnden, dQ})) return SSC_ERR_INVALID_ARG;
  const PfLayout L = make_pf_layout(true, n_N, n_M, m, k);
  if (ws == nullptr || ws_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  const Buf bQ{Q, (size_t)n_N * d * 2}, bK{K, (size_t)n_M * d * 2}, bV{V, (size_t)n_M * k * 2};
  const Buf bW{W, (size_t)m * d * 2}, bO{O, (size_t)n_N * k * 4}, bdO{dO, (size_t)n_N * k * 2};
  const Buf bd{lnden, (size_t)n_N * 4};
  const Buf bdQ{dQ, (size_t)n_N * d * 4}, bdK{dK, (size_t)n_M * d * 4}, bdV{dV, (size_t)n_M * k * 4};
  const Buf bw{ws, ws_bytes};
  if (!disjoint({bdQ, bdK, bdV, bw}, {bQ, bK, bV, bW, bO, bdO, bd})) return SSC_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* den = at<float>(ws, L.den);
  st = pf_features(d, m, L, ws, n_N, n_M, Q, K, W, scale, 3, nullptr, lnden, den, s);
  if (st != SSC_OK) return st;
  const int KP = kpad_lin(k);
  LinArgs a{};
  a.Q = at<bf16>(ws, L.FQ); a.K = at<bf16>(ws, L.FK); a.V = V; a.dO = dO; a.O = const_cast<float*>(O);
  a.den = den; a.rden = at<float>(ws, L.lin.rden); a.s = at<float>(ws, L.lin.s); a.part = at<float>(ws, L.lin.part);
  a.M = at<char>(ws, L.lin.M); a.MT = at<char>(ws, L.lin.MT); a.dM = at<char>(ws, L.lin.dM);
  a.dMT = at<char>(ws, L.lin.dMT);
  a.Mlo = at<char>(ws, L.Mlo); a.MTlo = at<char>(ws, L.MTlo); a.dMlo = at<char>(ws, L.dMlo);
  a.dMTlo = at<char>(ws, L.dMTlo);
  a.dQ = at<float>(ws, L.dFQ); a.dK = at<float>(ws, L.dFK); a.dV = dV;
  a.n_N = n_N; a.n_M = n_M; a.k = k; a.gram_rows = L.lin.gram_rows;
  a.partN = a.part + (size_t)L.lin.parts_M * m * KP;
  SSC_TRY(launch_lin_gram_bwd(m, KP, true, a, L.lin.parts_M, L.lin.parts_N, s));
  SSC_TRY(launch_lin_reduce2(m, KP, a.part, L.lin.parts_M, at<char>(ws, L.lin.M), at<char>(ws, L.lin.MT),
                             at<char>(ws, L.Mlo), at<char>(ws, L.MTlo), a.partN, L.lin.parts_N,
                             at<char>(ws, L.lin.dM), at<char>(ws, L.lin.dMT), at<char>(ws, L.dMlo),
                             at<char>(ws, L.dMTlo), s));
  SSC_TRY(launch_lin_apply_bwd(m, KP, true, a, s));
  // dQ and dK from the feature gradients, in one launch
  PfArgs pq{};
  pq.W = W; pq.scale = scale;
  pq.X = Q; pq.n = n_N; pq.F = at<bf16>(ws, L.FQ); pq.dF = at<float>(ws, L.dFQ); pq.dX = dQ;
  PfArgs pk = pq;
  pk.X = K; pk.n = n_M; pk.F = at<bf16>(ws, L.FK); pk.dF = at<float>(ws, L.dFK); pk.dX = dK;
  SSC_TRY(launch_pf_dx2(d, m, pq, pk, s));
  return SSC_OK;
}

ssc_status fmap_solve_fwd(ssc_dtype dtype, int n, int k, const void* PhiN, const float* O, float* C, void* ws,
                          size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_fmap(dtype, n, k);
  if (st != SSC_OK) return st;
  if (!all_ok({PhiN, O, C})) return SSC_ERR_INVALID_ARG;
  const FmLayout L = make_fm_layout(false, n, k);
  if (ws == nullptr || ws_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  const Buf bP{PhiN, (size_t)n * k * 2}, bO{O, (size_t)n * k * 4}, bC{C, (size_t)k * k * 4}, bw{ws, ws_bytes};
  if (!disjoint({bC, bw}, {bP, bO})) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_for(k);
  FmArgs a{};
  a.Phi = PhiN; a.O = O; a.C = C; a.n = n; a.k = k;
  a.part = at<float>(ws, L.part); a.G = at<float>(ws, L.G); a.R = at<float>(ws, L.R);
  a.Lrow = at<float>(ws, L.Lrow); a.Lcol = at<float>(ws, L.Lcol); a.rdiag = at<float>(ws, L.rdiag);
  a.rows = L.rows;
  SSC_TRY(timed("fm_gram", s, [&] { return launch_fm_gram(KP, true, a, L.nblk, s); }));
  SSC_TRY(launch_fm_reduce(KP, true, a, L.nblk, s));
  SSC_TRY(timed("fm_chol", s, [&] { return launch_fm_chol(KP, a, s); }));
  SSC_TRY(timed("fm_solve", s, [&] { return launch_fm_solve(KP, 0, a, s); }));
  return SSC_OK;
}

ssc_status fmap_solve_bwd(ssc_dtype dtype, int n, int k, const void* PhiN, const float* dC, float* dO, void* ws,
                          size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_fmap(dtype, n, k);
  if (st != SSC_OK) return st;
  if (!all_ok({PhiN, dC, dO})) return SSC_ERR_INVALID_ARG;
  const FmLayout L = make_fm_layout(true, n, k);
  if (ws == nullptr || ws_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  const Buf bP{PhiN, (size_t)n * k * 2}, bdC{dC, (size_t)k * k * 4}, bdO{dO, (size_t)n * k * 4}, bw{ws, ws_bytes};
  if (!disjoint({bdO, bw}, {bP, bdC})) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int KP = kpad_for(k);
  FmArgs a{};
  a.Phi = PhiN; a.dC = dC; a.dO = dO; a.n = n; a.k = k;
  a.part = at<float>(ws, L.part); a.G = at<float>(ws, L.G); a.X = at<bf16>(ws, L.X);
  a.Lrow = at<float>(ws, L.Lrow); a.Lcol = at<float>(ws, L.Lcol); a.rdiag = at<float>(ws, L.rdiag);
  a.rows = L.rows;
  SSC_TRY(timed("fm_gram", s, [&] { return launch_fm_gram(KP, false, a, L.nblk, s); }));
  SSC_TRY(launch_fm_reduce(KP, false, a, L.nblk, s));
  SSC_TRY(timed("fm_chol", s, [&] { return launch_fm_chol(KP, a, s); }));
  SSC_TRY(timed("fm_solve", s, [&] { return launch_fm_solve(KP, 1, a, s); }));
  SSC_TRY(timed("fm_apply", s, [&] { return launch_fm_apply(KP, a, s); }));
  return SSC_OK;
}

ssc_status fps_partition(int n, int nnz, const double* x, const int* off, const int* adj, int P, int* seeds,
                         int* labels, double* dist, void* ws, size_t ws_bytes, ssc_stream stream) {
  ssc_status st = check_fps(n, nnz, P);
  if (st != SSC_OK) return st;
  if (!all_ok({x, off, seeds, labels, dist}) || (nnz > 0 && adj == nullptr)) return SSC_ERR_INVALID_ARG;
  const FpsLayout L = make_fps_layout(n, nnz);
  if (ws == nullptr || ws_bytes < L.total) return SSC_ERR_WORKSPACE;
  if (!aligned16(ws)) return SSC_ERR_INVALID_ARG;
  const Buf bx{x, (size_t)n * 24}, bo{off, (size_t)(n + 1) * 4}, ba{adj, (size_t)nnz * 4};
  const Buf bs{seeds, (size_t)P * 4}, bl{labels, (size_t)n * 4}, bd{dist, (size_t)n * 8}, bw{ws, ws_bytes};
  if (!disjoint({bs, bl, bd, bw}, {bx, bo, ba})) return SSC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  FpsArgs a{};
  a.x = x; a.off = off; a.adj = adj; a.n = n; a.nnz = nnz; a.P = P;
  a.seeds = seeds; a.labels = labels; a.dist = dist;
  a.w = at<double>(ws, L.w); a.stamp = at<int>(ws, L.stamp); a.queue = at<int>(ws, L.queue);
  a.adjp = at<int>(ws, L.adjp); a.wp = at<double>(ws, L.wp);
  a.cmax = at<unsigned long long>(ws, L.cmax); a.cflag = at<int>(ws, L.cflag); a.bad = at<int>(ws, L.bad);
  a.nchunk = L.nchunk; a.nblk = L.nblk;
  a.ctl = at<FpsCtl>(ws, L.ctl);
  // from kFpsWideMin vertices the first steps run on 16 workgroups until a
  // step's largest round queue stays below 1024 vertices.  Overrides (tests
  // and tuning): SSC_FPS_WIDE_STEPS caps those steps (0: none),
  // SSC_FPS_WIDE_BLOCKS sets the workgroups, SSC_FPS_WIDE_FRONTIER the queue
  // threshold, SSC_FPS_SPIN_LIMIT the polls of a barrier wait (0: every wait
  // gives up at once, so the one-workgroup kernel redoes every step).
  a.wide_steps = n >= kFpsWideMin ? P : 0;
  a.spin = 1u << 20;
  a.wide_blocks = 16;
  a.wide_frontier = 1024;
  if (const char* e = std::getenv("SSC_FPS_WIDE_FRONTIER")) a.wide_frontier = std::atoi(e);
  if (const char* e = std::getenv("SSC_FPS_WIDE_STEPS")) a.wide_steps = std::max(0, std::min(P, std::atoi(e)));
  if (const char* e = std::getenv("SSC_FPS_WIDE_BLOCKS")) a.wide_blocks = std::max(1, std::atoi(e));
  if (const char* e = std::getenv("SSC_FPS_SPIN_LIMIT")) a.spin = (unsigned)std::strtoul(e, nullptr, 10);
  SSC_TRY(timed("fps", s, [&] { return launch_fps(a, s); }));
  return SSC_OK;
}

}  // extern "C"
