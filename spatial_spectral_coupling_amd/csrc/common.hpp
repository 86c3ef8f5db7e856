// Shared device definitions for the coupling kernels (gfx950 / CDNA4).
//
// Matrix-core building block: v_mfma_f32_32x32x16_bf16 (bf16) or eight
// v_mfma_f32_32x32x2_f32 (fp32).  Lane layouts (wave64, l = lane, h = l / 32):
//   operand A (M x K): lane holds row l % 32 and 8 k-elements of group h;
//   operand B (K x N): lane holds column l % 32 and 8 k-elements of group h;
//   result C (32 x 32 fp32, 16 per lane): column l % 32,
//       rows 8 * (i / 4) + 4 * h + (i % 4), i = 0..15.
// Which 8 k-indices a lane's group covers is arbitrary as long as A and B use
// the same assignment.  A C-layout tile can therefore be fed straight back as
// an operand whose contraction runs over C's rows: for the 16 rows of half
// `hk` of a 32-row block, lane group h holds rows
//   hk*16 + {4h, 4h+1, 4h+2, 4h+3, 8+4h, 8+4h+1, 8+4h+2, 8+4h+3}  (j = 0..7),
// and the matching partner operand is read from a transposed LDS tile with
// two 4-element reads.  This is how softmax probabilities move from the
// score product into the value product without leaving registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssc {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 16;      // row-group granularity of the padded patch layout
constexpr int kTile = 64;       // positions per streamed tile (4 groups)
constexpr int kGroupsPerTile = kTile / kGroup;
constexpr int kWaves = 4;       // waves per workgroup of the block kernels
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsPerWG = kWaves * 32;  // query rows (fwd, dQ) or key rows (dK/dV) per WG

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct FragT;
template <> struct FragT<bf16> { typedef bf16x8 type; };
template <> struct FragT<float> { typedef f32x8 type; };

__device__ __forceinline__ f32x16 mma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// 8 consecutive elements from LDS (row-layout tile).
template <typename T>
__device__ __forceinline__ typename FragT<T>::type lds_row8(const T* p) {
  return *reinterpret_cast<const typename FragT<T>::type*>(p);
}

// Elements [p[0..3], p[8..11]] from LDS (transposed tile, see header comment).
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* p) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 8);
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 lds_tr8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 8);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Eight C-layout values (c[i0 .. i0+7]) as an operand fragment of type T.
template <typename T>
__device__ __forceinline__ typename FragT<T>::type c_to_frag(const f32x16& c, int i0);
template <>
__device__ __forceinline__ bf16x8 c_to_frag<bf16>(const f32x16& c, int i0) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)c[i0 + j];
  return r;
}
template <>
__device__ __forceinline__ f32x8 c_to_frag<float>(const f32x16& c, int i0) {
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = c[i0 + j];
  return r;
}

// Row index (within a 32-row block) of C-layout element i for lane group h.
__device__ __forceinline__ int c_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// 16-byte global load / store helpers.
struct alignas(16) Chunk { uint32_t w[4]; };

__device__ __forceinline__ Chunk ld_chunk(const void* p) { return *reinterpret_cast<const Chunk*>(p); }
__device__ __forceinline__ void st_chunk(void* p, const Chunk& c) { *reinterpret_cast<Chunk*>(p) = c; }
__device__ __forceinline__ Chunk zero_chunk() { return Chunk{{0u, 0u, 0u, 0u}}; }

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// One source (or target) run of the padded patch layout: a contiguous range
// of padded positions [pos0, pos0 + ngroups * kGroup) whose first `nvalid`
// positions hold real rows.
struct Run {
  int pos0, ngroups, nvalid;
};

// Stream of runs.  `list == nullptr` means one run covering positions
// [0, npad) with `nvalid_all` real rows (the dense coupling); otherwise run r
// is patch list[r] of a layout with padded offsets `poff` and true offsets
// `off`.
struct RunStream {
  const int* list;
  int nruns;
  const int* poff;
  const int* off;
  int npad_all, nvalid_all;

  __device__ __forceinline__ Run get(int r) const {
    if (list == nullptr) return Run{0, npad_all / kGroup, nvalid_all};
    int q = list[r];
    int p0 = poff[q];
    return Run{p0, (poff[q + 1] - p0) / kGroup, off[q + 1] - off[q]};
  }
  __device__ __forceinline__ int count() const { return list == nullptr ? 1 : nruns; }
};

// Walks a RunStream kGroup positions at a time.
struct GroupCursor {
  int r, g;         // current run and group within it
  Run cur;
  bool live;

  __device__ __forceinline__ void start(const RunStream& rs) {
    r = 0;
    g = 0;
    live = false;
    advance_to_nonempty(rs);
  }
  __device__ __forceinline__ void advance_to_nonempty(const RunStream& rs) {
    const int n = rs.count();
    while (r < n) {
      cur = rs.get(r);
      if (g < cur.ngroups) {
        live = true;
        return;
      }
      ++r;
      g = 0;
    }
    live = false;
  }
  // Next group: base position and number of real rows in it (0 = none).
  __device__ __forceinline__ void next(const RunStream& rs, int& base, int& valid) {
    if (!live) {
      base = -1;
      valid = 0;
      return;
    }
    base = cur.pos0 + g * kGroup;
    int v = cur.nvalid - g * kGroup;
    valid = v < 0 ? 0 : (v > kGroup ? kGroup : v);
    ++g;
    if (g >= cur.ngroups) {
      ++r;
      g = 0;
      advance_to_nonempty(rs);
    }
  }
};

__device__ __forceinline__ int total_groups(const RunStream& rs) {
  int t = 0;
  const int n = rs.count();
  for (int r = 0; r < n; ++r) t += rs.get(r).ngroups;
  return t;
}

}  // namespace ssc
