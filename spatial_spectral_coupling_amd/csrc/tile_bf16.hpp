// Tile machinery shared by the bf16 block kernels of the spatial-spectral
// coupling on gfx950 (attn_bf16_q.hip: forward and dQ; attn_bf16_kv.hip:
// dK / dV).
//
// Same mathematics as attn.hip (forward with online softmax; dQ pass; dK/dV
// pass; project page "Spatial-Spectral Coupling as Attention", sections
// "How it works" and "Geo-FlashAttention"), with a data movement built for
// CDNA4:
//  * tiles of 64 streamed rows are copied global -> LDS with direct buffer
//    loads (16 bytes per lane) into one of two statically distinct buffers,
//    spread over the MFMA pipeline of the tile before;
//  * only row-layout tiles are staged.  Operands whose contraction runs along
//    the tile's rows (V^T in the forward, K^T in dQ, Q^T and dO^T in dK/dV)
//    are read with ds_read_b64_tr_b16: in a 16-lane group, lane j addresses
//    row r0 + j/4, columns c0 + 4(j%4) .. +3, and lane i receives rows
//    r0..r0+3 of column c0 + i -- four k-elements of an MFMA operand;
//  * rows are gathered one by one from the caller's arrays, so the geo
//    support (concatenated source patches) needs no padding: a tile may span
//    several patches and only the stream's last tile is partial;
//  * LDS rows carry pad chunks so that row-fragment reads (32 rows, one
//    chunk) and transposed reads (4 rows x 32 bytes per 16 lanes) spread
//    over the banks with purely affine addresses.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

#include <math.h>

#include <type_traits>
#include <utility>

namespace ssc {
namespace tb {

// f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at compile time
// (no loop for the unroller to give up on; every index is a constant).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// Row pitch (in 16-byte chunks) of an LDS tile with cw data chunks per row:
// the smallest cw + e (e >= 1) such that
//  * the pitch is an odd number of chunks -- 16 consecutive rows of a
//    row-fragment read (16 bytes per lane) then start in 16 distinct
//    16-byte bank groups of the 256-byte bank window;
//  * the 4 rows x 32 bytes of a 16-lane transposed read are pairwise
//    disjoint modulo the bank window.
// Measured on gfx950 (512 threads per CU): row-fragment reads run at about
// 195 B/clk per CU with such a pitch and at half that with an even one;
// transposed reads at about 104 B/clk per CU.
constexpr bool tr_rows_disjoint(int pitch_bytes) {
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b) {
      const int d = ((b - a) * pitch_bytes) % 256;
      if (d < 32 || d > 256 - 32) return false;
    }
  return true;
}
constexpr int tile_pitch_chunks(int cw) {
  int p = cw + 1;
  while (!((p & 1) && tr_rows_disjoint(p * 16))) ++p;
  return p;
}

// Geometry of a 64-row tile of W bf16 columns: CW data chunks of 16 bytes per
// row, stored with a pitch of CP chunks; every LDS address of a lane stays a
// per-lane base plus a compile-time offset.
template <int W>
struct Geo {
  static constexpr int CW = W / 8;
  static constexpr int CP = tile_pitch_chunks(CW);
  static constexpr int PITCH = CP * 16;           // bytes per row
  static constexpr int BYTES = kTile * PITCH;
  static constexpr int SLOTS = kTile * CP;        // 16-byte slots, a multiple of 64
};
static_assert(Geo<128>::CP == 19 && Geo<224>::CP == 29 && Geo<64>::CP == 9, "tile pitch");

// Row-fragment reads for MFMA operands: rows rb*32 + l32, chunk 2*cc + h.
template <int W>
struct RowReader {
  int lane_off;
  __device__ __forceinline__ void init(int l32, int h) { lane_off = l32 * Geo<W>::PITCH + h * 16; }
  __device__ __forceinline__ bf16x8 read(const char* tile, int rb, int cc) const {
    return *reinterpret_cast<const bf16x8*>(tile + lane_off + rb * 32 * Geo<W>::PITCH + cc * 32);
  }
};

// Transposed-operand reads with ds_read_b64_tr_b16: rows kc*16 + tr_r and
// kc*16 + 8 + tr_r, columns cb*32 + tr_c .. +3 (tr_r = 4h + (i>>2),
// tr_c = 16(G&1) + 4(i&3) for lane i of 16-lane group G), giving the 8
// k-elements rows kc*16 + {4h..4h+3, 8+4h..8+4h+3} of column cb*32 + l32.
template <int W>
struct TrReader {
  int lane_off;
  __device__ __forceinline__ void init(int tr_r, int tr_c) { lane_off = tr_r * Geo<W>::PITCH + tr_c * 2; }
  __device__ __forceinline__ bf16x8 frag(const char* tile, int cb, int kc) const {
    const char* base = tile + lane_off + cb * 64 + kc * 16 * Geo<W>::PITCH;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + 8 * Geo<W>::PITCH));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

// Elements 2m, 2m+1 of a bf16 operand fragment from two fp32 values (one
// packed conversion, round to nearest even).
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void put_pair(bf16x8& v, int m, float a, float b) {
  u32x4 w = __builtin_bit_cast(u32x4, v);
  w[m] = __builtin_bit_cast(unsigned, bf16x2{(bf16)a, (bf16)b});
  v = __builtin_bit_cast(bf16x8, w);
}

// Eight probabilities (C-layout elements i0..i0+7) as a bf16 operand.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& c, int i0) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)c[i0 + j];
  return r;
}

// Buffer resource of a global array (base, byte size): raw buffer loads
// take a 32-bit byte offset from it and return zero outside the range.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long p = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(p & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;  // raw 32-bit data format (gfx9)
  return r;
}

// Direct buffer load of `size` bytes per lane into LDS at lds + 4 * lane
// (size 4) or lds + 16 * lane (size 16).
extern "C" __device__ void ssc_raw_buffer_load_lds(i32x4 rsrc, __attribute__((address_space(3))) void* lds,
                                                   int size, int voffset, int soffset, int offset,
                                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Division of a tile slot index s < nslots by the constant CP as a 24-bit
// multiply and shift (checked exhaustively at compile time).
constexpr unsigned slot_magic(int cp) { return (1u << 20) / (unsigned)cp + 1u; }
constexpr bool slot_magic_exact(int cp, int nslots) {
  for (unsigned s = 0; s < (unsigned)nslots; ++s)
    if (((s * slot_magic(cp)) >> 20) != s / (unsigned)cp) return false;
  return true;
}

// Direct loads of 64-row tiles of one source array (row-major, W bf16 or
// W / 2 fp32 columns, `limit` rows present) into LDS.  Slot s of a tile (16
// bytes at s * 16) is tile row r = s / CP, chunk s - r CP; the pad chunks
// of a row fetch the first chunks of the next row (never read).  The j-th
// load of a wave is tile instruction wave + j * NW.  Every wave issues the
// same number of loads (no wave-uniform branches inside the pipelines): the
// LDS buffer of a tile is rounded up to whole rounds of NW loads (ALLOC
// bytes), and the slots past the tile's 64 rows fetch rows 64.. of the
// window (dense; zeros past the array's end) or the array's end (geo) into
// that never-read tail.
//  * dense tiles are windows of consecutive rows: a buffer resource based at
//    the tile's first row and bounded by the array's end (rows past it read
//    zeros), so a lane's byte offset is the tile-independent 16 (s - r PADC);
//  * geo tiles gather rows listed in an LDS table: phase 1 fetches this
//    lane's row from the table, phase 2 (a few pipeline steps later) issues
//    the load; a missing row reads past the end of the array (zeros).
template <int W, int NW>
struct TileSrc {
  static constexpr int CP = Geo<W>::CP, CW = Geo<W>::CW, RB = 2 * W;
  static constexpr int NI = Geo<W>::SLOTS / 64;      // instructions per tile
  static constexpr int NJ = (NI + NW - 1) / NW;      // per wave
  static constexpr int ALLOC = NJ * NW * 1024;        // LDS bytes of a tile buffer
  static constexpr unsigned MAGIC = slot_magic(CP);
  static_assert(slot_magic_exact(CP, NJ * NW * 64), "slot division");

  const char* base;
  int limit;

  __device__ __forceinline__ void init(const void* b, int lim) {
    base = reinterpret_cast<const char*>(b);
    limit = lim;
  }
  __device__ __forceinline__ static int slot(int wave, int lane, int j) { return (wave + j * NW) * 64 + lane; }
  __device__ __forceinline__ static int slot_row(int s) { return (int)(__umul24((unsigned)s, MAGIC) >> 20); }
  __device__ __forceinline__ i32x4 window(int row0) const {
    const int n = limit - row0;
    return make_rsrc(base + (size_t)row0 * RB, n > 0 ? (unsigned)(n * RB) : 0u);
  }
  __device__ __forceinline__ i32x4 whole() const { return make_rsrc(base, (unsigned)(limit * RB)); }

  // byte offset of this lane's chunk within a dense window (tile-independent)
  __device__ __forceinline__ static int dense_offset(int wave, int lane, int j) {
    const int s = slot(wave, lane, j);
    return (s - slot_row(s) * (CP - CW)) * 16;
  }
  __device__ __forceinline__ static void load_dense(char* tile, const i32x4& win, int wave, int lane, int j) {
    asm volatile("" : "+v"(lane));
    ssc_raw_buffer_load_lds(win, (lds_void_t*)(tile + (wave + j * NW) * 1024), 16, dense_offset(wave, lane, j), 0,
                            0, 0);
  }
  // the same with the offset computed once outside the tile loop
  __device__ __forceinline__ static void load_dense_at(char* tile, const i32x4& win, int off, int wave, int j) {
    ssc_raw_buffer_load_lds(win, (lds_void_t*)(tile + (wave + j * NW) * 1024), 16, off, 0, 0, 0);
  }
  // geo: the row-table index of this lane's load j (its tile row, or kTile,
  // the table's sentinel entry, for the slots past the tile) and the byte
  // offset of its chunk within the row; both tile-independent
  __device__ __forceinline__ static int geo_index(int wave, int lane, int j) {
    const int r = slot_row(slot(wave, lane, j));
    return r < kTile ? r : kTile;
  }
  __device__ __forceinline__ static int geo_chunk(int wave, int lane, int j) {
    const int s = slot(wave, lane, j);
    return (s - slot_row(s) * CP) * 16;
  }
  // grow: the table entry (a row of the array, or a sentinel row at or past
  // `limit`, which reads zeros); rows and sentinels stay below 2^24
  __device__ __forceinline__ void load_geo_at(char* tile, const i32x4& all, int grow, int coff, int wave,
                                              int j) const {
    ssc_raw_buffer_load_lds(all, (lds_void_t*)(tile + (wave + j * NW) * 1024), 16,
                            (int)(__umul24((unsigned)grow, (unsigned)RB) + (unsigned)coff), 0, 0, 0);
  }
  // The whole tile at once (first tile of a stream).
  template <bool GEO>
  __device__ __forceinline__ void load_tile(char* tile, const int* rows, int row0, int wave, int lane) const {
    const i32x4 rs = GEO ? whole() : window(row0);
    static_for<NJ>([&](auto j) {
      if (GEO) load_geo_at(tile, rs, rows[geo_index(wave, lane, j)], geo_chunk(wave, lane, j), wave, j);
      else load_dense(tile, rs, wave, lane, j);
    });
  }
};

// Direct loads of 64 positions of a GROUPED-TRANSPOSED array into an LDS tile
// of ROWS rows x 64 positions.  The array holds groups of 16 positions, each
// group a contiguous [ROWS][16] block (32 bytes per row): group g starts at
// byte g * ROWS * 32, so the 4 groups of a dense tile are one contiguous
// block and a gathered stream can place any group in any of a tile's four
// slots.  An MFMA operand whose contraction runs along the positions (8
// consecutive positions of one row) is one 16-byte LDS read.
// LDS tile: row r at r * 128 bytes, no pad; its logical 16-byte chunk cc
// (positions 8 cc .. 8 cc + 7) sits in physical chunk cc ^ ((r >> 1) & 7), so
// the 16 rows of a 16-lane row-fragment read land in 16 distinct bank groups.
// Slot s of a tile is row s / 8, physical chunk s % 8; every slot is data.
template <int ROWS, int NW>
struct TileSrcG {
  static constexpr int SLOTS = ROWS * 8;
  static constexpr int NI = (SLOTS + 63) / 64;       // instructions per tile
  static constexpr int NJ = (NI + NW - 1) / NW;      // per wave
  static constexpr int ALLOC = NJ * NW * 1024;        // LDS bytes of a tile buffer
  static constexpr int GROUP = ROWS * 32;             // bytes of one 16-position group

  const char* base;
  unsigned bytes;  // groups * GROUP

  __device__ __forceinline__ void init(const void* b, int groups) {
    base = reinterpret_cast<const char*>(b);
    bytes = (unsigned)groups * GROUP;
  }
  // logical chunk of slot s (tile row s / 8)
  __device__ __forceinline__ static int chunk_of(int s) { return (s & 7) ^ ((s >> 4) & 7); }
  // dense: resource of the 4 groups starting at group g0 (zeros past the end)
  __device__ __forceinline__ i32x4 window(int g0) const {
    const unsigned o = (unsigned)g0 * GROUP;
    return make_rsrc(base + o, bytes > o ? bytes - o : 0u);
  }
  __device__ __forceinline__ i32x4 whole() const { return make_rsrc(base, bytes); }
  // byte offset of this lane's chunk j within its group, and which of the
  // tile's four group slots it belongs to (rows past ROWS read the next
  // groups' data into slots that are never read)
  __device__ __forceinline__ static unsigned in_group(int wave, int lane, int j) {
    const int s = (wave + j * NW) * 64 + lane, r = s >> 3, cc = chunk_of(s);
    return (unsigned)(r * 32 + (cc & 1) * 16);
  }
  __device__ __forceinline__ static int group_slot(int wave, int lane, int j) {
    return chunk_of((wave + j * NW) * 64 + lane) >> 1;
  }
  // dense: offset from the window's first group
  __device__ __forceinline__ static unsigned dense_offset(int wave, int lane, int j) {
    return (unsigned)group_slot(wave, lane, j) * GROUP + in_group(wave, lane, j);
  }
  __device__ __forceinline__ static void load_at(char* tile, const i32x4& win, unsigned off, int wave, int j) {
    ssc_raw_buffer_load_lds(win, (lds_void_t*)(tile + (wave + j * NW) * 1024), 16, (int)off, 0, 0, 0);
  }
};

// Row-fragment reads of a TileSrcG tile: row cb * 32 + l32, logical chunk
// 2 kc + h (positions 16 kc + 8 h .. + 7) for kc = 0..3.
struct GroupReader {
  int off[4];
  __device__ __forceinline__ void init(int l32, int h) {
    const int x = (l32 >> 1) & 7;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      off[kc] = l32 * 128 + (((2 * kc + h) ^ x) << 4);
      // opaque to the range analysis: the block offset below is then added
      // (folded into the read's immediate), not or-ed in a VALU instruction
      asm volatile("" : "+v"(off[kc]));
    }
  }
  __device__ __forceinline__ bf16x8 read(const char* tile, int cb, int kc) const {
    return *reinterpret_cast<const bf16x8*>(tile + off[kc] + cb * 32 * 128);
  }
};

// The same reads restricted to the two 16-position chunks 2 kh, 2 kh + 1 of
// one half of the tile (kh wave-uniform, known only at run time): the two
// lane offsets are formed once, so no register array is indexed at run time.
struct GroupReaderHalf {
  int off[2];
  __device__ __forceinline__ void init(int l32, int h, int kh) {
    const int x = (l32 >> 1) & 7;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      off[kk] = l32 * 128 + (((4 * kh + 2 * kk + h) ^ x) << 4);
      asm volatile("" : "+v"(off[kk]));
    }
  }
  __device__ __forceinline__ bf16x8 read(const char* tile, int cb, int kk) const {
    return *reinterpret_cast<const bf16x8*>(tile + off[kk] + cb * 32 * 128);
  }
};

// Row permutation within a 32-row MFMA block that makes the C layout of a
// product over these rows hand each lane eight CONSECUTIVE rows as the k
// elements of the next product: C element i of lane group h sits in row
// c_row(i, h) = 8 (i / 4) + 4 h + i % 4; reading A row r from tile row
// sigma(r) (bits 2 and 3 of r swapped) puts tile rows 16 (i / 8) + 8 h +
// i % 8 there, so the partner operand of 16-row chunk kc is the 16 bytes at
// positions 16 kc + 8 h .. + 7 of a transposed tile.
__device__ __forceinline__ constexpr int sigma_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Row-fragment reads like RowReader, with the block rows permuted by sigma_row.
template <int W>
struct RowReaderP {
  int lane_off;
  // rb0: a run-time row block folded into the lane offset
  __device__ __forceinline__ void init(int l32, int h, int rb0 = 0) {
    lane_off = (rb0 * 32 + sigma_row(l32)) * Geo<W>::PITCH + h * 16;
  }
  __device__ __forceinline__ bf16x8 read(const char* tile, int rb, int cc) const {
    return *reinterpret_cast<const bf16x8*>(tile + lane_off + rb * 32 * Geo<W>::PITCH + cc * 32);
  }
};

// 64 fp32 values of a per-row vector (`limit` entries) for the rows of a
// tile: dense row0 + lane, geo the table row (missing rows read zero).
struct VecSrc {
  const float* base;
  int limit;
  __device__ __forceinline__ void init(const float* b, int lim) {
    base = b;
    limit = lim;
  }
  __device__ __forceinline__ void load_dense(float* dst, int row0, int lane) const {
    const int n = limit - row0;
    const i32x4 win = make_rsrc(base + row0, n > 0 ? (unsigned)(n * 4) : 0u);
    ssc_raw_buffer_load_lds(win, (lds_void_t*)dst, 4, lane * 4, 0, 0, 0);
  }
  // grow: a row, or a sentinel at or past `limit` (reads zero)
  __device__ __forceinline__ void load_geo(float* dst, int grow, int lane) const {
    const i32x4 all = make_rsrc(base, (unsigned)(limit * 4));
    ssc_raw_buffer_load_lds(all, (lds_void_t*)dst, 4, grow * 4, 0, 0, 0);
  }
};

// Quiet NaN into x[0 .. n) by the whole grid (outputs of a rejected geo plan).
__device__ __forceinline__ void fill_nan_grid(float* x, size_t n) {
  if (x == nullptr) return;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) x[i] = __builtin_nanf("");
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Depth of the operand-read pipelines (reads issued this many MFMAs ahead).
constexpr int kAhead = 4;

// Scheduling hints for the instruction scheduler (groups are filled in
// order within the current scheduling region): R DS reads first, then
// (1 MFMA, R/NA... ) pairs -- a pipelined chain of n MFMAs whose operand
// reads (rpm reads per MFMA) run `ahead` MFMAs in front of their use.
constexpr int kMaskMFMA = 0x008, kMaskDSRead = 0x100;
template <int N, int RPM, int AHEAD>
__device__ __forceinline__ void pipeline_hint() {
  __builtin_amdgcn_sched_group_barrier(kMaskDSRead, RPM * AHEAD, 0);
#pragma unroll
  for (int j = 0; j < N - AHEAD; ++j) {
    __builtin_amdgcn_sched_group_barrier(kMaskMFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kMaskDSRead, RPM, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMaskMFMA, AHEAD, 0);
}

// Position -> row cursor over a run stream (one per thread; positions of a
// thread only grow).  Run r covers the positions from the end of run r - 1
// up to tab[r].end and maps position x to row x + tab[r].base; positions at
// or past `total` map to the sentinel row `none`.  The entry of the run after
// the current one is fetched ahead, when the cursor enters a run, so a later
// crossing finds it in registers (the tile loop's end-of-step wait covers
// the fetch); runs shorter than a tile fall back to direct reads.  Dense
// (tab == nullptr): position x is row x.
struct RowCursor {
  const RunEntry* tab;
  int nruns, total, none;
  int r;
  RunEntry cur, pre;

  __device__ __forceinline__ void init() {
    r = 0;
    cur = RunEntry{total, 0};
    pre = cur;
    if (tab == nullptr || nruns <= 0) return;
    cur = tab[0];
    pre = tab[nruns > 1 ? 1 : 0];
  }
  __device__ __forceinline__ int row(int x) {
    if (x >= total) return none;
    if (tab != nullptr && x >= cur.end) {
      ++r;
      cur = pre;
      while (x >= cur.end) cur = tab[++r];
      pre = tab[r + 1 < nruns ? r + 1 : r];
    }
    return x + cur.base;
  }
};

}  // namespace tb
}  // namespace ssc
