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
//  * LDS rows carry pad chunks so that row-fragment reads (32 rows, one
//    chunk) and transposed reads (4 rows x 32 bytes per 16 lanes) spread
//    over the banks with purely affine addresses.
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

// Division of a tile slot index s < 64 CP by the constant CP as a 24-bit
// multiply and shift (checked exhaustively at compile time).
constexpr unsigned slot_magic(int cp) { return (1u << 20) / (unsigned)cp + 1u; }
constexpr bool slot_magic_exact(int cp) {
  for (unsigned s = 0; s < 64u * (unsigned)cp; ++s)
    if (((s * slot_magic(cp)) >> 20) != s / (unsigned)cp) return false;
  return true;
}

// Direct loads of 64-row tiles of one source array (row-major, W bf16 or
// W / 2 fp32 columns, `limit` rows present) into LDS.  Slot s of a tile (16
// bytes at s * 16) is tile row r = s / CP, chunk s - r CP; the pad chunks
// of a row fetch the first chunks of the next row (never read).  The j-th
// load of a wave is tile instruction wave + j * NW.
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
  static constexpr int NJ = (NI + NW - 1) / NW;      // per wave (at most)
  static constexpr unsigned MAGIC = slot_magic(CP);
  static_assert(slot_magic_exact(CP), "slot division");

  const char* base;
  int limit;

  __device__ __forceinline__ void init(const void* b, int lim) {
    base = reinterpret_cast<const char*>(b);
    limit = lim;
  }
  __device__ __forceinline__ static bool present(int wave, int j) {
    return NJ * NW == NI || j < NJ - 1 || wave + j * NW < NI;
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
    if (!present(wave, j)) return;  // wave-uniform
    asm volatile("" : "+v"(lane));
    ssc_raw_buffer_load_lds(win, (lds_void_t*)(tile + (wave + j * NW) * 1024), 16, dense_offset(wave, lane, j), 0,
                            0, 0);
  }
  // the same with the offset computed once outside the tile loop
  __device__ __forceinline__ static void load_dense_at(char* tile, const i32x4& win, int off, int wave, int j) {
    if (!present(wave, j)) return;
    ssc_raw_buffer_load_lds(win, (lds_void_t*)(tile + (wave + j * NW) * 1024), 16, off, 0, 0, 0);
  }
  __device__ __forceinline__ static int geo_row(const int* rows, int wave, int lane, int j) {
    if (!present(wave, j)) return -1;
    asm volatile("" : "+v"(lane));
    return rows[slot_row(slot(wave, lane, j))];
  }
  __device__ __forceinline__ void load_geo(char* tile, const i32x4& all, int grow, int wave, int lane, int j) const {
    if (!present(wave, j)) return;
    asm volatile("" : "+v"(lane));
    const int s = slot(wave, lane, j);
    const int r = slot_row(s);
    const int off = grow < 0 ? limit * RB : grow * RB + (s - r * CP) * 16;
    ssc_raw_buffer_load_lds(all, (lds_void_t*)(tile + (wave + j * NW) * 1024), 16, off, 0, 0, 0);
  }
  // The whole tile at once (first tile of a stream).
  template <bool GEO>
  __device__ __forceinline__ void load_tile(char* tile, const int* rows, int row0, int wave, int lane) const {
    const i32x4 rs = GEO ? whole() : window(row0);
    static_for<NJ>([&](auto j) {
      if (GEO) load_geo(tile, rs, geo_row(rows, wave, lane, j), wave, lane, j);
      else load_dense(tile, rs, wave, lane, j);
    });
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
  __device__ __forceinline__ void load_geo(float* dst, int grow, int lane) const {
    const i32x4 all = make_rsrc(base, (unsigned)(limit * 4));
    ssc_raw_buffer_load_lds(all, (lds_void_t*)dst, 4, grow < 0 ? limit * 4 : grow * 4, 0, 0, 0);
  }
};

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
// Exact sign flip of eight bf16 values.
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 neg_bf16x8(const bf16x8& x) {
  return __builtin_bit_cast(bf16x8, __builtin_bit_cast(u16x8, x) ^ (unsigned short)0x8000);
}

// One wave owns 32 query rows (their Q fragments stay in registers); the
// workgroup streams the key rows through LDS in tiles of 64.  A tile's MFMAs
// form four chains run as one software pipeline:
//   c = 0, 1: scores of key half c (keys 32c .. 32c+31), A = K rows;
//   c = 2, 3: O += P V over key half c - 2, A = transposed V reads.
// Operand reads run AH steps ahead of their MFMA.  The softmax of half 0
// (row maximum, exp2, row sum, bf16 packing) runs in slices during chain 1,
// that of half 1 during chain 2.  The next tile's direct loads are spread
// over the first half of the pipeline; scheduling fences between steps keep
// this order.
//
// Softmax reference: the probabilities of a tile are taken relative to a
// reference fixed for the whole tile (the first tile: the maximum of its
// first half; later tiles: the running reference), and the accumulators are
// rescaled only between tiles, when the running maximum has moved more than
// 8 (log2 units) above the reference.  A tile whose maximum exceeds its
// reference by more than 32 could overflow; a workgroup that saw one redoes
// its rows in a second pass with the exact row maxima of the first pass as a
// fixed reference (probabilities <= 1), so the result is exact either way.
template <int D, int KP, int NW, bool GEO>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void fwd_bf16(FwdArgs a) {
  constexpr int KB = Geo<D>::BYTES, VB = Geo<KP>::BYTES;
  __shared__ __attribute__((aligned(1024))) char sm0[KB + VB];
  __shared__ __attribute__((aligned(1024))) char sm1[KB + VB];
  __shared__ int rowtab[2][kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int q_begin, q_end;
  RowCursor rc;
  if (!GEO) {
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
  // streamed source rows: K (n_M rows) and the k-padded V (n_M + 1 rows,
  // a zero row at n_M)
  TileSrc<D, NW> sK;
  sK.init(a.Kp, a.n_M);
  TileSrc<KP, NW> sV;
  sV.init(a.Vp, a.n_M + 1);
  const int row = q_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;

  const bf16* Q = reinterpret_cast<const bf16*>(a.Q);
  RowReader<D> rk;
  rk.init(l32, h);
  TrReader<KP> tv;
  tv.init(tr_r, tr_c);

  // A negative scale is folded into Q (exact sign flip), so the reference is
  // always a maximum.
  const bool neg = a.c2 < 0.f;
  const float c2 = neg ? -a.c2 : a.c2;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc) {
    qf[dc] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + (size_t)row * D + dc * 16 + h * 8) : bf16x8{};
    if (neg) qf[dc] = neg_bf16x8(qf[dc]);
  }

  f32x16 acc[KP / 32];
  float m_run, l_run, m_true = -INFINITY;
  bool fixed = false;

  constexpr int NS = D / 16, NCB = KP / 32, NPV = 2 * NCB;
  constexpr int C1 = NS, C2 = 2 * NS, C3 = 2 * NS + NPV, U = 2 * NS + 2 * NPV, AH = 5;
  constexpr int SLICES = 10;  // 2 maximum, 8 element pairs
  constexpr int NJK = TileSrc<D, NW>::NJ, NJV = TileSrc<KP, NW>::NJ;
  constexpr int NL = NJK + NJV, LOAD0 = 2, LSTRIDE = (U / 2 - LOAD0) / NL > 2 ? (U / 2 - LOAD0) / NL : 2;
  // dense: the per-lane load offsets do not depend on the tile; kept in registers
  int loff[NL];
  static_for<NL>([&](auto j) {
    loff[j] = GEO ? 0 : j < NJK ? TileSrc<D, NW>::dense_offset(wave, lane, j)
                                : TileSrc<KP, NW>::dense_offset(wave, lane, j - NJK);
  });

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) acc[cb] = f32x16{};
    l_run = 0.f;
    m_run = fixed ? m_true : -INFINITY;
    bool lagged = false;

    if (GEO && tid < kTile) {
      rc.init();
      rowtab[0][tid] = rc.row(tid);
      rowtab[1][tid] = rc.row(kTile + tid);
    }
    __syncthreads();
    if (ntiles > 0) {
      sK.template load_tile<GEO>(sm0, rowtab[0], 0, wave, lane);
      sV.template load_tile<GEO>(sm0 + KB, rowtab[0], 0, wave, lane);
    }
    wait_loads();
    __syncthreads();

    // Two statically distinct buffers: the step that reads one fills the
    // other, so the compiler can tell the direct loads in flight from the LDS
    // reads.  The stream's last tile may be partial: its keys at or past
    // nvalid are masked (a wave-uniform branch inside the softmax slices).
    auto step = [&](const int t, const int b, char* Kt, char* Kn) {
      char* Vt = Kt + KB;
      const int nvalid = total - t * kTile;
      const bool part = nvalid < kTile;
      const bool first = t == 0 && !fixed;
      f32x16 sc[2];
      float sv[2][16];
      bf16x8 pf[2][2];
      float mx[2], mh[2], mref = m_run, lsum = 0.f;
      sc[0] = sc[1] = f32x16{};

      auto operand = [&](const int u) -> bf16x8 {
        if (u < C2) return rk.read(Kt, u / NS, u % NS);
        const int hb = u < C3 ? 0 : 1, j = u - (hb ? C3 : C2);
        return tv.frag(Vt, j % NCB, 2 * hb + j / NCB);
      };
      auto mma_step = [&](const int u, const bf16x8& x) {
        if (u < C2) {
          sc[u / NS] = mma(x, qf[u % NS], sc[u / NS]);
          return;
        }
        const int hb = u < C3 ? 0 : 1, j = u - (hb ? C3 : C2);
        acc[j % NCB] = mma(x, pf[hb][j / NCB], acc[j % NCB]);
      };
      auto valid = [&](const int hb, const int i) { return hb * 32 + c_row(i, h) < nvalid; };
      // Slice k of the softmax of key half hb (the scores are copied once out
      // of the MFMA accumulators into sv): 0, 1 copy and row maximum (the
      // first tile takes its reference from half 0); 2..9 element pairs
      // 2m, 2m+1 = 2(k-2) .. : exp2, row sum and packed bf16 probabilities.
      auto slice = [&](const int hb, const int k) {
        if (k <= 1) {
          if (k == 0 && part) {
            // masked keys get a score of -inf (the branch is kept: asm)
            asm volatile("");
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[hb][i] = valid(hb, i) ? sc[hb][i] : -INFINITY;
          } else if (!part) {
#pragma unroll
            for (int i = 8 * k; i < 8 * k + 8; ++i) sv[hb][i] = sc[hb][i];
          }
          float m = k == 0 ? -INFINITY : mx[hb];
#pragma unroll
          for (int i = 8 * k; i < 8 * k + 8; ++i) m = fmaxf(m, sv[hb][i]);
          mx[hb] = m;
          if (k == 1) {
            float ml = m * c2;
            ml = fmaxf(ml, xor32(ml));
            mh[hb] = ml;
            if (hb == 0) mref = first ? ml : m_run;
          }
        } else {
          const int m = k - 2;
          const float p0 = fexp2(fmaf(sv[hb][2 * m], c2, -mref));
          const float p1 = fexp2(fmaf(sv[hb][2 * m + 1], c2, -mref));
          lsum += p0 + p1;
          put_pair(pf[hb][m >> 2], m & 3, p0, p1);
        }
      };
      const int* rn = rowtab[b ^ 1];
      const int row0n = (t + 1) * kTile;
      const i32x4 winK = GEO ? sK.whole() : sK.window(row0n), winV = GEO ? sV.whole() : sV.window(row0n);
      int grow = -1;
      auto load_row = [&](const int j) {  // geo phase 1
        grow = j < NJK ? sK.geo_row(rn, wave, lane, j) : sV.geo_row(rn, wave, lane, j - NJK);
      };
      auto issue_load = [&](const int j) {
        if (j < NJK) {
          if (GEO) sK.load_geo(Kn, winK, grow, wave, lane, j);
          else sK.load_dense_at(Kn, winK, loff[j], wave, j);
        } else {
          if (GEO) sV.load_geo(Kn + KB, winV, grow, wave, lane, j - NJK);
          else sV.load_dense_at(Kn + KB, winV, loff[j], wave, j - NJK);
        }
      };
      auto side = [&](const int u) {
        if (u >= LOAD0 && (u - LOAD0) % LSTRIDE == 0 && (u - LOAD0) / LSTRIDE < NL) issue_load((u - LOAD0) / LSTRIDE);
        if (GEO && u + 2 >= LOAD0 && (u + 2 - LOAD0) % LSTRIDE == 0 && (u + 2 - LOAD0) / LSTRIDE < NL)
          load_row((u + 2 - LOAD0) / LSTRIDE);
        if (u >= C1 && u < C2) {
          static_for<SLICES>([&](auto k) {
            if (k * NS / SLICES == u - C1) slice(0, k);
          });
        } else if (u >= C2 && u < C3) {
          static_for<SLICES>([&](auto k) {
            if (k * NPV / SLICES == u - C2) slice(1, k);
          });
        }
      };

      bf16x8 ring[AH];
      static_for<AH>([&](auto u) { ring[u] = operand(u); });
      static_for<U>([&](auto u) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 cur = ring[u % AH];
        if (u + AH < U) ring[u % AH] = operand(u + AH);
        mma_step(u, cur);
        side(u);
      });
      __builtin_amdgcn_sched_barrier(0);

      // Between tiles: the sums of this tile join the running sum at the
      // tile's reference; move the reference up when the maximum ran ahead.
      l_run += lsum;
      m_run = mref;
      const float tmax = fmaxf(mh[0], mh[1]);
      m_true = fmaxf(m_true, tmax);
      lagged = lagged || tmax > mref + 32.f;
      if (!fixed && __any(tmax > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = fexp2(m_run - m_new);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      if (GEO && tid < kTile && t + 2 < ntiles) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
      wait_loads();
      __syncthreads();
    };
    for (int t = 0; t < ntiles; t += 2) {
      step(t, 0, sm0, sm1);
      if (t + 1 < ntiles) step(t + 1, 1, sm1, sm0);
    }
    if (fixed || !__syncthreads_or(lagged)) break;
    fixed = true;
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
// One wave owns 32 query rows (Q and dO fragments, lse and D in registers);
// the workgroup streams key tiles of 64 rows.  Per key half h of tile t:
//   A_h(t): scores and dP = dO V^T, A = K and V rows (two accumulations
//           interleaved);
//   B_h(t): dQ += dS K, A = transposed K fragments;
// and between them the softmax (P = exp2(S c2 - lse2), dS = P (dP - D),
// bf16 packing).  Iteration t runs A0(t), B1(t-1), A1(t), B0(t): B1 of the
// previous tile uses transposed K fragments kept in registers, so every
// softmax gets a window of a full A chain plus a B chain to hide in.
template <int D, int KP, int NW, bool GEO>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void dq_bf16(DqArgs a) {
  constexpr int KB = Geo<D>::BYTES, VB = Geo<KP>::BYTES;
  __shared__ __attribute__((aligned(1024))) char sm0[KB + VB];
  __shared__ __attribute__((aligned(1024))) char sm1[KB + VB];
  __shared__ int rowtab[2][kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int q_begin, q_end;
  RowCursor rc;
  if (!GEO) {
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
  // streamed source rows: K (n_M rows) and the k-padded V (n_M + 1 rows,
  // a zero row at n_M)
  TileSrc<D, NW> sK;
  sK.init(a.Kp, a.n_M);
  TileSrc<KP, NW> sV;
  sV.init(a.Vp, a.n_M + 1);
  const int row = q_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;

  const bf16* Q = reinterpret_cast<const bf16*>(a.Qp);
  const bf16* dOp = reinterpret_cast<const bf16*>(a.dOp);
  RowReader<D> rk;
  rk.init(l32, h);
  RowReader<KP> rv;
  rv.init(l32, h);
  TrReader<D> tk;
  tk.init(tr_r, tr_c);

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

  if (GEO && tid < kTile) {
    rc.init();
    rowtab[0][tid] = rc.row(tid);
    rowtab[1][tid] = rc.row(kTile + tid);
  }
  __syncthreads();
  if (ntiles > 0) {
    sK.template load_tile<GEO>(sm0, rowtab[0], 0, wave, lane);
    sV.template load_tile<GEO>(sm0 + KB, rowtab[0], 0, wave, lane);
  }
  wait_loads();
  __syncthreads();

  constexpr int NA = D / 16, NB = KP / 16, PAIRS = NA < NB ? NA : NB, LA = NA + NB;
  constexpr int NK = D / 32, LB = 2 * NK;
  // chains of iteration t: A0(t) | B1(t-1) | A1(t) | B0(t)
  constexpr int CY = LA, CZ = LA + LB, CW = 2 * LA + LB, U = 2 * LA + 2 * LB, AH = 5;
  constexpr int SLICES = 8;  // element pairs
  constexpr int NJK = TileSrc<D, NW>::NJ, NJV = TileSrc<KP, NW>::NJ;
  constexpr int NL = NJK + NJV, LOAD0 = 2, LSTRIDE = (U / 2 - LOAD0) / NL > 2 ? (U / 2 - LOAD0) / NL : 2;
  // dense: the per-lane load offsets do not depend on the tile; kept in registers
  int loff[NL];
  static_for<NL>([&](auto j) {
    loff[j] = GEO ? 0 : j < NJK ? TileSrc<D, NW>::dense_offset(wave, lane, j)
                                : TileSrc<KP, NW>::dense_offset(wave, lane, j - NJK);
  });
  // position of softmax slice k of a half over its window
  constexpr int WIN = LA + LB;

  // Half 1 of the previous tile, finished in the next iteration: its scores
  // and dP (slices still to run), its packed dS and its transposed K
  // fragments.  Before the first tile they stand for an empty half: zero
  // K fragments, and values whose remaining slices produce dS = 0 exactly
  // (-inf scores; elements already past their slice hold 0), so the first
  // iteration's B1 chain adds exactly 0.
  f32x16 sc1, dp1;
  bf16x8 ds1[2], kt[LB];
  static_for<16>([&](auto ic) {
    constexpr int i = ic, k = i / 2;
    sc1[i] = k * WIN / SLICES < LB ? 0.f : -INFINITY;
  });
  dp1 = f32x16{};
  ds1[0] = ds1[1] = bf16x8{};
#pragma unroll
  for (int j = 0; j < LB; ++j) kt[j] = bf16x8{};

  // Slice k of the softmax of one half (scores sv, dP dv, packed dS out):
  // element pair 2k, 2k+1 (P = exp2(S c2 - lse2), dS = P (dP - D)) packed
  // into out; slice 0 first masks keys at or past nvalid (scores -inf, so
  // P = dS = 0).
  auto slice = [&](f32x16& sv, f32x16& dv, bf16x8* out, const int kb, const int k, const bool part,
                   const int nvalid) {
    if (k == 0 && part) {
      asm volatile("");  // keeps the branch
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = kb * 32 + c_row(i, h) < nvalid ? sv[i] : -INFINITY;
    }
    const float d0 = fexp2(fmaf(sv[2 * k], c2, -lse2)) * (dv[2 * k] - Dq);
    const float d1 = fexp2(fmaf(sv[2 * k + 1], c2, -lse2)) * (dv[2 * k + 1] - Dq);
    put_pair(out[k >> 2], k & 3, d0, d1);
  };

  // Iteration t: the MFMAs of A0(t), B1(t-1), A1(t), B0(t) as one pipeline;
  // the softmax of half 0 runs during B1(t-1) and A1(t), that of half 1
  // during B0(t) and A0(t+1), so each has a 30-step window.  Two statically
  // distinct buffers: the step that reads one fills the other.
  auto step = [&](const int t, const int b, char* Kt, char* Kn) {
    char* Vt = Kt + KB;
    const int nvalid = total - t * kTile;
    const bool part = nvalid < kTile;
    f32x16 sc0 = f32x16{}, dp0 = f32x16{};
    bf16x8 ds0[2];

    auto operand = [&](const int u) -> bf16x8 {
      if (u < CY || (u >= CZ && u < CW)) {
        const int kb = u < CY ? 0 : 1, j = u < CY ? u : u - CZ;
        if (j < 2 * PAIRS) return (j & 1) ? rv.read(Vt, kb, j >> 1) : rk.read(Kt, kb, j >> 1);
        return NA > NB ? rk.read(Kt, kb, j - PAIRS) : rv.read(Vt, kb, j - PAIRS);
      }
      if (u < CZ) return kt[u - CY];
      const int j = u - CW;
      return tk.frag(Kt, j % NK, j / NK);
    };
    auto mma_step = [&](const int u, const bf16x8& x) {
      if (u < CY || (u >= CZ && u < CW)) {
        const int j = u < CY ? u : u - CZ;
        const bool is_s = j < 2 * PAIRS ? (j & 1) == 0 : NA > NB;
        const int chunk = j < 2 * PAIRS ? j >> 1 : j - PAIRS;
        f32x16& sv = u < CY ? sc0 : sc1;
        f32x16& dv = u < CY ? dp0 : dp1;
        if (is_s) sv = mma(x, qf[chunk], sv);
        else dv = mma(x, of[chunk], dv);
        return;
      }
      const int j = u < CZ ? u - CY : u - CW;
      dq[j % NK] = mma(x, u < CZ ? ds1[j / NK] : ds0[j / NK], dq[j % NK]);
    };
    const int* rn = rowtab[b ^ 1];
    const int row0n = (t + 1) * kTile;
    const i32x4 winK = GEO ? sK.whole() : sK.window(row0n), winV = GEO ? sV.whole() : sV.window(row0n);
    int grow = -1;
    auto load_row = [&](const int j) {  // geo phase 1
      grow = j < NJK ? sK.geo_row(rn, wave, lane, j) : sV.geo_row(rn, wave, lane, j - NJK);
    };
    auto issue_load = [&](const int j) {
      if (j < NJK) {
        if (GEO) sK.load_geo(Kn, winK, grow, wave, lane, j);
        else sK.load_dense_at(Kn, winK, loff[j], wave, j);
      } else {
        if (GEO) sV.load_geo(Kn + KB, winV, grow, wave, lane, j - NJK);
        else sV.load_dense_at(Kn + KB, winV, loff[j], wave, j - NJK);
      }
    };
    auto side = [&](const int u) {
      if (u >= LOAD0 && (u - LOAD0) % LSTRIDE == 0 && (u - LOAD0) / LSTRIDE < NL) issue_load((u - LOAD0) / LSTRIDE);
      if (GEO && u + 2 >= LOAD0 && (u + 2 - LOAD0) % LSTRIDE == 0 && (u + 2 - LOAD0) / LSTRIDE < NL)
        load_row((u + 2 - LOAD0) / LSTRIDE);
      if (u < CY) {
        // half 1 of the previous tile: window positions LB .. WIN-1
        static_for<SLICES>([&](auto k) {
          if (k * WIN / SLICES >= LB && k * WIN / SLICES - LB == u) slice(sc1, dp1, ds1, 1, k, false, kTile);
        });
      } else if (u < CW) {
        // half 0 of this tile: window positions 0 .. WIN-1 over B1 and A1
        static_for<SLICES>([&](auto k) {
          if (k * WIN / SLICES == u - CY) slice(sc0, dp0, ds0, 0, k, part, nvalid);
        });
      } else {
        // half 1 of this tile, window positions 0 .. LB-1; and its K^T
        // fragments for the B1 chain of the next iteration
        static_for<SLICES>([&](auto k) {
          if (k * WIN / SLICES < LB && k * WIN / SLICES == u - CW) slice(sc1, dp1, ds1, 1, k, part, nvalid);
        });
        const int j = u - CW;
        kt[j] = tk.frag(Kt, j % NK, 2 + j / NK);
      }
    };
    auto pre = [&](const int u) {
      if (u == CZ) {  // A1(t) starts: fresh accumulators for half 1
        sc1 = f32x16{};
        dp1 = f32x16{};
      }
    };

    bf16x8 ring[AH];
    static_for<AH>([&](auto u) { ring[u] = operand(u); });
    static_for<U>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 cur = ring[u % AH];
      if (u + AH < U) ring[u % AH] = operand(u + AH);
      pre(u);
      mma_step(u, cur);
      side(u);
    });
    __builtin_amdgcn_sched_barrier(0);
    if (GEO && tid < kTile && t + 2 < ntiles) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
    wait_loads();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, 0, sm0, sm1);
    if (t + 1 < ntiles) step(t + 1, 1, sm1, sm0);
  }
  // drain: the rest of the last tile's half-1 softmax, then its B1 chain
  static_for<SLICES>([&](auto k) {
    if (k * WIN / SLICES >= LB) slice(sc1, dp1, ds1, 1, k, false, kTile);
  });
  static_for<LB>([&](auto j) { dq[j % NK] = mma(kt[j], ds1[j / NK], dq[j % NK]); });

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
template <int D, int KP, int NW, bool GEO>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void dkv_bf16(DkvArgs a) {
  constexpr int QB = Geo<D>::BYTES, OB = Geo<KP>::BYTES;
  __shared__ __attribute__((aligned(1024))) char sm0[QB + OB];
  __shared__ __attribute__((aligned(1024))) char sm1[QB + OB];
  __shared__ __attribute__((aligned(16))) float ls0[kTile];
  __shared__ __attribute__((aligned(16))) float ls1[kTile];
  __shared__ __attribute__((aligned(16))) float ds0[kTile];
  __shared__ __attribute__((aligned(16))) float ds1[kTile];
  __shared__ int rowtab[2][kTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int k_begin, k_end;
  RowCursor rc;
  if (!GEO) {
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
  constexpr bool dense = !GEO;
  // streamed target rows: Q (n_N rows), dO, lse2 and D (n_N + 1 entries:
  // a zero / +inf sentinel row at n_N)
  TileSrc<D, NW> sQ;
  sQ.init(a.Qp, a.n_N);
  TileSrc<KP, NW> sO;
  sO.init(a.dOp, a.n_N + 1);
  VecSrc sL, sD;
  sL.init(a.lse2p, a.n_N + 1);
  sD.init(a.Dp, a.n_N + 1);
  const int krow = k_begin + wave * 32 + l32;
  const bool key_ok = krow < k_end;

  const bf16* K = reinterpret_cast<const bf16*>(a.Kp);
  const bf16* Vp = reinterpret_cast<const bf16*>(a.Vp);
  const bf16* Q = reinterpret_cast<const bf16*>(a.Qp);
  const bf16* dOp = reinterpret_cast<const bf16*>(a.dOp);
  RowReader<D> rq;
  rq.init(l32, h);
  RowReader<KP> ro;
  ro.init(l32, h);
  TrReader<D> tq;
  tq.init(tr_r, tr_c);
  TrReader<KP> to;
  to.init(tr_r, tr_c);

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

  if (GEO && tid < kTile) {
    rc.init();
    rowtab[0][tid] = rc.row(tid);
    rowtab[1][tid] = rc.row(kTile + tid);
  }
  __syncthreads();
  if (ntiles > 0) {
    sQ.template load_tile<GEO>(sm0, rowtab[0], 0, wave, lane);
    sO.template load_tile<GEO>(sm0 + QB, rowtab[0], 0, wave, lane);
    if (wave == 0) {
      if (GEO) sL.load_geo(ls0, rowtab[0][lane], lane);
      else sL.load_dense(ls0, 0, lane);
    }
    if (wave == NW - 1) {
      if (GEO) sD.load_geo(ds0, rowtab[0][lane], lane);
      else sD.load_dense(ds0, 0, lane);
    }
  }
  wait_loads();
  __syncthreads();

  // One tile = 64 query rows = two 32-row blocks qb.  Its MFMAs form four
  // chains of L steps each, run as one software pipeline of 4L steps:
  //   c = 0, 1: scores S = Q K^T and dP = dO V^T of block c (row reads);
  //   c = 2, 3: dV += P^T dO and dK += dS^T Q of block c - 2 (transposed
  //             reads), 2 (KP/32 + D/32) independent accumulators in turn.
  // Operand reads run AH steps ahead of their MFMA (also across chain
  // boundaries), and the softmax of block qb (P, dS and their bf16
  // packing) is cut into slices spread over chain qb + 1, so that its VALU
  // work issues while that chain's MFMAs execute.  Scheduling fences between
  // steps keep this order.
  constexpr int NA = D / 16, NB = KP / 16, PAIRS = NA < NB ? NA : NB;
  constexpr int NV = KP / 32, NK = D / 32, NVK = NV + NK;
  constexpr int L = NA + NB;  // == 2 * NVK
  static_assert(L == 2 * NVK, "chain lengths");
  constexpr int U = 4 * L, AH = 3;
  constexpr int SLICES = 12;  // 4 lse/D group reads, 8 element pairs
  // Direct loads of the next tile, spread over the first half of the
  // pipeline: NJQ + NJO tile loads and one lse or D vector load per wave.
  // The last tile loads a clamped (valid) copy into the idle buffer.
  constexpr int NJQ = TileSrc<D, NW>::NJ, NJO = TileSrc<KP, NW>::NJ;
  constexpr int NL = NJQ + NJO + 1, LOAD0 = 2, LSTRIDE = (U / 2 - LOAD0) / NL > 2 ? (U / 2 - LOAD0) / NL : 2;
  // dense: the per-lane tile load offsets do not depend on the tile
  int loff[NJQ + NJO];
  static_for<NJQ + NJO>([&](auto j) {
    loff[j] = GEO ? 0 : j < NJQ ? TileSrc<D, NW>::dense_offset(wave, lane, j)
                                : TileSrc<KP, NW>::dense_offset(wave, lane, j - NJQ);
  });

  // Two statically distinct buffers: the step that reads one fills the other.
  auto step = [&](const int t, const int b, char* Qt, char* Qn, const float* lsc, float* lsn, const float* dsc,
                  float* dsn) {
    char* Ot = Qt + QB;
    f32x16 sc[2], dp[2];
    bf16x8 pk[2][2], dk8[2][2];
    f32x4 lg[4], dg[4];
    sc[0] = sc[1] = dp[0] = dp[1] = f32x16{};

    auto operand = [&](const int u) -> bf16x8 {
      const int c = u / L, j = u % L;
      if (c < 2) {
        if (j < 2 * PAIRS) return (j & 1) ? ro.read(Ot, c, j >> 1) : rq.read(Qt, c, j >> 1);
        return NA > NB ? rq.read(Qt, c, j - PAIRS) : ro.read(Ot, c, j - PAIRS);
      }
      const int qb = c - 2, kk = j / NVK, m = j % NVK;
      return m < NV ? to.frag(Ot, m, 2 * qb + kk) : tq.frag(Qt, m - NV, 2 * qb + kk);
    };
    auto mma_step = [&](const int u, const bf16x8& x) {
      const int c = u / L, j = u % L;
      if (c < 2) {
        const bool is_s = j < 2 * PAIRS ? (j & 1) == 0 : NA > NB;
        const int chunk = j < 2 * PAIRS ? j >> 1 : j - PAIRS;
        if (is_s) sc[c] = mma(x, kf[chunk], sc[c]);
        else dp[c] = mma(x, vf[chunk], dp[c]);
        return;
      }
      const int qb = c - 2, kk = j / NVK, m = j % NVK;
      if (m < NV) dv[m] = mma(x, pk[qb][kk], dv[m]);
      else dk[m - NV] = mma(x, dk8[qb][kk], dk[m - NV]);
    };
    // Slice k of the softmax of block qb, in dependency order: the lse / D
    // values of element group g (elements 4g .. 4g+3) are read two slices
    // ahead of their use, and each element pair m (elements 2m, 2m+1 of
    // group m / 2) computes P = exp2(S c2 - lse2), dS = P (dP - D) and
    // packs both into their bf16 operands.
    //   k:  0  1  2  3  4  5  6  7  8  9  10 11
    //       r0 r1 p0 p1 r2 p2 p3 r3 p4 p5 p6 p7
    auto slice = [&](const int qb, const int k) {
      constexpr int kRead[4] = {0, 1, 4, 7};
      if (k == kRead[0] || k == kRead[1] || k == kRead[2] || k == kRead[3]) {
        const int g = k == kRead[0] ? 0 : k == kRead[1] ? 1 : k == kRead[2] ? 2 : 3;
        lg[g] = *reinterpret_cast<const f32x4*>(lsc + qb * 32 + 4 * h + 8 * g);
        dg[g] = *reinterpret_cast<const f32x4*>(dsc + qb * 32 + 4 * h + 8 * g);
      } else {
        const int m = k < 4 ? k - 2 : k < 7 ? k - 3 : k - 4;
        const int i = 2 * m, g = i >> 2, e = i & 3;
        const float p0 = fexp2(fmaf(sc[qb][i], c2, -lg[g][e]));
        const float p1 = fexp2(fmaf(sc[qb][i + 1], c2, -lg[g][e + 1]));
        put_pair(pk[qb][m >> 2], m & 3, p0, p1);
        put_pair(dk8[qb][m >> 2], m & 3, p0 * (dp[qb][i] - dg[g][e]), p1 * (dp[qb][i + 1] - dg[g][e + 1]));
      }
    };
    const int* rn = rowtab[b ^ 1];
    const int row0n = (t + 1) * kTile;
    const i32x4 winQ = GEO ? sQ.whole() : sQ.window(row0n), winO = GEO ? sO.whole() : sO.window(row0n);
    int grow = -1;
    auto load_row = [&](const int j) {  // geo phase 1
      if (j < NJQ) grow = sQ.geo_row(rn, wave, lane, j);
      else if (j < NJQ + NJO) grow = sO.geo_row(rn, wave, lane, j - NJQ);
      else grow = rn[lane];
    };
    auto issue_load = [&](const int j) {
      if (j < NJQ) {
        if (GEO) sQ.load_geo(Qn, winQ, grow, wave, lane, j);
        else sQ.load_dense_at(Qn, winQ, loff[j], wave, j);
      } else if (j < NJQ + NJO) {
        if (GEO) sO.load_geo(Qn + QB, winO, grow, wave, lane, j - NJQ);
        else sO.load_dense_at(Qn + QB, winO, loff[j], wave, j - NJQ);
      } else if (wave == 0) {
        if (GEO) sL.load_geo(lsn, grow, lane);
        else sL.load_dense(lsn, row0n, lane);
      } else if (wave == NW - 1) {
        if (GEO) sD.load_geo(dsn, grow, lane);
        else sD.load_dense(dsn, row0n, lane);
      }
    };
    auto side = [&](const int u) {
      if (u >= LOAD0 && (u - LOAD0) % LSTRIDE == 0 && (u - LOAD0) / LSTRIDE < NL) issue_load((u - LOAD0) / LSTRIDE);
      if (GEO && u + 2 >= LOAD0 && (u + 2 - LOAD0) % LSTRIDE == 0 && (u + 2 - LOAD0) / LSTRIDE < NL)
        load_row((u + 2 - LOAD0) / LSTRIDE);
      const int c = u / L, j = u % L;
      if (c != 1 && c != 2) return;
      static_for<SLICES>([&](auto k) {
        if (k * L / SLICES == j) slice(c - 1, k);
      });
    };

    bf16x8 ring[AH];
    static_for<AH>([&](auto u) { ring[u] = operand(u); });
    static_for<U>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 cur = ring[u % AH];
      if (u + AH < U) ring[u % AH] = operand(u + AH);
      mma_step(u, cur);
      side(u);
    });
    __builtin_amdgcn_sched_barrier(0);
    if (GEO && tid < kTile && t + 2 < ntiles) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
    wait_loads();
    __syncthreads();
  };
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(t, 0, sm0, sm1, ls0, ls1, ds0, ds1);
    step(t + 1, 1, sm1, sm0, ls1, ls0, ds1, ds0);
  }
  if (t < ntiles) step(t, 0, sm0, sm1, ls0, ls1, ds0, ds1);

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
    if (a.items != nullptr)                                                                                 \
      hipLaunchKernelGGL((tb::fwd_bf16<DD, KK, kWavesQ, true>), dim3(grid), dim3(kWavesQ * 64), 0, st, a);  \
    else                                                                                                    \
      hipLaunchKernelGGL((tb::fwd_bf16<DD, KK, kWavesQ, false>), dim3(grid), dim3(kWavesQ * 64), 0, st, a); \
    return hipGetLastError();                                                                               \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_dq_bf16(int D, int KP, const DqArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                       \
  if (D == DD && KP == KK) {                                                                                \
    if (a.items != nullptr)                                                                                 \
      hipLaunchKernelGGL((tb::dq_bf16<DD, KK, kWavesQ, true>), dim3(grid), dim3(kWavesQ * 64), 0, st, a);  \
    else                                                                                                    \
      hipLaunchKernelGGL((tb::dq_bf16<DD, KK, kWavesQ, false>), dim3(grid), dim3(kWavesQ * 64), 0, st, a); \
    return hipGetLastError();                                                                               \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_dkv_bf16(int D, int KP, const DkvArgs& a, int grid, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                       \
  if (D == DD && KP == KK) {                                                                                \
    if (a.items != nullptr)                                                                                 \
      hipLaunchKernelGGL((tb::dkv_bf16<DD, KK, kWavesK, true>), dim3(grid), dim3(kWavesK * 64), 0, st, a);  \
    else                                                                                                    \
      hipLaunchKernelGGL((tb::dkv_bf16<DD, KK, kWavesK, false>), dim3(grid), dim3(kWavesK * 64), 0, st, a); \
    return hipGetLastError();                                                                               \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
