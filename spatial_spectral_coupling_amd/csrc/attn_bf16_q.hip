// bf16 forward and dQ kernels of the spatial-spectral coupling on gfx950
// (project page "Spatial-Spectral Coupling as Attention", sections "How it
// works" and "Geo-FlashAttention").  Built with MFMA results in VGPRs
// (-mllvm -amdgpu-mfma-vgpr-form=1, see build.py): their softmax reads the
// score accumulators with plain VALU instructions.
#include "tile_bf16.hpp"

namespace ssc {
namespace tb {

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
// (row maximum if tracked, exp2, bf16 packing) runs in slices during chain 1,
// that of half 1 during chain 2.  The next tile's direct loads are spread
// over the first half of the pipeline; scheduling fences between steps keep
// this order.
//
// Row sums: with ONES, column k of the padded V holds 1 for every source
// row (0 past the end), so the PV MFMAs also accumulate the row sums of the
// bf16 probabilities in that column of O; without a spare column (k = KP)
// the softmax slices add them up.
//
// Softmax reference.  First pass: one fixed reference per row, the bound
// c2 |q| max_j |k_j| on its scores, so no probability exceeds 1 and no row
// maximum is tracked.  Only if that bound sits so far above a row's scores
// that its row sum falls below 2^-60 (an underflow risk) does the workgroup
// redo its rows with a running reference: the probabilities of a tile are
// taken relative to a reference fixed for the whole tile (the first tile:
// the maximum of its first half; later tiles: the running reference), and
// the accumulators are rescaled only between tiles, when the running maximum
// has moved more than 8 (log2 units) above the reference.  A tile whose
// maximum exceeds its reference by more than 32 could overflow; a workgroup
// that saw one redoes its rows once more with the exact row maxima as a
// fixed reference, so the result is exact in every case.
// Output of one row (held by lanes l and l ^ 32): O = acc / l and lse in
// natural log, from the accumulators relative to reference m.
template <int KP, bool ONES>
__device__ __forceinline__ void fwd_store(const FwdArgs& a, int row, bool row_ok, int h, const f32x16* acc, float l_run,
                                          float m) {
  float l_part = l_run;
  if (ONES) {
    // the row sum sits in column k of O, held by the lanes of one half
    l_part = 0.f;
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (cb * 32 + c_row(i, h) == a.k) l_part = acc[cb][i];
  }
  const float l_tot = l_part + xor32(l_part);
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
    if (h == 0) a.lse[row] = l_tot > 0.f ? (m + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// VT (dense only): V arrives grouped-transposed (a.Vt, groups of 16 source
// rows as [KP][16] blocks), the key rows are read in the sigma_row order, so
// every value-product operand is one 16-byte read of the transposed tile
// (GroupReader) instead of two transposed reads of a row tile.
template <int D, int KP, int NW, bool GEO, bool ONES, bool VT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void fwd_bf16(FwdArgs a) {
  static_assert(!(GEO && VT), "the transposed value tile is dense only");
  constexpr int KB = TileSrc<D, NW>::ALLOC, VB = VT ? TileSrcG<KP, NW>::ALLOC : TileSrc<KP, NW>::ALLOC;
  __shared__ __attribute__((aligned(1024))) char sm0[KB + VB];
  __shared__ __attribute__((aligned(1024))) char sm1[KB + VB];
  __shared__ int rowtab[2][kTile + 1];  // rows of the next tiles, sentinel at kTile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int q_begin, q_end;
  RowCursor rc;
  Item it{0, 0, 0, 0, -1};
  // gathered key rows missing from a tile read the sentinel row n_M + 1
  // (past the end of K and of the padded V)
  if (!GEO) {
    // after the paired-wave forward: only the workgroups it marked
    if (VT && a.fallback != nullptr && a.fallback[blockIdx.x] == 0) return;
    q_begin = blockIdx.x * (NW * 32);
    q_end = a.n_N;
    rc = RowCursor{nullptr, 1, a.n_M, a.n_M + 1};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    it = a.items[blockIdx.x];
    q_begin = a.offN[it.patch] + it.row0;
    q_end = a.offN[it.patch + 1];
    const RunEntry* tab = a.run_tab + (size_t)it.patch * a.s;
    rc = RowCursor{tab, a.s, tab[a.s - 1].end, a.n_M + 1};
  }
  const int total = rc.total;
  const int ntiles = (total + kTile - 1) / kTile;
  // tiles [t0, t1) of the stream (one part of a split item, or all of it)
  const int t0 = GEO ? it.t0 : 0, t1 = GEO ? min(it.t1, ntiles) : ntiles;
  // streamed source rows: K (n_M rows) and the k-padded V (n_M + 1 rows,
  // a zero row at n_M)
  TileSrc<D, NW> sK;
  sK.init(a.Kp, a.n_M);
  TileSrc<KP, NW> sV;
  sV.init(a.Vp, a.n_M + 1);
  TileSrcG<KP, NW> sVt;
  if (VT) sVt.init(a.Vt, a.groupsVt);
  const int row = q_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;
  // A geo item's waves past the patch's last row own no rows: they take
  // part in the loads and barriers only (not at KP = 256, where the second
  // copy of the pipeline would spill).
  const bool wave_rows = !GEO || KP > 224 || q_begin + wave * 32 < q_end;

  const bf16* Q = reinterpret_cast<const bf16*>(a.Q);
  std::conditional_t<VT, RowReaderP<D>, RowReader<D>> rk;
  rk.init(l32, h);
  TrReader<KP> tv;
  tv.init(tr_r, tr_c);
  GroupReader rvt;
  rvt.init(l32, h);
  // key of C-layout element i (lane group h) within a 32-key half
  auto key_of = [&](const int i) { return VT ? sigma_row(c_row(i, h)) : c_row(i, h); };

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
  // Bounded reference: every score of this row is at most |q| max_j |k_j|
  // (Cauchy-Schwarz), so probabilities relative to c2 |q| Kmax never exceed 1
  // and need no running maximum.  Kmax comes from the per-workgroup partial
  // maxima of the key-row norms.
  float m_bound;
  {
    float qn2 = 0.f;
#pragma unroll
    for (int dc = 0; dc < D / 16; ++dc)
#pragma unroll
      for (int e = 0; e < 8; ++e) qn2 = fmaf((float)qf[dc][e], (float)qf[dc][e], qn2);
    qn2 += xor32(qn2);
    float km2 = 0.f;
    for (int j = lane; j < kNormParts; j += 64) km2 = fmaxf(km2, a.knorm2[j]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) km2 = fmaxf(km2, __shfl_xor(km2, m, 64));
    m_bound = c2 * sqrtf(qn2 * km2);
  }

  f32x16 acc[KP / 32];
  // Initial score accumulators: zero, except in a partial last tile, where
  // keys at or past its end start at -inf (their probabilities are then 0).
  f32x16 bias[2];
  float m_run, l_run, m_true = -INFINITY;
  // mode 0: bounded reference; 1: running reference (when the bound left a
  // row sum below 2^-60, i.e. the bound was far above the scores); 2: the
  // exact row maxima of mode 1 as a fixed reference.  A workgroup redone
  // after the paired-wave forward (which ran mode 0) starts in mode 1.
  int mode = (!GEO && VT && a.fallback != nullptr) ? 1 : 0;

  constexpr int NS = D / 16, NCB = KP / 32, NPV = 2 * NCB;
  constexpr int C1 = NS, C2 = 2 * NS, C3 = 2 * NS + NPV, U = 2 * NS + 2 * NPV, AH = 5;
  constexpr int SLICES = 10;  // 2 maximum, 8 element pairs
  constexpr int NJK = TileSrc<D, NW>::NJ, NJV = VT ? TileSrcG<KP, NW>::NJ : TileSrc<KP, NW>::NJ;
  constexpr int NL = NJK + NJV, LOAD0 = 2, LSTRIDE = (U / 2 - LOAD0) / NL > 2 ? (U / 2 - LOAD0) / NL : 2;
  // dense: the per-lane load offsets do not depend on the tile; kept in registers
  int loff[NL];
  static_for<NL>([&](auto j) {
    loff[j] = GEO ? (j < NJK ? TileSrc<D, NW>::geo_chunk(wave, lane, j) : TileSrc<KP, NW>::geo_chunk(wave, lane, j - NJK))
                  : (j < NJK ? TileSrc<D, NW>::dense_offset(wave, lane, j)
                             : VT ? (int)TileSrcG<KP, NW>::dense_offset(wave, lane, j - NJK)
                                  : TileSrc<KP, NW>::dense_offset(wave, lane, j - NJK));
  });
  // geo: the row-table entry each load reads
  int gidx[NL];
  static_for<NL>([&](auto j) {
    gidx[j] = !GEO ? 0 : j < NJK ? TileSrc<D, NW>::geo_index(wave, lane, j)
                                 : TileSrc<KP, NW>::geo_index(wave, lane, j - NJK);
  });
  // the whole tile at t0 (the stream's first tile of this item)
  auto load_first = [&](char* tile) {
    sK.template load_tile<GEO>(tile, rowtab[0], t0 * kTile, wave, lane);
    if constexpr (VT) {
      const i32x4 w = sVt.window(t0 * kGroupsPerTile);
      static_for<NJV>([&](auto j) { sVt.load_at(tile + KB, w, (unsigned)loff[NJK + j], wave, j); });
    } else {
      sV.template load_tile<GEO>(tile + KB, rowtab[0], t0 * kTile, wave, lane);
    }
  };

  // row sum of this lane's row (both halves)
  auto row_sum = [&]() {
    float l_part = l_run;
    if (ONES) {
      // the row sum sits in column k of O, held by the lanes of one half
      l_part = 0.f;
#pragma unroll
      for (int cb = 0; cb < KP / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (cb * 32 + c_row(i, h) == a.k) l_part = acc[cb][i];
    }
    return l_part + xor32(l_part);
  };

  for (;;) {
    const bool fixed = mode == 2;
#pragma unroll
    for (int cb = 0; cb < KP / 32; ++cb) acc[cb] = f32x16{};
    bias[0] = bias[1] = f32x16{};
    l_run = 0.f;
    m_run = mode == 0 ? m_bound : fixed ? m_true : -INFINITY;
    bool lagged = false;

    if (GEO && tid < kTile) {
      rc.init();
      rowtab[0][tid] = rc.row(t0 * kTile + tid);
      rowtab[1][tid] = rc.row((t0 + 1) * kTile + tid);
      if (tid == 0) rowtab[0][kTile] = rowtab[1][kTile] = rc.none;
    }
    __syncthreads();
    if (t1 > t0) load_first(sm0);
    wait_loads();
    __syncthreads();

    // Two statically distinct buffers: the step that reads one fills the
    // other, so the compiler can tell the direct loads in flight from the LDS
    // reads.  The stream's last tile may be partial: its keys at or past
    // nvalid start from a score of -inf (bias, set before the pipeline).
    auto step = [&](auto bound_c, auto rows_c, const int t, const int b, char* Kt, char* Kn)
                    __attribute__((always_inline)) {
      constexpr bool BOUND = decltype(bound_c)::value;
      constexpr bool ROWS = decltype(rows_c)::value;  // false: loads and barrier only
      char* Vt = Kt + KB;
      const int nvalid = total - t * kTile;
      const bool first = !BOUND && t == t0 && !fixed;
      // Keys past the end of the last tile: with VT, the bounded reference and
      // the row sums taken from the ones column they need no mask (K and the
      // transposed V read zeros there, so their probabilities are at most 1
      // and multiply zero values and a zero ones column); otherwise their
      // scores start at -inf.
      constexpr bool MASK = !(VT && BOUND && ONES);
      if (MASK && __builtin_expect(nvalid < kTile, 0)) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 16; ++i) bias[hb][i] = hb * 32 + key_of(i) < nvalid ? 0.f : -INFINITY;
      }
      f32x16 sc[2];
      float sv[2][16];
      bf16x8 pf[2][2];
      float mx[2], mh[2], mref = m_run, lsum = 0.f;
      sc[0] = MASK ? bias[0] : f32x16{};
      sc[1] = MASK ? bias[1] : f32x16{};

      auto operand = [&](const int u) -> bf16x8 {
        if (u < C2) return rk.read(Kt, u / NS, u % NS);
        const int hb = u < C3 ? 0 : 1, j = u - (hb ? C3 : C2);
        if constexpr (VT) return rvt.read(Vt, j % NCB, 2 * hb + j / NCB);
        else return tv.frag(Vt, j % NCB, 2 * hb + j / NCB);
      };
      auto mma_step = [&](const int u, const bf16x8& x) {
        if (u < C2) {
          sc[u / NS] = mma(x, qf[u % NS], sc[u / NS]);
          return;
        }
        const int hb = u < C3 ? 0 : 1, j = u - (hb ? C3 : C2);
        acc[j % NCB] = mma(x, pf[hb][j / NCB], acc[j % NCB]);
      };
      // Slice k of the softmax of key half hb (the scores are copied once out
      // of the MFMA accumulators into sv): 0, 1 copy and row maximum (the
      // first tile takes its reference from half 0); 2..9 element pairs
      // 2m, 2m+1 = 2(k-2) .. : exp2, row sum and packed bf16 probabilities.
      auto slice = [&](const int hb, const int k) {
        if (k <= 1) {
#pragma unroll
          for (int i = 8 * k; i < 8 * k + 8; ++i) sv[hb][i] = sc[hb][i];
          if (BOUND) return;
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
          if (!ONES) lsum += p0 + p1;
          put_pair(pf[hb][m >> 2], m & 3, p0, p1);
        }
      };
      const int* rn = rowtab[b ^ 1];
      const int row0n = (t + 1) * kTile;
      const i32x4 winK = GEO ? sK.whole() : sK.window(row0n);
      const i32x4 winV = GEO ? sV.whole() : VT ? sVt.window((t + 1) * kGroupsPerTile) : sV.window(row0n);
      int grow = -1;
      auto load_row = [&](const int j) {  // geo phase 1
        grow = rn[gidx[j]];
      };
      auto issue_load = [&](const int j) {
        if (j < NJK) {
          if (GEO) sK.load_geo_at(Kn, winK, grow, loff[j], wave, j);
          else sK.load_dense_at(Kn, winK, loff[j], wave, j);
        } else {
          if (GEO) sV.load_geo_at(Kn + KB, winV, grow, loff[j], wave, j - NJK);
          else if (VT) sVt.load_at(Kn + KB, winV, (unsigned)loff[j], wave, j - NJK);
          else sV.load_dense_at(Kn + KB, winV, loff[j], wave, j - NJK);
        }
      };
      auto side = [&](const int u) {
        if (u >= LOAD0 && (u - LOAD0) % LSTRIDE == 0 && (u - LOAD0) / LSTRIDE < NL) issue_load((u - LOAD0) / LSTRIDE);
        if (GEO && u + 2 >= LOAD0 && (u + 2 - LOAD0) % LSTRIDE == 0 && (u + 2 - LOAD0) / LSTRIDE < NL)
          load_row((u + 2 - LOAD0) / LSTRIDE);
        if (!ROWS) return;
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
      if (ROWS) static_for<AH>([&](auto u) { ring[u] = operand(u); });
      static_for<U>([&](auto u) {
        __builtin_amdgcn_sched_barrier(0);
        if (ROWS) {
          const bf16x8 cur = ring[u % AH];
          if (u + AH < U) ring[u % AH] = operand(u + AH);
          mma_step(u, cur);
        }
        side(u);
      });
      __builtin_amdgcn_sched_barrier(0);

      // Between tiles: the sums of this tile join the running sum at the
      // tile's reference; move the reference up when the maximum ran ahead.
      l_run += lsum;
      if (!BOUND && ROWS) {
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
      }
      if (GEO && tid < kTile && t + 2 < t1) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
      wait_loads();
      __syncthreads();
    };
    auto run = [&](auto bound_c) __attribute__((always_inline)) {
      const int nt = t1 - t0;  // (this loop form keeps the accumulators in registers)
      if (!GEO || KP > 224 || wave_rows) {
        for (int i = 0; i < nt; i += 2) {
          step(bound_c, std::true_type{}, t0 + i, 0, sm0, sm1);
          if (i + 1 < nt) step(bound_c, std::true_type{}, t0 + i + 1, 1, sm1, sm0);
        }
      } else {
        for (int i = 0; i < nt; i += 2) {
          step(bound_c, std::false_type{}, t0 + i, 0, sm0, sm1);
          if (i + 1 < nt) step(bound_c, std::false_type{}, t0 + i + 1, 1, sm1, sm0);
        }
      }
    };
    if (mode == 0) {
      run(std::true_type{});
      const float lt = row_sum();
      if (!__syncthreads_or(t1 > t0 && row_ok && !(lt >= 0x1p-60f))) break;
      mode = 1;
      continue;
    }
    run(std::false_type{});
    if (fixed || !__syncthreads_or(lagged)) break;
    mode = 2;
  }

  if (GEO && it.slot >= 0) {
    // one part of a split item: partial sums for the merge pass
    constexpr int F = (KP / 32) * 16 + 2;
    float* out = a.part + (size_t)it.slot * F * (NW * 64) + tid;
    static_for<(KP / 32) * 16>([&](auto f) {
      constexpr int cb = f / 16, i = f % 16;
      out[f * (NW * 64)] = acc[cb][i];
    });
    out[(F - 2) * (NW * 64)] = m_run;
    out[(F - 1) * (NW * 64)] = l_run;
    return;
  }
  fwd_store<KP, ONES>(a, row, row_ok, h, acc, l_run, m_run);
}

// Merge of the parts of split items (one workgroup per split item and
// 32-column block of O, the producer's thread layout).  A part's sums are relative to its own
// reference m_q (the bound, or a running maximum where that part fell back),
// so the parts are combined at the reference of the largest part mass,
// M = max_q (m_q + log2 l_q): acc = sum_q 2^(m_q - M) acc_q, where every
// weighted part sum stays <= 1 and a part only underflows when its mass is
// below 2^-126 of the largest.
template <int D, int KP, int NW, bool ONES>
__global__ __launch_bounds__(NW * 64) void fwd_merge_bf16(FwdArgs a) {
  // every block recomputes the rows' common reference, weights and row sums
  // with the same operations in the same order (so the blocks agree bit for
  // bit); block 0 writes lse
  constexpr int NB = KP / 32;
  if (*a.status != 0) {
    // the planner rejected the offsets or the selection: nothing was computed
    fill_nan_grid(a.O, (size_t)a.n_N * a.k);
    fill_nan_grid(a.lse, (size_t)a.n_N);
    return;
  }
  const int item = blockIdx.x / NB, cb = blockIdx.x - item * NB;
  if (item >= *a.n_split) return;
  const SplitItem sp = a.split[item];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int row = a.offN[sp.patch] + sp.row0 + wave * 32 + l32;
  const bool row_ok = row < a.offN[sp.patch + 1];
  constexpr int F = NB * 16 + 2, T = NW * 64;
  const float* in = a.part + (size_t)sp.slot0 * F * T + tid;
  // row sum of part q (both halves of the row); with ONES, column k of O is
  // field (k/32) 16 + 4 ((k%32)/8) + k%4 of the lanes of half ((k%32)/4) % 2
  const int kk = a.k & 31, hk = (kk >> 2) & 1, fk = (a.k >> 5) * 16 + 4 * (kk >> 3) + (kk & 3);
  // every part's values are loaded first (at most kMaxParts), then combined
  // in part order: the reference m, then the weighted sums
  float ref[kMaxParts], lh[kMaxParts], lt[kMaxParts], v[kMaxParts][16];
  static_for<kMaxParts>([&](auto q) {
    if (q < sp.nparts) {
      const float* pq = in + (size_t)q * F * T;
      ref[q] = pq[(F - 2) * T];
      lh[q] = ONES ? (h == hk ? pq[(size_t)fk * T] : 0.f) : pq[(F - 1) * T];
      static_for<16>([&](auto i) { v[q][i] = pq[(cb * 16 + i) * T]; });
    }
  });
  static_for<kMaxParts>([&](auto q) {
    if (q < sp.nparts) lt[q] = lh[q] + xor32(lh[q]);
  });
  float m = -INFINITY;
  static_for<kMaxParts>([&](auto q) {
    if (q < sp.nparts && lt[q] > 0.f) m = fmaxf(m, ref[q] + log2f(lt[q]));
  });
  float acc[16];
  static_for<16>([&](auto i) { acc[i] = 0.f; });
  float l = 0.f;  // this half's row sum (with ONES: column k, on its half only)
  static_for<kMaxParts>([&](auto q) {
    if (q < sp.nparts) {
      const float w = lt[q] > 0.f ? fexp2(ref[q] - m) : 0.f;
      static_for<16>([&](auto i) { acc[i] = fmaf(w, v[q][i], acc[i]); });
      l = fmaf(w, lh[q], l);
    }
  });
  const float l_tot = l + xor32(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!row_ok) return;
  float* Orow = a.O + (size_t)row * a.k;
  const bool vec = (a.k & 3) == 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = cb * 32 + 8 * g + 4 * h;
    if (vec) {
      if (c < a.k)
        *reinterpret_cast<f32x4*>(Orow + c) =
            f32x4{acc[4 * g] * inv, acc[4 * g + 1] * inv, acc[4 * g + 2] * inv, acc[4 * g + 3] * inv};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e < a.k) Orow[c + e] = acc[4 * g + e] * inv;
    }
  }
  if (cb == 0 && h == 0) a.lse[row] = l_tot > 0.f ? (m + log2f(l_tot)) * kLn2 : -INFINITY;
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
template <int D>
__device__ __forceinline__ void dq_store(const DqArgs& a, int row, bool row_ok, int h, const f32x16* dq) {
  if (!row_ok) return;
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

template <int D, int KP, int NW, bool GEO, bool DCOL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void dq_bf16(DqArgs a) {
  constexpr int KB = TileSrc<D, NW>::ALLOC, VB = TileSrc<KP, NW>::ALLOC;
  __shared__ __attribute__((aligned(1024))) char sm0[KB + VB];
  __shared__ __attribute__((aligned(1024))) char sm1[KB + VB];
  __shared__ int rowtab[2][kTile + 1];  // rows of the next tiles, sentinel at kTile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int q_begin, q_end;
  RowCursor rc;
  Item it{0, 0, 0, 0, -1};
  // gathered key rows missing from a tile read the sentinel row n_M + 1
  // (past the end of K and of the padded V)
  if (!GEO) {
    q_begin = blockIdx.x * (NW * 32);
    q_end = a.n_N;
    rc = RowCursor{nullptr, 1, a.n_M, a.n_M + 1};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    it = a.items[blockIdx.x];
    q_begin = a.offN[it.patch] + it.row0;
    q_end = a.offN[it.patch + 1];
    const RunEntry* tab = a.run_tab + (size_t)it.patch * a.s;
    rc = RowCursor{tab, a.s, tab[a.s - 1].end, a.n_M + 1};
  }
  const int total = rc.total;
  const int ntiles = (total + kTile - 1) / kTile;
  // tiles [t0, t1) of the stream (one part of a split item, or all of it)
  const int t0 = GEO ? it.t0 : 0, t1 = GEO ? min(it.t1, ntiles) : ntiles;
  // streamed source rows: K (n_M rows) and the k-padded V (n_M + 1 rows,
  // a zero row at n_M)
  TileSrc<D, NW> sK;
  sK.init(a.Kp, a.n_M);
  TileSrc<KP, NW> sV;
  sV.init(a.Vp, a.n_M + 1);
  const int row = q_begin + wave * 32 + l32;
  const bool row_ok = row < q_end;
  // A geo item's waves past the patch's last row own no rows: they take
  // part in the loads and barriers only.
  const bool wave_rows = !GEO || q_begin + wave * 32 < q_end;

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
  // dP accumulators end at dP - D: with DCOL the ones / -D columns of V and
  // dO subtract D inside the MFMAs, otherwise they start at -D
  const float Dq = !DCOL && row_ok ? a.Dp[row] : 0.f;
  f32x16 dinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) dinit[i] = -Dq;
  const float c2 = a.c2;

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  if (GEO && tid < kTile) {
    rc.init();
    rowtab[0][tid] = rc.row(t0 * kTile + tid);
    rowtab[1][tid] = rc.row((t0 + 1) * kTile + tid);
    if (tid == 0) rowtab[0][kTile] = rowtab[1][kTile] = rc.none;
  }
  __syncthreads();
  if (t1 > t0) {
    sK.template load_tile<GEO>(sm0, rowtab[0], t0 * kTile, wave, lane);
    sV.template load_tile<GEO>(sm0 + KB, rowtab[0], t0 * kTile, wave, lane);
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
    loff[j] = GEO ? (j < NJK ? TileSrc<D, NW>::geo_chunk(wave, lane, j) : TileSrc<KP, NW>::geo_chunk(wave, lane, j - NJK))
                  : (j < NJK ? TileSrc<D, NW>::dense_offset(wave, lane, j)
                             : TileSrc<KP, NW>::dense_offset(wave, lane, j - NJK));
  });
  // geo: the row-table entry each load reads
  int gidx[NL];
  static_for<NL>([&](auto j) {
    gidx[j] = !GEO ? 0 : j < NJK ? TileSrc<D, NW>::geo_index(wave, lane, j)
                                 : TileSrc<KP, NW>::geo_index(wave, lane, j - NJK);
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
  // Initial score accumulators of the two key halves: zero, except in a
  // partial last tile, where keys at or past its end start at -inf (P = dS
  // = 0 for them).
  f32x16 bias[2];
  bias[0] = bias[1] = f32x16{};
  static_for<16>([&](auto ic) {
    constexpr int i = ic, k = i / 2;
    sc1[i] = k * WIN / SLICES < LB ? 0.f : -INFINITY;
  });
  dp1 = f32x16{};
  ds1[0] = ds1[1] = bf16x8{};
#pragma unroll
  for (int j = 0; j < LB; ++j) kt[j] = bf16x8{};

  // Slice k of the softmax of one half (scores sv, dv = dP - D, packed dS
  // out): element pair 2k, 2k+1 (P = exp2(S c2 - lse2), dS = P (dP - D))
  // packed into out.
  auto slice = [&](f32x16& sv, f32x16& dv, bf16x8* out, const int k) {
    const float d0 = fexp2(fmaf(sv[2 * k], c2, -lse2)) * dv[2 * k];
    const float d1 = fexp2(fmaf(sv[2 * k + 1], c2, -lse2)) * dv[2 * k + 1];
    put_pair(out[k >> 2], k & 3, d0, d1);
  };

  // Iteration t: the MFMAs of A0(t), B1(t-1), A1(t), B0(t) as one pipeline;
  // the softmax of half 0 runs during B1(t-1) and A1(t), that of half 1
  // during B0(t) and A0(t+1), so each has a 30-step window.  Two statically
  // distinct buffers: the step that reads one fills the other.
  auto step = [&](auto rows_c, const int t, const int b, char* Kt, char* Kn) __attribute__((always_inline)) {
    constexpr bool ROWS = decltype(rows_c)::value;  // false: loads and barrier only
    char* Vt = Kt + KB;
    const int nvalid = total - t * kTile;
    if (ROWS && nvalid < kTile) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) bias[kb][i] = kb * 32 + c_row(i, h) < nvalid ? 0.f : -INFINITY;
    }
    f32x16 sc0 = bias[0], dp0 = dinit;
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
      grow = rn[gidx[j]];
    };
    auto issue_load = [&](const int j) {
      if (j < NJK) {
        if (GEO) sK.load_geo_at(Kn, winK, grow, loff[j], wave, j);
        else sK.load_dense_at(Kn, winK, loff[j], wave, j);
      } else {
        if (GEO) sV.load_geo_at(Kn + KB, winV, grow, loff[j], wave, j - NJK);
        else sV.load_dense_at(Kn + KB, winV, loff[j], wave, j - NJK);
      }
    };
    auto side = [&](const int u) {
      if (u >= LOAD0 && (u - LOAD0) % LSTRIDE == 0 && (u - LOAD0) / LSTRIDE < NL) issue_load((u - LOAD0) / LSTRIDE);
      if (GEO && u + 2 >= LOAD0 && (u + 2 - LOAD0) % LSTRIDE == 0 && (u + 2 - LOAD0) / LSTRIDE < NL)
        load_row((u + 2 - LOAD0) / LSTRIDE);
      if (!ROWS) return;
      if (u < CY) {
        // half 1 of the previous tile: window positions LB .. WIN-1
        static_for<SLICES>([&](auto k) {
          if (k * WIN / SLICES >= LB && k * WIN / SLICES - LB == u) slice(sc1, dp1, ds1, k);
        });
      } else if (u < CW) {
        // half 0 of this tile: window positions 0 .. WIN-1 over B1 and A1
        static_for<SLICES>([&](auto k) {
          if (k * WIN / SLICES == u - CY) slice(sc0, dp0, ds0, k);
        });
      } else {
        // half 1 of this tile, window positions 0 .. LB-1; and its K^T
        // fragments for the B1 chain of the next iteration
        static_for<SLICES>([&](auto k) {
          if (k * WIN / SLICES < LB && k * WIN / SLICES == u - CW) slice(sc1, dp1, ds1, k);
        });
        const int j = u - CW;
        kt[j] = tk.frag(Kt, j % NK, 2 + j / NK);
      }
    };
    auto pre = [&](const int u) {
      if (u == CZ) {  // A1(t) starts: fresh accumulators for half 1
        sc1 = bias[1];
        dp1 = dinit;
      }
    };

    bf16x8 ring[AH];
    if (ROWS) static_for<AH>([&](auto u) { ring[u] = operand(u); });
    static_for<U>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      if (ROWS) {
        const bf16x8 cur = ring[u % AH];
        if (u + AH < U) ring[u % AH] = operand(u + AH);
        pre(u);
        mma_step(u, cur);
      }
      side(u);
    });
    __builtin_amdgcn_sched_barrier(0);
    if (GEO && tid < kTile && t + 2 < t1) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
    wait_loads();
    __syncthreads();
  };
  if (!GEO || wave_rows) {
    for (int t = t0; t < t1; t += 2) {
      step(std::true_type{}, t, 0, sm0, sm1);
      if (t + 1 < t1) step(std::true_type{}, t + 1, 1, sm1, sm0);
    }
    // drain: the rest of the last tile's half-1 softmax, then its B1 chain
    static_for<SLICES>([&](auto k) {
      if (k * WIN / SLICES >= LB) slice(sc1, dp1, ds1, k);
    });
    static_for<LB>([&](auto j) { dq[j % NK] = mma(kt[j], ds1[j / NK], dq[j % NK]); });
  } else {
    for (int t = t0; t < t1; t += 2) {
      step(std::false_type{}, t, 0, sm0, sm1);
      if (t + 1 < t1) step(std::false_type{}, t + 1, 1, sm1, sm0);
    }
  }

  if (GEO && it.slot >= 0) {
    // one part of a split item: partial sums for the merge pass
    constexpr int F = (D / 32) * 16;
    float* out = a.part + (size_t)it.slot * F * (NW * 64) + tid;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) out[(db * 16 + i) * (NW * 64)] = dq[db][i];
    return;
  }
  dq_store<D>(a, row, row_ok, h, dq);
}

// Merge of the parts of split items: dQ = scale * (sum of the parts, in part
// order), one workgroup per split item and 32-column block.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void dq_merge_bf16(DqArgs a) {
  constexpr int NB = D / 32;
  if (*a.status != 0) {
    fill_nan_grid(a.dQ, (size_t)a.n_N * D);
    return;
  }
  const int item = blockIdx.x / NB, db = blockIdx.x - item * NB;
  if (item >= *a.n_split) return;
  const SplitItem sp = a.split[item];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int row = a.offN[sp.patch] + sp.row0 + wave * 32 + l32;
  const bool row_ok = row < a.offN[sp.patch + 1];
  constexpr int F = NB * 16, T = NW * 64;
  const float* in = a.part + (size_t)sp.slot0 * F * T + (size_t)db * 16 * T + tid;
  // all loads of a part are issued before its sums
  float sum[16];
  static_for<16>([&](auto f) { sum[f] = 0.f; });
  for (int q = 0; q < sp.nparts; ++q) {
    const float* pq = in + (size_t)q * F * T;
    float v[16];
    static_for<16>([&](auto f) { v[f] = __builtin_nontemporal_load(pq + f * T); });
    static_for<16>([&](auto f) { sum[f] += v[f]; });
  }
  if (!row_ok) return;
  float* out = a.dQ + (size_t)row * D;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = db * 32 + 8 * g + 4 * h;
    *reinterpret_cast<f32x4*>(out + c) =
        f32x4{a.scale * sum[4 * g], a.scale * sum[4 * g + 1], a.scale * sum[4 * g + 2], a.scale * sum[4 * g + 3]};
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

// The forward takes the row sums from a ones column of V whenever k < KP;
// only KP = 256 also has the variant without one (k = 256).
hipError_t launch_fwd_bf16(int D, int KP, bool ones, const FwdArgs& a, int grid, hipStream_t st) {
#define SSC_L1(DD, KK, OO)                                                                                          \
  if (a.items != nullptr)                                                                                         \
    hipLaunchKernelGGL((tb::fwd_bf16<DD, KK, kWavesQ, true, OO, false>), dim3(grid), dim3(kWavesQ * 64), 0, st, a); \
  else                                                                                                            \
    hipLaunchKernelGGL((tb::fwd_bf16<DD, KK, kWavesQ, false, OO, true>), dim3(grid), dim3(kWavesQ * 64), 0, st, a); \
  return hipGetLastError();
#define SSC_L(DD, KK)                   \
  if (ones && D == DD && KP == KK) {    \
    SSC_L1(DD, KK, true)                \
  }
  SSC_BF16_INSTANCES(SSC_L)
  if (!ones && KP == 256) {
    if (D == 128) {
      SSC_L1(128, 256, false)
    }
    if (D == 64) {
      SSC_L1(64, 256, false)
    }
  }
#undef SSC_L
#undef SSC_L1
  return hipErrorInvalidValue;
}

hipError_t launch_dq_bf16(int D, int KP, bool dcol, const DqArgs& a, int grid, hipStream_t st) {
#define SSC_L1(DD, KK, CC)                                                                                   \
  if (a.items != nullptr)                                                                                  \
    hipLaunchKernelGGL((tb::dq_bf16<DD, KK, kWavesQ, true, CC>), dim3(grid), dim3(kWavesQ * 64), 0, st, a);  \
  else                                                                                                     \
    hipLaunchKernelGGL((tb::dq_bf16<DD, KK, kWavesQ, false, CC>), dim3(grid), dim3(kWavesQ * 64), 0, st, a); \
  return hipGetLastError();
#define SSC_L(DD, KK)                   \
  if (dcol && D == DD && KP == KK) {    \
    SSC_L1(DD, KK, true)                \
  }
  SSC_BF16_INSTANCES(SSC_L)
  if (!dcol && KP == 256) {
    if (D == 128) {
      SSC_L1(128, 256, false)
    }
    if (D == 64) {
      SSC_L1(64, 256, false)
    }
  }
#undef SSC_L
#undef SSC_L1
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_merge_bf16(int D, int KP, bool ones, const FwdArgs& a, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                          \
  if (D == DD && KP == KK) {                                                                                   \
    if (ones)                                                                                                  \
      hipLaunchKernelGGL((tb::fwd_merge_bf16<DD, KK, kWavesQ, true>), dim3(kRoundCUs * (KK / 32)), dim3(kWavesQ * 64), \
                         0, st, a);                                                                                \
    else                                                                                                       \
      hipLaunchKernelGGL((tb::fwd_merge_bf16<DD, KK, kWavesQ, false>), dim3(kRoundCUs * (KK / 32)),             \
                         dim3(kWavesQ * 64), 0, st, a);                                                        \
    return hipGetLastError();                                                                                  \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

hipError_t launch_dq_merge_bf16(int D, const DqArgs& a, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL((tb::dq_merge_bf16<128, kWavesQ>), dim3(kRoundCUs * 4), dim3(kWavesQ * 64), 0, st, a);
  else if (D == 64)
    hipLaunchKernelGGL((tb::dq_merge_bf16<64, kWavesQ>), dim3(kRoundCUs * 2), dim3(kWavesQ * 64), 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ssc
