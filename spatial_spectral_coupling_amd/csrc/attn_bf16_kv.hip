// bf16 dK / dV kernel of the spatial-spectral coupling on gfx950 (project
// page "Spatial-Spectral Coupling as Attention", sections "How it works" and
// "Geo-FlashAttention").
#include "tile_bf16.hpp"

namespace ssc {
namespace tb {

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
// Output of one source row (held by lanes l and l ^ 32): dK = scale * dk, dV.
template <int D, int KP, bool DV>
__device__ __forceinline__ void dkv_store(const DkvArgs& a, int krow, bool key_ok, int h, const f32x16* dk,
                                          const f32x16* dv) {
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
    if (!DV) return;
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

template <int D, int KP, int NW, bool GEO, bool DCOL, bool DV>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void dkv_bf16(DkvArgs a) {
  constexpr int QB = TileSrc<D, NW>::ALLOC, OB = TileSrc<KP, NW>::ALLOC;
  __shared__ __attribute__((aligned(1024))) char sm0[QB + OB];
  __shared__ __attribute__((aligned(1024))) char sm1[QB + OB];
  __shared__ __attribute__((aligned(16))) float ls0[kTile];
  __shared__ __attribute__((aligned(16))) float ls1[kTile];
  __shared__ __attribute__((aligned(16))) float ds0[kTile];
  __shared__ __attribute__((aligned(16))) float ds1[kTile];
  __shared__ int rowtab[2][kTile + 1];  // rows of the next tiles, sentinel at kTile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int tr_r = 4 * h + ((lane & 15) >> 2), tr_c = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  int k_begin, k_end;
  RowCursor rc;
  Item it{0, 0, 0, 0, -1};
  // gathered query rows missing from a tile read the sentinel row n_N + 1
  // (past the end of Q, of the padded dO and of lse2 / D)
  if (!GEO) {
    k_begin = blockIdx.x * (NW * 32);
    k_end = a.n_M;
    rc = RowCursor{nullptr, 1, a.n_N, a.n_N + 1};
  } else {
    if ((int)blockIdx.x >= *a.n_items) return;
    it = a.items[blockIdx.x];
    k_begin = a.offM[it.patch] + it.row0;
    k_end = a.offM[it.patch + 1];
    const int i0 = a.inv_off[it.patch];
    const int nr = a.inv_off[it.patch + 1] - i0;
    const RunEntry* tab = a.inv_tab + i0;
    rc = RowCursor{tab, nr, nr > 0 ? tab[nr - 1].end : 0, a.n_N + 1};
  }
  const int total = rc.total;
  const int ntiles = (total + kTile - 1) / kTile;
  // tiles [t0, t1) of the stream (one part of a split item, or all of it)
  const int t0 = GEO ? it.t0 : 0, t1 = GEO ? min(it.t1, ntiles) : ntiles;
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
  // A geo item's waves past the patch's last row own no keys: they take
  // part in the loads and barriers only.
  const bool wave_keys = !GEO || k_begin + wave * 32 < k_end;

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

  // without DV the dV accumulators are never touched (no MFMA, no store)
  f32x16 dv[DV ? KP / 32 : 1], dk[D / 32];
#pragma unroll
  for (int cb = 0; cb < (DV ? KP / 32 : 1); ++cb) dv[cb] = f32x16{};
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dk[db] = f32x16{};

  if (GEO && tid < kTile) {
    rc.init();
    rowtab[0][tid] = rc.row(t0 * kTile + tid);
    rowtab[1][tid] = rc.row((t0 + 1) * kTile + tid);
    if (tid == 0) rowtab[0][kTile] = rowtab[1][kTile] = rc.none;
  }
  __syncthreads();
  if (t1 > t0) {
    sQ.template load_tile<GEO>(sm0, rowtab[0], t0 * kTile, wave, lane);
    sO.template load_tile<GEO>(sm0 + QB, rowtab[0], t0 * kTile, wave, lane);
    if (wave == 0) {
      if (GEO) sL.load_geo(ls0, rowtab[0][lane], lane);
      else sL.load_dense(ls0, t0 * kTile, lane);
    }
    if (!DCOL && wave == NW - 1) {
      if (GEO) sD.load_geo(ds0, rowtab[0][lane], lane);
      else sD.load_dense(ds0, t0 * kTile, lane);
    }
  }
  wait_loads();
  __syncthreads();

  // One tile = 64 query rows = two 32-row blocks qb.  Its MFMAs form four
  // chains run as one software pipeline:
  //   c = 0, 1: scores S = Q K^T and dP = dO V^T of block c (row reads), L
  //             steps each;
  //   c = 2, 3: dV += P^T dO and dK += dS^T Q of block c - 2 (transposed
  //             reads), 2 (KP/32 + D/32) independent accumulators in turn
  //             (2 D/32 without DV: dK only), LB steps each.
  // Operand reads run AH steps ahead of their MFMA (also across chain
  // boundaries), and the softmax of block qb (P, dS and their bf16
  // packing) is cut into slices spread over chain qb + 1, so that its VALU
  // work issues while that chain's MFMAs execute.  Scheduling fences between
  // steps keep this order.
  constexpr int NA = D / 16, NB = KP / 16, PAIRS = NA < NB ? NA : NB;
  constexpr int NV = DV ? KP / 32 : 0, NK = D / 32, NVK = NV + NK;
  constexpr int L = NA + NB;
  constexpr int LB = 2 * NVK;
  static_assert(!DV || L == LB, "chain lengths");
  constexpr int C2 = 2 * L, C3 = 2 * L + LB, U = 2 * L + 2 * LB, AH = 3;
  // chain of step u and the step's index within it
  auto chain_of = [](const int u) { return u < L ? 0 : u < C2 ? 1 : u < C3 ? 2 : 3; };
  auto index_in = [](const int u) { return u < L ? u : u < C2 ? u - L : u < C3 ? u - C2 : u - C3; };
  auto chain_len = [](const int c) { return c < 2 ? L : LB; };
  constexpr int SLICES = 12;  // 4 lse/D group reads, 8 element pairs
  // Direct loads of the next tile, spread over the first half of the
  // pipeline: NJQ + NJO tile loads and one lse or D vector load per wave.
  // The last tile loads a clamped (valid) copy into the idle buffer.
  constexpr int NJQ = TileSrc<D, NW>::NJ, NJO = TileSrc<KP, NW>::NJ;
  constexpr int NL = NJQ + NJO + 1, LOAD0 = 2, LSTRIDE = (U / 2 - LOAD0) / NL > 2 ? (U / 2 - LOAD0) / NL : 2;
  // dense: the per-lane tile load offsets do not depend on the tile
  int loff[NJQ + NJO];
  static_for<NJQ + NJO>([&](auto j) {
    loff[j] = GEO ? (j < NJQ ? TileSrc<D, NW>::geo_chunk(wave, lane, j) : TileSrc<KP, NW>::geo_chunk(wave, lane, j - NJQ))
                  : (j < NJQ ? TileSrc<D, NW>::dense_offset(wave, lane, j)
                             : TileSrc<KP, NW>::dense_offset(wave, lane, j - NJQ));
  });
  // geo: the row-table entry each load reads (the vector load: this lane's row)
  int gidx[NL];
  static_for<NL>([&](auto j) {
    gidx[j] = !GEO ? 0 : j < NJQ ? TileSrc<D, NW>::geo_index(wave, lane, j)
                      : j < NJQ + NJO ? TileSrc<KP, NW>::geo_index(wave, lane, j - NJQ) : lane;
  });

  // Two statically distinct buffers: the step that reads one fills the other.
  auto step = [&](auto keys_c, const int t, const int b, char* Qt, char* Qn, const float* lsc, float* lsn,
                  const float* dsc, float* dsn) __attribute__((always_inline)) {
    constexpr bool KEYS = decltype(keys_c)::value;  // false: loads and barrier only
    char* Ot = Qt + QB;
    f32x16 sc[2], dp[2];
    bf16x8 pk[2][2], dk8[2][2];
    f32x4 lg[4], dg[4];
    sc[0] = sc[1] = dp[0] = dp[1] = f32x16{};

    auto operand = [&](const int u) -> bf16x8 {
      const int c = chain_of(u), j = index_in(u);
      if (c < 2) {
        if (j < 2 * PAIRS) return (j & 1) ? ro.read(Ot, c, j >> 1) : rq.read(Qt, c, j >> 1);
        return NA > NB ? rq.read(Qt, c, j - PAIRS) : ro.read(Ot, c, j - PAIRS);
      }
      const int qb = c - 2, kk = j / NVK, m = j % NVK;
      return m < NV ? to.frag(Ot, m, 2 * qb + kk) : tq.frag(Qt, m - NV, 2 * qb + kk);
    };
    auto mma_step = [&](const int u, const bf16x8& x) {
      const int c = chain_of(u), j = index_in(u);
      if (c < 2) {
        const bool is_s = j < 2 * PAIRS ? (j & 1) == 0 : NA > NB;
        const int chunk = j < 2 * PAIRS ? j >> 1 : j - PAIRS;
        if (is_s) sc[c] = mma(x, kf[chunk], sc[c]);
        else dp[c] = mma(x, vf[chunk], dp[c]);
        return;
      }
      const int qb = c - 2, kk = j / NVK, m = j % NVK;
      if (m < NV) {
        if constexpr (DV) dv[m] = mma(x, pk[qb][kk], dv[m]);
      } else {
        dk[m - NV] = mma(x, dk8[qb][kk], dk[m - NV]);
      }
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
        if (!DCOL) dg[g] = *reinterpret_cast<const f32x4*>(dsc + qb * 32 + 4 * h + 8 * g);
      } else {
        const int m = k < 4 ? k - 2 : k < 7 ? k - 3 : k - 4;
        const int i = 2 * m, g = i >> 2, e = i & 3;
        const float p0 = fexp2(fmaf(sc[qb][i], c2, -lg[g][e]));
        const float p1 = fexp2(fmaf(sc[qb][i + 1], c2, -lg[g][e + 1]));
        if (DV) put_pair(pk[qb][m >> 2], m & 3, p0, p1);
        // with DCOL the ones / -D columns already made dp = dP - D
        const float e0 = DCOL ? dp[qb][i] : dp[qb][i] - dg[g][e];
        const float e1 = DCOL ? dp[qb][i + 1] : dp[qb][i + 1] - dg[g][e + 1];
        put_pair(dk8[qb][m >> 2], m & 3, p0 * e0, p1 * e1);
      }
    };
    const int* rn = rowtab[b ^ 1];
    const int row0n = (t + 1) * kTile;
    const i32x4 winQ = GEO ? sQ.whole() : sQ.window(row0n), winO = GEO ? sO.whole() : sO.window(row0n);
    int grow = -1;
    auto load_row = [&](const int j) {  // geo phase 1
      grow = rn[gidx[j]];
    };
    auto issue_load = [&](const int j) {
      if (j < NJQ) {
        if (GEO) sQ.load_geo_at(Qn, winQ, grow, loff[j], wave, j);
        else sQ.load_dense_at(Qn, winQ, loff[j], wave, j);
      } else if (j < NJQ + NJO) {
        if (GEO) sO.load_geo_at(Qn + QB, winO, grow, loff[j], wave, j - NJQ);
        else sO.load_dense_at(Qn + QB, winO, loff[j], wave, j - NJQ);
      } else {
        // even waves fetch lse, odd waves D (duplicate fetches write the
        // same values; with DCOL every wave fetches lse); a wave-uniform
        // select, no branch in the pipeline
        const bool odd = !DCOL && (wave & 1);
        const VecSrc src = odd ? sD : sL;
        float* dst = odd ? dsn : lsn;
        if (GEO) src.load_geo(dst, grow, lane);
        else src.load_dense(dst, row0n, lane);
      }
    };
    auto side = [&](const int u) {
      if (u >= LOAD0 && (u - LOAD0) % LSTRIDE == 0 && (u - LOAD0) / LSTRIDE < NL) issue_load((u - LOAD0) / LSTRIDE);
      if (GEO && u + 2 >= LOAD0 && (u + 2 - LOAD0) % LSTRIDE == 0 && (u + 2 - LOAD0) / LSTRIDE < NL)
        load_row((u + 2 - LOAD0) / LSTRIDE);
      if (!KEYS) return;
      const int c = chain_of(u), j = index_in(u);
      if (c != 1 && c != 2) return;
      static_for<SLICES>([&](auto k) {
        if (k * chain_len(c) / SLICES == j) slice(c - 1, k);
      });
    };

    bf16x8 ring[AH];
    if (KEYS) static_for<AH>([&](auto u) { ring[u] = operand(u); });
    static_for<U>([&](auto u) {
      __builtin_amdgcn_sched_barrier(0);
      if (KEYS) {
        const bf16x8 cur = ring[u % AH];
        if (u + AH < U) ring[u % AH] = operand(u + AH);
        mma_step(u, cur);
      }
      side(u);
    });
    __builtin_amdgcn_sched_barrier(0);
    if (GEO && tid < kTile && t + 2 < t1) rowtab[b][tid] = rc.row((t + 2) * kTile + tid);
    wait_loads();
    __syncthreads();
  };
  auto run = [&](auto keys_c) __attribute__((always_inline)) {
    int t = t0;
    for (; t + 1 < t1; t += 2) {
      step(keys_c, t, 0, sm0, sm1, ls0, ls1, ds0, ds1);
      step(keys_c, t + 1, 1, sm1, sm0, ls1, ls0, ds1, ds0);
    }
    if (t < t1) step(keys_c, t, 0, sm0, sm1, ls0, ls1, ds0, ds1);
  };
  if (GEO && !wave_keys) {
    // no keys, no outputs (the merge of a split item stores existing keys
    // only, so this wave's rows of the partial buffer may stay unwritten)
    run(std::false_type{});
    return;
  }
  run(std::true_type{});

  if (GEO && it.slot >= 0) {
    // one part of a split item: partial sums for the merge pass
    constexpr int F = (D / 32 + (DV ? KP / 32 : 0)) * 16;
    float* out = a.part + (size_t)it.slot * F * (NW * 64) + tid;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) out[(db * 16 + i) * (NW * 64)] = dk[db][i];
    if constexpr (DV) {
#pragma unroll
      for (int cb = 0; cb < KP / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) out[((D / 32 + cb) * 16 + i) * (NW * 64)] = dv[cb][i];
    }
    return;
  }
  dkv_store<D, KP, DV>(a, krow, key_ok, h, dk, dv);
}

// Merge of the parts of split items: dK = scale * sum, dV = sum (part order),
// one workgroup per 32-column block (D/32 of dK, then KP/32 of dV with DV).
template <int D, int KP, int NW, bool DV>
__global__ __launch_bounds__(NW * 64) void dkv_merge_bf16(DkvArgs a) {
  constexpr int NK = D / 32, NB = NK + (DV ? KP / 32 : 0);
  if (*a.status != 0) {
    // the planner rejected the offsets or the selection: nothing was computed
    fill_nan_grid(a.dK, (size_t)a.n_M * D);
    if (DV) fill_nan_grid(a.dV, (size_t)a.n_M * a.k);
    return;
  }
  const int item = blockIdx.x / NB, blk = blockIdx.x - item * NB;
  if (item >= *a.n_split) return;
  const SplitItem sp = a.split[item];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int krow = a.offM[sp.patch] + sp.row0 + wave * 32 + l32;
  const bool key_ok = krow < a.offM[sp.patch + 1];
  constexpr int F = NB * 16, T = NW * 64;
  const float* in = a.part + (size_t)sp.slot0 * F * T + (size_t)blk * 16 * T + tid;
  // all loads of a part are issued before its sums
  float sum[16];
  static_for<16>([&](auto f) { sum[f] = 0.f; });
  for (int q = 0; q < sp.nparts; ++q) {
    const float* pq = in + (size_t)q * F * T;
    float v[16];
    static_for<16>([&](auto f) { v[f] = __builtin_nontemporal_load(pq + f * T); });
    static_for<16>([&](auto f) { sum[f] += v[f]; });
  }
  if (!key_ok) return;
  if (blk < NK) {
    float* okr = a.dK + (size_t)krow * D;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = blk * 32 + 8 * g + 4 * h;
      *reinterpret_cast<f32x4*>(okr + c) =
          f32x4{a.scale * sum[4 * g], a.scale * sum[4 * g + 1], a.scale * sum[4 * g + 2], a.scale * sum[4 * g + 3]};
    }
    return;
  }
  if (!DV) return;
  float* ovr = a.dV + (size_t)krow * a.k;
  const bool vec = (a.k & 3) == 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int c = (blk - NK) * 32 + 8 * g + 4 * h;
    if (vec) {
      if (c < a.k) *reinterpret_cast<f32x4*>(ovr + c) = f32x4{sum[4 * g], sum[4 * g + 1], sum[4 * g + 2], sum[4 * g + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (c + e < a.k) ovr[c + e] = sum[4 * g + e];
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

hipError_t launch_dkv_bf16(int D, int KP, bool dcol, bool dv, const DkvArgs& a, int grid, hipStream_t st) {
#define SSC_L2(DD, KK, CC, VV)                                                                                      \
  if (a.items != nullptr)                                                                                         \
    hipLaunchKernelGGL((tb::dkv_bf16<DD, KK, kWavesK, true, CC, VV>), dim3(grid), dim3(kWavesK * 64), 0, st, a);  \
  else                                                                                                            \
    hipLaunchKernelGGL((tb::dkv_bf16<DD, KK, kWavesK, false, CC, VV>), dim3(grid), dim3(kWavesK * 64), 0, st, a); \
  return hipGetLastError();
#define SSC_L1(DD, KK, CC)      \
  if (dv) {                     \
    SSC_L2(DD, KK, CC, true)    \
  } else {                      \
    SSC_L2(DD, KK, CC, false)   \
  }
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
#undef SSC_L2
  return hipErrorInvalidValue;
}

hipError_t launch_dkv_merge_bf16(int D, int KP, bool dv, const DkvArgs& a, hipStream_t st) {
#define SSC_L(DD, KK)                                                                                           \
  if (D == DD && KP == KK) {                                                                                    \
    if (dv)                                                                                                     \
      hipLaunchKernelGGL((tb::dkv_merge_bf16<DD, KK, kWavesK, true>), dim3(kRoundCUs * (DD / 32 + KK / 32)),    \
                         dim3(kWavesK * 64), 0, st, a);                                                         \
    else                                                                                                        \
      hipLaunchKernelGGL((tb::dkv_merge_bf16<DD, KK, kWavesK, false>), dim3(kRoundCUs * (DD / 32)),             \
                         dim3(kWavesK * 64), 0, st, a);                                                         \
    return hipGetLastError();                                                                                   \
  }
  SSC_BF16_INSTANCES(SSC_L)
#undef SSC_L
  return hipErrorInvalidValue;
}

}  // namespace ssc
