// Host-visible argument blocks and launchers of the coupling kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace ssc {

enum class DType { F32 = 0, BF16 = 1 };

// Waves per workgroup of the bf16 kernels: query-side kernels (forward, dQ)
// own kWavesQ * 32 rows, the dK/dV kernel owns kWavesK * 32 source rows.
constexpr int kWavesQ = 4;
constexpr int kWavesK = 4;
// Rows owned by one workgroup of each bf16 kernel (work-item sizes).
constexpr int kRowsFwd = kWavesQ * 32; // forward
constexpr int kRowsDq = kWavesQ * 32;  // dQ
constexpr int kRowsDkv = kWavesK * 32; // dK / dV

// Work item of the row-block kernels: (patch, first row within the patch).
// One run of a gathered row stream (the rows of one patch, in order): the
// stream positions before `end` that are past the previous run map to rows
// position + base.
struct RunEntry {
  int end, base;
};

// A work item: rows row0 .. row0 + (rows per item) of a patch, and the
// tiles [t0, t1) of its gathered stream (t1 past the end = to the end).
// slot < 0: the item covers the whole stream and writes the outputs; slot
// >= 0: one part of a split item, whose partial sums go to partial-buffer
// slot `slot` and are combined by the merge pass in part order.
struct Item {
  int patch, row0, t0, t1, slot;
};

// A split item: its rows, number of parts and first partial-buffer slot.
struct SplitItem {
  int patch, row0, nparts, slot0;
};

// Geo scheduling: one round = one workgroup per CU of an MI355X (one
// workgroup of the bf16 block kernels fills a CU).  The items left over
// after the full rounds (the cheapest ones) are split into up to
// kMaxParts parts along their stream, so the last round is not a tail of a
// few long items; partial buffers hold at most kRoundCUs parts.
constexpr int kRoundCUs = 256;
constexpr int kMaxParts = 8;

// Forward: O = softmax(Q K^T scale) V over each row's key stream.
struct FwdArgs {
  const void* Q;        // caller's Q [n_N x D], patch-sorted rows
  const void* Kp;       // source rows, padded layout [npadM x D]
  const void* Vg;       // source V, grouped-transposed [npadM/16][KP][16]
  float* O;             // [n_N x k]
  float* lse;           // [n_N]
  int n_N, k;
  float c2;             // scale * log2(e)
  const Item* items;    // nullptr: dense (item = blockIdx.x)
  const int* n_items;
  const int* offN;      // geo: target offsets [P_N + 1]
  const int* idx;       // geo: [P_N x s]
  int s;
  const int* poffM;     // geo: padded source offsets
  const int* offM;      // geo: source offsets
  int npadM, n_M;       // dense key stream
  // bf16 kernels: Kp is the caller's K (row-major), Vp the k-padded copy of V,
  // run_tab [P_N][s] the run table of each target patch's key stream.
  const void* Vp;
  const RunEntry* run_tab;
  const float* knorm2;  // [kNormParts] partial maxima of |k_j|^2 over the key rows
  // geo splitting: partial sums [slot][field][256 threads] and split items
  float* part;
  const SplitItem* split;
  const int* n_split;
  // geo: the planner's verdict (nonzero: offsets or selection invalid; the
  // merge pass then fills the outputs with NaN)
  const int* status;
  // dense bf16: V grouped-transposed, [groupsVt][KP][16] (row k = ones)
  const void* Vt;
  int groupsVt;
  // dense bf16, paired-wave forward: per 128-row workgroup, 1 where a
  // row sum underflowed against the bounded reference (fwd_pair writes every
  // entry); fwd_bf16 given `fallback` redoes exactly those workgroups
  int* fallback_out;
  const int* fallback;
};

// Partial maxima of the squared key-row norms (bf16 forward): kNormParts
// workgroups, one partial each.
constexpr int kNormParts = 1024;
hipError_t launch_keynorm(const void* K, int n, int d, float* part, hipStream_t st);

// dQ pass.
struct DqArgs {
  const void* Qp;       // target rows, padded layout [npadN x D]
  const void* dOp;      // [npadN x KP]
  const float* lse2p;   // [npadN] lse * log2(e); +inf on padding
  const float* Dp;      // [npadN] rowdot(dO, O); 0 on padding
  const void* Kp;       // [npadM x D]
  const void* Vp;       // [npadM x KP]
  const void* Kg;       // [npadM/16][D][16]
  float* dQ;            // [n_N x D]
  int n_N;
  float c2, scale;
  const Item* items;
  const int* n_items;
  const int* offN;
  const int* poffN;
  const int* idx;
  int s;
  const int* poffM;
  const int* offM;
  int npadM, n_M;
  const RunEntry* run_tab;  // bf16 kernels (Qp, Kp = caller rows; lse2p, Dp by row)
  float* part;
  const SplitItem* split;
  const int* n_split;
  const int* status;        // geo: the planner's verdict (see FwdArgs)
};

// dK / dV pass.
struct DkvArgs {
  const void* Kp;       // [npadM x D]
  const void* Vp;       // [npadM x KP]
  const void* Qp;       // [npadN x D]
  const void* dOp;      // [npadN x KP]
  const void* Qg;       // [npadN/16][D][16]
  const void* dOg;      // [npadN/16][KP][16]
  const float* lse2p;
  const float* Dp;
  float* dK;            // [n_M x D]
  float* dV;            // [n_M x k]
  int n_M, k;
  float c2, scale;
  const Item* items;    // (source patch, first key row); nullptr: dense
  const int* n_items;
  const int* offM;
  const int* poffM;
  const int* inv_off;   // geo: [P_M + 1] CSR of target patches selecting q
  const int* inv_idx;
  const int* poffN;
  const int* offN;
  int npadN, n_N;       // dense query stream
  // bf16 kernels: run table of each source patch's query stream, entries
  // inv_tab[inv_off[q] .. inv_off[q+1]) (one per selecting target patch).
  const RunEntry* inv_tab;
  float* part;
  const SplitItem* split;
  const int* n_split;
  const int* status;    // geo: the planner's verdict (see FwdArgs)
};

// Packing of one tensor into the padded patch layout.
struct PackArgs {
  const void* X;        // [n x w] rows in patch-sorted order
  void* Xp;             // [npad x W] or nullptr
  void* Xg;             // [npad/16][W][16] or nullptr
  int n, w, W;
  int ones;             // columns w .. w + ones - 1 of every row present hold 1
  int dcol;             // with O: columns w, w + 1 hold -D as bf16 high + low parts
  const int* poff;      // nullptr: dense (position = row)
  const int* off;
  int P;
  const int* n_groups;  // geo: total groups (written by the planner)
  // rowdot / lse extras (target side only; may be nullptr)
  const float* O;       // [n x w]
  const float* lse;     // [n]
  float* Dp;            // [npad]
  float* lse2p;         // [npad]
};

// Planner of the geo layout: padded offsets, work items, inverse lists.
struct PlanArgs {
  const int* offN;
  const int* offM;
  const int* idx;
  int n_N, n_M, P_N, P_M, s;
  int* poffN;           // [P_N + 1]
  int* poffM;           // [P_M + 1]
  Item* itemsQ;         // row blocks of target patches
  Item* itemsK;         // row blocks of source patches
  int* counters;        // [0] n itemsQ, [1] n itemsK, [2] groups N, [3] groups M, [4] status,
                        // [5] n splitQ, [6] n splitK
  SplitItem* splitQ;    // [kRoundCUs] or nullptr (no splitting)
  SplitItem* splitK;    // [kRoundCUs] or nullptr
  int* inv_off;         // [P_M + 1] or nullptr
  int* inv_idx;         // [P_N * s]
  int* scratch;         // [3 (max(P_N, P_M) + 1)] per workgroup (two with inverse lists): scans
  int rowsQ, rowsK;     // rows per work item (target, source side)
  RunEntry* run_tab;    // [P_N * s] or nullptr: source runs of each target patch
  RunEntry* inv_tab;    // [P_N * s] or nullptr: target runs of each source patch
};

struct PoolArgs {
  const void* Q;
  const void* K;
  const int* offN;
  const int* offM;
  int n_N, n_M, P_N, P_M, d;
  double* Qbar;         // [P_N x d]
  double* KbarT;        // [d x P_M]
};

struct TopkArgs {
  const double* Qbar;
  const double* KbarT;
  int P_N, P_M, d, s;
  int* idx;
  double* scores;       // optional
};

// Linear-attention (ELU feature map) coupling: one argument block for all
// of its kernels.
constexpr int kLinGramRows = 256;  // least rows per workgroup of the Gram sums
struct LinArgs {
  const void* Q;        // [n_N x D] bf16
  const void* K;        // [n_M x D] bf16
  const void* V;        // [n_M x k] bf16
  const void* dO;       // [n_N x k] bf16 (backward)
  float* O;             // [n_N x k] (forward output; backward input)
  float* den;           // [n_N]     (forward output; backward input)
  float* rden;          // [n_N]     1 / den (backward scratch)
  float* s;             // [n_N]     (dO . O) / den (backward scratch)
  float* part;          // [nparts x D x KP] Gram partials (scratch)
  float* partN;         // backward: [nparts_N x D x KP] partials of the query-side Gram
  const void* M;        // [D x KP]  bf16 KVz_ext (row-major)
  const void* MT;       // [KP x D]  bf16 KVz_ext^T
  const void* dM;       // [D x KP]  bf16 dKVz_ext
  const void* dMT;      // [KP x D]  bf16 dKVz_ext^T
  // bf16 rounding remainders of the four matrices above (identity feature
  // map: each product runs on the high + low pair); null otherwise
  const void* Mlo;
  const void* MTlo;
  const void* dMlo;
  const void* dMTlo;
  float* dQ;            // [n_N x D]
  float* dK;            // [n_M x D]
  float* dV;            // [n_M x k]
  const float* rowoff;  // [n_N] identity feature map, forward: den is written as ln(den) + rowoff
  int n_N, n_M, k;
  int gram_rows;        // rows per workgroup of the Gram sums (a multiple of kLinGramRows)
};

// Performer (FAVOR+) coupling pieces (performer.hip); m = D random features.
struct PfArgs {
  const void* X;        // [n x D] bf16 rows (Q or K)
  const void* W;        // [M x D] bf16 random directions (rows), M features
  int n, nblk;          // rows; row blocks of 128
  float scale;          // softmax scale c (the features use sqrt(c))
  float* part;          // [nblk x M] per-block key maxima of the exponents (log2 units)
  float* M2;            // [M] per-feature key maximum (log2 units)
  bf16* F;              // [n x M] shifted features exp(...) (output of the feature passes)
  float* rowoff;        // [n] queries, forward: ln den - ln(den of the shifted features)
  const float* lnden;   // [n] queries, backward: ln den from the forward
  float* den;           // [n] queries, backward: den of the shifted features
  const float* dF;      // [n x M] gradient w.r.t. the shifted features (pf_dx)
  float* dX;            // [n x D] gradient w.r.t. the rows (pf_dx output)
};
// D = d, M = m in {64, 128}.  Per-block maxima of the key exponents (a.part).
hipError_t launch_pf_keymax(int D, int M, const PfArgs& a, hipStream_t st);
// key features (ak) and query features (aq) in one launch; qmode 2: with the
// row offset (forward), 3: with den from ln den (backward)
hipError_t launch_pf_feat_kq(int D, int M, int qmode, const PfArgs& ak, const PfArgs& aq, hipStream_t st);
hipError_t launch_pf_maxreduce(int M, const PfArgs& a, hipStream_t st);
// mode 0: queries (no row-sum term), 1: keys
// the query rows (aq, mode 0) and the key rows (ak, mode 1) of dX in one launch
hipError_t launch_pf_dx2(int D, int M, const PfArgs& aq, const PfArgs& ak, hipStream_t st);

// Functional-map solve after the coupling (fmap.hip): C = (Phi^T Phi)^-1 Phi^T O
// and its backward dO = Phi (Phi^T Phi)^-1 dC.
constexpr int kFmMaxK = 256;
struct FmArgs {
  const void* Phi;      // [n x k] bf16
  const float* O;       // [n x k] (forward)
  const float* dC;      // [k x k] (backward)
  float* part;          // [nblk][nprod][KP x KP] Gram partials (G; forward also R)
  float* G;             // [KP x KP] Phi^T Phi (lower 32-blocks)
  float* R;             // [KP x KP] Phi^T O (forward)
  float* Lrow;          // [k (k + 1) / 2] Cholesky factor packed by rows
  float* Lcol;          // [k (k + 1) / 2] the same packed by columns
  float* rdiag;         // [k] 1 / L_ii
  float* C;             // [k x k] (forward output)
  bf16* X;              // [KP x KP] G^-1 dC, zero padded (backward)
  float* dO;            // [n x k] (backward output)
  int n, k;
  int rows;             // rows per Gram block (a multiple of 64)
};
// Gram blocking for n rows at padded width KP (rows per block, block count).
void fm_blocks(int n, int KP, int* rows, int* nblk);

// Geodesic farthest-point-sampling partition (fps.hip).  Meshes whose
// vertices have at most kFpsSlots neighbours also get a padded adjacency.
constexpr int kFpsSlots = 8;
struct FpsArgs {
  const double* x;      // [n x 3] vertex positions
  const int* off;       // [n + 1] CSR offsets of the adjacency
  const int* adj;       // [nnz] neighbour indices (both directions of every edge)
  int n, nnz, P;
  int* seeds;           // [P] output: seed vertices in sampling order
  int* labels;          // [n] output: index of the nearest seed
  double* dist;         // [n] output (and working field): distance to the nearest seed
  double* w;            // [nnz] edge lengths (workspace)
  int* adjp;            // [n x kFpsSlots] neighbours per vertex, -1 past its degree (workspace)
  double* wp;           // [n x kFpsSlots] their edge lengths (workspace)
  int* stamp;           // [n] round in whose queue a vertex sits (workspace)
  int* queue;           // [2 n] frontier worklists of two rounds (workspace)
  unsigned long long* cmax;  // [nchunk] per-chunk maximum distance bits (workspace)
  int* cflag;           // [nchunk] chunk touched by the current step (workspace)
  int* bad;             // [nblk] per-block adjacency check (workspace)
  int nchunk, nblk;
  struct FpsCtl* ctl;   // control block of the multi-workgroup steps (workspace)
  int wide_steps;       // steps 0 .. wide_steps - 1 run on many workgroups (0: none)
  int wide_blocks;      // their workgroups (at most one per CU)
  int wide_frontier;    // a step whose largest round queue stays below this ends them
  unsigned spin;        // polls a grid-barrier wait may take before it gives up
};
// Control block of the multi-workgroup steps, zeroed by fps_prep.
struct FpsCtl {
  unsigned long long bar;  // grid-barrier arrivals
  int abort;               // a barrier wait gave up: the one-workgroup kernel redoes every step
  int status;              // 0: not run, 2: a step exceeded its round bound, 3: steps 0 .. t_end - 1 done
  int t_end, r_end;        // steps done and rounds run by the multi-workgroup kernel
  int cnt[3];              // queue counters of three consecutive rounds
  int pad[7];
};
static_assert(sizeof(FpsCtl) == 64, "FpsCtl layout");
// meshes from this many vertices run their first steps on many workgroups
constexpr int kFpsWideMin = 32768;
hipError_t launch_fps(const FpsArgs& a, hipStream_t st);

// Launchers (return hipGetLastError() after the launch).
hipError_t launch_fwd(DType t, int D, int KP, const FwdArgs& a, int grid, hipStream_t st);
// ones: column k of the padded V holds ones (k < KP); KP = 256 also runs
// without (k = 256)
hipError_t launch_fwd_bf16(int D, int KP, bool ones, const FwdArgs& a, int grid, hipStream_t st);
// paired-wave dense forward (8 waves, 128 rows a workgroup; needs k < KP)
hipError_t launch_fwd_pair(int D, int KP, const FwdArgs& a, int grid, hipStream_t st);
// wide-wave dense forward (4 waves, 256 rows a workgroup; needs k < KP <= 224);
// taken from kWideMinWGs workgroups on
constexpr int kWideMinWGs = 128;
hipError_t launch_fwd_wide(int D, int KP, const FwdArgs& a, int grid, hipStream_t st);
// dcol: V carries two ones columns and dO the high / low parts of -D there
// (k + 2 <= KP), so dP - D comes out of the MFMAs; KP = 256 also runs without
hipError_t launch_dq_bf16(int D, int KP, bool dcol, const DqArgs& a, int grid, hipStream_t st);
// dv: also form dV (false: dK only, a.dV unused)
hipError_t launch_dkv_bf16(int D, int KP, bool dcol, bool dv, const DkvArgs& a, int grid, hipStream_t st);
hipError_t launch_fm_gram(int KP, bool fwd, const FmArgs& a, int nblk, hipStream_t st);
hipError_t launch_fm_reduce(int KP, bool fwd, const FmArgs& a, int nblk, hipStream_t st);
hipError_t launch_fm_chol(int KP, const FmArgs& a, hipStream_t st);
hipError_t launch_fm_solve(int KP, int mode, const FmArgs& a, hipStream_t st);
hipError_t launch_fm_apply(int KP, const FmArgs& a, hipStream_t st);
// merge passes of split geo items (kRoundCUs workgroups, idle past the count)
hipError_t launch_fwd_merge_bf16(int D, int KP, bool ones, const FwdArgs& a, hipStream_t st);
hipError_t launch_dq_merge_bf16(int D, const DqArgs& a, hipStream_t st);
hipError_t launch_dkv_merge_bf16(int D, int KP, bool dv, const DkvArgs& a, hipStream_t st);
// Offsets check (debug builds): *flag = 1 unless off[0] = 0, off[P] = n and
// the entries do not decrease, for both offset arrays (one workgroup each)
hipError_t launch_check_offsets(const int* offN, int P_N, int n_N, const int* offM, int P_M, int n_M, int* flag,
                                hipStream_t st);
// Grouped-transposed bf16 copy: Xg[j / 16][c][j % 16] = X[j][c] for c < w,
// j < n (X [n x w] rows); rows w .. w + ones - 1 hold 1 for j < n; every other
// entry of the (npad / 16) x W x 16 array (npad a multiple of 64) is 0.
hipError_t launch_transpose_bf16(const void* X, int n, int w, int W, int ones, void* Xt, int npad, hipStream_t st);
// NaN into up to three fp32 outputs when *status is nonzero (a rejected geo
// plan); otherwise the workgroups exit at once
hipError_t launch_invalid_fill(const int* status, float* x0, size_t n0, float* x1, size_t n1, float* x2, size_t n2,
                               hipStream_t st);
hipError_t launch_dq(DType t, int D, int KP, const DqArgs& a, int grid, hipStream_t st);
hipError_t launch_dkv(DType t, int D, int KP, const DkvArgs& a, int grid, hipStream_t st);
bool supported(DType t, int D, int KP);
hipError_t launch_pack(DType t, const PackArgs& a, int grid, hipStream_t st);
// launch_pack takes the bf16 row-padding kernel for these jobs (and its
// 16-byte vector form for pad_bf16_vec ones)
bool pad_bf16_applies(DType t, const PackArgs& a);
bool pad_bf16_vec(const PackArgs& a);
hipError_t launch_plan(const PlanArgs& a, hipStream_t st);
// the plan and up to two bf16 row-padding jobs (pad_bf16_applies, grid =
// 16-row groups) in one launch
hipError_t launch_plan_pad(const PlanArgs& a, const PackArgs* jobs, const int* grids, int njobs, hipStream_t st);
hipError_t launch_pool(DType t, const PoolArgs& a, hipStream_t st);
// p[0..11]: offsets of one patch per side ({0, n_N} at p, {0, n_M} at p + 4)
// and its selection ({0} at p + 8), the rest zero
hipError_t launch_one_patch(int* p, int n_N, int n_M, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// ident: the rows of Q / K are precomputed features (identity feature map)
// Forward Gram sums phi(K)^T V_ext over `grid` row blocks into a.part.
hipError_t launch_lin_gram(int D, int KP, bool ident, const LinArgs& a, int grid, hipStream_t st);
// Backward: both Gram sums in one launch (gM key-row blocks into a.part, gN
// query-row blocks into a.partN; the query side also writes a.rden and a.s).
hipError_t launch_lin_gram_bwd(int D, int KP, bool ident, const LinArgs& a, int gM, int gN, hipStream_t st);
// Mlo / MTlo (optional, may be null): the bf16 rounding remainders
hipError_t launch_lin_reduce(int D, int KP, const float* part, int nparts, void* M, void* MT, void* Mlo, void* MTlo,
                             hipStream_t st);
// the backward's two reductions in one launch
hipError_t launch_lin_reduce2(int D, int KP, const float* part0, int nparts0, void* M0, void* MT0, void* Mlo0,
                              void* MTlo0, const float* part1, int nparts1, void* M1, void* MT1, void* Mlo1,
                              void* MTlo1, hipStream_t st);
// forward rows: O and den
hipError_t launch_lin_apply(int D, int KP, bool ident, const LinArgs& a, hipStream_t st);
// backward rows in one launch: dQ, dK and dV
hipError_t launch_lin_apply_bwd(int D, int KP, bool ident, const LinArgs& a, hipStream_t st);

}  // namespace ssc
