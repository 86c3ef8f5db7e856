/*
 * ssc.h -- spatial-spectral coupling on AMD Instinct MI355X (gfx950).
 *
 * The coupling of deep functional-map pipelines is the product
 *     Pi_NM Phi_M = softmax(F_N F_M^T * scale) Phi_M,
 * i.e. scaled dot-product attention with Q = F_N (target descriptors,
 * n_N x d), K = F_M (source descriptors, n_M x d) and V = Phi_M (source
 * Laplace-Beltrami basis, n_M x k); the softmax runs over source vertices
 * for every target vertex and scale is 1/sqrt(d) for the pages' coupling
 * ("Spatial-Spectral Coupling as Attention", project page, section
 * "How it works"; the map Pi_NM itself is never formed, section
 * "The bottleneck").
 *
 * Two variants, each with forward and backward:
 *   dense  -- the exact coupling;
 *   geo    -- Geo-FlashAttention (section "Geo-FlashAttention" and its
 *             pipeline figure): both shapes are split into patches, source
 *             keys are pooled per patch, source patches are scored against
 *             each target patch, the top s are kept, and every target row
 *             takes the exact softmax over the union of its patch's selected
 *             source patches only.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers to dense row-major arrays
 *   (row stride = width, no separate leading-dimension argument: the tile
 *   loads address rows by a compile-time width), 16-byte aligned.  A strided
 *   view must be made contiguous by the caller.  The caller owns every buffer;
 *   the library never allocates device memory.  Scratch space comes from
 *   the caller through (ws, ws_bytes); ssc_workspace_bytes() gives the size.
 * - dtype selects the storage of Q, K, V and dO: SSC_BF16 (bf16 bits,
 *   MFMA bf16 x bf16 -> fp32) or SSC_F32 (fp32 MFMA).  O, lse, dQ, dK, dV
 *   are always fp32.  lse is in natural log.
 * - Supported shapes: d in {64, 128}; 1 <= k <= 256 (padded internally to
 *   the next of 32, 64, 128, 224, 256); n_M >= 1; n_N >= 0 (n_N = 0: a
 *   forward computes nothing, a backward writes dK = dV = 0, and Q, O, dO,
 *   lse and dQ may be NULL); n_N, n_M <= 2^22 for the couplings (larger ->
 *   SSC_ERR_UNSUPPORTED).
 *   fp32 inputs: k <= 128.  Geo: 1 <= P_N, P_M <= 8192, 1 <= s <= P_M.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *   stream) and re-entrant: no global mutable state (the optional kernel
 *   timer below is per thread), no host sync.
 *   Argument validation happens before any HIP call; on failure nothing is
 *   launched and an error status is returned.  SSC_ERR_HIP means a launch
 *   failed; ssc_last_hip_error() returns that hipError_t (thread-local).
 * - Workspaces must not be shared by calls that may run concurrently.
 * - Outputs must not overlap inputs.  Non-finite inputs are undefined.
 */
#ifndef SSC_H
#define SSC_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSC_OK = 0,
  SSC_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment, overlap */
  SSC_ERR_UNSUPPORTED = 2,  /* d, k, P, s or a row count outside the compiled set */
  SSC_ERR_WORKSPACE = 3,    /* ws too small (or NULL with ws_bytes > 0) */
  SSC_ERR_HIP = 4           /* a HIP launch failed */
} ssc_status;

/* The dtype and op enumerations each carry two range markers (never valid
 * arguments): with them every 32-bit int is a value of the type, so a caller
 * passing an unknown code through the ABI gets SSC_ERR_INVALID_ARG or
 * SSC_ERR_UNSUPPORTED (0 from ssc_workspace_bytes) rather than undefined
 * behaviour. */
typedef enum {
  SSC_F32 = 0,
  SSC_BF16 = 1,
  SSC_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  SSC_DTYPE_RANGE_MAX_ = 2147483647
} ssc_dtype;

typedef enum {
  SSC_OP_DENSE_FWD = 0,
  SSC_OP_DENSE_BWD = 1,
  SSC_OP_PATCH_TOPK = 2,
  SSC_OP_GEO_FWD = 3,
  SSC_OP_GEO_BWD = 4,
  SSC_OP_LINEAR_FWD = 5,
  SSC_OP_LINEAR_BWD = 6,
  SSC_OP_FMAP_FWD = 7,
  SSC_OP_FMAP_BWD = 8,
  SSC_OP_FPS = 9,
  SSC_OP_PERFORMER_FWD = 10,
  SSC_OP_PERFORMER_BWD = 11,
  SSC_OP_RANGE_MIN_ = -2147483647 - 1,
  SSC_OP_RANGE_MAX_ = 2147483647
} ssc_op;

typedef void* ssc_stream; /* hipStream_t */

/* Bytes of scratch an entry point needs for these sizes (0 if the sizes are
 * invalid).  Arguments not used by an op are ignored.  For SSC_OP_FPS:
 * n_N = vertex count n, n_M = adjacency length nnz, P_N = seed count P.
 * For SSC_OP_PERFORMER_*: P_N = feature count m (0 means m = d). */
size_t ssc_workspace_bytes(ssc_op op, ssc_dtype dtype, int n_N, int n_M, int d, int k,
                           int P_N, int P_M, int s);

/*
 * Dense forward (project page, "How it works"):
 *   O[i, :] = sum_j softmax_j(scale * Q[i].K[j]) V[j, :],
 *   lse[i]  = log sum_j exp(scale * Q[i].K[j]).
 * Q [n_N x d], K [n_M x d], V [n_M x k] in `dtype`; O [n_N x k] fp32,
 * lse [n_N] fp32.
 */
ssc_status coupling_dense_fwd(ssc_dtype dtype, int n_N, int n_M, int d, int k,
                              const void* Q, const void* K, const void* V, float scale,
                              float* O, float* lse, void* ws, size_t ws_bytes,
                              ssc_stream stream);

/*
 * Dense backward: gradients of <dO, O> for the coupling above (project page,
 * "How it works": the pipelines train through the product Pi_NM Phi_M, so
 * the descriptors F_N = Q and F_M = K receive gradients through it;
 * "The bottleneck": the map is never stored), recomputing the softmax from
 * lse:
 *   D_i = sum_c dO_ic O_ic,  dS = P * (dO V^T - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO.
 * O and lse are the forward's outputs for the same inputs.  dO [n_N x k] in
 * `dtype`; dQ [n_N x d], dK [n_M x d], dV [n_M x k] fp32, fully overwritten.
 * dV may be NULL: V = Phi_M is the fixed Laplace-Beltrami basis in the
 * pages' pipelines, so its gradient is usually not needed; the dV products
 * are then skipped (dQ and dK are the same bits as with dV).
 */
ssc_status coupling_dense_bwd(ssc_dtype dtype, int n_N, int n_M, int d, int k,
                              const void* Q, const void* K, const void* V, float scale,
                              const float* O, const void* dO, const float* lse,
                              float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes,
                              ssc_stream stream);

/*
 * Patch scoring and top-s selection (project page, "Geo-FlashAttention":
 * pool source keys, score source patches, keep the top R per target patch).
 * Rows of Q are patch-sorted: target patch p owns rows [offN[p], offN[p+1]);
 * likewise offM for K.  offN [P_N+1] and offM [P_M+1] are int32 device
 * arrays with off[0] = 0, off[P] = n and non-decreasing entries.
 *   Qbar_p = mean of Q rows of patch p,  Kbar_q = mean of K rows of patch q
 *   (fp64 accumulation; an empty patch has mean 0),
 *   C[p, q] = <Qbar_p, Kbar_q>  (fp64, unscaled),
 *   idx[p, 0..s-1] = the s source patches with the largest C[p, :],
 *   ordered by (score descending, index ascending): ties go to the lower
 *   index, so the result is unique.
 * idx [P_N x s] int32.  scores [P_N x P_M] fp64 is optional (may be NULL).
 * Offsets that break the rules above give unspecified scores, but every read
 * stays inside rows [0, n) (they are clamped), so they cannot fault.
 */
ssc_status patch_score_topk(ssc_dtype dtype, int d, int n_N, int P_N, const int* offN,
                            const void* Q, int n_M, int P_M, const int* offM, const void* K,
                            int s, int* idx, double* scores, void* ws, size_t ws_bytes,
                            ssc_stream stream);

/*
 * patch_score_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * patch_score_topk minus (ws, ws_bytes); it allocates nothing.  Its scratch
 * (the fp64 patch means) is a static device array of 4 MiB + 256 bytes per
 * GPU, held until the process ends, which limits P_N, P_M <= 2048 (d <= 128):
 * larger patch counts return SSC_ERR_WORKSPACE.  Every call on one GPU shares
 * that array, so calls that may overlap on the same GPU (different streams
 * or threads) race: serialise them.  The first call on a device looks up the
 * array's device address (one hipGetSymbolAddress, no allocation).
 */
ssc_status patch_score_topk_noalloc(ssc_dtype dtype, int d, int n_N, int P_N, const int* offN,
                                    const void* Q, int n_M, int P_M, const int* offM, const void* K,
                                    int s, int* idx, double* scores, ssc_stream stream);

/*
 * Geo forward (project page, "Geo-FlashAttention" and its pipeline figure:
 * a fused block-sparse kernel takes the exact softmax over the selected
 * source patches only): for every target row i of patch p, the softmax of
 * scale * Q[i].K[j] over j in J_p = union of source patches idx[p, :]
 * (patch-sorted rows, offsets as above), and
 *   O[i] = sum_{j in J_p} softmax_j V[j],  lse[i] = log sum_{j in J_p} exp(.).
 * A row whose support is empty gets O = 0 and lse = -inf.  idx entries must
 * lie in [0, P_M) and be distinct within a row, and the offsets must follow
 * the rules above; these are checked on the device (the host cannot see
 * them without a sync): if any entry or offset breaks them, nothing is
 * computed, O and lse are filled with NaN and the call still returns SSC_OK
 * (the debug build, see SSC_DEBUG below, reports SSC_ERR_INVALID_ARG).
 */
ssc_status coupling_geo_fwd(ssc_dtype dtype, int d, int k, int n_N, int P_N, const int* offN,
                            int n_M, int P_M, const int* offM, int s, const int* idx,
                            const void* Q, const void* K, const void* V, float scale,
                            float* O, float* lse, void* ws, size_t ws_bytes, ssc_stream stream);

/*
 * Geo backward (project page, "Geo-FlashAttention": the block-sparse
 * coupling is trained end to end like the dense one): gradients of
 * <dO, O_geo> for the FIXED selection idx (the selection is piecewise
 * constant in the inputs).  Same formulas as the dense backward restricted
 * to the selected support; source rows outside every support get dK = dV =
 * 0.  Outputs are fully overwritten; dV may be NULL (skipped, as in the
 * dense backward).  Invalid offsets or selection entries (checked on the
 * device, as in the geo forward) compute nothing and fill dQ, dK and dV with
 * NaN.
 */
ssc_status coupling_geo_bwd(ssc_dtype dtype, int d, int k, int n_N, int P_N, const int* offN,
                            int n_M, int P_M, const int* offM, int s, const int* idx,
                            const void* Q, const void* K, const void* V, float scale,
                            const float* O, const void* dO, const float* lse,
                            float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes,
                            ssc_stream stream);

/*
 * Linear-attention (ELU feature map) coupling: the linearized baseline the
 * pages compare against (ai4snews digest, "Interpretation"; project page,
 * "Runtime and memory", Table 1 row "Linear attention (ELU)"), with the
 * softmax replaced by phi(x) = elu(x) + 1 on the raw descriptors:
 *   den[i]  = sum_j phi(Q[i]).phi(K[j]),
 *   O[i, :] = sum_j phi(Q[i]).phi(K[j]) V[j, :] / den[i],
 * evaluated in O(n (d + k)) as phi(Q) (phi(K)^T V) / (phi(Q) phi(K)^T 1).
 * bf16 inputs only (SSC_F32 -> SSC_ERR_UNSUPPORTED); d in {64, 128};
 * 1 <= k <= 255 (one padded column carries the normaliser); n_M >= 1;
 * n_N = 0 is a no-op.  Q [n_N x d], K [n_M x d], V [n_M x k] bf16; O
 * [n_N x k] and den [n_N] fp32.
 */
ssc_status coupling_linear_fwd(ssc_dtype dtype, int n_N, int n_M, int d, int k,
                               const void* Q, const void* K, const void* V,
                               float* O, float* den, void* ws, size_t ws_bytes,
                               ssc_stream stream);

/*
 * Linear-coupling backward: gradients of <dO, O> for the coupling above.
 * O and den are the forward's outputs for the same inputs; dO [n_N x k] bf16.
 * With g = dO / den, s = (dO . O) / den (per row):
 *   dQ = phi'(Q) * (g (phi(K)^T V)^T - s (phi(K)^T 1)^T),
 *   dK = phi'(K) * (V (phi(Q)^T g)^T - 1 (phi(Q)^T s)^T),
 *   dV = phi(K) (phi(Q)^T g).
 * dQ [n_N x d], dK [n_M x d], dV [n_M x k] fp32, fully overwritten
 * (n_N = 0: dK = dV = 0, and Q, O, dO, den or ln den and dQ may be NULL).
 */
ssc_status coupling_linear_bwd(ssc_dtype dtype, int n_N, int n_M, int d, int k,
                               const void* Q, const void* K, const void* V,
                               const float* O, const void* dO, const float* den,
                               float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes,
                               ssc_stream stream);

/*
 * Performer coupling: the second linearized baseline the pages compare
 * against (ai4snews digest, "Synopsis"; project page, "Abstract"), read as
 * the FAVOR+ estimator with positive random features
 *   phi(x)_i = exp(sqrt(scale) W[i] . x - scale |x|^2 / 2) / sqrt(m),
 *   den[i]   = phi(Q[i]) . sum_j phi(K[j]),
 *   O[i, :]  = phi(Q[i]) (sum_j phi(K[j]) V[j, :]) / den[i],
 * with m random directions W [m x d] bf16 (rows; drawn by the caller; the
 * estimator's variance falls as 1/m) and scale the softmax scale being
 * approximated (e.g. 1/sqrt(d)).  Internally the features are shifted by
 * per-feature and per-row maxima that cancel in the ratio (no overflow).
 * Outputs O [n_N x k] fp32 and lnden [n_N] = ln den[i] fp32.  bf16 inputs
 * only; d and m in {64, 128} (other m: SSC_ERR_UNSUPPORTED); 1 <= k <= 255;
 * n_M >= 1; n_N = 0 is a no-op.  Q [n_N x d], K [n_M x d], V [n_M x k]
 * bf16.  ssc_workspace_bytes takes m in its P_N argument (0 means m = d).
 */
ssc_status coupling_performer_fwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, int m,
                                  const void* Q, const void* K, const void* V, const void* W,
                                  float scale, float* O, float* lnden, void* ws, size_t ws_bytes,
                                  ssc_stream stream);

/*
 * Performer backward: gradients of <dO, O> w.r.t. Q, K, V (W is held
 * fixed), with O and lnden from the forward on the same inputs and dO
 * [n_N x k] bf16.  With g = dO / den, s = (dO . O) / den per row and
 * d phi_i / dx = phi_i (sqrt(scale) W[i] - scale x):
 *   dPhiQ = g (phi(K)^T V)^T - s (phi(K)^T 1)^T,
 *   dPhiK = V (phi(Q)^T g)^T - 1 (phi(Q)^T s)^T,
 *   dV = phi(K) (phi(Q)^T g), and dQ, dK through d phi / dx.
 * dQ [n_N x d], dK [n_M x d], dV [n_M x k] fp32, fully overwritten
 * (n_N = 0: dK = dV = 0, and Q, O, dO, den or ln den and dQ may be NULL).
 */
ssc_status coupling_performer_bwd(ssc_dtype dtype, int n_N, int n_M, int d, int k, int m,
                                  const void* Q, const void* K, const void* V, const void* W,
                                  float scale, const float* O, const void* dO, const float* lnden,
                                  float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes,
                                  ssc_stream stream);

/*
 * Functional-map solve after the coupling: the coupled pipelines consume only
 * the product Pi_NM Phi_M (project page, "How it works"); this is the
 * least-squares map between the two spectral bases,
 *   C = argmin_C || Phi_N C - O ||_F = (Phi_N^T Phi_N)^{-1} Phi_N^T O,
 * with O = Pi_NM Phi_M (e.g. a coupling forward's output) and Phi_N the
 * target basis.  Phi_N [n x k] bf16 (SSC_F32 -> SSC_ERR_UNSUPPORTED), O
 * [n x k] fp32, C [k x k] fp32 row-major (C[i*k + j]), fully overwritten.
 * 1 <= k <= 256, n >= 1; Phi_N must have full column rank (else C is NaN).
 * Rows are contiguous (row stride = width), pointers 16-byte aligned.
 */
ssc_status fmap_solve_fwd(ssc_dtype dtype, int n, int k, const void* PhiN, const float* O, float* C,
                          void* ws, size_t ws_bytes, ssc_stream stream);

/*
 * Backward of the solve above for an upstream gradient dC [k x k] fp32, with
 * the basis held fixed: dO = Phi_N (Phi_N^T Phi_N)^{-1} dC, [n x k] fp32,
 * fully overwritten.
 */
ssc_status fmap_solve_bwd(ssc_dtype dtype, int n, int k, const void* PhiN, const float* dC, float* dO,
                          void* ws, size_t ws_bytes, ssc_stream stream);

/*
 * Geodesic farthest-point-sampling partition of one mesh (project page,
 * sections "Abstract" and "Geo-FlashAttention": the surface is partitioned
 * with geodesic farthest-point sampling).  Geodesic distance = shortest path
 * on the edge graph, an edge weighing its Euclidean length
 * sqrt((dx^2 + dy^2) + dz^2) in fp64, path lengths summed from the start
 * vertex outward.  Seed 0 is vertex 0; seed t is the vertex farthest from
 * seeds 0..t-1 (ties to the lower vertex index); labels[v] = t of v's
 * nearest seed (ties to the earlier seed); dist[v] = that distance (+inf and
 * label 0 where no seed is reachable).
 *   x      [n x 3] fp64 positions
 *   off    [n + 1] int32 CSR offsets (off[0] = 0, nondecreasing, off[n] = nnz)
 *   adj    [nnz]   int32 neighbours; every undirected edge appears in both
 *          directions (a one-way entry makes a one-way edge)
 *   seeds  [P] int32, labels [n] int32, dist [n] fp64 -- outputs, fully written
 * 1 <= P <= n.  Sizes are checked on the host (SSC_ERR_INVALID_ARG); the
 * adjacency contents are checked on the device: an offset out of order or
 * a neighbour outside [0, n) computes nothing and writes seeds = labels = -1
 * and dist = NaN.  dtype is ignored (the path is fp64).
 * From n = 32768 (and every vertex with at most 8 neighbours) the first
 * steps run as a cooperative launch of 16 workgroups (fewer on a smaller
 * GPU); if the runtime refuses it, or a grid-barrier wait of it gives up,
 * one workgroup takes every step: the outputs are the same either way.
 * Environment overrides, read at each call (tests and tuning):
 * SSC_FPS_WIDE_STEPS (cap on those steps, 0 = none), SSC_FPS_WIDE_BLOCKS,
 * SSC_FPS_WIDE_FRONTIER (a step whose round queues stay below it ends them),
 * SSC_FPS_SPIN_LIMIT (polls of a barrier wait; 0 = give up at once).
 */
ssc_status fps_partition(int n, int nnz, const double* x, const int* off, const int* adj, int P, int* seeds,
                         int* labels, double* dist, void* ws, size_t ws_bytes, ssc_stream stream);

/*
 * Debug build.  libssc_debug.so is the same library compiled with SSC_DEBUG
 * defined.  Its geo calls and patch_score_topk additionally wait for their
 * stream after launching and read the device-side verdict on the
 * preconditions the host cannot see (offsets start at 0, end at n and do not
 * decrease; idx entries lie in [0, P_M) and are distinct within a row):
 * a violation returns SSC_ERR_INVALID_ARG instead of SSC_OK.  Every kernel
 * still runs to its normal end; only the host reports the flag.  It is meant
 * for development; the synchronisation makes every such call blocking.
 */
int ssc_debug_build(void); /* 1 in libssc_debug.so, 0 otherwise */

/* Static text for a status code. */
const char* ssc_status_string(ssc_status status);

/* hipError_t of the last SSC_ERR_HIP on this thread (0 if none). */
int ssc_last_hip_error(void);

/*
 * Kernel timer (measurement aid).  ssc_timer_arm(family, capacity) makes the
 * calling thread bracket each subsequent launch of one kernel family with a
 * pair of HIP events recorded on that launch's stream; `capacity` event pairs
 * are created up front (family NULL or capacity <= 0 disarms and frees them).
 * Families: "fwd", "dq", "dkv" (dense) and "geo_fwd", "geo_dq", "geo_dkv"
 * (dense calls on the one-patch route, see ssc_dense_split, are timed as
 * the geo families); "lin_gram", "lin_apply" (linear forward), "pf_feat"
 * (Performer features), "fm_gram", "fm_chol", "fm_solve", "fm_apply"
 * (functional-map solve) and "fps" (FPS partition).
 * ssc_timer_read() waits for the recorded events and returns the summed
 * milliseconds and the number of timed launches (negated if more launches
 * happened than pairs were available), then starts a new count.
 * Both return an ssc_status.
 */
int ssc_timer_arm(const char* family, int capacity);
int ssc_timer_read(float* total_ms, int* count);

/*
 * Route of the bf16 dense couplings on the calling thread (a tuning and test
 * aid, like the timer).  With few row blocks (at most 128 blocks of 128 rows:
 * n_N for the forward; n_N or n_M for the backward, whose dQ pass has n_N /
 * 128 and dK/dV pass n_M / 128 blocks) the dense calls run as a geo coupling
 * with one patch per side selecting the other, which is the same exact
 * softmax over every key; the geo planner then splits each short side's row
 * blocks along their streams into parts (merged after the block kernel), so
 * a small or lopsided call fills the chip.  mode = -1: by
 * size (the default), 0: always the dense kernels, 1: always the one-patch
 * geo route.  Other values leave the mode unchanged.  Returns the previous
 * mode.  ssc_workspace_bytes() for the dense ops covers both routes.
 */
int ssc_dense_split(int mode);

/* Internal tile constants, exposed for tests and FLOP accounting:
 * which = 0: padded k for a given k (returns 0 if unsupported),
 * which = 1: row-group granularity of the padded patch layout. */
int ssc_query(int which, int arg);

#ifdef __cplusplus
}
#endif

#endif /* SSC_H */
