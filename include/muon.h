/*
 * muon.h -- C ABI of the shape-fused Muon optimizer step for AMD MI355X (gfx950).
 *
 * One Muon step, per 2-D weight slice W of shape [R, C]:
 *   1. M <- beta * M + G                       (momentum of the gradient)
 *   2. X <- M, transposed when R > C            (so X is [m, n], m = min(R, C))
 *      (with the Nesterov option: X <- G + beta * M)
 *   3. X <- X / (||X||_F + eps)                 (whole-matrix Frobenius normalisation)
 *   4. k times: A = X X^T;  X <- a X + (b A + c A^2) X      (Newton-Schulz)
 *   5. O <- X, transposed back when R > C
 *   6. W <- W - lr * O
 *      (options: W <- W - lr * wd * W - lr * f * O, see muon_plan_opts_t)
 *
 * Sources, by page and section:
 *  - "关于分布式Muon的想法整合及讨论" (notes on distributed Muon), §1 Introduction:
 *    Muon keeps a momentum of the gradient, orthogonalises it approximately
 *    and steps along the result; it acts on 2-D matrices.  §2 (how a Muon
 *    step runs): the momentum is first normalised, which needs the whole
 *    matrix; the rest is a Gram matrix and a chain of matrix products.  §6
 *    (combining with tensor parallelism): the normaliser is a sum of squares
 *    over all parts, and the Gram matrix is recomputed every round.
 *  - "MindSpore HyperParallel X 盘古,Muon优化器实现6倍性能跃升", section
 *    三大性能挑战 (three challenges): the iteration takes 5 to 10 rounds of
 *    matrix products and additions, and small matrices make a per-matrix
 *    launch stream host-bound; section 专家切分 (expert split): a 3-D
 *    [E, M, N] tensor is E independent slices; section 矩阵融合优化 (matrix
 *    fusion, Fig. 6-7): parameters whose last two dimensions agree are run as
 *    one batched problem, which is what a plan does here.
 *  The Newton-Schulz form in step 4 and the transpose rule in step 2 are not
 *  printed on the pages; they are the standard quintic Muon iteration, with
 *  (a, b, c) supplied by the caller.
 *
 * Memory and ownership
 *  - params, grads and momentum are DEVICE pointers owned by the caller, on the
 *    device the plan was created on; each is a contiguous row-major tensor of
 *    the shape given at plan creation, 16-byte aligned.  params and momentum
 *    are updated in place, grads is only read.  Momentum is always float32.
 *  - The arrays of pointers passed to muon_step are HOST arrays of n_params
 *    entries, read during the call only.
 *  - A plan owns its device workspace (allocated once in muon_plan_create,
 *    never during muon_step), its device tables and, if enabled, its graph.
 *  - A plan is bound to the device that was current when it was created and
 *    is not thread-safe: one muon_step on a plan at a time.  Different plans
 *    are independent.
 *
 * Errors
 *  - Every function returns a muon_status_t; muon_last_error() gives a
 *    message for the last failure on the calling thread.  No C++ exception
 *    crosses this interface.
 *  - Shape and dtype problems are reported by muon_plan_create/describe.
 *    muon_step checks its pointers and scalars before it enqueues anything;
 *    on error nothing is enqueued and no memory is modified.
 *  - muon_step is asynchronous on `stream`: device faults surface at the
 *    caller's next synchronisation.  muon_plan_status() reports the plan's
 *    device-side error word (it waits for the plan's last step only).
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad shape, non-finite scalar ... */
  MUON_ERR_UNSUPPORTED = 2,      /* valid request this library does not support          */
  MUON_ERR_HIP = 3,              /* a HIP runtime call failed                             */
  MUON_ERR_OOM = 4,              /* workspace allocation failed or exceeds workspace_limit */
  MUON_ERR_DEVICE_MISMATCH = 5,  /* current device differs from the plan's device         */
  MUON_ERR_DEVICE = 6            /* the device reported an error (muon_plan_status)        */
} muon_status_t;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype_t;

/* Arithmetic of the Newton-Schulz iteration.
 *  MUON_MODE_FP32:      float32 storage and float32 products (matrix cores in fp32).
 *  MUON_MODE_BF16_MFMA: bfloat16 operands on the matrix cores with float32
 *                       accumulation; Gram matrices and polynomial in float32. */
typedef enum { MUON_MODE_FP32 = 0, MUON_MODE_BF16_MFMA = 1 } muon_mode_t;

/* Descriptor of one parameter.  ndim 2: shape = [R, C];  ndim 3: shape = [E, R, C]
 * holding E independent slices.  Momentum is always float32. */
typedef struct {
  int32_t ndim;
  int32_t param_dtype; /* muon_dtype_t of W */
  int32_t grad_dtype;  /* muon_dtype_t of G */
  int32_t reserved;
  int64_t shape[3];
} muon_param_desc_t;

typedef struct {
  int32_t mode;            /* muon_mode_t; default MUON_MODE_BF16_MFMA                        */
  int32_t use_graph;       /* 1: capture the step's launches in a HIP graph and replay it     */
  float eps;               /* normaliser offset, default 1e-7                                 */
  int32_t max_ns_steps;    /* muon_step rejects ns_steps > this; default 16                   */
  uint64_t workspace_limit;/* bytes; 0 = no limit.  Plans needing more fail with MUON_ERR_OOM */
  int32_t skinny_max_m;    /* slices with m <= this (<= 32) run the skinny path, which does
                              the rounds in the m x m Gram space; 0 = default 32,
                              -1 = never (every slice takes the streamed path)                */
  int32_t timing;          /* 1: time each kernel class with HIP events (muon_plan_timings)   */
  int32_t n_cu;            /* compute units to plan for; 0 = the device's (describe: 256)     */
  /* Update variants, all off by default (the pages print no update formula;
   * these are the standard Muon options):                                     */
  int32_t nesterov;        /* 1: orthogonalise G + beta M (M already updated) instead of M   */
  int32_t update_scale;    /* muon_update_scale_t: factor f on O, from the stored [R, C]    */
  float weight_decay;      /* wd >= 0: W <- W - lr wd W - lr f O (decoupled)                 */
  int32_t large_min_m;     /* bf16 mode: streamed slices with m >= this (>= 33) take the
                              256 x 256-tile products; 0 = default 129, -1 = never (every
                              streamed slice takes the 32- or 128-tile products)              */
} muon_plan_opts_t;

/* Shape factor f of the update of a slice stored as [R, C]. */
typedef enum {
  MUON_SCALE_NONE = 0,     /* f = 1                        */
  MUON_SCALE_ASPECT = 1,   /* f = sqrt(max(1, R / C))      */
  MUON_SCALE_RMS = 2       /* f = 0.2 sqrt(max(R, C))      */
} muon_update_scale_t;

/* How a bucket of same-shape slices is executed.
 *  MUON_PATH_SKINNY: m <= 32.  One pass forms the first Gram matrix (split over
 *    256-column chunks), the rounds run on m x m matrices (each round's P is a
 *    polynomial in A, so A' = P^2 A and X_k = P_{k-1}..P_0 X_0), and one pass
 *    applies X_k = Q X_0 and updates W.  Three launches per step cover every
 *    skinny bucket of the plan.
 *  MUON_PATH_STREAM: every round forms A = X X^T, P = bA + cA^2 and
 *    X <- aX + PX with batched matrix-core products over the bucket. */
typedef enum { MUON_PATH_SKINNY = 0, MUON_PATH_STREAM = 1 } muon_path_t;

#define MUON_MAX_BUCKETS 64

typedef struct {
  int64_t m, n;            /* oriented slice shape, m <= n                         */
  int32_t count;           /* slices in the bucket                                 */
  int32_t n_transposed;    /* of which stored as [n, m] (R > C)                    */
  int32_t path;            /* muon_path_t                                          */
  int32_t chunks;          /* skinny: 256-column chunks per slice (workgroups)     */
  int32_t reserved[2];
  uint64_t workspace_bytes;/* this bucket's share of the workspace                 */
} muon_bucket_info_t;

typedef struct {
  int32_t n_params;
  int32_t n_matrices;      /* 2-D slices after expanding 3-D parameters            */
  int32_t n_buckets;
  int32_t mode;
  uint64_t workspace_bytes;
  int32_t launches_fixed;  /* launches per step independent of ns_steps           */
  int32_t launches_per_ns; /* plus this many per Newton-Schulz round              */
  muon_bucket_info_t buckets[MUON_MAX_BUCKETS];
} muon_plan_info_t;

typedef struct muon_plan* muon_plan_t;

/* Fill *opts with the defaults listed above. */
void muon_default_opts(muon_plan_opts_t* opts);

/* Plan a step over n_params parameters (descs[0..n_params-1], in the order
 * muon_step will receive their pointers).  Slices are oriented, grouped by
 * oriented shape (m, n) and given a kernel path; the workspace is allocated
 * once on the current device.  opts may be NULL (defaults).
 * Errors: INVALID_ARGUMENT (null pointers, n_params <= 0, ndim not 2 or 3, a
 * dimension <= 0 or >= 2^31, unknown dtype or mode, bad eps/max_ns_steps,
 * nesterov not 0 or 1, unknown update_scale, weight_decay negative or not
 * finite),
 * UNSUPPORTED (more than MUON_MAX_BUCKETS shapes), OOM, HIP. */
int muon_plan_create(const muon_param_desc_t* descs, int32_t n_params,
                     const muon_plan_opts_t* opts, muon_plan_t* out_plan);

/* The same planning as muon_plan_create without touching any device: fills
 * *info as the plan would report it (opts->n_cu, or 256 compute units). */
int muon_plan_describe(const muon_param_desc_t* descs, int32_t n_params,
                       const muon_plan_opts_t* opts, muon_plan_info_t* info);

/* Report an existing plan's layout. */
int muon_plan_query(muon_plan_t plan, muon_plan_info_t* info);

/* Enqueue one Muon step on `stream` (a hipStream_t; NULL = the null stream).
 * params/grads/momentum: host arrays of n_params device pointers (see above).
 * ns_steps in [0, max_ns_steps]; lr, beta, a, b, c finite.  ns_steps = 0 steps
 * along the normalised momentum.  Does not synchronise the host and
 * allocates no memory, host or device.  A step on another stream than the
 * plan's previous step is ordered after that step (stream wait on an event). */
int muon_step(muon_plan_t plan, void* const* params, const void* const* grads,
              void* const* momentum, float lr, float beta, int32_t ns_steps,
              float a, float b, float c, void* stream);

/* Wait for the plan's last step (not for other work on the device), read the
 * plan's device-side error word and clear it.  Bit 0: some slice's momentum
 * had a non-finite norm (its update is then not finite either); every path
 * sets it.  Returns MUON_ERR_DEVICE when the word was nonzero. */
int muon_plan_status(muon_plan_t plan, uint32_t* device_error);

/* Kernel-class timings collected since the last call (opts.timing = 1):
 * out_ms[i] = total milliseconds, out_count[i] = launches, for i < n_out and
 * the classes 0 skinny_gram, 1 skinny_poly, 2 skinny_apply, 3 momentum,
 * 4 norm, 5 gram, 6 poly, 7 apply, 8 update.  Synchronises.  Returns the
 * number of classes. */
int muon_plan_timings(muon_plan_t plan, double* out_ms, int64_t* out_count, int32_t n_out);

/* Wait for the plan's last step, then release the plan and its device
 * memory.  NULL is a no-op. */
int muon_plan_destroy(muon_plan_t plan);

/* Size of the fixed device scratch array of muon_step_noalloc: 64 MiB per
 * device, held from the first call on that device until the process ends. */
#define MUON_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one Muon
 * step over the parameters described by descs/opts (as for
 * muon_plan_create), run in a fixed file-scope device array of
 * MUON_NOALLOC_SCRATCH_BYTES instead of a plan's workspace.  The results are
 * those of muon_plan_create + muon_step on the same arguments (same kernels,
 * same arithmetic).
 *  - params/grads/momentum, lr, beta, ns_steps, a, b, c, stream: as for
 *    muon_step.  opts->use_graph and opts->timing must be 0.
 *  - device_error: NULL, or a 4-byte aligned DEVICE word owned by the caller
 *    into which bit 0 is OR-ed when a slice's momentum norm is not finite
 *    (the word is not cleared by this call).
 *  - Calls no hipMalloc, hipFree or other device or pinned-host allocation.
 *    The plan is built on the host's C++ heap and freed before return; the
 *    scratch is cleared by a kernel, and its tables (a few KB) are copied
 *    from pageable host memory, which makes those copies synchronous with
 *    respect to the host.
 *  - Every call on one device shares that device's scratch and overwrites
 *    it: calls that overlap on one GPU (other streams, other threads) race.
 *    Steps enqueued one after another on one stream are ordered as usual.
 * Errors: those of muon_plan_create and muon_step, plus UNSUPPORTED when the
 * step needs more than MUON_NOALLOC_SCRATCH_BYTES of scratch (checked on the
 * host before any device call; use a plan instead), INVALID_ARGUMENT for
 * use_graph/timing or a misaligned device_error. */
int muon_step_noalloc(const muon_param_desc_t* descs, int32_t n_params, const muon_plan_opts_t* opts,
                      void* const* params, const void* const* grads, void* const* momentum, float lr,
                      float beta, int32_t ns_steps, float a, float b, float c, uint32_t* device_error,
                      void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* muon_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MUON_H */
