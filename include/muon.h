/*
 * muon.h - C ABI of libmuon: the single-GPU Muon optimizer step and the
 * periodic-RowNorm non-refresh step on AMD Instinct MI355X (gfx950).
 *
 * Sources for what the calls compute (page title, then section/equation):
 *   "Infra Optimizers" (summary of "Muon is Scalable for LLM Training"):
 *       Background eq. (1) momentum, the Nesterov remark, the Frobenius
 *       normalisation, eq. (2) quintic Newton-Schulz with a, b, c;
 *       "Scaling Up Muon" eq. (3) decoupled weight decay, Lemma 1 and
 *       eq. (4) the 0.2*sqrt(max(A, B)) update scale, N = 5, mu = 0.95.
 *   "Scaling Muon for Diffusion Transformers": 2.1 (update
 *       W <- (1 - lr*wd) W - lr*s(W)*Phi_5(M)), 3.1 (short-side orientation
 *       and the row-normalisation operator R_eps), abstract (refresh every
 *       K steps, RowNorm on the current momentum otherwise).
 *   "DMuon: Efficient Distributed Muon Training with Near-Adam Overhead":
 *       2.2 (Gram-space Newton-Schulz on the short side, symmetric SYRK-style
 *       Gram product, batching of same-shape matrices).
 *
 * Conventions shared by every call:
 *   - A matrix i is m_i x n_i, row-major and contiguous (the [out, in]
 *     layout of a linear layer).  r = min(m, n), c = max(m, n).
 *   - W (fp32 master weights) and M (fp32 momentum) are updated in place;
 *     G (gradient, fp32 or bf16 as planned) is read only.
 *   - Every pointer inside the W / M / G / O_out / R_out arrays is a HIP
 *     device pointer owned by the caller.  The arrays themselves are host
 *     arrays of length num_matrices, in the order given to muon_plan.
 *   - The workspace is a caller-owned device buffer of at least the size
 *     muon_plan reported, 256-byte aligned.  Its contents between calls are
 *     irrelevant (every call rewrites what it reads).  Step calls allocate
 *     no device memory: the workspace is their only scratch (the plan's
 *     internal streams and events, and a pinned host ring for pointer
 *     tables of more than 960 matrices, are created on first use).
 *   - Calls enqueue work on `stream` and return without synchronising.
 *     Results are valid once the stream has reached that point.  When every
 *     bucket of a plan is too small to fill the GPU on its own and their
 *     scratch fits the cap together, muon_step_batched runs the buckets
 *     concurrently on `stream` and up to 3 internal streams of the plan
 *     (default priority, created on the first such call, destroyed with the
 *     plan): they wait for `stream` on entry and `stream` waits for all of
 *     them on return, so the call behaves as one operation on `stream`.  Each
 *     stream's launches are enqueued from its own host thread (the calling
 *     thread for `stream`; the others are worker threads the plan
 *     starts on its first such call and stops in muon_plan_destroy; each
 *     makes the caller's current device current), and the call returns when
 *     all have enqueued their launches (the calling thread enqueues every
 *     stream when the launch profiler is on).  The internal streams belong
 *     to the device that is current at
 *     that first call: later calls on the plan must keep the same device
 *     current, as the workspace and the matrices live there.
 *   - Errors: all validation happens on the host before anything is
 *     enqueued.  On any status other than MUON_OK and MUON_ERR_HIP nothing
 *     was enqueued and no memory was touched.  MUON_ERR_HIP means a HIP
 *     runtime call failed after work may have been enqueued; W and M are
 *     then undefined.  No C++ exception crosses this interface.
 *   - Concurrency: at most one call per plan may be in flight on the GPU
 *     with a given workspace; different plans with different workspaces are
 *     independent.  A plan may be used from one host thread at a time.
 *   - The step counter and the refresh schedule (call muon_step_batched when
 *     t mod K == 0, rownorm_step otherwise) belong to the caller.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct muon_plan_s* muon_plan_t;

typedef enum {
  MUON_OK = 0,
  MUON_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad count/shape/value */
  MUON_ERR_UNSUPPORTED = 2,        /* valid but not implemented (dtype, steps,
                                      coefficients the 16-bit path cannot scale) */
  MUON_ERR_WORKSPACE_TOO_SMALL = 3,
  MUON_ERR_HIP = 4                 /* a HIP runtime call failed */
} muon_status;

typedef enum { MUON_F32 = 0, MUON_BF16 = 1 } muon_dtype;

/* How the Newton-Schulz iteration of eq. (2) ("Infra Optimizers",
 * Background) is evaluated.  Both compute the same X_N in exact arithmetic.
 *   MUON_FORM_GRAM:   in the r x r Gram space ("DMuon" 2.2): one SYRK
 *                     G0 = X0 X0^T, the recursion on r x r polynomials of G0,
 *                     one final product Q X0.  3 r^2 c + 17 r^3 flops.
 *   MUON_FORM_DIRECT: eq. (2) on X itself, N times A = X X^T (SYRK),
 *                     P~ = b A + c A^2, X <- a X + P~ X.  15 r^2 c + 5 r^3
 *                     flops.  16-bit path only (ns_dtype MUON_BF16): X is
 *                     kept as scaled fp16 in both layouts; the products
 *                     use the tile width of the planner's rule (64 or 128
 *                     for small r, 256 above).
 *   MUON_FORM_AUTO:   per bucket: the direct form for near-square matrices
 *                     (c <= 1.125 r) on the 16-bit path, the Gram form
 *                     otherwise (fewer flops whenever c > r).
 * On the 16-bit path the Gram form is refused (MUON_ERR_UNSUPPORTED, plan-
 * wide or per hint) for near-square buckets: the recursion on X X^T squares
 * the spectrum, and fp16 resolves the small singular values of near-square
 * inputs too coarsely (measured NS error up to 3.2e-2 on squares against
 * the 2e-2 bound; 0.8e-2 at most from c > 1.125 r on). */
typedef enum { MUON_FORM_AUTO = 0, MUON_FORM_GRAM = 1, MUON_FORM_DIRECT = 2 } muon_formulation;

/* Per-shape override of the planner's choices for one bucket (the matrices
 * of exactly rows x cols): the shape-adaptive tuning hook.  "DMuon" 2.4
 * searches tile configurations per target and matrix shape and caches the
 * winners; 2.3 times every distinct shape at initialisation.  Here a tuner
 * (tune.py) times the candidate settings of each shape on the device and
 * passes the winners back through these hints.
 *   tile:        0 = the planner's rule; 64 or 128 = the small-tile kernels;
 *                256 = the 256-wide tile kernels (ns_dtype MUON_BF16 only).
 *   formulation: MUON_FORM_AUTO = the plan-wide setting decides; GRAM or
 *                DIRECT force the form for this bucket (DIRECT needs
 *                ns_dtype MUON_BF16).
 * The remaining fields set how the 256-wide kernels walk and run their
 * tiles (they need a 256-wide tile; 0 keeps the rule):
 *   group:       tile rows per tile-order group, 1..64 (rule: 8 for full
 *                grids, 4 for the lower-triangular grids of symmetric
 *                products); consecutive tiles of a group share operand panels
 *                in an XCD's L2.
 *   xcd_chunk:   consecutive tiles per XCD run, applied to every launch of
 *                the bucket: -1 = one contiguous range of the launch per XCD,
 *                1..65536 = runs of that many (rule: 32).
 *   waves:       wave64s per workgroup of the SYRK and final-product
 *                launches: 8 (rule; two per SIMD, 128 x 64 each) or 4 (one
 *                per SIMD, 128 x 128 each).  The other products always use
 *                8, and so does the final product of buckets with rows <=
 *                cols (it reads X0 across K).
 * Hints whose shape matches no planned matrix are ignored.  Two hints for
 * the same shape, or a value outside these ranges, give
 * MUON_ERR_INVALID_ARGUMENT; combinations the kernels do not provide give
 * MUON_ERR_UNSUPPORTED. */
typedef struct {
  int64_t rows, cols;
  int tile;
  muon_formulation formulation;
  int group;
  int xcd_chunk;
  int waves;
} muon_bucket_hint;

/* Hyper-parameters fixed at plan time.  muon_default_hparams fills the
 * values the pages give: mu = 0.95 and N = 5 ("Infra Optimizers", Scaling Up
 * Muon), a = 3.4445, b = -4.7750, c = 2.0315 (Background, eq. (2)), the 0.2
 * RMS-matching factor (eq. (4)), and eps = 1e-8 for R_eps (the pages leave
 * eps open). */
typedef struct {
  float momentum;      /* mu in M <- mu*M + G                               */
  int   nesterov;      /* 1: NS / RowNorm input U = mu*M' + G; 0: U = M'      */
  int   ns_steps;      /* Newton-Schulz iterations: 1..12 on the 16-bit path
                          (where the 2e-2 accuracy bound holds), 1..16 on
                          the fp32 path                                     */
  float a, b, c;       /* quintic coefficients                              */
  float scale_coeff;   /* s(W) = scale_coeff * sqrt(max(m, n))              */
  float rownorm_eps;   /* eps of R_eps, > 0                                 */
} muon_hparams;

typedef struct {
  int64_t num_matrices;      /* >= 1                                         */
  const int64_t* rows;       /* host array [num_matrices], each m >= 1       */
  const int64_t* cols;       /* host array [num_matrices], each n >= 1       */
  muon_dtype grad_dtype;     /* storage type of G: MUON_F32 or MUON_BF16     */
  muon_dtype ns_dtype;       /* MUON_F32: fp32-MFMA Newton-Schulz path;
                                MUON_BF16: bf16-MFMA Gram/final products with
                                an fp16-MFMA r x r recursion                 */
  muon_hparams hp;
  int64_t max_workspace_bytes; /* cap for the Newton-Schulz scratch; 0 = the
                                  library default (32 GiB).  Buckets of
                                  same-shape matrices are split into chunks
                                  that fit; a single matrix always fits.     */
  muon_formulation formulation; /* see above; 0 = MUON_FORM_AUTO            */
  const muon_bucket_hint* hints; /* nullable host array [num_hints]; copied   */
  int64_t num_hints;             /* 0 = no hints                              */
} muon_plan_desc;

/* Fill *hp with the defaults listed above.  Returns MUON_ERR_INVALID_ARGUMENT
 * if hp is NULL. */
muon_status muon_default_hparams(muon_hparams* hp);

/* Validate the description, bucket same-shape matrices ("DMuon" 2.2
 * batching), choose the orientation per bucket ("Scaling Muon for Diffusion
 * Transformers" 3.1) and lay out the workspace.  Host only: no device work,
 * no device allocation.  On success *plan owns host memory only and
 * *workspace_bytes (nullable) receives the workspace size needed by both
 * step calls.  MUON_ERR_UNSUPPORTED for MUON_FORM_DIRECT with ns_dtype
 * MUON_F32; MUON_ERR_INVALID_ARGUMENT for an unknown formulation.
 * ns_dtype MUON_BF16 keeps every operand of the recursion in fp16 with a
 * power-of-two scale derived here from (a, b, c) and ns_steps (bounds of the
 * iterated polynomials over singular values in [0, 1]); it gives
 * MUON_ERR_UNSUPPORTED when c == 0, |b / c| > 2^60, or a bound needs a scale
 * below 2^-14 (coefficients whose iteration grows without limit). */
muon_status muon_plan(const muon_plan_desc* desc, muon_plan_t* plan, size_t* workspace_bytes);

/* Release a plan.  NULL is accepted.  The caller must ensure no work using
 * the plan is still pending on the GPU. */
muon_status muon_plan_destroy(muon_plan_t plan);

/* Workspace size of an existing plan. */
muon_status muon_plan_workspace_size(muon_plan_t plan, size_t* workspace_bytes);

/* Number of same-shape buckets and launch chunks the planner formed. */
muon_status muon_plan_info(muon_plan_t plan, int64_t* num_buckets, int64_t* num_chunks);

/* What the planner decided for bucket `index` (0 .. num_buckets-1, in order
 * of first appearance of each shape). */
typedef struct {
  int64_t rows, cols;        /* the shape of the bucket's matrices           */
  int64_t count;             /* matrices in the bucket                       */
  int64_t chunks;            /* launch chunks (workspace cap)                */
  int tile;                  /* 64, 128 or 256                               */
  muon_formulation formulation; /* MUON_FORM_GRAM or MUON_FORM_DIRECT        */
  int transposed;            /* 1 iff rows > cols (X0 = U^T)                 */
  int fused_recursion;       /* 1: the whole Newton-Schulz iteration runs as
                                one launch, one workgroup per matrix: the Gram
                                form's r x r recursion (16-bit path, tiles
                                below 256, r padded to <= 128), or the direct
                                form's products and the update (16-bit path,
                                tiles below 256, padded squares of 128 or
                                256, rows <= cols)                           */
  float operand_scales[5];   /* fp16 operand scales of G, P~, H, Q and the
                                direct form's X (plan-wide; all 1 on the fp32
                                path); see muon_plan                         */
  int group, xcd_chunk, waves; /* the bucket's hint values (0: the rule)     */
} muon_bucket_info;

/* Fill *info for one bucket.  MUON_ERR_INVALID_ARGUMENT for a NULL plan or
 * info, or an index out of range. */
muon_status muon_plan_bucket_info(muon_plan_t plan, int64_t index, muon_bucket_info* info);

/* Non-finite inputs: a NaN or an infinity in a matrix's U (its gradient or
 * momentum), or a squared norm past fp32's range, makes that matrix's
 * direction and weights NaN in muon_step_batched, as the plain formula
 * X0 = U / ||U||_F does (no silently finite step); rownorm_step confines it
 * to the affected oriented rows.  Other matrices of the call are unaffected.
 *
 * Newton-Schulz (refresh) step for every planned matrix (Gram form shown;
 * the direct form evaluates the same X_N by iterating eq. (2) on X):
 *   M  <- mu*M + G                                   ("Infra Optimizers" eq. (1))
 *   U   = mu*M + G  (updated M; U = M if nesterov=0)  (Background, Nesterov)
 *   X0  = O(U) / ||U||_F,  O = transpose iff m > n     (eq. (2) preamble; DiT 3.1)
 *   X_N = N quintic steps a X + b (X X^T) X + c (X X^T)^2 X, evaluated in
 *         the r x r Gram space X_N = p(A_{N-1})...p(A_0) X0  (eq. (2); DMuon 2.2)
 *   W  <- (1 - lr*wd) W - lr * scale_coeff*sqrt(max(m,n)) * O^{-1}(X_N)
 *                                                      (eq. (4); DiT 2.1)
 * A matrix with ||U||_F == 0 gets X_N = 0 (pure decay).
 * G[i] points to fp32 or bf16 data as planned.  O_out is NULL or a host
 * array of nullable device pointers; a non-NULL O_out[i] (fp32, m x n)
 * receives O^{-1}(X_N) for matrix i (a parity/debug output).
 * lr and wd must be finite; workspace_bytes must be >= the planned size. */
muon_status muon_step_batched(muon_plan_t plan, float* const* W, float* const* M,
                              const void* const* G, float lr, float weight_decay,
                              void* workspace, size_t workspace_bytes, hipStream_t stream,
                              float* const* O_out);

/* Non-refresh step of periodic RowNorm Muon ("Scaling Muon for Diffusion
 * Transformers", abstract and 3.1): the same M update and U, then
 *   R = O^{-1}(R_eps(O(U))),  R_eps(X)_i = X_i / max(||X_i||_2, eps)
 * over the r rows of the oriented matrix (the columns of U when m > n), and
 *   W <- (1 - lr*wd) W - lr * scale_coeff*sqrt(max(m,n)) * R.
 * R_out works like O_out.  Always computed in fp32. */
muon_status rownorm_step(muon_plan_t plan, float* const* W, float* const* M,
                         const void* const* G, float lr, float weight_decay,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         float* const* R_out);

/* Size of the scratch array the library keeps on every GPU it runs on for
 * muon_step_batched_noalloc (64 MiB; allocated when the library's code is
 * loaded onto a GPU and held until the process ends). */
#define MUON_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

/* muon_step_batched for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, arguments and results, with the
 * workspace taken from the library's own per-GPU scratch array of
 * MUON_NOALLOC_WORKSPACE_BYTES instead of a caller buffer.  The call
 * allocates nothing (no hipMalloc / hipFree, no pinned host staging; the
 * pointer table is written by a kernel from its arguments).
 *   - The plan's single-stream workspace (every bucket on `stream`; plan
 *     with max_workspace_bytes a few MiB below the limit so that the
 *     Newton-Schulz scratch is chunked to fit) must not exceed
 *     MUON_NOALLOC_WORKSPACE_BYTES: else MUON_ERR_WORKSPACE_TOO_SMALL and
 *     nothing is enqueued.  Buckets never run on internal streams here.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on
 *     the GPU (other streams, other host threads, other plans) race and give
 *     undefined results; order them on one stream or synchronise.
 *   - The array's contents between calls are irrelevant (every call rewrites
 *     what it reads).  The launch profiler does not record these calls.
 * Errors as for muon_step_batched; MUON_ERR_HIP also when the current
 * device's scratch address cannot be obtained. */
muon_status muon_step_batched_noalloc(muon_plan_t plan, float* const* W, float* const* M,
                                      const void* const* G, float lr, float weight_decay,
                                      hipStream_t stream, float* const* O_out);

/* Kernel classes reported by the launch profiler. */
typedef enum {
  MUON_K_PREP = 0,        /* momentum, Nesterov blend, ||U|| partials, X0 */
  MUON_K_NORM = 1,        /* fixed-order norm reduction                  */
  MUON_K_SYRK = 2,        /* G0 = X0 X0^T, lower tiles                   */
  MUON_K_POLY = 3,        /* G^2 and P~ = b G + c G^2                    */
  MUON_K_PQPG = 4,        /* P~ Q and P~ G                               */
  MUON_K_PH = 5,          /* P~ H                                        */
  MUON_K_FINAL = 6,       /* Q X0 fused with the weight update           */
  MUON_K_ROWNORM = 7,     /* RowNorm, one pass (m <= n)                  */
  MUON_K_COLSUM = 8,      /* RowNorm m > n: M update + column sums        */
  MUON_K_COLFINAL = 9,    /* RowNorm m > n: column scale                 */
  MUON_K_COLAPPLY = 10,   /* RowNorm m > n: apply                         */
  MUON_K_XCAST = 11,      /* direct form: X0 = U / ||U|| as scaled fp16   */
  MUON_K_XUPD = 12,       /* direct form: X <- a X + P~ X (both layouts)  */
  MUON_K_WUPD = 13,       /* direct form: weight update from X_N          */
  MUON_K_COUNT = 14
} muon_kernel_class;

/* Launch profiler (measurement support, off by default).  While enabled,
 * each kernel launch of the step calls is bracketed by a pair of HIP events
 * recorded on the caller's stream.  muon_plan_kernel_times waits for the
 * recorded events, adds their elapsed times into per-class totals, and
 * returns the totals accumulated since the last reset: total milliseconds,
 * number of launches, and the algorithmic flops and HBM bytes of those
 * launches (flops: symmetric products counted on the lower triangle; bytes:
 * each operand read once and each result written once).  Enabling or
 * disabling resets the totals.  Arrays have MUON_K_COUNT entries; any may be
 * NULL. */
muon_status muon_plan_set_profiling(muon_plan_t plan, int enable);
muon_status muon_plan_kernel_times(muon_plan_t plan, double* total_ms, int64_t* launches,
                                   double* flops, double* bytes);

/* Static, human-readable name of a status code. */
const char* muon_status_string(muon_status s);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */
