/*
 * muon.h - C ABI of the owner-side Gram Newton-Schulz Muon step on one gfx950 GPU.
 *
 * What is computed (per owned weight matrix W of shape rows x cols):
 *   1. momentum accumulation   M <- beta*M + G            (heavy-ball; DMuon summary §1,
 *                                                          "momentum-aggregated gradients")
 *   2. orientation             X = M if rows <= cols, else M^T, so X is m x n, m <= n
 *                                                         (DMuon summary §2.2: the Gram
 *                                                          saving holds for m < n)
 *   3. Frobenius normalisation X0 = X / (||X||_F + eps)
 *   4. Newton-Schulz, ns_steps iterations of X <- aX + b(XX^T)X + c(XX^T)^2X, evaluated in
 *      the m x m Gram space G = X X^T (DMuon summary §2.2): P = aI + bG + cG^2,
 *      G <- P G P, Q <- P Q, output O = Q X0.  Only the lower triangle of every symmetric
 *      product is computed (DMuon summary §2.2, symmetric SYRK-type path) and mirrored on
 *      store.  Same-shape matrices are batched into shared launches (DMuon summary §2.2,
 *      batching).
 *   5. update                  W <- W - lr * sqrt(max(1, rows/cols)) * O
 *   The owner runs this once per matrix with no communication (DMuon summary §2.1;
 *   MatrixFSDP summary, Methodology §1).  The 1D tail uses AdamW (MatrixFSDP summary,
 *   Methodology §1) through adamw_step().
 *
 * Precision: bf16 matrices run bf16 MFMA products with fp32 accumulation and bf16 storage
 * of every m x m iterate (round to nearest even); fp32 matrices run fp32 MFMA products
 * with fp32 storage.  Elementwise math is fp32.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers on the current HIP device.  Matrices are
 *     row-major and contiguous (leading dimension = cols).
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream) and the
 *     call returns before it completes.  Buffers must stay valid and untouched until the
 *     stream has reached that point.
 *   - Every argument is validated on the host before the first HIP call; a validation
 *     failure returns a negative status and enqueues nothing.
 *   - No C++ exception crosses the ABI.  Status codes are muon_status values.
 *   - The library allocates no device memory.  It keeps a small pinned host staging ring
 *     for launch descriptors, released by muon_shutdown().
 *   - Calls may come from several host threads and go to several streams at once, each
 *     with its own workspace; results do not depend on how they interleave.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muon_status {
  MUON_OK = 0,
  MUON_EINVAL = -1,      /* null pointer, bad size, unknown dtype, non-finite hyperparameter */
  MUON_ENOSPC = -2,      /* workspace smaller than muon_workspace_size() */
  MUON_EALIAS = -3,      /* grad overlaps an output (param/momentum) of any matrix, or
                            outputs of two matrices overlap */
  MUON_EHIP = -4,        /* a HIP runtime call failed; muon_last_error() has the text */
  MUON_EUNSUPPORTED = -5, /* valid request this library cannot run (e.g. no gfx950 device) */
  MUON_ESTALE = -6        /* a tuning table measured on other kernels (another build) */
} muon_status;

typedef enum muon_dtype { MUON_BF16 = 1, MUON_F32 = 2 } muon_dtype;

/* One owned matrix.  param and momentum are updated in place; grad is read only.
 * All three have shape rows x cols, dtype `dtype`, row-major, contiguous. */
typedef struct muon_matrix {
  void* param;
  const void* grad;
  void* momentum;
  int64_t rows;
  int64_t cols;
  int32_t dtype;    /* muon_dtype */
  int32_t reserved; /* must be 0 */
} muon_matrix;

/* Restart set: bit k (1 <= k < ns_steps) re-anchors at the start of iteration k:
 * X <- Q X, G <- X X^T, Q <- I.  Exact in real arithmetic (the result does not change);
 * it bounds the bf16 error of the Gram iterate on near-square matrices.
 * MUON_RESTART_AUTO picks, per matrix, {2, 3, ..., ns_steps-1} when n < 1.5 m (near-square:
 * a restart costs no extra flops when m == n) and none otherwise. */
#define MUON_RESTART_AUTO 0xFFFFFFFFu

typedef struct muon_hparams {
  float lr;       /* step size before the shape factor sqrt(max(1, rows/cols)) */
  float beta;     /* momentum coefficient */
  float ns_a;     /* Newton-Schulz polynomial a x + b x^3 + c x^5 */
  float ns_b;
  float ns_c;
  int32_t ns_steps; /* 0..31; 0 gives O = X0 */
  float eps;        /* added to ||X||_F before dividing; >= 0 */
  uint32_t restart_mask;
} muon_hparams;

/* Bytes of device workspace muon_step() needs for this list.  Host only, no HIP call.
 * Returns MUON_OK and writes *bytes, or MUON_EINVAL. */
int muon_workspace_size(const muon_matrix* mats, int32_t count, const muon_hparams* hp,
                        size_t* bytes);

/* One Muon step over `count` owned matrices (count == 0 is a no-op).  `workspace` is a
 * device buffer of at least muon_workspace_size() bytes, 256-byte aligned, owned by the
 * caller and not touched by anything else until the stream passes this call; two calls
 * in flight at once need two workspaces.  Matrices may mix dtypes. */
int muon_step(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* workspace,
              size_t workspace_bytes, void* hip_stream);

/* AdamW on a packed fp32 vector of n values (MatrixFSDP summary, Methodology §1: the
 * non-matrix tail keeps standard AdamW).  With t = step >= 1:
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
 *   p <- p - lr * ( (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps) + weight_decay * p ).
 * p, m, v are updated in place; g is read only; all device pointers, 4-byte aligned. */
typedef struct adamw_hparams {
  float lr;
  float beta1;
  float beta2;
  float eps;
  float weight_decay;
  int32_t step;
} adamw_hparams;

int adamw_step(float* p, const float* g, float* m, float* v, int64_t n, const adamw_hparams* hp,
               void* hip_stream);

/* Algorithmic work of one muon_step over this list (host only): flops count a symmetric
 * m x m x k product as m(m+1)k and a full product as 2*m*n*k; bytes count the compulsory
 * HBM traffic of the elementwise phases.  Either output pointer may be NULL. */
int muon_step_cost(const muon_matrix* mats, int32_t count, const muon_hparams* hp,
                   double* flops, double* bytes);

/* Owner assignment (DMuon summary §2.3: each matrix gets one owner rank; the assignment
 * minimises the predicted makespan, the largest total cost of one owner; the summary poses
 * it as a mixed-integer program with a greedy fallback for large instances).  Host only.
 *   cost[i]    predicted cost of matrix i (e.g. its measured step time), finite, >= 0;
 *   count      number of matrices (>= 0), ranks the number of owners (>= 1);
 *   node_limit budget of the exact search (0: greedy only);
 *   owner[i]   receives the owner, in [0, ranks), of matrix i (count ints, caller-owned);
 *   *makespan  receives the largest owner load (may be NULL);
 *   *optimal   receives 1 when the result is proven optimal, else 0 (may be NULL).
 * Greedy longest-first: matrices in decreasing cost (ties in list order), each to the owner
 * with the smallest load so far (lowest index on ties).  Then, for count <= 64 and
 * node_limit > 0, an exact depth-first search from the greedy makespan.  It returns the
 * optimum when it finishes within node_limit nodes, else the best assignment found.  A
 * result is also proven optimal when it meets max(largest cost, total / ranks).  Errors:
 * MUON_EINVAL for bad sizes, NULL arrays or a negative or non-finite cost; nothing is
 * written then. */
int muon_owner_assign(const double* cost, int32_t count, int32_t ranks, int64_t node_limit,
                      int32_t* owner, double* makespan, int32_t* optimal);

/* Shape-adaptive kernel selection (DMuon summary §2.4: the tile shape is searched per
 * target and matrix shape, and the best configuration is cached and reused by later steps).
 * The library has six MFMA kernel configurations: 0 = 256 x 256 output tiles, 1 = 256 x 384
 * output tiles (8 waves of 128 x 96), 4 = 256 x 256 tiles with a deeper load pipeline (four
 * LDS stages of 32 contraction elements, three k-steps of loads in flight), 5 = 128 x 128
 * output tiles (4 waves of 64 x 64, two workgroups per compute unit: for launches with fewer
 * tiles than compute units or short contractions), 2 and 3 = 0 and 1 with the tail split: the tiles of
 * a launch's last, partial round of workgroups (one per compute unit) are cut along the
 * contraction into pieces run by the otherwise idle units, and the last piece of a tile to
 * finish adds the others' fp32 partial sums in piece order (so results are deterministic,
 * but they may differ from configurations 0 and 1 by the rounding of those additions).  The
 * last piece waits for the others' sums with a bounded wait; should it ever run out, the
 * tile is stored as NaN and the workspace's status word is set (muon_workspace_check).  A
 * launch with no tail worth cutting runs 2 as 0 and 3 as 1.  Each MFMA launch of a plan has
 * a signature string
 * (dtype, then per shape group its kind, symmetry, orientation and run-length shapes); a
 * process-wide table maps signatures to configurations; for a signature the table does not
 * hold, muon_step uses configuration 5 when the launch has fewer than 64 tiles of 256 x 256
 * and configuration 0 otherwise.  The table is shared by all threads and devices.
 * Configuration 1 addresses operands with 32-bit offsets: a launch holding a matrix whose
 * larger side d has (d + 384) * (d rounded up to 128) * element size >= 2^31 bytes always
 * runs configuration 0 (or 2), whatever the table or muon_tune_force say.  An fp32 launch
 * (fp32 matrices, and bf16 ones with at most 128 Gram rows) whose last tiles contract over
 * 2^17 elements or more always runs with the tail split (3 under 1 or 3, else 2), whatever the table or
 * muon_tune_force say.  Only the launch's tail tiles (those past its last whole round of
 * one tile per compute unit: all of them when it has fewer tiles than units) are cut: into
 * 8 pieces when there are at most units/8 of them, into units/R pieces for R tail tiles up
 * to units/2, and once (about n/(n+1) and 1/(n+1)) beyond that.  Whole-round tiles still
 * sum the whole contraction in one fp32 sum; they exist only for launches of at least one
 * tile per unit (an fp32 Gram formation with m above about 5600 rows).
 *
 * muon_tune_scratch_size: device bytes muon_tune needs in `scratch` for the list (its params
 *   and momenta, each copy 256-byte aligned); 0 for an empty list.  Host only; errors as
 *   muon_workspace_size.
 * muon_tune: runs one step over copies of the list's params and momenta, made in the
 *   caller's `scratch` (scratch_bytes >= muon_tune_scratch_size, 256-byte aligned, device
 *   memory the caller owns; the caller's matrices are not modified).  After each MFMA launch
 *   of that step it times the same launch in `reps` rounds (1 <= reps <= 64), each round
 *   running it once under every configuration that applies to it.  The configuration with
 *   the smallest median time is stored under the launch's signature when its median is at
 *   least 1 % below that of the launch's untuned default (5 or 0, above), else the default.
 *   A set-up call: it synchronises the stream before returning, after which the scratch is
 *   free again.  Arguments and
 *   errors as muon_step, plus MUON_EINVAL for reps outside [1, 64] or a NULL or misaligned
 *   scratch, and MUON_ENOSPC when scratch_bytes is too small (nothing enqueued then).
 * muon_tune_force: cfg in 0 .. 5 forces that configuration for every launch, -1
 *   restores the table.  MUON_EINVAL for other values.  For tests and measurements.
 * muon_tune_clear: empties the table.
 * muon_tune_export: writes the table as text, NUL-terminated, into buf (len bytes): a first
 *   line "# muon-tune <hash>" naming the kernels it was measured on (muon_kernel_hash),
 *   then one "signature cfg" line per entry, sorted.  *needed (may be NULL) receives the
 *   size with the NUL; buf == NULL only queries it.  MUON_ENOSPC when len is too small (buf
 *   untouched).
 * muon_tune_import: adds the lines of such a text to the table (existing signatures are
 *   overwritten).  A "# muon-tune <hash>" line naming other kernels than this library's
 *   makes it MUON_ESTALE, with nothing added (a table is valid only for the kernels it was
 *   measured on); a text without one is taken as it is; other lines starting with '#' are
 *   comments.  MUON_EINVAL, with nothing added, on a malformed line.  Host only.
 * muon_kernel_hash: 16 hex digits identifying the kernel sources this library was built
 *   from (the version of its tuning tables).  Host only. */
int muon_tune_scratch_size(const muon_matrix* mats, int32_t count, const muon_hparams* hp, size_t* bytes);
int muon_tune(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* workspace,
              size_t workspace_bytes, void* scratch, size_t scratch_bytes, void* hip_stream, int32_t reps);
int muon_tune_force(int32_t cfg);
void muon_tune_clear(void);
int muon_tune_export(char* buf, size_t len, size_t* needed);
int muon_tune_import(const char* text);
const char* muon_kernel_hash(void);

/* Host-side description of the launch plan (buckets, restart sets, launches) as a
 * NUL-terminated JSON string written to buf (truncated to len).  Host only.  For tests. */
int muon_plan_describe(const muon_matrix* mats, int32_t count, const muon_hparams* hp, char* buf,
                       size_t len);

/* Per-kernel timing.  Between muon_profile_begin() and muon_profile_end(), each launch made
 * by muon_step()/adamw_step() is bracketed by HIP events on its stream.  The events serve
 * timing only and carry no system-scope memory fence.  muon_profile_end() waits for them and
 * writes one record per kernel kind. */
typedef struct muon_kernel_stat {
  char name[32];
  int64_t launches;
  double ms;     /* summed event time of those launches */
  double flops;  /* algorithmic flops of those launches */
  double bytes;  /* algorithmic bytes of those launches */
} muon_kernel_stat;

int muon_profile_begin(void);
int muon_profile_end(muon_kernel_stat* out, int32_t max, int32_t* count);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): muon_step with no workspace argument.  The
 * library holds one 128 MiB scratch array per GPU it runs on (a file-scope device array, for
 * the life of the process) and runs exactly muon_step's plan and kernels in it, so results
 * equal muon_step's bitwise.  It calls no device or host allocator: the launch descriptors
 * reach the device in kernel arguments.  Every call on one GPU shares that GPU's array and
 * leaves its contents behind (each step clears what must start at zero), so calls that
 * overlap on one GPU (two streams, two threads) race: serialise them.  A list whose
 * muon_workspace_size exceeds 128 MiB returns MUON_ENOSPC with nothing enqueued; other
 * arguments and errors as muon_step.  muon_workspace_check(NULL, 0, stream) reports the
 * last such step's status on the current device. */
int muon_step_noalloc(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* hip_stream);

/* Status of the last step run on a workspace (muon_step or shampoo_step; the first
 * 256 bytes of every workspace hold a status word that the step's first launch clears).
 * Synchronises hip_stream, reads the word and clears it.  MUON_OK when the step completed
 * normally; MUON_EHIP, with the reason in muon_last_error(), when a tail-split tile's bounded
 * wait for the other pieces' partial sums timed out (that tile was stored as NaN, and the
 * step's results are not to be used).  A NULL workspace means the current device's
 * muon_step_noalloc scratch (workspace_bytes is then ignored).  MUON_EINVAL for
 * workspace_bytes < 256.  It reports the last step enqueued on the stream before it; check
 * after every step whose results matter. */
int muon_workspace_check(void* workspace, size_t workspace_bytes, void* hip_stream);

const char* muon_strerror(int status); /* static string */
const char* muon_last_error(void);     /* detail of the last failure on this thread */
const char* muon_version(void);
void muon_shutdown(void);              /* frees the pinned staging ring; idempotent */

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */
