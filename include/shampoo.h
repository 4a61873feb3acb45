/*
 * shampoo.h - C ABI of the owner-side Shampoo step on one gfx950 GPU (same library,
 * same conventions and status codes as muon.h).
 *
 * Why it is here: the owner-centric placement holds the whole 2D gradient of a matrix on
 * its owner rank, so matrix optimizers other than Muon run there unchanged and need no
 * distributed preconditioner ("Resumen Técnico: MatrixFSDP", Contribuciones Clave, item 4,
 * generality; "기술 요약: MatrixFSDP", key contributions, generality: both name Muon,
 * Shampoo and SOAP).  The pages do not define
 * Shampoo; this is the published method for a matrix parameter (Gupta, Koren and Singer,
 * 2018, "Shampoo: Preconditioned Stochastic Tensor Optimization"), with each inverse
 * fourth root computed by the coupled Newton iteration for inverse p-th roots (Guo and
 * Higham, 2006), which needs only matrix products.
 *
 * What is computed, per matrix W (rows x cols, fp32 or bf16) with gradient G (same dtype) and
 * fp32 statistics L (rows x rows) and R (cols x cols):
 *   1. L <- beta2 L + G G^T,  R <- beta2 R + G^T G           (statistics, in place)
 *   2. for S in {L, R}: A = S + eps I, nu = ||S||_F + eps (>= the largest eigenvalue of A);
 *      X_0 = nu^(-1/4) I, M_0 = A / nu, and root_iters times
 *        T = (5 I - M) / 4,  X <- X T,  M <- T^4 M
 *      (X tends to A^(-1/4) and M to I as the eigenvalues of A / nu lie in (0, 1]);
 *   3. W <- W - lr X_L G X_R.
 * Every iterate is a polynomial in A, hence symmetric: the products are computed on
 * lower-triangle tiles and mirrored on store, as in muon_step.  The statistics of all
 * matrices share each launch.
 *
 * Precision: fp32 statistics, copies of G and iterates; fp32 MFMA products (fp32 inputs, fp32
 * accumulation).  A bf16 W and G are read as bf16 (G is widened to fp32 exactly) and W' is
 * rounded to bf16 (round to nearest even) from the fp32 update.  A statistic's eigenvalues below about 1e-7 of its largest are not
 * resolved in fp32, so directions that weak get a root with a large relative error when
 * eps is that small (this is the arithmetic, not the kernels: a float32 run of the same
 * iteration on the CPU shows it too).
 *
 * Workspace: per matrix about 4 (rows + cols) round_up(., 128) words for copies of G and
 * G^T and the product Y_L G, plus 5 m x round_up(m, 128) fp32 iterates for each statistic
 * (m = rows, then cols); shampoo_workspace_size() gives the exact figure.
 */
#ifndef SHAMPOO_H
#define SHAMPOO_H

#include "muon.h"

#ifdef __cplusplus
extern "C" {
#endif

/* One owned matrix: param, stat_left and stat_right are updated in place, grad is read only.
 * param and grad are rows x cols of `dtype`; stat_left (rows x rows) and stat_right
 * (cols x cols) are fp32; all row-major, contiguous device pointers aligned to their element
 * size, 1 <= rows, cols <= 65536.  Matrices of both dtypes may be mixed in one call. */
typedef struct shampoo_matrix {
  void* param;
  const void* grad;
  void* stat_left;
  void* stat_right;
  int64_t rows;
  int64_t cols;
  int32_t dtype;    /* MUON_F32 or MUON_BF16: the dtype of param and grad */
  int32_t reserved; /* must be 0 */
} shampoo_matrix;

typedef struct shampoo_hparams {
  float lr;           /* step size, finite */
  float beta2;        /* statistics decay, in [0, 1] (1: plain sums) */
  float eps;          /* added to each statistic's diagonal and norm; finite and > 0 */
  int32_t root_iters; /* coupled Newton steps per inverse root, in [1, 64] */
} shampoo_hparams;

/* Bytes of device workspace shampoo_step() needs for this list.  Host only, no HIP call.
 * Returns MUON_OK and writes *bytes, or MUON_EINVAL. */
int shampoo_workspace_size(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                           size_t* bytes);

/* One Shampoo step over `count` owned matrices (count == 0 is a no-op).  Same contract as
 * muon_step: validation on the host before any HIP call (MUON_EINVAL for null pointers,
 * sizes, dtype, hyperparameters; MUON_EALIAS when an output (param, stat_left, stat_right)
 * overlaps another output or any grad); `workspace` is a caller-owned device buffer of at
 * least shampoo_workspace_size() bytes, 256-byte aligned (MUON_ENOSPC if smaller); work is
 * enqueued on hip_stream and the call returns before it completes.  The kernel
 * configuration is always the 256 x 256 tiles without the tail split (the tuning table
 * does not apply). */
int shampoo_step(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                 void* workspace, size_t workspace_bytes, void* hip_stream);

/* Host-side description of the launch plan as a NUL-terminated JSON string (truncated to
 * len; MUON_ENOSPC when truncated).  Host only.  For tests and cost figures: "flops"
 * counts a symmetric m x m x k product as m(m+1)k and a full one as 2 m n k. */
int shampoo_plan_describe(const shampoo_matrix* mats, int32_t count, const shampoo_hparams* hp,
                          char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* SHAMPOO_H */
