/*
 * ortho.h -- C-ABI of libortho.so: the per-matrix orthonormalized optimizer step
 * on one AMD Instinct MI355X (gfx950).
 *
 * Four operations, each for one matrix and for a group of same-shape matrices:
 *
 *   dion_step      Dion's amortised power iteration with error feedback.
 *                  MSR talk "Dion: The distributed orthonormal update revolution
 *                  is here" (passages on amortised power iteration, and on the
 *                  low-rank fraction with error feedback); agentlenshq
 *                  "microsoft/dion", section "How it works"; paper page "Dion:
 *                  Distributed Orthonormalized Updates", abstract (decoupled
 *                  momentum, orthonormalized update).  With B = M + G:
 *                      P  = Q-factor of the thin QR of B Q   (diag(R) > 0)
 *                      R  = B^T P
 *                      M' = B - (1 - mu) P R^T               (error feedback)
 *                      Q' = R with unit-norm columns
 *                      X' = X - lr * scale * P Q'^T          (SGD form)
 *   muon_step      the whole Muon step around newton_schulz: momentum buffer,
 *                  its orthogonalisation, SGD-form update (declared below).
 *   normuon_step   muon_step with the orthogonalised momentum normalised per
 *                  neuron (row) before the update (declared below).
 *   dion2_step     Dion2: the rows of largest norm orthonormalised and applied,
 *                  with error feedback (declared below).
 *   newton_schulz  Muon's Newton-Schulz orthogonalisation, the full-rank
 *                  comparison path.  Same talk, passage contrasting SGD with an
 *                  orthonormal update (take U V^T of the SVD) and the passage on
 *                  Muon's dense matrix-product iteration.  With X = G/(|G|_F+eps)
 *                  (on G^T when G is tall), repeated `steps` times:
 *                      A = X X^T,  X = a X + (b A + c A A) X.
 *
 * Conventions shared by every call
 *   - Every matrix is an ortho_mat: a DEVICE pointer to a row-major matrix with
 *     `rows` x `cols` elements and leading dimension `ld` (elements, >= cols).
 *     The caller allocates and owns all device memory, including the
 *     workspace; the library never allocates or frees memory inside a call.
 *   - All work is enqueued on `stream` (a hipStream_t, NULL = the default
 *     stream) and the calls return without synchronising.  Argument errors are
 *     reported synchronously, before anything is enqueued.
 *   - A call keeps no state between calls: everything it needs is in the
 *     caller's buffers.  Concurrent calls must use different workspaces.
 *   - No call performs host synchronisation or allocation, so a sequence of
 *     calls can be captured into a HIP graph.
 *   - Numerical breakdown cannot be reported synchronously; when `dev_status`
 *     is non-NULL the kernels OR these bits into the device int32 it points to
 *     (the caller zeroes it):
 *       ORTHO_DEV_CHOL_SHIFT   a non-positive Cholesky pivot was replaced by a
 *                              shifted one (B Q was numerically rank deficient)
 *       ORTHO_DEV_ZERO_COLUMN  a column of R had zero norm; that column of Q'
 *                              is set to zero
 */
#ifndef ORTHO_H_
#define ORTHO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORTHO_ABI_VERSION 1

typedef enum { ORTHO_F32 = 0, ORTHO_BF16 = 1 } ortho_dtype;

/* A row-major device matrix view.  `data` must be 16-byte aligned for the
 * vectorised loads; other alignments and ragged sizes are handled element by
 * element. */
typedef struct {
  void* data;
  int64_t rows;
  int64_t cols;
  int64_t ld;      /* elements between consecutive rows, >= cols */
  int32_t dtype;   /* ortho_dtype */
} ortho_mat;

typedef enum {
  ORTHO_OK = 0,
  ORTHO_E_NULL = 1,       /* a required pointer is NULL */
  ORTHO_E_SHAPE = 2,      /* shapes disagree, or a dimension is < 1 */
  ORTHO_E_DTYPE = 3,      /* unsupported or mismatched dtype */
  ORTHO_E_RANK = 4,       /* r outside [1, min(m, n)] or r != Q.cols */
  ORTHO_E_LAYOUT = 5,     /* ld < cols, or a size too large to index */
  ORTHO_E_WORKSPACE = 6,  /* ws is NULL or ws_bytes is below the required size */
  ORTHO_E_PARAM = 7,      /* mu outside [0,1], non-finite lr/scale/abc, steps < 0, batch < 1 */
  ORTHO_E_HIP = 8,        /* a HIP launch failed (no device, invalid stream, ...) */
  ORTHO_E_SCRATCH = 9     /* dion_step_noalloc: the problem needs more than
                             ORTHO_NOALLOC_SCRATCH_BYTES of workspace */
} ortho_status;

#define ORTHO_DEV_CHOL_SHIFT 1
#define ORTHO_DEV_ZERO_COLUMN 2

/* Bytes of device workspace that dion_step / dion_step_ex (batch = 1) or
 * dion_step_batched need for `batch` matrices of m x n at rank r.  Returns 0 for
 * invalid sizes.  The workspace must be 256-byte aligned. */
size_t ortho_dion_workspace_size(int64_t m, int64_t n, int32_t r, int32_t batch);

/* Bytes of device workspace for newton_schulz (batch = 1) or
 * newton_schulz_batched on `batch` matrices of m x n.  Returns 0 for invalid
 * sizes.  256-byte alignment required. */
size_t ortho_ns_workspace_size(int64_t m, int64_t n, int32_t batch);

/* One Dion step on one matrix (see the top of this file for the formulas).
 *   X  m x n, ORTHO_BF16 or ORTHO_F32, updated in place (rounded to nearest
 *      even when stored as bf16).
 *   G  m x n, same dtype as X, read only.
 *   M  m x n, ORTHO_F32 momentum, updated in place (becomes M').
 *   Q  n x r, ORTHO_F32 right factor, updated in place (becomes Q').
 *   r  rank, 1 <= r <= min(m, n), equal to Q.cols.
 *   mu error-feedback decay in [0, 1];  lr finite.
 * bf16 inputs use bf16 matrix-core products with fp32 accumulation (the B Q and
 * B^T P sweeps split fp32 operands into two bf16 terms); fp32 inputs use split
 * products throughout.  The Gram matrix of the orthonormalisation is formed in
 * fp64. */
ortho_status dion_step(ortho_mat X, ortho_mat G, ortho_mat M, ortho_mat Q, int32_t r,
                       float mu, float lr, void* ws, size_t ws_bytes, void* stream);

/* dion_step with an update scale (X' = X - lr*scale*P Q'^T) and optional
 * outputs: P_out (m x r, ORTHO_F32) receives P, R_out (n x r, ORTHO_F32)
 * receives R, dev_status (device int32) receives breakdown bits.  Each of the
 * three pointers may be NULL. */
ortho_status dion_step_ex(ortho_mat X, ortho_mat G, ortho_mat M, ortho_mat Q, int32_t r,
                          float mu, float lr, float scale, const ortho_mat* P_out,
                          const ortho_mat* R_out, int32_t* dev_status, void* ws,
                          size_t ws_bytes, void* stream);

/* dion_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same step, arguments, layouts and errors as dion_step, with no workspace
 * argument.  The workspace comes from a static device array of
 * ORTHO_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends (enough for, e.g., 4096 x 4096 at r = 256 or
 * 256 x 256 at r = 64); a problem whose workspace
 * (ortho_dion_workspace_size(m, n, r, 1)) is larger returns ORTHO_E_SCRATCH
 * before anything is enqueued.  The array of the current device is used, so
 * the stream must belong to the current device.  The call itself allocates and
 * frees nothing; its first call on a device looks up that device's copy of the
 * array once.  All calls on one GPU share the array: two calls that overlap on
 * one GPU (different streams, or different host threads) race and give wrong
 * results; serialise them on one stream.  No part of the array needs to start
 * at zero. */
#define ORTHO_NOALLOC_SCRATCH_BYTES (64u << 20)
ortho_status dion_step_noalloc(ortho_mat X, ortho_mat G, ortho_mat M, ortho_mat Q, int32_t r,
                               float mu, float lr, void* stream);

/* Dion on a group of `batch` independent matrices that share (m, n, dtype) and
 * rank r: the shape-grouped round that the repository summary describes for
 * its megabatch base class (thehardwarestore.ai "microsoft/dion").  X, G, M, Q
 * are HOST arrays of `batch` descriptors each, read during the call only.
 * Equivalent to `batch` calls of dion_step_ex, in fewer launches. */
ortho_status dion_step_batched(int32_t batch, const ortho_mat* X, const ortho_mat* G,
                               const ortho_mat* M, const ortho_mat* Q, int32_t r, float mu,
                               float lr, float scale, int32_t* dev_status, void* ws,
                               size_t ws_bytes, void* stream);

/* Newton-Schulz on one matrix.
 *   G    m x n, ORTHO_BF16 or ORTHO_F32, read only.
 *   Out  m x n, same dtype as G; may be the same memory as G.
 *   steps >= 0 iterations.
 *   abc  HOST pointer to 3 floats (a, b, c), or NULL for Muon's quintic
 *        (3.4445, -4.7750, 2.0315).
 * The iterate is kept in fp32.  For ORTHO_BF16 inputs the three products per
 * iteration use bf16 matrix-core operands with fp32 accumulation; for ORTHO_F32
 * inputs they use fp32-accurate products (each fp32 operand split into three
 * bf16 pieces, the six leading piece products accumulated in fp32), so the
 * result holds fp32-level accuracy.  eps = 1e-7; G = 0 gives 0. */
ortho_status newton_schulz(ortho_mat G, ortho_mat Out, int32_t steps, const float* abc,
                           void* ws, size_t ws_bytes, void* stream);

/* Newton-Schulz on `batch` independent same-shape matrices, each normalised by
 * its own Frobenius norm -- e.g. the per-head blocks of an attention projection
 * (agentlenshq "microsoft/dion", section "Highlights": per-head orthogonalisation
 * so heads do not blend).  G and Out are HOST arrays of descriptors. */
ortho_status newton_schulz_batched(int32_t batch, const ortho_mat* G, const ortho_mat* Out,
                                   int32_t steps, const float* abc, void* ws, size_t ws_bytes,
                                   void* stream);

/* Bytes of device workspace for muon_step (batch = 1) or muon_step_batched on
 * `batch` matrices of m x n.  Returns 0 for invalid arguments. */
size_t ortho_muon_workspace_size(int64_t m, int64_t n, int32_t batch);

/* One Muon step on one matrix: the steps on either side of newton_schulz.
 * MSR talk "Dion: The distributed orthonormal update revolution is here",
 * passage on Muon orthogonalising the momentum-accumulated gradient with dense
 * Newton-Schulz matrix products, and passage on the SGD-form update:
 *     M  = mu M + G                     (heavy-ball momentum buffer)
 *     U  = newton_schulz(M, steps, abc) (as newton_schulz above)
 *     X  = X - lr * scale * U,  rounded to nearest even into X's dtype.
 *   X      m x n, ORTHO_BF16 or ORTHO_F32, updated in place.
 *   G      m x n, same dtype as X, read only.
 *   M      m x n, ORTHO_F32, updated in place (start it at zero).
 *   steps  >= 0 Newton-Schulz iterations; abc as for newton_schulz.  The
 *          products are fp32-accurate when X is ORTHO_F32 and bf16 when X is
 *          ORTHO_BF16 (the momentum is fp32 either way).
 *   mu in [0, 1]; lr and scale finite, else ORTHO_E_PARAM.
 *   ws     >= ortho_muon_workspace_size(m, n, 1) bytes, 256-byte aligned.
 * Errors are returned before anything is enqueued. */
ortho_status muon_step(ortho_mat X, ortho_mat G, ortho_mat M, int32_t steps, const float* abc,
                       float mu, float lr, float scale, void* ws, size_t ws_bytes, void* stream);

/* muon_step on `batch` independent same-shape matrices (HOST arrays of
 * descriptors; every member shares (m, n, dtype) and each operand's ld), each
 * orthogonalised on its own. */
ortho_status muon_step_batched(int32_t batch, const ortho_mat* X, const ortho_mat* G,
                               const ortho_mat* M, int32_t steps, const float* abc, float mu,
                               float lr, float scale, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace for normuon_step (batch = 1) or
 * normuon_step_batched on `batch` matrices of m x n: the Muon workspace plus m
 * floats per member.  Returns 0 for invalid arguments. */
size_t ortho_normuon_workspace_size(int64_t m, int64_t n, int32_t batch);

/* One NorMuon step: muon_step with the orthogonalised momentum normalised per
 * neuron (row) before it is applied.  agentlenshq "microsoft/dion", section
 * "How it works" (NorMuon adds neuron-wise normalisation to Muon); hysenlabs
 * "Microsoft Dion: orthonormal optimizers that assume DTensor parallelism",
 * section "Dion3 is not a retuning of Dion2, and the README says so"
 * (per-neuron normalisation redistributes the update across rows).  The pages
 * print no formula; this is the stateless reading that keeps the total norm:
 *     M  = mu M + G
 *     U  = newton_schulz(M, steps, abc)
 *     V  = U with row i scaled by t / |U_i|,  t = |U|_F / sqrt(m)
 *          (a zero row stays zero)
 *     X  = X - lr * scale * V,  rounded to nearest even into X's dtype.
 * Arguments, layouts, ownership and errors as for muon_step, with
 *   ws     >= ortho_normuon_workspace_size(m, n, 1) bytes, 256-byte aligned. */
ortho_status normuon_step(ortho_mat X, ortho_mat G, ortho_mat M, int32_t steps, const float* abc,
                          float mu, float lr, float scale, void* ws, size_t ws_bytes,
                          void* stream);

/* normuon_step on `batch` independent same-shape matrices (HOST arrays of
 * descriptors, as for muon_step_batched); each member's rows are normalised
 * against its own total norm. */
ortho_status normuon_step_batched(int32_t batch, const ortho_mat* X, const ortho_mat* G,
                                  const ortho_mat* M, int32_t steps, const float* abc, float mu,
                                  float lr, float scale, void* ws, size_t ws_bytes,
                                  void* stream);

/* Bytes of device workspace for dion2_step on an m x n matrix selecting k
 * rows.  Returns 0 for invalid arguments. */
size_t ortho_dion2_workspace_size(int64_t m, int64_t n, int32_t k);

/* One Dion2 step on one matrix: submatrix selection with error feedback.
 * agentlenshq "microsoft/dion", sections "How it works" (Dion2 selects a
 * submatrix; the Dion variants keep error feedback) and "Highlights" (only a
 * fraction of the momentum takes part); hysenlabs "Microsoft Dion: orthonormal
 * optimizers that assume DTensor parallelism", section "Dion3 is not a
 * retuning of Dion2, and the README says so" (mu is Dion2's error-feedback
 * decay).  The pages print no selection rule; the reading taken:
 *     B  = M + G
 *     S  = the k rows of B with the largest l2 norm (equal norms: the lower
 *          row index first; a NaN norm after every other)
 *     U  = newton_schulz(B[S], steps, abc)   (the rows stacked in that order)
 *     X[S] = X[S] - lr * scale * U,  rounded to nearest even into X's dtype;
 *            the other rows of X are untouched
 *     M  = B, with the rows S replaced by mu * B[S]
 *   X      m x n, ORTHO_BF16 or ORTHO_F32, updated in place; m <= 65535.
 *   G      m x n, same dtype as X, read only.
 *   M      m x n, ORTHO_F32, updated in place (start it at zero).
 *   k      1 <= k <= m, else ORTHO_E_RANK.
 *   steps, abc as for newton_schulz (fp32-accurate products for ORTHO_F32
 *          weights, bf16 products for ORTHO_BF16).
 *   mu in [0, 1]; lr and scale finite, else ORTHO_E_PARAM.
 *   selected  NULL, or a DEVICE array of k int32 that receives S in the order
 *          above.
 *   ws     >= ortho_dion2_workspace_size(m, n, k) bytes, 256-byte aligned.
 * Errors are returned before anything is enqueued. */
ortho_status dion2_step(ortho_mat X, ortho_mat G, ortho_mat M, int32_t k, int32_t steps,
                        const float* abc, float mu, float lr, float scale, int32_t* selected,
                        void* ws, size_t ws_bytes, void* stream);

/* Static English description of a status code. */
const char* ortho_status_str(int32_t status);

/* ORTHO_ABI_VERSION of the built library. */
int32_t ortho_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ORTHO_H_ */
