/*
 * pamm.h -- C ABI of the PAMM library for AMD Instinct MI355X (gfx950).
 *
 * Point-Approximate Matrix Multiplication (PAMM), after the page "QKV
 * Projections Require a Fraction of Their Memory" (gist.science summary of
 * arXiv 2506.02939).  Instead of saving the input activations X [n x d] of a
 * QKV projection for the weight gradient, PAMM keeps k generator rows C, and
 * for every token an index f(i) and a scale alpha_i with X_i ~ alpha_i *
 * C_f(i).  The weight gradient is then approximated from that compressed
 * form without rebuilding X.
 *
 * Conventions for every call:
 *   - Matrices are row-major; a leading dimension (ld*) is the distance in
 *     elements between consecutive rows and must be >= the row length.
 *   - Pointers are DEVICE pointers unless the parameter name ends in _host.
 *     The caller allocates and owns every buffer, including the workspace;
 *     the library never allocates device memory and keeps no state between
 *     calls (pamm_wgrad_noalloc aside, whose workspace is a fixed device
 *     array the library's code object carries).
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  Work is enqueued asynchronously; nothing synchronises.
 *   - dtype: PAMM_F32 or PAMM_BF16.  X, C, dY and the reconstruction share
 *     one dtype; alpha is always fp32, f always int32, dW always fp32.
 *   - Base pointers of X, C, dY, dW and the reconstruction must be 16-byte
 *     aligned and their leading dimensions multiples of 16 bytes (8 bf16 or
 *     4 fp32 elements); f, alpha and gen_idx need 4-byte alignment; the
 *     workspace needs 256-byte alignment.
 *   - A workspace holds a call's intermediate results until its kernels
 *     finish: calls that may run concurrently need workspaces of their own.
 *   - Every call returns a pamm_status_t.  Arguments are fully validated
 *     before anything is enqueued; on any error nothing is launched and no
 *     output is written.  No C++ exception crosses this interface.
 *   - Sizes: 0 <= k <= n < 2^31, k <= PAMM_MAX_K, d >= 1, d_out >= 1, and
 *     every matrix spans at most 2^40 elements ((rows - 1) * ld + row
 *     length); otherwise PAMM_ERR_SHAPE.
 */
#ifndef PAMM_H
#define PAMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAMM_ABI_VERSION 3
/* Largest generator count the segment sort of pamm_wgrad supports. */
#define PAMM_MAX_K 4096

typedef enum { PAMM_F32 = 0, PAMM_BF16 = 1 } pamm_dtype_t;

typedef enum {
    PAMM_OK = 0,
    PAMM_ERR_NULL = 1,        /* a required pointer is NULL                     */
    PAMM_ERR_SHAPE = 2,       /* a size or leading dimension is out of range    */
    PAMM_ERR_DTYPE = 3,       /* unknown dtype code                             */
    PAMM_ERR_ALIGN = 4,       /* pointer or leading dimension misaligned        */
    PAMM_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required     */
    PAMM_ERR_UNSUPPORTED = 6, /* valid request the library does not implement   */
    PAMM_ERR_HIP = 7,         /* the HIP runtime reported an error at launch    */
    PAMM_ERR_VALUE = 8,       /* a scalar argument is out of range (e.g. eps)   */
    PAMM_ERR_TOO_LARGE = 9    /* needs more memory than available: the no-allocation
                                 scratch array, or host memory for sampling          */
} pamm_status_t;

/* PAMM_ABI_VERSION of the loaded library. */
int pamm_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *pamm_status_string(int status);

/*
 * Draw the generator rows (page section 2 "Metodologia", "Algoritmo in Due
 * Fasi", compression: the generators are rows of the activation matrix taken
 * at random).  Host-only, no GPU involved.
 *
 * Writes k distinct row indices in [0, n), sorted ascending, to
 * gen_idx_host[0..k).  Sampling is uniform without replacement: Floyd's
 * algorithm (j = n-k .. n-1: draw t uniform in [0, j], take t unless already
 * taken, else j) driven by SplitMix64 seeded with `seed`; a uniform integer in
 * [0, m) is the high 64 bits of the 128-bit product of a SplitMix64 output
 * and m.  Host memory: n bits for the set of rows taken.  Errors:
 * PAMM_ERR_SHAPE if k < 0, k > n or n >= 2^31; PAMM_ERR_NULL if k > 0 and
 * gen_idx_host is NULL; PAMM_ERR_TOO_LARGE if those n bits cannot be
 * allocated.
 */
int pamm_sample_generators(int64_t n, int64_t k, uint64_t seed, int32_t *gen_idx_host);

/* Bytes of workspace pamm_compress needs: 0 for fp32 with k <= 256 and for
 * bf16 with k <= 128; otherwise per-tile winners and |x|^2 (k > 256) and
 * the generator norms |c_j|^2 (bf16, k > 128). */
size_t pamm_compress_workspace_size(int64_t n, int64_t d, int64_t k, int dtype);

/*
 * Compression, the forward-pass phase (page section 2 "Metodologia",
 * "Algoritmo in Due Fasi", compression steps).
 *
 *   X        [n x d], leading dimension ldx, dtype      (read)
 *   gen_idx  [k] int32 row indices of X that serve as generators (read);
 *            values must lie in [0, n): an out-of-range value is clamped
 *            into range (no out-of-bounds access), and that generator is
 *            then an unspecified row of X
 *   eps      similarity threshold, 0 <= eps (finite)
 *   C        [k x d], leading dimension d, dtype (written): C_j = X[gen_idx_j]
 *   f        [n] int32 (written): generator slot of each row, -1 if dropped
 *   alpha    [n] fp32 (written): scale of each row, 0 if dropped
 *   ws       workspace of at least pamm_compress_workspace_size bytes
 *
 * For every row x_i: score_j = |<x_i, c_j>| / |c_j| (0 for a zero
 * generator); f*(i) = the lowest j of maximal score (NaN never wins); the row
 * is kept iff score/|x_i| >= eps (cosine 0 for a zero row), with then
 * f(i) = f*(i) and alpha_i = <x_i, c_f> / |c_f|^2; otherwise f(i) = -1 and
 * alpha_i = 0.  Dot products are accumulated in fp32 from exact products of
 * the stored values; the decision is taken in fp32.  The result is bitwise
 * deterministic.  |c_j|^2 is the same accumulation as a dot product, so a row
 * equal to a power-of-two multiple s of a generator gets alpha = s exactly,
 * with one exception: bf16 with k > 128 on inputs that fill the device (at
 * least one (128-row block, 256-generator tile) pair per compute unit) runs
 * a GEMM-shaped kernel that sums |c_j|^2 in fp32 in another order, so there
 * such an alpha is s to a few fp32 ulps (its bf16 reconstruction alpha*c
 * still equals the row).
 */
int pamm_compress(const void *X, int64_t n, int64_t d, int64_t ldx, int dtype,
                  const int32_t *gen_idx, int64_t k, float eps,
                  void *C, int32_t *f, float *alpha,
                  void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace pamm_forward_compress needs: the generator norms
 * |c_j|^2, plus per-tile winners and |x|^2 when k > 256. */
size_t pamm_forward_compress_workspace_size(int64_t n, int64_t d, int64_t k, int dtype);

/*
 * The projection and the compression in one pass over X (page section 2
 * "Metodologia", "Algoritmo in Due Fasi": the compressed form is computed
 * during the forward pass of the QKV projection, whose input X it replaces):
 *
 *   Y = X W^T (+ bias)       [n x d_out], fp32 accumulation, rounded to bf16
 *                            (nearest even) after the bias is added in fp32
 *   (C, f, alpha)            exactly as pamm_compress defines them
 *
 *   X     [n x d] bf16, leading dimension ldx            (read)
 *   W     [d_out x d] bf16, leading dimension ldw >= d   (read; the layout
 *         of a linear layer's weight)
 *   bias  [d_out] bf16, or NULL                          (read)
 *   Y     [n x d_out] bf16, leading dimension ldy >= d_out (written)
 *   gen_idx, k, eps, C, f, alpha as for pamm_compress
 *   ws    workspace of at least pamm_forward_compress_workspace_size bytes
 *
 * Alignment as for pamm_compress, plus W and Y 16-byte aligned with ldw and
 * ldy multiples of 8 elements, and bias 2-byte aligned.  Only bf16:
 * PAMM_ERR_UNSUPPORTED for fp32, and also when n x ldx or d_out x ldw spans
 * 4 GiB or more.  The indices and alpha follow the rules of pamm_compress's
 * GEMM-shaped kernel (|c_j|^2 summed outside the matrix product, so a
 * power-of-two multiple of a generator gets alpha exact to a few fp32 ulps).
 * Deterministic.
 */
int pamm_forward_compress(const void *X, int64_t n, int64_t d, int64_t ldx, int dtype,
                          const void *W, int64_t d_out, int64_t ldw, const void *bias,
                          void *Y, int64_t ldy,
                          const int32_t *gen_idx, int64_t k, float eps,
                          void *C, int32_t *f, float *alpha,
                          void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace pamm_wgrad needs. */
size_t pamm_wgrad_workspace_size(int64_t n, int64_t k, int64_t d, int64_t d_out, int dtype);

/*
 * Approximate weight gradient, the backward-pass phase (page section 2
 * "Metodologia", "Algoritmo in Due Fasi", gradient approximation):
 *   B~[j, :] = sum over rows i with f(i) = j of alpha_i * dY[i, :]
 *   dW       = C^T B~            ([d x d_out], page orientation A^T dZ)
 *
 *   C        [k x d] dtype, f [n] int32, alpha [n] fp32  (read; the triple
 *            saved by pamm_compress)
 *   dY       [n x d_out], leading dimension lddy, dtype  (read)
 *   dW       [d x d_out] fp32, leading dimension lddw >= d_out (written;
 *            when `accumulate` is non-zero the result is added to dW); with
 *            `transpose_out` non-zero it is dW^T [d_out x d], lddw >= d, the
 *            orientation of a framework's weight gradient for a layer
 *            Y = X W^T (same values, written directly in that layout)
 *   ws       workspace of at least pamm_wgrad_workspace_size bytes
 *
 * Rows with f outside [0, k) (the -1 of dropped rows) are skipped and their
 * dY rows are never read; with no kept row (or k = 0) dW is zero (unchanged
 * when accumulating).  Rows are grouped by generator with a stable
 * counting sort and summed in a fixed order, so the result is bitwise
 * deterministic.  fp32 accumulation; for bf16 the generator product splits
 * B~ into two bf16 terms (about 16 significant bits), for fp32 it uses fp32
 * MFMA.
 */
int pamm_wgrad(const void *C, const int32_t *f, const float *alpha,
               int64_t n, int64_t k, int64_t d,
               const void *dY, int64_t d_out, int64_t lddy, int dtype,
               float *dW, int64_t lddw, int accumulate, int transpose_out,
               void *ws, size_t ws_bytes, void *stream);

/* Bytes of the device array that serves as pamm_wgrad_noalloc's workspace
 * (one copy per GPU, held until the process ends). */
#define PAMM_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * pamm_wgrad for callers that cannot allocate device memory: code under
 * stream capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and errors as pamm_wgrad, without the workspace:
 * the library uses a fixed device array of PAMM_NOALLOC_SCRATCH_BYTES
 * instead, one per GPU, created with the library's code object and kept
 * until the process ends.  Nothing is allocated or freed by this call.
 *
 * Errors: those of pamm_wgrad; PAMM_ERR_TOO_LARGE (nothing enqueued) when
 * pamm_wgrad_workspace_size(n, k, d, d_out, dtype) exceeds
 * PAMM_NOALLOC_SCRATCH_BYTES (36 MiB are needed for 32768 tokens, 6144
 * outputs and 1024 generators, 31 MiB for 131072 tokens, 6144 outputs and
 * 256 generators); PAMM_ERR_HIP if the array's device address cannot be
 * obtained.
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind: calls that may overlap on one GPU (different streams, or host
 * threads without ordering) race on it and must be serialised by the
 * caller.  Calls on one stream are ordered and safe.
 */
int pamm_wgrad_noalloc(const void *C, const int32_t *f, const float *alpha,
                       int64_t n, int64_t k, int64_t d,
                       const void *dY, int64_t d_out, int64_t lddy, int dtype,
                       float *dW, int64_t lddw, int accumulate, int transpose_out,
                       void *stream);

/*
 * Reconstruction X~_i = alpha_i * C_f(i) (page section 2 "Metodologia",
 * "Algoritmo in Due Fasi": the approximation of a row by its generator), or a
 * zero row where f(i) is outside [0, k).  The product is formed in fp32 and
 * rounded to dtype (nearest-even).
 *
 *   C [k x d] dtype, f [n], alpha [n]   (read)
 *   Xt [n x d] dtype, leading dimension ldxt (written)
 */
int pamm_decompress(const void *C, const int32_t *f, const float *alpha,
                    int64_t n, int64_t k, int64_t d, int dtype,
                    void *Xt, int64_t ldxt, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAMM_H */
