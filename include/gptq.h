/*
 * gptq.h -- C ABI of libgptq, a GPTQ layer quantizer for AMD MI355X (gfx950).
 *
 * The method (web pages on GPTQ, cited by page title and section):
 *   - "GPTQ (GPT Quantization)" (brain.gartu.xyz), "Fondation theorique : OBQ":
 *     H = 2 X^T X over calibration inputs; quantize a column, then move the
 *     remaining columns by -e_i / (H^-1)_ii * (H^-1)_{i,F}.
 *   - same page, "Algorithme complet (pseudo-code)": damp H with lambda*I,
 *     invert through Cholesky, quantize in batches with a lazy update of the
 *     later columns.
 *   - "Optimization Gptq" (skillsdirectory.com), "Quantizacao group-wise" and
 *     "Configuracoes de quantizacao": per-group scale and zero point; bits,
 *     group_size, desc_act, damp_percent.
 *
 * Conventions for every entry point:
 *   - Pointers named X, W, H, Qpacked, scales, zeros, perm, workspace are
 *     DEVICE pointers (HIP global memory); every size is in elements unless
 *     it says bytes.  All matrices are row-major and densely packed.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it; calls return before the GPU finishes unless
 *     stated otherwise.  The caller keeps every buffer alive until the stream
 *     has passed the call.
 *   - The caller owns all memory.  The library never allocates or frees
 *     device memory; the one exception is the fixed static scratch that
 *     gptq_hessian_accumulate_noalloc keeps per GPU (see there).
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     GPTQ_EINVAL nothing was launched and no output was written;
 *     gptq_last_error() gives a detail string (thread-local).
 *   - No C++ exception crosses this interface.
 *   - Calls on different streams with distinct workspaces and outputs may run
 *     concurrently.
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define GPTQ_API __attribute__((visibility("default")))
#else
#define GPTQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GPTQ_OK = 0,
    GPTQ_EINVAL = 1,   /* bad argument (checked on the host, nothing launched) */
    GPTQ_ENOTSPD = 2,  /* damped Hessian not positive definite (a pivot <= 0 or NaN) */
    GPTQ_EHIP = 3,     /* a HIP runtime call failed, or a kernel's bounded wait for
                          another work group gave up (reported, never hung on) */
    GPTQ_ENOMEM = 4    /* workspace smaller than the size query returned */
} gptq_status;

typedef enum {
    GPTQ_F32 = 0,      /* IEEE binary32 */
    GPTQ_BF16 = 1      /* bfloat16 (upper 16 bits of a binary32) */
} gptq_dtype;

/* ---------------------------------------------------------------------------
 * Stage 1: Hessian accumulation.
 * "GPTQ (GPT Quantization)", sections "Fondation theorique : OBQ" and
 * "Algorithme complet (pseudo-code)" step 1: H = 2 X^T X.
 *
 * Computes H[i][j] += 2 * sum_t X[t][i] * X[t][j] for all i, j.
 *   X        device, [n][d_in] row-major, dtype x_dtype.  Products are formed
 *            exactly and accumulated in fp32 (bf16 inputs on bf16 MFMA, fp32
 *            inputs on fp32 MFMA).
 *   H        device, [d_in][d_in] fp32.  Read and written (accumulated): zero
 *            it before the first call.  Both triangles are written and the
 *            result is bitwise symmetric if H was.
 *   workspace device scratch of at least gptq_hessian_workspace_size(n, d_in,
 *            x_dtype) bytes (may be NULL when that size is 0).
 * n == 0 is a no-op.  Calling it on consecutive token chunks equals one call
 * on their concatenation up to fp32 rounding; results are deterministic.
 * Errors: EINVAL (null pointer, n < 0, d_in outside [1, 2^20], bad dtype), ENOMEM
 * (workspace too small), EHIP.
 * ------------------------------------------------------------------------- */
GPTQ_API size_t gptq_hessian_workspace_size(int64_t n, int64_t d_in, gptq_dtype x_dtype);

GPTQ_API gptq_status gptq_hessian_accumulate(const void *X, gptq_dtype x_dtype, int64_t n, int64_t d_in,
                                    float *H, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* ---------------------------------------------------------------------------
 * Stage 1 without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same operation, arguments and results as
 * gptq_hessian_accumulate (equal up to fp32 summation order: the token split
 * is chosen to fit the scratch), but the partial tiles live in a scratch
 * array that the library holds statically: 256 MiB per GPU it runs on, kept
 * until the process ends.  Calls nothing that allocates.  Every call on one
 * GPU shares that GPU's scratch, so calls that overlap on one GPU (other
 * streams, other threads) race and must be serialized by the caller.
 * EINVAL (before anything is enqueued) when the partial tiles do not fit:
 * d_in above gptq_hessian_noalloc_max_d_in(x_dtype), or at large d_in a token
 * range long enough to need several token splits (32-bit row offsets limit a
 * split to 2^30 / d_in tokens); other errors as gptq_hessian_accumulate.
 * ------------------------------------------------------------------------- */
GPTQ_API gptq_status gptq_hessian_accumulate_noalloc(const void *X, gptq_dtype x_dtype, int64_t n, int64_t d_in,
                                                     float *H, void *stream);
GPTQ_API int64_t gptq_hessian_noalloc_max_d_in(gptq_dtype x_dtype);   /* host only; -1 for a bad dtype */

/* ---------------------------------------------------------------------------
 * Stages 2-5: quantize one layer.
 * "GPTQ (GPT Quantization)", "Algorithme complet (pseudo-code)" steps 1-3 and
 * "Fondation theorique : OBQ"; "Optimization Gptq", "Quantizacao group-wise"
 * and "Configuracoes de quantizacao" (bits, group_size, desc_act,
 * damp_percent).
 *
 * Inputs (read-only):
 *   W          device, [d_out][d_in], dtype w_dtype (one row per output
 *              channel, one column per input channel).
 *   H          device, [d_in][d_in] fp32, the undamped Hessian from stage 1.
 *   bits       2, 3, 4 or 8.
 *   group_size -1 (one group per row) or a multiple of 16; values >= d_in
 *              also mean one group per row.  Unless one group spans the row,
 *              block_size must be a multiple of group_size (or >= d_in).
 *   block_size >= 1: columns per lazy batch (clamped to d_in).
 *   damp       relative damping, lambda = damp * mean(diag H); finite, >= 0.
 *   act_order  0: natural column order; 1: columns processed by descending
 *              diag(H) (stable, ties to the lower index).
 * Outputs (caller-allocated, device, all in processing order):
 *   Qpacked    uint32 [gptq_packed_words(d_in, bits)][d_out].  Row r's codes
 *              form a little-endian bit stream, code k at stream bits
 *              [bits*k, bits*k + bits); word w holds stream bits [32w, 32w+32).
 *   scales     fp32 [gptq_num_groups(d_in, group_size)][d_out].
 *   zeros      fp32 [gptq_num_groups(d_in, group_size)][d_out], integers in
 *              [0, 2^bits - 1].
 *   perm       int32 [d_in]: perm[k] is the original column processed k-th.
 *   Dequantization: W_hat[r][perm[k]] = scales[k/g][r] * (code(r,k) - zeros[k/g][r]).
 * workspace   device scratch of at least gptq_quantize_layer_workspace_size(...)
 *             bytes.
 * Everything is enqueued on `stream`; the call then synchronizes `stream` once,
 * at the end, to read the factorization's positive-definiteness flag.
 * Errors: EINVAL, ENOMEM (nothing launched); ENOTSPD (outputs undefined);
 * EHIP (also when the factorization's look-ahead gave up waiting for the
 * groups updating its diagonal tile; outputs undefined).
 * ------------------------------------------------------------------------- */
GPTQ_API size_t gptq_quantize_layer_workspace_size(int64_t d_out, int64_t d_in, int bits, int group_size,
                                          int block_size, int act_order);

GPTQ_API gptq_status gptq_quantize_layer(const void *W, gptq_dtype w_dtype, int64_t d_out, int64_t d_in,
                                const float *H, int bits, int group_size, int block_size,
                                float damp, int act_order,
                                uint32_t *Qpacked, float *scales, float *zeros, int32_t *perm,
                                void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Several layers that read the same input (q/k/v of an attention block,
 * gate/up of an MLP) share one Hessian, hence one order and one inverse
 * factor: "GPTQ" (wikiprompt.org), "Abordagem Tecnica" (the model is
 * quantized layer by layer from each layer's own inputs) and "GPTQ (GPT
 * Quantization)", "Fondation theorique : OBQ" (H depends only on the inputs
 * X).  Rows are independent given the factor, so this factors H once and
 * then quantizes each layer exactly as gptq_quantize_layer would (the same
 * kernels in the same order: the results are bitwise those of one
 * gptq_quantize_layer call per layer).
 *   n_layers   1 .. 4096.
 *   W, d_out, Qpacked, scales, zeros: HOST arrays of n_layers entries (the
 *              pointers they hold are device pointers; each layer has its own
 *              d_out and its own outputs, laid out as for
 *              gptq_quantize_layer).
 *   perm       one int32 [d_in] for all the layers.
 *   workspace  gptq_quantize_layers_workspace_size(...) bytes (that of the
 *              widest layer).
 * Every other argument, the synchronization and the errors are those of
 * gptq_quantize_layer.  Layers are processed in order on `stream`.
 * ------------------------------------------------------------------------- */
GPTQ_API size_t gptq_quantize_layers_workspace_size(int n_layers, const int64_t *d_out, int64_t d_in, int bits,
                                                    int group_size, int block_size, int act_order);

GPTQ_API gptq_status gptq_quantize_layers(int n_layers, const void *const *W, gptq_dtype w_dtype,
                                          const int64_t *d_out, int64_t d_in, const float *H, int bits,
                                          int group_size, int block_size, float damp, int act_order,
                                          uint32_t *const *Qpacked, float *const *scales, float *const *zeros,
                                          int32_t *perm, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Stage 2 alone, for inspection: activation order and the inverse factor.
 * "Algorithme complet (pseudo-code)" steps 1-2 (damping, inverse through
 * Cholesky).  Writes perm (int32 [d_in]) and U (fp32 [d_in][d_in], device):
 * the upper Cholesky factor of (H[perm][:,perm] + lambda I)^-1, i.e.
 * H_d^-1 = U^T U; entries below the diagonal are set to 0.  Uses the same
 * workspace as gptq_quantize_layer (size query with d_out = 1).  Synchronizes
 * `stream` once, at the end.  Errors as for gptq_quantize_layer.
 * ------------------------------------------------------------------------- */
GPTQ_API gptq_status gptq_inverse_factor(const float *H, int64_t d_in, float damp, int act_order,
                                int32_t *perm, float *U, void *workspace, size_t workspace_bytes,
                                void *stream);

/* ---------------------------------------------------------------------------
 * Products with a quantized layer: what inference runs on the packed weights.
 * "Optimization Gptq", "Backends de kernel" (kernels computing with the 4-bit
 * weights) and "GPTQ (GPT Quantization)", "Limitations" (the weights are
 * dequantized for each product).
 *
 * Y[i][r] = sum_c A[i][c] * W_hat[r][c] for i < m, r < d_out, where
 * W_hat[r][perm[k]] = scales[k/g][r] * (code(r, k) - zeros[k/g][r]) is the
 * layer exactly as gptq_quantize_layer stored it (g the effective group size).
 *   A        device, [m][d_in], a_dtype BF16 or F32, original column order
 *            (the kernels gather it into processing order through perm).
 *   Qpacked, scales, zeros, perm
 *            device, gptq_quantize_layer's outputs for a d_out x d_in layer
 *            quantized with `bits` and `group_size`.  perm may be NULL
 *            (identity, as act_order = 0 writes it).
 *   Y        device, [m][d_out], y_dtype F32 or BF16 (rounded to nearest
 *            even from the fp32 result).
 * Two paths, both deterministic:
 *   - skinny (m < 16, or fp32 activations, or d_in % 8 != 0; the decode
 *     shape, bound by reading the packed weights): codes are multiplied in
 *     fp32 with the fp32-widened activations, every 16 codes the group's
 *     scale and zero point are applied as s * (sum A q) - s z * (sum A), and
 *     the k-ranges' partial sums are added in a fixed order; up to 8 rows of
 *     A per launch, larger m in chunks of 8;
 *   - wide (m >= 16 bf16 rows, d_in % 8 == 0; prefill): per group the exact
 *     integers q - z meet the activations on bf16 matrix cores (every product
 *     exact, fp32 sums), and Y += s * (group sum).
 * workspace  device scratch of gptq_dequant_matmul_workspace_size(m, d_out,
 *            d_in, bits, group_size) bytes (0 when m == 0; may then be NULL).
 *            It holds the k-ranges' partial sums and one completion counter
 *            per output tile: it must be ZEROED before its first use; every
 *            call leaves it ready for the next (counters back at zero).
 *            A workspace serves one call at a time.
 * m == 0 is a no-op.  Errors: EINVAL (bad sizes, bits, group_size or dtype,
 * NULL pointer; nothing launched), ENOMEM (workspace too small), EHIP.
 * ------------------------------------------------------------------------- */
GPTQ_API size_t gptq_dequant_matmul_workspace_size(int64_t m, int64_t d_out, int64_t d_in, int bits,
                                                   int group_size);
GPTQ_API gptq_status gptq_dequant_matmul(const void *A, gptq_dtype a_dtype, int64_t m, int64_t d_in,
                                         const uint32_t *Qpacked, const float *scales, const float *zeros,
                                         const int32_t *perm, int64_t d_out, int bits, int group_size,
                                         void *Y, gptq_dtype y_dtype, void *workspace, size_t workspace_bytes,
                                         void *stream);

/* ---------------------------------------------------------------------------
 * Stage timing (tracing aid).  gptq_profile_enable(stage_mask): bit s set
 * makes every later call record a pair of hipEvents around stage s's launches
 * on the caller's stream (GPTQ_PROFILE_ALL: every stage; 0: none).  Reading
 * waits for those events and returns the summed GPU time per stage since the
 * last reset.  Process-wide state: enable it only while one thread drives
 * the library.  Stages:
 *   0 hessian product kernel      1 hessian reduce/mirror kernel
 *   2 damping, order and gathers   3 blocked Cholesky + inverse
 *   4 flip to U                    5 in-block quantize kernels
 *   6 trailing-update kernels      7 bit packing
 * ------------------------------------------------------------------------- */
#define GPTQ_NUM_STAGES 8
#define GPTQ_PROFILE_ALL ((1 << GPTQ_NUM_STAGES) - 1)
typedef struct {
    double ms[GPTQ_NUM_STAGES];        /* summed GPU milliseconds */
    int64_t launches[GPTQ_NUM_STAGES]; /* timed launch groups */
} gptq_profile;

GPTQ_API void gptq_profile_enable(int stage_mask);
GPTQ_API gptq_status gptq_profile_read(gptq_profile *out, int reset);
GPTQ_API const char *gptq_profile_stage_name(int stage);

/* Host-only helpers (no GPU work). */
GPTQ_API int64_t gptq_packed_words(int64_t d_in, int bits);          /* ceil(bits*d_in/32), -1 if invalid */
GPTQ_API int64_t gptq_num_groups(int64_t d_in, int group_size);      /* ceil(d_in/g), -1 if invalid */
GPTQ_API const char *gptq_status_string(gptq_status s);
GPTQ_API const char *gptq_last_error(void);                          /* detail of the last failure on this thread */
GPTQ_API const char *gptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H */
