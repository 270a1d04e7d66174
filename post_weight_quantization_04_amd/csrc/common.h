// Internal declarations shared by the HIP sources of libgptq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <algorithm>

namespace gptq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// ceil(a / b) for b > 0, exact for every int64 a (no intermediate overflow)
static inline int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b > 0); }
static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Hessian (hessian.hip)
// ---------------------------------------------------------------------------
struct HessPlan {
    int tile;          // output tile edge (256 for bf16, 128 for fp32)
    int nb;            // tile blocks along d_in
    int ntiles;        // nb*(nb+1)/2 lower-triangle tiles
    int s_off;         // token splits for off-diagonal tiles
    int s_diag;        // token splits for diagonal tiles
    int nwg;           // work groups of the product kernel
    int64_t slots;     // partial tiles written (= nwg)
};
// max_slots caps the partial tiles (the token split is chosen within it);
// the returned plan may still exceed it when even one split does not fit.
HessPlan hessian_plan(int64_t n, int64_t d, int is_bf16, int64_t max_slots = INT64_MAX);
size_t hessian_ws_bytes(const HessPlan &p);
// The library's own scratch for the allocation-free entry point: a static
// device array of HESS_STATIC_SCRATCH_BYTES per GPU; *ptr = its device
// address on the current device (resolved on first use, then cached).
constexpr size_t HESS_STATIC_SCRATCH_BYTES = (size_t)256 << 20;
hipError_t hessian_static_scratch(void **ptr);
// product kernel: lower tiles of X^T X per token split -> partial slots
hipError_t hessian_product_launch(const void *X, int is_bf16, int64_t n, int64_t d, float *partials,
                                  const HessPlan &p, hipStream_t st);
// H += 2 * (sum of a tile's slots in split order), mirrored to the upper triangle
hipError_t hessian_reduce_launch(int64_t d, float *H, const float *partials, const HessPlan &p,
                                 hipStream_t st);

// ---------------------------------------------------------------------------
// Preparation (prep.hip): diag / lambda, activation order, gathers
// ---------------------------------------------------------------------------
// diag(H) -> dg[d]; lam[0] = damp * mean(dg) (fixed-order reduction).
hipError_t prep_diag_lambda(const float *H, int64_t d, float damp, float *dg, float *lam,
                            hipStream_t st);
// perm[rank(i)] = i with rank by descending dg, ties to the lower index
// (identity when act_order == 0).  rank: int32 [d] scratch.
hipError_t prep_perm(const float *dg, int64_t d, int act_order, int32_t *rank, int32_t *perm, hipStream_t st);
// R[a][b] = H[p(a)][p(b)] (+lam on the diagonal) for a >= b, p(a) = perm[d-1-a].
hipError_t prep_gather_h(const float *H, const int32_t *perm, const float *lam, int64_t d,
                         float *R, hipStream_t st);
// Wp[r][k] = W[r][perm[k]] as fp32.
hipError_t prep_gather_w(const void *W, int is_bf16, const int32_t *perm, int64_t d_out,
                         int64_t d_in, float *Wp, hipStream_t st);

// ---------------------------------------------------------------------------
// Factorization (factor.hip): in-place lower Cholesky of R fused with the
// lower triangular inverse, then the flip that yields U.
// ---------------------------------------------------------------------------
constexpr int FACT_NB = 128;
// panel: d * FACT_NB floats; dinv: 2 * FACT_NB^2 floats (the inverse of the
// current diagonal block and, written ahead by the fused update, the next one).
// info: 2 int32, zero on entry.  info[0] receives the first bad pivot + 1, or
// FACTOR_SYNC_TIMEOUT if the look-ahead's wait for its helpers gave up;
// info[1] counts the helpers' completed diagonal-tile updates.
constexpr int32_t FACTOR_SYNC_TIMEOUT = -1;
// Large matrices take the steps in batches of FACT_BATCH (two-level update):
// inside a batch each step updates only the batch's own later columns and
// rows, and one far update with K = 128 FACT_BATCH then applies the whole
// batch to the rows below it.  factor_batch(d): the batch length used for
// d (1: every step updates the whole trailing matrix).
constexpr int FACT_BATCH = 8;
constexpr int FACT_BATCH_MIN_BLOCKS = 64;
int factor_batch(int64_t d);
// pt: FACT_BATCH * FACT_NB * d floats when factor_batch(d) > 1 (the batch's
// panels transposed), else unused.
hipError_t factor_launch(float *R, int64_t d, float *panel, float *pt, float *dinv, int32_t *info,
                         hipStream_t st);
// U[k][j] = M[d-1-k][d-1-j] for k < j (in place, upper triangle);
// ud[k] = M[d-1-k][d-1-k]; uinv[k] = 1/ud[k].  zero_lower: clear the strictly
// lower triangle afterwards (inspection output only).
hipError_t factor_flip(float *R, int64_t d, float *ud, float *uinv, int zero_lower,
                       hipStream_t st);

// ---------------------------------------------------------------------------
// Quantization loop (quant.hip, trail.hip) and packing (pack.hip)
// ---------------------------------------------------------------------------
struct QuantArgs {
    float *Wp;             // [d_out][d_in] working weights (processing order)
    const float *U;        // [d_in][d_in] upper factor (row-major, upper part valid)
    const float *ud;       // [d_in] U diagonal
    const float *uinv;     // [d_in] 1 / U diagonal
    float *E;              // [K][d_out] pending blocks' errors (block at column b: rows b - near_row0 ..)
    const float *En;       // the same errors as read for the near update (rows < b - near_row0)
    int64_t near_row0;     // first column of the pending blocks (their rows of U)
    int near_k;            // pending columns before the block being quantized (set per block)
    uint8_t *codes;        // [d_in][d_out]
    float *scales;         // [G][d_out]
    float *zeros;          // [G][d_out]
    int64_t d_out, d_in;
    int bits, group, block;   // group: effective group size (d_in when one group)
    int ring_ok;           // the launch's LDS holds the near-update ring (set by the launcher)
};
size_t quant_lds_bytes(int block);
// blocks [b0 + t*B, min(b0 + (t+1)*B, d_in)) for t < nblocks, one launch
hipError_t quant_block_launch(const QuantArgs &a, int64_t b0, int nblocks, int64_t B, hipStream_t st);
// Blocks whose errors are applied to the far columns together (two-level
// lazy update): each block's in-block kernel first takes the pending blocks'
// errors on its own columns, and after far_blocks(B) blocks one product
// applies all pending errors to the columns beyond.  Blocks up to 128 columns
// wide go eight at a time; wider ones (whose near update has no LDS left for a
// staging ring) as many as fill 1024 columns.
constexpr int FAR_BLOCKS = 8;
constexpr int FAR_COLS_WIDE = 1024;
inline int far_blocks(int64_t B) { return B <= 128 ? FAR_BLOCKS : (int)std::max<int64_t>(1, FAR_COLS_WIDE / B); }
// W[:, c_begin:c_end) -= E[0:K) (as [K][d_out]) U[u_row0 : u_row0+K, c_begin:c_end)
hipError_t trail_launch(const QuantArgs &a, int64_t u_row0, int64_t K, int64_t c_begin, int64_t c_end,
                        hipStream_t st);
hipError_t pack_launch(const uint8_t *codes, int64_t d_out, int64_t d_in, int bits,
                       uint32_t *Qpacked, hipStream_t st);

// ---------------------------------------------------------------------------
// Products with a packed layer (dequant.hip): Y = A W_hat^T
// ---------------------------------------------------------------------------
constexpr int GV_MAX_M = 8;   // activation rows per skinny launch
struct DequantArgs {
    const void *A;          // [m][d_in] activations, original column order
    int a_bf16;             // A is bf16 (else fp32)
    const int32_t *perm;    // [d_in] processing order, NULL: identity
    const uint32_t *Q;      // [words][d_out] packed codes
    const float *scales;    // [G][d_out]
    const float *zeros;     // [G][d_out]
    void *Y;                // [m][d_out]
    int y_bf16;             // Y is bf16 (else fp32)
    float *part;            // workspace: partial sums of the k-ranges
    int32_t *counters;      // workspace: one per output tile, zero between calls
    uint16_t *ap;           // workspace: activations in processing order (wide path)
    int64_t m, d_in, d_out;
    int bits, group;        // group: effective group size
    int ngroups;
};
struct DequantWs {
    size_t counters_off, counters_bytes, ap_off, bytes;
};
DequantWs dequant_ws_layout(int64_t m, int64_t d_out, int64_t d_in, int bits);
hipError_t dequant_matmul_launch(const DequantArgs &a, hipStream_t st);

}  // namespace gptq
