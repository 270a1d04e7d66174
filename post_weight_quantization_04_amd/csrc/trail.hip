// Stage 4: the lazy trailing update
//   W[:, c_begin:c_end) -= E U[u_row0 : u_row0 + K, c_begin:c_end)
// ("GPTQ (GPT Quantization)", "Algorithme complet (pseudo-code)" step 3: a
// batch's errors are pushed onto the remaining columns once per batch).  E
// holds the errors of one or more consecutive blocks, already divided by
// U_kk, so the product uses U's rows as they are.  With more than one block
// per far update it is applied in two levels: after each block to the next
// block's columns only, and every few blocks to all columns beyond, with the
// pending blocks' errors stacked (the same sum, fewer passes over W).  fp32
// operands on fp32 MFMA; the W tile is read into the accumulators, updated
// and written back.
#include "common.h"
#include "tile_gemm.h"

#include <algorithm>

namespace gptq {

namespace {

__global__ __launch_bounds__(256) void trail_kernel(QuantArgs a, int u_row0, int K, int c_begin, int c_end) {
    __shared__ __attribute__((aligned(16))) float lds[4 * GSTAGE];
    const int64_t row0 = (int64_t)blockIdx.x * GT;
    const int64_t col0 = (int64_t)c_begin + (int64_t)blockIdx.y * GT;
    const int rows = (int)std::min<int64_t>(GT, a.d_out - row0);
    const int cols = (int)std::min<int64_t>(GT, c_end - col0);
    const float *A = a.E + row0;                                   // A(m, k) = E[k][row0 + m]
    const float *B = a.U + (int64_t)u_row0 * a.d_in + col0;        // B(k, n) = U[u_row0 + k][col0 + n]
    float *C = a.Wp + row0 * a.d_in + col0;
    f32x16 acc[4];
    load_c(acc, C, a.d_in, rows, cols);
    gemm_tile<false, false>(acc, A, a.d_out, B, a.d_in, rows, cols, K, -1.f,
                            aligned16(A, a.d_out) && aligned16(B, a.d_in), lds);
    store_c(acc, C, a.d_in, rows, cols);
}

}  // namespace

hipError_t trail_launch(const QuantArgs &a, int64_t u_row0, int64_t K, int64_t c_begin, int64_t c_end,
                        hipStream_t st) {
    if (c_end <= c_begin || K <= 0) return hipSuccess;
    dim3 grid((unsigned)cdiv(a.d_out, GT), (unsigned)cdiv(c_end - c_begin, GT));
    trail_kernel<<<grid, 256, 0, st>>>(a, (int)u_row0, (int)K, (int)c_begin, (int)c_end);
    return hipGetLastError();
}

}  // namespace gptq
