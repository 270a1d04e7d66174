// Stage 4: the lazy trailing update after a block [b, e):
//   W[:, e:] -= E[:, b:e] U[b:e, e:]
// ("GPTQ (GPT Quantization)", "Algorithme complet (pseudo-code)" step 3: the
// batch error is pushed onto the remaining columns once per batch).  E holds
// the block's errors already divided by U_kk, so the product uses U's rows as
// they are.  fp32 operands on fp32 MFMA; the W tile is read into the
// accumulators, updated and written back.
#include "common.h"
#include "tile_gemm.h"

#include <algorithm>

namespace gptq {

namespace {

__global__ __launch_bounds__(256) void trail_kernel(QuantArgs a, int b, int e) {
    __shared__ __attribute__((aligned(16))) float lds[4 * GSTAGE];
    const int64_t row0 = (int64_t)blockIdx.x * GT;
    const int64_t col0 = (int64_t)e + (int64_t)blockIdx.y * GT;
    const int rows = (int)std::min<int64_t>(GT, a.d_out - row0);
    const int cols = (int)std::min<int64_t>(GT, a.d_in - col0);
    const int K = e - b;
    const float *A = a.E + row0;                                   // A(m, k) = E[k][row0 + m]
    const float *B = a.U + (int64_t)b * a.d_in + col0;             // B(k, n) = U[b + k][col0 + n]
    float *C = a.Wp + row0 * a.d_in + col0;
    f32x16 acc[4];
    load_c(acc, C, a.d_in, rows, cols);
    gemm_tile<false, false>(acc, A, a.d_out, B, a.d_in, rows, cols, K, -1.f,
                            aligned16(A, a.d_out) && aligned16(B, a.d_in), lds);
    store_c(acc, C, a.d_in, rows, cols);
}

}  // namespace

hipError_t trail_launch(const QuantArgs &a, int64_t b, int64_t e, hipStream_t st) {
    if (e >= a.d_in) return hipSuccess;
    dim3 grid((unsigned)cdiv(a.d_out, GT), (unsigned)cdiv(a.d_in - e, GT));
    trail_kernel<<<grid, 256, 0, st>>>(a, (int)b, (int)e);
    return hipGetLastError();
}

}  // namespace gptq
