// fp32-MFMA 128x128 tile product shared by the factorization and the
// trailing update: acc += alpha * A(128 x K) * B(K x 128), with both operands
// given by a strided view and staged through LDS in k-major layout.
// Four waves own 64x64 quadrants, each as 2x2 v_mfma_f32_32x32x2_f32 tiles.
#pragma once
#include "common.h"

namespace gptq {
namespace {

constexpr int GT = 128;       // product tile edge
constexpr int GK = 32;        // k chunk staged per pass

struct MatRef {
    const float *p;
    int64_t s0, s1;           // element (a, b) at p[a*s0 + b*s1]
    int rows, cols;           // valid range
};

__device__ __forceinline__ float mref(const MatRef &m, int a, int b) {
    return (a < m.rows && b < m.cols) ? m.p[a * m.s0 + b * m.s1] : 0.f;
}

__device__ __forceinline__ void tile_coords(int t, int &I, int &J) {
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > t) --i;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    I = i;
    J = t - i * (i + 1) / 2;
}

// acc[ma*2+mb] holds the wave's 32x32 sub-tile (ma, mb) of a 128x128 tile in
// MFMA layout: lane (h, li), register 4a+b <-> row 8a+4h+b, column li.
__device__ __forceinline__ void tile_rc(int ma, int mb, int a, int b, int &r, int &c) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    r = wr * 64 + ma * 32 + 8 * a + 4 * h + b;
    c = wc * 64 + mb * 32 + li;
}

__device__ __forceinline__ void load_c(f32x16 (&acc)[4], const float *C, int64_t ldc, int rows, int cols) {
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    int r, c;
                    tile_rc(ma, mb, a, b, r, c);
                    acc[ma * 2 + mb][4 * a + b] = (r < rows && c < cols) ? C[r * ldc + c] : 0.f;
                }
}

__device__ __forceinline__ void store_c(const f32x16 (&acc)[4], float *C, int64_t ldc, int rows, int cols) {
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    int r, c;
                    tile_rc(ma, mb, a, b, r, c);
                    if (r < rows && c < cols) C[r * ldc + c] = acc[ma * 2 + mb][4 * a + b];
                }
}

// acc += alpha * A(128 x K) * B(K x 128), operands staged through LDS.
__device__ void gemm_tile(f32x16 (&acc)[4], const MatRef &A, const MatRef &B, int K, float alpha,
                          float (*As)[GK * GT], float (*Bs)[GK * GT]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    const int nch = (K + GK - 1) / GK;
    for (int ch = 0; ch < nch; ++ch) {
        const int kb = ch * GK;
#pragma unroll 4
        for (int e = 0; e < (GK * GT) / 256; ++e) {
            const int idx = tid + 256 * e;
            const int kk = idx / GT, m = idx % GT;
            As[0][idx] = alpha * mref(A, m, kb + kk);
            Bs[0][idx] = mref(B, kb + kk, m);
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < GK / 2; ++s) {
            const int row = 2 * s + h;
            float fa[2], fb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                fa[m] = As[0][row * GT + wr * 64 + m * 32 + li];
                fb[m] = Bs[0][row * GT + wc * 64 + m * 32 + li];
            }
#pragma unroll
            for (int ma = 0; ma < 2; ++ma)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[ma * 2 + mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[ma], fb[mb], acc[ma * 2 + mb], 0, 0, 0);
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace gptq
