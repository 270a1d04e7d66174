// Stage 2: the inverse factor U with H_d^-1 = U^T U (U upper, positive
// diagonal).  "GPTQ (GPT Quantization)", "Algorithme complet (pseudo-code)"
// step 2: invert the damped Hessian through Cholesky.
//
// Route: with J the index reversal, R = J H_d J is factored R = L L^T
// (lower, in place, blocked right-looking, block NB = 128) and at the same
// time M = L^-1 is formed in place (right-looking triangular inverse).  Then
// H_d = V V^T with V = J L J upper, so H_d^-1 = (V^-1)^T V^-1 and
// U = V^-1 = J M J, i.e. U[k][j] = M[d-1-k][d-1-j] (flip kernel).  The
// reversal is applied by the gather that builds R, so the kernels here are a
// plain lower factorization.
//
// Step kb-block k (rows/cols [k0, k1)):
//   potrf  : L_kk = chol(A_kk) and Dinv_k = L_kk^-1 in LDS (one work group);
//            a non-positive or NaN pivot sets *info = first bad index + 1.
//   panel  : P = L[k1:, k] = A[k1:, k] Dinv_k^T (to a panel buffer);
//            M[k, :k0] = -Dinv_k S[k, :k0]; M_kk = Dinv_k (written into R).
//   update : for every lower tile (i, j), i > k:
//              j >  k: A_ij -= P_i P_j^T      (Cholesky trailing update)
//              j == k: S_ik  = P_i Dinv_k     (first term of the inverse sum)
//              j <  k: S_ij += P_i M_kj       (inverse accumulation)
//            where S_ij = sum_{m=j}^{i-1} L_im M_mj occupies the strictly lower
//            blocks already consumed by the Cholesky.
// The tile products run on fp32 MFMA (v_mfma_f32_32x32x2_f32).
#include "common.h"
#include "tile_gemm.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int NB = FACT_NB;   // 128
// ---------------------------------------------------------------------------
// diagonal block: L_kk and Dinv_k = L_kk^-1 (Gauss-Jordan on [L | I] fused
// into the right-looking column loop)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void potrf_kernel(const float *__restrict__ R, int64_t d, int k0, int kb,
                                                    float *__restrict__ dinv, int32_t *__restrict__ info) {
    __shared__ float A[NB][NB + 1];
    __shared__ float X[NB][NB + 1];
    const int tid = threadIdx.x;
    for (int idx = tid; idx < NB * NB; idx += 256) {
        const int i = idx / NB, c = idx % NB;
        A[i][c] = (i < kb && c <= i) ? R[(int64_t)(k0 + i) * d + k0 + c] : 0.f;
        X[i][c] = (i == c) ? 1.f : 0.f;
    }
    __syncthreads();
    const int tx = tid & 15, ty = tid >> 4;
    for (int j = 0; j < kb; ++j) {
        const float piv = A[j][j];
        if (!(piv > 0.f) && tid == 0 && info[0] == 0) info[0] = k0 + j + 1;
        const float ljj = sqrtf(piv);
        const float inv = 1.f / ljj;
        __syncthreads();
        for (int i = j + tid; i < kb; i += 256) A[i][j] = (i == j) ? ljj : A[i][j] * inv;
        for (int c = tid; c <= j; c += 256) X[j][c] *= inv;
        __syncthreads();
        // trailing Cholesky update (rows/cols > j) and inverse update (rows > j, cols <= j)
        for (int i = j + 1 + ty; i < kb; i += 16) {
            const float lij = A[i][j];
            for (int c = j + 1 + tx; c <= i; c += 16) A[i][c] -= lij * A[c][j];
            for (int c = tx; c <= j; c += 16) X[i][c] -= lij * X[j][c];
        }
        __syncthreads();
    }
    for (int idx = tid; idx < NB * NB; idx += 256) {
        const int i = idx / NB, c = idx % NB;
        dinv[idx] = (i < kb && c <= i) ? X[i][c] : 0.f;
    }
}

// part A (row blocks below k): P_i = A_ik Dinv^T -> panel
// part B (column tiles left of k): M_kj = -Dinv S_kj (in place)
// last group: M_kk = Dinv
__global__ __launch_bounds__(256) void panel_kernel(float *__restrict__ R, int64_t d, int k, int nblk,
                                                    float *__restrict__ panel, const float *__restrict__ dinv) {
    __shared__ float As[1][GK * GT];
    __shared__ float Bs[1][GK * GT];
    const int k0 = k * NB, kb = (int)std::min<int64_t>(NB, d - k0), k1 = k0 + kb;
    const int na = nblk - k - 1;
    const int bid = blockIdx.x;
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
    if (bid < na) {
        const int row0 = (k + 1 + bid) * NB;
        const int rows = (int)std::min<int64_t>(NB, d - row0);
        MatRef A{R + (int64_t)row0 * d + k0, d, 1, rows, kb};
        MatRef B{dinv, 1, NB, kb, kb};               // B(kk, n) = Dinv[n][kk]
        gemm_tile(acc, A, B, kb, 1.f, As, Bs);
        store_c(acc, panel + (int64_t)(row0 - k1) * NB, NB, rows, kb);
    } else if (bid < na + k) {
        const int col0 = (bid - na) * NB;
        MatRef A{dinv, NB, 1, kb, kb};
        MatRef B{R + (int64_t)k0 * d + col0, d, 1, kb, NB};
        gemm_tile(acc, A, B, kb, -1.f, As, Bs);
        store_c(acc, R + (int64_t)k0 * d + col0, d, kb, NB);
    } else {
        for (int idx = threadIdx.x; idx < kb * kb; idx += 256) {
            const int i = idx / kb, c = idx % kb;
            R[(int64_t)(k0 + i) * d + k0 + c] = dinv[i * NB + c];
        }
    }
}

__global__ __launch_bounds__(256) void update_kernel(float *__restrict__ R, int64_t d, int k, int nblk,
                                                     const float *__restrict__ panel,
                                                     const float *__restrict__ dinv) {
    __shared__ float As[1][GK * GT];
    __shared__ float Bs[1][GK * GT];
    int i, j;
    tile_coords(blockIdx.x + (k + 1) * (k + 2) / 2, i, j);
    const int k0 = k * NB, kb = (int)std::min<int64_t>(NB, d - k0), k1 = k0 + kb;
    const int row0 = i * NB, col0 = j * NB;
    const int rows = (int)std::min<int64_t>(NB, d - row0);
    const int cols = (int)std::min<int64_t>(NB, d - col0);
    float *C = R + (int64_t)row0 * d + col0;
    MatRef A{panel + (int64_t)(row0 - k1) * NB, NB, 1, rows, kb};
    f32x16 acc[4];
    if (j == k) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = f32x16{};
        MatRef B{dinv, NB, 1, kb, kb};
        gemm_tile(acc, A, B, kb, 1.f, As, Bs);
    } else if (j < k) {
        load_c(acc, C, d, rows, cols);
        MatRef B{R + (int64_t)k0 * d + col0, d, 1, kb, cols};
        gemm_tile(acc, A, B, kb, 1.f, As, Bs);
    } else {
        load_c(acc, C, d, rows, cols);
        MatRef B{panel + (int64_t)(col0 - k1) * NB, 1, NB, kb, cols};   // B(kk, n) = P[col0+n][kk]
        gemm_tile(acc, A, B, kb, -1.f, As, Bs);
    }
    store_c(acc, C, d, rows, cols);
}

__global__ void flip_kernel(float *__restrict__ R, int64_t d, float *__restrict__ ud) {
    // one row r per block: U[r][c] = M[d-1-r][d-1-c] for c > r, ud[r] = M[d-1-r][d-1-r]
    const int64_t r = blockIdx.x;
    const int64_t src = (d - 1 - r) * d + (d - 1);
    for (int64_t c = r + 1 + threadIdx.x; c < d; c += blockDim.x) R[r * d + c] = R[src - c];
    if (threadIdx.x == 0) ud[r] = R[(d - 1 - r) * d + (d - 1 - r)];
}

__global__ void finish_diag_kernel(float *__restrict__ R, int64_t d, const float *__restrict__ ud,
                                   float *__restrict__ uinv, int zero_lower) {
    const int64_t r = blockIdx.x;
    if (threadIdx.x == 0) {
        R[r * d + r] = ud[r];
        uinv[r] = 1.f / ud[r];
    }
    if (zero_lower)
        for (int64_t c = threadIdx.x; c < r; c += blockDim.x) R[r * d + c] = 0.f;
}

}  // namespace

hipError_t factor_launch(float *R, int64_t d, float *panel, float *dinv, int32_t *info, hipStream_t st) {
    const int nblk = (int)cdiv(d, NB);
    for (int k = 0; k < nblk; ++k) {
        const int k0 = k * NB, kb = (int)std::min<int64_t>(NB, d - k0);
        potrf_kernel<<<1, 256, 0, st>>>(R, d, k0, kb, dinv, info);
        const int na = nblk - k - 1;
        panel_kernel<<<na + k + 1, 256, 0, st>>>(R, d, k, nblk, panel, dinv);
        const int nup = nblk * (nblk + 1) / 2 - (k + 1) * (k + 2) / 2;
        if (nup > 0) update_kernel<<<nup, 256, 0, st>>>(R, d, k, nblk, panel, dinv);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t factor_flip(float *R, int64_t d, float *ud, float *uinv, int zero_lower, hipStream_t st) {
    // the diagonal of R is read before any write to it: flip_kernel only writes
    // strictly-upper entries and ud; finish_diag_kernel then writes the diagonal.
    flip_kernel<<<(unsigned)d, 256, 0, st>>>(R, d, ud);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    finish_diag_kernel<<<(unsigned)d, 256, 0, st>>>(R, d, ud, uinv, zero_lower);
    return hipGetLastError();
}

}  // namespace gptq
