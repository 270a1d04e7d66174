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
// Step over block k (rows/cols [k0, k1)):
//   potrf  : Dinv_k = chol(A_kk)^-1, one work group (run inside the previous
//            step's update kernel as look-ahead, or alone for k = 0); a
//            non-positive or NaN pivot sets *info = first bad index + 1.
//   panel  : P = L[k1:, k] = A[k1:, k] Dinv_k^T (to a panel buffer);
//            M[k, :k0] = -Dinv_k S[k, :k0]; M_kk = Dinv_k (written into R).
//   update : for every lower tile (i, j), i > k:
//              j >  k: A_ij -= P_i P_j^T      (Cholesky trailing update)
//              j == k: S_ik  = P_i Dinv_k     (first term of the inverse sum)
//              j <  k: S_ij += P_i M_kj       (inverse accumulation)
//            where S_ij = sum_{m=j}^{i-1} L_im M_mj occupies the strictly lower
//            blocks already consumed by the Cholesky.  Work group 0 takes tile
//            (k+1, k+1) and then factors it (potrf of the next step).
// Dinv alternates between two buffers by step parity because the fused
// potrf writes the next step's while the rest of the kernel reads this one.
// The tile products run on fp32 MFMA (v_mfma_f32_32x32x2_f32).
#include "common.h"
#include "tile_gemm.h"

#include <algorithm>
#include <utility>

namespace gptq {

namespace {

constexpr int NB = FACT_NB;   // 128

// ---------------------------------------------------------------------------
// Diagonal block: X = chol(A)^-1 by an in-place Gauss-Jordan sweep.
// Thread (ty, tx) = (tid%16, tid/16) keeps the 8x8 tile of rows 8ty.., cols
// 8tx.. in registers, so a wave owns four whole tile columns.  At column j
// the tile holds L^-1 for rows/cols <= j (the finished part) and the
// trailing Cholesky matrix beyond.  Column j becomes l_ij = a_ij / l_jj; the
// vector v[i] = l_ij (i > j), X[j][i] (i < j), 0 (i = j) is broadcast through
// LDS and every element with row i > j takes T[i][c] -= l_ij * v[c]: the
// Cholesky update for c > j and the inverse update for c < j in one pass;
// column j itself becomes -l_ij / l_jj.
// Latency choices: every thread tracks the eight pivots of the current tile
// column with the same fused multiply-add the owning thread applies, so all
// threads derive bitwise-identical pivots without a broadcast; only the wave
// owning tile column j computes column j; row j of the inverse is published
// unscaled at the end of the previous column and scaled by 1/l_jj on read.
// One barrier per column (double-buffered v) plus one per tile column.
// Rows/cols beyond kb are padded with the identity.
// ---------------------------------------------------------------------------
template <int JJ>
__device__ __forceinline__ void potrf_publish_row(const float (&T)[8][8], int ty, int tx, int jt, float *vb) {
    // row j = 8*jt + JJ of the inverse (columns < j), unscaled
    if (ty == jt) {
        if (tx < jt) {
            *(f32x4 *)(vb + 8 * tx) = f32x4{T[JJ][0], T[JJ][1], T[JJ][2], T[JJ][3]};
            *(f32x4 *)(vb + 8 * tx + 4) = f32x4{T[JJ][4], T[JJ][5], T[JJ][6], T[JJ][7]};
        } else if (tx == jt) {
#pragma unroll
            for (int c = 0; c < JJ; ++c) vb[8 * tx + c] = T[JJ][c];
        }
    }
}

template <int JJ>
__device__ __forceinline__ void potrf_step(float (&T)[8][8], float (&d8)[8], int ty, int tx, int jt, int tid, int kb,
                                           int info_base, int32_t *__restrict__ info, float *vbuf) {
    const int j = 8 * jt + JJ;
    float *vb = vbuf + (JJ & 1) * NB;
    const float p = d8[JJ];
    if (tid == 0 && !(p > 0.f) && j < kb && info[0] == 0) info[0] = info_base + j + 1;
    // 1/l_jj from the hardware reciprocal square root (about 1 ulp)
    const float il = __builtin_amdgcn_rsqf(p);
    if (tx == jt) {
        // column j: l_ij for rows below, the inverse's column j in place
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int i = 8 * ty + r;
            const float lij = T[r][JJ] * il;
            T[r][JJ] = (i > j) ? -lij * il : ((i == j) ? il : T[r][JJ]);
            if (i >= j) vb[i] = (i > j) ? lij : 0.f;
        }
    }
    if (ty == jt && tx <= jt) {
        // row j of the inverse takes its 1/l_jj (it was published unscaled)
#pragma unroll
        for (int c = 0; c < 8; ++c) T[JJ][c] = (8 * tx + c < j) ? T[JJ][c] * il : T[JJ][c];
    }
    __syncthreads();
    const f32x4 r0 = *(const f32x4 *)(vb + 8 * ty), r1 = *(const f32x4 *)(vb + 8 * ty + 4);
    const f32x4 c0 = *(const f32x4 *)(vb + 8 * tx), c1 = *(const f32x4 *)(vb + 8 * tx + 4);
    const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    float lr[8], vc[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) lr[r] = (8 * ty + r > j) ? rv[r] : 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) vc[c] = (8 * tx + c < j) ? cv[c] * il : cv[c];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) T[r][c] = fmaf(-lr[r], vc[c], T[r][c]);
    // the remaining pivots of this tile column take the same update
#pragma unroll
    for (int q = JJ + 1; q < 8; ++q) {
        const float lq = vb[8 * jt + q];
        d8[q] = fmaf(-lq, lq, d8[q]);
    }
    // publish row j+1 of the inverse for the next column (other buffer)
    float *vn = vbuf + ((JJ + 1) & 1) * NB;
    if (JJ < 7) potrf_publish_row<(JJ + 1) & 7>(T, ty, tx, jt, vn);
    else potrf_publish_row<0>(T, ty, tx, jt + 1, vn);
}

template <int... S>
__device__ __forceinline__ void potrf_tile_column(float (&T)[8][8], float (&d8)[8], int ty, int tx, int jt, int tid,
                                                  int kb, int info_base, int32_t *__restrict__ info, float *vbuf,
                                                  std::integer_sequence<int, S...>) {
    (potrf_step<S>(T, d8, ty, tx, jt, tid, kb, info_base, info, vbuf), ...);
}

__device__ __forceinline__ void potrf_block(const float *__restrict__ src, int64_t ld, int kb, int info_base,
                                            float *__restrict__ dinv, int32_t *__restrict__ info, float *vbuf,
                                            float *dgbuf) {
    const int tid = threadIdx.x;
    const int ty = tid & 15, tx = tid >> 4;
    float T[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = 8 * ty + r, cc = 8 * tx + c;
            float v = (i == cc) ? 1.f : 0.f;
            if (i < kb && cc < kb && cc <= i) v = src[(int64_t)i * ld + cc];
            T[r][c] = v;
        }
    for (int jt = 0; jt < 16; ++jt) {
        // pivots of tile column jt: the diagonal of tile (jt, jt), current
        if (ty == jt && tx == jt) {
#pragma unroll
            for (int q = 0; q < 8; ++q) dgbuf[q] = T[q][q];
        }
        __syncthreads();
        float d8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) d8[q] = dgbuf[q];
        potrf_tile_column(T, d8, ty, tx, jt, tid, kb, info_base, info, vbuf, std::make_integer_sequence<int, 8>{});
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = 8 * ty + r, cc = 8 * tx + c;
            dinv[i * NB + cc] = (i < kb && cc < kb && cc <= i) ? T[r][c] : 0.f;
        }
}

__global__ __launch_bounds__(256) void potrf_kernel(const float *__restrict__ R, int64_t d, int k0, int kb,
                                                    float *__restrict__ dinv, int32_t *__restrict__ info) {
    __shared__ __attribute__((aligned(16))) float vbuf[2 * NB];
    __shared__ float dgbuf[8];
    potrf_block(R + (int64_t)k0 * d + k0, d, kb, k0, dinv, info, vbuf, dgbuf);
}

// part A (row blocks below k): P_i = A_ik Dinv^T -> panel
// part B (column tiles left of k): M_kj = -Dinv S_kj (in place)
// last group: M_kk = Dinv
__global__ __launch_bounds__(256) void panel_kernel(float *__restrict__ R, int64_t d, int k, int nblk,
                                                    float *__restrict__ panel, const float *__restrict__ dinv) {
    __shared__ __attribute__((aligned(16))) float lds[4 * GSTAGE];
    const int k0 = k * NB, kb = (int)std::min<int64_t>(NB, d - k0), k1 = k0 + kb;
    const int na = nblk - k - 1;
    const int bid = blockIdx.x;
    f32x16 acc[4];
    zero_acc(acc);
    if (bid < na) {
        const int row0 = (k + 1 + bid) * NB;
        const int rows = (int)std::min<int64_t>(NB, d - row0);
        const float *A = R + (int64_t)row0 * d + k0;          // A(m, k) = R[row0+m][k0+k]
        // B(k, n) = Dinv[n][k]: k-contiguous rows of Dinv
        gemm_tile<true, true>(acc, A, d, dinv, NB, rows, kb, kb, 1.f, aligned16(A, d), lds);
        store_c(acc, panel + (int64_t)(row0 - k1) * NB, NB, rows, kb);
    } else if (bid < na + k) {
        const int col0 = (bid - na) * NB;
        float *S = R + (int64_t)k0 * d + col0;                 // S(k, n) = R[k0+k][col0+n]
        gemm_tile<true, false>(acc, dinv, NB, S, d, kb, NB, kb, -1.f, aligned16(S, d), lds);
        store_c(acc, S, d, kb, NB);
    } else {
        for (int idx = threadIdx.x; idx < kb * kb; idx += 256) {
            const int i = idx / kb, c = idx % kb;
            R[(int64_t)(k0 + i) * d + k0 + c] = dinv[i * NB + c];
        }
    }
}

// Update of step k plus look-ahead factorization of block k+1 (work group 0).
__global__ __launch_bounds__(256) void update_kernel(float *__restrict__ R, int64_t d, int k, int nblk,
                                                     const float *__restrict__ panel,
                                                     const float *__restrict__ dinv_k,
                                                     float *__restrict__ dinv_next, int32_t *__restrict__ info) {
    __shared__ __attribute__((aligned(16))) float lds[4 * GSTAGE];
    __shared__ __attribute__((aligned(16))) float vbuf[2 * NB];
    __shared__ float dgbuf[8];
    // work group 0 -> tile (k+1, k+1); 1..k+1 -> (k+1, 0..k); the rest in order
    const int base = (k + 1) * (k + 2) / 2;
    int i, j;
    if (blockIdx.x == 0) {
        i = k + 1;
        j = k + 1;
    } else if ((int)blockIdx.x <= k + 1) {
        i = k + 1;
        j = blockIdx.x - 1;
    } else {
        tile_coords(base + blockIdx.x, i, j);
    }
    const int k0 = k * NB, kb = (int)std::min<int64_t>(NB, d - k0), k1 = k0 + kb;
    const int row0 = i * NB, col0 = j * NB;
    const int rows = (int)std::min<int64_t>(NB, d - row0);
    const int cols = (int)std::min<int64_t>(NB, d - col0);
    float *C = R + (int64_t)row0 * d + col0;
    const float *A = panel + (int64_t)(row0 - k1) * NB;       // A(m, k) = P[row0+m][k]
    f32x16 acc[4];
    if (j == k) {
        zero_acc(acc);
        // B(k, n) = Dinv[k][n]: n-contiguous
        gemm_tile<true, false>(acc, A, NB, dinv_k, NB, rows, cols, kb, 1.f, true, lds);
    } else if (j < k) {
        load_c(acc, C, d, rows, cols);
        const float *B = R + (int64_t)k0 * d + col0;           // M[k0+k][col0+n]
        gemm_tile<true, false>(acc, A, NB, B, d, rows, cols, kb, 1.f, aligned16(B, d), lds);
    } else {
        load_c(acc, C, d, rows, cols);
        const float *B = panel + (int64_t)(col0 - k1) * NB;    // B(k, n) = P[col0+n][k]
        gemm_tile<true, true>(acc, A, NB, B, NB, rows, cols, kb, -1.f, true, lds);
    }
    store_c(acc, C, d, rows, cols);
    if (blockIdx.x == 0) {
        // look-ahead: the tile just updated is the next diagonal block
        __syncthreads();
        potrf_block(C, d, rows, row0, dinv_next, info, vbuf, dgbuf);
    }
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
    float *dbuf[2] = {dinv, dinv + NB * NB};
    potrf_kernel<<<1, 256, 0, st>>>(R, d, 0, (int)std::min<int64_t>(NB, d), dbuf[0], info);
    for (int k = 0; k < nblk; ++k) {
        const int na = nblk - k - 1;
        panel_kernel<<<na + k + 1, 256, 0, st>>>(R, d, k, nblk, panel, dbuf[k & 1]);
        const int nup = nblk * (nblk + 1) / 2 - (k + 1) * (k + 2) / 2;
        if (nup > 0)
            update_kernel<<<nup, 256, 0, st>>>(R, d, k, nblk, panel, dbuf[k & 1], dbuf[(k + 1) & 1], info);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t factor_flip(float *R, int64_t d, float *ud, float *uinv, int zero_lower, hipStream_t st) {
    // flip_kernel writes only strictly-upper entries and ud; finish_diag_kernel
    // then writes the diagonal.
    flip_kernel<<<(unsigned)d, 256, 0, st>>>(R, d, ud);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    finish_diag_kernel<<<(unsigned)d, 256, 0, st>>>(R, d, ud, uinv, zero_lower);
    return hipGetLastError();
}

}  // namespace gptq
