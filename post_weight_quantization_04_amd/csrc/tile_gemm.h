// fp32-MFMA 128x128 tile product of the factorization:
// acc += alpha * A(128 x K) * B(K x 128).
//
// Operands are strided views: A(m, k) = A[m*lda + k] when A is k-contiguous,
// else A[k*lda + m]; B(k, n) = B[k*ldb + n] when B is n-contiguous, else
// B[n*ldb + k].  Both are staged through LDS in k-major layout ([k][m] and
// [k][n]) in 32-deep chunks, double-buffered through registers so the next
// chunk's global loads overlap the current chunk's MFMAs.  Interior tiles
// with aligned rows use 16-byte loads; edges fall back to guarded scalar
// loads.  Four waves own 64x64 quadrants, each as 2x2 v_mfma_f32_32x32x2_f32
// tiles computed transposed (D = B^T A^T), so that the accumulator of lane
// (h, li), register 4a+b, holds row li, column 8a+4h+b of the 32x32 sub-tile:
// every lane owns four consecutive columns of a row, and C moves with
// 16-byte accesses.
#pragma once
#include "common.h"

namespace gptq {
namespace {

constexpr int GT = 128;       // product tile edge
constexpr int GK = 32;        // k chunk staged per pass
constexpr int GLD = GT + 1;   // LDS row stride (floats): transposed scalar writes stay conflict-free
constexpr int GSTAGE = GK * GLD;

__device__ __forceinline__ void tile_coords(int t, int &I, int &J) {
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > t) --i;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    I = i;
    J = t - i * (i + 1) / 2;
}

__device__ __forceinline__ void tile_rc(int ma, int mb, int a, int b, int &r, int &c) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    r = wr * 64 + ma * 32 + li;
    c = wc * 64 + mb * 32 + 8 * a + 4 * h + b;
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
}

// C tile (rows x cols at C, row stride ldc) <-> accumulators.  Registers
// 4a .. 4a+3 are four consecutive columns of one row: 16-byte accesses when
// they are all inside the tile and C's rows are 16-byte aligned.
__device__ __forceinline__ void load_c(f32x16 (&acc)[4], const float *C, int64_t ldc, int rows, int cols) {
    const bool vec = ((reinterpret_cast<uintptr_t>(C) & 15) == 0) && (ldc % 4 == 0);
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                int r, c;
                tile_rc(ma, mb, a, 0, r, c);
                const float *src = C + (int64_t)r * ldc + c;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (r < rows) {
                    if (vec && c + 3 < cols) {
                        x = *(const f32x4 *)src;
                    } else {
                        if (c + 0 < cols) x.x = src[0];
                        if (c + 1 < cols) x.y = src[1];
                        if (c + 2 < cols) x.z = src[2];
                        if (c + 3 < cols) x.w = src[3];
                    }
                }
                acc[ma * 2 + mb][4 * a + 0] = x.x;
                acc[ma * 2 + mb][4 * a + 1] = x.y;
                acc[ma * 2 + mb][4 * a + 2] = x.z;
                acc[ma * 2 + mb][4 * a + 3] = x.w;
            }
}

__device__ __forceinline__ void store_c(const f32x16 (&acc)[4], float *C, int64_t ldc, int rows, int cols) {
    const bool vec = ((reinterpret_cast<uintptr_t>(C) & 15) == 0) && (ldc % 4 == 0);
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                int r, c;
                tile_rc(ma, mb, a, 0, r, c);
                float *dst = C + (int64_t)r * ldc + c;
                const f32x4 x = {acc[ma * 2 + mb][4 * a + 0], acc[ma * 2 + mb][4 * a + 1],
                                 acc[ma * 2 + mb][4 * a + 2], acc[ma * 2 + mb][4 * a + 3]};
                if (r < rows) {
                    if (vec && c + 3 < cols) {
                        *(f32x4 *)dst = x;
                    } else {
                        if (c + 0 < cols) dst[0] = x.x;
                        if (c + 1 < cols) dst[1] = x.y;
                        if (c + 2 < cols) dst[2] = x.z;
                        if (c + 3 < cols) dst[3] = x.w;
                    }
                }
            }
}

// C += acc on the tile: the products are summed apart from C and applied to
// it once, one rounding onto C per step instead of one per MFMA.
__device__ __forceinline__ void add_store_c(const f32x16 (&acc)[4], float *C, int64_t ldc, int rows, int cols) {
    f32x16 cur[4];
    load_c(cur, C, ldc, rows, cols);
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] += acc[i];
    store_c(cur, C, ldc, rows, cols);
}

// One operand chunk: 32 (k) x 128 (m or n) values held as 16 floats per thread.
// KCONTIG: the source is contiguous along k (element (m, k) at p[m*ld + k]).
template <bool KCONTIG>
struct Chunk {
    float v[16];

    // thread mapping: KCONTIG -> t%8 picks a 4-wide k quad, t/8 + 32q the row;
    // otherwise t%32 picks a 4-wide m quad, t/32 + 8q the k row.
    __device__ __forceinline__ void load(const float *p, int64_t ld, int kbase, int mlim, int klim, bool fast) {
        const int t = threadIdx.x;
        if (KCONTIG) {
            const int kq = (t & 7) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = (t >> 3) + 32 * q;
                const float *src = p + (int64_t)m * ld + kbase + kq;
                if (fast) {
                    const f32x4 x = *(const f32x4 *)src;
                    v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[4 * q + e] = (m < mlim && kbase + kq + e < klim) ? src[e] : 0.f;
                }
            }
        } else {
            const int mq = (t & 31) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = (t >> 5) + 8 * q;
                const float *src = p + (int64_t)(kbase + k) * ld + mq;
                if (fast) {
                    const f32x4 x = *(const f32x4 *)src;
                    v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[4 * q + e] = (kbase + k < klim && mq + e < mlim) ? src[e] : 0.f;
                }
            }
        }
    }

    // write into LDS stage s[k][m] (row stride GLD), scaled by alpha
    __device__ __forceinline__ void store(float *s, float alpha) const {
        const int t = threadIdx.x;
        if (KCONTIG) {
            const int kq = (t & 7) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = (t >> 3) + 32 * q;
#pragma unroll
                for (int e = 0; e < 4; ++e) s[(kq + e) * GLD + m] = alpha * v[4 * q + e];
            }
        } else {
            const int mq = (t & 31) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = (t >> 5) + 8 * q;
#pragma unroll
                for (int e = 0; e < 4; ++e) s[k * GLD + mq + e] = alpha * v[4 * q + e];
            }
        }
    }
};

// acc += alpha * A * B over K.  lds: 4 * GSTAGE floats (two stages of A and B).
// rows/cols bound A's m and B's n; K bounds k.  vec_ok: both bases and
// leading dimensions are 16-byte aligned (enables 16-byte loads on full chunks).
template <bool A_KCONTIG, bool B_KCONTIG>
__device__ __forceinline__ void gemm_tile(f32x16 (&acc)[4], const float *A, int64_t lda, const float *B, int64_t ldb,
                          int rows, int cols, int K, float alpha, bool vec_ok, float *lds) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    const int nch = (K + GK - 1) / GK;
    if (nch == 0) return;
    const bool full_mn = rows >= GT && cols >= GT && vec_ok;
    Chunk<A_KCONTIG> ca;
    Chunk<B_KCONTIG> cb;
    ca.load(A, lda, 0, rows, K, full_mn && GK <= K);
    cb.load(B, ldb, 0, cols, K, full_mn && GK <= K);
    ca.store(lds, alpha);
    cb.store(lds + GSTAGE, 1.f);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int buf = ch & 1;
        const bool more = ch + 1 < nch;
        if (more) {
            const int kb = (ch + 1) * GK;
            const bool fast = full_mn && kb + GK <= K;
            ca.load(A, lda, kb, rows, K, fast);
            cb.load(B, ldb, kb, cols, K, fast);
        }
        const float *as = lds + (2 * buf) * GSTAGE;
        const float *bs = lds + (2 * buf + 1) * GSTAGE;
#pragma unroll
        for (int s = 0; s < GK / 2; ++s) {
            const int row = 2 * s + h;
            float fa[2], fb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                fa[m] = as[row * GLD + wr * 64 + m * 32 + li];
                fb[m] = bs[row * GLD + wc * 64 + m * 32 + li];
            }
#pragma unroll
            for (int ma = 0; ma < 2; ++ma)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[ma * 2 + mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[mb], fa[ma], acc[ma * 2 + mb], 0, 0, 0);
        }
        if (more) {
            ca.store(lds + (2 * (buf ^ 1)) * GSTAGE, alpha);
            cb.store(lds + (2 * (buf ^ 1) + 1) * GSTAGE, 1.f);
        }
        __syncthreads();
    }
}

__device__ __forceinline__ bool aligned16(const void *p, int64_t ld) {
    return ((reinterpret_cast<uintptr_t>(p) & 15) == 0) && (ld % 4 == 0);
}

}  // namespace
}  // namespace gptq
