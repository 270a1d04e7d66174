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
//            blocks already consumed by the Cholesky.  Work groups 1..3
//            update the next diagonal tile (k+1, k+1), one 64x64 quadrant
//            each, and count their completion in info[1]; work group 0 waits
//            for that count, then factors the tile (potrf of the next step).
// Dinv alternates between two buffers by step parity because the fused
// potrf writes the next step's while the rest of the kernel reads this one.
// The tile products run on fp32 MFMA (v_mfma_f32_32x32x2_f32).
//
// Batched schedule (factor_batch(d) = T > 1, large d): every step above
// rewrites the whole trailing matrix with a K = 128 product, so for large d
// the factorization streams the matrix through HBM once per step.  Instead
// the steps go in batches [s, e) of T.  Inside a batch, step k's update
// kernel touches only what the batch's later panels read: the rows k+1..e-1
// left of column k+1 (their S) and the columns k+1..e-1 from the diagonal
// down (their A), with the look-ahead as before.  After the batch's last
// panel one far update (far_kernel, K = 128 T) applies all T steps to the
// rows below the batch, and potrf_kernel factors block e.  The panels also
// go to pt transposed for it.  Same sums, fewer passes over the matrix.
#include "common.h"
#include "dma_tile.h"
#include "tile_gemm.h"

#include <algorithm>
#include <utility>

namespace gptq {

namespace {

constexpr int NB = FACT_NB;   // 128

// ---------------------------------------------------------------------------
// Diagonal block: X = chol(A)^-1 for one 128x128 block, by the same blocked
// right-looking scheme as the whole factorization, on 32-wide sub-blocks and
// entirely in LDS (matrix F, row stride FLD).  For sub-block b (rows/cols
// [32b, 32b+32)):
//   1. one wave: X_bb = chol(A_bb)^-1 in place (potrf32);
//   2. panel  : P_i = A_ib X_bb^T for i > b, kept transposed in the unused
//               upper block (b, i);  inverse rows: M_bj = -X_bb S_bj, j < b;
//   3. update : A_ic -= P_i P_c^T (b < c <= i);  S_ij += P_i M_bj (j < b);
//               S_ib = P_i X_bb,
// with S_ij = sum_{m=j}^{i-1} L_im M_mj held in the consumed lower blocks.
// Block products are 32x32x32 on v_mfma_f32_32x32x2_f32, one per wave.
// Wave 0 runs potrf32 of sub-block b+1 during step b's trailing products.
// Rows/cols at or past kb hold the identity.
// ---------------------------------------------------------------------------
constexpr int FLD = NB + 1;   // LDS row stride of the 128x128 block (floats)
static_assert(NB * FLD <= 4 * GSTAGE, "the diagonal block reuses the tile-product staging area");

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// X = chol(A)^-1 of the 32x32 block at (s, s) of F, by one wave.  Lane c
// (both halves hold the same column) keeps column c of the working matrix in
// registers: the trailing Cholesky matrix (both triangles, so that row j can
// stand in for column j) and, left of the current column, the finished rows
// of the inverse.  Step j: pivot p = T_jj, il = 1/sqrt(p); every column
// c != j takes T_ic -= r_i (T_jc / p) for i > j with r_i = T_ji, which is the
// Cholesky update for c > j and the inverse update for c < j; row j of the
// inverse is finished as T_jc * il (c < j) and the diagonal becomes il.
// Row j (T_jc over all lanes c, pivot included) reaches every lane through
// bc (2 x 32 floats of LDS, 16-byte aligned): each lane writes its T_jc and
// reads the row back as broadcast 16-byte reads.  A wave's LDS operations
// complete in order, so no barrier is needed.  Row j+1 is updated and
// published first in step j, so the next row's reads overlap this step's
// remaining updates.
// Column j of the inverse below the diagonal is -T_ij / p followed by the
// later inverse updates, all of which are linear in that column alone (their
// multipliers come from the column itself), so lane j leaves its column as
// it is at step j and scales rows below the diagonal by -1/p once at the end.
__device__ __forceinline__ void potrf32(float *F, int s, int kb, int info_base, int32_t *__restrict__ info,
                                        float *bc) {
    // the lane's column, opaque to the optimizer: otherwise the 64 per-step
    // lane masks (c == j, c < j) are hoisted out of the caller's loop and
    // spill the scalar registers
    int c;
    asm volatile("v_and_b32 %0, 31, %1" : "=v"(c) : "v"((int)threadIdx.x));
    float T[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) T[i] = (i >= c) ? F[(s + i) * FLD + s + c] : F[(s + c) * FLD + s + i];
    bc[c] = T[0];
    float r[32];   // row j, read from bc
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const f32x4 v = *(const f32x4 *)(bc + 4 * q);
        r[4 * q + 0] = v.x;
        r[4 * q + 1] = v.y;
        r[4 * q + 2] = v.z;
        r[4 * q + 3] = v.w;
    }
    int bad = 0;       // first non-positive (or NaN) pivot of this block, 1-based
    float ilc = 0.f;   // this lane's own 1/l_cc
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        __builtin_amdgcn_sched_barrier(0);
        const float p = r[j];
        bad = (bad == 0 && !(p > 0.f) && s + j < kb) ? j + 1 : bad;
        // 1/l_jj from the hardware reciprocal square root (about 1 ulp)
        const float il = __builtin_amdgcn_rsqf(p);
        const float il2 = il * il;
        const float tj = T[j];
        const bool me = (c == j);
        const float w = me ? 0.f : tj * il2;
        ilc = me ? il : ilc;
        float rn[32];   // row j+1
        if (j + 1 < 32) {
            T[j + 1] = fmaf(-r[j + 1], w, T[j + 1]);
            float *nrow = bc + 32 * ((j + 1) & 1);
            nrow[c] = T[j + 1];
#pragma unroll
            for (int q = (j + 1) >> 2; q < 8; ++q) {
                const f32x4 v = *(const f32x4 *)(nrow + 4 * q);
                rn[4 * q + 0] = v.x;
                rn[4 * q + 1] = v.y;
                rn[4 * q + 2] = v.z;
                rn[4 * q + 3] = v.w;
            }
        }
        // the next row's reads are in flight during this step's updates
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = j + 2; i < 32; ++i) T[i] = fmaf(-r[i], w, T[i]);
        T[j] = me ? il : ((c < j) ? tj * il : tj);
        if (j + 1 < 32) {
#pragma unroll
            for (int i = j + 1; i < 32; ++i) r[i] = rn[i];
        }
    }
    if (threadIdx.x == 0 && bad != 0 && info[0] == 0) info[0] = info_base + s + bad;
    const float sc = -ilc * ilc;
    if (threadIdx.x < 32) {
#pragma unroll
        for (int i = 0; i < 32; ++i) F[(s + i) * FLD + s + c] = (i > c) ? T[i] * sc : ((i == c) ? T[i] : 0.f);
    }
}

// acc (+)= sum_k A(m, k) B(k, n) over k < 32 for one 32x32 block; A(m, k) =
// F[a0 + m*am + k*ak], B(k, n) = F[b0 + k*bk + n*bn].  Accumulator layout:
// lane (h, li), register 4a+b <-> row 8a+4h+b, column li.
__device__ __forceinline__ void blk_mfma(f32x16 &acc, const float *F, int a0, int am, int ak, int b0, int bk, int bn) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, li = lane & 31;
#pragma unroll
    for (int k = 0; k < 32; k += 2) {
        const float av = F[a0 + li * am + (k + h) * ak];
        const float bv = F[b0 + (k + h) * bk + li * bn];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ void blk_load(f32x16 &acc, const float *F, int r0, int c0) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, li = lane & 31;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[4 * a + b] = F[(r0 + 8 * a + 4 * h + b) * FLD + c0 + li];
}

// C = scale * acc, stored as block (r0, c0); transposed: element (m, n) goes to (r0 + n, c0 + m)
__device__ __forceinline__ void blk_store(const f32x16 &acc, float *F, int r0, int c0, float scale, bool transposed) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, li = lane & 31;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = 8 * a + 4 * h + b;
            if (transposed)
                F[(r0 + li) * FLD + c0 + m] = scale * acc[4 * a + b];
            else
                F[(r0 + m) * FLD + c0 + li] = scale * acc[4 * a + b];
        }
}

// F = the kb x kb block at src (row stride ld; lower triangle read), identity
// past kb.  Thread t takes 4-column group t % 32 of rows t / 32 + 8q, all of
// its loads issued before any store.
__device__ __forceinline__ void potrf_block_load(const float *__restrict__ src, int64_t ld, int kb, float *F) {
    const int t = threadIdx.x, c4 = 4 * (t & 31);
    const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15) == 0) && (ld % 4 == 0) && (kb % 4 == 0);
    f32x4 v[16];
    if (vec && kb == NB) {
        // full block: every load unguarded (the upper triangle is read and
        // dropped below), so that all sixteen are in flight together
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = *(const f32x4 *)(src + (int64_t)((t >> 5) + 8 * q) * ld + c4);
    } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = (t >> 5) + 8 * q;
            const float *p = src + (int64_t)i * ld + c4;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (i < kb && c4 <= i) {
                if (vec) {
                    x = *(const f32x4 *)p;
                } else {
                    if (c4 + 0 < kb) x.x = p[0];
                    if (c4 + 1 < kb) x.y = p[1];
                    if (c4 + 2 < kb) x.z = p[2];
                    if (c4 + 3 < kb) x.w = p[3];
                }
            }
            v[q] = x;
        }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int i = (t >> 5) + 8 * q;
        const float e[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = c4 + u;
            F[i * FLD + c] = (i < kb && c < kb && c <= i) ? e[u] : (i == c ? 1.f : 0.f);
        }
    }
}

// dinv = the lower triangle of F restricted to kb x kb, zero elsewhere.
// Thread t takes 4-column group t % 32 of rows t / 32 + 8q: 16-byte stores.
__device__ __forceinline__ void potrf_block_store(const float *F, int kb, float *__restrict__ dinv) {
    const int t = threadIdx.x, c4 = 4 * (t & 31);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int i = (t >> 5) + 8 * q;
        float e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            // kept iff c <= i < kb (then c < kb too), as an all-ones mask:
            // plain integer arithmetic rather than 64 live lane masks
            const int c = c4 + u;
            const int keep = ((c - i - 1) & (i - kb)) >> 31;
            e[u] = __builtin_bit_cast(float, __builtin_bit_cast(int, F[i * FLD + c]) & keep);
        }
        *(f32x4 *)(dinv + i * NB + c4) = f32x4{e[0], e[1], e[2], e[3]};
    }
}

// F (NB x FLD floats in LDS, identity past kb) := chol(F)^-1 in its lower
// triangle.  256 threads; F must be complete and visible (after a barrier).
// bc: 64 floats of LDS, 16-byte aligned (row broadcasts of the 32x32 steps).
__device__ __forceinline__ void potrf_block_lds(float *F, int kb, int info_base, int32_t *__restrict__ info,
                                                float *bc) {
    const int wave = threadIdx.x >> 6;
    constexpr int SB = 32, NSB = NB / SB;
    // Sub-block b + 1's own chain needs only its diagonal block's update from
    // step b, so wave 0 takes that one trailing product and goes straight on
    // to potrf32 of b + 1 while waves 1-3 take the rest of step b's trailing
    // products (the chain of one wave is most of the routine's time).
    if (wave == 0) potrf32(F, 0, kb, info_base, info, bc);
    __syncthreads();
    for (int b = 0; b < NSB; ++b) {
        const int s = SB * b;
        // panel blocks i = b+1.. (transposed into block (b, i)) and inverse rows j < b
        {
            const int ntask = (NSB - 1 - b) + b;
            for (int t = wave; t < ntask; t += 4) {
                f32x16 acc = f32x16{};
                if (t < NSB - 1 - b) {
                    const int i = b + 1 + t;
                    // P_i(m, n) = sum_k A_ib(m, k) X_bb(n, k)
                    blk_mfma(acc, F, (SB * i) * FLD + s, FLD, 1, s * FLD + s, 1, FLD);
                    blk_store(acc, F, s, SB * i, 1.f, true);
                } else {
                    const int j = t - (NSB - 1 - b);
                    // M_bj(m, n) = -sum_k X_bb(m, k) S_bj(k, n), in place
                    blk_mfma(acc, F, s * FLD + s, FLD, 1, s * FLD + SB * j, FLD, 1);
                    blk_store(acc, F, s, SB * j, -1.f, false);
                }
            }
        }
        __syncthreads();
        // trailing Cholesky blocks (i, c), b < c <= i, then inverse sums (i, j),
        // j <= b; task 0 is the next diagonal block (b+1, b+1)
        const int nr = NSB - 1 - b;
        const int nchol = nr * (nr + 1) / 2;
        const int ntask = nchol + nr * (b + 1);
        auto task = [&](int t) {
            f32x16 acc;
            if (t < nchol) {
                int ii = 0;
                while ((ii + 1) * (ii + 2) / 2 <= t) ++ii;
                const int i = b + 1 + ii, cc = b + 1 + (t - ii * (ii + 1) / 2);
                blk_load(acc, F, SB * i, SB * cc);
                // A_ic -= P_i P_c^T with P_x(m, k) at F[(s + k) * FLD + 32x + m]
                f32x16 prod = f32x16{};
                blk_mfma(prod, F, s * FLD + SB * i, 1, FLD, s * FLD + SB * cc, FLD, 1);
                acc -= prod;
                blk_store(acc, F, SB * i, SB * cc, 1.f, false);
            } else {
                const int u = t - nchol;
                const int i = b + 1 + u / (b + 1), j = u % (b + 1);
                if (j < b) {
                    blk_load(acc, F, SB * i, SB * j);
                    // S_ij += P_i M_bj
                    blk_mfma(acc, F, s * FLD + SB * i, 1, FLD, s * FLD + SB * j, FLD, 1);
                } else {
                    acc = f32x16{};
                    // S_ib = P_i X_bb
                    blk_mfma(acc, F, s * FLD + SB * i, 1, FLD, s * FLD + s, FLD, 1);
                }
                blk_store(acc, F, SB * i, SB * j, 1.f, false);
            }
        };
        if (nr > 0) {
            if (wave == 0) {
                // the block is this wave's own: potrf32 reads it after this
                // wave's stores (a wave's LDS operations complete in order)
                task(0);
                potrf32(F, s + SB, kb, info_base, info, bc);
            } else {
                for (int t = wave; t < ntask; t += 3) task(t);
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256, 2) void potrf_kernel(const float *__restrict__ R, int64_t d, int k0, int kb,
                                                    float *__restrict__ dinv, int32_t *__restrict__ info) {
    __shared__ __attribute__((aligned(16))) float F[NB * FLD];
    __shared__ __attribute__((aligned(16))) float bc[64];
    potrf_block_load(R + (int64_t)k0 * d + k0, d, kb, F);
    __syncthreads();
    potrf_block_lds(F, kb, k0, info, bc);
    potrf_block_store(F, kb, dinv);
}

// Narrow operand chunk for the strip products: 32 (k) x 32 (x) values, four
// per thread.  KCONTIG: element (x, k) at p[x*ld + k] (thread t: x = t/8,
// k quad t%8); otherwise at p[k*ld + x] (x quad t%8, k = t/8).  Staged in
// LDS as [k][x] with row stride 33.
constexpr int SLD = 33;
template <bool KCONTIG>
struct NChunk {
    float v[4];
    __device__ __forceinline__ void load(const float *p, int64_t ld, int kbase, int xlim, int klim, bool fast) {
        const int t = threadIdx.x;
        if (KCONTIG) {
            const int x = t >> 3, kq = (t & 7) * 4;
            const float *src = p + (int64_t)x * ld + kbase + kq;
            if (fast) {
                const f32x4 q = *(const f32x4 *)src;
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (x < xlim && kbase + kq + e < klim) ? src[e] : 0.f;
            }
        } else {
            const int xq = (t & 7) * 4, k = t >> 3;
            const float *src = p + (int64_t)(kbase + k) * ld + xq;
            if (fast) {
                const f32x4 q = *(const f32x4 *)src;
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (kbase + k < klim && xq + e < xlim) ? src[e] : 0.f;
            }
        }
    }
    __device__ __forceinline__ void store(float *st, float alpha) const {
        const int t = threadIdx.x;
        if (KCONTIG) {
            const int x = t >> 3, kq = (t & 7) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[(kq + e) * SLD + x] = alpha * v[e];
        } else {
            const int xq = (t & 7) * 4, k = t >> 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[k * SLD + xq + e] = alpha * v[e];
        }
    }
};

// Strip products for the panel step: a 128x128 tile product split four ways
// so that four groups share it.  ROWS: out is 32 rows x 128 cols (A narrow,
// B wide; wave w owns columns 32w..32w+31); else 128 rows x 32 cols (A wide,
// B narrow; wave w owns rows 32w..).  acc += alpha A B over K, computed
// transposed as in the tile product (lane (h, li), register 4a+b: row li /
// 32w+li, column 8a+4h+b of the wave's 32x32 block).  lds: 2 * (32*GLD +
// 32*SLD) floats.
template <bool ROWS, bool A_KCONTIG, bool B_KCONTIG>
__device__ __forceinline__ void gemm_strip(f32x16 &acc, const float *A, int64_t lda, const float *B, int64_t ldb,
                                           int rows, int cols, int K, float alpha, bool vec_ok, float *lds) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, li = lane & 31;
    constexpr int WST = GK * GLD, NST = GK * SLD;
    float *wide = lds;                  // [2][WST]
    float *narrow = lds + 2 * WST;      // [2][NST]
    const int nch = (K + GK - 1) / GK;
    if (nch == 0) return;
    const bool full = (ROWS ? (rows >= 32 && cols >= GT) : (rows >= GT && cols >= 32)) && vec_ok;
    Chunk<ROWS ? B_KCONTIG : A_KCONTIG> cw;
    NChunk<ROWS ? A_KCONTIG : B_KCONTIG> cn;
    auto load = [&](int kb, bool fast) {
        if (ROWS) {
            cn.load(A, lda, kb, rows, K, fast);
            cw.load(B, ldb, kb, cols, K, fast);
        } else {
            cw.load(A, lda, kb, rows, K, fast);
            cn.load(B, ldb, kb, cols, K, fast);
        }
    };
    auto store = [&](int buf) {
        // alpha goes with A
        cw.store(wide + buf * WST, ROWS ? 1.f : alpha);
        cn.store(narrow + buf * NST, ROWS ? alpha : 1.f);
    };
    if (full && K == NB) {
        // full strip, full K: all four chunks' loads go out unguarded at the
        // start (one memory latency), then pass through the two LDS buffers
        constexpr int MAXC = NB / GK;
        Chunk<ROWS ? B_KCONTIG : A_KCONTIG> xw[MAXC];
        NChunk<ROWS ? A_KCONTIG : B_KCONTIG> xn[MAXC];
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            if (ROWS) {
                xn[c].load(A, lda, c * GK, rows, K, true);
                xw[c].load(B, ldb, c * GK, cols, K, true);
            } else {
                xw[c].load(A, lda, c * GK, rows, K, true);
                xn[c].load(B, ldb, c * GK, cols, K, true);
            }
        }
        xw[0].store(wide, ROWS ? 1.f : alpha);
        xn[0].store(narrow, ROWS ? alpha : 1.f);
        __syncthreads();
#pragma unroll
        for (int ch = 0; ch < MAXC; ++ch) {
            const int buf = ch & 1;
            const float *ws = wide + buf * WST;
            const float *ns = narrow + buf * NST;
#pragma unroll
            for (int s = 0; s < GK / 2; ++s) {
                const int row = 2 * s + h;
                const float fw = ws[row * GLD + wave * 32 + li];
                const float fn = ns[row * SLD + li];
                if (ROWS) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fw, fn, acc, 0, 0, 0);
                else acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fn, fw, acc, 0, 0, 0);
            }
            if (ch + 1 < MAXC) {
                xw[ch + 1].store(wide + (buf ^ 1) * WST, ROWS ? 1.f : alpha);
                xn[ch + 1].store(narrow + (buf ^ 1) * NST, ROWS ? alpha : 1.f);
            }
            __syncthreads();
        }
        return;
    }
    load(0, full && GK <= K);
    store(0);
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int buf = ch & 1;
        const bool more = ch + 1 < nch;
        if (more) load((ch + 1) * GK, full && (ch + 2) * GK <= K);
        const float *ws = wide + buf * WST;
        const float *ns = narrow + buf * NST;
#pragma unroll
        for (int s = 0; s < GK / 2; ++s) {
            const int row = 2 * s + h;
            const float fw = ws[row * GLD + wave * 32 + li];
            const float fn = ns[row * SLD + li];
            // D = B^T A^T: the first operand indexes the output columns
            if (ROWS) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fw, fn, acc, 0, 0, 0);
            else acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fn, fw, acc, 0, 0, 0);
        }
        if (more) store(buf ^ 1);
        __syncthreads();
    }
}

// store of a strip product's accumulator (rows x cols at C, row stride ldc)
template <bool ROWS>
__device__ __forceinline__ void store_strip(const f32x16 &acc, float *C, int64_t ldc, int rows, int cols) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, li = lane & 31;
    const bool vec = ((reinterpret_cast<uintptr_t>(C) & 15) == 0) && (ldc % 4 == 0);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int r = ROWS ? li : wave * 32 + li;
        const int c = (ROWS ? wave * 32 : 0) + 8 * a + 4 * h;
        float *dst = C + (int64_t)r * ldc + c;
        const f32x4 x = {acc[4 * a + 0], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
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

// Panel step, four groups per 128x128 tile:
// part A (row blocks below k, 32-row strips): P_i = A_ik Dinv^T -> panel
// part B (column blocks left of k, 32-column strips): M_kj = -Dinv S_kj, in
//        place (each group reads and writes only its own columns of S)
// last group: M_kk = Dinv
// pt (batched schedule only, else null): part A also writes P transposed,
// pt[pt_k + c][row] = P[row][c], for the batch's far update.
__global__ __launch_bounds__(256) void panel_kernel(float *__restrict__ R, int64_t d, int k, int nblk,
                                                    float *__restrict__ panel, const float *__restrict__ dinv,
                                                    float *__restrict__ pt, int pt_k) {
    __shared__ __attribute__((aligned(16))) float lds[2 * GK * (GLD + SLD)];
    const int k0 = k * NB, kb = (int)std::min<int64_t>(NB, d - k0), k1 = k0 + kb;
    const int na = nblk - k - 1;
    const int bid = blockIdx.x;
    f32x16 acc = f32x16{};
    if (bid < 4 * na) {
        const int row0 = (k + 1 + bid / 4) * NB + 32 * (bid % 4);
        const int rows = (int)std::min<int64_t>(32, d - row0);
        if (rows <= 0) return;                                   // whole group: nothing to do
        const float *A = R + (int64_t)row0 * d + k0;            // A(m, k) = R[row0+m][k0+k]
        // B(k, n) = Dinv[n][k]: k-contiguous rows of Dinv
        gemm_strip<true, true, true>(acc, A, d, dinv, NB, rows, kb, kb, 1.f, aligned16(A, d), lds);
        store_strip<true>(acc, panel + (int64_t)(row0 - k1) * NB, NB, rows, kb);
        if (pt) {
            // lane (h, li) holds row li, columns 32 w + 8a + 4h + b: each
            // store puts 32 consecutive rows of one transposed row
            const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, li = lane & 31;
            if (li < rows) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int c = wave * 32 + 8 * a + 4 * h + b;
                        if (c < kb) pt[(int64_t)(pt_k + c) * d + row0 + li] = acc[4 * a + b];
                    }
            }
        }
    } else if (bid < 4 * na + 4 * k) {
        const int col0 = ((bid - 4 * na) / 4) * NB + 32 * ((bid - 4 * na) % 4);
        float *S = R + (int64_t)k0 * d + col0;                   // S(k, n) = R[k0+k][col0+n]
        gemm_strip<false, true, false>(acc, dinv, NB, S, d, kb, 32, kb, -1.f, aligned16(S, d), lds);
        store_strip<false>(acc, S, d, kb, 32);
    } else {
        // M_kk = Dinv (kb x kb, upper part zero): thread t copies 4-column
        // group t % 32 of rows t / 32 + 8q, all loads before any store
        const int t = threadIdx.x, c4 = 4 * (t & 31);
        const bool vec = (d % 4 == 0);
        f32x4 v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = (t >> 5) + 8 * q;
            v[q] = (i < kb) ? *(const f32x4 *)(dinv + i * NB + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int i = (t >> 5) + 8 * q;
            if (i >= kb) continue;
            float *dst = R + (int64_t)(k0 + i) * d + k0 + c4;
            if (vec && c4 + 3 < kb) {
                *(f32x4 *)dst = v[q];
            } else {
                if (c4 + 0 < kb) dst[0] = v[q].x;
                if (c4 + 1 < kb) dst[1] = v[q].y;
                if (c4 + 2 < kb) dst[2] = v[q].z;
                if (c4 + 3 < kb) dst[3] = v[q].w;
            }
        }
    }
}

// Step counter shared by the diagonal-update helpers and the look-ahead
// factorization (info[1], zero at the start of each factorization): after
// step k's update kernel it reads 3 (k + 1).  The waiting thread polls with
// device-scope atomic loads and a short sleep, at most STEP_SPIN_LIMIT times;
// on time-out it records FACTOR_SYNC_TIMEOUT in info[0] (unless a pivot error
// is already there) and goes on, so every group finishes.  The helpers are
// dispatched right after the waiting group and wait for nothing.
constexpr int STEP_SPIN_LIMIT = 1 << 20;

__device__ __forceinline__ void wait_count(int32_t *cnt, int target, int32_t *info) {
    if (threadIdx.x == 0) {
        int v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int it = 0; v < target && it < STEP_SPIN_LIMIT; ++it) {
            __builtin_amdgcn_s_sleep(2);
            v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (v < target) atomicCAS(info, 0, FACTOR_SYNC_TIMEOUT);
        // what the helpers wrote before their release is visible after this
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

__device__ __forceinline__ void signal_count(int32_t *cnt) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // this wave's stores
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Helper q of step k: quadrant (qa, qb) = (0,0), (1,0), (1,1) of the next
// diagonal tile (k+1, k+1) of R takes C -= P_a P_b^T in place, with P the
// panel rows of block k+1 (rows x NB, k-contiguous, at the panel's start).
// Wave w takes the 32x32 sub-block (w/2, w%2) of the quadrant (none above
// the diagonal of a diagonal quadrant) on fp32 MFMA, computed transposed
// (lane (h, li), register 4a+b: row li, column 8a+4h+b).  The products run
// over k in any order as long as both operands agree, so lane half h
// supplies k = 64h + s at step s.  The two 64-row blocks of P (one for a
// diagonal quadrant) go to LDS first with coalesced 16-byte loads (each
// 32-lane half reads 512 contiguous bytes of one row; loaded per lane along
// its own row, every load instruction touched 64 cache lines and the 32 of
// them took 3-6 k cycles to issue), rows padded to 132 floats so that the
// 16-byte fragment reads, one row per lane, hit distinct banks; then the 64
// products run back to back.  Rows past the block repeat the last row and
// only feed entries that are not stored.
constexpr int QLD = NB + 4;                                // LDS row stride of the staged P rows
constexpr int QSTAGE = 2 * 64 * QLD;                       // both 64-row blocks (floats)
__device__ __forceinline__ void diag_quadrant(float *__restrict__ R, int64_t d, int n0, int rows, int q,
                                              const float *__restrict__ P, float *lds) {
    const int qa = (q >= 1) ? 1 : 0, qb = (q == 2) ? 1 : 0;
    const int ra = 64 * qa, rb = 64 * qb;
    if (ra >= rows) return;   // the block has no such quadrant (uniform over the group)
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, h = lane >> 5, li = lane & 31;
    const int sa = wave >> 1, sb = wave & 1;
    const bool active = !(qa == qb && sa < sb);            // above the diagonal: not needed
    const int r = ra + 32 * sa + li;                       // this lane's row of the tile (P_a row)
    const int cb = rb + 32 * sb;                           // the sub-block's first column
    float *Crow = R + (int64_t)(n0 + r) * d + n0;
    // acc = -C, then acc += P_b P_a^T (transposed), C = -acc.  The C loads go
    // out first (a full tile without guards), then the P rows, so that both
    // sets are in flight together.
    f32x4 cv[4];
    if (rows == NB && active) {
#pragma unroll
        for (int a = 0; a < 4; ++a) cv[a] = *(const f32x4 *)(Crow + cb + 8 * a + 4 * h);
    } else {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int c = cb + 8 * a + 4 * h;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (active && r < rows) {
                if (c + 3 < rows) {
                    x = *(const f32x4 *)(Crow + c);
                } else {
                    if (c + 0 < rows) x.x = Crow[c + 0];
                    if (c + 1 < rows) x.y = Crow[c + 1];
                    if (c + 2 < rows) x.z = Crow[c + 2];
                }
            }
            cv[a] = x;
        }
    }
    // stage P rows ra.. (block 0) and rb.. (block 1, off-diagonal quadrant
    // only): piece t + 256 i is row ((t + 256 i) / 32) % 64 of block
    // (t + 256 i) / 2048, 16-byte column group t % 32
    const int nblkrows = (qa == qb) ? 1 : 2;
    {
        f32x4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int piece = tid + 256 * i;
            const int blk = piece >> 11, row = (piece >> 5) & 63, c4 = 4 * (piece & 31);
            const int src_row = min((blk ? rb : ra) + row, rows - 1);
            v[i] = (blk < nblkrows) ? *(const f32x4 *)(P + (int64_t)src_row * NB + c4) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int piece = tid + 256 * i;
            const int blk = piece >> 11, row = (piece >> 5) & 63, c4 = 4 * (piece & 31);
            if (blk < nblkrows) *(f32x4 *)(lds + (blk * 64 + row) * QLD + c4) = v[i];
        }
    }
    __syncthreads();
    if (!active) return;
    // A row 32 sa + li of block 0; B row 32 sb + li of block 1 (block 0 for
    // a diagonal quadrant, whose two blocks are the same rows)
    const float *pa = lds + (32 * sa + li) * QLD + 64 * h;
    const float *pb = lds + ((qa == qb ? 0 : 64) + 32 * sb + li) * QLD + 64 * h;
    f32x4 av[16], bv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        av[j] = *(const f32x4 *)(pa + 4 * j);
        bv[j] = *(const f32x4 *)(pb + 4 * j);
    }
    // every read goes out before the first product
    __builtin_amdgcn_sched_barrier(0);
    // the 128-term sums apart from C, applied to it once
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < 64; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[s >> 2][s & 3], av[s >> 2][s & 3], acc, 0, 0, 0);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int c = cb + 8 * a + 4 * h;
        const f32x4 x = {cv[a].x - acc[4 * a + 0], cv[a].y - acc[4 * a + 1], cv[a].z - acc[4 * a + 2],
                         cv[a].w - acc[4 * a + 3]};
        if (r < rows) {
            if (c + 3 < rows) {
                *(f32x4 *)(Crow + c) = x;
            } else {
                if (c + 0 < rows) Crow[c + 0] = x.x;
                if (c + 1 < rows) Crow[c + 1] = x.y;
                if (c + 2 < rows) Crow[c + 2] = x.z;
            }
        }
    }
}

// Update of step k plus the look-ahead factorization of block k+1.
//   group 0     : waits for the three helpers, then loads the next diagonal
//                 tile (k+1, k+1) from R and factors it (look-ahead), writing
//                 Dinv_{k+1} to dinv_next.
//   groups 1..3 : the next diagonal tile's update, one 64x64 quadrant each.
//   groups 4..  : every other tile that step k updates now.  Unbatched
//                 (e == nblk): all tiles in rows > k, (k+1, 0..k) first,
//                 then the rows below in order.  Inside a batch of steps
//                 ending at block e < nblk: the rows k+1 .. e-1 left of
//                 column k+1 (row by row), then the columns k+1 .. e-1 from
//                 their diagonal down (column by column); the rest of the
//                 step's update waits for the batch's far update.
// target: the helpers' count that group 0 waits for (three per launch).
__global__ __launch_bounds__(256, 2) void update_kernel(float *__restrict__ R, int64_t d, int k, int nblk, int e,
                                                     const float *__restrict__ panel,
                                                     const float *__restrict__ dinv_k,
                                                     float *__restrict__ dinv_next, int32_t *__restrict__ info,
                                                     int target) {
    __shared__ __attribute__((aligned(16))) float lds[std::max(4 * GSTAGE, QSTAGE)];
    __shared__ __attribute__((aligned(16))) float bc[64];
    const int k0 = k * NB, kb = (int)std::min<int64_t>(NB, d - k0), k1 = k0 + kb;
    const int b = blockIdx.x;
    if (b < 4) {
        const int n0 = (k + 1) * NB;
        const int rows = (int)std::min<int64_t>(NB, d - n0);
        if (b > 0) {
            diag_quadrant(R, d, n0, rows, b - 1, panel + (int64_t)(n0 - k1) * NB, lds);
            signal_count(info + 1);
            return;
        }
        wait_count(info + 1, target, info);
        float *F = lds;
        potrf_block_load(R + (int64_t)n0 * d + n0, d, rows, F);
        __syncthreads();
        potrf_block_lds(F, rows, n0, info, bc);
        potrf_block_store(F, rows, dinv_next);
        return;
    }
    int i, j;
    if (e >= nblk) {
        // (k+1, 0..k), then the rows below in order
        const int bb = b - 3;
        if (bb <= k + 1) {
            i = k + 1;
            j = bb - 1;
        } else {
            tile_coords((k + 1) * (k + 2) / 2 + bb, i, j);
        }
    } else {
        int t = b - 4;
        const int nrow = (e - k - 1) * (k + 1);
        if (t < nrow) {
            i = k + 1 + t / (k + 1);
            j = t % (k + 1);
        } else {
            // column c holds rows c .. nblk-1, without (k+1, k+1)
            t -= nrow;
            int c = k + 1, n = nblk - k - 2;
            while (t >= n && c < e) {
                t -= n;
                ++c;
                n = nblk - c;
            }
            if (c >= e) return;   // past the last tile (the grid is sized exactly)
            j = c;
            i = (c == k + 1) ? c + 1 + t : c + t;
        }
    }
    const int row0 = i * NB, col0 = j * NB;
    const int rows = (int)std::min<int64_t>(NB, d - row0);
    const int cols = (int)std::min<int64_t>(NB, d - col0);
    float *C = R + (int64_t)row0 * d + col0;
    const float *A = panel + (int64_t)(row0 - k1) * NB;       // A(m, k) = P[row0+m][k]
    f32x16 acc[4];
    zero_acc(acc);
    if (j == k) {
        // B(k, n) = Dinv[k][n]: n-contiguous
        gemm_tile<true, false>(acc, A, NB, dinv_k, NB, rows, cols, kb, 1.f, true, lds);
        store_c(acc, C, d, rows, cols);
        return;
    }
    // the products summed apart from C, added to it once
    if (j < k) {
        const float *B = R + (int64_t)k0 * d + col0;           // M[k0+k][col0+n]
        gemm_tile<true, false>(acc, A, NB, B, d, rows, cols, kb, 1.f, aligned16(B, d), lds);
    } else {
        const float *B = panel + (int64_t)(col0 - k1) * NB;    // B(k, n) = P[col0+n][k]
        gemm_tile<true, true>(acc, A, NB, B, NB, rows, cols, kb, -1.f, true, lds);
    }
    add_store_c(acc, C, d, rows, cols);
}

// Far update of the batch of steps s .. e-1 (e < nblk), one 128 x 128 tile
// (i, j) of the rows below the batch per work group, i >= e, j <= i, in row
// order.  pt holds the batch's panels transposed ([(m - s) * 128 + c][row]
// = L[row][128 m + c]), so with K = 128 (e - s):
//   j >= e      : A_ij -= sum_m P_i^(m) P_j^(m)^T        (Cholesky part)
//   s <= j < e  : S_ij  = sum_{m >= j} P_i^(m) M_mj      (M_jj = Dinv_j)
//   j <  s      : S_ij += sum_m P_i^(m) M_mj
// with the batch's rows of M read from R (final after its panels; the
// diagonal blocks carry zeros above the diagonal).  The sums over the batch
// equal the steps' own updates applied one after another, so the result is
// the same factorization up to rounding order.  Two groups per compute unit
// (a 64 KB ring each: four stages of 16 k-rows), so that one group's tile
// start (its C loads and first chunks) overlaps the other's products: at
// d = 28672 this took the factorization from 157 to 137 ms against one group
// per unit with four stages of 32 k-rows.
constexpr int FAR_NST = 4, FAR_KC = 16;
__global__ __launch_bounds__(256, 2) void far_kernel(float *__restrict__ R, int64_t d, int s, int e,
                                                  const float *__restrict__ pt) {
    __shared__ __attribute__((aligned(16))) float lds[DmaShape<128, FAR_NST, FAR_KC>::LDS_FLOATS];
    int i, j;
    tile_coords(e * (e + 1) / 2 + (int)blockIdx.x, i, j);
    const int64_t row0 = (int64_t)i * NB, col0 = (int64_t)j * NB;
    const int rows = (int)std::min<int64_t>(NB, d - row0);
    const int cols = (int)std::min<int64_t>(NB, d - col0);
    if (rows <= 0) return;
    const int kt = (e - s) * NB;   // every block of a batch that has a far update is full
    int koff = 0, mode = DMA_ADD;
    const float *B;
    if (j >= e) {
        mode = DMA_SUB;
        B = pt + col0;
    } else {
        if (j >= s) {
            koff = (j - s) * NB;
            mode = DMA_SET;
        }
        B = R + (int64_t)(s * NB + koff) * d + col0;
    }
    const int K = kt - koff;
    const float *A = pt + (int64_t)koff * d + row0;
    dma_tile_product<128, FAR_NST, FAR_KC>(R + row0 * d + col0, d, rows, cols, A, d, ((int64_t)K * d - row0) * 4, B + 0, d,
                          ((int64_t)K * d - col0) * 4, K, mode, lds);
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

int factor_batch(int64_t d) {
    const int64_t nblk = cdiv(d, NB);
    // the far update moves 16-byte rows with 32-bit offsets
    if (d % 4 != 0 || (int64_t)FACT_BATCH * NB * d * 4 + (int64_t)DK * DNST * d * 4 >= ((int64_t)1 << 31)) return 1;
    return nblk >= FACT_BATCH_MIN_BLOCKS ? FACT_BATCH : 1;
}

hipError_t factor_launch(float *R, int64_t d, float *panel, float *pt, float *dinv, int32_t *info, hipStream_t st) {
    const int nblk = (int)cdiv(d, NB);
    const int T = factor_batch(d);
    float *dbuf[2] = {dinv, dinv + NB * NB};
    potrf_kernel<<<1, 256, 0, st>>>(R, d, 0, (int)std::min<int64_t>(NB, d), dbuf[0], info);
    int target = 0;   // helpers' completions so far
    for (int s = 0, e = 0; s < nblk; s = e) {
        // batch [s, e); unbatched, one batch of all steps and no far update
        e = (T > 1) ? std::min(nblk, s + T) : nblk;
        const bool far = e < nblk;
        for (int k = s; k < e; ++k) {
            const int na = nblk - k - 1;
            panel_kernel<<<4 * (na + k) + 1, 256, 0, st>>>(R, d, k, nblk, panel, dbuf[k & 1], far ? pt : nullptr,
                                                           (k - s) * NB);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
            if (far && k == e - 1) break;   // the far update takes the rest of this step
            // tiles updated now, the next diagonal one included: that one goes
            // to the three helpers, and group 0 is the look-ahead
            int nup;
            if (!far) {
                nup = nblk * (nblk + 1) / 2 - (k + 1) * (k + 2) / 2;
            } else {
                nup = (e - k - 1) * (k + 1);
                for (int c = k + 1; c < e; ++c) nup += nblk - c;
            }
            if (nup > 0) {
                target += 3;
                update_kernel<<<nup + 3, 256, 0, st>>>(R, d, k, nblk, e, panel, dbuf[k & 1], dbuf[(k + 1) & 1], info,
                                                       target);
                err = hipGetLastError();
                if (err != hipSuccess) return err;
            }
        }
        if (far) {
            const int ntile = nblk * (nblk + 1) / 2 - e * (e + 1) / 2;
            far_kernel<<<ntile, 256, 0, st>>>(R, d, s, e, pt);
            potrf_kernel<<<1, 256, 0, st>>>(R, d, e * NB, (int)std::min<int64_t>(NB, d - (int64_t)e * NB), dbuf[e & 1],
                                            info);
            hipError_t err = hipGetLastError();
            if (err != hipSuccess) return err;
        }
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
