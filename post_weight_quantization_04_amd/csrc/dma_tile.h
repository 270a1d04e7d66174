// fp32-MFMA tile product with both operands streamed from global memory
// straight into LDS, shared by the lazy trailing update and the
// factorization's batched far update:
//
//   C(m, n) <- C(m, n) - P(m, n)   (DMA_SUB)
//   C(m, n) <- C(m, n) + P(m, n)   (DMA_ADD)
//   C(m, n) <- P(m, n)             (DMA_SET)
//   P(m, n) = sum_{k < K} A[k * lda + m] B[k * ldb + n]
//
// for one 128 x TN tile of C (row stride ldc): both operands are k-major,
// contiguous along the tile's rows (A) and columns (B).  Chunks of KC k-rows
// move by 16-byte buffer loads through an NST-stage LDS ring, NST - 1 chunks
// in flight while one is multiplied (by default 32 k-rows and four stages,
// 128 KB: one work group per compute unit; both users take 16 k-rows, 64 KB,
// two groups per unit).  The buffer resources end where the caller says the
// operand ends (normally at k-row K), so the ragged last chunk reads zeros
// without a branch; rows and columns past the tile's edge only feed entries
// that are not stored.
// Requires lda, ldb, ldc and the operand and tile origins to be 16-byte
// aligned, and K * max(lda, ldb) * 4 + 4 chunks < 2^31 (32-bit offsets).
#pragma once
#include "common.h"

#include <algorithm>

namespace gptq {
namespace {

constexpr int DT = 128;               // tile rows
constexpr int DK = 32;                // default k-rows per chunk
constexpr int DNST = 4;               // default ring stages

enum DmaMode { DMA_SUB = 0, DMA_ADD = 1, DMA_SET = 2 };

typedef __attribute__((address_space(3))) void dma_lds_void_t;
typedef __attribute__((address_space(3))) char dma_lds_char;

template <int N>
__device__ __forceinline__ void dma_wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Work-group barrier without __syncthreads()' fence, which would also wait
// for the chunks still meant to be in flight; this wave's LDS operations are
// drained first, and chunk arrival is covered by the vmcnt waits.
__device__ __forceinline__ void dma_lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// buffer resource over [p, p + bytes), base and size kept in scalar registers
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const float *p, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)b);
    const int n = __builtin_amdgcn_readfirstlane((int)std::max<int64_t>(bytes, 0));
    return __builtin_amdgcn_make_buffer_rsrc((void *)bu, (short)0, n, 0x00020000);
}

// Tiles are 128 rows x TN columns (TN = 128 or 64).  Waves form a 2 x 2 grid
// of 64 x TN/2 blocks (MB = TN/64 MFMA blocks across).  Each of the four
// waves moves KC/4 k-rows of every chunk.
template <int TN, int NST = DNST, int KC = DK>
struct DmaShape {
    static_assert(KC % 16 == 0 && NST >= 2, "chunk of whole 16-row groups, at least two stages");
    static constexpr int MB = TN / 64;                 // 32-column MFMA blocks per wave
    static constexpr int AST = KC * DT;                // A chunk (floats)
    static constexpr int BST = KC * TN;                // B chunk (floats)
    static constexpr int STAGE = AST + BST;            // one ring stage: A chunk then B chunk
    static constexpr int RPW = KC / 4;                 // k-rows per wave per chunk
    static constexpr int AINS = RPW / 2;               // A load instructions per wave (2 rows each)
    static constexpr int BROWS = 1024 / (TN * 4);      // B k-rows per 1 KB load instruction (2 or 4)
    static constexpr int BINS = RPW / BROWS;           // B load instructions per wave per stage
    static constexpr int PER_STAGE = AINS + BINS;      // vector-memory instructions per stage per wave
    static constexpr int LDS_FLOATS = NST * STAGE;
};

typedef __attribute__((ext_vector_type(16))) float dma_f32x16;

// One tile.  rows / cols: the tile's extent inside C (at most 128 / TN).
// a_bytes / b_bytes: readable bytes from A / B (reads past them give zero).
// lds: DmaShape<TN, NST, KC>::LDS_FLOATS floats, 16-byte aligned.
template <int TN, int NST = DNST, int KC = DK>
__device__ __forceinline__ void dma_tile_product(float *C, int64_t ldc, int rows, int cols, const float *A, int64_t lda,
                                                 int64_t a_bytes, const float *B, int64_t ldb, int64_t b_bytes, int K,
                                                 int mode, float *lds) {
    typedef DmaShape<TN, NST, KC> S;
    constexpr int MB = S::MB;
    constexpr int STAGE = S::STAGE;
    constexpr int AST = S::AST;
    constexpr int RPW = S::RPW;
    constexpr int AINS = S::AINS;
    constexpr int BROWS = S::BROWS;
    constexpr int BINS = S::BINS;
    constexpr int PER_STAGE = S::PER_STAGE;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    const int nch = (K + KC - 1) / KC;
    // accumulator (ma, mb), register group g: C row wr*64 + ma*32 + li,
    // columns wc*TN/2 + mb*32 + 8g + 4h + [0, 4)

    // the C tile first: its loads are the oldest, covered by the first wait
    f32x4 cv[2][MB][4];
    const bool full_tile = rows == DT && cols == TN;
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r = wr * 64 + ma * 32 + li, c = wc * (TN / 2) + mb * 32 + 8 * g + 4 * h;
                const float *src = C + (int64_t)r * ldc + c;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (mode != DMA_SET) {
                    if (full_tile) {
                        x = *(const f32x4 *)src;
                    } else if (r < rows) {
                        if (c + 3 < cols) {
                            x = *(const f32x4 *)src;
                        } else {
                            if (c + 0 < cols) x.x = src[0];
                            if (c + 1 < cols) x.y = src[1];
                            if (c + 2 < cols) x.z = src[2];
                        }
                    }
                }
                cv[ma][mb][g] = x;
            }

    const __amdgpu_buffer_rsrc_t ra = dma_rsrc(A, a_bytes);
    const __amdgpu_buffer_rsrc_t rb = dma_rsrc(B, b_bytes);
    // wave w moves k-rows RPW w .. RPW w + RPW-1 of each chunk: A two rows
    // per instruction (32 lanes x 16 bytes each), B BROWS rows per instruction
    int offa[AINS], offb[BINS];
#pragma unroll
    for (int q = 0; q < AINS; ++q) offa[q] = (int)(((RPW * wave + 2 * q + h) * lda + 4 * li) * 4);
    {
        const int lpr = TN / 4;   // lanes per B row
#pragma unroll
        for (int q = 0; q < BINS; ++q)
            offb[q] = (int)(((RPW * wave + BROWS * q + lane / lpr) * ldb + 4 * (lane % lpr)) * 4);
    }
    auto issue = [&](int st) {
        dma_lds_char *buf = (dma_lds_char *)lds + (st % NST) * STAGE * 4;
        const int sa = (int)(st * KC * lda * 4), sb = (int)(st * KC * ldb * 4);
#pragma unroll
        for (int q = 0; q < AINS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (dma_lds_void_t *)(buf + (RPW * wave + 2 * q) * DT * 4), 16,
                                                     offa[q] + sa, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < BINS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (dma_lds_void_t *)(buf + (AST + (RPW * wave + BROWS * q) * TN) * 4), 16, offb[q] + sb, 0, 0, 0);
    };
    for (int st = 0; st < NST - 1 && st < nch; ++st) issue(st);

    dma_f32x16 acc[2][MB];
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[ma][mb] = dma_f32x16{};
    for (int ch = 0; ch < nch; ++ch) {
        // chunk ch landed: the chunks issued after it may stay in flight
        const int ahead = std::min(NST - 2, nch - 1 - ch);
        static_assert(NST <= 4, "waits written out for up to two chunks ahead");
        if (ahead >= 2)
            dma_wait_vm<2 * PER_STAGE>();
        else if (ahead == 1)
            dma_wait_vm<PER_STAGE>();
        else
            dma_wait_vm<0>();
        dma_lds_barrier();   // and every wave is done with chunk ch - 1's buffer
        if (ch + NST - 1 < nch) issue(ch + NST - 1);
        const float *as = lds + (ch % NST) * STAGE;
        const float *bs = as + AST;
        // the whole chunk's operands first (LDS reads return in order, so the
        // products wait only for the reads they use), then the products
        float fa[KC / 2][2], fb[KC / 2][MB];
#pragma unroll
        for (int s = 0; s < KC / 2; ++s) {
            const int k = 2 * s + h;
#pragma unroll
            for (int m = 0; m < 2; ++m) fa[s][m] = as[k * DT + wr * 64 + m * 32 + li];
#pragma unroll
            for (int m = 0; m < MB; ++m) fb[s][m] = bs[k * TN + wc * (TN / 2) + m * 32 + li];
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
        for (int s = 0; s < KC / 2; ++s)
            // D[n][m] += sum_k B(k, n) A(k, m): the tile transposed
#pragma unroll
            for (int ma = 0; ma < 2; ++ma)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[ma][mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[s][mb], fa[s][ma], acc[ma][mb], 0, 0, 0);
    }

    // accumulator register 4g + b is column c + b of row r
    const float sg = (mode == DMA_SUB) ? -1.f : 1.f;
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r = wr * 64 + ma * 32 + li, c = wc * (TN / 2) + mb * 32 + 8 * g + 4 * h;
                f32x4 x = cv[ma][mb][g];
                x.x = fmaf(sg, acc[ma][mb][4 * g + 0], x.x);
                x.y = fmaf(sg, acc[ma][mb][4 * g + 1], x.y);
                x.z = fmaf(sg, acc[ma][mb][4 * g + 2], x.z);
                x.w = fmaf(sg, acc[ma][mb][4 * g + 3], x.w);
                float *dst = C + (int64_t)r * ldc + c;
                if (full_tile) {
                    *(f32x4 *)dst = x;
                } else if (r < rows) {
                    if (c + 3 < cols) {
                        *(f32x4 *)dst = x;
                    } else {
                        if (c + 0 < cols) dst[0] = x.x;
                        if (c + 1 < cols) dst[1] = x.y;
                        if (c + 2 < cols) dst[2] = x.z;
                    }
                }
            }
}

}  // namespace
}  // namespace gptq
