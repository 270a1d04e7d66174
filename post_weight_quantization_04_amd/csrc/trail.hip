// Stage 4: the lazy trailing update
//   W[:, c_begin:c_end) -= E U[u_row0 : u_row0 + K, c_begin:c_end)
// ("GPTQ (GPT Quantization)", "Algorithme complet (pseudo-code)" step 3: a
// batch's errors are pushed onto the remaining columns once per batch).  E
// holds the errors of one or more consecutive blocks, already divided by
// U_kk, so the product uses U's rows as they are.  With more than one block
// per far update it is applied in two levels: after each block to the next
// block's columns only, and every few blocks to all columns beyond, with the
// pending blocks' errors stacked (the same sum, fewer passes over W).
//
// Main kernel (trail_dma_kernel, 16-byte aligned shapes): one work group per
// 128 x 128 tile and two groups per compute unit, the operand chunks moved
// from global memory straight into LDS by 16-byte buffer loads through a
// four-stage ring of 16 k-rows, three chunks in flight while one is
// multiplied, so that a tile keeps the matrix cores busy even when it has its
// unit to itself (a launch's last, partial round).  The buffer resources end at row K of E
// and U, so the ragged last chunk reads zeros without a branch; rows and
// columns past the tile's edge only feed entries that are not stored.  The
// tile body (dma_tile.h) is shared with the factorization's far update.
//
// Fallback (trail_kernel, any shape): one work group per 128 x 128 tile of W, fp32 operands on fp32 MFMA
// (v_mfma_f32_32x32x2_f32).  Both operands arrive as k-rows (E is [k][row],
// U is [k][col]), 32 k-rows per chunk, staged in LDS as [k][128] with 16-byte
// stores, double-buffered.  The MFMA computes the tile transposed
// (D = U_chunk^T E_chunk^T), so each lane's accumulator holds 4 consecutive
// columns of one W row: the W tile moves with 16-byte loads and stores.  Its
// loads go out after the first chunk's and the product starts from zero, so
// the W tile's latency passes during the product; it is added at the end.
#include "common.h"
#include "dma_tile.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int TT = 128;          // tile edge
constexpr int TK = 32;           // k-rows per chunk
constexpr int TLD = TT;          // LDS row stride (floats)
constexpr int TSTAGE = TK * TLD; // one operand chunk

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// 32 k-rows x 128 values (from p, rows ld apart), 16 per thread: thread t
// takes the 4-value group t % 32 of k-rows t / 32 + 8 q.  vec: the base and
// ld are 16-byte aligned and every group is inside [klim) x [nlim).
struct KChunk {
    f32x4 v[4];
    __device__ __forceinline__ void load(const float *p, int64_t ld, int k0, int klim, int nlim, bool vec) {
        const int t = threadIdx.x;
        const int n4 = (t & 31) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = k0 + (t >> 5) + 8 * q;
            const float *src = p + (int64_t)k * ld + n4;
            if (vec) {
                v[q] = *(const f32x4 *)src;
            } else {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (k < klim) {
                    if (n4 + 0 < nlim) x.x = src[0];
                    if (n4 + 1 < nlim) x.y = src[1];
                    if (n4 + 2 < nlim) x.z = src[2];
                    if (n4 + 3 < nlim) x.w = src[3];
                }
                v[q] = x;
            }
        }
    }
    __device__ __forceinline__ void store(float *s, float alpha) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int q = 0; q < 4; ++q) *(f32x4 *)(s + ((t >> 5) + 8 * q) * TLD + (t & 31) * 4) = alpha * v[q];
    }
};

// Accumulator (ma, mb) of wave (wr, wc) covers W rows wr*64 + ma*32 + li and
// columns wc*64 + mb*32 + 8a + 4h + [0, 4) in register group a (lane h, li).
__device__ __forceinline__ void tile_rowcol(int ma, int mb, int a, int &r, int &c) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    r = wr * 64 + ma * 32 + li;
    c = wc * 64 + mb * 32 + 8 * a + 4 * h;
}

__global__ __launch_bounds__(256, 2) void trail_kernel(QuantArgs a, int u_row0, int K, int c_begin, int c_end) {
    __shared__ __attribute__((aligned(16))) float lds[4 * TSTAGE];
    const int64_t row0 = (int64_t)blockIdx.x * TT;
    const int64_t col0 = (int64_t)c_begin + (int64_t)blockIdx.y * TT;
    const int rows = (int)std::min<int64_t>(TT, a.d_out - row0);
    const int cols = (int)std::min<int64_t>(TT, c_end - col0);
    const float *A = a.E + row0;                                   // A(k, m) = E[k][row0 + m]
    const float *B = a.U + (int64_t)u_row0 * a.d_in + col0;        // B(k, n) = U[u_row0 + k][col0 + n]
    float *C = a.Wp + row0 * a.d_in + col0;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    const bool vec_rows = rows == TT && ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && (a.d_out % 4 == 0);
    const bool vec_cols = cols == TT && ((reinterpret_cast<uintptr_t>(B) & 15) == 0) && (a.d_in % 4 == 0);
    const bool vec_c = vec_cols && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
    const int nch = (K + TK - 1) / TK;

    KChunk ca, cb;
    ca.load(A, a.d_out, 0, K, rows, vec_rows && TK <= K);
    cb.load(B, a.d_in, 0, K, cols, vec_cols && TK <= K);
    // the W tile, after the first chunk's loads
    f32x4 cv[2][2][4];
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                int r, c;
                tile_rowcol(ma, mb, g, r, c);
                const float *src = C + (int64_t)r * a.d_in + c;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (r < rows) {
                    if (vec_c) {
                        x = *(const f32x4 *)src;
                    } else {
                        if (c + 0 < cols) x.x = src[0];
                        if (c + 1 < cols) x.y = src[1];
                        if (c + 2 < cols) x.z = src[2];
                        if (c + 3 < cols) x.w = src[3];
                    }
                }
                cv[ma][mb][g] = x;
            }
    ca.store(lds, -1.f);
    cb.store(lds + TSTAGE, 1.f);
    __syncthreads();

    f32x16_t acc[2][2];
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[ma][mb] = f32x16_t{};
    for (int ch = 0; ch < nch; ++ch) {
        const int buf = ch & 1;
        const bool more = ch + 1 < nch;
        if (more) {
            const int k0 = (ch + 1) * TK;
            const bool full = k0 + TK <= K;
            ca.load(A, a.d_out, k0, K, rows, vec_rows && full);
            cb.load(B, a.d_in, k0, K, cols, vec_cols && full);
        }
        const float *as = lds + (2 * buf) * TSTAGE;
        const float *bs = lds + (2 * buf + 1) * TSTAGE;
#pragma unroll
        for (int s = 0; s < TK / 2; ++s) {
            const int k = 2 * s + h;
            float fa[2], fb[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                fa[m] = as[k * TLD + wr * 64 + m * 32 + li];
                fb[m] = bs[k * TLD + wc * 64 + m * 32 + li];
            }
            // D[n][m] += sum_k B(k, n) A(k, m): the tile transposed
#pragma unroll
            for (int ma = 0; ma < 2; ++ma)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[ma][mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[mb], fa[ma], acc[ma][mb], 0, 0, 0);
        }
        if (more) {
            ca.store(lds + (2 * (buf ^ 1)) * TSTAGE, -1.f);
            cb.store(lds + (2 * (buf ^ 1) + 1) * TSTAGE, 1.f);
        }
        __syncthreads();
    }

    // W tile += product; accumulator register 4g + b is column c + b of row r
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                int r, c;
                tile_rowcol(ma, mb, g, r, c);
                f32x4 x = cv[ma][mb][g];
                x.x += acc[ma][mb][4 * g + 0];
                x.y += acc[ma][mb][4 * g + 1];
                x.z += acc[ma][mb][4 * g + 2];
                x.w += acc[ma][mb][4 * g + 3];
                float *dst = C + (int64_t)r * a.d_in + c;
                if (r < rows) {
                    if (vec_c) {
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

// Main kernel: tile t is row tile t % tiles_m of column tile t / tiles_m,
// 128 rows x TN columns (TN = 128, or 64 for the last columns of a launch
// whose 128-wide tiles would leave a half-empty last round).  Requires
// d_out % 4 == 0, d_in % 4 == 0, c_begin % 4 == 0 (16-byte aligned rows and
// tile origins) and K * max(d_out, d_in) * 4 < 2^31.
// A(k, m) = E[k][row0 + m] and B(k, n) = U[u_row0 + k][col0 + n] for k < K:
// the buffer resources end at row K of E and U.
// Two groups per compute unit (a 64 KB ring each: four stages of 16 k-rows),
// so that one group's tile start overlaps the other's products (against one
// group per unit with four stages of 32 k-rows: q_proj's far launches
// 0.54 -> 0.50 ms per layer, down_proj's 4.42 -> 3.85 ms).
constexpr int TRAIL_NST = 4, TRAIL_KC = 16;
template <int TN>
__global__ __launch_bounds__(256, 2) void trail_dma_kernel(QuantArgs a, int u_row0, int K, int c_begin, int c_end,
                                                        int tiles_m) {
    __shared__ __attribute__((aligned(16))) float lds[DmaShape<TN, TRAIL_NST, TRAIL_KC>::LDS_FLOATS];
    const int t = blockIdx.x;
    const int64_t row0 = (int64_t)(t % tiles_m) * TT;
    const int64_t col0 = (int64_t)c_begin + (int64_t)(t / tiles_m) * TN;
    const int rows = (int)std::min<int64_t>(TT, a.d_out - row0);
    const int cols = (int)std::min<int64_t>(TN, c_end - col0);
    dma_tile_product<TN, TRAIL_NST, TRAIL_KC>(a.Wp + row0 * a.d_in + col0, a.d_in, rows, cols, a.E + row0, a.d_out,
                         ((int64_t)K * a.d_out - row0) * 4, a.U + (int64_t)u_row0 * a.d_in + col0, a.d_in,
                         ((int64_t)K * a.d_in - col0) * 4, K, DMA_SUB, lds);
}

int trail_cu_count() {
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            cached = cus;
        else
            cached = 256;
    }
    return cached;
}

}  // namespace

hipError_t trail_launch(const QuantArgs &a, int64_t u_row0, int64_t K, int64_t c_begin, int64_t c_end,
                        hipStream_t st) {
    if (c_end <= c_begin || K <= 0) return hipSuccess;
    const bool aligned = a.d_out % 4 == 0 && a.d_in % 4 == 0 && c_begin % 4 == 0 &&
                         reinterpret_cast<uintptr_t>(a.E) % 16 == 0 && reinterpret_cast<uintptr_t>(a.U) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(a.Wp) % 16 == 0 &&
                         K * std::max(a.d_out, a.d_in) * 4 + (int64_t)DK * std::max(a.d_out, a.d_in) * 4 * DNST < ((int64_t)1 << 31);
    if (aligned) {
        // 128-wide tiles, except that when they would leave a last round of
        // at most half the compute units, that round's whole column tiles go
        // to a second launch as twice as many 64-wide tiles
        const int64_t tiles_m = cdiv(a.d_out, TT);
        const int64_t tiles_n = cdiv(c_end - c_begin, TT);
        const int cus = trail_cu_count();
        const int64_t last = (tiles_m * tiles_n) % cus;
        int64_t narrow_cols = 0;   // column tiles done 64 wide
        if (last > 0 && last <= cus / 2 && last % tiles_m == 0) narrow_cols = last / tiles_m;
        const int64_t wide_end = std::min<int64_t>(c_end, c_begin + (tiles_n - narrow_cols) * TT);
        if (wide_end > c_begin) {
            trail_dma_kernel<128><<<(unsigned)(tiles_m * (tiles_n - narrow_cols)), 256, 0, st>>>(
                a, (int)u_row0, (int)K, (int)c_begin, (int)wide_end, (int)tiles_m);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (wide_end < c_end) {
            trail_dma_kernel<64><<<(unsigned)(tiles_m * cdiv(c_end - wide_end, 64)), 256, 0, st>>>(
                a, (int)u_row0, (int)K, (int)wide_end, (int)c_end, (int)tiles_m);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    dim3 grid((unsigned)cdiv(a.d_out, TT), (unsigned)cdiv(c_end - c_begin, TT));
    trail_kernel<<<grid, 256, 0, st>>>(a, (int)u_row0, (int)K, (int)c_begin, (int)c_end);
    return hipGetLastError();
}

}  // namespace gptq
