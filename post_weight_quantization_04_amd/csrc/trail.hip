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
// 128 x 128 tile and one group per compute unit, the operand chunks moved
// from global memory straight into LDS by 16-byte buffer loads through a
// four-stage ring, three chunks in flight while one is multiplied, so that a
// tile runs at the matrix cores' rate even when it has its unit to itself
// (a launch's last, partial round).  The buffer resources end at row K of E
// and U, so the ragged last chunk reads zeros without a branch; rows and
// columns past the tile's edge only feed entries that are not stored.
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

constexpr int NST = 4;   // LDS ring stages of the main kernel

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char;

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Work-group barrier without __syncthreads()' fence, which would also wait
// for the chunks still meant to be in flight; this wave's LDS operations are
// drained first, and chunk arrival is covered by the vmcnt waits.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// buffer resource over [p, p + bytes), base and size kept in scalar registers
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *p, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)b);
    const int n = __builtin_amdgcn_readfirstlane((int)std::max<int64_t>(bytes, 0));
    return __builtin_amdgcn_make_buffer_rsrc((void *)bu, (short)0, n, 0x00020000);
}

// Requires d_out % 4 == 0, d_in % 4 == 0, c_begin % 4 == 0 (16-byte aligned
// rows and tile origins) and K * max(d_out, d_in) * 4 < 2^31.  Tiles are
// 128 rows x TN columns (TN = 128, or 64 for the last columns of a launch
// whose 128-wide tiles would leave a half-empty last round); tile t is row
// tile t % tiles_m of column tile t / tiles_m.  Waves form a 2 x 2 grid of
// 64 x TN/2 blocks (MB = TN/64 MFMA blocks across).
template <int TN>
struct DmaShape {
    static constexpr int MB = TN / 64;                 // 32-column MFMA blocks per wave
    static constexpr int BST = TK * TN;                // B chunk (floats)
    static constexpr int STAGE = TSTAGE + BST;         // one ring stage: A chunk then B chunk
    static constexpr int BROWS = 1024 / (TN * 4);      // B k-rows per 1 KB load instruction (2 or 4)
    static constexpr int BINS = 8 / BROWS;             // B load instructions per wave per stage
    static constexpr int PER_STAGE = 4 + BINS;         // vector-memory instructions per stage per wave
};

// one tile; lds: NST * DmaShape<TN>::STAGE floats.  (The body lives in a
// device function: the host pass instantiates a kernel template's body, and
// the buffer-resource type exists only for the device.)
template <int TN>
__device__ __forceinline__ void trail_dma_tile(const QuantArgs &a, int u_row0, int K, int c_begin, int c_end, int tiles_m,
                                               float *lds) {
    constexpr int MB = DmaShape<TN>::MB;
    constexpr int STAGE = DmaShape<TN>::STAGE;
    constexpr int BROWS = DmaShape<TN>::BROWS;
    constexpr int BINS = DmaShape<TN>::BINS;
    constexpr int PER_STAGE = DmaShape<TN>::PER_STAGE;
    const int t = blockIdx.x;
    const int64_t row0 = (int64_t)(t % tiles_m) * TT;
    const int64_t col0 = (int64_t)c_begin + (int64_t)(t / tiles_m) * TN;
    const int rows = (int)std::min<int64_t>(TT, a.d_out - row0);
    const int cols = (int)std::min<int64_t>(TN, c_end - col0);
    const int64_t d_out = a.d_out, d_in = a.d_in;
    float *C = a.Wp + row0 * d_in + col0;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int wr = wave >> 1, wc = wave & 1, h = lane >> 5, li = lane & 31;
    const int nch = (K + TK - 1) / TK;
    // accumulator (ma, mb), register group g: W row wr*64 + ma*32 + li,
    // columns wc*TN/2 + mb*32 + 8g + 4h + [0, 4)

    // the W tile first: its loads are the oldest, covered by the first wait
    f32x4 cv[2][MB][4];
    const bool full_tile = rows == TT && cols == TN;
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r = wr * 64 + ma * 32 + li, c = wc * (TN / 2) + mb * 32 + 8 * g + 4 * h;
                const float *src = C + (int64_t)r * d_in + c;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
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
                cv[ma][mb][g] = x;
            }

    // A(k, m) = E[k][row0 + m] for k < K; B(k, n) = U[u_row0 + k][col0 + n]
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.E + row0, ((int64_t)K * d_out - row0) * 4);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.U + (int64_t)u_row0 * d_in + col0, ((int64_t)K * d_in - col0) * 4);
    // wave w moves k-rows 8w .. 8w+7 of each chunk: A two rows per
    // instruction (32 lanes x 16 bytes each), B BROWS rows per instruction
    int offa[4], offb[BINS];
#pragma unroll
    for (int q = 0; q < 4; ++q) offa[q] = (int)(((8 * wave + 2 * q + h) * d_out + 4 * li) * 4);
    {
        const int lpr = TN / 4;   // lanes per B row
#pragma unroll
        for (int q = 0; q < BINS; ++q)
            offb[q] = (int)(((8 * wave + BROWS * q + lane / lpr) * d_in + 4 * (lane % lpr)) * 4);
    }
    auto issue = [&](int st) {
        lds_char *buf = (lds_char *)lds + (st % NST) * STAGE * 4;
        const int sa = (int)(st * TK * d_out * 4), sb = (int)(st * TK * d_in * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)(buf + (8 * wave + 2 * q) * TLD * 4), 16,
                                                     offa[q] + sa, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < BINS; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)(buf + (TSTAGE + (8 * wave + BROWS * q) * TN) * 4),
                                                     16, offb[q] + sb, 0, 0, 0);
    };
    for (int st = 0; st < NST - 1 && st < nch; ++st) issue(st);

    f32x16_t acc[2][MB];
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[ma][mb] = f32x16_t{};
    for (int ch = 0; ch < nch; ++ch) {
        // chunk ch landed: the chunks issued after it may stay in flight
        const int ahead = std::min(NST - 2, nch - 1 - ch);
        if (ahead >= 2)
            wait_vm<2 * PER_STAGE>();
        else if (ahead == 1)
            wait_vm<PER_STAGE>();
        else
            wait_vm<0>();
        lds_barrier();   // and every wave is done with chunk ch - 1's buffer
        if (ch + NST - 1 < nch) issue(ch + NST - 1);
        const float *as = lds + (ch % NST) * STAGE;
        const float *bs = as + TSTAGE;
        // the whole chunk's operands first (LDS reads return in order, so the
        // products wait only for the reads they use), then the products
        float fa[TK / 2][2], fb[TK / 2][MB];
#pragma unroll
        for (int s = 0; s < TK / 2; ++s) {
            const int k = 2 * s + h;
#pragma unroll
            for (int m = 0; m < 2; ++m) fa[s][m] = as[k * TLD + wr * 64 + m * 32 + li];
#pragma unroll
            for (int m = 0; m < MB; ++m) fb[s][m] = bs[k * TN + wc * (TN / 2) + m * 32 + li];
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
        for (int s = 0; s < TK / 2; ++s)
            // D[n][m] += sum_k B(k, n) A(k, m): the tile transposed
#pragma unroll
            for (int ma = 0; ma < 2; ++ma)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[ma][mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[s][mb], fa[s][ma], acc[ma][mb], 0, 0, 0);
    }

    // W tile -= product; accumulator register 4g + b is column c + b of row r
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r = wr * 64 + ma * 32 + li, c = wc * (TN / 2) + mb * 32 + 8 * g + 4 * h;
                f32x4 x = cv[ma][mb][g];
                x.x -= acc[ma][mb][4 * g + 0];
                x.y -= acc[ma][mb][4 * g + 1];
                x.z -= acc[ma][mb][4 * g + 2];
                x.w -= acc[ma][mb][4 * g + 3];
                float *dst = C + (int64_t)r * d_in + c;
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

template <int TN>
__global__ __launch_bounds__(256, 1) void trail_dma_kernel(QuantArgs a, int u_row0, int K, int c_begin, int c_end,
                                                        int tiles_m) {
    __shared__ __attribute__((aligned(16))) float lds[NST * DmaShape<TN>::STAGE];
    trail_dma_tile<TN>(a, u_row0, K, c_begin, c_end, tiles_m, lds);
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
                         K * std::max(a.d_out, a.d_in) * 4 + (int64_t)TK * std::max(a.d_out, a.d_in) * 4 * NST < ((int64_t)1 << 31);
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
