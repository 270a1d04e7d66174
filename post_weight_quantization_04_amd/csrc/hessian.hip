// Stage 1: H += 2 X^T X  ("GPTQ (GPT Quantization)", "Fondation theorique :
// OBQ" definition of H and "Algorithme complet (pseudo-code)" step 1).
//
// X is row-major [n][d] and the contraction runs over tokens (rows).  The
// product kernel computes lower-triangle output tiles of X^T X with the token
// range split S ways; every work group writes its fp32 partial tile to a
// scratch slot.  A second kernel sums the slots of each tile in split order
// (deterministic, no float atomics), adds 2*sum into H and mirrors it to the
// upper triangle through LDS so that H stays bitwise symmetric.
//
// bf16 path: 256x256 tiles, 4 waves of 128x128, v_mfma_f32_32x32x16_bf16.
// X is staged through LDS as loaded (token-major rows of 512 bytes), with the
// 16-byte units of each row XOR-swizzled by the token index.  MFMA operands
// need 8 consecutive tokens of one channel per lane; the LDS transpose read
// ds_read_b64_tr_b16 delivers them directly: within each 16-lane group, lane
// i points at 4 channels of token i/4 and receives 4 tokens of one channel.
// Two such reads form one operand, so no register regrouping is needed, and
// the swizzle keeps each 32-lane half of a read on distinct banks.
//
// fp32 path: 128x128 tiles, 4 waves of 64x64, v_mfma_f32_32x32x2_f32.
#include "common.h"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

namespace gptq {

namespace {

constexpr int BT = 256;   // bf16 tile
constexpr int BBK = 32;   // tokens per LDS stage (bf16)
constexpr int NBUF = 4;   // LDS ring of stages (bf16): three stages in flight while one is computed
constexpr int FT = 128;   // fp32 tile
constexpr int FBK = 16;   // tokens per LDS stage (fp32)

__device__ __forceinline__ void tile_coords(int t, int &I, int &J) {
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > t) --i;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    I = i;
    J = t - i * (i + 1) / 2;
}

constexpr int SLAB_PASSES = BBK / 8;   // 16-byte chunks per thread per slab

// LDS position (in 16-byte units) of channel unit u (8 channels) of token t
// inside a slab: row t holds 32 units, permuted by u ^ 4 (t % 4).
__device__ __forceinline__ int slab_unit(int t, int u) { return t * 32 + (u ^ (4 * (t & 3))); }

// Load one BBK-token x 256-channel bf16 slab (A or B operand) into registers.
template <bool VEC>
__device__ __forceinline__ void load_slab_bf16(const uint16_t *__restrict__ X, int64_t n, int d,
                                               int64_t k, int c0, u32x4 (&r)[SLAB_PASSES]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < SLAB_PASSES; ++p) {
        const int row = (tid >> 5) + 8 * p;
        const int col = (tid & 31) * 8;
        const int64_t t = k + row;
        const int ch = c0 + col;
        if (VEC) {
            if (t < n && ch < d) {
                r[p] = *(const u32x4 *)(X + t * (int64_t)d + ch);
            } else {
                r[p] = u32x4{0u, 0u, 0u, 0u};
            }
        } else {
            unsigned w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                unsigned lo = 0, hi = 0;
                if (t < n && ch + 2 * e < d) lo = X[t * (int64_t)d + ch + 2 * e];
                if (t < n && ch + 2 * e + 1 < d) hi = X[t * (int64_t)d + ch + 2 * e + 1];
                w[e] = lo | (hi << 16);
            }
            r[p] = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

__device__ __forceinline__ void store_slab_bf16(uint16_t *s, const u32x4 (&r)[SLAB_PASSES]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < SLAB_PASSES; ++p) {
        const int row = (tid >> 5) + 8 * p;
        *(u32x4 *)(s + 8 * slab_unit(row, tid & 31)) = r[p];
    }
}

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

// One MFMA operand: tokens t0..t0+7 (k slots 0..7) of 32 channels.  off is
// this lane's byte offset for tokens t0..t0+3; tokens t0+4..t0+7 sit four
// rows (2 KB) further on with the same swizzle (t % 4 unchanged).
__device__ __forceinline__ bf16x8 tr_operand(const lds_char *base, int off) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(base + off + 4 * 512));
    const __attribute__((ext_vector_type(8))) short v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// p-th tile of the lower triangle in blocked order: super-tiles of 4x4 tiles
// row by row (off-diagonal super-tiles, then the diagonal one), tiles inside
// a super-tile row by row.
__device__ __forceinline__ void blocked_tile(int p, int nb, int &I, int &J) {
    constexpr int S = 4;
    const int nsb = (nb + S - 1) / S;
    for (int si = 0; si < nsb; ++si) {
        const int rows = min(S, nb - S * si);
        const int off = si * rows * S;                 // tiles in off-diagonal super-tiles of this row
        const int dg = rows * (rows + 1) / 2;
        if (p < off) {
            const int sj = p / (rows * S), q = p % (rows * S);
            I = S * si + q / S;
            J = S * sj + q % S;
            return;
        }
        p -= off;
        if (p < dg) {
            int r = 0;
            while ((r + 1) * (r + 2) / 2 <= p) ++r;
            I = S * si + r;
            J = S * si + (p - r * (r + 1) / 2);
            return;
        }
        p -= dg;
    }
    I = J = 0;
}

typedef __attribute__((address_space(3))) void lds_void_t;

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Work-group barrier without the release/acquire fence of __syncthreads():
// that fence would wait for every outstanding LDS DMA, including the stages
// still meant to be in flight.  LDS stores of this wave are drained first;
// DMA completion is covered by the explicit vmcnt waits before it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// wait until at most `left` of this wave's vector-memory instructions are outstanding
__device__ __forceinline__ void wait_vm_left(int left) {
    switch (left) {
        case 0: wait_vm<0>(); break;
        case 4: wait_vm<4>(); break;
        case 8: wait_vm<8>(); break;
        case 12: wait_vm<12>(); break;
        case 16: wait_vm<16>(); break;
        case 20: wait_vm<20>(); break;
        case 24: wait_vm<24>(); break;
        default: wait_vm<0>(); break;
    }
}

// Instruction order for each half of a stage (16 MFMAs): the next half's 16
// operand reads go out two per MFMA over the first eight, then the half's
// share of the refill DMAs, one per one or two MFMAs.  Reads in a burst (four
// per MFMA) or DMAs mixed in among them queue up behind each other in LDS and
// leave the matrix core waiting; spread this way the product runs ≈ 8%
// faster.  (The reads must precede the DMAs: LDS aliasing is unknown to the
// compiler.)
template <int NDMA>
__device__ __forceinline__ void interleave_refill() {
    constexpr int MFMA = 0x008, VMEM = 0x010, DSR = 0x100;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(DSR, 2, 0);
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < NDMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(VMEM, 1, 0);
        __builtin_amdgcn_sched_group_barrier(MFMA, 8 / NDMA, 0);
    }
}

// One (split, tile) unit over tokens [k0, k1).  DIAG: I == J, only the A slab
// is staged and the B operands read it too.
//
// VEC (d % 8 == 0): every stage is moved by 16-byte buffer loads straight into
// LDS through a buffer resource that spans exactly this unit's token rows, so
// rows at or past k1 (the ragged last stage, and the stages issued past the
// end to keep the ring uniform) arrive as zeros without a branch.  Channels
// past d inside a row only feed partial-tile rows and columns past d, which
// the reduction never reads.  Otherwise every stage goes through registers
// with per-element guards.
template <bool VEC, bool DIAG>
__device__ __forceinline__ void bf16_unit(const uint16_t *__restrict__ X, int64_t d, int I, int J, int64_t k0,
                                          int64_t k1, float *__restrict__ out, uint16_t *smem) {
    constexpr int SLAB = BBK * BT;
    constexpr int per_stage = (DIAG ? 1 : 2) * (BBK / 8);   // vector-memory instructions per stage per wave
    const int nst = (k1 > k0) ? (int)((k1 - k0 + BBK - 1) / BBK) : 0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: LDS DMA bases go to M0
    const int lane = threadIdx.x & 63;
    const int wr = wave >> 1, wc = wave & 1;
    const int h = lane >> 5, li = lane & 31;

    f32x16 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x16{};

    // DMA addressing: wave chunk q covers token rows 2 (wave * BBK/8 + q) and
    // +1 of a stage; lane l's 16 bytes land at chunk base + 16 l and hold the
    // channel unit that the swizzle places there.
    // base and size go through readfirstlane so the descriptor lives in SGPRs
    const uint64_t xbase = reinterpret_cast<uint64_t>(X + k0 * d);
    // (readfirstlane returns int: widen through uint32_t, never sign-extend)
    const uint64_t xb = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(xbase >> 32)) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)xbase);
    const int nrec = __builtin_amdgcn_readfirstlane((int)(std::max<int64_t>(k1 - k0, 0) * d * 2));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)xb, (short)0, nrec, 0x00020000);
    int dma_off[BBK / 8];
    if (VEC) {
#pragma unroll
        for (int q = 0; q < BBK / 8; ++q) {
            const int row = 2 * (wave * (BBK / 8) + q) + (lane >> 5);
            const int unit = (lane & 31) ^ (4 * (row & 3));
            dma_off[q] = (int)((row * d + unit * 8) * 2);
        }
    }
    auto dma_part = [&](int st, int q0, int q1) {
        const int stage_off = (int)((int64_t)st * BBK * d * 2);
        lds_void_t *buf = (lds_void_t *)(smem + (st % NBUF) * 2 * SLAB);
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            const int chunk = wave * (BBK / 8) + q;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)((lds_char *)buf + chunk * 1024), 16,
                                                     dma_off[q] + stage_off + I * BT * 2, 0, 0, 0);
            if (!DIAG)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)((lds_char *)buf + SLAB * 2 + chunk * 1024),
                                                         16, dma_off[q] + stage_off + J * BT * 2, 0, 0, 0);
        }
    };
    auto dma = [&](int st) { dma_part(st, 0, BBK / 8); };
    auto reg_issue = [&](int st) {
        if (st >= nst) return;
        const int64_t k = k0 + (int64_t)st * BBK;
        uint16_t *buf = smem + (st % NBUF) * 2 * SLAB;
        u32x4 r[SLAB_PASSES];
        load_slab_bf16<VEC>(X, k1, (int)d, k, I * BT, r);
        wait_vm<0>();
        store_slab_bf16(buf, r);
        if (!DIAG) {
            load_slab_bf16<VEC>(X, k1, (int)d, k, J * BT, r);
            wait_vm<0>();
            store_slab_bf16(buf + SLAB, r);
        }
    };
    auto issue = [&](int st) {
        if (VEC)
            dma(st);
        else
            reg_issue(st);
    };
    if (nst > 0) {
        for (int st = 0; st < NBUF - 1; ++st) issue(st);
    }

    // Transpose-read addressing.  Lane l sits in 16-lane group g = l / 16 at
    // index i = l % 16; for operand block m (32 channels at 32 m of the wave's
    // 128) it points at token 8 (g / 2) + i / 4 of the k step and channels
    // 16 (g % 2) + 4 (i % 4) .. +3, swizzled by the token's i / 4.
    const int g = lane >> 4, i16 = lane & 15;
    const int q4 = i16 >> 2;
    const int lane_row = (8 * (g >> 1) + q4) * 512 + (i16 & 1) * 8;
    const int lane_unit = 2 * (g & 1) + ((i16 & 3) >> 1);
    int offa[4], offb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        offa[m] = lane_row + 16 * (wr * 16 + 4 * (m ^ q4) + lane_unit);
        offb[m] = lane_row + 16 * (wc * 16 + 4 * (m ^ q4) + lane_unit) + (DIAG ? 0 : SLAB * 2);
    }
    const lds_char *lds = (const lds_char *)smem;
    // operands of k step ks (16 tokens) of stage st
    auto frags = [&](int st, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
        const lds_char *a = lds + (st % NBUF) * 2 * SLAB * 2 + ks * 16 * 512;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            fa[m] = tr_operand(a, offa[m]);
            fb[m] = tr_operand(a, offb[m]);
        }
    };
    auto mfma16 = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[4]) {
#pragma unroll
        for (int ma = 0; ma < 4; ++ma)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                acc[ma * 4 + mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ma], fb[mb], acc[ma * 4 + mb], 0, 0, 0);
    };
    // Software pipeline over the two k steps of a stage: the first operands
    // of stage st+1 are read while the second half of stage st multiplies, so
    // the wait for the next stage and the barrier sit behind queued MFMAs.
    // Ring: stage j lives in buffer j % NBUF, and NBUF-2 stages beyond the
    // one waited for are always in flight (past the end they load zeros).
    // Each barrier is passed only once every wave has finished reading the
    // stage before it (lds_barrier drains this wave's LDS reads), so that
    // stage's buffer is free from there on: half of its refill goes out with
    // the MFMAs after the barrier, the other half with the next half stage's
    // (DMA writes spread over the whole stage instead of crowding LDS in one
    // half).  Every stage is wholly issued before the wait that counts it.
    static_assert(BBK == 32, "two k steps per stage");
    if (DIAG && VEC && wr < wc) {
        // The wave above the diagonal of a diagonal tile: its quadrant is never
        // stored, so it only moves its share of every stage and meets every
        // barrier of the others (same DMA order, same waits).
        if (nst > 0) {
            wait_vm_left((NBUF - 2) * per_stage);
            lds_barrier();
            dma_part(NBUF - 1, 0, BBK / 16);
            for (int st = 0; st < nst - 1; ++st) {
                dma_part(st - 1 + NBUF, BBK / 16, BBK / 8);
                wait_vm_left((NBUF - 2) * per_stage);
                lds_barrier();
                dma_part(st + NBUF, 0, BBK / 16);
            }
            wait_vm<0>();
        }
        return;
    }
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    if (nst > 0) {
        wait_vm_left((NBUF - 2) * per_stage);                   // stage 0 landed
        lds_barrier();
        if (VEC)
            dma_part(NBUF - 1, 0, BBK / 16);                     // the one buffer still free: first half
        else
            issue(NBUF - 1);
        frags(0, 0, fa0, fb0);
        for (int st = 0; st < nst - 1; ++st) {
            frags(st, 1, fa1, fb1);
            if (VEC) {
                dma_part(st - 1 + NBUF, BBK / 16, BBK / 8);      // second half of the refill begun before
                mfma16(fa0, fb0);
                interleave_refill<per_stage / 2>();
            } else {
                mfma16(fa0, fb0);
            }
            // keep the first half's MFMAs ahead of the wait and the barrier
            __builtin_amdgcn_sched_barrier(0);
            wait_vm_left((NBUF - 2) * per_stage);               // stage st+1 landed
            lds_barrier();                                       // all reads of stage st are done
            __builtin_amdgcn_sched_barrier(0);
            frags(st + 1, 0, fa0, fb0);
            if (VEC)
                dma_part(st + NBUF, 0, BBK / 16);                // first half of the refill of stage st's buffer
            else
                issue(st + NBUF);                                // into the buffer of stage st
            mfma16(fa1, fb1);
            if (VEC) interleave_refill<per_stage / 2>();
            __builtin_amdgcn_sched_barrier(0);
        }
        frags(nst - 1, 1, fa1, fb1);
        mfma16(fa0, fb0);
        mfma16(fa1, fb1);
        wait_vm<0>();   // stages issued past the end must land before the group's LDS is released
    }
    // (register-staged path) the wave above the diagonal of a diagonal tile
    // computed nothing useful
    if (DIAG && wr < wc) return;
    // accumulator layout: lane (h, li), register 4a+b <-> row 8a+4h+b, column li
#pragma unroll
    for (int ma = 0; ma < 4; ++ma)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int r = wr * 128 + 32 * ma + 8 * a + 4 * h + b;
                    const int c = wc * 128 + 32 * mb + li;
                    out[r * BT + c] = acc[ma * 4 + mb][4 * a + b];
                }
}

template <bool VEC>
__global__ __launch_bounds__(256) void hess_bf16_kernel(const uint16_t *__restrict__ X, int64_t n, int d,
                                                        float *__restrict__ part, int ntiles, int nb, int nsplit,
                                                        int64_t tok_per_split, int round_wgs) {
    // smem[buf][op]: op 0 = A slab (channels of tile row I), op 1 = B slab (tile column J)
    __shared__ __attribute__((aligned(16))) uint16_t smem[NBUF * 2 * BBK * BT];

    // Units (split-major, blocked tile order) are handed out one round of
    // round_wgs groups (one per CU) at a time.  Work-group ids go round-robin
    // over the 8 XCDs; inside a round each XCD takes a contiguous run of units,
    // so the groups it runs at once share a token range and few column blocks
    // (reuse in its L2), while all XCDs stream the same token range together
    // (reuse in the memory-side cache instead of one HBM read per XCD).
    const int base = (int)(blockIdx.x / round_wgs) * round_wgs;
    const int m = min(round_wgs, (int)gridDim.x - base);    // multiple of 8
    const int q = (int)blockIdx.x - base;
    const int unit = base + (m / 8) * (q % 8) + q / 8;
    if (unit >= ntiles * nsplit) return;
    const int split = unit / ntiles;
    int I, J;
    blocked_tile(unit % ntiles, nb, I, J);
    const int w = split * ntiles + I * (I + 1) / 2 + J;    // partial slot: split-major, row-major tile
    const int64_t k0 = (int64_t)split * tok_per_split;
    const int64_t k1 = std::min<int64_t>(n, k0 + tok_per_split);
    float *out = part + (int64_t)w * BT * BT;
    if (I == J)
        bf16_unit<VEC, true>(X, d, I, J, k0, k1, out, smem);
    else
        bf16_unit<VEC, false>(X, d, I, J, k0, k1, out, smem);
}

template <bool VEC>
__device__ __forceinline__ void load_slab_f32(const float *__restrict__ X, int64_t n, int d, int64_t k,
                                              int c0, f32x4 (&r)[2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int row = (tid >> 5) + 8 * p;
        const int col = (tid & 31) * 4;
        const int64_t t = k + row;
        const int ch = c0 + col;
        if (VEC) {
            r[p] = (t < n && ch < d) ? *(const f32x4 *)(X + t * (int64_t)d + ch) : f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) r[p][e] = (t < n && ch + e < d) ? X[t * (int64_t)d + ch + e] : 0.f;
        }
    }
}

__device__ __forceinline__ void store_slab_f32(float *s, const f32x4 (&r)[2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int row = (tid >> 5) + 8 * p;
        const int col = (tid & 31) * 4;
        *(f32x4 *)(s + row * FT + col) = r[p];
    }
}

template <bool VEC>
__global__ __launch_bounds__(256) void hess_f32_kernel(const float *__restrict__ X, int64_t n, int d,
                                                       float *__restrict__ part, int ntiles,
                                                       int64_t tok_per_split) {
    __shared__ __attribute__((aligned(16))) float sA[2][FBK * FT];
    __shared__ __attribute__((aligned(16))) float sB[2][FBK * FT];
    const int w = blockIdx.x;
    const int split = w / ntiles;
    int I, J;
    tile_coords(w % ntiles, I, J);
    const bool diag = (I == J);
    const int64_t k0 = (int64_t)split * tok_per_split;
    const int64_t k1 = std::min<int64_t>(n, k0 + tok_per_split);
    const int nst = (k1 > k0) ? (int)((k1 - k0 + FBK - 1) / FBK) : 0;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wr = wave >> 1, wc = wave & 1;
    const int h = lane >> 5, li = lane & 31;
    const bool active = !(diag && wr < wc);

    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
    f32x4 ra[2], rb[2];
    if (nst > 0) {
        load_slab_f32<VEC>(X, k1, d, k0, I * FT, ra);
        store_slab_f32(sA[0], ra);
        if (!diag) {
            load_slab_f32<VEC>(X, k1, d, k0, J * FT, rb);
            store_slab_f32(sB[0], rb);
        }
    }
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nst;
        if (more) {
            const int64_t k = k0 + (int64_t)(st + 1) * FBK;
            load_slab_f32<VEC>(X, k1, d, k, I * FT, ra);
            if (!diag) load_slab_f32<VEC>(X, k1, d, k, J * FT, rb);
        }
        if (active) {
            const float *a = sA[buf];
            const float *b = diag ? sA[buf] : sB[buf];
#pragma unroll
            for (int ks = 0; ks < FBK / 2; ++ks) {
                const int row = 2 * ks + h;
                float fa[2], fb[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    fa[m] = a[row * FT + wr * 64 + m * 32 + li];
                    fb[m] = b[row * FT + wc * 64 + m * 32 + li];
                }
#pragma unroll
                for (int ma = 0; ma < 2; ++ma)
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
                        acc[ma * 2 + mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[ma], fb[mb], acc[ma * 2 + mb], 0, 0, 0);
            }
        }
        if (more) {
            store_slab_f32(sA[buf ^ 1], ra);
            if (!diag) store_slab_f32(sB[buf ^ 1], rb);
        }
        __syncthreads();
    }
    if (!active) return;
    float *out = part + (int64_t)w * FT * FT;
#pragma unroll
    for (int ma = 0; ma < 2; ++ma)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int r = wr * 64 + ma * 32 + 8 * a + 4 * h + b;
                    const int c = wc * 64 + mb * 32 + li;
                    out[r * FT + c] = acc[ma * 2 + mb][4 * a + b];
                }
}

// Sum the split partials of each lower tile (fixed order), H += 2*sum, mirror.
// One work group per 64x64 sub-block; VEC (d % 4 == 0): each thread owns four
// adjacent columns of four rows, read and written 16 bytes at a time, and the
// mirrored (upper) copy is written as 16-byte runs of four source rows.
template <bool VEC>
__global__ __launch_bounds__(256) void hess_reduce_kernel(const float *__restrict__ part, float *__restrict__ H,
                                                          int d, int T, int ntiles, int nsplit) {
    __shared__ float tileT[64][65];
    const int sub_per = T / 64;
    const int t = blockIdx.x / (sub_per * sub_per);
    const int sb = blockIdx.x % (sub_per * sub_per);
    const int sr = sb / sub_per, sc = sb % sub_per;
    int I, J;
    tile_coords(t, I, J);
    const bool diag = (I == J);
    if (diag && sr < sc) return;
    const int row0 = I * T + sr * 64, col0 = J * T + sc * 64;
    if (row0 >= d || col0 >= d) return;
    const int64_t tile_stride = (int64_t)ntiles * T * T;
    const float *pt = part + (int64_t)t * T * T;
    if (VEC) {
        const int cg = threadIdx.x & 15, ty = threadIdx.x >> 4;
        const int c4 = 4 * cg;
        const int gc = col0 + c4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = ty + 16 * i;
            const int gr = row0 + rr;
            const int64_t po = (int64_t)(sr * 64 + rr) * T + sc * 64 + c4;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int sp = 0; sp < nsplit; ++sp) {
                const f32x4 p = *(const f32x4 *)(pt + sp * tile_stride + po);
                s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
            }
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (gr < d && gc < d) {     // d % 4 == 0: the four columns are all in range
                float *hp = H + (int64_t)gr * d + gc;
                const f32x4 h = *(const f32x4 *)hp;
                v = f32x4{h.x + 2.f * s.x, h.y + 2.f * s.y, h.z + 2.f * s.z, h.w + 2.f * s.w};
                if (!diag || gc + 3 <= gr) {
                    *(f32x4 *)hp = v;
                } else {
                    // diagonal sub-block: the lower part only (the mirror writes the rest)
                    if (gc + 0 <= gr) hp[0] = v.x; else v.x = 0.f;
                    if (gc + 1 <= gr) hp[1] = v.y; else v.y = 0.f;
                    if (gc + 2 <= gr) hp[2] = v.z; else v.z = 0.f;
                    if (gc + 3 <= gr) hp[3] = v.w; else v.w = 0.f;
                }
            }
            tileT[rr][c4 + 0] = v.x;
            tileT[rr][c4 + 1] = v.y;
            tileT[rr][c4 + 2] = v.z;
            tileT[rr][c4 + 3] = v.w;
        }
        __syncthreads();
        // mirror: H[col0 + cc][row0 + rr .. rr+3] = tileT[rr .. rr+3][cc]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = ty + 16 * i, rr = c4;
            const int gr = col0 + cc, gcol = row0 + rr;   // destination row, first column
            if (gr >= d || gcol >= d) continue;
            float *hp = H + (int64_t)gr * d + gcol;
            const f32x4 v = {tileT[rr + 0][cc], tileT[rr + 1][cc], tileT[rr + 2][cc], tileT[rr + 3][cc]};
            if (gcol > gr) {
                *(f32x4 *)hp = v;
            } else {
                if (gcol + 0 > gr) hp[0] = v.x;
                if (gcol + 1 > gr) hp[1] = v.y;
                if (gcol + 2 > gr) hp[2] = v.z;
                if (gcol + 3 > gr) hp[3] = v.w;
            }
        }
        return;
    }
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int rr = ty; rr < 64; rr += 4) {
        const int r = sr * 64 + rr, c = sc * 64 + tx;
        const int gr = row0 + rr, gc = col0 + tx;
        float v = 0.f;
        if (gr < d && gc < d && !(diag && gc > gr)) {
            float s = 0.f;
            for (int sp = 0; sp < nsplit; ++sp) s += pt[sp * tile_stride + (int64_t)r * T + c];
            v = H[(int64_t)gr * d + gc] + 2.0f * s;
            H[(int64_t)gr * d + gc] = v;
        }
        tileT[rr][tx] = v;
    }
    __syncthreads();
    // mirror: H[col0 + cc][row0 + rr] = tileT[rr][cc]
    for (int cc = ty; cc < 64; cc += 4) {
        const int gr = col0 + cc, gc = row0 + tx;   // destination (upper triangle)
        if (gr < d && gc < d && gc > gr) H[(int64_t)gr * d + gc] = tileT[tx][cc];
    }
}

int cu_count() {
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

HessPlan hessian_plan(int64_t n, int64_t d, int is_bf16, int64_t max_slots) {
    HessPlan p{};
    p.tile = is_bf16 ? BT : FT;
    const int bk = is_bf16 ? BBK : FBK;
    p.nb = (int)cdiv(d, p.tile);
    p.ntiles = p.nb * (p.nb + 1) / 2;
    const int cus = 256;   // planning assumes one work group per CU on a 256-CU part
    // pick the token split that minimises rounds * per-group work + partial traffic
    const double flop_rate_cu = 0.6 * (is_bf16 ? 2.5e15 : 1.57e14) / 256.0;
    const double t_tok = 2.0 * p.tile * p.tile / flop_rate_cu;
    const double bw = 4.0e12;
    int best_s = 1;
    double best = 1e300;
    const int smax = (int)std::max<int64_t>(1, std::min<int64_t>(32, cdiv(std::max<int64_t>(n, 1), 4 * bk)));
    // bf16 units address their token rows with 32-bit byte offsets from the
    // unit's first row, including the ring stages issued past the end
    const int64_t tok_limit = is_bf16 ? ((int64_t)1 << 31) / (2 * std::max<int64_t>(d, 1)) - (NBUF + 1) * BBK
                                      : INT64_MAX;
    for (int s = 1; s <= std::max(smax, 1); ++s) {
        const int64_t nwg = (int64_t)s * p.ntiles;
        const int64_t tok = cdiv(cdiv(std::max<int64_t>(n, 1), s), bk) * bk;
        if (tok > tok_limit || nwg > max_slots) continue;
        const double rounds = (double)cdiv(nwg, cus);
        const double bytes = 2.0 * (double)nwg * p.tile * p.tile * 4.0;
        const double t = rounds * tok * t_tok + bytes / bw;
        if (t < best * 0.98) {
            best = t;
            best_s = s;
        }
    }
    if (best >= 1e300) {   // token range too long for the split cap: split further
        best_s = (int)cdiv(std::max<int64_t>(n, 1), std::max<int64_t>(tok_limit / bk * bk, bk));
        while (cdiv(cdiv(std::max<int64_t>(n, 1), best_s), bk) * bk > tok_limit) ++best_s;
    }
    p.s_off = p.s_diag = best_s;
    p.nwg = best_s * p.ntiles;
    p.slots = p.nwg;
    return p;
}

size_t hessian_ws_bytes(const HessPlan &p) {
    return align256((size_t)p.slots * p.tile * p.tile * sizeof(float));
}

// ---------------------------------------------------------------------------
// Library-owned scratch for callers that cannot allocate.  Every GPU that
// runs the library holds one copy of this array until the process ends; its
// device address is resolved once per device (with that device current) and
// kept, because in host code the array's name is only a host-side stand-in.
// Calls that overlap on one GPU share it and race.
// ---------------------------------------------------------------------------
namespace {
__device__ __attribute__((aligned(256))) unsigned char scratch[HESS_STATIC_SCRATCH_BYTES];
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};
}  // namespace

hipError_t hessian_static_scratch(void **ptr) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t hessian_product_launch(const void *X, int is_bf16, int64_t n, int64_t d, float *partials,
                                  const HessPlan &p, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int round_wgs = std::max(8, cu_count() / 8 * 8);   // grid and rounds stay multiples of 8
    const int bk = is_bf16 ? BBK : FBK;
    const int64_t tok = cdiv(cdiv(n, p.s_off), bk) * bk;
    if (is_bf16) {
        const unsigned grid = (unsigned)(cdiv(p.nwg, 8) * 8);
        if (d % 8 == 0)
            hess_bf16_kernel<true><<<grid, 256, 0, st>>>((const uint16_t *)X, n, (int)d, partials, p.ntiles, p.nb,
                                                         p.s_off, tok, round_wgs);
        else
            hess_bf16_kernel<false><<<grid, 256, 0, st>>>((const uint16_t *)X, n, (int)d, partials, p.ntiles, p.nb,
                                                          p.s_off, tok, round_wgs);
    } else {
        if (d % 4 == 0)
            hess_f32_kernel<true><<<p.nwg, 256, 0, st>>>((const float *)X, n, (int)d, partials, p.ntiles, tok);
        else
            hess_f32_kernel<false><<<p.nwg, 256, 0, st>>>((const float *)X, n, (int)d, partials, p.ntiles, tok);
    }
    return hipGetLastError();
}

hipError_t hessian_reduce_launch(int64_t d, float *H, const float *partials, const HessPlan &p, hipStream_t st) {
    const int sub = p.tile / 64;
    if (d % 4 == 0)
        hess_reduce_kernel<true><<<p.ntiles * sub * sub, 256, 0, st>>>(partials, H, (int)d, p.tile, p.ntiles, p.s_off);
    else
        hess_reduce_kernel<false><<<p.ntiles * sub * sub, 256, 0, st>>>(partials, H, (int)d, p.tile, p.ntiles, p.s_off);
    return hipGetLastError();
}

}  // namespace gptq
