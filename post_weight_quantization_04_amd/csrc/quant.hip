// Stage 3: the in-block sequential quantize-and-compensate loop.
// "GPTQ (GPT Quantization)", "Fondation theorique : OBQ" (quantize column i,
// take its error, move the remaining columns) and "Algorithme complet
// (pseudo-code)" step 3 (columns in batches); "Optimization Gptq",
// "Quantizacao group-wise" (per-group scale and zero point).
//
// For block columns [b, e) of the processing order and every row r:
//   at a group start: xmin = min(0, min w), xmax = max(0, max w) over the
//     group's current values (an all-zero group uses [0, 1]);
//     s = (xmax - xmin) / maxq, z = rint(-xmin / s)
//   for k = b .. e-1:  q = clamp(rint(w_k / s) + z, 0, maxq),
//     E_k = (w_k - s (q - z)) / U_kk,  w_j -= E_k U_kj  for k < j < e.
// The update of the columns after e is left to the trailing product.
//
// Layout: a work group owns 16 rows; each row is spread over one 16-lane DPP
// row (lane c holds column c of the current 16-column chunk), so a wave
// holds four rows.  The block's W tile, the strict upper part of the block's
// U, 1/U_kk and the packed rows' offsets are staged in LDS.  Per column step
// the current value is broadcast across the 16 lanes with DPP row_newbcast;
// every lane then computes the same quantization and updates its own column
// with a coefficient preloaded into registers for the chunk.  After a chunk,
// its 16 x 16 errors go to LDS and the rest of the block takes
// W[16 rows, j] -= E[16 x 16] U[16, j] as 16 x 16 column tiles on fp32 MFMA
// (v_mfma_f32_16x16x4_f32), the four waves taking every fourth tile.  Before
// the first chunk the pending blocks' errors are applied to the block's own
// columns (the near update); for full 128-column blocks their U and E rows
// stream through an LDS ring of 64-row chunks moved by 16-byte buffer loads.
#include "common.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace gptq {

namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int QROWS = 16;     // rows per work group
constexpr int CH = 16;        // columns per chunk (= lanes per row)

__host__ __device__ inline int roundup16(int x) { return (x + 15) & ~15; }

// packed upper-triangle layout of the U block: row i keeps columns
// [4*floor(i/4), Bp); offsets stay 16-byte aligned.
__host__ __device__ inline int uoff(int i, int Bp) {
    const int A = i >> 2, r = i & 3;
    return 4 * A * Bp - 8 * A * (A - 1) + r * (Bp - 4 * A);
}
__host__ __device__ inline int usize(int Bp) { return uoff(Bp, Bp); }
__device__ __forceinline__ int uidx(int i, int j, int Bp) { return uoff(i, Bp) + j - 4 * (i >> 2); }
constexpr int ELD = CH + 1;   // row stride of the chunk's error tile in LDS

// Near-update ring (full 128-column blocks with 16-byte aligned rows): 64
// k-rows of U (128 columns) and of E (the group's 16 rows) per chunk, three
// chunks in LDS, moved by 16-byte buffer loads straight into LDS.
constexpr int NCH = 64;                        // k-rows per chunk
constexpr int NUF = NCH * 128;                 // U chunk (floats), [k][128], 16-byte groups swizzled
constexpr int NEF = NCH * QROWS;               // E chunk (floats), [k][16]
constexpr int NSTG = 3;                        // ring stages
constexpr int NRING = NSTG * (NUF + NEF);      // ring (floats)
constexpr int NDMA = 9;                        // buffer loads per wave per chunk: 8 of U, 1 of E

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char;

template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// work-group barrier without __syncthreads()' fence, which would also wait for
// the chunks still meant to be in flight; this wave's LDS operations are
// drained first, and chunk arrival is covered by the vmcnt waits
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

// W[16 rows][0:128) -= E[16 rows][0:nk) U[0:nk)[0:128) for a full 128-column
// block, the near update's fast path.  Wl: the staged W tile (row stride LW);
// ring: NRING floats of LDS, 16-byte aligned.  U rows come from u (row
// stride d_in), E rows from En (row stride d_out) at the group's row row0;
// the buffer resources end at row nk, so the ragged last chunk reads zeros.
// U chunk layout: k-row r holds column group g (4 columns) at slot
// g ^ 4 (r % 4), so that the product's reads (16 columns of 4 k-rows per
// instruction) hit 64 distinct banks.  Wave w takes column tiles 16w and
// 16w + 64 on v_mfma_f32_16x16x4_f32 (A[i][k] at lane i + 16k, B[k][j] at
// lane j + 16k, D[i][j] at lane 16 (i/4) + j, register i % 4), its
// accumulators kept across all chunks.  They hold -W and add E U (negation
// is exact, so the result is bitwise that of W - E U): the operands then go
// from LDS to the MFMAs untouched, and every read of a chunk is issued before
// its first product instead of each pair waiting for its own reads.
__device__ __forceinline__ void near_update_ring(float *Wl, int LW, float *ring, const float *u, const float *En,
                                                 int64_t row0, int64_t d_in, int64_t d_out, int nk) {
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, li = lane & 15, lk = lane >> 4;
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(u, ((int64_t)(nk - 1) * d_in + 128) * 4);
    // E ends exactly at row nk (its rows past nk may hold anything, even
    // NaN, which a zero U row would not cancel); rows of the group past d_out
    // in its last k-row read zeros, and earlier ones only feed rows not stored
    const __amdgpu_buffer_rsrc_t re = make_rsrc(En + row0, ((int64_t)nk * d_out - row0) * 4);
    // U: instruction q of wave w moves k-rows 16w + 2q (lanes 0-31) and +1
    // (lanes 32-63), slot lane % 32 of each; E: one instruction per wave,
    // k-rows 16w + lane / 4, 16-byte group lane % 4 of the 16 rows
    int offu[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int r = 16 * wave + 2 * q + (lane >> 5);
        const int g = (lane & 31) ^ (4 * (r & 3));
        offu[q] = (int)((r * d_in + 4 * g) * 4);
    }
    const int offe = (int)(((16 * wave + (lane >> 2)) * d_out + 4 * (lane & 3)) * 4);
    const int nch = (nk + NCH - 1) / NCH;
    auto issue = [&](int c) {
        lds_char *st = (lds_char *)(ring + (c % NSTG) * (NUF + NEF));
        const int su = (int)(c * NCH * d_in * 4), se = (int)(c * NCH * d_out * 4);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (lds_void_t *)(st + (16 * wave + 2 * q) * 128 * 4), 16,
                                                     offu[q] + su, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void_t *)(st + (NUF + 16 * wave * QROWS) * 4), 16, offe + se,
                                                 0, 0, 0);
    };
    issue(0);
    if (nch > 1) issue(1);
    const int jp = 16 * wave, j1 = jp + 64;
    f32x4 acc0, acc1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        acc0[r] = -Wl[(4 * lk + r) * LW + jp + li];
        acc1[r] = -Wl[(4 * lk + r) * LW + j1 + li];
    }
    // this lane's U columns jp + li and j1 + li, swizzled by its k-row's r % 4 = lk
    const int cu0 = 4 * (((jp + li) >> 2) ^ (4 * lk)) + (li & 3);
    const int cu1 = 4 * (((j1 + li) >> 2) ^ (4 * lk)) + (li & 3);
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch)
            wait_vm<NDMA>();   // chunk c landed, chunk c + 1 may be in flight
        else
            wait_vm<0>();
        lds_barrier();         // every wave's part of chunk c, and every wave done with chunk c - 1
        if (c + 2 < nch) issue(c + 2);
        const float *st = ring + (c % NSTG) * (NUF + NEF);
        float ea[16], ub0[16], ub1[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int k = 4 * t + lk;
            ea[t] = st[NUF + k * QROWS + li];
            ub0[t] = st[k * 128 + cu0];
            ub1[t] = st[k * 128 + cu1];
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[t], ub0[t], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[t], ub1[t], acc1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 48, 0);   // every operand read of the chunk
        __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);   // then its MFMAs
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        Wl[(4 * lk + r) * LW + jp + li] = -acc0[r];
        Wl[(4 * lk + r) * LW + j1 + li] = -acc1[r];
    }
}

// lane S of each 16-lane DPP row to the whole row (every lane is written, so
// no old value is needed)
template <int S>
__device__ __forceinline__ float bcast16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + S, 0xF, 0xF, true));
}

// lo = -z and hi = maxq - z bound the code relative to the zero point:
// clamp(rint(t) + z, 0, maxq) - z == clamp(rint(t), -z, maxq - z) exactly (z is
// an integer), which keeps the add and subtract of z off the column chain.
struct Quantizer {
    float s, inv_s, z, lo, hi;
};

__device__ __forceinline__ Quantizer make_quantizer(float xmin, float xmax, float maxq) {
    xmin = fminf(xmin, 0.f);
    xmax = fmaxf(xmax, 0.f);
    if (xmax == xmin) xmax = 1.f;       // all-zero group
    Quantizer Q;
    Q.s = (xmax - xmin) / maxq;
    Q.z = rintf(-xmin / Q.s);
    Q.inv_s = 1.f / Q.s;
    Q.lo = -Q.z;
    Q.hi = maxq - Q.z;
    return Q;
}

__device__ __forceinline__ Quantizer reuse_quantizer(float s, float z, float maxq) {
    Quantizer Q;
    Q.s = s;
    Q.inv_s = 1.f / s;
    Q.z = z;
    Q.lo = -z;
    Q.hi = maxq - z;
    return Q;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// min and max over the 16 lanes of a DPP row, in every lane: rotations by 8
// and 4 within the row, then swaps of lane pairs 2 and 1 apart in each quad
__device__ __forceinline__ void minmax16(float &mn, float &mx) {
    mn = fminf(mn, dpp_f<0x128>(mn));
    mx = fmaxf(mx, dpp_f<0x128>(mx));
    mn = fminf(mn, dpp_f<0x124>(mn));
    mx = fmaxf(mx, dpp_f<0x124>(mx));
    mn = fminf(mn, dpp_f<0x4E>(mn));
    mx = fmaxf(mx, dpp_f<0x4E>(mx));
    mn = fminf(mn, dpp_f<0xB1>(mn));
    mx = fmaxf(mx, dpp_f<0xB1>(mx));
}

// Column S of the chunk (i = c0 + S): every lane of the row quantizes the
// broadcast value x and applies the error to its own column c:
//   w_c -= E U_{i,c} = w_c - x U_{i,c}/U_ii + r s U_{i,c}/U_ii
// with uu[S] = U_{i,c}/U_ii and sv[S] = s U_{i,c}/U_ii (both 0 for c <= S),
// so that only the code (round, clamp) and one fma stay on the chain from
// one column to the next.  Lane S's own value is never changed again from
// step S on (its coefficients are zero there), so its code and error are
// taken from its final value after the chunk, off the chain.
template <int S, bool RAGGED>
__device__ __forceinline__ void qstep(float &w, int c0, int nb, const Quantizer &Q, const float (&uu)[CH],
                                      const float (&sv)[CH]) {
    if (RAGGED && c0 + S >= nb) return;       // uniform: ragged last chunk
    const float x = bcast16<S>(w);
    const float r = __builtin_amdgcn_fmed3f(rintf(x * Q.inv_s), Q.lo, Q.hi);   // code - z
    const float t = fmaf(-x, uu[S], w);
    w = fmaf(r, sv[S], t);
}

template <bool RAGGED, int... S>
__device__ __forceinline__ void run_chunk(float &w, int c0, int nb, const Quantizer &Q, const float (&uu)[CH],
                                          const float (&sv)[CH], std::integer_sequence<int, S...>) {
    (qstep<S, RAGGED>(w, c0, nb, Q, uu, sv), ...);
}

// u[S] = U_{c0+S, c0+c} for c > S and 0 for c <= S (the packed block holds
// zeros on and below the diagonal, and max(c, S) reads the diagonal), and
// ui[S] = 1/U_{c0+S, c0+S}, for the 16 rows of chunk c0.  c0 and Bp are
// multiples of 16, so rows c0..c0+15 all exist (past nb they hold zeros) and
// max(c, S) stays inside row c0+S's packed range, which starts at column
// c0 + 4 floor(S/4).
__device__ __forceinline__ void load_coef(const float *Ul, const float *uil, int c0, int Bp, int cl, float (&u)[CH],
                                          float (&ui)[CH]) {
#pragma unroll
    for (int q = 0; q < CH / 4; ++q) {
        const f32x4 x = *(const f32x4 *)(uil + c0 + 4 * q);
        ui[4 * q + 0] = x.x;
        ui[4 * q + 1] = x.y;
        ui[4 * q + 2] = x.z;
        ui[4 * q + 3] = x.w;
    }
    // row c0 + S of the packed block starts at column c0 + 4 floor(S/4) and
    // holds Bp - c0 - 4 floor(S/4) values: walk the row starts by adding
    // lengths (uniform) instead of evaluating the packed offset per row
    int start = uoff(c0, Bp);
#pragma unroll
    for (int S = 0; S < CH; ++S) {
        const int q4 = 4 * (S >> 2);
        u[S] = Ul[start + max(cl, S) - q4];
        start += Bp - c0 - q4;
    }
}

// Block [b, e) for this group's 16 rows.  a.E is the block's error slot and
// a.near_k the pending columns before b.  Q carries a group's parameters
// from one block to the next; first: b is the launch's first block (a group
// that began before it has its parameters read back from scales/zeros).
__device__ __forceinline__ void quant_one_block(const QuantArgs &a, int b, int e, Quantizer &Q, bool first) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int nb = e - b;
    const int Bp = roundup16(nb);
    const int LW = Bp + 4;                 // W tile row stride (floats)
    float *Wl = lds;                       // [16][LW]
    float *Ul = lds + QROWS * LW;          // packed upper U block
    float *uil = Ul + usize(Bp);           // 1/U_kk of the block
    int *rbl = (int *)(uil + Bp);          // rbl[i] + j = packed index of U_ij (for the MFMA lanes)
    float *El = (float *)(rbl + Bp);       // the chunk's errors [16 rows][ELD]
    const int tid = threadIdx.x;
    const int rl = tid >> 4, c = tid & 15;
    const int64_t row0 = (int64_t)blockIdx.x * QROWS;
    const int64_t row = row0 + rl;
    const bool row_ok = row < a.d_out;
    const int64_t d_in = a.d_in, d_out = a.d_out;

    // Stage the W tile, the packed upper part of the U block and 1/U_kk.
    // Only the strict upper part of U is ever read (1/U_kk comes from uil);
    // row i's packed range starts at column 4 floor(i/4), zeros on and below
    // the diagonal.  full: every 4-column group of the block is 4 valid,
    // 16-byte aligned columns.  Then all of a thread's 16-byte loads are
    // issued before any is stored (U comes from HBM and one latency per block
    // is the goal), each from an address clamped into range and zeroed
    // afterwards, so that they carry no branches.  Thread mapping without
    // divisions: lane & 31 picks the 4-column group (plus 32 per half for
    // blocks wider than 128 columns), tid >> 5 plus 8q the row.  Otherwise
    // (unaligned shapes) one element at a time on its own bounds.
    const bool full = (d_in % 4 == 0) && (b % 4 == 0) && (nb % 4 == 0);
    const int G = Bp / 4;                  // 4-column groups per row (<= 64)
    const int jg0 = tid & 31, ri = tid >> 5;
    auto store_u = [&](int i, int jg, f32x4 x) {
        const int j = 4 * jg;
        if (i < Bp && jg < G && j >= 4 * (i >> 2)) {
            x.x = (j + 0 > i) ? x.x : 0.f;
            x.y = (j + 1 > i) ? x.y : 0.f;
            x.z = (j + 2 > i) ? x.z : 0.f;
            x.w = (j + 3 > i) ? x.w : 0.f;
            *(f32x4 *)(Ul + uidx(i, j, Bp)) = x;
        }
    };
    auto stage_full = [&](auto nh_c) {
        constexpr int NH = decltype(nh_c)::value;        // 32-group halves: 1 up to 128 columns, else 2
        // rows and columns past the block (or past d_out) are read from a
        // clamped, in-range address and zeroed when stored; 32-bit element
        // offsets from a per-block base keep the address arithmetic short
        const int di = (int)d_in, nbq = nb / 4;
        const int rows_here = (int)std::min<int64_t>(QROWS, d_out - row0);
        const float *wb = a.Wp + row0 * d_in + b;
        const float *ub = a.U + (int64_t)b * d_in + b;
        f32x4 wv[NH][2], uv[NH][16];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int jc = 4 * min(jg0 + 32 * hh, nbq - 1);
                wv[hh][q] = *(const f32x4 *)(wb + (unsigned)(min(ri + 8 * q, rows_here - 1) * di + jc));
            }
        // U block rows 0..127 (rows 128..255 of a wider block in a second pass)
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int jc = 4 * min(jg0 + 32 * hh, nbq - 1);
                uv[hh][q] = *(const f32x4 *)(ub + (unsigned)(min(ri + 8 * q, nb - 1) * di + jc));
            }
        const float uiv0 = a.uinv[b + min(tid, nb - 1)];   // Bp <= 256: one per thread
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int jg = jg0 + 32 * hh, r = ri + 8 * q;
                if (jg < G) *(f32x4 *)(Wl + r * LW + 4 * jg) = (r < rows_here && jg < nbq) ? wv[hh][q] : z;
            }
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int jg = jg0 + 32 * hh, i = ri + 8 * q;
                store_u(i, jg, (i < nb && jg < nbq) ? uv[hh][q] : z);
            }
        if (tid < Bp) uil[tid] = (tid < nb) ? uiv0 : 0.f;
        if (NH > 1) {
            // rows 128..Bp-1 (only their columns >= 128 are in the packed range)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int jc = 4 * min(jg0 + 32, nbq - 1);
                uv[0][q] = *(const f32x4 *)(ub + (unsigned)(min(128 + ri + 8 * q, nb - 1) * di + jc));
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int jg = jg0 + 32, i = 128 + ri + 8 * q;
                store_u(i, jg, (i < nb && jg < nbq) ? uv[0][q] : z);
            }
        }
    };
    if (full) {
        if (G <= 32)
            stage_full(std::integral_constant<int, 1>{});
        else
            stage_full(std::integral_constant<int, 2>{});
    } else {
        for (int it = tid; it < QROWS * G; it += 256) {
            const int r = it / G, j = 4 * (it % G);
            const int64_t gr = row0 + r;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (gr < d_out) {
                const float *p = a.Wp + gr * d_in + b + j;
                if (j + 0 < nb) v.x = p[0];
                if (j + 1 < nb) v.y = p[1];
                if (j + 2 < nb) v.z = p[2];
                if (j + 3 < nb) v.w = p[3];
            }
            *(f32x4 *)(Wl + r * LW + j) = v;
        }
        for (int it = tid; it < Bp * G; it += 256) {
            const int i = it / G, jg = it % G, j = 4 * jg;
            if (j < 4 * (i >> 2)) continue;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (i < nb) {
                const float *p = a.U + (int64_t)(b + i) * d_in + b + j;
                if (j + 0 < nb && j + 0 > i) v.x = p[0];
                if (j + 1 < nb && j + 1 > i) v.y = p[1];
                if (j + 2 < nb && j + 2 > i) v.z = p[2];
                if (j + 3 < nb && j + 3 > i) v.w = p[3];
            }
            store_u(i, jg, v);
        }
        if (tid < Bp) uil[tid] = (tid < nb) ? a.uinv[b + tid] : 0.f;
    }
    if (tid < Bp) rbl[tid] = uidx(tid, 0, Bp);
    __syncthreads();

    const bool near_fast = nb == 128 && a.ring_ok && d_in % 4 == 0 && d_out % 4 == 0 && b % 4 == 0 &&
                           a.near_k * std::max(d_in, d_out) * 4 + (int64_t)NSTG * NCH * std::max(d_in, d_out) * 4 <
                               ((int64_t)1 << 31);
    if (a.near_k > 0 && near_fast) {
        float *ring = El + ((QROWS * ELD + 3) & ~3);   // 16-byte aligned after the error tile
        near_update_ring(Wl, LW, ring, a.U + a.near_row0 * d_in + b, a.En, row0, d_in, d_out, a.near_k);
        __syncthreads();
    } else if (a.near_k > 0) {
        // The pending blocks' errors on this block's columns:
        //   W[16 rows][j] -= sum_{k < near_k} En[k][row] U[near_row0 + k][b + j]
        // as 16 x 16 tiles on v_mfma_f32_16x16x4_f32 (A[i][k] at lane i + 16k,
        // B[k][j] at lane j + 16k, D[i][j] at lane 16 (i/4) + j, register
        // i % 4).  Wave w takes column tiles w, w + 4, w + 8 and w + 12 (those
        // inside the block), all four accumulated over one pass of k, so each
        // error value is loaded once; k goes in batches of 32 whose operand
        // loads (from L2) go out one batch ahead of the products.
        const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;
        // every load reads an address clamped into range and the value is
        // zeroed afterwards, so that the loads carry no branches and go out
        // together
        const int64_t ra = row0 + li;
        const bool ra_ok = ra < d_out;
        const float *ep = a.En + (ra_ok ? ra : d_out - 1);              // En[k][ra]
        const float *up = a.U + a.near_row0 * d_in + b;                 // U[near_row0 + k][b + j]
        const int nk = a.near_k;
        constexpr int NT = 4, KB = 32, KT = KB / 4;
        int cc[NT];
        bool c_ok[NT], t_on[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int jt = 16 * wave + 64 * t;
            t_on[t] = jt < nb;
            c_ok[t] = jt + li < nb;
            cc[t] = c_ok[t] ? jt + li : nb - 1;
        }
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = t_on[t] ? Wl[(4 * lk + r) * LW + 16 * wave + 64 * t + li] : 0.f;
        float ea[KT], ub[NT][KT];
        auto load = [&](int k0, float (&e_)[KT], float (&u_)[NT][KT]) {
#pragma unroll
            for (int q = 0; q < KT; ++q) {
                const int k = k0 + 4 * q + lk;
                const int64_t kc = k < nk ? k : nk - 1;
                e_[q] = ep[kc * d_out];
#pragma unroll
                for (int t = 0; t < NT; ++t) u_[t][q] = up[kc * d_in + cc[t]];
            }
        };
        load(0, ea, ub);
        for (int k0 = 0; k0 < nk; k0 += KB) {
            float en[KT], un[NT][KT];
            if (k0 + KB < nk) load(k0 + KB, en, un);
            // zero what lies past the matrix, after the loads are in flight
#pragma unroll
            for (int q = 0; q < KT; ++q) {
                const bool k_ok = k0 + 4 * q + lk < nk;
                ea[q] = (k_ok && ra_ok) ? -ea[q] : 0.f;
#pragma unroll
                for (int t = 0; t < NT; ++t) ub[t][q] = (k_ok && c_ok[t]) ? ub[t][q] : 0.f;
            }
#pragma unroll
            for (int q = 0; q < KT; ++q)
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[q], ub[t][q], acc[t], 0, 0, 0);
#pragma unroll
            for (int q = 0; q < KT; ++q) {
                ea[q] = en[q];
#pragma unroll
                for (int t = 0; t < NT; ++t) ub[t][q] = un[t][q];
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (t_on[t])
#pragma unroll
                for (int r = 0; r < 4; ++r) Wl[(4 * lk + r) * LW + 16 * wave + 64 * t + li] = acc[t][r];
        __syncthreads();
    }

    const float maxq = (float)((1 << a.bits) - 1);
    const int g = a.group;
    if (first && b % g != 0) {
        // the current group began in an earlier block: reuse its parameters
        const int64_t gi = b / g;
        Q = reuse_quantizer(row_ok ? a.scales[gi * d_out + row] : 1.f, row_ok ? a.zeros[gi * d_out + row] : 0.f,
                            maxq);
    }

    const int cl = c;
    // the first chunk's coefficients; later chunks' are read one chunk ahead
    float u[CH], ui[CH];
    load_coef(Ul, uil, 0, Bp, cl, u, ui);
    for (int c0 = 0; c0 < nb; c0 += CH) {
        const int k = b + c0;
        if (k % g == 0) {
            // group start: parameters from the current values of the group's columns
            float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
            if (c0 + std::min<int64_t>(g, d_in - k) > nb) {
                // the group reaches past this block: its columns from W
                const int gl = (int)std::min<int64_t>(g, d_in - k);
                if (row_ok)
                    for (int j = c; j < gl; j += CH) {
                        const float v = a.Wp[row * d_in + k + j];
                        mn = fminf(mn, v);
                        mx = fmaxf(mx, v);
                    }
            } else {
                // the group's columns from the staged tile, all reads in
                // flight together: lanes past the group's end reread its last
                // column, which leaves min and max unchanged
                const int gl = std::min(g, nb - c0);
                const float *wr = Wl + rl * LW + c0;
                if (gl <= 8 * CH) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float v = wr[min(c + CH * q, gl - 1)];
                        mn = fminf(mn, v);
                        mx = fmaxf(mx, v);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const float v = wr[min(c + CH * q, gl - 1)];
                        mn = fminf(mn, v);
                        mx = fmaxf(mx, v);
                    }
                }
            }
            minmax16(mn, mx);
            if (!row_ok) mn = mx = 0.f;
            Q = make_quantizer(mn, mx, maxq);
            if (row_ok && c == 0) {
                const int64_t gi = k / g;
                a.scales[gi * d_out + row] = Q.s;
                a.zeros[gi * d_out + row] = Q.z;
            }
        }
        float w = Wl[rl * LW + c0 + c];
        const float uic = uil[c0 + c];         // 1/U_kk of this lane's column
        // U_kc / U_kk and s U_kc / U_kk for the chunk's steps (the group's
        // parameters are fixed within a chunk)
        float uu[CH], sv[CH];
#pragma unroll
        for (int S = 0; S < CH; ++S) {
            uu[S] = u[S] * ui[S];
            sv[S] = uu[S] * Q.s;
        }
        // the next chunk's coefficients: their LDS reads go out after this
        // chunk's own (LDS reads return in order) and are in flight during
        // this chunk's steps.  Unconditional (the last chunk rereads its
        // own), so that the waits before the steps count exactly.
        __builtin_amdgcn_sched_barrier(0);
        load_coef(Ul, uil, (c0 + CH < nb) ? c0 + CH : c0, Bp, cl, u, ui);
        __builtin_amdgcn_sched_barrier(0);
        if (c0 + CH <= nb)
            run_chunk<false>(w, c0, nb, Q, uu, sv, std::make_integer_sequence<int, CH>{});
        else
            run_chunk<true>(w, c0, nb, Q, uu, sv, std::make_integer_sequence<int, CH>{});
        // this lane's column: code and error, (w - s (q - z)) / U_kk
        const float rq = __builtin_amdgcn_fmed3f(rintf(w * Q.inv_s), Q.lo, Q.hi);
        const float myq = rq + Q.z;
        const float myE = fmaf(-Q.s, rq, w) * uic;
        if (row_ok && c0 + c < nb) {
            a.codes[(int64_t)(k + c) * d_out + row] = (uint8_t)myq;
            a.E[(int64_t)(c0 + c) * d_out + row] = myE;
        }
        // apply this chunk's errors to the rest of the block:
        // W[16 rows, j] -= E[16 rows][16] U[c0 .. c0+15][j] for j >= c0 + 16
        El[rl * ELD + c] = myE;
        __syncthreads();
        {
            const int wave = tid >> 6, lane = tid & 63;
            const int li = lane & 15, lk = lane >> 4;
            // A[i][k] = -E[i][4t + k] at lane i + 16 k
            float ea[4];
            int rbk[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ea[t] = -El[li * ELD + 4 * t + lk];
                rbk[t] = rbl[c0 + 4 * t + lk];
            }
            for (int j0 = c0 + CH * (1 + wave); j0 < nb; j0 += 4 * CH) {
                // D[i][j] at lane 16 (i / 4) + j, register i % 4
                f32x4 acc;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = Wl[(4 * lk + r) * LW + j0 + li];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // B[k][j] = U[c0 + 4t + k][j0 + j] at lane j + 16 k
                    const float ub = Ul[rbk[t] + j0 + li];
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[t], ub, acc, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) Wl[(4 * lk + r) * LW + j0 + li] = acc[r];
            }
        }
        __syncthreads();
    }
}

// One launch takes nblocks blocks of width B from b0 (the blocks between two
// far updates): each group takes its 16 rows through all of them.  Nothing
// crosses groups within a batch (a block's near update uses this group's own
// earlier errors), so the blocks need no grid-wide synchronization, and a
// grid larger than the CUs simply runs in several rounds of whole batches.
// (One launch per block instead, with its own rounds, was slower where the
// grid exceeds the CUs: up_proj's in-block stage 2.22 -> 2.05 ms batched.)
// a.E / a.En: the batch's error slots ([k][d_out], block t at rows t*B);
// a.near_row0: the batch's first column.
// Grid: ceil(d_out / 16) groups of 256 threads.
__global__ __launch_bounds__(256) void quant_block_kernel(QuantArgs a, int b0, int nblocks, int B) {
    Quantizer Q = reuse_quantizer(1.f, 0.f, (float)((1 << a.bits) - 1));
    for (int t = 0; t < nblocks; ++t) {
        QuantArgs ab = a;
        const int b = b0 + t * B;
        const int e = (int)std::min<int64_t>(b + B, ab.d_in);
        ab.E = ab.E + (int64_t)(b - ab.near_row0) * ab.d_out;
        ab.near_k = b - (int)ab.near_row0;
        quant_one_block(ab, b, e, Q, t == 0);
        __syncthreads();   // the next block restages the LDS
    }
}

}  // namespace

size_t quant_lds_bytes(int block) {
    const int Bp = roundup16(block);
    const size_t base = (size_t)QROWS * (Bp + 4) + (size_t)usize(Bp) + 2 * (size_t)Bp + (size_t)((QROWS * ELD + 3) & ~3);
    // blocks of 128 columns take the near update through the LDS ring
    return sizeof(float) * (base + (block == 128 ? (size_t)NRING : 0));
}

// LDS of a launch over blocks of width B from b0 (nblocks of them): every
// block but the last is B wide, the last may be narrower.  A 128-wide last
// block after wider ones needs the near-update ring, which can take more
// than the first block's staging (154944 bytes against 152896 at B = 256),
// so the launch takes the larger of the two.
static size_t quant_launch_lds(int64_t d_in, int64_t b0, int nblocks, int64_t B) {
    const int w_first = (int)std::min<int64_t>(B, d_in - b0);
    const int w_last = (int)std::min<int64_t>(B, d_in - (b0 + (int64_t)(nblocks - 1) * B));
    return std::max(quant_lds_bytes(w_first), quant_lds_bytes(w_last));
}

hipError_t quant_block_launch(const QuantArgs &a, int64_t b0, int nblocks, int64_t B, hipStream_t st) {
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t err = hipFuncSetAttribute((const void *)quant_block_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err != hipSuccess) return err;
        attr_done = true;
    }
    if (B < 1 || B > 256 || nblocks < 1 || b0 + (nblocks - 1) * B >= a.d_in || b0 < a.near_row0)
        return hipErrorInvalidValue;   // the kernel stages at most 256 columns per block
    const unsigned grid = (unsigned)cdiv(a.d_out, QROWS);
    // ring_ok: the allocation holds the near-update ring after a 128-wide
    // block's staging (the kernel takes the ring only then)
    const size_t ring_need = quant_lds_bytes(128);
    const size_t lds = quant_launch_lds(a.d_in, b0, nblocks, B);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    QuantArgs ar = a;
    ar.ring_ok = lds >= ring_need;
    quant_block_kernel<<<grid, 256, lds, st>>>(ar, (int)b0, nblocks, (int)B);
    return hipGetLastError();
}

}  // namespace gptq
