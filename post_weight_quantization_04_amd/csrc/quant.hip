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
// (v_mfma_f32_16x16x4_f32), the four waves taking every fourth tile.
#include "common.h"

#include <algorithm>
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

template <int S>
__device__ __forceinline__ float bcast16(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + S, 0xF, 0xF, false));
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

struct StepCtx {
    int c0, c, nb;
};

// Column S of the chunk: every lane of the row quantizes the broadcast value
// x and applies the error to its own column c:
//   w_c -= E U_{i,c} = w_c - x U_{i,c}/U_ii + r s U_{i,c}/U_ii
// with uu[S] = U_{i,c}/U_ii and sv[S] = s U_{i,c}/U_ii (both 0 for c <= S),
// so that only the code (round, clamp) and one fma stay on the chain from
// one column to the next.  The error itself, (x - s r)/U_ii, is only output.
template <int S, bool RAGGED>
__device__ __forceinline__ void qstep(float &w, float &myq, float &myE, const StepCtx &cx, const Quantizer &Q,
                                      const float (&uu)[CH], const float (&sv)[CH], const float (&ui)[CH],
                                      const float (&su)[CH]) {
    if (RAGGED && cx.c0 + S >= cx.nb) return;       // uniform: ragged last chunk
    const float x = bcast16<S>(w);
    const float r = __builtin_amdgcn_fmed3f(rintf(x * Q.inv_s), Q.lo, Q.hi);   // code - z
    const float t = fmaf(-x, uu[S], w);
    const float err = fmaf(-su[S], r, x * ui[S]);                              // (w - s (q - z)) / U_kk
    myq = (cx.c == S) ? r + Q.z : myq;
    myE = (cx.c == S) ? err : myE;
    w = fmaf(r, sv[S], t);
}

template <bool RAGGED, int... S>
__device__ __forceinline__ void run_chunk(float &w, float &myq, float &myE, const StepCtx &cx, const Quantizer &Q,
                                          const float (&uu)[CH], const float (&sv)[CH], const float (&ui)[CH],
                                          const float (&su)[CH], std::integer_sequence<int, S...>) {
    (qstep<S, RAGGED>(w, myq, myE, cx, Q, uu, sv, ui, su), ...);
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
    int *rbl = (int *)(uil + Bp);          // rbl[i] + j = packed index of U_ij
    float *El = (float *)(rbl + Bp);       // the chunk's errors [16 rows][ELD]
    const int tid = threadIdx.x;
    const int rl = tid >> 4, c = tid & 15;
    const int64_t row0 = (int64_t)blockIdx.x * QROWS;
    const int64_t row = row0 + rl;
    const bool row_ok = row < a.d_out;
    const int64_t d_in = a.d_in, d_out = a.d_out;

    // Stage the W tile, the packed upper part of the U block and 1/U_kk with
    // 16-byte loads (4-column groups), all of a thread's loads issued before
    // any is stored: U comes from HBM and one latency per block is the goal.
    // Thread mapping without divisions: lane & 31 picks the 4-column group
    // (plus 32 per half for blocks wider than 128 columns), tid >> 5 plus 8q
    // the row.  full: every group of the block is 4 valid, 16-byte aligned
    // columns, so no load needs a per-column bound.
    const bool full = (d_in % 4 == 0) && (b % 4 == 0) && (nb % 4 == 0);
    auto load4 = [&](const float *p, int nvalid) -> f32x4 {
        if (full) return *(const f32x4 *)p;
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (nvalid > 0) v.x = p[0];
        if (nvalid > 1) v.y = p[1];
        if (nvalid > 2) v.z = p[2];
        if (nvalid > 3) v.w = p[3];
        return v;
    };
    const int G = Bp / 4;                  // 4-column groups per row (<= 64)
    const int jg0 = tid & 31, ri = tid >> 5;
    {
        const int nhalf = (G + 31) / 32;   // 1 or 2
        f32x4 wv[2][2], uv[2][16];
        // W tile: 16 rows
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int jg = jg0 + 32 * hh, r = ri + 8 * q, j = 4 * jg;
                const int64_t gr = row0 + r;
                wv[hh][q] = (hh < nhalf && jg < G && gr < d_out && j < nb) ? load4(a.Wp + gr * d_in + b + j, nb - j)
                                                                          : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        // U block rows 0..127 (rows 128..255 of a wider block in a second pass)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int jg = jg0 + 32 * hh, i = ri + 8 * q, j = 4 * jg;
                uv[hh][q] = (hh < nhalf && jg < G && i < nb && j + 3 > i && j < nb)
                                ? load4(a.U + (int64_t)(b + i) * d_in + b + j, nb - j)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        const float uiv = (tid < nb) ? a.uinv[b + tid] : 0.f;   // Bp <= 256: one per thread
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int jg = jg0 + 32 * hh, r = ri + 8 * q;
                if (hh < nhalf && jg < G) *(f32x4 *)(Wl + r * LW + 4 * jg) = wv[hh][q];
            }
        // only the strict upper part of U is ever read (1/U_kk comes from uil);
        // row i's packed range starts at column 4 floor(i/4)
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
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (hh < nhalf) store_u(ri + 8 * q, jg0 + 32 * hh, uv[hh][q]);
        if (tid < Bp) {
            uil[tid] = uiv;
            rbl[tid] = uidx(tid, 0, Bp);
        }
        if (Bp > 128) {
            // rows 128..Bp-1 (only their columns >= 128 are in the packed range)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int jg = jg0 + 32, i = 128 + ri + 8 * q, j = 4 * jg;
                uv[0][q] = (jg < G && i < nb && j + 3 > i && j < nb)
                               ? load4(a.U + (int64_t)(b + i) * d_in + b + j, nb - j)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int q = 0; q < 16; ++q) store_u(128 + ri + 8 * q, jg0 + 32, uv[0][q]);
        }
    }
    __syncthreads();

    if (a.near_k > 0) {
        // The pending blocks' errors on this block's columns:
        //   W[16 rows][j] -= sum_{k < near_k} En[k][row] U[near_row0 + k][b + j]
        // as 16 x 16 tiles on v_mfma_f32_16x16x4_f32 (A[i][k] at lane i + 16k,
        // B[k][j] at lane j + 16k, D[i][j] at lane 16 (i/4) + j, register
        // i % 4).  Wave w takes column tiles w and w + 4 (then w + 8, w + 12
        // for blocks past 128 columns); k goes in batches of 64 whose
        // operand loads (from L2) are all issued before their products.
        const int wave = tid >> 6, lane = tid & 63, li = lane & 15, lk = lane >> 4;
        // every load reads an address clamped into range and the value is
        // zeroed afterwards, so that the loads carry no branches and go out
        // together
        const int64_t ra = row0 + li;
        const bool ra_ok = ra < d_out;
        const float *ep = a.En + (ra_ok ? ra : d_out - 1);              // En[k][ra]
        const float *up = a.U + a.near_row0 * d_in + b;                 // U[near_row0 + k][b + j]
        const int nk = a.near_k;
        for (int jp = 16 * wave; jp < nb; jp += 128) {
            const int j1 = jp + 64;                                     // second tile of the pair
            const bool c0_ok = jp + li < nb, c1_ok = j1 + li < nb;
            const int cc0 = c0_ok ? jp + li : nb - 1, cc1 = c1_ok ? j1 + li : nb - 1;
            for (int k0 = 0; k0 < nk; k0 += 64) {
                float ea[16], ub0[16], ub1[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const int k = k0 + 4 * t + lk;
                    const bool k_ok = k < nk;
                    const int64_t kc = k_ok ? k : nk - 1;
                    const float e = ep[kc * d_out];
                    const float u0 = up[kc * d_in + cc0];
                    const float u1 = up[kc * d_in + cc1];
                    ea[t] = (k_ok && ra_ok) ? -e : 0.f;
                    ub0[t] = (k_ok && c0_ok) ? u0 : 0.f;
                    ub1[t] = (k_ok && c1_ok) ? u1 : 0.f;
                }
                f32x4 acc0, acc1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    acc0[r] = Wl[(4 * lk + r) * LW + jp + li];
                    acc1[r] = (j1 < Bp) ? Wl[(4 * lk + r) * LW + j1 + li] : 0.f;
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[t], ub0[t], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[t], ub1[t], acc1, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Wl[(4 * lk + r) * LW + jp + li] = acc0[r];
                    if (j1 < Bp) Wl[(4 * lk + r) * LW + j1 + li] = acc1[r];
                }
            }
        }
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
                const int gl = std::min(g, nb - c0);
                for (int j = c; j < gl; j += CH) {
                    const float v = Wl[rl * LW + c0 + j];
                    mn = fminf(mn, v);
                    mx = fmaxf(mx, v);
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
        float myq = 0.f, myE = 0.f;
        // this chunk's coefficients in registers, off the dependency chain:
        // u[S] = U_{c0+S, c0+c} for c > S (0 otherwise), ui[S] = 1/U_{c0+S, c0+S}
        float u[CH], ui[CH];
        // the lane's column, opaque to the optimizer: keeps the per-step lane
        // masks from being hoisted out of the chunk loop (scalar spills)
        int cl;
        asm volatile("v_mov_b32 %0, %1" : "=v"(cl) : "v"(c));
        {
            // c0 is a multiple of 16 and Bp of 16: rows c0..c0+15 all exist in
            // LDS (past nb they hold zeros); max(cl, S) stays inside row
            // c0+S's packed range, which starts at column c0 + 4 floor(S/4)
            int rb[CH];
#pragma unroll
            for (int q = 0; q < CH / 4; ++q) {
                const f32x4 x = *(const f32x4 *)(uil + c0 + 4 * q);
                ui[4 * q + 0] = x.x;
                ui[4 * q + 1] = x.y;
                ui[4 * q + 2] = x.z;
                ui[4 * q + 3] = x.w;
                const i32x4 y = *(const i32x4 *)(rbl + c0 + 4 * q);
                rb[4 * q + 0] = y.x;
                rb[4 * q + 1] = y.y;
                rb[4 * q + 2] = y.z;
                rb[4 * q + 3] = y.w;
            }
#pragma unroll
            for (int S = 0; S < CH; ++S) {
                const float x = Ul[rb[S] + c0 + max(cl, S)];
                u[S] = (cl > S) ? x : 0.f;
            }
        }
        // s / U_kk, U_kc / U_kk and s U_kc / U_kk (the group's parameters are
        // fixed within a chunk)
        float su[CH], uu[CH], sv[CH];
#pragma unroll
        for (int S = 0; S < CH; ++S) {
            su[S] = Q.s * ui[S];
            uu[S] = u[S] * ui[S];
            sv[S] = u[S] * su[S];
        }
        StepCtx cx{c0, cl, nb};
        if (c0 + CH <= nb)
            run_chunk<false>(w, myq, myE, cx, Q, uu, sv, ui, su, std::make_integer_sequence<int, CH>{});
        else
            run_chunk<true>(w, myq, myE, cx, Q, uu, sv, ui, su, std::make_integer_sequence<int, CH>{});
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

// BATCH: one launch takes nblocks blocks of width B from b0 (the blocks
// between two far updates): each group takes its 16 rows through all of them.
// Nothing crosses groups within a batch (a block's near update uses this
// group's own earlier errors), so the blocks need no grid-wide
// synchronization.  The loop keeps the kernel's arguments live across the
// whole body (≈ 340 VGPRs, one group per SIMD set), so it is used when the grid
// fits in one group per CU; otherwise one launch per block (nblocks = 1).
// a.E / a.En: the batch's error slots ([k][d_out], block t at rows t*B);
// a.near_row0: the batch's first column.
// Grid: ceil(d_out / 16) groups of 256 threads.
template <bool BATCH>
__global__ __launch_bounds__(256) void quant_block_kernel(QuantArgs a, int b0, int nblocks, int B) {
    Quantizer Q = reuse_quantizer(1.f, 0.f, (float)((1 << a.bits) - 1));
    for (int t = 0; t < (BATCH ? nblocks : 1); ++t) {
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
    return sizeof(float) * ((size_t)QROWS * (Bp + 4) + (size_t)usize(Bp) + 2 * (size_t)Bp + (size_t)QROWS * ELD);
}

int quant_cu_count() {
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

hipError_t quant_block_launch(const QuantArgs &a, int64_t b0, int nblocks, int64_t B, hipStream_t st) {
    static bool attr_done = false;
    if (!attr_done) {
        hipError_t err = hipFuncSetAttribute((const void *)quant_block_kernel<true>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err == hipSuccess)
            err = hipFuncSetAttribute((const void *)quant_block_kernel<false>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (err != hipSuccess) return err;
        attr_done = true;
    }
    if (B < 1 || B > 256 || nblocks < 1 || b0 + (nblocks - 1) * B >= a.d_in || b0 < a.near_row0)
        return hipErrorInvalidValue;   // the kernel stages at most 256 columns per block
    const size_t lds = quant_lds_bytes((int)std::min<int64_t>(B, a.d_in - b0));   // the widest block is the first
    const unsigned grid = (unsigned)cdiv(a.d_out, QROWS);
    if ((int64_t)grid <= quant_cu_count()) {
        quant_block_kernel<true><<<grid, 256, lds, st>>>(a, (int)b0, nblocks, (int)B);
        return hipGetLastError();
    }
    for (int t = 0; t < nblocks; ++t) {
        quant_block_kernel<false><<<grid, 256, lds, st>>>(a, (int)(b0 + t * B), 1, (int)B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gptq
