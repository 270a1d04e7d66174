// Products with a GPTQ-packed layer: Y = A W_hat^T, the weights dequantized
// on the fly.  "Optimization Gptq", "Backends de kernel" (kernels that run
// the quantized model on its 4-bit weights) and "GPTQ (GPT Quantization)",
// "Limitations" (weights are dequantized for each product).
//
// Storage (as the quantizer writes it): codes in processing order as a
// little-endian bit stream per row, word-major Qpacked [words][d_out];
// scales and zeros [groups][d_out]; W_hat[r][perm[k]] = s[k/g][r] (q - z).
// With A_p[i][k] = A[i][perm[k]] (activations moved into processing order),
//   Y[i][r] = sum_k A_p[i][k] s[k/g][r] (q[r][k] - z[k/g][r]).
//
// Skinny path (m <= 8 activation rows; decode), bound by reading the packed
// weights once.  A work group owns 256 output rows (four adjacent rows per
// lane, so a packed word row is one contiguous kilobyte read by a wave as
// 16-byte loads) and one of `nsplit` ranges of k; k is cut into 32-code units
// (a unit is `bits` consecutive words of a row) and the group's waves take
// every fourth (or eighth) unit of its range: eight waves for one activation
// row on layers under 16 MB of packed words, whose few work groups would
// otherwise leave half the SIMDs idle, with all of a wave's words in flight.  The group gathers its range of A_p
// into LDS as fp32, with the sum of every 16 consecutive activations.  Codes
// are extracted with constant shifts and multiplied with the broadcast
// activations into a 16-code dot product (two or more bf16 activation rows:
// code pairs as exact bf16 pairs through v_dot2c_f32_bf16), folded as
//   acc += s dot - (s z) sum16(A_p),
// so the group's scale and zero point are applied once per 16 codes and a
// group may end at any multiple of 16.  The units' packed words, scales and
// zero points are loaded a few units ahead, the first ones before the
// activations are staged.  The waves' sums meet in LDS; the k-ranges'
// partial sums go to the workspace, and the last work group of a row tile to
// finish (a device-scope counter per tile, reset by that group) adds them in
// split order and writes Y as fp32 or bf16: deterministic, one launch.  No
// work group ever waits for another.
#include "common.h"

#include <algorithm>

namespace gptq {

namespace {

constexpr int UNIT = 32;          // codes per unit
constexpr int GV_ROWS = 256;      // output rows per work group
constexpr int GV_LDS = 15360;     // staged activations (floats, 60 KB)

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (unsigned)b << 16);
}

// code k (compile-time, 0..31) of a unit held in BITS words
template <int BITS, int K>
__device__ __forceinline__ unsigned unit_code(const unsigned (&w)[BITS]) {
    constexpr int pos = BITS * K, j = pos >> 5, sh = pos & 31;
    constexpr unsigned mask = (1u << BITS) - 1u;
    if constexpr (sh + BITS <= 32) {
        return __builtin_amdgcn_ubfe(w[j], sh, BITS);
    } else {
        return __builtin_amdgcn_alignbit(w[j + 1], w[j], sh) & mask;
    }
}

// dot[j][i] += sum over codes 16H .. 16H+15 of the unit of al[i][k] * code_k
// of row j; each activation is read once and used for the four rows
template <int BITS, int M, int H, int... KK>
__device__ __forceinline__ void half_unit_dot(const u32x4 (&w)[BITS], const float *al, int astride,
                                              float (&dot)[4][M], std::integer_sequence<int, KK...>) {
    auto one = [&](auto kc) {
        constexpr int k = decltype(kc)::value + 16 * H;
        float a[M];
#pragma unroll
        for (int i = 0; i < M; ++i) a[i] = al[i * astride + k];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            unsigned wj[BITS];
#pragma unroll
            for (int b = 0; b < BITS; ++b) wj[b] = w[b][j];
            const float c = (float)unit_code<BITS, k>(wj);
#pragma unroll
            for (int i = 0; i < M; ++i) dot[j][i] = fmaf(a[i], c, dot[j][i]);
        }
    };
    (one(std::integral_constant<int, KK>{}), ...);
}

// The same sums for bf16 activations (staged as bf16 pairs, a2[i][k / 2]):
// codes k, k+1 become an exact bf16 pair and one v_dot2c_f32_bf16 adds both
// products per activation row
typedef __attribute__((ext_vector_type(2))) __bf16 gv_bf16x2;
template <int BITS, int M, int H, int... PP>
__device__ __forceinline__ void half_unit_dot2(const u32x4 (&w)[BITS], const unsigned *a2, int astride2,
                                               float (&dot)[4][M], std::integer_sequence<int, PP...>) {
    auto one = [&](auto pc) {
        constexpr int k = 2 * decltype(pc)::value + 16 * H;
        gv_bf16x2 a[M];
#pragma unroll
        for (int i = 0; i < M; ++i) a[i] = __builtin_bit_cast(gv_bf16x2, a2[i * astride2 + k / 2]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            unsigned wj[BITS];
#pragma unroll
            for (int b = 0; b < BITS; ++b) wj[b] = w[b][j];
            const gv_bf16x2 q = {(__bf16)(float)unit_code<BITS, k>(wj), (__bf16)(float)unit_code<BITS, k + 1>(wj)};
#pragma unroll
            for (int i = 0; i < M; ++i) dot[j][i] = __builtin_amdgcn_fdot2_f32_bf16(a[i], q, dot[j][i], false);
        }
    };
    (one(std::integral_constant<int, PP>{}), ...);
}

// units whose packed words are in flight per lane: about 16 words of
// registers for one activation row in eight-wave groups, 8 otherwise
template <int BITS, int M, int NW>
constexpr int prefetch_units() {
    return (M == 1 && NW == 8) ? (BITS <= 2 ? 6 : (BITS <= 4 ? 16 / BITS : 2))
                               : (BITS <= 2 ? 4 : (BITS <= 4 ? 2 : 1));
}

// D2: bf16 activations summed in pairs by v_dot2c_f32_bf16 (staged as bf16)
template <int BITS, int M, int NW, bool VEC, bool G32, bool D2>
__global__ __launch_bounds__(64 * NW) void dq_gemv_kernel(const void *__restrict__ A, int a_bf16,
                                                      const int32_t *__restrict__ perm,
                                                      const uint32_t *__restrict__ Q,
                                                      const float *__restrict__ scales,
                                                      const float *__restrict__ zeros, void *__restrict__ Y,
                                                      int y_bf16, float *__restrict__ part,
                                                      int32_t *__restrict__ counters, int64_t m_total, int64_t m0,
                                                      int64_t d_in, int64_t d_out, int g, int ngroups, int nunits,
                                                      int nsplit, int64_t nwords) {
    constexpr int PF = prefetch_units<BITS, M, NW>();
    constexpr int NT = 64 * NW;
    __shared__ __attribute__((aligned(16))) float a_lds[GV_LDS];
    __shared__ float hs_lds[GV_LDS / 16];
    __shared__ int last_flag;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int split = blockIdx.y;
    const int u0 = (int)((int64_t)split * nunits / nsplit), u1 = (int)((int64_t)(split + 1) * nunits / nsplit);
    const int nu = u1 - u0;                    // M * nu * 32 <= GV_LDS (host plan)
    const int kw = nu * UNIT;
    const int64_t r0 = (int64_t)blockIdx.x * GV_ROWS + 4 * lane;
    bool rv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rv[j] = r0 + j < d_out;
    const bool any_row = rv[0];

    auto load4 = [&](const uint32_t *base, int64_t off, u32x4 &out) {
        if (VEC) {   // d_out % 4 == 0: the lane's four rows exist together
            out = any_row ? *(const u32x4 *)(base + off + r0) : u32x4{0u, 0u, 0u, 0u};
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) out[j] = rv[j] ? base[off + r0 + j] : 0u;
        }
    };
    auto loadf4 = [&](const float *base, int64_t off, f32x4 &out) {
        if (VEC) {
            out = any_row ? *(const f32x4 *)(base + off + r0) : f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) out[j] = rv[j] ? base[off + r0 + j] : 0.f;
        }
    };
    // a unit's words (zero past the end of the stream), scales and zero
    // points (G32: both halves of every unit lie in one group)
    struct Slot {
        u32x4 w[BITS];
        f32x4 s[G32 ? 1 : 2], z[G32 ? 1 : 2];
    };
    auto fetch = [&](int u, Slot &sl) {
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            const int64_t wi = (int64_t)u * BITS + b;
            if (wi < nwords)
                load4(Q, wi * d_out, sl.w[b]);
            else
                sl.w[b] = u32x4{0u, 0u, 0u, 0u};
        }
        // past d_in (a ragged last unit) the activations are zero; the last
        // group's parameters stand in for the missing ones
#pragma unroll
        for (int h = 0; h < (G32 ? 1 : 2); ++h) {
            const int64_t gi = std::min<int64_t>(((int64_t)u * UNIT + 16 * h) / g, ngroups - 1);
            loadf4(scales, gi * d_out, sl.s[h]);
            loadf4(zeros, gi * d_out, sl.z[h]);
        }
    };

    float acc[4][M];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < M; ++i) acc[j][i] = 0.f;

    // this wave's units of the range: wave, wave + NW, ...
    const int nmy = wave < nu ? (nu - 1 - wave) / NW + 1 : 0;
    Slot sl[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < nmy) fetch(u0 + wave + NW * p, sl[p]);
    // stage A_p for the range (rows past m_total read 0): fp32, or the bf16
    // values themselves for D2
    const int64_t k0 = (int64_t)u0 * UNIT;
    uint16_t *a16 = (uint16_t *)a_lds;
    for (int idx = tid; idx < M * kw; idx += NT) {
        const int i = idx / kw, kk = idx - i * kw;
        const int64_t k = k0 + kk, row = m0 + i;
        if (D2) {
            uint16_t v = 0;
            if (k < d_in && row < m_total) v = ((const uint16_t *)A)[row * d_in + (perm ? (int64_t)perm[k] : k)];
            a16[i * kw + kk] = v;
        } else {
            float v = 0.f;
            if (k < d_in && row < m_total) {
                const int64_t c = perm ? (int64_t)perm[k] : k;
                v = a_bf16 ? bf16_bits_to_f32(((const uint16_t *)A)[row * d_in + c])
                           : ((const float *)A)[row * d_in + c];
            }
            a_lds[i * kw + kk] = v;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < M * 2 * nu; idx += NT) {
        const int i = idx / (2 * nu), h = idx - i * 2 * nu;
        float s = 0.f;
        if (D2) {
            const uint16_t *p = a16 + i * kw + 16 * h;
#pragma unroll
            for (int t = 0; t < 16; ++t) s += bf16_bits_to_f32(p[t]);
        } else {
            const float *p = a_lds + i * kw + 16 * h;
#pragma unroll
            for (int t = 0; t < 16; ++t) s += p[t];
        }
        hs_lds[i * 2 * nu + h] = s;
    }
    __syncthreads();
    for (int i0 = 0; i0 < nmy; i0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int it = i0 + p;
            if (it < nmy) {
                const int ul = wave + NW * it;         // unit within the range
                const float *al = a_lds + ul * UNIT;
                const unsigned *al2 = (const unsigned *)(a16 + ul * UNIT);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float hs[M];
#pragma unroll
                    for (int i = 0; i < M; ++i) hs[i] = hs_lds[i * 2 * nu + 2 * ul + h];
                    float dot[4][M];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int i = 0; i < M; ++i) dot[j][i] = 0.f;
                    if (D2) {
                        if (h == 0)
                            half_unit_dot2<BITS, M, 0>(sl[p].w, al2, kw / 2, dot, std::make_integer_sequence<int, 8>{});
                        else
                            half_unit_dot2<BITS, M, 1>(sl[p].w, al2, kw / 2, dot, std::make_integer_sequence<int, 8>{});
                    } else {
                        if (h == 0)
                            half_unit_dot<BITS, M, 0>(sl[p].w, al, kw, dot, std::make_integer_sequence<int, 16>{});
                        else
                            half_unit_dot<BITS, M, 1>(sl[p].w, al, kw, dot, std::make_integer_sequence<int, 16>{});
                    }
                    const int hh = G32 ? 0 : h;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float sj = sl[p].s[hh][j], szj = sj * sl[p].z[hh][j];
#pragma unroll
                        for (int i = 0; i < M; ++i) acc[j][i] = fmaf(sj, dot[j][i], fmaf(-szj, hs[i], acc[j][i]));
                    }
                }
                if (it + PF < nmy) fetch(u0 + wave + NW * (it + PF), sl[p]);
            }
        }
    }

    // the waves' sums, added in wave order: red[wave][row][i]
    __syncthreads();
    float *red = a_lds;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < M; ++i) red[(wave * GV_ROWS + 4 * lane + j) * M + i] = acc[j][i];
    __syncthreads();
    // thread t < 256: row t of the tile, all M activation rows
    const bool row_thread = tid < GV_ROWS;
    const int64_t r = (int64_t)blockIdx.x * GV_ROWS + tid;
    float mine[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        float v = 0.f;
        if (row_thread)
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[(w * GV_ROWS + tid) * M + i];
        mine[i] = v;
    }
    auto store_y = [&](int i, float v) {
        const int64_t o = (m0 + i) * d_out + r;
        if (y_bf16) {
            const unsigned u = __builtin_bit_cast(unsigned, v);   // round to nearest even
            ((uint16_t *)Y)[o] = (uint16_t)((u + ((u >> 16) & 1u) + 0x7FFFu) >> 16);
        } else {
            ((float *)Y)[o] = v;
        }
    };
    if (nsplit == 1) {
        if (row_thread && r < d_out)
#pragma unroll
            for (int i = 0; i < M; ++i)
                if (m0 + i < m_total) store_y(i, mine[i]);
        return;
    }
    // Partial sums of this k-range, then the tile's last group adds them all.
    // The partials are device-scope atomic stores and loads (written through
    // to, and read from, the point where all XCDs see memory alike, past the
    // per-XCD L2), and every store has completed (vmcnt drained) before this
    // group's count is added; the group that adds the last count therefore
    // reads every partial.  This is the ordering a device-scope release and
    // acquire give, without writing back and invalidating the whole L2 in
    // every group (which made the product three times slower).
    if (row_thread && r < d_out)
#pragma unroll
        for (int i = 0; i < M; ++i)
            __hip_atomic_store(&part[((int64_t)split * M + i) * d_out + r], mine[i], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(&counters[blockIdx.x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = old == nsplit - 1;
    }
    __syncthreads();
    if (!last_flag) return;
    if (row_thread && r < d_out) {
#pragma unroll
        for (int i = 0; i < M; ++i) {
            // split order, eight loads in flight at a time
            float v = 0.f;
            for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
                float t[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int sp = sp0 + q;
                    t[q] = (sp >= nsplit) ? 0.f
                         : (sp == split ? mine[i]
                                        : __hip_atomic_load(&part[((int64_t)sp * M + i) * d_out + r],
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                }
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (sp0 + q < nsplit) v += t[q];
            }
            if (m0 + i < m_total) store_y(i, v);
        }
    }
    if (tid == 0) counters[blockIdx.x] = 0;    // ready for the next call on this workspace
}

// waves per work group: eight for one activation row on layers under 16 MB
// of packed words (few work groups there, so every SIMD gets a share), four
// otherwise (the streaming shapes and the wider accumulators)
int gemv_waves(int M, int64_t d_out, int64_t d_in, int bits) {
    const int64_t packed = d_out * cdiv((int64_t)bits * d_in, 32) * 4;
    return (M == 1 && packed < ((int64_t)16 << 20)) ? 8 : 4;
}

// work groups along k for a launch of M activation rows (measured on q_proj,
// up_proj, down_proj and the 70B down_proj): about 128 work groups in all for
// layers under 16 MB of packed words (fixed costs per group dominate there)
// and 512 above.  With eight rows (more arithmetic per word) at most one group
// per CU, 256 in all, unless a wave would then take more than 16 units, where
// 512 (two per CU) hide the longer streams better; with two or four rows the
// same only where it keeps at least 240 of the CUs busy.  A count just above
// the CU count is the one to avoid: the CUs that take two groups finish last
// (up_proj, 8 rows: 258 groups 54 us, 172 groups 40 us).  Each wave gets at
// least one unit and the staged range fits in LDS.
int gemv_splits(int M, int64_t d_out, int64_t d_in, int bits) {
    const int nunits = (int)cdiv(d_in, UNIT);
    const int64_t tiles = cdiv(d_out, GV_ROWS);
    const int max_units = GV_LDS / (M * UNIT);
    const int waves = gemv_waves(M, d_out, d_in, bits);
    const int64_t packed = d_out * cdiv((int64_t)bits * d_in, 32) * 4;
    int64_t target = packed < ((int64_t)16 << 20) ? 128 : 512;
    if (M > 1) {
        const int64_t s1 = std::max<int64_t>(1, 256 / tiles);
        if (nunits / s1 > 16 * waves)
            target = 512;
        else if (M == GV_MAX_M || s1 * tiles >= 240)
            target = 256;
    }
    int64_t s = std::max<int64_t>(1, target / tiles);
    s = std::min<int64_t>(s, std::max(1, nunits / waves));
    s = std::max<int64_t>(s, cdiv(nunits, max_units));
    return (int)s;
}

int pad_m(int64_t mc) { return mc <= 1 ? 1 : (mc <= 2 ? 2 : (mc <= 4 ? 4 : 8)); }

template <int BITS, int M, bool VEC, bool G32, bool D2>
void launch_gemv_k(const DequantArgs &a, int64_t m0, hipStream_t st) {
    const int nsplit = gemv_splits(M, a.d_out, a.d_in, BITS);
    const dim3 grid((unsigned)cdiv(a.d_out, GV_ROWS), (unsigned)nsplit);
    const int nunits = (int)cdiv(a.d_in, UNIT);
    const int64_t nwords = cdiv((int64_t)BITS * a.d_in, 32);
    if constexpr (M == 1) {
        if (gemv_waves(M, a.d_out, a.d_in, BITS) == 8) {
            dq_gemv_kernel<BITS, M, 8, VEC, G32, D2><<<grid, 512, 0, st>>>(
                a.A, a.a_bf16, a.perm, a.Q, a.scales, a.zeros, a.Y, a.y_bf16, a.part, a.counters, a.m, m0, a.d_in,
                a.d_out, a.group, a.ngroups, nunits, nsplit, nwords);
            return;
        }
    }
    dq_gemv_kernel<BITS, M, 4, VEC, G32, D2><<<grid, 256, 0, st>>>(a.A, a.a_bf16, a.perm, a.Q, a.scales, a.zeros, a.Y,
                                                            a.y_bf16, a.part, a.counters, a.m, m0, a.d_in, a.d_out,
                                                            a.group, a.ngroups, nunits, nsplit, nwords);
}

template <int BITS, int M, bool D2>
hipError_t launch_gemv_md(const DequantArgs &a, int64_t m0, hipStream_t st) {
    const bool vec = a.d_out % 4 == 0;
    const bool g32 = a.group % 32 == 0 || a.ngroups == 1;
    if (vec && g32)
        launch_gemv_k<BITS, M, true, true, D2>(a, m0, st);
    else if (vec)
        launch_gemv_k<BITS, M, true, false, D2>(a, m0, st);
    else if (g32)
        launch_gemv_k<BITS, M, false, true, D2>(a, m0, st);
    else
        launch_gemv_k<BITS, M, false, false, D2>(a, m0, st);
    return hipGetLastError();
}

// bf16 activations in launches of two or more rows take the pairwise dot
template <int BITS, int M>
hipError_t launch_gemv_m(const DequantArgs &a, int64_t m0, hipStream_t st) {
    if constexpr (M >= 2) {
        if (a.a_bf16) return launch_gemv_md<BITS, M, true>(a, m0, st);
    }
    return launch_gemv_md<BITS, M, false>(a, m0, st);
}

template <int BITS>
hipError_t launch_gemv_bits(const DequantArgs &a, hipStream_t st) {
    for (int64_t m0 = 0; m0 < a.m; m0 += GV_MAX_M) {
        const int M = pad_m(std::min<int64_t>(GV_MAX_M, a.m - m0));
        hipError_t e;
        if (M == 1)
            e = launch_gemv_m<BITS, 1>(a, m0, st);
        else if (M == 2)
            e = launch_gemv_m<BITS, 2>(a, m0, st);
        else if (M == 4)
            e = launch_gemv_m<BITS, 4>(a, m0, st);
        else
            e = launch_gemv_m<BITS, 8>(a, m0, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}


// code k (0..31, a constant after unrolling) of a unit held in BITS words
template <int BITS>
__device__ __forceinline__ unsigned unit_code_w(const unsigned (&w)[BITS], int k) {
    const int pos = BITS * k, j = pos >> 5, sh = pos & 31;
    if (sh + BITS <= 32) return __builtin_amdgcn_ubfe(w[j], sh, BITS);
    return __builtin_amdgcn_alignbit(w[j + 1 < BITS ? j + 1 : j], w[j], sh) & ((1u << BITS) - 1u);
}

// ---------------------------------------------------------------------------
// Wide path (m >= 16 bf16 activation rows; prefill): bf16 MFMA on exact
// integer weights.  For every group, D = A_p[:, group] (q - z)[group, :]^T is
// formed with v_mfma_f32_32x32x16_bf16: q - z is an integer in [-255, 255]
// and exact in bf16, every product of two bf16 values is exact in fp32, and
// D accumulates in fp32; at the group's end Y += s D (one fp32 fma per
// output and group).  A work group (8 waves, 4 x 2, each 64 x 64 as 2 x 2
// tiles of 32 x 32) owns 256 x 128 of Y and walks k in chunks of 64: the
// chunk's activations (256 x 64 bf16) and its weights as q - z in bf16
// (128 x 64; each thread dequantizes 16 codes of one row) go through LDS,
// the next chunk's loads issued before the current chunk's products; staged
// rows are padded by 8 bf16 so that the 16-byte operand reads of a wave fall
// on distinct banks.  The chunk's scales are staged with them.  Activations
// of an act-order layer are first gathered into processing order into the
// workspace by a separate kernel.
// ---------------------------------------------------------------------------
constexpr int GM_BM = 256, GM_BN = 128, GM_KC = 64;
constexpr int GM_LDA = GM_KC + 8;            // bf16 per staged row (padding)
constexpr int GM_MAXG = GM_KC / 16;          // groups a chunk can touch (g >= 16)
constexpr int GM_MIN_M = 16;                 // fewest activation rows for the wide path

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// A_p[i][k] = A[i][perm[k]] (bf16), the activations in processing order
__global__ __launch_bounds__(256) void dq_permute_kernel(const uint16_t *__restrict__ A,
                                                         const int32_t *__restrict__ perm,
                                                         uint16_t *__restrict__ Ap, int64_t m, int64_t d_in) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= m * d_in) return;
    const int64_t i = idx / d_in, k = idx - i * d_in;
    Ap[idx] = A[i * d_in + perm[k]];
}

// The same, one work group per activation row (d_in % 8 == 0): the row is
// staged in LDS with 16-byte loads, gathered from there and written as
// 16-byte pieces (a gather straight from global memory touches a scattered
// 2-byte value per lane).
constexpr int64_t PERMUTE_LDS_MAX = 80 * 1024;   // bf16 values of a staged row (160 KB)
__global__ __launch_bounds__(256) void dq_permute_lds_kernel(const uint16_t *__restrict__ A,
                                                             const int32_t *__restrict__ perm,
                                                             uint16_t *__restrict__ Ap, int64_t d_in) {
    extern __shared__ __attribute__((aligned(16))) uint16_t srow16[];
    const int64_t i = blockIdx.x;
    const int np = (int)(d_in / 8);
    const u32x4 *src = (const u32x4 *)(A + i * d_in);
    for (int p = threadIdx.x; p < np; p += 256) *(u32x4 *)(srow16 + 8 * p) = src[p];
    __syncthreads();
    u32x4 *dst = (u32x4 *)(Ap + i * d_in);
    for (int p = threadIdx.x; p < np; p += 256) {
        int c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = perm[8 * p + e];
        unsigned w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (unsigned)srow16[c[2 * e]] | ((unsigned)srow16[c[2 * e + 1]] << 16);
        dst[p] = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// dynamic LDS above the default limit must be allowed once
bool permute_lds_ok(int64_t d_in) {
    static int state = 0;   // 0 unknown, 1 allowed, -1 refused
    if (d_in > PERMUTE_LDS_MAX) return false;
    if (state == 0)
        state = hipFuncSetAttribute((const void *)dq_permute_lds_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)(PERMUTE_LDS_MAX * 2)) == hipSuccess
                    ? 1
                    : -1;
    if (state < 0) (void)hipGetLastError();
    return state > 0;
}

// d_in % 8 == 0 (whole 16-byte pieces of activation rows)
template <int BITS>
__global__ __launch_bounds__(512) void dq_gemm_kernel(const uint16_t *__restrict__ A, const uint32_t *__restrict__ Q,
                                                      const float *__restrict__ scales,
                                                      const float *__restrict__ zeros, void *__restrict__ Y,
                                                      int y_bf16, int64_t m, int64_t d_in, int64_t d_out, int g,
                                                      int ngroups, int64_t nwords) {
    __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][GM_BM * GM_LDA];
    __shared__ __attribute__((aligned(16))) uint16_t b_lds[2][GM_BN * GM_LDA];
    __shared__ float s_lds[2][GM_MAXG * GM_BN];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.x * GM_BM, n0 = (int64_t)blockIdx.y * GM_BN;
    const int nchunks = (int)((d_in + GM_KC - 1) / GM_KC);

    // staging roles.  Activations: row tid / 2, pieces 4 (tid % 2) .. +3 (8
    // bf16 each).  Weights: row tid % 128, codes 16 q .. 16 q + 15 of the
    // chunk (q = tid / 128), from the unit's words.  Scales: slot tid / 128 of
    // row tid % 128.
    const int64_t arow = m0 + (tid >> 1);
    const int apiece = 4 * (tid & 1);
    const int bn = tid & (GM_BN - 1), bq = tid >> 7;
    const int64_t nrow = n0 + bn;
    u32x4 ra[4];
    unsigned rw[BITS];
    float rz = 0.f, rs = 0.f;
    auto load_chunk = [&](int c) {
        const int64_t k0 = (int64_t)c * GM_KC;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t k = k0 + 8 * (apiece + q);
            ra[q] = (arow < m && k < d_in) ? *(const u32x4 *)(A + arow * d_in + k) : u32x4{0u, 0u, 0u, 0u};
        }
        const int64_t u = (k0 >> 5) + (bq >> 1);   // 32-code unit of this thread's codes
#pragma unroll
        for (int b = 0; b < BITS; ++b) {
            const int64_t wi = u * BITS + b;
            rw[b] = (nrow < d_out && wi < nwords) ? Q[wi * d_out + nrow] : 0u;
        }
        const int64_t gz = std::min<int64_t>((k0 + 16 * bq) / g, ngroups - 1);
        rz = nrow < d_out ? zeros[gz * d_out + nrow] : 0.f;
        const int64_t gs = std::min<int64_t>(k0 / g + bq, ngroups - 1);
        rs = nrow < d_out ? scales[gs * d_out + nrow] : 0.f;
    };
    auto store_chunk = [&](int buf) {
        uint16_t *ad = a_lds[buf] + (tid >> 1) * GM_LDA + 8 * apiece;
#pragma unroll
        for (int q = 0; q < 4; ++q) *(u32x4 *)(ad + 8 * q) = ra[q];
        // codes 16 (bq % 2) .. +15 of the unit as q - z in bf16
        unsigned pk[8];
        const int c0 = 16 * (bq & 1);
#pragma unroll
        for (int kk = 0; kk < 16; kk += 2) {
            const float v0 = (float)unit_code_w<BITS>(rw, c0 + kk) - rz;
            const float v1 = (float)unit_code_w<BITS>(rw, c0 + kk + 1) - rz;
            const bf16x2 p = {(__bf16)v0, (__bf16)v1};
            pk[kk >> 1] = __builtin_bit_cast(unsigned, p);
        }
        uint16_t *bd = b_lds[buf] + bn * GM_LDA + 16 * bq;
        *(u32x4 *)(bd) = u32x4{pk[0], pk[1], pk[2], pk[3]};
        *(u32x4 *)(bd + 8) = u32x4{pk[4], pk[5], pk[6], pk[7]};
        s_lds[buf][bq * GM_BN + bn] = rs;
    };

    f32x16 acc[2][2], dg[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            acc[a][b] = f32x16{};
            dg[a][b] = f32x16{};
        }
    // operand reads: lane l supplies row / column l % 32, k 8 (l / 32) .. +7
    const int orow = lane & 31, ok = 8 * (lane >> 5);

    load_chunk(0);
    store_chunk(0);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < nchunks) load_chunk(c + 1);   // in flight during this chunk's products
        const int64_t k0 = (int64_t)c * GM_KC;
        const uint16_t *ab = a_lds[buf] + (wm * 64 + orow) * GM_LDA + ok;
        const uint16_t *bb = b_lds[buf] + (wn * 64 + orow) * GM_LDA + ok;
#pragma unroll
        for (int ks = 0; ks < GM_KC / 16; ++ks) {
            const int64_t k = k0 + 16 * ks;
            if (k >= d_in) break;   // uniform
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) fa[a] = *(const bf16x8 *)(ab + a * 32 * GM_LDA + 16 * ks);
#pragma unroll
            for (int b = 0; b < 2; ++b) fb[b] = *(const bf16x8 *)(bb + b * 32 * GM_LDA + 16 * ks);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    dg[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], dg[a][b], 0, 0, 0);
            // a group ends after this k step: Y += s D, D = 0 (uniform)
            const int64_t kn = k + 16;
            if (kn >= d_in || kn % g == 0) {
                const int slot = (int)(k / g - k0 / g);
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const float sc = s_lds[buf][slot * GM_BN + wn * 64 + 32 * b + orow];
#pragma unroll
                    for (int a = 0; a < 2; ++a) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[a][b][r] = fmaf(sc, dg[a][b][r], acc[a][b][r]);
                        dg[a][b] = f32x16{};
                    }
                }
            }
        }
        __syncthreads();   // every wave is done with the other buffer's previous chunk
        if (c + 1 < nchunks) store_chunk(buf ^ 1);
        __syncthreads();
    }
    // Y: tile (a, b) of wave (wm, wn), register 4 i + j <-> row 8 i + 4 (l / 32) + j, column l % 32
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t n = n0 + wn * 64 + 32 * b + orow;
            if (n >= d_out) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + 32 * a + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= m) continue;
                const float v = acc[a][b][r];
                if (y_bf16) {
                    const unsigned u = __builtin_bit_cast(unsigned, v);
                    ((uint16_t *)Y)[row * d_out + n] = (uint16_t)((u + ((u >> 16) & 1u) + 0x7FFFu) >> 16);
                } else {
                    ((float *)Y)[row * d_out + n] = v;
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Wide path, streamed form (d_in a multiple of the stage width KC).  The same
// product and the same 256 x 128 tiles of Y (8 waves, 4 x 2, each 64 x 64),
// but k moves in stages of KC (32 or 64 codes, one or two units) through an
// LDS ring that buffer loads fill directly (no register round trip): per
// stage the unit's packed words, the scales and zero points of its 16-code
// halves, then the activations (256 x KC bf16, 16-byte pieces).  While the
// products of stage c run, stage c+1's codes are dequantized (q - z, bf16)
// into one of two LDS weight tiles, in the same branch-free block, so that
// the conversions fill the issue slots between the matrix instructions.  One
// barrier per stage; at its end a wave waits only until the next stage's
// codes have landed, so the activations (issued last) have two stages to
// arrive.  Stages of 64 (codes of up to 4 bits) halve the barriers and
// per-stage costs per product; 8-bit codes take stages of 32 (a 64-wide
// ring would not fit the LDS).  Activation pieces are swizzled within their
// LDS row so that the 16-byte operand reads of 8 or 16 consecutive rows fall
// on distinct banks.  Waves with no packed-word load of their own in a stage
// issue a dummy one, so that every wave counts the same loads per stage.
// ---------------------------------------------------------------------------
constexpr int GR_NW = 8;          // waves per work group
constexpr int GR_MAX_SPLIT = 16;  // k splits of a small grid, at most

template <int BITS, int KC>
struct GrLayout {
    static constexpr int KS = KC / 16;                    // k steps of 16 per stage
    static constexpr int UPS = KC / 32;                   // 32-code units per stage
    static constexpr int NST = KC == 32 ? 6 : 3;          // ring stages
    static constexpr int AROW = KC * 2;                   // bytes of one activation row per stage
    static constexpr int A_STAGE = GM_BM * AROW;
    static constexpr int BROW = KC + 8;                   // bf16 per staged weight row (padding)
    static constexpr int Q_STAGE = UPS * BITS * GM_BN * 4;
    static constexpr int SZ_STAGE = 2 * KS * GM_BN * 4;   // [s, z][half][128] floats
    static constexpr int Q_OFF = NST * A_STAGE;
    static constexpr int SZ_OFF = Q_OFF + NST * Q_STAGE;
    static constexpr int B_OFF = SZ_OFF + NST * SZ_STAGE;
    static constexpr int B_BUF = GM_BN * BROW * 2;
    static constexpr int JUNK_OFF = B_OFF + 2 * B_BUF;    // target of the dummy loads
    static constexpr int BYTES = JUNK_OFF + 256;
    static constexpr int ADMA = A_STAGE / 1024 / GR_NW;   // activation loads per wave and stage (1 KB)
    static constexpr int QDMA = (2 * BITS * UPS + GR_NW - 1) / GR_NW;   // packed-word loads (256 B)
    static constexpr int SDMA = 4 * KS / GR_NW;           // scale / zero-point loads (256 B)
    static constexpr int PER_STAGE = ADMA + QDMA + SDMA;
    static constexpr int NCH = GM_BN * KC / (64 * GR_NW) / 8;   // 8-code chunks each thread dequantizes
    static_assert(BYTES <= 160 * 1024, "the ring fits the LDS");
};

typedef __attribute__((address_space(3))) void gr_lds_void_t;

template <int N>
__device__ __forceinline__ void gr_wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// barrier without __syncthreads()' fence (which would wait for every stage
// in flight); this wave's LDS operations are drained first
__device__ __forceinline__ void gr_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// buffer resource over [p, p + bytes), base and size in SGPRs
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gr_rsrc(const void *p, int64_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) << 32) |
                        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((unsigned)b);
    const int n = __builtin_amdgcn_readfirstlane((int)std::min<int64_t>(std::max<int64_t>(bytes, 0), (int64_t)0x7fffffff));
    return __builtin_amdgcn_make_buffer_rsrc((void *)bu, (short)0, n, 0x00020000);
}

// 16-byte piece position of an activation row inside its LDS row: four
// pieces (stages of 32) or eight (stages of 64)
template <int KC>
__device__ __forceinline__ int gr_swz(int row) {
    if constexpr (KC == 32)
        return ((row >> 1) & 3) ^ ((row >> 3) & 1);
    else
        return ((row >> 1) ^ ((row & 1) << 2)) & 7;
}

// Split k (small grids): work group z takes stages [st_begin, st_end), cut
// at multiples of `align` stages (whole groups), folds its own pieces of the
// groups (s D is linear in D), and the tile's last group to finish adds the
// splits' partial sums in split order.
template <int BITS, int KC, bool SPLIT>
__global__ __launch_bounds__(64 * GR_NW) void dq_gemm_ring_kernel(const uint16_t *__restrict__ A,
                                                                  const uint32_t *__restrict__ Q,
                                                                  const float *__restrict__ scales,
                                                                  const float *__restrict__ zeros,
                                                                  void *__restrict__ Y, int y_bf16, int64_t m,
                                                                  int64_t d_in, int64_t d_out, int g, int ngroups,
                                                                  int64_t nwords, float *__restrict__ part,
                                                                  int32_t *__restrict__ counters, int nsplit,
                                                                  int align) {
    using L = GrLayout<BITS, KC>;
    // (arrays that the lambdas below capture have literal sizes, their
    // largest counts: with value-dependent sizes the host pass drops the
    // kernel's launch stub)
    constexpr int NST = L::NST, KS = L::KS, ADMA = L::ADMA, QDMA = L::QDMA, SDMA = L::SDMA, NCH = L::NCH;
    static_assert(ADMA <= 4 && QDMA <= 2 && SDMA <= 2 && NCH <= 2, "per-thread array bounds");
    constexpr int RPI = 1024 / L::AROW, PPR = L::AROW / 16;   // activation rows per load, pieces per row
    __shared__ __attribute__((aligned(16))) char lds[L::BYTES];
    __shared__ int last_flag;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.x * GM_BM, n0 = (int64_t)blockIdx.y * GM_BN;
    const int split = SPLIT ? (int)blockIdx.z : 0;
    const int nst_all = (int)(d_in / KC);
    int st_begin = 0, st_end = nst_all;
    if (SPLIT) {
        // (32-bit arithmetic, kept in scalar registers: the loads' scalar
        // offsets derive from these)
        const int nal = nst_all / align;
        st_begin = __builtin_amdgcn_readfirstlane(align * (nal * split / nsplit));
        st_end = __builtin_amdgcn_readfirstlane(split == nsplit - 1 ? nst_all : align * (nal * (split + 1) / nsplit));
    }
    const int nst = st_end - st_begin;   // this split's stages

    // Every load address is clamped into its operand (rows past m re-read
    // the last row, columns past d_out the last column, stages past the end
    // the last stage: all only feed entries that are never stored), so no
    // load relies on buffer range checks; per-lane offsets are fixed and the
    // stage moves only the scalar offset.
    const int rows = (int)(std::min<int64_t>(m, m0 + GM_BM) - m0);
    const int cols = (int)(std::min<int64_t>(d_out, n0 + GM_BN) - n0);
    const __amdgpu_buffer_rsrc_t arsrc = gr_rsrc(A + m0 * d_in, (int64_t)rows * d_in * 2);
    const __amdgpu_buffer_rsrc_t qrsrc = gr_rsrc(Q + n0, (nwords * d_out - n0) * 4);
    const __amdgpu_buffer_rsrc_t srsrc = gr_rsrc(scales + n0, ((int64_t)ngroups * d_out - n0) * 4);
    const __amdgpu_buffer_rsrc_t zrsrc = gr_rsrc(zeros + n0, ((int64_t)ngroups * d_out - n0) * 4);
    // activation load j = ADMA wave + q of a stage fills LDS rows RPI j ..
    // RPI j + RPI - 1; lane l lands in row RPI j + l / PPR at piece position
    // l % PPR, holding the piece that the swizzle places there
    int aoff[4];
#pragma unroll
    for (int q = 0; q < ADMA; ++q) {
        const int r = RPI * (ADMA * wave + q) + lane / PPR;
        const int p = (lane % PPR) ^ gr_swz<KC>(r);
        aoff[q] = std::min(r, rows - 1) * (int)d_in * 2 + 16 * p;
    }
    // packed-word load i = wave + 8 t: word row i / 2 of the stage, columns
    // 64 (i % 2) .. +63 (a dummy re-read of row 0 when i >= 2 bits units)
    int qoff[2];
#pragma unroll
    for (int t = 0; t < QDMA; ++t) {
        const int i = wave + GR_NW * t;
        qoff[t] = i < 2 * BITS * L::UPS ? ((i >> 1) * (int)d_out + std::min(64 * (i & 1) + lane, cols - 1)) * 4
                                        : std::min(lane, cols - 1) * 4;
    }
    // scale / zero-point load i = wave + 8 t: tensor i / (2 KS) (s, z), half
    // i / 2 % KS of the stage, columns 64 (i % 2) .. +63
    int szoff[2];
#pragma unroll
    for (int t = 0; t < SDMA; ++t) szoff[t] = std::min(64 * ((wave + GR_NW * t) & 1) + lane, cols - 1) * 4;
    // k steps of 16 per group: 1, 2 or a multiple of KS (16, 32, whole
    // stages or one group per row)
    const int gsteps = g / 16;
    const int qstride = L::UPS * BITS * (int)d_out * 4, gstride = (int)d_out * 4;
    // issue tracker: the stage to issue (clamped when loaded), the group of
    // its first k step and that step's place in the group
    int iss_st = st_begin, iss_g = __builtin_amdgcn_readfirstlane(st_begin * KS / gsteps);
    int iss_r = __builtin_amdgcn_readfirstlane(st_begin * KS - iss_g * gsteps);

    auto issue = [&](int slot) {
        const int st = std::min(iss_st, st_end - 1);
        // packed words and scales first: the next stage's conversions need
        // them one stage before its products need the activations
        char *qbase = lds + L::Q_OFF + slot * L::Q_STAGE;
        const int qsoff = __builtin_amdgcn_readfirstlane(st * qstride);
#pragma unroll
        for (int t = 0; t < QDMA; ++t) {
            const int i = wave + GR_NW * t;
            gr_lds_void_t *dst = (gr_lds_void_t *)(i < 2 * BITS * L::UPS ? qbase + (i >> 1) * 512 + (i & 1) * 256
                                                                         : lds + L::JUNK_OFF);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qrsrc, dst, 4, qoff[t], qsoff, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < SDMA; ++t) {
            const int i = wave + GR_NW * t, ten = i / (2 * KS), h = (i >> 1) % KS;
            // the half's group (g of 16: one per half; of 32: one per two
            // halves, the stage starting a group; otherwise one per stage)
            const int gh = iss_g + (gsteps == 1 ? h : (gsteps == 2 ? (h >> 1) : 0));
            const int soff = __builtin_amdgcn_readfirstlane(std::min(gh, ngroups - 1) * gstride);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ten ? zrsrc : srsrc,
                (gr_lds_void_t *)(lds + L::SZ_OFF + slot * L::SZ_STAGE + (ten * KS + h) * GM_BN * 4 + (i & 1) * 256),
                4, szoff[t], soff, 0, 0);
        }
        char *base = lds + slot * L::A_STAGE;
#pragma unroll
        for (int q = 0; q < ADMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (gr_lds_void_t *)(base + (ADMA * wave + q) * 1024), 16,
                                                     aoff[q], st * KC * 2, 0, 0);
        ++iss_st;
        iss_r += KS;
        while (iss_r >= gsteps) {
            iss_r -= gsteps;
            ++iss_g;
        }
    };

    // dequantization: thread t turns codes 8 (NCH (t / 128) + j) .. +7 of a
    // stage (j < NCH) in tile row t % 128 into q - z (bf16)
    const int bn = tid & (GM_BN - 1), bpart = tid >> 7;
    int dq_w0[2], dq_w1[2], dq_sh[2];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int q8 = NCH * bpart + j, uo = q8 >> 2, cpos = BITS * 8 * (q8 & 3), cj0 = cpos >> 5;
        dq_w0[j] = L::Q_OFF + ((uo * BITS + cj0) * GM_BN + bn) * 4;
        dq_w1[j] = L::Q_OFF + ((uo * BITS + std::min(cj0 + 1, BITS - 1)) * GM_BN + bn) * 4;
        dq_sh[j] = cpos & 31;
    }
    // a thread's chunks lie in one 16-code half
    const int dq_z = L::SZ_OFF + ((KS + (NCH * bpart) / 2) * GM_BN + bn) * 4;
    const int dq_dst = L::B_OFF + bn * L::BROW * 2 + 16 * NCH * bpart;
    auto dq_convert = [&](unsigned lo, unsigned hi, int sh, float z) {
        const uint64_t w = (((uint64_t)hi << 32) | (uint64_t)lo) >> sh;
        unsigned pk[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const float v0 = (float)(unsigned)((w >> (BITS * j)) & ((1u << BITS) - 1u)) - z;
            const float v1 = (float)(unsigned)((w >> (BITS * (j + 1))) & ((1u << BITS) - 1u)) - z;
            const bf16x2 p = {(__bf16)v0, (__bf16)v1};
            pk[j >> 1] = __builtin_bit_cast(unsigned, p);
        }
        return u32x4{pk[0], pk[1], pk[2], pk[3]};
    };
    auto dequant = [&](int slot, int tile) {
        const char *qs = lds + slot * L::Q_STAGE;
        const float z = *(const float *)(lds + slot * L::SZ_STAGE + dq_z);
        unsigned w0[2], w1[2];
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            w0[j] = *(const unsigned *)(qs + dq_w0[j]);
            w1[j] = *(const unsigned *)(qs + dq_w1[j]);
        }
#pragma unroll
        for (int j = 0; j < NCH; ++j)
            *(u32x4 *)(lds + tile * L::B_BUF + dq_dst + 16 * j) = dq_convert(w0[j], w1[j], dq_sh[j], z);
    };

    f32x16 acc[2][2], dg[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            acc[a][b] = f32x16{};
            dg[a][b] = f32x16{};   // (every group overwrites it at its first step)
        }
    // operand reads: lane l supplies row / column l % 32, k 8 (l / 32) .. +7
    const int orow = lane & 31, oh = lane >> 5;
    const int aswz = gr_swz<KC>(orow);   // rows of a lane differ by multiples of 32
    const int op_a = (wm * 64 + orow) * L::AROW, op_b = L::B_OFF + (wn * 64 + orow) * L::BROW * 2;
    const int op_s = L::SZ_OFF + (wn * 64 + orow) * 4;

    // One stage: the products of stage st (slot `slot`, weight tile st % 2)
    // and the dequantization of stage st + 1 (slot `nslot`, the other
    // tile).  Group structure of the stage's KS k steps, fixed at compile
    // time: bit s of FR, a group starts at step s (D begins from zero); bit
    // s of EN, a group ends after step s (Y += s D).
    auto stage = [&](auto frc, auto enc, int st, int slot, int nslot) {
        constexpr int FR = decltype(frc)::value, EN = decltype(enc)::value;
        const char *ab = lds + slot * L::A_STAGE + op_a;
        const char *bb = lds + (st & 1) * L::B_BUF + op_b;
        const float *sc = (const float *)(lds + slot * L::SZ_STAGE + op_s);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int p = 2 * ks + oh;
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) fa[a] = *(const bf16x8 *)(ab + a * 32 * L::AROW + 16 * (p ^ aswz));
#pragma unroll
            for (int b = 0; b < 2; ++b) fb[b] = *(const bf16x8 *)(bb + b * 32 * L::BROW * 2 + 16 * p);
            const bool fresh = (FR >> ks) & 1;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    dg[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[b], fresh ? f32x16{} : dg[a][b], 0,
                                                                       0, 0);
            if ((EN >> ks) & 1) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const float s = sc[ks * GM_BN + 32 * b];
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[a][b][r] = fmaf(s, dg[a][b][r], acc[a][b][r]);
                }
                // a group starting at the next step overwrites D: keep its
                // products behind these reads
                if (ks + 1 < KS && ((FR >> (ks + 1)) & 1)) __builtin_amdgcn_sched_barrier(0);
            }
        }
        dequant(nslot, (st + 1) & 1);
    };

    // Ring: stage j lives in slot j % NST.  Loads go out in stage order, each
    // stage's packed words and scales before its activations; at the end of
    // iteration c the next stage's words and scales (stage c + 2 in the ring:
    // its conversions run in iteration c + 1) and stage c + 1's activations
    // have landed, so stage c + 2's activations and everything later may
    // still be outstanding.  Stages issued past the end re-read the last one,
    // unused (the dequantization of the stage after the last one writes a
    // weight tile that is never read).
    constexpr int PS = L::PER_STAGE;
    for (int st = 0; st < NST - 1; ++st) issue(st);
    gr_wait_vm<ADMA + (NST - 2) * PS>();   // stage 0's words and scales
    gr_barrier();
    dequant(0, 0);
    gr_wait_vm<ADMA + (NST - 3) * PS>();   // stage 0's activations, stage 1's words and scales
    gr_barrier();
    int c = 0, slot = 0;
    auto iteration = [&](auto frc, auto enc) {
        const int next = slot == NST - 1 ? 0 : slot + 1;
        issue(slot == 0 ? NST - 1 : slot - 1);   // stage c + NST - 1, into the slot of stage c - 1
        stage(frc, enc, c, slot, next);
        gr_wait_vm<ADMA + (NST - 3) * PS>();
        gr_barrier();
        slot = next;
        ++c;
    };
    using IC0 = std::integral_constant<int, 0>;
    using ICA = std::integral_constant<int, (1 << KS) - 1>;            // every step
    using ICF = std::integral_constant<int, 1>;                        // first step
    using ICL = std::integral_constant<int, 1 << (KS - 1)>;            // last step
    using ICE = std::integral_constant<int, KS == 4 ? 0b0101 : 0b01>;  // even steps
    using ICO = std::integral_constant<int, KS == 4 ? 0b1010 : 0b10>;  // odd steps
    if (gsteps == 1) {
        // groups of 16: each k step is a group
        while (c < nst) iteration(ICA{}, ICA{});
    } else if (gsteps == 2 && KS == 4) {
        // groups of 32 in stages of 64: two per stage
        while (c < nst) iteration(ICE{}, ICO{});
    } else {
        // groups of whole stages (or one group per row)
        const int spg = gsteps / KS;
        while (c < nst) {
            const int len = std::min(spg, nst - c);
            if (len == 1) {
                iteration(ICF{}, ICL{});
            } else {
                iteration(ICF{}, IC0{});
                for (int j = 1; j < len - 1; ++j) iteration(IC0{}, IC0{});
                iteration(IC0{}, ICL{});
            }
        }
    }
    gr_wait_vm<0>();   // no load may still write LDS when the group ends

    // Y: tile (a, b) of wave (wm, wn), register 4 i + j <-> row 8 i + 4 (l / 32) + j, column l % 32
    auto store_y = [&](int64_t row, int64_t n, float v) {
        if (y_bf16) {
            const unsigned u = __builtin_bit_cast(unsigned, v);
            ((uint16_t *)Y)[row * d_out + n] = (uint16_t)((u + ((u >> 16) & 1u) + 0x7FFFu) >> 16);
        } else {
            ((float *)Y)[row * d_out + n] = v;
        }
    };
    if constexpr (SPLIT) {
        // This split's partial sums, then the tile's last group adds them
        // all.  Device-scope atomic stores and loads (written through to, and
        // read from, the point where all XCDs see memory alike), every store
        // drained (vmcnt) before the group's count is added: the ordering of
        // a device-scope release and acquire without writing back and
        // invalidating the whole L2 in every group.
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int64_t n = n0 + wn * 64 + 32 * b + orow;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * 64 + 32 * a + 8 * (r >> 2) + 4 * oh + (r & 3);
                    if (n < d_out && row < m)
                        __hip_atomic_store(&part[((int64_t)split * m + row) * d_out + n], acc[a][b][r],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int tile = (int)(blockIdx.x + gridDim.x * blockIdx.y);
        if (tid == 0) {
            const int old = __hip_atomic_fetch_add(&counters[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_flag = old == nsplit - 1;
        }
        __syncthreads();
        if (!last_flag) return;
        // every split's partial sums (this group's own included: the
        // accumulators are reused for the sum), one split at a time with
        // all of the lane's 64 outputs in flight together, added in split
        // order
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
        // (32-bit element offsets: m d_out is small whenever k is split)
        int eo[2][16];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int n = (int)std::min<int64_t>(n0 + wn * 64 + 32 * b + orow, d_out - 1);
                const int row = (int)std::min<int64_t>(m0 + wm * 64 + 8 * (r >> 2) + 4 * oh + (r & 3), m - 1);
                eo[b][r] = row * (int)d_out + n;
            }
        const int md = (int)(m * d_out);
#pragma unroll 1
        for (int sp = 0; sp < nsplit; ++sp) {
            const float *ps = part + (int64_t)sp * md;
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                // rows of block a past m re-read row m - 1 (never stored)
                f32x16 t[2];
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = a == 0 ? eo[b][r] : std::min(eo[b][r] + 32 * (int)d_out, md - 1);
                        t[b][r] = __hip_atomic_load(ps + off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] += t[b];
            }
        }
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int64_t n = n0 + wn * 64 + 32 * b + orow;
                if (n >= d_out) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = m0 + wm * 64 + 32 * a + 8 * (r >> 2) + 4 * oh + (r & 3);
                    if (row < m) store_y(row, n, acc[a][b][r]);
                }
            }
        if (tid == 0) counters[tile] = 0;   // ready for the next call on this workspace
        return;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t n = n0 + wn * 64 + 32 * b + orow;
            if (n >= d_out) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + 32 * a + 8 * (r >> 2) + 4 * oh + (r & 3);
                if (row >= m) continue;
                store_y(row, n, acc[a][b][r]);
            }
        }
}

// the streamed form in stages of KC: whole stages, groups of 16, of 32 (or
// of whole stages, or one group per row), codes of up to 4 bits for stages
// of 64, and 32-bit buffer offsets (a row tile of activations, the packed
// words, the scales)
bool gemm_ring_ok(int kc, int64_t d_in, int64_t d_out, int bits, int g) {
    const int64_t lim = (int64_t)1 << 31;
    if (kc == 64 && bits > 4) return false;
    return d_in % kc == 0 && (g == 16 || g == 32 || g % kc == 0 || g == d_in) && (int64_t)GM_BM * d_in * 2 < lim &&
           bits * (d_in / 32) * d_out * 4 < lim && (d_in / 16) * d_out * 4 < lim;
}

// k splits of the wide path for a small grid (fewer tiles than CUs), each
// split at least four stages of 32 and at most GR_MAX_SPLIT (the workspace
// holds their partial sums); a launch may take fewer so that splits hold
// whole groups
int gemm_splits(int64_t m, int64_t d_out, int64_t d_in) {
    const int64_t tiles = cdiv(m, GM_BM) * cdiv(d_out, GM_BN);
    if (tiles >= 256) return 1;
    // the most splits that still fit one round of the CUs: a count just above
    // it (ceil(256 / tiles) groups per tile) leaves a second, nearly empty
    // round, and a round of 128 tiles alone leaves half the CUs idle
    int64_t s = std::max<int64_t>(1, 256 / tiles);
    s = std::min<int64_t>(s, std::max<int64_t>(1, d_in / 32 / 4));
    return (int)std::min<int64_t>(s, GR_MAX_SPLIT);
}

template <int BITS, int KC>
hipError_t launch_gemm_ring(const uint16_t *A, const DequantArgs &a, int64_t nwords, hipStream_t st) {
    // splits hold whole groups: stages per group when a group spans several
    // stages (one group per row may split anywhere: its fold is linear)
    const int gsteps = a.group / 16, ks = KC / 16;
    const int align = (gsteps > ks && a.group != a.d_in) ? gsteps / ks : 1;
    const int nal = (int)(a.d_in / KC) / align;
    const int nsplit = std::max(1, std::min(gemm_splits(a.m, a.d_out, a.d_in), nal));
    const dim3 grid((unsigned)cdiv(a.m, GM_BM), (unsigned)cdiv(a.d_out, GM_BN), (unsigned)nsplit);
    if (nsplit > 1)
        dq_gemm_ring_kernel<BITS, KC, true><<<grid, 64 * GR_NW, 0, st>>>(A, a.Q, a.scales, a.zeros, a.Y, a.y_bf16,
                                                                        a.m, a.d_in, a.d_out, a.group, a.ngroups,
                                                                        nwords, a.part, a.counters, nsplit, align);
    else
        dq_gemm_ring_kernel<BITS, KC, false><<<grid, 64 * GR_NW, 0, st>>>(A, a.Q, a.scales, a.zeros, a.Y, a.y_bf16,
                                                                         a.m, a.d_in, a.d_out, a.group, a.ngroups,
                                                                         nwords, a.part, a.counters, 1, 1);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_gemm_bits(const DequantArgs &a, hipStream_t st) {
    const uint16_t *A = (const uint16_t *)a.A;
    if (a.perm) {
        if (permute_lds_ok(a.d_in)) {
            dq_permute_lds_kernel<<<(unsigned)a.m, 256, (size_t)a.d_in * 2, st>>>(A, a.perm, a.ap, a.d_in);
        } else {
            const int64_t n = a.m * a.d_in;
            dq_permute_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(A, a.perm, a.ap, a.m, a.d_in);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        A = a.ap;
    }
    const dim3 grid((unsigned)cdiv(a.m, GM_BM), (unsigned)cdiv(a.d_out, GM_BN));
    const int64_t nwords = cdiv((int64_t)BITS * a.d_in, 32);
    if constexpr (BITS <= 4) {
        if (gemm_ring_ok(64, a.d_in, a.d_out, BITS, a.group)) return launch_gemm_ring<BITS, 64>(A, a, nwords, st);
    }
    if (gemm_ring_ok(32, a.d_in, a.d_out, BITS, a.group)) return launch_gemm_ring<BITS, 32>(A, a, nwords, st);
    dq_gemm_kernel<BITS><<<grid, 512, 0, st>>>(A, a.Q, a.scales, a.zeros, a.Y, a.y_bf16, a.m, a.d_in, a.d_out,
                                               a.group, a.ngroups, nwords);
    return hipGetLastError();
}
}  // namespace

// The wide (MFMA) path takes bf16 activations with at least GM_MIN_M rows
// and whole 16-byte row pieces; everything else runs on the skinny path.
bool dequant_wide(int64_t m, int a_bf16, int64_t d_in) { return m >= GM_MIN_M && a_bf16 && d_in % 8 == 0; }

// Workspace: the skinny path's partial sums of its widest launch
// ([nsplit][M][d_out] fp32), then one counter per row tile (zero between
// calls), then (m >= GM_MIN_M) room for the activations in processing order.
DequantWs dequant_ws_layout(int64_t m, int64_t d_out, int64_t d_in, int bits) {
    DequantWs w{};
    size_t part = 0;
    for (int64_t m0 = 0; m0 < m; m0 += GV_MAX_M) {
        const int M = pad_m(std::min<int64_t>(GV_MAX_M, m - m0));
        const int s = gemv_splits(M, d_out, d_in, bits);
        if (s > 1) part = std::max(part, (size_t)s * M * d_out * sizeof(float));
    }
    size_t ncount = (size_t)cdiv(d_out, GV_ROWS);
    if (m >= GM_MIN_M) {
        // the wide path's split partial sums and one counter per tile
        const int s = gemm_splits(m, d_out, d_in);
        if (s > 1) part = std::max(part, (size_t)s * m * d_out * sizeof(float));
        ncount = std::max(ncount, (size_t)(cdiv(m, GM_BM) * cdiv(d_out, GM_BN)));
    }
    w.counters_off = align256(part);
    w.counters_bytes = ncount * sizeof(int32_t);
    w.ap_off = align256(w.counters_off + w.counters_bytes);
    const size_t ap = m >= GM_MIN_M ? (size_t)m * d_in * sizeof(uint16_t) : 0;
    w.bytes = m > 0 ? align256(w.ap_off + ap) : 0;
    return w;
}

hipError_t dequant_matmul_launch(const DequantArgs &a, hipStream_t st) {
    if (dequant_wide(a.m, a.a_bf16, a.d_in)) {
        switch (a.bits) {
            case 2: return launch_gemm_bits<2>(a, st);
            case 3: return launch_gemm_bits<3>(a, st);
            case 4: return launch_gemm_bits<4>(a, st);
            case 8: return launch_gemm_bits<8>(a, st);
        }
        return hipErrorInvalidValue;
    }
    switch (a.bits) {
        case 2: return launch_gemv_bits<2>(a, st);
        case 3: return launch_gemv_bits<3>(a, st);
        case 4: return launch_gemv_bits<4>(a, st);
        case 8: return launch_gemv_bits<8>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace gptq
