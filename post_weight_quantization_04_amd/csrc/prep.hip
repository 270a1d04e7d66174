// Stage 2a: damping constant, activation order and the gathers that build the
// factorization input and the fp32 working weights.
//   lambda = damp * mean(diag H)   ("Algorithme complet (pseudo-code)" step 1,
//                                   damp_percent of "Configuracoes de quantizacao")
//   perm   = columns by descending diag(H), ties to the lower index
//            (desc_act, "ordre par importance" in "Quantification avec AutoGPTQ")
#include "common.h"

#include <algorithm>

namespace gptq {

namespace {

// diag(H) and lambda; one work group, fixed-order reduction in fp64.
__global__ __launch_bounds__(1024) void diag_lambda_kernel(const float *__restrict__ H, int64_t d, float damp,
                                                           float *__restrict__ dg, float *__restrict__ lam) {
    __shared__ double part[1024];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < d; i += 1024) {
        const float v = H[i * d + i];
        dg[i] = v;
        s += (double)v;
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) lam[0] = (float)((double)damp * (part[0] / (double)d));
}

// Ordering key: NaN sorts last; i precedes j iff key_i > key_j or equal keys
// and i < j.  That is a strict total order, so the ranks form a permutation.
__device__ __forceinline__ float order_key(float v) { return (v != v) ? -__builtin_huge_valf() : v; }

constexpr int RANK_TILE = 256;

// rank[i] += #{j in this group's slice : j precedes i}.  The slice's keys go
// to LDS, padded with -inf past d (a padded j >= d never precedes any i < d),
// and are read back four at a time.  Slices of 256 give d = 4096 a grid of
// 256 groups; with slices of 1024 read one key per step, the 64 groups of
// that size waited on LDS for every comparison (≈ 120 us at d = 4096).
__global__ __launch_bounds__(256) void rank_kernel(const float *__restrict__ dg, int64_t d,
                                                   int32_t *__restrict__ rank) {
    __shared__ __attribute__((aligned(16))) float kj[RANK_TILE];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t j0 = (int64_t)blockIdx.y * RANK_TILE;
    for (int t = threadIdx.x; t < RANK_TILE; t += 256)
        kj[t] = (j0 + t < d) ? order_key(dg[j0 + t]) : -__builtin_huge_valf();
    __syncthreads();
    if (i >= d) return;
    const float ki = order_key(dg[i]);
    int cnt = 0;
#pragma unroll 8
    for (int t = 0; t < RANK_TILE; t += 4) {
        const f32x4 v = *(const f32x4 *)(kj + t);
        const int64_t j = j0 + t;
        cnt += (v.x > ki) || (v.x == ki && j + 0 < i);
        cnt += (v.y > ki) || (v.y == ki && j + 1 < i);
        cnt += (v.z > ki) || (v.z == ki && j + 2 < i);
        cnt += (v.w > ki) || (v.w == ki && j + 3 < i);
    }
    if (cnt) atomicAdd(rank + i, cnt);
}

__global__ void scatter_perm_kernel(const int32_t *__restrict__ rank, int64_t d, int32_t *__restrict__ perm) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < d) perm[rank[i]] = (int32_t)i;
}

__global__ void iota_kernel(int32_t *__restrict__ perm, int64_t d) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < d) perm[i] = (int32_t)i;
}

__global__ void zero_i32_kernel(int32_t *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

constexpr int GATHER_UNROLL = 8;   // elements per thread in flight

// R[a][b] = H[p(a)][p(b)] (+ lambda if a == b), p(a) = perm[d-1-a]; one row per
// block, eight elements per thread at a time (index loads, then the gathered
// loads, then the stores).
__global__ __launch_bounds__(256) void gather_h_kernel(const float *__restrict__ H, const int32_t *__restrict__ perm,
                                                       const float *__restrict__ lam, int64_t d,
                                                       float *__restrict__ R) {
    const int64_t a = blockIdx.x;
    const int64_t pa = perm[d - 1 - a];
    const float l = lam[0];
    const float *hrow = H + pa * d;
    float *rrow = R + a * d;
    for (int64_t b0 = threadIdx.x; b0 < d; b0 += 256 * GATHER_UNROLL) {
        int32_t pb[GATHER_UNROLL];
        float v[GATHER_UNROLL];
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) {
            const int64_t b = b0 + 256 * u;
            pb[u] = (b < d) ? perm[d - 1 - b] : 0;
        }
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) v[u] = hrow[pb[u]];
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) {
            const int64_t b = b0 + 256 * u;
            if (b < d) rrow[b] = (b == a) ? v[u] + l : v[u];
        }
    }
}

// Row gathers through LDS (16-byte aligned rows of at most LDS_GATHER_MAX
// values): one row per work group; the source row is copied into LDS with
// coalesced 16-byte loads (indices clamped into the row, so the loads carry
// no guards), the permuted values are read back from LDS and the output row
// is written with 16-byte stores.  Read from global memory one 4-byte element
// per lane at permuted positions, every load instruction touched up to 64
// cache lines.
//   H: dst[a][b] = H[p(a)][p(b)] (+ lambda if a == b), p(x) = perm[d-1-x]
//   W: dst[r][k] = W[r][perm[k]] (bf16 widened exactly to fp32)
constexpr int64_t LDS_GATHER_MAX = 40960;   // floats of one staged row (160 KB)
constexpr int GATHER_BATCH = 8;             // 16-byte pieces per thread in flight

template <int MODE>   // 0: H, 1: fp32 W, 2: bf16 W
__global__ __launch_bounds__(256) void gather_lds_kernel(const void *__restrict__ src, const int32_t *__restrict__ perm,
                                                         const float *__restrict__ lam, int64_t n,
                                                         float *__restrict__ dst) {
    extern __shared__ __attribute__((aligned(16))) float srow[];
    const int64_t a = blockIdx.x;
    const int tid = threadIdx.x;
    // stage the source row: n / 4 fp32 pieces, or n / 8 bf16 pieces
    if (MODE == 2) {
        const u32x4 *s8 = (const u32x4 *)((const uint16_t *)src + a * n);
        const int np = (int)(n / 8);
        for (int i0 = tid; i0 < np; i0 += 256 * GATHER_BATCH) {
            u32x4 v[GATHER_BATCH];
#pragma unroll
            for (int u = 0; u < GATHER_BATCH; ++u) v[u] = s8[min(i0 + 256 * u, np - 1)];
#pragma unroll
            for (int u = 0; u < GATHER_BATCH; ++u) {
                const int i = i0 + 256 * u;
                if (i < np) {
                    f32x4 lo, hi;
                    lo.x = __uint_as_float(v[u].x << 16); lo.y = __uint_as_float(v[u].x & 0xffff0000u);
                    lo.z = __uint_as_float(v[u].y << 16); lo.w = __uint_as_float(v[u].y & 0xffff0000u);
                    hi.x = __uint_as_float(v[u].z << 16); hi.y = __uint_as_float(v[u].z & 0xffff0000u);
                    hi.z = __uint_as_float(v[u].w << 16); hi.w = __uint_as_float(v[u].w & 0xffff0000u);
                    *(f32x4 *)(srow + 8 * i) = lo;
                    *(f32x4 *)(srow + 8 * i + 4) = hi;
                }
            }
        }
    } else {
        const int64_t srow_idx = (MODE == 0) ? (int64_t)perm[n - 1 - a] : a;
        const f32x4 *s4 = (const f32x4 *)((const float *)src + srow_idx * n);
        const int np = (int)(n / 4);
        for (int i0 = tid; i0 < np; i0 += 256 * GATHER_BATCH) {
            f32x4 v[GATHER_BATCH];
#pragma unroll
            for (int u = 0; u < GATHER_BATCH; ++u) v[u] = s4[min(i0 + 256 * u, np - 1)];
#pragma unroll
            for (int u = 0; u < GATHER_BATCH; ++u) {
                const int i = i0 + 256 * u;
                if (i < np) *(f32x4 *)(srow + 4 * i) = v[u];
            }
        }
    }
    __syncthreads();
    // output pieces of four: indices as one 16-byte load (reversed for H)
    const float l = (MODE == 0) ? lam[0] : 0.f;
    float *drow = dst + a * n;
    const int nq = (int)(n / 4);
    for (int j0 = tid; j0 < nq; j0 += 256 * GATHER_BATCH) {
        int32_t pc[GATHER_BATCH][4];
#pragma unroll
        for (int u = 0; u < GATHER_BATCH; ++u) {
            const int64_t b = 4 * (int64_t)min(j0 + 256 * u, nq - 1);
            if (MODE == 0) {
                const int4 q = *(const int4 *)(perm + (n - 4 - b));   // perm[n-1-b-3 .. n-1-b]
                pc[u][0] = q.w; pc[u][1] = q.z; pc[u][2] = q.y; pc[u][3] = q.x;
            } else {
                const int4 q = *(const int4 *)(perm + b);
                pc[u][0] = q.x; pc[u][1] = q.y; pc[u][2] = q.z; pc[u][3] = q.w;
            }
        }
#pragma unroll
        for (int u = 0; u < GATHER_BATCH; ++u) {
            const int j = j0 + 256 * u;
            if (j < nq) {
                const int64_t b = 4 * (int64_t)j;
                f32x4 v = {srow[pc[u][0]], srow[pc[u][1]], srow[pc[u][2]], srow[pc[u][3]]};
                if (MODE == 0 && a >= b && a < b + 4) {
                    if (a == b + 0) v.x += l;
                    if (a == b + 1) v.y += l;
                    if (a == b + 2) v.z += l;
                    if (a == b + 3) v.w += l;
                }
                *(f32x4 *)(drow + b) = v;
            }
        }
    }
}

// dynamic LDS above the default limit must be allowed per kernel, once
template <int MODE>
bool gather_lds_ok(int64_t n, bool aligned) {
    if (!aligned || n <= 0 || n > LDS_GATHER_MAX) return false;
    static int state = 0;   // 0 unknown, 1 allowed, -1 refused
    if (state == 0)
        state = (hipFuncSetAttribute((const void *)gather_lds_kernel<MODE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)(LDS_GATHER_MAX * 4)) == hipSuccess)
                    ? 1
                    : -1;
    if (state < 0) (void)hipGetLastError();
    return state > 0;
}

template <bool BF16>
__global__ __launch_bounds__(256) void gather_w_kernel(const void *__restrict__ W, const int32_t *__restrict__ perm,
                                                       int64_t d_in, float *__restrict__ Wp) {
    const int64_t r = blockIdx.x;
    for (int64_t k0 = threadIdx.x; k0 < d_in; k0 += 256 * GATHER_UNROLL) {
        int32_t c[GATHER_UNROLL];
        float v[GATHER_UNROLL];
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) {
            const int64_t k = k0 + 256 * u;
            c[u] = (k < d_in) ? perm[k] : 0;
        }
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) {
            if (BF16) {
                const unsigned short b = ((const unsigned short *)W)[r * d_in + c[u]];
                v[u] = __uint_as_float((unsigned)b << 16);
            } else {
                v[u] = ((const float *)W)[r * d_in + c[u]];
            }
        }
#pragma unroll
        for (int u = 0; u < GATHER_UNROLL; ++u) {
            const int64_t k = k0 + 256 * u;
            if (k < d_in) Wp[r * d_in + k] = v[u];
        }
    }
}

}  // namespace

hipError_t prep_diag_lambda(const float *H, int64_t d, float damp, float *dg, float *lam, hipStream_t st) {
    diag_lambda_kernel<<<1, 1024, 0, st>>>(H, d, damp, dg, lam);
    return hipGetLastError();
}

hipError_t prep_perm(const float *dg, int64_t d, int act_order, int32_t *rank, int32_t *perm, hipStream_t st) {
    const unsigned g = (unsigned)cdiv(d, 256);
    if (!act_order) {
        iota_kernel<<<g, 256, 0, st>>>(perm, d);
        return hipGetLastError();
    }
    zero_i32_kernel<<<g, 256, 0, st>>>(rank, d);
    dim3 grid(g, (unsigned)cdiv(d, RANK_TILE));
    rank_kernel<<<grid, 256, 0, st>>>(dg, d, rank);
    scatter_perm_kernel<<<g, 256, 0, st>>>(rank, d, perm);
    return hipGetLastError();
}

hipError_t prep_gather_h(const float *H, const int32_t *perm, const float *lam, int64_t d, float *R,
                         hipStream_t st) {
    const bool aligned = d % 4 == 0 && reinterpret_cast<uintptr_t>(H) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(R) % 16 == 0 && reinterpret_cast<uintptr_t>(perm) % 16 == 0;
    if (gather_lds_ok<0>(d, aligned))
        gather_lds_kernel<0><<<(unsigned)d, 256, (size_t)d * 4, st>>>(H, perm, lam, d, R);
    else
        gather_h_kernel<<<(unsigned)d, 256, 0, st>>>(H, perm, lam, d, R);
    return hipGetLastError();
}

hipError_t prep_gather_w(const void *W, int is_bf16, const int32_t *perm, int64_t d_out, int64_t d_in, float *Wp,
                         hipStream_t st) {
    const bool aligned = d_in % (is_bf16 ? 8 : 4) == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0 &&
                         reinterpret_cast<uintptr_t>(Wp) % 16 == 0 && reinterpret_cast<uintptr_t>(perm) % 16 == 0;
    if (is_bf16 && gather_lds_ok<2>(d_in, aligned))
        gather_lds_kernel<2><<<(unsigned)d_out, 256, (size_t)d_in * 4, st>>>(W, perm, nullptr, d_in, Wp);
    else if (!is_bf16 && gather_lds_ok<1>(d_in, aligned))
        gather_lds_kernel<1><<<(unsigned)d_out, 256, (size_t)d_in * 4, st>>>(W, perm, nullptr, d_in, Wp);
    else if (is_bf16)
        gather_w_kernel<true><<<(unsigned)d_out, 256, 0, st>>>(W, perm, d_in, Wp);
    else
        gather_w_kernel<false><<<(unsigned)d_out, 256, 0, st>>>(W, perm, d_in, Wp);
    return hipGetLastError();
}

}  // namespace gptq
