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

constexpr int RANK_TILE = 1024;

// rank[i] += #{j in this group's slice : j precedes i}
__global__ __launch_bounds__(256) void rank_kernel(const float *__restrict__ dg, int64_t d,
                                                   int32_t *__restrict__ rank) {
    __shared__ float kj[RANK_TILE];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t j0 = (int64_t)blockIdx.y * RANK_TILE;
    const int64_t j1 = std::min<int64_t>(d, j0 + RANK_TILE);
    for (int64_t j = j0 + threadIdx.x; j < j1; j += 256) kj[j - j0] = order_key(dg[j]);
    __syncthreads();
    if (i >= d) return;
    const float ki = order_key(dg[i]);
    int cnt = 0;
    for (int64_t j = j0; j < j1; ++j) {
        const float v = kj[j - j0];
        cnt += (v > ki) || (v == ki && j < i);
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
    gather_h_kernel<<<(unsigned)d, 256, 0, st>>>(H, perm, lam, d, R);
    return hipGetLastError();
}

hipError_t prep_gather_w(const void *W, int is_bf16, const int32_t *perm, int64_t d_out, int64_t d_in, float *Wp,
                         hipStream_t st) {
    if (is_bf16)
        gather_w_kernel<true><<<(unsigned)d_out, 256, 0, st>>>(W, perm, d_in, Wp);
    else
        gather_w_kernel<false><<<(unsigned)d_out, 256, 0, st>>>(W, perm, d_in, Wp);
    return hipGetLastError();
}

}  // namespace gptq
