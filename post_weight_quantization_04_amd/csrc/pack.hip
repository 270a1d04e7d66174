// Stage 5: bit packing of the codes.  Row r's codes form a little-endian bit
// stream (code k at stream bits [bits*k, bits*k + bits)); word w holds stream
// bits [32w, 32w + 32).  For 4 bits that is eight codes per word; for 3 bits,
// 32 codes per three words with codes 10 and 21 straddling word boundaries.
// Storage form implied by the pages' 4x memory figures ("Optimization Gptq",
// memory table; "GPTQ" (wikiprompt.org), "Desempenho e Precisao").
// codes: [d_in][d_out] uint8 -> Qpacked: [words][d_out] uint32; one thread per
// (word, row) with rows fastest, so reads and writes are coalesced.
#include "common.h"

#include <algorithm>

namespace gptq {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ codes, int64_t d_out, int64_t d_in,
                                                   int bits, int64_t nwords, uint32_t *__restrict__ Q) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t w = blockIdx.y;
    if (r >= d_out) return;
    const int64_t bit0 = 32 * w;
    const int64_t k0 = bit0 / bits;
    const int64_t k1 = std::min<int64_t>(d_in - 1, (bit0 + 31) / bits);
    uint64_t acc = 0;
    for (int64_t k = k0; k <= k1; ++k) {
        const uint64_t v = codes[k * d_out + r];
        const int64_t pos = bits * k - bit0;
        acc |= (pos >= 0) ? (v << pos) : (v >> (-pos));
    }
    Q[w * d_out + r] = (uint32_t)acc;
}

// The same for d_out % 4 == 0 with four consecutive rows per thread: one
// 4-byte load per code (its four rows) and one 16-byte store per word.
__global__ __launch_bounds__(256) void pack4_kernel(const uint8_t *__restrict__ codes, int64_t d_out, int64_t d_in,
                                                    int bits, int64_t nwords, uint32_t *__restrict__ Q) {
    const int64_t r = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    const int64_t w = blockIdx.y;
    if (r >= d_out) return;
    const int64_t bit0 = 32 * w;
    const int64_t k0 = bit0 / bits;
    const int64_t k1 = std::min<int64_t>(d_in - 1, (bit0 + 31) / bits);
    uint64_t acc[4] = {0, 0, 0, 0};
    for (int64_t k = k0; k <= k1; ++k) {
        const uint32_t v4 = *(const uint32_t *)(codes + k * d_out + r);
        const int64_t pos = bits * k - bit0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint64_t v = (v4 >> (8 * u)) & 0xffu;
            acc[u] |= (pos >= 0) ? (v << pos) : (v >> (-pos));
        }
    }
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    *(u32x4 *)(Q + w * d_out + r) = u32x4{(unsigned)acc[0], (unsigned)acc[1], (unsigned)acc[2], (unsigned)acc[3]};
}

}  // namespace

hipError_t pack_launch(const uint8_t *codes, int64_t d_out, int64_t d_in, int bits, uint32_t *Qpacked,
                       hipStream_t st) {
    const int64_t nwords = cdiv(bits * d_in, 32);
    const bool vec = (d_out % 4 == 0) && ((reinterpret_cast<uintptr_t>(codes) & 3) == 0) &&
                     ((reinterpret_cast<uintptr_t>(Qpacked) & 15) == 0);
    if (vec) {
        dim3 grid((unsigned)cdiv(d_out / 4, 256), (unsigned)nwords);
        pack4_kernel<<<grid, 256, 0, st>>>(codes, d_out, d_in, bits, nwords, Qpacked);
    } else {
        dim3 grid((unsigned)cdiv(d_out, 256), (unsigned)nwords);
        pack_kernel<<<grid, 256, 0, st>>>(codes, d_out, d_in, bits, nwords, Qpacked);
    }
    return hipGetLastError();
}

}  // namespace gptq
