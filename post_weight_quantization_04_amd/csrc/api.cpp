// C ABI of libgptq: argument validation, workspace layout and the launch
// sequence of the GPTQ layer quantizer.  Every stage of the method runs in the
// HIP kernels of this library; this file only checks arguments and enqueues.
#include "gptq.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace {

thread_local std::string g_err;

gptq_status fail(gptq_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
gptq_status fail(gptq_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

// An enum argument from a C caller (or a foreign-function binding) may hold
// any int.  Its bits are read as an int, since loading an out-of-range value
// as the C++ enum type is undefined.
template <class E>
int raw(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "C enums here are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}
bool valid_dtype(const gptq_dtype &t) { return raw(t) == GPTQ_F32 || raw(t) == GPTQ_BF16; }

#define HIPCHECK(expr)                                                                      \
    do {                                                                                    \
        hipError_t e_ = (expr);                                                             \
        if (e_ != hipSuccess) return fail(GPTQ_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

// ---------------------------------------------------------------------------
// stage timing
// ---------------------------------------------------------------------------
struct Profiler {
    unsigned mask = 0;   // bit s: stage s is timed
    std::mutex mu;
    std::vector<hipEvent_t> pool;
    struct Pending { int stage; hipEvent_t a, b; };
    std::vector<Pending> pending;
    double ms[GPTQ_NUM_STAGES] = {};
    int64_t launches[GPTQ_NUM_STAGES] = {};

    hipEvent_t get() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
};
Profiler g_prof;

// RAII: records an event pair around the enclosed launches when profiling is on
struct StageTimer {
    int stage;
    hipStream_t st;
    hipEvent_t a = nullptr;
    StageTimer(int s, hipStream_t stream) : stage(s), st(stream) {
        if (!((g_prof.mask >> s) & 1u)) return;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        a = g_prof.get();
        if (a && hipEventRecord(a, st) != hipSuccess) a = nullptr;
    }
    ~StageTimer() {
        if (!a) return;
        std::lock_guard<std::mutex> lk(g_prof.mu);
        hipEvent_t b = g_prof.get();
        if (b && hipEventRecord(b, st) == hipSuccess) g_prof.pending.push_back({stage, a, b});
    }
};

using gptq::align256;
using gptq::cdiv;

constexpr int BI_MAX = 256;   // widest block staged by the in-block kernel

struct LayerShape {
    int64_t d_out, d_in;
    int bits, group, block, block_int;   // group: effective (d_in for one group per row)
    int64_t groups, words;
};

bool valid_bits(int b) { return b == 2 || b == 3 || b == 4 || b == 8; }

// Internal block width: the requested block when it fits the in-block kernel,
// otherwise the widest width that keeps every group start on a block start.
int internal_block(int B, int g, int64_t d_in) {
    if (B <= BI_MAX) return B;
    if (g >= d_in) return BI_MAX;
    if (g <= BI_MAX) return (BI_MAX / g) * g;
    for (int c = BI_MAX; c >= 16; c -= 16)
        if (g % c == 0) return c;
    return 16;
}

gptq_status check_layer(int64_t d_out, int64_t d_in, int bits, int group_size, int block_size, LayerShape &L) {
    if (d_out < 1 || d_in < 1) return fail(GPTQ_EINVAL, "d_out and d_in must be >= 1 (got %lld, %lld)", (long long)d_out, (long long)d_in);
    if (d_in > (int64_t)1 << 30 || d_out > (int64_t)1 << 30) return fail(GPTQ_EINVAL, "dimension too large");
    if (!valid_bits(bits)) return fail(GPTQ_EINVAL, "bits must be 2, 3, 4 or 8 (got %d)", bits);
    if (block_size < 1) return fail(GPTQ_EINVAL, "block_size must be >= 1 (got %d)", block_size);
    int g;
    if (group_size == -1 || group_size >= d_in) {
        g = (int)d_in;
    } else {
        if (group_size < 1) return fail(GPTQ_EINVAL, "group_size must be -1 or >= 1 (got %d)", group_size);
        if (group_size % 16 != 0) return fail(GPTQ_EINVAL, "group_size must be a multiple of 16 (got %d)", group_size);
        if (block_size < d_in && block_size % group_size != 0)
            return fail(GPTQ_EINVAL, "block_size (%d) must be a multiple of group_size (%d)", block_size, group_size);
        g = group_size;
    }
    L.d_out = d_out;
    L.d_in = d_in;
    L.bits = bits;
    L.group = g;
    L.block = (int)std::min<int64_t>(block_size, d_in);
    L.block_int = internal_block(L.block, g, d_in);
    L.groups = cdiv(d_in, g);
    L.words = cdiv(bits * d_in, 32);
    return GPTQ_OK;
}

struct Workspace {
    float *R, *Wp, *E, *panel, *pt, *dinv, *dg, *ud, *uinv, *lam;
    uint8_t *codes;
    int32_t *rank, *info;
    size_t bytes;
};

Workspace layout(const LayerShape &L, char *base) {
    Workspace w{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *p = base ? base + off : nullptr;
        off += align256(bytes);
        return p;
    };
    const int64_t d = L.d_in;
    w.R = (float *)take(sizeof(float) * (size_t)d * d);
    w.Wp = (float *)take(sizeof(float) * (size_t)L.d_out * d);
    w.E = (float *)take(sizeof(float) * (size_t)gptq::far_blocks(L.block_int) * L.block_int * L.d_out);
    w.codes = (uint8_t *)take((size_t)d * L.d_out);
    w.panel = (float *)take(sizeof(float) * (size_t)d * gptq::FACT_NB);
    w.pt = (float *)take(gptq::factor_batch(d) > 1 ? sizeof(float) * (size_t)gptq::FACT_BATCH * gptq::FACT_NB * d : 0);
    w.dinv = (float *)take(sizeof(float) * 2 * gptq::FACT_NB * gptq::FACT_NB);  // ping-pong pair
    w.dg = (float *)take(sizeof(float) * d);
    w.ud = (float *)take(sizeof(float) * d);
    w.uinv = (float *)take(sizeof(float) * d);
    w.rank = (int32_t *)take(sizeof(int32_t) * d);
    w.lam = (float *)take(sizeof(float));
    w.info = (int32_t *)take(2 * sizeof(int32_t));   // pivot flag, step counter
    w.bytes = off;
    return w;
}

// damping, order, gathers, factorization, status sync, flip.
gptq_status run_factor(const float *H, int64_t d, float damp, int act_order, int32_t *perm, Workspace &w,
                       hipStream_t st) {
    HIPCHECK(hipMemsetAsync(w.info, 0, 2 * sizeof(int32_t), st));
    {
        StageTimer t(2, st);
        HIPCHECK(gptq::prep_diag_lambda(H, d, damp, w.dg, w.lam, st));
        HIPCHECK(gptq::prep_perm(w.dg, d, act_order, w.rank, perm, st));
        HIPCHECK(gptq::prep_gather_h(H, perm, w.lam, d, w.R, st));
    }
    {
        StageTimer t(3, st);
        HIPCHECK(gptq::factor_launch(w.R, d, w.panel, w.pt, w.dinv, w.info, st));
    }
    return GPTQ_OK;
}

// Stages 3-5 for one layer on the factor already in the workspace: gather
// the layer's weights into processing order, the batched in-block and
// trailing updates, packing.
gptq_status quantize_rows(const void *W, int w_bf16, int64_t d_out, int64_t d_in, int bits, int group, int block_int,
                          const int32_t *perm, uint32_t *Qpacked, float *scales, float *zeros, Workspace &w,
                          hipStream_t st) {
    {
        StageTimer t(2, st);
        HIPCHECK(gptq::prep_gather_w(W, w_bf16, perm, d_out, d_in, w.Wp, st));
    }
    gptq::QuantArgs qa{};
    qa.Wp = w.Wp;
    qa.U = w.R;
    qa.ud = w.ud;
    qa.uinv = w.uinv;
    qa.E = w.E;
    qa.codes = w.codes;
    qa.scales = scales;
    qa.zeros = zeros;
    qa.d_out = d_out;
    qa.d_in = d_in;
    qa.bits = bits;
    qa.group = group;
    qa.block = block_int;
    // Blocks go in batches of far_blocks(B); the errors of a batch's blocks are
    // stacked in E (block t of the batch at rows t*B..).  One in-block launch
    // takes the whole batch, each block first applying the batch's earlier
    // errors to its own columns (the near update); then one product applies
    // all of them to every column beyond.  A group wider than a block takes
    // its parameters from all its columns at its start, so a batch also ends
    // before such a group begins.
    const int64_t B = block_int;
    for (int64_t pend0 = 0; pend0 < d_in;) {
        // one batch: up to far_blocks(B) blocks, ending early after a block whose
        // end starts a group wider than a block
        int nblk = 0;
        int64_t e = pend0;
        while (nblk < gptq::far_blocks(B) && e < d_in) {
            e = std::min<int64_t>(e + B, d_in);
            ++nblk;
            if (group > B && e % group == 0) break;
        }
        {
            StageTimer t(5, st);
            gptq::QuantArgs qb = qa;
            qb.E = w.E;
            qb.En = w.E;
            qb.near_row0 = pend0;
            HIPCHECK(gptq::quant_block_launch(qb, pend0, nblk, B, st));
        }
        if (e >= d_in) break;
        {
            StageTimer t(6, st);
            HIPCHECK(gptq::trail_launch(qa, pend0, e - pend0, e, d_in, st));
        }
        pend0 = e;
    }
    {
        StageTimer t(7, st);
        HIPCHECK(gptq::pack_launch(w.codes, d_out, d_in, bits, Qpacked, st));
    }
    return GPTQ_OK;
}

// The factorization's pivot flag, read once everything has been enqueued so
// that the device never idles waiting for the host in the middle of a layer.
// On a bad pivot the later stages ran on non-finite values; they index no
// memory by data, so they finish normally and their outputs are discarded.
gptq_status read_pivot_flag(const Workspace &w, hipStream_t st) {
    int32_t info = 0;
    HIPCHECK(hipMemcpyAsync(&info, w.info, sizeof(int32_t), hipMemcpyDeviceToHost, st));
    HIPCHECK(hipStreamSynchronize(st));
    if (info == gptq::FACTOR_SYNC_TIMEOUT)
        return fail(GPTQ_EHIP, "factorization: the look-ahead gave up waiting for the diagonal update");
    if (info != 0)
        return fail(GPTQ_ENOTSPD, "damped Hessian is not positive definite (pivot %lld of the reversed order)",
                    (long long)info - 1);
    return GPTQ_OK;
}

gptq_status check_dequant(int64_t m, int64_t d_out, int64_t d_in, int bits, int group_size, int &g_eff) {
    if (m < 0) return fail(GPTQ_EINVAL, "m must be >= 0");
    if (d_out < 1 || d_in < 1) return fail(GPTQ_EINVAL, "d_out and d_in must be >= 1");
    if (d_in > (int64_t)1 << 30 || d_out > (int64_t)1 << 30) return fail(GPTQ_EINVAL, "dimension too large");
    if (!valid_bits(bits)) return fail(GPTQ_EINVAL, "bits must be 2, 3, 4 or 8 (got %d)", bits);
    if (group_size == -1 || group_size >= d_in) {
        g_eff = (int)d_in;
    } else {
        if (group_size < 1 || group_size % 16 != 0)
            return fail(GPTQ_EINVAL, "group_size must be -1 or a multiple of 16 (got %d)", group_size);
        g_eff = group_size;
    }
    return GPTQ_OK;
}

}  // namespace

extern "C" {

const char *gptq_version(void) { return "libgptq 0.1 (gfx950)"; }

void gptq_profile_enable(int stage_mask) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    g_prof.mask = (unsigned)stage_mask & ((1u << GPTQ_NUM_STAGES) - 1u);
}

const char *gptq_profile_stage_name(int stage) {
    static const char *names[GPTQ_NUM_STAGES] = {"hessian_product", "hessian_reduce", "prep_gather", "factor",
                                                 "flip", "quant_block", "trail_update", "pack"};
    return (stage >= 0 && stage < GPTQ_NUM_STAGES) ? names[stage] : "";
}

gptq_status gptq_profile_read(gptq_profile *out, int reset) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    size_t done = 0;
    for (; done < g_prof.pending.size(); ++done) {
        const auto &p = g_prof.pending[done];
        float ms = 0.f;
        if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
            // the pairs already summed go back to the pool exactly once
            g_prof.pending.erase(g_prof.pending.begin(), g_prof.pending.begin() + done);
            return fail(GPTQ_EHIP, "profile event query failed");
        }
        g_prof.ms[p.stage] += ms;
        g_prof.launches[p.stage] += 1;
        g_prof.pool.push_back(p.a);
        g_prof.pool.push_back(p.b);
    }
    g_prof.pending.clear();
    if (out) {
        for (int i = 0; i < GPTQ_NUM_STAGES; ++i) {
            out->ms[i] = g_prof.ms[i];
            out->launches[i] = g_prof.launches[i];
        }
    }
    if (reset) {
        for (int i = 0; i < GPTQ_NUM_STAGES; ++i) {
            g_prof.ms[i] = 0.0;
            g_prof.launches[i] = 0;
        }
    }
    return GPTQ_OK;
}

const char *gptq_last_error(void) { return g_err.c_str(); }

const char *gptq_status_string(gptq_status s) {
    switch (raw(s)) {
        case GPTQ_OK: return "ok";
        case GPTQ_EINVAL: return "invalid argument";
        case GPTQ_ENOTSPD: return "damped Hessian not positive definite";
        case GPTQ_EHIP: return "HIP runtime error";
        case GPTQ_ENOMEM: return "workspace too small";
    }
    return "unknown status";
}

int64_t gptq_packed_words(int64_t d_in, int bits) {
    if (d_in < 0 || !valid_bits(bits)) return -1;
    // ceil(bits * d_in / 32) without forming bits * d_in (no overflow for any d_in)
    return (d_in / 32) * bits + cdiv((d_in % 32) * bits, 32);
}

int64_t gptq_num_groups(int64_t d_in, int group_size) {
    if (d_in < 1) return -1;
    if (group_size == -1 || group_size >= d_in) return 1;
    if (group_size < 1) return -1;
    return cdiv(d_in, group_size);
}

size_t gptq_hessian_workspace_size(int64_t n, int64_t d_in, gptq_dtype x_dtype) {
    if (n < 0 || d_in < 1 || d_in > (int64_t)1 << 20 || !valid_dtype(x_dtype)) return 0;
    if (n == 0) return 0;
    return gptq::hessian_ws_bytes(gptq::hessian_plan(n, d_in, x_dtype == GPTQ_BF16));
}

gptq_status gptq_hessian_accumulate(const void *X, gptq_dtype x_dtype, int64_t n, int64_t d_in, float *H,
                                    void *workspace, size_t workspace_bytes, void *stream) {
    g_err.clear();
    if (!valid_dtype(x_dtype)) return fail(GPTQ_EINVAL, "x_dtype must be GPTQ_F32 or GPTQ_BF16");
    if (n < 0) return fail(GPTQ_EINVAL, "n must be >= 0");
    if (d_in < 1 || d_in > (int64_t)1 << 20) return fail(GPTQ_EINVAL, "d_in must be in [1, 2^20]");
    if (!H) return fail(GPTQ_EINVAL, "H is NULL");
    if (n == 0) return GPTQ_OK;
    if (!X) return fail(GPTQ_EINVAL, "X is NULL");
    const gptq::HessPlan p = gptq::hessian_plan(n, d_in, x_dtype == GPTQ_BF16);
    const size_t need = gptq::hessian_ws_bytes(p);
    if (!workspace || workspace_bytes < need)
        return fail(GPTQ_ENOMEM, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    hipStream_t st = (hipStream_t)stream;
    {
        StageTimer t(0, st);
        HIPCHECK(gptq::hessian_product_launch(X, x_dtype == GPTQ_BF16, n, d_in, (float *)workspace, p, st));
    }
    {
        StageTimer t(1, st);
        HIPCHECK(gptq::hessian_reduce_launch(d_in, H, (const float *)workspace, p, st));
    }
    return GPTQ_OK;
}

int64_t gptq_hessian_noalloc_max_d_in(gptq_dtype x_dtype) {
    if (!valid_dtype(x_dtype)) return -1;
    // the largest d_in whose lower tiles fit the scratch with one token split
    const gptq::HessPlan p1 = gptq::hessian_plan(1, 1, x_dtype == GPTQ_BF16);
    const int64_t max_slots = (int64_t)(gptq::HESS_STATIC_SCRATCH_BYTES / ((size_t)p1.tile * p1.tile * sizeof(float)));
    int64_t nb = 0;
    while ((nb + 1) * (nb + 2) / 2 <= max_slots) ++nb;
    return nb * p1.tile;
}

gptq_status gptq_hessian_accumulate_noalloc(const void *X, gptq_dtype x_dtype, int64_t n, int64_t d_in, float *H,
                                            void *stream) {
    g_err.clear();
    if (!valid_dtype(x_dtype)) return fail(GPTQ_EINVAL, "x_dtype must be GPTQ_F32 or GPTQ_BF16");
    if (n < 0) return fail(GPTQ_EINVAL, "n must be >= 0");
    if (d_in < 1 || d_in > (int64_t)1 << 20) return fail(GPTQ_EINVAL, "d_in must be in [1, 2^20]");
    if (!H) return fail(GPTQ_EINVAL, "H is NULL");
    if (n == 0) return GPTQ_OK;
    if (!X) return fail(GPTQ_EINVAL, "X is NULL");
    const int bf = x_dtype == GPTQ_BF16;
    const gptq::HessPlan p1 = gptq::hessian_plan(1, 1, bf);
    const int64_t max_slots = (int64_t)(gptq::HESS_STATIC_SCRATCH_BYTES / ((size_t)p1.tile * p1.tile * sizeof(float)));
    const gptq::HessPlan p = gptq::hessian_plan(n, d_in, bf, max_slots);
    if (p.slots > max_slots || gptq::hessian_ws_bytes(p) > gptq::HESS_STATIC_SCRATCH_BYTES)
        return fail(GPTQ_EINVAL, "d_in = %lld needs %lld partial tiles; the static scratch of %zu MiB holds %lld "
                    "(d_in <= %lld)", (long long)d_in, (long long)p.slots, gptq::HESS_STATIC_SCRATCH_BYTES >> 20,
                    (long long)max_slots, (long long)gptq_hessian_noalloc_max_d_in(x_dtype));
    void *scratch = nullptr;
    HIPCHECK(gptq::hessian_static_scratch(&scratch));
    hipStream_t st = (hipStream_t)stream;
    {
        StageTimer t(0, st);
        HIPCHECK(gptq::hessian_product_launch(X, bf, n, d_in, (float *)scratch, p, st));
    }
    {
        StageTimer t(1, st);
        HIPCHECK(gptq::hessian_reduce_launch(d_in, H, (const float *)scratch, p, st));
    }
    return GPTQ_OK;
}

size_t gptq_quantize_layer_workspace_size(int64_t d_out, int64_t d_in, int bits, int group_size, int block_size,
                                          int act_order) {
    (void)act_order;
    LayerShape L{};
    if (check_layer(d_out, d_in, bits, group_size, block_size, L) != GPTQ_OK) return 0;
    return layout(L, nullptr).bytes;
}

gptq_status gptq_quantize_layer(const void *W, gptq_dtype w_dtype, int64_t d_out, int64_t d_in, const float *H,
                                int bits, int group_size, int block_size, float damp, int act_order,
                                uint32_t *Qpacked, float *scales, float *zeros, int32_t *perm, void *workspace,
                                size_t workspace_bytes, void *stream) {
    // checked before w_dtype is passed on as an enum value
    if (!valid_dtype(w_dtype)) return fail(GPTQ_EINVAL, "w_dtype must be GPTQ_F32 or GPTQ_BF16");
    return gptq_quantize_layers(1, &W, w_dtype, &d_out, d_in, H, bits, group_size, block_size, damp, act_order,
                                &Qpacked, &scales, &zeros, perm, workspace, workspace_bytes, stream);
}

size_t gptq_quantize_layers_workspace_size(int n_layers, const int64_t *d_out, int64_t d_in, int bits, int group_size,
                                           int block_size, int act_order) {
    if (n_layers < 1 || !d_out) return 0;
    int64_t dmax = 0;
    for (int l = 0; l < n_layers; ++l) dmax = std::max(dmax, d_out[l]);
    return gptq_quantize_layer_workspace_size(dmax, d_in, bits, group_size, block_size, act_order);
}

gptq_status gptq_quantize_layers(int n_layers, const void *const *W, gptq_dtype w_dtype, const int64_t *d_out,
                                 int64_t d_in, const float *H, int bits, int group_size, int block_size, float damp,
                                 int act_order, uint32_t *const *Qpacked, float *const *scales, float *const *zeros,
                                 int32_t *perm, void *workspace, size_t workspace_bytes, void *stream) {
    g_err.clear();
    if (n_layers < 1 || n_layers > 4096) return fail(GPTQ_EINVAL, "n_layers must be in [1, 4096] (got %d)", n_layers);
    if (!W || !d_out || !Qpacked || !scales || !zeros) return fail(GPTQ_EINVAL, "a required array is NULL");
    LayerShape Lmax{};
    int64_t dmax = 0;
    for (int l = 0; l < n_layers; ++l) {
        LayerShape Ll{};
        gptq_status s = check_layer(d_out[l], d_in, bits, group_size, block_size, Ll);
        if (s != GPTQ_OK) return s;
        if (!W[l] || !Qpacked[l] || !scales[l] || !zeros[l])
            return fail(GPTQ_EINVAL, "a required pointer of layer %d is NULL", l);
        if (d_out[l] > dmax) {
            dmax = d_out[l];
            Lmax = Ll;
        }
    }
    if (!valid_dtype(w_dtype)) return fail(GPTQ_EINVAL, "w_dtype must be GPTQ_F32 or GPTQ_BF16");
    if (!std::isfinite(damp) || damp < 0.f) return fail(GPTQ_EINVAL, "damp must be finite and >= 0");
    if (act_order != 0 && act_order != 1) return fail(GPTQ_EINVAL, "act_order must be 0 or 1");
    if (!H || !perm) return fail(GPTQ_EINVAL, "a required pointer is NULL");
    const size_t need = layout(Lmax, nullptr).bytes;
    if (!workspace || workspace_bytes < need)
        return fail(GPTQ_ENOMEM, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    hipStream_t st = (hipStream_t)stream;
    // every buffer sized for the widest layer serves the narrower ones too
    // (their row strides are their own d_out)
    Workspace w = layout(Lmax, (char *)workspace);

    gptq_status s = run_factor(H, d_in, damp, act_order, perm, w, st);
    if (s != GPTQ_OK) return s;
    {
        StageTimer t(4, st);
        HIPCHECK(gptq::factor_flip(w.R, d_in, w.ud, w.uinv, 0, st));
    }
    for (int l = 0; l < n_layers; ++l) {
        s = quantize_rows(W[l], w_dtype == GPTQ_BF16, d_out[l], d_in, bits, Lmax.group, Lmax.block_int, perm,
                          Qpacked[l], scales[l], zeros[l], w, st);
        if (s != GPTQ_OK) return s;
    }
    return read_pivot_flag(w, st);
}

size_t gptq_dequant_matmul_workspace_size(int64_t m, int64_t d_out, int64_t d_in, int bits, int group_size) {
    int g = 0;
    if (check_dequant(m, d_out, d_in, bits, group_size, g) != GPTQ_OK) return 0;
    if (m == 0) return 0;
    return gptq::dequant_ws_layout(m, d_out, d_in, bits).bytes;
}

gptq_status gptq_dequant_matmul(const void *A, gptq_dtype a_dtype, int64_t m, int64_t d_in, const uint32_t *Qpacked,
                                const float *scales, const float *zeros, const int32_t *perm, int64_t d_out,
                                int bits, int group_size, void *Y, gptq_dtype y_dtype, void *workspace,
                                size_t workspace_bytes, void *stream) {
    g_err.clear();
    int g = 0;
    gptq_status s = check_dequant(m, d_out, d_in, bits, group_size, g);
    if (s != GPTQ_OK) return s;
    if (!valid_dtype(a_dtype)) return fail(GPTQ_EINVAL, "a_dtype must be GPTQ_F32 or GPTQ_BF16");
    if (!valid_dtype(y_dtype)) return fail(GPTQ_EINVAL, "y_dtype must be GPTQ_F32 or GPTQ_BF16");
    if (m == 0) return GPTQ_OK;
    if (!A || !Qpacked || !scales || !zeros || !Y) return fail(GPTQ_EINVAL, "a required pointer is NULL");
    const gptq::DequantWs wl = gptq::dequant_ws_layout(m, d_out, d_in, bits);
    const size_t need = wl.bytes;
    if (!workspace || workspace_bytes < need)
        return fail(GPTQ_ENOMEM, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    gptq::DequantArgs a{};
    a.A = A;
    a.a_bf16 = a_dtype == GPTQ_BF16;
    a.perm = perm;
    a.Q = Qpacked;
    a.scales = scales;
    a.zeros = zeros;
    a.Y = Y;
    a.y_bf16 = y_dtype == GPTQ_BF16;
    a.part = (float *)workspace;
    a.counters = (int32_t *)((char *)workspace + wl.counters_off);
    a.ap = (uint16_t *)((char *)workspace + wl.ap_off);
    a.m = m;
    a.d_in = d_in;
    a.d_out = d_out;
    a.bits = bits;
    a.group = g;
    a.ngroups = (int)cdiv(d_in, g);
    HIPCHECK(gptq::dequant_matmul_launch(a, (hipStream_t)stream));
    return GPTQ_OK;
}

gptq_status gptq_inverse_factor(const float *H, int64_t d_in, float damp, int act_order, int32_t *perm, float *U,
                                void *workspace, size_t workspace_bytes, void *stream) {
    g_err.clear();
    LayerShape L{};
    gptq_status s = check_layer(1, d_in, 4, -1, 1, L);
    if (s != GPTQ_OK) return s;
    if (!std::isfinite(damp) || damp < 0.f) return fail(GPTQ_EINVAL, "damp must be finite and >= 0");
    if (act_order != 0 && act_order != 1) return fail(GPTQ_EINVAL, "act_order must be 0 or 1");
    if (!H || !perm || !U) return fail(GPTQ_EINVAL, "a required pointer is NULL");
    const size_t need = layout(L, nullptr).bytes;
    if (!workspace || workspace_bytes < need)
        return fail(GPTQ_ENOMEM, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
    hipStream_t st = (hipStream_t)stream;
    Workspace w = layout(L, (char *)workspace);
    s = run_factor(H, d_in, damp, act_order, perm, w, st);
    if (s != GPTQ_OK) return s;
    HIPCHECK(gptq::factor_flip(w.R, d_in, w.ud, w.uinv, 1, st));
    HIPCHECK(hipMemcpyAsync(U, w.R, sizeof(float) * (size_t)d_in * d_in, hipMemcpyDeviceToDevice, st));
    return read_pivot_flag(w, st);
}

}  // extern "C"
