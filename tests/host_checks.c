/* Host-side checks of libgptq's C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host code of the library (see
 * test_host_sanitizers.py).  Every call here fails argument validation on the
 * host or is a host-only helper, so nothing reaches a GPU: the program runs on
 * a machine without one.  Exit status 0 and a final "ok" line on success. */
#include "gptq.h"

#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                               \
        }                                                             \
    } while (0)

/* the status and that the detail string names the argument */
#define EXPECT(call, status, needle)                                  \
    do {                                                              \
        gptq_status s_ = (call);                                      \
        if (s_ != (status)) {                                         \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d (%s)\n", __FILE__, __LINE__, #call, (int)s_, \
                    (int)(status), gptq_last_error());                \
            ++failures;                                               \
        } else if ((needle) != NULL && strstr(gptq_last_error(), (needle)) == NULL) { \
            fprintf(stderr, "%s:%d: detail '%s' lacks '%s'\n", __FILE__, __LINE__, gptq_last_error(), \
                    (const char *)(needle));                          \
            ++failures;                                               \
        }                                                             \
    } while (0)

/* never dereferenced: validation fails before any use */
#define FAKE ((void *)(uintptr_t)0x1000)

static void helpers(void) {
    CHECK(gptq_packed_words(4096, 4) == 512);
    CHECK(gptq_packed_words(33, 3) == 4);
    CHECK(gptq_packed_words(10, 5) == -1);
    CHECK(gptq_packed_words(-1, 4) == -1);
    CHECK(gptq_packed_words(INT64_MAX, 8) == -1 || gptq_packed_words(INT64_MAX, 8) > 0);
    CHECK(gptq_num_groups(11008, 128) == 86);
    CHECK(gptq_num_groups(4096, -1) == 1);
    CHECK(gptq_num_groups(100, 0) == -1);
    CHECK(gptq_num_groups(INT64_MAX, 16) > 0 || gptq_num_groups(INT64_MAX, 16) == -1);
    for (int s = -3; s < 8; ++s) CHECK(gptq_status_string((gptq_status)s) != NULL);
    for (int s = -3; s < GPTQ_NUM_STAGES + 3; ++s) CHECK(gptq_profile_stage_name(s) != NULL);
    CHECK(strstr(gptq_version(), "gfx950") != NULL);
}

static void sizes(void) {
    CHECK(gptq_quantize_layer_workspace_size(4096, 4096, 4, 128, 128, 0) > 0);
    CHECK(gptq_quantize_layer_workspace_size(4096, 4096, 5, 128, 128, 0) == 0);
    CHECK(gptq_quantize_layer_workspace_size(4096, 4096, 4, 100, 128, 0) == 0);
    CHECK(gptq_quantize_layer_workspace_size(0, 4096, 4, 128, 128, 0) == 0);
    CHECK(gptq_quantize_layer_workspace_size(INT64_MAX, INT64_MAX, 4, 128, 128, 1) == 0 ||
          gptq_quantize_layer_workspace_size(INT64_MAX, INT64_MAX, 4, 128, 128, 1) > 0);
    CHECK(gptq_hessian_workspace_size(262144, 4096, GPTQ_BF16) % 256 == 0);
    CHECK(gptq_hessian_workspace_size(0, 4096, GPTQ_BF16) == 0);
    CHECK(gptq_hessian_workspace_size(INT64_MAX, 4096, GPTQ_BF16) >= 0);
    CHECK(gptq_hessian_noalloc_max_d_in((gptq_dtype)7) == -1);
    CHECK(gptq_dequant_matmul_workspace_size(1, 4096, 4096, 4, 128) > 0);
    CHECK(gptq_dequant_matmul_workspace_size(1, 4096, 4096, 5, 128) == 0);
    const int64_t dout[3] = {4096, 1024, 1024};
    CHECK(gptq_quantize_layers_workspace_size(3, dout, 4096, 4, 128, 128, 0) ==
          gptq_quantize_layer_workspace_size(4096, 4096, 4, 128, 128, 0));
    CHECK(gptq_quantize_layers_workspace_size(0, dout, 4096, 4, 128, 128, 0) == 0);
    CHECK(gptq_quantize_layers_workspace_size(3, NULL, 4096, 4, 128, 128, 0) == 0);
}

static gptq_status q(const void *W, int dt, int64_t d_out, int64_t d_in, int bits, int g, int B, float damp,
                     int act, void *ws, size_t wsb) {
    return gptq_quantize_layer(W, (gptq_dtype)dt, d_out, d_in, (const float *)FAKE, bits, g, B, damp, act,
                               (uint32_t *)FAKE, (float *)FAKE, (float *)FAKE, (int32_t *)FAKE, ws, wsb, NULL);
}

static void quantize_rejections(void) {
    const size_t big = (size_t)1 << 40;
    EXPECT(q(NULL, 1, 64, 256, 4, 128, 128, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "NULL");
    EXPECT(q(FAKE, 1, 0, 256, 4, 128, 128, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "d_out");
    EXPECT(q(FAKE, 1, 64, -3, 4, 128, 128, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "d_in");
    EXPECT(q(FAKE, 1, 64, 256, 5, 128, 128, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "bits");
    EXPECT(q(FAKE, 1, 64, 256, 4, 100, 128, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "multiple of 16");
    EXPECT(q(FAKE, 1, 64, 256, 4, 64, 96, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "multiple of group_size");
    EXPECT(q(FAKE, 1, 64, 256, 4, 128, 0, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "block_size");
    EXPECT(q(FAKE, 1, 64, 256, 4, 128, 128, NAN, 0, FAKE, big), GPTQ_EINVAL, "damp");
    EXPECT(q(FAKE, 1, 64, 256, 4, 128, 128, -1.f, 0, FAKE, big), GPTQ_EINVAL, "damp");
    EXPECT(q(FAKE, 1, 64, 256, 4, 128, 128, 0.01f, 2, FAKE, big), GPTQ_EINVAL, "act_order");
    EXPECT(q(FAKE, 7, 64, 256, 4, 128, 128, 0.01f, 0, FAKE, big), GPTQ_EINVAL, "w_dtype");
    EXPECT(q(FAKE, 1, 64, 256, 4, 128, 128, 0.01f, 0, FAKE, 1024), GPTQ_ENOMEM, NULL);
    EXPECT(q(FAKE, 1, 64, 256, 4, 128, 128, 0.01f, 0, NULL, big), GPTQ_ENOMEM, NULL);
    EXPECT(q(FAKE, 1, INT64_MAX, INT64_MAX, 4, 128, 128, 0.01f, 0, FAKE, big), GPTQ_EINVAL, NULL);

    const void *W2[2] = {FAKE, NULL};
    const int64_t dout[2] = {64, 32};
    uint32_t *Q2[2] = {(uint32_t *)FAKE, (uint32_t *)FAKE};
    float *S2[2] = {(float *)FAKE, (float *)FAKE};
    EXPECT(gptq_quantize_layers(2, W2, GPTQ_BF16, dout, 256, (const float *)FAKE, 4, 128, 128, 0.01f, 0, Q2, S2, S2,
                                (int32_t *)FAKE, FAKE, big, NULL),
           GPTQ_EINVAL, NULL);
    EXPECT(gptq_quantize_layers(0, W2, GPTQ_BF16, dout, 256, (const float *)FAKE, 4, 128, 128, 0.01f, 0, Q2, S2, S2,
                                (int32_t *)FAKE, FAKE, big, NULL),
           GPTQ_EINVAL, NULL);
}

static void other_rejections(void) {
    const size_t big = (size_t)1 << 30;
    EXPECT(gptq_hessian_accumulate(FAKE, (gptq_dtype)5, 10, 10, (float *)FAKE, FAKE, big, NULL), GPTQ_EINVAL, NULL);
    EXPECT(gptq_hessian_accumulate(FAKE, GPTQ_BF16, -1, 10, (float *)FAKE, FAKE, big, NULL), GPTQ_EINVAL, NULL);
    EXPECT(gptq_hessian_accumulate(FAKE, GPTQ_BF16, 10, 0, (float *)FAKE, FAKE, big, NULL), GPTQ_EINVAL, NULL);
    EXPECT(gptq_hessian_accumulate(FAKE, GPTQ_BF16, 10, (int64_t)1 << 21, (float *)FAKE, FAKE, big, NULL),
           GPTQ_EINVAL, NULL);
    EXPECT(gptq_hessian_accumulate(NULL, GPTQ_BF16, 10, 10, (float *)FAKE, FAKE, big, NULL), GPTQ_EINVAL, NULL);
    EXPECT(gptq_hessian_accumulate(FAKE, GPTQ_BF16, 10, 10, (float *)FAKE, FAKE, 8, NULL), GPTQ_ENOMEM, NULL);
    EXPECT(gptq_hessian_accumulate(NULL, GPTQ_BF16, 0, 10, (float *)FAKE, NULL, 0, NULL), GPTQ_OK, NULL);
    EXPECT(gptq_hessian_accumulate_noalloc(FAKE, GPTQ_BF16, 100, gptq_hessian_noalloc_max_d_in(GPTQ_BF16) + 1,
                                           (float *)FAKE, NULL),
           GPTQ_EINVAL, "static scratch");
    EXPECT(gptq_hessian_accumulate_noalloc(FAKE, GPTQ_BF16, 10, 10, NULL, NULL), GPTQ_EINVAL, NULL);
    EXPECT(gptq_inverse_factor(NULL, 10, 0.01f, 0, (int32_t *)FAKE, (float *)FAKE, FAKE, big, NULL), GPTQ_EINVAL,
           NULL);
    EXPECT(gptq_inverse_factor((const float *)FAKE, 10, INFINITY, 0, (int32_t *)FAKE, (float *)FAKE, FAKE, big, NULL),
           GPTQ_EINVAL, NULL);
    EXPECT(gptq_inverse_factor((const float *)FAKE, 10, 0.01f, 0, (int32_t *)FAKE, (float *)FAKE, FAKE, 4, NULL),
           GPTQ_ENOMEM, NULL);
    EXPECT(gptq_dequant_matmul(FAKE, GPTQ_BF16, 2, 256, (const uint32_t *)FAKE, (const float *)FAKE,
                               (const float *)FAKE, NULL, 64, 5, 128, FAKE, GPTQ_F32, FAKE, big, NULL),
           GPTQ_EINVAL, NULL);
    EXPECT(gptq_dequant_matmul(FAKE, GPTQ_BF16, 2, 256, (const uint32_t *)FAKE, (const float *)FAKE,
                               (const float *)FAKE, NULL, 64, 4, 128, FAKE, GPTQ_F32, FAKE, 16, NULL),
           GPTQ_ENOMEM, NULL);
    EXPECT(gptq_dequant_matmul(NULL, GPTQ_BF16, 0, 256, (const uint32_t *)FAKE, (const float *)FAKE,
                               (const float *)FAKE, NULL, 64, 4, 128, FAKE, GPTQ_F32, NULL, 0, NULL),
           GPTQ_OK, NULL);
    gptq_profile p;
    gptq_profile_enable(0);
    CHECK(gptq_profile_read(&p, 1) == GPTQ_OK);
    CHECK(gptq_profile_read(NULL, 1) == GPTQ_OK);   /* a reset alone */
}

/* the detail string is per thread: concurrent failures do not mix */
static void *worker(void *arg) {
    const int id = (int)(intptr_t)arg;
    for (int i = 0; i < 2000; ++i) {
        gptq_status s = q(FAKE, 1, id % 2 ? 0 : 64, 256, id % 2 ? 4 : 5, 128, 128, 0.01f, 0, FAKE, 1 << 20);
        const char *want = id % 2 ? "d_out" : "bits";
        if (s != GPTQ_EINVAL || strstr(gptq_last_error(), want) == NULL) return (void *)1;
    }
    return NULL;
}

static void threads(void) {
    pthread_t t[8];
    for (int i = 0; i < 8; ++i) CHECK(pthread_create(&t[i], NULL, worker, (void *)(intptr_t)i) == 0);
    for (int i = 0; i < 8; ++i) {
        void *r = NULL;
        CHECK(pthread_join(t[i], &r) == 0);
        CHECK(r == NULL);
    }
}

int main(void) {
    helpers();
    sizes();
    quantize_rejections();
    other_rejections();
    threads();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
