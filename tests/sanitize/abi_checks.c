/* Host-side argument checks of every entry point in lora_batch.h, run as a
 * plain executable built with AddressSanitizer and UndefinedBehaviorSanitizer
 * over the library's host code.  Every call here either fails validation or
 * has nothing to do (zero rows), so no GPU work is enqueued and no device
 * pointer is dereferenced: FAKE is a 16-byte aligned address that validation
 * never reaches past.  The size queries are also asked for extreme sizes, so
 * an overflow in their arithmetic shows up as a sanitizer report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lora_batch.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, \
                    __LINE__, #cond);                                     \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

#define FAKE ((void*)(uintptr_t)0x10000)
#define FAKEB(off) ((void*)((uintptr_t)0x10000 + (off)))

static lora_segments seg_of(int ok) {
    lora_segments s;
    s.counts = (int32_t*)FAKE;
    s.offsets = (int32_t*)FAKE;
    s.perm = (int32_t*)FAKE;
    s.err = (int32_t*)FAKE;
    s.sched = ok ? (int32_t*)FAKE : NULL;
    return s;
}

static void queries(void) {
    EXPECT(lora_abi_version() == LORA_ABI_VERSION);
    for (int s = -6; s <= 3; ++s) EXPECT(lora_status_string(s) != NULL && strlen(lora_status_string(s)) > 0);
    const int32_t big = INT32_MAX;
    /* pure size queries at the extremes: no overflow, monotone in T */
    EXPECT(lora_segments_workspace_bytes(-1, 4) == 0);
    EXPECT(lora_segments_workspace_bytes(big, 1024) > lora_segments_workspace_bytes(big / 2, 1024));
    EXPECT(lora_segments_sched_elems(big, big) > 0);
    EXPECT(lora_shrink_workspace_bytes(LORA_BF16, big, big, LORA_MAX_RANK) > 0);
    EXPECT(lora_shrink_workspace_bytes(LORA_F32, big, 8, 1) > 0);
    EXPECT(lora_shrink_workspace_bytes(LORA_BF16, 100, 4096, 20) == (size_t)8 * 100 * 24 * 4);
    EXPECT(lora_shrink_workspace_bytes(LORA_BF16, 100, 4096, 129) == 0);
    EXPECT(lora_backward_workspace_bytes(LORA_BF16, big, big, big, LORA_MAX_RANK) > 0);
    EXPECT(lora_backward_workspace_bytes(LORA_BF16, 16, 256, 256, 0) == 0);
    EXPECT(lora_backward_workspace_bytes(7, 16, 256, 256, 8) == 0);
}

static void segments(void) {
    const size_t need = lora_segments_workspace_bytes(100, 4);
    EXPECT(lora_segments_build(FAKE, -1, 4, seg_of(1), FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_segments_build(FAKE, 100, 0, seg_of(1), FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_segments_build(NULL, 100, 4, seg_of(1), FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_segments_build(FAKE, 100, 4, seg_of(0), FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_segments_build(FAKE, 100, 4, seg_of(1), FAKE, need - 1, NULL) == LORA_ERR_WORKSPACE);
    EXPECT(lora_segments_build(FAKE, 100, 4, seg_of(1), NULL, need, NULL) == LORA_ERR_WORKSPACE);
    EXPECT(lora_segments_build(NULL, 0, 4, seg_of(1), NULL, 0, NULL) == LORA_OK);
    lora_segments_job jobs[2];
    jobs[0].adapter_ids = FAKE;
    jobs[0].T = 100;
    jobs[0].seg = seg_of(1);
    jobs[0].ws = FAKE;
    jobs[0].ws_bytes = need;
    jobs[1] = jobs[0];
    jobs[1].T = -1;
    EXPECT(lora_segments_build_batch(NULL, 0, 4, NULL) == LORA_OK);
    EXPECT(lora_segments_build_batch(NULL, -1, 4, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_segments_build_batch(jobs, 2, 4, NULL) == LORA_ERR_INVALID_ARG);
    jobs[1].T = 100;
    jobs[1].ws_bytes = need - 1;
    EXPECT(lora_segments_build_batch(jobs, 2, 4, NULL) == LORA_ERR_WORKSPACE);
    EXPECT(lora_segments_build_batch(jobs, 1, 0, NULL) == LORA_ERR_INVALID_ARG);
}

static void shrink_expand(void) {
    const size_t need = lora_shrink_workspace_bytes(LORA_BF16, 64, 256, 8);
    const lora_adapter* ad = (const lora_adapter*)FAKE;
    float* v = (float*)FAKE;
    EXPECT(lora_shrink(5, FAKE, 256, 64, 256, ad, 4, 8, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, -1, 256, ad, 4, 8, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 0, 8, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 4, 0, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 4, 129, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, NULL, 4, 8, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 4, 8, seg_of(0), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKEB(4), 256, 64, 256, ad, 4, 8, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 100, 64, 256, ad, 4, 8, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 100, 64, 100, ad, 4, 8, seg_of(1), v, 8, FAKE, need, NULL) == LORA_ERR_UNSUPPORTED);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 4, 8, seg_of(1), NULL, 8, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 4, 8, seg_of(1), v, 4, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 4, 8, seg_of(1), v, 8, FAKE, need - 1, NULL) == LORA_ERR_WORKSPACE);
    EXPECT(lora_shrink(0, FAKE, 256, 64, 256, ad, 4, 8, seg_of(1), v, 8, FAKEB(4), need, NULL) == LORA_ERR_WORKSPACE);
    EXPECT(lora_shrink(0, NULL, 0, 0, 256, ad, 4, 8, seg_of(1), NULL, 0, NULL, 0, NULL) == LORA_OK);
    EXPECT(lora_shrink_noalloc(5, FAKE, 256, 64, 256, ad, 4, 8, seg_of(1), v, 8, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink_noalloc(0, FAKE, 256, 64, 256, ad, 4, 8, seg_of(1), v, 4, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_shrink_noalloc(0, NULL, 0, 0, 256, ad, 4, 8, seg_of(1), NULL, 0, NULL) == LORA_OK);
    EXPECT(lora_shrink_noalloc(0, FAKE, 8192, 1 << 20, 8192, ad, 4, 128, seg_of(1), v, 128, NULL) ==
           LORA_ERR_TOO_LARGE);
    EXPECT(lora_expand_add(5, v, 8, 64, 256, ad, 4, 8, seg_of(1), FAKE, 256, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_expand_add(0, v, 8, 64, 0, ad, 4, 8, seg_of(1), FAKE, 256, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_expand_add(0, v, 8, 64, 256, ad, 4, 8, seg_of(1), FAKEB(8), 256, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_expand_add(0, v, 12, 64, 256, ad, 4, 8, seg_of(1), FAKE, 256, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_expand_add(0, v, 8, 64, 260, ad, 4, 8, seg_of(1), FAKE, 264, NULL) == LORA_ERR_UNSUPPORTED);
    EXPECT(lora_expand_add(0, NULL, 0, 0, 256, ad, 4, 8, seg_of(1), NULL, 0, NULL) == LORA_OK);
}

static void fused(void) {
    const lora_adapter* ad = (const lora_adapter*)FAKE;
    EXPECT(lora_forward(2, FAKE, 256, 10, 256, 512, ad, 4, 16, seg_of(1), FAKE, 512, NULL, 0, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_forward(0, FAKE, 128, 10, 256, 512, ad, 4, 16, seg_of(1), FAKE, 512, NULL, 0, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_forward(0, FAKE, 264, 10, 260, 512, ad, 4, 16, seg_of(1), FAKE, 512, NULL, 0, NULL) == LORA_ERR_UNSUPPORTED);
    EXPECT(lora_forward(0, FAKE, 256, 10, 256, 512, ad, 4, 16, seg_of(1), FAKE, 512, (float*)FAKE, 8, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_forward(0, NULL, 0, 0, 256, 256, ad, 4, 8, seg_of(1), NULL, 0, NULL, 0, NULL) == LORA_OK);
    lora_slice sl[4];
    for (int i = 0; i < 4; ++i) {
        sl[i].adapters = ad;
        sl[i].y = FAKE;
        sl[i].ldy = 512;
        sl[i].v = NULL;
        sl[i].ldv = 0;
        sl[i].d_out = 512;
        sl[i].reserved = 0;
    }
    EXPECT(lora_forward_multi(0, FAKE, 256, 10, 256, sl, 0, 4, 16, seg_of(1), NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_forward_multi(0, FAKE, 256, 10, 256, sl, 4, 4, 16, seg_of(1), NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_forward_multi(0, FAKE, 256, 10, 256, NULL, 1, 4, 16, seg_of(1), NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_forward_multi(0, FAKE, 256, 10, 256, sl, 2, 4, 72, seg_of(1), NULL) == LORA_ERR_UNSUPPORTED);
    sl[1].reserved = 1;
    EXPECT(lora_forward_multi(0, FAKE, 256, 10, 256, sl, 2, 4, 16, seg_of(1), NULL) == LORA_ERR_INVALID_ARG);
}

static void backward(void) {
    const size_t need = lora_backward_workspace_bytes(LORA_BF16, 16, 256, 256, 8);
    const lora_adapter* ad = (const lora_adapter*)FAKE;
    const lora_adapter_grad* gr = (const lora_adapter_grad*)FAKE;
    EXPECT(lora_backward(0, FAKE, 256, FAKE, 256, FAKE, 256, 16, 256, 256, ad, NULL, 4, 8, seg_of(1), NULL, 0, FAKE,
                         need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_backward(0, FAKE, 256, FAKE, 256, FAKE, 256, 16, 256, 256, ad, (const lora_adapter_grad*)FAKEB(4), 4,
                         8, seg_of(1), NULL, 0, FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_backward(0, FAKE, 256, NULL, 256, FAKE, 256, 16, 256, 256, ad, gr, 4, 8, seg_of(1), NULL, 0, FAKE,
                         need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_backward(0, FAKE, 256, FAKE, 100, FAKE, 256, 16, 256, 100, ad, gr, 4, 8, seg_of(1), NULL, 0, FAKE,
                         need, NULL) == LORA_ERR_UNSUPPORTED);
    EXPECT(lora_backward(0, FAKE, 256, FAKE, 256, FAKEB(2), 256, 16, 256, 256, ad, gr, 4, 8, seg_of(1), NULL, 0,
                         FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_backward(0, FAKE, 256, FAKE, 256, FAKE, 256, 16, 256, 256, ad, gr, 4, 8, seg_of(1), (float*)FAKE, 4,
                         FAKE, need, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_backward(0, FAKE, 256, FAKE, 256, FAKE, 256, 16, 256, 256, ad, gr, 4, 8, seg_of(1), NULL, 0, FAKE,
                         need - 1, NULL) == LORA_ERR_WORKSPACE);
    EXPECT(lora_backward(0, NULL, 0, NULL, 0, NULL, 0, 0, 256, 256, ad, gr, 4, 8, seg_of(1), NULL, 0, NULL, 0,
                         NULL) == LORA_OK);
    EXPECT(lora_backward_preemptible(0, FAKE, 256, FAKE, 256, NULL, 0, 64, 256, 512, ad, gr, 4, 16, seg_of(1), NULL,
                                     0, FAKE, need, NULL, (int32_t*)FAKE, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_backward_preemptible(0, FAKE, 256, FAKE, 256, NULL, 0, 64, 256, 512, ad, gr, 4, 16, seg_of(1), NULL,
                                     0, FAKE, need, (const int32_t*)FAKEB(2), (int32_t*)FAKE,
                                     NULL) == LORA_ERR_INVALID_ARG);
}

static void adamw(void) {
    lora_adamw_tensor t[33];
    for (int i = 0; i < 33; ++i) {
        t[i].w = FAKE;
        t[i].master = NULL;
        t[i].grad = (float*)FAKE;
        t[i].m = (float*)FAKE;
        t[i].v = (float*)FAKE;
        t[i].n = 1024;
    }
    lora_adamw_params hp = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, 1.0f, 1, 0};
    EXPECT(lora_adamw_step(0, NULL, 0, hp, NULL) == LORA_OK);
    EXPECT(lora_adamw_step(2, t, 1, hp, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_adamw_step(0, t, 33, hp, NULL) == LORA_ERR_INVALID_ARG);
    EXPECT(lora_adamw_step(0, t, -1, hp, NULL) == LORA_ERR_INVALID_ARG);
    lora_adamw_params h2 = hp;
    h2.lr = NAN;
    EXPECT(lora_adamw_step(0, t, 1, h2, NULL) == LORA_ERR_INVALID_ARG);
    h2 = hp;
    h2.beta1 = 1.0f;
    EXPECT(lora_adamw_step(0, t, 1, h2, NULL) == LORA_ERR_INVALID_ARG);
    h2 = hp;
    h2.step = 0;
    EXPECT(lora_adamw_step(0, t, 1, h2, NULL) == LORA_ERR_INVALID_ARG);
    t[1].w = FAKEB(4);
    EXPECT(lora_adamw_step(0, t, 2, hp, NULL) == LORA_ERR_INVALID_ARG);
    t[1].w = FAKE;
    t[1].n = -1;
    EXPECT(lora_adamw_step(0, t, 2, hp, NULL) == LORA_ERR_INVALID_ARG);
}

int main(void) {
    queries();
    segments();
    shrink_expand();
    fused();
    backward();
    adamw();
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("abi checks: ok\n");
    return 0;
}
