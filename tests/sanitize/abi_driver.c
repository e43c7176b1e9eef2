/* Drives the library's host-side argument checks from C: every call below is
 * invalid and must be refused with its documented status before anything is
 * enqueued, so no GPU is involved.  Built with the library's host code under
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lpq.h"

static int failures = 0;
#define EXPECT(call, want)                                                         \
    do {                                                                           \
        const int got_ = (int)(call);                                              \
        if (got_ != (want)) {                                                      \
            printf("%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, got_, (want)); \
            failures++;                                                            \
        }                                                                          \
    } while (0)

int main(void) {
    /* aligned, never dereferenced: every call below fails its checks first */
    void* P = (void*)(uintptr_t)(1u << 20);
    const uint16_t* W = (const uint16_t*)P;
    uint16_t* H = (uint16_t*)P;
    uint8_t* B = (uint8_t*)P;
    float* F = (float*)P;
    const uint16_t* W2 = (const uint16_t*)((const char*)P + 2);
    const uint16_t* W1 = (const uint16_t*)((const char*)P + 1);
    for (int st = -1; st < 9; st++) EXPECT(strlen(lpq_status_string((lpq_status)st)) > 0, 1);
    EXPECT(lpq_quantize_mxfp8(NULL, 4, 32, B, B, NULL), LPQ_ERR_NULL);
    EXPECT(lpq_quantize_mxfp8(W, 4, 48, B, B, NULL), LPQ_ERR_SHAPE);
    EXPECT(lpq_quantize_mxfp8(W, INT64_MAX, 32, B, B, NULL), LPQ_ERR_SHAPE);   /* element-count overflow guard */
    EXPECT(lpq_quantize_mxfp8(W, 4, INT64_MIN, B, B, NULL), LPQ_ERR_SHAPE);
    EXPECT(lpq_quantize_mxfp8(W2, 4, 32, B, B, NULL), LPQ_ERR_ALIGN);
    EXPECT(lpq_quantize_fp8blk(W, INT64_MAX, INT64_MAX, B, F, NULL), LPQ_ERR_SHAPE);
    EXPECT(lpq_quantize_fp8blk(W1, 5, 5, B, F, NULL), LPQ_ERR_ALIGN);
    EXPECT(lpq_dequantize_fp8blk(B, F, 5, 5, NULL, NULL), LPQ_ERR_NULL);
    EXPECT(lpq_quantize_nvfp4(W, 4, 24, F, B, B, F, NULL), LPQ_ERR_SHAPE);
    EXPECT(lpq_quantize_nvfp4(W, 4, 32, NULL, B, B, NULL, NULL), LPQ_ERR_NULL);
    EXPECT(lpq_nvfp4_qdq(W, 4, 32, NULL, H, NULL), LPQ_ERR_ARG);   /* amax computed into y: x, y overlap */
    EXPECT(lpq_quantize_nvfp4_ex(W, 4, 32, F, 300, B, B, F, NULL), LPQ_ERR_ARG);
    EXPECT(lpq_nvfp4_observe(W, 4, 32, 7, 0.5f, F, F, NULL), LPQ_ERR_ARG);
    EXPECT(lpq_nvfp4_observe_noalloc(W, 4, 32, 7, 0.5f, F, F, NULL), LPQ_ERR_ARG);
    EXPECT(lpq_nvfp4_observe_noalloc(W, 4, 32, 1, 0.5f, NULL, F, NULL), LPQ_ERR_NULL);
    EXPECT(lpq_quantize_int4(W, 4, 128, 64, B, F, NULL), LPQ_ERR_ARG);
    EXPECT(lpq_requantize_fp8blk_mxfp8(B, F, (int64_t)1 << 31, 32, B, B, NULL), LPQ_ERR_SHAPE);
    EXPECT(lpq_nvfp4_global_scale_reciprocal(F, -5, F, NULL), LPQ_ERR_SHAPE);

    lpq_tensor t[3];
    memset(t, 0, sizeof t);
    for (int i = 0; i < 3; i++) {
        t[i].src = t[i].dst = t[i].scale = P;
        t[i].rows = 8;
        t[i].cols = 64;
        t[i].group = i;
    }
    EXPECT(lpq_quantize_nvfp4_grouped(t, (lpq_tensor*)P, 3, F, 2, 0, F, NULL), LPQ_ERR_GROUP);
    EXPECT(lpq_nvfp4_qdq_grouped(t, (lpq_tensor*)P, 3, F, 2, 1, NULL), LPQ_ERR_GROUP);
    EXPECT(lpq_quantize_mxfp8_grouped(t, (lpq_tensor*)P, 0, NULL), LPQ_ERR_SHAPE);
    EXPECT(lpq_quantize_mxfp8_grouped(t, (lpq_tensor*)P, -1, NULL), LPQ_ERR_SHAPE);
    t[2].rows = INT64_MAX;
    EXPECT(lpq_quantize_fp8blk_grouped(t, (lpq_tensor*)P, 3, NULL), LPQ_ERR_SHAPE);
    t[2].rows = 8;
    t[1].reserved = 3;
    EXPECT(lpq_dequantize_mxfp8_grouped(t, (lpq_tensor*)P, 3, NULL), LPQ_ERR_ARG);
    EXPECT(lpq_int4_qdq_grouped(t, (lpq_tensor*)P, 3, 33, NULL), LPQ_ERR_ARG);

    lpq_requant_tensor r[2];
    memset(r, 0, sizeof r);
    for (int i = 0; i < 2; i++) {
        r[i].src = B;
        r[i].src_scale = F;
        r[i].dst = r[i].dst_scale = P;
        r[i].rows = 8;
        r[i].cols = 64;
        r[i].group = 5;
    }
    EXPECT(lpq_requantize_fp8blk_nvfp4_grouped(r, (lpq_requant_tensor*)P, 2, F, 2, F, NULL), LPQ_ERR_GROUP);
    EXPECT(lpq_fp8blk_amax_grouped(r, (lpq_requant_tensor*)P, 2, NULL, 2, 0, NULL), LPQ_ERR_NULL);
    EXPECT(lpq_last_hip_error(), 0);
    printf("%s\n", failures ? "FAIL" : "abi: every invalid call refused, clean under ASan/UBSan");
    return failures ? 1 : 0;
}
