/*
 * A plain C consumer of liblpq.so: device buffers from the HIP runtime's C
 * API, the codecs through their C entry points (include/lpq.h), and every
 * output checked bit for bit against the C oracle (oracle/lpq_oracle.c).  No
 * Python and no torch are involved.
 *
 * TEST INFRASTRUCTURE: built by the build step, run by
 * tests/test_gpu_c_consumer.py on a GPU.  Exit status 0 when every call
 * returns LPQ_OK and every array matches; the per-array mismatch counts go to
 * stdout.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lpq.h"

/* The oracle's entry points used here (see oracle/lpq_oracle.c). */
void oc_fp8blk_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, float* s);
void oc_fp8blk_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t N, uint16_t* y);
void oc_mxfp8_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e);
void oc_mxfp8_dequantize(const uint8_t* q, const uint8_t* e, int64_t M, int64_t N, uint16_t* y);
float oc_amax_bf16(const uint16_t* w, int64_t n);
float oc_nvfp4_global_scale(float A);
void oc_nvfp4_quantize(const uint16_t* w, int64_t M, int64_t N, float g, uint8_t* p, uint8_t* s);
void oc_nvfp4_dequantize(const uint8_t* p, const uint8_t* s, float g, int64_t M, int64_t N, uint16_t* y);
void oc_nvfp4_qdq(const uint16_t* x, int64_t M, int64_t N, float g, uint16_t* y);
void oc_int4_quantize(const uint16_t* w, int64_t M, int64_t N, int64_t G, uint8_t* p, float* s);
void oc_int4_dequantize(const uint8_t* p, const float* s, int64_t M, int64_t N, int64_t G, uint16_t* y);
void oc_int4_qdq(const uint16_t* x, int64_t M, int64_t N, int64_t G, uint16_t* y);
float oc_observer_update(int kind, float c, float* state, const uint16_t* x, int64_t n);

static int failures = 0;

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));         \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

static void lpq_ok(lpq_status st, const char* what) {
    if (st != LPQ_OK) {
        printf("%s returned %d (%s)\n", what, (int)st, lpq_status_string(st));
        failures++;
    }
}

/* Compares n bytes of a device array with the oracle's host array. */
static void check(const char* name, const void* dev, const void* want, size_t n) {
    unsigned char* got = (unsigned char*)malloc(n);
    HIP_OK(hipMemcpy(got, dev, n, hipMemcpyDeviceToHost));
    size_t bad = 0;
    for (size_t i = 0; i < n; i++) bad += got[i] != ((const unsigned char*)want)[i];
    printf("%-22s %zu mismatching bytes of %zu\n", name, bad, n);
    if (bad) failures++;
    free(got);
}

static void* dev_alloc(size_t n) {
    void* p = NULL;
    HIP_OK(hipMalloc(&p, n));
    return p;
}

/* Deterministic BF16 test data: a linear congruential generator drives
 * mantissas and exponents over a wide range (round to nearest even). */
static void make_input(uint16_t* w, size_t n) {
    uint64_t x = 0x9E3779B97F4A7C15ull;
    for (size_t i = 0; i < n; i++) {
        x = x * 6364136223846793005ull + 1442695040888963407ull;
        uint32_t r = (uint32_t)(x >> 32);
        uint32_t sign = r & 0x80000000u, exp = 100u + ((r >> 23) & 31u), man = r & 0x7fffffu;
        uint32_t u = sign | (exp << 23) | man;
        uint32_t bf = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
        w[i] = (uint16_t)bf;
    }
}

int main(void) {
    const int64_t M = 300, N = 1024, n = M * N;
    const int64_t tm = (M + 127) / 128, tn = (N + 127) / 128;
    uint16_t* w = (uint16_t*)malloc(n * 2);
    make_input(w, (size_t)n);

    uint16_t* dw = (uint16_t*)dev_alloc(n * 2);
    uint8_t* dq = (uint8_t*)dev_alloc(n);
    float* ds = (float*)dev_alloc(tm * tn * 4);
    uint8_t* de = (uint8_t*)dev_alloc(n / 16);
    uint16_t* dy = (uint16_t*)dev_alloc(n * 2);
    float* damax = (float*)dev_alloc(4);
    float* dg = (float*)dev_alloc(4);
    float* ds4 = (float*)dev_alloc(n / 128 * 4);
    HIP_OK(hipMemcpy(dw, w, n * 2, hipMemcpyHostToDevice));

    uint8_t* q = (uint8_t*)malloc(n);
    float* s = (float*)malloc(tm * tn * 4);
    uint8_t* e = (uint8_t*)malloc(n / 16);
    uint16_t* y = (uint16_t*)malloc(n * 2);
    float* s4 = (float*)malloc(n / 128 * 4);

    /* block-wise FP8 */
    lpq_ok(lpq_quantize_fp8blk(dw, M, N, dq, ds, NULL), "lpq_quantize_fp8blk");
    lpq_ok(lpq_dequantize_fp8blk(dq, ds, M, N, dy, NULL), "lpq_dequantize_fp8blk");
    HIP_OK(hipDeviceSynchronize());
    oc_fp8blk_quantize(w, M, N, q, s);
    oc_fp8blk_dequantize(q, s, M, N, y);
    check("fp8blk codes", dq, q, n);
    check("fp8blk scales", ds, s, tm * tn * 4);
    check("fp8blk dequantized", dy, y, n * 2);

    /* MXFP8 */
    lpq_ok(lpq_quantize_mxfp8(dw, M, N, dq, de, NULL), "lpq_quantize_mxfp8");
    lpq_ok(lpq_dequantize_mxfp8(dq, de, M, N, dy, NULL), "lpq_dequantize_mxfp8");
    HIP_OK(hipDeviceSynchronize());
    oc_mxfp8_quantize(w, M, N, q, e);
    oc_mxfp8_dequantize(q, e, M, N, y);
    check("mxfp8 codes", dq, q, n);
    check("mxfp8 scale bytes", de, e, n / 32);
    check("mxfp8 dequantized", dy, y, n * 2);

    /* NVFP4: the tensor is its own sibling group */
    lpq_ok(lpq_nvfp4_amax(dw, M, N, damax, 0, NULL), "lpq_nvfp4_amax");
    lpq_ok(lpq_quantize_nvfp4(dw, M, N, damax, dq, de, dg, NULL), "lpq_quantize_nvfp4");
    HIP_OK(hipDeviceSynchronize());
    const float A = oc_amax_bf16(w, n), g = oc_nvfp4_global_scale(A);
    oc_nvfp4_quantize(w, M, N, g, q, e);
    check("nvfp4 amax", damax, &A, 4);
    check("nvfp4 global scale", dg, &g, 4);
    check("nvfp4 packed", dq, q, n / 2);
    check("nvfp4 block scales", de, e, n / 16);
    lpq_ok(lpq_dequantize_nvfp4(dq, de, dg, M, N, dy, NULL), "lpq_dequantize_nvfp4");
    HIP_OK(hipDeviceSynchronize());
    oc_nvfp4_dequantize(q, e, g, M, N, y);
    check("nvfp4 dequantized", dy, y, n * 2);
    lpq_ok(lpq_nvfp4_qdq(dw, M, N, damax, dy, NULL), "lpq_nvfp4_qdq");
    HIP_OK(hipDeviceSynchronize());
    oc_nvfp4_qdq(w, M, N, g, y);
    check("nvfp4 qdq", dy, y, n * 2);
    /* no amax given: the call computes the tensor's own (in the g word) */
    HIP_OK(hipMemset(dq, 0, n / 2));
    lpq_ok(lpq_quantize_nvfp4(dw, M, N, NULL, dq, de, dg, NULL), "lpq_quantize_nvfp4 (amax NULL)");
    HIP_OK(hipDeviceSynchronize());
    check("nvfp4 global scale, own amax", dg, &g, 4);
    check("nvfp4 packed, own amax", dq, q, n / 2);
    check("nvfp4 block scales, own amax", de, e, n / 16);
    HIP_OK(hipMemset(dy, 0xff, n * 2));
    lpq_ok(lpq_nvfp4_qdq(dw, M, N, NULL, dy, NULL), "lpq_nvfp4_qdq (amax NULL)");   /* A held in y meanwhile */
    HIP_OK(hipDeviceSynchronize());
    oc_nvfp4_qdq(w, M, N, g, y);
    check("nvfp4 qdq, own amax", dy, y, n * 2);
    if (lpq_nvfp4_qdq(dw, M, N, NULL, (uint16_t*)dw + 8, NULL) != LPQ_ERR_ARG) {   /* y overlapping x */
        printf("lpq_nvfp4_qdq with amax NULL and overlapping x, y was not refused with LPQ_ERR_ARG\n");
        failures++;
    }

    /* W4A4 observer (moving average), twice in a row on the same batch: with the
     * caller's full state, and with the library's own control block and a
     * 3-word state (lpq_nvfp4_observe_noalloc) */
    float* dstate = (float*)dev_alloc(LPQ_OBSERVER_STATE_FLOATS * 4);
    float* dstats = (float*)dev_alloc(3 * 4);
    float* damax2 = (float*)dev_alloc(4);
    float ostate[3] = {0.0f, 0.0f, 0.0f}, oamax[2];
    lpq_ok(lpq_observer_reset(dstate, NULL), "lpq_observer_reset");
    HIP_OK(hipMemset(dstats, 0, 3 * 4));
    for (int t = 0; t < 2; t++) {
        const int64_t rows = t == 0 ? M : M / 3;   /* the second batch smaller */
        lpq_ok(lpq_nvfp4_observe(dw, rows, N, LPQ_OBSERVER_MINMAX, 0.25f, dstate, damax, NULL), "lpq_nvfp4_observe");
        lpq_ok(lpq_nvfp4_observe_noalloc(dw, rows, N, LPQ_OBSERVER_MINMAX, 0.25f, dstats, damax2, NULL),
               "lpq_nvfp4_observe_noalloc");
        HIP_OK(hipDeviceSynchronize());
        oamax[t] = oc_observer_update(LPQ_OBSERVER_MINMAX, 0.25f, ostate, w, rows * N);
        check(t == 0 ? "observer amax 1" : "observer amax 2", damax, &oamax[t], 4);
        check(t == 0 ? "no-alloc amax 1" : "no-alloc amax 2", damax2, &oamax[t], 4);
    }
    check("observer state", dstate, ostate, 3 * 4);
    check("no-alloc statistics", dstats, ostate, 3 * 4);

    /* group-wise INT4, group 128 */
    lpq_ok(lpq_quantize_int4(dw, M, N, 128, dq, ds4, NULL), "lpq_quantize_int4");
    lpq_ok(lpq_dequantize_int4(dq, ds4, M, N, 128, dy, NULL), "lpq_dequantize_int4");
    HIP_OK(hipDeviceSynchronize());
    oc_int4_quantize(w, M, N, 128, q, s4);
    oc_int4_dequantize(q, s4, M, N, 128, y);
    check("int4 packed", dq, q, n / 2);
    check("int4 scales", ds4, s4, n / 128 * 4);
    check("int4 dequantized", dy, y, n * 2);
    lpq_ok(lpq_int4_qdq(dw, M, N, 128, dy, NULL), "lpq_int4_qdq");
    HIP_OK(hipDeviceSynchronize());
    oc_int4_qdq(w, M, N, 128, y);
    check("int4 qdq", dy, y, n * 2);

    /* a refused call enqueues nothing and says why */
    if (lpq_quantize_mxfp8(dw, M, 48, dq, de, NULL) != LPQ_ERR_SHAPE) {
        printf("N = 48 was not refused with LPQ_ERR_SHAPE\n");
        failures++;
    }

    printf("%s\n", failures ? "FAIL" : "OK: every C entry point matches the oracle bit for bit");
    return failures ? 1 : 0;
}
