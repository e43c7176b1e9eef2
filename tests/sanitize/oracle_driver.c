/* Drives every function of the C oracle over edge shapes (one element, ragged
 * 128x128 tiles, a single block, all zeros, signed zeros, extreme magnitudes)
 * under AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds
 * access, overflow or undefined shift aborts the program.  Test
 * infrastructure; built and run by tests/test_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oc_bf16_to_f32(uint16_t h);
uint16_t oc_f32_to_bf16(float f);
float oc_e4m3_decode(uint8_t c);
uint8_t oc_e4m3_encode(float v);
float oc_e2m1_decode(uint8_t c);
uint8_t oc_e2m1_encode(float v);
float oc_ue8m0_decode(uint8_t b);
uint8_t oc_mxfp8_scale_byte(float amax);
uint8_t oc_mxfp8_floor_scale_byte(float amax);
void oc_fp8blk_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, float* s);
void oc_fp8blk_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t N, uint16_t* y);
void oc_mxfp8_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e);
void oc_mxfp8_floor_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e);
void oc_mxfp8_dequantize(const uint8_t* q, const uint8_t* e, int64_t M, int64_t N, uint16_t* y);
float oc_amax_bf16(const uint16_t* w, int64_t n);
float oc_nvfp4_global_scale(float A);
float oc_nvfp4_global_scale_max(float A, int e4m3_max);
float oc_nvfp4_global_scale_reciprocal(float A);
uint8_t oc_nvfp4_block_scale(float b, float g);
float oc_nvfp4_effective_scale(uint8_t scode, float g);
void oc_nvfp4_quantize(const uint16_t* w, int64_t M, int64_t N, float g, uint8_t* p, uint8_t* s);
void oc_nvfp4_dequantize(const uint8_t* p, const uint8_t* s, float g, int64_t M, int64_t N, uint16_t* y);
void oc_nvfp4_qdq(const uint16_t* x, int64_t M, int64_t N, float g, uint16_t* y);
float oc_observer_update(int kind, float c, float* state, const uint16_t* x, int64_t n);
float oc_int4_scale(float amax);
void oc_int4_quantize(const uint16_t* w, int64_t M, int64_t N, int64_t G, uint8_t* p, float* s);
void oc_int4_dequantize(const uint8_t* p, const float* s, int64_t M, int64_t N, int64_t G, uint16_t* y);
void oc_int4_qdq(const uint16_t* x, int64_t M, int64_t N, int64_t G, uint16_t* y);

static uint64_t rng = 0x5EED;
static uint16_t rand_bf16(void) {   /* any finite BF16 pattern */
    for (;;) {
        rng = rng * 6364136223846793005ull + 1442695040888963407ull;
        uint16_t h = (uint16_t)(rng >> 40);
        if (((h >> 7) & 0xff) != 0xff) return h;
    }
}

/* exactly sized heap buffers, so that ASan sees any access past the end */
static void* buf(size_t n) { return malloc(n ? n : 1); }

static void run(int64_t M, int64_t N, int fill) {
    const int64_t n = M * N, tm = (M + 127) / 128, tn = (N + 127) / 128;
    uint16_t* w = buf(2 * n);
    for (int64_t i = 0; i < n; i++)
        w[i] = fill == 0 ? 0 : fill == 1 ? (uint16_t)((i & 1) ? 0x8000 : 0) : rand_bf16();
    uint8_t* q = buf(n);
    uint16_t* y = buf(2 * n);
    float* s = buf(4 * tm * tn);
    oc_fp8blk_quantize(w, M, N, q, s);
    oc_fp8blk_dequantize(q, s, M, N, y);
    if (N % 32 == 0) {
        uint8_t* e = buf(n / 32);
        oc_mxfp8_quantize(w, M, N, q, e);
        oc_mxfp8_dequantize(q, e, M, N, y);
        oc_mxfp8_floor_quantize(w, M, N, q, e);
        free(e);
    }
    if (N % 16 == 0) {
        uint8_t* p = buf(n / 2);
        uint8_t* sb = buf(n / 16);
        const float g = oc_nvfp4_global_scale(oc_amax_bf16(w, n));
        oc_nvfp4_quantize(w, M, N, g, p, sb);
        oc_nvfp4_dequantize(p, sb, g, M, N, y);
        oc_nvfp4_qdq(w, M, N, g, y);
        oc_nvfp4_qdq(w, M, N, oc_nvfp4_global_scale_max(oc_amax_bf16(w, n), 256), y);
        float st[3] = {0, 0, 0};
        for (int kind = 0; kind < 3; kind++) oc_observer_update(kind, 0.01f, st, w, n);
        free(p);
        free(sb);
    }
    for (int64_t G = 32; G <= 128; G *= 4) {
        if (N % G) continue;
        uint8_t* p = buf(n / 2);
        float* sg = buf(4 * (n / G));
        oc_int4_quantize(w, M, N, G, p, sg);
        oc_int4_dequantize(p, sg, M, N, G, y);
        oc_int4_qdq(w, M, N, G, y);
        free(p);
        free(sg);
    }
    free(w);
    free(q);
    free(y);
    free(s);
}

int main(void) {
    /* scalar casts over every BF16 pattern and a few binary32 edge values */
    for (uint32_t h = 0; h < 65536; h++) {
        const float f = oc_bf16_to_f32((uint16_t)h);
        (void)oc_f32_to_bf16(f);
        (void)oc_e4m3_encode(f);
        (void)oc_e2m1_encode(f);
        if (f == f && f >= 0.0f && f < 3.4e38f) {
            (void)oc_mxfp8_scale_byte(f);
            (void)oc_mxfp8_floor_scale_byte(f);
            (void)oc_nvfp4_global_scale_reciprocal(f);
            (void)oc_nvfp4_block_scale(f, oc_nvfp4_global_scale(f));
            (void)oc_int4_scale(f);
        }
    }
    for (int c = 0; c < 256; c++) {
        (void)oc_e4m3_decode((uint8_t)c);
        (void)oc_e2m1_decode((uint8_t)(c & 15));
        (void)oc_ue8m0_decode((uint8_t)c);
        (void)oc_nvfp4_effective_scale((uint8_t)c, 1e-30f);
    }
    const int64_t shapes[][2] = {{1, 1}, {1, 2}, {7, 3}, {1, 16}, {1, 32}, {3, 128}, {129, 130}, {130, 256},
                                 {256, 512}, {5, 160}};
    for (size_t k = 0; k < sizeof shapes / sizeof shapes[0]; k++)
        for (int fill = 0; fill < 3; fill++) run(shapes[k][0], shapes[k][1], fill);
    puts("oracle: clean under ASan/UBSan");
    return 0;
}
