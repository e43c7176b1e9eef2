/*
 * lpq_oracle.c -- plain, slow CPU oracle for the BF16 -> low-precision weight
 * codecs (block-wise FP8, MXFP8, NVFP4, group-wise INT4) and their fake-quant
 * (QDQ).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no source, header, table or helper with the
 * HIP kernels.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -shared -fPIC
 * Every floating-point operation below is one IEEE-754 binary32 operation,
 * rounded to nearest-even (x86-64 SSE, FLT_EVAL_METHOD == 0, no FMA
 * contraction), so "fl(a op b)" in the comments is exactly what the C
 * expression computes.
 *
 * Sources (web pages; cited by title and section):
 *  [LPRL]  "Low Precision RL" (Miles documentation) -- "Choose a precision"
 *          table: block-wise FP8 = 128x128 tiles with FP32 scales; MXFP8 = 1x32
 *          blocks with UE8M0 scales; NVFP4 = E2M1, 1x16 blocks, two-level
 *          (FP8 + FP32) scale.  "3. Unified MXFP8": UE8M0 power-of-two scales
 *          stored as uint8, values stored as float8_e4m3fn.  "2. Unified
 *          block-wise FP8": FP32 (not power-of-two) scales.
 *  [VERL]  "verl NVFP4 QAT" article (capital-peak.com), section 2.3: global
 *          scale = amax / (FP4_E2M1_MAX * FP8_E4M3_MAX) with 6.0 and 448.0;
 *          per-16 block amax converted to an E4M3 block scale; values snapped
 *          to the nearest point of {0, 0.5, 1, 1.5, 2, 3, 4, 6} and multiplied
 *          back by the block scale.  Section 2.4: sibling q/k/v and gate/up
 *          share one global scale taken from the group maximum.  Section 3.3:
 *          weight_scale_2 = w_amax / (6.0 * 448.0).
 *  [PR503] vime pull request 503 review: fake QAT requires exact
 *          round-to-nearest numerics (no fast math).
 *
 * Readings where the pages are silent:
 *  - every rounding is round-to-nearest, ties-to-even (the "exact RN" rule);
 *  - FP8 block scale s = fl(amax / 448), stored as the dequant multiplier;
 *  - MXFP8 exponent: smallest e with amax <= 448 * 2^e, clamped to e >= -127;
 *  - NVFP4 block scale = E4M3(fl(fl(b / 6) / g)), effective scale
 *    S = fl(E4M3value * g);
 *  - E4M3 and E2M1 casts saturate to +-448 / +-6 and keep the sign of zero;
 *  - a zero scale encodes every element as a zero of the element's sign;
 *  - packed E2M1: element 2j in the low nibble of byte j;
 *  - group-wise INT4 (the page gives only the group sizes 32 and 128):
 *    s = fl(amax / 7) per group of a row, code = the nearest integer of
 *    fl(x / s), ties to even, clamped to [-8, 7], two's-complement nibbles
 *    with element 2j low, y = BF16(fl(code * s));
 *  - activation observers (the page names them): the latest batch's extremes,
 *    the running extremes, or the moving average m + c * (b - m).
 *
 * Parity unpinned against the pages: they fix no value for the multiplier
 * form of the scales, the MXFP8 exponent rule, the FP32 evaluation order, the
 * observer rules, the E4M3 maximum of 256 or the INT4 convention.  The tests
 * pin each function to its stated definition instead (closed forms, exact
 * rational arithmetic, brute force over BF16 patterns).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OC_API __attribute__((visibility("default")))

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ------------------------------------------------------------------------ */
/* Scalar codecs                                                             */
/* ------------------------------------------------------------------------ */

/* BF16 is the upper half of a binary32 pattern: widening is exact. */
OC_API float oc_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* binary32 -> BF16, round to nearest, ties to even; overflow gives +-Inf. */
OC_API uint16_t oc_f32_to_bf16(float f) {
    uint32_t u = f2u(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u); /* NaN stays NaN */
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;                  /* the 16 bits dropped */
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;  /* carries into exponent */
    return (uint16_t)keep;
}

/* E4M3 (float8_e4m3fn): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, NaN = S.1111.111, largest finite 0x7E = 448 ([LPRL] dtype;
 * [VERL] 2.3 gives FP8_E4M3_MAX = 448.0). */
OC_API float oc_e4m3_decode(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9)                 /* m/8 * 2^-6 */
                          : ldexp(8.0 + (double)m, e - 7 - 3);  /* (1+m/8) * 2^(e-7) */
    return (float)(sign ? -mag : mag);
}

/* Saturating round-to-nearest-even cast of a binary32 value to E4M3. */
OC_API uint8_t oc_e4m3_encode(float v) {
    uint32_t u = f2u(v);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint8_t)(sign | 0x7f);         /* NaN in: outside the contract */
    float mag = u2f(a);
    if (mag >= 448.0f) return (uint8_t)(sign | 0x7e);           /* saturate (Inf included) */
    if (mag < 0.015625f) {
        /* below 2^-6 the E4M3 grid is k * 2^-9, k = 0..7 (k = 8 is the first
         * normal, code 0x08).  mag * 512 is exact; round half to even. */
        float k = mag * 512.0f;
        float fl = floorf(k);
        float frac = k - fl;                                     /* exact */
        unsigned ki = (unsigned)fl;
        if (frac > 0.5f || (frac == 0.5f && (ki & 1u))) ki += 1u;
        return (uint8_t)(sign | ki);
    }
    /* normal: 1.m * 2^e, e in [-6, 8]; keep 3 of the 23 mantissa bits */
    int e = (int)(a >> 23) - 127;
    uint32_t man = a & 0x7fffffu;
    uint32_t keep = man >> 20, rest = man & 0xfffffu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep += 1u;
    if (keep == 8u) { keep = 0u; e += 1; }                       /* mantissa overflow */
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | (int)keep));
}

/* E2M1: 1 sign bit (bit 3), 2 exponent bits (bias 1), 1 mantissa bit.
 * Magnitudes 0..7 <-> {0, 0.5, 1, 1.5, 2, 3, 4, 6} ([VERL] 2.3). */
static const float oc_e2m1_grid[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

OC_API float oc_e2m1_decode(uint8_t c) {
    float mag = oc_e2m1_grid[c & 7];
    return (c & 8) ? -mag : mag;
}

/* Nearest grid point, ties to the even code, saturating at 6; the sign bit is
 * kept even when the magnitude rounds to zero.  Each threshold is the
 * midpoint of two neighbouring grid values; whether the midpoint itself goes
 * up or down is decided by which neighbour has the even code. */
OC_API uint8_t oc_e2m1_encode(float v) {
    uint8_t sign = (f2u(v) >> 31) ? 8 : 0;
    float a = fabsf(v);
    uint8_t c;
    if (a <= 0.25f) c = 0;        /* 0.25: between 0 (code 0) and 0.5 (code 1) -> 0 */
    else if (a < 0.75f) c = 1;    /* 0.75: 0.5 (1) vs 1.0 (2) -> 2 */
    else if (a <= 1.25f) c = 2;   /* 1.25: 1.0 (2) vs 1.5 (3) -> 2 */
    else if (a < 1.75f) c = 3;    /* 1.75: 1.5 (3) vs 2.0 (4) -> 4 */
    else if (a <= 2.5f) c = 4;    /* 2.5: 2.0 (4) vs 3.0 (5) -> 4 */
    else if (a < 3.5f) c = 5;     /* 3.5: 3.0 (5) vs 4.0 (6) -> 6 */
    else if (a <= 5.0f) c = 6;    /* 5.0: 4.0 (6) vs 6.0 (7) -> 6 */
    else c = 7;                   /* saturate */
    return (uint8_t)(sign | c);
}

/* UE8M0: an unsigned biased exponent byte, value 2^(byte-127).  The byte 255
 * (NaN) is never produced by the quantizer. */
OC_API float oc_ue8m0_decode(uint8_t b) { return (float)ldexp(1.0, (int)b - 127); }

/* MXFP8 shared exponent ([LPRL] "3. Unified MXFP8" fixes only that it is a
 * power of two).  Reading: the power-of-two counterpart of amax / 448 -- the
 * smallest integer e with amax <= 448 * 2^e, so no element of the block
 * saturates -- clamped to the UE8M0 range (e >= -127).  Evaluated exactly in
 * double precision (448 * 2^e is exact there for every e used). */
OC_API uint8_t oc_mxfp8_scale_byte(float amax) {
    double a = (double)amax;
    int e = -127;
    while (a > ldexp(448.0, e)) e++;
    return (uint8_t)(e + 127);
}

/* ------------------------------------------------------------------------ */
/* Block-wise FP8, 128 x 128 tiles, FP32 scales ([LPRL] "Choose a precision",  */
/* "2. Unified block-wise FP8")                                               */
/* ------------------------------------------------------------------------ */

/* w: [M, N] BF16 row-major.  q: [M, N] E4M3 codes.  s: [ceil(M/128),
 * ceil(N/128)] FP32, row-major; tile (i, j) covers rows [128i, 128i+128) and
 * columns [128j, 128j+128), clipped at the tensor edge. */
OC_API void oc_fp8blk_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, float* s) {
    const int64_t T = 128;
    int64_t tiles_m = (M + T - 1) / T, tiles_n = (N + T - 1) / T;
    for (int64_t ti = 0; ti < tiles_m; ti++) {
        for (int64_t tj = 0; tj < tiles_n; tj++) {
            int64_t r0 = ti * T, r1 = (r0 + T < M) ? r0 + T : M;
            int64_t c0 = tj * T, c1 = (c0 + T < N) ? c0 + T : N;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = c0; c < c1; c++) {
                    float a = fabsf(oc_bf16_to_f32(w[r * N + c]));
                    if (a > amax) amax = a;
                }
            float scale = amax / 448.0f;                  /* fl(amax / 448) */
            s[ti * tiles_n + tj] = scale;
            for (int64_t r = r0; r < r1; r++)
                for (int64_t c = c0; c < c1; c++) {
                    float x = oc_bf16_to_f32(w[r * N + c]);
                    uint8_t code;
                    if (scale == 0.0f) code = (f2u(x) >> 31) ? 0x80 : 0x00;
                    else code = oc_e4m3_encode(x / scale);  /* E4M3(fl(x / s)) */
                    q[r * N + c] = code;
                }
        }
    }
}

/* y = BF16(fl(E4M3value * s_tile)). */
OC_API void oc_fp8blk_dequantize(const uint8_t* q, const float* s, int64_t M, int64_t N, uint16_t* y) {
    const int64_t T = 128;
    int64_t tiles_n = (N + T - 1) / T;
    for (int64_t r = 0; r < M; r++)
        for (int64_t c = 0; c < N; c++) {
            float scale = s[(r / T) * tiles_n + (c / T)];
            y[r * N + c] = oc_f32_to_bf16(oc_e4m3_decode(q[r * N + c]) * scale);
        }
}

/* ------------------------------------------------------------------------ */
/* MXFP8: 1 x 32 blocks along a row, UE8M0 scale byte, E4M3 values            */
/* ([LPRL] "3. Unified MXFP8")                                               */
/* ------------------------------------------------------------------------ */

/* N must be a multiple of 32.  q: [M, N] codes; e: [M, N/32] scale bytes.
 * `rule` turns the block amax into the scale byte. */
static void mxfp8_quantize_with(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e,
                                uint8_t (*rule)(float)) {
    int64_t nb = N / 32;
    for (int64_t r = 0; r < M; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint16_t* blk = w + r * N + b * 32;
            float amax = 0.0f;
            for (int k = 0; k < 32; k++) {
                float a = fabsf(oc_bf16_to_f32(blk[k]));
                if (a > amax) amax = a;
            }
            uint8_t byte = rule(amax);
            e[r * nb + b] = byte;
            float X = oc_ue8m0_decode(byte);              /* 2^(byte-127) */
            for (int k = 0; k < 32; k++)
                q[r * N + b * 32 + k] = oc_e4m3_encode(oc_bf16_to_f32(blk[k]) / X);
        }
}

OC_API void oc_mxfp8_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e) {
    mxfp8_quantize_with(w, M, N, q, e, oc_mxfp8_scale_byte);
}

/* MXFP8 with the floor exponent rule of the OCP Microscaling (MX) Formats
 * specification v1.0 (conversion of FP32 vectors to MX, section 6.3): the
 * shared exponent is floor(log2(amax)) minus the largest exponent of the
 * element format (8 for E4M3, whose maximum is 1.75 * 2^8), and a scaled
 * element beyond 448 saturates.  The pages fix only "UE8M0 power-of-two
 * scales"; this is the alternative to the no-saturation rule above.  A block
 * of zeros gets byte 0; the byte is clamped to [0, 254]. */
OC_API uint8_t oc_mxfp8_floor_scale_byte(float amax) {
    if (amax == 0.0f) return 0;
    int k;
    (void)frexp((double)amax, &k);          /* amax = m * 2^k, 0.5 <= m < 1 */
    int e = (k - 1) - 8;                    /* floor(log2 amax) - 8 */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (uint8_t)(e + 127);
}

/* Same layout as oc_mxfp8_quantize; codes E4M3(fl(x / 2^(byte-127))), saturating. */
OC_API void oc_mxfp8_floor_quantize(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e) {
    mxfp8_quantize_with(w, M, N, q, e, oc_mxfp8_floor_scale_byte);
}

/* y = BF16(fl(E4M3value * 2^(byte-127))). */
OC_API void oc_mxfp8_dequantize(const uint8_t* q, const uint8_t* e, int64_t M, int64_t N, uint16_t* y) {
    int64_t nb = N / 32;
    for (int64_t r = 0; r < M; r++)
        for (int64_t c = 0; c < N; c++) {
            float X = oc_ue8m0_decode(e[r * nb + c / 32]);
            y[r * N + c] = oc_f32_to_bf16(oc_e4m3_decode(q[r * N + c]) * X);
        }
}

/* ------------------------------------------------------------------------ */
/* NVFP4: E2M1 values, 1 x 16 blocks, E4M3 block scale, FP32 global scale     */
/* ([LPRL] "4. NVFP4"; [VERL] 2.3, 2.4, 2.5, 3.3)                             */
/* ------------------------------------------------------------------------ */

/* max |x| over n BF16 values (exact: a maximum needs no rounding). */
OC_API float oc_amax_bf16(const uint16_t* w, int64_t n) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(oc_bf16_to_f32(w[i]));
        if (a > amax) amax = a;
    }
    return amax;
}

/* Global scale g = fl(A / (6 * 448)); 6 * 448 = 2688 is exact.  A is the
 * amax of the tensor, or of its whole sibling group ([VERL] 2.4). */
OC_API float oc_nvfp4_global_scale(float A) { return A / (6.0f * 448.0f); }

/* The global scale with another E4M3 maximum in the denominator:
 * fl(A / (6 * e4m3_max)).  The vime pull request 503 review quotes a
 * configuration in which the NVFP4 "4over6" switch with its "E4M3 use 256"
 * flag sets e4m3_max to 256 instead of 448; the global scale of "verl NVFP4
 * QAT" 2.3 is amax over (FP4 max x FP8 max), so it becomes A / 1536.  The
 * per-block choice that gives "4over6" its name is not described on the
 * pages and is not modelled here. */
OC_API float oc_nvfp4_global_scale_max(float A, int e4m3_max) { return A / (6.0f * (float)e4m3_max); }

/* The same global scale in the reciprocal form some exporters store
 * ("verl NVFP4 QAT" 2.5: a compressed-tensors export whose sibling groups
 * are fused by taking the minimum of this form): fl(2688 / A).  A group of
 * zeros gives +Inf (the IEEE quotient). */
OC_API float oc_nvfp4_global_scale_reciprocal(float A) { return (6.0f * 448.0f) / A; }

/* The E4M3 block-scale code of a block with amax b under global scale g. */
OC_API uint8_t oc_nvfp4_block_scale(float b, float g) {
    if (g == 0.0f) return 0x00;
    float t = b / 6.0f;                                   /* fl(b / FP4_E2M1_MAX) */
    return oc_e4m3_encode(t / g);                         /* E4M3(fl(t / g)) */
}

/* The effective FP32 multiplier of a block: S = fl(E4M3value * g). */
OC_API float oc_nvfp4_effective_scale(uint8_t scode, float g) {
    return oc_e4m3_decode(scode) * g;
}

static uint8_t oc_nvfp4_code(float x, float S) {
    if (S == 0.0f) return (f2u(x) >> 31) ? 8 : 0;
    return oc_e2m1_encode(x / S);                         /* E2M1(fl(x / S)) */
}

/* N must be a multiple of 16.  p: [M, N/2] packed codes (element 2j in the
 * low nibble of byte j); s: [M, N/16] E4M3 block-scale codes. */
OC_API void oc_nvfp4_quantize(const uint16_t* w, int64_t M, int64_t N, float g, uint8_t* p, uint8_t* s) {
    int64_t nb = N / 16;
    for (int64_t r = 0; r < M; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint16_t* blk = w + r * N + b * 16;
            float bmax = 0.0f;
            for (int k = 0; k < 16; k++) {
                float a = fabsf(oc_bf16_to_f32(blk[k]));
                if (a > bmax) bmax = a;
            }
            uint8_t scode = oc_nvfp4_block_scale(bmax, g);
            s[r * nb + b] = scode;
            float S = oc_nvfp4_effective_scale(scode, g);
            for (int k = 0; k < 16; k += 2) {
                uint8_t lo = oc_nvfp4_code(oc_bf16_to_f32(blk[k]), S);
                uint8_t hi = oc_nvfp4_code(oc_bf16_to_f32(blk[k + 1]), S);
                p[(r * N + b * 16 + k) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
}

/* y = BF16(fl(E2M1value * S)), S = fl(E4M3value * g). */
OC_API void oc_nvfp4_dequantize(const uint8_t* p, const uint8_t* s, float g, int64_t M, int64_t N, uint16_t* y) {
    int64_t nb = N / 16;
    for (int64_t r = 0; r < M; r++)
        for (int64_t c = 0; c < N; c++) {
            float S = oc_nvfp4_effective_scale(s[r * nb + c / 16], g);
            uint8_t byte = p[(r * N + c) / 2];
            uint8_t code = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
            y[r * N + c] = oc_f32_to_bf16(oc_e2m1_decode(code) * S);
        }
}

/* Fake quantization ([VERL] 2.3): snap each element to the E2M1 grid under
 * its block's two-level scale and multiply back, BF16 in and BF16 out.  Per
 * element this is the quantizer's code followed by the dequantizer's product;
 * no codes are stored. */
OC_API void oc_nvfp4_qdq(const uint16_t* x, int64_t M, int64_t N, float g, uint16_t* y) {
    int64_t nb = N / 16;
    for (int64_t r = 0; r < M; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint16_t* blk = x + r * N + b * 16;
            float bmax = 0.0f;
            for (int k = 0; k < 16; k++) {
                float a = fabsf(oc_bf16_to_f32(blk[k]));
                if (a > bmax) bmax = a;
            }
            float S = oc_nvfp4_effective_scale(oc_nvfp4_block_scale(bmax, g), g);
            for (int k = 0; k < 16; k++) {
                uint8_t code = oc_nvfp4_code(oc_bf16_to_f32(blk[k]), S);
                y[r * N + b * 16 + k] = oc_f32_to_bf16(oc_e2m1_decode(code) * S);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* W4A4 activation observers ("verl NVFP4 QAT" 2.2: activation_observer,     */
/* default static_minmax, used only in W4A4 mode; 3.1: the choices           */
/* static_minmax, memoryless_minmax, minmax).  The pages name the observers  */
/* but do not define them.  Readings: each tracks the activations' min and   */
/* max per tensor; memoryless_minmax keeps only the latest batch's,          */
/* static_minmax the running extremes over every batch seen, and minmax a    */
/* moving average m += c * (batch - m) (c is the caller's averaging         */
/* constant; the first batch initialises it).  The activation global amax    */
/* is max(|min|, |max|).  Min and max order -0 below +0.                     */
/* ------------------------------------------------------------------------ */

static int oc_below(float a, float b) {        /* a < b in the order with -0 < +0 */
    return a < b || (a == b && signbit(a) && !signbit(b));
}

/* state[0] = min, state[1] = max, state[2] = batches seen (a count held in a
 * float).  Returns the activation amax after the update. */
OC_API float oc_observer_update(int kind, float c, float* state, const uint16_t* x, int64_t n) {
    float bmin = oc_bf16_to_f32(x[0]), bmax = bmin;
    for (int64_t i = 1; i < n; i++) {
        float v = oc_bf16_to_f32(x[i]);
        if (oc_below(v, bmin)) bmin = v;
        if (oc_below(bmax, v)) bmax = v;
    }
    if (kind == 0 || state[2] == 0.0f) {        /* memoryless, or the first batch */
        state[0] = bmin;
        state[1] = bmax;
    } else if (kind == 1) {                     /* static: running extremes */
        if (oc_below(bmin, state[0])) state[0] = bmin;
        if (oc_below(state[1], bmax)) state[1] = bmax;
    } else {                                    /* minmax: moving average */
        state[0] = state[0] + c * (bmin - state[0]);
        state[1] = state[1] + c * (bmax - state[1]);
    }
    state[2] = state[2] + 1.0f;
    float lo = fabsf(state[0]), hi = fabsf(state[1]);
    return lo > hi ? lo : hi;
}

/* ------------------------------------------------------------------------ */
/* INT4, symmetric, one FP32 scale per group of G elements along a row        */
/* ("低精度训练与 Rollout", "INT4 QAT 训练")                                  */
/* ------------------------------------------------------------------------ */
/* The page fixes only the group size (OPEN_TRAINING_INT4_GROUP_SIZE: 128 for
 * Moonlight-16B-A3B, Qwen3-30B-A3B and Qwen3-235B-A22B, 32 for
 * Kimi-K2-Thinking) and that QAT trains through a straight-through
 * estimator, whose forward pass is quantize then dequantize.  Readings (the
 * plainest ones):
 *  - groups run along a row (the GEMM reduction dimension), as the other
 *    block formats' blocks do; N % G == 0;
 *  - symmetric: s = fl(amax / 7), so the group's largest magnitude maps to
 *    the largest positive code, 7;
 *  - q = the integer nearest to fl(x / s), ties to even, clamped to [-8, 7]
 *    (a finite input never reaches the clamp); a zero scale gives code 0;
 *  - stored as two's-complement nibbles, element 2j in the low nibble of
 *    byte j; s is FP32 [M, N / G];
 *  - y = BF16(fl(q * s)).  An integer code has no sign of zero: -0 and
 *    negative values that round to 0 come back as +0. */

OC_API float oc_int4_scale(float amax) { return amax / 7.0f; }   /* fl(amax / 7) */

static int oc_int4_code(float x, float s) {
    if (s == 0.0f) return 0;
    float t = nearbyintf(x / s);   /* fl(x / s), then the nearest integer, ties to even */
    if (t > 7.0f) t = 7.0f;
    if (t < -8.0f) t = -8.0f;
    return (int)t;
}

static int oc_int4_decode(uint8_t nibble) { return (nibble & 8) ? (int)nibble - 16 : (int)nibble; }

static float oc_int4_group_amax(const uint16_t* grp, int64_t G) {
    float amax = 0.0f;
    for (int64_t k = 0; k < G; k++) {
        float a = fabsf(oc_bf16_to_f32(grp[k]));
        if (a > amax) amax = a;
    }
    return amax;
}

/* N % G == 0.  p: [M, N/2] packed codes; s: [M, N/G] FP32 scales. */
OC_API void oc_int4_quantize(const uint16_t* w, int64_t M, int64_t N, int64_t G, uint8_t* p, float* s) {
    int64_t ng = N / G;
    for (int64_t r = 0; r < M; r++)
        for (int64_t gi = 0; gi < ng; gi++) {
            const uint16_t* grp = w + r * N + gi * G;
            float scale = oc_int4_scale(oc_int4_group_amax(grp, G));
            s[r * ng + gi] = scale;
            for (int64_t k = 0; k < G; k += 2) {
                int lo = oc_int4_code(oc_bf16_to_f32(grp[k]), scale);
                int hi = oc_int4_code(oc_bf16_to_f32(grp[k + 1]), scale);
                p[(r * N + gi * G + k) / 2] = (uint8_t)((lo & 15) | ((hi & 15) << 4));
            }
        }
}

/* y = BF16(fl(q * s)). */
OC_API void oc_int4_dequantize(const uint8_t* p, const float* s, int64_t M, int64_t N, int64_t G, uint16_t* y) {
    int64_t ng = N / G;
    for (int64_t r = 0; r < M; r++)
        for (int64_t c = 0; c < N; c++) {
            float scale = s[r * ng + c / G];
            uint8_t byte = p[(r * N + c) / 2];
            uint8_t nibble = (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
            y[r * N + c] = oc_f32_to_bf16((float)oc_int4_decode(nibble) * scale);
        }
}

/* Fake quantization (the straight-through estimator's forward pass): each
 * element's code, multiplied back by its group's scale; no codes stored. */
OC_API void oc_int4_qdq(const uint16_t* x, int64_t M, int64_t N, int64_t G, uint16_t* y) {
    int64_t ng = N / G;
    for (int64_t r = 0; r < M; r++)
        for (int64_t gi = 0; gi < ng; gi++) {
            const uint16_t* grp = x + r * N + gi * G;
            float scale = oc_int4_scale(oc_int4_group_amax(grp, G));
            for (int64_t k = 0; k < G; k++) {
                int q = oc_int4_code(oc_bf16_to_f32(grp[k]), scale);
                y[r * N + gi * G + k] = oc_f32_to_bf16((float)q * scale);
            }
        }
}

/* Vectorised scalar entry points for the tests (n independent elements). */
OC_API void oc_e4m3_encode_n(const float* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oc_e4m3_encode(v[i]);
}
OC_API void oc_e2m1_encode_n(const float* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oc_e2m1_encode(v[i]);
}
OC_API void oc_f32_to_bf16_n(const float* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oc_f32_to_bf16(v[i]);
}
OC_API void oc_mxfp8_scale_byte_n(const float* amax, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oc_mxfp8_scale_byte(amax[i]);
}
OC_API void oc_mxfp8_floor_scale_byte_n(const float* amax, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; i++) out[i] = oc_mxfp8_floor_scale_byte(amax[i]);
}
