/*
 * Design check of the kernels' division (not part of the oracle): the GPU
 * computes RN(x / S) as  q0 = x*r;  t = fma(q0, S, -x);  q = fma(-t, r, q0)
 * with r = RN(1/S) (Markstein's correction step; P. Markstein, IBM J. Res.
 * Dev. 34(1), 1990).  This program replays that sequence with the C library's
 * fused multiply-add and compares it with the correctly rounded quotient
 * x / S for
 *   - every divisor significand in [1, 2) with index % stride == 0,
 *   - numerators: the 128 BF16 significands (mode 0) or RN(b / 6) for them
 *     (mode 1, the block-scale numerator of NVFP4),
 *   - numerator/divisor exponent offsets -12..12 and both signs.
 * The computation is scale-invariant while nothing under- or overflows, so
 * stride 1 is an exhaustive proof for the normal range.  Prints the number of
 * mismatches and returns non-zero if there is any.
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -o quotient_check quotient_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
    int mode = argc > 1 ? atoi(argv[1]) : 0;
    uint32_t stride = argc > 2 ? (uint32_t)atoi(argv[2]) : 1;
    float nums[128];
    for (uint32_t k = 0; k < 128; k++) {
        float b = bf(0x3f800000u | (k << 16));
        nums[k] = mode ? b / 6.0f : b;
    }
    long long bad = 0, checked = 0;
    for (uint32_t m = 0; m < (1u << 23); m += stride) {
        float S = bf(0x3f800000u | m);
        float r = 1.0f / S;
        for (int i = 0; i < 128; i++)
            for (int d = -12; d <= 12; d++)
                for (int sg = 0; sg < 2; sg++) {
                    float x = ldexpf(nums[i], d);
                    if (sg) x = -x;
                    float q0 = x * r;
                    float t = fmaf(q0, S, -x);
                    float q = fmaf(-t, r, q0);
                    checked++;
                    if (fb(q) != fb(x / S)) bad++;
                }
    }
    /* signed zeros and a zero divisor with r = 0 */
    float zs[2] = {0.0f, -0.0f};
    for (int i = 0; i < 2; i++) {
        float x = zs[i], S = 3.0f, r = 1.0f / S;
        float q0 = x * r, t = fmaf(q0, S, -x), q = fmaf(-t, r, q0);
        if (fb(q) != fb(x)) bad++;
        S = 0.0f; r = 0.0f;
        q0 = x * r; t = fmaf(q0, S, -x); q = fmaf(-t, r, q0);
        if (fb(q) != fb(x)) bad++;
        float y = i ? -1.5f : 1.5f;
        q0 = y * r; t = fmaf(q0, S, -y); q = fmaf(-t, r, q0);
        if (fb(q) != fb(i ? -0.0f : 0.0f)) bad++;
    }
    printf("mode %d stride %u checked %lld mismatches %lld\n", mode, stride, checked, bad);
    return bad != 0;
}
