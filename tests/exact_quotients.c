/*
 * Exhaustive check of the activation quantizer's division-free quotients (test code; the device
 * versions are div6_rn and div_rn in the HIP library's device header). Both use only IEEE fp32
 * products and fused multiply-adds, which the host reproduces bit for bit, so the check runs on
 * the host over the whole domain the quantizer feeds them:
 *   ab: every non-negative finite bf16 value (a block's max |x|);
 *   A:  every positive finite bf16 value (a row's max |x|) with s = RN(A / 2688) >= 2^-96;
 *   q:  RN(ab / 6) and ab / 4 for every ab <= A.
 * It prints the mismatch counts: div6 against the IEEE quotient ab / 6, and div against q / s
 * where that quotient is at least 2^-11 (below it both results encode as E4M3 zero), plus any
 * case below 2^-11 where the fast result reaches 2^-10.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp exact_quotients.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float div6_fast(float a)
{
    const float y = from_bits(0x3E2AAAABu);   /* RN(1/6) */
    const float q = a * y;
    const float r = fmaf(-q, 6.0f, a);
    return fmaf(r, y, q);
}

static float div_fast(float q, float s, float ys)
{
    const float t = q * ys;
    const float r = fmaf(-t, s, q);
    return fmaf(r, ys, t);
}

int main(void)
{
    long bad6 = 0, bad = 0, bad_small = 0, pairs = 0;
    for (uint32_t h = 0; h < 0x7F80u; h++) {
        const float a = from_bits(h << 16);
        volatile float ieee = a / 6.0f;
        if (to_bits(div6_fast(a)) != to_bits(ieee)) bad6++;
    }
#pragma omp parallel for reduction(+ : bad, bad_small, pairs) schedule(dynamic, 16)
    for (uint32_t H = 1; H < 0x7F80u; H++) {
        const float A = from_bits(H << 16);
        const float s = A / 2688.0f;
        if (s < 0x1p-96f) continue;
        volatile float ys_v = 1.0f / s;
        const float ys = ys_v;
        for (uint32_t h = 0; h <= H; h++) {
            const float ab = from_bits(h << 16);
            for (int c = 0; c < 2; c++) {
                const float q = c ? ab * 0.25f : ab / 6.0f;
                volatile float ieee_v = q / s;
                const float ieee = ieee_v;
                const float fast = div_fast(q, s, ys);
                pairs++;
                if (ieee >= 0x1p-11f) bad += to_bits(fast) != to_bits(ieee);
                else bad_small += fast >= 0x1p-10f;
            }
        }
    }
    printf("div6 %ld div %ld small %ld pairs %ld\n", bad6, bad, bad_small, pairs);
    return 0;
}
