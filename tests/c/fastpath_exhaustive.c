/*
 * Exhaustive CPU check of the division-free tile arithmetic that the gfx950
 * store kernels use on their fast path (test infrastructure; built and run by
 * tests/test_fastpath_exhaustive.py).
 *
 * The kernels quantize a 128-element bf16 tile with scale = RN32(amax / 448)
 * and code = e4m3(RN32(x / scale)).  For tiles whose amax has a biased bf16
 * exponent E in [72, 254] (scale >= 2^-64, normal) they avoid both divisions:
 *   n  = 128 + m (m: the 7 mantissa bits of amax), c = RN32(1/448)
 *   q0 = n * c;  S = fma(fma(-q0, 448, n), c, q0)        -> RN32(n / 448)
 *   Y  = fma(fma(-S, y0, 1), y0, y0), y0 a reciprocal estimate of S
 *   scale = S * 2^(E-134),  y = Y * 2^(134-E)
 *   q = x * y;  t = fma(q, scale, -x);  q' = fma(-t, y, q)
 * This program walks that whole domain: every amax pattern with E in
 * [72, 254] and, for each, every bf16 x with |x| <= amax, both signs.  It
 * checks that
 *   - scale equals the IEEE binary32 division amax / 448 bit for bit,
 *   - Y equals RN32(1/S) for every estimate y0 within 3 ulp of it, and y
 *     equals the IEEE division 1 / scale,
 *   - the e4m3 code of q' equals the e4m3 code of the IEEE division x / scale
 *     (the encoder is the oracle's kvo_e4m3_encode, linked in).
 * q' itself may differ from RN32(x / scale) in its last bit; those pairs are
 * counted and reported, and each one's code is compared.
 *
 * With the arguments "product E" the program instead takes q' = x * y (a
 * plain reciprocal multiply) over the one binade of amax exponent E, so that
 * a test can show it does report code differences where they exist.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp, with
 * oracle/kvpub_oracle.c, -lm.  Exit status 0 iff no check failed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t kvo_e4m3_encode(float v);

static float from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t to_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float bf16(uint32_t b) { return from_bits(b << 16); }

int main(int argc, char **argv)
{
    const float c = 1.0f / 448.0f; /* RN32(1/448) */
    const int product = argc == 3 && strcmp(argv[1], "product") == 0;
    const int first = product ? atoi(argv[2]) << 7 : 72 << 7;
    const int last = product ? (atoi(argv[2]) << 7) + 127 : (255 << 7) - 1;
    long long pairs = 0, quotient_bits_differ = 0, code_differs = 0;
    long long scale_bad = 0, recip_bad = 0, estimate_bad = 0;
    int ab;

#pragma omp parallel for schedule(dynamic, 16) \
    reduction(+ : pairs, quotient_bits_differ, code_differs, scale_bad, recip_bad, estimate_bad)
    for (ab = first; ab <= last; ++ab) {
        const float amax = bf16((uint32_t)ab);
        const int E = ab >> 7;
        const float n = (float)((ab & 127) | 128);
        const float q0 = n * c;
        const float S = fmaf(fmaf(-q0, 448.0f, n), c, q0);
        const float Yref = 1.0f / S;
        int d;
        for (d = -3; d <= 3; ++d) {
            const float y0 = from_bits(to_bits(Yref) + (uint32_t)d);
            const float Y = fmaf(fmaf(-S, y0, 1.0f), y0, y0);
            if (to_bits(Y) != to_bits(Yref)) ++estimate_bad;
        }
        const float scale = ldexpf(S, E - 134);
        const float y = ldexpf(Yref, 134 - E);
        if (to_bits(scale) != to_bits(amax / 448.0f)) ++scale_bad;
        if (to_bits(y) != to_bits(1.0f / scale)) ++recip_bad;
        uint32_t xb;
        for (xb = 0; xb <= (uint32_t)ab; ++xb) {
            int sgn;
            for (sgn = 0; sgn < 2; ++sgn) {
                const float x = bf16(xb | (sgn ? 0x8000u : 0u));
                const float q = x * y;
                const float t = fmaf(q, scale, -x);
                const float qf = product ? q : fmaf(-t, y, q);
                const float qd = x / scale;
                ++pairs;
                if (to_bits(qf) != to_bits(qd)) {
                    ++quotient_bits_differ;
                    if (kvo_e4m3_encode(qf) != kvo_e4m3_encode(qd)) ++code_differs;
                }
            }
        }
    }
    printf("amax_patterns %d pairs %lld quotient_bits_differ %lld code_differs %lld "
           "scale_bad %lld recip_bad %lld estimate_bad %lld\n",
           last - first + 1, pairs, quotient_bits_differ, code_differs, scale_bad, recip_bad,
           estimate_bad);
    return (code_differs || scale_bad || recip_bad || estimate_bad) ? 1 : 0;
}
