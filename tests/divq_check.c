/* Checks the division identity the quantizer kernels use for the group
 * scale: with y = fl(1/d), q0 = fl(x*y), res = fma(-q0, d, x), the value
 * fma(res, y, q0) equals the IEEE quotient fl(x/d).
 *
 *   divq_check D STRIDE   checks x = every STRIDE-th non-negative finite fp32
 *                         bit pattern, plus every subnormal and every x of
 *                         the top binade when STRIDE > 1
 * Prints the number of mismatches and the first one. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int check(uint32_t i, float d, float y) {
    const float x = from_bits(i);
    const float ref = x / d;
    const float q0 = x * y;
    const float res = fmaf(-q0, d, x);
    const float q1 = fmaf(res, y, q0);
    return to_bits(q1) != to_bits(ref);
}

int main(int argc, char** argv) {
    if (argc < 3) return 2;
    volatile float dv = (float)atof(argv[1]);
    const float d = dv;
    const float y = 1.0f / dv;
    const uint32_t stride = (uint32_t)strtoul(argv[2], NULL, 10);
    uint64_t bad = 0, n = 0;
    uint32_t first = 0;
    for (uint64_t i = 0; i < 0x7f800000ull; i += stride, ++n)
        if (check((uint32_t)i, d, y) && !bad++) first = (uint32_t)i;
    if (stride > 1) {
        for (uint32_t i = 0; i < 0x00800000u; ++i, ++n)          /* subnormals */
            if (check(i, d, y) && !bad++) first = i;
        for (uint32_t i = 0x7f000000u; i < 0x7f800000u; ++i, ++n) /* top binade */
            if (check(i, d, y) && !bad++) first = i;
    }
    printf("%llu %llu 0x%08x\n", (unsigned long long)bad, (unsigned long long)n, first);
    return 0;
}
