/* Exhaustive check of the division by 6 used by the NVFP4 block-scale
 * kernels: for every fp32 bit pattern a with 2^-125 <= a < +inf,
 *   q = RN(a * RN(1/6)),  t = fma(-q, 6, a),  fma(t, RN(1/6), q)
 * equals the correctly rounded quotient RN(a / 6). (Below 2^-125 the kernels
 * divide.) Exit status 0 when every value agrees; the count of disagreeing
 * values, and the first few, are printed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

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

int main(void)
{
    const float zh = from_bits(0x3E2AAAABu); /* RN(1/6) */
    volatile float six = 6.0f, one = 1.0f;
    if (to_bits(one / six) != 0x3E2AAAABu) {
        printf("RN(1/6) is not 0x3E2AAAAB\n");
        return 2;
    }
    uint64_t bad = 0, n = 0;
    for (uint32_t u = 0x01000000u; u < 0x7F800000u; ++u, ++n) {
        const float a = from_bits(u);
        const float q = a * zh;
        const float got = fmaf(fmaf(-q, 6.0f, a), zh, q);
        const float want = a / six;
        if (to_bits(got) != to_bits(want)) {
            if (bad < 5)
                printf("a=%08x want %08x got %08x\n", u, to_bits(want), to_bits(got));
            ++bad;
        }
    }
    printf("checked %llu values, %llu disagree\n", (unsigned long long)n, (unsigned long long)bad);
    return bad != 0;
}
