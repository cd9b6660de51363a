/* The quantize's division by 127 as three IEEE f32 operations (a product with
 * the rounded reciprocal, then one fused correction of the remainder), against
 * the correctly rounded quotient a / 127, for every finite non-negative f32
 * (subnormals included). Prints the number of inputs where they differ and the
 * first such input. Built and run by tests/test_quantize_arithmetic.py. (Dynamic
 * scheduling: the inputs whose quotient is subnormal are far slower on a CPU.) */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_to_float(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}
static uint32_t float_to_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

int main(void) {
    const float c = 1.0f / 127.0f; /* the reciprocal rounded to f32 */
    long long bad = 0;
    uint32_t first = 0xFFFFFFFFu;
#pragma omp parallel for schedule(dynamic, 1 << 20) reduction(+ : bad) reduction(min : first)
    for (long long i = 0; i <= 0x7F7FFFFFLL; ++i) {
        const float a = bits_to_float((uint32_t)i);
        const float q = a * c;
        const float r = fmaf(fmaf(-q, 127.0f, a), c, q);
        const volatile float want = a / 127.0f;
        if (float_to_bits(r) != float_to_bits(want)) {
            ++bad;
            if ((uint32_t)i < first) first = (uint32_t)i;
        }
    }
    printf("%lld %08x\n", bad, first);
    return 0;
}
