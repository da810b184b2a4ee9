// The kernels' fold() (csrc/la_tile.h) on the host: for fp32 a and c of any magnitudes, s is the
// fp32 rounding of a + c and s + res equals a + c exactly (checked in fp64, where the sum of two
// fp32 values is exact).  Pairs with |c| > |a| are the case a compensation term can reach when
// the running sum it belongs to cancels towards zero.  Exit status 0 when every pair holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "la_tile.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float rand_float() {  // random sign, mantissa and exponent in [2^-40, 2^40)
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    const uint32_t sign = (uint32_t)(rng >> 63) << 31, mant = (uint32_t)(rng >> 20) & 0x7fffff;
    const uint32_t expo = (uint32_t)(127 - 40 + (rng % 80)) << 23;
    const uint32_t bits = sign | expo | mant;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

int main() {
    int failures = 0, big_c = 0;
    for (int i = 0; i < 1000000; ++i) {
        float a = rand_float(), c = rand_float();
        if (i % 3 == 0) c = -a * (1.f + 1e-6f * (float)(i % 7));  // near-total cancellation
        if (fabsf(c) > fabsf(a)) ++big_c;
        float s, res;
        lachunk::fold(a, c, s, res);
        const volatile float fs = a + c;
        if (s != fs || (double)s + (double)res != (double)a + (double)c) {
            if (failures < 10) printf("FAIL a=%a c=%a: s=%a res=%a\n", a, c, s, res);
            ++failures;
        }
    }
    printf("%s: %d failures in 1000000 pairs (%d with |c| > |a|)\n", failures ? "FAILED" : "ok", failures, big_c);
    return failures || big_c < 100000 ? 1 : 0;
}
