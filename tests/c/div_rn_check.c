/* CPU check of the quotient scheme the dynamic-quantization kernels use
 * (div_rn in the library's device code, restated here in C): one correctly
 * rounded reciprocal per group, then Markstein's FMA correction per value,
 * groups whose maximum is below 2^-60 scaled by 2^64 first, and the sign of
 * x copied onto the result.  Claim: the result equals the correctly rounded
 * x / s wherever |x / s| >= 2^-12 and has the sign of x / s elsewhere, for
 * every finite 16-bit x within the group maximum.  Usage:
 *   div_rn_check <stride over bf16 maxima> <0 = bf16 x, 1 = fp16 x>
 * Prints "checked N mismatches M". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bf16(uint16_t b) { uint32_t u = (uint32_t)b << 16; float f; memcpy(&f, &u, 4); return f; }
static float from_fp16(uint16_t b) {
    int s = b >> 15, e = (b >> 10) & 31, m = b & 1023;
    float v;
    if (e == 31) return NAN;
    v = e ? ldexpf((float)(m | 1024), e - 25) : ldexpf((float)m, -24);
    return s ? -v : v;
}
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char **argv) {
    const int stride = argc > 1 ? atoi(argv[1]) : 61;
    const int fp16 = argc > 2 ? atoi(argv[2]) : 0;
    long checked = 0, bad = 0;
    for (int qi = 0; qi < 2; ++qi) {
        const float qmax = qi ? 127.0f : 448.0f;
        for (uint32_t ab = 1; ab < 0x7F80; ab += stride) {
            const float amax = from_bf16((uint16_t)ab);
            const float s = amax / qmax;
            if (!(s > 0)) continue;
            const float k = amax < 0x1p-60f ? 0x1p64f : 1.0f;
            const float sk = s * k, y = 1.0f / sk;
            for (uint32_t b = 0; b < 65536; ++b) {
                const float x = fp16 ? from_fp16((uint16_t)b) : from_bf16((uint16_t)b);
                if (!isfinite(x) || fabsf(x) > amax) continue;
                const float ref = x / s;
                const float xk = x * k, q = xk * y;
                const float r = fmaf(-sk, q, xk);
                const float got = copysignf(fmaf(r, y, q), x);
                ++checked;
                if (fabsf(ref) >= 0x1p-12f ? bits(got) != bits(ref) : signbit(got) != signbit(ref))
                    ++bad;
            }
        }
    }
    printf("checked %ld mismatches %ld\n", checked, bad);
    return bad != 0;
}
