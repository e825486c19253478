/* Exhaustive check of the reciprocal quotient the quantisation kernels use
 * for bf16 rows.  For every positive finite bf16 value a (a row maximum) with
 * s = fl(a / 127) >= 2^-100, and every bf16 x with 0 <= x <= a:
 *   r = fl(1 / s), q0 = fl(x * r), e = fma(-q0, s, x), q = fma(e, r, q0)
 * must satisfy rint(q) == rint(fl(x / s)).  Negative x need no check: every
 * step is symmetric in the sign of x.  The kernels take the code as the low
 * bits of fl(q + 1.5 * 2^23) with no clamp: that is checked against the
 * clamped rint of the IEEE quotient for x and for -x.  Prints the number of
 * pairs checked and the number of mismatches of the quotient, of the bare
 * product q0 (not exact: the check can tell the two apart) and of the code. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int code_from_sum(float q)
{
    const float t = q + 0x1.8p23f;
    uint32_t u;
    memcpy(&u, &t, sizeof u);
    return (int)(u - 0x4B400000u);
}

static int clamped(float v)
{
    return (int)fminf(fmaxf(v, -127.0f), 127.0f);
}

static float bf16(uint32_t h)
{
    uint32_t u = h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int main(void)
{
    long long pairs = 0, bad = 0, bad_product = 0, bad_code = 0;
#pragma omp parallel for reduction(+ : pairs, bad, bad_product, bad_code) schedule(dynamic, 64)
    for (uint32_t ha = 1; ha < 0x7f80; ha++) {
        const float a = bf16(ha);
        const float s = a / 127.0f;
        if (!(s >= 0x1p-100f)) continue;
        const float r = 1.0f / s;
        for (uint32_t hx = 0; hx <= ha; hx++) {
            const float x = bf16(hx);
            const float ref = rintf(x / s);
            const float q0 = x * r;
            const float e = fmaf(-q0, s, x);
            const float q = fmaf(e, r, q0);
            bad += rintf(q) != ref;
            bad_product += rintf(q0) != ref;
            /* -x: the same steps with every sign flipped */
            const float nq0 = -x * r;
            const float nq = fmaf(fmaf(-nq0, s, -x), r, nq0);
            bad_code += code_from_sum(q) != clamped(ref);
            bad_code += code_from_sum(nq) != clamped(rintf(-x / s));
            pairs++;
        }
    }
    printf("%lld %lld %lld %lld\n", pairs, bad, bad_product, bad_code);
    return 0;
}
