"""The density encode's quotient method, checked on the host.

The GPU encode divides a row's values by its scale s without a full IEEE division per
value: with k = 1 - exponent(s), s' = s 2^k in [1, 2) and v' = v 2^k (exact scalings),
y = RN(1 / s') (one IEEE division per row), q0 = RN(v' y), r = v' - q0 s' (one FMA,
exact) and q = RN(q0 + r y) -- Markstein's correction, which returns RN(v / s) when y
is within half an ulp of 1/s' and q0 within an ulp of v'/s'.  This test runs the same
sequence in C (fmaf, IEEE single precision, no contraction) against the IEEE quotient
over random and adversarial (v, s) pairs in every exponent range of s -- subnormal to
the largest finite, plus 0 and infinity -- and requires the densities (q + 1) / 2 to
agree bit for bit, and the quotients wherever |v / s| >= 2^-100.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

C_SRC = r"""
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t U(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static long bad_u = 0, bad_q = 0, n = 0;
static void one(float v, float s) {
    int ex;
    frexpf(s, &ex);
    int fin = s > 0.0f && s <= FLT_MAX;
    int k = fin ? 1 - ex : (s > 0.0f ? -300 : 0);
    float sp = fin ? ldexpf(s, k) : 1.0f;
    volatile float y = 1.0f / sp;
    float vp = ldexpf(v, k);
    volatile float q0 = vp * y;
    float r = fmaf(-q0, sp, vp);
    float q = fmaf(r, y, q0);
    volatile float ref = s > 0.0f ? v / s : 0.0f;
    volatile float u1 = (q + 1.0f) * 0.5f, u2 = (ref + 1.0f) * 0.5f;
    n++;
    if (U(u1) != U(u2) && !(isnan(u1) && isnan(u2))) bad_u++;
    if (fabsf(ref) >= 0x1p-100f && U(q) != U(ref)) bad_q++;
}
int main(void) {
    for (int es = -149; es <= 128; ++es) {
        for (long i = 0; i < 20000; ++i) {
            uint64_t a = rnd(), b = rnd();
            float s = es - 1 < -126 ? f((uint32_t)(a % 0x800000u) | 1u)
                                    : ldexpf(1.0f + (float)(a & 0x7fffff) / 8388608.0f, es - 1);
            if (!(s > 0.0f) || isinf(s)) continue;
            float v;
            switch (b & 3) {
                case 0: v = s * ((float)((b >> 2) & 0xffffff) / 16777216.0f); break;
                case 1: v = f(U(s) - (uint32_t)((b >> 2) % 4096)); break;
                case 2: v = ldexpf(1.0f + (float)((b >> 8) & 0x7fffff) / 8388608.0f, es - 1 - (int)((b >> 40) % 160)); break;
                default: v = f((U(s) & 0xff800000u) | (uint32_t)((b >> 2) & 0x7fffff)); break;
            }
            if (!(fabsf(v) <= s)) v = s;
            if (b & (1ull << 50)) v = -v;
            one(v, s);
        }
    }
    const float specials[] = {0.0f, INFINITY, FLT_MAX, f(1), f(0x007fffff), 0x1p-126f, 0x1p127f, f(0x3f7fffff)};
    for (int j = 0; j < 8; ++j)
        for (long i = 0; i < 20000; ++i) {
            float s = specials[j];
            uint64_t b = rnd();
            float v = s == 0.0f ? 0.0f
                      : isinf(s) ? ldexpf((float)(b & 0xffffff), (int)((b >> 30) % 200) - 100)
                                 : s * ((float)((b >> 2) & 0xffffff) / 16777216.0f);
            if (b & (1ull << 51)) v = -v;
            one(v, s);
        }
    /* every significand of v against an all-ones-significand scale, and against 1 */
    for (uint32_t m = 0; m < (1u << 23); m += 7) {
        one(f(0x3f000000u | m), f(0x3f7fffffu));
        one(-f(0x3f000000u | m), f(0x3f800000u));
    }
    one(INFINITY, INFINITY);
    one(-INFINITY, INFINITY);
    printf("%ld %ld %ld\n", n, bad_u, bad_q);
    return 0;
}
"""


def test_markstein_quotient_matches_ieee_division():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "q.c"), os.path.join(tmp, "q")
        with open(src, "w") as fh:
            fh.write(C_SRC)
        subprocess.run([cc, "-O2", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    n, bad_u, bad_q = (int(t) for t in out)
    assert n > 5_000_000
    assert bad_u == 0, f"{bad_u} of {n} densities differ from the IEEE quotient's"
    assert bad_q == 0, f"{bad_q} of {n} quotients differ from the IEEE quotient"
