"""Host check of the quantiser's scale division (CPU; no GPU involved).

The INT8/INT4 quantiser kernels divide the row or group absolute maximum by
the largest code (127 or 7) without a division instruction: with
r = RN(1/qmax), q = RN(amax r), e = fma(-q, qmax, amax) (exact) and
y = fma(e, r, q).  The scales must equal the oracle's binary32 quotient bit
for bit, so y must be the correctly rounded quotient for every finite
amax >= 0.  This test compiles a few lines of C (IEEE binary32 with
subnormals, hardware fma) and compares y with amax / qmax over every 61st
non-negative finite bit pattern plus all subnormals and the values around
powers of two; the full sweep over all 2^31 patterns (about a minute) runs
with GEMV_FULL_DIVISION_SWEEP=1 and found no mismatch.  A planted mistake
(the product amax r without the remainder correction) must be caught."""
import os
import subprocess
import tempfile

import pytest

SRC = r"""
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static int plant;
static int bad(float x, float c, float r)
{
    const float q = x * r;
    const float e = fmaf(-q, c, x);
    const float y = plant ? q : fmaf(e, r, q);
    const float want = x / c;
    return u_of(y) != u_of(want);
}
int main(int argc, char** argv)
{
    const uint32_t stride = (uint32_t)strtoul(argv[1], 0, 10);
    plant = atoi(argv[2]);
    const float cs[2] = {7.0f, 127.0f};
    unsigned long long n = 0, fails = 0;
    for (int k = 0; k < 2; ++k) {
        const float c = cs[k];
        const float r = 1.0f / c;
        for (uint32_t u = 0; u < 0x7F800000u; u += stride) { fails += bad(f_of(u), c, r); ++n; }
        for (uint32_t u = 0; u < 0x00800000u; u += 7) { fails += bad(f_of(u), c, r); ++n; }
        for (int e = 1; e < 255; ++e)
            for (int d = -64; d <= 64; ++d) { fails += bad(f_of(((uint32_t)e << 23) + (uint32_t)d), c, r); ++n; }
    }
    printf("%llu %llu\n", n, fails);
    return 0;
}
"""


def _run(stride: int, plant: int):
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div.c"), os.path.join(d, "div")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
        out = subprocess.run([exe, str(stride), str(plant)], check=True, capture_output=True, text=True).stdout
    n, fails = map(int, out.split())
    return n, fails


def test_scale_division_is_correctly_rounded():
    full = os.environ.get("GEMV_FULL_DIVISION_SWEEP") == "1"
    n, fails = _run(1 if full else 61, 0)
    assert n > 60_000_000 and fails == 0, (n, fails)


def test_planted_missing_correction_is_caught():
    n, fails = _run(4099, 1)
    assert fails > 0, (n, fails)
