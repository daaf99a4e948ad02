"""The activation quantizer's rounding on the device (the shared quant_quad
routine) takes round-half-away-from-zero of y = x * (1/d) as a truncating
conversion of y + copysign(0.5 - 2^-25, y), the addition in fp32.  This
checks that identity against C's roundf for every non-negative fp32 below
256 (the quantizer's |y| is at most 127; both forms are odd functions of y,
so the negative half is the mirror image).  Plain C on the host, compiled
here; it shares nothing with the oracle."""
import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
    const float h = 0.49999997f;                 /* 0.5 - 2^-25 */
    unsigned long long bad = 0, n = 0;
    for (uint32_t b = 0; b < 0x43800000u; b++) { /* +0 .. the float below 256 */
        float x;
        memcpy(&x, &b, 4);
        volatile float s = x + copysignf(h, x);
        if ((long)truncf(s) != (long)roundf(x)) {
            if (bad < 5) printf("mismatch at %a\n", x);
            bad++;
        }
        n++;
    }
    printf("%llu %llu\n", n, bad);
    return bad != 0;
}
"""


def test_round_half_away_identity():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "r.c"), os.path.join(d, "r")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.run([cc, "-O2", "-std=c99", "-o", exe, src, "-lm"], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    n, bad = map(int, r.stdout.split()[-2:])
    assert n == 0x43800000 and bad == 0, r.stdout
