"""The quantizers compute the block scale's fp32(bamax / 6) as x * RN(1/6)
followed by one FMA correction step (device_common.h, div6) instead of the
division sequence.  This checks, on the host with C's fmaf, that the
three-operation sequence returns the IEEE quotient for every non-negative
finite fp32 from 2^-120 up (below 2^-120 the kernels divide), over all 2^31
bit patterns."""
import os
import subprocess
import tempfile

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
int main(void) {
    const float c = 0.16666667163372039794921875f;   /* RN(1/6) */
    unsigned long long bad = 0;
    #pragma omp parallel for reduction(+:bad) schedule(static)
    for (long long u = 0x03800000LL; u < 0x7F800000LL; u++) {   /* 2^-120 .. FLT_MAX */
        uint32_t b = (uint32_t)u;
        float x;
        memcpy(&x, &b, 4);
        volatile float want = x / 6.0f;
        float q0 = x * c;
        float q1 = fmaf(fmaf(-q0, 6.0f, x), c, q0);
        if (q1 != want) bad++;
    }
    printf("%llu\n", bad);
    return 0;
}
"""


def test_fma_corrected_division_by_six_is_exact():
    assert float.fromhex("0x1p-120") == 2.0 ** -120
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "div6.c")
        exe = os.path.join(d, "div6")
        open(c, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", c, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=300).stdout
    assert out.strip() == "0"
