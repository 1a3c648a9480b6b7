"""The append kernels form Delta = fp16(fp32(r / 15)) and the INT8 scale
s = fp16(fp32(amax / 127)) (KV4-RL Section 3 eq. 3.3 and Appendix A.3
"Encoding and allocation"; the binary32 quotient is the reading the oracle
takes) without a division instruction: q0 = a * RN(1/B), e = fma(-B, q0, a),
q = fma(e, RN(1/B), q0).  This test runs that sequence in IEEE binary32 (C
fmaf, subnormals kept, no contraction) over EVERY finite binary32 a >= 0 and
compares it with the binary64 quotient rounded to binary32, which is the
correctly rounded quotient (53 >= 2 * 24 + 2 bits).  It pins the arithmetic
identity the kernels rely on; the kernels' own bytes are compared with the
oracle in the GPU tests."""
import os
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
int main(int argc, char** argv)
{
    const float B = (float)atoi(argv[1]);
    const float y = 1.0f / B;
    long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 20)
    for (long long i = 0; i < 0x7F800000LL; ++i) {
        const float a = u2f((uint32_t)i);
        const float ref = (float)((double)a / (double)B);
        const float q0 = a * y;
        const float e = fmaf(-B, q0, a);
        const float q = fmaf(e, y, q0);
        if (f2u(q) != f2u(ref)) ++bad;
    }
    printf("%lld\n", bad);
    return 0;
}
"""


@pytest.mark.parametrize("divisor", [15, 127])
def test_correction_step_is_correctly_rounded_for_every_input(divisor):
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "div.c")
        exe = os.path.join(d, "div")
        open(src, "w").write(SRC)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-include", "stdlib.h",
                        src, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe, str(divisor)], check=True, capture_output=True, text=True,
                             timeout=600, env={**os.environ, "OMP_NUM_THREADS": str(min(8, os.cpu_count() or 1))})
    assert int(out.stdout.strip()) == 0
