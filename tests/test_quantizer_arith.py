"""Arithmetic identities the quantizer kernels rely on, checked on the CPU.

The group scale s = (wmax - wmin)/Q (and the symmetric wmax/(2^(b-1) - 1))
is computed in the kernels without a division: q0 = fl(x y) with
y = fl(1/Q), then one fused multiply-add for the exact residual and one to
correct q0.  For the codes to stay bit-exact to the quantizer's definition
this must equal the IEEE quotient for every non-negative finite x and every
divisor that bit widths 2..8 produce.  The default run samples every 251st
fp32 bit pattern plus all subnormals and the top binade; with
AR_EXHAUSTIVE=1 it checks all 2^31 - 2^23 patterns (about 25 s per
divisor)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DIVISORS = [1, 3, 7, 15, 31, 63, 127, 255]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path_factory.mktemp("divq") / "divq_check")
    # no contraction: the program's fmaf calls are the only fused operations
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "divq_check.c"), "-lm"],
                   check=True)
    return exe


@pytest.mark.parametrize("d", DIVISORS)
def test_corrected_product_equals_ieee_quotient(checker, d):
    stride = 1 if os.environ.get("AR_EXHAUSTIVE") == "1" else 251
    out = subprocess.run([checker, str(d), str(stride)], check=True, capture_output=True, text=True).stdout.split()
    bad, n, first = int(out[0]), int(out[1]), out[2]
    assert n > 8_000_000
    assert bad == 0, f"divisor {d}: {bad} of {n} differ, first x bits {first}"
