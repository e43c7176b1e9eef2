"""Design checks of the kernels' arithmetic that run on the CPU.

The GPU's quotient RN(x / S) is one multiply and one Markstein correction
from r = RN(1/S); tests/kernel_arith/quotient_check.c replays that sequence
with C's fused multiply-add.  The default run samples every 256th divisor
significand; LPQ_EXHAUSTIVE=1 runs all 2^23 (about a minute per mode on 8
cores' worth of single-thread time; done once when the kernels were designed,
0 mismatches in both modes).
"""
import os
import subprocess

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kernel_arith")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("qc") / "quotient_check")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", exe,
                           os.path.join(HERE, "quotient_check.c"), "-lm"])
    return exe


@pytest.mark.parametrize("mode", [0, 1], ids=["bf16-numerators", "b-over-6-numerators"])
def test_markstein_quotient(checker, mode):
    stride = "1" if os.environ.get("LPQ_EXHAUSTIVE") == "1" else "256"
    out = subprocess.run([checker, str(mode), stride], capture_output=True, text=True, timeout=1200)
    print(out.stdout)
    assert out.returncode == 0 and " mismatches 0" in out.stdout
