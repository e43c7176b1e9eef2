"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C oracle, built with -fsanitize=address,undefined, over every scalar
  cast and BF16 pattern and over edge shapes of every format (one element,
  ragged tiles, all-zero and signed-zero tensors, random finite patterns).
* The library's host code (argument checks, launch planning) built with the
  same sanitizers on the host side only, driven with invalid calls from C:
  each must be refused with its documented status before any launch, so no
  GPU is needed.
Any out-of-bounds access, signed overflow or undefined shift ends the program
with an error.
"""
import os
import shlex
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = "-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    return res.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", *SAN.split(), "-o", exe,
         os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "lpq_oracle.c"), "-lm"])
    out = run([exe], env=ENV, timeout=600)
    assert "clean under ASan/UBSan" in out


def test_library_host_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "precision_weight_quantization_amd", "csrc")
    # the host pass only is instrumented: -Xarch_host before each -fsanitize= option
    cmd = (f"{ROCM}/bin/hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -ffp-contract=off "
           f"-Xclang -target-feature -Xclang -packed-fp32-ops "
           f"-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
           f"-Xarch_host -fno-sanitize-recover=all -I{ROOT}/include -I{csrc} "
           f"-x c++ {os.path.join(HERE, 'abi_driver.c')} -x hip {os.path.join(csrc, 'lpq_kernels.hip')} -o {exe}")
    run(shlex.split(cmd), timeout=900)
    out = run([exe], env=ENV, timeout=300)
    assert "every invalid call refused" in out
