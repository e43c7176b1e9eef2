"""Build step of the plain C consumer of liblpq.so (test infrastructure).

gcc compiles lpq_c_consumer.c against the HIP runtime's C API, the library
and the C oracle; the library paths are relative to the binary, so it runs
from any copy of the repository.  Needs no GPU to build.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "lpq_c_consumer.c")
BIN = os.path.join(HERE, "lpq_c_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    rpath = "$ORIGIN/../../precision_weight_quantization_amd:$ORIGIN/../../oracle:" + os.path.join(ROCM, "lib")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"), SRC, "-o", BIN + ".tmp",
           "-L" + os.path.join(ROOT, "precision_weight_quantization_amd"), "-llpq",
           "-L" + os.path.join(ROOT, "oracle"), "-llpq_oracle",
           "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + rpath]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("gcc failed building the C consumer")
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build())
