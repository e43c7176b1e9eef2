"""Device-side generation of the synthetic tensors of ``synth.synth`` (bit-identical)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

from . import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "synth_gen.hip")
LIB = os.path.join(_HERE, "libsynth.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    subprocess.check_call(["/opt/rocm/bin/hipcc", *FLAGS, "-o", LIB + ".tmp", SRC],
                          stderr=subprocess.DEVNULL)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is missing: run synth.gpu.build()")
        L = ctypes.CDLL(LIB)
        L.synth_fill_bf16.restype = ctypes.c_int
        L.synth_fill_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                      ctypes.c_uint64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_double, ctypes.c_void_p]
        _lib = L
    return _lib


def fill(out: torch.Tensor, seed: int, stream_id: int, dist) -> torch.Tensor:
    """Fill a 2-D bfloat16 device tensor with the tensor ``synth.generate(seed, stream_id, M, N, *dist)``."""
    assert out.dim() == 2 and out.is_contiguous() and out.element_size() == 2
    M, N = out.shape
    sigma, row_sigma, p, f = dist
    rc = _L().synth_fill_bf16(out.data_ptr(), M, N, seed, stream_id, float(sigma), float(row_sigma), float(p),
                              float(f), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_bf16 failed ({rc})")
    return out


def generate(seed: int, stream_id: int, M: int, N: int, dist, device="cuda") -> torch.Tensor:
    return fill(torch.empty((M, N), dtype=torch.bfloat16, device=device), seed, stream_id, dist)


def single_linear(device="cuda") -> torch.Tensor:
    w = generate(synth.seed_of(1), synth.stream_of(0, 0, 0), 256, 512, synth.DIST_MOE, device)
    w[128:256, 128:256] = 0
    return w
