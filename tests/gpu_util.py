"""Helpers shared by the GPU tests: host <-> device transfers of bit patterns."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def to_dev_bf16(w: np.ndarray) -> torch.Tensor:
    """uint16 BF16 bit patterns (numpy) -> bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(DEV).view(torch.bfloat16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits32(x) -> np.ndarray:
    """binary32 bit patterns of a device tensor, a numpy array or a Python float:
    FP32 results are compared as bits (a -0 / +0 or NaN-payload difference counts)."""
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.atleast_1d(np.asarray(x, np.float32)).view(np.uint32)


def same_bits(a, b) -> bool:
    return np.array_equal(bits32(a), bits32(b))


def mismatches(a: np.ndarray, b: np.ndarray) -> int:
    assert a.shape == b.shape, (a.shape, b.shape)
    return int(np.count_nonzero(a != b))


def report(name: str, a: np.ndarray, b: np.ndarray) -> int:
    n = mismatches(a, b)
    print(f"  {name}: {n} mismatches of {a.size}", flush=True)
    return n


# --------------------------------------------------------------------------- brute force over BF16

def finite_bf16():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (u.astype(np.uint32) << 16).view(np.float32)
    return u[np.isfinite(f)]


def f2bf(x):
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def brute_blocks(width, seed):
    """Two blocks per finite BF16 pattern p: {p alone with zeros} and {p with an
    anchor a >= |p| and fillers inside [-|a|, |a|]}; p sits at a random position."""
    rng = np.random.default_rng(seed)
    pats = finite_bf16()
    n = pats.size
    pf = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    A = np.zeros((n, width), np.uint16)
    pos = rng.integers(0, width, n)
    A[np.arange(n), pos] = pats
    fac = rng.choice(np.array([1.0, 1.0000001, 1.5, 2.0, 3.0, 7.9, 100.0, 6.0, 448.0, 2688.0]), n)
    a = np.minimum(np.abs(pf) * fac, 3.3e38)
    a = np.where(a == 0, rng.choice(np.array([0.0, 1e-40, 1.0]), n), a)
    fill = rng.uniform(-1, 1, (n, width)) * a[:, None]
    B = f2bf(fill.astype(np.float32))
    apos = (pos + 1 + rng.integers(0, width - 1, n)) % width
    B[np.arange(n), apos] = f2bf((a * rng.choice([-1.0, 1.0], n)).astype(np.float32))
    B[np.arange(n), pos] = pats
    return np.concatenate([A, B])
