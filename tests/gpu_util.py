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


def mismatches(a: np.ndarray, b: np.ndarray) -> int:
    assert a.shape == b.shape, (a.shape, b.shape)
    return int(np.count_nonzero(a != b))


def report(name: str, a: np.ndarray, b: np.ndarray) -> int:
    n = mismatches(a, b)
    print(f"  {name}: {n} mismatches of {a.size}", flush=True)
    return n
