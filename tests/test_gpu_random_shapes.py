"""Seeded random shapes and magnitudes through every format, bit for bit against
the oracle: block-wise FP8, MXFP8, NVFP4 (quantize, dequantize, QDQ) and INT4
with groups of 32 and, where N allows, 128; and 12 more shapes through the fused
FP8 re-quantizers (tile scales 2^lo .. 2^hi of both signs, lo from -60 to 19),
and 12 with power-of-two tile scales from 2^-121 to 2^119.

24 shapes are drawn once from a fixed seed: M from 1 to 1500, N a multiple of
32 from 32 to 8192, so that most shapes end in a ragged chunk, tile or row band.
Each tensor is the synthetic weight distribution (N(0, sigma) times a lognormal
row factor, 0.1% outliers x 50) with sigma drawn log-uniformly from 1e-6 to 1e3,
drawn on the device by the generator's GPU twin (the same bits as
``synth.generate``) and copied to the host for the oracle."""
import numpy as np
import pytest
import torch

from tests.gpu_util import host_u16
from tests.test_gpu_int4 import check_int4
from tests.test_gpu_parity import check_fp8blk, check_mxfp8, check_nvfp4

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(24):
        M = int(rng.integers(1, 1501))
        N = 32 * int(rng.integers(1, 257))
        sigma = float(10.0 ** rng.uniform(-6.0, 3.0))
        out.append((i, M, N, sigma))
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


@pytest.mark.parametrize("i,M,N,sigma", CASES, ids=[f"{M}x{N}" for _, M, N, _ in CASES])
def test_random_shape_all_formats(lpq, i, M, N, sigma):
    from synth import gpu as sgpu
    w = host_u16(sgpu.generate(150, i, M, N, (sigma, 0.5, 0.001, 50.0)))
    name = f"{M}x{N} sigma {sigma:.3g}"
    print(f"  case {i}: {name}", flush=True)
    check_fp8blk(lpq, w, name)
    check_mxfp8(lpq, w, name)
    check_nvfp4(lpq, w, name)
    check_int4(lpq, w, 32, name)
    if N % 128 == 0:
        check_int4(lpq, w, 128, name)


def _requant_cases():
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(12):
        M = int(rng.integers(1, 1501))
        N = 32 * int(rng.integers(1, 257))
        lo = int(rng.integers(-60, 20))
        out.append((i, M, N, lo, lo + int(rng.integers(0, 30))))
    return out


RQ_CASES = _requant_cases()


@pytest.mark.parametrize("i,M,N,lo,hi", RQ_CASES, ids=[f"{M}x{N}" for _, M, N, _, _ in RQ_CASES])
def test_random_shape_requant(lpq, i, M, N, lo, hi):
    """Seeded E4M3 codes and tile scales 2^lo .. 2^hi of both signs, through the
    three fused FP8 re-quantizers."""
    from tests.test_gpu_requant import check_fp8, check_mx, check_nv, random_case
    q, s = random_case(M, N, 400 + i, lo, hi, signed=True)
    name = f"{M}x{N} scales 2^[{lo},{hi}]"
    print(f"  requant case {i}: {name}", flush=True)
    assert check_fp8(lpq, q, s, name) + check_mx(lpq, q, s, name) + check_nv(lpq, q, s, name) == 0


def _pow2_cases():
    rng = np.random.default_rng(20261205)
    out = []
    for i in range(12):
        M = int(rng.integers(1, 1501))
        N = 32 * int(rng.integers(1, 257))
        lo = int(rng.integers(-121, 100))
        out.append((i, M, N, lo, min(119, lo + int(rng.integers(0, 60)))))
    return out


POW2_CASES = _pow2_cases()


@pytest.mark.parametrize("i,M,N,lo,hi", POW2_CASES, ids=[f"{M}x{N}" for _, M, N, _, _ in POW2_CASES])
def test_random_shape_requant_pow2(lpq, i, M, N, lo, hi):
    """Seeded E4M3 codes under power-of-two tile scales 2^lo .. 2^hi (inside the
    range where FP8 -> NVFP4 takes its scaled decode, up to both of its edges),
    through the three fused FP8 re-quantizers."""
    from oracle import oracle as O
    from synth import synth
    from tests.test_gpu_requant import check_fp8, check_mx, check_nv, pow2_scales
    q = synth.e4m3_codes(500 + i, 1, M, N)
    s = pow2_scales(O.fp8blk_scale_shape(M, N), 600 + i, list(range(lo, hi + 1)))
    name = f"{M}x{N} scales 2^[{lo},{hi}]"
    print(f"  requant pow2 case {i}: {name}", flush=True)
    assert check_fp8(lpq, q, s, name) + check_mx(lpq, q, s, name) + check_nv(lpq, q, s, name) == 0
