"""W4A4 activation observers on the GPU against the oracle, bit for bit: the
observer state after every batch, the activation amax, and the activation
fake-quant (QDQ) under that amax.  Batches are seeded synthetic activations
(N(0, 1) with 0.01% outliers x 100, the W4A4 workload's distribution) at
growing scales, plus all-zero and sign-of-zero batches."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import host_u16, report, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


def batches(M, N, n, seed):
    out = []
    for t in range(n):
        sigma = float(np.ldexp(1.0, t % 5 - 2)) * (1.0 + 0.37 * t)
        out.append(synth.generate(seed, t, M, N, sigma, 0.0, 1e-4, 100.0))
    return out


def f32_bits(v):
    return np.asarray(v, np.float32).view(np.uint32)


@pytest.mark.parametrize("kind", ["memoryless_minmax", "static_minmax", "minmax"])
@pytest.mark.parametrize("M,N", [(1, 16), (37, 48), (512, 2048)])
def test_observer_sequence(lpq, kind, M, N):
    c = 0.01 if kind == "minmax" else 0.0
    state = lpq.lpq_observer_reset(device="cuda")
    ost = np.zeros(3, np.float32)
    bad = 0
    for t, x_np in enumerate(batches(M, N, 6, 1000 + M + N)):
        x = to_dev_bf16(x_np)
        amax = lpq.lpq_nvfp4_observe(x, state, kind, averaging_constant=c)
        a = O.observer_update(kind, ost, x_np, c=c)
        st = state.cpu().numpy()[:3]
        bad += int(not np.array_equal(f32_bits(st), f32_bits(ost))) + int(f32_bits(amax.item()) != f32_bits(a))
        if t in (0, 5):
            y = lpq.lpq_nvfp4_qdq(x, amax)
            bad += report(f"W4A4 QDQ {kind} {M}x{N} batch {t}", host_u16(y), O.nvfp4_qdq(x_np, O.nvfp4_global_scale(a)))
    print(f"  {kind} {M}x{N}: state {ost}", flush=True)
    assert bad == 0


def test_observer_zeros_and_moving_average(lpq):
    """All-zero and signed-zero batches, then a moving average with c = 1/2."""
    state = lpq.lpq_observer_reset(device="cuda")
    ost = np.zeros(3, np.float32)
    bad = 0
    seq = [np.zeros((2, 16), np.uint16), np.array([[0x8000] * 8 + [0x0000] * 8] * 2, np.uint16)]
    seq += batches(64, 64, 5, 7)
    for x_np in seq:
        amax = lpq.lpq_nvfp4_observe(to_dev_bf16(x_np), state, "minmax", averaging_constant=0.5)
        a = O.observer_update("minmax", ost, x_np, c=0.5)
        bad += int(not np.array_equal(f32_bits(state.cpu().numpy()[:3]), f32_bits(ost)))
        bad += int(f32_bits(amax.item()) != f32_bits(a))
    assert bad == 0


def test_global_scale_forms(lpq):
    rng = np.random.default_rng(3)
    A = rng.integers(0, 0x7F800000, 10000, dtype=np.uint32).view(np.float32)
    A = np.concatenate([A, np.array([0.0, 2688.0, 1e-45], np.float32)])
    g = lpq.lpq_nvfp4_global_scale(torch.from_numpy(A).cuda()).cpu().numpy()
    want = np.array([O.nvfp4_global_scale(a) for a in A], np.float32)
    assert report("global scale (multiplier form)", f32_bits(g), f32_bits(want)) == 0
