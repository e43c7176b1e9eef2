"""The amax, observer and QDQ passes on large single tensors, against the oracle.

8177 x 16384 and 8192 x 16384 BF16 tensors (268 MB each, about 2,000 workgroups,
each folding its maximum into one slot with an atomic) go through the
single-tensor amax, a grouped amax with a second tensor in another group, and
two batches of the static min/max observer.  The inputs are drawn on the device
by the synthetic generator's GPU twin (the same bits as ``synth.generate``) and
copied to the host for the oracle.

A short-chunk form for calls of fewer than 2,048 workgroups was measured and not
kept: eight times the workgroups meant eight times the atomics on one address,
and the activation amax ran at half the speed."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import host_u16

pytestmark = pytest.mark.gpu

SMALL = (8177, 16384)   # 2,044 full chunks of 65,536 elements and a ragged one
LARGE = (8192, 16384)   # 2,048 full chunks


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


@pytest.fixture(scope="module")
def tensors():
    from synth import gpu as sgpu
    out = {}
    for i, (name, (M, N)) in enumerate((("small", SMALL), ("large", LARGE))):
        x = sgpu.generate(140, i, M, N, synth.DIST_MOE)
        out[name] = (x, host_u16(x))
    return out


def bits(v):
    return np.asarray(v, np.float32).view(np.uint32)


@pytest.mark.parametrize("name", ["small", "large"])
def test_amax_single(lpq, tensors, name):
    x, x_np = tensors[name]
    got = lpq.lpq_nvfp4_amax(x).item()
    want = O.amax(x_np)
    print(f"  amax {name} {tuple(x.shape)}: {got!r} vs {want!r}", flush=True)
    assert bits(got) == bits(want)


def test_amax_grouped_two_groups(lpq, tensors):
    """Two groups in one launch: the large tensor and a 64-row companion."""
    x, x_np = tensors["small"]
    from synth import gpu as sgpu
    c = sgpu.generate(141, 0, 64, 16384, synth.DIST_MOE)
    c_np = host_u16(c)
    amax = torch.empty(2, dtype=torch.float32, device="cuda")
    lpq.lpq_nvfp4_amax_grouped(lpq.TensorTable([(x, None, None, *SMALL, 0), (c, None, None, 64, 16384, 1)]), amax)
    got = amax.cpu().numpy()
    want = np.array([O.amax(x_np), O.amax(c_np)], np.float32)
    print(f"  grouped amax: {got} vs {want}", flush=True)
    assert np.array_equal(bits(got), bits(want))


@pytest.mark.parametrize("name", ["small", "large"])
def test_observer_large(lpq, tensors, name):
    """Two batches through the static min/max observer: state and amax after each."""
    x, x_np = tensors[name]
    state = lpq.lpq_observer_reset(device="cuda")
    ost = np.zeros(3, np.float32)
    for batch in range(2):
        amax = lpq.lpq_nvfp4_observe(x, state, "static_minmax")
        a = O.observer_update("static_minmax", ost, x_np)
        st = state.cpu().numpy()[:3]
        assert np.array_equal(bits(st), bits(ost)), (name, batch, st, ost)
        assert bits(amax.item()) == bits(a), (name, batch)


@pytest.mark.parametrize("M,N", [(8192, 2048), (2048, 16384), (2049, 16384), (8177, 16384)])
def test_qdq_single_both_shapes(lpq, M, N):
    """Single-tensor QDQ on both sides of the switch between the wide launch
    shape (at most 2^25 elements: the 8192 x 2048 activation, 2048 x 16384)
    and the streaming one (2049 x 16384, 8177 x 16384 with a ragged last
    chunk).  The global scale comes from the whole tensor; the QDQ output is
    compared on every 61st row and the last row."""
    from synth import gpu as sgpu
    x = sgpu.generate(142, M, M, N, synth.DIST_ACT)
    amax = lpq.lpq_nvfp4_amax(x)
    y = lpq.lpq_nvfp4_qdq(x, amax)
    A = O.amax(host_u16(x))
    assert bits(amax.item()) == bits(A)
    rows = np.unique(np.concatenate([np.arange(0, M, 61), [M - 1]]))
    idx = torch.as_tensor(rows, device=x.device)
    want = O.nvfp4_qdq(host_u16(x[idx]), O.nvfp4_global_scale(A))
    got = host_u16(y[idx])
    bad = int((got != want).sum())
    y2 = lpq.lpq_nvfp4_qdq(x)   # amax computed by the call (held in y's first word meanwhile)
    bad += int((host_u16(y2[idx]) != want).sum())
    print(f"  qdq {M}x{N}: {len(rows)} rows, {bad} mismatches", flush=True)
    assert bad == 0
