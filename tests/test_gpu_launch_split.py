"""Grouped calls whose tables the library must split into several launches.

A launch's work map holds at most 8 runs of tensors with equal work-unit
counts.  Here 40 tensors cycle through 20 shapes, so every tensor starts a new
run and each call becomes several launches, with tensor offsets and work-unit
origins that restart in each.  Every format's grouped call is compared with
the oracle per tensor, bit for bit; NVFP4 sibling groups pair tensors that
fall on both sides of a launch boundary."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import host_u8, host_u16, report, same_bits, to_dev_bf16

pytestmark = pytest.mark.gpu

SHAPES = [(m, n) for m in (1, 64, 129, 300) for n in (128, 384, 640, 1024, 2176)]   # 20 shapes, N % 128 == 0
TENSORS = [SHAPES[i % len(SHAPES)] for i in range(40)]


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


@pytest.fixture(scope="module")
def weights():
    ws = [synth.generate(130, i, M, N, *synth.DIST_MOE) for i, (M, N) in enumerate(TENSORS)]
    return ws, [to_dev_bf16(w) for w in ws]


def _empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def test_split_fp8blk(lpq, weights):
    ws, dw = weights
    qs = [_empty((M, N), torch.uint8) for M, N in TENSORS]
    ss = [_empty(O.fp8blk_scale_shape(M, N), torch.float32) for M, N in TENSORS]
    ys = [_empty((M, N), torch.bfloat16) for M, N in TENSORS]
    lpq.lpq_quantize_fp8blk_grouped(lpq.TensorTable([(dw[i], qs[i], ss[i], M, N, 0) for i, (M, N) in enumerate(TENSORS)]))
    lpq.lpq_dequantize_fp8blk_grouped(lpq.TensorTable([(qs[i], ys[i], ss[i], M, N, 0) for i, (M, N) in enumerate(TENSORS)]))
    bad = 0
    for i in range(len(TENSORS)):
        oq, os_ = O.fp8blk_quantize(ws[i])
        bad += report(f"fp8blk codes {i}", host_u8(qs[i]), oq) + report("  scales", ss[i].cpu().numpy(), os_)
        bad += report("  dequant", host_u16(ys[i]), O.fp8blk_dequantize(oq, os_))
    assert bad == 0


def test_split_mxfp8(lpq, weights):
    ws, dw = weights
    qs = [_empty((M, N), torch.uint8) for M, N in TENSORS]
    es = [_empty((M, N // 32), torch.uint8) for M, N in TENSORS]
    ys = [_empty((M, N), torch.bfloat16) for M, N in TENSORS]
    lpq.lpq_quantize_mxfp8_grouped(lpq.TensorTable([(dw[i], qs[i], es[i], M, N, 0) for i, (M, N) in enumerate(TENSORS)]))
    lpq.lpq_dequantize_mxfp8_grouped(lpq.TensorTable([(qs[i], ys[i], es[i], M, N, 0) for i, (M, N) in enumerate(TENSORS)]))
    bad = 0
    for i in range(len(TENSORS)):
        oq, oe = O.mxfp8_quantize(ws[i])
        bad += report(f"mxfp8 codes {i}", host_u8(qs[i]), oq) + report("  bytes", host_u8(es[i]), oe)
        bad += report("  dequant", host_u16(ys[i]), O.mxfp8_dequantize(oq, oe))
    assert bad == 0


def test_split_nvfp4_siblings(lpq, weights):
    """Tensors 2k and 2k+21 share sibling group k (20 groups), so each group spans launches."""
    ws, dw = weights
    n = len(TENSORS)
    group = [(i // 2) if i % 2 == 0 else ((i - 21) // 2) % 20 for i in range(n)]
    members = {}
    for i, gid in enumerate(group):
        members.setdefault(gid, []).append(i)
    ps = [_empty((M, N // 2), torch.uint8) for M, N in TENSORS]
    ss = [_empty((M, N // 16), torch.uint8) for M, N in TENSORS]
    ys = [_empty((M, N), torch.bfloat16) for M, N in TENSORS]
    yq = [_empty((M, N), torch.bfloat16) for M, N in TENSORS]
    amax = _empty(20, torch.float32)
    g = _empty(20, torch.float32)
    tq = lpq.TensorTable([(dw[i], ps[i], ss[i], M, N, group[i]) for i, (M, N) in enumerate(TENSORS)])
    lpq.lpq_nvfp4_amax_grouped(tq, amax)
    lpq.lpq_quantize_nvfp4_grouped(tq, amax, g)
    lpq.lpq_dequantize_nvfp4_grouped(lpq.TensorTable([(ps[i], ys[i], ss[i], M, N, group[i])
                                                      for i, (M, N) in enumerate(TENSORS)]), g)
    lpq.lpq_nvfp4_qdq_grouped(lpq.TensorTable([(dw[i], yq[i], None, M, N, group[i])
                                               for i, (M, N) in enumerate(TENSORS)]), amax)
    bad = 0
    for gid, idx in sorted(members.items()):
        A, og, res = O.nvfp4_quantize_group([ws[i] for i in idx])
        assert same_bits(amax[gid], A) and same_bits(g[gid], og), gid
        for i, (op, os_) in zip(idx, res):
            oy = O.nvfp4_dequantize(op, os_, og)
            bad += report(f"nvfp4 packed {i}", host_u8(ps[i]), op) + report("  scales", host_u8(ss[i]), os_)
            bad += report("  dequant", host_u16(ys[i]), oy) + report("  qdq", host_u16(yq[i]), oy)
    assert bad == 0


@pytest.mark.parametrize("G", [32, 128])
def test_split_int4(lpq, weights, G):
    ws, dw = weights
    ps = [_empty((M, N // 2), torch.uint8) for M, N in TENSORS]
    ss = [_empty((M, N // G), torch.float32) for M, N in TENSORS]
    ys = [_empty((M, N), torch.bfloat16) for M, N in TENSORS]
    lpq.lpq_quantize_int4_grouped(lpq.TensorTable([(dw[i], ps[i], ss[i], M, N, 0) for i, (M, N) in enumerate(TENSORS)]), G)
    lpq.lpq_dequantize_int4_grouped(lpq.TensorTable([(ps[i], ys[i], ss[i], M, N, 0) for i, (M, N) in enumerate(TENSORS)]), G)
    bad = 0
    for i in range(len(TENSORS)):
        op, os_ = O.int4_quantize(ws[i], G)
        bad += report(f"int4/{G} packed {i}", host_u8(ps[i]), op)
        bad += report("  scales", ss[i].cpu().numpy().view(np.uint32), os_.view(np.uint32))
        bad += report("  dequant", host_u16(ys[i]), O.int4_dequantize(op, os_, G))
    assert bad == 0
