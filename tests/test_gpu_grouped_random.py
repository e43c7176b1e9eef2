"""Grouped calls over seeded random tables, bit for bit against the oracle.

Each table holds 1 to 69 tensors drawn from up to five random shapes in random
order, so that runs of equal work-unit counts start and end at random places and
the library splits the call into launches wherever its work map fills up. NVFP4
and FP8 -> NVFP4 tables also get random sibling groups, whose amax the library
fills itself (amax_valid 0). Every grouped entry point takes part: block FP8,
MXFP8 (both exponent rules), NVFP4 quantize / dequantize / QDQ, INT4 with groups
of 32 or 128, and the three fused re-quantizations under FP32 or power-of-two
tile scales. Weights are the synthetic weight distribution at a random scale."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import host_u8, host_u16, report, to_dev_bf16

pytestmark = pytest.mark.gpu

POW2_MASK = np.uint32(0x7F800000)   # exponent field: each tile scale cut to the power of two at or below it


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


def _empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _table(trial):
    rng = np.random.default_rng(20261206 + trial)
    n = int(rng.integers(1, 70))
    pool = [(int(rng.integers(1, 700)), 128 * int(rng.integers(1, 24))) for _ in range(int(rng.integers(1, 6)))]
    shapes = [pool[int(rng.integers(0, len(pool)))] for _ in range(n)]
    sigma = float(10.0 ** rng.uniform(-4, 2))
    ws = [synth.generate(31000, 100 * trial + i, M, N, sigma, 0.5, 0.001, 50.0) for i, (M, N) in enumerate(shapes)]
    ng = int(rng.integers(1, n + 1))
    groups = [int(rng.integers(0, ng)) for _ in range(n)]
    return rng, shapes, ws, ng, groups


def _members(groups, ng):
    return [(k, [i for i, g in enumerate(groups) if g == k]) for k in range(ng)]


@pytest.mark.parametrize("trial", range(2))
def test_random_table_fp8blk_mxfp8(lpq, trial):
    rng, shapes, ws, _, _ = _table(trial)
    dw = [to_dev_bf16(w) for w in ws]
    floor = trial % 2 == 1
    print(f"  trial {trial}: {len(shapes)} tensors, shapes {sorted(set(shapes))}", flush=True)
    fq = [_empty((M, N), torch.uint8) for M, N in shapes]
    fs = [_empty(O.fp8blk_scale_shape(M, N), torch.float32) for M, N in shapes]
    fy = [_empty((M, N), torch.bfloat16) for M, N in shapes]
    mq = [_empty((M, N), torch.uint8) for M, N in shapes]
    me = [_empty((M, N // 32), torch.uint8) for M, N in shapes]
    my = [_empty((M, N), torch.bfloat16) for M, N in shapes]
    T, idx = lpq.TensorTable, list(enumerate(shapes))
    lpq.lpq_quantize_fp8blk_grouped(T([(dw[i], fq[i], fs[i], M, N, 0) for i, (M, N) in idx]))
    lpq.lpq_dequantize_fp8blk_grouped(T([(fq[i], fy[i], fs[i], M, N, 0) for i, (M, N) in idx]))
    mx_q = lpq.lpq_quantize_mxfp8_floor_grouped if floor else lpq.lpq_quantize_mxfp8_grouped
    mx_q(T([(dw[i], mq[i], me[i], M, N, 0) for i, (M, N) in idx]))
    lpq.lpq_dequantize_mxfp8_grouped(T([(mq[i], my[i], me[i], M, N, 0) for i, (M, N) in idx]))
    bad = 0
    for i in range(len(shapes)):
        oq, os_ = O.fp8blk_quantize(ws[i])
        bad += report(f"fp8blk {i}", host_u8(fq[i]), oq) + report("  scales", _bits(fs[i].cpu().numpy()), _bits(os_))
        bad += report("  dequant", host_u16(fy[i]), O.fp8blk_dequantize(oq, os_))
        oq, oe = (O.mxfp8_floor_quantize if floor else O.mxfp8_quantize)(ws[i])
        bad += report(f"mxfp8 {i}", host_u8(mq[i]), oq) + report("  bytes", host_u8(me[i]), oe)
        bad += report("  dequant", host_u16(my[i]), O.mxfp8_dequantize(oq, oe))
    assert bad == 0


@pytest.mark.parametrize("trial", range(2, 4))
def test_random_table_nvfp4(lpq, trial):
    rng, shapes, ws, ng, groups = _table(trial)
    dw = [to_dev_bf16(w) for w in ws]
    print(f"  trial {trial}: {len(shapes)} tensors in {ng} sibling groups", flush=True)
    ps = [_empty((M, N // 2), torch.uint8) for M, N in shapes]
    sb = [_empty((M, N // 16), torch.uint8) for M, N in shapes]
    ys = [_empty((M, N), torch.bfloat16) for M, N in shapes]
    yq = [_empty((M, N), torch.bfloat16) for M, N in shapes]
    amax, g, amax2 = _empty(ng, torch.float32), _empty(ng, torch.float32), _empty(ng, torch.float32)
    T, idx = lpq.TensorTable, list(enumerate(shapes))
    lpq.lpq_quantize_nvfp4_grouped(T([(dw[i], ps[i], sb[i], M, N, groups[i]) for i, (M, N) in idx]), amax, g,
                                   amax_valid=False)
    lpq.lpq_dequantize_nvfp4_grouped(T([(ps[i], ys[i], sb[i], M, N, groups[i]) for i, (M, N) in idx]), g)
    lpq.lpq_nvfp4_qdq_grouped(T([(dw[i], yq[i], None, M, N, groups[i]) for i, (M, N) in idx]), amax2,
                              amax_valid=False)
    ga, gg, ga2 = amax.cpu().numpy(), g.cpu().numpy(), amax2.cpu().numpy()
    bad = 0
    for k, mem in _members(groups, ng):
        if not mem:
            continue
        A, og = O.nvfp4_group_scale([ws[i] for i in mem])
        bad += int(_bits(ga[k]) != _bits(A)) + int(_bits(ga2[k]) != _bits(A)) + int(_bits(gg[k]) != _bits(og))
        for i in mem:
            op, os_ = O.nvfp4_quantize(ws[i], og)
            bad += report(f"nvfp4 {i}", host_u8(ps[i]), op) + report("  block scales", host_u8(sb[i]), os_)
            bad += report("  dequant", host_u16(ys[i]), O.nvfp4_dequantize(op, os_, og))
            bad += report("  qdq", host_u16(yq[i]), O.nvfp4_qdq(ws[i], og))
    assert bad == 0


@pytest.mark.parametrize("trial", range(4, 6))
def test_random_table_int4(lpq, trial):
    rng, shapes, ws, _, _ = _table(trial)
    dw = [to_dev_bf16(w) for w in ws]
    G = 32 if trial % 2 == 0 else 128
    print(f"  trial {trial}: {len(shapes)} tensors, group {G}", flush=True)
    ps = [_empty((M, N // 2), torch.uint8) for M, N in shapes]
    ss = [_empty((M, N // G), torch.float32) for M, N in shapes]
    ys = [_empty((M, N), torch.bfloat16) for M, N in shapes]
    yq = [_empty((M, N), torch.bfloat16) for M, N in shapes]
    T, idx = lpq.TensorTable, list(enumerate(shapes))
    lpq.lpq_quantize_int4_grouped(T([(dw[i], ps[i], ss[i], M, N, 0) for i, (M, N) in idx]), G)
    lpq.lpq_dequantize_int4_grouped(T([(ps[i], ys[i], ss[i], M, N, 0) for i, (M, N) in idx]), G)
    lpq.lpq_int4_qdq_grouped(T([(dw[i], yq[i], None, M, N, 0) for i, (M, N) in idx]), G)
    bad = 0
    for i in range(len(shapes)):
        op, os_ = O.int4_quantize(ws[i], G)
        bad += report(f"int4 {i}", host_u8(ps[i]), op) + report("  scales", _bits(ss[i].cpu().numpy()), _bits(os_))
        bad += report("  dequant", host_u16(ys[i]), O.int4_dequantize(op, os_, G))
        bad += report("  qdq", host_u16(yq[i]), O.int4_qdq(ws[i], G))
    assert bad == 0


@pytest.mark.parametrize("trial,pow2", [(6, False), (7, True)])
def test_random_table_requant(lpq, trial, pow2):
    rng, shapes, ws, ng, groups = _table(trial)
    print(f"  trial {trial}: {len(shapes)} tensors in {ng} sibling groups, power-of-two scales {pow2}", flush=True)
    src = [O.fp8blk_quantize(w) for w in ws]   # the oracle's own block-FP8 copy of each weight
    if pow2:
        src = [(q, (s.view(np.uint32) & POW2_MASK).view(np.float32)) for q, s in src]
    dq = [torch.from_numpy(q).cuda() for q, _ in src]
    ds = [torch.from_numpy(s).cuda() for _, s in src]
    fq = [_empty((M, N), torch.uint8) for M, N in shapes]
    fs = [_empty(O.fp8blk_scale_shape(M, N), torch.float32) for M, N in shapes]
    mq = [_empty((M, N), torch.uint8) for M, N in shapes]
    me = [_empty((M, N // 32), torch.uint8) for M, N in shapes]
    ps = [_empty((M, N // 2), torch.uint8) for M, N in shapes]
    sb = [_empty((M, N // 16), torch.uint8) for M, N in shapes]
    amax, g = _empty(ng, torch.float32), _empty(ng, torch.float32)
    R, idx = lpq.RequantTable, list(enumerate(shapes))
    lpq.lpq_requantize_fp8blk_grouped(R([(dq[i], ds[i], fq[i], fs[i], M, N, 0) for i, (M, N) in idx]))
    lpq.lpq_requantize_fp8blk_mxfp8_grouped(R([(dq[i], ds[i], mq[i], me[i], M, N, 0) for i, (M, N) in idx]))
    lpq.lpq_fp8blk_amax_grouped(R([(dq[i], ds[i], None, None, M, N, groups[i]) for i, (M, N) in idx]), amax)
    lpq.lpq_requantize_fp8blk_nvfp4_grouped(R([(dq[i], ds[i], ps[i], sb[i], M, N, groups[i]) for i, (M, N) in idx]),
                                           amax, g)
    bad = 0
    for i in range(len(shapes)):
        oq, os_ = O.fp8blk_requantize_fp8blk(*src[i])
        bad += report(f"to fp8blk {i}", host_u8(fq[i]), oq) + report("  scales", _bits(fs[i].cpu().numpy()), _bits(os_))
        oq, oe = O.fp8blk_requantize_mxfp8(*src[i])
        bad += report(f"to mxfp8 {i}", host_u8(mq[i]), oq) + report("  bytes", host_u8(me[i]), oe)
    ga, gg = amax.cpu().numpy(), g.cpu().numpy()
    for k, mem in _members(groups, ng):
        if not mem:
            continue
        A, og, res = O.fp8blk_requantize_nvfp4_group([src[i] for i in mem])
        bad += int(_bits(ga[k]) != _bits(A)) + int(_bits(gg[k]) != _bits(og))
        for i, (op, os_) in zip(mem, res):
            bad += report(f"to nvfp4 {i}", host_u8(ps[i]), op) + report("  block scales", host_u8(sb[i]), os_)
    assert bad == 0
