"""The grouped calls under HIP graph capture.

One bucket of six tensors goes through every format's grouped calls: block-wise
FP8, MXFP8, NVFP4 (sibling amax, quantize, dequantize, QDQ) and INT4 (group
128). The sequence is captured once with torch.cuda.graph and replayed three
times. Between replays, new weights are copied into the captured input buffers,
and there is other eager work and a synchronisation. Every replay's outputs
are compared bit for bit with the oracle on those weights, and then with an
eager run of the same calls on the same inputs.

The library enqueues only kernels on the caller's stream (no memset, copy,
allocation or synchronisation), so the whole sequence is capturable. The
NVFP4 group amax is cleared by a fill kernel, not a memset."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import host_u8, host_u16, report, same_bits, to_dev_bf16

pytestmark = pytest.mark.gpu

SHAPES = [(256, 384), (64, 384), (384, 256), (128, 128), (300, 1024), (129, 2048)]
GROUPS = [0, 0, 1, 2, 3, 3]   # NVFP4 sibling groups (pairs share a global scale)
NG = 4


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


def weights(seed):
    return [synth.generate(seed, i, M, N, *synth.DIST_MOE) for i, (M, N) in enumerate(SHAPES)]


def test_grouped_calls_in_a_graph(lpq):
    dev = "cuda"
    e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
    w = [e((M, N), torch.bfloat16) for M, N in SHAPES]
    fq = [e((M, N), torch.uint8) for M, N in SHAPES]
    fs = [e(O.fp8blk_scale_shape(M, N), torch.float32) for M, N in SHAPES]
    fy = [e((M, N), torch.bfloat16) for M, N in SHAPES]
    mq = [e((M, N), torch.uint8) for M, N in SHAPES]
    me = [e((M, N // 32), torch.uint8) for M, N in SHAPES]
    my = [e((M, N), torch.bfloat16) for M, N in SHAPES]
    np_ = [e((M, N // 2), torch.uint8) for M, N in SHAPES]
    ns = [e((M, N // 16), torch.uint8) for M, N in SHAPES]
    ny = [e((M, N), torch.bfloat16) for M, N in SHAPES]
    nq = [e((M, N), torch.bfloat16) for M, N in SHAPES]
    ip = [e((M, N // 2), torch.uint8) for M, N in SHAPES]
    iS = [e((M, N // 128), torch.float32) for M, N in SHAPES]
    iy = [e((M, N), torch.bfloat16) for M, N in SHAPES]
    amax, g = e(NG, torch.float32), e(NG, torch.float32)
    T = lpq.TensorTable
    idx = list(enumerate(SHAPES))
    t_fq = T([(w[i], fq[i], fs[i], M, N, 0) for i, (M, N) in idx])
    t_fd = T([(fq[i], fy[i], fs[i], M, N, 0) for i, (M, N) in idx])
    t_mq = T([(w[i], mq[i], me[i], M, N, 0) for i, (M, N) in idx])
    t_md = T([(mq[i], my[i], me[i], M, N, 0) for i, (M, N) in idx])
    t_nq = T([(w[i], np_[i], ns[i], M, N, GROUPS[i]) for i, (M, N) in idx])
    t_nd = T([(np_[i], ny[i], ns[i], M, N, GROUPS[i]) for i, (M, N) in idx])
    t_nqdq = T([(w[i], nq[i], None, M, N, GROUPS[i]) for i, (M, N) in idx])
    t_iq = T([(w[i], ip[i], iS[i], M, N, 0) for i, (M, N) in idx])
    t_id = T([(ip[i], iy[i], iS[i], M, N, 0) for i, (M, N) in idx])

    def run():
        lpq.lpq_quantize_fp8blk_grouped(t_fq)
        lpq.lpq_dequantize_fp8blk_grouped(t_fd)
        lpq.lpq_quantize_mxfp8_grouped(t_mq)
        lpq.lpq_dequantize_mxfp8_grouped(t_md)
        lpq.lpq_nvfp4_amax_grouped(t_nq, amax)
        lpq.lpq_quantize_nvfp4_grouped(t_nq, amax, g)
        lpq.lpq_dequantize_nvfp4_grouped(t_nd, g)
        lpq.lpq_nvfp4_qdq_grouped(t_nqdq, amax)
        lpq.lpq_quantize_int4_grouped(t_iq, 128)
        lpq.lpq_dequantize_int4_grouped(t_id, 128)

    outputs = fq + fs + fy + mq + me + my + np_ + ns + ny + nq + ip + iS + iy + [amax, g]

    def snapshot():   # raw bits (BF16 through an int16 view)
        return [(o.view(torch.int16) if o.dtype == torch.bfloat16 else o).cpu().numpy().copy() for o in outputs]

    # warm up on a side stream, as torch's graph capture expects, then capture
    for i, a in enumerate(weights(160)):
        w[i].copy_(to_dev_bf16(a))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    bad = 0
    for rep in range(3):
        ws = weights(161 + rep)
        for i, a in enumerate(ws):
            w[i].copy_(to_dev_bf16(a))
        for o in outputs:   # stale results would be caught
            o.zero_()
        junk = torch.randn(1 << 20, device=dev).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for i, (M, N) in idx:
            oq, os_ = O.fp8blk_quantize(ws[i])
            bad += report(f"graph {rep} fp8blk codes {i}", host_u8(fq[i]), oq)
            bad += report("  scales", fs[i].cpu().numpy().view(np.uint32), os_.view(np.uint32))
            bad += report("  dequant", host_u16(fy[i]), O.fp8blk_dequantize(oq, os_))
            oq, oe = O.mxfp8_quantize(ws[i])
            bad += report(f"graph {rep} mxfp8 codes {i}", host_u8(mq[i]), oq)
            bad += report("  bytes", host_u8(me[i]), oe)
            bad += report("  dequant", host_u16(my[i]), O.mxfp8_dequantize(oq, oe))
            op, os_ = O.int4_quantize(ws[i], 128)
            bad += report(f"graph {rep} int4 packed {i}", host_u8(ip[i]), op)
            bad += report("  scales", iS[i].cpu().numpy().view(np.uint32), os_.view(np.uint32))
            bad += report("  dequant", host_u16(iy[i]), O.int4_dequantize(op, os_, 128))
        for gid in range(NG):
            members = [i for i in range(len(SHAPES)) if GROUPS[i] == gid]
            A, og, res = O.nvfp4_quantize_group([ws[i] for i in members])
            assert same_bits(amax[gid], A) and same_bits(g[gid], og), (rep, gid)
            for i, (op, os_) in zip(members, res):
                oy = O.nvfp4_dequantize(op, os_, og)
                bad += report(f"graph {rep} nvfp4 packed {i}", host_u8(np_[i]), op)
                bad += report("  scales", host_u8(ns[i]), os_)
                bad += report("  dequant", host_u16(ny[i]), oy)
                bad += report("  qdq", host_u16(nq[i]), oy)
        # the same calls run eagerly on the same inputs give the same bits
        run()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, snapshot())):
            assert np.array_equal(a, b), (rep, k)
        del junk
    assert bad == 0


def test_w4a4_activation_path_in_a_graph(lpq):
    """The W4A4 activation forward, the static min/max observer then the QDQ under
    its amax, captured once and replayed over a sequence of batches: between
    replays a new batch is copied into the captured input, with eager work and a
    synchronisation. After every replay the observer state, the amax and the
    QDQ output must equal the oracle's sequence, bit for bit; the observer's
    batch keys and arrival counter re-arm themselves inside the replay."""
    M, N = 2048, 2048
    x = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    state = lpq.lpq_observer_reset(device="cuda")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lpq.lpq_nvfp4_observe(x, state, "static_minmax", amax=amax)
        lpq.lpq_nvfp4_qdq(x, amax, y)
    lpq.lpq_observer_reset(state)   # capture ran nothing; start the sequence from a reset state
    ost = np.zeros(3, np.float32)
    bad = 0
    for t in range(4):
        sigma = float(np.ldexp(1.0, t - 1)) * (1.0 + 0.3 * t)
        x_np = synth.generate(777, t, M, N, sigma, 0.0, 1e-4, 100.0)
        x.copy_(to_dev_bf16(x_np))
        torch.zeros(1024, device="cuda").sum().item()   # other eager work and a synchronisation
        graph.replay()
        torch.cuda.synchronize()
        a = O.observer_update("static_minmax", ost, x_np)
        bad += int(not same_bits(state[:3], ost))
        bad += int(not same_bits(amax, np.float32(a)))
        bad += report(f"graph W4A4 replay {t}", host_u16(y), O.nvfp4_qdq(x_np, O.nvfp4_global_scale(a)))
        print(f"  replay {t}: amax {a!r}", flush=True)
    assert bad == 0
