"""Calls on two streams at once share nothing, from one host thread or two.

The library keeps no state of its own between or during calls (the observer
state and the NVFP4 amax slots are the caller's), so independent calls may run
concurrently on different streams. Two default-priority streams each run a
sequence of grouped calls (MXFP8 quantize, the NVFP4 group amax and quantize,
block-FP8 quantize and dequantize) and a W4A4 observer + QDQ on their own
buffers, their launches interleaved from the host; afterwards every output of
both streams is compared with the oracle, bit for bit."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import host_u8, host_u16, report, same_bits, to_dev_bf16

pytestmark = pytest.mark.gpu

SHAPES = [(768, 2048), (2048, 768), (512, 2048), (300, 1024)]
GROUPS = [0, 0, 1, 2]


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


class Lane:
    """One stream's buffers and calls."""

    def __init__(self, lpq, seed):
        self.lpq = lpq
        self.stream = torch.cuda.Stream()
        self.w_np = [synth.generate(seed, i, M, N, *synth.DIST_MOE) for i, (M, N) in enumerate(SHAPES)]
        self.x_np = synth.generate(seed, 99, 1024, 2048, *synth.DIST_ACT)
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
        self.w = [to_dev_bf16(w) for w in self.w_np]
        self.x = to_dev_bf16(self.x_np)
        self.mq = [e((M, N), torch.uint8) for M, N in SHAPES]
        self.me = [e((M, N // 32), torch.uint8) for M, N in SHAPES]
        self.np_ = [e((M, N // 2), torch.uint8) for M, N in SHAPES]
        self.ns = [e((M, N // 16), torch.uint8) for M, N in SHAPES]
        self.fq = [e((M, N), torch.uint8) for M, N in SHAPES]
        self.fs = [e(O.fp8blk_scale_shape(M, N), torch.float32) for M, N in SHAPES]
        self.fy = [e((M, N), torch.bfloat16) for M, N in SHAPES]
        self.amax = e(3, torch.float32)
        self.g = e(3, torch.float32)
        self.y = torch.empty_like(self.x)
        self.xa = e(1, torch.float32)
        T = lpq.TensorTable
        idx = list(enumerate(SHAPES))
        self.t_mx = T([(self.w[i], self.mq[i], self.me[i], M, N, 0) for i, (M, N) in idx])
        self.t_nv = T([(self.w[i], self.np_[i], self.ns[i], M, N, GROUPS[i]) for i, (M, N) in idx])
        self.t_fq = T([(self.w[i], self.fq[i], self.fs[i], M, N, 0) for i, (M, N) in idx])
        self.t_fd = T([(self.fq[i], self.fy[i], self.fs[i], M, N, 0) for i, (M, N) in idx])
        self.state = lpq.lpq_observer_reset(device="cuda")
        torch.cuda.synchronize()

    def steps(self):
        L, s = self.lpq, self.stream
        return [lambda: L.lpq_quantize_mxfp8_grouped(self.t_mx, stream=s),
                lambda: L.lpq_nvfp4_amax_grouped(self.t_nv, self.amax, stream=s),
                lambda: L.lpq_quantize_nvfp4_grouped(self.t_nv, self.amax, self.g, stream=s),
                lambda: L.lpq_quantize_fp8blk_grouped(self.t_fq, stream=s),
                lambda: L.lpq_dequantize_fp8blk_grouped(self.t_fd, stream=s),
                lambda: L.lpq_nvfp4_observe(self.x, self.state, "static_minmax", amax=self.xa, stream=s),
                lambda: L.lpq_nvfp4_qdq(self.x, self.xa, self.y, stream=s)]

    def check(self, tag):
        bad = 0
        for i, w in enumerate(self.w_np):
            q, e = O.mxfp8_quantize(w)
            bad += report(f"{tag} mxfp8 {i}", host_u8(self.mq[i]), q) + report(f"{tag} mxfp8 e {i}", host_u8(self.me[i]), e)
            q, sc = O.fp8blk_quantize(w)
            bad += report(f"{tag} fp8blk {i}", host_u8(self.fq[i]), q) + int(not same_bits(self.fs[i], sc))
            bad += report(f"{tag} fp8blk y {i}", host_u16(self.fy[i]), O.fp8blk_dequantize(q, sc))
        for gid in range(3):
            members = [i for i in range(len(SHAPES)) if GROUPS[i] == gid]
            A, g, res = O.nvfp4_quantize_group([self.w_np[i] for i in members])
            bad += int(not same_bits(self.amax[gid], np.float32(A))) + int(not same_bits(self.g[gid], np.float32(g)))
            for i, (p, sb) in zip(members, res):
                bad += report(f"{tag} nvfp4 {i}", host_u8(self.np_[i]), p) + report(f"{tag} nvfp4 s {i}", host_u8(self.ns[i]), sb)
        ost = np.zeros(3, np.float32)
        a = O.observer_update("static_minmax", ost, self.x_np)
        bad += int(not same_bits(self.state[:3], ost)) + int(not same_bits(self.xa, np.float32(a)))
        bad += report(f"{tag} W4A4 qdq", host_u16(self.y), O.nvfp4_qdq(self.x_np, O.nvfp4_global_scale(a)))
        return bad


def test_two_streams_interleaved(lpq):
    a, b = Lane(lpq, 501), Lane(lpq, 502)
    for fa, fb in zip(a.steps(), b.steps()):
        fa()
        fb()
    torch.cuda.synchronize()
    assert a.check("stream A") + b.check("stream B") == 0


def test_two_host_threads(lpq):
    """The same calls driven from two host threads at once (the binding releases the
    interpreter lock inside each C call), each thread on its own stream and buffers,
    each repeating its weight calls five times before its observer + QDQ: both
    threads' outputs must still equal the oracle's, bit for bit."""
    import threading
    a, b = Lane(lpq, 503), Lane(lpq, 504)
    errors = []

    def drive(lane):
        try:
            steps = lane.steps()
            for _ in range(5):
                for f in steps[:5]:   # the weight calls
                    f()
            for f in steps[5:]:       # observer, then QDQ under its amax
                f()
            lane.stream.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=drive, args=(lane,)) for lane in (a, b)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    torch.cuda.synchronize()
    assert not errors, errors
    assert a.check("thread A") + b.check("thread B") == 0
