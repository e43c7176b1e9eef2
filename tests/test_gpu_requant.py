"""Re-quantization of block-wise FP8 weights (FP8 codes + FP32 tile scales) into
block-wise FP8, MXFP8 and NVFP4, HIP path vs the CPU oracle, bit for bit.

The oracle is the unfused composition: block-FP8 dequantization to BF16, then
the target format's quantizer.  All calls go through the C ABI; the tolerance is
zero for codes, scale bytes, the group amax and the global scale.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import DEV, host_u8, host_u16, report, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def f32_bits(t) -> np.ndarray:
    return np.asarray(t, np.float32).view(np.uint32)


def check_fp8(lpq, q_np, s_np, name, q_dev=None, out=None):
    q = dev_u8(q_np) if q_dev is None else q_dev
    qo, so = lpq.lpq_requantize_fp8blk(q, dev_f32(s_np), *(out or (None, None)))
    oq, os_ = O.fp8blk_requantize_fp8blk(q_np, s_np)
    bad = report(f"requant fp8blk codes {name}", host_u8(qo), oq)
    bad += report(f"requant fp8blk scales {name}", f32_bits(so.cpu().numpy()), f32_bits(os_))
    return bad


def check_mx(lpq, q_np, s_np, name):
    qo, eo = lpq.lpq_requantize_fp8blk_mxfp8(dev_u8(q_np), dev_f32(s_np))
    oq, oe = O.fp8blk_requantize_mxfp8(q_np, s_np)
    bad = report(f"requant mxfp8 codes {name}", host_u8(qo), oq)
    bad += report(f"requant mxfp8 bytes {name}", host_u8(eo), oe)
    return bad


def check_nv(lpq, q_np, s_np, name):
    q, s = dev_u8(q_np), dev_f32(s_np)
    amax = lpq.lpq_fp8blk_amax(q, s)
    p, sb, g = lpq.lpq_requantize_fp8blk_nvfp4(q, s, amax)
    A, og, [(op, os_)] = O.fp8blk_requantize_nvfp4_group([(q_np, s_np)])
    bad = int(f32_bits(amax.item()) != f32_bits(A)) + int(f32_bits(g.item()) != f32_bits(og))
    print(f"  requant nvfp4 amax {name}: gpu {amax.item()!r} oracle {A!r}", flush=True)
    bad += report(f"requant nvfp4 packed {name}", host_u8(p), op)
    bad += report(f"requant nvfp4 block scales {name}", host_u8(sb), os_)
    return bad


def random_case(M, N, seed, lo=-20, hi=10, signed=False, zero_tile=True):
    q = synth.e4m3_codes(seed, 1, M, N)
    s = synth.random_f32(seed, 2, O.fp8blk_scale_shape(M, N), lo, hi, signed)
    if zero_tile:
        s[-1, 0] = 0.0
    return q, s


def pow2_scales(shape, seed, ks, signs=(1.0,)):
    """Tile scales +-2^k, k drawn from ``ks`` and the sign from ``signs`` by seeded bytes
    (the block scales a trainer without FP32 block scales writes)."""
    n = int(np.prod(shape))
    kb = synth.random_bytes(seed, 3, n).astype(np.int64)
    sb = synth.random_bytes(seed, 4, n).astype(np.int64)
    k = np.asarray(ks, np.int64)[kb % len(ks)]
    sg = np.asarray(signs, np.float64)[sb % len(signs)]
    return (sg * np.ldexp(1.0, k)).astype(np.float32).reshape(shape)


SHAPES = [(1, 32), (3, 64), (200, 320), (130, 2080), (257, 96), (40, 4128), (2, 16416), (1000, 7168)]


@pytest.mark.parametrize("M,N", [(1, 1), (7, 3), (130, 200), (128, 128), (257, 1000), (1000, 544), (256, 2048),
                                 (129, 4100)])
def test_requant_fp8blk_random(lpq, M, N):
    q, s = random_case(M, N, 700 + M + N)
    assert check_fp8(lpq, q, s, f"{M}x{N}") == 0


def test_requant_fp8blk_unaligned(lpq):
    """Code arrays that are not 16-byte aligned, in and out (the per-byte path)."""
    M, N = 256, 384
    q, s = random_case(M, N, 77)
    buf = torch.zeros(M * N + 64, dtype=torch.uint8, device=DEV)
    qin = buf[3:3 + M * N].view(M, N)
    qin.copy_(dev_u8(q))
    obuf = torch.zeros(M * N + 64, dtype=torch.uint8, device=DEV)
    qout = obuf[5:5 + M * N].view(M, N)
    sout = torch.empty(O.fp8blk_scale_shape(M, N), dtype=torch.float32, device=DEV)
    assert check_fp8(lpq, q, s, "unaligned", q_dev=qin, out=(qout, sout)) == 0


@pytest.mark.parametrize("M,N", SHAPES)
def test_requant_mxfp8_random(lpq, M, N):
    q, s = random_case(M, N, 100 + M + N)
    assert check_mx(lpq, q, s, f"{M}x{N}") == 0


@pytest.mark.parametrize("M,N", SHAPES + [(64, 16), (7, 48), (129, 2064)])
def test_requant_nvfp4_random(lpq, M, N):
    q, s = random_case(M, N, 200 + M + N)
    assert check_nv(lpq, q, s, f"{M}x{N}") == 0


@pytest.mark.parametrize("lo,hi,signed", [(-126, -100, False), (100, 118, False), (-126, 118, True),
                                          (-30, 30, True), (-84, -80, False)])
def test_requant_scale_extremes(lpq, lo, hi, signed):
    """Tile scales from the bottom of the normal range (dequantized values in BF16's
    subnormal range or flushed to zero by rounding) to the top (values near BF16's
    largest finite), and negative scales.  [-84, -80] puts the NVFP4 global scale
    between 2^-90 and 2^-81 (some block multipliers pre-scaled, g not)."""
    M, N = 300, 544
    q, s = random_case(M, N, 300 + lo + hi, lo, hi, signed)
    bad = check_mx(lpq, q, s, f"[{lo},{hi}] signed={signed}")
    bad += check_nv(lpq, q, s, f"[{lo},{hi}] signed={signed}")
    bad += check_fp8(lpq, q, s, f"[{lo},{hi}] signed={signed}")
    assert bad == 0


def test_requant_zero_and_sign(lpq):
    """Zero codes of both signs, zero tile scales over nonzero codes, and all-zero blocks."""
    M, N = 256, 384
    q = synth.e4m3_codes(7, 3, M, N)
    q[:, :64] = np.where(np.arange(64) % 2 == 0, 0x00, 0x80)[None, :]
    q[128:, 128:256] = 0x80
    s = synth.random_f32(7, 4, O.fp8blk_scale_shape(M, N), -8, 8)
    s[0, 1] = 0.0
    s[1, 2] = -0.0
    bad = check_mx(lpq, q, s, "zeros")
    bad += check_nv(lpq, q, s, "zeros")
    bad += check_fp8(lpq, q, s, "zeros")
    assert bad == 0


def test_requant_quantized_weights(lpq):
    """Realistic FP8 weights: the MoE-distributed synthetic weight of a gate projection
    quantized block-wise by the oracle, then re-quantized."""
    w = synth.generate(synth.seed_of(3), synth.stream_of(0, 5, 0), 768, 2048, *synth.DIST_MOE)
    q, s = O.fp8blk_quantize(w)
    bad = check_mx(lpq, q, s, "gate 768x2048")
    bad += check_nv(lpq, q, s, "gate 768x2048")
    bad += check_fp8(lpq, q, s, "gate 768x2048")
    assert bad == 0


def test_requant_matches_unfused_kernels(lpq):
    """The fused path equals this library's own dequantize-then-quantize kernels."""
    M, N = 384, 1024
    q_np, s_np = random_case(M, N, 41)
    q, s = dev_u8(q_np), dev_f32(s_np)
    y = lpq.lpq_dequantize_fp8blk(q.view(torch.float8_e4m3fn), s)
    mq, me = lpq.lpq_quantize_mxfp8(y)
    fq, fe = lpq.lpq_requantize_fp8blk_mxfp8(q, s)
    bad = report("fused vs unfused mxfp8 codes", host_u8(fq), host_u8(mq))
    bad += report("fused vs unfused mxfp8 bytes", host_u8(fe), host_u8(me))
    a1 = lpq.lpq_nvfp4_amax(y)
    a2 = lpq.lpq_fp8blk_amax(q, s)
    bad += int(not same_bits(a1, a2))
    p1, s1, g1 = lpq.lpq_quantize_nvfp4(y, a1)
    p2, s2, g2 = lpq.lpq_requantize_fp8blk_nvfp4(q, s, a2)
    bad += report("fused vs unfused nvfp4 packed", host_u8(p2), host_u8(p1))
    bad += report("fused vs unfused nvfp4 scales", host_u8(s2), host_u8(s1))
    bq, bs = lpq.lpq_quantize_fp8blk(y)
    fq8, fs8 = lpq.lpq_requantize_fp8blk(q, s)
    bad += report("fused vs unfused fp8blk codes", host_u8(fq8), host_u8(bq))
    bad += report("fused vs unfused fp8blk scales", f32_bits(fs8.cpu().numpy()), f32_bits(bs.cpu().numpy()))
    assert bad == 0


def test_requant_grouped(lpq):
    """Grouped calls over tensors of many shapes (more distinct sizes than one launch
    holds, so the call is split), NVFP4 sibling groups spanning shapes, and the
    amax pre-pass in overwrite and accumulate modes."""
    shapes = [(64, 96), (128, 256), (40, 2080), (3, 32), (129, 160), (256, 64), (17, 4128), (64, 96),
              (300, 544), (1, 32), (96, 352), (128, 256)]
    groups = [0, 0, 1, 2, 2, 2, 3, 4, 5, 5, 6, 7]
    n_groups = max(groups) + 1
    src = [random_case(M, N, 500 + i, zero_tile=(i % 3 == 0)) for i, (M, N) in enumerate(shapes)]
    qd = [dev_u8(q) for q, _ in src]
    sd = [dev_f32(s) for _, s in src]

    # block-wise FP8 (ragged shapes added: any N)
    fshapes = shapes + [(5, 7), (130, 333)]
    fsrc = src + [random_case(M, N, 900 + i) for i, (M, N) in enumerate(fshapes[len(shapes):])]
    fq = [torch.empty((M, N), dtype=torch.uint8, device=DEV) for M, N in fshapes]
    fs = [torch.empty(O.fp8blk_scale_shape(M, N), dtype=torch.float32, device=DEV) for M, N in fshapes]
    t = lpq.RequantTable([(dev_u8(q), dev_f32(s), fq[i], fs[i], M, N, 0)
                          for i, ((q, s), (M, N)) in enumerate(zip(fsrc, fshapes))])
    lpq.lpq_requantize_fp8blk_grouped(t)
    bad = 0
    for i, (q, s) in enumerate(fsrc):
        oq, os_ = O.fp8blk_requantize_fp8blk(q, s)
        bad += report(f"grouped fp8blk codes #{i}", host_u8(fq[i]), oq)
        bad += report(f"grouped fp8blk scales #{i}", f32_bits(fs[i].cpu().numpy()), f32_bits(os_))

    # MXFP8
    mq = [torch.empty((M, N), dtype=torch.uint8, device=DEV) for M, N in shapes]
    me = [torch.empty((M, N // 32), dtype=torch.uint8, device=DEV) for M, N in shapes]
    t = lpq.RequantTable([(qd[i], sd[i], mq[i], me[i], M, N, 0) for i, (M, N) in enumerate(shapes)])
    lpq.lpq_requantize_fp8blk_mxfp8_grouped(t)
    for i, (q, s) in enumerate(src):
        oq, oe = O.fp8blk_requantize_mxfp8(q, s)
        bad += report(f"grouped mxfp8 codes #{i}", host_u8(mq[i]), oq)
        bad += report(f"grouped mxfp8 bytes #{i}", host_u8(me[i]), oe)

    # NVFP4 amax + quantize
    p = [torch.empty((M, N // 2), dtype=torch.uint8, device=DEV) for M, N in shapes]
    sb = [torch.empty((M, N // 16), dtype=torch.uint8, device=DEV) for M, N in shapes]
    t = lpq.RequantTable([(qd[i], sd[i], p[i], sb[i], M, N, groups[i]) for i, (M, N) in enumerate(shapes)])
    amax = torch.full((n_groups,), 1e30, dtype=torch.float32, device=DEV)
    lpq.lpq_fp8blk_amax_grouped(t, amax, accumulate=False)
    g = torch.zeros(n_groups, dtype=torch.float32, device=DEV)
    lpq.lpq_requantize_fp8blk_nvfp4_grouped(t, amax, g)
    amax_h, g_h = amax.cpu().numpy(), g.cpu().numpy()
    for gid in range(n_groups):
        idx = [i for i in range(len(shapes)) if groups[i] == gid]
        A, og, outs = O.fp8blk_requantize_nvfp4_group([src[i] for i in idx])
        bad += int(f32_bits(amax_h[gid]) != f32_bits(A)) + int(f32_bits(g_h[gid]) != f32_bits(og))
        for i, (op, os_) in zip(idx, outs):
            bad += report(f"grouped nvfp4 packed #{i} (group {gid})", host_u8(p[i]), op)
            bad += report(f"grouped nvfp4 scales #{i} (group {gid})", host_u8(sb[i]), os_)
    # accumulate: a second pass over the same tensors leaves the maxima unchanged,
    # and a larger preset value survives
    amax2 = amax.clone()
    amax2[0] = 3.0e38
    lpq.lpq_fp8blk_amax_grouped(t, amax2, accumulate=True)
    a2 = amax2.cpu().numpy()
    bad += int(a2[0] != np.float32(3.0e38)) + int(not np.array_equal(a2[1:], amax_h[1:]))
    assert bad == 0


# Power-of-two tile scales: every wave whose lanes all hold a scale 2^k with
# -121 <= k <= 119 forms the dequantized values with the scaled convert (exact
# there), the rest through multiply and BF16 rounding.  Both must give the same
# bits, at the range's edges too.

@pytest.mark.parametrize("M,N", [(1, 32), (200, 320), (130, 2080), (40, 4128), (1000, 7168)])
def test_requant_pow2_scales(lpq, M, N):
    q = synth.e4m3_codes(900 + M, 1, M, N)
    s = pow2_scales(O.fp8blk_scale_shape(M, N), 900 + N, list(range(-121, 120)))
    bad = check_mx(lpq, q, s, f"pow2 {M}x{N}") + check_nv(lpq, q, s, f"pow2 {M}x{N}")
    bad += check_fp8(lpq, q, s, f"pow2 {M}x{N}")
    assert bad == 0


@pytest.mark.parametrize("ks,signs", [
    ([-123, -122, -121, -120], (1.0,)),          # the bottom edge: 2^-122 and below take the general path
    ([118, 119, 120, 121, 126], (1.0,)),         # the top edge: 2^120 and above take it
    ([-121, -60, 0, 60, 119], (1.0, -1.0)),      # negative powers of two take it as well
])
def test_requant_pow2_scale_edges(lpq, ks, signs):
    M, N = 384, 2048
    q = synth.e4m3_codes(950, 1, M, N)
    if max(ks) > 119:   # codes below 2 in magnitude keep every dequantized value finite (the contract)
        q = q & np.uint8(0xB7)
    s = pow2_scales(O.fp8blk_scale_shape(M, N), 951 + ks[0], ks, signs)
    name = f"pow2 k in {ks} signs {signs}"
    bad = check_mx(lpq, q, s, name) + check_nv(lpq, q, s, name) + check_fp8(lpq, q, s, name)
    assert bad == 0


def test_requant_pow2_mixed_waves(lpq):
    """Half the tiles with power-of-two scales and half without, so that waves
    straddle the two (they take the general path), on a trainer's real block-FP8
    weight whose scales were rounded to powers of two in alternate tiles."""
    M, N = 512, 2048
    w = synth.generate(960, 1, M, N, *synth.DIST_MOE)
    q, s = O.fp8blk_quantize(w)
    s2 = s.copy()
    s2[:, ::2] = np.ldexp(1.0, np.round(np.log2(s[:, ::2])).astype(np.int64)).astype(np.float32)
    bad = check_mx(lpq, q, s2, "mixed pow2") + check_nv(lpq, q, s2, "mixed pow2") + check_fp8(lpq, q, s2, "mixed pow2")
    s3 = np.ldexp(1.0, np.round(np.log2(s)).astype(np.int64)).astype(np.float32)
    bad += check_mx(lpq, q, s3, "all pow2") + check_nv(lpq, q, s3, "all pow2") + check_fp8(lpq, q, s3, "all pow2")
    assert bad == 0
