"""HIP path vs the CPU oracle, bit for bit (codes, scale bytes/values, BF16 outputs).

All calls go through the C ABI (via the thin Python binding).  Floating-point
outputs are compared as bit patterns: the tolerance is zero (0 ulp) for every
array, QDQ included.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import (bits32, brute_blocks, f2bf, finite_bf16, host_u8, host_u16, mismatches, report,
                            same_bits, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


# --------------------------------------------------------------------------- helpers

def check_fp8blk(lpq, w_np, name=""):
    w = to_dev_bf16(w_np)
    q, s = lpq.lpq_quantize_fp8blk(w)
    y = lpq.lpq_dequantize_fp8blk(q, s)
    oq, os_ = O.fp8blk_quantize(w_np)
    oy = O.fp8blk_dequantize(oq, os_)
    bad = report(f"fp8blk codes {name}", host_u8(q), oq)
    bad += report(f"fp8blk scales {name}", s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    bad += report(f"fp8blk dequant {name}", host_u16(y), oy)
    assert bad == 0


def check_mxfp8(lpq, w_np, name=""):
    w = to_dev_bf16(w_np)
    q, e = lpq.lpq_quantize_mxfp8(w)
    y = lpq.lpq_dequantize_mxfp8(q, e)
    oq, oe = O.mxfp8_quantize(w_np)
    oy = O.mxfp8_dequantize(oq, oe)
    bad = report(f"mxfp8 codes {name}", host_u8(q), oq)
    bad += report(f"mxfp8 scale bytes {name}", host_u8(e), oe)
    bad += report(f"mxfp8 dequant {name}", host_u16(y), oy)
    assert bad == 0


def check_nvfp4(lpq, w_np, name=""):
    w = to_dev_bf16(w_np)
    amax = lpq.lpq_nvfp4_amax(w)
    p, s, g = lpq.lpq_quantize_nvfp4(w, amax)
    y = lpq.lpq_dequantize_nvfp4(p, s, g)
    yq = lpq.lpq_nvfp4_qdq(w, amax)
    A, og, [(op, os_)] = O.nvfp4_quantize_group([w_np])
    oy = O.nvfp4_dequantize(op, os_, og)
    assert same_bits(amax, A), (float(amax.item()), A)
    assert same_bits(g, og)
    # the same call with no amax given: the library computes the tensor's own
    p2, s2, g2 = lpq.lpq_quantize_nvfp4(w)
    assert same_bits(g2, og)
    bad = report(f"nvfp4 packed, amax computed by the call {name}", host_u8(p2), op)
    bad += report(f"nvfp4 block scales, amax computed by the call {name}", host_u8(s2), os_)
    bad += report(f"nvfp4 packed {name}", host_u8(p), op)
    bad += report(f"nvfp4 block scales {name}", host_u8(s), os_)
    bad += report(f"nvfp4 dequant {name}", host_u16(y), oy)
    bad += report(f"nvfp4 qdq {name}", host_u16(yq), O.nvfp4_qdq(w_np, og))
    bad += report(f"nvfp4 qdq vs dequant(quant) {name}", host_u16(yq), host_u16(y))
    # QDQ with no amax given: the library computes it, holding A in y's first word meanwhile
    yq2 = torch.full_like(w, -7.0)
    lpq.lpq_nvfp4_qdq(w, None, yq2)
    bad += report(f"nvfp4 qdq, amax computed by the call {name}", host_u16(yq2), O.nvfp4_qdq(w_np, og))
    assert bad == 0


# --------------------------------------------------------------------------- single-Linear workload

def test_generator_twin(lpq):
    """The GPU twin of the input generator reproduces the host generator bit for bit."""
    from synth import gpu as sg
    for (M, N, dist, st) in ((256, 512, synth.DIST_MOE, 1), (77, 96, synth.DIST_DENSE, 2),
                             (64, 2048, synth.DIST_ACT, 3), (3, 5, synth.DIST_MOE, 4)):
        dev = sg.generate(123, st, M, N, dist)
        assert mismatches(host_u16(dev), synth.generate(123, st, M, N, *dist)) == 0
    assert mismatches(host_u16(sg.single_linear()), synth.single_linear()) == 0


def test_single_linear_all_formats(lpq):
    w = synth.single_linear()
    check_fp8blk(lpq, w, "single-linear")
    check_mxfp8(lpq, w, "single-linear")
    check_nvfp4(lpq, w, "single-linear")


@pytest.mark.parametrize("M,N", [(1, 32), (3, 96), (128, 128), (131, 160), (300, 2048), (1000, 544)])
def test_shapes_mx_nv(lpq, M, N):
    w = synth.generate(77, M * 10007 + N, M, N, *synth.DIST_MOE)
    check_mxfp8(lpq, w, f"{M}x{N}")
    check_nvfp4(lpq, w, f"{M}x{N}")


@pytest.mark.parametrize("M,N", [(1, 16), (5, 48), (7, 80)])
def test_shapes_nv_only(lpq, M, N):
    check_nvfp4(lpq, synth.generate(78, M * 31 + N, M, N, *synth.DIST_MOE), f"{M}x{N}")


@pytest.mark.parametrize("M,N", [(1, 1), (1, 2), (7, 3), (128, 128), (129, 130), (300, 200), (256, 1000),
                                 (200, 264), (640, 384)])
def test_shapes_fp8blk(lpq, M, N):
    check_fp8blk(lpq, synth.generate(79, M * 31 + N, M, N, *synth.DIST_MOE), f"{M}x{N}")


def test_fp8blk_unaligned_pointers(lpq):
    """Rows whose base is not 16-byte aligned take the element-wise path."""
    M, N = 256, 256
    w_np = synth.generate(80, 1, M, N, *synth.DIST_MOE)
    buf = torch.zeros(M * N + 8, dtype=torch.bfloat16, device="cuda")
    buf[1:1 + M * N] = to_dev_bf16(w_np).view(-1)
    w = buf[1:1 + M * N].view(M, N)
    qbuf = torch.zeros(M * N + 8, dtype=torch.uint8, device="cuda")
    q = qbuf[3:3 + M * N].view(M, N)
    s = torch.empty((2, 2), dtype=torch.float32, device="cuda")
    raw = lpq.raw()
    st = raw.lpq_quantize_fp8blk(w.data_ptr(), M, N, q.data_ptr(), s.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    oq, os_ = O.fp8blk_quantize(w_np)
    assert mismatches(host_u8(q), oq) == 0 and mismatches(bits32(s), bits32(os_)) == 0


def test_extreme_values(lpq):
    """Tiny (subnormal-scale), huge (near the BF16 maximum) and mixed-magnitude tensors.
    1e-22 puts the NVFP4 global scale g between 2^-90 and 2^-81: g itself is not
    pre-scaled but block multipliers can be, in full chunks as well as the tail."""
    rng = np.random.default_rng(5)
    for scale in (1e-38, 1e-30, 1e-22, 1e-12, 1.0, 1e30, 3e38):
        x = (rng.standard_normal((64, 256)) * scale / 4).astype(np.float32)
        x = np.clip(x, -3.38e38, 3.38e38)
        w = (((x.view(np.uint32).astype(np.uint64) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16)
             .astype(np.uint16))
        fin = np.isfinite(((w.astype(np.uint32) << 16).view(np.float32)))
        w = np.where(fin, w, 0).astype(np.uint16)
        check_fp8blk(lpq, w, f"scale {scale}")
        check_mxfp8(lpq, w, f"scale {scale}")
        check_nvfp4(lpq, w, f"scale {scale}")


# --------------------------------------------------------------------------- brute force over BF16

def test_bruteforce_mxfp8(lpq):
    w = brute_blocks(32, 1)
    check_mxfp8(lpq, w, "bruteforce")


def test_bruteforce_mxfp8_floor(lpq):
    """The OCP floor exponent rule (saturating) over every finite BF16 pattern, alone and
    beside a larger anchor, and the default rule's dequantizer on its output."""
    w_np = brute_blocks(32, 5)
    w = to_dev_bf16(w_np)
    q, e = lpq.lpq_quantize_mxfp8_floor(w)
    y = lpq.lpq_dequantize_mxfp8(q, e)
    oq, oe = O.mxfp8_floor_quantize(w_np)
    bad = report("mxfp8 floor codes", host_u8(q), oq)
    bad += report("mxfp8 floor bytes", host_u8(e), oe)
    bad += report("mxfp8 floor dequant", host_u16(y), O.mxfp8_dequantize(oq, oe))
    assert bad == 0


@pytest.mark.parametrize("M,N", [(1, 32), (131, 160), (1000, 544)])
def test_mxfp8_floor_shapes_grouped(lpq, M, N):
    w_np = synth.generate(77, M + N, M, N, *synth.DIST_MOE)
    oq, oe = O.mxfp8_floor_quantize(w_np)
    w = to_dev_bf16(w_np)
    q, e = lpq.lpq_quantize_mxfp8_floor(w)
    bad = report(f"mxfp8 floor codes {M}x{N}", host_u8(q), oq) + report("bytes", host_u8(e), oe)
    q2 = torch.empty((M, N), dtype=torch.uint8, device=w.device)
    e2 = torch.empty((M, N // 32), dtype=torch.uint8, device=w.device)
    lpq.lpq_quantize_mxfp8_floor_grouped(lpq.TensorTable([(w, q2, e2, M, N, 0), (w, q2, e2, M, N, 0)]))
    bad += report("grouped codes", host_u8(q2), oq) + report("grouped bytes", host_u8(e2), oe)
    assert bad == 0


@pytest.mark.parametrize("M,N", [(1, 16), (131, 160), (1000, 544)])
def test_nvfp4_e4m3_max_256_single(lpq, M, N):
    w_np = synth.generate(91, M + N, M, N, *synth.DIST_MOE)
    w = to_dev_bf16(w_np)
    amax = lpq.lpq_nvfp4_amax(w)
    p, s, g = lpq.lpq_quantize_nvfp4_ex(w, amax, 256)
    yq = lpq.lpq_nvfp4_qdq_ex(w, amax, 256)
    A, og, [(op, os_)] = O.nvfp4_quantize_group([w_np], 256)
    bad = int(not same_bits(g, og))
    p2, s2, g2 = lpq.lpq_quantize_nvfp4_ex(w, None, 256)     # amax computed by the call
    bad += int(not same_bits(g2, og)) + report("packed, own amax", host_u8(p2), op) + report("scales", host_u8(s2), os_)
    bad += report(f"nvfp4/256 packed {M}x{N}", host_u8(p), op) + report("scales", host_u8(s), os_)
    bad += report("qdq", host_u16(yq), O.nvfp4_qdq(w_np, og))
    bad += report("qdq, own amax", host_u16(lpq.lpq_nvfp4_qdq_ex(w, None, 256)), O.nvfp4_qdq(w_np, og))
    assert int(host_u8(s).max()) <= 0x78   # block-scale codes stay at or below 256 (0x78)
    assert bad == 0


def test_nvfp4_global_scale_reciprocal(lpq):
    """fl(2688 / A) on random, tiny, huge, exact and zero amax values."""
    rng = np.random.default_rng(9)
    bits = rng.integers(0, 0x7F800000, 20000, dtype=np.uint32)
    A = np.concatenate([bits.view(np.float32), np.ldexp(np.float32(2688.0), np.arange(-40, 40)).astype(np.float32),
                        np.array([0.0, 1e-45, 3.4e38], np.float32)]).astype(np.float32)
    out = lpq.lpq_nvfp4_global_scale_reciprocal(torch.from_numpy(A).cuda())
    want = np.array([O.nvfp4_global_scale_reciprocal(a) for a in A], np.float32)
    assert report("reciprocal global scale", out.cpu().numpy().view(np.uint32), want.view(np.uint32)) == 0


@pytest.mark.parametrize("e4m3_max", [448, 256])
def test_bruteforce_nvfp4_grouped(lpq, e4m3_max):
    """Each 1x16 block is its own tensor and its own sibling group (own global scale);
    with E4M3 maximum 448 (the default calls) and 256 (the *_ex calls)."""
    w_np = brute_blocks(16, 2 if e4m3_max == 448 else 6)
    n = w_np.shape[0]
    w = to_dev_bf16(w_np)
    p = torch.empty((n, 8), dtype=torch.uint8, device="cuda")
    s = torch.empty((n, 1), dtype=torch.uint8, device="cuda")
    yq = torch.empty((n, 16), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((n, 16), dtype=torch.bfloat16, device="cuda")
    amax = torch.empty(n, dtype=torch.float32, device="cuda")
    g = torch.empty(n, dtype=torch.float32, device="cuda")
    tq = lpq.TensorTable([(w[i:i + 1], p[i:i + 1], s[i:i + 1], 1, 16, i) for i in range(n)])
    tdq = lpq.TensorTable([(p[i:i + 1], y[i:i + 1], s[i:i + 1], 1, 16, i) for i in range(n)])
    tqdq = lpq.TensorTable([(w[i:i + 1], yq[i:i + 1], None, 1, 16, i) for i in range(n)])
    lpq.lpq_nvfp4_amax_grouped(tq, amax)
    if e4m3_max == 448:
        lpq.lpq_quantize_nvfp4_grouped(tq, amax, g)
        lpq.lpq_nvfp4_qdq_grouped(tqdq, amax)
    else:
        lpq.lpq_quantize_nvfp4_grouped_ex(tq, amax, g, e4m3_max)
        lpq.lpq_nvfp4_qdq_grouped_ex(tqdq, amax, e4m3_max)
    lpq.lpq_dequantize_nvfp4_grouped(tdq, g)
    hp, hs, hy, hyq = host_u8(p), host_u8(s), host_u16(y), host_u16(yq)
    hg = g.cpu().numpy()
    # the same calls with amax_valid False: each call fills the group amax itself
    # (slots start as NaN here: the call must overwrite every one)
    amax2 = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    amax3 = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    g2 = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    lpq.lpq_quantize_nvfp4_grouped_ex(tq, amax2, g2, e4m3_max, amax_valid=False)
    hp2, hs2 = host_u8(p), host_u8(s)
    lpq.lpq_nvfp4_qdq_grouped_ex(tqdq, amax3, e4m3_max, amax_valid=False)
    hyq2 = host_u16(yq)
    op = np.empty_like(hp); os_ = np.empty_like(hs); oy = np.empty_like(hy); og = np.empty(n, np.float32)
    for i in range(n):
        A, og[i], [(a, b)] = O.nvfp4_quantize_group([w_np[i:i + 1]], e4m3_max)
        op[i], os_[i] = a[0], b[0]
    for i in range(n):
        oy[i] = O.nvfp4_dequantize(op[i:i + 1], os_[i:i + 1], float(og[i]))[0]
    bad = report("bruteforce nvfp4 g", hg.view(np.uint32), og.view(np.uint32))
    bad += report("bruteforce nvfp4 packed", hp, op)
    bad += report("bruteforce nvfp4 scales", hs, os_)
    bad += report("bruteforce nvfp4 dequant", hy, oy)
    bad += report("bruteforce nvfp4 qdq", hyq, oy)
    bad += report("bruteforce nvfp4 amax filled by quantize", bits32(amax2), bits32(amax))
    bad += report("bruteforce nvfp4 amax filled by qdq", bits32(amax3), bits32(amax))
    bad += report("bruteforce nvfp4 g, amax filled", bits32(g2), og.view(np.uint32))
    bad += report("bruteforce nvfp4 packed, amax filled", hp2, op)
    bad += report("bruteforce nvfp4 scales, amax filled", hs2, os_)
    bad += report("bruteforce nvfp4 qdq, amax filled", hyq2, oy)
    assert bad == 0


def test_bruteforce_fp8blk_grouped(lpq):
    """Each 1x2 (ragged) tensor is its own tile: p with a zero, and p with an anchor."""
    pats = finite_bf16()
    rng = np.random.default_rng(3)
    n = pats.size
    pf = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.minimum(np.abs(pf) * rng.choice(np.array([1.0, 1.3, 2.0, 448.0, 1e6]), n), 3.3e38)
    w_np = np.zeros((2 * n, 2), np.uint16)
    w_np[:n, 0] = pats
    w_np[n:, 1] = pats
    w_np[n:, 0] = f2bf(a.astype(np.float32))
    N = 2 * n
    w = to_dev_bf16(w_np)
    q = torch.empty((N, 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((N, 1), dtype=torch.float32, device="cuda")
    y = torch.empty((N, 2), dtype=torch.bfloat16, device="cuda")
    tq = lpq.TensorTable([(w[i:i + 1], q[i:i + 1], s[i:i + 1], 1, 2, 0) for i in range(N)])
    tdq = lpq.TensorTable([(q[i:i + 1], y[i:i + 1], s[i:i + 1], 1, 2, 0) for i in range(N)])
    lpq.lpq_quantize_fp8blk_grouped(tq)
    lpq.lpq_dequantize_fp8blk_grouped(tdq)
    oq = np.empty((N, 2), np.uint8); os_ = np.empty((N, 1), np.float32)
    for i in range(N):
        a_, b_ = O.fp8blk_quantize(w_np[i:i + 1])
        oq[i], os_[i] = a_[0], b_[0]
    oy = np.concatenate([O.fp8blk_dequantize(oq[i:i + 1], os_[i:i + 1]) for i in range(N)])
    bad = report("bruteforce fp8blk codes", host_u8(q), oq)
    bad += report("bruteforce fp8blk scales", s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    bad += report("bruteforce fp8blk dequant", host_u16(y), oy)
    assert bad == 0


def test_fp8blk_wide_strips(lpq):
    """Calls with at least 8192 strips of 4 tiles (the library's threshold) take the
    4-tile-per-workgroup quantizer.  Tiles are independent, so bands of whole tiles
    (edge bands included) are checked against the oracle run on the same band."""
    from synth import gpu as sgpu
    bad = 0
    # one ragged tensor: 257 tile rows x 33 strips = 8481 strips
    M, N = 32768 + 37, 16384 + 40
    w = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sgpu.fill(w, 92, 1, synth.DIST_MOE)
    q, s = lpq.lpq_quantize_fp8blk(w)
    for r0, r1, c0, c1 in [(0, 128, 0, N), (12800, 13056, 0, N), (32768, M, 0, N), (0, M, 16384, N)]:
        oq, os_ = O.fp8blk_quantize(host_u16(w[r0:r1, c0:c1]))
        bad += report(f"wide single codes rows {r0}:{r1} cols {c0}:{c1}", host_u8(q[r0:r1, c0:c1]), oq)
        bad += report("  scales", s[r0 // 128:(r1 + 127) // 128, c0 // 128:(c1 + 127) // 128].cpu().numpy().view(np.uint32),
                      os_.view(np.uint32))
    del w, q, s
    # grouped: 4 ragged shapes, 274 outputs each from one source per shape (8220 strips)
    shapes = [(300, 1000), (256, 1536), (129, 2056), (512, 520)]
    copies = 274
    srcs = [to_dev_bf16(synth.generate(93, i, M, N, *synth.DIST_MOE)) for i, (M, N) in enumerate(shapes)]
    qs = [torch.empty((copies, M, N), dtype=torch.uint8, device="cuda") for M, N in shapes]
    ss = [torch.empty((copies, (M + 127) // 128, (N + 127) // 128), dtype=torch.float32, device="cuda") for M, N in shapes]
    lpq.lpq_quantize_fp8blk_grouped(lpq.TensorTable(
        [(srcs[k], qs[k][j], ss[k][j], M, N, 0) for k, (M, N) in enumerate(shapes) for j in range(copies)]))
    for k, (M, N) in enumerate(shapes):
        oq, os_ = O.fp8blk_quantize(host_u16(srcs[k]))
        bad += report(f"wide grouped codes {M}x{N} (x{copies})", host_u8(qs[k]), np.broadcast_to(oq, (copies, M, N)))
        bad += report("  scales", ss[k].cpu().numpy().view(np.uint32),
                      np.broadcast_to(os_.view(np.uint32), (copies,) + os_.shape))
    assert bad == 0


# --------------------------------------------------------------------------- grouped calls

def test_grouped_mixed_shapes_and_siblings(lpq):
    """Several shapes in one launch; q/k/v and gate/up sibling groups share g."""
    shapes = [("q", 256, 320), ("k", 64, 320), ("v", 64, 320), ("o", 320, 256),
              ("gate", 384, 320), ("up", 384, 320), ("down", 320, 384)]
    groups = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
    ws = [synth.generate(90, i, M, N, *synth.DIST_MOE) for i, (_, M, N) in enumerate(shapes)]
    dw = [to_dev_bf16(w) for w in ws]
    # NVFP4
    ps = [torch.empty((M, N // 2), dtype=torch.uint8, device="cuda") for _, M, N in shapes]
    ss = [torch.empty((M, N // 16), dtype=torch.uint8, device="cuda") for _, M, N in shapes]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _, M, N in shapes]
    yq = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _, M, N in shapes]
    tq = lpq.TensorTable([(dw[i], ps[i], ss[i], M, N, groups[nm]) for i, (nm, M, N) in enumerate(shapes)])
    tdq = lpq.TensorTable([(ps[i], ys[i], ss[i], M, N, groups[nm]) for i, (nm, M, N) in enumerate(shapes)])
    tqdq = lpq.TensorTable([(dw[i], yq[i], None, M, N, groups[nm]) for i, (nm, M, N) in enumerate(shapes)])
    amax = torch.empty(4, dtype=torch.float32, device="cuda")
    g = torch.empty(4, dtype=torch.float32, device="cuda")
    lpq.lpq_nvfp4_amax_grouped(tq, amax)
    lpq.lpq_quantize_nvfp4_grouped(tq, amax, g)
    lpq.lpq_dequantize_nvfp4_grouped(tdq, g)
    lpq.lpq_nvfp4_qdq_grouped(tqdq, amax)
    bad = 0
    # amax_valid False: quantize and QDQ fill their group amax themselves (from NaN)
    ps2 = [torch.empty_like(t) for t in ps]
    ss2 = [torch.empty_like(t) for t in ss]
    yq2 = [torch.empty_like(t) for t in yq]
    amax2 = torch.full((4,), float("nan"), dtype=torch.float32, device="cuda")
    amax3 = torch.full((4,), float("nan"), dtype=torch.float32, device="cuda")
    g2 = torch.full((4,), float("nan"), dtype=torch.float32, device="cuda")
    lpq.lpq_quantize_nvfp4_grouped(lpq.TensorTable([(dw[i], ps2[i], ss2[i], M, N, groups[nm])
                                                    for i, (nm, M, N) in enumerate(shapes)]), amax2, g2,
                                   amax_valid=False)
    lpq.lpq_nvfp4_qdq_grouped(lpq.TensorTable([(dw[i], yq2[i], None, M, N, groups[nm])
                                               for i, (nm, M, N) in enumerate(shapes)]), amax3, amax_valid=False)
    bad += mismatches(bits32(amax2), bits32(amax)) + mismatches(bits32(amax3), bits32(amax))
    bad += mismatches(bits32(g2), bits32(g))
    for i in range(len(shapes)):
        bad += mismatches(host_u8(ps2[i]), host_u8(ps[i])) + mismatches(host_u8(ss2[i]), host_u8(ss[i]))
        bad += mismatches(host_u16(yq2[i]), host_u16(yq[i]))
    for gid in range(4):
        members = [i for i, (nm, _, _) in enumerate(shapes) if groups[nm] == gid]
        A, og, outs = O.nvfp4_quantize_group([ws[i] for i in members])
        assert same_bits(amax[gid], A) and same_bits(g[gid], og)
        for i, (op, os_) in zip(members, outs):
            bad += mismatches(host_u8(ps[i]), op) + mismatches(host_u8(ss[i]), os_)
            oy = O.nvfp4_dequantize(op, os_, og)
            bad += mismatches(host_u16(ys[i]), oy) + mismatches(host_u16(yq[i]), oy)
    # MXFP8 and block-wise FP8 over the same set
    qs = [torch.empty((M, N), dtype=torch.uint8, device="cuda") for _, M, N in shapes]
    es = [torch.empty((M, N // 32), dtype=torch.uint8, device="cuda") for _, M, N in shapes]
    lpq.lpq_quantize_mxfp8_grouped(lpq.TensorTable([(dw[i], qs[i], es[i], M, N, 0) for i, (_, M, N) in enumerate(shapes)]))
    lpq.lpq_dequantize_mxfp8_grouped(lpq.TensorTable([(qs[i], ys[i], es[i], M, N, 0) for i, (_, M, N) in enumerate(shapes)]))
    for i in range(len(shapes)):
        oq, oe = O.mxfp8_quantize(ws[i])
        bad += mismatches(host_u8(qs[i]), oq) + mismatches(host_u8(es[i]), oe)
        bad += mismatches(host_u16(ys[i]), O.mxfp8_dequantize(oq, oe))
    sc = [torch.empty(((M + 127) // 128, (N + 127) // 128), dtype=torch.float32, device="cuda") for _, M, N in shapes]
    lpq.lpq_quantize_fp8blk_grouped(lpq.TensorTable([(dw[i], qs[i], sc[i], M, N, 0) for i, (_, M, N) in enumerate(shapes)]))
    lpq.lpq_dequantize_fp8blk_grouped(lpq.TensorTable([(qs[i], ys[i], sc[i], M, N, 0) for i, (_, M, N) in enumerate(shapes)]))
    for i in range(len(shapes)):
        oq, os_ = O.fp8blk_quantize(ws[i])
        bad += mismatches(host_u8(qs[i]), oq) + mismatches(bits32(sc[i]), bits32(os_))
        bad += mismatches(host_u16(ys[i]), O.fp8blk_dequantize(oq, os_))
    assert bad == 0


def test_determinism(lpq):
    w = to_dev_bf16(synth.generate(91, 1, 512, 1024, *synth.DIST_MOE))
    a1 = lpq.lpq_nvfp4_amax(w)
    r1 = [host_u8(x) for x in lpq.lpq_quantize_nvfp4(w, a1)[:2]] + [host_u8(x) for x in lpq.lpq_quantize_mxfp8(w)]
    a2 = lpq.lpq_nvfp4_amax(w)
    r2 = [host_u8(x) for x in lpq.lpq_quantize_nvfp4(w, a2)[:2]] + [host_u8(x) for x in lpq.lpq_quantize_mxfp8(w)]
    assert all(np.array_equal(x, y) for x, y in zip(r1, r2))


def test_amax_accumulate(lpq):
    a = to_dev_bf16(synth.generate(92, 1, 64, 64, *synth.DIST_MOE))
    b = to_dev_bf16(synth.generate(92, 2, 64, 64, 1.0, 0.0, 0.0, 1.0))
    m = lpq.lpq_nvfp4_amax(a)
    lpq.lpq_nvfp4_amax(b, m, accumulate=True)
    want = max(O.amax(host_u16(a)), O.amax(host_u16(b)))
    assert same_bits(m, want)


def test_binding_refuses_undersized_and_host_tensors(lpq):
    """The Python binding checks every tensor before its address reaches a kernel."""
    w = to_dev_bf16(synth.generate(94, 1, 64, 256, *synth.DIST_MOE))
    with pytest.raises(ValueError):
        lpq.lpq_quantize_mxfp8(w, q=torch.empty((64, 255), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        lpq.lpq_quantize_nvfp4(w, amax=torch.zeros(1))                       # host amax
    with pytest.raises(ValueError):
        lpq.lpq_dequantize_nvfp4(torch.empty((64, 128), dtype=torch.uint8, device="cuda"),
                                 torch.empty((64, 15), dtype=torch.uint8, device="cuda"), torch.ones(1, device="cuda"))
    with pytest.raises(ValueError):
        lpq.lpq_nvfp4_qdq(w, lpq.lpq_nvfp4_amax(w), y=torch.empty((64, 256), dtype=torch.bfloat16,
                                                                  device="cuda").t().contiguous().t())
    short = torch.empty((64, 100), dtype=torch.uint8, device="cuda")
    t = lpq.TensorTable([(w, short, short, 64, 256, 0)])
    with pytest.raises(ValueError):
        lpq.lpq_quantize_mxfp8_grouped(t)
    torch.cuda.synchronize()
