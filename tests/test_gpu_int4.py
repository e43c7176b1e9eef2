"""Group-wise INT4 ("INT4 QAT 训练"): the HIP path against the CPU oracle, bit for
bit -- packed nibbles, FP32 group scales, dequantized BF16 and the fake-quant
(QDQ) output.  Group sizes 32 and 128; single and grouped calls; every finite
BF16 pattern inside a group; extreme magnitudes."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import synth
from tests.gpu_util import brute_blocks, f2bf, host_u8, host_u16, report, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lpq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import precision_weight_quantization_amd as m
    return m


def check_int4(lpq, w_np, G, name=""):
    w = to_dev_bf16(w_np)
    p, s = lpq.lpq_quantize_int4(w, G)
    y = lpq.lpq_dequantize_int4(p, s, G)
    yq = lpq.lpq_int4_qdq(w, G)
    op, os_ = O.int4_quantize(w_np, G)
    oy = O.int4_dequantize(op, os_, G)
    bad = report(f"int4/{G} packed {name}", host_u8(p), op)
    bad += report(f"int4/{G} scales {name}", s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    bad += report(f"int4/{G} dequant {name}", host_u16(y), oy)
    bad += report(f"int4/{G} qdq {name}", host_u16(yq), oy)
    assert bad == 0


@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("M,N", [(1, 128), (3, 256), (131, 384), (128, 128), (300, 2048), (1000, 640), (7, 4224)])
def test_int4_shapes(lpq, G, M, N):
    """MoE-like values: one row up to several 4,096-element chunks, ragged in the chunk."""
    check_int4(lpq, synth.generate(110 + G, 7 * M + N, M, N, *synth.DIST_MOE), G, f"{M}x{N}")


@pytest.mark.parametrize("M,N", [(1, 32), (5, 96), (33, 160)])
def test_int4_shapes_group32_only(lpq, M, N):
    check_int4(lpq, synth.generate(112, 7 * M + N, M, N, *synth.DIST_MOE), 32, f"{M}x{N}")


@pytest.mark.parametrize("G", [32, 128])
def test_int4_extreme_values(lpq, G):
    """Subnormal-scale, huge (near the BF16 maximum) and ordinary magnitudes."""
    rng = np.random.default_rng(17)
    for scale in (1e-39, 1e-38, 1e-30, 1e-12, 1.0, 1e30, 3e38):
        x = np.clip(rng.standard_normal((64, 256)) * scale / 4, -3.38e38, 3.38e38).astype(np.float32)
        w = f2bf(x)
        fin = np.isfinite((w.astype(np.uint32) << 16).view(np.float32))
        check_int4(lpq, np.where(fin, w, 0).astype(np.uint16), G, f"scale {scale}")


@pytest.mark.parametrize("G", [32, 128])
def test_int4_bruteforce(lpq, G):
    """Each row is one group: every finite BF16 pattern alone among zeros, and with
    an anchor of larger magnitude and random fillers."""
    check_int4(lpq, brute_blocks(G, 21 + G), G, "bruteforce")


@pytest.mark.parametrize("G", [32, 128])
def test_int4_grouped(lpq, G):
    """One grouped launch per operation over mixed shapes matches the oracle per tensor."""
    shapes = [(256, 384), (64, 384), (384, 256), (1, 128), (300, 1024), (129, 2048)]
    ws = [synth.generate(120 + G, i, M, N, *synth.DIST_MOE) for i, (M, N) in enumerate(shapes)]
    dw = [to_dev_bf16(w) for w in ws]
    ps = [torch.empty((M, N // 2), dtype=torch.uint8, device="cuda") for M, N in shapes]
    ss = [torch.empty((M, N // G), dtype=torch.float32, device="cuda") for M, N in shapes]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for M, N in shapes]
    yq = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for M, N in shapes]
    lpq.lpq_quantize_int4_grouped(lpq.TensorTable([(dw[i], ps[i], ss[i], M, N, 0) for i, (M, N) in enumerate(shapes)]), G)
    lpq.lpq_dequantize_int4_grouped(lpq.TensorTable([(ps[i], ys[i], ss[i], M, N, 0) for i, (M, N) in enumerate(shapes)]), G)
    lpq.lpq_int4_qdq_grouped(lpq.TensorTable([(dw[i], yq[i], None, M, N, 0) for i, (M, N) in enumerate(shapes)]), G)
    bad = 0
    for i, (M, N) in enumerate(shapes):
        op, os_ = O.int4_quantize(ws[i], G)
        oy = O.int4_dequantize(op, os_, G)
        bad += report(f"grouped int4/{G} packed {M}x{N}", host_u8(ps[i]), op)
        bad += report("  scales", ss[i].cpu().numpy().view(np.uint32), os_.view(np.uint32))
        bad += report("  dequant", host_u16(ys[i]), oy)
        bad += report("  qdq", host_u16(yq[i]), oy)
    assert bad == 0
