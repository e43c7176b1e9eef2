"""Full-size synthetic workloads of the weight codecs, shared by bench.py and the
full-size GPU parity test.

Shapes follow the model families the pages train and serve ("Low Precision
RL": Qwen3-4B, Qwen3-30B-A3B, DeepSeek-V3; "verl NVFP4 QAT" 2.4: q/k/v and
gate/up sibling groups).  No checkpoints are available, so every weight is
drawn by the seeded generator (``synth``), on the device, with the
distributions named for each workload.

  dense   Qwen3-4B: 36 layers x {q 4096x2560, k 1024x2560, v 1024x2560,
          o 2560x4096, gate 9728x2560, up 9728x2560, down 2560x9728}
          -> block-wise FP8 quantize + dequantize
  moe     Qwen3-30B-A3B experts: 48 layers x 128 experts x {gate 768x2048,
          up 768x2048, down 2048x768} -> MXFP8 quantize + dequantize
  nvfp4   the same experts plus 48 x {q 4096x2048, k 512x2048, v 512x2048};
          sibling groups {gate_e, up_e}, {down_e}, {q, k, v} (12,336 groups)
          -> NVFP4 amax, quantize, dequantize and weight QDQ; plus W4A4
          activation QDQ on 8192x2048 tokens
  dsv3    DeepSeek-V3 MoE layer: 256 experts x {gate 2048x7168, up 2048x7168,
          down 7168x2048} -> block-wise FP8 quantize + dequantize
  fp8train  the nvfp4 workload's weights held in block-wise FP8 (as an FP8
          trainer keeps them; made once by this library's quantizer) ->
          fused re-quantization into block-wise FP8 (all tensors), MXFP8
          (experts) and NVFP4 (experts and q/k/v, sibling groups as above),
          each next to the unfused dequantize-then-quantize sequence on the
          same data; and the same fused re-quantizations with every tile scale
          rounded to a power of two (the block scales a trainer writes unless
          FP32 block scales are asked for, "Low Precision RL" 2).  Timed apart
          from the step.
  int4    the moe workload's experts -> group-wise INT4 (group 128, the size
          "INT4 QAT 训练" gives for Qwen3-30B-A3B) quantize, dequantize and
          fake-quant.  Timed apart from the step.

Buckets: one grouped launch per weight-sync bucket of about 1-3 GB (a
Qwen3-30B-A3B layer, four Qwen3-4B layers, one DeepSeek-V3 expert-parallel
rank's 32 experts), per transformer layer, or over the whole workload.
"""
from __future__ import annotations

import dataclasses

import torch

import precision_weight_quantization_amd as lpq
from synth import gpu as sgpu
from synth import synth

GB = 1e9

# projection ids inside a layer (part of each tensor's generator stream id)
P_Q, P_K, P_V, P_O, P_GATE, P_UP, P_DOWN = range(7)


@dataclasses.dataclass
class TensorSpec:
    name: str
    layer: int
    expert: int
    proj: int
    M: int
    N: int
    group: int = 0

    @property
    def numel(self) -> int:
        return self.M * self.N


def dense_specs(layers=36):
    shapes = [(P_Q, 4096, 2560), (P_K, 1024, 2560), (P_V, 1024, 2560), (P_O, 2560, 4096),
              (P_GATE, 9728, 2560), (P_UP, 9728, 2560), (P_DOWN, 2560, 9728)]
    return [TensorSpec(f"L{l}.p{p}", l, 0, p, M, N) for l in range(layers) for (p, M, N) in shapes]


def moe_specs(layers=48, experts=128, attention=False):
    out = []
    g = 0
    for l in range(layers):
        if attention:
            for p, M in ((P_Q, 4096), (P_K, 512), (P_V, 512)):
                out.append(TensorSpec(f"L{l}.attn.p{p}", l, 0xFFFF, p, M, 2048, g))
            g += 1
        for e in range(experts):
            out.append(TensorSpec(f"L{l}.e{e}.gate", l, e, P_GATE, 768, 2048, g))
            out.append(TensorSpec(f"L{l}.e{e}.up", l, e, P_UP, 768, 2048, g))
            g += 1
            out.append(TensorSpec(f"L{l}.e{e}.down", l, e, P_DOWN, 2048, 768, g))
            g += 1
    return out


def dsv3_specs(experts=256):
    out = []
    for e in range(experts):
        out.append(TensorSpec(f"e{e}.gate", 0, e, P_GATE, 2048, 7168))
        out.append(TensorSpec(f"e{e}.up", 0, e, P_UP, 2048, 7168))
        out.append(TensorSpec(f"e{e}.down", 0, e, P_DOWN, 7168, 2048))
    return out


class Slab:
    """One device allocation carved into 256-byte aligned per-tensor views."""

    def __init__(self, sizes_bytes, device, dtype=torch.uint8):
        self.offsets = []
        off = 0
        for b in sizes_bytes:
            self.offsets.append(off)
            off += (b + 255) // 256 * 256
        self.buf = torch.empty(max(off, 256), dtype=torch.uint8, device=device)
        self.nbytes = off

    def view(self, i, shape, dtype):
        n = 1
        for s in shape:
            n *= s
        nb = n * torch.empty((), dtype=dtype).element_size()
        return self.buf[self.offsets[i]:self.offsets[i] + nb].view(dtype).view(shape)


class WeightSet:
    """BF16 weights of one workload, generated on the device."""

    def __init__(self, config: int, specs, dist, device="cuda"):
        self.config = config
        self.specs = specs
        self.seed = synth.seed_of(config)
        self.dist = dist
        self.slab = Slab([s.numel * 2 for s in specs], device)
        self.w = [self.slab.view(i, (s.M, s.N), torch.bfloat16) for i, s in enumerate(specs)]
        for s, w in zip(specs, self.w):
            sgpu.fill(w, self.seed, synth.stream_of(s.layer, s.expert, s.proj), dist)

    @property
    def numel(self) -> int:
        return sum(s.numel for s in self.specs)

    def layers(self):
        out = {}
        for i, s in enumerate(self.specs):
            out.setdefault(s.layer, []).append(i)
        return [out[k] for k in sorted(out)]


# --------------------------------------------------------------------------- operations

@dataclasses.dataclass
class Op:
    name: str              # e.g. "mxfp8.quantize"
    workload: str
    bytes: float           # algorithmic bytes (in + out) of one run
    launches: list         # callables, one per grouped launch
    counted: bool = True   # False: in the step's time, not in its algorithmic bytes

    def run(self):
        for f in self.launches:
            f()


# Weight-sync buckets: the tensors one grouped launch covers.  A weight sync
# streams its buckets one after another; "sync" (the default) keeps each at
# about 1-3 GB of BF16: a Qwen3-30B-A3B layer (384 expert tensors, 1.2 GB), four
# Qwen3-4B layers (28 tensors, 1.2 GB), one DeepSeek-V3 expert-parallel rank's
# share (32 of 256 experts, 96 tensors, 2.8 GB).  Measured on the DeepSeek-V3
# layer: block-FP8 quantize 73% of HBM peak as one 22.5 GB launch against 78%
# in such buckets (MXFP8 quantize on the same tensors: 77% against 82%); on
# Qwen3-4B, 70% per layer against 75% for four layers.  A Qwen3-4B bucket lists
# its tensors by shape (q and o, then k and v, then gate, up and down: three runs
# of equal work-unit counts), so that it is one launch rather than two of at
# most 8 runs each: about one more point for quantize and dequantize.  "layer"
# and "all" are one launch per transformer layer and one launch over everything.
DENSE_LAYERS_PER_BUCKET = 4
EP_RANK_EXPERTS = 32


def _buckets(ws: WeightSet, bucket: str):
    if bucket == "all":
        return [list(range(len(ws.specs)))]
    if bucket == "layer":
        return ws.layers()
    if ws.config == 2:      # Qwen3-4B dense
        layers = ws.layers()
        buckets = [sum(layers[i:i + DENSE_LAYERS_PER_BUCKET], [])
                   for i in range(0, len(layers), DENSE_LAYERS_PER_BUCKET)]
        return [sorted(b, key=lambda i: (ws.specs[i].numel, ws.specs[i].M, i)) for b in buckets]
    if ws.config == 5:      # DeepSeek-V3 MoE layer: per expert-parallel rank
        out = {}
        for i, s in enumerate(ws.specs):
            out.setdefault(s.expert // EP_RANK_EXPERTS, []).append(i)
        return [out[k] for k in sorted(out)]
    return ws.layers()


def fp8blk_ops(tag: str, ws: WeightSet, codes: Slab, scales: Slab, out: Slab, bucket: str):
    specs = ws.specs
    q = [codes.view(i, (s.M, s.N), torch.uint8) for i, s in enumerate(specs)]
    sc = [scales.view(i, ((s.M + 127) // 128, (s.N + 127) // 128), torch.float32) for i, s in enumerate(specs)]
    y = [out.view(i, (s.M, s.N), torch.bfloat16) for i, s in enumerate(specs)]
    tq, tdq = [], []
    for idx in _buckets(ws, bucket):
        tq.append(lpq.TensorTable([(ws.w[i], q[i], sc[i], specs[i].M, specs[i].N, 0) for i in idx]))
        tdq.append(lpq.TensorTable([(q[i], y[i], sc[i], specs[i].M, specs[i].N, 0) for i in idx]))
    tiles = sum(((s.M + 127) // 128) * ((s.N + 127) // 128) for s in specs)
    nbytes = 3 * ws.numel + 4 * tiles
    return ([Op(f"fp8blk.quantize[{tag}]", tag, nbytes, [lambda t=t: lpq.lpq_quantize_fp8blk_grouped(t) for t in tq]),
             Op(f"fp8blk.dequantize[{tag}]", tag, nbytes, [lambda t=t: lpq.lpq_dequantize_fp8blk_grouped(t) for t in tdq])],
            dict(q=q, s=sc, y=y))


def mxfp8_ops(tag: str, ws: WeightSet, codes: Slab, ebytes: Slab, out: Slab, bucket: str):
    specs = ws.specs
    q = [codes.view(i, (s.M, s.N), torch.uint8) for i, s in enumerate(specs)]
    e = [ebytes.view(i, (s.M, s.N // 32), torch.uint8) for i, s in enumerate(specs)]
    y = [out.view(i, (s.M, s.N), torch.bfloat16) for i, s in enumerate(specs)]
    tq, tdq = [], []
    for idx in _buckets(ws, bucket):
        tq.append(lpq.TensorTable([(ws.w[i], q[i], e[i], specs[i].M, specs[i].N, 0) for i in idx]))
        tdq.append(lpq.TensorTable([(q[i], y[i], e[i], specs[i].M, specs[i].N, 0) for i in idx]))
    nbytes = 3 * ws.numel + ws.numel // 32
    return ([Op(f"mxfp8.quantize[{tag}]", tag, nbytes, [lambda t=t: lpq.lpq_quantize_mxfp8_grouped(t) for t in tq]),
             Op(f"mxfp8.dequantize[{tag}]", tag, nbytes, [lambda t=t: lpq.lpq_dequantize_mxfp8_grouped(t) for t in tdq])],
            dict(q=q, e=e, y=y),
            # the OCP floor-rule variant (a widening row): same tensors and outputs
            [Op(f"mxfp8.quantize.floor[{tag}]", tag, nbytes,
                [lambda t=t: lpq.lpq_quantize_mxfp8_floor_grouped(t) for t in tq])])


def nvfp4_ops(tag: str, ws: WeightSet, packed: Slab, sbytes: Slab, out: Slab, bucket: str, device="cuda"):
    specs = ws.specs
    n_groups = max(s.group for s in specs) + 1
    amax = torch.zeros(n_groups, dtype=torch.float32, device=device)
    g = torch.zeros(n_groups, dtype=torch.float32, device=device)
    p = [packed.view(i, (s.M, s.N // 2), torch.uint8) for i, s in enumerate(specs)]
    sb = [sbytes.view(i, (s.M, s.N // 16), torch.uint8) for i, s in enumerate(specs)]
    y = [out.view(i, (s.M, s.N), torch.bfloat16) for i, s in enumerate(specs)]
    tq, tdq, tqdq = [], [], []
    # the amax pre-pass covers the whole model in one grouped call; tensors of
    # equal shape are put next to each other so that the call is one launch
    by_shape = sorted(range(len(specs)), key=lambda i: (specs[i].M, specs[i].N, i))
    tamax = lpq.TensorTable([(ws.w[i], None, None, specs[i].M, specs[i].N, specs[i].group) for i in by_shape])
    for idx in _buckets(ws, bucket):
        tq.append(lpq.TensorTable([(ws.w[i], p[i], sb[i], specs[i].M, specs[i].N, specs[i].group) for i in idx]))
        tdq.append(lpq.TensorTable([(p[i], y[i], sb[i], specs[i].M, specs[i].N, specs[i].group) for i in idx]))
        tqdq.append(lpq.TensorTable([(ws.w[i], y[i], None, specs[i].M, specs[i].N, specs[i].group) for i in idx]))
    n = ws.numel
    qbytes = 2 * n + n // 2 + n // 16 + 4 * n_groups
    # the amax pass accumulates: zero all group slots first (a fill kernel), then max in
    ops = [
        Op(f"nvfp4.amax[{tag}]", tag, 2 * n,
           [lambda: lpq.lpq_nvfp4_amax_grouped(tamax, amax, accumulate=False)], counted=False),
        Op(f"nvfp4.quantize[{tag}]", tag, qbytes, [lambda t=t: lpq.lpq_quantize_nvfp4_grouped(t, amax, g) for t in tq]),
        Op(f"nvfp4.dequantize[{tag}]", tag, qbytes, [lambda t=t: lpq.lpq_dequantize_nvfp4_grouped(t, g) for t in tdq]),
        Op(f"nvfp4.qdq[{tag}]", tag, 4 * n, [lambda t=t: lpq.lpq_nvfp4_qdq_grouped(t, amax) for t in tqdq]),
    ]
    return ops, dict(p=p, s=sb, y=y, amax=amax, g=g, n_groups=n_groups)


INT4_GROUP = 128


def int4_ops(tag: str, ws: WeightSet, packed: Slab, scales: Slab, out: Slab, bucket: str, group: int = INT4_GROUP):
    specs = ws.specs
    p = [packed.view(i, (s.M, s.N // 2), torch.uint8) for i, s in enumerate(specs)]
    sc = [scales.view(i, (s.M, s.N // group), torch.float32) for i, s in enumerate(specs)]
    y = [out.view(i, (s.M, s.N), torch.bfloat16) for i, s in enumerate(specs)]
    tq, tdq, tqdq = [], [], []
    for idx in _buckets(ws, bucket):
        tq.append(lpq.TensorTable([(ws.w[i], p[i], sc[i], specs[i].M, specs[i].N, 0) for i in idx]))
        tdq.append(lpq.TensorTable([(p[i], y[i], sc[i], specs[i].M, specs[i].N, 0) for i in idx]))
        tqdq.append(lpq.TensorTable([(ws.w[i], y[i], None, specs[i].M, specs[i].N, 0) for i in idx]))
    n = ws.numel
    qbytes = 2 * n + n // 2 + 4 * (n // group)
    ops = [
        Op(f"int4.quantize[{tag}]", tag, qbytes, [lambda t=t: lpq.lpq_quantize_int4_grouped(t, group) for t in tq]),
        Op(f"int4.dequantize[{tag}]", tag, qbytes, [lambda t=t: lpq.lpq_dequantize_int4_grouped(t, group) for t in tdq]),
        Op(f"int4.qdq[{tag}]", tag, 4 * n, [lambda t=t: lpq.lpq_int4_qdq_grouped(t, group) for t in tqdq]),
    ]
    return ops, dict(p=p, s=sc, y=y, group=group)


def tiles_of(s: TensorSpec) -> int:
    return ((s.M + 127) // 128) * ((s.N + 127) // 128)


def fp8_source(ws: WeightSet, device):
    """Block-wise FP8 copies (codes, tile scales) of every weight of ``ws``."""
    specs = ws.specs
    qslab = Slab([s.numel for s in specs], device)
    sslab = Slab([4 * tiles_of(s) for s in specs], device)
    q = [qslab.view(i, (s.M, s.N), torch.uint8) for i, s in enumerate(specs)]
    sc = [sslab.view(i, ((s.M + 127) // 128, (s.N + 127) // 128), torch.float32) for i, s in enumerate(specs)]
    for idx in ws.layers():
        lpq.lpq_quantize_fp8blk_grouped(lpq.TensorTable([(ws.w[i], q[i], sc[i], specs[i].M, specs[i].N, 0)
                                                         for i in idx]))
    return q, sc, (qslab, sslab)


POW2_MASK = 0x7F800000   # the exponent field (the scales here are non-negative)


def pow2_tile_scales(s8):
    """Each tile scale cut to the power of two at or below it (its significand bits
    cleared): the same codes then stand for a block-FP8 tensor with power-of-two
    block scales."""
    return [(s.view(torch.int32) & POW2_MASK).view(torch.float32) for s in s8]


def requant_ops(ws: WeightSet, q8, s8, codes: Slab, out: Slab, bucket: str, device="cuda", tag="fp8train",
                fused_only=False):
    """Fused FP8 -> MXFP8 (experts) and FP8 -> NVFP4 (all tensors) re-quantization,
    and (unless fused_only) the unfused sequences they replace, writing into the
    shared slabs."""
    specs = ws.specs
    ex = [i for i, s in enumerate(specs) if s.expert != 0xFFFF]
    n_ex, t_ex = sum(specs[i].numel for i in ex), sum(tiles_of(specs[i]) for i in ex)
    n, t = ws.numel, sum(tiles_of(s) for s in specs)
    n_groups = max(s.group for s in specs) + 1
    exset = set(ex)

    # block-FP8 targets of every tensor (the page's FP8 -> BF16 -> FP8 sync)
    fcodes = reslab(codes, specs, 1)
    fsl = Slab([4 * tiles_of(s) for s in specs], device)
    fq = [fcodes.view(i, (s.M, s.N), torch.uint8) for i, s in enumerate(specs)]
    fs = [fsl.view(i, ((s.M + 127) // 128, (s.N + 127) // 128), torch.float32) for i, s in enumerate(specs)]
    # MXFP8 targets of the experts
    mcodes = reslab(codes, [specs[i] for i in ex], 1)
    eb = Slab([specs[i].numel // 32 for i in ex], device)
    mq = {i: mcodes.view(k, (specs[i].M, specs[i].N), torch.uint8) for k, i in enumerate(ex)}
    me = {i: eb.view(k, (specs[i].M, specs[i].N // 32), torch.uint8) for k, i in enumerate(ex)}
    # NVFP4 targets of every tensor; BF16 staging of the unfused sequences
    packed = reslab(codes, specs, 0.5)
    sbs = Slab([s.numel // 16 for s in specs], device)
    p = [packed.view(i, (s.M, s.N // 2), torch.uint8) for i, s in enumerate(specs)]
    sb = [sbs.view(i, (s.M, s.N // 16), torch.uint8) for i, s in enumerate(specs)]
    ys = reslab(out, specs, 2)
    y = [ys.view(i, (s.M, s.N), torch.bfloat16) for i, s in enumerate(specs)]
    amax = torch.zeros(n_groups, dtype=torch.float32, device=device)
    g = torch.zeros(n_groups, dtype=torch.float32, device=device)

    by_shape = sorted(range(len(specs)), key=lambda i: (specs[i].M, specs[i].N, i))
    tamax = lpq.RequantTable([(q8[i], s8[i], None, None, specs[i].M, specs[i].N, specs[i].group) for i in by_shape])
    rmx, rnv, dq_mx, q_mx, dq_nv, a_nv, q_nv = [], [], [], [], [], [], []
    rf8, q_f8 = [], []
    for idx in _buckets(ws, bucket):
        ie = [i for i in idx if i in exset]
        rf8.append(lpq.RequantTable([(q8[i], s8[i], fq[i], fs[i], specs[i].M, specs[i].N, 0) for i in idx]))
        q_f8.append(lpq.TensorTable([(y[i], fq[i], fs[i], specs[i].M, specs[i].N, 0) for i in idx]))
        rmx.append(lpq.RequantTable([(q8[i], s8[i], mq[i], me[i], specs[i].M, specs[i].N, 0) for i in ie]))
        rnv.append(lpq.RequantTable([(q8[i], s8[i], p[i], sb[i], specs[i].M, specs[i].N, specs[i].group)
                                     for i in idx]))
        dq_mx.append(lpq.TensorTable([(q8[i], y[i], s8[i], specs[i].M, specs[i].N, 0) for i in ie]))
        q_mx.append(lpq.TensorTable([(y[i], mq[i], me[i], specs[i].M, specs[i].N, 0) for i in ie]))
        dq_nv.append(lpq.TensorTable([(q8[i], y[i], s8[i], specs[i].M, specs[i].N, 0) for i in idx]))
        q_nv.append(lpq.TensorTable([(y[i], p[i], sb[i], specs[i].M, specs[i].N, specs[i].group) for i in idx]))
    # the unfused NVFP4 sequence stages every BF16 tensor, takes the model-wide amax
    # over them (as the fused sequence does over the FP8 copies), then quantizes
    a_nv = lpq.TensorTable([(y[i], None, None, specs[i].M, specs[i].N, specs[i].group) for i in by_shape])

    def unfused_mx(k):
        lpq.lpq_dequantize_fp8blk_grouped(dq_mx[k])
        lpq.lpq_quantize_mxfp8_grouped(q_mx[k])


    f8_bytes = 2 * n + 8 * t
    mx_bytes = 2 * n_ex + n_ex // 32 + 4 * t_ex
    amax_bytes = n + 4 * t
    nv_bytes = n + 4 * t + n // 2 + n // 16 + 4 * n_groups
    fused = [
        Op(f"requant.fp8blk[{tag}]", tag, f8_bytes,
           [lambda r=r: lpq.lpq_requantize_fp8blk_grouped(r) for r in rf8]),
        Op(f"requant.mxfp8[{tag}]", tag, mx_bytes,
           [lambda r=r: lpq.lpq_requantize_fp8blk_mxfp8_grouped(r) for r in rmx]),
        Op(f"requant.amax[{tag}]", tag, amax_bytes,
           [lambda: lpq.lpq_fp8blk_amax_grouped(tamax, amax, accumulate=False)]),
        Op(f"requant.nvfp4[{tag}]", tag, nv_bytes,
           [lambda r=r: lpq.lpq_requantize_fp8blk_nvfp4_grouped(r, amax, g) for r in rnv]),
    ]
    unfused = [
        Op(f"requant.fp8blk.unfused[{tag}]", tag, f8_bytes,
           [f for k in range(len(rf8)) for f in (lambda k=k: lpq.lpq_dequantize_fp8blk_grouped(dq_nv[k]),
                                                  lambda k=k: lpq.lpq_quantize_fp8blk_grouped(q_f8[k]))]),
        Op(f"requant.mxfp8.unfused[{tag}]", tag, mx_bytes,
           [lambda k=k: unfused_mx(k) for k in range(len(rmx))]),
        Op(f"requant.nvfp4.unfused[{tag}]", tag, amax_bytes + nv_bytes,
           [lambda t=t: lpq.lpq_dequantize_fp8blk_grouped(t) for t in dq_nv]
           + [lambda: lpq.lpq_nvfp4_amax_grouped(a_nv, amax, accumulate=False)]
           + [lambda t=t: lpq.lpq_quantize_nvfp4_grouped(t, amax, g) for t in q_nv]),
    ]
    ops = fused if fused_only else [fused[0], unfused[0], fused[1], unfused[1], fused[2], fused[3], unfused[2]]
    return ops, dict(ex=ex, fq=fq, fs=fs, mq=mq, me=me, p=p, sb=sb, amax=amax, g=g, n_groups=n_groups, q8=q8, s8=s8)


def activation_ops(x: torch.Tensor, y: torch.Tensor):
    amax = torch.zeros(1, dtype=torch.float32, device=x.device)
    n = x.numel()
    # the W4A4 path with the default observer (a widening row): observe the batch, then QDQ
    state = lpq.lpq_observer_reset(device=x.device)
    oamax = torch.zeros(1, dtype=torch.float32, device=x.device)
    return ([Op("nvfp4.amax[act]", "act", 2 * n, [lambda: lpq.lpq_nvfp4_amax(x, amax)], counted=False),
             Op("nvfp4.qdq[act]", "act", 4 * n, [lambda: lpq.lpq_nvfp4_qdq(x, amax, y)])],
            dict(amax=amax, state=state, observer_amax=oamax),
            [Op("nvfp4.observe+qdq[act]", "act", 6 * n,
                [lambda: lpq.lpq_nvfp4_observe(x, state, "static_minmax", amax=oamax),
                 lambda: lpq.lpq_nvfp4_qdq(x, oamax, y)])])


WORKLOADS = ("dense", "moe", "nvfp4", "dsv3")
NEXT_WORKLOADS = ("fp8train", "int4")


def reslab(slab: Slab, specs, bytes_per_elem):
    """A view-only slab over `slab`'s buffer laid out for `specs`."""
    s = Slab.__new__(Slab)
    s.buf = slab.buf
    s.offsets = []
    off = 0
    for sp in specs:
        s.offsets.append(off)
        off += (int(sp.numel * bytes_per_elem) + 255) // 256 * 256
    assert off <= slab.buf.numel(), "output slab too small"
    s.nbytes = off
    return s


class Bench:
    """All workloads' tensors and operations, buffers shared where the order allows."""

    def __init__(self, which=WORKLOADS, bucket="sync", device="cuda", log=print, scale_layers=None):
        self.ops = []
        self.next_ops = []      # widening rows: timed apart from the step
        self.outputs = {}
        self.sets = {}
        L = scale_layers
        need_moe = any(w in which for w in ("moe", "nvfp4", "fp8train", "int4"))
        if "dense" in which:
            self.sets["dense"] = WeightSet(2, dense_specs(L or 36), synth.DIST_DENSE, device)
            log(f"generated dense weights: {self.sets['dense'].numel * 2 / GB:.2f} GB")
        if need_moe:
            self.sets["moe"] = WeightSet(3, moe_specs(L or 48, attention=True), synth.DIST_MOE, device)
            log(f"generated MoE expert + attention weights: {self.sets['moe'].numel * 2 / GB:.2f} GB")
        if "dsv3" in which:
            self.sets["dsv3"] = WeightSet(5, dsv3_specs(256 if L is None else max(4, L)), synth.DIST_MOE, device)
            log(f"generated DeepSeek-V3 layer weights: {self.sets['dsv3'].numel * 2 / GB:.2f} GB")
        # shared output slabs, sized for the largest user
        maxspecs = max((ws.specs for ws in self.sets.values()), key=lambda sp: sum(s.numel for s in sp))
        self.codes = Slab([s.numel for s in maxspecs], device)
        self.out = Slab([2 * s.numel for s in maxspecs], device)
        if "dense" in which:
            ws = self.sets["dense"]
            codes = self._reslab(self.codes, ws.specs, 1)
            sc = Slab([4 * ((s.M + 127) // 128) * ((s.N + 127) // 128) for s in ws.specs], device)
            out = self._reslab(self.out, ws.specs, 2)
            ops, o = fp8blk_ops("dense", ws, codes, sc, out, bucket)
            self.ops += ops
            self.outputs["dense"] = o
        if "moe" in which:
            ws = self._experts_only(self.sets["moe"])
            codes = self._reslab(self.codes, ws.specs, 1)
            eb = Slab([s.numel // 32 for s in ws.specs], device)
            out = self._reslab(self.out, ws.specs, 2)
            ops, o, nxt = mxfp8_ops("moe", ws, codes, eb, out, bucket)
            self.ops += ops
            self.next_ops += nxt
            self.outputs["moe"] = o
            self.sets["moe_experts"] = ws
        if "nvfp4" in which:
            ws = self.sets["moe"]
            packed = self._reslab(self.codes, ws.specs, 0.5)
            sb = Slab([s.numel // 16 for s in ws.specs], device)
            out = self._reslab(self.out, ws.specs, 2)
            ops, o = nvfp4_ops("nvfp4", ws, packed, sb, out, bucket, device)
            self.ops += ops
            self.outputs["nvfp4"] = o
            x = torch.empty((8192, 2048), dtype=torch.bfloat16, device=device)
            sgpu.fill(x, synth.seed_of(4), synth.stream_of(0xFFFF, 0xFFFFFF, 0xFFFF), synth.DIST_ACT)
            ya = torch.empty_like(x)
            ops, o, nxt = activation_ops(x, ya)
            self.ops += ops
            self.next_ops += nxt
            self.outputs["act"] = dict(x=x, y=ya, **o)
        if "dsv3" in which:
            ws = self.sets["dsv3"]
            codes = self._reslab(self.codes, ws.specs, 1)
            sc = Slab([4 * ((s.M + 127) // 128) * ((s.N + 127) // 128) for s in ws.specs], device)
            out = self._reslab(self.out, ws.specs, 2)
            ops, o = fp8blk_ops("dsv3", ws, codes, sc, out, bucket)
            self.ops += ops
            self.outputs["dsv3"] = o
        if "fp8train" in which:
            ws = self.sets["moe"]
            q8, s8, keep = fp8_source(ws, device)
            log(f"block-wise FP8 copies of the MoE + attention weights: {sum(k.nbytes for k in keep) / GB:.2f} GB")
            ops, o = requant_ops(ws, q8, s8, self.codes, self.out, bucket, device)
            o["keep"] = keep
            self.next_ops += ops
            self.outputs["fp8train"] = o
            s8p = pow2_tile_scales(s8)
            ops, o2 = requant_ops(ws, q8, s8p, self.codes, self.out, bucket, device, tag="fp8train-pow2",
                                  fused_only=True)
            o2["keep"] = s8p
            self.next_ops += ops
            self.outputs["fp8train-pow2"] = o2
        if "int4" in which:
            ws = self.sets.get("moe_experts") or self._experts_only(self.sets["moe"])
            self.sets["moe_experts"] = ws
            packed = self._reslab(self.codes, ws.specs, 0.5)
            sc = Slab([4 * (s.numel // INT4_GROUP) for s in ws.specs], device)
            out = self._reslab(self.out, ws.specs, 2)
            ops, o = int4_ops("int4", ws, packed, sc, out, bucket)
            self.next_ops += ops
            self.outputs["int4"] = o

    _reslab = staticmethod(reslab)

    @staticmethod
    def _experts_only(ws: WeightSet) -> WeightSet:
        sub = WeightSet.__new__(WeightSet)
        keep = [i for i, s in enumerate(ws.specs) if s.expert != 0xFFFF]
        sub.config, sub.seed, sub.dist = 3, ws.seed, ws.dist
        sub.specs = [ws.specs[i] for i in keep]
        sub.w = [ws.w[i] for i in keep]
        sub.slab = ws.slab
        return sub

    def counted_bytes(self) -> float:
        return sum(op.bytes for op in self.ops if op.counted)

    def step(self):
        for op in self.ops:
            op.run()

    def next_step(self):
        for op in self.next_ops:
            op.run()
