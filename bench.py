"""Throughput of the low-precision weight codecs on one MI355X.

One step = one pass of the whole hot path over every full-size weight
workload (see workloads.py): block-wise FP8 quantize + dequantize of the
Qwen3-4B dense weights and of a DeepSeek-V3 MoE layer, MXFP8 quantize +
dequantize of the Qwen3-30B-A3B experts, and NVFP4 group amax + quantize +
dequantize + weight QDQ of those experts with q/k/v, plus the W4A4 activation
amax + QDQ.  Inputs are generated on the device before timing; the timed
region holds only the codec launches.

value = algorithmic bytes of the step (each input and output byte counted
once; the NVFP4 amax pre-passes are timed but not counted) / step time.

The widening rows -- the fp8train workload (fused re-quantization of
block-wise FP8 weights into block-wise FP8 / MXFP8 / NVFP4, next to the
unfused sequences), the OCP floor-rule MXFP8 quantizer, the W4A4 observer,
and group-wise INT4 of the Qwen3-30B-A3B experts -- are timed after the
step, over the same number of iterations, and reported under "next_rows";
they are not part of value or ms_per_step.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, GB/s
GB = 1e9
NEXT_CPU_STRIDE = 48   # the widening rows' oracle sample: every 48th tensor or sibling group


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# every source of the kernel library (the .hip translation unit and the parts it includes), in a fixed order
KERNEL_SOURCES = tuple(sorted(os.path.relpath(f, ROOT) for ext in ("*.hip", "*.hpp")
                              for f in glob.glob(os.path.join(ROOT, "precision_weight_quantization_amd", "csrc", ext))))


def code_text(src: str) -> str:
    """C++ source without its comments and blank lines, spaces at line ends removed:
    what the compiler sees, so that a comment-only edit keeps recorded counters valid."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_hash(root: str = ROOT) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(op_name: str):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel source, if recorded."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = rec.get("ops", {}).get(op_name)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------- CPU baseline

def cpu_baseline(bench, stride: int, threads: int):
    """Time the oracle on every `stride`-th tensor (NVFP4: sibling group) of each
    workload, on `threads` host threads, and compare its outputs with the GPU's."""
    import numpy as np
    import torch

    from oracle import oracle as O

    def h8(t):
        return t.contiguous().view(torch.uint8).cpu().numpy()

    def h16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    jobs = []        # (callable, algorithmic bytes); each callable returns a mismatch count
    for op in bench.ops:
        op.run()
        torch.cuda.synchronize()
        wl = op.workload
        if wl in ("dense", "dsv3") or wl == "moe":
            ws = bench.sets["moe_experts" if wl == "moe" else wl]
            out = bench.outputs[wl]
            for i in range(0, len(ws.specs), stride):
                sp = ws.specs[i]
                x = h16(ws.w[i])
                if op.name.startswith("fp8blk.quantize"):
                    q, s = h8(out["q"][i]), out["s"][i].cpu().numpy()

                    def job(x=x, q=q, s=s):
                        oq, os_ = O.fp8blk_quantize(x)
                        return int((oq != q).sum() + (os_ != s).sum())
                    jobs.append((job, 3 * sp.numel + 4 * s.size, "fp8blk"))
                elif op.name.startswith("fp8blk.dequantize"):
                    q, s, y = h8(out["q"][i]), out["s"][i].cpu().numpy(), h16(out["y"][i])
                    jobs.append((lambda q=q, s=s, y=y: int((O.fp8blk_dequantize(q, s) != y).sum()),
                                 3 * sp.numel + 4 * s.size, "fp8blk"))
                elif op.name.startswith("mxfp8.quantize"):
                    q, e = h8(out["q"][i]), h8(out["e"][i])
                    jobs.append((lambda x=x, q=q, e=e: (lambda r: int((r[0] != q).sum() + (r[1] != e).sum()))(
                        O.mxfp8_quantize(x)), 3 * sp.numel + sp.numel // 32, "mxfp8"))
                elif op.name.startswith("mxfp8.dequantize"):
                    q, e, y = h8(out["q"][i]), h8(out["e"][i]), h16(out["y"][i])
                    jobs.append((lambda q=q, e=e, y=y: int((O.mxfp8_dequantize(q, e) != y).sum()),
                                 3 * sp.numel + sp.numel // 32, "mxfp8"))
        elif wl == "nvfp4" and op.counted:
            ws = bench.sets["moe"]
            out = bench.outputs["nvfp4"]
            groups = {}
            for i, sp in enumerate(ws.specs):
                groups.setdefault(sp.group, []).append(i)
            g_dev = out["g"].cpu().numpy()
            for gid in sorted(groups)[::stride]:
                idx = groups[gid]
                xs = [h16(ws.w[i]) for i in idx]
                n = sum(ws.specs[i].numel for i in idx)
                if op.name.startswith("nvfp4.quantize"):
                    ps, ss = [h8(out["p"][i]) for i in idx], [h8(out["s"][i]) for i in idx]
                    gg = np.float32(g_dev[gid])

                    def job(xs=xs, ps=ps, ss=ss, gg=gg):
                        A, g, res = O.nvfp4_quantize_group(xs)
                        bad = int(np.float32(g) != gg)
                        for (p, s), pp, sg in zip(res, ps, ss):
                            bad += int((p != pp).sum() + (s != sg).sum())
                        return bad
                    jobs.append((job, 2 * n + n // 2 + n // 16 + 4, "nvfp4"))
                elif op.name.startswith("nvfp4.dequantize") or op.name.startswith("nvfp4.qdq"):
                    ys = [h16(out["y"][i]) for i in idx]
                    gg = float(g_dev[gid])
                    if op.name.startswith("nvfp4.dequantize"):
                        ps, ss = [h8(out["p"][i]) for i in idx], [h8(out["s"][i]) for i in idx]
                        jobs.append((lambda ps=ps, ss=ss, ys=ys, gg=gg: sum(
                            int((O.nvfp4_dequantize(p, s, gg) != y).sum()) for p, s, y in zip(ps, ss, ys)),
                            2 * n + n // 2 + n // 16 + 4, "nvfp4"))
                    else:
                        jobs.append((lambda xs=xs, ys=ys: (lambda g: sum(
                            int((O.nvfp4_qdq(x, g) != y).sum()) for x, y in zip(xs, ys)))(
                            O.nvfp4_group_scale(xs)[1]), 4 * n, "nvfp4"))
        elif wl == "act" and op.counted:
            a = bench.outputs["act"]
            x, y = h16(a["x"]), h16(a["y"])
            jobs.append((lambda x=x, y=y: int((O.nvfp4_qdq(x, O.nvfp4_group_scale([x])[1]) != y).sum()),
                         4 * x.size, "nvfp4"))
    O.default()
    t0 = time.perf_counter()
    res = O.run_parallel(lambda j: j[0](), jobs, threads)
    dt = time.perf_counter() - t0
    total = sum(j[1] for j in jobs)
    # one host thread on a short prefix of the same calls (the Qwen3-4B block-FP8 ones come first)
    one, one_bytes = [], 0
    for j in jobs:
        if one_bytes >= 0.25 * GB:
            break
        one.append(j)
        one_bytes += j[1]
    t1 = time.perf_counter()
    bad1 = sum(j[0]() for j in one)
    dt1 = time.perf_counter() - t1
    lin = linear_single_thread()
    return {
        "value": round(total / dt / GB, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"every {stride}th tensor (NVFP4: every {stride}th sibling group) of each workload op, plus the "
                  f"whole activation QDQ: {len(jobs)} oracle calls, {total / GB:.2f} GB algorithmic, {dt:.1f} s",
        "seconds": round(dt, 2),
        "parity_mismatches": int(sum(res)) + int(bad1),
        "single_thread": {"value": round(one_bytes / dt1 / GB, 3), "unit": "GB/s", "cores": 1,
                          "workload": "Qwen3-4B dense block-FP8 quantize",
                          "sample": f"the first {len(one)} of those calls ({one_bytes / GB:.2f} GB algorithmic), "
                                    f"{dt1:.1f} s"},
        "single_thread_linear": lin,
    }


def linear_single_thread(min_seconds: float = 1.0):
    """One host thread on the 256x512 single-Linear case: block-FP8, MXFP8 and
    NVFP4 quantize + dequantize and the NVFP4 QDQ, repeated for `min_seconds`."""
    from oracle import oracle as O
    from synth import synth

    w = synth.single_linear()
    n, M, N = w.size, w.shape[0], w.shape[1]
    tiles = -(-M // 128) * -(-N // 128)
    per_pass = (2 * (3 * n + 4 * tiles) + 2 * (3 * n + n // 32) + 2 * (2 * n + n // 2 + n // 16 + 4) + 4 * n)
    orc = O.default()

    def one_pass():
        q, s = orc.fp8blk_quantize(w)
        orc.fp8blk_dequantize(q, s)
        q, e = orc.mxfp8_quantize(w)
        orc.mxfp8_dequantize(q, e)
        _, g, ((p, sb),) = orc.nvfp4_quantize_group([w])
        orc.nvfp4_dequantize(p, sb, g)
        orc.nvfp4_qdq(w, g)

    one_pass()
    passes, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(passes * per_pass / dt / GB, 3), "unit": "GB/s", "cores": 1,
            "workload": f"single Linear {M}x{N}, all formats quantize + dequantize + NVFP4 QDQ",
            "sample": f"{passes} passes of {per_pass} algorithmic bytes, {dt:.2f} s"}


def next_rows_parity(bench, stride: int, threads: int):
    """Run each widening-row op and compare every `stride`-th tensor (NVFP4: sibling
    group) of its outputs with the oracle, timing the oracle per op.

    The oracle starts from the BF16 weights: for the re-quantization rows it forms
    its own block-wise FP8 copy (untimed, before the op's timed jobs), then
    re-quantizes that.  Each op's sample is credited with the op's algorithmic
    bytes in proportion to its share of the op's elements.  Returns the totals and,
    per op, the oracle's rate on its sample (the unfused rows are checked, not timed:
    their oracle is the fused rows')."""
    import numpy as np
    import torch

    import workloads as W
    from oracle import oracle as O

    def h8(t):
        return t.contiguous().view(torch.uint8).cpu().numpy()

    def h16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    per_op = []   # (op, [(prep, job, elements)], elements of the op)
    for op in bench.next_ops:
        op.run()
        torch.cuda.synchronize()
        jobs = []
        if op.name.startswith("mxfp8.quantize.floor"):
            ws = bench.sets["moe_experts"]
            out = bench.outputs["moe"]
            for i in range(0, len(ws.specs), stride):
                x, q, e = h16(ws.w[i]), h8(out["q"][i]), h8(out["e"][i])

                def job(_, x=x, q=q, e=e):
                    oq, oe = O.mxfp8_floor_quantize(x)
                    return int((oq != q).sum() + (oe != e).sum())
                jobs.append((None, job, ws.specs[i].numel))
            per_op.append((op, jobs, sum(sp.numel for sp in ws.specs)))
            continue
        if op.name.startswith("nvfp4.observe+qdq"):
            # the same batch every time: the static observer's extremes are that batch's
            a = bench.outputs["act"]
            x, y = h16(a["x"]), h16(a["y"])
            jobs.append((None, lambda _, x=x, y=y: int((O.nvfp4_qdq(x, O.nvfp4_group_scale([x])[1]) != y).sum()),
                         x.size))
            per_op.append((op, jobs, x.size))
            continue
        if op.workload == "int4":
            ws = bench.sets["moe_experts"]
            out = bench.outputs["int4"]
            G = out["group"]
            for i in range(0, len(ws.specs), stride):
                x = h16(ws.w[i])
                if op.name.startswith("int4.quantize"):
                    p, s = h8(out["p"][i]), out["s"][i].cpu().numpy()

                    def job(_, x=x, p=p, s=s):
                        op_, os_ = O.int4_quantize(x, G)
                        return int((op_ != p).sum() + (os_.view(np.uint32) != s.view(np.uint32)).sum())
                    jobs.append((None, job, ws.specs[i].numel))
                elif op.name.startswith("int4.dequantize"):   # from the oracle's own codes (untimed)
                    y = h16(out["y"][i])
                    jobs.append((lambda x=x: O.int4_quantize(x, G),
                                 lambda c, y=y: int((O.int4_dequantize(*c, G) != y).sum()), ws.specs[i].numel))
                else:   # QDQ: BF16(fl(code * s)) of the codes of the input, as the dequantized weight
                    y = h16(out["y"][i])
                    jobs.append((None, lambda _, x=x, y=y: int((O.int4_qdq(x, G) != y).sum()), ws.specs[i].numel))
            per_op.append((op, jobs, sum(sp.numel for sp in ws.specs)))
            continue
        if op.workload not in ("fp8train", "fp8train-pow2") or op.name.startswith("requant.amax"):
            continue
        ws = bench.sets["moe"]
        out = bench.outputs[op.workload]
        if op.workload == "fp8train-pow2":   # the oracle's own block-FP8 copy, scales cut to powers of two
            def fp8_of(x):
                q, s = O.fp8blk_quantize(x)
                return q, (s.view(np.uint32) & np.uint32(W.POW2_MASK)).view(np.float32)
        else:
            fp8_of = O.fp8blk_quantize
        if op.name.startswith("requant.fp8blk"):
            for i in range(0, len(ws.specs), stride):
                x, q, s8 = h16(ws.w[i]), h8(out["fq"][i]), out["fs"][i].cpu().numpy()

                def job(src, q=q, s8=s8):
                    oq, os_ = O.fp8blk_requantize_fp8blk(*src)
                    return int((oq != q).sum() + (os_.view(np.uint32) != s8.view(np.uint32)).sum())
                jobs.append((lambda x=x, f=fp8_of: f(x), job, ws.specs[i].numel))
            per_op.append((op, jobs, sum(sp.numel for sp in ws.specs)))
        elif op.name.startswith("requant.mxfp8"):
            for i in out["ex"][::stride]:
                x, q, e = h16(ws.w[i]), h8(out["mq"][i]), h8(out["me"][i])

                def job(src, q=q, e=e):
                    oq, oe = O.fp8blk_requantize_mxfp8(*src)
                    return int((oq != q).sum() + (oe != e).sum())
                jobs.append((lambda x=x, f=fp8_of: f(x), job, ws.specs[i].numel))
            per_op.append((op, jobs, sum(ws.specs[i].numel for i in out["ex"])))
        elif op.name.startswith("requant.nvfp4"):
            groups = {}
            for i, sp in enumerate(ws.specs):
                groups.setdefault(sp.group, []).append(i)
            amax_d, g_d = out["amax"].cpu().numpy(), out["g"].cpu().numpy()
            for gid in sorted(groups)[::stride]:
                idx = groups[gid]
                xs = [h16(ws.w[i]) for i in idx]
                ps, ss = [h8(out["p"][i]) for i in idx], [h8(out["sb"][i]) for i in idx]
                A_d, gg_d = np.float32(amax_d[gid]), np.float32(g_d[gid])

                def job(srcs, ps=ps, ss=ss, A_d=A_d, gg_d=gg_d):
                    A, g, res = O.fp8blk_requantize_nvfp4_group(srcs)
                    bad = int(np.float32(A) != A_d) + int(np.float32(g) != gg_d)
                    for (p, s), pp, sg in zip(res, ps, ss):
                        bad += int((p != pp).sum() + (s != sg).sum())
                    return bad
                jobs.append((lambda xs=xs, f=fp8_of: [f(x) for x in xs], job, sum(ws.specs[i].numel for i in idx)))
            per_op.append((op, jobs, sum(sp.numel for sp in ws.specs)))
    O.default()
    t_all, bad_all, n_all, rows = 0.0, 0, 0, {}
    for op, jobs, op_elems in per_op:
        preps = O.run_parallel(lambda j: j[0]() if j[0] else None, jobs, threads)   # untimed inputs
        t0 = time.perf_counter()
        res = O.run_parallel(lambda jp: jp[0][1](jp[1]), list(zip(jobs, preps)), threads)
        dt = time.perf_counter() - t0
        elems = sum(j[2] for j in jobs)
        bad = int(sum(res))
        t_all, bad_all, n_all = t_all + dt, bad_all + bad, n_all + len(jobs)
        if ".unfused" not in op.name:
            sample = op.bytes * elems / op_elems
            rows[op.name] = {"GB/s": round(sample / dt / GB, 3), "sample_GB": round(sample / GB, 3),
                             "seconds": round(dt, 2), "calls": len(jobs), "mismatches": bad}
    return {"checked": n_all, "parity_mismatches": bad_all, "seconds": round(t_all, 2), "ops": rows}


# --------------------------------------------------------------------------- HBM copy reference

COPY_BYTES = 4 * (1 << 30)


def copy_bandwidth(reps: int = 10) -> float:
    """Device-to-device copy rate (GB/s, read + write) of a plain 4 GiB copy on the
    current stream: the achievable-bandwidth context for the codec figures, and
    the kernel of known traffic used to calibrate the HBM byte counters."""
    import torch
    x = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) / 1e3 / reps
    del x, y
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / sec / GB


def summarize_pmc(path: str) -> None:
    """Per-kernel mean of each counter per dispatch, from rocprofv3 counter CSVs
    found under `path` (grouped by kernel name and grid size)."""
    import csv
    import glob
    import re
    rows = []
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name", "?").replace("(anonymous namespace)::", "").replace("void ", "")
        name = re.sub(r"\(.*", "", name)
        key = (name, r.get("Grid_Size", "?"), r.get("Counter_Name", "?"))
        d = acc.setdefault(key, [0, 0.0, set()])
        d[1] += float(r.get("Counter_Value", 0))
        d[2].add(r.get("Dispatch_Id", len(d[2])))
    print("| kernel | grid size | counter | dispatches | mean per dispatch |")
    print("|---|---|---|---|---|")
    for (name, grid, ctr), (_, tot, disp) in sorted(acc.items()):
        print(f"| {name} | {grid} | {ctr} | {len(disp)} | {tot / max(len(disp), 1):.1f} |")


# --------------------------------------------------------------------------- launch floor

def launch_floor_us(reps: int = 50) -> float:
    """Median time between two events around one launch of the library's
    smallest kernel (one workgroup: the multiplier form of one global scale),
    with the pairs queued back to back behind a long fill so that the GPU, not
    the host, paces them, as the ops of a step are paced: the fixed cost of
    any single launch timed this way, which bounds the small activation ops
    from below."""
    import statistics

    import torch

    import precision_weight_quantization_amd as lpq
    a = torch.full((1,), 2688.0, dtype=torch.float32, device="cuda")
    out = torch.empty_like(a)
    block = torch.empty(1 << 29, dtype=torch.float32, device="cuda")   # 2 GiB
    for _ in range(5):
        lpq.lpq_nvfp4_global_scale(a, out)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for _ in range(4):
        block.fill_(1.0)
    for e0, e1 in ev:
        e0.record()
        lpq.lpq_nvfp4_global_scale(a, out)
        e1.record()
    torch.cuda.synchronize()
    del block
    return round(statistics.median(e0.elapsed_time(e1) for e0, e1 in ev) * 1e3, 2)


# --------------------------------------------------------------------------- widening rows

def time_next_rows(bench, steps: int):
    """Time the widening-row ops (outside the step) and compare fused with unfused."""
    import torch
    ops = bench.next_ops
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in ops]
          for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        for j, op in enumerate(ops):
            ev[k][j][0].record()
            op.run()
            ev[k][j][1].record()
    torch.cuda.synchronize()
    out = {"ops": {}}
    ms = {}
    for j, op in enumerate(ops):
        m = sum(ev[k][j][0].elapsed_time(ev[k][j][1]) for k in range(steps)) / steps
        ms[op.name] = m
        gbs = op.bytes / (m / 1e3) / GB
        out["ops"][op.name] = {"ms": round(m, 3), "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                               "launches": len(op.launches), "algorithmic_bytes": int(op.bytes),
                               "traffic_hbm_bytes_per_launch": load_traffic(op.name)}
        log(f"  {op.name:36s} {m:8.3f} ms  {gbs:8.1f} GB/s  {100 * gbs / HBM_PEAK_GBS:5.1f}% of peak")
    sp = {}
    if "requant.fp8blk[fp8train]" in ms and "requant.fp8blk.unfused[fp8train]" in ms:
        sp["fp8blk"] = round(ms["requant.fp8blk.unfused[fp8train]"] / ms["requant.fp8blk[fp8train]"], 3)
    if "requant.mxfp8[fp8train]" in ms and "requant.mxfp8.unfused[fp8train]" in ms:
        sp["mxfp8"] = round(ms["requant.mxfp8.unfused[fp8train]"] / ms["requant.mxfp8[fp8train]"], 3)
    if all(k in ms for k in ("requant.amax[fp8train]", "requant.nvfp4[fp8train]", "requant.nvfp4.unfused[fp8train]")):
        sp["nvfp4"] = round(ms["requant.nvfp4.unfused[fp8train]"]
                            / (ms["requant.amax[fp8train]"] + ms["requant.nvfp4[fp8train]"]), 3)
    out["fused_speedup_vs_unfused"] = sp
    out["workload"] = ("W4A4 activations 8192x2048: static_minmax observer update, then QDQ under its amax; "
                       "Qwen3-30B-A3B experts (18,432 tensors) quantized to MXFP8 with the OCP floor exponent rule; "
                       "the Qwen3-30B-A3B weights held in block-wise FP8 (128x128 tiles, FP32 scales): the experts + "
                       "48 q/k/v (18,576 tensors) -> block-wise FP8; the 18,432 expert tensors -> MXFP8; the experts "
                       "+ q/k/v (12,336 sibling groups) -> NVFP4 with the model-wide amax pass; unfused = dequantize "
                       "to BF16 in HBM, then quantize; [fp8train-pow2] = the same fused re-quantizations with every tile "
                       "scale cut to the power of two at or below it; the Qwen3-30B-A3B experts (18,432 tensors) -> "
                       "group-wise INT4 (group 128) quantize, dequantize and QDQ")
    log(f"  fused speedup vs unfused: {sp}")
    return out


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--bucket", choices=("sync", "layer", "all"), default="sync")
    ap.add_argument("--workloads", default="dense,moe,nvfp4,dsv3,fp8train,int4")
    ap.add_argument("--cpu-stride", type=int, default=12)
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--layers", type=int, default=0, help="reduced layer/expert count for quick checks (0 = full size)")
    ap.add_argument("--ops", default="", help="regex: time only the matching ops (warmup still runs every op)")
    ap.add_argument("--copy-only", action="store_true", help="only measure the plain HBM copy reference")
    ap.add_argument("--summarize-pmc", default="", help="print a per-kernel summary of rocprofv3 counter CSVs")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the codecs need no cross-GPU exchange on this path "
              "(each GPU would run the same kernels on its own share of the tensors); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads

    torch.cuda.init()
    dev = torch.device("cuda:0")
    if args.copy_only:
        log(f"plain copy: {copy_bandwidth():.1f} GB/s")
        return
    copy_gbs = copy_bandwidth()
    log(f"plain {COPY_BYTES >> 30} GiB device copy: {copy_gbs:.1f} GB/s")
    which = tuple(w for w in args.workloads.split(",") if w)
    log(f"building workloads {which} (bucket={args.bucket}) on {torch.cuda.get_device_name(0)}")
    t0 = time.perf_counter()
    bench = workloads.Bench(which, bucket=args.bucket, device=dev, log=log, scale_layers=args.layers or None)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; "
        f"{torch.cuda.memory_allocated() / GB:.1f} GB allocated; {len(bench.ops)} ops per step")

    for i in range(args.warmup):
        bench.step()
        bench.next_step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    if args.ops:
        import re
        bench.ops = [op for op in bench.ops if re.search(args.ops, op.name)]
        bench.next_ops = [op for op in bench.next_ops if re.search(args.ops, op.name)]
        log(f"timing only: {[op.name for op in bench.ops + bench.next_ops]}")
    nops = len(bench.ops)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nops)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for j, op in enumerate(bench.ops):
            ev[k][j][0].record()
            op.run()
            ev[k][j][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")

    op_ms = [sum(ev[k][j][0].elapsed_time(ev[k][j][1]) for k in range(args.steps)) / args.steps for j in range(nops)]
    ms_per_step = wall * 1e3 / args.steps
    counted = bench.counted_bytes()
    value = counted / (ms_per_step / 1e3) / GB
    per_op = {}
    for op, ms in zip(bench.ops, op_ms):
        gbs = op.bytes / (ms / 1e3) / GB
        per_op[op.name] = {"ms": round(ms, 3), "GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                           "launches": len(op.launches), "algorithmic_GB": round(op.bytes / GB, 3),
                           "algorithmic_bytes": int(op.bytes),
                           "in_metric": op.counted}
        log(f"  {op.name:32s} {ms:8.3f} ms  {gbs:8.1f} GB/s  {100 * gbs / HBM_PEAK_GBS:5.1f}% of peak")

    next_rows = time_next_rows(bench, args.steps) if bench.next_ops else None
    floor_us = launch_floor_us()
    log(f"launch floor (one-workgroup kernel between two events): {floor_us} us")

    roofline = None
    if nops:
        dom = max(range(nops), key=lambda j: op_ms[j])
        dop = bench.ops[dom]
        launches = len(dop.launches)
        per_launch_bytes = dop.bytes / launches
        per_launch_s = op_ms[dom] / 1e3 / launches
        achieved = per_launch_bytes / per_launch_s / GB
        traffic = load_traffic(dop.name)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": dop.name, "bytes_per_launch": int(per_launch_bytes),
                    "avg_launch_us": round(per_launch_s * 1e6, 2)}

    cpu = None
    if not args.no_cpu and not args.ops:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        log(f"cpu baseline: oracle on a 1/{args.cpu_stride} sample with {threads} threads")
        cpu = cpu_baseline(bench, args.cpu_stride, threads)
        log(f"cpu baseline: {cpu['value']} GB/s, {cpu['parity_mismatches']} mismatches vs GPU, {cpu['seconds']} s; "
            f"one thread: {cpu['single_thread']['value']} GB/s ({cpu['single_thread']['sample']}); "
            f"one thread on the single Linear: {cpu['single_thread_linear']['value']} GB/s")
        if next_rows is not None:
            nr = next_rows_parity(bench, NEXT_CPU_STRIDE, threads)
            next_rows["cpu_baseline"] = {
                "kind": "oracle", "cores": threads, "unit": "GB/s",
                "sample": f"every {NEXT_CPU_STRIDE}th tensor (NVFP4: sibling group) of each widening-row op, "
                          "the whole activation for the observer row; the oracle's own block-FP8 copy of the "
                          "weights is formed first, untimed",
                "parity_mismatches": nr["parity_mismatches"], "seconds": nr["seconds"], "ops": nr["ops"]}
            log(f"next rows, oracle: {nr['checked']} calls, {nr['parity_mismatches']} mismatches vs GPU, "
                f"{nr['seconds']} s; " + ", ".join(f"{k} {v['GB/s']} GB/s" for k, v in nr["ops"].items()))

    result = {
        "metric": "quantize+dequant GB/s (bytes in+out) and % of HBM peak, per format, 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "hbm_copy_GBs": round(copy_gbs, 1),
        "config": {
            "workload": "all weight workloads at full size: Qwen3-4B dense (252 tensors) block-FP8 q+dq; "
                        "Qwen3-30B-A3B experts (18,432 tensors) MXFP8 q+dq; the same experts + q/k/v "
                        "(18,576 tensors, 12,336 sibling groups) NVFP4 amax+q+dq+QDQ and W4A4 activation "
                        "QDQ 8192x2048; DeepSeek-V3 MoE layer (768 tensors) block-FP8 q+dq",
            "workloads": list(which),
            "bucket": args.bucket,
            "algorithmic_GB_per_step": round(counted / GB, 3),
        },
        "per_op": per_op,
        "launch_floor_us": floor_us,
        "roofline": roofline,
        "next_rows": next_rows,
        "cpu_baseline": cpu,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
