"""Parity at full size, in the launch configuration bench.py times.

Builds every weight workload at its full size on the device (Qwen3-4B dense,
Qwen3-30B-A3B experts with q/k/v sibling groups, DeepSeek-V3 MoE layer, W4A4
activations, the block-wise FP8 copy of the Qwen3-30B-A3B weights for
re-quantization, and INT4 of its experts), runs each operation exactly as the
benchmark does (grouped
launches per weight-sync bucket), and compares sampled outputs -- every 48th tensor, every
48th NVFP4 sibling group, and the whole activation QDQ -- with the oracle,
bit for bit.  The sampled inputs are copied back from the device; the
generator that produced them is checked against its host twin elsewhere.
"""
import os

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def full_bench():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info()
    if free < 230e9:
        pytest.skip(f"full-size workloads need ~215 GB of device memory, {free / 1e9:.0f} GB free")
    import workloads
    b = workloads.Bench(workloads.WORKLOADS + workloads.NEXT_WORKLOADS, bucket="sync", device="cuda",
                        log=lambda *a: print(*a, flush=True))
    b.step()
    torch.cuda.synchronize()
    yield b
    del b
    torch.cuda.empty_cache()


def test_fullsize_sampled_parity(full_bench):
    import bench
    res = bench.cpu_baseline(full_bench, stride=48, threads=min(16, os.cpu_count() or 1))
    print(res["sample"], flush=True)
    assert res["parity_mismatches"] == 0


def test_fullsize_requant_sampled_parity(full_bench):
    """The widening rows at full size, sampled, against the oracle: fused and unfused
    FP8 re-quantization, floor-rule MXFP8, the observed activation QDQ and
    group-wise INT4 of the Qwen3-30B-A3B experts."""
    import bench
    res = bench.next_rows_parity(full_bench, stride=48, threads=min(16, os.cpu_count() or 1))
    print(res, flush=True)
    assert res["checked"] > 0 and res["parity_mismatches"] == 0


def test_fullsize_group_scales_shared(full_bench):
    """Every member of a sibling group reports the same global scale (one slot per group),
    and every group slot was written."""
    out = full_bench.outputs["nvfp4"]
    g = out["g"].cpu()
    amax = out["amax"].cpu()
    assert g.numel() == out["n_groups"] == 12336
    assert torch.all(amax > 0) and torch.all(g > 0)
    assert torch.equal(g.view(torch.int32), (amax / 2688.0).view(torch.int32))   # bit patterns
