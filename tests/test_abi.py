"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects invalid arguments on the host before anything is enqueued."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lpq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lpq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import precision_weight_quantization_amd as m
    return m


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 19
    raw = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(lib.EXPORTED)


def test_status_strings(lib):
    L = lib.raw()
    for code in range(7):
        assert len(L.lpq_status_string(code)) > 0
    assert L.lpq_version() == 10000
    assert L.lpq_last_hip_error() == 0


P = 1 << 20          # a fake, suitably aligned address: the checks below must fail before any use of it


def test_single_call_validation(lib):
    L = lib.raw()
    assert L.lpq_quantize_mxfp8(None, 4, 32, P, P, None) == 1
    assert L.lpq_quantize_mxfp8(P, 0, 32, P, P, None) == 2
    assert L.lpq_quantize_mxfp8(P, 4, 48, P, P, None) == 2
    assert L.lpq_quantize_mxfp8(P, -1, 32, P, P, None) == 2
    assert L.lpq_quantize_mxfp8(P + 2, 4, 32, P, P, None) == 3
    assert L.lpq_quantize_mxfp8(P, 4, 32, P + 4, P, None) == 3
    assert L.lpq_quantize_mxfp8_floor(P, 4, 48, P, P, None) == 2
    assert L.lpq_quantize_mxfp8_floor(P + 2, 4, 32, P, P, None) == 3
    assert L.lpq_quantize_mxfp8_floor(P, 4, 32, None, P, None) == 1
    assert L.lpq_nvfp4_global_scale_reciprocal(None, 4, P, None) == 1
    assert L.lpq_nvfp4_global_scale_reciprocal(P, 0, P, None) == 2
    assert L.lpq_nvfp4_global_scale_reciprocal(P, 4, P + 2, None) == 3
    assert L.lpq_quantize_nvfp4_ex(P, 4, 32, P, 300, P, P, P, None) == 6     # E4M3 maximum 448 or 256
    assert L.lpq_nvfp4_qdq_ex(P, 4, 32, P, 0, P, None) == 6
    assert L.lpq_nvfp4_qdq_ex(P, 4, 24, P, 256, P, None) == 2
    assert L.lpq_nvfp4_global_scale(None, 4, P, None) == 1
    assert L.lpq_nvfp4_global_scale(P, -1, P, None) == 2
    assert L.lpq_observer_reset(None, None) == 1
    assert L.lpq_observer_reset(P + 2, None) == 3
    assert L.lpq_nvfp4_observe(P, 4, 32, 1, 0.01, None, P, None) == 1
    assert L.lpq_nvfp4_observe(P, 4, 32, 3, 0.01, P, P, None) == 6            # unknown observer
    assert L.lpq_nvfp4_observe(P, 4, 24, 1, 0.01, P, P, None) == 2            # N % 16
    assert L.lpq_nvfp4_observe(P + 8, 4, 32, 1, 0.01, P, P, None) == 3
    # the allocation-free observer refuses the same arguments before touching its device block
    assert L.lpq_nvfp4_observe_noalloc(P, 4, 32, 1, 0.01, None, P, None) == 1
    assert L.lpq_nvfp4_observe_noalloc(P, 4, 32, 1, 0.01, P, None, None) == 1
    assert L.lpq_nvfp4_observe_noalloc(P, 4, 32, -1, 0.01, P, P, None) == 6
    assert L.lpq_nvfp4_observe_noalloc(P, 4, 24, 1, 0.01, P, P, None) == 2
    assert L.lpq_nvfp4_observe_noalloc(P, 0, 32, 1, 0.01, P, P, None) == 2
    assert L.lpq_nvfp4_observe_noalloc(P, 4, 32, 1, 0.01, P + 2, P, None) == 3
    assert L.lpq_nvfp4_observe_noalloc(P + 8, 4, 32, 1, 0.01, P, P, None) == 3
    assert L.lpq_nvfp4_observe_noalloc(P, 1 << 40, 1 << 20, 1, 0.01, P, P, None) == 2   # beyond the grid limit
    assert L.lpq_dequantize_mxfp8(P, P, 4, 33, P, None) == 2
    assert L.lpq_dequantize_mxfp8(P + 4, P, 4, 32, P, None) == 3
    assert L.lpq_quantize_nvfp4(P, 4, 24, P, P, P, P, None) == 2
    assert L.lpq_quantize_nvfp4(P, 4, 32, P, P, P, None, None) == 1
    # amax NULL: the call computes the tensor's own amax into g, so g stays required
    assert L.lpq_quantize_nvfp4(P, 4, 32, None, P, P, None, None) == 1
    assert L.lpq_quantize_nvfp4(P, 4, 24, None, P, P, P, None) == 2
    assert L.lpq_quantize_nvfp4(P, 4, 32, None, P, P, P + 2, None) == 3
    assert L.lpq_quantize_nvfp4_ex(P, 4, 32, None, 256, P, P, None, None) == 1
    assert L.lpq_quantize_nvfp4(P, 4, 32, P + 1, P, P, P, None) == 3
    assert L.lpq_quantize_nvfp4(P + 8, 4, 32, P, P, P, P, None) == 3
    assert L.lpq_quantize_nvfp4(P, 4, 32, P, P + 2, P, P, None) == 3
    assert L.lpq_dequantize_nvfp4(P, P, None, 4, 32, P, None) == 1
    assert L.lpq_dequantize_nvfp4(P, P, P, 4, 32, P + 8, None) == 3
    assert L.lpq_nvfp4_qdq(P, 4, 32, None, P, None) == 6      # amax computed into y: x and y may not overlap
    assert L.lpq_nvfp4_qdq(P, 4, 32, None, P + 240, None) == 6
    assert L.lpq_nvfp4_qdq(P + 240, 4, 32, None, P, None) == 6
    assert L.lpq_nvfp4_qdq_ex(P, 4, 32, None, 448, P, None) == 6
    assert L.lpq_nvfp4_qdq_ex(P, 4, 32, None, 100, P + 4096, None) == 6   # bad maximum before anything else
    assert L.lpq_nvfp4_qdq(P, 4, 32, P, None, None) == 1
    assert L.lpq_nvfp4_amax(P, 4, 32, None, 0, None) == 1
    assert L.lpq_nvfp4_amax(P, 4, 8, P, 0, None) == 2
    assert L.lpq_quantize_fp8blk(P, 0, 5, P, P, None) == 2
    assert L.lpq_quantize_fp8blk(P, 5, 5, P, None, None) == 1
    assert L.lpq_quantize_fp8blk(P + 1, 5, 5, P, P, None) == 3
    assert L.lpq_quantize_fp8blk(P, 5, 5, P, P + 2, None) == 3
    assert L.lpq_dequantize_fp8blk(P, P, 5, 5, None, None) == 1
    assert L.lpq_last_hip_error() == 0


def _table(lib, rows):
    t = (lib.lpq_tensor * len(rows))()
    for i, (src, dst, scale, M, N, group, reserved) in enumerate(rows):
        t[i].src, t[i].dst, t[i].scale = src, dst, scale
        t[i].rows, t[i].cols, t[i].group, t[i].reserved = M, N, group, reserved
    return t


def test_grouped_validation(lib):
    L = lib.raw()
    good = (P, P, P, 8, 64, 0, 0)
    t = _table(lib, [good, (P, P, P, 8, 64, 3, 0)])
    for valid in (1, 0):   # amax_valid 0 (the call fills group_amax): the same checks, before anything runs
        assert L.lpq_quantize_nvfp4_grouped(t, P, 2, P, 2, valid, P, None) == 4     # group 3 >= n_groups 2
        assert L.lpq_quantize_nvfp4_grouped(t, P, 2, P, 4, valid, None, None) == 1
        assert L.lpq_quantize_nvfp4_grouped(t, P, 2, None, 4, valid, P, None) == 1
        assert L.lpq_quantize_nvfp4_grouped(t, P, 2, P + 2, 4, valid, P, None) == 3
        assert L.lpq_quantize_nvfp4_grouped(t, P, 0, P, 4, valid, P, None) == 2
        assert L.lpq_quantize_nvfp4_grouped(None, P, 2, P, 4, valid, P, None) == 1
        assert L.lpq_quantize_nvfp4_grouped(t, None, 2, P, 4, valid, P, None) == 1
        assert L.lpq_quantize_nvfp4_grouped(t, P + 4, 2, P, 4, valid, P, None) == 3
        assert L.lpq_nvfp4_qdq_grouped(t, P, 2, P, 2, valid, None) == 4
        assert L.lpq_nvfp4_qdq_grouped(t, P, 2, P, 0, valid, None) == 2
        assert L.lpq_nvfp4_qdq_grouped(t, P, 2, None, 4, valid, None) == 1
        assert L.lpq_nvfp4_qdq_grouped(t, P, 2, P + 2, 4, valid, None) == 3
        assert L.lpq_quantize_nvfp4_grouped_ex(t, P, 2, P, 4, valid, 300, P, None) == 6
        assert L.lpq_quantize_nvfp4_grouped_ex(t, P, 2, P, 2, valid, 256, P, None) == 4
        assert L.lpq_nvfp4_qdq_grouped_ex(t, P, 2, P, 4, valid, 100, None) == 6
        assert L.lpq_nvfp4_qdq_grouped_ex(t, P, 2, P, 2, valid, 256, None) == 4
    t2 = _table(lib, [good, (P, P, P, 8, 63, 0, 0)])
    assert L.lpq_quantize_mxfp8_grouped(t2, P, 2, None) == 2
    assert L.lpq_quantize_mxfp8_floor_grouped(t2, P, 2, None) == 2
    t3 = _table(lib, [good, (P, P, P, 8, 64, 0, 7)])
    assert L.lpq_quantize_mxfp8_grouped(t3, P, 2, None) == 6
    t4 = _table(lib, [good, (0, P, P, 8, 64, 0, 0)])
    assert L.lpq_quantize_fp8blk_grouped(t4, P, 2, None) == 1
    assert L.lpq_nvfp4_amax_grouped(t, P, 2, P, 2, 0, None) == 4
    assert L.lpq_nvfp4_amax_grouped(t, P, 2, None, 4, 0, None) == 1
    assert L.lpq_dequantize_nvfp4_grouped(t, P, 2, None, 4, None) == 1
    assert L.lpq_last_hip_error() == 0


def test_int4_validation(lib):
    L = lib.raw()
    assert L.lpq_quantize_int4(P, 4, 128, 64, P, P, None) == 6          # group 32 or 128 only
    assert L.lpq_quantize_int4(P, 4, 128, 0, P, P, None) == 6
    assert L.lpq_quantize_int4(None, 4, 128, 128, P, P, None) == 1
    assert L.lpq_quantize_int4(P, 4, 128, 128, None, P, None) == 1
    assert L.lpq_quantize_int4(P, 4, 128, 128, P, None, None) == 1
    assert L.lpq_quantize_int4(P, 4, 96, 128, P, P, None) == 2          # N % group
    assert L.lpq_quantize_int4(P, 0, 128, 128, P, P, None) == 2
    assert L.lpq_quantize_int4(P + 8, 4, 128, 128, P, P, None) == 3      # BF16 input needs 16 bytes
    assert L.lpq_quantize_int4(P, 4, 128, 128, P + 2, P, None) == 3      # packed needs 4
    assert L.lpq_quantize_int4(P, 4, 128, 128, P, P + 2, None) == 3      # FP32 scales
    assert L.lpq_dequantize_int4(P, P, 4, 96, 32, None, None) == 1
    assert L.lpq_dequantize_int4(P, None, 4, 96, 32, P, None) == 1
    assert L.lpq_dequantize_int4(P, P, 4, 80, 32, P, None) == 2
    assert L.lpq_dequantize_int4(P, P, 4, 96, 32, P + 8, None) == 3      # BF16 output needs 16 bytes
    assert L.lpq_dequantize_int4(P, P, 4, 96, 16, P, None) == 6
    assert L.lpq_int4_qdq(P, 4, 96, 128, P, None) == 2
    assert L.lpq_int4_qdq(P, 4, 96, 32, None, None) == 1
    assert L.lpq_int4_qdq(P, 4, 96, 32, P + 8, None) == 3
    assert L.lpq_int4_qdq(P, 4, 96, 33, P, None) == 6
    good = (P, P, P, 8, 256, 0, 0)
    t = _table(lib, [good, (P, P, P, 8, 160, 0, 0)])                      # 160 % 128 != 0, 160 % 32 == 0
    assert L.lpq_quantize_int4_grouped(t, P, 2, 128, None) == 2
    assert L.lpq_dequantize_int4_grouped(t, P, 2, 128, None) == 2
    assert L.lpq_int4_qdq_grouped(t, P, 2, 128, None) == 2
    assert L.lpq_quantize_int4_grouped(t, P, 2, 64, None) == 6
    assert L.lpq_quantize_int4_grouped(None, P, 2, 32, None) == 1
    assert L.lpq_quantize_int4_grouped(t, P, 0, 32, None) == 2
    t2 = _table(lib, [good, (P, P, P, 8, 256, 0, 5)])                     # reserved != 0
    assert L.lpq_int4_qdq_grouped(t2, P, 2, 32, None) == 6
    assert L.lpq_last_hip_error() == 0


def test_requant_validation(lib):
    L = lib.raw()
    assert L.lpq_requantize_fp8blk(None, P, 4, 5, P, P, None) == 1
    assert L.lpq_requantize_fp8blk(P, P, 4, 5, P, None, None) == 1
    assert L.lpq_requantize_fp8blk(P, P, 0, 5, P, P, None) == 2
    assert L.lpq_requantize_fp8blk(P, P + 2, 4, 5, P, P, None) == 3          # FP32 scales
    assert L.lpq_requantize_fp8blk(P, P, 4, 5, P, P + 1, None) == 3
    assert L.lpq_requantize_fp8blk_mxfp8(None, P, 4, 32, P, P, None) == 1
    assert L.lpq_requantize_fp8blk_mxfp8(P, None, 4, 32, P, P, None) == 1
    assert L.lpq_requantize_fp8blk_mxfp8(P, P, 4, 32, None, P, None) == 1
    assert L.lpq_requantize_fp8blk_mxfp8(P, P, 4, 32, P, None, None) == 1
    assert L.lpq_requantize_fp8blk_mxfp8(P, P, 4, 48, P, P, None) == 2       # N % 32
    assert L.lpq_requantize_fp8blk_mxfp8(P, P, 0, 32, P, P, None) == 2
    assert L.lpq_requantize_fp8blk_mxfp8(P + 8, P, 4, 32, P, P, None) == 3   # codes need 16 bytes
    assert L.lpq_requantize_fp8blk_mxfp8(P, P + 2, 4, 32, P, P, None) == 3   # FP32 scales
    assert L.lpq_requantize_fp8blk_mxfp8(P, P, 4, 32, P + 8, P, None) == 3
    assert L.lpq_requantize_fp8blk_mxfp8(P, P, 1 << 31, 32, P, P, None) == 2  # flat targets: M < 2^31
    assert L.lpq_fp8blk_amax(P, P, 4, 32, None, 0, None) == 1
    assert L.lpq_fp8blk_amax(P, P, 4, 24, P, 0, None) == 2                   # N % 16
    assert L.lpq_fp8blk_amax(P, P, 4, 32, P + 2, 0, None) == 3
    assert L.lpq_requantize_fp8blk_nvfp4(P, P, 4, 32, None, P, P, P, None) == 1
    assert L.lpq_requantize_fp8blk_nvfp4(P, P, 4, 32, P, P, P, None, None) == 1
    assert L.lpq_requantize_fp8blk_nvfp4(P, P, 4, 32, P, P + 4, P, P, None) == 3   # packed needs 8 bytes
    assert L.lpq_requantize_fp8blk_nvfp4(P, P, 4, 40, P, P, P, P, None) == 2
    t = (lib.lpq_requant_tensor * 2)()
    for i in range(2):
        t[i].src = t[i].src_scale = t[i].dst = t[i].dst_scale = P
        t[i].rows, t[i].cols, t[i].group, t[i].reserved = 8, 64, i, 0
    assert L.lpq_requantize_fp8blk_nvfp4_grouped(t, P, 2, P, 1, P, None) == 4    # group 1 >= n_groups 1
    assert L.lpq_fp8blk_amax_grouped(t, P, 2, P, 1, 0, None) == 4
    assert L.lpq_fp8blk_amax_grouped(t, P, 2, None, 2, 0, None) == 1
    assert L.lpq_requantize_fp8blk_nvfp4_grouped(t, P, 2, P, 2, None, None) == 1
    assert L.lpq_requantize_fp8blk_mxfp8_grouped(t, P + 4, 2, None) == 3
    assert L.lpq_requantize_fp8blk_mxfp8_grouped(t, P, 0, None) == 2
    t[1].reserved = 1
    assert L.lpq_requantize_fp8blk_mxfp8_grouped(t, P, 2, None) == 6
    t[1].reserved, t[1].src_scale = 0, 0
    assert L.lpq_requantize_fp8blk_mxfp8_grouped(t, P, 2, None) == 1
    assert L.lpq_last_hip_error() == 0


def test_product_path_has_no_oracle_or_fallback():
    """The package neither imports the oracle nor carries a CPU code path."""
    pkg = os.path.join(ROOT, "precision_weight_quantization_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


# --------------------------------------------------------------------------- the Python binding's checks

class _FakeDevice(torch.Tensor):
    """A host tensor that reports itself as a device tensor on ``FAKE_DEVICE``:
    enough to drive the binding's argument checks without a GPU."""

    FAKE_DEVICE = torch.device("cuda", 0)

    @property
    def is_cuda(self):
        return True

    @property
    def device(self):
        return self.FAKE_DEVICE


def fake(t):
    return torch.Tensor._make_subclass(_FakeDevice, t)


class _OtherDevice(_FakeDevice):
    FAKE_DEVICE = torch.device("cuda", 1)


class _Recorder:
    """Stands in for the C library: records any call (none may happen)."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def recorder(lib, monkeypatch):
    r = _Recorder()
    monkeypatch.setattr(lib, "_L", r)
    return r


def test_binding_refuses_bad_tensors_before_any_call(lib, recorder):
    bf = lambda *shape: fake(torch.zeros(shape, dtype=torch.bfloat16))
    u8 = lambda *shape: fake(torch.zeros(shape, dtype=torch.uint8))
    f32 = lambda *shape: fake(torch.zeros(shape, dtype=torch.float32))
    w = bf(4, 64)
    cases = [
        (ValueError, lambda: lib.lpq_quantize_mxfp8(torch.zeros(4, 64, dtype=torch.bfloat16))),    # host tensor
        (TypeError, lambda: lib.lpq_quantize_mxfp8(fake(torch.zeros(4, 64)))),                     # FP32, not BF16
        (ValueError, lambda: lib.lpq_quantize_mxfp8(bf(4, 64, 1))),                                 # not 2-D
        (ValueError, lambda: lib.lpq_quantize_mxfp8(fake(torch.zeros(64, 4, dtype=torch.bfloat16).t()))),
        (ValueError, lambda: lib.lpq_quantize_mxfp8(w, q=u8(4, 63))),                               # too small
        (ValueError, lambda: lib.lpq_quantize_mxfp8(w, e=u8(4, 1))),
        (ValueError, lambda: lib.lpq_quantize_mxfp8(w, q=u8(64, 4).t())),                           # strided out
        (TypeError, lambda: lib.lpq_quantize_fp8blk(w, s=fake(torch.zeros(1, 1, dtype=torch.float16)))),
        (ValueError, lambda: lib.lpq_dequantize_fp8blk(u8(4, 64), f32(1, 1), y=bf(4, 63))),
        (ValueError, lambda: lib.lpq_dequantize_fp8blk(u8(200, 64), f32(1, 1))),                    # 2 tiles
        (ValueError, lambda: lib.lpq_dequantize_mxfp8(u8(4, 64), u8(4, 1))),
        (ValueError, lambda: lib.lpq_quantize_nvfp4(w, amax=torch.zeros(1))),                       # host amax
        (ValueError, lambda: lib.lpq_quantize_nvfp4(w, amax=torch.Tensor._make_subclass(_OtherDevice,
                                                                                         torch.zeros(1)))),
        (TypeError, lambda: lib.lpq_quantize_nvfp4(w, amax=fake(torch.zeros(1, dtype=torch.float64)))),
        (ValueError, lambda: lib.lpq_quantize_nvfp4(w, p=u8(4, 31))),
        (ValueError, lambda: lib.lpq_quantize_nvfp4(w, g=f32(0))),
        (ValueError, lambda: lib.lpq_dequantize_nvfp4(u8(4, 32), u8(4, 3), f32(1))),
        (ValueError, lambda: lib.lpq_nvfp4_qdq(w, f32(1), y=bf(4, 32))),
        (ValueError, lambda: lib.lpq_quantize_int4(w, 32, s=f32(4, 1))),
        (ValueError, lambda: lib.lpq_dequantize_int4(u8(4, 32), f32(4, 1), 32)),
        (ValueError, lambda: lib.lpq_requantize_fp8blk_nvfp4(u8(4, 64), f32(1, 1), f32(1), sb=u8(4, 3))),
        (ValueError, lambda: lib.lpq_nvfp4_observe(w, f32(lib.OBSERVER_STATE_FLOATS - 1))),         # state too short
        (ValueError, lambda: lib.lpq_nvfp4_observe_noalloc(w, f32(2))),                            # 3 words needed
        (ValueError, lambda: lib.lpq_nvfp4_observe_noalloc(w, torch.zeros(3))),                    # host state
        (ValueError, lambda: lib.lpq_nvfp4_global_scale(f32(4), out=f32(3))),
    ]
    for exc, call in cases:
        with pytest.raises(exc):
            call()
    assert recorder.calls == []


def test_tensor_table_checks(lib, recorder):
    with pytest.raises(ValueError):   # a host tensor in an entry: refused before the table is copied anywhere
        lib.TensorTable([(fake(torch.zeros(4, 64, dtype=torch.bfloat16)), torch.zeros(4, 64, dtype=torch.uint8),
                          None, 4, 64, 0)])
    with pytest.raises(ValueError):
        lib.TensorTable([])
    # the per-operation size check, on a table whose device copy is skipped
    t = lib.TensorTable.__new__(lib.TensorTable)
    src = fake(torch.zeros(4, 64, dtype=torch.bfloat16))
    t.host = (lib.lpq_tensor * 1)()
    t.host[0].rows, t.host[0].cols = 4, 64
    t.keep = [(src, fake(torch.zeros(4 * 32 - 1, dtype=torch.uint8)), fake(torch.zeros(16, dtype=torch.uint8)))]
    t._checked = set()
    with pytest.raises(ValueError):
        t.check("nvfp4_q")           # packed output one byte short
    t.check("nvfp4_amax")            # the amax pass reads src only
    t.keep = [(src, None, None)]
    with pytest.raises(ValueError):
        t.check("nvfp4_qdq")         # QDQ needs dst
    assert recorder.calls == []


def test_header_constants_match_binding(lib):
    """The binding's copies of the header's constants (status codes, observer
    kinds and the observer state size) are the header's values."""
    import re
    text = open(os.path.join(ROOT, "include", "lpq.h")).read()
    defs = {k: int(v) for k, v in re.findall(r"#define (LPQ_\w+) (\d+)", text)}
    assert defs["LPQ_OBSERVER_STATE_FLOATS"] == lib.OBSERVER_STATE_FLOATS
    assert {k: defs["LPQ_OBSERVER_" + k.upper()] for k in lib.OBSERVERS} == lib.OBSERVERS
    enum = dict((k, int(v)) for k, v in re.findall(r"(LPQ_(?:OK|ERR_\w+)) = (\d+)", text))
    assert enum["LPQ_OK"] == lib.LPQ_OK
    assert lib.STATUS_NAMES == {v: k for k, v in enum.items()}
