"""Python binding of liblpq.so, the gfx950 low-precision weight codec library.

Argument marshalling only: every step of the codecs runs in the HIP kernels
behind the C ABI (include/lpq.h).  PyTorch supplies device memory and the
current stream.  The functions carry the C names; each accepts CUDA (HIP)
tensors, allocates any output that is not passed in, launches on the current
stream and returns the outputs.  BF16 data is a ``torch.bfloat16`` tensor (or
its ``int16``/``uint16`` bit view), E4M3 codes come back as
``torch.float8_e4m3fn``, scale bytes and packed FP4 as ``torch.uint8``.

If the library has not been built the import fails: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# LPQ_LIBRARY may name another build of the same library (e.g. one compiled
# with different launch parameters); the default is the in-tree build.
LIB_PATH = os.environ.get("LPQ_LIBRARY") or os.path.join(_PKG, "liblpq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -c \"import __graft_entry__ as g; g.build()\"`")

_L = ctypes.CDLL(LIB_PATH)

LPQ_OK = 0
STATUS_NAMES = {0: "LPQ_OK", 1: "LPQ_ERR_NULL", 2: "LPQ_ERR_SHAPE", 3: "LPQ_ERR_ALIGN",
                4: "LPQ_ERR_GROUP", 5: "LPQ_ERR_HIP", 6: "LPQ_ERR_ARG"}


class LpqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _L.lpq_status_string(status).decode()
        if status == 5:
            msg += f" (hipError {_L.lpq_last_hip_error()})"
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


class lpq_tensor(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("group", ctypes.c_int32), ("reserved", ctypes.c_int32)]


assert ctypes.sizeof(lpq_tensor) == 48


class lpq_requant_tensor(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("src_scale", ctypes.c_void_p), ("dst", ctypes.c_void_p),
                ("dst_scale", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("group", ctypes.c_int32), ("reserved", ctypes.c_int32)]


assert ctypes.sizeof(lpq_requant_tensor) == 56

_vp, _i64, _i32, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
_tp = ctypes.POINTER(lpq_tensor)
_rp = ctypes.POINTER(lpq_requant_tensor)
_SIG = {
    "lpq_status_string": (ctypes.c_char_p, [_int]),
    "lpq_last_hip_error": (_int, []),
    "lpq_version": (_int, []),
    "lpq_quantize_fp8blk": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "lpq_dequantize_fp8blk": (_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "lpq_quantize_mxfp8": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "lpq_dequantize_mxfp8": (_int, [_vp, _vp, _i64, _i64, _vp, _vp]),
    "lpq_quantize_mxfp8_floor": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "lpq_quantize_mxfp8_floor_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_nvfp4_global_scale_reciprocal": (_int, [_vp, _i32, _vp, _vp]),
    "lpq_nvfp4_global_scale": (_int, [_vp, _i32, _vp, _vp]),
    "lpq_quantize_nvfp4_ex": (_int, [_vp, _i64, _i64, _vp, _int, _vp, _vp, _vp, _vp]),
    "lpq_nvfp4_qdq_ex": (_int, [_vp, _i64, _i64, _vp, _int, _vp, _vp]),
    "lpq_quantize_nvfp4_grouped_ex": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _vp, _vp]),
    "lpq_nvfp4_qdq_grouped_ex": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _vp]),
    "lpq_observer_reset": (_int, [_vp, _vp]),
    "lpq_nvfp4_observe": (_int, [_vp, _i64, _i64, _int, ctypes.c_float, _vp, _vp, _vp]),
    "lpq_nvfp4_amax": (_int, [_vp, _i64, _i64, _vp, _int, _vp]),
    "lpq_quantize_nvfp4": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "lpq_dequantize_nvfp4": (_int, [_vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "lpq_nvfp4_qdq": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "lpq_quantize_fp8blk_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_dequantize_fp8blk_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_quantize_mxfp8_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_dequantize_mxfp8_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_nvfp4_amax_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _vp]),
    "lpq_quantize_nvfp4_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _vp, _vp]),
    "lpq_dequantize_nvfp4_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _vp]),
    "lpq_nvfp4_qdq_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _vp]),
    "lpq_requantize_fp8blk": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "lpq_requantize_fp8blk_grouped": (_int, [_rp, _vp, _i32, _vp]),
    "lpq_requantize_fp8blk_mxfp8": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp]),
    "lpq_fp8blk_amax": (_int, [_vp, _vp, _i64, _i64, _vp, _int, _vp]),
    "lpq_requantize_fp8blk_nvfp4": (_int, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "lpq_requantize_fp8blk_mxfp8_grouped": (_int, [_rp, _vp, _i32, _vp]),
    "lpq_fp8blk_amax_grouped": (_int, [_rp, _vp, _i32, _vp, _i32, _int, _vp]),
    "lpq_requantize_fp8blk_nvfp4_grouped": (_int, [_rp, _vp, _i32, _vp, _i32, _vp, _vp]),
    "lpq_quantize_int4": (_int, [_vp, _i64, _i64, _i32, _vp, _vp, _vp]),
    "lpq_dequantize_int4": (_int, [_vp, _vp, _i64, _i64, _i32, _vp, _vp]),
    "lpq_int4_qdq": (_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "lpq_quantize_int4_grouped": (_int, [_tp, _vp, _i32, _i32, _vp]),
    "lpq_dequantize_int4_grouped": (_int, [_tp, _vp, _i32, _i32, _vp]),
    "lpq_int4_qdq_grouped": (_int, [_tp, _vp, _i32, _i32, _vp]),
}
for _name, (_res, _args) in _SIG.items():
    _fn = getattr(_L, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = sorted(k for k in _SIG)


def _check(status: int, where: str) -> None:
    if status != LPQ_OK:
        raise LpqError(status, where)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _bf16_in(x: torch.Tensor, name: str) -> torch.Tensor:
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D [M, N]")
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (or its 16-bit view), got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return x.contiguous()


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


# --------------------------------------------------------------------------- block-wise FP8

def fp8blk_scale_shape(M: int, N: int):
    return ((M + 127) // 128, (N + 127) // 128)


def lpq_quantize_fp8blk(w, q=None, s=None, stream=None):
    """BF16 [M,N] -> (codes [M,N] float8_e4m3fn, FP32 tile scales [ceil(M/128), ceil(N/128)])."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    q = _empty((M, N), torch.float8_e4m3fn, w) if q is None else q
    s = _empty(fp8blk_scale_shape(M, N), torch.float32, w) if s is None else s
    _check(_L.lpq_quantize_fp8blk(w.data_ptr(), M, N, q.data_ptr(), s.data_ptr(), _stream(stream)),
           "lpq_quantize_fp8blk")
    return q, s


def lpq_dequantize_fp8blk(q, s, y=None, stream=None):
    M, N = q.shape
    y = _empty((M, N), torch.bfloat16, q) if y is None else y
    _check(_L.lpq_dequantize_fp8blk(q.data_ptr(), s.data_ptr(), M, N, y.data_ptr(), _stream(stream)),
           "lpq_dequantize_fp8blk")
    return y


# --------------------------------------------------------------------------- MXFP8

def lpq_quantize_mxfp8(w, q=None, e=None, stream=None):
    """BF16 [M,N] (N % 32 == 0) -> (codes [M,N] float8_e4m3fn, UE8M0 bytes [M,N/32] uint8)."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    q = _empty((M, N), torch.float8_e4m3fn, w) if q is None else q
    e = _empty((M, max(N // 32, 1)), torch.uint8, w) if e is None else e
    _check(_L.lpq_quantize_mxfp8(w.data_ptr(), M, N, q.data_ptr(), e.data_ptr(), _stream(stream)),
           "lpq_quantize_mxfp8")
    return q, e


def lpq_quantize_mxfp8_floor(w, q=None, e=None, stream=None):
    """As lpq_quantize_mxfp8, with the OCP MX floor exponent rule (saturating)."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    q = _empty((M, N), torch.float8_e4m3fn, w) if q is None else q
    e = _empty((M, max(N // 32, 1)), torch.uint8, w) if e is None else e
    _check(_L.lpq_quantize_mxfp8_floor(w.data_ptr(), M, N, q.data_ptr(), e.data_ptr(), _stream(stream)),
           "lpq_quantize_mxfp8_floor")
    return q, e


def lpq_dequantize_mxfp8(q, e, y=None, stream=None):
    M, N = q.shape
    y = _empty((M, N), torch.bfloat16, q) if y is None else y
    _check(_L.lpq_dequantize_mxfp8(q.data_ptr(), e.data_ptr(), M, N, y.data_ptr(), _stream(stream)),
           "lpq_dequantize_mxfp8")
    return y


# --------------------------------------------------------------------------- NVFP4

def lpq_nvfp4_amax(w, amax=None, accumulate=False, stream=None):
    """max |w| into a 1-element FP32 device tensor (max-accumulated when accumulate)."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    amax = _empty((1,), torch.float32, w) if amax is None else amax
    _check(_L.lpq_nvfp4_amax(w.data_ptr(), M, N, amax.data_ptr(), int(bool(accumulate)), _stream(stream)),
           "lpq_nvfp4_amax")
    return amax


def lpq_quantize_nvfp4_ex(w, amax, e4m3_max=448, p=None, s=None, g=None, stream=None):
    """lpq_quantize_nvfp4 with the global scale fl(A / (6 * e4m3_max)), e4m3_max 448 or 256."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    p = _empty((M, max(N // 2, 1)), torch.uint8, w) if p is None else p
    s = _empty((M, max(N // 16, 1)), torch.float8_e4m3fn, w) if s is None else s
    g = _empty((1,), torch.float32, w) if g is None else g
    _check(_L.lpq_quantize_nvfp4_ex(w.data_ptr(), M, N, amax.data_ptr(), int(e4m3_max), p.data_ptr(), s.data_ptr(),
                                    g.data_ptr(), _stream(stream)), "lpq_quantize_nvfp4_ex")
    return p, s, g


def lpq_nvfp4_qdq_ex(x, amax, e4m3_max=448, y=None, stream=None):
    x = _bf16_in(x, "x")
    M, N = x.shape
    y = _empty((M, N), torch.bfloat16, x) if y is None else y
    _check(_L.lpq_nvfp4_qdq_ex(x.data_ptr(), M, N, amax.data_ptr(), int(e4m3_max), y.data_ptr(), _stream(stream)),
           "lpq_nvfp4_qdq_ex")
    return y


def lpq_quantize_nvfp4(w, amax, p=None, s=None, g=None, stream=None):
    """BF16 [M,N] (N % 16 == 0) with group amax (1-element FP32 device tensor) ->
    (packed [M,N/2] uint8, E4M3 block scales [M,N/16] float8_e4m3fn, global scale [1] FP32)."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    p = _empty((M, max(N // 2, 1)), torch.uint8, w) if p is None else p
    s = _empty((M, max(N // 16, 1)), torch.float8_e4m3fn, w) if s is None else s
    g = _empty((1,), torch.float32, w) if g is None else g
    _check(_L.lpq_quantize_nvfp4(w.data_ptr(), M, N, amax.data_ptr(), p.data_ptr(), s.data_ptr(), g.data_ptr(),
                                 _stream(stream)), "lpq_quantize_nvfp4")
    return p, s, g


def lpq_nvfp4_global_scale_reciprocal(group_amax, out=None, stream=None):
    """fl(2688 / A) per group (the reciprocal export form of the global scale)."""
    out = torch.empty_like(group_amax) if out is None else out
    _check(_L.lpq_nvfp4_global_scale_reciprocal(group_amax.data_ptr(), group_amax.numel(), out.data_ptr(),
                                                _stream(stream)), "lpq_nvfp4_global_scale_reciprocal")
    return out


def lpq_nvfp4_global_scale(amax, out=None, stream=None):
    """fl(A / 2688) per entry (the multiplier form of a global scale)."""
    out = torch.empty_like(amax) if out is None else out
    _check(_L.lpq_nvfp4_global_scale(amax.data_ptr(), amax.numel(), out.data_ptr(), _stream(stream)),
           "lpq_nvfp4_global_scale")
    return out


# W4A4 activation observers (the C constants of the same names)
OBSERVERS = {"memoryless_minmax": 0, "static_minmax": 1, "minmax": 2}
OBSERVER_STATE_FLOATS = 8


def lpq_observer_reset(state=None, device=None, stream=None):
    """A reset observer state (8 FP32 words on the device; allocated when not given)."""
    if state is None:
        state = torch.empty(OBSERVER_STATE_FLOATS, dtype=torch.float32, device=device or "cuda")
    _check(_L.lpq_observer_reset(state.data_ptr(), _stream(stream)), "lpq_observer_reset")
    return state


def lpq_nvfp4_observe(x, state, observer="static_minmax", averaging_constant=0.01, amax=None, stream=None):
    """Update the observer state with the BF16 batch x; returns the activation amax (1 FP32, device)."""
    x = _bf16_in(x, "x")
    M, N = x.shape
    amax = _empty((1,), torch.float32, x) if amax is None else amax
    kind = OBSERVERS[observer] if isinstance(observer, str) else int(observer)
    _check(_L.lpq_nvfp4_observe(x.data_ptr(), M, N, kind, float(averaging_constant), state.data_ptr(),
                                amax.data_ptr(), _stream(stream)), "lpq_nvfp4_observe")
    return amax


def lpq_dequantize_nvfp4(p, s, g, y=None, stream=None):
    M, N = p.shape[0], p.shape[1] * 2
    y = _empty((M, N), torch.bfloat16, p) if y is None else y
    _check(_L.lpq_dequantize_nvfp4(p.data_ptr(), s.data_ptr(), g.data_ptr(), M, N, y.data_ptr(), _stream(stream)),
           "lpq_dequantize_nvfp4")
    return y


def lpq_nvfp4_qdq(x, amax, y=None, stream=None):
    """NVFP4 fake quantization of BF16 [M,N] under the group amax; returns BF16 [M,N]."""
    x = _bf16_in(x, "x")
    M, N = x.shape
    y = _empty((M, N), torch.bfloat16, x) if y is None else y
    _check(_L.lpq_nvfp4_qdq(x.data_ptr(), M, N, amax.data_ptr(), y.data_ptr(), _stream(stream)), "lpq_nvfp4_qdq")
    return y


# --------------------------------------------------------------------------- INT4, group-wise

INT4_GROUPS = (32, 128)


def lpq_quantize_int4(w, group=128, p=None, s=None, stream=None):
    """BF16 [M,N] (N % group == 0) -> (packed two's-complement nibbles [M,N/2] uint8,
    FP32 group scales [M,N/group])."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    g = max(int(group), 1)
    p = _empty((M, max(N // 2, 1)), torch.uint8, w) if p is None else p
    s = _empty((M, max(N // g, 1)), torch.float32, w) if s is None else s
    _check(_L.lpq_quantize_int4(w.data_ptr(), M, N, int(group), p.data_ptr(), s.data_ptr(), _stream(stream)),
           "lpq_quantize_int4")
    return p, s


def lpq_dequantize_int4(p, s, group=128, y=None, stream=None):
    M, N = p.shape[0], p.shape[1] * 2
    y = _empty((M, N), torch.bfloat16, p) if y is None else y
    _check(_L.lpq_dequantize_int4(p.data_ptr(), s.data_ptr(), M, N, int(group), y.data_ptr(), _stream(stream)),
           "lpq_dequantize_int4")
    return y


def lpq_int4_qdq(x, group=128, y=None, stream=None):
    """INT4 fake quantization (the straight-through estimator's forward pass) of BF16 [M,N]."""
    x = _bf16_in(x, "x")
    M, N = x.shape
    y = _empty((M, N), torch.bfloat16, x) if y is None else y
    _check(_L.lpq_int4_qdq(x.data_ptr(), M, N, int(group), y.data_ptr(), _stream(stream)), "lpq_int4_qdq")
    return y


def lpq_quantize_int4_grouped(table, group=128, stream=None):
    _check(_L.lpq_quantize_int4_grouped(*table.args(), int(group), _stream(stream)), "lpq_quantize_int4_grouped")


def lpq_dequantize_int4_grouped(table, group=128, stream=None):
    _check(_L.lpq_dequantize_int4_grouped(*table.args(), int(group), _stream(stream)), "lpq_dequantize_int4_grouped")


def lpq_int4_qdq_grouped(table, group=128, stream=None):
    _check(_L.lpq_int4_qdq_grouped(*table.args(), int(group), _stream(stream)), "lpq_int4_qdq_grouped")


# --------------------------------------------------------------------------- FP8 re-quantization

def _codes_in(q, name: str):
    if q.dim() != 2:
        raise ValueError(f"{name} must be 2-D [M, N]")
    if q.element_size() != 1:
        raise TypeError(f"{name} must hold 1-byte E4M3 codes, got {q.dtype}")
    if not q.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return q.contiguous()


def lpq_requantize_fp8blk(q, s, q_out=None, s_out=None, stream=None):
    """Block-wise FP8 (codes [M,N], FP32 tile scales) -> block-wise FP8 of the dequantized
    BF16 values (codes [M,N] float8_e4m3fn, new FP32 tile scales), in one pass."""
    q = _codes_in(q, "q")
    M, N = q.shape
    q_out = _empty((M, N), torch.float8_e4m3fn, q) if q_out is None else q_out
    s_out = _empty(fp8blk_scale_shape(M, N), torch.float32, q) if s_out is None else s_out
    _check(_L.lpq_requantize_fp8blk(q.data_ptr(), s.data_ptr(), M, N, q_out.data_ptr(), s_out.data_ptr(),
                                    _stream(stream)), "lpq_requantize_fp8blk")
    return q_out, s_out


def lpq_requantize_fp8blk_mxfp8(q, s, q_out=None, e_out=None, stream=None):
    """Block-wise FP8 (codes [M,N], FP32 tile scales) -> MXFP8 (codes [M,N] float8_e4m3fn,
    UE8M0 bytes [M,N/32] uint8) of the dequantized BF16 values, in one pass."""
    q = _codes_in(q, "q")
    M, N = q.shape
    q_out = _empty((M, N), torch.float8_e4m3fn, q) if q_out is None else q_out
    e_out = _empty((M, max(N // 32, 1)), torch.uint8, q) if e_out is None else e_out
    _check(_L.lpq_requantize_fp8blk_mxfp8(q.data_ptr(), s.data_ptr(), M, N, q_out.data_ptr(), e_out.data_ptr(),
                                          _stream(stream)), "lpq_requantize_fp8blk_mxfp8")
    return q_out, e_out


def lpq_fp8blk_amax(q, s, amax=None, accumulate=False, stream=None):
    """max |y| of the dequantized BF16 values into a 1-element FP32 device tensor."""
    q = _codes_in(q, "q")
    M, N = q.shape
    amax = _empty((1,), torch.float32, q) if amax is None else amax
    _check(_L.lpq_fp8blk_amax(q.data_ptr(), s.data_ptr(), M, N, amax.data_ptr(), int(bool(accumulate)),
                              _stream(stream)), "lpq_fp8blk_amax")
    return amax


def lpq_requantize_fp8blk_nvfp4(q, s, amax, p=None, sb=None, g=None, stream=None):
    """Block-wise FP8 -> NVFP4 (packed [M,N/2] uint8, E4M3 block scales [M,N/16], global scale [1])
    of the dequantized BF16 values under the group amax (1-element FP32 device tensor)."""
    q = _codes_in(q, "q")
    M, N = q.shape
    p = _empty((M, max(N // 2, 1)), torch.uint8, q) if p is None else p
    sb = _empty((M, max(N // 16, 1)), torch.float8_e4m3fn, q) if sb is None else sb
    g = _empty((1,), torch.float32, q) if g is None else g
    _check(_L.lpq_requantize_fp8blk_nvfp4(q.data_ptr(), s.data_ptr(), M, N, amax.data_ptr(), p.data_ptr(),
                                          sb.data_ptr(), g.data_ptr(), _stream(stream)),
           "lpq_requantize_fp8blk_nvfp4")
    return p, sb, g


# --------------------------------------------------------------------------- grouped

class TensorTable:
    """The n descriptors of a grouped call, in host memory and on the device.

    ``entries`` is a list of (src, dst, scale, rows, cols, group): torch tensors
    (dst / scale may be None where the call ignores them), the logical shape
    M x N of the BF16 tensor, and the NVFP4 sibling group.  The tensors must
    stay alive while the table is used."""

    def __init__(self, entries, device=None):
        n = len(entries)
        self.host = (lpq_tensor * n)()
        self.keep = []
        for i, (src, dst, scale, rows, cols, group) in enumerate(entries):
            self.host[i].src = _ptr(src)
            self.host[i].dst = _ptr(dst)
            self.host[i].scale = _ptr(scale)
            self.host[i].rows = int(rows)
            self.host[i].cols = int(cols)
            self.host[i].group = int(group)
            self.host[i].reserved = 0
            self.keep.append((src, dst, scale))
        raw = torch.frombuffer(bytearray(bytes(self.host)), dtype=torch.uint8)
        dev = device if device is not None else entries[0][0].device
        self.dev = raw.to(dev)
        self.n = n

    def args(self):
        return self.host, self.dev.data_ptr(), self.n


class RequantTable:
    """Descriptors of a grouped re-quantization call: ``entries`` is a list of
    (src codes, src tile scales, dst, dst scales, rows, cols, group)."""

    def __init__(self, entries, device=None):
        n = len(entries)
        self.host = (lpq_requant_tensor * n)()
        self.keep = []
        for i, (src, src_scale, dst, dst_scale, rows, cols, group) in enumerate(entries):
            h = self.host[i]
            h.src, h.src_scale, h.dst, h.dst_scale = _ptr(src), _ptr(src_scale), _ptr(dst), _ptr(dst_scale)
            h.rows, h.cols, h.group, h.reserved = int(rows), int(cols), int(group), 0
            self.keep.append((src, src_scale, dst, dst_scale))
        raw = torch.frombuffer(bytearray(bytes(self.host)), dtype=torch.uint8)
        dev = device if device is not None else entries[0][0].device
        self.dev = raw.to(dev)
        self.n = n

    def args(self):
        return self.host, self.dev.data_ptr(), self.n


def lpq_quantize_fp8blk_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_quantize_fp8blk_grouped(*table.args(), _stream(stream)), "lpq_quantize_fp8blk_grouped")


def lpq_dequantize_fp8blk_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_dequantize_fp8blk_grouped(*table.args(), _stream(stream)), "lpq_dequantize_fp8blk_grouped")


def lpq_quantize_mxfp8_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_quantize_mxfp8_grouped(*table.args(), _stream(stream)), "lpq_quantize_mxfp8_grouped")


def lpq_quantize_mxfp8_floor_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_quantize_mxfp8_floor_grouped(*table.args(), _stream(stream)), "lpq_quantize_mxfp8_floor_grouped")


def lpq_dequantize_mxfp8_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_dequantize_mxfp8_grouped(*table.args(), _stream(stream)), "lpq_dequantize_mxfp8_grouped")


def lpq_nvfp4_amax_grouped(table: TensorTable, group_amax, accumulate=False, stream=None):
    _check(_L.lpq_nvfp4_amax_grouped(*table.args(), group_amax.data_ptr(), group_amax.numel(),
                                     int(bool(accumulate)), _stream(stream)), "lpq_nvfp4_amax_grouped")
    return group_amax


def lpq_quantize_nvfp4_grouped(table: TensorTable, group_amax, group_g, stream=None):
    _check(_L.lpq_quantize_nvfp4_grouped(*table.args(), group_amax.data_ptr(), group_amax.numel(),
                                         group_g.data_ptr(), _stream(stream)), "lpq_quantize_nvfp4_grouped")
    return group_g


def lpq_quantize_nvfp4_grouped_ex(table: TensorTable, group_amax, group_g, e4m3_max=448, stream=None):
    _check(_L.lpq_quantize_nvfp4_grouped_ex(*table.args(), group_amax.data_ptr(), group_amax.numel(), int(e4m3_max),
                                            group_g.data_ptr(), _stream(stream)), "lpq_quantize_nvfp4_grouped_ex")
    return group_g


def lpq_nvfp4_qdq_grouped_ex(table: TensorTable, group_amax, e4m3_max=448, stream=None):
    _check(_L.lpq_nvfp4_qdq_grouped_ex(*table.args(), group_amax.data_ptr(), group_amax.numel(), int(e4m3_max),
                                       _stream(stream)), "lpq_nvfp4_qdq_grouped_ex")


def lpq_dequantize_nvfp4_grouped(table: TensorTable, group_g, stream=None):
    _check(_L.lpq_dequantize_nvfp4_grouped(*table.args(), group_g.data_ptr(), group_g.numel(), _stream(stream)),
           "lpq_dequantize_nvfp4_grouped")


def lpq_nvfp4_qdq_grouped(table: TensorTable, group_amax, stream=None):
    _check(_L.lpq_nvfp4_qdq_grouped(*table.args(), group_amax.data_ptr(), group_amax.numel(), _stream(stream)),
           "lpq_nvfp4_qdq_grouped")


def lpq_requantize_fp8blk_grouped(table: RequantTable, stream=None):
    _check(_L.lpq_requantize_fp8blk_grouped(*table.args(), _stream(stream)), "lpq_requantize_fp8blk_grouped")


def lpq_requantize_fp8blk_mxfp8_grouped(table: RequantTable, stream=None):
    _check(_L.lpq_requantize_fp8blk_mxfp8_grouped(*table.args(), _stream(stream)),
           "lpq_requantize_fp8blk_mxfp8_grouped")


def lpq_fp8blk_amax_grouped(table: RequantTable, group_amax, accumulate=False, stream=None):
    _check(_L.lpq_fp8blk_amax_grouped(*table.args(), group_amax.data_ptr(), group_amax.numel(),
                                      int(bool(accumulate)), _stream(stream)), "lpq_fp8blk_amax_grouped")
    return group_amax


def lpq_requantize_fp8blk_nvfp4_grouped(table: RequantTable, group_amax, group_g, stream=None):
    _check(_L.lpq_requantize_fp8blk_nvfp4_grouped(*table.args(), group_amax.data_ptr(), group_amax.numel(),
                                                  group_g.data_ptr(), _stream(stream)),
           "lpq_requantize_fp8blk_nvfp4_grouped")
    return group_g


def raw():
    """The ctypes handle of liblpq.so (for tests of the C ABI itself)."""
    return _L
