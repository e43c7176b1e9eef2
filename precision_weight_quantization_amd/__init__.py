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
    "lpq_quantize_nvfp4_grouped_ex": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _int, _vp, _vp]),
    "lpq_nvfp4_qdq_grouped_ex": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _int, _vp]),
    "lpq_observer_reset": (_int, [_vp, _vp]),
    "lpq_nvfp4_observe": (_int, [_vp, _i64, _i64, _int, ctypes.c_float, _vp, _vp, _vp]),
    "lpq_nvfp4_observe_noalloc": (_int, [_vp, _i64, _i64, _int, ctypes.c_float, _vp, _vp, _vp]),
    "lpq_nvfp4_amax": (_int, [_vp, _i64, _i64, _vp, _int, _vp]),
    "lpq_quantize_nvfp4": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "lpq_dequantize_nvfp4": (_int, [_vp, _vp, _vp, _i64, _i64, _vp, _vp]),
    "lpq_nvfp4_qdq": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "lpq_quantize_fp8blk_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_dequantize_fp8blk_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_quantize_mxfp8_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_dequantize_mxfp8_grouped": (_int, [_tp, _vp, _i32, _vp]),
    "lpq_nvfp4_amax_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _vp]),
    "lpq_quantize_nvfp4_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _vp, _vp]),
    "lpq_dequantize_nvfp4_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _vp]),
    "lpq_nvfp4_qdq_grouped": (_int, [_tp, _vp, _i32, _vp, _i32, _int, _vp]),
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


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _arg(t, name: str, like=None, nbytes: int = 0, esize=None, dtypes=None, dims=None):
    """Check a tensor argument before its address reaches a kernel: a device
    tensor, on the device of ``like`` (the call's data), contiguous, of the
    given element size or dtypes and rank, holding at least ``nbytes`` bytes.
    Raises TypeError or ValueError; nothing has been launched then."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor, got one on {t.device}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the call's data on {like.device}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {[str(d) for d in dtypes]}, got {t.dtype}")
    if esize is not None and t.element_size() != esize:
        raise TypeError(f"{name} must have {esize}-byte elements, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must be {dims}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes; the call accesses {nbytes}")
    return t


def _bf16_in(x, name: str):
    """A BF16 [M, N] device tensor (or its 16-bit integer view)."""
    return _arg(x, name, dtypes=_BF16, dims=2)


def _out(t, name: str, like, nbytes: int, shape, dtype, esize):
    """A caller-supplied output, checked; or a new one of ``shape`` and ``dtype``."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return _arg(t, name, like, nbytes, esize=esize)


def _outs(like, *specs):
    """Several outputs, each (tensor or None, name, nbytes, shape, dtype, esize):
    every tensor the caller gave is checked before any missing one is allocated."""
    for t, name, nbytes, _, _, esize in specs:
        if t is not None:
            _arg(t, name, like, nbytes, esize=esize)
    return [t if t is not None else torch.empty(shape, dtype=dtype, device=like.device)
            for t, _, _, shape, dtype, _ in specs]


def _f32_words(t, name: str, like, n: int = 1):
    """``n`` FP32 words on the device (an amax, a global scale, ...)."""
    return _arg(t, name, like, 4 * n, dtypes=(torch.float32,))


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


def _tiles(M: int, N: int) -> int:
    return ((M + 127) // 128) * ((N + 127) // 128)


# --------------------------------------------------------------------------- block-wise FP8

def fp8blk_scale_shape(M: int, N: int):
    return ((M + 127) // 128, (N + 127) // 128)


def _codes_in(q, name: str):
    """A 2-D device tensor of 1-byte codes (E4M3 or packed FP4/INT4)."""
    return _arg(q, name, esize=1, dims=2)


def lpq_quantize_fp8blk(w, q=None, s=None, stream=None):
    """BF16 [M,N] -> (codes [M,N] float8_e4m3fn, FP32 tile scales [ceil(M/128), ceil(N/128)])."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    q, s = _outs(w, (q, "q", M * N, (M, N), torch.float8_e4m3fn, 1),
                 (s, "s", 4 * _tiles(M, N), fp8blk_scale_shape(M, N), torch.float32, 4))
    _check(_L.lpq_quantize_fp8blk(w.data_ptr(), M, N, q.data_ptr(), s.data_ptr(), _stream(stream)),
           "lpq_quantize_fp8blk")
    return q, s


def lpq_dequantize_fp8blk(q, s, y=None, stream=None):
    q = _codes_in(q, "q")
    M, N = q.shape
    _arg(s, "s", q, 4 * _tiles(M, N), esize=4)
    y = _out(y, "y", q, 2 * M * N, (M, N), torch.bfloat16, 2)
    _check(_L.lpq_dequantize_fp8blk(q.data_ptr(), s.data_ptr(), M, N, y.data_ptr(), _stream(stream)),
           "lpq_dequantize_fp8blk")
    return y


# --------------------------------------------------------------------------- MXFP8

def _mxfp8_quantize(fn, where, w, q, e, stream):
    w = _bf16_in(w, "w")
    M, N = w.shape
    q, e = _outs(w, (q, "q", M * N, (M, N), torch.float8_e4m3fn, 1),
                 (e, "e", M * (N // 32), (M, max(N // 32, 1)), torch.uint8, 1))
    _check(fn(w.data_ptr(), M, N, q.data_ptr(), e.data_ptr(), _stream(stream)), where)
    return q, e


def lpq_quantize_mxfp8(w, q=None, e=None, stream=None):
    """BF16 [M,N] (N % 32 == 0) -> (codes [M,N] float8_e4m3fn, UE8M0 bytes [M,N/32] uint8)."""
    return _mxfp8_quantize(_L.lpq_quantize_mxfp8, "lpq_quantize_mxfp8", w, q, e, stream)


def lpq_quantize_mxfp8_floor(w, q=None, e=None, stream=None):
    """As lpq_quantize_mxfp8, with the OCP MX floor exponent rule (saturating)."""
    return _mxfp8_quantize(_L.lpq_quantize_mxfp8_floor, "lpq_quantize_mxfp8_floor", w, q, e, stream)


def lpq_dequantize_mxfp8(q, e, y=None, stream=None):
    q = _codes_in(q, "q")
    M, N = q.shape
    _arg(e, "e", q, M * (N // 32), esize=1)
    y = _out(y, "y", q, 2 * M * N, (M, N), torch.bfloat16, 2)
    _check(_L.lpq_dequantize_mxfp8(q.data_ptr(), e.data_ptr(), M, N, y.data_ptr(), _stream(stream)),
           "lpq_dequantize_mxfp8")
    return y


# --------------------------------------------------------------------------- NVFP4

def lpq_nvfp4_amax(w, amax=None, accumulate=False, stream=None):
    """max |w| into a 1-element FP32 device tensor (max-accumulated when accumulate)."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    amax = _empty((1,), torch.float32, w) if amax is None else _f32_words(amax, "amax", w)
    _check(_L.lpq_nvfp4_amax(w.data_ptr(), M, N, amax.data_ptr(), int(bool(accumulate)), _stream(stream)),
           "lpq_nvfp4_amax")
    return amax


def lpq_quantize_nvfp4_ex(w, amax=None, e4m3_max=448, p=None, s=None, g=None, stream=None):
    """BF16 [M,N] (N % 16 == 0) -> (packed [M,N/2] uint8, E4M3 block scales [M,N/16]
    float8_e4m3fn, global scale [1] FP32 = fl(A / (6 * e4m3_max))), e4m3_max 448 or 256.
    amax: 1-element FP32 device tensor holding the group amax A, or None for the
    tensor's own (computed by the call)."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    if amax is not None:
        _f32_words(amax, "amax", w)
    p, s, g = _outs(w, (p, "p", M * (N // 2), (M, max(N // 2, 1)), torch.uint8, 1),
                    (s, "s", M * (N // 16), (M, max(N // 16, 1)), torch.float8_e4m3fn, 1),
                    (g, "g", 4, (1,), torch.float32, 4))
    _check(_L.lpq_quantize_nvfp4_ex(w.data_ptr(), M, N, _ptr(amax), int(e4m3_max), p.data_ptr(), s.data_ptr(),
                                    g.data_ptr(), _stream(stream)), "lpq_quantize_nvfp4_ex")
    return p, s, g


def lpq_quantize_nvfp4(w, amax=None, p=None, s=None, g=None, stream=None):
    """BF16 [M,N] (N % 16 == 0) with group amax (1-element FP32 device tensor, or None
    for the tensor's own, computed by the call) -> (packed [M,N/2] uint8, E4M3 block
    scales [M,N/16] float8_e4m3fn, global scale [1] FP32)."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    if amax is not None:
        _f32_words(amax, "amax", w)
    p, s, g = _outs(w, (p, "p", M * (N // 2), (M, max(N // 2, 1)), torch.uint8, 1),
                    (s, "s", M * (N // 16), (M, max(N // 16, 1)), torch.float8_e4m3fn, 1),
                    (g, "g", 4, (1,), torch.float32, 4))
    _check(_L.lpq_quantize_nvfp4(w.data_ptr(), M, N, _ptr(amax), p.data_ptr(), s.data_ptr(), g.data_ptr(),
                                 _stream(stream)), "lpq_quantize_nvfp4")
    return p, s, g


def lpq_nvfp4_qdq_ex(x, amax, e4m3_max=448, y=None, stream=None):
    x = _bf16_in(x, "x")
    M, N = x.shape
    if amax is not None:
        _f32_words(amax, "amax", x)
    y = _out(y, "y", x, 2 * M * N, (M, N), torch.bfloat16, 2)
    _check(_L.lpq_nvfp4_qdq_ex(x.data_ptr(), M, N, _ptr(amax), int(e4m3_max), y.data_ptr(), _stream(stream)),
           "lpq_nvfp4_qdq_ex")
    return y


def lpq_nvfp4_global_scale_reciprocal(group_amax, out=None, stream=None):
    """fl(2688 / A) per group (the reciprocal export form of the global scale)."""
    _f32_words(group_amax, "group_amax", None, group_amax.numel() if isinstance(group_amax, torch.Tensor) else 1)
    out = torch.empty_like(group_amax) if out is None else _f32_words(out, "out", group_amax, group_amax.numel())
    _check(_L.lpq_nvfp4_global_scale_reciprocal(group_amax.data_ptr(), group_amax.numel(), out.data_ptr(),
                                                _stream(stream)), "lpq_nvfp4_global_scale_reciprocal")
    return out


def lpq_nvfp4_global_scale(amax, out=None, stream=None):
    """fl(A / 2688) per entry (the multiplier form of a global scale)."""
    _f32_words(amax, "amax", None, amax.numel() if isinstance(amax, torch.Tensor) else 1)
    out = torch.empty_like(amax) if out is None else _f32_words(out, "out", amax, amax.numel())
    _check(_L.lpq_nvfp4_global_scale(amax.data_ptr(), amax.numel(), out.data_ptr(), _stream(stream)),
           "lpq_nvfp4_global_scale")
    return out


# W4A4 activation observers (the C constants of the same names)
OBSERVERS = {"memoryless_minmax": 0, "static_minmax": 1, "minmax": 2}
OBSERVER_STATE_FLOATS = 128


def lpq_observer_reset(state=None, device=None, stream=None):
    """A reset observer state (8 FP32 words on the device; allocated when not given)."""
    if state is None:
        state = torch.empty(OBSERVER_STATE_FLOATS, dtype=torch.float32, device=device or "cuda")
    else:
        _f32_words(state, "state", None, OBSERVER_STATE_FLOATS)
    _check(_L.lpq_observer_reset(state.data_ptr(), _stream(stream)), "lpq_observer_reset")
    return state


def lpq_nvfp4_observe(x, state, observer="static_minmax", averaging_constant=0.01, amax=None, stream=None):
    """Update the observer state with the BF16 batch x; returns the activation amax (1 FP32, device)."""
    x = _bf16_in(x, "x")
    M, N = x.shape
    _f32_words(state, "state", x, OBSERVER_STATE_FLOATS)
    amax = _empty((1,), torch.float32, x) if amax is None else _f32_words(amax, "amax", x)
    kind = OBSERVERS[observer] if isinstance(observer, str) else int(observer)
    _check(_L.lpq_nvfp4_observe(x.data_ptr(), M, N, kind, float(averaging_constant), state.data_ptr(),
                                amax.data_ptr(), _stream(stream)), "lpq_nvfp4_observe")
    return amax


def lpq_nvfp4_observe_noalloc(x, state, observer="static_minmax", averaging_constant=0.01, amax=None, stream=None):
    """lpq_nvfp4_observe with the call's control words in a block the library holds on
    the device: ``state`` needs only 3 FP32 words (min, max, batches seen).  Calls
    that overlap on one device race.  Pass ``amax`` (1 FP32 on the device) for a call
    that allocates nothing; without it this wrapper allocates the output."""
    x = _bf16_in(x, "x")
    M, N = x.shape
    _f32_words(state, "state", x, 3)
    amax = _empty((1,), torch.float32, x) if amax is None else _f32_words(amax, "amax", x)
    kind = OBSERVERS[observer] if isinstance(observer, str) else int(observer)
    _check(_L.lpq_nvfp4_observe_noalloc(x.data_ptr(), M, N, kind, float(averaging_constant), state.data_ptr(),
                                        amax.data_ptr(), _stream(stream)), "lpq_nvfp4_observe_noalloc")
    return amax


def lpq_dequantize_nvfp4(p, s, g, y=None, stream=None):
    p = _codes_in(p, "p")
    M, N = p.shape[0], p.shape[1] * 2
    _arg(s, "s", p, M * (N // 16), esize=1)
    _f32_words(g, "g", p)
    y = _out(y, "y", p, 2 * M * N, (M, N), torch.bfloat16, 2)
    _check(_L.lpq_dequantize_nvfp4(p.data_ptr(), s.data_ptr(), g.data_ptr(), M, N, y.data_ptr(), _stream(stream)),
           "lpq_dequantize_nvfp4")
    return y


def lpq_nvfp4_qdq(x, amax=None, y=None, stream=None):
    """NVFP4 fake quantization of BF16 [M,N] under the group amax (1-element FP32 device
    tensor); returns BF16 [M,N].  amax None: the tensor's own, computed by the library."""
    x = _bf16_in(x, "x")
    M, N = x.shape
    if amax is not None:
        _f32_words(amax, "amax", x)
    y = _out(y, "y", x, 2 * M * N, (M, N), torch.bfloat16, 2)
    _check(_L.lpq_nvfp4_qdq(x.data_ptr(), M, N, _ptr(amax), y.data_ptr(), _stream(stream)), "lpq_nvfp4_qdq")
    return y


# --------------------------------------------------------------------------- INT4, group-wise

INT4_GROUPS = (32, 128)


def _int4_group(group) -> int:
    return max(int(group), 1)


def lpq_quantize_int4(w, group=128, p=None, s=None, stream=None):
    """BF16 [M,N] (N % group == 0) -> (packed two's-complement nibbles [M,N/2] uint8,
    FP32 group scales [M,N/group])."""
    w = _bf16_in(w, "w")
    M, N = w.shape
    G = _int4_group(group)
    p, s = _outs(w, (p, "p", M * (N // 2), (M, max(N // 2, 1)), torch.uint8, 1),
                 (s, "s", 4 * M * (N // G), (M, max(N // G, 1)), torch.float32, 4))
    _check(_L.lpq_quantize_int4(w.data_ptr(), M, N, int(group), p.data_ptr(), s.data_ptr(), _stream(stream)),
           "lpq_quantize_int4")
    return p, s


def lpq_dequantize_int4(p, s, group=128, y=None, stream=None):
    p = _codes_in(p, "p")
    M, N = p.shape[0], p.shape[1] * 2
    _arg(s, "s", p, 4 * M * (N // _int4_group(group)), esize=4)
    y = _out(y, "y", p, 2 * M * N, (M, N), torch.bfloat16, 2)
    _check(_L.lpq_dequantize_int4(p.data_ptr(), s.data_ptr(), M, N, int(group), y.data_ptr(), _stream(stream)),
           "lpq_dequantize_int4")
    return y


def lpq_int4_qdq(x, group=128, y=None, stream=None):
    """INT4 fake quantization (the straight-through estimator's forward pass) of BF16 [M,N]."""
    x = _bf16_in(x, "x")
    M, N = x.shape
    y = _out(y, "y", x, 2 * M * N, (M, N), torch.bfloat16, 2)
    _check(_L.lpq_int4_qdq(x.data_ptr(), M, N, int(group), y.data_ptr(), _stream(stream)), "lpq_int4_qdq")
    return y


# --------------------------------------------------------------------------- FP8 re-quantization

def lpq_requantize_fp8blk(q, s, q_out=None, s_out=None, stream=None):
    """Block-wise FP8 (codes [M,N], FP32 tile scales) -> block-wise FP8 of the dequantized
    BF16 values (codes [M,N] float8_e4m3fn, new FP32 tile scales), in one pass."""
    q = _codes_in(q, "q")
    M, N = q.shape
    _arg(s, "s", q, 4 * _tiles(M, N), esize=4)
    q_out, s_out = _outs(q, (q_out, "q_out", M * N, (M, N), torch.float8_e4m3fn, 1),
                         (s_out, "s_out", 4 * _tiles(M, N), fp8blk_scale_shape(M, N), torch.float32, 4))
    _check(_L.lpq_requantize_fp8blk(q.data_ptr(), s.data_ptr(), M, N, q_out.data_ptr(), s_out.data_ptr(),
                                    _stream(stream)), "lpq_requantize_fp8blk")
    return q_out, s_out


def lpq_requantize_fp8blk_mxfp8(q, s, q_out=None, e_out=None, stream=None):
    """Block-wise FP8 (codes [M,N], FP32 tile scales) -> MXFP8 (codes [M,N] float8_e4m3fn,
    UE8M0 bytes [M,N/32] uint8) of the dequantized BF16 values, in one pass."""
    q = _codes_in(q, "q")
    M, N = q.shape
    _arg(s, "s", q, 4 * _tiles(M, N), esize=4)
    q_out, e_out = _outs(q, (q_out, "q_out", M * N, (M, N), torch.float8_e4m3fn, 1),
                         (e_out, "e_out", M * (N // 32), (M, max(N // 32, 1)), torch.uint8, 1))
    _check(_L.lpq_requantize_fp8blk_mxfp8(q.data_ptr(), s.data_ptr(), M, N, q_out.data_ptr(), e_out.data_ptr(),
                                          _stream(stream)), "lpq_requantize_fp8blk_mxfp8")
    return q_out, e_out


def lpq_fp8blk_amax(q, s, amax=None, accumulate=False, stream=None):
    """max |y| of the dequantized BF16 values into a 1-element FP32 device tensor."""
    q = _codes_in(q, "q")
    M, N = q.shape
    _arg(s, "s", q, 4 * _tiles(M, N), esize=4)
    amax = _empty((1,), torch.float32, q) if amax is None else _f32_words(amax, "amax", q)
    _check(_L.lpq_fp8blk_amax(q.data_ptr(), s.data_ptr(), M, N, amax.data_ptr(), int(bool(accumulate)),
                              _stream(stream)), "lpq_fp8blk_amax")
    return amax


def lpq_requantize_fp8blk_nvfp4(q, s, amax, p=None, sb=None, g=None, stream=None):
    """Block-wise FP8 -> NVFP4 (packed [M,N/2] uint8, E4M3 block scales [M,N/16], global scale [1])
    of the dequantized BF16 values under the group amax (1-element FP32 device tensor)."""
    q = _codes_in(q, "q")
    M, N = q.shape
    _arg(s, "s", q, 4 * _tiles(M, N), esize=4)
    _f32_words(amax, "amax", q)
    p, sb, g = _outs(q, (p, "p", M * (N // 2), (M, max(N // 2, 1)), torch.uint8, 1),
                     (sb, "sb", M * (N // 16), (M, max(N // 16, 1)), torch.float8_e4m3fn, 1),
                     (g, "g", 4, (1,), torch.float32, 4))
    _check(_L.lpq_requantize_fp8blk_nvfp4(q.data_ptr(), s.data_ptr(), M, N, amax.data_ptr(), p.data_ptr(),
                                          sb.data_ptr(), g.data_ptr(), _stream(stream)),
           "lpq_requantize_fp8blk_nvfp4")
    return p, sb, g


# --------------------------------------------------------------------------- grouped

# Bytes each descriptor array of a grouped call accesses, per operation, for a
# tensor of M x N elements: (src, dst, scale) of lpq_tensor, or (src,
# src_scale, dst, dst_scale) of lpq_requant_tensor; None = not accessed.
def _grouped_bytes(op: str, M: int, N: int, G: int = 128):
    MN, t = M * N, 4 * _tiles(M, N)
    return _GROUPED_BYTES[op](MN, t, G)


_GROUPED_BYTES = {
    "fp8blk_q": lambda MN, t, G: (2 * MN, MN, t),
    "fp8blk_dq": lambda MN, t, G: (MN, 2 * MN, t),
    "mxfp8_q": lambda MN, t, G: (2 * MN, MN, MN // 32),
    "mxfp8_dq": lambda MN, t, G: (MN, 2 * MN, MN // 32),
    "nvfp4_amax": lambda MN, t, G: (2 * MN, None, None),
    "nvfp4_q": lambda MN, t, G: (2 * MN, MN // 2, MN // 16),
    "nvfp4_dq": lambda MN, t, G: (MN // 2, 2 * MN, MN // 16),
    "nvfp4_qdq": lambda MN, t, G: (2 * MN, 2 * MN, None),
    "int4_q": lambda MN, t, G: (2 * MN, MN // 2, 4 * (MN // G)),
    "int4_dq": lambda MN, t, G: (MN // 2, 2 * MN, 4 * (MN // G)),
    "int4_qdq": lambda MN, t, G: (2 * MN, 2 * MN, None),
    "rq_fp8": lambda MN, t, G: (MN, t, MN, t),
    "rq_mx": lambda MN, t, G: (MN, t, MN, MN // 32),
    "rq_amax": lambda MN, t, G: (MN, t, None, None),
    "rq_nv": lambda MN, t, G: (MN, t, MN // 2, MN // 16),
}


class _Table:
    """Descriptors of a grouped call in host memory and, copied once, on the device.

    The device copy is a blocking host-to-device copy: it has completed when the
    constructor returns, so the table serves calls on any stream.  The tensors
    named by the entries must stay alive while the table is used."""

    _CTYPE = None
    _FIELDS = ()

    def __init__(self, entries, device=None):
        n = len(entries)
        if n == 0:
            raise ValueError("a grouped call needs at least one tensor")
        first = entries[0][0]
        _arg(first, f"entry 0 {self._FIELDS[0]}")
        dev = torch.device(device) if device is not None else first.device
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.host = (self._CTYPE * n)()
        self.keep = []
        for i, e in enumerate(entries):
            tensors, (rows, cols, group) = e[:-3], e[-3:]
            for name, t in zip(self._FIELDS, tensors):
                if t is not None and (not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev
                                      or not t.is_contiguous()):
                    raise ValueError(f"entry {i} {name}: a contiguous tensor on {dev} is required")
            h = self.host[i]
            for name, t in zip(self._FIELDS, tensors):
                setattr(h, name, _ptr(t))
            h.rows, h.cols, h.group, h.reserved = int(rows), int(cols), int(group), 0
            self.keep.append(tuple(tensors))
        raw = torch.frombuffer(bytearray(bytes(self.host)), dtype=torch.uint8)
        self.dev = torch.empty(raw.numel(), dtype=torch.uint8, device=dev)
        self.dev.copy_(raw, non_blocking=False)
        self.device = dev
        self.n = n
        self._checked = set()

    def check(self, op: str, G: int = 128):
        """Raise ValueError unless every tensor an operation accesses is large enough
        (checked once per operation and group size: the entries do not change)."""
        if (op, G) in self._checked:
            return self
        for i, tensors in enumerate(self.keep):
            h = self.host[i]
            for name, t, need in zip(self._FIELDS, tensors, _grouped_bytes(op, h.rows, h.cols, G)):
                if need is None:
                    continue
                if t is None:
                    raise ValueError(f"entry {i}: {op} needs {name}")
                have = t.numel() * t.element_size()
                if have < need:
                    raise ValueError(f"entry {i} {name} holds {have} bytes; {op} accesses {need}")
        self._checked.add((op, G))
        return self

    def args(self):
        return self.host, self.dev.data_ptr(), self.n


class TensorTable(_Table):
    """The n descriptors of a grouped call.  ``entries`` is a list of (src, dst,
    scale, rows, cols, group): device tensors (dst / scale may be None where the
    call ignores them), the logical shape M x N of the BF16 tensor, and the
    NVFP4 sibling group."""

    _CTYPE = lpq_tensor
    _FIELDS = ("src", "dst", "scale")


class RequantTable(_Table):
    """Descriptors of a grouped re-quantization call: ``entries`` is a list of
    (src codes, src tile scales, dst, dst scales, rows, cols, group)."""

    _CTYPE = lpq_requant_tensor
    _FIELDS = ("src", "src_scale", "dst", "dst_scale")


def _group_words(t, name, table, n=None):
    return _f32_words(t, name, table.dev, t.numel() if n is None and isinstance(t, torch.Tensor) else (n or 1))


def lpq_quantize_fp8blk_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_quantize_fp8blk_grouped(*table.check("fp8blk_q").args(), _stream(stream)),
           "lpq_quantize_fp8blk_grouped")


def lpq_dequantize_fp8blk_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_dequantize_fp8blk_grouped(*table.check("fp8blk_dq").args(), _stream(stream)),
           "lpq_dequantize_fp8blk_grouped")


def lpq_quantize_mxfp8_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_quantize_mxfp8_grouped(*table.check("mxfp8_q").args(), _stream(stream)),
           "lpq_quantize_mxfp8_grouped")


def lpq_quantize_mxfp8_floor_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_quantize_mxfp8_floor_grouped(*table.check("mxfp8_q").args(), _stream(stream)),
           "lpq_quantize_mxfp8_floor_grouped")


def lpq_dequantize_mxfp8_grouped(table: TensorTable, stream=None):
    _check(_L.lpq_dequantize_mxfp8_grouped(*table.check("mxfp8_dq").args(), _stream(stream)),
           "lpq_dequantize_mxfp8_grouped")


def lpq_nvfp4_amax_grouped(table: TensorTable, group_amax, accumulate=False, stream=None):
    _group_words(group_amax, "group_amax", table)
    _check(_L.lpq_nvfp4_amax_grouped(*table.check("nvfp4_amax").args(), group_amax.data_ptr(), group_amax.numel(),
                                     int(bool(accumulate)), _stream(stream)), "lpq_nvfp4_amax_grouped")
    return group_amax


def lpq_quantize_nvfp4_grouped(table: TensorTable, group_amax, group_g, amax_valid=True, stream=None):
    """amax_valid False: the call fills group_amax (every member's max |w| folded into
    its group's slot) before it encodes."""
    _group_words(group_amax, "group_amax", table)
    _group_words(group_g, "group_g", table, group_amax.numel())
    _check(_L.lpq_quantize_nvfp4_grouped(*table.check("nvfp4_q").args(), group_amax.data_ptr(), group_amax.numel(),
                                         int(bool(amax_valid)), group_g.data_ptr(), _stream(stream)),
           "lpq_quantize_nvfp4_grouped")
    return group_g


def lpq_quantize_nvfp4_grouped_ex(table: TensorTable, group_amax, group_g, e4m3_max=448, amax_valid=True,
                                  stream=None):
    _group_words(group_amax, "group_amax", table)
    _group_words(group_g, "group_g", table, group_amax.numel())
    _check(_L.lpq_quantize_nvfp4_grouped_ex(*table.check("nvfp4_q").args(), group_amax.data_ptr(), group_amax.numel(),
                                            int(bool(amax_valid)), int(e4m3_max), group_g.data_ptr(),
                                            _stream(stream)), "lpq_quantize_nvfp4_grouped_ex")
    return group_g


def lpq_nvfp4_qdq_grouped_ex(table: TensorTable, group_amax, e4m3_max=448, amax_valid=True, stream=None):
    _group_words(group_amax, "group_amax", table)
    _check(_L.lpq_nvfp4_qdq_grouped_ex(*table.check("nvfp4_qdq").args(), group_amax.data_ptr(), group_amax.numel(),
                                       int(bool(amax_valid)), int(e4m3_max), _stream(stream)),
           "lpq_nvfp4_qdq_grouped_ex")


def lpq_dequantize_nvfp4_grouped(table: TensorTable, group_g, stream=None):
    _group_words(group_g, "group_g", table)
    _check(_L.lpq_dequantize_nvfp4_grouped(*table.check("nvfp4_dq").args(), group_g.data_ptr(), group_g.numel(),
                                           _stream(stream)), "lpq_dequantize_nvfp4_grouped")


def lpq_nvfp4_qdq_grouped(table: TensorTable, group_amax, amax_valid=True, stream=None):
    """amax_valid False: the call fills group_amax before it encodes."""
    _group_words(group_amax, "group_amax", table)
    _check(_L.lpq_nvfp4_qdq_grouped(*table.check("nvfp4_qdq").args(), group_amax.data_ptr(), group_amax.numel(),
                                    int(bool(amax_valid)), _stream(stream)), "lpq_nvfp4_qdq_grouped")


def lpq_quantize_int4_grouped(table: TensorTable, group=128, stream=None):
    _check(_L.lpq_quantize_int4_grouped(*table.check("int4_q", _int4_group(group)).args(), int(group),
                                        _stream(stream)), "lpq_quantize_int4_grouped")


def lpq_dequantize_int4_grouped(table: TensorTable, group=128, stream=None):
    _check(_L.lpq_dequantize_int4_grouped(*table.check("int4_dq", _int4_group(group)).args(), int(group),
                                          _stream(stream)), "lpq_dequantize_int4_grouped")


def lpq_int4_qdq_grouped(table: TensorTable, group=128, stream=None):
    _check(_L.lpq_int4_qdq_grouped(*table.check("int4_qdq").args(), int(group), _stream(stream)),
           "lpq_int4_qdq_grouped")


def lpq_requantize_fp8blk_grouped(table: RequantTable, stream=None):
    _check(_L.lpq_requantize_fp8blk_grouped(*table.check("rq_fp8").args(), _stream(stream)),
           "lpq_requantize_fp8blk_grouped")


def lpq_requantize_fp8blk_mxfp8_grouped(table: RequantTable, stream=None):
    _check(_L.lpq_requantize_fp8blk_mxfp8_grouped(*table.check("rq_mx").args(), _stream(stream)),
           "lpq_requantize_fp8blk_mxfp8_grouped")


def lpq_fp8blk_amax_grouped(table: RequantTable, group_amax, accumulate=False, stream=None):
    _group_words(group_amax, "group_amax", table)
    _check(_L.lpq_fp8blk_amax_grouped(*table.check("rq_amax").args(), group_amax.data_ptr(), group_amax.numel(),
                                      int(bool(accumulate)), _stream(stream)), "lpq_fp8blk_amax_grouped")
    return group_amax


def lpq_requantize_fp8blk_nvfp4_grouped(table: RequantTable, group_amax, group_g, stream=None):
    _group_words(group_amax, "group_amax", table)
    _group_words(group_g, "group_g", table, group_amax.numel())
    _check(_L.lpq_requantize_fp8blk_nvfp4_grouped(*table.check("rq_nv").args(), group_amax.data_ptr(),
                                                  group_amax.numel(), group_g.data_ptr(), _stream(stream)),
           "lpq_requantize_fp8blk_nvfp4_grouped")
    return group_g


def raw():
    """The ctypes handle of liblpq.so (for tests of the C ABI itself)."""
    return _L
