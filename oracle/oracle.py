"""Python binding of the CPU oracle (``oracle/lpq_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; the product library never imports
it.  All arrays are numpy; BF16 tensors travel as ``uint16`` bit patterns,
codes and scale bytes as ``uint8``, FP32 scales as ``float32``.

The arithmetic lives in the C file (one IEEE binary32 operation per step,
round-to-nearest-even, no FMA contraction); this module only marshals
arguments, forms the sibling-group global scale of an NVFP4 group (the
maximum of the members' amax values, "verl NVFP4 QAT" section 2.4), and runs
independent tensors on a thread pool.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "lpq_oracle.c")
LIB = os.path.join(_HERE, "liblpq_oracle.so")
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no GPU involved)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def build_variant(src_text: str, out_path: str) -> str:
    """Compile a modified copy of the oracle source (used by the tests that plant
    mistakes in the oracle to show that its pins catch them)."""
    c_path = out_path[:-3] + ".c" if out_path.endswith(".so") else out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *CFLAGS, "-o", out_path, c_path, "-lm"])
    return out_path


_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_i64 = ctypes.c_int64

_SIG = {
    "oc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "oc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
    "oc_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
    "oc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
    "oc_e2m1_decode": (ctypes.c_float, [ctypes.c_uint8]),
    "oc_e2m1_encode": (ctypes.c_uint8, [ctypes.c_float]),
    "oc_ue8m0_decode": (ctypes.c_float, [ctypes.c_uint8]),
    "oc_mxfp8_scale_byte": (ctypes.c_uint8, [ctypes.c_float]),
    "oc_amax_bf16": (ctypes.c_float, [_u16p, _i64]),
    "oc_nvfp4_global_scale": (ctypes.c_float, [ctypes.c_float]),
    "oc_nvfp4_block_scale": (ctypes.c_uint8, [ctypes.c_float, ctypes.c_float]),
    "oc_nvfp4_effective_scale": (ctypes.c_float, [ctypes.c_uint8, ctypes.c_float]),
    "oc_fp8blk_quantize": (None, [_u16p, _i64, _i64, _u8p, _f32p]),
    "oc_fp8blk_dequantize": (None, [_u8p, _f32p, _i64, _i64, _u16p]),
    "oc_mxfp8_quantize": (None, [_u16p, _i64, _i64, _u8p, _u8p]),
    "oc_mxfp8_dequantize": (None, [_u8p, _u8p, _i64, _i64, _u16p]),
    "oc_nvfp4_quantize": (None, [_u16p, _i64, _i64, ctypes.c_float, _u8p, _u8p]),
    "oc_nvfp4_dequantize": (None, [_u8p, _u8p, ctypes.c_float, _i64, _i64, _u16p]),
    "oc_nvfp4_qdq": (None, [_u16p, _i64, _i64, ctypes.c_float, _u16p]),
    "oc_e4m3_encode_n": (None, [_f32p, _i64, _u8p]),
    "oc_e2m1_encode_n": (None, [_f32p, _i64, _u8p]),
    "oc_f32_to_bf16_n": (None, [_f32p, _i64, _u16p]),
    "oc_mxfp8_scale_byte_n": (None, [_f32p, _i64, _u8p]),
    "oc_mxfp8_floor_scale_byte_n": (None, [_f32p, _i64, _u8p]),
    "oc_mxfp8_floor_quantize": (None, [_u16p, _i64, _i64, _u8p, _u8p]),
    "oc_nvfp4_global_scale_reciprocal": (ctypes.c_float, [ctypes.c_float]),
    "oc_observer_update": (ctypes.c_float, [ctypes.c_int, ctypes.c_float, _f32p, _u16p, _i64]),
    "oc_nvfp4_global_scale_max": (ctypes.c_float, [ctypes.c_float, ctypes.c_int]),
    "oc_int4_scale": (ctypes.c_float, [ctypes.c_float]),
    "oc_int4_quantize": (None, [_u16p, _i64, _i64, _i64, _u8p, _f32p]),
    "oc_int4_dequantize": (None, [_u8p, _f32p, _i64, _i64, _i64, _u16p]),
    "oc_int4_qdq": (None, [_u16p, _i64, _i64, _i64, _u16p]),
}


def _p(a: np.ndarray, ptype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ptype)


def _bf16(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w)
    assert w.dtype == np.uint16 and w.ndim == 2, "BF16 tensors are 2-D uint16 bit patterns"
    return w


def fp8blk_scale_shape(M: int, N: int) -> tuple[int, int]:
    return ((M + 127) // 128, (N + 127) // 128)


def bf16_to_f32(w: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns (numpy, no rounding involved)."""
    return (np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Oracle:
    """The oracle's functions, bound to one compiled copy of ``lpq_oracle.c``."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIG.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        self.path = path
        self.L = L

    # ------------------------------------------------------------------ scalar casts
    def _vec(self, fn, v, dtype):
        v = np.ascontiguousarray(np.asarray(v, dtype=np.float32).ravel())
        out = np.empty(v.size, dtype)
        fn(_p(v, _f32p), v.size, _p(out, _u8p if dtype == np.uint8 else _u16p))
        return out

    def e4m3_encode(self, v) -> np.ndarray:
        return self._vec(self.L.oc_e4m3_encode_n, v, np.uint8)

    def e2m1_encode(self, v) -> np.ndarray:
        return self._vec(self.L.oc_e2m1_encode_n, v, np.uint8)

    def f32_to_bf16(self, v) -> np.ndarray:
        return self._vec(self.L.oc_f32_to_bf16_n, v, np.uint16)

    def mxfp8_scale_byte(self, amax) -> np.ndarray:
        return self._vec(self.L.oc_mxfp8_scale_byte_n, amax, np.uint8)

    def e4m3_decode(self, c: int) -> float:
        return float(self.L.oc_e4m3_decode(int(c)))

    def e2m1_decode(self, c: int) -> float:
        return float(self.L.oc_e2m1_decode(int(c)))

    def ue8m0_decode(self, b: int) -> float:
        return float(self.L.oc_ue8m0_decode(int(b)))

    # ------------------------------------------------------------------ block-wise FP8
    def fp8blk_quantize(self, w: np.ndarray):
        """BF16 [M,N] -> (E4M3 codes [M,N] uint8, FP32 tile scales [ceil(M/128), ceil(N/128)])."""
        w = _bf16(w)
        M, N = w.shape
        q = np.empty((M, N), np.uint8)
        s = np.empty(fp8blk_scale_shape(M, N), np.float32)
        self.L.oc_fp8blk_quantize(_p(w, _u16p), M, N, _p(q, _u8p), _p(s, _f32p))
        return q, s

    def fp8blk_dequantize(self, q: np.ndarray, s: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.float32)
        M, N = q.shape
        assert s.shape == fp8blk_scale_shape(M, N)
        y = np.empty((M, N), np.uint16)
        self.L.oc_fp8blk_dequantize(_p(q, _u8p), _p(s, _f32p), M, N, _p(y, _u16p))
        return y

    # ------------------------------------------------------------------ MXFP8
    def mxfp8_quantize(self, w: np.ndarray):
        """BF16 [M,N] (N % 32 == 0) -> (E4M3 codes [M,N], UE8M0 bytes [M,N/32])."""
        w = _bf16(w)
        M, N = w.shape
        assert N % 32 == 0
        q = np.empty((M, N), np.uint8)
        e = np.empty((M, N // 32), np.uint8)
        self.L.oc_mxfp8_quantize(_p(w, _u16p), M, N, _p(q, _u8p), _p(e, _u8p))
        return q, e

    def mxfp8_floor_scale_byte(self, amax) -> np.ndarray:
        return self._vec(self.L.oc_mxfp8_floor_scale_byte_n, amax, np.uint8)

    def mxfp8_floor_quantize(self, w: np.ndarray):
        """BF16 [M,N] (N % 32 == 0) -> (E4M3 codes, UE8M0 bytes) under the floor exponent rule."""
        w = _bf16(w)
        M, N = w.shape
        assert N % 32 == 0
        q = np.empty((M, N), np.uint8)
        e = np.empty((M, N // 32), np.uint8)
        self.L.oc_mxfp8_floor_quantize(_p(w, _u16p), M, N, _p(q, _u8p), _p(e, _u8p))
        return q, e

    def mxfp8_dequantize(self, q: np.ndarray, e: np.ndarray) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        e = np.ascontiguousarray(e, dtype=np.uint8)
        M, N = q.shape
        assert e.shape == (M, N // 32)
        y = np.empty((M, N), np.uint16)
        self.L.oc_mxfp8_dequantize(_p(q, _u8p), _p(e, _u8p), M, N, _p(y, _u16p))
        return y

    # ------------------------------------------------------------------ NVFP4
    def amax(self, w: np.ndarray) -> float:
        w = np.ascontiguousarray(w, dtype=np.uint16)
        return float(self.L.oc_amax_bf16(_p(w, _u16p), w.size))

    def nvfp4_global_scale(self, A: float, e4m3_max: int = 448) -> float:
        if e4m3_max == 448:
            return float(self.L.oc_nvfp4_global_scale(float(A)))
        return float(self.L.oc_nvfp4_global_scale_max(float(A), int(e4m3_max)))

    def nvfp4_global_scale_reciprocal(self, A: float) -> float:
        return float(self.L.oc_nvfp4_global_scale_reciprocal(float(A)))

    def nvfp4_block_scale(self, b: float, g: float) -> int:
        return int(self.L.oc_nvfp4_block_scale(float(b), float(g)))

    def nvfp4_effective_scale(self, scode: int, g: float) -> float:
        return float(self.L.oc_nvfp4_effective_scale(int(scode), float(g)))

    def nvfp4_quantize(self, w: np.ndarray, g: float):
        """BF16 [M,N] (N % 16 == 0) under global scale g -> (packed [M,N/2], E4M3 block scales [M,N/16])."""
        w = _bf16(w)
        M, N = w.shape
        assert N % 16 == 0
        p = np.empty((M, N // 2), np.uint8)
        s = np.empty((M, N // 16), np.uint8)
        self.L.oc_nvfp4_quantize(_p(w, _u16p), M, N, float(g), _p(p, _u8p), _p(s, _u8p))
        return p, s

    def nvfp4_dequantize(self, p: np.ndarray, s: np.ndarray, g: float) -> np.ndarray:
        p = np.ascontiguousarray(p, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.uint8)
        M, N = p.shape[0], p.shape[1] * 2
        assert s.shape == (M, N // 16)
        y = np.empty((M, N), np.uint16)
        self.L.oc_nvfp4_dequantize(_p(p, _u8p), _p(s, _u8p), float(g), M, N, _p(y, _u16p))
        return y

    def nvfp4_qdq(self, x: np.ndarray, g: float) -> np.ndarray:
        x = _bf16(x)
        M, N = x.shape
        assert N % 16 == 0
        y = np.empty((M, N), np.uint16)
        self.L.oc_nvfp4_qdq(_p(x, _u16p), M, N, float(g), _p(y, _u16p))
        return y

    # ------------------------------------------------------------------ INT4, group-wise ("INT4 QAT 训练")
    INT4_GROUPS = (32, 128)

    def int4_scale(self, amax: float) -> float:
        return float(self.L.oc_int4_scale(float(amax)))

    def int4_quantize(self, w: np.ndarray, group: int):
        """BF16 [M,N] (N % group == 0) -> (packed [M,N/2] two's-complement nibbles, FP32 scales [M,N/group])."""
        w = _bf16(w)
        M, N = w.shape
        assert group in self.INT4_GROUPS and N % group == 0
        p = np.empty((M, N // 2), np.uint8)
        s = np.empty((M, N // group), np.float32)
        self.L.oc_int4_quantize(_p(w, _u16p), M, N, group, _p(p, _u8p), _p(s, _f32p))
        return p, s

    def int4_dequantize(self, p: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
        p = np.ascontiguousarray(p, dtype=np.uint8)
        s = np.ascontiguousarray(s, dtype=np.float32)
        M, N = p.shape[0], p.shape[1] * 2
        assert group in self.INT4_GROUPS and s.shape == (M, N // group)
        y = np.empty((M, N), np.uint16)
        self.L.oc_int4_dequantize(_p(p, _u8p), _p(s, _f32p), M, N, group, _p(y, _u16p))
        return y

    def int4_qdq(self, x: np.ndarray, group: int) -> np.ndarray:
        x = _bf16(x)
        M, N = x.shape
        assert group in self.INT4_GROUPS and N % group == 0
        y = np.empty((M, N), np.uint16)
        self.L.oc_int4_qdq(_p(x, _u16p), M, N, group, _p(y, _u16p))
        return y

    # ------------------------------------------------------------------ W4A4 activation observers
    OBSERVERS = {"memoryless_minmax": 0, "static_minmax": 1, "minmax": 2}

    def observer_update(self, kind: str, state: np.ndarray, x: np.ndarray, c: float = 0.01) -> float:
        """Update ``state`` (float32 [3]: min, max, batches seen) with the BF16 batch ``x``
        under the named observer; returns the activation amax max(|min|, |max|)."""
        assert state.dtype == np.float32 and state.shape == (3,) and state.flags["C_CONTIGUOUS"]
        x = np.ascontiguousarray(x, dtype=np.uint16)
        assert x.size > 0
        return float(self.L.oc_observer_update(self.OBSERVERS[kind], float(c), _p(state, _f32p),
                                               _p(x, _u16p), x.size))

    def nvfp4_group_scale(self, members, e4m3_max: int = 448) -> tuple[float, float]:
        """Sibling group: A = max over every member's amax, g = fl(A / (6 * e4m3_max))."""
        A = max(self.amax(m) for m in members) if members else 0.0
        return A, self.nvfp4_global_scale(A, e4m3_max)

    def nvfp4_quantize_group(self, members, e4m3_max: int = 448):
        """Quantize the tensors of one sibling group under their shared global scale.

        Returns (A, g, [(packed, scales), ...])."""
        A, g = self.nvfp4_group_scale(members, e4m3_max)
        return A, g, [self.nvfp4_quantize(m, g) for m in members]

    # ------------------------------------------------------------------ re-quantization of FP8 weights
    # "低精度训练与 Rollout" (vime and slime documentation), section
    # "FP8 训练 + FP8 Rollout", implementation note 3: with FP8 training, the
    # weight update first turns the trainer's block-wise FP8 weights back into
    # BF16 and then quantizes that BF16 tensor for the rollout engine.  The
    # oracle is that composition, step by step, with nothing fused.
    def fp8blk_requantize_fp8blk(self, q: np.ndarray, s: np.ndarray):
        """Block-wise FP8 (codes, tile scales) -> BF16 -> block-wise FP8 (codes, new tile scales)."""
        return self.fp8blk_quantize(self.fp8blk_dequantize(q, s))

    def fp8blk_requantize_mxfp8(self, q: np.ndarray, s: np.ndarray):
        """Block-wise FP8 (codes, tile scales) -> BF16 -> MXFP8 (codes, UE8M0 bytes)."""
        return self.mxfp8_quantize(self.fp8blk_dequantize(q, s))

    def fp8blk_amax(self, q: np.ndarray, s: np.ndarray) -> float:
        """max |y| of the dequantized BF16 tensor y (the NVFP4 amax of the re-quantized weight)."""
        return self.amax(self.fp8blk_dequantize(q, s))

    def fp8blk_requantize_nvfp4_group(self, members):
        """One sibling group of block-wise FP8 tensors [(q, s), ...] -> BF16 -> NVFP4 under the
        group's shared global scale.  Returns (A, g, [(packed, scales), ...])."""
        return self.nvfp4_quantize_group([self.fp8blk_dequantize(q, s) for q, s in members])


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(build())
    return _default


def __getattr__(name):
    # module-level access to the default oracle's methods: oracle.fp8blk_quantize(...)
    if hasattr(Oracle, name) and not name.startswith("_"):
        return getattr(default(), name)
    raise AttributeError(name)


# --------------------------------------------------------------------------- threading

def run_parallel(fn, items, threads: int):
    """Run ``fn`` over independent items on ``threads`` host threads (ctypes drops the GIL)."""
    if threads <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))
