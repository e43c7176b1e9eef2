"""Seeded synthetic weights and activations (host side, numpy).

This module holds none of the quantization arithmetic: it only draws BF16
inputs.  Both the CPU oracle and the GPU path consume what it produces, and
``synth_gen.hip`` is its bit-identical GPU twin for full-size workloads (the
twin is checked against this file by a GPU test).

Recipe (a stand-in for the trained checkpoints the pages train on, which are
not available):

  w[r, c] = sigma * z[r, c] * rowf[r] * (factor if outlier[r, c] else 1)

* z: a standard normal variate approximated by the Irwin-Hall sum of twelve
  32-bit uniforms minus 6 (mean 0, variance 1, support +-6).  Only integer
  operations and exactly rounded float64 additions/multiplications are used,
  so numpy and the GPU produce identical bits.
* rowf: lognormal(0, row_sigma) per output row, exp(row_sigma * z_row), with
  exp evaluated by a fixed range reduction and Taylor polynomial in float64
  basic operations (again bit-reproducible on both sides).  row_sigma = 0
  gives rowf = 1.
* outlier: Bernoulli(outlier_p) per element, multiplying by ``factor``.
* The float64 product is rounded to float32, then to BF16, both to nearest
  even.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) used counter-style: the k-th
output of the stream with key K is mix(K + (k + 1) * GAMMA).
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB
TAG_ROW = 0x524F57F4C7A1B2C3
TAG_OUT = 0x4F55544C49455221

# exp(): y = k*ln2 + f, |f| <= ln2/2; ln2 split so that k*LN2_HI is exact for |k| < 2^11.
INV_LN2 = 1.4426950408889634
LN2_HI = 0.6931471803691238      # 0x3FE62E42FEE00000
LN2_LO = 1.9082149292705877e-10  # ln2 - LN2_HI
EXP_TERMS = 14


def _mix_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MUL1) & MASK64
    z = ((z ^ (z >> 27)) * MUL2) & MASK64
    return z ^ (z >> 31)


def _mix(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=False)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MUL1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MUL2)
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> int:
    """Key of one tensor's stream: a hash of (seed, stream)."""
    return _mix_int((seed * GAMMA + stream) & MASK64)


def _draw(key: int, counter: np.ndarray) -> np.ndarray:
    c = counter.astype(np.uint64, copy=False)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(key) + (c + np.uint64(1)) * np.uint64(GAMMA))


def _irwin_hall12(key: int, idx: np.ndarray) -> np.ndarray:
    """Approximate N(0,1): sum of 12 uniforms from 6 draws per index, minus 6."""
    base = idx.astype(np.uint64) * np.uint64(6)
    total = np.zeros(idx.shape, np.uint64)
    for j in range(6):
        d = _draw(key, base + np.uint64(j))
        total += (d >> np.uint64(32)) + (d & np.uint64(0xFFFFFFFF))
    centred = total.astype(np.int64) - np.int64(6 << 32)
    return centred.astype(np.float64) * 2.0 ** -32


def exp_det(y: np.ndarray) -> np.ndarray:
    """exp(y) from float64 basic operations only (bit-reproducible)."""
    y = np.asarray(y, np.float64)
    k = np.rint(y * INV_LN2)
    f = (y - k * LN2_HI) - k * LN2_LO
    p = np.ones_like(f)
    for n in range(EXP_TERMS, 0, -1):          # Horner: 1 + f/1 (1 + f/2 (1 + ...))
        p = 1.0 + (f / float(n)) * p
    return np.ldexp(p, k.astype(np.int64))


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x32, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def row_factors(seed: int, stream: int, rows: np.ndarray, row_sigma: float) -> np.ndarray:
    if row_sigma == 0.0:
        return np.ones(rows.shape, np.float64)
    rk = _mix_int(stream_key(seed, stream) ^ TAG_ROW)
    return exp_det(row_sigma * _irwin_hall12(rk, rows))


def generate(seed: int, stream: int, M: int, N: int, sigma: float, row_sigma: float,
             outlier_p: float, outlier_factor: float, rows=None, cols=None) -> np.ndarray:
    """BF16 bit patterns of the tensor (or of the sub-block rows x cols of it)."""
    rows = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    cols = np.arange(N, dtype=np.int64) if cols is None else np.asarray(cols, np.int64)
    key = stream_key(seed, stream)
    idx = rows[:, None] * np.int64(N) + cols[None, :]
    z = _irwin_hall12(key, idx)
    w = (sigma * z) * row_factors(seed, stream, rows, row_sigma)[:, None]
    if outlier_p > 0.0:
        ok = _mix_int(key ^ TAG_OUT)
        u = (_draw(ok, idx) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        w = w * np.where(u < outlier_p, outlier_factor, 1.0)
    return f32_to_bf16_bits(w.astype(np.float32))


def random_bytes(seed: int, stream: int, n: int, exclude=()) -> np.ndarray:
    """n uniform bytes from the (seed, stream) stream, skipping the values in
    ``exclude`` (redrawn from the next counter block)."""
    key = stream_key(seed, stream)
    out = np.empty(0, np.uint8)
    base = 0
    while out.size < n:
        m = max(n - out.size, 64)
        b = (_draw(key, np.arange(base, base + m, dtype=np.uint64)) >> np.uint64(56)).astype(np.uint8)
        if exclude:
            b = b[~np.isin(b, np.asarray(exclude, np.uint8))]
        out = np.concatenate([out, b])
        base += m
    return out[:n]


def e4m3_codes(seed: int, stream: int, M: int, N: int) -> np.ndarray:
    """[M, N] float8_e4m3fn bit patterns, uniform over the 254 that are not NaN
    (0x7F and 0xFF are the format's only NaNs)."""
    return random_bytes(seed, stream, M * N, exclude=(0x7F, 0xFF)).reshape(M, N)


def random_f32(seed: int, stream: int, shape, lo_exp: int, hi_exp: int, signed: bool = False) -> np.ndarray:
    """float32 values 1.m * 2^e with a uniform 23-bit m and e uniform in [lo_exp, hi_exp]
    (normal floats; subnormal exponents are not produced)."""
    n = int(np.prod(shape))
    d = _draw(stream_key(seed, stream), np.arange(n, dtype=np.uint64))
    mant = (d & np.uint64(0x7FFFFF)).astype(np.uint32)
    span = hi_exp - lo_exp + 1
    e = ((d >> np.uint64(23)) % np.uint64(span)).astype(np.int64) + lo_exp
    assert -126 <= lo_exp and hi_exp <= 127
    bits = ((e + 127).astype(np.uint32) << np.uint32(23)) | mant
    if signed:
        bits |= ((d >> np.uint64(63)).astype(np.uint32) << np.uint32(31))
    return bits.view(np.float32).reshape(shape)


# --------------------------------------------------------------------------- named workloads

# (sigma, row_sigma, outlier_p, outlier_factor) of each distribution named by the workloads.
DIST_DENSE = (0.02, 0.5, 0.0, 1.0)          # N(0, 0.02) x lognormal(0, 0.5) per row
DIST_MOE = (0.02, 0.5, 0.001, 50.0)         # ... plus 0.1 % outliers x 50
DIST_ACT = (1.0, 0.0, 0.0001, 100.0)        # N(0, 1) tokens, 0.01 % outliers x 100


def seed_of(config: int) -> int:
    return 0x5EED0000 + config


def stream_of(layer: int, expert: int, proj: int) -> int:
    """Stream id of one tensor: (layer, expert, projection) packed into 64 bits."""
    return ((layer & 0xFFFF) << 40) | ((expert & 0xFFFFFF) << 16) | (proj & 0xFFFF)


def single_linear(config: int = 1) -> np.ndarray:
    """The 256 x 512 parity weight: MoE distribution, and tile (1, 1) of the 128 x 128
    grid (rows 128-255, columns 128-255) set to +0."""
    w = generate(seed_of(config), stream_of(0, 0, 0), 256, 512, *DIST_MOE)
    w[128:256, 128:256] = 0
    return w
