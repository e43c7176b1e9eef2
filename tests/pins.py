"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function takes an oracle instance (``oracle.oracle.Oracle``)
and raises AssertionError on failure.  ``test_oracle_pins.py`` runs them on
the oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with
planted mistakes and requires every mistake to be caught.

Independent routes used here (none re-types the oracle's own arithmetic):
  * E4M3 decoding comes from PyTorch's float8_e4m3fn dtype (a library);
  * nearest-with-ties-to-even is decided by comparing against grid midpoints
    in float64, where every quantity involved is exact;
  * BF16 rounding is cross-checked against PyTorch's CPU cast;
  * the MXFP8 exponent is checked against a closed form read off the bits;
  * block formats are checked on inputs built to be exactly representable,
    where the whole round trip must be the identity and every scale is a
    known power of two (a different power per tile/block, so that tile and
    block indexing is exercised), on hand-worked examples whose values were
    derived from the printed formulas, and on invariants (QDQ equals
    dequantize-of-quantize, idempotence, sibling sharing, nearest-code).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------- helpers

def f32_bits(x) -> np.ndarray:
    return np.asarray(x, np.float32).view(np.uint32)


def bf16_f32(w) -> np.ndarray:
    return (np.asarray(w, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_torch(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def all_finite_bf16() -> np.ndarray:
    """The 65,280 finite BF16 bit patterns (both zeros, subnormals included)."""
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = bf16_f32(u)
    return u[np.isfinite(f)]


def e4m3_table():
    """Decoded value of every E4M3 code, from PyTorch's float8_e4m3fn."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def e4m3_positive_grid():
    vals = e4m3_table()[:0x7F]          # codes 0x00..0x7E: 0 .. 448, increasing
    return vals.astype(np.float64), np.arange(0x7F, dtype=np.int64)


def read_grid_file() -> np.ndarray:
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_grid.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                vals.append(float(line))
    return np.array(vals, np.float64)


def read_constants() -> dict:
    out = {}
    with open(os.path.join(GOLDEN, "format_constants.txt")) as f:
        for line in f:
            line = line.split("--")[0].split("#")[0].strip()
            if line:
                k, v = line.split()[:2]
                out[k] = float(v)
    return out


def nearest_even_codes(v, grid, codes) -> np.ndarray:
    """Code of the grid point nearest to |v| (ties to the even code, saturating at
    the top of the grid), with the sign bit supplied by the caller.  float64
    comparisons against midpoints of neighbouring grid points are exact here."""
    a = np.abs(np.asarray(v, np.float64))
    hi = np.searchsorted(grid, a, side="left")           # first grid point >= a
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = grid[hi] == a
    mid = (grid[lo] + grid[hi]) / 2.0
    pick_lo = a < mid
    pick_hi = a > mid
    tie_lo = (codes[lo] % 2) == 0
    out = np.where(pick_lo, codes[lo], np.where(pick_hi, codes[hi], np.where(tie_lo, codes[lo], codes[hi])))
    out = np.where(exact, codes[hi], out)
    out = np.where(a >= grid[-1], codes[-1], out)
    return out


def midpoint_probes(grid) -> np.ndarray:
    """float32 values at, and one float32 ulp either side of, each grid midpoint."""
    mids = ((grid[1:] + grid[:-1]) / 2.0).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    return np.concatenate([mids, up, dn])


def random_f32(n, seed, lo_exp=-140, hi_exp=12) -> np.ndarray:
    rng = np.random.default_rng(seed)
    m = rng.integers(0, 1 << 23, n, dtype=np.uint32)
    e = rng.integers(max(lo_exp + 127, 0), min(hi_exp + 127, 254), n, dtype=np.uint32)
    s = rng.integers(0, 2, n, dtype=np.uint32)
    return ((s << 31) | (e << 23) | m).view(np.float32)


def rn_f32_of(x: Fraction) -> np.float32:
    """The binary32 value nearest to the exact rational x (ties to even), by comparing
    exact distances to the float32 neighbours of a first guess."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def sign_bit(v) -> np.ndarray:
    return (f32_bits(np.asarray(v, np.float32)) >> 31).astype(np.int64)


# --------------------------------------------------------------------------- scalar pins

def pin_constants(O):
    """The pages' constants: E4M3 max 448, E2M1 max 6, 6 * 448 = 2688."""
    c = read_constants()
    assert c["E4M3_MAX"] == 448.0 and c["E2M1_MAX"] == 6.0
    assert c["NVFP4_GLOBAL_DIVISOR"] == c["E2M1_MAX"] * c["E4M3_MAX"]
    assert O.e4m3_decode(0x7E) == c["E4M3_MAX"] and O.e4m3_decode(0xFE) == -c["E4M3_MAX"]
    assert O.e2m1_decode(7) == c["E2M1_MAX"] and O.e2m1_decode(15) == -c["E2M1_MAX"]
    # global scale of an amax equal to the divisor is exactly one
    assert O.nvfp4_global_scale(c["NVFP4_GLOBAL_DIVISOR"]) == 1.0


def pin_e4m3_decode_library(O):
    """Every non-NaN E4M3 code decodes to PyTorch's float8_e4m3fn value (sign of zero too)."""
    tab = e4m3_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = O.e4m3_decode(c)
        assert f32_bits(np.float32(v)) == f32_bits(tab[c]), (c, v, tab[c])


def pin_e4m3_encode_exact(O):
    """E4M3 encode == nearest E4M3 value, ties to even code, saturating, sign kept:
    on all finite BF16 values, FP32 probes around every midpoint, and random FP32."""
    grid, codes = e4m3_positive_grid()
    v = np.concatenate([bf16_f32(all_finite_bf16()), midpoint_probes(grid), -midpoint_probes(grid),
                        random_f32(200000, 1), np.float32([448.0, 464.0, 479.9, 480.0, 1e30, -1e30, np.inf, -np.inf])])
    want = nearest_even_codes(v, grid, codes) | (sign_bit(v) << 7)
    got = O.e4m3_encode(v).astype(np.int64)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {v[bad[:5]]} got {got[bad[:5]]} want {want[bad[:5]]}"


def pin_e4m3_encode_library(O):
    """E4M3 encode == PyTorch's round-to-nearest cast after clamping to +-448."""
    v = np.concatenate([random_f32(400000, 2, -20, 10), bf16_f32(all_finite_bf16())])
    t = torch.from_numpy(v).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode(v)
    assert np.array_equal(got, t)


def pin_e2m1_table(O):
    """The pages' E2M1 ladder: code k decodes to the k-th grid value, each grid
    value encodes back to its code, anything above 6 saturates to code 7."""
    grid = read_grid_file()
    assert len(grid) == 8 and grid[-1] == read_constants()["E2M1_MAX"]
    for c in range(16):
        want = grid[c & 7] * (-1.0 if c & 8 else 1.0)
        got = O.e2m1_decode(c)
        assert got == want and (np.signbit(got) == bool(c & 8)), (c, got, want)
    assert list(O.e2m1_encode(grid)) == list(range(8))
    assert list(O.e2m1_encode(-grid)) == [8 + k for k in range(8)]
    assert list(O.e2m1_encode([6.0001, 7.0, 100.0, 1e30, -7.0])) == [7, 7, 7, 7, 15]


def pin_e2m1_encode_exact(O):
    """E2M1 encode == nearest grid value, ties to even code, on all finite BF16 values,
    FP32 probes around every midpoint and random FP32."""
    grid = read_grid_file()
    codes = np.arange(8, dtype=np.int64)
    v = np.concatenate([bf16_f32(all_finite_bf16()), midpoint_probes(grid), -midpoint_probes(grid),
                        random_f32(200000, 3, -10, 5)])
    want = nearest_even_codes(v, grid, codes) | (sign_bit(v) << 3)
    got = O.e2m1_encode(v).astype(np.int64)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {v[bad[:5]]} got {got[bad[:5]]} want {want[bad[:5]]}"


def pin_bf16_library(O):
    """FP32 -> BF16 equals PyTorch's CPU cast (nearest even, overflow to Inf)."""
    rng = np.random.default_rng(4)
    u = rng.integers(0, 1 << 32, 400000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    ties = ((rng.integers(0, 1 << 16, 1000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    edge = np.float32([3.3895314e38, 3.3961775e38, 3.4028235e38, -3.4028235e38, 0.0, -0.0, 1e-45, -1e-45])
    v = np.concatenate([v, ties, edge])
    assert np.array_equal(O.f32_to_bf16(v), f32_to_bf16_torch(v))


def pin_mxfp8_byte_closed_form(O):
    """On all 32,640 non-negative finite BF16 amax values: the shared exponent e is the
    smallest integer with amax <= 448 * 2^e (or -127), and equals the closed form read
    off the bits, e + 127 = max(0, Eb - 8 + [m7 > 96]) (448 = 1.75 * 2^8, 0.75 = 96/128)."""
    u = all_finite_bf16()
    u = u[u < 0x8000]
    amax = bf16_f32(u)
    got = O.mxfp8_scale_byte(amax).astype(np.int64)
    Eb = (u.astype(np.int64) >> 7) & 0xFF
    m7 = u.astype(np.int64) & 0x7F
    closed = np.maximum(0, Eb - 8 + (m7 > 96))
    assert np.array_equal(got, closed)
    e = got - 127
    a = amax.astype(np.float64)
    assert np.all(a <= np.ldexp(448.0, e))
    assert np.all((e == -127) | (a > np.ldexp(448.0, e - 1)))
    assert got.max() <= 254


def pin_mxfp8_floor_byte_closed_form(O):
    """The floor rule of the OCP MX specification on all 32,640 non-negative finite BF16
    amax values: byte = max(0, Eb - 8) read off the exponent bits (floor(log2 amax) = Eb - 127
    for normal values, and E4M3's largest exponent is 8); it is the ceiling rule's byte
    whenever the significand is at most 1.75 and one less otherwise."""
    u = all_finite_bf16()
    u = u[u < 0x8000]
    amax = bf16_f32(u)
    got = O.mxfp8_floor_scale_byte(amax).astype(np.int64)
    Eb = (u.astype(np.int64) >> 7) & 0xFF
    m7 = u.astype(np.int64) & 0x7F
    assert np.array_equal(got, np.maximum(0, Eb - 8))
    ceil = O.mxfp8_scale_byte(amax).astype(np.int64)
    big = (m7 > 96) & (Eb >= 8)
    assert np.array_equal(got[~big], ceil[~big]) and np.array_equal(got[big], ceil[big] - 1)


def pin_mxfp8_floor_quantize(O):
    """Floor-rule MXFP8 on blocks of E4M3 values times 2^k: with the block amax in
    [256, 448] * 2^k the byte is 127 + k and every code is the value's own; with one
    element at 480 * 2^k (a BF16 value above E4M3's 448) the byte is still 127 + k, that
    element saturates to 448 and the others keep their codes.  Elsewhere (random MoE-like
    data) each code is the nearest-even E4M3 point of w / 2^(byte-127), saturating."""
    rng = np.random.default_rng(31)
    M, N = 24, 256
    nb = N // 32
    k = rng.integers(-100, 100, (M, nb))
    vals = _e4m3_values(rng, M * N).reshape(M, N)
    vals = np.where(np.abs(vals) > 240.0, vals / 4.0, vals)    # still E4M3 values, all below 256
    sat = rng.integers(0, 2, (M, nb)).astype(bool)
    pos = rng.integers(0, 32, (M, nb))
    for r in range(M):
        for b in range(nb):
            sgn = 1.0 if rng.integers(0, 2) else -1.0
            vals[r, 32 * b + pos[r, b]] = sgn * (480.0 if sat[r, b] else 448.0)
    x = np.ldexp(vals, np.repeat(k, 32, 1)).astype(np.float32)
    w = f32_to_bf16_torch(x).reshape(M, N)
    assert np.array_equal(bf16_f32(w), x)
    q, e = O.mxfp8_floor_quantize(w)
    assert np.array_equal(e.astype(np.int64), 127 + k)
    want = np.clip(vals, -448.0, 448.0)
    assert np.array_equal(e4m3_table()[q].astype(np.float64), want)
    w2 = _moe_like(rng, 16, 128)
    q2, e2 = O.mxfp8_floor_quantize(w2)
    grid, codes = e4m3_positive_grid()
    v = bf16_f32(w2).astype(np.float64) / np.ldexp(1.0, np.repeat(e2.astype(np.int64) - 127, 32, 1))
    mag = nearest_even_codes(v.ravel(), grid, codes).reshape(v.shape)
    assert np.array_equal(q2 & 0x7F, mag)
    assert np.array_equal(q2 >> 7, sign_bit(bf16_f32(w2)))


def pin_nvfp4_e4m3_max_256(O):
    """With E4M3 maximum 256 the global scale is fl(A / 1536): 2^k for A = 1536 * 2^k, and the
    float64 quotient rounded once elsewhere.  A group anchored at A = 1536 * 2^k whose blocks
    hold E2M1 grid values times s_b * 2^k (s_b <= 256, one +-6 per block) round-trips exactly,
    with block-scale codes s_b."""
    rng = np.random.default_rng(34)
    for k in range(-30, 30):
        assert O.nvfp4_global_scale(np.ldexp(1536.0, k), 256) == np.ldexp(1.0, k)
    A = np.abs(random_f32(2000, 35, lo_exp=-120, hi_exp=120)).astype(np.float32)
    got = np.array([O.nvfp4_global_scale(a, 256) for a in A], np.float32)
    want = (A.astype(np.float64) / 1536.0).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    grid = read_grid_file()
    M, N, k = 16, 64, 3
    nb = N // 16
    sb = np.abs(_e4m3_values(rng, M * nb, normal_only=True)).reshape(M, nb)
    sb = np.where(sb > 256.0, sb / 4.0, sb)
    gc = rng.integers(0, 16, (M, N))
    for r in range(M):
        for b in range(nb):
            gc[r, 16 * b + int(rng.integers(0, 16))] = 7 | (8 if rng.integers(0, 2) else 0)
    gv = grid[gc & 7] * np.where(gc & 8, -1.0, 1.0)
    x = np.ldexp(gv * np.repeat(sb, 16, 1), k).astype(np.float32)
    w1 = f32_to_bf16_torch(x).reshape(M, N)
    assert np.array_equal(bf16_f32(w1), x)
    anchor = np.zeros((1, 16), np.float32)
    anchor[0, 2] = np.ldexp(1536.0, k)
    A_, g, outs = O.nvfp4_quantize_group([w1, f32_to_bf16_torch(anchor).reshape(1, 16)], e4m3_max=256)
    assert g == np.ldexp(1.0, k)
    p, s = outs[0]
    assert np.array_equal(e4m3_table()[s].astype(np.float64), sb)
    assert np.array_equal(O.nvfp4_dequantize(p, s, g), w1)


def pin_nvfp4_reciprocal_global_scale(O):
    """fl(2688 / A), the reciprocal form of the global scale: equal to the float64 quotient
    rounded once to binary32 (double rounding of a quotient of binary32 values through a
    53-bit format is harmless, 53 >= 2 * 24 + 2), exactly 2^-k for A = 2688 * 2^k, +Inf for 0."""
    rng = np.random.default_rng(32)
    A = np.concatenate([random_f32(4000, 33, lo_exp=-140, hi_exp=127), np.ldexp(2688.0, np.arange(-20, 20))])
    A = np.abs(A[np.isfinite(A) & (A != 0)]).astype(np.float32)
    got = np.array([O.nvfp4_global_scale_reciprocal(a) for a in A], np.float32)
    with np.errstate(over="ignore"):      # quotients beyond binary32's range round to +Inf
        want = (np.float64(2688.0) / A.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert O.nvfp4_global_scale_reciprocal(0.0) == np.inf
    assert all(O.nvfp4_global_scale_reciprocal(np.ldexp(2688.0, k)) == np.ldexp(1.0, -k) for k in range(-30, 30))


def pin_observers(O):
    """W4A4 activation observers against closed forms: memoryless keeps the last batch's
    extremes, static the extremes of everything seen (numpy min/max of the concatenation);
    the moving average with c = 0 stays at the first batch and with c = 1/2 over batches
    whose max is 2^k after a first batch of zeros reaches 2^k (1 - 2^-(t-1)) exactly;
    -0 orders below +0; amax = max(|min|, |max|)."""
    rng = np.random.default_rng(41)
    batches = [_moe_like(rng, 8, 64, scale=float(sc)) for sc in (0.5, 2.0, 0.1, 1.0, 3.0)]
    f = [bf16_f32(b).astype(np.float64) for b in batches]
    for kind in ("memoryless_minmax", "static_minmax"):
        st = np.zeros(3, np.float32)
        for t, b in enumerate(batches):
            a = O.observer_update(kind, st, b)
            seen = np.concatenate([x.ravel() for x in (f[t:t + 1] if kind == "memoryless_minmax" else f[:t + 1])])
            assert st[0] == seen.min() and st[1] == seen.max() and st[2] == t + 1
            assert a == max(abs(seen.min()), abs(seen.max())) == O.amax(np.concatenate(
                [x.ravel() for x in (batches[t:t + 1] if kind == "memoryless_minmax" else batches[:t + 1])]))
    st = np.zeros(3, np.float32)
    for t, b in enumerate(batches):
        O.observer_update("minmax", st, b, c=0.0)
        assert st[0] == f[0].min() and st[1] == f[0].max()
    for k in (-20, 0, 30):
        st = np.zeros(3, np.float32)
        O.observer_update("minmax", st, np.zeros((2, 16), np.uint16), c=0.5)
        for t in range(2, 20):
            x = np.zeros((2, 16), np.float32)
            x[1, 3], x[0, 5] = np.ldexp(1.0, k), -np.ldexp(1.0, k - 1)
            a = O.observer_update("minmax", st, f32_to_bf16_torch(x).reshape(2, 16), c=0.5)
            assert st[1] == np.ldexp(1.0 - 2.0 ** -(t - 1), k) and st[0] == -np.ldexp(1.0 - 2.0 ** -(t - 1), k - 1)
            assert a == st[1]
    st = np.zeros(3, np.float32)
    O.observer_update("static_minmax", st, np.array([[0x8000, 0x0000]], np.uint16))
    assert st[0] == 0 and np.signbit(st[0]) and st[1] == 0 and not np.signbit(st[1])


# --------------------------------------------------------------------------- worked examples

def _read_examples():
    ex = {}
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            fmt, key, *vals = line.split()
            ex.setdefault(fmt, {})[key] = vals
    return ex


def _num(v):
    return [int(x, 0) if x.startswith("0x") or x.isdigit() else float(x) for x in v]


def _to_bf16(vals) -> np.ndarray:
    return f32_to_bf16_torch(np.float32(vals))


def pin_worked_examples(O):
    ex = _read_examples()
    # NVFP4: the block, in a group with an anchor tensor of amax A
    nv = ex["nvfp4"]
    x = _to_bf16(_num(nv["x"])).reshape(1, 16)
    anchor = _to_bf16([float(nv["A"][0])] + [0.0] * 15).reshape(1, 16)
    A, g, outs = O.nvfp4_quantize_group([x, anchor])
    assert A == float(nv["A"][0]) and g == float(nv["g"][0])
    p, s = outs[0]
    assert int(s[0, 0]) == int(nv["block_scale_code"][0], 0)
    assert O.nvfp4_effective_scale(int(s[0, 0]), g) == float(nv["S"][0])
    codes = _num(nv["codes"])
    want_p = np.array([codes[2 * j] | (codes[2 * j + 1] << 4) for j in range(8)], np.uint8)
    assert np.array_equal(p[0], want_p), (p[0], want_p)
    y = O.nvfp4_dequantize(p, s, g)
    assert np.array_equal(y[0], _to_bf16(_num(nv["y"])))
    assert np.array_equal(O.nvfp4_qdq(x, g)[0], _to_bf16(_num(nv["y"])))
    # MXFP8: one 1x32 block
    mx = ex["mxfp8"]
    xs = _num(mx["x"])
    x = _to_bf16(xs + [0.0] * (32 - len(xs))).reshape(1, 32)
    q, e = O.mxfp8_quantize(x)
    assert int(e[0, 0]) == int(mx["byte"][0])
    assert list(q[0, :len(xs)]) == _num(mx["codes"]) and not q[0, len(xs):].any()
    y = O.mxfp8_dequantize(q, e)
    assert np.array_equal(y[0, :len(xs)], _to_bf16(_num(mx["y"])))
    # block-wise FP8: one tile (a 1 x 5 tensor is a single clipped tile)
    fb = ex["fp8blk"]
    x = _to_bf16(_num(fb["x"])).reshape(1, -1)
    q, s = O.fp8blk_quantize(x)
    assert float(s[0, 0]) == float(fb["s"][0])
    assert list(q[0]) == _num(fb["codes"])
    assert np.array_equal(O.fp8blk_dequantize(q, s)[0], _to_bf16(_num(fb["y"])))


# --------------------------------------------------------------------------- exact round trips

def _e4m3_values(rng, n, normal_only=False):
    tab = e4m3_table()
    pool = np.array([c for c in range(256) if c not in (0x7F, 0xFF) and (not normal_only or (c & 0x78))])
    return tab[rng.choice(pool, n)].astype(np.float64)


def pin_round_trip_fp8blk(O):
    """Tiles built from E4M3 values times 2^k_tile, each holding +-448 * 2^k_tile:
    s == 2^k_tile, the codes are those values, and dequantize returns the input.
    Ragged 300 x 200 tensor (2 x 3 ... partial tiles), a different k per tile."""
    rng = np.random.default_rng(10)
    M, N = 300, 200
    tm, tn = (M + 127) // 128, (N + 127) // 128
    k = rng.integers(-30, 20, (tm, tn))
    vals = _e4m3_values(rng, M * N).reshape(M, N)
    kk = np.repeat(np.repeat(k, 128, 0), 128, 1)[:M, :N]
    for i in range(tm):
        for j in range(tn):
            r, c = 128 * i + int(rng.integers(0, min(128, M - 128 * i))), 128 * j + int(rng.integers(0, min(128, N - 128 * j)))
            vals[r, c] = 448.0 * (1 if rng.integers(0, 2) else -1)
    x = np.ldexp(vals, kk).astype(np.float32)
    w = f32_to_bf16_torch(x).reshape(M, N)
    assert np.array_equal(bf16_f32(w), x), "construction must be BF16-exact"
    q, s = O.fp8blk_quantize(w)
    assert np.array_equal(s, np.ldexp(1.0, k).astype(np.float32))
    want_codes = O.e4m3_encode(vals.astype(np.float32)).reshape(M, N)
    assert np.array_equal(q, want_codes)
    assert np.array_equal(e4m3_table()[q].astype(np.float64), vals)
    assert np.array_equal(O.fp8blk_dequantize(q, s), w)


def pin_round_trip_mxfp8(O):
    """Blocks of E4M3 values times 2^k_block holding +-448 * 2^k_block: byte == 127 + k,
    codes are those values, dequantize returns the input (a different k per block)."""
    rng = np.random.default_rng(11)
    M, N = 37, 256
    nb = N // 32
    k = rng.integers(-100, 100, (M, nb))
    vals = _e4m3_values(rng, M * N).reshape(M, N)
    for r in range(M):
        for b in range(nb):
            vals[r, 32 * b + int(rng.integers(0, 32))] = 448.0 * (1 if rng.integers(0, 2) else -1)
    x = np.ldexp(vals, np.repeat(k, 32, 1)).astype(np.float32)
    w = f32_to_bf16_torch(x).reshape(M, N)
    assert np.array_equal(bf16_f32(w), x)
    q, e = O.mxfp8_quantize(w)
    assert np.array_equal(e.astype(np.int64), 127 + k)
    assert np.array_equal(e4m3_table()[q].astype(np.float64), vals)
    assert np.array_equal(O.mxfp8_dequantize(q, e), w)


def pin_round_trip_nvfp4(O):
    """Group amax A = 2688 * 2^k, so g = 2^k; each block holds E2M1 grid values times
    s_b * 2^k with one +-6 * s_b * 2^k (s_b a normal E4M3 value): the block-scale code
    is s_b's, the element codes are the grid codes, dequantize returns the input."""
    rng = np.random.default_rng(12)
    grid = read_grid_file()
    for k in (-20, 0, 7):
        M, N = 24, 64
        nb = N // 16
        sb = _e4m3_values(rng, M * nb, normal_only=True).reshape(M, nb)
        sb = np.abs(sb)
        gc = rng.integers(0, 16, (M, N))
        gv = grid[gc & 7] * np.where(gc & 8, -1.0, 1.0)
        for r in range(M):
            for b in range(nb):
                gc[r, 16 * b + int(rng.integers(0, 16))] = 7 | (8 if rng.integers(0, 2) else 0)
        gv = grid[gc & 7] * np.where(gc & 8, -1.0, 1.0)
        x = np.ldexp(gv * np.repeat(sb, 16, 1), k).astype(np.float32)
        w1 = f32_to_bf16_torch(x).reshape(M, N)
        assert np.array_equal(bf16_f32(w1), x)
        anchor = np.zeros((2, 32), np.float32)
        anchor[1, 5] = np.ldexp(2688.0, k)
        w2 = f32_to_bf16_torch(anchor).reshape(2, 32)
        A, g, outs = O.nvfp4_quantize_group([w1, w2])
        assert g == np.ldexp(1.0, k)
        p, s = outs[0]
        assert np.array_equal(e4m3_table()[s].astype(np.float64), sb)
        codes = np.empty((M, N), np.int64)
        codes[:, 0::2] = p & 15
        codes[:, 1::2] = p >> 4
        mag_ok = (codes & 7) == (gc & 7)
        sign_ok = ((codes & 8) == (gc & 8)) | ((gc & 7) == 0)
        assert np.all(mag_ok & sign_ok)
        assert np.array_equal(O.nvfp4_dequantize(p, s, g), w1)


# --------------------------------------------------------------------------- exact quotients

# The oracle's divisions (the block-FP8 tile scale and element quotient, the NVFP4
# global scale, block scale and element quotient) are each one correctly rounded
# binary32 operation.  The pins below recompute every such quotient from the exact
# rational value of its operands with integer arithmetic alone, and check the
# oracle's codes and scale bits against it.  Power-of-two scales would hide a
# reciprocal-multiply mistake (x * (1/s) is exact there), so the inputs use scales
# that are not powers of two, including quotients that land exactly on a rounding
# midpoint of the E4M3 or E2M1 grid, where only a correctly rounded quotient gives
# the tie (ties go to the even code).

_F32_EMIN_Q = -149          # exponent of binary32's smallest subnormal step


def rn_f32_ratio(n: int, d: int) -> float:
    """The binary32 value nearest to the rational n / d (d != 0), ties to the even
    significand, returned as a Python float; overflow gives +-inf, and a nonzero
    quotient that rounds to zero keeps its sign.  Integer arithmetic only: the
    24-bit significand is the integer part of n / (d * 2^e) for the right e, and
    the remainder decides the rounding."""
    if d < 0:
        n, d = -n, -d
    neg = n < 0
    n = -n if neg else n
    if n == 0:
        return -0.0 if neg else 0.0

    def split(e):
        num, den = (n, d << e) if e >= 0 else (n << -e, d)
        q, r = divmod(num, den)
        return q, r, den

    e = n.bit_length() - d.bit_length() - 24     # n / (d 2^e) lies in [2^23, 2^25)
    q, r, den = split(e)
    if q >= 1 << 24:
        e += 1
        q, r, den = split(e)
    if e < _F32_EMIN_Q:                          # subnormal result: fixed quantum
        e = _F32_EMIN_Q
        q, r, den = split(e)
    if 2 * r > den or (2 * r == den and q & 1):
        q += 1
    if e > 104 or (e == 104 and q >= 1 << 24):   # at or beyond 2^128
        val = float("inf")
    else:
        val = math.ldexp(q, e)                   # exact: q <= 2^24, e >= -149
    return -val if neg else val


def _ratio(v: float):
    n, d = float(v).as_integer_ratio()
    return n, d


def rn_div_f32(a, b) -> np.ndarray:
    """Elementwise RN32(a / b) of binary32 operands, exactly (b != 0).  The sign of a
    zero quotient is the XOR of the operands' signs, as in IEEE division."""
    a, b = (v.ravel() for v in np.broadcast_arrays(np.asarray(a, np.float64), np.asarray(b, np.float64)))
    out = np.empty(a.size, np.float64)
    for i in range(a.size):
        x, y = float(a[i]), float(b[i])
        if x == 0.0:
            out[i] = math.copysign(0.0, math.copysign(1.0, x) * math.copysign(1.0, y))
            continue
        nx, dx = _ratio(x)
        ny, dy = _ratio(y)
        out[i] = rn_f32_ratio(nx * dy, dx * ny)
    return out.astype(np.float32)


def rn_mul_f32(a, b) -> np.ndarray:
    """Elementwise RN32(a * b) of binary32 operands, exactly."""
    a, b = (v.ravel() for v in np.broadcast_arrays(np.asarray(a, np.float64), np.asarray(b, np.float64)))
    out = np.empty(a.size, np.float64)
    for i in range(a.size):
        x, y = float(a[i]), float(b[i])
        if x == 0.0 or y == 0.0:
            out[i] = math.copysign(0.0, math.copysign(1.0, x) * math.copysign(1.0, y))
            continue
        nx, dx = _ratio(x)
        ny, dy = _ratio(y)
        out[i] = rn_f32_ratio(nx * ny, dx * dy)
    return out.astype(np.float32)


def _e4m3_nearest(t) -> np.ndarray:
    """Saturating nearest-even E4M3 code of binary32 values (sign of zero kept)."""
    grid, codes = e4m3_positive_grid()
    t = np.asarray(t, np.float32)
    return (nearest_even_codes(t, grid, codes) | (sign_bit(t) << 7)).astype(np.uint8)


def _e2m1_nearest(t) -> np.ndarray:
    t = np.asarray(t, np.float32)
    return (nearest_even_codes(t, read_grid_file(), np.arange(8, dtype=np.int64)) | (sign_bit(t) << 3)).astype(np.uint8)


def _short_significands(max_bits: int) -> list:
    """Significands in (1, 2) with at most ``max_bits`` bits after the leading one."""
    return [1.0 + k / 2.0 ** max_bits for k in range(1, 1 << max_bits)]


def _bf16_exact(v) -> bool:
    v = np.float32(v)
    return bool(np.isfinite(v)) and (int(v.view(np.uint32)) & 0xFFFF) == 0


def exact_fp8blk(w: np.ndarray):
    """Block-wise FP8 of a BF16 [M, N] tensor by exact rationals: per tile
    s = RN32(amax / 448); code = E4M3(RN32(x / s)), a signed zero when s = 0;
    y = BF16(RN32(E4M3value * s))."""
    M, N = w.shape
    x = bf16_f32(w)
    tm, tn = (M + 127) // 128, (N + 127) // 128
    pad = np.zeros((tm * 128, tn * 128), np.float32)
    pad[:M, :N] = np.abs(x)
    amax = pad.reshape(tm, 128, tn, 128).max(axis=(1, 3))
    s = rn_div_f32(amax, 448.0).reshape(tm, tn)
    sf = np.repeat(np.repeat(s, 128, 0), 128, 1)[:M, :N]
    nz = sf != 0
    t = np.zeros((M, N), np.float32)
    t[nz] = rn_div_f32(x[nz], sf[nz])
    t[~nz] = np.copysign(np.float32(0), x[~nz])
    q = _e4m3_nearest(t).reshape(M, N)
    y = f32_to_bf16_torch(rn_mul_f32(e4m3_table()[q], sf)).reshape(M, N)
    return q, s, y


def exact_nvfp4(w: np.ndarray, g: float, e4m3_max: int = 448):
    """NVFP4 of a BF16 [M, N] tensor under global scale g by exact rationals: per
    1x16 block with amax b, scode = E4M3(RN32(RN32(b / 6) / g)) (0 when g = 0),
    S = RN32(E4M3value * g), code = E2M1(RN32(x / S)) (a signed zero when S = 0),
    y = BF16(RN32(E2M1value * S)).  Returns (codes [M, N], scodes [M, N/16], y)."""
    M, N = w.shape
    x = bf16_f32(w)
    b = np.abs(x).reshape(M, N // 16, 16).max(-1).ravel()
    if g == 0.0:
        sc = np.zeros(b.size, np.uint8)
    else:
        sc = _e4m3_nearest(rn_div_f32(rn_div_f32(b, 6.0), g))
    S = rn_mul_f32(e4m3_table()[sc], g).reshape(M, N // 16)
    Sf = np.repeat(S, 16, 1)
    nz = Sf != 0
    t = np.zeros((M, N), np.float32)
    t[nz] = rn_div_f32(x[nz], Sf[nz])
    t[~nz] = np.copysign(np.float32(0), x[~nz])
    codes = _e2m1_nearest(t).reshape(M, N)
    grid = read_grid_file()
    val = (grid[codes & 7] * np.where(codes & 8, -1.0, 1.0)).astype(np.float32)
    y = f32_to_bf16_torch(rn_mul_f32(val, Sf)).reshape(M, N)
    return codes, sc.reshape(M, N // 16), y


def _unpack_e2m1(p: np.ndarray) -> np.ndarray:
    codes = np.empty((p.shape[0], p.shape[1] * 2), np.uint8)
    codes[:, 0::2] = p & 15
    codes[:, 1::2] = p >> 4
    return codes


def pin_exact_global_scale(O):
    """g = RN32(A / 2688) on every positive finite BF16 amax (the amax of BF16 weights
    is a BF16 value) and on 20,000 random binary32 A (a caller-supplied or observed
    amax), against the exact rational quotient; likewise A / 1536 (E4M3 maximum 256)
    and the reciprocal export RN32(2688 / A).  Then 2,000 random tensors, whose A is
    recomputed with numpy: the group call reports that A and its exact quotient
    ("verl NVFP4 QAT" 2.3 and 3.3: amax / (6.0 * 448.0))."""
    u = all_finite_bf16()
    A = np.concatenate([bf16_f32(u[(u > 0) & (u < 0x8000)]), np.abs(random_f32(20000, 60, -140, 127))])
    A = A[A > 0]
    got = np.array([O.nvfp4_global_scale(float(a)) for a in A], np.float32)
    assert np.array_equal(f32_bits(got), f32_bits(rn_div_f32(A, 2688.0)))
    got256 = np.array([O.nvfp4_global_scale(float(a), 256) for a in A[::4]], np.float32)
    assert np.array_equal(f32_bits(got256), f32_bits(rn_div_f32(A[::4], 1536.0)))
    rec = np.array([O.nvfp4_global_scale_reciprocal(float(a)) for a in A[::4]], np.float32)
    want = np.array([rn_f32_ratio(2688 * _ratio(a)[1], _ratio(a)[0]) for a in A[::4]], np.float32)
    assert np.array_equal(f32_bits(rec), f32_bits(want))
    rng = np.random.default_rng(61)
    for _ in range(2000):
        m = int(rng.integers(1, 4))
        w = _moe_like(rng, m, 16, float(np.exp(rng.uniform(-60, 60))), 0.05)
        Ar = float(np.abs(bf16_f32(w).astype(np.float64)).max())
        A2, g2 = O.nvfp4_group_scale([w])
        assert A2 == Ar and f32_bits(np.float32(g2)) == f32_bits(rn_div_f32([Ar], 2688.0)[0])


def pin_exact_fp8blk(O):
    """Block-wise FP8 tile scales, codes and dequantized values against exact rationals:
    (1) one 1x128 tile per positive finite BF16 amax (32,640 tiles), scale bits only;
    (2) tiles whose scale s = sigma * 2^k is not a power of two, holding every
    BF16-representable x = m * s for m an E4M3 rounding midpoint (an exact tie that
    only a correctly rounded x / s produces), plus the other grid points times s;
    (3) a MoE-like ragged tensor (0.1% outliers x 50) and tiles of subnormal and
    huge magnitudes, every element."""
    u = all_finite_bf16()
    amax = u[(u > 0) & (u < 0x8000)]
    w = np.zeros((1, 128 * amax.size), np.uint16)
    w[0, ::128] = amax
    w[0, 1::128] = amax | 0x8000          # a negative element of the same magnitude
    _, s = O.fp8blk_quantize(w)
    assert np.array_equal(f32_bits(s[0]), f32_bits(rn_div_f32(bf16_f32(amax), 448.0)))

    grid, _ = e4m3_positive_grid()
    mids = (grid[1:] + grid[:-1]) / 2.0
    rows = []
    rng = np.random.default_rng(62)
    for sigma in _short_significands(3):
        for k in (-20, -3, 0, 5):
            sc = np.ldexp(sigma, k)
            if not _bf16_exact(448.0 * sc):
                continue
            rest = [m * sc for m in mids if _bf16_exact(m * sc)]
            rest += [v * sc for v in grid[1:-1] if _bf16_exact(v * sc)]
            for j in range(0, len(rest), 127):       # every tile holds its amax 448 * s
                vals = np.array([448.0 * sc] + rest[j:j + 127])
                vals *= np.where(rng.integers(0, 2, len(vals)) == 1, -1.0, 1.0)
                rows.append(vals[rng.permutation(len(vals))])
    tiles = np.zeros((len(rows), 128), np.float32)
    for i, r in enumerate(rows):
        tiles[i, :len(r)] = r
    # each row is its own 1 x 128 tile: lay the rows side by side in one row
    wt = f32_to_bf16_torch(tiles.reshape(1, -1)).reshape(1, -1)
    assert np.array_equal(bf16_f32(wt).ravel(), tiles.ravel()), "tie construction must be BF16-exact"
    cases = [wt]
    cases.append(_moe_like(np.random.default_rng(63), 200, 296, 0.02, 0.001))
    cases.append(_moe_like(np.random.default_rng(64), 130, 136, 1e-39, 0.01))
    cases.append(_moe_like(np.random.default_rng(65), 130, 136, 1e34, 0.01))
    for w in cases:
        q, s = O.fp8blk_quantize(w)
        eq, es, ey = exact_fp8blk(w)
        assert np.array_equal(f32_bits(s), f32_bits(es))
        bad = np.nonzero(q != eq)
        assert bad[0].size == 0, f"{bad[0].size} codes differ from the exact quotient"
        assert np.array_equal(O.fp8blk_dequantize(q, s), ey)


def pin_exact_nvfp4(O):
    """NVFP4 block-scale codes, element codes and dequantized values against exact
    rationals, RN32(RN32(b / 6) / g) and RN32(x / S):
    (1) groups whose g = gamma * 2^k is not a power of two, with blocks whose
    RN32(b / 6) / g is an E4M3 rounding midpoint, or whose elements x / S are E2M1
    midpoints (0.25, 0.75, ..., 5): exact ties;
    (2) block scales of (b, g) pairs built so that RN32(b / 6) / g is an E4M3 midpoint;
    (3) a 1-in-4 sample of positive finite BF16 patterns, each in a block with a larger
    anchor and 14 random elements below it;
    (4) MoE-like tensors, tiny and huge magnitudes; the E4M3-256 form on one of them."""
    rng = np.random.default_rng(66)
    grid, _ = e4m3_positive_grid()
    e4_mids = (grid[1:] + grid[:-1]) / 2.0
    e4_normal = grid[grid >= 2.0 ** -6]
    e2 = read_grid_file()
    e2_mids = (e2[1:] + e2[:-1]) / 2.0

    def check(members, e4m3_max=448):
        A, g, outs = O.nvfp4_quantize_group(members, e4m3_max)
        assert A == max(float(np.abs(bf16_f32(m)).max()) for m in members)
        assert f32_bits(np.float32(g)) == f32_bits(rn_div_f32([A], 6.0 * e4m3_max)[0])
        for m, (p, s) in zip(members, outs):
            ec, es, ey = exact_nvfp4(m, g, e4m3_max)
            assert np.array_equal(s, es), f"{np.count_nonzero(s != es)} block scales differ"
            codes = _unpack_e2m1(p)
            assert np.array_equal(codes, ec), f"{np.count_nonzero(codes != ec)} codes differ"
            assert np.array_equal(O.nvfp4_dequantize(p, s, g), ey)
            assert np.array_equal(O.nvfp4_qdq(m, g), ey)

    # (1) exact ties under g = gamma * 2^k
    for gamma in _short_significands(3):
        for k in (-24, -7, 0):
            gk = np.ldexp(gamma, k)
            if not _bf16_exact(2688.0 * gk):
                continue
            blocks = []
            for m in e4_mids[40:]:                  # block-scale ties: b = 6 * m * g
                b = 6.0 * m * gk
                if _bf16_exact(b):
                    blocks.append([b] + [0.0] * 15)
            for v in e4_normal[::3]:                # element ties: x = mu * v * g
                S = v * gk
                if not _bf16_exact(6.0 * S):
                    continue
                xs = [6.0 * S] + [mu * S for mu in e2_mids if _bf16_exact(mu * S)]
                xs += [mu * S for mu in e2[1:7] if _bf16_exact(mu * S)]
                blocks.append((xs + [0.0] * 16)[:16])
            if not blocks:
                continue
            x = np.array(blocks, np.float64)
            x *= np.where(rng.integers(0, 2, x.shape) == 1, -1.0, 1.0)
            w = f32_to_bf16_torch(x.astype(np.float32)).reshape(x.shape)
            assert np.array_equal(bf16_f32(w), x.astype(np.float32)), "tie construction must be BF16-exact"
            anchor = np.zeros((1, 16), np.float32)
            anchor[0, 3] = 2688.0 * gk
            check([w, f32_to_bf16_torch(anchor).reshape(1, 16)])

    # (2) block-scale ties from the first division: b is any BF16 value whose RN32(b / 6)
    # has an integer significand divisible by the odd part o of an E4M3 midpoint m;
    # then g = RN32(b / 6) / m is exact and RN32(b / 6) / g = m, a tie only when both
    # divisions are correctly rounded in this order.
    u = all_finite_bf16()
    bs = bf16_f32(u[(u > 0) & (u < 0x8000)])
    bs = bs[(bs > 2.0 ** -100) & (bs < 2.0 ** 100)]
    t1 = rn_div_f32(bs[::7], 6.0)
    pairs = []
    for b, t in zip(bs[::7], t1):
        n, d = _ratio(float(t))
        for m in e4_mids[40:120:3]:
            mn, md = _ratio(float(m))
            if n % mn == 0:
                g = np.float32(float(t) / float(m))
                if float(g) * float(m) == float(t):
                    pairs.append((float(b), float(g)))
    assert len(pairs) > 500
    pb = np.array([p_[0] for p_ in pairs], np.float32)
    pg = np.array([p_[1] for p_ in pairs], np.float32)
    got = np.array([O.nvfp4_block_scale(float(b), float(g)) for b, g in pairs], np.uint8)
    want = _e4m3_nearest(rn_div_f32(rn_div_f32(pb, 6.0), pg))
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} block-scale codes differ"

    # (3) a sample of positive finite BF16 patterns p, each in a block with a seeded
    # larger anchor and 14 random elements below it; blocks sorted by anchor and
    # quantized 256 to a group, so that every group spans a few binades
    pats = bf16_f32(u[(u > 0) & (u < 0x7B00)][::4]).astype(np.float64)      # anchors stay below 2^126
    a = pats * rng.uniform(1.0, 64.0, pats.size)
    rows = np.concatenate([a[:, None], pats[:, None], rng.uniform(-1.0, 1.0, (pats.size, 14)) * a[:, None]], 1)
    rows *= np.where(rng.integers(0, 2, rows.shape) == 1, -1.0, 1.0)
    rows = rows[np.argsort(a)].astype(np.float32)
    for j in range(0, rows.shape[0], 256):
        check([f32_to_bf16_torch(rows[j:j + 256]).reshape(-1, 16)])

    # (4) MoE-like tensors and extreme magnitudes
    check([_moe_like(np.random.default_rng(67), 96, 512, 0.02, 0.001)])
    check([_moe_like(np.random.default_rng(68), 32, 256, 1e-38, 0.01)])
    check([_moe_like(np.random.default_rng(69), 32, 256, 1e34, 0.01)])
    check([_moe_like(np.random.default_rng(70), 32, 256, 0.02, 0.001)], 256)


# --------------------------------------------------------------------------- invariants on random data

def _moe_like(rng, M, N, scale=0.02, p_out=0.01, factor=50.0):
    z = rng.standard_normal((M, N)) * scale * np.exp(0.5 * rng.standard_normal((M, 1)))
    z = z * np.where(rng.random((M, N)) < p_out, factor, 1.0)
    return f32_to_bf16_torch(z.astype(np.float32)).reshape(M, N)


def pin_nearest_fp8blk(O):
    """Every code is the E4M3 value nearest to x / s (up to the FP32 rounding of the
    quotient), the tile max lands on +-448, and s is a multiple of its tile's
    amax by 1/448 within one FP32 rounding."""
    rng = np.random.default_rng(13)
    M, N = 200, 300
    w = _moe_like(rng, M, N)
    q, s = O.fp8blk_quantize(w)
    x = bf16_f32(w).astype(np.float64)
    tab = e4m3_table().astype(np.float64)
    sf = np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:M, :N]
    qq = x / sf
    grid, _ = e4m3_positive_grid()
    d_chosen = np.abs(tab[q] - qq)
    d_best = np.min(np.abs(np.abs(qq)[..., None] - grid[None, None, :]), axis=-1)
    assert np.all(d_chosen <= d_best + 2.0 ** -22 * np.abs(qq))
    assert np.all(np.sign(tab[q]) * np.sign(qq) >= 0)
    pad = np.zeros((256, 384))
    pad[:M, :N] = np.abs(x)
    tmax = pad.reshape(2, 128, 3, 128).max(axis=(1, 3))
    assert np.all(np.abs(s.astype(np.float64) * 448.0 / tmax - 1.0) <= 2.0 ** -23)


def pin_nearest_mxfp8(O):
    """Every code is the E4M3 value nearest to x * 2^-e, and no element saturates."""
    rng = np.random.default_rng(14)
    M, N = 64, 512
    w = _moe_like(rng, M, N)
    q, e = O.mxfp8_quantize(w)
    x = bf16_f32(w).astype(np.float64)
    qq = x * np.ldexp(1.0, 127 - np.repeat(e.astype(np.int64), 32, 1))
    assert np.all(np.abs(qq) <= 448.0)
    tab = e4m3_table().astype(np.float64)
    grid, _ = e4m3_positive_grid()
    d_chosen = np.abs(tab[q] - qq)
    d_best = np.min(np.abs(np.abs(qq)[..., None] - grid[None, None, :]), axis=-1)
    assert np.all(d_chosen <= d_best)


def pin_nearest_nvfp4(O):
    """Every element code is the E2M1 value nearest to x / S; each block's largest
    element lands within the E4M3 rounding of the block scale of 6 (normal scales)."""
    rng = np.random.default_rng(15)
    M, N = 64, 256
    w = _moe_like(rng, M, N)
    A, g, [(p, s)] = O.nvfp4_quantize_group([w])
    grid = read_grid_file()
    x = bf16_f32(w).astype(np.float64)
    S = np.array([[O.nvfp4_effective_scale(int(c), g) for c in row] for row in s])
    Sf = np.repeat(S, 16, 1)
    codes = np.empty((M, N), np.int64)
    codes[:, 0::2] = p & 15
    codes[:, 1::2] = p >> 4
    val = grid[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    nz = Sf > 0
    qq = np.where(nz, x / np.where(nz, Sf, 1.0), 0.0)
    d_best = np.min(np.abs(np.abs(qq)[..., None] - grid[None, None, :]), axis=-1)
    assert np.all(np.abs(val - qq) <= d_best + 2.0 ** -22 * np.abs(qq))
    tab = e4m3_table()
    normal = (s & 0x78) != 0
    bmax = np.abs(x).reshape(M, N // 16, 16).max(-1)
    ratio = bmax[normal] / S[normal]
    assert np.all((ratio >= 6.0 / (1 + 2.0 ** -4) * (1 - 2.0 ** -20)) & (ratio <= 6.0 / (1 - 2.0 ** -4) * (1 + 2.0 ** -20)))
    assert A == np.abs(x).max()
    assert np.all(tab[s] >= 0)


def pin_sibling_sharing(O):
    """Members of a sibling group share one global scale, the largest of the members'
    own scales (fl(. / 2688) is monotone), and the group amax is the members' max."""
    rng = np.random.default_rng(16)
    q = _moe_like(rng, 64, 128, 0.02, 0.0)
    k = _moe_like(rng, 16, 128, 0.05, 0.0)
    v = _moe_like(rng, 16, 128, 0.01, 0.0)
    members = [q, k, v]
    A, g, outs = O.nvfp4_quantize_group(members)
    solo = [O.nvfp4_group_scale([m])[1] for m in members]
    assert g == max(solo)
    assert A == max(float(np.abs(bf16_f32(m)).max()) for m in members)
    for m, (p, s) in zip(members, outs):
        p2, s2 = O.nvfp4_quantize(m, g)
        assert np.array_equal(p, p2) and np.array_equal(s, s2)


def pin_qdq_equals_dequant_quant(O):
    """Fake quantization equals dequantize(quantize(x)) bit for bit."""
    rng = np.random.default_rng(17)
    for M, N, sc in ((32, 128, 0.02), (8, 2048, 1.0), (16, 64, 1e-30)):
        x = _moe_like(rng, M, N, sc)
        _, g = O.nvfp4_group_scale([x])
        p, s = O.nvfp4_quantize(x, g)
        assert np.array_equal(O.nvfp4_qdq(x, g), O.nvfp4_dequantize(p, s, g))


def pin_idempotence(O):
    """QDQ(QDQ(x)) == QDQ(x) on blocks whose E4M3 scale is zero or normal;
    FP8 block: quantize(dequantize(quantize(x))) == quantize(x);
    MXFP8: dequantize(quantize(.)) is idempotent on values."""
    rng = np.random.default_rng(18)
    x = _moe_like(rng, 64, 256)
    _, g = O.nvfp4_group_scale([x])
    y = O.nvfp4_qdq(x, g)
    _, g2 = O.nvfp4_group_scale([y])
    z = O.nvfp4_qdq(y, g2)
    _, s = O.nvfp4_quantize(x, g)
    ok = np.repeat((s == 0) | ((s & 0x78) != 0), 16, 1)
    assert np.array_equal(z[ok], y[ok])
    q, sc = O.fp8blk_quantize(x)
    q2, sc2 = O.fp8blk_quantize(O.fp8blk_dequantize(q, sc))
    assert np.array_equal(q, q2) and np.array_equal(sc, sc2)
    qm, em = O.mxfp8_quantize(x)
    y1 = O.mxfp8_dequantize(qm, em)
    y2 = O.mxfp8_dequantize(*O.mxfp8_quantize(y1))
    assert np.array_equal(y1, y2)


def pin_zero_and_sign(O):
    """All-zero tiles/blocks/groups and negative zeros round-trip exactly, with the sign
    of zero kept in codes and outputs; a zero global scale zeroes every block scale."""
    w = np.zeros((128, 128), np.uint16)
    w[::3, ::5] = 0x8000                              # -0
    q, s = O.fp8blk_quantize(w)
    assert s[0, 0] == 0.0 and np.array_equal(q, np.where(w == 0x8000, 0x80, 0).astype(np.uint8))
    assert np.array_equal(O.fp8blk_dequantize(q, s), w)
    q, e = O.mxfp8_quantize(w)
    assert not e.any() and np.array_equal(q, np.where(w == 0x8000, 0x80, 0).astype(np.uint8))
    assert np.array_equal(O.mxfp8_dequantize(q, e), w)
    A, g, [(p, s)] = O.nvfp4_quantize_group([w])
    assert A == 0.0 and g == 0.0 and not s.any()
    assert np.array_equal(O.nvfp4_dequantize(p, s, g), w)
    assert np.array_equal(O.nvfp4_qdq(w, g), w)
    # negative values whose code rounds to zero keep the sign bit
    x = f32_to_bf16_torch(np.float32([-1e-4] + [0.0] * 14 + [448.0])).reshape(1, 16)
    q, s = O.fp8blk_quantize(x)
    assert q[0, 0] == 0x80
    anchor = f32_to_bf16_torch(np.float32([2688.0] + [0.0] * 15)).reshape(1, 16)
    _, g, [(p, s), _] = O.nvfp4_quantize_group([x, anchor])
    assert (p[0, 0] & 15) == 8


def pin_config1_layout(O):
    """The parity weight of the single-Linear workload: its zero tile has scale 0 and
    zero codes in every format."""
    from synth import synth
    w = synth.single_linear()
    q, s = O.fp8blk_quantize(w)
    assert s[1, 1] == 0.0 and not q[128:256, 128:256].any() and (s[0, 0] > 0) and (s[1, 2] > 0)
    q, e = O.mxfp8_quantize(w)
    assert not e[128:, 4:8].any() and not q[128:, 128:256].any()
    _, g, [(p, s)] = O.nvfp4_quantize_group([w])
    assert not s[128:, 8:16].any() and not p[128:, 64:128].any()


# --------------------------------------------------------------------------- re-quantization of FP8 weights

def pin_requant_mxfp8_identity(O):
    """Block-wise FP8 tensor with a power-of-two scale 2^k per tile (a different k per
    tile, ragged 200 x 320 so that the last tile column is 64 wide) and a +-448 code
    in every 1x32 block: the dequantized BF16 values are code * 2^k exactly, so the
    MXFP8 re-quantization keeps every code and sets each byte to 127 + k of its tile."""
    rng = np.random.default_rng(21)
    M, N = 200, 320
    tm, tn = (M + 127) // 128, (N + 127) // 128
    k = rng.integers(-100, 100, (tm, tn))
    tab = e4m3_table()
    pool = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    q = rng.choice(pool, (M, N)).astype(np.uint8)
    for r in range(M):
        for b in range(N // 32):
            q[r, 32 * b + int(rng.integers(0, 32))] = 0x7E | (0x80 if rng.integers(0, 2) else 0)
    s = np.ldexp(1.0, k).astype(np.float32)
    qo, e = O.fp8blk_requantize_mxfp8(q, s)
    kk = np.repeat(np.repeat(k, 128, 0), 128, 1)[:M, :N]
    assert np.array_equal(e.astype(np.int64), (127 + kk)[:, ::32])
    assert np.array_equal(qo, q)
    y = O.fp8blk_dequantize(q, s)
    assert np.array_equal(bf16_f32(y).astype(np.float64), np.ldexp(tab[q].astype(np.float64), kk))


def pin_requant_fp8blk(O):
    """Block-wise FP8 -> BF16 -> block-wise FP8.  With a power-of-two scale 2^k per tile and a
    +-448 code in every tile, the BF16 values are code * 2^k exactly, so the new scale is 2^k
    and the codes come back unchanged.  With a tile scale s that is not a power of two, the
    new scale is fl(BF16(448 * s) / 448) (the tile holds a 448 code), worked here in float64
    from PyTorch's BF16 cast."""
    rng = np.random.default_rng(23)
    M, N = 300, 200
    tm, tn = (M + 127) // 128, (N + 127) // 128
    pool = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    q = rng.choice(pool, (M, N)).astype(np.uint8)
    for i in range(tm):
        for j in range(tn):
            r = 128 * i + int(rng.integers(0, min(128, M - 128 * i)))
            c = 128 * j + int(rng.integers(0, min(128, N - 128 * j)))
            q[r, c] = 0x7E | (0x80 if rng.integers(0, 2) else 0)
    k = rng.integers(-60, 60, (tm, tn))
    s = np.ldexp(1.0, k).astype(np.float32)
    q2, s2 = O.fp8blk_requantize_fp8blk(q, s)
    assert np.array_equal(s2, s) and np.array_equal(q2, q)
    s = (s * np.float32(1.3)).astype(np.float32)
    _, s3 = O.fp8blk_requantize_fp8blk(q, s)
    amax = bf16_f32(f32_to_bf16_torch((s.astype(np.float64) * 448.0).astype(np.float32)))
    want = np.array([rn_f32_of(Fraction(float(a)) / 448) for a in amax.ravel()], np.float32).reshape(s.shape)
    assert np.array_equal(s3, want)


def pin_requant_nvfp4_round_trip(O):
    """A sibling group of two block-wise FP8 tensors.  The first dequantizes to E2M1
    grid values times s_b * 2^k per 1x16 block (one +-6 per block, s_b in {2^j,
    1.5 * 2^j}), with a different power-of-two tile scale per tile; the second holds
    one code 448 under the tile scale 6 * 2^k, so the group amax is 2688 * 2^k and
    g = 2^k.  Then the block-scale codes are s_b, the element codes the grid codes,
    and the NVFP4 dequantization returns the FP8 tensor's BF16 values."""
    rng = np.random.default_rng(22)
    grid = read_grid_file()
    tab = e4m3_table()
    code_of = {float(v): c for c, v in enumerate(tab[:0x7F])}
    for k in (-30, 0, 9):
        M, N = 140, 272
        nb = N // 16
        tm, tn = (M + 127) // 128, (N + 127) // 128
        sb = np.ldexp(np.where(rng.integers(0, 2, (M, nb)) == 1, 1.5, 1.0), rng.integers(-3, 4, (M, nb)))
        gc = rng.integers(0, 16, (M, N))
        for r in range(M):
            for b in range(nb):
                gc[r, 16 * b + int(rng.integers(0, 16))] = 7 | (8 if rng.integers(0, 2) else 0)
        gv = grid[gc & 7] * np.where(gc & 8, -1.0, 1.0)
        kt = k + rng.integers(-2, 3, (tm, tn))
        ktt = np.repeat(np.repeat(kt, 128, 0), 128, 1)[:M, :N]
        cv = gv * np.repeat(sb, 16, 1) * np.ldexp(1.0, k - ktt)
        q1 = np.array([code_of[abs(v)] | (0x80 if v < 0 else 0) for v in cv.ravel()], np.uint8).reshape(M, N)
        s1 = np.ldexp(1.0, kt).astype(np.float32)
        q2 = np.zeros((2, 32), np.uint8)
        q2[1, 7] = 0x7E
        s2 = np.full((1, 1), np.ldexp(6.0, k), np.float32)
        assert O.fp8blk_amax(q2, s2) == np.ldexp(2688.0, k)
        A, g, outs = O.fp8blk_requantize_nvfp4_group([(q1, s1), (q2, s2)])
        assert A == np.ldexp(2688.0, k) and g == np.ldexp(1.0, k)
        p, s = outs[0]
        assert np.array_equal(tab[s].astype(np.float64), sb)
        codes = np.empty((M, N), np.int64)
        codes[:, 0::2] = p & 15
        codes[:, 1::2] = p >> 4
        assert np.all((codes & 7) == (gc & 7))
        assert np.all(((codes & 8) == (gc & 8)) | ((gc & 7) == 0))
        assert np.array_equal(O.nvfp4_dequantize(p, s, g), O.fp8blk_dequantize(q1, s1))


# --------------------------------------------------------------------------- INT4, group-wise
# "低精度训练与 Rollout", "INT4 QAT 训练": only the group sizes (128, 32) are on
# the page; the readings (symmetric, s = amax / 7, nearest integer with ties to
# even, two's-complement nibbles) are the oracle's and are pinned here from
# independent routes: exact rationals, numpy's int8 bit patterns, and inputs
# built to be exactly representable.

def _int4_pack_numpy(q: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles from numpy's int8 bit patterns, element 2j low."""
    nib = q.astype(np.int8).view(np.uint8) & 0x0F
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def pin_int4_grid_round_trip(O):
    """Integer codes times a power of two per group, with a +-7 in every group:
    the scale is exactly that power, the codes come back packed as numpy's int8
    nibbles, and dequantize and QDQ return the input bit for bit."""
    rng = np.random.default_rng(41)
    for G in (32, 128):
        M, N = 6, 4 * G
        q = rng.integers(-7, 8, (M, N)).astype(np.int64)
        k = rng.integers(-30, 30, (M, N // G))
        for r in range(M):
            for gi in range(N // G):
                q[r, gi * G + rng.integers(0, G)] = 7 if rng.integers(0, 2) else -7
        scale = np.ldexp(1.0, np.repeat(k, G, axis=1))
        w = f32_to_bf16_torch((q * scale).astype(np.float32))
        assert np.array_equal(bf16_f32(w).astype(np.float64), q * scale)   # exact by construction
        p, s = O.int4_quantize(w, G)
        assert np.array_equal(s.astype(np.float64), np.ldexp(1.0, k)), G
        assert np.array_equal(p, _int4_pack_numpy(q)), G
        y = O.int4_dequantize(p, s, G)
        assert np.array_equal(bf16_f32(y).astype(np.float64), q * scale), G
        assert np.array_equal(O.int4_qdq(w, G), y), G


def _int4_exact(xs: np.ndarray):
    """Scale, codes and BF16 outputs of one group by exact rational arithmetic:
    s = RN32(amax / 7), t = RN32(x / s), q = round-half-even(t) clamped to
    [-8, 7], y = BF16(RN32(q * s))."""
    vals = [Fraction(float(v)) for v in bf16_f32(xs)]
    amax = max(abs(v) for v in vals)
    s = rn_f32_of(amax / 7)
    qs, ys = [], []
    for v in vals:
        if s == 0:
            q = 0
        else:
            t = Fraction(float(rn_f32_of(v / Fraction(float(s)))))
            q = min(7, max(-8, round(t)))          # Python rounds half to even
        qs.append(q)
        ys.append(rn_f32_of(Fraction(q) * Fraction(float(s))))
    return s, np.array(qs, np.int64), f32_to_bf16_torch(np.array(ys, np.float32))


def pin_int4_nearest_exact(O):
    """Codes, scales and QDQ outputs against exact rationals, on MoE-like groups,
    groups of subnormals, groups spanning wide exponent ranges, and groups whose
    quotients land exactly on half-integers (ties to even) under power-of-two scales
    and under scales sigma * 2^k that are not (only a correctly rounded x / s gives
    the tie there)."""
    rng = np.random.default_rng(42)
    for G in (32, 128):
        groups = []
        for j in range(6):   # MoE-like values with outliers
            v = rng.standard_normal(G) * 0.02
            v[rng.integers(0, G)] *= 50
            groups.append(v.astype(np.float32))
        groups.append(random_f32(G, 43 + G, -133, -120))   # subnormal and tiny amax
        groups.append(random_f32(G, 44 + G, -60, 60))      # wide exponent range
        halves = np.array([7, -7, 0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 3.5, -3.5, 4.5, 5.5, 6.5, -6.5, 0, 3])
        for k in (-12, 0, 9):                              # half-integer quotients under s = 2^k
            groups.append(np.ldexp(np.resize(halves, G), k).astype(np.float32))
        for sigma in _short_significands(3):               # the same ties under s = sigma * 2^k
            t = np.resize(halves, G) * sigma
            if all(_bf16_exact(v) for v in t):
                groups.append(np.ldexp(t, -5).astype(np.float32))
        w = np.stack([f32_to_bf16_torch(g) for g in groups])
        p, s = O.int4_quantize(w, G)
        y = O.int4_qdq(w, G)
        for r in range(w.shape[0]):
            es, eq, ey = _int4_exact(w[r])
            assert f32_bits(s[r, 0]) == f32_bits(es), (G, r)
            assert np.array_equal(p[r], _int4_pack_numpy(eq[None])[0]), (G, r)
            assert np.array_equal(y[r], ey), (G, r)


def pin_int4_zero_and_layout(O):
    """A zero group has scale 0, codes 0 and +0 outputs (integers carry no sign of
    zero), a group's scale sits at [row, column / G], and QDQ is dequantize of
    quantize on random data."""
    for G in (32, 128):
        M, N = 3, 3 * G
        w = f32_to_bf16_torch(np.linspace(-1.0, 1.0, M * N, dtype=np.float32).reshape(M, N))
        w[1, G:2 * G] = 0x8000            # -0 group
        w[2, 0:G] = 0
        p, s = O.int4_quantize(w, G)
        assert s.shape == (M, N // G) and s[1, 1] == 0 and s[2, 0] == 0
        assert np.all(p[1, G // 2:G] == 0) and np.all(p[2, :G // 2] == 0)
        y = O.int4_dequantize(p, s, G)
        assert np.all(y[1, G:2 * G] == 0) and np.all(y[2, :G] == 0)     # +0, not -0
        # scale of group (r, gi) is the amax of exactly those G elements over 7
        for r in range(M):
            for gi in range(N // G):
                amax = np.max(np.abs(bf16_f32(w[r, gi * G:(gi + 1) * G]).astype(np.float64)))
                assert f32_bits(s[r, gi]) == f32_bits(rn_f32_of(Fraction(float(amax)) / 7)), (G, r, gi)
        rng = np.random.default_rng(45)
        x = f32_to_bf16_torch((rng.standard_normal((4, 2 * G)) * 0.03).astype(np.float32))
        assert np.array_equal(O.int4_qdq(x, G), O.int4_dequantize(*O.int4_quantize(x, G), G))


# The exact-quotient pins take seconds each; they run last, so that a planted mistake
# that a cheaper pin catches never waits for them.
_SLOW_PINS = ("pin_exact_global_scale", "pin_exact_fp8blk", "pin_exact_nvfp4")
ALL_PINS = ([v for k, v in sorted(globals().items()) if k.startswith("pin_") and k not in _SLOW_PINS]
            + [globals()[k] for k in _SLOW_PINS])
