"""Plant plausible mistakes in copies of the oracle (on the CPU) and require the
pins to catch every one: evidence that the pins constrain each step."""
import os

import pytest

from oracle import oracle as O
from tests import pins

MUTANTS = [
    ("e4m3 ties away from zero",
     "if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep += 1u;",
     "if (rest >= 0x80000u) keep += 1u;"),
    ("e4m3 subnormal ties up",
     "if (frac > 0.5f || (frac == 0.5f && (ki & 1u))) ki += 1u;",
     "if (frac >= 0.5f) ki += 1u;"),
    ("e4m3 no saturation",
     "if (mag >= 448.0f) return (uint8_t)(sign | 0x7e);",
     "if (mag >= 480.0f) return (uint8_t)(sign | 0x7f);"),
    ("e4m3 drops sign of zero",
     "uint8_t sign = (uint8_t)((u >> 24) & 0x80u);",
     "uint8_t sign = (uint8_t)((v < 0.0f) ? 0x80u : 0u);"),
    ("e2m1 tie at 0.25 goes up",
     "if (a <= 0.25f) c = 0;",
     "if (a < 0.25f) c = 0;"),
    ("e2m1 tie at 2.5 goes up",
     "else if (a <= 2.5f) c = 4;",
     "else if (a < 2.5f) c = 4;"),
    ("bf16 truncates",
     "if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;",
     ""),
    ("fp8blk scale divisor 256",
     "float scale = amax / 448.0f;",
     "float scale = amax / 256.0f;"),
    ("fp8blk tile index transposed",
     "s[ti * tiles_n + tj] = scale;",
     "s[tj * tiles_m + ti] = scale;"),
    ("fp8blk amax without abs",
     "float a = fabsf(oc_bf16_to_f32(w[r * N + c]));\n                    if (a > amax) amax = a;",
     "float a = oc_bf16_to_f32(w[r * N + c]);\n                    if (a > amax) amax = a;"),
    ("fp8blk dequant divides",
     "y[r * N + c] = oc_f32_to_bf16(oc_e4m3_decode(q[r * N + c]) * scale);",
     "y[r * N + c] = oc_f32_to_bf16(oc_e4m3_decode(q[r * N + c]) / scale);"),
    ("fp8blk ragged tile clipped wrong",
     "int64_t r0 = ti * T, r1 = (r0 + T < M) ? r0 + T : M;",
     "int64_t r0 = ti * T, r1 = (r0 + T < M) ? r0 + T - 1 : M;"),
    ("mxfp8 floor exponent rule",
     "while (a > ldexp(448.0, e)) e++;",
     "while (a >= ldexp(512.0, e)) e++;"),
    ("mxfp8 scale index transposed",
     "e[r * nb + b] = byte;",
     "e[b * M + r] = byte;"),
    ("mxfp8 dequant block width 16",
     "float X = oc_ue8m0_decode(e[r * nb + c / 32]);",
     "float X = oc_ue8m0_decode(e[r * nb + (c / 16) % nb]);"),
    ("nvfp4 global divisor 448",
     "OC_API float oc_nvfp4_global_scale(float A) { return A / (6.0f * 448.0f); }",
     "OC_API float oc_nvfp4_global_scale(float A) { return A / 448.0f; }"),
    ("nvfp4 block scale drops /6",
     "float t = b / 6.0f;",
     "float t = b;"),
    ("nvfp4 effective scale drops g",
     "return oc_e4m3_decode(scode) * g;",
     "return oc_e4m3_decode(scode);"),
    ("nvfp4 nibbles swapped",
     "p[(r * N + b * 16 + k) / 2] = (uint8_t)(lo | (hi << 4));",
     "p[(r * N + b * 16 + k) / 2] = (uint8_t)(hi | (lo << 4));"),
    ("nvfp4 dequant scale index by 8",
     "float S = oc_nvfp4_effective_scale(s[r * nb + c / 16], g);",
     "float S = oc_nvfp4_effective_scale(s[r * nb + (c / 8) % nb], g);"),
    ("nvfp4 zero scale loses sign",
     "if (S == 0.0f) return (f2u(x) >> 31) ? 8 : 0;",
     "if (S == 0.0f) return 0;"),
    ("nvfp4 qdq block amax over 8 elements",
     "const uint16_t* blk = x + r * N + b * 16;\n            float bmax = 0.0f;\n            for (int k = 0; k < 16; k++) {",
     "const uint16_t* blk = x + r * N + b * 16;\n            float bmax = 0.0f;\n            for (int k = 0; k < 8; k++) {"),
    ("mxfp8 floor rule off by one",
     "int e = (k - 1) - 8;",
     "int e = k - 8;"),
    ("mxfp8 floor quantizer uses the ceiling byte",
     "mxfp8_quantize_with(w, M, N, q, e, oc_mxfp8_floor_scale_byte);",
     "mxfp8_quantize_with(w, M, N, q, e, oc_mxfp8_scale_byte);"),
    ("nvfp4 reciprocal global scale formed from the multiplier",
     "return (6.0f * 448.0f) / A;",
     "return 1.0f / (A / (6.0f * 448.0f));"),
    ("observer: static keeps the latest batch",
     "if (oc_below(bmin, state[0])) state[0] = bmin;",
     "state[0] = bmin;"),
    ("observer: moving average without the constant",
     "state[1] = state[1] + c * (bmax - state[1]);",
     "state[1] = state[1] + (bmax - state[1]);"),
    ("observer: amax from the max only",
     "return lo > hi ? lo : hi;",
     "return hi;"),
    ("nvfp4 global scale ignores the E4M3 maximum",
     "OC_API float oc_nvfp4_global_scale_max(float A, int e4m3_max) { return A / (6.0f * (float)e4m3_max); }",
     "OC_API float oc_nvfp4_global_scale_max(float A, int e4m3_max) { return A / (6.0f * 448.0f); }"),
    ("nvfp4 qdq does not multiply back by the global scale",
     "float S = oc_nvfp4_effective_scale(oc_nvfp4_block_scale(bmax, g), g);",
     "float S = oc_e4m3_decode(oc_nvfp4_block_scale(bmax, g)) * (g > 0.0f ? 1.0f : 0.0f);"),
    ("int4 scale divisor 8",
     "OC_API float oc_int4_scale(float amax) { return amax / 7.0f; }",
     "OC_API float oc_int4_scale(float amax) { return amax / 8.0f; }"),
    ("int4 rounds half away from zero",
     "float t = nearbyintf(x / s);",
     "float t = roundf(x / s);"),
    ("int4 truncates the quotient",
     "float t = nearbyintf(x / s);",
     "float t = truncf(x / s);"),
    ("int4 nibbles swapped",
     "p[(r * N + gi * G + k) / 2] = (uint8_t)((lo & 15) | ((hi & 15) << 4));",
     "p[(r * N + gi * G + k) / 2] = (uint8_t)((hi & 15) | ((lo & 15) << 4));"),
    ("int4 decode without sign extension",
     "static int oc_int4_decode(uint8_t nibble) { return (nibble & 8) ? (int)nibble - 16 : (int)nibble; }",
     "static int oc_int4_decode(uint8_t nibble) { return (int)nibble; }"),
    ("int4 dequant scale of the 32-element group",
     "float scale = s[r * ng + c / G];",
     "float scale = s[r * ng + (c / 32) % ng];"),
    ("int4 group amax without abs",
     "float a = fabsf(oc_bf16_to_f32(grp[k]));",
     "float a = oc_bf16_to_f32(grp[k]);"),
    ("int4 qdq keeps the quotient unrounded",
     "y[r * N + gi * G + k] = oc_f32_to_bf16((float)q * scale);",
     "y[r * N + gi * G + k] = oc_f32_to_bf16((scale == 0.0f ? 0.0f : oc_bf16_to_f32(grp[k]) / scale) * scale);"),
]


@pytest.fixture(scope="module")
def source():
    with open(O.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation site not found exactly once: {name}"
    path = O.build_variant(source.replace(old, new), str(tmp_path / "mutant.so"))
    mutant = O.Oracle(path)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append((pin.__name__, type(exc).__name__))
            break
    assert caught, f"no pin caught the planted mistake: {name}"
