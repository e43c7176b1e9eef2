// Device-side building blocks of the gfx950 codec kernels.
//
// Everything here is exact: each helper either reproduces one correctly rounded
// IEEE binary32 operation, or one round-to-nearest-even conversion, bit for bit.
// The choices were checked as follows (the checks are described with the
// kernels' design notes in the repository's documentation):
//  * v_cvt_pk_fp8_f32 rounds to nearest even into OCP E4M3 and keeps the sign
//    of zero, but turns overflow into NaN -> inputs are clamped to +-448 first
//    (an exhaustive sweep over all binary32 patterns then matched a software
//    saturating cast everywhere);
//  * v_cvt_scalef32_pk_fp8_f32 computes the E4M3 rounding of src / 2^scale
//    (one rounding) and v_cvt_scalef32_pk_bf16_fp8 the BF16 rounding of
//    code * 2^scale; the scale operand carries a UE8M0 byte in the binary32
//    exponent field;
//  * v_cvt_scalef32_pk_fp4_f32 with scale 1.0 is the saturating
//    nearest-even E2M1 cast (sign of zero kept); v_cvt_scalef32_pk_f32_fp4
//    decodes E2M1 exactly; element 0 sits in the low nibble;
//  * v_cvt_pk_bf16_f32 is the nearest-even BF16 rounding, subnormals and
//    overflow to Inf included;
//  * rcp_rn(): v_rcp_f32 followed by one Newton step with FMA returns the
//    correctly rounded reciprocal for every binary32 input in [2^-125, 2^126);
//  * quot_rn(): x * r, then one Markstein correction, returns the correctly
//    rounded quotient RN(x / S) when r = RN(1/S), S in [2^-90, 2^126) and x is
//    a BF16 value or RN(BF16 / 6) (exhaustive over all significand pairs),
//    and a zero with x's sign when S == 0 and r == 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lpq {

typedef short short2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));   // 16 bytes: 8 BF16 values
typedef uint32_t v2u __attribute__((ext_vector_type(2)));   // 8 bytes

// Global loads and stores, optionally marked non-temporal (streamed data that
// is not read again soon: keeps it from displacing useful cache lines).  The
// pointers are taken to the global address space so that global_load /
// global_store (not flat) instructions are emitted.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;

template <bool NT, typename T>
__device__ __forceinline__ T load(const T* p) {
    auto g = (__attribute__((address_space(1))) const T*)(p);
    if constexpr (NT) return __builtin_nontemporal_load(g);
    else return *g;
}
template <bool NT, typename T>
__device__ __forceinline__ void store(T* p, T v) {
    auto g = (gptr<T>)(p);
    if constexpr (NT) __builtin_nontemporal_store(v, g);
    else *g = v;
}

// Plain global byte access (scale bytes).
__device__ __forceinline__ uint32_t load_u8(const uint8_t* p) {
    return *(__attribute__((address_space(1))) const uint8_t*)(p);
}
__device__ __forceinline__ void store_u8(uint8_t* p, uint32_t v) { *(gptr<uint8_t>)(p) = (uint8_t)v; }

constexpr float kE4M3Max = 448.0f;      // largest finite E4M3 value
constexpr float kTinyScale = 0x1p-90f;  // below this a scale is pre-scaled by 2^64
constexpr float kPreScale = 0x1p64f;
constexpr float kRcp6 = 0x1.555556p-3f; // RN(1/6)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Correctly rounded 1/s for s in [2^-125, 2^126).
__device__ __forceinline__ float rcp_rn(float s) {
    float y = __builtin_amdgcn_rcpf(s);
    float e = __builtin_fmaf(-s, y, 1.0f);
    return __builtin_fmaf(e, y, y);
}

// RN(x / S) from r = RN(1/S) (see the header comment for the domain).  The
// residual is formed as fma(q0, S, -x) and subtracted, which keeps the sign of
// a zero quotient.
__device__ __forceinline__ float quot_rn(float x, float S, float r) {
    float q0 = x * r;
    float t = __builtin_fmaf(q0, S, -x);
    return __builtin_fmaf(-t, r, q0);
}

// Two binary32 values -> two E4M3 codes (saturating, nearest even) in the
// low (HI == false) or high 16 bits of `old`.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2(float a, float b, uint32_t old) {
    a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
    b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// E4M3 code (low byte) -> binary32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0];
}

// Packed pair of BF16 (low = a) from two binary32 values, nearest even: one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
    const float2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// True for the whole wave when any active lane has `p` (a wave-uniform branch
// condition for rare slow paths).
__device__ __forceinline__ bool any_lane(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// A pointer the caller knows to be wave-uniform, pinned to scalar registers:
// lane addresses formed from it are the scalar base plus a 32-bit lane offset
// (global_load's saddr form) instead of a 64-bit address per lane.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Maximum of two non-negative binary32 values through their bit patterns.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// |x| maximum over the 8 BF16 values of a 16-byte vector, as binary32 bits.
// BF16 magnitudes order like their 15-bit patterns, so the maximum is taken on
// the masked integers and widened once.
__device__ __forceinline__ uint32_t absmax8_bits(const v4u& v) {
    uint32_t a = v.x & 0x7fff7fffu, b = v.y & 0x7fff7fffu, c = v.z & 0x7fff7fffu, d = v.w & 0x7fff7fffu;
    uint32_t m0 = umax(umax(a & 0xffffu, a >> 16), umax(b & 0xffffu, b >> 16));
    uint32_t m1 = umax(umax(c & 0xffffu, c >> 16), umax(d & 0xffffu, d >> 16));
    return umax(m0, m1) << 16;
}

// The 8 BF16 values of a 16-byte vector widened to binary32 (exact).
struct F8 {
    float x[8];
};
__device__ __forceinline__ F8 widen8(const v4u& v) {
    F8 f;
    f.x[0] = bf16_lo(v.x); f.x[1] = bf16_hi(v.x); f.x[2] = bf16_lo(v.y); f.x[3] = bf16_hi(v.y);
    f.x[4] = bf16_lo(v.z); f.x[5] = bf16_hi(v.z); f.x[6] = bf16_lo(v.w); f.x[7] = bf16_hi(v.w);
    return f;
}

// max |x| of 8 widened values as binary32 bits (three-input maximum with
// absolute-value operands: 4 instructions).
__device__ __forceinline__ uint32_t absmax8_f32(const F8& f) {
    float m = fmaxf(fmaxf(fabsf(f.x[0]), fabsf(f.x[1])), fabsf(f.x[2]));
    m = fmaxf(fmaxf(m, fabsf(f.x[3])), fabsf(f.x[4]));
    m = fmaxf(fmaxf(m, fabsf(f.x[5])), fabsf(f.x[6]));
    m = fmaxf(m, fabsf(f.x[7]));
    return __float_as_uint(m);
}

// Cross-lane maxima inside groups of 2 / 4 lanes (DPP quad permutations).
__device__ __forceinline__ uint32_t pair_max(uint32_t v) {
    return umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = pair_max(v);
    return umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = quad_max(v);
    v = umax(v, (uint32_t)__shfl_xor((int)v, 4));
    v = umax(v, (uint32_t)__shfl_xor((int)v, 8));
    v = umax(v, (uint32_t)__shfl_xor((int)v, 16));
    v = umax(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// MXFP8 scale byte of a block amax given as binary32 bits (a BF16 value, so
// the low 16 bits are zero): byte = max(0, Eb - 8 + [m7 > 96]), the smallest
// e with amax <= 448 * 2^e (448 = 1.75 * 2^8) biased by 127.  Adding 31 to
// the 7-bit mantissa field carries into the exponent exactly when m7 > 96.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
    int e = (int)((amax_bits + (31u << 16)) >> 23) - 8;
    return (uint32_t)(e > 0 ? e : 0);
}

// The floor rule of the OCP MX specification: byte = floor(log2 amax) - 8 + 127
// = max(0, Eb - 8) from the biased exponent of a BF16 amax (a subnormal amax
// clamps to 0).
__device__ __forceinline__ uint32_t mx_floor_scale_byte(uint32_t amax_bits) {
    const int e = (int)(amax_bits >> 23) - 8;
    return (uint32_t)(e > 0 ? e : 0);
}

// The binary32 operand that carries a UE8M0 byte for the scaled converts.
__device__ __forceinline__ float ue8m0_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

}  // namespace lpq
