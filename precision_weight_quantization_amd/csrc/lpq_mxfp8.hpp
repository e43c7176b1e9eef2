// MXFP8 quantize (default and floor exponent rules) and dequantize.
//
// Part of lpq_kernels.hip, which includes each part once, in this order: one
// translation unit.
#pragma once

namespace {

// ---------------------------------------------------------------------------
// MXFP8
// ---------------------------------------------------------------------------

// 8 values -> 8 E4M3 codes of RN(x / 2^(byte - 127)), X carrying the byte.
__device__ __forceinline__ v2u mx_encode8(const F8& f, float X) {
    short2_t c01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((short2_t){0, 0}, f.x[0], f.x[1], X, false);
    c01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c01, f.x[2], f.x[3], X, true);
    short2_t c23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((short2_t){0, 0}, f.x[4], f.x[5], X, false);
    c23 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(c23, f.x[6], f.x[7], X, true);
    return v2u{__builtin_bit_cast(uint32_t, c01), __builtin_bit_cast(uint32_t, c23)};
}

// FLOOR selects the shared-exponent rule of the OCP MX specification
// (floor(log2 amax) - 8, elements beyond 448 saturate) instead of the default
// no-saturation rule.
template <int U, int TH, bool GROUPED, bool FLOOR = false, bool AHEAD = LPQ_MXQ_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_mxfp8_quant(const lpq_tensor* table, lpq_tensor one, ChunkMap map) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const v4u* src = reinterpret_cast<const v4u*>(d.src);
    v2u* dst = reinterpret_cast<v2u*>(d.dst);
    uint8_t* esc = reinterpret_cast<uint8_t*>(d.scale);
    const int tid = threadIdx.x;
    by_fullness<chunk_elems<U, TH>()>(base, total, [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
        v4u v[U];
        auto fetch = [&](int u) { v[u] = load_vec<TH, FULL>(src, base, total, u); };
        fetch_start<U, AHEAD>(fetch);
#pragma unroll
        for (int u = 0; u < U; u++) {
            fetch_step<U, AHEAD>(u, fetch, v[u].x);
            const int64_t e0 = base + (int64_t)(u * TH + tid) * 8;
            // a quad of lanes is one 32-element block; blocks never straddle the end
            F8 f = widen8(v[u]);
            const uint32_t amax = quad_max(absmax8_f32(f));
            const uint32_t byte = FLOOR ? mx_floor_scale_byte(amax) : mx_scale_byte(amax);
            if constexpr (FLOOR) {
                // saturation: clamp to +-448 * 2^(byte-127) (exact; byte <= 246 keeps it finite)
                const float L = __uint_as_float(((byte + 8u) << 23) | 0x600000u);
#pragma unroll
                for (int k = 0; k < 8; k++) f.x[k] = __builtin_amdgcn_fmed3f(f.x[k], -L, L);
            }
            const v2u codes = mx_encode8(f, ue8m0_operand(byte));
            if (FULL || e0 < total) {
                store<kNTS>(dst + (e0 >> 3), codes);
                if ((tid & 3) == 0) store_u8(esc + (e0 >> 5), byte);
            }
        }
    });
}

template <int U, int TH, bool GROUPED, bool AHEAD = LPQ_MXD_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_mxfp8_dequant(const lpq_tensor* table, lpq_tensor one, ChunkMap map) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const v2u* src = reinterpret_cast<const v2u*>(d.src);
    v4u* dst = reinterpret_cast<v4u*>(d.dst);
    const uint8_t* esc = reinterpret_cast<const uint8_t*>(d.scale);
    const int tid = threadIdx.x;
    by_fullness<chunk_elems<U, TH>()>(base, total, [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
        v2u c[U];
        uint32_t b[U];
        auto fetch = [&](int u) {
            const int64_t e0 = base + (int64_t)(u * TH + tid) * 8;
            c[u] = load_vec<TH, FULL>(src, base, total, u);
            b[u] = (FULL || e0 < total) ? load_u8(esc + (e0 >> 5)) : 127u;
        };
        fetch_start<U, AHEAD>(fetch);
#pragma unroll
        for (int u = 0; u < U; u++) {
            fetch_step<U, AHEAD>(u, fetch, c[u].x, b[u]);
            const int64_t e0 = base + (int64_t)(u * TH + tid) * 8;
            const float X = ue8m0_operand(b[u]);
            v4u o;
            o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[u].x, X, false));
            o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[u].x, X, true));
            o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[u].y, X, false));
            o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[u].y, X, true));
            if (FULL || e0 < total) store<kNTS>(dst + (e0 >> 3), o);
        }
    });
}

}  // namespace
