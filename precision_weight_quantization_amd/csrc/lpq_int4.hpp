// Group-wise INT4 quantize, dequantize and QDQ.
//
// Part of lpq_kernels.hip, which includes each part once, in this order: one
// translation unit.
#pragma once

namespace {

// ---------------------------------------------------------------------------
// INT4: symmetric, one FP32 scale per group of G = 32 or 128 elements of a row
// ---------------------------------------------------------------------------
//
// "低精度训练与 Rollout", "INT4 QAT 训练" fixes the group size (128, or 32 for
// Kimi-K2) and a straight-through estimator, whose forward pass is QDQ.
// Readings: s = fl(amax / 7); code = the integer nearest to fl(x / s), ties
// to even, clamped to [-8, 7] (a zero scale gives 0); two's-complement
// nibbles, element 2j low; y = BF16(fl(code * s)).  Flat layout as for
// NVFP4: 8 elements per lane, a group is G / 8 consecutive lanes.

constexpr float kRcp7 = 0x1.24924ap-3f;   // RN(1/7)
constexpr float kRound = 0x1.8p23f;       // fl(t + 1.5 * 2^23) = 1.5 * 2^23 + RN_int(t) for |t| <= 2^22

// Maximum over the G / 8 lanes of a group: a quad, or a DPP row of 16 lanes
// (rotations by 4 and 8 lanes inside the row: no LDS round trip).
template <int G>
__device__ __forceinline__ uint32_t int4_group_max(uint32_t m) {
    m = quad_max(m);
    if constexpr (G == 128) {
        m = umax(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x124, 0xF, 0xF, false));   // row_ror:4
        m = umax(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xF, 0xF, false));   // row_ror:8
    }
    return m;
}

struct Int4Scale {
    float s;        // the group scale
    float sd;       // divisor for the quotients: s, or s * 2^64 when s is tiny
    float r;        // RN(1 / sd), or 0 when s == 0
    float xpre;     // 1, or 2^64 when s is tiny
    bool any_tiny;  // wave-uniform
};

__device__ __forceinline__ Int4Scale int4_scale(uint32_t amax_bits) {
    Int4Scale I;
    const float a = __uint_as_float(amax_bits);
    // fl(a / 7): the short sequence is exact while the quotient is normal;
    // tinier groups take the full correctly rounded division
    float s = quot_rn(a, 7.0f, kRcp7);
    if (any_lane(a < 0x1p-100f)) {
        float aa = a;
        __asm__ volatile("" : "+v"(aa));   // keeps the long division inside the branch
        if (aa < 0x1p-100f) s = aa / 7.0f;
    }
    I.s = s;
    I.any_tiny = any_lane(s > 0.0f && s < kTinyScale);
    I.xpre = 1.0f;
    I.sd = s;
    if (I.any_tiny) {   // wave-uniform and rare: the pre-scaling selects stay inside the branch
        float ss = s;
        __asm__ volatile("" : "+v"(ss));
        const bool tiny = ss > 0.0f && ss < kTinyScale;
        I.xpre = tiny ? kPreScale : 1.0f;
        I.sd = tiny ? ss * kPreScale : ss;
    }
    I.r = s > 0.0f ? rcp_rn(I.sd) : 0.0f;
    return I;
}

// fl(x / s) of the 8 values, clamped to [-8, 7] (so that rounding stays in range).
__device__ __forceinline__ void int4_quotients(const F8& f, const Int4Scale& I, float (&t)[8]) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; k++) x[k] = f.x[k];
    if (I.any_tiny) {
#pragma unroll
        for (int k = 0; k < 8; k++) x[k] *= I.xpre;
    }
#pragma unroll
    for (int k = 0; k < 8; k++) t[k] = __builtin_amdgcn_fmed3f(quot_rn(x[k], I.sd, I.r), -8.0f, 7.0f);
}

// 8 values -> 8 nibbles (element 0 low).  The low four bits of fl(t + 1.5 *
// 2^23) are RN_int(t) in two's complement.
__device__ __forceinline__ uint32_t int4x8(const F8& f, const Int4Scale& I) {
    float t[8];
    int4_quotients(f, I, t);
    // byte j = nibbles 2j, 2j+1 (the bits above the byte are don't-cares), then
    // the four low bytes gathered with byte permutes
    uint32_t b[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
        b[j] = (__float_as_uint(t[2 * j] + kRound) & 15u) | (__float_as_uint(t[2 * j + 1] + kRound) << 4);
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);   // b0.byte0, b1.byte0
    const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u);   // b2.byte0, b3.byte0
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);                    // lo.bytes 0-1, hi.bytes 0-1
}

// 8 values -> their fake-quantized BF16 values BF16(fl(RN_int(fl(x / s)) * s)).
__device__ __forceinline__ v4u int4x8_qdq(const F8& f, const Int4Scale& I) {
    float t[8], y[8];
    int4_quotients(f, I, t);
#pragma unroll
    for (int k = 0; k < 8; k++) y[k] = ((t[k] + kRound) - kRound) * I.s;   // the integer, exactly, times s
    return v4u{bf16x2(y[0], y[1]), bf16x2(y[2], y[3]), bf16x2(y[4], y[5]), bf16x2(y[6], y[7])};
}

// 8 nibbles (one word) times s -> 8 BF16 values.
__device__ __forceinline__ v4u int4x8_to_bf16(uint32_t p, float s) {
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; k++) y[k] = (float)((int32_t)(p << (28 - 4 * k)) >> 28) * s;   // sign-extended nibble
    return v4u{bf16x2(y[0], y[1]), bf16x2(y[2], y[3]), bf16x2(y[4], y[5]), bf16x2(y[6], y[7])};
}

template <int U, int TH, bool GROUPED, int G, bool AHEAD = LPQ_I4Q_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_int4_quant(const lpq_tensor* table, lpq_tensor one, ChunkMap map) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const int tid = threadIdx.x;
    // the chunk's origins (uniform); a lane's vector i = u * TH + tid, and its
    // group's scale, are addressed with 32-bit offsets from them
    const v4u* src = reinterpret_cast<const v4u*>(d.src) + base / 8;
    uint32_t* dst = reinterpret_cast<uint32_t*>(d.dst) + base / 8;
    float* scale = reinterpret_cast<float*>(d.scale) + base / G;
    const int64_t left = total - base;   // elements from the chunk origin to the end
    const bool leader = (tid & (G / 8 - 1)) == 0;   // the first lane of its group
    by_fullness<chunk_elems<U, TH>()>(base, total, [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
        auto in = [&](int i) { return FULL || (int64_t)i * 8 < left; };
        v4u v[U];
        auto fetch = [&](int u) {
            const int i = u * TH + tid;
            v[u] = in(i) ? load<kNTL>(uniform_ptr(src + u * TH) + tid) : v4u{};
        };
        fetch_start<U, AHEAD>(fetch);
#pragma unroll
        for (int u = 0; u < U; u++) {
            fetch_step<U, AHEAD>(u, fetch, v[u].x);
            const int i = u * TH + tid;
            // G / 8 lanes are one group; groups never straddle the end (N % G == 0)
            const F8 f = widen8(v[u]);
            const Int4Scale I = int4_scale(int4_group_max<G>(absmax8_f32(f)));
            const uint32_t p = int4x8(f, I);
            if (in(i)) {
                store<kNTS>(uniform_ptr(dst + u * TH) + tid, p);
                if (leader) store<false>(uniform_ptr(scale + u * (TH * 8 / G)) + tid / (G / 8), I.s);
            }
        }
    });
}

template <int U, int TH, bool GROUPED, int G, bool AHEAD = LPQ_I4D_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_int4_dequant(const lpq_tensor* table, lpq_tensor one, ChunkMap map) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const uint32_t* src = reinterpret_cast<const uint32_t*>(d.src);
    const float* scale = reinterpret_cast<const float*>(d.scale);
    v4u* dst = reinterpret_cast<v4u*>(d.dst);
    const int tid = threadIdx.x;
    by_fullness<chunk_elems<U, TH>()>(base, total, [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
        uint32_t p[U];
        float sc[U];
        auto fetch = [&](int u) {
            const int64_t e0 = base + (int64_t)(u * TH + tid) * 8;
            p[u] = load_vec<TH, FULL>(src, base, total, u);
            sc[u] = (FULL || e0 < total) ? load<false>(scale + e0 / G) : 0.0f;
        };
        fetch_start<U, AHEAD>(fetch);
#pragma unroll
        for (int u = 0; u < U; u++) {
            fetch_step<U, AHEAD>(u, fetch, p[u], __float_as_uint(sc[u]));
            const int64_t e0 = base + (int64_t)(u * TH + tid) * 8;
            const v4u o = int4x8_to_bf16(p[u], sc[u]);
            if (FULL || e0 < total) store<kNTS>(dst + (e0 >> 3), o);
        }
    });
}

template <int U, int TH, bool GROUPED, int G, bool AHEAD = LPQ_I4QDQ_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_int4_qdq(const lpq_tensor* table, lpq_tensor one, ChunkMap map) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const v4u* src = reinterpret_cast<const v4u*>(d.src);
    v4u* dst = reinterpret_cast<v4u*>(d.dst);
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
            const F8 f = widen8(v[u]);
            const v4u o = int4x8_qdq(f, int4_scale(int4_group_max<G>(absmax8_f32(f))));
            if (FULL || e0 < total) store<kNTS>(dst + (e0 >> 3), o);
        }
    });
}

}  // namespace
