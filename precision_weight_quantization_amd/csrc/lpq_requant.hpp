// Fused re-quantization of block-wise FP8 weights (to block FP8, MXFP8, NVFP4,
// and their amax) and the flat block-FP8 dequantizer, which shares their tile-
// scale walk.
//
// Part of lpq_kernels.hip, which includes each part once, in this order: one
// translation unit.
#pragma once

namespace {

// ---------------------------------------------------------------------------
// Re-quantization of block-wise FP8 weights into MXFP8 / NVFP4
// ---------------------------------------------------------------------------
//
// The source is E4M3 codes with one FP32 scale per 128x128 tile; the values
// re-quantized are the BF16 dequantization y = BF16(fl(code * s_tile)),
// formed in registers and never stored.  Flat layout as above, but a lane
// takes 16 codes (one 16-byte vector) per step: a 1x16 NVFP4 block is one
// lane, a 1x32 MXFP8 block a pair of lanes.  N % 16 == 0 keeps a lane's 16
// elements inside one row and one 128-column tile, so each step needs one
// tile-scale lookup, found from the lane's (row, column).  These kernels do
// little memory traffic per element, so the per-wave set-up and per-step
// index work are kept to 32-bit integer steps (the host limits M and N to
// below 2^31), and full chunks run a straight-line body.

template <int U, int TH = kThreads>
constexpr int64_t rq_chunk_elems() {
    static_assert(TH % 64 == 0 && TH >= 64 && TH <= kMaxFlatThreads, "whole waves, at most kMaxFlatThreads");
    return (int64_t)TH * 16 * U;
}

constexpr uint32_t kRqStepMax = kMaxFlatThreads * 16;   // the largest step between a lane's vectors

// Walks the (row, column) of a lane's vectors (TH-thread workgroup, EV
// elements per vector) and looks up their tile scales.
template <int EV, int TH = kThreads>
struct TileCursor {
    static constexpr uint32_t kStep = TH * EV;   // elements between a lane's consecutive vectors
    const float* scale;   // tile scales of the tensor
    uint32_t N, tn;       // columns, tiles per row
    uint32_t sr, sc;      // kStep = sr * N + sc
    uint32_t r, c;        // position of the lane's current vector

    __device__ __forceinline__ TileCursor(const float* tile_scales, int64_t cols, int64_t base) {
        scale = tile_scales;
        N = (uint32_t)cols;
        tn = (N + kTile - 1) / kTile;
        sr = kStep / N;
        sc = kStep - sr * N;
        // chunk origin (uniform): a double-precision quotient estimate (base < 2^40,
        // error below 2^-11), corrected by one step
        const double invN = 1.0 / (double)N;
        int64_t r0 = (int64_t)((double)base * invN);
        int64_t c0 = base - r0 * (int64_t)N;
        if (c0 < 0) {
            r0 -= 1;
            c0 += N;
        } else if (c0 >= (int64_t)N) {
            r0 += 1;
            c0 -= N;
        }
        // the lane's offset from the origin: t < N + kStep < 2^32 and
        // t / N <= kStep <= 8192, so the single-precision estimate is within one
        const uint32_t t = (uint32_t)c0 + threadIdx.x * (uint32_t)EV;
        uint32_t q = (uint32_t)((float)t * __builtin_amdgcn_rcpf((float)N));
        if (q * N > t) q -= 1;
        else if (t - q * N >= N) q += 1;
        r = (uint32_t)r0 + q;
        c = t - q * N;
    }

    __device__ __forceinline__ const float* ptr() const { return scale + (r >> 7) * tn + (c >> 7); }   // 128 = kTile

    __device__ __forceinline__ void next() {
        r += sr;
        c += sc;
        if (c >= N) {
            c -= N;
            r += 1;
        }
    }
};

// RN-to-BF16 of x as binary32 bits, in one convert: the pair (0, x) packs
// BF16(x) into the high half over a zero low half.
__device__ __forceinline__ uint32_t bf16_in_f32(float x) { return bf16x2(0.0f, x); }

// The 16 codes of a vector times s, rounded to BF16 and widened back to
// binary32 (exact): the dequantized values, in two halves of 8.  `amax` is
// max |y| as binary32 bits: BF16 rounding is monotone, so it is the rounding
// of the largest |product| (taken on the products, which the compiler knows
// to be canonical floats).
struct Y16 {
    F8 lo, hi;
    uint32_t amax;
};

// POW2: the tile scale is 2^k with -121 <= k <= 119 (positive, significand bits
// clear, biased exponent 6 to 246).  A code
// has at most 4 significant bits and |code| lies in {0} or [2^-9, 448], so
// code * 2^k is then exact in binary32 and in BF16 (|y| in [2^-130, 1.75 * 2^127]
// keeps the 4 bits above BF16's last place, subnormal range included): y is
// the product itself, which the scaled convert forms from the scale's exponent
// (measured equal to the correctly rounded product for every code and every
// k from -126 to 127), with no multiply and no BF16 rounding.
template <bool POW2 = false>
__device__ __forceinline__ Y16 fp8blk_values16(const v4u& c, float s) {
    float p[16];
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        if constexpr (POW2) {
            const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[k], s, false);
            const float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[k], s, true);
            p[4 * k + 0] = a[0];
            p[4 * k + 1] = a[1];
            p[4 * k + 2] = b[0];
            p[4 * k + 3] = b[1];
        } else {
            const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
            const float2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
            p[4 * k + 0] = a[0] * s;
            p[4 * k + 1] = a[1] * s;
            p[4 * k + 2] = b[0] * s;
            p[4 * k + 3] = b[1] * s;
        }
    }
    float m = fmaxf(fmaxf(fabsf(p[0]), fabsf(p[1])), fabsf(p[2]));
#pragma unroll
    for (int k = 3; k < 15; k += 2) m = fmaxf(fmaxf(m, fabsf(p[k])), fabsf(p[k + 1]));
    m = fmaxf(m, fabsf(p[15]));
    Y16 y;
    if constexpr (POW2) {
        y.amax = __float_as_uint(m);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            y.lo.x[k] = p[k];
            y.hi.x[k] = p[8 + k];
        }
    } else {
        y.amax = bf16_in_f32(m);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            y.lo.x[k] = __uint_as_float(bf16_in_f32(p[k]));
            y.hi.x[k] = __uint_as_float(bf16_in_f32(p[8 + k]));
        }
    }
    return y;
}

// The block-FP8 codes and tile scales a descriptor names.
__device__ __forceinline__ const void* codes_of(const lpq_requant_tensor& d) { return d.src; }
__device__ __forceinline__ const float* tile_scales_of(const lpq_requant_tensor& d) { return d.src_scale; }
__device__ __forceinline__ const void* codes_of(const lpq_tensor& d) { return d.src; }
__device__ __forceinline__ const float* tile_scales_of(const lpq_tensor& d) { return reinterpret_cast<const float*>(d.scale); }

// Loads of a lane's U code vectors and their tile scales; with FULL every
// vector is in range, else vectors past the end read as codes 0, scale 0.
template <int U, bool FULL, int TH, typename D>
__device__ __forceinline__ void rq_load(v4u (&c)[U], float (&s)[U], const D& d, int64_t base, int64_t total) {
    const v4u* src = reinterpret_cast<const v4u*>(codes_of(d)) + base / 16 + threadIdx.x;
    TileCursor<16, TH> cur(tile_scales_of(d), d.cols, base);
#pragma unroll
    for (int u = 0; u < U; u++) {
        if (FULL) {
            c[u] = load<kNTL>(src + u * TH);
            s[u] = load<false>(cur.ptr());
        } else {
            const bool in = base + (int64_t)(u * TH + threadIdx.x) * 16 < total;
            c[u] = in ? load<kNTL>(src + u * TH) : v4u{0u, 0u, 0u, 0u};
            s[u] = in ? load<false>(cur.ptr()) : 0.0f;
        }
        cur.next();
    }
}

// The code vectors and tile scales of a lane's U steps, issued in the order of
// fetch_start / fetch_step (all up front, or one step ahead of the work);
// body(u, codes, scale) runs on each step.  Steps past the end read as codes 0,
// scale 0.
template <int U, bool FULL, bool AHEAD, int TH, typename D, typename Body>
__device__ __forceinline__ void rq_stream(const D& d, int64_t base, int64_t total, Body&& body) {
    const v4u* src = reinterpret_cast<const v4u*>(codes_of(d)) + base / 16 + threadIdx.x;
    TileCursor<16, TH> cur(tile_scales_of(d), d.cols, base);
    v4u c[U];
    float s[U];
    auto fetch = [&](int u) {   // called for u = 0, 1, ... in order: the cursor walks along
        const bool in = FULL || base + (int64_t)(u * TH + threadIdx.x) * 16 < total;
        c[u] = in ? load<kNTL>(src + u * TH) : v4u{0u, 0u, 0u, 0u};
        s[u] = in ? load<false>(cur.ptr()) : 0.0f;
        cur.next();
    };
    fetch_start<U, AHEAD>(fetch);
#pragma unroll
    for (int u = 0; u < U; u++) {
        fetch_step<U, AHEAD>(u, fetch, c[u].x, __float_as_uint(s[u]));
        body(u, c[u], s[u]);
    }
}

template <int U, bool FULL, int TH>
__device__ __forceinline__ void rq_mxfp8_body(const lpq_requant_tensor& d, int64_t base, int64_t total) {
    v4u* dst = reinterpret_cast<v4u*>(d.dst);
    uint8_t* esc = reinterpret_cast<uint8_t*>(d.dst_scale);
    const int tid = threadIdx.x;
    rq_stream<U, FULL, LPQ_RQM_AHEAD != 0, TH>(d, base, total, [&](int u, const v4u& c, float s) {
        const int64_t e0 = base + (int64_t)(u * TH + tid) * 16;
        const Y16 y = fp8blk_values16(c, s);
        // a pair of lanes is one 32-element block
        const uint32_t byte = mx_scale_byte(pair_max(y.amax));
        const float X = ue8m0_operand(byte);
        const v2u q0 = mx_encode8(y.lo, X);
        const v2u q1 = mx_encode8(y.hi, X);
        if (FULL || e0 < total) {
            store<kNTS>(dst + (e0 >> 4), v4u{q0.x, q0.y, q1.x, q1.y});
            if ((tid & 1) == 0) store_u8(esc + (e0 >> 5), byte);
        }
    });
}

template <int U, int TH, bool GROUPED>
__global__ __launch_bounds__(TH) void k_requant_mxfp8(const lpq_requant_tensor* table, lpq_requant_tensor one,
                                                            ChunkMap map) {
    const WorkT<lpq_requant_tensor> W = locate<GROUPED>(table, one, map);
    const int64_t total = W.d.rows * W.d.cols;
    const int64_t base = W.unit * rq_chunk_elems<U, TH>();
    if (base + rq_chunk_elems<U, TH>() <= total) rq_mxfp8_body<U, true, TH>(W.d, base, total);
    else rq_mxfp8_body<U, false, TH>(W.d, base, total);
}

// max |y| of each tensor's dequantized values, max-accumulated into its group
// slot.  |fl(code * s)| = fl(|code| * |s|) and BF16 rounding is monotone, so
// the maximum is taken over fl(max|code| * |s|) and rounded once.
template <int U, bool FULL, int TH>
__device__ __forceinline__ float rq_amax_body(const lpq_requant_tensor& d, int64_t base, int64_t total) {
    v4u c[U];
    float s[U];
    rq_load<U, FULL, TH>(c, s, d, base, total);
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < U; u++) {
        float cm = 0.0f;
        const uint32_t w[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
            const float2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
            cm = fmaxf(fmaxf(cm, fabsf(a[0])), fabsf(a[1]));
            cm = fmaxf(fmaxf(cm, fabsf(b[0])), fabsf(b[1]));
        }
        m = fmaxf(m, cm * fabsf(s[u]));   // vectors past the end have codes and scale 0
    }
    return m;
}

template <int U, int TH, bool GROUPED>
__global__ __launch_bounds__(TH) void k_requant_amax(const lpq_requant_tensor* table, lpq_requant_tensor one,
                                                           ChunkMap map, float* group_amax) {
    const WorkT<lpq_requant_tensor> W = locate<GROUPED>(table, one, map);
    const int64_t total = W.d.rows * W.d.cols;
    const int64_t base = W.unit * rq_chunk_elems<U, TH>();
    const int tid = threadIdx.x;
    const float m = base + rq_chunk_elems<U, TH>() <= total ? rq_amax_body<U, true, TH>(W.d, base, total)
                                                        : rq_amax_body<U, false, TH>(W.d, base, total);
    uint32_t mb = (bf16x2(m, 0.0f) & 0xffffu) << 16;
    mb = wave_max(mb);
    __shared__ uint32_t part[TH / 64];
    if ((tid & 63) == 0) part[tid >> 6] = mb;
    __syncthreads();
    if (tid == 0) {
        uint32_t r = part[0];
#pragma unroll
        for (int k = 1; k < TH / 64; k++) r = umax(r, part[k]);
        atomicMax(reinterpret_cast<unsigned int*>(group_amax + (GROUPED ? W.d.group : 0)), r);
    }
}

template <int U, bool FULL, bool LARGE, bool POW2, int TH>
__device__ __forceinline__ void rq_nvfp4_steps(const lpq_requant_tensor& d, int64_t base, int64_t total,
                                               const GlobalScale& G, const v4u (&c)[U], const float (&s)[U]) {
    // the chunk's origins (uniform): one 8-byte code word and one scale byte per lane and step
    v2u* dst = reinterpret_cast<v2u*>(d.dst) + base / 16;
    uint8_t* ssc = reinterpret_cast<uint8_t*>(d.dst_scale) + base / 16;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int i = u * TH + threadIdx.x;
        const Y16 y = fp8blk_values16<POW2>(c[u], s[u]);
        // one lane is one 16-element block
        const BlockScale B = block_scale<LARGE>(y.amax, G);
        const v2u p = v2u{e2m1x8(y.lo, B), e2m1x8(y.hi, B)};
        if (FULL || base + (int64_t)i * 16 < total) {
            store<kNTS>(dst + i, p);
            store_u8(ssc + i, B.code);
        }
    }
}

// Every load of a lane issued up front, its U tile scales first (one scale when
// all its steps fall in one tile): the wave then learns from the scales alone
// (without waiting for its codes) whether all its tiles have power-of-two
// scales, and runs the steps with the exact scaled-convert dequantization if so
// (the block scales a trainer writes unless FP32 block scales are asked for:
// "Low Precision RL", "2. Unified block-wise FP8"), else with multiply and
// rounding.  Both paths test the same range, 2^k with -121 <= k <= 119.
template <int U, bool FULL, bool LARGE, int TH>
__device__ __forceinline__ void rq_nvfp4_body(const lpq_requant_tensor& d, int64_t base, int64_t total,
                                              const GlobalScale& G) {
    const v4u* src = reinterpret_cast<const v4u*>(d.src) + base / 16 + threadIdx.x;
    TileCursor<16, TH> cur(d.src_scale, d.cols, base);
    v4u c[U];
    // A full chunk whose steps are whole rows apart (N divides the step) and whose
    // rows stay inside every lane's tile row gives each lane one tile for all its
    // steps: one scale load, no walk (uniform test).
    if (FULL && cur.sc == 0u && !any_lane((cur.r >> 7) != ((cur.r + (U - 1) * cur.sr) >> 7))) {
        const float s0 = load<false>(cur.ptr());
#pragma unroll
        for (int u = 0; u < U; u++) {
            c[u] = load<kNTL>(src + u * TH);
            __asm__ volatile("" ::: "memory");
        }
        const uint32_t b0 = __float_as_uint(s0);
        const bool pow2 = (b0 & 0x807fffffu) == 0u && b0 >= (6u << 23) && b0 <= (246u << 23);
        float s[U];
#pragma unroll
        for (int u = 0; u < U; u++) s[u] = s0;
        if (!any_lane(!pow2)) rq_nvfp4_steps<U, FULL, LARGE, true, TH>(d, base, total, G, c, s);
        else rq_nvfp4_steps<U, FULL, LARGE, false, TH>(d, base, total, G, c, s);
        return;
    }
    float s[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
        const bool in = FULL || base + (int64_t)(u * TH + threadIdx.x) * 16 < total;
        s[u] = in ? load<false>(cur.ptr()) : 0.0f;
        cur.next();
    }
    // the code vectors in step order (an empty asm that clobbers memory after each
    // load keeps the compiler from regrouping them), so that step u waits for its
    // own vector only
#pragma unroll
    for (int u = 0; u < U; u++) {
        const bool in = FULL || base + (int64_t)(u * TH + threadIdx.x) * 16 < total;
        c[u] = in ? load<kNTL>(src + u * TH) : v4u{0u, 0u, 0u, 0u};
        __asm__ volatile("" ::: "memory");
    }
    // every scale 2^k, -121 <= k <= 119 (fp8blk_values16<true> is exact there): sign
    // and significand bits all clear, the smallest and largest bit patterns in range
    uint32_t frac = 0u, lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const uint32_t b = __float_as_uint(s[u]);
        frac |= b & 0x807fffffu;
        lo = umin(lo, b);
        hi = umax(hi, b);
    }
    const bool pow2 = frac == 0u && lo >= (6u << 23) && hi <= (246u << 23);
    if (!any_lane(!pow2)) rq_nvfp4_steps<U, FULL, LARGE, true, TH>(d, base, total, G, c, s);
    else rq_nvfp4_steps<U, FULL, LARGE, false, TH>(d, base, total, G, c, s);
}

template <int U, int TH, bool GROUPED>
__global__ __launch_bounds__(TH) void k_requant_nvfp4(const lpq_requant_tensor* table, lpq_requant_tensor one,
                                                            ChunkMap map, const float* group_amax, float* group_g) {
    const WorkT<lpq_requant_tensor> W = locate<GROUPED>(table, one, map);
    const int64_t total = W.d.rows * W.d.cols;
    const int64_t base = W.unit * rq_chunk_elems<U, TH>();
    const int gi = GROUPED ? W.d.group : 0;
    const GlobalScale G = global_scale(group_amax[gi], map.gdiv);
    if (W.unit == 0 && threadIdx.x == 0) group_g[gi] = G.g;   // same value from every member
    if (base + rq_chunk_elems<U, TH>() <= total) {   // uniform, as is G.large
        if (G.large) rq_nvfp4_body<U, true, true, TH>(W.d, base, total, G);
        else rq_nvfp4_body<U, true, false, TH>(W.d, base, total, G);
    } else {
        rq_nvfp4_body<U, false, false, TH>(W.d, base, total, G);
    }
}

// Block-wise FP8 dequantization in the flat layout: used when N % 16 == 0 and
// the arrays are 16-byte aligned (the host checks every tensor of the call), so
// the codes stream contiguously instead of in 128-byte tile rows.  Same
// arithmetic as k_fp8blk_dequant: y = BF16(fl(code * s_tile)).
// A lane takes 8 codes (8 bytes) per step so that its 16 output bytes make
// each store instruction one contiguous span across the wave.
template <int U, bool FULL, bool AHEAD, int TH>
__device__ __forceinline__ void fp8blk_dequant_flat_body(const lpq_tensor& d, int64_t base, int64_t total) {
    const v2u* src = reinterpret_cast<const v2u*>(d.src) + base / 8 + threadIdx.x;
    v4u* dst = reinterpret_cast<v4u*>(d.dst);
    TileCursor<8, TH> cur(reinterpret_cast<const float*>(d.scale), d.cols, base);
    v2u c[U];
    float s[U];
    auto fetch = [&](int u) {   // called for u = 0, 1, ... in order: the cursor walks along
        const bool in = FULL || base + (int64_t)(u * TH + threadIdx.x) * 8 < total;
        c[u] = in ? load<kNTL>(src + u * TH) : v2u{0u, 0u};
        s[u] = in ? load<false>(cur.ptr()) : 0.0f;
        cur.next();
    };
    fetch_start<U, AHEAD>(fetch);
#pragma unroll
    for (int u = 0; u < U; u++) {
        fetch_step<U, AHEAD>(u, fetch, c[u].x, __float_as_uint(s[u]));
        const int64_t e0 = base + (int64_t)(u * TH + threadIdx.x) * 8;
        const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[u].x, false);
        const float2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[u].x, true);
        const float2_t e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[u].y, false);
        const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[u].y, true);
        const float sc = s[u];
        const v4u o = v4u{bf16x2(a[0] * sc, a[1] * sc), bf16x2(b[0] * sc, b[1] * sc), bf16x2(e[0] * sc, e[1] * sc),
                          bf16x2(f[0] * sc, f[1] * sc)};
        if (FULL || e0 < total) store<kNTS>(dst + (e0 >> 3), o);
    }
}

template <int U, int TH = kThreads>
constexpr int64_t dqf_chunk_elems() {
    static_assert(TH % 64 == 0 && TH >= 64 && TH <= kMaxFlatThreads, "whole waves, at most kMaxFlatThreads");
    return (int64_t)TH * 8 * U;
}

template <int U, int TH, bool GROUPED>
__global__ __launch_bounds__(TH) void k_fp8blk_dequant_flat(const lpq_tensor* table, lpq_tensor one,
                                                                  ChunkMap map) {
    const Work W = locate<GROUPED>(table, one, map);
    const int64_t total = W.d.rows * W.d.cols;
    const int64_t base = W.unit * dqf_chunk_elems<U, TH>();
    constexpr bool AHEAD = LPQ_DQF_AHEAD != 0;
    if (base + dqf_chunk_elems<U, TH>() <= total) fp8blk_dequant_flat_body<U, true, AHEAD, TH>(W.d, base, total);
    else fp8blk_dequant_flat_body<U, false, AHEAD, TH>(W.d, base, total);
}

// Block-wise FP8 -> block-wise FP8, TW adjacent 128x128 tiles per workgroup:
// each tile's codes stay in registers (16 per lane per pass); the amax of the
// dequantized values y = BF16(fl(code * s)) gives the new scale
// s' = fl(amax/448), and each y is encoded as E4M3(fl(y / s')).  Lane t covers
// codes 16*(t % (8 TW)) .. +16 of rows (TW*256/(8 TW))*pass + t / (8 TW).
// The new code depends on the old code alone once s and s' are fixed, so each
// tile's 256 possible codes are encoded once (one per lane of the tile, the
// same operations as per element) into a table in LDS, and every element then
// takes its new code from the table.
template <int TW>
struct RqWideShape {
    static constexpr int threads = 256 * TW;
    static constexpr int lanes_per_row = 8 * TW;
    static constexpr int rows_per_pass = threads / lanes_per_row;   // 32
    static constexpr int passes = kTile / rows_per_pass;             // 4
};

template <int TW, bool GROUPED>
__global__ __launch_bounds__(256 * TW) void k_requant_fp8blk(const lpq_requant_tensor* table, lpq_requant_tensor one,
                                                             ChunkMap map) {
    using S = RqWideShape<TW>;
    const WorkT<lpq_requant_tensor> W = locate<GROUPED>(table, one, map);
    const lpq_requant_tensor& d = W.d;
    const int64_t M = d.rows, N = d.cols;
    const int64_t tn = (N + kTile - 1) / kTile, tnw = (tn + TW - 1) / TW;
    const int64_t tr = W.unit / tnw, tcw = W.unit % tnw;
    const int64_t r0 = tr * kTile, c0 = tcw * kTile * TW;
    const int64_t rows = M - r0 < kTile ? M - r0 : kTile;
    const int64_t cols = N - c0 < kTile * TW ? N - c0 : kTile * TW;
    const uint8_t* q = d.src;
    uint8_t* qo = reinterpret_cast<uint8_t*>(d.dst);
    const int tid = threadIdx.x;
    const int lr = tid / S::lanes_per_row;          // row inside a pass
    const int lc = (tid % S::lanes_per_row) * 16;   // first column of the lane's 16 codes in the strip
    const int sub = lc / kTile;                     // the lane's tile within the strip
    const bool present = sub * kTile < cols;
    const float s = present ? d.src_scale[tr * tn + tcw * TW + sub] : 0.0f;
    const int64_t origin = r0 * N + c0;             // offset of the strip in the tensor
    __shared__ uint32_t recode[TW * 64];            // new code of each old code, 256 bytes per tile

    // FAST: 16-byte aligned rows (N % 16 == 0, so a lane's 16 columns are all inside
    // the tensor or all outside) whose buffer offsets (< 128 * N) fit 32 bits; edge
    // strips included, lanes outside the tensor taking code 0 and storing nothing.
    // It keeps the strip's codes in registers between the amax and the encode.  The
    // general body (any other tensor) reads each pass twice, the second time from
    // cache, so that its registers stay below the fast body's.
    auto body = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
        const uint32_t lane_off = (uint32_t)lr * (uint32_t)N + (uint32_t)lc;   // < 2^27 when FAST
        const __amdgpu_buffer_rsrc_t rs = buffer_of(q + origin, M * N - origin);
        const bool in_c = lc < cols;   // the lane's columns are inside the tensor
        auto in_r = [&](int p) { return S::rows_per_pass * p + lr < rows; };
        auto gather = [&](int p) {   // general body: pass p of the lane, code 0 outside the tensor
            const int64_t r = S::rows_per_pass * p + lr;
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            for (int k = 0; k < 16; k++)
                if (r < rows && lc + k < cols) w[k >> 2] |= (uint32_t)q[(r0 + r) * N + c0 + lc + k] << (8 * (k & 3));
            return v4u{w[0], w[1], w[2], w[3]};
        };
        // tile amax of y: BF16 rounding is monotone, so round fl(max|code| * |s|) once
        auto code_max = [](const v4u& c, float cm) {
            const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
                const float2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
                cm = fmaxf(fmaxf(cm, fabsf(a[0])), fabsf(a[1]));
                cm = fmaxf(fmaxf(cm, fabsf(b[0])), fabsf(b[1]));
            }
            return cm;
        };
        v4u c[FAST ? S::passes : 1];
        float cm = 0.0f;
        if constexpr (FAST) {
            // lanes outside the columns read the strip's first code of their row
            // (rows past the end of the tensor read as 0: buffer range check), then zero
            const uint32_t ld_off = in_c ? lane_off : 0u;
#pragma unroll
            for (int p = 0; p < S::passes; p++) c[p] = buffer_load16(rs, ld_off, (uint32_t)(S::rows_per_pass * p * N));
#pragma unroll
            for (int p = 0; p < S::passes; p++) {
                if (!(in_c && in_r(p))) c[p] = v4u{0u, 0u, 0u, 0u};
                cm = code_max(c[p], cm);
            }
        } else {
#pragma unroll 1
            for (int p = 0; p < S::passes; p++) cm = code_max(gather(p), cm);
        }
        const uint32_t mb = bf16_in_f32(cm * fabsf(s));   // codes outside the tensor read as 0
        const float amax = __uint_as_float(strip_reduce_max<8, TW, S::threads>(mb, sub));
        const float s2 = amax / kE4M3Max;   // correctly rounded division
        if (lr == 0 && (lc & (kTile - 1)) == 0 && present)
            reinterpret_cast<float*>(d.dst_scale)[tr * tn + tcw * TW + sub] = s2;
        const bool tiny = s2 > 0.0f && s2 < kTinyScale;
        const float sd = tiny ? s2 * kPreScale : s2;
        const float r = s2 > 0.0f ? rcp_rn(sd) : 0.0f;
        {
            // this lane's entry of its tile's table: old code `cd` (the tile's 256
            // lanes take the 256 codes), y = BF16(fl(code * s)), then E4M3(fl(y / s'))
            // (y and s' pre-scaled alike when s' is tiny)
            const uint32_t cd = ((uint32_t)lr << 3) | ((uint32_t)tid & 7u);
            const float2_t v = __builtin_amdgcn_cvt_pk_f32_fp8((int)cd, false);
            float x = __uint_as_float(bf16_in_f32(v[0] * s));
            if (tiny) x *= kPreScale;
            const float qv = quot_rn(x, sd, r);
            reinterpret_cast<uint8_t*>(recode)[sub * 256 + cd] = (uint8_t)e4m3x2<false>(qv, qv, 0u);
        }
        __syncthreads();
        const uint8_t* lut = reinterpret_cast<const uint8_t*>(recode) + sub * 256;

        auto encode = [&](int p, const v4u& cp) {
            const uint32_t w[4] = {cp.x, cp.y, cp.z, cp.w};
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; k++)
                o[k] = (uint32_t)lut[w[k] & 0xffu] | ((uint32_t)lut[(w[k] >> 8) & 0xffu] << 8) |
                       ((uint32_t)lut[(w[k] >> 16) & 0xffu] << 16) | ((uint32_t)lut[w[k] >> 24] << 24);
            const int64_t row = S::rows_per_pass * p + lr;
            if constexpr (FAST) {
                if (in_c && row < rows)
                    store_at(qo + origin + (int64_t)S::rows_per_pass * p * N, lane_off, v4u{o[0], o[1], o[2], o[3]});
            } else if (row < rows) {
                for (int k = 0; k < 16; k++)
                    if (lc + k < cols) qo[(r0 + row) * N + c0 + lc + k] = (uint8_t)(o[k >> 2] >> (8 * (k & 3)));
            }
        };
        if constexpr (FAST) {
#pragma unroll
            for (int p = 0; p < S::passes; p++) encode(p, c[p]);
        } else {
#pragma unroll 1
            for (int p = 0; p < S::passes; p++) encode(p, gather(p));
        }
    };
    if ((N & 15) == 0 && N <= (1 << 23) &&
        ((reinterpret_cast<uintptr_t>(d.src) | reinterpret_cast<uintptr_t>(d.dst)) & 15) == 0)
        body(Full<true>{});
    else
        body(Full<false>{});
}

}  // namespace
