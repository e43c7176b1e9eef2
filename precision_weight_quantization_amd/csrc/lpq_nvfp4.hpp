// NVFP4: global and block scales, E2M1 encode/decode, the W4A4 observers, the
// amax pass, quantize, dequantize and QDQ.
//
// Part of lpq_kernels.hip, which includes each part once, in this order: one
// translation unit.
#pragma once

namespace {

// ---------------------------------------------------------------------------
// NVFP4
// ---------------------------------------------------------------------------

// Per-tensor quantities derived from the group amax A: g = fl(A / 2688) and
// what the block-scale division by g needs.
struct GlobalScale {
    float g;       // the global scale
    float gd;      // divisor used for fl(t / g): g, or g * 2^64 when g is tiny
    float rg;      // RN(1 / gd)
    bool tiny;     // g < 2^-90: t and g are pre-scaled by 2^64
    bool large;    // g >= 2^-81: every nonzero block multiplier S = E4M3value * g
                   // is at least 2^-9 * 2^-81 = 2^-90, so none is pre-scaled
};

__device__ __forceinline__ GlobalScale global_scale(float A, float gdiv) {
    GlobalScale G;
    G.g = A / gdiv;  // correctly rounded division (gdiv = 6 * E4M3 maximum)
    G.tiny = G.g < kTinyScale;
    G.large = G.g >= 0x1p-81f;
    G.gd = G.tiny ? G.g * kPreScale : G.g;
    G.rg = G.g > 0.0f ? rcp_rn(G.gd) : 0.0f;
    return G;
}

// Block of 16 with amax b (binary32 bits): E4M3 block-scale code, the block
// multiplier S = fl(E4M3value * g), and the divisor state for the elements.
struct BlockScale {
    uint32_t code;
    float S;       // multiplier for dequantization
    float Sd;      // divisor for the quotient: S, or S * 2^64 when S is tiny
    float r;       // RN(1 / Sd), or 0 when S == 0
    float xpre;    // 1, or 2^64 when S is tiny
    bool maybe_tiny;   // wave-uniform: some S of the group could be tiny
};

// LARGE: the caller has established G.large (a group-uniform fact), so neither g
// nor any block multiplier is pre-scaled and the pre-scaling selects drop out.
// LARGE = false is correct for every G.
template <bool LARGE = false>
__device__ __forceinline__ BlockScale block_scale(uint32_t bmax_bits, const GlobalScale& G) {
    BlockScale B;
    const float b = __uint_as_float(bmax_bits);
    // fl(b / 6): the short sequence is exact while the quotient is normal;
    // tinier blocks take the full correctly rounded division.
    float t6 = quot_rn(b, 6.0f, kRcp6);
    if (any_lane(b < 0x1p-100f)) {
        float bb = b;
        __asm__ volatile("" : "+v"(bb));   // an empty barrier: keeps the long division inside the branch
        if (bb < 0x1p-100f) t6 = bb / 6.0f;
    }
    const float t = (!LARGE && G.tiny) ? t6 * kPreScale : t6;   // group-uniform pre-scaling
    const float u = quot_rn(t, G.gd, G.rg);                      // fl(fl(b / 6) / g)
    const float uc = __builtin_amdgcn_fmed3f(u, -kE4M3Max, kE4M3Max);
    // the conversion writes the low 16 bits (the code, then E4M3(0) = 0) and keeps
    // the rest of its last operand, here the dead bits of b
    const uint32_t c8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(uc, 0.0f, (int)bmax_bits, false) & 0xffu;
    B.code = (LARGE || G.g > 0.0f) ? c8 : 0u;
    B.S = e4m3_to_f32(B.code) * G.g;
    B.maybe_tiny = !LARGE && !G.large;
    if (LARGE || G.large) {   // group-uniform: no block multiplier is tiny
        B.xpre = 1.0f;
        B.Sd = B.S;
    } else {
        const bool tiny = B.S > 0.0f && B.S < kTinyScale;
        B.xpre = tiny ? kPreScale : 1.0f;
        B.Sd = tiny ? B.S * kPreScale : B.S;
    }
    B.r = B.S > 0.0f ? rcp_rn(B.Sd) : 0.0f;
    return B;
}

// 8 BF16 values -> 8 E2M1 codes (one 32-bit word, element 0 in the low nibble).
__device__ __forceinline__ uint32_t e2m1x8(const F8& f, const BlockScale& B) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; k++) x[k] = f.x[k];
    if (B.maybe_tiny && any_lane(B.xpre != 1.0f)) {
#pragma unroll
        for (int k = 0; k < 8; k++) x[k] *= B.xpre;
    }
    float q[8];
#pragma unroll
    for (int k = 0; k < 8; k++) q[k] = quot_rn(x[k], B.Sd, B.r);
    // the four converts write the word's four bytes, so it starts from any value
    // (one already in a register)
    uint32_t p = __float_as_uint(q[0]);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, q[0], q[1], 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, q[2], q[3], 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, q[4], q[5], 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, q[6], q[7], 1.0f, 3);
    return p;
}

// 8 E2M1 codes (one word) times S -> 8 BF16 values.
__device__ __forceinline__ v4u e2m1x8_to_bf16(uint32_t p, float S) {
    float2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 0);
    float2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 1);
    float2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 2);
    float2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.0f, 3);
    v4u o;
    o.x = bf16x2(f0[0] * S, f0[1] * S);
    o.y = bf16x2(f1[0] * S, f1[1] * S);
    o.z = bf16x2(f2[0] * S, f2[1] * S);
    o.w = bf16x2(f3[0] * S, f3[1] * S);
    return o;
}

// ---------------------------------------------------------------------------
// W4A4 activation observers
// ---------------------------------------------------------------------------
//
// Observer state (caller-owned device memory, LPQ_OBSERVER_STATE_FLOATS
// words): [0] min, [1] max, [2] batches seen (FP32); then the call's control
// words, each on a cache line of its own so that the workgroups' atomics on
// them do not queue behind one another: [32] / [64] the current batch's min /
// max as order-preserving keys and [96] the number of workgroups of the
// current call that have folded in their keys.  The kernels take the control
// words through a pointer of their own (`ctl`, at the same offsets): the
// state itself, or a block the library holds.  Keys map binary32 bits to
// unsigned integers whose order is the values' order with -0 below +0:
// non-negative values get the sign bit set, negative values have every bit
// flipped.
constexpr int kObsKeyMin = 32, kObsKeyMax = 64, kObsArrived = 96;
constexpr int kObsCtlWords = 128;   // a control block: 512 bytes

__device__ __forceinline__ uint32_t order_key(uint32_t u) { return (u >> 31) ? ~u : (u | 0x80000000u); }
__device__ __forceinline__ uint32_t key_bits(uint32_t k) { return (k >> 31) ? (k & 0x7fffffffu) : ~k; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

constexpr uint32_t kKeyMinIdentity = 0xffffffffu;
constexpr uint32_t kKeyMaxIdentity = 0u;

__device__ __forceinline__ void observer_arm(uint32_t* ctl) {
    ctl[kObsKeyMin] = kKeyMinIdentity;
    ctl[kObsKeyMax] = kKeyMaxIdentity;
    ctl[kObsArrived] = 0u;
}

__global__ void k_observer_reset(uint32_t* state) {
    const int i = threadIdx.x;
    if (i < 3) state[i] = 0u;
    if (i == 0) observer_arm(state);
}

// Keys at their identities and no arrivals: a control block ready for a call.
__global__ void k_observer_arm(uint32_t* ctl) {
    if (threadIdx.x == 0) observer_arm(ctl);
}

__device__ __forceinline__ uint32_t dev_atomic_xchg(uint32_t* p, uint32_t v) {
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Applies the observer rule to the batch extremes (one thread), writes the
// activation amax and re-arms the batch keys.  Same operations, in the same
// order, as the definition: m += c * (b - m) for the moving average.  The keys
// are taken (and reset to their identities) with device-scope atomic
// exchanges, performed where the other workgroups' key atomics were.
__device__ void observer_apply(int kind, float c, float* f, uint32_t* ctl, float* amax) {
    const uint32_t kmin = dev_atomic_xchg(ctl + kObsKeyMin, kKeyMinIdentity);
    const uint32_t kmax = dev_atomic_xchg(ctl + kObsKeyMax, kKeyMaxIdentity);
    const float bmin = __uint_as_float(key_bits(kmin)), bmax = __uint_as_float(key_bits(kmax));
    float mn = f[0], mx = f[1];
    if (kind == LPQ_OBSERVER_MEMORYLESS_MINMAX || f[2] == 0.0f) {
        mn = bmin;
        mx = bmax;
    } else if (kind == LPQ_OBSERVER_STATIC_MINMAX) {
        if (kmin < order_key(__float_as_uint(mn))) mn = bmin;
        if (kmax > order_key(__float_as_uint(mx))) mx = bmax;
    } else {
        mn = mn + c * (bmin - mn);
        mx = mx + c * (bmax - mx);
    }
    f[0] = mn;
    f[1] = mx;
    f[2] = f[2] + 1.0f;
    *amax = fmaxf(fabsf(mn), fabsf(mx));
}

// min / max of one BF16 tensor into the batch keys of the state; the last
// workgroup to fold in its keys applies the observer rule (no workgroup waits
// for another: each counts its arrival after its keys are in, and the one
// that arrives last finds every key there).
template <int U>
__global__ __launch_bounds__(kThreads) void k_minmax(lpq_tensor one, int kind, float c, float* state, uint32_t* ctl,
                                                     float* amax) {
    const int64_t total = one.rows * one.cols;
    const int64_t base = (int64_t)blockIdx.x * chunk_elems<U>();
    const v4u* src = reinterpret_cast<const v4u*>(one.src);
    uint32_t lo = kKeyMinIdentity, hi = kKeyMaxIdentity;
    by_fullness<chunk_elems<U>()>(base, total, [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
        v4u v[U];
        load_chunk<U, FULL>(v, src, base, total);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t e0 = base + (int64_t)(u * kThreads + threadIdx.x) * 8;
            if (!FULL && e0 >= total) continue;   // past the end (N % 8 == 0: vectors are whole)
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t a = order_key(w[k] << 16), b = order_key(w[k] & 0xffff0000u);
                lo = umin(lo, umin(a, b));
                hi = umax(hi, umax(a, b));
            }
        }
    });
    lo = ~wave_max(~lo);   // min through the max reduction on complements
    hi = wave_max(hi);
    __shared__ uint32_t plo[kThreads / 64], phi[kThreads / 64];
    if ((threadIdx.x & 63) == 0) {
        plo[threadIdx.x >> 6] = lo;
        phi[threadIdx.x >> 6] = hi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t l = plo[0], h = phi[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; k++) {
            l = umin(l, plo[k]);
            h = umax(h, phi[k]);
        }
        atomicMin(ctl + kObsKeyMin, l);
        atomicMax(ctl + kObsKeyMax, h);
        // this workgroup's keys before its arrival; the last arriver's reads after every arrival
        if (__hip_atomic_fetch_add(ctl + kObsArrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
            gridDim.x - 1) {
            observer_apply(kind, c, state, ctl, amax);
            __hip_atomic_store(ctl + kObsArrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // re-armed
        }
    }
}

// fl(A / gdiv) per entry, gdiv = 6 * the E4M3 maximum (2688 or 1536): the
// multiplier form of a global scale.  out may be amax itself (each entry is
// read, then written, by one thread).
__global__ __launch_bounds__(kThreads) void k_global_scale(const float* amax, int32_t n, float* out, float gdiv) {
    const int32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) out[i] = amax[i] / gdiv;   // correctly rounded division
}

// fl(2688 / A) per group: the reciprocal form of the global scale.
__global__ __launch_bounds__(kThreads) void k_global_scale_reciprocal(const float* amax, int32_t n, float* out) {
    const int32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) out[i] = 2688.0f / amax[i];   // correctly rounded division
}

__global__ __launch_bounds__(kThreads) void k_fill_f32(float* p, int64_t n, float v) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = v;
}

// max |w| of each tensor, max-accumulated into its group slot (binary32 bits
// of non-negative values order like unsigned integers).
template <int U, int TH, bool GROUPED>
__global__ __launch_bounds__(TH) void k_amax(const lpq_tensor* table, lpq_tensor one, ChunkMap map,
                                                   float* group_amax) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const v4u* src = reinterpret_cast<const v4u*>(d.src);
    const int tid = threadIdx.x;
    uint32_t m = 0;
    by_fullness<chunk_elems<U, TH>()>(base, total, [&](auto full) {
        v4u v[U];   // vectors past the end read as zero
        load_chunk<U, decltype(full)::value, TH>(v, src, base, total);
#pragma unroll
        for (int u = 0; u < U; u++) m = umax(m, absmax8_bits(v[u]));
    });
    m = wave_max(m);
    __shared__ uint32_t part[TH / 64];
    if ((tid & 63) == 0) part[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        uint32_t w = part[0];
#pragma unroll
        for (int k = 1; k < TH / 64; k++) w = umax(w, part[k]);
        atomicMax(reinterpret_cast<unsigned int*>(group_amax + (GROUPED ? d.group : 0)), w);
    }
}

template <int U, int TH, bool GROUPED, bool AHEAD = LPQ_NVQ_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_nvfp4_quant(const lpq_tensor* table, lpq_tensor one, ChunkMap map,
                                                          const float* group_amax, float* group_g) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const int gi = GROUPED ? d.group : 0;
    const GlobalScale G = global_scale(group_amax[gi], map.gdiv);
    const int tid = threadIdx.x;
    // same value from every member; no g pointer: the amax slot is turned into g
    // by a later launch (the call whose amax the library computes)
    if (group_g != nullptr && W.unit == 0 && tid == 0) group_g[gi] = G.g;
    // the chunk's origins (uniform); a lane's vector i = u * TH + tid is addressed
    // with a 32-bit offset from them
    const v4u* src = reinterpret_cast<const v4u*>(d.src) + base / 8;
    uint32_t* dst = reinterpret_cast<uint32_t*>(d.dst) + base / 8;
    uint8_t* ssc = reinterpret_cast<uint8_t*>(d.scale) + base / 16;
    const int64_t left = total - base;   // elements from the chunk origin to the end

    auto run = [&](auto full, auto large) {
        constexpr bool FULL = decltype(full)::value, LARGE = decltype(large)::value;
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
            const F8 f = widen8(v[u]);
            const BlockScale B = block_scale<LARGE>(pair_max(absmax8_f32(f)), G);
            const uint32_t p = e2m1x8(f, B);
            if (in(i)) {
                store<kNTS>(dst + i, p);
                if ((tid & 1) == 0) store_u8(ssc + u * (TH / 2) + (tid >> 1), B.code);
            }
        }
    };
    const bool full = base + chunk_elems<U, TH>() <= total;   // uniform, as is G.large
    if (full) {
        if (G.large) run(Full<true>{}, Full<true>{});
        else run(Full<true>{}, Full<false>{});
    } else {
        run(Full<false>{}, Full<false>{});
    }
}

template <int U, int TH, bool GROUPED, bool AHEAD = LPQ_NVD_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_nvfp4_dequant(const lpq_tensor* table, lpq_tensor one, ChunkMap map,
                                                            const float* group_g) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const float g = group_g[GROUPED ? d.group : 0];
    const uint32_t* src = reinterpret_cast<const uint32_t*>(d.src);
    const uint8_t* ssc = reinterpret_cast<const uint8_t*>(d.scale);
    v4u* dst = reinterpret_cast<v4u*>(d.dst);
    const int tid = threadIdx.x;

    by_fullness<chunk_elems<U, TH>()>(base, total, [&](auto full) {
        constexpr bool FULL = decltype(full)::value;
        uint32_t p[U], sb[U];
        auto fetch = [&](int u) {
            const int64_t e0 = base + (int64_t)(u * TH + tid) * 8;
            p[u] = load_vec<TH, FULL>(src, base, total, u);
            sb[u] = (FULL || e0 < total) ? load_u8(ssc + (e0 >> 4)) : 0u;
        };
        fetch_start<U, AHEAD>(fetch);
#pragma unroll
        for (int u = 0; u < U; u++) {
            fetch_step<U, AHEAD>(u, fetch, p[u], sb[u]);
            const int64_t e0 = base + (int64_t)(u * TH + tid) * 8;
            const float S = e4m3_to_f32(sb[u]) * g;
            const v4u o = e2m1x8_to_bf16(p[u], S);
            if (FULL || e0 < total) store<kNTS>(dst + (e0 >> 3), o);
        }
    });
}

template <int U, int TH, bool GROUPED, bool AHEAD = LPQ_QDQ_AHEAD != 0>
__global__ __launch_bounds__(TH) void k_nvfp4_qdq(const lpq_tensor* table, lpq_tensor one, ChunkMap map,
                                                        const float* group_amax) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t total = d.rows * d.cols;
    const int64_t base = W.unit * chunk_elems<U, TH>();
    const GlobalScale G = global_scale(group_amax[GROUPED ? d.group : 0], map.gdiv);
    const int tid = threadIdx.x;
    // the chunk's origins (uniform); a lane's vector i = u * TH + tid is addressed
    // with a 32-bit offset from them
    const v4u* src = reinterpret_cast<const v4u*>(d.src) + base / 8;
    v4u* dst = reinterpret_cast<v4u*>(d.dst) + base / 8;
    const int64_t left = total - base;   // elements from the chunk origin to the end

    auto run = [&](auto full, auto large) {
        constexpr bool FULL = decltype(full)::value, LARGE = decltype(large)::value;
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
            const F8 f = widen8(v[u]);
            const BlockScale B = block_scale<LARGE>(pair_max(absmax8_f32(f)), G);
            const v4u o = e2m1x8_to_bf16(e2m1x8(f, B), B.S);
            if (in(i)) store<kNTS>(uniform_ptr(dst + u * TH) + tid, o);
        }
    };
    const bool full = base + chunk_elems<U, TH>() <= total;   // uniform, as is G.large
    if (full) {
        if (G.large) run(Full<true>{}, Full<true>{});
        else run(Full<true>{}, Full<false>{});
    } else {
        run(Full<false>{}, Full<false>{});
    }
}

}  // namespace
