// gfx950 kernels of the low-precision weight codecs and the C ABI that
// launches them (declared in include/lpq.h).
//
// Formats ("Low Precision RL", "Choose a precision"; "verl NVFP4 QAT",
// sections 2.3-2.5 and 3.3): block-wise FP8 (E4M3, FP32 scale per 128x128
// tile), MXFP8 (E4M3, UE8M0 byte per 1x32 block) and NVFP4 (E2M1, E4M3 scale
// per 1x16 block, FP32 global scale amax / 2688 shared by a sibling group),
// plus the NVFP4 fake-quant.  All of it is streaming work bound by HBM
// bandwidth: no kernel here is a contraction, so none uses MFMA.
//
// Launch shape.  A grouped call covers many tensors in one launch.  The grid
// is one-dimensional and dense: the host lays the tensors' work units
// (chunks, or 128x128 tiles) end to end and passes a short table of
// equal-size runs in the kernel arguments; each workgroup finds its tensor
// from that table with scalar compares and one division, then reads the
// descriptor into scalar registers.
// No workgroup is launched without work.
//  * MXFP8 / NVFP4 / INT4 are flat in memory (N is a multiple of the block),
//    so a workgroup (128, 256 or 512 threads, chosen per kernel) streams
//    16-byte BF16 vectors, 8 elements per lane, U vectors per lane; a 1x32 block is a quad of lanes and a 1x16 block a pair,
//    reduced with DPP lane permutations.  U is 2 to 4 (16 for the read-only
//    amax pass): enough bytes in flight per CU, short-lived workgroups.  A
//    lane's U loads go out either all at once or one vector ahead of the
//    work, chosen per kernel by measurement: the encoders and the MXFP8
//    decoder run faster with fewer reads in flight per wave.  Full chunks
//    (all but a tensor's last) take a body compiled without bounds checks.
//  * Block-wise FP8 quantization gives one workgroup a strip of 2 or 4
//    adjacent 128x128 tiles (one per 256 threads): 16 lanes per 256-byte row
//    segment of a tile, 8 row passes, all values kept in registers between the
//    per-tile amax reduction (DPP + LDS across the waves) and the encode, so
//    HBM is read once.  Dequantization streams flat when the layout allows,
//    else one tile per workgroup.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "lpq.h"
#include "lpq_device.hpp"

// Launch parameters (vectors per lane, workgroup size, non-temporal access);
// the values are the measured best on MI355X for each kernel.
#ifndef LPQ_MXQ_U
#define LPQ_MXQ_U 2
#endif
#ifndef LPQ_MXD_U
#define LPQ_MXD_U 2
#endif
#ifndef LPQ_NVQ_U
#define LPQ_NVQ_U 4
#endif
#ifndef LPQ_NVD_U
#define LPQ_NVD_U 2
#endif
#ifndef LPQ_QDQ_U
#define LPQ_QDQ_U 2
#endif
#ifndef LPQ_AMAX_U
#define LPQ_AMAX_U 32
#endif
#ifndef LPQ_I4Q_U
#define LPQ_I4Q_U 4
#endif
#ifndef LPQ_I4D_U
#define LPQ_I4D_U 2
#endif
#ifndef LPQ_I4QDQ_U
#define LPQ_I4QDQ_U 2
#endif
#ifndef LPQ_RQM_U
#define LPQ_RQM_U 2
#endif
#ifndef LPQ_RQA_U
#define LPQ_RQA_U 16
#endif
#ifndef LPQ_RQN_U
#define LPQ_RQN_U 8
#endif
#ifndef LPQ_DQF_U
#define LPQ_DQF_U 2
#endif
#ifndef LPQ_RQT_TW
#define LPQ_RQT_TW 2
#endif
#ifndef LPQ_TILEQ_TW
#define LPQ_TILEQ_TW 2
#endif
// Block-FP8 quantize launches with at least this many 4-tile strips take 4
// tiles per workgroup instead of LPQ_TILEQ_TW.
#ifndef LPQ_TILEQ_WIDE_TW
#define LPQ_TILEQ_WIDE_TW 4
#endif
#ifndef LPQ_TILEQ_WIDE_MIN
#define LPQ_TILEQ_WIDE_MIN 8192
#endif
#ifndef LPQ_TILEQ_WAVES_PER_SIMD
#define LPQ_TILEQ_WAVES_PER_SIMD 4
#endif
#ifndef LPQ_TILED_THREADS
#define LPQ_TILED_THREADS 1024
#endif
// Load order of the flat kernels (1: one vector ahead, 0: all U up front).
#ifndef LPQ_MXQ_AHEAD
#define LPQ_MXQ_AHEAD 1
#endif
#ifndef LPQ_NVQ_AHEAD
#define LPQ_NVQ_AHEAD 1
#endif
#ifndef LPQ_QDQ_AHEAD
#define LPQ_QDQ_AHEAD 1
#endif
#ifndef LPQ_MXD_AHEAD
#define LPQ_MXD_AHEAD 1
#endif
#ifndef LPQ_NVD_AHEAD
#define LPQ_NVD_AHEAD 0
#endif
#ifndef LPQ_DQF_AHEAD
#define LPQ_DQF_AHEAD 0
#endif
#ifndef LPQ_RQM_AHEAD
#define LPQ_RQM_AHEAD 1
#endif
#ifndef LPQ_RQN_AHEAD
#define LPQ_RQN_AHEAD 0
#endif
#ifndef LPQ_I4Q_AHEAD
#define LPQ_I4Q_AHEAD 0
#endif
#ifndef LPQ_I4D_AHEAD
#define LPQ_I4D_AHEAD 0
#endif
#ifndef LPQ_I4QDQ_AHEAD
#define LPQ_I4QDQ_AHEAD 1
#endif
#ifndef LPQ_NTL
#define LPQ_NTL 1
#endif
#ifndef LPQ_NTS
#define LPQ_NTS 1
#endif

using namespace lpq;

namespace {

#ifndef LPQ_FLAT_THREADS
#define LPQ_FLAT_THREADS 256
#endif
// Workgroup size of each flat kernel (64 to 512, a multiple of 64), measured
// per kernel: the NVFP4 encoder runs best with one wave, MXFP8 encoding and the
// QDQs with 128 threads, the NVFP4 and INT4 decoders and the INT4 encoder with
// 512, the rest with 256.
#ifndef LPQ_MXQ_T
#define LPQ_MXQ_T 128
#endif
#ifndef LPQ_MXD_T
#define LPQ_MXD_T LPQ_FLAT_THREADS
#endif
#ifndef LPQ_AMAX_T
#define LPQ_AMAX_T LPQ_FLAT_THREADS
#endif
#ifndef LPQ_NVQ_T
#define LPQ_NVQ_T 64
#endif
#ifndef LPQ_NVD_T
#define LPQ_NVD_T 512
#endif
#ifndef LPQ_QDQ_T
#define LPQ_QDQ_T 128
#endif
#ifndef LPQ_I4Q_T
#define LPQ_I4Q_T 512
#endif
#ifndef LPQ_I4D_T
#define LPQ_I4D_T 512
#endif
#ifndef LPQ_I4QDQ_T
#define LPQ_I4QDQ_T 128
#endif
#ifndef LPQ_DQF_T
#define LPQ_DQF_T LPQ_FLAT_THREADS
#endif
#ifndef LPQ_RQM_T
#define LPQ_RQM_T LPQ_FLAT_THREADS
#endif
#ifndef LPQ_RQA_T
#define LPQ_RQA_T LPQ_FLAT_THREADS
#endif
#ifndef LPQ_RQN_T
#define LPQ_RQN_T LPQ_FLAT_THREADS
#endif
constexpr int kThreads = LPQ_FLAT_THREADS;   // flat kernels
constexpr int kTile = 128;
constexpr bool kNTL = LPQ_NTL != 0;
constexpr bool kNTS = LPQ_NTS != 0;
constexpr int kMaxSeg = 8;               // segments per launch (longer lists are split)

constexpr int kMaxFlatThreads = 512;   // the largest flat workgroup

// Elements of one flat work unit.  Whole waves per workgroup keep every chunk
// origin a multiple of 512 elements, which the kernels' split of a lane's
// address into a uniform chunk origin plus a lane offset relies on.
template <int U, int TH = kThreads>
constexpr int64_t chunk_elems() {
    static_assert(TH % 64 == 0 && TH >= 64 && TH <= kMaxFlatThreads, "whole waves, at most kMaxFlatThreads");
    return (int64_t)TH * 8 * U;
}

// Loads the lane's U vectors of a flat chunk of a TH-thread workgroup: lane t
// of vector u holds the EV elements starting at base + (u * TH + t) * EV.  A
// full chunk (the common case) loads without per-lane bounds checks.
template <int U, bool FULL, int TH = kThreads, int EV = 8, typename T>
__device__ __forceinline__ void load_chunk(T (&v)[U], const T* src, int64_t base, int64_t total) {
    const T* p = src + base / EV + threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const bool in = FULL || base + (int64_t)(u * TH + threadIdx.x) * EV < total;
        v[u] = in ? load<kNTL>(p + u * TH) : T{};
    }
}

// Waits until the loads that produce x (and y) have arrived, and keeps every
// later memory access behind that point: an empty asm that reads the values
// (the compiler puts the memory-counter wait in front of it) and clobbers
// memory.
__device__ __forceinline__ void arrived(uint32_t x) { __asm__ volatile("" ::"v"(x) : "memory"); }
__device__ __forceinline__ void arrived(uint32_t x, uint32_t y) { __asm__ volatile("" ::"v"(x), "v"(y) : "memory"); }

// Issue order of a lane's U vectors, fetch(u) issuing the loads of vector u.
// All U up front puts the most bytes in flight per wave; one ahead issues
// vector u + 1 once vector u has arrived (step(u, ...) before the work on
// vector u), so a wave holds at most two vectors in flight.  Which is faster
// depends on the kernel's read / write mix and is measured per kernel.
template <int U, bool ONE_AHEAD, typename Fetch>
__device__ __forceinline__ void fetch_start(Fetch&& fetch) {
    fetch(0);
    if constexpr (!ONE_AHEAD) {
#pragma unroll
        for (int u = 1; u < U; u++) fetch(u);
    }
}
template <int U, bool ONE_AHEAD, typename Fetch, typename... X>
__device__ __forceinline__ void fetch_step(int u, Fetch&& fetch, X... have) {
    if constexpr (ONE_AHEAD) {
        if (u + 1 < U) {
            arrived(have...);
            fetch(u + 1);
        }
    }
}

// Vector u of a lane in a flat chunk of EV-element vectors (TH-thread
// workgroup), zero past the end.
template <int TH, bool FULL, int EV = 8, typename T>
__device__ __forceinline__ T load_vec(const T* src, int64_t base, int64_t total, int u) {
    const bool in = FULL || base + (int64_t)(u * TH + threadIdx.x) * EV < total;
    return in ? load<kNTL>(src + base / EV + threadIdx.x + u * TH) : T{};
}

template <bool B>
struct Full {
    static constexpr bool value = B;
};

// Runs body(Full<true>) for a full chunk (every chunk of a tensor but its
// last) and body(Full<false>) otherwise.  Fullness is uniform over the
// workgroup; as a compile-time constant it gives full chunks a straight-line
// body whose loads are all issued before the first wait, where a run-time
// flag would let the compiler merge the two paths around per-lane branches.
template <int64_t CHUNK, typename Body>
__device__ __forceinline__ void by_fullness(int64_t base, int64_t total, Body&& body) {
    if (base + CHUNK <= total) body(Full<true>{});
    else body(Full<false>{});
}

// Dense work map of one launch.  Consecutive tensors with the same number of
// work units form a segment: segment s starts at work unit first[s] and at
// tensor tensor0[s], and each of its tensors owns units[s] work units.
// Grouped calls over expert lists are one to a few segments, so a workgroup
// finds its tensor with a handful of scalar compares and one division (no
// dependent memory access).
struct ChunkMap {
    int32_t nseg;
    float gdiv;                  // NVFP4 global-scale divisor 6 * E4M3 maximum (2688, or 1536)
    uint32_t first[kMaxSeg];
    uint32_t tensor0[kMaxSeg];
    uint32_t units[kMaxSeg];
    double inv_units[kMaxSeg];   // 1 / units[s]
};

template <typename D>
struct WorkT {
    D d;
    int64_t unit;    // chunk or tile index inside the tensor
};
using Work = WorkT<lpq_tensor>;

template <typename T>
using cptr = const __attribute__((address_space(4))) T*;   // constant address space: uniform scalar loads

__device__ __forceinline__ void read_desc(lpq_tensor& o, cptr<lpq_tensor> t) {
    o.src = t->src;
    o.dst = t->dst;
    o.scale = t->scale;
    o.rows = t->rows;
    o.cols = t->cols;
    o.group = t->group;
    o.reserved = 0;
}

__device__ __forceinline__ void read_desc(lpq_requant_tensor& o, cptr<lpq_requant_tensor> t) {
    o.src = t->src;
    o.src_scale = t->src_scale;
    o.dst = t->dst;
    o.dst_scale = t->dst_scale;
    o.rows = t->rows;
    o.cols = t->cols;
    o.group = t->group;
    o.reserved = 0;
}

// The tensor and work unit of this workgroup.  Every quantity is uniform
// across the workgroup and kept in scalar registers, so the descriptor of a
// grouped call is fetched with scalar loads.
template <bool G, typename D>
__device__ __forceinline__ WorkT<D> locate(const D* table, const D& one, const ChunkMap& m) {
    WorkT<D> w;
    if constexpr (!G) {
        w.d = one;
        w.unit = blockIdx.x;
        return w;
    } else {
        const uint32_t b = blockIdx.x;
        // every table entry is read at a constant offset (one batch of scalar
        // loads from the kernel arguments); the segment search stops at the
        // first segment past b (a launch of one segment does no search)
        uint32_t f = 0, u = m.units[0], t0 = 0;
        double inv = m.inv_units[0];
#pragma unroll
        for (int k = 1; k < kMaxSeg; k++) {
            if (k >= m.nseg || m.first[k] > b) break;
            f = m.first[k];
            u = m.units[k];
            t0 = m.tensor0[k];
            inv = m.inv_units[k];
        }
        const uint32_t x = b - f;
        // x / u from a double-precision estimate (off by at most one), corrected
        uint32_t q = (uint32_t)((double)x * inv);
        if ((uint64_t)(q + 1) * u <= x) q += 1;
        else if ((uint64_t)q * u > x) q -= 1;
        q = __builtin_amdgcn_readfirstlane(q);
        read_desc(w.d, (cptr<D>)(table) + t0 + q);
        w.unit = (int64_t)(x - q * u);
        return w;
    }
}

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
    uint32_t p = 0;
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
// Observer state (caller-owned device memory, 8 words): [0] min, [1] max,
// [2] batches seen (FP32), [4] / [5] the current batch's min / max as
// order-preserving keys, [6] the number of workgroups of the current call
// that have folded in their keys.  Keys map binary32 bits to unsigned integers whose
// order is the values' order with -0 below +0: non-negative values get the
// sign bit set, negative values have every bit flipped.

__device__ __forceinline__ uint32_t order_key(uint32_t u) { return (u >> 31) ? ~u : (u | 0x80000000u); }
__device__ __forceinline__ uint32_t key_bits(uint32_t k) { return (k >> 31) ? (k & 0x7fffffffu) : ~k; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

constexpr uint32_t kKeyMinIdentity = 0xffffffffu;
constexpr uint32_t kKeyMaxIdentity = 0u;

__global__ void k_observer_reset(uint32_t* state) {
    const int i = threadIdx.x;
    if (i < 8) state[i] = i == 4 ? kKeyMinIdentity : (i == 5 ? kKeyMaxIdentity : 0u);
}

// Applies the observer rule to the batch extremes (one thread), writes the
// activation amax and re-arms the batch keys.  Same operations, in the same
// order, as the definition: m += c * (b - m) for the moving average.  The keys
// were folded in by device-scope atomics of other workgroups: they are read
// with device-scope atomic loads.
__device__ void observer_apply(int kind, float c, uint32_t* state, float* amax) {
    float* f = reinterpret_cast<float*>(state);
    const uint32_t kmin = __hip_atomic_load(state + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t kmax = __hip_atomic_load(state + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    state[4] = kKeyMinIdentity;
    state[5] = kKeyMaxIdentity;
    *amax = fmaxf(fabsf(mn), fabsf(mx));
}

// min / max of one BF16 tensor into the batch keys of the state; the last
// workgroup to fold in its keys applies the observer rule (no workgroup waits
// for another: each counts its arrival after its keys are in, and the one
// that arrives last finds every key there).
template <int U>
__global__ __launch_bounds__(kThreads) void k_minmax(lpq_tensor one, int kind, float c, uint32_t* state,
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
        atomicMin(state + 4, l);
        atomicMax(state + 5, h);
        __threadfence();   // this workgroup's keys before its arrival
        if (atomicAdd(state + 6, 1u) == gridDim.x - 1) {
            __threadfence();   // every other workgroup's keys before the rule reads them
            observer_apply(kind, c, state, amax);
            state[6] = 0u;     // re-armed for the next call
        }
    }
}

// fl(A / 2688) per entry: the multiplier form of a global scale.
__global__ __launch_bounds__(kThreads) void k_global_scale(const float* amax, int32_t n, float* out) {
    const int32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) out[i] = amax[i] / 2688.0f;   // correctly rounded division
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
    if (W.unit == 0 && tid == 0) group_g[gi] = G.g;   // same value from every member
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

// ---------------------------------------------------------------------------
// Block-wise FP8, one 128 x 128 tile per workgroup
// ---------------------------------------------------------------------------

// Lane layout inside a tile: lane t covers columns 8*(t%16) .. +8 of rows
// R*pass + t/16, R = TT/16 rows per pass for TT threads.
template <int TT>
struct TileShape {
    static constexpr int rows_per_pass = TT / 16;
    static constexpr int passes = kTile / rows_per_pass;
    static constexpr int waves = TT / 64;
};

struct TileGeom {
    int64_t r0, c0, rows, cols;   // tile origin and clipped extent
    int64_t index;                // position in the [ceil(M/128), ceil(N/128)] scale grid
    bool fast;                    // full tile and 16-byte aligned rows
};

__device__ __forceinline__ TileGeom tile_geom(const lpq_tensor& d, int64_t tile) {
    const int64_t tn = (d.cols + kTile - 1) / kTile;
    TileGeom T;
    T.index = tile;
    T.r0 = (tile / tn) * kTile;
    T.c0 = (tile % tn) * kTile;
    T.rows = d.rows - T.r0 < kTile ? d.rows - T.r0 : kTile;
    T.cols = d.cols - T.c0 < kTile ? d.cols - T.c0 : kTile;
    T.fast = T.rows == kTile && T.cols == kTile && (d.cols & 7) == 0 &&
             ((reinterpret_cast<uintptr_t>(d.src) | reinterpret_cast<uintptr_t>(d.dst)) & 15) == 0;
    return T;
}

// The quantizer's workgroup covers TW adjacent tiles of one tile row (128
// rows x 128*TW columns, 256*TW threads): each pass reads one 256*TW-byte run
// per row instead of 256 bytes, which the memory system serves better (an
// access-pattern probe with no arithmetic: 70-72% of HBM peak for one tile,
// 75-79% for two).  TW is 2, or 4 for calls with many strips (the host's
// choice, fp8blk_quant_kind).  Lane t covers columns 8*(t % (16 TW)) .. +8 of
// rows 16*pass + t / (16 TW); its tile within the strip is (t % (16 TW)) / 16.
template <int TW>
struct WideShape {
    static constexpr int threads = 256 * TW;
    static constexpr int lanes_per_row = 16 * TW;
    static constexpr int rows_per_pass = threads / lanes_per_row;   // 16
    static constexpr int passes = kTile / rows_per_pass;             // 8
    static constexpr int waves = threads / 64;
    static constexpr int rows_per_wave = 64 / lanes_per_row;         // 4 / TW
};

// Maximum of m over the lanes of each tile of a strip of TW tiles, for a
// workgroup of THREADS lanes with LPT lanes per tile row (a row of the strip
// is LPT * TW lanes); every lane gets its own tile's value.
template <int LPT, int TW, int THREADS>
__device__ __forceinline__ uint32_t strip_reduce_max(uint32_t m, int sub) {
    constexpr int waves = THREADS / 64;
    m = quad_max(m);
#pragma unroll
    for (int k = 4; k < LPT; k <<= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, k));   // one row segment
#pragma unroll
    for (int k = LPT * TW; k < 64; k <<= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, k));   // rows of the wave
    __shared__ uint32_t part[waves][TW];
    const int lane = threadIdx.x & 63;
    if (lane < LPT * TW && lane % LPT == 0) part[threadIdx.x >> 6][lane / LPT] = m;
    __syncthreads();
    uint32_t r = part[0][sub];
#pragma unroll
    for (int k = 1; k < waves; k++) r = umax(r, part[k][sub]);
    return r;
}

// A raw buffer resource over the `bytes` bytes from p (at most 2^32 - 1; the
// resource's third word is the gfx9 default).  Loads through it take a
// 32-bit per-lane offset plus a uniform one in a scalar register, so the
// addresses of a tile's row passes cost one vector register in all.
// Stores do not go through buffers: a buffer store of more than 8 bytes with
// a scalar-register offset gets no wait state before a following VALU write
// of its data registers, and such a store was seen to write a stale first
// dword.  Stores use global_store with a uniform 64-bit base and the 32-bit
// lane offset (store_at), which costs no more vector registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* p, int64_t bytes) {
    const int32_t n = bytes >= 0xffffffffLL ? -1 : (int32_t)(uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
constexpr int kBufNT = 2;   // cache-policy bits of a non-temporal buffer access
__device__ __forceinline__ v4u buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, kNTL ? kBufNT : 0);
}
// Stores x at byte offset lane_off from the uniform address base.
template <typename T>
__device__ __forceinline__ void store_at(uint8_t* base, uint32_t lane_off, T x) {
    store<kNTS>(reinterpret_cast<T*>(base + lane_off), x);
}

template <int TW, bool GROUPED>
__global__ __launch_bounds__(256 * TW, LPQ_TILEQ_WAVES_PER_SIMD) void k_fp8blk_quant(const lpq_tensor* table,
                                                                                      lpq_tensor one, ChunkMap map) {
    using S = WideShape<TW>;
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const int64_t M = d.rows, N = d.cols;
    const int64_t tn = (N + kTile - 1) / kTile, tnw = (tn + TW - 1) / TW;
    const int64_t tr = W.unit / tnw, tcw = W.unit % tnw;
    const int64_t r0 = tr * kTile, c0 = tcw * kTile * TW;
    const int64_t rows = M - r0 < kTile ? M - r0 : kTile;
    const int64_t cols = N - c0 < kTile * TW ? N - c0 : kTile * TW;   // columns of the strip inside the tensor
    const uint16_t* w = reinterpret_cast<const uint16_t*>(d.src);
    uint8_t* q = reinterpret_cast<uint8_t*>(d.dst);
    const int tid = threadIdx.x;
    const int lr = tid / S::lanes_per_row;          // row inside a pass
    const int lc = (tid % S::lanes_per_row) * 8;    // first column of the lane's segment in the strip
    const int sub = lc / kTile;                     // the lane's tile within the strip
    const int64_t origin = r0 * N + c0;             // element offset of the strip in the tensor

    // FAST: 16-byte aligned rows (N % 8 == 0, so a lane's 8 columns are all inside
    // the tensor or all outside) whose buffer offsets (< 2 * 128 * N bytes) fit 32
    // bits; edge strips included, lanes outside the tensor taking zeros and storing
    // nothing.  It keeps the strip in registers between the amax and the encode.  The
    // general body (any other tensor) reads the strip twice, the second time from
    // cache, one pass at a time, so that its registers stay below the fast body's.
    auto body = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
        const uint32_t lane_off = (uint32_t)lr * (uint32_t)N + (uint32_t)lc;   // elements, < 2^29 when FAST
        const __amdgpu_buffer_rsrc_t rw = buffer_of(w + origin, (M * N - origin) * 2);
        const bool in_c = lc < cols;   // the lane's columns are inside the tensor
        auto in_r = [&](int p) { return S::rows_per_pass * p + lr < rows; };
        auto gather = [&](int p) {   // general body: pass p of the lane, zero outside the tensor
            const int64_t r = S::rows_per_pass * p + lr;
            uint32_t h[8];
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const bool in = r < rows && lc + k < cols;
                h[k] = in ? w[(r0 + r) * N + c0 + lc + k] : 0u;
            }
            return v4u{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        };
        v4u v[FAST ? S::passes : 1];
        uint32_t m = 0;
        if constexpr (FAST) {
            // lanes outside the columns read the strip's first element of their row
            // (rows past the end of the tensor read as 0: buffer range check), then zero
            const uint32_t ld_off = in_c ? lane_off * 2 : 0u;
#pragma unroll
            for (int p = 0; p < S::passes; p++)
                v[p] = buffer_load16(rw, ld_off, (uint32_t)(S::rows_per_pass * p * N * 2));
#pragma unroll
            for (int p = 0; p < S::passes; p++) {
                if (!(in_c && in_r(p))) v[p] = v4u{0u, 0u, 0u, 0u};
                m = umax(m, absmax8_bits(v[p]));
            }
        } else {
#pragma unroll 1
            for (int p = 0; p < S::passes; p++) m = umax(m, absmax8_bits(gather(p)));
        }
        const float amax = __uint_as_float(strip_reduce_max<16, TW, S::threads>(m, sub));
        const float s = amax / kE4M3Max;   // correctly rounded division
        if (lr == 0 && (lc & (kTile - 1)) == 0 && sub * kTile < cols)
            reinterpret_cast<float*>(d.scale)[tr * tn + tcw * TW + sub] = s;
        const bool tiny = s > 0.0f && s < kTinyScale;
        const float sd = tiny ? s * kPreScale : s;
        const float r = s > 0.0f ? rcp_rn(sd) : 0.0f;
        const bool any_tiny = any_lane(tiny);

        auto encode = [&](int p, const v4u& x8) {
            float x[8] = {bf16_lo(x8.x), bf16_hi(x8.x), bf16_lo(x8.y), bf16_hi(x8.y),
                          bf16_lo(x8.z), bf16_hi(x8.z), bf16_lo(x8.w), bf16_hi(x8.w)};
            if (any_tiny) {
#pragma unroll
                for (int k = 0; k < 8; k++) x[k] *= tiny ? kPreScale : 1.0f;
            }
            float qq[8];
#pragma unroll
            for (int k = 0; k < 8; k++) qq[k] = quot_rn(x[k], sd, r);
            uint32_t lo = e4m3x2<false>(qq[0], qq[1], 0u);
            lo = e4m3x2<true>(qq[2], qq[3], lo);
            uint32_t hi = e4m3x2<false>(qq[4], qq[5], 0u);
            hi = e4m3x2<true>(qq[6], qq[7], hi);
            const int64_t row = S::rows_per_pass * p + lr;
            if constexpr (FAST) {
                if (in_c && row < rows) store_at(q + origin + (int64_t)S::rows_per_pass * p * N, lane_off, v2u{lo, hi});
            } else if (row < rows) {
                const uint32_t c8[2] = {lo, hi};
                for (int k = 0; k < 8; k++)
                    if (lc + k < cols) q[(r0 + row) * N + c0 + lc + k] = (uint8_t)(c8[k >> 2] >> (8 * (k & 3)));
            }
        };
        if constexpr (FAST) {
#pragma unroll
            for (int p = 0; p < S::passes; p++) encode(p, v[p]);
        } else {
#pragma unroll 1
            for (int p = 0; p < S::passes; p++) encode(p, gather(p));
        }
    };
    if ((N & 7) == 0 && N <= (1 << 22) &&
        ((reinterpret_cast<uintptr_t>(d.src) | reinterpret_cast<uintptr_t>(d.dst)) & 15) == 0)
        body(Full<true>{});
    else
        body(Full<false>{});
}

template <int TT, bool GROUPED>
__global__ __launch_bounds__(TT) void k_fp8blk_dequant(const lpq_tensor* table, lpq_tensor one, ChunkMap map) {
    const Work W = locate<GROUPED>(table, one, map);
    const lpq_tensor& d = W.d;
    const TileGeom T = tile_geom(d, W.unit);
    const uint8_t* q = reinterpret_cast<const uint8_t*>(d.src);
    uint16_t* y = reinterpret_cast<uint16_t*>(d.dst);
    const float s = reinterpret_cast<const float*>(d.scale)[T.index];
    const int tid = threadIdx.x;
    const int lr = tid >> 4;
    const int lc = (tid & 15) * 8;

    v2u c[TileShape<TT>::passes];
    if (T.fast) {
#pragma unroll
        for (int p = 0; p < TileShape<TT>::passes; p++)
            c[p] = load<kNTL>(reinterpret_cast<const v2u*>(q + (T.r0 + TileShape<TT>::rows_per_pass * p + lr) * d.cols + T.c0 + lc));
    } else {
        for (int p = 0; p < TileShape<TT>::passes; p++) {
            const int64_t r = TileShape<TT>::rows_per_pass * p + lr;
            uint32_t b[8];
            for (int k = 0; k < 8; k++) {
                const bool in = r < T.rows && lc + k < T.cols;
                b[k] = in ? q[(T.r0 + r) * d.cols + T.c0 + lc + k] : 0u;
            }
            c[p] = v2u{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
        }
    }
#pragma unroll
    for (int p = 0; p < TileShape<TT>::passes; p++) {
        const float2_t f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[p].x, false);
        const float2_t f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[p].x, true);
        const float2_t f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[p].y, false);
        const float2_t f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[p].y, true);
        v4u o;
        o.x = bf16x2(f0[0] * s, f0[1] * s);
        o.y = bf16x2(f1[0] * s, f1[1] * s);
        o.z = bf16x2(f2[0] * s, f2[1] * s);
        o.w = bf16x2(f3[0] * s, f3[1] * s);
        const int64_t r = TileShape<TT>::rows_per_pass * p + lr;
        if (T.fast) {
            store<kNTS>(reinterpret_cast<v4u*>(y + (T.r0 + r) * d.cols + T.c0 + lc), o);
        } else if (r < T.rows) {
            const uint32_t h[4] = {o.x, o.y, o.z, o.w};
            for (int k = 0; k < 8; k++)
                if (lc + k < T.cols) y[(T.r0 + r) * d.cols + T.c0 + lc + k] = (uint16_t)(h[k >> 1] >> (16 * (k & 1)));
        }
    }
}

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

__device__ __forceinline__ Y16 fp8blk_values16(const v4u& c, float s) {
    float p[16];
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const float2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
        const float2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
        p[4 * k + 0] = a[0] * s;
        p[4 * k + 1] = a[1] * s;
        p[4 * k + 2] = b[0] * s;
        p[4 * k + 3] = b[1] * s;
    }
    float m = fmaxf(fmaxf(fabsf(p[0]), fabsf(p[1])), fabsf(p[2]));
#pragma unroll
    for (int k = 3; k < 15; k += 2) m = fmaxf(fmaxf(m, fabsf(p[k])), fabsf(p[k + 1]));
    m = fmaxf(m, fabsf(p[15]));
    Y16 y;
    y.amax = bf16_in_f32(m);
#pragma unroll
    for (int k = 0; k < 8; k++) {
        y.lo.x[k] = __uint_as_float(bf16_in_f32(p[k]));
        y.hi.x[k] = __uint_as_float(bf16_in_f32(p[8 + k]));
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

template <int U, bool FULL, bool LARGE, int TH>
__device__ __forceinline__ void rq_nvfp4_body(const lpq_requant_tensor& d, int64_t base, int64_t total,
                                              const GlobalScale& G) {
    // the chunk's origins (uniform): one 8-byte code word and one scale byte per lane and step
    v2u* dst = reinterpret_cast<v2u*>(d.dst) + base / 16;
    uint8_t* ssc = reinterpret_cast<uint8_t*>(d.dst_scale) + base / 16;
    rq_stream<U, FULL, LPQ_RQN_AHEAD != 0, TH>(d, base, total, [&](int u, const v4u& c, float s) {
        const int i = u * TH + threadIdx.x;
        const Y16 y = fp8blk_values16(c, s);
        // one lane is one 16-element block
        const BlockScale B = block_scale<LARGE>(y.amax, G);
        const v2u p = v2u{e2m1x8(y.lo, B), e2m1x8(y.hi, B)};
        if (FULL || base + (int64_t)i * 16 < total) {
            store<kNTS>(dst + i, p);
            store_u8(ssc + i, B.code);
        }
    });
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
// each tile's dequantized values y = BF16(fl(code * s)) stay in registers (16
// codes per lane per pass), their amax gives the new scale s' = fl(amax/448),
// and each y is encoded as E4M3(fl(y / s')).  Lane t covers codes
// 16*(t % (8 TW)) .. +16 of rows (TW*256/(8 TW))*pass + t / (8 TW).
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
        const bool any_tiny = any_lane(tiny);

        auto encode = [&](int p, const v4u& cp) {
            const Y16 y = fp8blk_values16(cp, s);
            float x[16];
#pragma unroll
            for (int k = 0; k < 8; k++) {
                x[k] = y.lo.x[k];
                x[8 + k] = y.hi.x[k];
            }
            if (any_tiny) {
#pragma unroll
                for (int k = 0; k < 16; k++) x[k] *= tiny ? kPreScale : 1.0f;
            }
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const float q0 = quot_rn(x[4 * k + 0], sd, r), q1 = quot_rn(x[4 * k + 1], sd, r);
                const float q2 = quot_rn(x[4 * k + 2], sd, r), q3 = quot_rn(x[4 * k + 3], sd, r);
                o[k] = e4m3x2<true>(q2, q3, e4m3x2<false>(q0, q1, 0u));
            }
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

// ===========================================================================
// Host side: argument checks and launches
// ===========================================================================

namespace {

thread_local int g_last_hip_error = 0;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline lpq_status launched() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return LPQ_ERR_HIP;
    }
    return LPQ_OK;
}

enum Kind {
    FP8BLK_Q, FP8BLK_QW, FP8BLK_DQ, FP8BLK_DQF, MXFP8_Q, MXFP8_QF, MXFP8_DQ, NV_AMAX, NV_Q, NV_DQ, NV_QDQ,
    I4_Q32, I4_Q128, I4_DQ32, I4_DQ128, I4_QDQ32, I4_QDQ128,
    RQ_FP8, RQ_MX, RQ_AMAX, RQ_NV
};

// The INT4 group size of an INT4 kind (0 for other kinds).
constexpr int int4_group(Kind k) {
    return (k == I4_Q32 || k == I4_DQ32 || k == I4_QDQ32) ? 32 : (k == I4_Q128 || k == I4_DQ128 || k == I4_QDQ128) ? 128 : 0;
}

// Shape and pointer checks of one tensor for one kind of call.
lpq_status check_tensor(Kind k, const lpq_tensor& t, int32_t n_groups) {
    if (t.rows <= 0 || t.cols <= 0) return LPQ_ERR_SHAPE;
    if (t.rows > (int64_t(1) << 40) / t.cols) return LPQ_ERR_SHAPE;   // element count overflow guard
    if (!t.src) return LPQ_ERR_NULL;
    if (k != NV_AMAX && !t.dst) return LPQ_ERR_NULL;
    if (k != NV_AMAX && k != NV_QDQ && k != I4_QDQ32 && k != I4_QDQ128 && !t.scale) return LPQ_ERR_NULL;
    if (t.reserved != 0) return LPQ_ERR_ARG;
    switch (k) {
    case FP8BLK_Q:
    case FP8BLK_QW:   // not a caller-visible kind: the wide-strip quantizer
    case FP8BLK_DQ:
        if (!aligned(k == FP8BLK_DQ ? t.dst : t.src, 2) || !aligned(t.scale, 4)) return LPQ_ERR_ALIGN;
        break;
    case FP8BLK_DQF:   // not a caller-visible kind: the flat layout's extra conditions
        if (t.cols % 8 || t.rows >= (int64_t(1) << 31) || t.cols >= (int64_t(1) << 31) - kRqStepMax) return LPQ_ERR_SHAPE;
        if (!aligned(t.src, 8) || !aligned(t.dst, 16) || !aligned(t.scale, 4)) return LPQ_ERR_ALIGN;
        break;
    case MXFP8_Q:
    case MXFP8_QF:
        if (t.cols % 32) return LPQ_ERR_SHAPE;
        if (!aligned(t.src, 16) || !aligned(t.dst, 8)) return LPQ_ERR_ALIGN;
        break;
    case MXFP8_DQ:
        if (t.cols % 32) return LPQ_ERR_SHAPE;
        if (!aligned(t.src, 8) || !aligned(t.dst, 16)) return LPQ_ERR_ALIGN;
        break;
    case NV_AMAX:
    case NV_Q:
    case NV_DQ:
    case NV_QDQ:
        if (t.cols % 16) return LPQ_ERR_SHAPE;
        if (k == NV_DQ ? !aligned(t.src, 4) : !aligned(t.src, 16)) return LPQ_ERR_ALIGN;
        if (k == NV_Q && !aligned(t.dst, 4)) return LPQ_ERR_ALIGN;
        if ((k == NV_DQ || k == NV_QDQ) && !aligned(t.dst, 16)) return LPQ_ERR_ALIGN;
        if (n_groups > 0 && (t.group < 0 || t.group >= n_groups)) return LPQ_ERR_GROUP;
        break;
    case I4_Q32:
    case I4_Q128:
        if (t.cols % int4_group(k)) return LPQ_ERR_SHAPE;
        if (!aligned(t.src, 16) || !aligned(t.dst, 4) || !aligned(t.scale, 4)) return LPQ_ERR_ALIGN;
        break;
    case I4_DQ32:
    case I4_DQ128:
        if (t.cols % int4_group(k)) return LPQ_ERR_SHAPE;
        if (!aligned(t.src, 4) || !aligned(t.dst, 16) || !aligned(t.scale, 4)) return LPQ_ERR_ALIGN;
        break;
    case I4_QDQ32:
    case I4_QDQ128:
        if (t.cols % int4_group(k)) return LPQ_ERR_SHAPE;
        if (!aligned(t.src, 16) || !aligned(t.dst, 16)) return LPQ_ERR_ALIGN;
        break;
    default: return LPQ_ERR_ARG;
    }
    return LPQ_OK;
}

lpq_status check_tensor(Kind k, const lpq_requant_tensor& t, int32_t n_groups) {
    if (t.rows <= 0 || t.cols <= 0) return LPQ_ERR_SHAPE;
    if (t.rows > (int64_t(1) << 40) / t.cols) return LPQ_ERR_SHAPE;
    if (!t.src || !t.src_scale) return LPQ_ERR_NULL;
    if (k != RQ_AMAX && (!t.dst || !t.dst_scale)) return LPQ_ERR_NULL;
    if (t.reserved != 0) return LPQ_ERR_ARG;
    if (k == RQ_FP8) return aligned(t.src_scale, 4) && aligned(t.dst_scale, 4) ? LPQ_OK : LPQ_ERR_ALIGN;
    if (t.cols % (k == RQ_MX ? 32 : 16)) return LPQ_ERR_SHAPE;
    if (t.rows >= (int64_t(1) << 31) || t.cols >= (int64_t(1) << 31) - kRqStepMax) return LPQ_ERR_SHAPE;
    if (!aligned(t.src, 16) || !aligned(t.src_scale, 4)) return LPQ_ERR_ALIGN;
    if (k == RQ_MX && !aligned(t.dst, 16)) return LPQ_ERR_ALIGN;
    if (k == RQ_NV && !aligned(t.dst, 8)) return LPQ_ERR_ALIGN;
    if (k != RQ_MX && n_groups > 0 && (t.group < 0 || t.group >= n_groups)) return LPQ_ERR_GROUP;
    return LPQ_OK;
}

// Work units (workgroups) of one tensor.
int64_t units(Kind k, const lpq_tensor& t) {
    const int64_t n = t.rows * t.cols;
    switch (k) {
    case FP8BLK_Q: return ((t.rows + kTile - 1) / kTile) * ((t.cols + kTile * LPQ_TILEQ_TW - 1) / (kTile * LPQ_TILEQ_TW));
    case FP8BLK_QW:
        return ((t.rows + kTile - 1) / kTile) * ((t.cols + kTile * LPQ_TILEQ_WIDE_TW - 1) / (kTile * LPQ_TILEQ_WIDE_TW));
    case FP8BLK_DQ: return ((t.rows + kTile - 1) / kTile) * ((t.cols + kTile - 1) / kTile);
    case FP8BLK_DQF: return (n + dqf_chunk_elems<LPQ_DQF_U, LPQ_DQF_T>() - 1) / dqf_chunk_elems<LPQ_DQF_U, LPQ_DQF_T>();
    case MXFP8_Q:
    case MXFP8_QF: return (n + chunk_elems<LPQ_MXQ_U, LPQ_MXQ_T>() - 1) / chunk_elems<LPQ_MXQ_U, LPQ_MXQ_T>();
    case MXFP8_DQ: return (n + chunk_elems<LPQ_MXD_U, LPQ_MXD_T>() - 1) / chunk_elems<LPQ_MXD_U, LPQ_MXD_T>();
    case NV_AMAX: return (n + chunk_elems<LPQ_AMAX_U, LPQ_AMAX_T>() - 1) / chunk_elems<LPQ_AMAX_U, LPQ_AMAX_T>();
    case NV_Q: return (n + chunk_elems<LPQ_NVQ_U, LPQ_NVQ_T>() - 1) / chunk_elems<LPQ_NVQ_U, LPQ_NVQ_T>();
    case NV_DQ: return (n + chunk_elems<LPQ_NVD_U, LPQ_NVD_T>() - 1) / chunk_elems<LPQ_NVD_U, LPQ_NVD_T>();
    case NV_QDQ: return (n + chunk_elems<LPQ_QDQ_U, LPQ_QDQ_T>() - 1) / chunk_elems<LPQ_QDQ_U, LPQ_QDQ_T>();
    case I4_Q32:
    case I4_Q128: return (n + chunk_elems<LPQ_I4Q_U, LPQ_I4Q_T>() - 1) / chunk_elems<LPQ_I4Q_U, LPQ_I4Q_T>();
    case I4_DQ32:
    case I4_DQ128: return (n + chunk_elems<LPQ_I4D_U, LPQ_I4D_T>() - 1) / chunk_elems<LPQ_I4D_U, LPQ_I4D_T>();
    case I4_QDQ32:
    case I4_QDQ128: return (n + chunk_elems<LPQ_I4QDQ_U, LPQ_I4QDQ_T>() - 1) / chunk_elems<LPQ_I4QDQ_U, LPQ_I4QDQ_T>();
    default: return 0;
    }
}

int64_t units(Kind k, const lpq_requant_tensor& t) {
    const int64_t n = t.rows * t.cols;
    switch (k) {
    case RQ_FP8: return ((t.rows + kTile - 1) / kTile) * ((t.cols + kTile * LPQ_RQT_TW - 1) / (kTile * LPQ_RQT_TW));
    case RQ_MX: return (n + rq_chunk_elems<LPQ_RQM_U, LPQ_RQM_T>() - 1) / rq_chunk_elems<LPQ_RQM_U, LPQ_RQM_T>();
    case RQ_AMAX: return (n + rq_chunk_elems<LPQ_RQA_U, LPQ_RQA_T>() - 1) / rq_chunk_elems<LPQ_RQA_U, LPQ_RQA_T>();
    case RQ_NV: return (n + rq_chunk_elems<LPQ_RQN_U, LPQ_RQN_T>() - 1) / rq_chunk_elems<LPQ_RQN_U, LPQ_RQN_T>();
    default: return 0;
    }
}

constexpr int64_t kMaxGridX = 0x7fffffffLL;

void dispatch(Kind k, dim3 grid, hipStream_t stream, const lpq_tensor* tab, const lpq_tensor& one, const ChunkMap& map,
              const float* fa, float* fb) {
    const dim3 tileq(256 * LPQ_TILEQ_TW), tileqw(256 * LPQ_TILEQ_WIDE_TW), tiled(LPQ_TILED_THREADS);
    if (tab) {
        switch (k) {
        case FP8BLK_Q: hipLaunchKernelGGL((k_fp8blk_quant<LPQ_TILEQ_TW, true>), grid, tileq, 0, stream, tab, one, map); break;
        case FP8BLK_QW:
            hipLaunchKernelGGL((k_fp8blk_quant<LPQ_TILEQ_WIDE_TW, true>), grid, tileqw, 0, stream, tab, one, map);
            break;
        case FP8BLK_DQ: hipLaunchKernelGGL((k_fp8blk_dequant<LPQ_TILED_THREADS, true>), grid, tiled, 0, stream, tab, one, map); break;
        case FP8BLK_DQF: hipLaunchKernelGGL((k_fp8blk_dequant_flat<LPQ_DQF_U, LPQ_DQF_T, true>), grid, dim3(LPQ_DQF_T), 0, stream, tab, one, map); break;
        case MXFP8_Q: hipLaunchKernelGGL((k_mxfp8_quant<LPQ_MXQ_U, LPQ_MXQ_T, true>), grid, dim3(LPQ_MXQ_T), 0, stream, tab, one, map); break;
        case MXFP8_QF: hipLaunchKernelGGL((k_mxfp8_quant<LPQ_MXQ_U, LPQ_MXQ_T, true, true>), grid, dim3(LPQ_MXQ_T), 0, stream, tab, one, map); break;
        case MXFP8_DQ: hipLaunchKernelGGL((k_mxfp8_dequant<LPQ_MXD_U, LPQ_MXD_T, true>), grid, dim3(LPQ_MXD_T), 0, stream, tab, one, map); break;
        case NV_AMAX: hipLaunchKernelGGL((k_amax<LPQ_AMAX_U, LPQ_AMAX_T, true>), grid, dim3(LPQ_AMAX_T), 0, stream, tab, one, map, fb); break;
        case NV_Q: hipLaunchKernelGGL((k_nvfp4_quant<LPQ_NVQ_U, LPQ_NVQ_T, true>), grid, dim3(LPQ_NVQ_T), 0, stream, tab, one, map, fa, fb); break;
        case NV_DQ: hipLaunchKernelGGL((k_nvfp4_dequant<LPQ_NVD_U, LPQ_NVD_T, true>), grid, dim3(LPQ_NVD_T), 0, stream, tab, one, map, fa); break;
        case NV_QDQ: hipLaunchKernelGGL((k_nvfp4_qdq<LPQ_QDQ_U, LPQ_QDQ_T, true>), grid, dim3(LPQ_QDQ_T), 0, stream, tab, one, map, fa); break;
        case I4_Q32: hipLaunchKernelGGL((k_int4_quant<LPQ_I4Q_U, LPQ_I4Q_T, true, 32>), grid, dim3(LPQ_I4Q_T), 0, stream, tab, one, map); break;
        case I4_Q128: hipLaunchKernelGGL((k_int4_quant<LPQ_I4Q_U, LPQ_I4Q_T, true, 128>), grid, dim3(LPQ_I4Q_T), 0, stream, tab, one, map); break;
        case I4_DQ32: hipLaunchKernelGGL((k_int4_dequant<LPQ_I4D_U, LPQ_I4D_T, true, 32>), grid, dim3(LPQ_I4D_T), 0, stream, tab, one, map); break;
        case I4_DQ128: hipLaunchKernelGGL((k_int4_dequant<LPQ_I4D_U, LPQ_I4D_T, true, 128>), grid, dim3(LPQ_I4D_T), 0, stream, tab, one, map); break;
        case I4_QDQ32: hipLaunchKernelGGL((k_int4_qdq<LPQ_I4QDQ_U, LPQ_I4QDQ_T, true, 32>), grid, dim3(LPQ_I4QDQ_T), 0, stream, tab, one, map); break;
        case I4_QDQ128: hipLaunchKernelGGL((k_int4_qdq<LPQ_I4QDQ_U, LPQ_I4QDQ_T, true, 128>), grid, dim3(LPQ_I4QDQ_T), 0, stream, tab, one, map); break;
        default: break;
        }
    } else {
        switch (k) {
        case FP8BLK_Q: hipLaunchKernelGGL((k_fp8blk_quant<LPQ_TILEQ_TW, false>), grid, tileq, 0, stream, tab, one, map); break;
        case FP8BLK_QW:
            hipLaunchKernelGGL((k_fp8blk_quant<LPQ_TILEQ_WIDE_TW, false>), grid, tileqw, 0, stream, tab, one, map);
            break;
        case FP8BLK_DQ: hipLaunchKernelGGL((k_fp8blk_dequant<LPQ_TILED_THREADS, false>), grid, tiled, 0, stream, tab, one, map); break;
        case FP8BLK_DQF: hipLaunchKernelGGL((k_fp8blk_dequant_flat<LPQ_DQF_U, LPQ_DQF_T, false>), grid, dim3(LPQ_DQF_T), 0, stream, tab, one, map); break;
        case MXFP8_Q: hipLaunchKernelGGL((k_mxfp8_quant<LPQ_MXQ_U, LPQ_MXQ_T, false>), grid, dim3(LPQ_MXQ_T), 0, stream, tab, one, map); break;
        case MXFP8_QF: hipLaunchKernelGGL((k_mxfp8_quant<LPQ_MXQ_U, LPQ_MXQ_T, false, true>), grid, dim3(LPQ_MXQ_T), 0, stream, tab, one, map); break;
        case MXFP8_DQ: hipLaunchKernelGGL((k_mxfp8_dequant<LPQ_MXD_U, LPQ_MXD_T, false>), grid, dim3(LPQ_MXD_T), 0, stream, tab, one, map); break;
        case NV_AMAX: hipLaunchKernelGGL((k_amax<LPQ_AMAX_U, LPQ_AMAX_T, false>), grid, dim3(LPQ_AMAX_T), 0, stream, tab, one, map, fb); break;
        case NV_Q: hipLaunchKernelGGL((k_nvfp4_quant<LPQ_NVQ_U, LPQ_NVQ_T, false>), grid, dim3(LPQ_NVQ_T), 0, stream, tab, one, map, fa, fb); break;
        case NV_DQ: hipLaunchKernelGGL((k_nvfp4_dequant<LPQ_NVD_U, LPQ_NVD_T, false>), grid, dim3(LPQ_NVD_T), 0, stream, tab, one, map, fa); break;
        case NV_QDQ: hipLaunchKernelGGL((k_nvfp4_qdq<LPQ_QDQ_U, LPQ_QDQ_T, false>), grid, dim3(LPQ_QDQ_T), 0, stream, tab, one, map, fa); break;
        case I4_Q32: hipLaunchKernelGGL((k_int4_quant<LPQ_I4Q_U, LPQ_I4Q_T, false, 32>), grid, dim3(LPQ_I4Q_T), 0, stream, tab, one, map); break;
        case I4_Q128: hipLaunchKernelGGL((k_int4_quant<LPQ_I4Q_U, LPQ_I4Q_T, false, 128>), grid, dim3(LPQ_I4Q_T), 0, stream, tab, one, map); break;
        case I4_DQ32: hipLaunchKernelGGL((k_int4_dequant<LPQ_I4D_U, LPQ_I4D_T, false, 32>), grid, dim3(LPQ_I4D_T), 0, stream, tab, one, map); break;
        case I4_DQ128: hipLaunchKernelGGL((k_int4_dequant<LPQ_I4D_U, LPQ_I4D_T, false, 128>), grid, dim3(LPQ_I4D_T), 0, stream, tab, one, map); break;
        case I4_QDQ32: hipLaunchKernelGGL((k_int4_qdq<LPQ_I4QDQ_U, LPQ_I4QDQ_T, false, 32>), grid, dim3(LPQ_I4QDQ_T), 0, stream, tab, one, map); break;
        case I4_QDQ128: hipLaunchKernelGGL((k_int4_qdq<LPQ_I4QDQ_U, LPQ_I4QDQ_T, false, 128>), grid, dim3(LPQ_I4QDQ_T), 0, stream, tab, one, map); break;
        default: break;
        }
    }
}

void dispatch(Kind k, dim3 grid, hipStream_t stream, const lpq_requant_tensor* tab, const lpq_requant_tensor& one,
              const ChunkMap& map, const float* fa, float* fb) {
    const dim3 tile(256 * LPQ_RQT_TW);
    if (tab) {
        switch (k) {
        case RQ_FP8: hipLaunchKernelGGL((k_requant_fp8blk<LPQ_RQT_TW, true>), grid, tile, 0, stream, tab, one, map); break;
        case RQ_MX: hipLaunchKernelGGL((k_requant_mxfp8<LPQ_RQM_U, LPQ_RQM_T, true>), grid, dim3(LPQ_RQM_T), 0, stream, tab, one, map); break;
        case RQ_AMAX: hipLaunchKernelGGL((k_requant_amax<LPQ_RQA_U, LPQ_RQA_T, true>), grid, dim3(LPQ_RQA_T), 0, stream, tab, one, map, fb); break;
        case RQ_NV: hipLaunchKernelGGL((k_requant_nvfp4<LPQ_RQN_U, LPQ_RQN_T, true>), grid, dim3(LPQ_RQN_T), 0, stream, tab, one, map, fa, fb); break;
        default: break;
        }
    } else {
        switch (k) {
        case RQ_FP8: hipLaunchKernelGGL((k_requant_fp8blk<LPQ_RQT_TW, false>), grid, tile, 0, stream, tab, one, map); break;
        case RQ_MX: hipLaunchKernelGGL((k_requant_mxfp8<LPQ_RQM_U, LPQ_RQM_T, false>), grid, dim3(LPQ_RQM_T), 0, stream, tab, one, map); break;
        case RQ_AMAX: hipLaunchKernelGGL((k_requant_amax<LPQ_RQA_U, LPQ_RQA_T, false>), grid, dim3(LPQ_RQA_T), 0, stream, tab, one, map, fb); break;
        case RQ_NV: hipLaunchKernelGGL((k_requant_nvfp4<LPQ_RQN_U, LPQ_RQN_T, false>), grid, dim3(LPQ_RQN_T), 0, stream, tab, one, map, fa, fb); break;
        default: break;
        }
    }
}

// Where the launch over tensors [i0, count) stops: the first tensor that would
// exceed kMaxSeg segments (runs of equal work-unit counts) or 2^31-1 work units.
// Fills map and total; returns -1 when one tensor alone is too large.
template <typename D>
int32_t slice_end(Kind k, const D* host, int32_t count, int32_t i0, const D& one, ChunkMap& map, int64_t& total) {
    map = ChunkMap{};
    total = 0;
    int32_t nseg = 0, i = i0;
    while (i < count) {
        const int64_t u = units(k, host ? host[i] : one);
        if (u > kMaxGridX) return -1;
        if (total + u > kMaxGridX) break;
        if (nseg == 0 || (int64_t)map.units[nseg - 1] != u) {
            if (nseg == kMaxSeg) break;
            map.first[nseg] = (uint32_t)total;
            map.tensor0[nseg] = (uint32_t)(i - i0);
            map.units[nseg] = (uint32_t)u;
            map.inv_units[nseg] = 1.0 / (double)u;
            nseg++;
        }
        total += u;
        i++;
    }
    map.nseg = nseg;
    return i;
}

// Number of launches a call of kind k over host[0, n) takes (-1: a tensor is too large).
template <typename D>
int64_t launch_count(Kind k, const D* host, int32_t n) {
    int64_t launches = 0;
    ChunkMap map;
    int64_t total;
    for (int32_t i0 = 0; i0 < n; launches++) {
        const int32_t i = slice_end(k, host, n, i0, D{}, map, total);
        if (i < 0) return -1;
        i0 = i;
    }
    return launches;
}

// Launch kernel `k` over tensors [0, n) of `host`/`dev` (single tensor: dev ==
// nullptr, `one` used), in slices of at most kMaxSeg segments and 2^31-1 work
// units.
template <typename D>
lpq_status launch(Kind k, const D* host, const D* dev, int32_t n, const D& one, const float* fa, float* fb,
                  hipStream_t stream, float gdiv = 2688.0f) {
    const int32_t count = dev ? n : 1;
    int32_t i0 = 0;
    while (i0 < count) {
        ChunkMap map;
        int64_t total;
        const int32_t i = slice_end(k, dev ? host : nullptr, count, i0, one, map, total);
        if (i < 0) return LPQ_ERR_SHAPE;
        map.gdiv = gdiv;
        dispatch(k, dim3((unsigned)total), stream, dev ? dev + i0 : nullptr, one, map, fa, fb);
        lpq_status st = launched();
        if (st != LPQ_OK) return st;
        i0 = i;
    }
    return LPQ_OK;
}

lpq_tensor make_one(const void* src, void* dst, void* scale, int64_t M, int64_t N) {
    lpq_tensor t;
    t.src = src;
    t.dst = dst;
    t.scale = scale;
    t.rows = M;
    t.cols = N;
    t.group = 0;
    t.reserved = 0;
    return t;
}

template <typename D>
lpq_status single(Kind k, const D& one, const float* fa, float* fb, void* stream, float gdiv = 2688.0f) {
    lpq_status st = check_tensor(k, one, 0);
    if (st != LPQ_OK) return st;
    return launch<D>(k, nullptr, nullptr, 0, one, fa, fb, (hipStream_t)stream, gdiv);
}

template <typename D>
lpq_status grouped(Kind k, const D* host, const D* dev, int32_t n, int32_t n_groups, const float* fa, float* fb,
                   void* stream, float gdiv = 2688.0f) {
    if (!host || !dev) return LPQ_ERR_NULL;
    if (n <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(dev, 8)) return LPQ_ERR_ALIGN;
    for (int32_t i = 0; i < n; i++) {
        lpq_status st = check_tensor(k, host[i], n_groups);
        if (st != LPQ_OK) return st;
    }
    return launch<D>(k, host, dev, n, D{}, fa, fb, (hipStream_t)stream, gdiv);
}

// Strip width of a block-FP8 quantize call: 4 tiles per workgroup when the
// call has at least LPQ_TILEQ_WIDE_MIN 4-tile strips and takes no more
// launches that way, else LPQ_TILEQ_TW.  Measured: wide strips run faster on
// large launches (longer contiguous row runs) and slower on short ones, where
// fewer, longer workgroups leave more of the chip idle at the end.  The launch
// count matters when the table alternates shapes: Qwen3-30B-A3B experts
// (768x2048, 2048x768) have equal 2-tile strip counts, one run of equal work
// units, but unequal 4-tile counts, a new run at every tensor.  Any tensor that
// fails the checks keeps the narrow kind (the call is refused later).
Kind fp8blk_quant_kind(const lpq_tensor* t, int32_t n) {
    if (!t || n <= 0) return FP8BLK_Q;
    int64_t strips = 0;
    for (int32_t i = 0; i < n; i++) {
        if (check_tensor(FP8BLK_QW, t[i], 0) != LPQ_OK) return FP8BLK_Q;
        strips += units(FP8BLK_QW, t[i]);
    }
    if (strips < LPQ_TILEQ_WIDE_MIN) return FP8BLK_Q;
    const int64_t wide = launch_count(FP8BLK_QW, t, n), narrow = launch_count(FP8BLK_Q, t, n);
    return wide > 0 && wide <= narrow ? FP8BLK_QW : FP8BLK_Q;
}

// The kind of an INT4 operation ("INT4 QAT 训练") for a group size of 32 or
// 128; -1 for any other group size (the call returns LPQ_ERR_ARG).
int int4_kind(Kind k32, Kind k128, int32_t group) { return group == 32 ? k32 : group == 128 ? k128 : -1; }

// 6 * the E4M3 maximum of an NVFP4 call, or 0 for an unsupported maximum.
float gdiv_of(int e4m3_max) { return e4m3_max == 448 ? 2688.0f : (e4m3_max == 256 ? 1536.0f : 0.0f); }

lpq_requant_tensor make_requant(const uint8_t* q, const float* s, void* dst, void* dst_scale, int64_t M, int64_t N) {
    lpq_requant_tensor t;
    t.src = q;
    t.src_scale = s;
    t.dst = dst;
    t.dst_scale = dst_scale;
    t.rows = M;
    t.cols = N;
    t.group = 0;
    t.reserved = 0;
    return t;
}

lpq_status fill(float* p, int64_t n, float v, void* stream) {
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       (hipStream_t)stream, p, n, v);
    return launched();
}

}  // namespace

extern "C" {

const char* lpq_status_string(int status) {
    switch (status) {
    case LPQ_OK: return "ok";
    case LPQ_ERR_NULL: return "a required pointer is NULL";
    case LPQ_ERR_SHAPE: return "invalid shape (M or N <= 0, N not a multiple of the block, or count <= 0)";
    case LPQ_ERR_ALIGN: return "a pointer is not aligned as required";
    case LPQ_ERR_GROUP: return "sibling-group index out of range";
    case LPQ_ERR_HIP: return "HIP launch failed (see lpq_last_hip_error)";
    case LPQ_ERR_ARG: return "invalid argument";
    default: return "unknown status";
    }
}

int lpq_last_hip_error(void) { return g_last_hip_error; }

int lpq_version(void) { return 10000; }

lpq_status lpq_quantize_fp8blk(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, float* s, void* stream) {
    const lpq_tensor one = make_one(w, q, s, M, N);
    return single(fp8blk_quant_kind(&one, 1), one, nullptr, nullptr, stream);
}

lpq_status lpq_dequantize_fp8blk(const uint8_t* q, const float* s, int64_t M, int64_t N, uint16_t* y, void* stream) {
    const lpq_tensor one = make_one(q, y, const_cast<float*>(s), M, N);
    const bool flat = check_tensor(FP8BLK_DQ, one, 0) == LPQ_OK && check_tensor(FP8BLK_DQF, one, 0) == LPQ_OK;
    return single(flat ? FP8BLK_DQF : FP8BLK_DQ, one, nullptr, nullptr, stream);
}

lpq_status lpq_quantize_mxfp8(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e, void* stream) {
    return single(MXFP8_Q, make_one(w, q, e, M, N), nullptr, nullptr, stream);
}

lpq_status lpq_quantize_mxfp8_floor(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e, void* stream) {
    return single(MXFP8_QF, make_one(w, q, e, M, N), nullptr, nullptr, stream);
}

lpq_status lpq_quantize_mxfp8_floor_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, void* stream) {
    return grouped(MXFP8_QF, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_nvfp4_global_scale_reciprocal(const float* group_amax, int32_t n_groups, float* out, void* stream) {
    if (!group_amax || !out) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4) || !aligned(out, 4)) return LPQ_ERR_ALIGN;
    hipLaunchKernelGGL(k_global_scale_reciprocal, dim3((unsigned)((n_groups + kThreads - 1) / kThreads)), dim3(kThreads),
                       0, (hipStream_t)stream, group_amax, n_groups, out);
    return launched();
}

lpq_status lpq_nvfp4_global_scale(const float* amax, int32_t n, float* out, void* stream) {
    if (!amax || !out) return LPQ_ERR_NULL;
    if (n <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(amax, 4) || !aligned(out, 4)) return LPQ_ERR_ALIGN;
    hipLaunchKernelGGL(k_global_scale, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       (hipStream_t)stream, amax, n, out);
    return launched();
}

lpq_status lpq_observer_reset(float* state, void* stream) {
    if (!state) return LPQ_ERR_NULL;
    if (!aligned(state, 4)) return LPQ_ERR_ALIGN;
    hipLaunchKernelGGL(k_observer_reset, dim3(1), dim3(64), 0, (hipStream_t)stream, reinterpret_cast<uint32_t*>(state));
    return launched();
}

lpq_status lpq_nvfp4_observe(const uint16_t* x, int64_t M, int64_t N, int observer, float averaging_constant,
                             float* state, float* amax, void* stream) {
    if (!state || !amax) return LPQ_ERR_NULL;
    if (!aligned(state, 4) || !aligned(amax, 4)) return LPQ_ERR_ALIGN;
    if (observer < LPQ_OBSERVER_MEMORYLESS_MINMAX || observer > LPQ_OBSERVER_MINMAX) return LPQ_ERR_ARG;
    const lpq_tensor one = make_one(x, nullptr, nullptr, M, N);
    lpq_status st = check_tensor(NV_AMAX, one, 0);   // same shape and alignment rules as the amax pass
    if (st != LPQ_OK) return st;
    const int64_t units = (M * N + chunk_elems<LPQ_AMAX_U>() - 1) / chunk_elems<LPQ_AMAX_U>();
    if (units > kMaxGridX) return LPQ_ERR_SHAPE;
    hipLaunchKernelGGL((k_minmax<LPQ_AMAX_U>), dim3((unsigned)units), dim3(kThreads), 0, (hipStream_t)stream, one,
                       observer, averaging_constant, reinterpret_cast<uint32_t*>(state), amax);
    return launched();
}

lpq_status lpq_dequantize_mxfp8(const uint8_t* q, const uint8_t* e, int64_t M, int64_t N, uint16_t* y, void* stream) {
    return single(MXFP8_DQ, make_one(q, y, const_cast<uint8_t*>(e), M, N), nullptr, nullptr, stream);
}

lpq_status lpq_nvfp4_amax(const uint16_t* w, int64_t M, int64_t N, float* amax, int accumulate, void* stream) {
    if (!amax) return LPQ_ERR_NULL;
    if (!aligned(amax, 4)) return LPQ_ERR_ALIGN;
    const lpq_tensor one = make_one(w, nullptr, nullptr, M, N);
    lpq_status st = check_tensor(NV_AMAX, one, 0);
    if (st != LPQ_OK) return st;
    if (!accumulate && (st = fill(amax, 1, 0.0f, stream)) != LPQ_OK) return st;
    return launch<lpq_tensor>(NV_AMAX, nullptr, nullptr, 0, one, nullptr, amax, (hipStream_t)stream);
}

lpq_status lpq_quantize_nvfp4(const uint16_t* w, int64_t M, int64_t N, const float* amax, uint8_t* p, uint8_t* s,
                              float* g, void* stream) {
    if (!amax || !g) return LPQ_ERR_NULL;
    if (!aligned(amax, 4) || !aligned(g, 4)) return LPQ_ERR_ALIGN;
    return single(NV_Q, make_one(w, p, s, M, N), amax, g, stream);
}

lpq_status lpq_dequantize_nvfp4(const uint8_t* p, const uint8_t* s, const float* g, int64_t M, int64_t N, uint16_t* y,
                                void* stream) {
    if (!g) return LPQ_ERR_NULL;
    if (!aligned(g, 4)) return LPQ_ERR_ALIGN;
    return single(NV_DQ, make_one(p, y, const_cast<uint8_t*>(s), M, N), g, nullptr, stream);
}

lpq_status lpq_nvfp4_qdq(const uint16_t* x, int64_t M, int64_t N, const float* amax, uint16_t* y, void* stream) {
    if (!amax) return LPQ_ERR_NULL;
    if (!aligned(amax, 4)) return LPQ_ERR_ALIGN;
    return single(NV_QDQ, make_one(x, y, nullptr, M, N), amax, nullptr, stream);
}

lpq_status lpq_quantize_nvfp4_ex(const uint16_t* w, int64_t M, int64_t N, const float* amax, int e4m3_max, uint8_t* p,
                                 uint8_t* s, float* g, void* stream) {
    if (!amax || !g) return LPQ_ERR_NULL;
    if (!aligned(amax, 4) || !aligned(g, 4)) return LPQ_ERR_ALIGN;
    if (gdiv_of(e4m3_max) == 0.0f) return LPQ_ERR_ARG;
    return single(NV_Q, make_one(w, p, s, M, N), amax, g, stream, gdiv_of(e4m3_max));
}

lpq_status lpq_nvfp4_qdq_ex(const uint16_t* x, int64_t M, int64_t N, const float* amax, int e4m3_max, uint16_t* y,
                            void* stream) {
    if (!amax) return LPQ_ERR_NULL;
    if (!aligned(amax, 4)) return LPQ_ERR_ALIGN;
    if (gdiv_of(e4m3_max) == 0.0f) return LPQ_ERR_ARG;
    return single(NV_QDQ, make_one(x, y, nullptr, M, N), amax, nullptr, stream, gdiv_of(e4m3_max));
}

lpq_status lpq_quantize_nvfp4_grouped_ex(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                         const float* group_amax, int32_t n_groups, int e4m3_max, float* group_g,
                                         void* stream) {
    if (!group_amax || !group_g) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4) || !aligned(group_g, 4)) return LPQ_ERR_ALIGN;
    if (gdiv_of(e4m3_max) == 0.0f) return LPQ_ERR_ARG;
    return grouped(NV_Q, host, dev, n, n_groups, group_amax, group_g, stream, gdiv_of(e4m3_max));
}

lpq_status lpq_nvfp4_qdq_grouped_ex(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, const float* group_amax,
                                    int32_t n_groups, int e4m3_max, void* stream) {
    if (!group_amax) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4)) return LPQ_ERR_ALIGN;
    if (gdiv_of(e4m3_max) == 0.0f) return LPQ_ERR_ARG;
    return grouped(NV_QDQ, host, dev, n, n_groups, group_amax, nullptr, stream, gdiv_of(e4m3_max));
}

lpq_status lpq_quantize_fp8blk_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, void* stream) {
    return grouped(fp8blk_quant_kind(host, n), host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_dequantize_fp8blk_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, void* stream) {
    // the flat kernel when every tensor allows it, else the tile kernel for all
    bool flat = host != nullptr && n > 0;
    for (int32_t i = 0; flat && i < n; i++) flat = check_tensor(FP8BLK_DQF, host[i], 0) == LPQ_OK;
    return grouped(flat ? FP8BLK_DQF : FP8BLK_DQ, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_quantize_mxfp8_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, void* stream) {
    return grouped(MXFP8_Q, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_dequantize_mxfp8_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, void* stream) {
    return grouped(MXFP8_DQ, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_nvfp4_amax_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, float* group_amax,
                                  int32_t n_groups, int accumulate, void* stream) {
    if (!group_amax) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4)) return LPQ_ERR_ALIGN;
    if (!host || !dev) return LPQ_ERR_NULL;
    if (n <= 0) return LPQ_ERR_SHAPE;
    for (int32_t i = 0; i < n; i++) {
        lpq_status st = check_tensor(NV_AMAX, host[i], n_groups);
        if (st != LPQ_OK) return st;
    }
    if (!accumulate) {
        lpq_status st = fill(group_amax, n_groups, 0.0f, stream);
        if (st != LPQ_OK) return st;
    }
    return grouped(NV_AMAX, host, dev, n, n_groups, nullptr, group_amax, stream);
}

lpq_status lpq_quantize_nvfp4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                      const float* group_amax, int32_t n_groups, float* group_g, void* stream) {
    if (!group_amax || !group_g) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4) || !aligned(group_g, 4)) return LPQ_ERR_ALIGN;
    return grouped(NV_Q, host, dev, n, n_groups, group_amax, group_g, stream);
}

lpq_status lpq_dequantize_nvfp4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                        const float* group_g, int32_t n_groups, void* stream) {
    if (!group_g) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_g, 4)) return LPQ_ERR_ALIGN;
    return grouped(NV_DQ, host, dev, n, n_groups, group_g, nullptr, stream);
}

lpq_status lpq_nvfp4_qdq_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, const float* group_amax,
                                 int32_t n_groups, void* stream) {
    if (!group_amax) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4)) return LPQ_ERR_ALIGN;
    return grouped(NV_QDQ, host, dev, n, n_groups, group_amax, nullptr, stream);
}

lpq_status lpq_requantize_fp8blk(const uint8_t* q, const float* s, int64_t M, int64_t N, uint8_t* q_out, float* s_out,
                                 void* stream) {
    return single(RQ_FP8, make_requant(q, s, q_out, s_out, M, N), nullptr, nullptr, stream);
}

lpq_status lpq_requantize_fp8blk_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev, int32_t n,
                                         void* stream) {
    return grouped(RQ_FP8, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_requantize_fp8blk_mxfp8(const uint8_t* q, const float* s, int64_t M, int64_t N, uint8_t* q_out,
                                       uint8_t* e_out, void* stream) {
    return single(RQ_MX, make_requant(q, s, q_out, e_out, M, N), nullptr, nullptr, stream);
}

lpq_status lpq_fp8blk_amax(const uint8_t* q, const float* s, int64_t M, int64_t N, float* amax, int accumulate,
                           void* stream) {
    if (!amax) return LPQ_ERR_NULL;
    if (!aligned(amax, 4)) return LPQ_ERR_ALIGN;
    const lpq_requant_tensor one = make_requant(q, s, nullptr, nullptr, M, N);
    lpq_status st = check_tensor(RQ_AMAX, one, 0);
    if (st != LPQ_OK) return st;
    if (!accumulate && (st = fill(amax, 1, 0.0f, stream)) != LPQ_OK) return st;
    return launch<lpq_requant_tensor>(RQ_AMAX, nullptr, nullptr, 0, one, nullptr, amax, (hipStream_t)stream);
}

lpq_status lpq_requantize_fp8blk_nvfp4(const uint8_t* q, const float* s, int64_t M, int64_t N, const float* amax,
                                       uint8_t* p, uint8_t* sb, float* g, void* stream) {
    if (!amax || !g) return LPQ_ERR_NULL;
    if (!aligned(amax, 4) || !aligned(g, 4)) return LPQ_ERR_ALIGN;
    return single(RQ_NV, make_requant(q, s, p, sb, M, N), amax, g, stream);
}

lpq_status lpq_requantize_fp8blk_mxfp8_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev,
                                               int32_t n, void* stream) {
    return grouped(RQ_MX, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_fp8blk_amax_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev, int32_t n,
                                   float* group_amax, int32_t n_groups, int accumulate, void* stream) {
    if (!group_amax) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4)) return LPQ_ERR_ALIGN;
    if (!host || !dev) return LPQ_ERR_NULL;
    if (n <= 0) return LPQ_ERR_SHAPE;
    for (int32_t i = 0; i < n; i++) {
        lpq_status st = check_tensor(RQ_AMAX, host[i], n_groups);
        if (st != LPQ_OK) return st;
    }
    if (!accumulate) {
        lpq_status st = fill(group_amax, n_groups, 0.0f, stream);
        if (st != LPQ_OK) return st;
    }
    return grouped(RQ_AMAX, host, dev, n, n_groups, nullptr, group_amax, stream);
}

lpq_status lpq_requantize_fp8blk_nvfp4_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev,
                                               int32_t n, const float* group_amax, int32_t n_groups,
                                               float* group_g, void* stream) {
    if (!group_amax || !group_g) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4) || !aligned(group_g, 4)) return LPQ_ERR_ALIGN;
    return grouped(RQ_NV, host, dev, n, n_groups, group_amax, group_g, stream);
}

lpq_status lpq_quantize_int4(const uint16_t* w, int64_t M, int64_t N, int32_t group, uint8_t* p, float* s,
                             void* stream) {
    const int k = int4_kind(I4_Q32, I4_Q128, group);
    if (k < 0) return LPQ_ERR_ARG;
    return single((Kind)k, make_one(w, p, s, M, N), nullptr, nullptr, stream);
}

lpq_status lpq_dequantize_int4(const uint8_t* p, const float* s, int64_t M, int64_t N, int32_t group, uint16_t* y,
                               void* stream) {
    const int k = int4_kind(I4_DQ32, I4_DQ128, group);
    if (k < 0) return LPQ_ERR_ARG;
    return single((Kind)k, make_one(p, y, const_cast<float*>(s), M, N), nullptr, nullptr, stream);
}

lpq_status lpq_int4_qdq(const uint16_t* x, int64_t M, int64_t N, int32_t group, uint16_t* y, void* stream) {
    const int k = int4_kind(I4_QDQ32, I4_QDQ128, group);
    if (k < 0) return LPQ_ERR_ARG;
    return single((Kind)k, make_one(x, y, nullptr, M, N), nullptr, nullptr, stream);
}

lpq_status lpq_quantize_int4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, int32_t group,
                                     void* stream) {
    const int k = int4_kind(I4_Q32, I4_Q128, group);
    if (k < 0) return LPQ_ERR_ARG;
    return grouped((Kind)k, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_dequantize_int4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, int32_t group,
                                       void* stream) {
    const int k = int4_kind(I4_DQ32, I4_DQ128, group);
    if (k < 0) return LPQ_ERR_ARG;
    return grouped((Kind)k, host, dev, n, 0, nullptr, nullptr, stream);
}

lpq_status lpq_int4_qdq_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, int32_t group,
                                void* stream) {
    const int k = int4_kind(I4_QDQ32, I4_QDQ128, group);
    if (k < 0) return LPQ_ERR_ARG;
    return grouped((Kind)k, host, dev, n, 0, nullptr, nullptr, stream);
}

}  // extern "C"
