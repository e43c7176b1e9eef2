// Shared device-side machinery: constants, flat work units, the dense work map
// and its lookup, load order.
//
// Part of lpq_kernels.hip, which includes each part once, in this order: one
// translation unit.
#pragma once

namespace {

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

}  // namespace
