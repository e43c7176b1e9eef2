// Block-wise FP8: the tile quantizer (strips of 2 or 4 tiles) and the tile
// dequantizer.
//
// Part of lpq_kernels.hip, which includes each part once, in this order: one
// translation unit.
#pragma once

namespace {

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

}  // namespace
