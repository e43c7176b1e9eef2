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

#include <atomic>

#include "lpq.h"
#include "lpq_device.hpp"

// Launch parameters, then the kernels, format by format.
#include "lpq_tuning.hpp"

using namespace lpq;

#include "lpq_flat.hpp"
#include "lpq_mxfp8.hpp"
#include "lpq_nvfp4.hpp"
#include "lpq_int4.hpp"
#include "lpq_fp8blk.hpp"
#include "lpq_requant.hpp"


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
    FP8BLK_Q, FP8BLK_QW, FP8BLK_DQ, FP8BLK_DQF, MXFP8_Q, MXFP8_QF, MXFP8_DQ, NV_AMAX, NV_Q, NV_DQ, NV_QDQ, NV_QDQ_W,
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
    case NV_QDQ_W: return (n + chunk_elems<LPQ_QDQW_U, LPQ_QDQW_T>() - 1) / chunk_elems<LPQ_QDQW_U, LPQ_QDQW_T>();
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
        case NV_QDQ_W:
            hipLaunchKernelGGL((k_nvfp4_qdq<LPQ_QDQW_U, LPQ_QDQW_T, false, LPQ_QDQW_AHEAD != 0>), grid, dim3(LPQ_QDQW_T), 0,
                               stream, tab, one, map, fa);
            break;
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

// Checks of a grouped call's tables and of every descriptor for kind k.
template <typename D>
lpq_status check_grouped(Kind k, const D* host, const D* dev, int32_t n, int32_t n_groups) {
    if (!host || !dev) return LPQ_ERR_NULL;
    if (n <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(dev, 8)) return LPQ_ERR_ALIGN;
    for (int32_t i = 0; i < n; i++) {
        lpq_status st = check_tensor(k, host[i], n_groups);
        if (st != LPQ_OK) return st;
    }
    return LPQ_OK;
}

template <typename D>
lpq_status grouped(Kind k, const D* host, const D* dev, int32_t n, int32_t n_groups, const float* fa, float* fb,
                   void* stream, float gdiv = 2688.0f) {
    lpq_status st = check_grouped(k, host, dev, n, n_groups);
    if (st != LPQ_OK) return st;
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

lpq_status global_scale(const float* amax, int32_t n, float* out, float gdiv, void* stream) {
    hipLaunchKernelGGL(k_global_scale, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       (hipStream_t)stream, amax, n, out, gdiv);
    return launched();
}

// The single-tensor QDQ kind for n elements: a tensor of at most a few waves
// of full-CU workgroups takes the wide shape (every load of a lane issued up
// front); larger ones stream.
Kind qdq_kind(int64_t n) { return n <= LPQ_QDQW_MAX_ELEMS ? NV_QDQ_W : NV_QDQ; }

// NVFP4 quantize (k = NV_Q) or QDQ (k = NV_QDQ) of one tensor.  With amax ==
// NULL the tensor's own amax is the group amax ("verl NVFP4 QAT" 2.3: a tensor
// of its own is a group of one), computed by the call into a word the caller
// already owns, and every launch goes on the caller's stream, so each sees the
// previous one's result:
//   quantize: the g word is cleared, receives max |w| from the amax pass, is
//     read as A by the encode (which then leaves it alone), and is finally
//     turned into fl(A / gdiv);
//   QDQ: the first word of y is cleared and receives max |x|; the QDQ of every
//     element but the first 16-element block reads A from it; the QDQ of that
//     block runs last, reading A before it writes the block over the word
//     (only its first wave holds elements, and each lane reads A before its
//     store).  x and y must not overlap.
lpq_status nvfp4_single(Kind k, const uint16_t* w, int64_t M, int64_t N, const float* amax, int e4m3_max, void* dst,
                        void* scale, float* g, void* stream) {
    if (k == NV_Q && !g) return LPQ_ERR_NULL;
    if ((amax && !aligned(amax, 4)) || (g && !aligned(g, 4))) return LPQ_ERR_ALIGN;
    const float gdiv = gdiv_of(e4m3_max);
    if (gdiv == 0.0f) return LPQ_ERR_ARG;
    const lpq_tensor one = make_one(w, dst, scale, M, N);
    lpq_status st = check_tensor(k, one, 0);
    if (st != LPQ_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    const int64_t n = M * N;
    if (amax) {
        const Kind kk = k == NV_QDQ ? qdq_kind(n) : k;
        return launch<lpq_tensor>(kk, nullptr, nullptr, 0, one, amax, k == NV_Q ? g : nullptr, s, gdiv);
    }
    if (k == NV_Q) {
        if ((st = fill(g, 1, 0.0f, stream)) != LPQ_OK) return st;
        if ((st = launch<lpq_tensor>(NV_AMAX, nullptr, nullptr, 0, one, nullptr, g, s)) != LPQ_OK) return st;
        if ((st = launch<lpq_tensor>(NV_Q, nullptr, nullptr, 0, one, g, nullptr, s, gdiv)) != LPQ_OK) return st;
        return global_scale(g, 1, g, gdiv, stream);
    }
    uint16_t* y = static_cast<uint16_t*>(dst);
    const uintptr_t xa = reinterpret_cast<uintptr_t>(w), ya = reinterpret_cast<uintptr_t>(y);
    if (xa < ya + 2 * (uint64_t)n && ya < xa + 2 * (uint64_t)n) return LPQ_ERR_ARG;   // overlapping x and y
    float* a = reinterpret_cast<float*>(y);
    if ((st = fill(a, 1, 0.0f, stream)) != LPQ_OK) return st;
    if ((st = launch<lpq_tensor>(NV_AMAX, nullptr, nullptr, 0, one, nullptr, a, s)) != LPQ_OK) return st;
    if (n > 16) {
        const lpq_tensor tail = make_one(w + 16, y + 16, nullptr, 1, n - 16);
        if ((st = launch<lpq_tensor>(qdq_kind(n - 16), nullptr, nullptr, 0, tail, a, nullptr, s, gdiv)) != LPQ_OK)
            return st;
    }
    const lpq_tensor head = make_one(w, y, nullptr, 1, 16);
    return launch<lpq_tensor>(NV_QDQ_W, nullptr, nullptr, 0, head, a, nullptr, s, gdiv);
}

// Grouped NVFP4 quantize (NV_Q) or QDQ (NV_QDQ).  amax_valid != 0: group_amax
// holds each group's A (a cached or observed value, or lpq_nvfp4_amax_grouped's
// result) and is only read.  amax_valid == 0: the call fills it first -- the
// slots are cleared and the amax pass folds every member's max |w| into its
// group's slot (the group maximum, "verl NVFP4 QAT" 2.4) -- then encodes.
lpq_status nvfp4_grouped(Kind k, const lpq_tensor* host, const lpq_tensor* dev, int32_t n, float* group_amax,
                         int32_t n_groups, int amax_valid, int e4m3_max, float* group_g, void* stream) {
    if (!group_amax || (k == NV_Q && !group_g)) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_amax, 4) || (group_g && !aligned(group_g, 4))) return LPQ_ERR_ALIGN;
    const float gdiv = gdiv_of(e4m3_max);
    if (gdiv == 0.0f) return LPQ_ERR_ARG;
    lpq_status st = check_grouped(k, host, dev, n, n_groups);   // every amax-pass condition included
    if (st != LPQ_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    if (!amax_valid) {
        if ((st = fill(group_amax, n_groups, 0.0f, stream)) != LPQ_OK) return st;
        if ((st = launch<lpq_tensor>(NV_AMAX, host, dev, n, lpq_tensor{}, nullptr, group_amax, s)) != LPQ_OK) return st;
    }
    return launch<lpq_tensor>(k, host, dev, n, lpq_tensor{}, group_amax, k == NV_Q ? group_g : nullptr, s, gdiv);
}

// Host-side checks of an observer call; the workgroup count on success.
lpq_status observe_args(const uint16_t* x, int64_t M, int64_t N, int observer, const float* state, const float* amax,
                        lpq_tensor* one, int64_t* units) {
    if (!state || !amax) return LPQ_ERR_NULL;
    if (!aligned(state, 4) || !aligned(amax, 4)) return LPQ_ERR_ALIGN;
    if (observer < LPQ_OBSERVER_MEMORYLESS_MINMAX || observer > LPQ_OBSERVER_MINMAX) return LPQ_ERR_ARG;
    *one = make_one(x, nullptr, nullptr, M, N);
    lpq_status st = check_tensor(NV_AMAX, *one, 0);   // same shape and alignment rules as the amax pass
    if (st != LPQ_OK) return st;
    *units = (M * N + chunk_elems<LPQ_AMAX_U>() - 1) / chunk_elems<LPQ_AMAX_U>();
    return *units > kMaxGridX ? LPQ_ERR_SHAPE : LPQ_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// The allocation-free observer call keeps the control words of a call (batch
// keys and arrival counter) in a block the library holds, instead of in the
// caller's state.  Every device the library runs on holds its own copy of the
// block until the process ends.  All such calls on one device share it: each
// call re-arms it first, and calls that overlap on one device race.

static __device__ __align__(256) uint32_t scratch[kObsCtlWords];

namespace {

constexpr int kMaxScratchDevices = 64;
std::atomic<uint32_t*> g_scratch_ptr[kMaxScratchDevices];

inline lpq_status hip_failed(hipError_t e) {
    g_last_hip_error = (int)e;
    return LPQ_ERR_HIP;
}

// The device address of `scratch` on the device that `stream` runs on (the
// current device for the null stream).  It is looked up once per device, with
// that device current, and kept: on the host the name `scratch` is a stand-in,
// not a device address, and each device holds the block at its own address.
lpq_status scratch_on(hipStream_t stream, uint32_t** out) {
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_failed(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return hip_failed(hipErrorInvalidDevice);
    uint32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_failed(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_failed(e);
        void* q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return hip_failed(e);
        if (!q) return hip_failed(hipErrorInvalidSymbol);
        p = static_cast<uint32_t*>(q);
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return LPQ_OK;
}

}  // namespace

extern "C" {

const char* lpq_status_string(lpq_status status) {
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
    return global_scale(amax, n, out, 2688.0f, stream);
}

lpq_status lpq_observer_reset(float* state, void* stream) {
    if (!state) return LPQ_ERR_NULL;
    if (!aligned(state, 4)) return LPQ_ERR_ALIGN;
    hipLaunchKernelGGL(k_observer_reset, dim3(1), dim3(64), 0, (hipStream_t)stream, reinterpret_cast<uint32_t*>(state));
    return launched();
}

lpq_status lpq_nvfp4_observe(const uint16_t* x, int64_t M, int64_t N, int observer, float averaging_constant,
                             float* state, float* amax, void* stream) {
    lpq_tensor one;
    int64_t units = 0;
    const lpq_status st = observe_args(x, M, N, observer, state, amax, &one, &units);
    if (st != LPQ_OK) return st;
    hipLaunchKernelGGL((k_minmax<LPQ_AMAX_U>), dim3((unsigned)units), dim3(kThreads), 0, (hipStream_t)stream, one,
                       observer, averaging_constant, state, reinterpret_cast<uint32_t*>(state), amax);
    return launched();
}

lpq_status lpq_nvfp4_observe_noalloc(const uint16_t* x, int64_t M, int64_t N, int observer,
                                     float averaging_constant, float* state, float* amax, void* stream) {
    lpq_tensor one;
    int64_t units = 0;
    lpq_status st = observe_args(x, M, N, observer, state, amax, &one, &units);
    if (st != LPQ_OK) return st;
    uint32_t* ctl = nullptr;
    if ((st = scratch_on((hipStream_t)stream, &ctl)) != LPQ_OK) return st;
    hipLaunchKernelGGL(k_observer_arm, dim3(1), dim3(64), 0, (hipStream_t)stream, ctl);
    if ((st = launched()) != LPQ_OK) return st;
    hipLaunchKernelGGL((k_minmax<LPQ_AMAX_U>), dim3((unsigned)units), dim3(kThreads), 0, (hipStream_t)stream, one,
                       observer, averaging_constant, state, ctl, amax);
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
    return nvfp4_single(NV_Q, w, M, N, amax, 448, p, s, g, stream);
}

lpq_status lpq_dequantize_nvfp4(const uint8_t* p, const uint8_t* s, const float* g, int64_t M, int64_t N, uint16_t* y,
                                void* stream) {
    if (!g) return LPQ_ERR_NULL;
    if (!aligned(g, 4)) return LPQ_ERR_ALIGN;
    return single(NV_DQ, make_one(p, y, const_cast<uint8_t*>(s), M, N), g, nullptr, stream);
}

lpq_status lpq_nvfp4_qdq(const uint16_t* x, int64_t M, int64_t N, const float* amax, uint16_t* y, void* stream) {
    return nvfp4_single(NV_QDQ, x, M, N, amax, 448, y, nullptr, nullptr, stream);
}

lpq_status lpq_quantize_nvfp4_ex(const uint16_t* w, int64_t M, int64_t N, const float* amax, int e4m3_max, uint8_t* p,
                                 uint8_t* s, float* g, void* stream) {
    return nvfp4_single(NV_Q, w, M, N, amax, e4m3_max, p, s, g, stream);
}

lpq_status lpq_nvfp4_qdq_ex(const uint16_t* x, int64_t M, int64_t N, const float* amax, int e4m3_max, uint16_t* y,
                            void* stream) {
    return nvfp4_single(NV_QDQ, x, M, N, amax, e4m3_max, y, nullptr, nullptr, stream);
}

lpq_status lpq_quantize_nvfp4_grouped_ex(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, float* group_amax,
                                         int32_t n_groups, int amax_valid, int e4m3_max, float* group_g,
                                         void* stream) {
    return nvfp4_grouped(NV_Q, host, dev, n, group_amax, n_groups, amax_valid, e4m3_max, group_g, stream);
}

lpq_status lpq_nvfp4_qdq_grouped_ex(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, float* group_amax,
                                    int32_t n_groups, int amax_valid, int e4m3_max, void* stream) {
    return nvfp4_grouped(NV_QDQ, host, dev, n, group_amax, n_groups, amax_valid, e4m3_max, nullptr, stream);
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

lpq_status lpq_quantize_nvfp4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, float* group_amax,
                                      int32_t n_groups, int amax_valid, float* group_g, void* stream) {
    return nvfp4_grouped(NV_Q, host, dev, n, group_amax, n_groups, amax_valid, 448, group_g, stream);
}

lpq_status lpq_dequantize_nvfp4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                        const float* group_g, int32_t n_groups, void* stream) {
    if (!group_g) return LPQ_ERR_NULL;
    if (n_groups <= 0) return LPQ_ERR_SHAPE;
    if (!aligned(group_g, 4)) return LPQ_ERR_ALIGN;
    return grouped(NV_DQ, host, dev, n, n_groups, group_g, nullptr, stream);
}

lpq_status lpq_nvfp4_qdq_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, float* group_amax,
                                 int32_t n_groups, int amax_valid, void* stream) {
    return nvfp4_grouped(NV_QDQ, host, dev, n, group_amax, n_groups, amax_valid, 448, nullptr, stream);
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
