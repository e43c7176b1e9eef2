// Launch parameters of the kernels (compile-time; each can be overridden with
// -D).
//
// Part of lpq_kernels.hip, which includes each part once, in this order: one
// translation unit.
#pragma once

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
// The single-tensor QDQ of at most LPQ_QDQW_MAX_ELEMS elements (the W4A4
// activation case): 512-thread workgroups of 16 vectors per lane, all loaded
// up front, so that a 8192 x 2048 activation is one pass of 256 workgroups.
#ifndef LPQ_QDQW_U
#define LPQ_QDQW_U 16
#endif
#ifndef LPQ_QDQW_T
#define LPQ_QDQW_T 512
#endif
#ifndef LPQ_QDQW_AHEAD
#define LPQ_QDQW_AHEAD 0
#endif
#ifndef LPQ_QDQW_MAX_ELEMS
#define LPQ_QDQW_MAX_ELEMS (int64_t(1) << 25)
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
#define LPQ_DQF_AHEAD 1
#endif
#ifndef LPQ_RQM_AHEAD
#define LPQ_RQM_AHEAD 1
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



#ifndef LPQ_FLAT_THREADS
#define LPQ_FLAT_THREADS 256
#endif
// Workgroup size of each flat kernel (64 to 512, a multiple of 64), measured
// per kernel: the NVFP4 encoder runs best with one wave, MXFP8 encoding, the
// QDQs and the flat block-FP8 decoder with 128 threads, the NVFP4 and INT4
// decoders and the INT4 encoder with 512, the rest with 256.
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
#define LPQ_DQF_T 128
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
