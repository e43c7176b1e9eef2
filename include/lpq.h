/*
 * lpq.h -- C ABI of the MI355X (gfx950) low-precision weight codec library
 * (liblpq.so): BF16 -> block-wise FP8 / MXFP8 / NVFP4 quantizers, their
 * dequantizers, and the NVFP4 fake-quant (quantize-dequantize, "QDQ").
 *
 * What the calls compute (web pages, cited by title and section):
 *  - "Low Precision RL" (Miles documentation), "Choose a precision" table and
 *    "Modes": block-wise FP8 = E4M3 codes with one FP32 scale per 128x128
 *    tile; MXFP8 = E4M3 codes with one UE8M0 (power-of-two, uint8) scale per
 *    1x32 block; NVFP4 = E2M1 codes in 1x16 blocks with a two-level scale
 *    (E4M3 per block, FP32 per tensor).  Weights are re-quantized from the BF16
 *    master copy at every weight-update sync.
 *  - "verl NVFP4 QAT" article (capital-peak.com), section 2.3: NVFP4 global
 *    scale = amax / (6 * 448); per-16-element block amax turned into an E4M3
 *    block scale; values snapped to the nearest of {0,0.5,1,1.5,2,3,4,6} and
 *    multiplied back (fake quantization).  Section 2.4: q/k/v and gate/up
 *    siblings share one global scale, taken from the group maximum.  Sections
 *    2.5 and 3.3: exported tensors are the packed FP4 weight, the E4M3 block
 *    scales and the FP32 global scale.
 *  - vime pull request 503 review: exact round-to-nearest numerics.
 * Every cast rounds to nearest, ties to even; E4M3 and E2M1 casts saturate
 * (+-448, +-6); zero scales give zero codes that keep the element's sign.
 * The exact arithmetic of each format is written out where it is declared.
 *
 * Conventions (all entry points):
 *  - Pointers are DEVICE pointers unless stated otherwise.  The caller owns
 *    every buffer; the library never allocates, frees or synchronizes, keeps
 *    no state between calls (apart from the thread-local last HIP error, and
 *    the per-device control block of lpq_nvfp4_observe_noalloc, whose calls
 *    must not overlap on one device) and is safe to call from several host
 *    threads.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; a kernel fault surfaces at the caller's
 *    next synchronization.  A call enqueues kernels only (no memset, copy or
 *    allocation), so it can be recorded by stream capture into a HIP graph
 *    and replayed; the host-side table of a grouped call is read when the
 *    call is made, and the device-side table must hold the same descriptors
 *    at every replay.
 *  - Tensors are row-major and contiguous: M rows (out_features) by N
 *    columns (in_features); blocks run along N.  BF16 values travel as
 *    uint16_t bit patterns, E4M3 codes as uint8_t (float8_e4m3fn).
 *  - Every argument check that can run on the host runs before anything is
 *    enqueued; on failure nothing is enqueued and the status says why.
 *  - Alignment (LPQ_ERR_ALIGN otherwise): MXFP8 and NVFP4 BF16 arrays 16
 *    bytes, MXFP8 code arrays 8 bytes, NVFP4 packed arrays 4 bytes; the
 *    block-wise FP8 calls accept any 2-byte aligned BF16 and any code array
 *    (rows that are not 16-byte aligned take a slower path).  FP32 arrays
 *    (scales, amax, global scales) must be 4-byte aligned; byte scale arrays
 *    have no requirement.
 *  - Inputs are finite; NaN and Inf inputs are outside the contract.
 */
#ifndef LPQ_H
#define LPQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* C++ sees a fixed 32-bit int underlying type, so that any int a C caller
 * passes (lpq_status_string of an unknown code) is a valid value there too. */
#ifdef __cplusplus
typedef enum lpq_status : int {
#else
typedef enum lpq_status {
#endif
    LPQ_OK = 0,
    LPQ_ERR_NULL = 1,   /* a required pointer is NULL                                   */
    LPQ_ERR_SHAPE = 2,  /* M or N <= 0, N not a multiple of the block (32 MXFP8, 16
                           NVFP4), a tensor count <= 0, or a tensor beyond the size
                           limits (M * N above 2^40 for every call; tighter limits are
                           stated where a call has one)                                 */
    LPQ_ERR_ALIGN = 3,  /* a pointer is not aligned as required (see above)             */
    LPQ_ERR_GROUP = 4,  /* an NVFP4 sibling-group index is outside [0, n_groups)        */
    LPQ_ERR_HIP = 5,    /* a HIP launch failed; lpq_last_hip_error() holds the code     */
    LPQ_ERR_ARG = 6     /* any other invalid argument (reserved field not 0, ...)      */
} lpq_status;

/* Static, NUL-terminated description of a status code ("unknown status" for a
 * value outside the enumeration). */
const char* lpq_status_string(lpq_status status);

/* hipError_t of the most recent LPQ_ERR_HIP on the calling thread (0 if none). */
int lpq_last_hip_error(void);

/* Library version, as MAJOR * 10000 + MINOR * 100 + PATCH. */
int lpq_version(void);

/* ======================================================================== */
/* Block-wise FP8 ("DeepSeek-style"): "Low Precision RL", "Choose a precision"
 * and "2. Unified block-wise FP8" -- 128 x 128 tiles, FP32 (not power-of-two)
 * scales.
 *   tile (i, j) = rows [128i, min(128i+128, M)) x cols [128j, min(128j+128, N))
 *   amax  = max |w| over the tile
 *   s     = fl(amax / 448)                       stored FP32, the dequant multiplier
 *   q     = E4M3(fl(w / s))   (s == 0: a zero with w's sign)
 *   y     = BF16(fl(E4M3value(q) * s))
 * w: [M, N] BF16.  q: [M, N] codes.  s: [ceil(M/128), ceil(N/128)] FP32. */
lpq_status lpq_quantize_fp8blk(const uint16_t* w, int64_t M, int64_t N,
                               uint8_t* q, float* s, void* stream);
lpq_status lpq_dequantize_fp8blk(const uint8_t* q, const float* s, int64_t M, int64_t N,
                                 uint16_t* y, void* stream);

/* ======================================================================== */
/* MXFP8: "Low Precision RL", "3. Unified MXFP8" -- 1 x 32 blocks along a row,
 * UE8M0 power-of-two scales stored as uint8, E4M3 values.  N % 32 == 0.
 *   amax  = max |w| over the 32 elements of the block
 *   e     = the smallest integer with amax <= 448 * 2^e, clamped to e >= -127
 *           (the power-of-two counterpart of amax / 448: no element saturates)
 *   byte  = e + 127                               (never 255)
 *   q     = E4M3(w * 2^-e)                        (exact scaling, one rounding)
 *   y     = BF16(E4M3value(q) * 2^e)
 * w: [M, N] BF16.  q: [M, N] codes.  e: [M, N/32] uint8. */
lpq_status lpq_quantize_mxfp8(const uint16_t* w, int64_t M, int64_t N,
                              uint8_t* q, uint8_t* e, void* stream);
lpq_status lpq_dequantize_mxfp8(const uint8_t* q, const uint8_t* e, int64_t M, int64_t N,
                                uint16_t* y, void* stream);

/* MXFP8 with the shared-exponent rule of the OCP Microscaling (MX) Formats
 * specification v1.0, section 6.3: X = 2^(floor(log2 amax) - 8) (8 is E4M3's
 * largest exponent), byte = max(0, floor(log2 amax) - 8 + 127), codes
 * E4M3(w / X) saturating at +-448 -- an element up to 1.14x beyond 448 * X
 * clamps.  The pages fix only power-of-two UE8M0 scales ("Low Precision RL",
 * "3. Unified MXFP8"); this is the alternative to lpq_quantize_mxfp8's rule,
 * for engines that expect it.  Same layouts, alignment and checks;
 * lpq_dequantize_mxfp8 decodes it. */
lpq_status lpq_quantize_mxfp8_floor(const uint16_t* w, int64_t M, int64_t N, uint8_t* q, uint8_t* e, void* stream);

/* ======================================================================== */
/* NVFP4: "Low Precision RL", "4. NVFP4"; "verl NVFP4 QAT", sections 2.3-2.5
 * and 3.3 -- E2M1 values in 1 x 16 blocks, an E4M3 block scale and an FP32
 * global scale.  N % 16 == 0.
 *   A     = max |w| over the tensor or its whole sibling group (the amax input)
 *   g     = fl(A / 2688)                           (2688 = 6 * 448)
 *   b     = max |w| over the 16-element block
 *   sb    = (g == 0) ? 0 : E4M3(fl(fl(b / 6) / g)) stored E4M3 block-scale code
 *   S     = fl(E4M3value(sb) * g)                  effective FP32 block multiplier
 *   code  = (S == 0) ? a zero with w's sign : E2M1(fl(w / S))
 *   y     = BF16(fl(E2M1value(code) * S))
 * Packed layout: element 2j in the low nibble of byte j. */

/* amax pre-pass: *amax = max(*amax, max |w|) when accumulate != 0; when
 * accumulate == 0 *amax is overwritten with max |w|.  amax: 1 FP32 on the
 * device.  The result does not depend on the order of the reduction. */
lpq_status lpq_nvfp4_amax(const uint16_t* w, int64_t M, int64_t N, float* amax,
                          int accumulate, void* stream);

/* amax: 1 FP32 (device) holding A (e.g. a cached amax, "verl NVFP4 QAT" 2.4,
 * or the group maximum of lpq_nvfp4_amax), or NULL: then A is this tensor's
 * own max |w| (a tensor of its own is a group of one), computed by the call
 * itself -- it reads w twice, and uses the caller's g word to hold A until g
 * is written.  p: [M, N/2] packed codes.  s: [M, N/16] E4M3 codes.  g: 1 FP32
 * (device), receives the global scale. */
lpq_status lpq_quantize_nvfp4(const uint16_t* w, int64_t M, int64_t N, const float* amax,
                              uint8_t* p, uint8_t* s, float* g, void* stream);

/* g: 1 FP32 (device), the global scale written by the quantizer. */
lpq_status lpq_dequantize_nvfp4(const uint8_t* p, const uint8_t* s, const float* g,
                                int64_t M, int64_t N, uint16_t* y, void* stream);

/* Fake quantization ("verl NVFP4 QAT" 2.3, also used on W4A4 activations):
 * y = dequantize(quantize(x)) bit for bit, without storing codes.
 * amax: 1 FP32 (device) holding A, or NULL: the tensor's own amax, computed
 * by the call.  The library allocates nothing, so between the amax pass and
 * the encode A is held in the first 4 bytes of y, which the last of the
 * call's four launches (the first 16-element block) overwrites with its
 * result; y is complete when the call's work on the stream is.
 * x, y: [M, N] BF16, and may not overlap (with amax NULL an overlap is
 * refused: LPQ_ERR_ARG). */
lpq_status lpq_nvfp4_qdq(const uint16_t* x, int64_t M, int64_t N, const float* amax,
                         uint16_t* y, void* stream);

/* ======================================================================== */
/* Grouped calls: one launch over many tensors (MoE experts, sibling groups).
 * Each call takes the same n descriptors twice: `host` (host memory, used to
 * validate every descriptor and size the launch) and `dev` (device memory,
 * read by the kernels).  The two must hold identical bytes.
 *
 *   call                        src            dst               scale
 *   quantize_fp8blk_grouped     BF16 [M,N]     codes [M,N]       FP32 tiles (out)
 *   dequantize_fp8blk_grouped   codes [M,N]    BF16 [M,N]        FP32 tiles (in)
 *   quantize_mxfp8_grouped      BF16           codes             uint8 [M,N/32] (out)
 *   dequantize_mxfp8_grouped    codes          BF16              uint8 (in)
 *   nvfp4_amax_grouped          BF16           unused            unused
 *   quantize_nvfp4_grouped      BF16           packed [M,N/2]    E4M3 [M,N/16] (out)
 *   dequantize_nvfp4_grouped    packed         BF16              E4M3 (in)
 *   nvfp4_qdq_grouped           BF16           BF16              unused
 * `group` is the NVFP4 sibling-group index of the tensor (q/k/v share one,
 * gate/up share one, a lone tensor has its own); other formats ignore it.
 * A call is split into one launch per run of up to 8 changes of tensor size:
 * placing tensors of equal shape next to each other (e.g. all experts of a
 * layer) keeps a call to a single launch.
 */
typedef struct lpq_tensor {
    const void* src;
    void* dst;
    void* scale;
    int64_t rows;      /* M */
    int64_t cols;      /* N */
    int32_t group;     /* NVFP4 sibling group, 0 <= group < n_groups */
    int32_t reserved;  /* must be 0 */
} lpq_tensor;

lpq_status lpq_quantize_fp8blk_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                       void* stream);
lpq_status lpq_dequantize_fp8blk_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                         void* stream);
lpq_status lpq_quantize_mxfp8_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                      void* stream);
lpq_status lpq_dequantize_mxfp8_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                        void* stream);

/* group_amax: n_groups FP32 (device).  accumulate == 0: the group slots are
 * first set to 0, then group_amax[group] = max over the group's members of
 * max |w|; accumulate != 0: max-accumulated into the existing values. */
lpq_status lpq_nvfp4_amax_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                  float* group_amax, int32_t n_groups, int accumulate, void* stream);

/* group_amax: n_groups FP32 (device), the A of each group.  amax_valid != 0:
 * group_amax already holds them (from lpq_nvfp4_amax_grouped, an observer or
 * a cached value, "verl NVFP4 QAT" 2.4) and is only read.  amax_valid == 0:
 * the call fills it first -- every slot set to 0, then each member's max |w|
 * max-folded into its group's slot (the group maximum) -- and then encodes;
 * the filled values stay there for the caller (e.g. to cache).  group_g:
 * n_groups FP32 (device, out): g of every group that has at least one
 * member. */
lpq_status lpq_quantize_nvfp4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                      float* group_amax, int32_t n_groups, int amax_valid, float* group_g,
                                      void* stream);

/* group_g: n_groups FP32 (device), the global scales written by the quantizer. */
lpq_status lpq_dequantize_nvfp4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                        const float* group_g, int32_t n_groups, void* stream);

/* group_amax, amax_valid: as for lpq_quantize_nvfp4_grouped.  src and dst of a
 * descriptor may not overlap. */
lpq_status lpq_nvfp4_qdq_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                 float* group_amax, int32_t n_groups, int amax_valid, void* stream);

/* ======================================================================== */
/* Re-quantization of block-wise FP8 weights, for the FP8-training weight
 * sync.  "低精度训练与 Rollout" (vime and slime documentation), section
 * "FP8 训练 + FP8 Rollout", implementation note 3: at a weight update the
 * trainer's FP8 weights go back to BF16 and are then quantized again for the
 * rollout engine.  These calls do both steps in one pass; the BF16 tensor
 * never reaches HBM.  Each result is bit-identical to lpq_dequantize_fp8blk
 * followed by the target format's quantizer (for NVFP4: the amax pass, then
 * lpq_quantize_nvfp4), applied to the dequantized BF16 values
 * y = BF16(fl(E4M3value(q) * s_tile)).
 *
 * Inputs: q, [M, N] E4M3 codes (never the NaN patterns 0x7F / 0xFF); s,
 * [ceil(M/128), ceil(N/128)] finite FP32 tile scales of either sign such that
 * every y is finite.  Outputs and their layouts are those of the target
 * format's quantizer. */

/* Grouped descriptor: both scale arrays are named. */
typedef struct lpq_requant_tensor {
    const uint8_t* src;        /* E4M3 codes [M, N] */
    const float* src_scale;    /* FP32 tile scales */
    void* dst;                 /* target codes: E4M3 [M, N] (block FP8, MXFP8) or NVFP4 packed [M, N/2] */
    void* dst_scale;           /* FP32 tile scales (block FP8), UE8M0 bytes [M, N/32] (MXFP8), or E4M3 block
                                  scales [M, N/16] (NVFP4) */
    int64_t rows;
    int64_t cols;
    int32_t group;             /* NVFP4 sibling group */
    int32_t reserved;          /* must be 0 */
} lpq_requant_tensor;

/* Block-wise FP8 -> block-wise FP8 (the page's own case).  Any M, N > 0; q and
 * q_out any alignment (16-byte aligned rows with N % 16 == 0 take the fast
 * path); s and s_out 4-byte aligned.  The new tile scale is fl(amax(y)/448). */
lpq_status lpq_requantize_fp8blk(const uint8_t* q, const float* s, int64_t M, int64_t N, uint8_t* q_out,
                                 float* s_out, void* stream);

/* The flat-target calls below need N % 32 == 0 (MXFP8) or N % 16 == 0 (amax,
 * NVFP4), and M, N < 2^31 - 4096, else LPQ_ERR_SHAPE.  Alignment: q 16 bytes,
 * MXFP8 q_out 16 bytes, NVFP4 p 8 bytes, FP32 arrays 4 bytes; scale-byte
 * arrays none. */
lpq_status lpq_requantize_fp8blk_mxfp8(const uint8_t* q, const float* s, int64_t M, int64_t N,
                                       uint8_t* q_out, uint8_t* e_out, void* stream);

/* max |y| of the dequantized tensor, max-accumulated into *amax when
 * accumulate != 0, else overwritten (1 FP32 on the device). */
lpq_status lpq_fp8blk_amax(const uint8_t* q, const float* s, int64_t M, int64_t N, float* amax,
                           int accumulate, void* stream);

/* amax: 1 FP32 (device) holding A of the sibling group of the dequantized
 * tensors.  p, sb, g as for lpq_quantize_nvfp4. */
lpq_status lpq_requantize_fp8blk_nvfp4(const uint8_t* q, const float* s, int64_t M, int64_t N,
                                       const float* amax, uint8_t* p, uint8_t* sb, float* g, void* stream);

/* Grouped forms, one launch per call where the work map allows (tensors of
 * equal size kept adjacent).  group_amax / group_g as for the NVFP4 grouped
 * calls; the amax call overwrites or max-accumulates as lpq_fp8blk_amax. */
lpq_status lpq_requantize_fp8blk_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev, int32_t n,
                                         void* stream);
lpq_status lpq_requantize_fp8blk_mxfp8_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev,
                                               int32_t n, void* stream);
lpq_status lpq_fp8blk_amax_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev, int32_t n,
                                   float* group_amax, int32_t n_groups, int accumulate, void* stream);
lpq_status lpq_requantize_fp8blk_nvfp4_grouped(const lpq_requant_tensor* host, const lpq_requant_tensor* dev,
                                               int32_t n, const float* group_amax, int32_t n_groups,
                                               float* group_g, void* stream);

/* Grouped form of lpq_quantize_mxfp8_floor (descriptors as for lpq_quantize_mxfp8_grouped). */
lpq_status lpq_quantize_mxfp8_floor_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, void* stream);

/* The NVFP4 global scale in its reciprocal form, out[i] = fl(2688 / A_i)
 * (correctly rounded; A_i = 0 gives +Inf), from the n_groups group amax
 * values (device, FP32).  "verl NVFP4 QAT" section 2.5: a compressed-tensors
 * export stores weight_global_scale in this form and fuses q/k/v and gate/up
 * by the minimum of it (the same value as the maximum amax).  Multiplying the
 * exported codes back needs the multiplier g of lpq_quantize_nvfp4*, which
 * is not 1/out[i] in general. */
lpq_status lpq_nvfp4_global_scale_reciprocal(const float* group_amax, int32_t n_groups, float* out, void* stream);

/* ======================================================================== */
/* NVFP4 with another E4M3 maximum in the global scale: g = fl(A / (6 *
 * e4m3_max)), e4m3_max 448 (the calls above) or 256, else LPQ_ERR_ARG.  The
 * vime pull request 503 review quotes a configuration where the NVFP4
 * "4over6" switch with its "E4M3 use 256" flag sets the E4M3 maximum to 256;
 * the global scale of "verl NVFP4 QAT" 2.3 divides amax by FP4 max x FP8 max.
 * Everything else is as for lpq_quantize_nvfp4 / lpq_nvfp4_qdq (and their
 * grouped forms: amax NULL, amax_valid); lpq_dequantize_nvfp4* decode the
 * output with the g it wrote.  The per-block choice between two scalings that gives "4over6" its
 * name is not described on the pages and is not implemented. */
lpq_status lpq_quantize_nvfp4_ex(const uint16_t* w, int64_t M, int64_t N, const float* amax, int e4m3_max,
                                 uint8_t* p, uint8_t* s, float* g, void* stream);
lpq_status lpq_nvfp4_qdq_ex(const uint16_t* x, int64_t M, int64_t N, const float* amax, int e4m3_max, uint16_t* y,
                            void* stream);
lpq_status lpq_quantize_nvfp4_grouped_ex(const lpq_tensor* host, const lpq_tensor* dev, int32_t n,
                                         float* group_amax, int32_t n_groups, int amax_valid, int e4m3_max,
                                         float* group_g, void* stream);
lpq_status lpq_nvfp4_qdq_grouped_ex(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, float* group_amax,
                                    int32_t n_groups, int amax_valid, int e4m3_max, void* stream);

/* ======================================================================== */
/* W4A4 activation observers.  "verl NVFP4 QAT" 2.2 (activation_observer,
 * default static_minmax, W4A4 mode only) and 3.1 (the choices static_minmax,
 * memoryless_minmax, minmax); the pages name them without defining them.
 * Readings: an observer tracks the activations' min and max per tensor --
 *   LPQ_OBSERVER_MEMORYLESS_MINMAX  the latest batch's extremes;
 *   LPQ_OBSERVER_STATIC_MINMAX      the extremes over every batch seen;
 *   LPQ_OBSERVER_MINMAX             a moving average, m = fl(m + fl(c * fl(b - m)))
 *                                   for each of min and max, c = averaging_constant;
 * the first batch after a reset initialises every kind.  The activation amax
 * is max(|min|, |max|); min and max order -0 below +0.
 *
 * state: LPQ_OBSERVER_STATE_FLOATS words of caller-owned device memory, 4-byte
 * aligned, one per observed tensor: [0] min, [1] max, [2] batches seen (FP32),
 * the rest lpq_nvfp4_observe's control words (on cache lines of their own: 512
 * bytes in all; lpq_nvfp4_observe_noalloc keeps them in the library and needs
 * the first 3 words only).  Reset it once before first use; calls
 * on one state must not overlap.  The amax feeds lpq_nvfp4_qdq (the W4A4
 * activation fake-quant) or lpq_nvfp4_global_scale[_reciprocal] (the exported
 * input_scale / input_global_scale). */
#define LPQ_OBSERVER_MEMORYLESS_MINMAX 0
#define LPQ_OBSERVER_STATIC_MINMAX 1
#define LPQ_OBSERVER_MINMAX 2
#define LPQ_OBSERVER_STATE_FLOATS 128

lpq_status lpq_observer_reset(float* state, void* stream);

/* Observe one BF16 batch x [M, N] (N % 16 == 0, x 16-byte aligned): updates
 * the state and writes the activation amax (1 FP32, device).  observer outside
 * the three kinds: LPQ_ERR_ARG. */
lpq_status lpq_nvfp4_observe(const uint16_t* x, int64_t M, int64_t N, int observer, float averaging_constant,
                             float* state, float* amax, void* stream);

/* For callers that cannot allocate device memory per observed tensor beyond
 * its statistics (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): lpq_nvfp4_observe with the call's control words (the
 * batch keys and the arrival counter) in a 512-byte block the library holds on
 * each device, instead of in the state.
 *   state: 3 FP32 words of caller-owned device memory, 4-byte aligned --
 *          [0] min, [1] max, [2] batches seen, as in lpq_nvfp4_observe's state
 *          (zero them, or lpq_observer_reset a full state, before first use);
 *          words past [2] are neither read nor written.
 *   Everything else (x, observer, averaging_constant, amax, the checks and
 *   their statuses) is as in lpq_nvfp4_observe; the control block is fixed
 *   in size, so the only size limit is that call's: M * N up to 2^40
 *   elements, LPQ_ERR_SHAPE beyond.
 * The block is re-armed by a one-workgroup kernel at the start of every call,
 * on the call's stream.  It is shared by every call of this function on one
 * device, and lives until the process ends: calls that overlap on one device
 * (two streams, two threads) race and give wrong statistics.  The first call
 * on a device looks up the block's address there (LPQ_ERR_HIP if that fails):
 * make one before capturing a graph that holds the call.  No call allocates
 * memory. */
lpq_status lpq_nvfp4_observe_noalloc(const uint16_t* x, int64_t M, int64_t N, int observer,
                                     float averaging_constant, float* state, float* amax, void* stream);

/* The multiplier form of a global scale, out[i] = fl(amax[i] / 2688), for n
 * device FP32 values (the input_scale / weight_scale_2 export of "verl NVFP4
 * QAT" 3.3). */
lpq_status lpq_nvfp4_global_scale(const float* amax, int32_t n, float* out, void* stream);

/* ======================================================================== */
/* Group-wise INT4.  "低精度训练与 Rollout" (vime and slime documentation),
 * "INT4 QAT 训练": INT4 weights for rollout and INT4 fake-quant training
 * through a straight-through estimator, with OPEN_TRAINING_INT4_GROUP_SIZE
 * 128 (Moonlight-16B-A3B, Qwen3-30B-A3B, Qwen3-235B-A22B) or 32
 * (Kimi-K2-Thinking).  The page fixes nothing else; readings:
 *   group  G = 32 or 128 consecutive elements of a row, N % G == 0
 *          (other group sizes: LPQ_ERR_ARG; N % G != 0: LPQ_ERR_SHAPE)
 *   s      = fl(amax / 7), amax = max |w| over the group (symmetric)
 *   code   = (s == 0) ? 0 : the integer nearest to fl(w / s), ties to even,
 *            clamped to [-8, 7] (finite inputs never reach the clamp)
 *   y      = BF16(fl(code * s))   (+0 for code 0: integers have no -0)
 * Packed layout: two's-complement nibbles, element 2j in the low nibble of
 * byte j.  p: [M, N/2] (4-byte aligned); s: [M, N/G] FP32 (4-byte aligned);
 * w, x, y: [M, N] BF16, 16-byte aligned. */
lpq_status lpq_quantize_int4(const uint16_t* w, int64_t M, int64_t N, int32_t group, uint8_t* p, float* s,
                             void* stream);
lpq_status lpq_dequantize_int4(const uint8_t* p, const float* s, int64_t M, int64_t N, int32_t group, uint16_t* y,
                               void* stream);

/* The straight-through estimator's forward pass: y = dequantize(quantize(x))
 * bit for bit, no codes stored.  x and y may not overlap. */
lpq_status lpq_int4_qdq(const uint16_t* x, int64_t M, int64_t N, int32_t group, uint16_t* y, void* stream);

/* Grouped forms (descriptors as for the NVFP4 grouped
 * calls: quantize {src = w, dst = p, scale = s}, dequantize {src = p, dst = y,
 * scale = s}, QDQ {src = x, dst = y, scale unused}; the group field is
 * ignored, reserved must be 0).  One group size per call. */
lpq_status lpq_quantize_int4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, int32_t group,
                                     void* stream);
lpq_status lpq_dequantize_int4_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, int32_t group,
                                       void* stream);
lpq_status lpq_int4_qdq_grouped(const lpq_tensor* host, const lpq_tensor* dev, int32_t n, int32_t group,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LPQ_H */
