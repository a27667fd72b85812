/*
 * mxq.h - C ABI of libmxq, the MI355X (gfx950) MX quantized linear.
 *
 * The operations follow the page "Quark Mixed-Precision Quantization for
 * Wan2.2 Video Generation on AMD Instinct GPUs":
 *   - section "Quantization formats": W4A4 = OCP MXFP4 weights with dynamic
 *     MXFP4 activations (the default, natively executed path); W4A8 = OCP
 *     MXFP4 weights with FP8 E4M3 activations (the promotion path);
 *   - section "Results" (rows marked RTN): weights are quantized by plain
 *     round-to-nearest;
 *   - section "Practical workflow" (step 6 and the paragraph after it): a
 *     per-expert, per-block policy artifact lets the runtime keep most blocks
 *     on W4A4 and spend W4A8 only on the blocks calibration flagged.
 *
 * Data formats:
 *   bf16 tensor      uint16 bit patterns, [rows][ld] with ld >= K, row-major.
 *   Code panels      MXFP4 codes are stored K-panel-major: K is cut into panels of
 *                    128 elements (the last one narrower, w = K - 128p, when
 *                    K % 128 != 0), and panel p holds every row's codes of
 *                    elements 128p .. 128p + w_p - 1, row after row. With B
 *                    bytes per element, element k of row r is at byte
 *                      128 p rows B + r w_p B + (k - 128 p) B,  p = k / 128.
 *                    The buffer has rows * K * B bytes, as a row-major one
 *                    would; a GEMM stage of 256 rows is then one contiguous
 *                    block (the pipelined GEMM copies it with 1 KiB loads).
 *   MXFP4 codes      B = 1/2, in code panels; element 2t of a row in the low
 *                    nibble of its byte, element 2t+1 in the high nibble.
 *                    Each nibble is E2M1 (sign bit 3; magnitudes 0, .5, 1,
 *                    1.5, 2, 3, 4, 6).
 *   MXFP4 scales     E8M0 bytes (value 2^(u-127)), one per 32 consecutive
 *                    elements along K, stored group-major as
 *                    uint8 [ceil(K/128)][rows][4]: the byte of row r, block j
 *                    (elements 32j .. 32j+31) is at ((j/4) * rows + r) * 4 +
 *                    j%4; bytes of blocks past K/32 are zero. One K stage of
 *                    a row tile is then one contiguous run (the GEMM copies
 *                    it with a few wide loads).
 *   FP8 codes        uint8 [M][K] row-major, E4M3FN (max 448, 0x7F/0xFF NaN).
 *                    (A GEMM stage already takes a full 128-byte line of each
 *                    FP8 row, so these stay row-major.)
 *   FP8 scales       float32 [M], one per row (token).
 *
 * Quantization rules:
 *   MXFP4 block: E = floor(log2 amax) - 2, clamped to [-127, 127]; an
 *     all-zero block has E = -127. code = E2M1 round-half-to-even of
 *     v / 2^E, saturating at +-6; the sign of v is kept (also for zeros).
 *   FP8 per token: s = fp32(amax) / 448 (IEEE fp32 division);
 *     code = E4M3FN round-half-to-even of the IEEE fp32 quotient x / s,
 *     saturating at +-448; a row of zeros has s = 0 and signed-zero codes.
 *   GEMM: y[m][n] = sum_k deqA[m][k] * deqW[n][k] accumulated in fp32, plus
 *     bias[n] (if given), optional tanh-GELU, rounded to bf16
 *     (round-half-to-even). For W4A8 the per-token scale multiplies the fp32
 *     sum of row m.
 *
 * Conventions of every entry point:
 *   - Device pointers are plain addresses in the current HIP device's memory;
 *     host pointers are marked as such. The caller owns every buffer and
 *     keeps it alive until the work on the stream has completed. The library
 *     allocates no device memory.
 *   - Work is only enqueued on `stream` (0 = the null stream); nothing
 *     synchronizes. Results are valid once the stream has reached that point.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is written. An empty problem (M == 0 or N == 0) enqueues
 *     nothing, returns MXQ_OK and accepts null pointers.
 *   - Device pointers must be 16-byte aligned and leading dimensions multiples
 *     of 8 elements (MXQ_ERR_ALIGN otherwise).
 *   - K must be a positive multiple of 32 (MXQ_ERR_SHAPE otherwise); sizes
 *     must stay below 2^31 elements per dimension and 2^31 rows.
 *   - Functions are thread-safe; calls that share output buffers must be
 *     ordered by the caller.
 *   - Inputs are assumed finite. With the environment variable
 *     MXQ_CHECK_FINITE set (not "0"), the entry points that read bf16
 *     activations or weights scan them before enqueueing anything and return
 *     MXQ_ERR_NONFINITE, writing nothing, when one holds an infinity or NaN;
 *     those that write bf16 outputs (mxq_gemm, mxq_lowrank_up,
 *     mxq_gemm_lowrank, and the quantized linears through them) scan the
 *     output afterwards and return MXQ_ERR_NONFINITE when it overflowed. Each
 *     scan synchronizes the stream: a debugging aid, the fail-closed guard
 *     the "Wan q8 performance investigation" page asks for after all-black
 *     outputs, not a mode for graph capture.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  MXQ_OK = 0,
  MXQ_ERR_NULL = 1,      /* a required pointer is null                      */
  MXQ_ERR_SHAPE = 2,     /* negative size, K not a positive multiple of 32,
                            ld < K, or a size beyond the supported range    */
  MXQ_ERR_ALIGN = 3,     /* device pointer not 16-byte aligned, or ld not a
                            multiple of 8                                   */
  MXQ_ERR_MODE = 4,      /* mode/epilogue not supported: W4A4 and W4A8 are
                            the quantized-linear modes (transform_on also a
                            policy entry); no silent fallback               */
  MXQ_ERR_WORKSPACE = 5, /* workspace missing or too small                  */
  MXQ_ERR_HIP = 6,       /* a HIP launch or runtime call failed             */
  MXQ_ERR_RANGE = 7,     /* policy index (expert, block) out of range       */
  MXQ_ERR_SCRATCH = 8,   /* problem too large for the allocation-free
                            scratch area (mxq_qlinear_noalloc)              */
  MXQ_ERR_NONFINITE = 9  /* MXQ_CHECK_FINITE: an input or output holds an
                            infinity or NaN                                 */
};

/* Precision modes: values of the policy table (the page's policy artifact,
 * "Practical workflow" step 6). MXQ_POLICY_TRANSFORM_ON is W4A4 with the
 * fixed Hadamard rotation + SmoothQuant transform ("Calibration-driven block
 * selection"): the policy accepts it, mxq_qlinear_transform runs it. The
 * artifact's "bf16" entry is not a mode of this layer (MXQ_ERR_MODE). */
enum { MXQ_W4A4 = 0, MXQ_W4A8 = 1, MXQ_POLICY_BF16 = 2, MXQ_POLICY_TRANSFORM_ON = 3 };

/* GEMM epilogues. The FFN's first projection is followed by tanh-GELU:
 * 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))). */
enum { MXQ_EPI_NONE = 0, MXQ_EPI_GELU_TANH = 1 };

/* Human-readable name of a status code (static string, never null). */
const char* mxq_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int mxq_version(void);

/*
 * Offline round-to-nearest MXFP4 weight packing (weights W [N][K] bf16,
 * nn.Linear layout) - the RTN weight quantization of the page's "Results"
 * table, in the MXFP4 format of "Quantization formats".
 *   w       device, bf16 [N][ldw]
 *   codes   device, uint8, N * K/2 bytes in code panels   (output)
 *   scales  device, uint8 [ceil(K/128)][N][4]  (output, E8M0, group-major)
 */
int mxq_quantize_weight_mxfp4(const void* w, int64_t N, int64_t K, int64_t ldw,
                              void* codes, void* scales, hipStream_t stream);

/*
 * Dynamic activation quantization ("Quantization formats"): MXQ_W4A4 gives
 * MXFP4 codes (M * K/2 bytes in code panels) + E8M0 scales [ceil(K/128)][M][4]
 * (group-major); MXQ_W4A8 gives E4M3FN codes [M][K] (row-major) + float32
 * per-token scales [M].
 *   x       device, bf16 [M][ldx]
 *   codes   device (output), scales device (output)
 */
int mxq_quantize_act(int mode, const void* x, int64_t M, int64_t K, int64_t ldx,
                     void* codes, void* scales, hipStream_t stream);

/*
 * Calibration for static FP8 activations. The page's format table calls the
 * W4A8 activations FP8 E4M3 "static", and its experimental setup runs a
 * calibration set (prompts x denoising steps) through the model: a static
 * scale is fixed from the largest activation magnitude seen there. This call
 * folds one calibration batch into a running maximum:
 *   *amax = max(*amax, max |x|)   over x [M][K] (bf16 [M][ldx], device)
 *   amax   device float32, one value; the caller sets it to 0 before the
 *          first batch and may call this any number of times (in any
 *          order: the result depends only on the set of batches). It is
 *          always the magnitude of one input element, exactly.
 * Finite inputs only (a NaN or infinity makes the result unspecified).
 */
int mxq_fp8_calibrate(const void* x, int64_t M, int64_t K, int64_t ldx, float* amax, hipStream_t stream);

/*
 * Static FP8 activation quantization (W4A8 with a calibrated per-tensor
 * scale): s = fp32(*amax) / 448 (IEEE), code = E4M3FN round-half-to-even of
 * the IEEE fp32 quotient x / s, saturating at +-448 (values past the
 * calibrated range clamp); *amax == 0 gives s = 0 and signed-zero codes.
 *   x       device, bf16 [M][ldx]
 *   amax    device float32 (e.g. from mxq_fp8_calibrate), finite, >= 0; read
 *           by the kernel, so it may be produced earlier on the same stream
 *   codes   device uint8 [M][K] E4M3FN (output)
 *   scales  device float32 [M] (output): s in every row, so the pair feeds
 *           mxq_gemm(MXQ_W4A8, ...) exactly as per-token activations do
 */
int mxq_quantize_act_fp8_static(const void* x, int64_t M, int64_t K, int64_t ldx, const float* amax,
                                void* codes, void* scales, hipStream_t stream);

/*
 * transform_on (sections "Calibration-driven block selection" and
 * "Mixed-Precision selection": fixed Hadamard rotation followed by
 * SmoothQuant, MXFP4 W4A4). For a linear y = x W^T the K dimension is rotated
 * by a block-diagonal Walsh-Hadamard matrix (one 128-point block per 128
 * consecutive elements, the MXFP4 code panel) and each channel is rescaled:
 *   x_t = (x H) / lambda (online),  W_t = (W H) * lambda (offline),
 * so x_t W_t^T = x W^T. The arithmetic is fp32 in a fixed order: the
 * unnormalized transform by butterflies (h = 1, 2, 4, ..., 64, each a + b and
 * a - b of the elements h apart), one multiply by the channel factor `mult`,
 * rounding to bf16, then the MXFP4 rule. K must be a multiple of 128.
 *
 * mxq_hadamard_channel_amax: SmoothQuant calibration statistic,
 *   amax[k] = max(amax[k], max over rows |unnormalized transform of x|[k])
 *   x      device bf16 [M][ldx]; amax device float32 [K], set to 0 by the
 *          caller before the first batch, then folded batch after batch (in
 *          any order). Use it on calibration activations, and on the bf16
 *          weight [N][K] for the weight's statistic.
 * mxq_smoothquant_factors: lambda = sqrt(act_amax / w_amax) (migration
 *   strength 0.5; 1 where either maximum is 0), then
 *   act_mult = RN(RN(1 / lambda) * c), w_mult = RN(lambda * c), c = RN(1 /
 *   sqrt(128)) (IEEE fp32 division and square root). All device float32 [K].
 * mxq_quantize_mxfp4_hadamard: MXFP4 codes (M * K/2 bytes in code panels) and
 *   E8M0 scales [K/128][M][4] of RN_bf16(transform(x) * mult). With act_mult
 *   it is the transform_on activation quantizer; with w_mult on the bf16
 *   weight [N][K] it packs the weight offline (use these codes with mxq_gemm(
 *   MXQ_W4A4, ...)). mult: device float32 [K], 16-byte aligned.
 * Finite inputs whose transform stays finite only.
 */
int mxq_hadamard_channel_amax(const void* x, int64_t M, int64_t K, int64_t ldx, float* amax, hipStream_t stream);
int mxq_smoothquant_factors(const float* act_amax, const float* w_amax, int64_t K, float* act_mult,
                            float* w_mult, hipStream_t stream);
int mxq_quantize_mxfp4_hadamard(const void* x, int64_t M, int64_t K, int64_t ldx, const float* mult,
                                void* codes, void* scales, hipStream_t stream);

/*
 * Calibration-driven block selection (section "Calibration-driven block
 * selection"): captured BF16 block inputs are replayed through two quantized
 * versions of each block, OFF = plain dynamic MXFP4 and ON = MXFP4 behind the
 * transform above, and the block output's SQNR against the captured BF16
 * output decides the block by a rule ladder with three tiers of thresholds.
 * A block here is its quantized linears; their outputs together are the
 * block output. SQNR = 10 log10(sum y_ref^2 / sum (y - y_ref)^2) dB.
 *
 * mxq_sqnr_accumulate: sums[0] += sum y_ref^2, sums[1] += sum (y - y_ref)^2
 *   over n elements of two bf16 device buffers (16-byte aligned), in fp64.
 *   sums: device double [2], set to 0 by the caller, then folded over any
 *   number of calls (the order of fp64 additions is not fixed).
 * mxq_block_replay_sqnr: one block's replay. For each linear, OFF quantizes
 *   x (mxq_quantize_act, MXQ_W4A4) and w (mxq_quantize_weight_mxfp4) and ON
 *   calibrates the transform on this x and w (mxq_hadamard_channel_amax,
 *   mxq_smoothquant_factors) and quantizes both with
 *   mxq_quantize_mxfp4_hadamard; both run mxq_gemm(MXQ_W4A4) into bf16 and
 *   fold their output against y_ref into sums_off / sums_on (device double
 *   [2] each, running). K % 128 == 0 for every linear. All inputs are
 *   validated before anything is enqueued; the linears run in order on
 *   `stream`, sharing the workspace (size from mxq_replay_workspace_bytes).
 *   linears is a host array.
 * mxq_policy_select: host only. From the host copies of per-block sums
 *   (double [n_experts][n_blocks][2] each) it writes the policy artifact
 *   modes [n_experts][n_blocks] (host): with best = max(SQNR_off, SQNR_on),
 *   best < floor -> MXQ_POLICY_BF16; best < w4a8 -> MXQ_W4A8;
 *   SQNR_on - SQNR_off > margin -> MXQ_POLICY_TRANSFORM_ON; else MXQ_W4A4.
 *   Tiers (floor, w4a8, margin) in dB: low (8, 21, 0.5), mid (10, 23, 0.5),
 *   high (12, 25, 0.5). No noise counts as +inf dB, no signal as -inf.
 */
enum { MXQ_TIER_LOW = 0, MXQ_TIER_MID = 1, MXQ_TIER_HIGH = 2 };
typedef struct mxq_replay_linear {
  const void* x;     /* device bf16 [M][K]: the captured input */
  const void* w;     /* device bf16 [N][K]: the linear's weight */
  const void* y_ref; /* device bf16 [M][N]: the captured BF16 output */
  int64_t M, N, K;
} mxq_replay_linear;
int mxq_sqnr_accumulate(const void* y, const void* y_ref, int64_t n, double* sums, hipStream_t stream);
int mxq_replay_workspace_bytes(const mxq_replay_linear* linears, int32_t n_linears, size_t* bytes);
int mxq_block_replay_sqnr(const mxq_replay_linear* linears, int32_t n_linears, void* workspace,
                          size_t workspace_bytes, double* sums_off, double* sums_on, hipStream_t stream);
int mxq_policy_select(const double* sums_off, const double* sums_on, int32_t n_experts, int32_t n_blocks,
                      int32_t tier, uint8_t* modes);

/*
 * SVDQuant's low-rank branch (the SVDQuant transform of sections
 * "Mixed-Precision selection" and "Results"): for a weight W ~ L2 L1^T + R of
 * rank r, the residual R is packed as MXFP4 like any weight and the layer is
 *   y = epilogue( Q(x) Q(R)^T + bias + (x L1) L2^T' )
 * with the branch in bf16 beside the quantized product. Run as: mxq_gemm
 * (or mxq_qlinear) with MXQ_EPI_NONE into y_pre (the GELU must follow the
 * whole sum), mxq_lowrank_down, then mxq_lowrank_up with the linear's
 * epilogue.
 * mxq_lowrank_down: t [M][r] = RN_bf16(x L1), fp32 accumulation.
 *   x    device bf16 [M][K] (dense), K a multiple of 128
 *   l1t  device bf16 [r][K]: L1 transposed (one rank vector per row)
 *   r    32, 64, 96 or 128
 *   t    device bf16 [M][r] (output)
 * mxq_lowrank_up: y [M][N] = RN_bf16(epilogue(y_pre + t L2^T)), fp32.
 *   y_pre device bf16 [M][N] (dense), N a multiple of 32
 *   l2    device bf16 [N][r] (one rank vector per output column)
 *   y     device bf16 [M][N] (output; may be y_pre itself)
 * All pointers 16-byte aligned.
 */
int mxq_lowrank_down(const void* x, int64_t M, int64_t K, const void* l1t, int64_t r, void* t, hipStream_t stream);
/*
 * mxq_quantize_act_lowrank: mxq_quantize_act(MXQ_W4A4, x, M, K, ldx = K, codes,
 *   scales) and mxq_lowrank_down(x, M, K, l1t, r, t) in one pass over x: the
 *   same codes and scales byte for byte, the same t. For a linear whose
 *   activation and branch both come from x (the quantizer and the branch's
 *   first half each read it whole). Arguments as for those two calls; K a
 *   multiple of 128; codes M * K/2 bytes, scales [K/128][M][4].
 */
int mxq_quantize_act_lowrank(const void* x, int64_t M, int64_t K, const void* l1t, int64_t r, void* codes,
                             void* scales, void* t, hipStream_t stream);
int mxq_lowrank_up(const void* y_pre, const void* t, const void* l2, int64_t M, int64_t N, int64_t r,
                   int epilogue, void* y, hipStream_t stream);

/*
 * SVDQuant's branch inside the W4A4 GEMM (same sections): the second half of
 * the branch joins the quantized product's fp32 sums, and the output is
 * rounded once,
 *   y [M][N] = RN_bf16(epilogue( sum_k deqA[m][k] deqR[n][k]
 *                                + sum_j t[m][j] l2[n][j] + bias[n] )),
 * with deqR the packed residual weight. Unlike mxq_gemm + mxq_lowrank_up it
 * does not round the quantized product to bf16 before the branch is added,
 * and it reads and writes the output once. Run mxq_lowrank_down first.
 *   a_codes/a_scales  device, from mxq_quantize_act(MXQ_W4A4, ...)
 *   w_codes/w_scales  device, the residual from mxq_quantize_weight_mxfp4
 *   bias              device bf16 [N], or null for none
 *   t                 device bf16 [M][r] (mxq_lowrank_down's output)
 *   l2                device bf16 [N][r]
 *   r                 32, 64, 96 or 128
 *   y_scales null:    y is device bf16 [M][N] (output)
 *   y_scales given:   y and y_scales are the MXFP4 activation of a next W4A4
 *                     layer, as mxq_gemm_mxfp4_out writes them (its shapes:
 *                     N a multiple of 128), of the bf16 values above
 * Only for the shapes of the pipelined kernel (mxq_gemm_kernel_name(MXQ_W4A4,
 * M, N, K) starts with "pipe_"): MXQ_ERR_SHAPE otherwise, and nothing is
 * written (use mxq_gemm and mxq_lowrank_up). All pointers 16-byte aligned.
 */
int mxq_gemm_lowrank(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                     const void* bias, const void* t, const void* l2, int64_t r, int epilogue, void* y,
                     void* y_scales, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Scaled GEMM on quantized operands (the native MXFP4 / W4A8 execution of
 * "Quantization formats", kernel note): y [M][N] bf16 =
 *   epilogue( sum_k deqA[m][k] deqW[n][k] + bias[n] ).
 *   a_codes/a_scales  device, from mxq_quantize_act(mode, ...)
 *   w_codes/w_scales  device, from mxq_quantize_weight_mxfp4
 *   bias              device bf16 [N], or null for none
 *   y                 device bf16 [M][N] (output, dense)
 */
int mxq_gemm(int mode, const void* a_codes, const void* a_scales,
             const void* w_codes, const void* w_scales, const void* bias,
             int epilogue, void* y, int64_t M, int64_t N, int64_t K,
             hipStream_t stream);

/*
 * W4A4 GEMM whose output is the W4A4 activation of a next layer: the FFN of a
 * W4A4 block takes the first projection (with tanh-GELU), quantizes the
 * hidden state to MXFP4 ("Quantization formats") and feeds it to the second
 * projection. This entry point does the first two in one kernel, without the
 * bf16 hidden state in memory. The result is exactly that of mxq_gemm(
 * MXQ_W4A4, ...) into a bf16 [M][N] buffer followed by mxq_quantize_act(
 * MXQ_W4A4, that buffer): the same bf16 values, quantized by the same rule.
 *   a_codes/a_scales  device, from mxq_quantize_act(MXQ_W4A4, ...)
 *   w_codes/w_scales  device, from mxq_quantize_weight_mxfp4
 *   bias              device bf16 [N], or null for none
 *   y_codes           device uint8, M * N/2 bytes in code panels (output;
 *                     its K is N)
 *   y_scales          device uint8 [N/128][M][4] (output)
 * Only for the shapes of the pipelined kernel (mxq_gemm_kernel_name(MXQ_W4A4,
 * M, N, K) starts with "pipe_") with N a multiple of 128 and M * N/2 below
 * 2^31 - 256: MXQ_ERR_SHAPE otherwise, and nothing is written (use mxq_gemm
 * and mxq_quantize_act).
 */
int mxq_gemm_mxfp4_out(const void* a_codes, const void* a_scales,
                       const void* w_codes, const void* w_scales, const void* bias,
                       int epilogue, void* y_codes, void* y_scales,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * The same for a next layer that runs transform_on (sections "Mixed-Precision
 * selection" and "Calibration-driven block selection": fixed Hadamard
 * rotation and SmoothQuant in front of the MXFP4 W4A4 linear): the FFN of a
 * transform_on block quantizes its hidden state with the second projection's
 * rotation and factors. The result is exactly that of mxq_gemm(MXQ_W4A4, ...)
 * into a bf16 [M][N] buffer followed by mxq_quantize_mxfp4_hadamard(that
 * buffer, mult): the same bf16 values, rotated and rescaled in the same fp32
 * order, quantized by the same rule; the hidden state never goes to memory.
 *   mult              device float32 [N], 16-byte aligned: the second
 *                     projection's act_mult (mxq_smoothquant_factors over
 *                     its K = N)
 *   other arguments   as for mxq_gemm_mxfp4_out
 * Same shapes as mxq_gemm_mxfp4_out (N a multiple of 128, the transform's
 * panel width): MXQ_ERR_SHAPE otherwise, and nothing is written. Finite
 * values whose transform stays finite only.
 */
int mxq_gemm_mxfp4_hadamard_out(const void* a_codes, const void* a_scales,
                                const void* w_codes, const void* w_scales, const void* bias,
                                int epilogue, const float* mult, void* y_codes, void* y_scales,
                                int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * W4A8 GEMM whose output is the static FP8 activation of a next W4A8 layer:
 * the FFN of a W4A8 block takes the first projection (with tanh-GELU),
 * quantizes the hidden state with its calibrated static scale (the FP8 E4M3
 * static activations of "Quantization formats") and feeds it to the second
 * projection. With a static scale no amax pass over the hidden state is
 * needed, so this entry point does the first two in one kernel. The result
 * is exactly that of mxq_gemm(MXQ_W4A8, ...) into a bf16 [M][N] buffer
 * followed by mxq_quantize_act_fp8_static(that buffer, out_amax).
 *   a_codes/a_scales  device, W4A8 activations (per-token or static scales)
 *   w_codes/w_scales  device, from mxq_quantize_weight_mxfp4
 *   bias              device bf16 [N], or null for none
 *   out_amax          device float32, the output's calibrated amax (>= 0)
 *   y_codes           device uint8 [M][N] E4M3FN (output)
 *   y_scales          device float32 [M] (output): out_amax / 448 in every row
 * Only for the shapes of the pipelined kernel (mxq_gemm_kernel_name(MXQ_W4A8,
 * M, N, K) starts with "pipe_") with N a multiple of 32 (N is the next
 * layer's K): MXQ_ERR_SHAPE otherwise, and nothing is written.
 */
int mxq_gemm_fp8_static_out(const void* a_codes, const void* a_scales,
                            const void* w_codes, const void* w_scales, const void* bias,
                            int epilogue, const float* out_amax, void* y_codes, void* y_scales,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Conversion between the library's MXFP4 layouts (code panels, group-major
 * scales; see "Data formats" above) and the canonical row-major layout of the
 * OCP MXFP4 format ("Quantization formats": OCP MXFP4, the page's reference
 * [7]): codes [rows][K/2] bytes with element 2t of a row in the low nibble of
 * byte t, and E8M0 scales [rows][K/32] bytes, one per 32 consecutive
 * elements of a row. The bytes themselves are unchanged; only their places
 * move.
 *   mxq_mxfp4_to_canonical: codes (M * K/2 bytes in code panels) and scales
 *     ([ceil(K/128)][rows][4]) -> codes_rm [rows][K/2], scales_rm [rows][K/32].
 *     Use it to hand the output of mxq_quantize_weight_mxfp4,
 *     mxq_quantize_act(MXQ_W4A4, ...) or mxq_gemm_mxfp4_out to code that
 *     expects the OCP layout.
 *   mxq_mxfp4_from_canonical: the inverse; the padding bytes of the last
 *     scale group (blocks past K/32) are written as zero. Use it to feed
 *     MXFP4 weights or activations held in the OCP layout to mxq_gemm.
 * All four buffers are device memory owned by the caller, 16-byte aligned,
 * and must not overlap; K is a positive multiple of 32 (MXQ_ERR_SHAPE
 * otherwise). rows == 0 enqueues nothing. Errors are detected before anything
 * is enqueued, so nothing is written on an error.
 */
int mxq_mxfp4_to_canonical(const void* codes, const void* scales, int64_t rows, int64_t K, void* codes_rm,
                           void* scales_rm, hipStream_t stream);
int mxq_mxfp4_from_canonical(const void* codes_rm, const void* scales_rm, int64_t rows, int64_t K, void* codes,
                             void* scales, hipStream_t stream);

/*
 * Name of the kernel that mxq_gemm runs for (mode, M, N, K), as a static
 * string: "pipe_..." for the LDS-pipelined persistent kernel (M, N >= 256,
 * N a multiple of 8, K a multiple of 128 with at least one ring of stages,
 * the activation codes and the packed weight each below 2^31 bytes; the
 * output may be larger), "direct_..." for the register-tiled kernel,
 * "invalid" for a mode that is
 * not W4A4 or W4A8. Host only: enqueues nothing, never fails.
 */
const char* mxq_gemm_kernel_name(int mode, int64_t M, int64_t N, int64_t K);

/*
 * Per-expert, per-block policy table ("Practical workflow", step 6).
 *   modes   host, uint8 [n_experts][n_blocks]; each entry MXQ_W4A4, MXQ_W4A8
 *           or MXQ_POLICY_TRANSFORM_ON (run by mxq_qlinear_transform);
 *           anything else, MXQ_POLICY_BF16 included, is MXQ_ERR_MODE (with
 *           MXQ_LOG set, the first offending (expert, block) is printed).
 *           A table written by mxq_policy_select may hold MXQ_POLICY_BF16
 *           entries: those blocks stay in bf16 outside this library, and the
 *           caller replaces their entries (by any quantized mode, never
 *           read for them) before creating the policy. Copied; the caller
 *           may free it after the call.
 *   policy  host, receives an opaque handle owned by the caller, released
 *           with mxq_policy_destroy.
 */
int mxq_policy_create(const uint8_t* modes, int32_t n_experts, int32_t n_blocks, void** policy);
int mxq_policy_destroy(void* policy);
/* Mode of (expert, block): MXQ_ERR_RANGE when out of range. mode: host out. */
int mxq_policy_mode(const void* policy, int32_t expert, int32_t block, int* mode);

/* Workspace bytes mxq_qlinear needs for the activation codes and scales of
 * an [M][K] input in `mode` (bytes: host out). */
int mxq_qlinear_workspace_bytes(int mode, int64_t M, int64_t K, size_t* bytes);

/*
 * One quantized linear layer: looks up the mode of (expert, block) in the
 * policy, quantizes x into the workspace with that mode's activation format,
 * then runs the scaled GEMM into y. Exactly mxq_quantize_act followed by
 * mxq_gemm.
 *   x          device bf16 [M][K] (dense)
 *   w_codes    device uint8, N * K/2 bytes in code panels, w_scales device uint8 [ceil(K/128)][N][4]
 *   bias       device bf16 [N] or null
 *   y          device bf16 [M][N] (output)
 *   workspace  device, at least mxq_qlinear_workspace_bytes(mode, M, K)
 */
int mxq_qlinear(const void* policy, int32_t expert, int32_t block,
                const void* x, int64_t M, int64_t K,
                const void* w_codes, const void* w_scales, int64_t N,
                const void* bias, int epilogue, void* y,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mxq_qlinear without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The activation codes and scales go to a scratch area of
 * MXQ_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends (a static device array; nothing is allocated). The
 * first call on a device looks up that device's address of the array (a host
 * call with no stream work): make one call there before capturing a graph; a
 * call with M == 0 does only that.
 *   Limits: mxq_qlinear_workspace_bytes(mode, M, K) <= MXQ_NOALLOC_SCRATCH_BYTES
 *   (64 MiB: e.g. M * K <= 126 M elements for W4A4, 67 M for W4A8), else
 *   MXQ_ERR_SCRATCH and nothing is written.
 *   Concurrency: every call on a device uses that device's one scratch area,
 *   so calls that overlap on one device (other streams, other threads) race;
 *   calls ordered on one stream do not. The area keeps the last call's
 *   activation codes (each call overwrites what it reads).
 * Otherwise exactly mxq_qlinear (same arguments without the workspace, same
 * validation, same kernels and results).
 */
#define MXQ_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int mxq_qlinear_noalloc(const void* policy, int32_t expert, int32_t block,
                        const void* x, int64_t M, int64_t K,
                        const void* w_codes, const void* w_scales, int64_t N,
                        const void* bias, int epilogue, void* y, hipStream_t stream);

/*
 * mxq_qlinear for tables that hold MXQ_POLICY_TRANSFORM_ON blocks. A
 * transform_on block quantizes x with mxq_quantize_mxfp4_hadamard(act_mult)
 * and multiplies with the weight packed by the same call on w_mult; its
 * workspace is the W4A4 one. Other blocks ignore act_mult and behave as
 * mxq_qlinear. (mxq_qlinear itself returns MXQ_ERR_MODE on a transform_on
 * block: it has no factors for it.)
 *   act_mult  device float32 [K] (16-byte aligned); required (MXQ_ERR_NULL)
 *             on a transform_on block; K a multiple of 128 there.
 */
int mxq_qlinear_transform(const void* policy, int32_t expert, int32_t block,
                          const void* x, int64_t M, int64_t K,
                          const void* w_codes, const void* w_scales, int64_t N,
                          const void* bias, int epilogue, const float* act_mult, void* y,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
