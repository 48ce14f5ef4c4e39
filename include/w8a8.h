/*
 * w8a8.h — C ABI of libw8a8.so, the W8A8 quantized-verification hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (Quasar, arXiv 2603.01399, "Quasar: Quantized Self-Speculative
 * Acceleration for Rapid Inference via Memory-Efficient Verification"):
 * a drafter proposes a block of tokens and the target model checks the
 * whole block in one forward pass; Quasar runs that verification pass with
 * a W8A8 copy of the target — weights smoothed and quantized to INT8
 * offline, activations scaled by the smoothing factor and quantized to
 * INT8 at run time, an INT8 product accumulated in INT32, and a dequant
 * back to high precision before acceptance reads the logits.  Sources, cited
 * by page and section below:
 *   [de] gist.science German summary, "Technische Zusammenfassung";
 *   [it] gist.science Italian summary, "Sommario tecnico";
 *   [fr] gist.science French summary, "Résumé technique";
 *   [zh] shd-paper.top Chinese summary and its English abstract;
 *   [ja] gist.science Japanese summary, "技術的サマリー".
 *
 * Conventions for every call:
 *   - Tensor arguments are DEVICE pointers owned by the caller; the library
 *     never frees or keeps them.  Tensors are dense and row-major (last
 *     dimension contiguous).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue kernels on it and return without synchronizing; results
 *     are valid once the caller synchronizes the stream.  No call allocates
 *     device or host memory, and none keeps state between calls, so calls
 *     are thread-safe; calls that share a workspace must be ordered on one
 *     stream.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     rejected call enqueues nothing.  Device data is not validated: inputs
 *     must be finite (non-finite values give unspecified but in-range
 *     results, never an out-of-bounds access).
 *   - Nothing throws across the ABI.  A non-zero status names the failure;
 *     w8a8_last_error() returns a message for the calling thread's most
 *     recent failure.
 *   - Sizes are int64_t; M == 0, N == 0 or B == 0 makes the call a no-op
 *     that returns W8A8_OK (its pointers may then be NULL).  K == 0 is a
 *     valid empty contraction (zero products, zero scales).
 */
#ifndef W8A8_H
#define W8A8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t w8a8_status;

#define W8A8_OK              0  /* success */
#define W8A8_ERR_INVALID_ARG 1  /* NULL pointer, bad size, misalignment, K out of range */
#define W8A8_ERR_UNSUPPORTED 2  /* valid request the library does not handle */
#define W8A8_ERR_WORKSPACE   3  /* workspace NULL or smaller than the query says */
#define W8A8_ERR_HIP         4  /* the HIP runtime reported an error at launch */

/* Largest K for which |sum_k qx*qw| <= 127*127*K fits an int32 accumulator. */
#define W8A8_MAX_K 133144

/* ABI version of this header; w8a8_abi_version() returns the library's. */
#define W8A8_ABI_VERSION 1

int32_t     w8a8_abi_version(void);

/* Static text for a status code; never NULL. */
const char* w8a8_status_string(w8a8_status status);

/* Message describing the calling thread's most recent failure ("" if none).
 * The pointer stays valid until the thread's next call into the library. */
const char* w8a8_last_error(void);

/*
 * Per-token dynamic activation quantization, BF16 -> INT8.
 *
 * Pages: activations arrive in BF16, are scaled by the per-channel smoothing
 * factor s and converted to INT8 at run time ([ja] §2.2 item 3; [de] §2
 * "Online-Prozess"; [it] §2 pipeline "Inferenza Online"); the quantization
 * is symmetric and uniform ([it] §2 "Componenti Tecnici" 1).
 * Computes, for each row m (one token):
 *   x'[k]      = fp32(x[m][k]) * smooth[k]      (smooth == NULL: x' = fp32(x))
 *   amax       = max_k |x'[k]|
 *   x_scale[m] = amax / 127                     (correctly rounded fp32)
 *   inv        = 127 / amax                     (0 when amax == 0)
 *   xq[m][k]   = 0 if x'[k] == 0, else clamp(round_half_even(x'[k] * inv), -127, 127)
 * Every fp32 operation is a single correctly rounded operation; no fused
 * multiply-add.
 *
 * x_bf16   [M][K] bf16 bit patterns, 16-byte aligned.
 * smooth   [K] fp32, positive and finite, 16-byte aligned; or NULL.
 * xq       [M][K] int8 output, 16-byte aligned.
 * x_scale  [M] fp32 output.
 * Requires 0 <= K <= W8A8_MAX_K and K % 16 == 0.
 */
w8a8_status w8a8_quantize_act(const uint16_t* x_bf16, const float* smooth,
                              int64_t M, int64_t K,
                              int8_t* xq, float* x_scale, void* stream);

/*
 * Offline per-output-channel weight quantization, FP32 -> INT8.
 *
 * Pages: the weights are smoothed and quantized to INT8 ahead of inference
 * and kept in device memory ([ja] §2.2 item 2; [it] §2 pipeline
 * "Preparazione Offline"); smoothing divides the weights by s per input
 * channel, Y = (W diag(s)^-1)(diag(s) X) ([ja] §2.2 item 1).
 * Computes, for each output channel n (a row of W):
 *   w'[k]      = w[n][k] / smooth[k]            (smooth == NULL: w' = w)
 *   then the same rule as w8a8_quantize_act, giving wq[n][k] and w_scale[n].
 *
 * w        [N][K] fp32 (nn.Linear order: K contiguous), 16-byte aligned.
 * smooth   [K] fp32, positive and finite, 16-byte aligned; or NULL.
 * wq       [N][K] int8 output, 16-byte aligned.
 * w_scale  [N] fp32 output.
 * Requires 0 <= K <= W8A8_MAX_K and K % 16 == 0.
 */
w8a8_status w8a8_quantize_weight(const float* w, const float* smooth,
                                 int64_t N, int64_t K,
                                 int8_t* wq, float* w_scale, void* stream);

/*
 * Tiled weight layout (the layout the W8A8 linear streams fastest).
 *
 * The INT8 weights live in device memory for the life of the verifier
 * ([ja] §2.2 item 2), so their layout is chosen for the kernel: for each
 * tile of 16 output channels and each 64-wide k step, the 1 KiB that one
 * int8 MFMA consumes is stored contiguously in lane order.  With
 * steps = ceil(K/64), element (n, k) of the row-major [N][K] matrix is at
 * byte
 *   ((n/16 * steps + k/64) * 64 + (n%16 + 16*((k%64)/16))) * 16 + k%16
 * and every other byte (rows n >= N of the last tile, k >= K) is zero.
 * Size: w8a8_tiled_weight_bytes(N, K) = ceil(N/16)*16 * ceil(K/64)*64.
 *
 * w8a8_quantize_weight_tiled: same arithmetic and arguments as
 *   w8a8_quantize_weight, writing the codes in the tiled layout (wq_tiled,
 *   16-byte aligned, w8a8_tiled_weight_bytes(N, K) bytes, every byte
 *   written).
 * w8a8_tile_weight: rearranges row-major int8 wq [N][K] into the tiled
 *   layout (no arithmetic).  Requires K % 16 == 0, 16-byte aligned pointers.
 */
size_t      w8a8_tiled_weight_bytes(int64_t N, int64_t K);
w8a8_status w8a8_quantize_weight_tiled(const float* w, const float* smooth,
                                       int64_t N, int64_t K,
                                       int8_t* wq_tiled, float* w_scale, void* stream);
w8a8_status w8a8_tile_weight(const int8_t* wq, int64_t N, int64_t K,
                             int8_t* wq_tiled, void* stream);

/*
 * One W8A8 linear: INT8 x INT8 product with INT32 accumulation, then the
 * dequant epilogue.
 *
 * Pages: the product runs on INT8 matrix units and accumulates in INT32;
 * the result is dequantized to BF16 before the nonlinear layers ([ja] §2.2
 * item 3; [de] §2 "Online-Prozess" and "De-Quantisierung"; [it] §2 pipeline
 * "Calcolo" / "Dequantizzazione").
 * Computes, for m < M, n < N:
 *   acc[m][n]    = sum_k xq[m][k] * wq[n][k]                  (exact int32)
 *   y_f32[m][n]  = fp32(fp32(fp32(acc) * x_scale[m]) * w_scale[n])
 *   y_bf16[m][n] = bf16 round-half-even of y_f32[m][n]
 *
 * xq       [M][K] int8 (from w8a8_quantize_act), 16-byte aligned.
 * x_scale  [M] fp32.
 * wq       [N][K] int8 (from w8a8_quantize_weight), 16-byte aligned.
 * w_scale  [N] fp32.
 * y_bf16   [M][N] bf16 output, or NULL.
 * y_f32    [M][N] fp32 output, or NULL (the LM head's logits).
 * acc      [M][N] int32 output, or NULL.   At least one output is non-NULL.
 * workspace / workspace_bytes: device scratch of at least
 *          w8a8_linear_workspace_bytes(M, N, K) bytes (NULL allowed when that
 *          is 0), 256-byte aligned.  It holds the int32 partials and arrival
 *          counters of a reduction split across workgroups: up to 16 rows a
 *          long or narrow product, or only the 16-channel tiles past the last
 *          whole round over the compute units of a long one; above 16 rows
 *          (tiled weights, K % 64 == 0) a long one on a mid-size grid.  The workspace must be zero-filled
 *          before its first use; every completed call leaves it zero-filled
 *          again.  Calls that share a workspace must not overlap in time.
 * Requires 0 <= K <= W8A8_MAX_K, K % 16 == 0; any N (ragged tails are
 * handled); any M (M <= 16 takes the skinny kernel, larger M the batched one).
 */
size_t      w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);
w8a8_status w8a8_linear(const int8_t* xq, const float* x_scale,
                        const int8_t* wq, const float* w_scale,
                        int64_t M, int64_t N, int64_t K,
                        uint16_t* y_bf16, float* y_f32, int32_t* acc,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * w8a8_linear_tiled: w8a8_linear with the weights in the tiled layout
 * (wq_tiled from w8a8_quantize_weight_tiled or w8a8_tile_weight for the
 * same N and K).  Same results bit for bit; same workspace rule.
 */
w8a8_status w8a8_linear_tiled(const int8_t* xq, const float* x_scale,
                              const int8_t* wq_tiled, const float* w_scale,
                              int64_t M, int64_t N, int64_t K,
                              uint16_t* y_bf16, float* y_f32, int32_t* acc,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tiled activations for the batched product (more than 16 token rows, e.g.
 * 32 sequences x 9 verified positions).  w8a8_quantize_act_tiled computes
 * exactly w8a8_quantize_act's codes and scales and writes the codes in the
 * weights' tiled layout with token rows in place of channels
 * (w8a8_tiled_weight_bytes(M, K) bytes; padding rows and k zero).
 * w8a8_linear_tiled_act is w8a8_linear_tiled (bit-identical outputs) with
 * xq in that layout; loading one contiguous KiB per 16-row block and k step
 * instead of 16 rows x 64 bytes makes the batched product ~30% faster.
 * workspace / workspace_bytes: at least
 * w8a8_linear_tiled_act_workspace_bytes(M, N, K) bytes (NULL allowed when
 * that is 0; e.g. 288 x 4096 x 12288 needs ~9.4 MB), under w8a8_linear's
 * workspace rule (256-byte aligned, zero-filled before first use, left
 * zero-filled by every completed call, no overlapping calls); one buffer may
 * serve both.  Errors as for w8a8_linear.
 */
w8a8_status w8a8_quantize_act_tiled(const uint16_t* x_bf16, const float* smooth,
                                    int64_t M, int64_t K,
                                    int8_t* xq_tiled, float* x_scale, void* stream);
size_t      w8a8_linear_tiled_act_workspace_bytes(int64_t M, int64_t N, int64_t K);
w8a8_status w8a8_linear_tiled_act(const int8_t* xq_tiled, const float* x_scale,
                                  const int8_t* wq_tiled, const float* w_scale,
                                  int64_t M, int64_t N, int64_t K,
                                  uint16_t* y_bf16, float* y_f32, int32_t* acc,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * LM-head argmax and greedy acceptance of a draft block.
 *
 * Pages: the target verifies the drafted block in one pass and the
 * acceptance reads the dequantized, high-precision logits ([ja] §2.2
 * item 4; [it] §2 "Campionamento di rifiuto"); correct drafts are accepted
 * together and decoding restarts at the first wrong one ([fr] lay summary);
 * evaluation is greedy, T = 0 ([ja] §4).
 * Row b*(G+1)+i of `logits` is the target's prediction after position i of
 * sequence b.  Computes:
 *   argmax[r]      = lowest n with logits[r][n] == max_j logits[r][j]
 *   accept_len[b]  = number of leading i < G with draft[b][i] == argmax[b*(G+1)+i]
 *   next_token[b]  = argmax[b*(G+1) + accept_len[b]]
 * (tokens emitted by the step: accept_len + 1).  Draft ids outside [0, V)
 * never match.
 *
 * logits     [B*(G+1)][V] fp32, 4-byte aligned.
 * draft      [B][G] int32 (may be NULL when G == 0).
 * argmax     [B*(G+1)] int32 output, or NULL.
 * accept_len [B] int32 output;  next_token [B] int32 output.
 * workspace: at least w8a8_verify_accept_workspace_bytes(B, G, V) bytes.
 * Requires 0 <= G <= W8A8_MAX_DRAFT and 1 <= V < 2^31.
 */
#define W8A8_MAX_DRAFT 255
size_t      w8a8_verify_accept_workspace_bytes(int64_t B, int64_t G, int64_t V);
w8a8_status w8a8_verify_accept(const float* logits, int64_t V,
                               const int32_t* draft, int64_t B, int64_t G,
                               int32_t* argmax, int32_t* accept_len,
                               int32_t* next_token,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The LM-head verification in two kernels: the LM-head W8A8 linear (tiled
 * weights) whose epilogue also folds each row's maximum (value, lowest
 * index) into 64-bit keys (64 per row) with device-scope atomic max, then a
 * tiny acceptance kernel that reads, combines and resets the keys.  Same results, bit
 * for bit, as w8a8_linear_tiled(..., y_f32 = logits) followed by
 * w8a8_verify_accept; it saves the separate pass over the logits (and their
 * write, when logits == NULL).
 * xq [B*(G+1)][K], x_scale [B*(G+1)]: the quantized hidden states of the
 *    verified rows (row b*(G+1)+i as in w8a8_verify_accept).
 * wq_tiled / w_scale: the LM head [V][K] in the tiled layout and its scales.
 * logits [B*(G+1)][V] fp32 output, or NULL; argmax [B*(G+1)] output or NULL;
 * accept_len, next_token [B] outputs.  draft [B][G].
 * workspace: w8a8_lm_head_verify_workspace_bytes(B, G, V, K) bytes (16 KiB
 *    per verified row), 256-byte aligned.  It must be zero-filled before its
 *    first use; every completed call leaves it zero-filled again.  Calls that
 *    share a workspace must not overlap in time.
 * Requires 0 <= G <= W8A8_MAX_DRAFT, 1 <= V <= 2^30, K as for w8a8_linear.
 */
size_t      w8a8_lm_head_verify_workspace_bytes(int64_t B, int64_t G, int64_t V, int64_t K);

/*
 * Streaming-read probe (measurement): reads `bytes` bytes of `buf` once with
 * 16-byte non-temporal loads, each workgroup of 256 threads one contiguous
 * 32 KiB chunk (its four waves taking consecutive KiB in turn, eight loads
 * per lane in flight).  Its duration gives the read bandwidth this chip
 * sustains for a plain stream, the practical ceiling for a weight stream
 * next to the nominal peak.
 *
 * Pages: verification time is the weight bytes read over the memory
 * bandwidth ([de] §3 item 4; [ja] §2.3).
 *
 * buf: device buffer, 16-byte aligned; bytes % 16 == 0 (0 reads nothing).
 * sink: W8A8_HBM_PROBE_SINK_WORDS device uint32 (4-byte aligned) that the
 *    kernel may overwrite with a fold of the bytes read (the value has no
 *    use; it keeps the loads from being dropped).  start_event / stop_event:
 *    both NULL, or two hipEvent_t handles created with timing enabled that
 *    receive the kernel's own start and end timestamps (as for
 *    w8a8_lm_head_argmax_timed).  Errors: W8A8_ERR_INVALID_ARG for a NULL
 *    pointer, misalignment, a ragged size or one event without the other.
 */
#define W8A8_HBM_PROBE_SINK_WORDS 1
w8a8_status w8a8_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                void* start_event, void* stop_event, void* stream);

/* The two phases of w8a8_lm_head_verify, for callers that schedule (or time)
 * them apart.  w8a8_lm_head_argmax runs the LM-head linear for M = B*(G+1)
 * rows and folds the row maxima into the workspace keys; a following
 * w8a8_accept_from_keys on the same stream and workspace reads and resets
 * the keys and accepts the drafts.  Arguments as for w8a8_lm_head_verify. */
w8a8_status w8a8_lm_head_argmax(const int8_t* xq, const float* x_scale,
                                const int8_t* wq_tiled, const float* w_scale,
                                int64_t M, int64_t V, int64_t K, float* logits,
                                void* workspace, size_t workspace_bytes, void* stream);
/* w8a8_lm_head_argmax launched with hipExtLaunchKernel, which records the
 * LM-head kernel's own start and end timestamps into start_event and
 * stop_event (hipEvent_t handles the caller created with timing enabled):
 * hipEventElapsedTime(start, stop) is then that kernel's execution time as a
 * profiler's kernel trace reports it, and no marker packets are added to the
 * stream.  For measurement.  Results, arguments and errors as for
 * w8a8_lm_head_argmax; both events are required (W8A8_ERR_INVALID_ARG if
 * NULL); M <= 16 (W8A8_ERR_UNSUPPORTED above). */
w8a8_status w8a8_lm_head_argmax_timed(const int8_t* xq, const float* x_scale,
                                      const int8_t* wq_tiled, const float* w_scale,
                                      int64_t M, int64_t V, int64_t K, float* logits,
                                      void* workspace, size_t workspace_bytes,
                                      void* start_event, void* stop_event, void* stream);
/* w8a8_lm_head_argmax for many verified rows (e.g. 32 sequences x 9 = 288)
 * with the activations in the tiled layout of w8a8_quantize_act_tiled: the
 * batched product (the 32 x 32 MFMA pipeline where the grid is wide enough)
 * folds each row's maximum into the same workspace keys, so a following
 * w8a8_accept_from_keys accepts the drafts.  Results bit-identical to
 * w8a8_lm_head_argmax on the row-major codes.  Arguments, workspace and
 * errors as for w8a8_lm_head_argmax, with xq_tiled (w8a8_tiled_weight_bytes(M,
 * K) bytes, 16-byte aligned) in place of xq; any M >= 1. */
w8a8_status w8a8_lm_head_argmax_tiled_act(const int8_t* xq_tiled, const float* x_scale,
                                          const int8_t* wq_tiled, const float* w_scale,
                                          int64_t M, int64_t V, int64_t K, float* logits,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);
w8a8_status w8a8_accept_from_keys(void* workspace, size_t workspace_bytes,
                                  const int32_t* draft, int64_t B, int64_t G,
                                  int32_t* argmax, int32_t* accept_len,
                                  int32_t* next_token, void* stream);

w8a8_status w8a8_lm_head_verify(const int8_t* xq, const float* x_scale,
                                const int8_t* wq_tiled, const float* w_scale,
                                int64_t V, int64_t K,
                                const int32_t* draft, int64_t B, int64_t G,
                                float* logits, int32_t* argmax,
                                int32_t* accept_len, int32_t* next_token,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * w8a8_lm_head_verify for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same results, bit for bit, with no workspace argument.
 * The argmax keys live in a scratch array inside the library, one per GPU
 * (W8A8_NOALLOC_MAX_ROWS rows of 16 KiB: 4.5 MiB of device memory, held by
 * each GPU the library runs on until the process ends).  The call allocates
 * nothing: each call clears the keys its rows use with a small kernel (no
 * hipMemsetAsync), then runs the LM-head kernel and the acceptance kernel,
 * which leaves them zero.  The array's device address is looked up on the
 * first call on each device (make the stream's device current; make that
 * first call outside graph capture).  Every call on one GPU shares the
 * array: calls that overlap in time on one GPU (other streams, other
 * threads) race on it and must be serialized by the caller.
 *
 * Arguments and errors as for w8a8_lm_head_verify, without workspace and
 * workspace_bytes; B*(G+1) > W8A8_NOALLOC_MAX_ROWS returns
 * W8A8_ERR_UNSUPPORTED (nothing is enqueued).
 */
#define W8A8_NOALLOC_MAX_ROWS 288
w8a8_status w8a8_lm_head_verify_noalloc(const int8_t* xq, const float* x_scale,
                                        const int8_t* wq_tiled, const float* w_scale,
                                        int64_t V, int64_t K,
                                        const int32_t* draft, int64_t B, int64_t G,
                                        float* logits, int32_t* argmax,
                                        int32_t* accept_len, int32_t* next_token,
                                        void* stream);

/*
 * The BF16 glue between linears, fused with the per-token int8
 * quantization of the next linear's input (it replaces that
 * w8a8_quantize_act call).
 *
 * Pages: the INT32 results are dequantized to BF16 before the non-linear
 * layers, which run in high precision ([de] §2 "De-Quantisierung"; [it] §2
 * pipeline; [fr] §2; [ja] §2.2 item 3).  For the Qwen3 shapes: RMSNorm and
 * the SiLU-gated MLP.  Computes, per token row m (fp32 arithmetic, bf16 =
 * round to nearest even):
 *
 * w8a8_residual_rmsnorm_quant:
 *   h1 = bf16(h + delta) (h1 = h when delta == NULL), written to h_out
 *        (may equal h) when delta and h_out are given;
 *   r  = 1 / sqrt(sum_k h1^2 / D + eps)   (summation order unspecified);
 *   n  = bf16(bf16(h1 * r) * gamma), written to normed if not NULL;
 *   xq, x_scale = w8a8_quantize_act(n, smooth).
 * w8a8_silu_mul_quant:
 *   a  = bf16(bf16(g / (1 + exp(-g))) * u), g = gate[m][k], u = up[m][k]
 *        (rows row_stride elements apart: gate and up may be the two halves
 *        of a fused [gate;up] linear's output), written to act [M][F] if not
 *        NULL;
 *   xq, x_scale = w8a8_quantize_act(a, smooth).
 * The int8 codes are those w8a8_quantize_act gives for the bf16 row the
 * call produced (n or a), bit for bit.
 *
 * h, delta, h_out, normed [M][D] bf16; gamma [D] bf16; smooth [D] fp32 or
 * NULL; xq [M][D] int8; x_scale [M] fp32.  Pointers 16-byte aligned
 * (x_scale 4); 16 <= D <= W8A8_MAX_GLUE_WIDTH, D % 16 == 0; eps >= 0.
 */
#define W8A8_MAX_GLUE_WIDTH 32768
w8a8_status w8a8_residual_rmsnorm_quant(const uint16_t* h, const uint16_t* delta,
                                        const uint16_t* gamma, float eps,
                                        const float* smooth, int64_t M, int64_t D,
                                        uint16_t* h_out, uint16_t* normed,
                                        int8_t* xq, float* x_scale, void* stream);
w8a8_status w8a8_silu_mul_quant(const uint16_t* gate, const uint16_t* up,
                                int64_t row_stride, const float* smooth,
                                int64_t M, int64_t F, uint16_t* act,
                                int8_t* xq, float* x_scale, void* stream);

/*
 * The steps between the [q;k;v] linear and w8a8_verify_attention (Qwen3's
 * attention block; the pages do not describe it).  For token row (b, i) of
 * qkv [B*T][(Hq + 2*Hkv) * Dh] bf16 (heads of q, then k, then v) and
 * position p = L_b - T + i (L_b = lengths[b] clamped into [T, Lmax]):
 *   q, k heads: per-head RMSNorm over Dh with bf16 gammas
 *     n = bf16(bf16(x * r) * gamma), r = 1/sqrt(mean(x^2) + eps);
 *   then rotary embedding: dims (d, d + 64), d < 64, turned by the fp32
 *     angle fp32(fp32(p) * f_d), f_d = fp32(rope_base^(-d/64)) (computed on the
 *     host in double): (x1, x2) -> bf16(x1 cos - x2 sin), bf16(x2 cos + x1 sin);
 *   q goes to q_out [B][T][Hq][Dh]; k is written into k_cache
 *   [B][Hkv][Lmax][Dh] and v (unchanged) into the blocked v_cache (layout
 *   at w8a8_verify_attention) at position p.
 * fp32 arithmetic (sine and cosine of the fp32 angle in fp32).  Dh == 128
 * (else W8A8_ERR_UNSUPPORTED); Hq % Hkv == 0; T <= Lmax <= 131072 with
 * Lmax % 16 == 0; rope_base > 1; eps >= 0.
 */
w8a8_status w8a8_qk_norm_rope_append(const uint16_t* qkv, int64_t B, int64_t T,
                                     int64_t Hq, int64_t Hkv, int64_t Dh,
                                     const uint16_t* q_gamma, const uint16_t* k_gamma,
                                     float eps, float rope_base, const int32_t* lengths,
                                     int64_t Lmax, uint16_t* q_out, uint16_t* k_cache,
                                     uint16_t* v_cache, void* stream);

/*
 * Attention of the verified block over the KV cache (the softmax part of
 * the verifier, kept in high precision after the dequant step: [de] §2
 * "De-Quantisierung"; [it] §2 pipeline; [ja] §2.2 item 3).
 * For sequence b with L_b = lengths[b] valid cache positions, the last T of
 * which are the verified block's own keys and values, query i (0 <= i < T)
 * and head h read kv head h / (Hq / Hkv) and positions j <= L_b - T + i:
 *   out[b][i][h] = softmax_j(q[b][i][h] . k[b][kvh][j] / sqrt(Dh)) . v[b][kvh][j]
 * in fp32 (summation order unspecified), rounded to bf16.
 *
 * q [B][T][Hq][Dh], k_cache [B][Hkv][Lmax][Dh] (one row per position),
 * out [B][T][Hq][Dh], all bf16.  v_cache is bf16 in a blocked layout of
 * the same size: for each (b, kv head) a slab of Lmax * Dh elements in
 * blocks of 16 positions, position p and dim d at element
 *   (p / 16) * 2048 + ((p % 16 / 4) * 16 + d % 16) * 32 + (d / 16) * 4 + p % 4
 * of slab (b * Hkv + kvh) (w8a8_pack_v_cache converts a row-major cache;
 * w8a8_qk_norm_rope_append appends in this layout).  Positions >= L_b may
 * hold any bits.  q, k, v 16-byte aligned; lengths [B] int32 on the device
 * (values outside [T, Lmax] are clamped into it).  Requires Dh == 128
 * (else W8A8_ERR_UNSUPPORTED), Hq % Hkv == 0, T * Hq / Hkv <= 64,
 * T <= Lmax <= 131072, Lmax % 16 == 0.
 * workspace: at least w8a8_verify_attention_workspace_bytes(B, Hkv, Lmax)
 * bytes (0 for arguments out of range), 256-byte aligned; no initial
 * contents needed.
 */
size_t      w8a8_verify_attention_workspace_bytes(int64_t B, int64_t Hkv, int64_t Lmax);
w8a8_status w8a8_verify_attention(const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* lengths,
                                  int64_t B, int64_t T, int64_t Hq, int64_t Hkv,
                                  int64_t Dh, int64_t Lmax, uint16_t* out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Converts a row-major V cache v [B][Hkv][Lmax][Dh] bf16 into the blocked
 * layout w8a8_verify_attention reads (written to v_blocked, same size, not
 * overlapping v; 16-byte aligned).  A pure permutation of the bf16 values.
 * Dh == 128 (else W8A8_ERR_UNSUPPORTED); Lmax a multiple of 16 in
 * [16, 131072].
 */
w8a8_status w8a8_pack_v_cache(const uint16_t* v, int64_t B, int64_t Hkv, int64_t Lmax,
                              int64_t Dh, uint16_t* v_blocked, void* stream);

/*
 * W4A8: the verifier's weights in 4 bits (int4 codes, one fp32 scale per
 * output channel), activations as in W8A8.
 *
 * Pages: lower-bit verifiers, INT4 among them, are named as explored and as
 * the next step ([zh] 关键设计; [it] §5; [ja] §5); no scheme is given.
 * Reading: the int8 weight scheme with codes in [-7, 7]:
 *   w_scale[n] = fp32(amax_n / 7); q = clip(rint(fp32(w' * fp32(7/amax_n))), -7, 7)
 *   (w' = fp32(w / smooth[k]) when smooth != NULL; q = 0 where w' == 0),
 * and the same exact contraction and dequant as w8a8_linear:
 *   acc[m][n] = sum_k xq[m][k] * q[n][k]; y_f32 = fp32(fp32(acc * x_scale[m]) * w_scale[n]).
 *
 * Layout (int4 tiled, w8a8_w4_weight_bytes(N, K) bytes): per 16-channel tile
 * t and 128-wide k pair p, 1 KiB at offset (t * ceil(K/128) + p) * 1024;
 * lane l = (n % 16) + 16 * ((k % 64) / 16) owns bytes l*16 .. l*16+15: bytes
 * 0..7 for k % 128 < 64, bytes 8..15 for k % 128 >= 64.  With j = k % 16,
 * the code of (n, k) sits in byte (j % 4) of word (j / 4) % 2 of that
 * 8-byte half, in the low nibble for j < 8 and the high nibble for j >= 8;
 * codes are two's-complement nibbles, padding (n >= N, k >= K) is 0.
 *
 * w (fp32 [N][K]) and wq4 16-byte aligned; K % 16 == 0; K <= W8A8_MAX_K.
 */
size_t      w8a8_w4_weight_bytes(int64_t N, int64_t K);
w8a8_status w8a8_quantize_weight_w4(const float* w, const float* smooth,
                                    int64_t N, int64_t K,
                                    int8_t* wq4, float* w_scale, void* stream);

/*
 * The W4A8 linear: w8a8_linear's arguments and outputs with int4 tiled
 * weights (bit-exact int32 acc, fp32 y32, bf16 y).  No workspace.
 */
w8a8_status w8a8_linear_w4(const int8_t* xq, const float* x_scale,
                           const int8_t* wq4, const float* w_scale,
                           int64_t M, int64_t N, int64_t K,
                           uint16_t* y_bf16, float* y_f32, int32_t* acc,
                           void* stream);

/*
 * The W4A8 LM head with the row argmax folded into its epilogue, as
 * w8a8_lm_head_argmax (same key workspace; follow it with
 * w8a8_accept_from_keys).
 */
w8a8_status w8a8_lm_head_argmax_w4(const int8_t* xq, const float* x_scale,
                                   const int8_t* wq4, const float* w_scale,
                                   int64_t M, int64_t V, int64_t K,
                                   float* logits,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Stochastic verification at temperature T > 0: speculative sampling of a
 * block of single-token drafts on the fp32 dequantized logits.
 *
 * Pages: the logits are restored to high precision before softmax and the
 * rejection-sampling test, so the lossless guarantee of speculative decoding
 * holds ([de] §2 "De-Quantisierung"; [it] §2 item 3; [fr] §2
 * "Échantillonnage de rejet"; [ja] §2.2 item 4); T = 0 .. 1 ([de] §3,
 * [ja] §4).  The drafter's distribution at each position is taken to be a
 * point mass on its draft (N-gram or greedy self-drafting).  With rows laid
 * out as in w8a8_verify_accept, for each sequence b:
 *   p_i = softmax(logits[b*(G+1)+i] / T), in the exact fixed-point form
 *         below;
 *   positions i = 0..G-1 in order: accept draft[b][i] with probability
 *         p_i(draft), decided by u_accept[b][i]; stop at the first rejection;
 *   accept_len[b] = n, the number accepted;
 *   next_token[b] ~ p_n with draft[b][n] removed and renormalised when
 *         n < G, else ~ p_G; decided by u_sample[b].
 * Exact form (every step one IEEE fp32 operation, no contraction):
 *   m = max_j y_j; x_j = max(fp32(fp32(y_j - m) * fp32(1/T)), -32);
 *   e_j = exp_f32(x_j): k = rint(x*log2e), r = (x - k*ln2_hi) - k*ln2_lo,
 *         degree-7 Taylor polynomial in Horner form at r, times 2^k;
 *   W_j = floor(e_j * 2^40) (uint64), Z = sum_j W_j (exact);
 *   accept iff u_accept * Z < W(draft) * 2^32 (exact integer compare);
 *   next_token = first j whose inclusive prefix sum of W (draft removed)
 *         exceeds floor(u_sample * Z' / 2^64), Z' the total.
 * Draft ids outside [0, V) have weight 0: never accepted, nothing removed.
 * The same inputs give the same outputs on any device.
 *
 * logits     [B*(G+1)][V] fp32, finite, 4-byte aligned.
 * draft      [B][G] int32; u_accept [B][G] uint32 (both may be NULL when
 *            G == 0); u_sample [B] uint64, 8-byte aligned: uniform random
 *            words drawn by the caller.
 * accept_len [B], next_token [B] int32 outputs.
 * temperature: finite, > 0, with 1/T finite in fp32.
 * workspace: at least w8a8_verify_sample_workspace_bytes(B, G, V) bytes,
 *            256-byte aligned; no initial contents needed.
 * Requires 1 <= V <= W8A8_MAX_SAMPLE_VOCAB (sums of W stay below 2^63) and
 * 0 <= G <= W8A8_MAX_DRAFT.
 */
#define W8A8_MAX_SAMPLE_VOCAB (1 << 23)
size_t      w8a8_verify_sample_workspace_bytes(int64_t B, int64_t G, int64_t V);
w8a8_status w8a8_verify_sample(const float* logits, int64_t V,
                               const int32_t* draft, int64_t B, int64_t G,
                               float temperature, const uint32_t* u_accept,
                               const uint64_t* u_sample,
                               int32_t* accept_len, int32_t* next_token,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * The fixed-point softmax numerators W_j of w8a8_verify_sample for every
 * element of R rows: weights[r][j] = W_j of row r at temperature T (the
 * same kernels and values the sampler uses).
 * logits [R][V] fp32; weights [R][V] uint64 output, 8-byte aligned;
 * workspace: at least w8a8_sample_weights_workspace_bytes(R, V) bytes.
 */
size_t      w8a8_sample_weights_workspace_bytes(int64_t R, int64_t V);
w8a8_status w8a8_sample_weights(const float* logits, int64_t R, int64_t V,
                                float temperature, uint64_t* weights,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * The BF16 verifier's linear at the same shapes, as the weight-traffic
 * reference (BF16 weights move twice the bytes of INT8 ones: [zh] abstract;
 * [de] §3 item 4, latency M*2B/BW against M*1B/BW).
 * Computes y_f32[m][n] = sum_k x[m][k] * w[n][k] with bf16 operands and
 * fp32 accumulation (summation order unspecified), y_bf16 = its bf16
 * round-half-even.
 *
 * x_bf16 [M][K] and w_bf16 [N][K] bf16 bit patterns, 16-byte aligned.
 * y_bf16 [M][N] and/or y_f32 [M][N] outputs (at least one non-NULL).
 * Requires 0 <= K, K % 16 == 0, M <= 16.
 */
w8a8_status w8a8_bf16_linear(const uint16_t* x_bf16, const uint16_t* w_bf16,
                             int64_t M, int64_t N, int64_t K,
                             uint16_t* y_bf16, float* y_f32, void* stream);

/*
 * The same bf16 reference on tiled weights (the layout that lets every
 * weight load be one contiguous KiB, as for the W8A8 weights): element
 * (n, k) of w[N][K] at bf16 offset
 *   ((n/16 * steps + k/32) * 64 + (n%16 + 16*((k%32)/8))) * 8 + k%8,
 * steps = ceil(K/32), w8a8_bf16_tiled_weight_bytes(N, K) bytes in all, the
 * padding (n >= N, k >= K) zero.  w8a8_tile_weight_bf16 writes it from a
 * row-major w_bf16 (both 16-byte aligned; K % 16 == 0).
 * w8a8_bf16_linear_tiled: w8a8_bf16_linear's arguments, outputs and
 * requirements with w_tiled in that layout (the fp32 sums may differ from
 * w8a8_bf16_linear's in the last bits: another summation order).
 */
size_t      w8a8_bf16_tiled_weight_bytes(int64_t N, int64_t K);
w8a8_status w8a8_tile_weight_bf16(const uint16_t* w_bf16, int64_t N, int64_t K,
                                  uint16_t* w_tiled, void* stream);
w8a8_status w8a8_bf16_linear_tiled(const uint16_t* x_bf16, const uint16_t* w_tiled,
                                   int64_t M, int64_t N, int64_t K,
                                   uint16_t* y_bf16, float* y_f32, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
