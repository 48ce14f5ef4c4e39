// C ABI of libw8a8.so: argument validation, workspace checks, error
// reporting, and dispatch to the kernel launchers.  Declarations and the
// contract of each call are in include/w8a8.h.
#include "../../include/w8a8.h"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_last_error;

w8a8_status fail(w8a8_status s, const char* fn, const char* what) {
  g_last_error = std::string(fn) + ": " + what;
  return s;
}

w8a8_status hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return W8A8_OK;
  g_last_error = std::string(fn) + ": HIP error: " + hipGetErrorString(e);
  return W8A8_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxRows = int64_t(1) << 30;    // token rows / output channels
constexpr int64_t kMaxVocab = (int64_t(1) << 31) - 1;

// Common checks on an [R][K] quantization problem.
w8a8_status check_rows_k(const char* fn, int64_t R, int64_t K) {
  if (R < 0 || R > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "row count out of range");
  if (K < 0 || K > W8A8_MAX_K) return fail(W8A8_ERR_INVALID_ARG, fn, "K out of range [0, 133144]");
  if (K % 16 != 0) return fail(W8A8_ERR_INVALID_ARG, fn, "K must be a multiple of 16");
  return W8A8_OK;
}

}  // namespace

extern "C" {

int32_t w8a8_abi_version(void) { return W8A8_ABI_VERSION; }

const char* w8a8_status_string(w8a8_status s) {
  switch (s) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_INVALID_ARG: return "invalid argument";
    case W8A8_ERR_UNSUPPORTED: return "unsupported";
    case W8A8_ERR_WORKSPACE: return "workspace missing or too small";
    case W8A8_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* w8a8_last_error(void) { return g_last_error.c_str(); }

w8a8_status w8a8_quantize_act(const uint16_t* x_bf16, const float* smooth, int64_t M, int64_t K,
                              int8_t* xq, float* x_scale, void* stream) {
  static const char* fn = "w8a8_quantize_act";
  g_last_error.clear();
  if (w8a8_status s = check_rows_k(fn, M, K)) return s;
  if (M == 0) return W8A8_OK;
  if (!x_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "x_scale is NULL");
  if (K > 0 && (!x_bf16 || !xq)) return fail(W8A8_ERR_INVALID_ARG, fn, "x_bf16 or xq is NULL");
  if (!aligned(x_bf16, 16) || !aligned(xq, 16) || !aligned(smooth, 16) || !aligned(x_scale, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (16 bytes for tensors, 4 for scales)");
  return hip_status(w8a8_launch_quantize_rows(x_bf16, true, smooth, false, M, K, false, xq,
                                              x_scale, reinterpret_cast<hipStream_t>(stream)), fn);
}

static w8a8_status quantize_weight_common(const char* fn, const float* w, const float* smooth,
                                          int64_t N, int64_t K, bool tiled, int8_t* wq,
                                          float* w_scale, void* stream) {
  g_last_error.clear();
  if (w8a8_status s = check_rows_k(fn, N, K)) return s;
  if (N == 0) return W8A8_OK;
  if (!w_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "w_scale is NULL");
  if (K > 0 && (!w || !wq)) return fail(W8A8_ERR_INVALID_ARG, fn, "w or wq is NULL");
  if (!aligned(w, 16) || !aligned(wq, 16) || !aligned(smooth, 16) || !aligned(w_scale, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (16 bytes for tensors, 4 for scales)");
  return hip_status(w8a8_launch_quantize_rows(w, false, smooth, true, N, K, tiled, wq, w_scale,
                                              reinterpret_cast<hipStream_t>(stream)), fn);
}

w8a8_status w8a8_quantize_weight(const float* w, const float* smooth, int64_t N, int64_t K,
                                 int8_t* wq, float* w_scale, void* stream) {
  return quantize_weight_common("w8a8_quantize_weight", w, smooth, N, K, false, wq, w_scale,
                                stream);
}

size_t w8a8_tiled_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N > kMaxRows || K > W8A8_MAX_K) return 0;
  return w8a8_tiled_weight_bytes_impl(N, K);
}

w8a8_status w8a8_quantize_weight_tiled(const float* w, const float* smooth, int64_t N, int64_t K,
                                       int8_t* wq_tiled, float* w_scale, void* stream) {
  return quantize_weight_common("w8a8_quantize_weight_tiled", w, smooth, N, K, true, wq_tiled,
                                w_scale, stream);
}

w8a8_status w8a8_tile_weight(const int8_t* wq, int64_t N, int64_t K, int8_t* wq_tiled,
                             void* stream) {
  static const char* fn = "w8a8_tile_weight";
  g_last_error.clear();
  if (w8a8_status s = check_rows_k(fn, N, K)) return s;
  if (N == 0 || K == 0) return W8A8_OK;
  if (!wq || !wq_tiled) return fail(W8A8_ERR_INVALID_ARG, fn, "wq or wq_tiled is NULL");
  if (!aligned(wq, 16) || !aligned(wq_tiled, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "wq and wq_tiled must be 16-byte aligned");
  return hip_status(w8a8_launch_tile_weight(wq, N, K, wq_tiled,
                                            reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t w8a8_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || M > kMaxRows || N > kMaxRows || K < 0 || K > W8A8_MAX_K) return 0;
  const size_t a = w8a8_gemm_workspace_bytes(M, N, K, false);
  const size_t b = w8a8_gemm_workspace_bytes(M, N, K, true);
  return a > b ? a : b;
}

static w8a8_status linear_common(const char* fn, const int8_t* xq, const float* x_scale,
                                 const int8_t* wq, const float* w_scale, int64_t M, int64_t N,
                                 int64_t K, bool tiled, uint16_t* y_bf16, float* y_f32,
                                 int32_t* acc, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  g_last_error.clear();
  if (w8a8_status s = check_rows_k(fn, M, K)) return s;
  if (N < 0 || N > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "N out of range");
  if (M == 0 || N == 0) return W8A8_OK;
  if (!y_bf16 && !y_f32 && !acc) return fail(W8A8_ERR_INVALID_ARG, fn, "all outputs are NULL");
  if (!x_scale || !w_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "x_scale or w_scale is NULL");
  if (K > 0 && (!xq || !wq)) return fail(W8A8_ERR_INVALID_ARG, fn, "xq or wq is NULL");
  if (!aligned(xq, 16) || !aligned(wq, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "xq and wq must be 16-byte aligned");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(y_bf16, 2) || !aligned(y_f32, 4) ||
      !aligned(acc, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "scale or output pointer misaligned");
  const size_t need = w8a8_gemm_workspace_bytes(M, N, K, tiled);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_linear_workspace_bytes()");
  if (need > 0 && !aligned(workspace, 256))
    return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_gemm(xq, x_scale, wq, w_scale, M, N, K, tiled, y_bf16, y_f32, acc,
                                     workspace, reinterpret_cast<hipStream_t>(stream)), fn);
}

w8a8_status w8a8_linear(const int8_t* xq, const float* x_scale, const int8_t* wq,
                        const float* w_scale, int64_t M, int64_t N, int64_t K, uint16_t* y_bf16,
                        float* y_f32, int32_t* acc, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return linear_common("w8a8_linear", xq, x_scale, wq, w_scale, M, N, K, false, y_bf16, y_f32,
                       acc, workspace, workspace_bytes, stream);
}

w8a8_status w8a8_linear_tiled(const int8_t* xq, const float* x_scale, const int8_t* wq_tiled,
                              const float* w_scale, int64_t M, int64_t N, int64_t K,
                              uint16_t* y_bf16, float* y_f32, int32_t* acc, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return linear_common("w8a8_linear_tiled", xq, x_scale, wq_tiled, w_scale, M, N, K, true, y_bf16,
                       y_f32, acc, workspace, workspace_bytes, stream);
}

size_t w8a8_verify_accept_workspace_bytes(int64_t B, int64_t G, int64_t V) {
  if (B <= 0 || G < 0 || G > W8A8_MAX_DRAFT || V <= 0 || V > kMaxVocab || B > kMaxRows) return 0;
  return w8a8_argmax_workspace_bytes(B * (G + 1), V);
}

w8a8_status w8a8_verify_accept(const float* logits, int64_t V, const int32_t* draft, int64_t B,
                               int64_t G, int32_t* argmax, int32_t* accept_len,
                               int32_t* next_token, void* workspace, size_t workspace_bytes,
                               void* stream) {
  static const char* fn = "w8a8_verify_accept";
  g_last_error.clear();
  if (B < 0 || B > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "B out of range");
  if (G < 0 || G > W8A8_MAX_DRAFT) return fail(W8A8_ERR_INVALID_ARG, fn, "G out of range [0, 255]");
  if (B == 0) return W8A8_OK;
  if (V < 1 || V > kMaxVocab) return fail(W8A8_ERR_INVALID_ARG, fn, "V out of range [1, 2^31)");
  if ((B * (G + 1)) * ((V + 4095) / 4096) > kMaxVocab)
    return fail(W8A8_ERR_INVALID_ARG, fn, "too many logits rows for one launch");
  if (!logits || !accept_len || !next_token || (G > 0 && !draft))
    return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(logits, 4) || !aligned(draft, 4) || !aligned(argmax, 4) ||
      !aligned(accept_len, 4) || !aligned(next_token, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (4 bytes)");
  const size_t need = w8a8_argmax_workspace_bytes(B * (G + 1), V);
  if (!workspace || workspace_bytes < need)
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_verify_accept_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_verify_accept(logits, V, draft, B, G, argmax, accept_len,
                                              next_token, workspace,
                                              reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t w8a8_lm_head_verify_workspace_bytes(int64_t B, int64_t G, int64_t V, int64_t K) {
  if (B <= 0 || G < 0 || G > W8A8_MAX_DRAFT || V <= 0 || V > kMaxRows || B > kMaxRows ||
      K < 0 || K > W8A8_MAX_K)
    return 0;
  return w8a8_lm_head_workspace_bytes(B * (G + 1));
}

// The LM-head operands (everything but the key workspace).
static w8a8_status check_lm_head_operands(const char* fn, const int8_t* xq, const float* x_scale,
                                          const int8_t* wq_tiled, const float* w_scale, int64_t M,
                                          int64_t V, int64_t K, const float* logits) {
  if (w8a8_status s = check_rows_k(fn, M, K)) return s;
  if (M == 0) return W8A8_OK;
  if (V < 1 || V > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "V out of range [1, 2^30]");
  if (!x_scale || !w_scale || (K > 0 && (!xq || !wq_tiled)))
    return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(xq, 16) || !aligned(wq_tiled, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "xq and wq_tiled must be 16-byte aligned");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(logits, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (4 bytes)");
  return W8A8_OK;
}

static w8a8_status check_lm_head(const char* fn, const int8_t* xq, const float* x_scale,
                                 const int8_t* wq_tiled, const float* w_scale, int64_t M,
                                 int64_t V, int64_t K, const float* logits, const void* keys,
                                 size_t keys_bytes) {
  if (w8a8_status s = check_lm_head_operands(fn, xq, x_scale, wq_tiled, w_scale, M, V, K, logits))
    return s;
  if (M == 0) return W8A8_OK;
  if (!keys || keys_bytes < w8a8_lm_head_workspace_bytes(M))
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_lm_head_verify_workspace_bytes()");
  if (!aligned(keys, 256)) return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return W8A8_OK;
}

static w8a8_status check_accept_keys(const char* fn, const int32_t* draft, int64_t B, int64_t G,
                                     const int32_t* argmax, const int32_t* accept_len,
                                     const int32_t* next_token) {
  if (B < 0 || B > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "B out of range");
  if (G < 0 || G > W8A8_MAX_DRAFT) return fail(W8A8_ERR_INVALID_ARG, fn, "G out of range [0, 255]");
  if (B == 0) return W8A8_OK;
  if (!accept_len || !next_token || (G > 0 && !draft))
    return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(draft, 4) || !aligned(argmax, 4) || !aligned(accept_len, 4) || !aligned(next_token, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (4 bytes)");
  return W8A8_OK;
}

w8a8_status w8a8_lm_head_argmax(const int8_t* xq, const float* x_scale, const int8_t* wq_tiled,
                                const float* w_scale, int64_t M, int64_t V, int64_t K,
                                float* logits, void* workspace, size_t workspace_bytes,
                                void* stream) {
  static const char* fn = "w8a8_lm_head_argmax";
  g_last_error.clear();
  if (w8a8_status s = check_lm_head(fn, xq, x_scale, wq_tiled, w_scale, M, V, K, logits,
                                    workspace, workspace_bytes))
    return s;
  if (M == 0) return W8A8_OK;
  return hip_status(w8a8_launch_lm_head_argmax(xq, x_scale, wq_tiled, w_scale, M, V, K, logits,
                                               workspace, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

w8a8_status w8a8_lm_head_argmax_timed(const int8_t* xq, const float* x_scale,
                                      const int8_t* wq_tiled, const float* w_scale, int64_t M,
                                      int64_t V, int64_t K, float* logits, void* workspace,
                                      size_t workspace_bytes, void* start_event,
                                      void* stop_event, void* stream) {
  static const char* fn = "w8a8_lm_head_argmax_timed";
  g_last_error.clear();
  if (w8a8_status s = check_lm_head(fn, xq, x_scale, wq_tiled, w_scale, M, V, K, logits,
                                    workspace, workspace_bytes))
    return s;
  if (!start_event || !stop_event)
    return fail(W8A8_ERR_INVALID_ARG, fn, "start_event and stop_event are required");
  if (M > 16) return fail(W8A8_ERR_UNSUPPORTED, fn, "kernel timestamps are taken for M <= 16 only");
  if (M == 0) return W8A8_OK;
  return hip_status(w8a8_launch_lm_head_argmax(xq, x_scale, wq_tiled, w_scale, M, V, K, logits,
                                               workspace, reinterpret_cast<hipStream_t>(stream),
                                               reinterpret_cast<hipEvent_t>(start_event),
                                               reinterpret_cast<hipEvent_t>(stop_event)),
                    fn);
}

w8a8_status w8a8_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* start_event,
                                void* stop_event, void* stream) {
  static const char* fn = "w8a8_hbm_read_probe";
  g_last_error.clear();
  if (bytes % 16 != 0) return fail(W8A8_ERR_INVALID_ARG, fn, "bytes must be a multiple of 16");
  if (!sink || (bytes > 0 && !buf)) return fail(W8A8_ERR_INVALID_ARG, fn, "buf or sink is NULL");
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (16 bytes for buf, 4 for sink)");
  if (!start_event != !stop_event)
    return fail(W8A8_ERR_INVALID_ARG, fn, "pass both events or neither");
  if (bytes / 16 / 2048 >= (size_t)INT32_MAX)
    return fail(W8A8_ERR_INVALID_ARG, fn, "bytes too large for one launch");
  return hip_status(w8a8_launch_hbm_read_probe(buf, bytes, sink,
                                               reinterpret_cast<hipStream_t>(stream),
                                               reinterpret_cast<hipEvent_t>(start_event),
                                               reinterpret_cast<hipEvent_t>(stop_event)),
                    fn);
}

w8a8_status w8a8_accept_from_keys(void* workspace, size_t workspace_bytes, const int32_t* draft,
                                  int64_t B, int64_t G, int32_t* argmax, int32_t* accept_len,
                                  int32_t* next_token, void* stream) {
  static const char* fn = "w8a8_accept_from_keys";
  g_last_error.clear();
  if (w8a8_status s = check_accept_keys(fn, draft, B, G, argmax, accept_len, next_token)) return s;
  if (B == 0) return W8A8_OK;
  if (!workspace || workspace_bytes < w8a8_lm_head_workspace_bytes(B * (G + 1)))
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_lm_head_verify_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_accept_from_keys(workspace, draft, B, G, argmax, accept_len,
                                                 next_token, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

w8a8_status w8a8_lm_head_verify(const int8_t* xq, const float* x_scale, const int8_t* wq_tiled,
                                const float* w_scale, int64_t V, int64_t K, const int32_t* draft,
                                int64_t B, int64_t G, float* logits, int32_t* argmax,
                                int32_t* accept_len, int32_t* next_token, void* workspace,
                                size_t workspace_bytes, void* stream) {
  static const char* fn = "w8a8_lm_head_verify";
  g_last_error.clear();
  if (w8a8_status s = check_accept_keys(fn, draft, B, G, argmax, accept_len, next_token)) return s;
  if (B == 0) return W8A8_OK;
  if (w8a8_status s = check_lm_head(fn, xq, x_scale, wq_tiled, w_scale, B * (G + 1), V, K, logits,
                                    workspace, workspace_bytes))
    return s;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (w8a8_status s = hip_status(w8a8_launch_lm_head_argmax(xq, x_scale, wq_tiled, w_scale,
                                                            B * (G + 1), V, K, logits, workspace,
                                                            st), fn))
    return s;
  return hip_status(w8a8_launch_accept_from_keys(workspace, draft, B, G, argmax, accept_len,
                                                 next_token, st), fn);
}

w8a8_status w8a8_lm_head_verify_noalloc(const int8_t* xq, const float* x_scale,
                                        const int8_t* wq_tiled, const float* w_scale, int64_t V,
                                        int64_t K, const int32_t* draft, int64_t B, int64_t G,
                                        float* logits, int32_t* argmax, int32_t* accept_len,
                                        int32_t* next_token, void* stream) {
  static const char* fn = "w8a8_lm_head_verify_noalloc";
  g_last_error.clear();
  if (w8a8_status s = check_accept_keys(fn, draft, B, G, argmax, accept_len, next_token)) return s;
  if (B == 0) return W8A8_OK;
  if (B * (G + 1) > W8A8_NOALLOC_MAX_ROWS)
    return fail(W8A8_ERR_UNSUPPORTED, fn,
                "B*(G+1) exceeds W8A8_NOALLOC_MAX_ROWS (288 rows of argmax keys in the library's "
                "scratch array); use w8a8_lm_head_verify with a workspace");
  if (w8a8_status s = check_lm_head_operands(fn, xq, x_scale, wq_tiled, w_scale, B * (G + 1), V, K,
                                             logits))
    return s;
  return hip_status(w8a8_launch_lm_head_verify_noalloc(xq, x_scale, wq_tiled, w_scale, V, K, draft,
                                                       B, G, logits, argmax, accept_len,
                                                       next_token,
                                                       reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

w8a8_status w8a8_bf16_linear(const uint16_t* x_bf16, const uint16_t* w_bf16, int64_t M, int64_t N,
                             int64_t K, uint16_t* y_bf16, float* y_f32, void* stream) {
  static const char* fn = "w8a8_bf16_linear";
  g_last_error.clear();
  if (M < 0 || N < 0 || N > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "M or N out of range");
  if (M > 16) return fail(W8A8_ERR_UNSUPPORTED, fn, "the bf16 reference handles M <= 16");
  if (K < 0 || K > (int64_t(1) << 24) || K % 16 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "K must be a multiple of 16 in [0, 2^24]");
  if (M == 0 || N == 0) return W8A8_OK;
  if (!y_bf16 && !y_f32) return fail(W8A8_ERR_INVALID_ARG, fn, "all outputs are NULL");
  if (K > 0 && (!x_bf16 || !w_bf16)) return fail(W8A8_ERR_INVALID_ARG, fn, "x_bf16 or w_bf16 is NULL");
  if (!aligned(x_bf16, 16) || !aligned(w_bf16, 16) || !aligned(y_bf16, 2) || !aligned(y_f32, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned");
  return hip_status(w8a8_launch_bf16_gemm(x_bf16, w_bf16, M, N, K, y_bf16, y_f32,
                                          reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t w8a8_bf16_tiled_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || N > kMaxRows || K <= 0 || K > (int64_t(1) << 24)) return 0;
  return w8a8_bf16_tiled_weight_bytes_impl(N, K);
}

w8a8_status w8a8_tile_weight_bf16(const uint16_t* w_bf16, int64_t N, int64_t K, uint16_t* w_tiled,
                                  void* stream) {
  static const char* fn = "w8a8_tile_weight_bf16";
  g_last_error.clear();
  if (N < 0 || N > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "N out of range");
  if (K < 0 || K > (int64_t(1) << 24) || K % 16 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "K must be a multiple of 16 in [0, 2^24]");
  if (N == 0 || K == 0) return W8A8_OK;
  if (!w_bf16 || !w_tiled) return fail(W8A8_ERR_INVALID_ARG, fn, "w_bf16 or w_tiled is NULL");
  if (!aligned(w_bf16, 16) || !aligned(w_tiled, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "w_bf16 and w_tiled must be 16-byte aligned");
  return hip_status(w8a8_launch_tile_bf16(w_bf16, N, K, w_tiled, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

w8a8_status w8a8_bf16_linear_tiled(const uint16_t* x_bf16, const uint16_t* w_tiled, int64_t M,
                                   int64_t N, int64_t K, uint16_t* y_bf16, float* y_f32,
                                   void* stream) {
  static const char* fn = "w8a8_bf16_linear_tiled";
  g_last_error.clear();
  if (M < 0 || N < 0 || N > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "M or N out of range");
  if (M > 16) return fail(W8A8_ERR_UNSUPPORTED, fn, "the bf16 reference handles M <= 16");
  if (K < 0 || K > (int64_t(1) << 24) || K % 16 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "K must be a multiple of 16 in [0, 2^24]");
  if (M == 0 || N == 0) return W8A8_OK;
  if (!y_bf16 && !y_f32) return fail(W8A8_ERR_INVALID_ARG, fn, "all outputs are NULL");
  if (K > 0 && (!x_bf16 || !w_tiled)) return fail(W8A8_ERR_INVALID_ARG, fn, "x_bf16 or w_tiled is NULL");
  if (!aligned(x_bf16, 16) || !aligned(w_tiled, 16) || !aligned(y_bf16, 2) || !aligned(y_f32, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned");
  return hip_status(w8a8_launch_bf16_gemm_tiled(x_bf16, w_tiled, M, N, K, y_bf16, y_f32,
                                                reinterpret_cast<hipStream_t>(stream)), fn);
}


// ---- stochastic verification (T > 0) ----

static w8a8_status check_sample_common(const char* fn, const float* logits, int64_t R, int64_t V,
                                       float temperature, float* inv_t) {
  if (V < 1 || V > W8A8_MAX_SAMPLE_VOCAB)
    return fail(W8A8_ERR_INVALID_ARG, fn, "V out of range [1, 2^23]");
  if (R * ((V + 2047) / 2048) > INT32_MAX)
    return fail(W8A8_ERR_INVALID_ARG, fn, "too many logits rows for one launch");
  if (!(std::isfinite(temperature) && temperature > 0.0f))
    return fail(W8A8_ERR_INVALID_ARG, fn, "temperature must be finite and > 0");
  const float inv = 1.0f / temperature;   // one correctly rounded fp32 division
  if (!std::isfinite(inv)) return fail(W8A8_ERR_INVALID_ARG, fn, "1/temperature overflows fp32");
  if (!logits) return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(logits, 4)) return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (4 bytes)");
  *inv_t = inv;
  return W8A8_OK;
}

size_t w8a8_sample_weights_workspace_bytes(int64_t R, int64_t V) {
  if (R <= 0 || R > kMaxRows || V <= 0 || V > W8A8_MAX_SAMPLE_VOCAB) return 0;
  return w8a8_sample_workspace_bytes_impl(R, V);
}

w8a8_status w8a8_sample_weights(const float* logits, int64_t R, int64_t V, float temperature,
                                uint64_t* weights, void* workspace, size_t workspace_bytes,
                                void* stream) {
  static const char* fn = "w8a8_sample_weights";
  g_last_error.clear();
  if (R < 0 || R > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "R out of range");
  if (R == 0) return W8A8_OK;
  float inv_t = 0.0f;
  if (w8a8_status st = check_sample_common(fn, logits, R, V, temperature, &inv_t)) return st;
  if (!weights) return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(weights, 8)) return fail(W8A8_ERR_INVALID_ARG, fn, "weights must be 8-byte aligned");
  if (!workspace || workspace_bytes < w8a8_sample_workspace_bytes_impl(R, V))
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_sample_weights_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_sample_weights(logits, R, V, inv_t, weights, workspace,
                                               reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t w8a8_verify_sample_workspace_bytes(int64_t B, int64_t G, int64_t V) {
  if (B <= 0 || B > kMaxRows || G < 0 || G > W8A8_MAX_DRAFT || V <= 0 ||
      V > W8A8_MAX_SAMPLE_VOCAB)
    return 0;
  return w8a8_sample_workspace_bytes_impl(B * (G + 1), V);
}

w8a8_status w8a8_verify_sample(const float* logits, int64_t V, const int32_t* draft, int64_t B,
                               int64_t G, float temperature, const uint32_t* u_accept,
                               const uint64_t* u_sample, int32_t* accept_len,
                               int32_t* next_token, void* workspace, size_t workspace_bytes,
                               void* stream) {
  static const char* fn = "w8a8_verify_sample";
  g_last_error.clear();
  if (B < 0 || B > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "B out of range");
  if (G < 0 || G > W8A8_MAX_DRAFT) return fail(W8A8_ERR_INVALID_ARG, fn, "G out of range [0, 255]");
  if (B == 0) return W8A8_OK;
  float inv_t = 0.0f;
  if (w8a8_status st = check_sample_common(fn, logits, B * (G + 1), V, temperature, &inv_t))
    return st;
  if (!u_sample || !accept_len || !next_token || (G > 0 && (!draft || !u_accept)))
    return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(draft, 4) || !aligned(u_accept, 4) || !aligned(accept_len, 4) ||
      !aligned(next_token, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (4 bytes)");
  if (!aligned(u_sample, 8)) return fail(W8A8_ERR_INVALID_ARG, fn, "u_sample must be 8-byte aligned");
  if (!workspace || workspace_bytes < w8a8_sample_workspace_bytes_impl(B * (G + 1), V))
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_verify_sample_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_verify_sample(logits, V, draft, B, G, inv_t, u_accept, u_sample,
                                              accept_len, next_token, workspace,
                                              reinterpret_cast<hipStream_t>(stream)), fn);
}


// ---- W4A8: int4 per-channel weights ----

size_t w8a8_w4_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N > kMaxRows || K > W8A8_MAX_K) return 0;
  return w8a8_w4_weight_bytes_impl(N, K);
}

w8a8_status w8a8_quantize_weight_w4(const float* w, const float* smooth, int64_t N, int64_t K,
                                    int8_t* wq4, float* w_scale, void* stream) {
  static const char* fn = "w8a8_quantize_weight_w4";
  g_last_error.clear();
  if (w8a8_status s = check_rows_k(fn, N, K)) return s;
  if (N == 0) return W8A8_OK;
  if (!w_scale || (K > 0 && (!w || !wq4)))
    return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(w, 16) || !aligned(wq4, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "w and wq4 must be 16-byte aligned");
  if (!aligned(smooth, 4) || !aligned(w_scale, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "smooth or w_scale misaligned");
  return hip_status(w8a8_launch_quantize_w4(w, smooth, N, K, wq4, w_scale,
                                            reinterpret_cast<hipStream_t>(stream)), fn);
}

static w8a8_status check_w4(const char* fn, const int8_t* xq, const float* x_scale,
                            const int8_t* wq4, const float* w_scale, int64_t M, int64_t N,
                            int64_t K) {
  if (w8a8_status s = check_rows_k(fn, M, K)) return s;
  if (N < 0 || N > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "N out of range");
  if (M == 0 || N == 0) return W8A8_OK;
  if (!x_scale || !w_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "x_scale or w_scale is NULL");
  if (K > 0 && (!xq || !wq4)) return fail(W8A8_ERR_INVALID_ARG, fn, "xq or wq4 is NULL");
  if (!aligned(xq, 16) || !aligned(wq4, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "xq and wq4 must be 16-byte aligned");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "scale pointer misaligned");
  return W8A8_OK;
}

w8a8_status w8a8_linear_w4(const int8_t* xq, const float* x_scale, const int8_t* wq4,
                           const float* w_scale, int64_t M, int64_t N, int64_t K,
                           uint16_t* y_bf16, float* y_f32, int32_t* acc, void* stream) {
  static const char* fn = "w8a8_linear_w4";
  g_last_error.clear();
  if (w8a8_status s = check_w4(fn, xq, x_scale, wq4, w_scale, M, N, K)) return s;
  if (M == 0 || N == 0) return W8A8_OK;
  if (!y_bf16 && !y_f32 && !acc) return fail(W8A8_ERR_INVALID_ARG, fn, "all outputs are NULL");
  if (!aligned(y_bf16, 2) || !aligned(y_f32, 4) || !aligned(acc, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "output pointer misaligned");
  return hip_status(w8a8_launch_gemm_w4(xq, x_scale, wq4, w_scale, M, N, K, y_bf16, y_f32, acc,
                                        nullptr, reinterpret_cast<hipStream_t>(stream)), fn);
}

w8a8_status w8a8_lm_head_argmax_w4(const int8_t* xq, const float* x_scale, const int8_t* wq4,
                                   const float* w_scale, int64_t M, int64_t V, int64_t K,
                                   float* logits, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  static const char* fn = "w8a8_lm_head_argmax_w4";
  g_last_error.clear();
  if (V < 1 || V > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "V out of range [1, 2^30]");
  if (w8a8_status s = check_w4(fn, xq, x_scale, wq4, w_scale, M, V, K)) return s;
  if (M == 0) return W8A8_OK;
  if (!aligned(logits, 4)) return fail(W8A8_ERR_INVALID_ARG, fn, "logits misaligned");
  if (!workspace || workspace_bytes < w8a8_lm_head_workspace_bytes(M))
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_lm_head_verify_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_gemm_w4(xq, x_scale, wq4, w_scale, M, V, K, nullptr, logits,
                                        nullptr, workspace, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}


// ---- BF16 glue fused with the next quantization ----

static w8a8_status check_glue_row(const char* fn, int64_t M, int64_t D) {
  if (M < 0 || M > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "row count out of range");
  if (D < 16 || D > W8A8_MAX_GLUE_WIDTH || D % 16 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "width must be a multiple of 16 in [16, 32768]");
  return W8A8_OK;
}

w8a8_status w8a8_residual_rmsnorm_quant(const uint16_t* h, const uint16_t* delta,
                                        const uint16_t* gamma, float eps, const float* smooth,
                                        int64_t M, int64_t D, uint16_t* h_out, uint16_t* normed,
                                        int8_t* xq, float* x_scale, void* stream) {
  static const char* fn = "w8a8_residual_rmsnorm_quant";
  g_last_error.clear();
  if (w8a8_status s = check_glue_row(fn, M, D)) return s;
  if (!(std::isfinite(eps) && eps >= 0.0f)) return fail(W8A8_ERR_INVALID_ARG, fn, "eps must be finite and >= 0");
  if (M == 0) return W8A8_OK;
  if (!h || !gamma || !xq || !x_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(h, 16) || !aligned(delta, 16) || !aligned(gamma, 16) || !aligned(h_out, 16) ||
      !aligned(normed, 16) || !aligned(xq, 16) || !aligned(smooth, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "tensors must be 16-byte aligned");
  if (!aligned(x_scale, 4)) return fail(W8A8_ERR_INVALID_ARG, fn, "x_scale misaligned");
  return hip_status(w8a8_launch_residual_rmsnorm_quant(h, delta, gamma, eps, smooth, M, D, h_out,
                                                       normed, xq, x_scale,
                                                       reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

w8a8_status w8a8_silu_mul_quant(const uint16_t* gate, const uint16_t* up, int64_t row_stride,
                                const float* smooth, int64_t M, int64_t F, uint16_t* act,
                                int8_t* xq, float* x_scale, void* stream) {
  static const char* fn = "w8a8_silu_mul_quant";
  g_last_error.clear();
  if (w8a8_status s = check_glue_row(fn, M, F)) return s;
  if (row_stride < F || row_stride % 8 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "row_stride must be >= F and a multiple of 8");
  if (M == 0) return W8A8_OK;
  if (!gate || !up || !xq || !x_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(gate, 16) || !aligned(up, 16) || !aligned(act, 16) || !aligned(xq, 16) ||
      !aligned(smooth, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "tensors must be 16-byte aligned");
  if (!aligned(x_scale, 4)) return fail(W8A8_ERR_INVALID_ARG, fn, "x_scale misaligned");
  return hip_status(w8a8_launch_silu_mul_quant(gate, up, row_stride, smooth, M, F, act, xq,
                                               x_scale, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}


// ---- tiled activations for the batched product ----

w8a8_status w8a8_quantize_act_tiled(const uint16_t* x_bf16, const float* smooth, int64_t M,
                                    int64_t K, int8_t* xq_tiled, float* x_scale, void* stream) {
  static const char* fn = "w8a8_quantize_act_tiled";
  g_last_error.clear();
  if (w8a8_status s = check_rows_k(fn, M, K)) return s;
  if (M == 0) return W8A8_OK;
  if (!x_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "x_scale is NULL");
  if (K > 0 && (!x_bf16 || !xq_tiled)) return fail(W8A8_ERR_INVALID_ARG, fn, "x_bf16 or xq_tiled is NULL");
  if (!aligned(x_bf16, 16) || !aligned(xq_tiled, 16) || !aligned(smooth, 16) ||
      !aligned(x_scale, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned (16 bytes for tensors, 4 for scales)");
  return hip_status(w8a8_launch_quantize_rows(x_bf16, true, smooth, false, M, K, true, xq_tiled,
                                              x_scale, reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t w8a8_linear_tiled_act_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || M > kMaxRows || N > kMaxRows || K < 0 || K > W8A8_MAX_K) return 0;
  return w8a8_batched_workspace_bytes(M, N, K, true);
}

w8a8_status w8a8_linear_tiled_act(const int8_t* xq_tiled, const float* x_scale,
                                  const int8_t* wq_tiled, const float* w_scale, int64_t M,
                                  int64_t N, int64_t K, uint16_t* y_bf16, float* y_f32,
                                  int32_t* acc, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  static const char* fn = "w8a8_linear_tiled_act";
  g_last_error.clear();
  if (w8a8_status s = check_rows_k(fn, M, K)) return s;
  if (N < 0 || N > kMaxRows) return fail(W8A8_ERR_INVALID_ARG, fn, "N out of range");
  if (M == 0 || N == 0) return W8A8_OK;
  if (!y_bf16 && !y_f32 && !acc) return fail(W8A8_ERR_INVALID_ARG, fn, "all outputs are NULL");
  if (!x_scale || !w_scale) return fail(W8A8_ERR_INVALID_ARG, fn, "x_scale or w_scale is NULL");
  if (K > 0 && (!xq_tiled || !wq_tiled)) return fail(W8A8_ERR_INVALID_ARG, fn, "xq_tiled or wq_tiled is NULL");
  if (!aligned(xq_tiled, 16) || !aligned(wq_tiled, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "xq_tiled and wq_tiled must be 16-byte aligned");
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(y_bf16, 2) || !aligned(y_f32, 4) ||
      !aligned(acc, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "scale or output pointer misaligned");
  const size_t need = w8a8_batched_workspace_bytes(M, N, K, true);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(W8A8_ERR_WORKSPACE, fn,
                "workspace NULL or smaller than w8a8_linear_tiled_act_workspace_bytes()");
  if (need > 0 && !aligned(workspace, 256))
    return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_gemm_batched(xq_tiled, x_scale, wq_tiled, w_scale, M, N, K, true,
                                             y_bf16, y_f32, acc, nullptr, 0, 0,
                                             reinterpret_cast<hipStream_t>(stream), true,
                                             need > 0 ? workspace : nullptr),
                    fn);
}

w8a8_status w8a8_lm_head_argmax_tiled_act(const int8_t* xq_tiled, const float* x_scale,
                                          const int8_t* wq_tiled, const float* w_scale,
                                          int64_t M, int64_t V, int64_t K, float* logits,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream) {
  static const char* fn = "w8a8_lm_head_argmax_tiled_act";
  g_last_error.clear();
  if (w8a8_status s = check_lm_head(fn, xq_tiled, x_scale, wq_tiled, w_scale, M, V, K, logits,
                                    workspace, workspace_bytes))
    return s;
  if (M == 0) return W8A8_OK;
  return hip_status(w8a8_launch_gemm_batched(xq_tiled, x_scale, wq_tiled, w_scale, M, V, K, true,
                                             nullptr, logits, nullptr, workspace,
                                             w8a8_argmax_subkeys(), w8a8_argmax_key_stride(),
                                             reinterpret_cast<hipStream_t>(stream), true),
                    fn);
}

// ---- attention of the verified block ----

size_t w8a8_verify_attention_workspace_bytes(int64_t B, int64_t Hkv, int64_t Lmax) {
  if (B <= 0 || Hkv <= 0 || Lmax <= 0 || B > 65535 || Hkv > 65535 || Lmax > (1 << 17) ||
      Lmax % 16 != 0)
    return 0;
  return w8a8_attention_workspace_bytes_impl(B, Hkv, Lmax);
}

w8a8_status w8a8_verify_attention(const uint16_t* q, const uint16_t* k_cache,
                                  const uint16_t* v_cache, const int32_t* lengths, int64_t B,
                                  int64_t T, int64_t Hq, int64_t Hkv, int64_t Dh, int64_t Lmax,
                                  uint16_t* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  static const char* fn = "w8a8_verify_attention";
  g_last_error.clear();
  if (B < 0 || B > 65535) return fail(W8A8_ERR_INVALID_ARG, fn, "B out of range");
  if (B == 0) return W8A8_OK;
  if (Dh != 128) return fail(W8A8_ERR_UNSUPPORTED, fn, "head dimension must be 128");
  if (T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hkv > 65535 || Hq > 65535)
    return fail(W8A8_ERR_INVALID_ARG, fn, "T, Hq, Hkv must be >= 1 with Hq % Hkv == 0");
  if (T * (Hq / Hkv) > 64)
    return fail(W8A8_ERR_UNSUPPORTED, fn, "T * Hq / Hkv must be <= 64");
  if (Lmax < T || Lmax > (1 << 17) || Lmax % 16 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "Lmax must be a multiple of 16 in [T, 131072]");
  if (!q || !k_cache || !v_cache || !lengths || !out)
    return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) ||
      !aligned(lengths, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "q/k/v must be 16-byte aligned, out and lengths 4");
  if (!workspace || workspace_bytes < w8a8_attention_workspace_bytes_impl(B, Hkv, Lmax))
    return fail(W8A8_ERR_WORKSPACE, fn, "workspace NULL or smaller than w8a8_verify_attention_workspace_bytes()");
  if (!aligned(workspace, 256)) return fail(W8A8_ERR_INVALID_ARG, fn, "workspace must be 256-byte aligned");
  return hip_status(w8a8_launch_verify_attention(q, k_cache, v_cache, lengths, B, T, Hq, Hkv, Lmax,
                                                 out, workspace,
                                                 reinterpret_cast<hipStream_t>(stream)), fn);
}


w8a8_status w8a8_pack_v_cache(const uint16_t* v, int64_t B, int64_t Hkv, int64_t Lmax,
                              int64_t Dh, uint16_t* v_blocked, void* stream) {
  static const char* fn = "w8a8_pack_v_cache";
  g_last_error.clear();
  if (B < 0 || Hkv < 0 || B > 65535 || Hkv > 65535) return fail(W8A8_ERR_INVALID_ARG, fn, "B, Hkv out of range");
  if (B == 0 || Hkv == 0) return W8A8_OK;
  if (Dh != 128) return fail(W8A8_ERR_UNSUPPORTED, fn, "head dimension must be 128");
  if (Lmax < 16 || Lmax > (1 << 17) || Lmax % 16 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "Lmax must be a multiple of 16 in [16, 131072]");
  if (!v || !v_blocked) return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(v, 2) || !aligned(v_blocked, 16))
    return fail(W8A8_ERR_INVALID_ARG, fn, "v must be 2-byte aligned, v_blocked 16");
  const char* vb = reinterpret_cast<const char*>(v);
  const char* ob = reinterpret_cast<const char*>(v_blocked);
  const size_t bytes = (size_t)B * Hkv * Lmax * 128 * 2;
  if (vb < ob + bytes && ob < vb + bytes) return fail(W8A8_ERR_INVALID_ARG, fn, "v and v_blocked overlap");
  return hip_status(w8a8_launch_pack_v_cache(v, B * Hkv, Lmax, v_blocked,
                                             reinterpret_cast<hipStream_t>(stream)), fn);
}


w8a8_status w8a8_qk_norm_rope_append(const uint16_t* qkv, int64_t B, int64_t T, int64_t Hq,
                                     int64_t Hkv, int64_t Dh, const uint16_t* q_gamma,
                                     const uint16_t* k_gamma, float eps, float rope_base,
                                     const int32_t* lengths, int64_t Lmax, uint16_t* q_out,
                                     uint16_t* k_cache, uint16_t* v_cache, void* stream) {
  static const char* fn = "w8a8_qk_norm_rope_append";
  g_last_error.clear();
  if (B < 0 || B > 65535) return fail(W8A8_ERR_INVALID_ARG, fn, "B out of range");
  if (B == 0) return W8A8_OK;
  if (Dh != 128) return fail(W8A8_ERR_UNSUPPORTED, fn, "head dimension must be 128");
  if (T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq + 2 * Hkv > 65535 || B * T > (1 << 30))
    return fail(W8A8_ERR_INVALID_ARG, fn, "T, Hq, Hkv out of range");
  if (Lmax < T || Lmax > (1 << 17) || Lmax % 16 != 0)
    return fail(W8A8_ERR_INVALID_ARG, fn, "Lmax must be a multiple of 16 in [T, 131072]");
  if (!(std::isfinite(eps) && eps >= 0.0f) || !(std::isfinite(rope_base) && rope_base > 1.0f))
    return fail(W8A8_ERR_INVALID_ARG, fn, "eps must be >= 0 and rope_base > 1");
  if (!qkv || !q_gamma || !k_gamma || !lengths || !q_out || !k_cache || !v_cache)
    return fail(W8A8_ERR_INVALID_ARG, fn, "required pointer is NULL");
  if (!aligned(qkv, 2) || !aligned(q_gamma, 2) || !aligned(k_gamma, 2) || !aligned(q_out, 2) ||
      !aligned(k_cache, 2) || !aligned(v_cache, 2) || !aligned(lengths, 4))
    return fail(W8A8_ERR_INVALID_ARG, fn, "pointer misaligned");
  return hip_status(w8a8_launch_qk_norm_rope_append(qkv, B, T, Hq, Hkv, q_gamma, k_gamma, eps,
                                                    rope_base, lengths, Lmax, q_out, k_cache,
                                                    v_cache, reinterpret_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
