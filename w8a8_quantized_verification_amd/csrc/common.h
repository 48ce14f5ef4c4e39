// Internal helpers shared by the HIP kernels of libw8a8.so (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kXcds = 8;   // MI355X: 8 XCDs, each with its own L2; workgroups go round-robin

// fp32 -> bf16 bit pattern, round to nearest with ties to even; NaN stays a
// quiet NaN with its sign.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Maximum over the 64 lanes of a wave (every lane receives it).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// (value, index) maximum with the lowest index on equal values, over a wave.
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float ov = __shfl_xor(v, off, kWave);
    int oi = __shfl_xor(idx, off, kWave);
    if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
  }
}

// Fused-argmax keys: row m keeps kArgmaxSubkeys running maxima; workgroup w
// folds into sub-key w % kArgmaxSubkeys, at keys[(m * kArgmaxSubkeys + s) *
// kArgmaxKeyStride].  Spreading the folds over 64 addresses 256 bytes apart
// keeps same-address atomics (which serialize) to a few dozen per key.
constexpr int kArgmaxSubkeys = 64;
constexpr int kArgmaxKeyStride = 32;  // in 8-byte words: 256 bytes

// Pack (value, index) into a 64-bit key whose unsigned order is "larger value
// first, then lower index": the value's bits mapped to an order-preserving
// unsigned (negatives complemented, positives with the sign bit set; -0 made
// +0 first so that it ties with +0), the index complemented.  Key 0 means
// "empty".
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(~(uint32_t)idx);
}

}  // namespace w8a8

// ---------------------------------------------------------------------------
// Launchers (host functions defined next to their kernels).  Arguments are
// validated by the C-ABI layer before these are called.  Each returns
// hipSuccess or the launch error.
// ---------------------------------------------------------------------------
hipError_t w8a8_launch_quantize_rows(const void* in, bool in_is_bf16, const float* smooth,
                                     bool smooth_divides, int64_t R, int64_t K, bool tiled,
                                     int8_t* q, float* scale, hipStream_t stream);
size_t w8a8_tiled_weight_bytes_impl(int64_t N, int64_t K);
hipError_t w8a8_launch_tile_weight(const int8_t* wq, int64_t N, int64_t K, int8_t* out,
                                   hipStream_t stream);

size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool tiled);
// workspace of the batched kernel's k split (0: none), and the launcher;
// `workspace` (zero-filled, left zero) may be null where that size is 0
size_t w8a8_batched_workspace_bytes(int64_t M, int64_t N, int64_t K, bool a_tiled);
hipError_t w8a8_launch_gemm_batched(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, int64_t M, int64_t N, int64_t K,
                                    bool tiled, uint16_t* y_bf16, float* y_f32, int32_t* acc,
                                    void* keys, int subkeys, int key_stride, hipStream_t stream,
                                    bool a_tiled = false, void* workspace = nullptr);
size_t w8a8_lm_head_workspace_bytes(int64_t M);
inline int w8a8_argmax_subkeys() { return w8a8::kArgmaxSubkeys; }
inline int w8a8_argmax_key_stride() { return w8a8::kArgmaxKeyStride; }
hipError_t w8a8_launch_lm_head_argmax(const int8_t* xq, const float* x_scale,
                                      const int8_t* wq_tiled, const float* w_scale, int64_t M,
                                      int64_t V, int64_t K, float* logits, void* keys,
                                      hipStream_t stream, hipEvent_t ev0 = nullptr,
                                      hipEvent_t ev1 = nullptr);
hipError_t w8a8_launch_accept_from_keys(void* keys, const int32_t* draft, int64_t B, int64_t G,
                                        int32_t* argmax, int32_t* accept_len, int32_t* next_token,
                                        hipStream_t stream);
hipError_t w8a8_launch_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, int64_t M, int64_t N, int64_t K, bool tiled,
                            uint16_t* y_bf16, float* y_f32, int32_t* acc,
                            void* workspace, hipStream_t stream);

size_t w8a8_argmax_workspace_bytes(int64_t R, int64_t V);
hipError_t w8a8_launch_verify_accept(const float* logits, int64_t V, const int32_t* draft,
                                     int64_t B, int64_t G, int32_t* argmax,
                                     int32_t* accept_len, int32_t* next_token,
                                     void* workspace, hipStream_t stream);

// parts: [B*(G+1)][nparts] 8-byte (float maximum bits, lowest index) pairs
hipError_t w8a8_launch_accept(const void* parts, int nparts, const int32_t* draft, int64_t B,
                              int64_t G, int32_t* argmax, int32_t* accept_len,
                              int32_t* next_token, hipStream_t stream);

hipError_t w8a8_launch_accept_keys(unsigned long long* keys, int subkeys, int key_stride,
                                   const int32_t* draft, int64_t B, int64_t G, int32_t* argmax,
                                   int32_t* accept_len, int32_t* next_token, hipStream_t stream);

hipError_t w8a8_launch_bf16_gemm(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                                 int64_t K, uint16_t* y_bf16, float* y_f32, hipStream_t stream);
size_t w8a8_bf16_tiled_weight_bytes_impl(int64_t N, int64_t K);
hipError_t w8a8_launch_tile_bf16(const uint16_t* w, int64_t N, int64_t K, uint16_t* out,
                                 hipStream_t stream);
hipError_t w8a8_launch_bf16_gemm_tiled(const uint16_t* x, const uint16_t* w_tiled, int64_t M,
                                       int64_t N, int64_t K, uint16_t* y_bf16, float* y_f32,
                                       hipStream_t stream);

size_t w8a8_sample_workspace_bytes_impl(int64_t R, int64_t V);
hipError_t w8a8_launch_sample_weights(const float* logits, int64_t R, int64_t V, float inv_t,
                                      uint64_t* weights, void* workspace, hipStream_t stream);
hipError_t w8a8_launch_verify_sample(const float* logits, int64_t V, const int32_t* draft,
                                     int64_t B, int64_t G, float inv_t, const uint32_t* u_accept,
                                     const uint64_t* u_sample, int32_t* accept_len,
                                     int32_t* next_token, void* workspace, hipStream_t stream);

size_t w8a8_w4_weight_bytes_impl(int64_t N, int64_t K);
hipError_t w8a8_launch_quantize_w4(const float* w, const float* smooth, int64_t N, int64_t K,
                                   int8_t* wq4, float* scale, hipStream_t stream);
hipError_t w8a8_launch_gemm_w4(const int8_t* xq, const float* x_scale, const int8_t* wq4,
                               const float* w_scale, int64_t M, int64_t N, int64_t K,
                               uint16_t* y_bf16, float* y_f32, int32_t* acc, void* keys,
                               hipStream_t stream);

hipError_t w8a8_launch_residual_rmsnorm_quant(const uint16_t* h, const uint16_t* delta,
                                              const uint16_t* gamma, float eps,
                                              const float* smooth, int64_t M, int64_t D,
                                              uint16_t* h_out, uint16_t* normed, int8_t* xq,
                                              float* x_scale, hipStream_t stream);
hipError_t w8a8_launch_silu_mul_quant(const uint16_t* gate, const uint16_t* up, int64_t stride,
                                      const float* smooth, int64_t M, int64_t F, uint16_t* act,
                                      int8_t* xq, float* x_scale, hipStream_t stream);

size_t w8a8_attention_workspace_bytes_impl(int64_t B, int64_t Hkv, int64_t Lmax);
hipError_t w8a8_launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const int32_t* lengths, int64_t B, int64_t T,
                                        int64_t Hq, int64_t Hkv, int64_t Lmax, uint16_t* out,
                                        void* workspace, hipStream_t stream);
hipError_t w8a8_launch_pack_v_cache(const uint16_t* v, int64_t BH, int64_t Lmax, uint16_t* out,
                                    hipStream_t stream);
hipError_t w8a8_launch_qk_norm_rope_append(const uint16_t* qkv, int64_t B, int64_t T, int64_t Hq,
                                           int64_t Hkv, const uint16_t* q_gamma,
                                           const uint16_t* k_gamma, float eps, float rope_base,
                                           const int32_t* lengths, int64_t Lmax, uint16_t* q_out,
                                           uint16_t* k_cache, uint16_t* v_cache,
                                           hipStream_t stream);

hipError_t w8a8_launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t w8a8_launch_lm_head_verify_noalloc(const int8_t* xq, const float* x_scale,
                                              const int8_t* wq_tiled, const float* w_scale,
                                              int64_t V, int64_t K, const int32_t* draft,
                                              int64_t B, int64_t G, float* logits,
                                              int32_t* argmax, int32_t* accept_len,
                                              int32_t* next_token, hipStream_t stream);
