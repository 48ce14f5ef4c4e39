// The BF16 glue between the verifier's W8A8 linears, fused with the
// per-token int8 quantization of the next linear's input (gfx950).
//
// The pages dequantize the INT32 results to BF16 before the non-linear
// layers (gist.science German summary, Technische Zusammenfassung §2
// "De-Quantisierung"; Italian summary §2 pipeline; French summary §2;
// Japanese summary §2.2 item 3).  For the Qwen3 shapes those layers are
// RMSNorm and the SiLU-gated MLP:
//   residual_rmsnorm_quant: h1 = bf16(h + delta); r = 1/sqrt(mean(h1^2) + eps);
//                           n = bf16(bf16(h1 * r) * gamma); then xq, x_scale of n
//   silu_mul_quant:         a = bf16(bf16(silu(g)) * u); then xq, x_scale of a
// The quantization is the one of w8a8_quantize_act on the bf16 row (n or a),
// optionally after the smoothing multiply; it replaces that launch, so a
// decoder layer needs no extra kernel for its glue.
//
// One workgroup per token row; every element of the row stays in registers
// between the passes (rows up to 4 * 8 * threads elements: 8192 with 256
// threads, 32768 with 1024).  Latency-bound at verification sizes.
#include "common.h"

namespace w8a8 {

constexpr int kGlueCache = 4;   // groups of 8 elements per thread

template <int T>
__device__ __forceinline__ float block_sum_f32(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < T / kWave; ++w) s += red[w];
  __syncthreads();
  return s;
}

template <int T>
__device__ __forceinline__ float block_max_f32(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int w = 1; w < T / kWave; ++w) s = fmaxf(s, red[w]);
  __syncthreads();
  return s;
}

__device__ __forceinline__ void load_bf16x8(const uint16_t* p, float v[8]) {
  const uint4 raw = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void store_bf16x8(uint16_t* p, const float v[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16_rne(v[2 * i]) | ((uint32_t)f32_to_bf16_rne(v[2 * i + 1]) << 16);
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16_rne(f)); }

// The tail shared by both kernels: optional smoothing multiply, row absmax,
// scale and codes (the rule of w8a8_quantize_act), from values in registers.
template <int T, bool kSmooth>
__device__ __forceinline__ void quantize_cached(float v[kGlueCache][8], int64_t K,
                                                const float* smooth, int8_t* q_row,
                                                float* scale_out, float* red) {
  const int tid = threadIdx.x;
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kGlueCache; ++c) {
    const int64_t k = (int64_t)tid * 8 + (int64_t)c * T * 8;
    if (k < K) {
      if constexpr (kSmooth) {
        const float4 s0 = *reinterpret_cast<const float4*>(smooth + k);
        const float4 s1 = *reinterpret_cast<const float4*>(smooth + k + 4);
        const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = v[c][i] * s[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    }
  }
  amax = block_max_f32<T>(amax, red);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (tid == 0) *scale_out = amax > 0.0f ? amax / 127.0f : 0.0f;
#pragma unroll
  for (int c = 0; c < kGlueCache; ++c) {
    const int64_t k = (int64_t)tid * 8 + (int64_t)c * T * 8;
    if (k < K) {
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float r = __builtin_rintf(v[c][i] * inv);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const int qi = (v[c][i] == 0.0f) ? 0 : (int)r;
        packed[i >> 2] |= ((uint32_t)(qi & 0xff)) << (8 * (i & 3));
      }
      *reinterpret_cast<uint2*>(q_row + k) = make_uint2(packed[0], packed[1]);
    }
  }
}

template <int T, bool kDelta, bool kSmooth>
__global__ __launch_bounds__(T) void residual_rmsnorm_quant_kernel(
    const uint16_t* h, const uint16_t* delta, const uint16_t* gamma, float eps,
    const float* smooth, int64_t D, uint16_t* h_out, uint16_t* normed, int8_t* xq,
    float* x_scale) {
  __shared__ float red[T / kWave];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t row = (size_t)m * (size_t)D;
  float v[kGlueCache][8];
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < kGlueCache; ++c) {
    const int64_t k = (int64_t)tid * 8 + (int64_t)c * T * 8;
    if (k < D) {
      load_bf16x8(h + row + k, v[c]);
      if constexpr (kDelta) {
        float d[8];
        load_bf16x8(delta + row + k, d);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[c][i] = round_bf16(v[c][i] + d[i]);
        if (h_out) store_bf16x8(h_out + row + k, v[c]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[c][i] * v[c][i];
    }
  }
  ss = block_sum_f32<T>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int c = 0; c < kGlueCache; ++c) {
    const int64_t k = (int64_t)tid * 8 + (int64_t)c * T * 8;
    if (k < D) {
      float g[8];
      load_bf16x8(gamma + k, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[c][i] = round_bf16(round_bf16(v[c][i] * r) * g[i]);
      if (normed) store_bf16x8(normed + row + k, v[c]);
    }
  }
  quantize_cached<T, kSmooth>(v, D, smooth, xq + row, x_scale + m, red);
}

template <int T, bool kSmooth>
__global__ __launch_bounds__(T) void silu_mul_quant_kernel(const uint16_t* gate, const uint16_t* up,
                                                           int64_t stride, const float* smooth,
                                                           int64_t F, uint16_t* act, int8_t* xq,
                                                           float* x_scale) {
  __shared__ float red[T / kWave];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  float v[kGlueCache][8];
#pragma unroll
  for (int c = 0; c < kGlueCache; ++c) {
    const int64_t k = (int64_t)tid * 8 + (int64_t)c * T * 8;
    if (k < F) {
      float g[8], u[8];
      load_bf16x8(gate + (size_t)m * stride + k, g);
      load_bf16x8(up + (size_t)m * stride + k, u);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s = g[i] / (1.0f + expf(-g[i]));
        v[c][i] = round_bf16(round_bf16(s) * u[i]);
      }
      if (act) store_bf16x8(act + (size_t)m * F + k, v[c]);
    }
  }
  quantize_cached<T, kSmooth>(v, F, smooth, xq + (size_t)m * F, x_scale + m, red);
}

}  // namespace w8a8

hipError_t w8a8_launch_residual_rmsnorm_quant(const uint16_t* h, const uint16_t* delta,
                                              const uint16_t* gamma, float eps,
                                              const float* smooth, int64_t M, int64_t D,
                                              uint16_t* h_out, uint16_t* normed, int8_t* xq,
                                              float* x_scale, hipStream_t stream) {
  using namespace w8a8;
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)M);
#define W8A8_RMS(T, DL, SM)                                                                     \
  hipLaunchKernelGGL((residual_rmsnorm_quant_kernel<T, DL, SM>), grid, dim3(T), 0, stream, h, \
                     delta, gamma, eps, smooth, D, h_out, normed, xq, x_scale)
#define W8A8_RMS_T(T)                                      \
  do {                                                     \
    if (delta) { if (smooth) W8A8_RMS(T, true, true); else W8A8_RMS(T, true, false); } \
    else { if (smooth) W8A8_RMS(T, false, true); else W8A8_RMS(T, false, false); }     \
  } while (0)
  if (D <= (int64_t)kGlueCache * 256 * 8) W8A8_RMS_T(256);
  else W8A8_RMS_T(1024);
#undef W8A8_RMS_T
#undef W8A8_RMS
  return hipGetLastError();
}

hipError_t w8a8_launch_silu_mul_quant(const uint16_t* gate, const uint16_t* up, int64_t stride,
                                      const float* smooth, int64_t M, int64_t F, uint16_t* act,
                                      int8_t* xq, float* x_scale, hipStream_t stream) {
  using namespace w8a8;
  if (M == 0) return hipSuccess;
  const dim3 grid((unsigned)M);
#define W8A8_SILU(T, SM)                                                                      \
  hipLaunchKernelGGL((silu_mul_quant_kernel<T, SM>), grid, dim3(T), 0, stream, gate, up, stride, \
                     smooth, F, act, xq, x_scale)
  if (F <= (int64_t)kGlueCache * 256 * 8) {
    if (smooth) W8A8_SILU(256, true);
    else W8A8_SILU(256, false);
  } else {
    if (smooth) W8A8_SILU(1024, true);
    else W8A8_SILU(1024, false);
  }
#undef W8A8_SILU
  return hipGetLastError();
}
