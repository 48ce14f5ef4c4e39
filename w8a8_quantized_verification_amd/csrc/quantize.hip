// Symmetric per-row INT8 quantization (activations per token, weights per
// output channel) for gfx950.
//
// Pages: activations are scaled by the smoothing factor s and converted to
// INT8 at run time; weights are smoothed (divided by s) and quantized to INT8
// offline; symmetric uniform quantization.  (gist.science Japanese summary,
// 技術的サマリー §2.2 items 1-3; gist.science Italian summary, Sommario
// tecnico §2, Componenti Tecnici 1 and the pipeline.)
//
// Per row: amax = max |v|, scale = amax/127, inv = 127/amax (0 if amax == 0),
// q = 0 where v == 0, else clamp(rint(v*inv), -127, 127).  All fp32
// operations are single correctly rounded operations (the library is built
// with -ffp-contract=off and correctly rounded division).
//
// One workgroup of 256 threads (4 waves) per row.  Each thread handles
// groups of 8 consecutive elements with 16-byte loads (bf16: one load; fp32:
// two); the row maximum is a wave reduction followed by a 4-entry LDS
// reduction; the second pass re-reads the row (an L2 hit) and writes 8 int8
// codes per store.
#include "common.h"

namespace w8a8 {

constexpr int kQuantThreads = 256;

template <bool kBf16In, bool kSmooth, bool kDivide>
__device__ __forceinline__ void load8(const void* __restrict__ in_row, const float* __restrict__ smooth,
                                      int64_t k, float v[8]) {
  if constexpr (kBf16In) {
    const uint4 raw = *reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(in_row) + k);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(in_row) + k);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(in_row) + k + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  if constexpr (kSmooth) {
    const float4 s0 = *reinterpret_cast<const float4*>(smooth + k);
    const float4 s1 = *reinterpret_cast<const float4*>(smooth + k + 4);
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = kDivide ? (v[i] / s[i]) : (v[i] * s[i]);
  }
}

template <bool kBf16In, bool kSmooth, bool kDivide>
__global__ __launch_bounds__(kQuantThreads) void quantize_rows_kernel(
    const void* __restrict__ in, const float* __restrict__ smooth, int64_t K,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[kQuantThreads / kWave];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t elt = kBf16In ? sizeof(uint16_t) : sizeof(float);
  const void* in_row = reinterpret_cast<const char*>(in) + (size_t)row * (size_t)K * elt;

  float amax = 0.0f;
  for (int64_t k = (int64_t)tid * 8; k < K; k += kQuantThreads * 8) {
    float v[8];
    load8<kBf16In, kSmooth, kDivide>(in_row, smooth, k, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const float s = amax / 127.0f;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (tid == 0) scale[row] = amax > 0.0f ? s : 0.0f;

  int8_t* q_row = q + (size_t)row * (size_t)K;
  for (int64_t k = (int64_t)tid * 8; k < K; k += kQuantThreads * 8) {
    float v[8];
    load8<kBf16In, kSmooth, kDivide>(in_row, smooth, k, v);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float r = __builtin_rintf(v[i] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      const int qi = (v[i] == 0.0f) ? 0 : (int)r;
      packed[i >> 2] |= ((uint32_t)(qi & 0xff)) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(q_row + k) = make_uint2(packed[0], packed[1]);
  }
}

}  // namespace w8a8

hipError_t w8a8_launch_quantize_rows(const void* in, bool in_is_bf16, const float* smooth,
                                     bool smooth_divides, int64_t R, int64_t K,
                                     int8_t* q, float* scale, hipStream_t stream) {
  using namespace w8a8;
  if (R == 0) return hipSuccess;
  const dim3 grid((unsigned)R), block(kQuantThreads);
#define W8A8_QLAUNCH(BF, SM, DIV) \
  hipLaunchKernelGGL((quantize_rows_kernel<BF, SM, DIV>), grid, block, 0, stream, in, smooth, K, q, scale)
  if (in_is_bf16) {
    if (!smooth) W8A8_QLAUNCH(true, false, false);
    else if (smooth_divides) W8A8_QLAUNCH(true, true, true);
    else W8A8_QLAUNCH(true, true, false);
  } else {
    if (!smooth) W8A8_QLAUNCH(false, false, false);
    else if (smooth_divides) W8A8_QLAUNCH(false, true, true);
    else W8A8_QLAUNCH(false, true, false);
  }
#undef W8A8_QLAUNCH
  return hipGetLastError();
}
