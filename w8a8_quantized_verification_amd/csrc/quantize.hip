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
// reduction; the second pass takes the first 4 groups per thread (rows of up
// to 8192 elements) from registers, re-reads the rest (an L2 hit), and writes
// 8 int8 codes per store.
//
// Weights can also be written in the tiled layout the W8A8 linear streams
// (one contiguous KiB per 16 channels x 64 k): element (n, k) goes to byte
//   ((n/16 * steps + k/64) * 64 + (n%16 + 16*((k%64)/16))) * 16 + k%16,
// steps = ceil(K/64); the grid then covers whole 16-row tiles and every
// padding byte (rows >= N, k >= K) is written as zero.
#include "common.h"

namespace w8a8 {

constexpr int kQuantThreads = 256;      // threads per row (weights, short activation rows)
constexpr int kQuantThreadsLong = 1024; // threads per row for activation rows longer than
constexpr int64_t kLongRow = 8192;      //   this: every element then stays in registers
constexpr int kCache = 4;  // groups of 8 elements kept in registers between the passes

__host__ __device__ __forceinline__ size_t tiled_offset(int64_t n, int64_t k, int64_t steps) {
  return ((((size_t)(n >> 4) * (size_t)steps + (size_t)(k >> 6)) << 6) +
          (size_t)((n & 15) | (((k >> 4) & 3) << 4))) * 16 + (size_t)(k & 15);
}

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

// Rows [0, R) are real; with kTiled the grid also covers the padding rows of
// the last 16-row tile and the k range is padded to a multiple of 64.
template <int kThreads, bool kBf16In, bool kSmooth, bool kDivide, bool kTiled>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(
    const void* __restrict__ in, const float* __restrict__ smooth, int64_t R, int64_t K,
    int8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int kWaves = kThreads / kWave;
  __shared__ float red[kWaves];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t steps = (K + 63) >> 6;
  const int64_t k_end = kTiled ? steps * 64 : K;

  if (kTiled && row >= R) {  // padding row of the last tile: zeros
    for (int64_t k = (int64_t)tid * 8; k < k_end; k += kThreads * 8)
      *reinterpret_cast<uint2*>(q + tiled_offset(row, k, steps)) = make_uint2(0u, 0u);
    return;
  }

  const size_t elt = kBf16In ? sizeof(uint16_t) : sizeof(float);
  const void* in_row = reinterpret_cast<const char*>(in) + (size_t)row * (size_t)K * elt;
  constexpr int64_t kStride = kThreads * 8;

  // pass 1: row maximum; the first kCache groups of 8 stay in registers
  float cache[kCache][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kCache; ++c) {
    const int64_t k = (int64_t)tid * 8 + c * kStride;
    if (k < K) {
      load8<kBf16In, kSmooth, kDivide>(in_row, smooth, k, cache[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(cache[c][i]));
    }
  }
  for (int64_t k = (int64_t)tid * 8 + kCache * kStride; k < K; k += kStride) {
    float v[8];
    load8<kBf16In, kSmooth, kDivide>(in_row, smooth, k, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) amax = fmaxf(amax, red[w]);

  const float s = amax / 127.0f;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (tid == 0) scale[row] = amax > 0.0f ? s : 0.0f;

  // pass 2: codes (cached groups from registers, the rest re-read)
  auto emit = [&](int64_t k, const float v[8], bool real) {
    uint32_t packed[2] = {0u, 0u};
    if (real) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float r = __builtin_rintf(v[i] * inv);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const int qi = (v[i] == 0.0f) ? 0 : (int)r;
        packed[i >> 2] |= ((uint32_t)(qi & 0xff)) << (8 * (i & 3));
      }
    }
    const size_t o = kTiled ? tiled_offset(row, k, steps) : (size_t)row * (size_t)K + (size_t)k;
    *reinterpret_cast<uint2*>(q + o) = make_uint2(packed[0], packed[1]);
  };
#pragma unroll
  for (int c = 0; c < kCache; ++c) {
    const int64_t k = (int64_t)tid * 8 + c * kStride;
    if (k < k_end) emit(k, cache[c], k < K);
  }
  for (int64_t k = (int64_t)tid * 8 + kCache * kStride; k < k_end; k += kStride) {
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (k < K) load8<kBf16In, kSmooth, kDivide>(in_row, smooth, k, v);
    emit(k, v, k < K);
  }
}

// Row-major int8 [N][K] -> tiled layout: one thread per 16-byte chunk of the
// tiled buffer, in tiled order (coalesced writes), zeros for padding.
__global__ __launch_bounds__(256) void tile_weight_kernel(const int8_t* __restrict__ wq, int64_t N,
                                                          int64_t K, int64_t steps, int64_t chunks,
                                                          int8_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int64_t t = c / (steps * 64);
  const int64_t rem = c - t * steps * 64;
  const int64_t s = rem >> 6;
  const int l = (int)(rem & 63);
  const int64_t n = t * 16 + (l & 15);
  const int64_t k = s * 64 + (int64_t)(l >> 4) * 16;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (n < N && k < K) v = *reinterpret_cast<const uint4*>(wq + (size_t)n * (size_t)K + (size_t)k);
  *reinterpret_cast<uint4*>(out + (size_t)c * 16) = v;
}

}  // namespace w8a8

size_t w8a8_tiled_weight_bytes_impl(int64_t N, int64_t K) {
  return (size_t)((N + 15) / 16) * 16 * (size_t)((K + 63) / 64) * 64;
}

hipError_t w8a8_launch_quantize_rows(const void* in, bool in_is_bf16, const float* smooth,
                                     bool smooth_divides, int64_t R, int64_t K, bool tiled,
                                     int8_t* q, float* scale, hipStream_t stream) {
  using namespace w8a8;
  if (R == 0) return hipSuccess;
  const int64_t grid_rows = tiled ? (R + 15) / 16 * 16 : R;
  const dim3 grid((unsigned)grid_rows), block(kQuantThreads);
#define W8A8_QLAUNCH(BF, SM, DIV, TL) \
  hipLaunchKernelGGL((quantize_rows_kernel<kQuantThreads, BF, SM, DIV, TL>), grid, block, 0, stream, in, smooth, R, K, q, scale)
#define W8A8_QLAUNCH_LONG(SM, TL) \
  hipLaunchKernelGGL((quantize_rows_kernel<kQuantThreadsLong, true, SM, false, TL>), grid, \
                     dim3(kQuantThreadsLong), 0, stream, in, smooth, R, K, q, scale)
  if (in_is_bf16) {
    // activations (row-major, or tiled for the batched GEMM); few rows, so
    // long rows get more threads
    if (K > kLongRow) {
      if (tiled) { if (!smooth) W8A8_QLAUNCH_LONG(false, true); else W8A8_QLAUNCH_LONG(true, true); }
      else if (!smooth) W8A8_QLAUNCH_LONG(false, false);
      else W8A8_QLAUNCH_LONG(true, false);
    } else if (tiled) {
      if (!smooth) W8A8_QLAUNCH(true, false, false, true);
      else W8A8_QLAUNCH(true, true, false, true);
    } else if (!smooth) W8A8_QLAUNCH(true, false, false, false);
    else W8A8_QLAUNCH(true, true, false, false);
  } else if (!tiled) {
    if (!smooth) W8A8_QLAUNCH(false, false, false, false);
    else if (smooth_divides) W8A8_QLAUNCH(false, true, true, false);
    else W8A8_QLAUNCH(false, true, false, false);
  } else {
    if (!smooth) W8A8_QLAUNCH(false, false, false, true);
    else if (smooth_divides) W8A8_QLAUNCH(false, true, true, true);
    else W8A8_QLAUNCH(false, true, false, true);
  }
#undef W8A8_QLAUNCH_LONG
#undef W8A8_QLAUNCH
  return hipGetLastError();
}

hipError_t w8a8_launch_tile_weight(const int8_t* wq, int64_t N, int64_t K, int8_t* out,
                                   hipStream_t stream) {
  using namespace w8a8;
  if (N == 0) return hipSuccess;
  const int64_t steps = (K + 63) / 64;
  const int64_t chunks = (N + 15) / 16 * steps * 64;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_weight_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                     stream, wq, N, K, steps, chunks, out);
  return hipGetLastError();
}
