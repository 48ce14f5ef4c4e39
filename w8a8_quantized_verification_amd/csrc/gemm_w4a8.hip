// W4A8 for gfx950: int4 per-output-channel weights, int8 per-token
// activations, exact int32 accumulation, the W8A8 dequant epilogue.
//
// The pages name lower-bit verifiers (INT4) as explored and as the next step
// (shd-paper.top Chinese summary, key design; gist.science Italian and
// Japanese summaries, §5), without a scheme; this is the int8 scheme with
// 4-bit weight codes:
//   w_scale[n] = amax_n / 7, q = clip(rint(w * (7 / amax_n)), -7, 7)
//   acc[m][n]  = sum_k xq[m][k] * q[n][k]            (exact in int32)
//   y32 = (fp32(acc) * x_scale[m]) * w_scale[n], y = bf16(y32)
// Halving the weight bytes again halves the time of the HBM-bound skinny
// product.
//
// Weight layout (int4 tiled): per 16-channel tile and per 128-wide k pair of
// MFMA steps, 1 KiB; lane l (channel l%16, k group g = l/16) owns 16 bytes:
// bytes 0..7 for k = 128p + 16g + j and bytes 8..15 for k = 128p + 64 + 16g
// + j (j = 0..15).  In each 8-byte half, with words w0 (bytes 0..3) and w1
// (bytes 4..7): byte i of w0 holds j = i in its low nibble and j = 8+i in
// its high nibble; byte i of w1 holds j = 4+i (low) and j = 12+i (high).
// Codes are two's-complement nibbles; padding (n >= N, k >= K) is 0.
//
// Unpacking is two masks per word: (w << 4) & 0xF0F0F0F0 puts every low
// nibble in the high half of its byte and w & 0xF0F0F0F0 keeps the high
// nibbles, each byte then holding 16 * code as an int8.  The MFMA therefore
// accumulates 16 * acc (|16 acc| <= 127 * 112 * K < 2^31 for K <= 133144)
// and one arithmetic shift by 4 at the end is exact.  Byte j of the
// unpacked operand is k = 16g + j, the same k the activation fragment holds,
// so the usual pairing of A and B lanes is kept.
#include "common.h"

#include <climits>

namespace w8a8 {

constexpr int kW4Threads = 256;
constexpr uint32_t kHiNibbles = 0xF0F0F0F0u;

__host__ __device__ __forceinline__ size_t w4_offset(int64_t n, int64_t k, int64_t pairs) {
  const int64_t kk = k & 127;
  const int64_t lane = (n & 15) | (((kk & 63) >> 4) << 4);
  return ((((size_t)(n >> 4) * (size_t)pairs + (size_t)(k >> 7)) << 6) + (size_t)lane) * 16 +
         (size_t)(kk >> 6) * 8;
}

// One row (output channel) per workgroup; rows up to the next multiple of 16
// are padding and written as zeros.
template <bool kSmooth>
__global__ __launch_bounds__(kW4Threads) void quantize_w4_kernel(const float* __restrict__ w,
                                                                 const float* __restrict__ smooth,
                                                                 int64_t N, int64_t K,
                                                                 int8_t* __restrict__ out,
                                                                 float* __restrict__ scale) {
  __shared__ float red[kW4Threads / kWave];
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t pairs = (K + 127) >> 7;
  const int64_t groups = pairs * 8;   // 16-wide k groups, padded
  const bool real = n < N;
  const float* row = w + (size_t)(real ? n : 0) * (size_t)K;

  auto load16f = [&](int64_t k, float v[16]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(row + k + 4 * i);
      v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
    }
    if constexpr (kSmooth) {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] / smooth[k + i];
    }
  };

  float amax = 0.0f;
  if (real) {
    for (int64_t g = tid; g * 16 < K; g += kW4Threads) {
      float v[16];
      load16f(g * 16, v);
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  }
  amax = wave_max(amax);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? 7.0f / amax : 0.0f;
  if (real && tid == 0) scale[n] = amax > 0.0f ? amax / 7.0f : 0.0f;

  for (int64_t g = tid; g < groups; g += kW4Threads) {
    const int64_t k = g * 16;
    uint32_t w0 = 0u, w1 = 0u;
    if (real && k < K) {
      float v[16];
      load16f(k, v);
      uint32_t c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float r = __builtin_rintf(v[i] * inv);
        r = fminf(fmaxf(r, -7.0f), 7.0f);
        c[i] = (v[i] == 0.0f) ? 0u : ((uint32_t)(int)r & 0xFu);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= (c[i] | (c[8 + i] << 4)) << (8 * i);
        w1 |= (c[4 + i] | (c[12 + i] << 4)) << (8 * i);
      }
    }
    *reinterpret_cast<uint2*>(out + w4_offset(n, k, pairs)) = make_uint2(w0, w1);
  }
}

struct W4Args {
  const int8_t* xq;
  const float* xs;
  const int8_t* wq;   // int4 tiled
  const float* ws;
  int M, N, K;
  int pairs;    // ceil(K / 128)
  int tiles16;  // ceil(N / 16)
  uint16_t* y_bf16;
  float* y_f32;
  int32_t* acc;
  unsigned long long* keys;  // fused argmax sub-keys (as for the int8 LM head), or null
};

__device__ __forceinline__ void unpack_w4(v4i raw, v4i& b0, v4i& b1) {
  const uint32_t x = (uint32_t)raw.x, y = (uint32_t)raw.y, z = (uint32_t)raw.z, w = (uint32_t)raw.w;
  b0 = v4i{(int)((x << 4) & kHiNibbles), (int)((y << 4) & kHiNibbles), (int)(x & kHiNibbles),
           (int)(y & kHiNibbles)};
  b1 = v4i{(int)((z << 4) & kHiNibbles), (int)((w << 4) & kHiNibbles), (int)(z & kHiNibbles),
           (int)(w & kHiNibbles)};
}

// grid (column workgroups, 1, 16-row blocks); WAVES waves take the k pairs
// round-robin, so the workgroup sweeps adjacent KiB blocks of its tiles
// with non-temporal 16-byte loads; partial tiles meet in LDS.
template <int TN, int WAVES, int U, bool kArgmax>
__global__ __launch_bounds__(WAVES * kWave) void gemm_w4a8_skinny(W4Args g) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int tile = blockIdx.x;
  const int m_base = blockIdx.z * 16;
  const int n0 = tile * 16 * TN;
  const int K = g.K;
  const int pairs = g.pairs;
  const int J = pairs > wave ? (pairs - wave + WAVES - 1) / WAVES : 0;

  const int m_a = m_base + col;
  const bool a_ok = m_a < g.M;
  const int8_t* a_ptr = g.xq + (size_t)(a_ok ? m_a : 0) * (size_t)K + grp * 16;
  const int8_t* b_ptr[TN];
  bool b_ok[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int t16 = tile * TN + t;
    b_ok[t] = t16 < g.tiles16;
    b_ptr[t] = g.wq + ((size_t)(b_ok[t] ? t16 : 0) * (size_t)pairs << 10) + (lane << 4);
  }

  v4i acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = v4i{0, 0, 0, 0};
  const v4i zero = v4i{0, 0, 0, 0};

  auto load_a = [&](int k) -> v4i {
    return (a_ok && k + grp * 16 < K) ? *reinterpret_cast<const v4i*>(a_ptr + k) : zero;
  };
  auto load_b = [&](int t, int p) -> v4i {
    return (TN == 1 || b_ok[t])
               ? __builtin_nontemporal_load(reinterpret_cast<const v4i*>(b_ptr[t] + ((size_t)p << 10)))
               : zero;
  };

  int j = 0;
  for (; j + U <= J; j += U) {
    v4i a0[U], a1[U], raw[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = wave + WAVES * (j + u);
      a0[u] = load_a(p * 128);
      a1[u] = load_a(p * 128 + 64);
#pragma unroll
      for (int t = 0; t < TN; ++t) raw[u][t] = load_b(t, p);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        v4i b0, b1;
        unpack_w4(raw[u][t], b0, b1);
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0[u], b0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1[u], b1, acc[t], 0, 0, 0);
      }
  }
  for (; j < J; ++j) {
    const int p = wave + WAVES * j;
    const v4i a0 = load_a(p * 128), a1 = load_a(p * 128 + 64);
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      v4i b0, b1;
      unpack_w4(load_b(t, p), b0, b1);
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc[t], 0, 0, 0);
    }
  }

  if constexpr (WAVES > 1) {
    __shared__ v4i red[WAVES][TN][kWave];
#pragma unroll
    for (int t = 0; t < TN; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      v4i sum = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][t][lane];
      acc[t] = sum;
    }
  }

  // wave 0: rows 4*grp + r, column col of each tile; acc holds 16 * the sums
  float bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  int bi[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + col;
    if (n >= g.N) continue;
    const float wsn = g.ws[n];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + 4 * grp + r;
      if (m < g.M) {
        const int32_t a = acc[t][r] >> 4;
        const float y = (static_cast<float>(a) * g.xs[m]) * wsn;
        const size_t o = (size_t)m * (size_t)g.N + (size_t)n;
        if (g.y_f32) g.y_f32[o] = y;
        if (g.y_bf16) g.y_bf16[o] = f32_to_bf16_rne(y);
        if (g.acc) g.acc[o] = a;
        if constexpr (kArgmax) {
          if (y > bv[r]) { bv[r] = y; bi[r] = n; }   // t ascending: first maximum kept
        }
      }
    }
  }
  if constexpr (kArgmax) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float ov = __shfl_xor(bv[r], off, kWave);
        const int oi = __shfl_xor(bi[r], off, kWave);
        if (ov > bv[r] || (ov == bv[r] && oi < bi[r])) { bv[r] = ov; bi[r] = oi; }
      }
      const int m = m_base + 4 * grp + r;
      if (col == 0 && m < g.M && bi[r] != INT_MAX) {
        const size_t sub = (size_t)m * kArgmaxSubkeys + (tile % kArgmaxSubkeys);
        __hip_atomic_fetch_max(&g.keys[sub * kArgmaxKeyStride], argmax_key(bv[r], bi[r]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

constexpr int kW4Unroll = 4;

}  // namespace w8a8

size_t w8a8_w4_weight_bytes_impl(int64_t N, int64_t K) {
  return (size_t)((N + 15) / 16) * 16 * (size_t)((K + 127) / 128) * 64;
}

hipError_t w8a8_launch_quantize_w4(const float* w, const float* smooth, int64_t N, int64_t K,
                                   int8_t* wq4, float* scale, hipStream_t stream) {
  using namespace w8a8;
  if (N == 0) return hipSuccess;   // (K == 0 writes scales of 0 and no codes)
  const dim3 grid((unsigned)((N + 15) / 16 * 16)), block(kW4Threads);
  if (smooth)
    hipLaunchKernelGGL((quantize_w4_kernel<true>), grid, block, 0, stream, w, smooth, N, K, wq4, scale);
  else
    hipLaunchKernelGGL((quantize_w4_kernel<false>), grid, block, 0, stream, w, smooth, N, K, wq4, scale);
  return hipGetLastError();
}

hipError_t w8a8_launch_gemm_w4(const int8_t* xq, const float* x_scale, const int8_t* wq4,
                               const float* w_scale, int64_t M, int64_t N, int64_t K,
                               uint16_t* y_bf16, float* y_f32, int32_t* acc, void* keys,
                               hipStream_t stream) {
  using namespace w8a8;
  if (M == 0 || N == 0) return hipSuccess;
  W4Args g{};
  g.xq = xq; g.xs = x_scale; g.wq = wq4; g.ws = w_scale;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.pairs = (int)((K + 127) / 128);
  g.tiles16 = (int)((N + 15) / 16);
  g.y_bf16 = y_bf16; g.y_f32 = y_f32; g.acc = acc;
  g.keys = reinterpret_cast<unsigned long long*>(keys);
  const int64_t mblocks = (M + 15) / 16;
  // as the int8 skinny plan: two tiles per workgroup once there are enough
  // tiles to go round; 4 waves per workgroup for big grids, more for small
  const int tn = ((int64_t)g.tiles16 * mblocks >= 2048) ? 2 : 1;
  const int64_t tiles = (g.tiles16 + tn - 1) / tn;
  const int64_t wgs = tiles * mblocks;
  const int waves = wgs >= 512 ? 4 : (wgs >= 32 ? 8 : 16);
  const dim3 grid((unsigned)tiles, 1, (unsigned)mblocks);
#define W8A8_W4(TN, W, AM) \
  hipLaunchKernelGGL((gemm_w4a8_skinny<TN, W, kW4Unroll, AM>), grid, dim3(W * kWave), 0, stream, g)
#define W8A8_W4_W(TN, AM)                        \
  do {                                           \
    if (waves == 4) W8A8_W4(TN, 4, AM);          \
    else if (waves == 8) W8A8_W4(TN, 8, AM);     \
    else W8A8_W4(TN, 16, AM);                    \
  } while (0)
  if (keys) {
    if (tn == 2) W8A8_W4_W(2, true);
    else W8A8_W4_W(1, true);
  } else {
    if (tn == 2) W8A8_W4_W(2, false);
    else W8A8_W4_W(1, false);
  }
#undef W8A8_W4_W
#undef W8A8_W4
  return hipGetLastError();
}
