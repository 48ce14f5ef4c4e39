// BF16 linear at the same shapes as the W8A8 one: the full-precision
// verifier's weight stream, kept as the two-times-traffic reference (BF16
// weights move twice the bytes of INT8 ones: shd-paper.top English abstract;
// gist.science German summary, Technische Zusammenfassung §3 item 4).
//
//   y32[m][n] = sum_k x[m][k] * w[n][k]   (bf16 operands, fp32 accumulation)
//   y  [m][n] = bf16_rne(y32)
//
// Same organisation as the W8A8 skinny kernel, on v_mfma_f32_16x16x32_bf16:
// lane l supplies A row / B column (l & 15) with the 8 k-values of group
// (l >> 4) of each 32-wide step, loaded as 16 bytes from the same
// k-positions for both operands; WAVES waves split K inside a workgroup and
// reduce their fp32 tiles through LDS in a fixed order.  Up to 16 token rows.
//
// Two weight layouts.  Row-major [N][K]: each 64-lane load gathers 16 rows
// x 64 bytes.  Tiled, as the W8A8 weights: one contiguous KiB per 16
// channels x 32 k, in the operand's lane order, element (n, k) at bf16
// offset
//   ((n/16 * steps + k/32) * 64 + (n%16 + 16*((k%32)/8))) * 8 + k%8,
// steps = ceil(K/32), padding (n >= N, k >= K) zero; every weight load is
// then one non-temporal KiB, the waves of a workgroup taking the k steps
// round-robin so that together they sweep adjacent KiB blocks.
#include "common.h"

namespace w8a8 {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct Bf16Args {
  const uint16_t* x;
  const uint16_t* w;
  int M, N, K;
  uint16_t* y_bf16;
  float* y_f32;
};

__device__ __forceinline__ v4i load16_bf(const void* p) { return *reinterpret_cast<const v4i*>(p); }
__device__ __forceinline__ v4i load16_bf_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

template <int WAVES, int U>
__global__ __launch_bounds__(WAVES * kWave) void gemm_bf16_skinny(Bf16Args g) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int K = g.K;
  const int steps = (K + 31) >> 5;
  const int s0 = (int)(((int64_t)steps * wave) / WAVES);
  const int s1 = (int)(((int64_t)steps * (wave + 1)) / WAVES);

  const bool a_ok = col < g.M;
  const int n = n0 + col;
  const bool b_ok = n < g.N;
  const uint16_t* a_ptr = g.x + (size_t)(a_ok ? col : 0) * (size_t)K + grp * 8;
  const uint16_t* b_ptr = g.w + (size_t)(b_ok ? n : 0) * (size_t)K + grp * 8;

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i zero = v4i{0, 0, 0, 0};
  int s = s0;
  for (; s + U <= s1; s += U) {
    v4i a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 32;
      const bool kin = k + grp * 8 < K;
      a[u] = (a_ok && kin) ? *reinterpret_cast<const v4i*>(a_ptr + k) : zero;
      b[u] = (b_ok && kin) ? *reinterpret_cast<const v4i*>(b_ptr + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u]),
                                                    __builtin_bit_cast(v8bf, b[u]), acc, 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const int k = s * 32;
    const bool kin = k + grp * 8 < K;
    const v4i a = (a_ok && kin) ? *reinterpret_cast<const v4i*>(a_ptr + k) : zero;
    const v4i b = (b_ok && kin) ? *reinterpret_cast<const v4i*>(b_ptr + k) : zero;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                  __builtin_bit_cast(v8bf, b), acc, 0, 0, 0);
  }

  if constexpr (WAVES > 1) {
    __shared__ v4f red[WAVES][kWave];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4f sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[w][lane];
    acc = sum;
  }
  if (!b_ok) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * grp + r;
    if (m >= g.M) continue;
    const size_t o = (size_t)m * (size_t)g.N + (size_t)n;
    if (g.y_f32) g.y_f32[o] = acc[r];
    if (g.y_bf16) g.y_bf16[o] = f32_to_bf16_rne(acc[r]);
  }
}

// The tiled layout from a row-major [N][K] bf16 weight (K % 16 == 0): one
// thread per 16-byte lane unit u = (tile * steps + s) * 64 + l.
__global__ __launch_bounds__(256) void tile_bf16_kernel(const uint16_t* __restrict__ w, int64_t N,
                                                        int64_t K, int64_t steps, int64_t units,
                                                        uint16_t* __restrict__ out) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  const int l = (int)(u & 63);
  const int64_t ts = u >> 6;
  const int64_t tile = ts / steps, s = ts - tile * steps;
  const int64_t n = tile * 16 + (l & 15);
  const int64_t k0 = s * 32 + (l >> 4) * 8;
  v4i v = v4i{0, 0, 0, 0};
  // (K % 16 == 0 and k0 % 8 == 0: a group that starts below K ends there)
  if (n < N && k0 < K) v = *reinterpret_cast<const v4i*>(w + n * K + k0);
  *reinterpret_cast<v4i*>(out + u * 8) = v;
}

// The same product on tiled weights: a workgroup owns TN 16-channel tiles;
// wave w takes k steps w, w + WAVES, ... in batches of U (a partial last
// batch requested together), then the waves' fp32 tiles meet in LDS.
template <int TN, int WAVES, int U>
__global__ __launch_bounds__(WAVES * kWave) void gemm_bf16_tiled(Bf16Args g) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int K = g.K;
  const int steps = (K + 31) >> 5;
  const int tiles16 = (g.N + 15) >> 4;
  const int J = steps > wave ? (steps - wave + WAVES - 1) / WAVES : 0;

  const bool a_ok = col < g.M;
  const uint16_t* a_ptr = g.x + (size_t)(a_ok ? col : 0) * (size_t)K + grp * 8;
  const char* b_ptr[TN];
  bool b_ok[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int t16 = blockIdx.x * TN + t;
    b_ok[t] = t16 < tiles16;
    b_ptr[t] = reinterpret_cast<const char*>(g.w) + ((size_t)(b_ok[t] ? t16 : 0) * (size_t)steps << 10) +
               (lane << 4);
  }
  v4f acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4i zero = v4i{0, 0, 0, 0};
  auto batch = [&](int j, int live_n) {
    v4i a[U], b[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = u < live_n;
      const int s = wave + WAVES * (live ? j + u : j);
      const int k = s * 32;
      const bool kin = k + grp * 8 < K;
      a[u] = (live && a_ok && kin) ? load16_bf(a_ptr + k) : zero;
#pragma unroll
      for (int t = 0; t < TN; ++t)
        b[u][t] = (live && (TN == 1 || b_ok[t])) ? load16_bf_stream(b_ptr[t] + ((size_t)s << 10)) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u]),
                                                         __builtin_bit_cast(v8bf, b[u][t]), acc[t], 0, 0, 0);
  };
  int j = 0;
  for (; j + U <= J; j += U) batch(j, U);
  if (j < J) batch(j, J - j);

  if constexpr (WAVES > 1) {
    __shared__ v4f red[WAVES][TN][kWave];
#pragma unroll
    for (int t = 0; t < TN; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      v4f sum = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) sum += red[w][t][lane];
      acc[t] = sum;
    }
  }
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = (blockIdx.x * TN + t) * 16 + col;
    if (n >= g.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * grp + r;
      if (m >= g.M) continue;
      const size_t o = (size_t)m * (size_t)g.N + (size_t)n;
      if (g.y_f32) g.y_f32[o] = acc[t][r];
      if (g.y_bf16) g.y_bf16[o] = f32_to_bf16_rne(acc[t][r]);
    }
  }
}

}  // namespace w8a8

size_t w8a8_bf16_tiled_weight_bytes_impl(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return (size_t)((N + 15) / 16) * (size_t)((K + 31) / 32) * 1024;
}

hipError_t w8a8_launch_tile_bf16(const uint16_t* w, int64_t N, int64_t K, uint16_t* out,
                                 hipStream_t stream) {
  using namespace w8a8;
  const int64_t steps = (K + 31) / 32;
  const int64_t units = (N + 15) / 16 * steps * 64;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(tile_bf16_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                     w, N, K, steps, units, out);
  return hipGetLastError();
}

// Launch shape as for the W8A8 skinny kernel: two tiles and 4 waves per
// workgroup on wide outputs (the LM head), one tile and 8 waves otherwise.
hipError_t w8a8_launch_bf16_gemm_tiled(const uint16_t* x, const uint16_t* w_tiled, int64_t M,
                                       int64_t N, int64_t K, uint16_t* y_bf16, float* y_f32,
                                       hipStream_t stream) {
  using namespace w8a8;
  if (M == 0 || N == 0) return hipSuccess;
  Bf16Args g{x, w_tiled, (int)M, (int)N, (int)K, y_bf16, y_f32};
  const int64_t tiles = (N + 15) / 16;
  if (tiles >= 2048)
    hipLaunchKernelGGL((gemm_bf16_tiled<2, 4, 8>), dim3((unsigned)((tiles + 1) / 2)), dim3(4 * kWave), 0,
                       stream, g);
  else
    hipLaunchKernelGGL((gemm_bf16_tiled<1, 8, 8>), dim3((unsigned)tiles), dim3(8 * kWave), 0, stream, g);
  return hipGetLastError();
}

hipError_t w8a8_launch_bf16_gemm(const uint16_t* x, const uint16_t* w, int64_t M, int64_t N,
                                 int64_t K, uint16_t* y_bf16, float* y_f32, hipStream_t stream) {
  using namespace w8a8;
  if (M == 0 || N == 0) return hipSuccess;
  Bf16Args g{x, w, (int)M, (int)N, (int)K, y_bf16, y_f32};
  const int tiles = (int)((N + 15) / 16);
  if (tiles >= 1024) {
    hipLaunchKernelGGL((gemm_bf16_skinny<4, 8>), dim3(tiles), dim3(4 * kWave), 0, stream, g);
  } else {
    hipLaunchKernelGGL((gemm_bf16_skinny<16, 8>), dim3(tiles), dim3(16 * kWave), 0, stream, g);
  }
  return hipGetLastError();
}
