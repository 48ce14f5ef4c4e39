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

}  // namespace w8a8

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
