// W8A8 linear for gfx950: INT8 x INT8 -> INT32 on the int8 MFMA, with the
// dequant epilogue fused.
//
// Pages: the matrix product runs on INT8 units and accumulates in INT32,
// then the result is dequantized back to BF16 (gist.science Japanese
// summary, 技術的サマリー §2.2 item 3; gist.science German summary,
// Technische Zusammenfassung §2 "Online-Prozess" / "De-Quantisierung").
// Verification time is weight bytes over memory bandwidth (German summary
// §3 item 4; Japanese summary §2.3), so with a handful of token rows this
// kernel is a weight stream: it is built to keep HBM busy, and uses the MFMA
// because the contraction is dense.
//
//   acc[m][n] = sum_k xq[m][k] * wq[n][k]                     (exact int32)
//   y32[m][n] = fp32(fp32(fp32(acc) * x_scale[m]) * w_scale[n])
//   y  [m][n] = bf16_rne(y32)
//
// Mapping onto v_mfma_i32_16x16x64_i8 (C[16x16] += A[16x64] * B[64x16]):
// lane l supplies A row (l & 15) and B column (l & 15), each with the 16
// k-values of group (l >> 4); it receives C rows 4*(l>>4)..+3 of column
// (l & 15).  A = 16 token rows of xq (rows >= M are zero), B = 16 weight
// rows (output channels).  Each lane loads its 16 bytes of A and of B from
// the SAME 16 k-positions (k = 64*step + 16*(l>>4)), so the pairing of A and
// B inside the instruction is right whatever order the hardware sums the
// 64 products in — and int32 sums are exact in any order.
//
// Work split: a workgroup owns TN tiles of 16 output channels and one
// k-range; its WAVES waves split that k-range, issue U steps of 16-byte
// loads (U*(TN+1) loads in flight per lane) before their MFMAs, and reduce
// their partial tiles through LDS.  When the output has too few tiles to
// fill the 256 CUs, the k-range is also split across SPLIT workgroups
// (grid.y); those add their int32 partials into a workspace with atomics
// (exact, order-free) and the last one to arrive, found with a per-tile
// counter, applies the epilogue and zeroes the workspace tile and counter
// behind it.  Token rows beyond 16 are handled by grid.z blocks of 16 rows.
#include "common.h"

namespace w8a8 {

struct GemmArgs {
  const int8_t* xq;
  const float* xs;
  const int8_t* wq;
  const float* ws;
  int M, N, K;
  int split;
  int tiles;  // number of workgroup column tiles (grid.x)
  uint16_t* y_bf16;
  float* y_f32;
  int32_t* acc;
  int32_t* part;    // [M][N] int32 split-K workspace (zero between calls)
  uint32_t* count;  // [grid.z][tiles] arrival counters (zero between calls)
};

__device__ __forceinline__ void epilogue_store(const GemmArgs& g, int m, int n, int32_t a) {
  const float y = (static_cast<float>(a) * g.xs[m]) * g.ws[n];
  const size_t o = (size_t)m * (size_t)g.N + (size_t)n;
  if (g.y_f32) g.y_f32[o] = y;
  if (g.y_bf16) g.y_bf16[o] = f32_to_bf16_rne(y);
  if (g.acc) g.acc[o] = a;
}

__device__ __forceinline__ v4i load16(const int8_t* p) {
  return *reinterpret_cast<const v4i*>(p);
}

template <int TN, int WAVES, int U>
__global__ __launch_bounds__(WAVES * kWave) void gemm_w8a8_skinny(GemmArgs g) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int tile = blockIdx.x;
  const int m_base = blockIdx.z * 16;
  const int n0 = tile * 16 * TN;
  const int K = g.K;
  const int steps = (K + 63) >> 6;

  // this workgroup's k-steps [g0, g1), then this wave's [s0, s1)
  const int g0 = (int)(((int64_t)steps * blockIdx.y) / g.split);
  const int g1 = (int)(((int64_t)steps * (blockIdx.y + 1)) / g.split);
  const int s0 = g0 + (int)(((int64_t)(g1 - g0) * wave) / WAVES);
  const int s1 = g0 + (int)(((int64_t)(g1 - g0) * (wave + 1)) / WAVES);

  const int m_a = m_base + col;
  const bool a_ok = m_a < g.M;
  const int8_t* a_ptr = g.xq + (size_t)(a_ok ? m_a : 0) * (size_t)K + grp * 16;
  const int8_t* b_ptr[TN];
  bool b_ok[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + col;
    b_ok[t] = n < g.N;
    b_ptr[t] = g.wq + (size_t)(b_ok[t] ? n : 0) * (size_t)K + grp * 16;
  }

  v4i acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = v4i{0, 0, 0, 0};

  const v4i zero = v4i{0, 0, 0, 0};
  int s = s0;
  for (; s + U <= s1; s += U) {
    v4i a[U], b[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s + u) * 64;
      const bool kin = k + grp * 16 < K;
      a[u] = (a_ok && kin) ? load16(a_ptr + k) : zero;
#pragma unroll
      for (int t = 0; t < TN; ++t) b[u][t] = (b_ok[t] && kin) ? load16(b_ptr[t] + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][t], acc[t], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const int k = s * 64;
    const bool kin = k + grp * 16 < K;
    const v4i a = (a_ok && kin) ? load16(a_ptr + k) : zero;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const v4i b = (b_ok[t] && kin) ? load16(b_ptr[t] + k) : zero;
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
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

  // wave 0 holds the workgroup's partial tile: rows 4*grp + r, column col.
  if (g.split == 1) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n = n0 + 16 * t + col;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m_base + 4 * grp + r;
        if (m < g.M) epilogue_store(g, m, n, acc[t][r]);
      }
    }
    return;
  }

#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + col;
    if (n >= g.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + 4 * grp + r;
      if (m < g.M) atomicAdd(&g.part[(size_t)m * g.N + n], acc[t][r]);
    }
  }
  __threadfence();
  uint32_t* counter = &g.count[(size_t)blockIdx.z * g.tiles + tile];
  uint32_t old = 0;
  if (lane == 0) old = atomicAdd(counter, 1u);
  old = __shfl(old, 0, kWave);
  if (old != (uint32_t)(g.split - 1)) return;
  __threadfence();
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + col;
    if (n >= g.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + 4 * grp + r;
      if (m < g.M) {
        const int32_t total = atomicExch(&g.part[(size_t)m * g.N + n], 0);
        epilogue_store(g, m, n, total);
      }
    }
  }
  if (lane == 0) atomicExch(counter, 0u);
}

// Launch shape: (tiles, split, mblocks) workgroups of WAVES waves.
struct SkinnyPlan {
  int tiles, split, mblocks;
};

constexpr int kTN = 1;
constexpr int kWaves = 4;
constexpr int kUnroll = 8;
constexpr int kTargetWorkgroups = 1024;  // 4 per CU on 256 CUs

static SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K) {
  SkinnyPlan p;
  p.tiles = (int)((N + 16 * kTN - 1) / (16 * kTN));
  p.mblocks = (int)((M + 15) / 16);
  const int64_t steps = (K + 63) / 64;
  p.split = 1;
  while ((int64_t)p.tiles * p.mblocks * p.split < kTargetWorkgroups &&
         steps / ((int64_t)p.split * 2 * kWaves) >= 2)
    p.split *= 2;
  return p;
}

}  // namespace w8a8

size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  using namespace w8a8;
  if (M <= 0 || N <= 0) return 0;
  const SkinnyPlan p = plan_skinny(M, N, K);
  if (p.split == 1) return 0;
  const size_t part = (size_t)M * (size_t)N * sizeof(int32_t);
  const size_t part_aligned = (part + 255) & ~(size_t)255;
  return part_aligned + (size_t)p.tiles * p.mblocks * sizeof(uint32_t);
}

hipError_t w8a8_launch_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, int64_t M, int64_t N, int64_t K,
                            uint16_t* y_bf16, float* y_f32, int32_t* acc,
                            void* workspace, hipStream_t stream) {
  using namespace w8a8;
  if (M == 0 || N == 0) return hipSuccess;
  const SkinnyPlan p = plan_skinny(M, N, K);
  GemmArgs g;
  g.xq = xq; g.xs = x_scale; g.wq = wq; g.ws = w_scale;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.split = p.split; g.tiles = p.tiles;
  g.y_bf16 = y_bf16; g.y_f32 = y_f32; g.acc = acc;
  g.part = nullptr; g.count = nullptr;
  if (p.split > 1) {
    const size_t part = (size_t)M * (size_t)N * sizeof(int32_t);
    g.part = reinterpret_cast<int32_t*>(workspace);
    g.count = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(workspace) +
                                          ((part + 255) & ~(size_t)255));
  }
  const dim3 grid((unsigned)p.tiles, (unsigned)p.split, (unsigned)p.mblocks);
  const dim3 block(kWaves * kWave);
  hipLaunchKernelGGL((gemm_w8a8_skinny<kTN, kWaves, kUnroll>), grid, block, 0, stream, g);
  return hipGetLastError();
}
