// Batched W8A8 linear for gfx950 (more than 16 token rows, e.g. 32
// sequences x (8 drafts + 1) = 288 rows): the same arithmetic as the skinny
// kernel — acc = sum_k xq[m][k]*wq[n][k] exact in int32 on
// v_mfma_i32_16x16x64_i8, y32 = (acc*x_scale[m])*w_scale[n], y = bf16(y32)
// (gist.science Japanese summary, 技術的サマリー §2.2 item 3) — organised
// for the point where the product stops being a pure weight stream: at
// M = 288 it does ~576 int-ops per weight byte, close to the MI355X ridge.
//
// Workgroup tile: WAVES x MB row blocks of 16 token rows x TN channel tiles
// of 16.  Wave w owns MB row blocks of the tile over the whole K: per
// 64-wide k step it loads its MB activation fragments and the TN weight
// fragments, then issues MB x TN MFMAs (each loaded fragment feeds several
// MFMAs from registers); U steps of loads are in flight before their
// MFMAs.  The waves of a workgroup read the same weight blocks at
// about the same time, so one HBM fetch serves them through L1/L2 (cached
// loads here, not the skinny kernel's non-temporal stream).  No LDS, no
// barrier; each wave writes its own rows.  Pairing of A and B k-positions
// inside an MFMA is as in the skinny kernel (lane l of both operands holds
// k = 64*step + 16*(l>>4) .. +15).
//
// The workgroups that share a set of weight tiles (the row tiles) are given
// ids that the dispatcher sends to the same XCD back to back (ids differ by
// multiples of 8), so the later reads of a weight block come from that
// XCD's L2 rather than HBM.  With few tiles the k loop is latency-bound
// (each wave waits about a microsecond per round of loads), so K is split
// across workgroups (grid.y) until the grid holds ~3 waves per SIMD; the
// int32 partials meet through the same atomic handoff as the skinny
// kernel's split-K.
#include "common.h"

#include <climits>

namespace w8a8 {

constexpr int kXcds = 8;

struct BatchedArgs {
  const int8_t* xq;
  const float* xs;
  const int8_t* wq;
  const float* ws;
  int M, N, K;
  int steps;    // ceil(K / 64)
  int tiles16;  // ceil(N / 16)
  int ngroups;  // ceil(tiles16 / TN): workgroup channel groups
  int mtiles;   // ceil(M / (16*WAVES)): workgroup row tiles
  uint16_t* y_bf16;
  float* y_f32;
  int32_t* acc;
  unsigned long long* keys;  // fused argmax sub-keys (as in the skinny kernel), or null
  int subkeys, key_stride;
  int split;        // k ranges per tile (grid.y)
  int32_t* part;    // [M][N] split-K partial sums (zero between calls) when split > 1
  uint32_t* count;  // [mtiles * ngroups] arrival counters (zero between calls)
};

__device__ __forceinline__ unsigned long long batched_argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(~(uint32_t)idx);
}

template <int MB, int TN, int WAVES, int U, bool kTiled, bool kArgmax>
__global__ __launch_bounds__(WAVES * kWave) void gemm_w8a8_batched(BatchedArgs g) {
  // workgroup id -> (row tile, channel group), XCD-aware (see header)
  const int b = blockIdx.x;
  const int xcd = b % kXcds;
  const int slot = b / kXcds;
  const int mt = slot % g.mtiles;
  const int ng = (slot / g.mtiles) * kXcds + xcd;
  if (ng >= g.ngroups) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int mb0 = (mt * WAVES + wave) * MB;     // this wave's first row block
  const bool live = mb0 * 16 < g.M;             // some of its rows are real
  if (!live && g.split == 1) return;            // (with split > 1 it still meets the barrier)
  const int K = g.K;
  const int steps = g.steps;
  const int col = lane & 15, grp = lane >> 4;
  // this workgroup's k steps [k0, k1)
  const int k0 = (int)(((int64_t)steps * blockIdx.y) / g.split);
  const int k1 = (int)(((int64_t)steps * (blockIdx.y + 1)) / g.split);
  const int nk = live ? k1 - k0 : 0;

  const int8_t* a_ptr[MB];
  bool a_ok[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m_a = (mb0 + i) * 16 + col;
    a_ok[i] = m_a < g.M;
    a_ptr[i] = g.xq + (size_t)(a_ok[i] ? m_a : 0) * (size_t)K + grp * 16;
  }
  const int8_t* b_ptr[TN];
  bool b_ok[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int t16 = ng * TN + t;
    if constexpr (kTiled) {
      b_ok[t] = t16 < g.tiles16;
      b_ptr[t] = g.wq + ((size_t)(b_ok[t] ? t16 : 0) * (size_t)steps << 10) + (lane << 4);
    } else {
      const int n = t16 * 16 + col;
      b_ok[t] = n < g.N;
      b_ptr[t] = g.wq + (size_t)(b_ok[t] ? n : 0) * (size_t)K + grp * 16;
    }
  }
  const v4i zero = v4i{0, 0, 0, 0};
  auto load_b = [&](int t, int s) -> v4i {
    if constexpr (kTiled) {
      return b_ok[t] ? *reinterpret_cast<const v4i*>(b_ptr[t] + ((size_t)s << 10)) : zero;
    } else {
      return (b_ok[t] && s * 64 + grp * 16 < K)
                 ? *reinterpret_cast<const v4i*>(b_ptr[t] + (size_t)s * 64) : zero;
    }
  };

  auto load_a = [&](int i, int s) -> v4i {
    const int k = s * 64 + grp * 16;
    return (a_ok[i] && k < K) ? *reinterpret_cast<const v4i*>(a_ptr[i] + (size_t)s * 64) : zero;
  };
  // Each workgroup walks the k steps from its own starting point (int32
  // sums are exact in any order).  Row-major activations put every row's
  // fragment of a given k step at the same address modulo the row pitch, so
  // workgroups marching in lockstep would all hit the same memory channel.
  const int rot = (int)(((int64_t)b * 4) % (nk > 0 ? nk : 1));
  auto kstep = [&](int s) { const int e = s + rot; return k0 + (e >= nk ? e - nk : e); };

  v4i acc[MB][TN];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = zero;

  int s = 0;
  for (; s + U <= nk; s += U) {
    v4i a[U][MB], bb[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int se = kstep(s + u);
#pragma unroll
      for (int i = 0; i < MB; ++i) a[u][i] = load_a(i, se);
#pragma unroll
      for (int t = 0; t < TN; ++t) bb[u][t] = load_b(t, se);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][i], bb[u][t], acc[i][t], 0, 0, 0);
  }
  for (; s < nk; ++s) {
    v4i a[MB], bb[TN];
    const int se = kstep(s);
#pragma unroll
    for (int i = 0; i < MB; ++i) a[i] = load_a(i, se);
#pragma unroll
    for (int t = 0; t < TN; ++t) bb[t] = load_b(t, se);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bb[t], acc[i][t], 0, 0, 0);
  }

  if (g.split > 1) {
    // Split-K handoff, as in the skinny kernel: device-scope atomic adds of
    // the partial tile, a wait for their completion, one arrival count per
    // workgroup; the last arriver takes the totals with atomic exchanges
    // (leaving zeros) and applies the epilogue.
    if (live) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int n = (ng * TN + t) * 16 + col;
        if (n >= g.N) continue;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = (mb0 + i) * 16 + 4 * grp + r;
            if (m < g.M)
              __hip_atomic_fetch_add(&g.part[(size_t)m * g.N + n], acc[i][t][r], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __shared__ uint32_t arrived;
    __syncthreads();
    uint32_t* counter = &g.count[(size_t)mt * g.ngroups + ng];
    if (threadIdx.x == 0)
      arrived = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != (uint32_t)(g.split - 1)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (threadIdx.x == 0)
      __hip_atomic_exchange(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!live) return;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n = (ng * TN + t) * 16 + col;
      if (n >= g.N) continue;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = (mb0 + i) * 16 + 4 * grp + r;
          if (m < g.M)
            acc[i][t][r] = __hip_atomic_exchange(&g.part[(size_t)m * g.N + n], 0,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
  }

  // epilogue: rows (mb0+i)*16 + 4*grp + r, columns (ng*TN + t)*16 + col
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int t16 = ng * TN + t;
    const int n = t16 * 16 + col;
    const bool n_ok = n < g.N;
    const float wsn = n_ok ? g.ws[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = (mb0 + i) * 16 + 4 * grp + r;
        float v = -INFINITY;
        int idx = INT_MAX;
        if (m < g.M && n_ok) {
          const int32_t a = acc[i][t][r];
          const float y = (static_cast<float>(a) * g.xs[m]) * wsn;
          const size_t o = (size_t)m * (size_t)g.N + (size_t)n;
          if (g.y_f32) g.y_f32[o] = y;
          if (g.y_bf16) g.y_bf16[o] = f32_to_bf16_rne(y);
          if (g.acc) g.acc[o] = a;
          v = y;
          idx = n;
        }
        if constexpr (kArgmax) {
          // (max, lowest index) of row m over this tile's 16 columns, then one
          // atomic fold into the row's sub-key for this tile
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) {
            const float ov = __shfl_xor(v, off, kWave);
            const int oi = __shfl_xor(idx, off, kWave);
            if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
          }
          if (col == 0 && m < g.M && idx != INT_MAX) {
            const size_t sub = (size_t)m * g.subkeys + (t16 % g.subkeys);
            __hip_atomic_fetch_max(&g.keys[sub * g.key_stride], batched_argmax_key(v, idx),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  }
}

constexpr int kBMB = 3;     // row blocks of 16 per wave
constexpr int kBTN = 2;     // channel tiles of 16 per workgroup
constexpr int kBWaves = 2;  // waves per workgroup (they split the rows)
constexpr int kBU = 4;      // k steps of loads in flight per wave
// Split k until the grid has this many waves.  Measured on MI355X at 288
// rows the split costs more in atomics than it gains in waves, so it is off.
constexpr int64_t kBTargetWaves = 0;

struct BatchedPlan {
  int ngroups, mtiles, split;
};

static BatchedPlan plan_batched(int64_t M, int64_t N, int64_t K, bool no_split) {
  BatchedPlan p;
  const int64_t tiles16 = (N + 15) / 16;
  p.ngroups = (int)((tiles16 + kBTN - 1) / kBTN);
  p.mtiles = (int)((M + 16 * kBMB * kBWaves - 1) / (16 * kBMB * kBWaves));
  const int64_t steps = (K + 63) / 64;
  const int64_t waves = (int64_t)p.ngroups * p.mtiles * kBWaves;
  p.split = 1;
  // more workgroups in flight: the k loop is latency-bound with few waves
  while (!no_split && waves * p.split < kBTargetWaves && steps / (p.split * 2) >= 8) p.split *= 2;
  return p;
}

}  // namespace w8a8

size_t w8a8_gemm_batched_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  using namespace w8a8;
  if (M <= 0 || N <= 0) return 0;
  const BatchedPlan p = plan_batched(M, N, K, false);
  if (p.split == 1) return 0;
  const size_t part = ((size_t)M * (size_t)N * sizeof(int32_t) + 255) & ~(size_t)255;
  return part + (size_t)p.mtiles * p.ngroups * sizeof(uint32_t);
}

hipError_t w8a8_launch_gemm_batched(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, int64_t M, int64_t N, int64_t K,
                                    bool tiled, uint16_t* y_bf16, float* y_f32, int32_t* acc,
                                    void* keys, int subkeys, int key_stride, void* workspace,
                                    hipStream_t stream) {
  using namespace w8a8;
  if (M == 0 || N == 0) return hipSuccess;
  const BatchedPlan p = plan_batched(M, N, K, workspace == nullptr);
  BatchedArgs g{};
  g.xq = xq; g.xs = x_scale; g.wq = wq; g.ws = w_scale;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.steps = (int)((K + 63) / 64);
  g.tiles16 = (int)((N + 15) / 16);
  g.ngroups = p.ngroups;
  g.mtiles = p.mtiles;
  g.y_bf16 = y_bf16; g.y_f32 = y_f32; g.acc = acc;
  g.keys = reinterpret_cast<unsigned long long*>(keys);
  g.subkeys = subkeys; g.key_stride = key_stride;
  g.split = p.split;
  if (p.split > 1) {
    const size_t part = ((size_t)M * (size_t)N * sizeof(int32_t) + 255) & ~(size_t)255;
    g.part = reinterpret_cast<int32_t*>(workspace);
    g.count = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(workspace) + part);
  }
  // grid: channel groups rounded up to a multiple of the XCD count, times row
  // tiles; grid.y: k ranges
  const int64_t ng_padded = ((int64_t)g.ngroups + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)(ng_padded * g.mtiles), (unsigned)p.split), block(kBWaves * kWave);
#define W8A8_BATCHED(TL, AM)                                                                    \
  hipLaunchKernelGGL((gemm_w8a8_batched<kBMB, kBTN, kBWaves, kBU, TL, AM>), grid, block, 0, \
                     stream, g)
  if (keys) {
    if (tiled) W8A8_BATCHED(true, true);
    else W8A8_BATCHED(false, true);
  } else {
    if (tiled) W8A8_BATCHED(true, false);
    else W8A8_BATCHED(false, false);
  }
#undef W8A8_BATCHED
  return hipGetLastError();
}
