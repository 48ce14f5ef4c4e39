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
// Two weight layouts:
//  * row-major [N][K]: one B load touches 16 rows x 64 bytes;
//  * tiled (see w8a8_quantize_weight_tiled): for each tile of 16 output
//    channels and each 64-wide k step, the 1 KiB the MFMA consumes is stored
//    contiguously in lane order, so every B load is one fully coalesced 1 KiB
//    read.  Tiles are zero-padded to 16 rows and K to a multiple of 64.
// Tiled weight loads are non-temporal (streamed once, kept out of the
// caches); that measured faster for the contiguous tiled stream and not for
// the row-major pattern, which keeps ordinary loads.
//
// Work split: a workgroup owns TN tiles of 16 output channels and one
// k-range; its WAVES waves share the k steps of that range, issue U steps of
// loads before their MFMAs, and reduce their partial tiles through LDS.
// When the output is too narrow to occupy the chip (a few dozen tiles), the
// k-range is also split across SPLIT workgroups (grid.y): they add their
// int32 partials into a workspace with atomics (exact, order-free) and the
// last one to arrive, found with a per-tile counter, applies the epilogue
// and zeroes the workspace tile and counter behind it.  More than 16 token
// rows go to the batched kernel (gemm_w8a8_batched.hip).
#include "common.h"

#include <hip/hip_ext.h>

#include <climits>
#include <cstdlib>

namespace w8a8 {

struct GemmArgs {
  const int8_t* xq;
  const float* xs;
  const int8_t* wq;
  const float* ws;
  int M, N, K;
  int steps;    // ceil(K / 64)
  int tiles16;  // ceil(N / 16): 16-channel tiles in the tiled weight layout
  int split;
  int tiles;  // number of workgroup column tiles
  int ntail;  // > 0: the last ntail tiles are split tsplit ways, the rest not (1-D grid)
  int tsplit;
  uint16_t* y_bf16;
  float* y_f32;
  int32_t* acc;
  int32_t* part;    // [M][N] int32 split-K workspace (zero between calls)
  uint32_t* count;  // [grid.z][tiles] arrival counters (zero between calls)
  unsigned long long* keys;  // fused argmax: packed (value, index) sub-keys, see
                             // kArgmaxSubkeys (zero before the call), or null
};

__device__ __forceinline__ float epilogue_store(const GemmArgs& g, int m, int n, int32_t a) {
  const float y = (static_cast<float>(a) * g.xs[m]) * g.ws[n];
  const size_t o = (size_t)m * (size_t)g.N + (size_t)n;
  if (g.y_f32) g.y_f32[o] = y;
  if (g.y_bf16) g.y_bf16[o] = f32_to_bf16_rne(y);
  if (g.acc) g.acc[o] = a;
  return y;
}

__device__ __forceinline__ v4i load16(const int8_t* p) {
  return *reinterpret_cast<const v4i*>(p);
}
__device__ __forceinline__ v4i load16_stream(const int8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

template <int TN, int WAVES, int U, bool kTiled, bool kArgmax>
__global__ __launch_bounds__(WAVES * kWave) void gemm_w8a8_skinny(GemmArgs g) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int col = lane & 15;
  const int grp = lane >> 4;
  // (tile, k slice, slices of that tile): grid (tiles, split, mblocks), or
  // with a split tail a 1-D grid whose first ntail*tsplit workgroups are the
  // tail tiles' slices (dispatched first, so that their hand-off overlaps
  // the whole tiles' streaming) and the rest the whole tiles
  int tile, slice, split;
  if (g.ntail > 0) {
    const int nt = g.ntail * g.tsplit;
    const int id = blockIdx.x;
    if (id < nt) {
      tile = g.tiles - g.ntail + id / g.tsplit;
      slice = id % g.tsplit;
      split = g.tsplit;
    } else {
      tile = id - nt;
      slice = 0;
      split = 1;
    }
  } else {
    tile = blockIdx.x;
    slice = blockIdx.y;
    split = g.split;
  }
  const int m_base = blockIdx.z * 16;
  const int n0 = tile * 16 * TN;
  const int K = g.K;
  const int steps = g.steps;

  // this workgroup's k steps [g0, g1).  Tiled weights: the waves take them
  // round-robin (s = g0 + wave + WAVES*j), so the workgroup sweeps adjacent
  // KiB blocks.  Row-major weights: each wave takes a contiguous share
  // (s = sw + j), so each of its loads continues the same 16 rows.
  const int g0 = (int)(((int64_t)steps * slice) / split);
  const int g1 = (int)(((int64_t)steps * (slice + 1)) / split);
  int J, sw;
  constexpr int kStride = kTiled ? WAVES : 1;
  if constexpr (kTiled) {
    J = (g1 - g0 > wave) ? (g1 - g0 - wave + WAVES - 1) / WAVES : 0;
    sw = g0 + wave;
  } else {
    sw = g0 + (int)(((int64_t)(g1 - g0) * wave) / WAVES);
    J = g0 + (int)(((int64_t)(g1 - g0) * (wave + 1)) / WAVES) - sw;
  }

  const int m_a = m_base + col;
  const bool a_ok = m_a < g.M;
  const int8_t* a_ptr = g.xq + (size_t)(a_ok ? m_a : 0) * (size_t)K + grp * 16;
  const int8_t* b_ptr[TN];
  bool b_ok[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    if constexpr (kTiled) {
      const int t16 = tile * TN + t;
      b_ok[t] = t16 < g.tiles16;
      b_ptr[t] = g.wq + ((size_t)(b_ok[t] ? t16 : 0) * (size_t)steps << 10) + (lane << 4);
    } else {
      const int n = n0 + 16 * t + col;
      b_ok[t] = n < g.N;
      b_ptr[t] = g.wq + (size_t)(b_ok[t] ? n : 0) * (size_t)K + grp * 16;
    }
  }
  // byte offset of k step s inside a B stream
  auto b_off = [](int s) -> size_t { return kTiled ? ((size_t)s << 10) : (size_t)s * 64; };

  v4i acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = v4i{0, 0, 0, 0};

  const v4i zero = v4i{0, 0, 0, 0};
  int j = 0;
  for (; j + U <= J; j += U) {
    v4i a[U], b[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = sw + kStride * (j + u);
      const int k = s * 64;
      const bool kin = k + grp * 16 < K;
      a[u] = (a_ok && kin) ? load16(a_ptr + k) : zero;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        if constexpr (kTiled) b[u][t] = (TN == 1 || b_ok[t]) ? load16_stream(b_ptr[t] + b_off(s)) : zero;
        else b[u][t] = (b_ok[t] && kin) ? load16(b_ptr[t] + b_off(s)) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][t], acc[t], 0, 0, 0);
  }
  if (j < J) {
    // the last J - j < U steps, requested together (one round trip); the
    // slots past J load nothing and multiply zeros, which add nothing
    v4i a[U], b[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = j + u < J;
      const int s = sw + kStride * (live ? j + u : j);
      const int k = s * 64;
      const bool kin = k + grp * 16 < K;
      a[u] = (live && a_ok && kin) ? load16(a_ptr + k) : zero;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        if constexpr (kTiled) b[u][t] = (live && (TN == 1 || b_ok[t])) ? load16_stream(b_ptr[t] + b_off(s)) : zero;
        else b[u][t] = (live && b_ok[t] && kin) ? load16(b_ptr[t] + b_off(s)) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][t], acc[t], 0, 0, 0);
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
  if (split == 1) {
    float bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    int bi[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int n = n0 + 16 * t + col;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m_base + 4 * grp + r;
        if (m < g.M) {
          const float y = epilogue_store(g, m, n, acc[t][r]);
          if constexpr (kArgmax) {
            if (y > bv[r]) { bv[r] = y; bi[r] = n; }  // t ascending: first maximum kept
          }
        }
      }
    }
    if constexpr (kArgmax) {
      // fused LM-head argmax: (max, lowest index) of each row over this
      // workgroup's columns, reduced over the 16 lanes that share the row
      // group (lane bits 0..3), then folded into one of the row's sub-keys
      // with one device-scope atomic max (performed at the coherence point,
      // so the acceptance kernel that follows sees every workgroup's fold)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float ov = __shfl_xor(bv[r], off, kWave);
          const int oi = __shfl_xor(bi[r], off, kWave);
          if (ov > bv[r] || (ov == bv[r] && oi < bi[r])) { bv[r] = ov; bi[r] = oi; }
        }
        const int m = m_base + 4 * grp + r;
        if (col == 0 && m < g.M) {
          const size_t sub = (size_t)m * kArgmaxSubkeys + (tile % kArgmaxSubkeys);
          __hip_atomic_fetch_max(&g.keys[sub * kArgmaxKeyStride], argmax_key(bv[r], bi[r]),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    return;
  }

  // Split-K handoff.  Every exchange goes through device-scope atomic
  // read-modify-writes, which the hardware performs at one coherence point
  // per address, so no cache write-back or invalidate (an agent-scope fence)
  // is needed: the wave waits for its partial adds to complete (vmcnt(0))
  // before lane 0 adds to the arrival counter, and the last arriver reads the
  // totals with atomic exchanges issued after its counter add returned.
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + col;
    if (n >= g.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + 4 * grp + r;
      if (m < g.M)
        __hip_atomic_fetch_add(&g.part[(size_t)m * g.N + n], acc[t][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // wait until this wave's adds have returned before counting the arrival
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  uint32_t* counter = &g.count[(size_t)blockIdx.z * g.tiles + tile];
  uint32_t old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, kWave);
  if (old != (uint32_t)(split - 1)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + col;
    if (n >= g.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m_base + 4 * grp + r;
      if (m < g.M) {
        const int32_t total = __hip_atomic_exchange(&g.part[(size_t)m * g.N + n], 0,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        epilogue_store(g, m, n, total);
      }
    }
  }
  if (lane == 0)
    __hip_atomic_exchange(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Launch shape: (tiles, split, mblocks) workgroups of `waves` waves, each
// owning tn 16-channel tiles.
struct SkinnyPlan {
  int tiles, split, mblocks, waves, tn;
  int ntail = 0, tsplit = 1;  // split tail (see plan_skinny)
};

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// k steps of loads issued per wave before their MFMAs.  Measured on the
// LM head at M = 5 (same box, interleaved builds): 4: 97.8 us, 6: 97.0,
// 8: 96.3-96.9, 10: 95.1-95.5 (three waves per SIMD), 12: 107 and 16: 101
// (two waves per SIMD).  10 everywhere cost the mid-size shapes their
// fourth wave per SIMD (gate/up 12288 x 4096 at M = 5: 12.5 against 10.7
// us; the Qwen3-32B stack 7.80 against 7.37 ms), so only the LM head's
// fused-argmax kernel takes 10.
#ifndef W8A8_SKINNY_UNROLL
#define W8A8_SKINNY_UNROLL 8
#endif
constexpr int kUnroll = W8A8_SKINNY_UNROLL;
constexpr int kUnrollArgmax = 10;
constexpr int64_t kSkinnyMaxRows = 16;  // more token rows go to the batched kernel
constexpr int kSplitBelowTiles = 32;  // split k across workgroups below this ...
constexpr int64_t kLongChain = 32;    // ... or above this many k steps per wave
constexpr int64_t kTailMinSteps = 80; // split tail only for tiles this long (see plan_skinny)

// Tuning overrides (results do not depend on them: int32 sums are exact in
// any order): W8A8_SPLITK forces the cross-workgroup split, W8A8_WAVES the
// waves per workgroup (4, 8 or 16).  Read on every call.
static int env_int(const char* name) {
  const char* v = getenv(name);
  return v ? atoi(v) : 0;
}

// Measured on MI355X at M=5 over the Qwen3-8B shapes (N = 1024..12288, K =
// 4096/12288), at M=8 over the Qwen3-32B shapes (K up to 25600) and on the
// LM head, sweeping tiles per workgroup, waves and slices: on the tiled
// layout 4 waves per workgroup with two tiles each (>= 2048 tiles: the LM
// heads, the 32B gate/up), 8 waves with one tile (Qwen3-8B gate/up at M=5:
// 17.3 against 17.8-19.1 us with 4 waves; 32B q/k/v at M=8: 13.1 against
// 13.3 us).  Splitting k across workgroups (its atomic handoff) pays only
// for outputs too narrow to occupy more than a few dozen CUs and for long
// reductions over no more tiles than CUs; once a wave would walk more than
// 32 k steps, the split goes on until it walks at most 16 (the 8B down at
// M=5, 24 steps per wave, is fastest unsplit).  Outputs with more tiles
// than CUs split only the tiles past the last whole round (the split tail):
// the 32B down, 5120 x 25600 with 400 steps per tile, took 37.2 us unsplit
// before that tail, 31.2 with 2 slices, 27.2-27.8 with 4, and 26.1 with
// the tail.
static SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, bool tiled, bool no_split = false) {
  SkinnyPlan p;
  const int64_t tiles16 = (N + 15) / 16;
  p.mblocks = (int)((M + 15) / 16);
  // two tiles per workgroup halve the activation loads per weight byte; it
  // pays on the tiled layout once there are enough tiles to go round
  p.tn = (tiled && tiles16 * p.mblocks >= 2048) ? 2 : 1;
  const int fn = env_int("W8A8_TN");
  if (fn == 1 || fn == 2) p.tn = fn;
  p.tiles = (int)((tiles16 + p.tn - 1) / p.tn);
  const int64_t steps = (K + 63) / 64;
  const int64_t wgs = (int64_t)p.tiles * p.mblocks;
  p.waves = (wgs >= 512 && (p.tn == 2 || !tiled)) ? 4 : (wgs >= kSplitBelowTiles ? 8 : 16);
  p.split = 1;
  while (!no_split && wgs * p.split < kSplitBelowTiles &&
         steps / ((int64_t)p.split * 2 * p.waves) >= 2)
    p.split *= 2;
  // long reductions over few tiles: more than kLongChain k steps per wave is
  // a chain of dependent round trips that the grid cannot hide, so K is cut
  // across workgroups until a wave walks at most about half of that.  With
  // more tiles than CUs the split tail below balances the CUs instead and
  // the long chains overlap across the grid (32B down, 320 tiles of 400
  // steps: 26.1 us unsplit with the tail against 27.8 with four slices)
  if (!no_split && steps / ((int64_t)p.split * p.waves) > kLongChain &&
      (int64_t)p.tiles * p.mblocks <= cu_count())
    while (p.split < 8 && steps / ((int64_t)p.split * p.waves) > kLongChain / 2) p.split *= 2;
  const int fw = env_int("W8A8_WAVES");
  if (fw == 4 || fw == 8 || fw == 16) p.waves = fw;
  const int fs = env_int("W8A8_SPLITK");
  if (!no_split && fs >= 1 && fs <= 64 && fs <= steps) p.split = fs;
  // Split tail: one CU streams little more than its share of HBM, so when
  // the tiles do not divide evenly over the CUs, the CUs that get one tile
  // more set the time (the Qwen3-32B o at M = 8: 320 tiles of 128 KiB over
  // 256 CUs, 64 of them stream two).  The remainder tiles are then cut into
  // tsplit k slices, about one per CU, with the atomic hand-off of the
  // split; their workgroups go first, so that the hand-off overlaps the
  // whole tiles' streaming.  Measured on MI355X (M = 8, graph-timed): 32B o
  // 12.68 -> 10.63 us, q/k/v (10240 x 5120) 13.06 -> 12.61, gate/up
  // (51200 x 5120) 46.1 -> 45.1.  It pays only for long tiles (>= 80 k
  // steps): at K = 4096 the hand-off costs more than the uneven round
  // (Qwen3-8B q/k/v at M = 5: 7.48 -> 7.73 us), and it needs whole tiles to
  // overlap (a 64-tile output split four ways: 4.63 -> 6.35 us).
  // W8A8_TAIL=-1 turns it off (a tuning override; results are exact either
  // way).
  if (!no_split && p.split == 1 && p.mblocks == 1 && steps >= kTailMinSteps &&
      env_int("W8A8_TAIL") >= 0) {
    const int cus = cu_count();
    const int rem = p.tiles > cus ? p.tiles % cus : 0;
    int ts = 1;
    while (rem > 0 && ts < 8 && rem * ts * 2 <= cus && ts * 2 <= steps) ts *= 2;
    if (ts > 1) {
      p.ntail = rem;
      p.tsplit = ts;
    }
  }
  return p;
}

}  // namespace w8a8

size_t w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, bool tiled) {
  using namespace w8a8;
  if (M <= 0 || N <= 0) return 0;
  if (M > kSkinnyMaxRows) return tiled ? w8a8_batched_workspace_bytes(M, N, K, false) : 0;
  const SkinnyPlan p = plan_skinny(M, N, K, tiled);
  if (p.split == 1 && p.ntail == 0) return 0;
  const size_t part = (size_t)M * (size_t)N * sizeof(int32_t);
  const size_t part_aligned = (part + 255) & ~(size_t)255;
  return part_aligned + (size_t)p.tiles * p.mblocks * sizeof(uint32_t);
}

// With ev0/ev1 set, the launch goes through hipExtLaunchKernel, which
// records the kernel's own start and end timestamps into the two events.
static hipError_t launch_plan(const w8a8::SkinnyPlan& p, const w8a8::GemmArgs& g, bool tiled,
                              bool argmax, hipStream_t stream, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr) {
  using namespace w8a8;
  const dim3 grid = p.ntail > 0
                        ? dim3((unsigned)(p.ntail * p.tsplit + p.tiles - p.ntail), 1u, (unsigned)p.mblocks)
                        : dim3((unsigned)p.tiles, (unsigned)p.split, (unsigned)p.mblocks);
#define W8A8_GEMM(TN, W, TL, AM)                                                              \
  do {                                                                                        \
    if (ev0)                                                                                  \
      hipExtLaunchKernelGGL((gemm_w8a8_skinny<TN, W, (AM ? kUnrollArgmax : kUnroll), TL, AM>),  \
                            grid, dim3(W * kWave), 0, stream, ev0, ev1, 0, g);               \
    else                                                                                      \
      hipLaunchKernelGGL((gemm_w8a8_skinny<TN, W, (AM ? kUnrollArgmax : kUnroll), TL, AM>),     \
                         grid, dim3(W * kWave), 0, stream, g);                                \
  } while (0)
#define W8A8_GEMM_W(TN, TL, AM)                   \
  do {                                            \
    if (p.waves == 4) W8A8_GEMM(TN, 4, TL, AM);   \
    else if (p.waves == 8) W8A8_GEMM(TN, 8, TL, AM); \
    else W8A8_GEMM(TN, 16, TL, AM);               \
  } while (0)
  if (argmax) {
    if (p.tn == 2) W8A8_GEMM_W(2, true, true);
    else W8A8_GEMM_W(1, true, true);
  } else if (tiled) {
    if (p.tn == 2) W8A8_GEMM_W(2, true, false);
    else W8A8_GEMM_W(1, true, false);
  } else {
    W8A8_GEMM_W(1, false, false);
  }
#undef W8A8_GEMM_W
#undef W8A8_GEMM
  return hipGetLastError();
}

static w8a8::GemmArgs make_args(const w8a8::SkinnyPlan& p, const int8_t* xq, const float* x_scale,
                                const int8_t* wq, const float* w_scale, int64_t M, int64_t N,
                                int64_t K, uint16_t* y_bf16, float* y_f32, int32_t* acc) {
  w8a8::GemmArgs g{};
  g.xq = xq; g.xs = x_scale; g.wq = wq; g.ws = w_scale;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.steps = (int)((K + 63) / 64);
  g.tiles16 = (int)((N + 15) / 16);
  g.split = p.split; g.tiles = p.tiles;
  g.ntail = p.ntail; g.tsplit = p.tsplit;
  g.y_bf16 = y_bf16; g.y_f32 = y_f32; g.acc = acc;
  return g;
}

hipError_t w8a8_launch_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, int64_t M, int64_t N, int64_t K, bool tiled,
                            uint16_t* y_bf16, float* y_f32, int32_t* acc, void* workspace,
                            hipStream_t stream) {
  using namespace w8a8;
  if (M == 0 || N == 0) return hipSuccess;
  if (M > kSkinnyMaxRows)
    return w8a8_launch_gemm_batched(xq, x_scale, wq, w_scale, M, N, K, tiled, y_bf16, y_f32, acc,
                                    nullptr, 0, 0, stream, false, workspace);
  const SkinnyPlan p = plan_skinny(M, N, K, tiled);
  GemmArgs g = make_args(p, xq, x_scale, wq, w_scale, M, N, K, y_bf16, y_f32, acc);
  if (p.split > 1 || p.ntail > 0) {
    const size_t part = (size_t)M * (size_t)N * sizeof(int32_t);
    g.part = reinterpret_cast<int32_t*>(workspace);
    g.count = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(workspace) +
                                          ((part + 255) & ~(size_t)255));
  }
  return launch_plan(p, g, tiled, false, stream);
}

// LM head with the argmax fused into the epilogue: every workgroup folds
// its per-row maxima into one of each row's sub-keys; the acceptance kernel
// reads the sub-keys, resets them to zero and accepts the draft.
size_t w8a8_lm_head_workspace_bytes(int64_t M) {
  using namespace w8a8;
  if (M <= 0) return 0;
  return (size_t)M * kArgmaxSubkeys * kArgmaxKeyStride * sizeof(unsigned long long);
}

hipError_t w8a8_launch_lm_head_argmax(const int8_t* xq, const float* x_scale,
                                      const int8_t* wq_tiled, const float* w_scale, int64_t M,
                                      int64_t V, int64_t K, float* logits, void* keys,
                                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  using namespace w8a8;
  if (M == 0) return hipSuccess;
  if (M > kSkinnyMaxRows) {
    if (ev0 || ev1) return hipErrorNotSupported;  // kernel timestamps: skinny kernel only
    return w8a8_launch_gemm_batched(xq, x_scale, wq_tiled, w_scale, M, V, K, true, nullptr, logits,
                                    nullptr, keys, kArgmaxSubkeys, kArgmaxKeyStride, stream);
  }
  const SkinnyPlan p = plan_skinny(M, V, K, true, true);
  GemmArgs g = make_args(p, xq, x_scale, wq_tiled, w_scale, M, V, K, nullptr, logits, nullptr);
  g.keys = reinterpret_cast<unsigned long long*>(keys);
  return launch_plan(p, g, true, true, stream, ev0, ev1);
}

hipError_t w8a8_launch_accept_from_keys(void* keys, const int32_t* draft, int64_t B, int64_t G,
                                        int32_t* argmax, int32_t* accept_len, int32_t* next_token,
                                        hipStream_t stream) {
  using namespace w8a8;
  return w8a8_launch_accept_keys(reinterpret_cast<unsigned long long*>(keys), kArgmaxSubkeys,
                                 kArgmaxKeyStride, draft, B, G, argmax, accept_len, next_token,
                                 stream);
}
