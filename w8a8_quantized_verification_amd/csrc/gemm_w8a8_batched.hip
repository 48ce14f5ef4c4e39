// Batched W8A8 linear for gfx950 (more than 16 token rows, e.g. 32
// sequences x (8 drafts + 1) = 288 rows): the same arithmetic as the skinny
// kernel — acc = sum_k xq[m][k]*wq[n][k] exact in int32 on
// v_mfma_i32_16x16x64_i8, y32 = (acc*x_scale[m])*w_scale[n], y = bf16(y32)
// (gist.science Japanese summary, 技術的サマリー §2.2 item 3) — organised
// for the point where the product stops being a pure weight stream: at
// M = 288 it does ~576 int-ops per weight byte, close to the MI355X ridge.
//
// Workgroup tile: WR x MB row blocks of 16 token rows x TN channel tiles of
// 16.  The workgroup's WR*KW waves form a WR x KW grid: wave (wr, wk) owns
// row blocks wr*MB .. wr*MB+MB-1 of the tile over the k steps of slice wk
// (K is cut into KW contiguous slices).  Per 64-wide k step a wave loads
// its MB activation fragments and TN weight fragments straight into
// registers, then issues MB x TN MFMAs (each loaded fragment feeds several
// MFMAs); U steps of loads are in flight before their MFMAs.  Cutting K
// across the waves of one workgroup shortens each wave's chain of
// dependent loads KW-fold without adding traffic: the chain length, not
// bandwidth, is what bounds this loop at a few waves per SIMD.  The KW
// partial int32 tiles meet in LDS once at the end (exact in any order), and
// the wk = 0 waves apply the epilogue.  Waves that share a weight fragment
// read it at about the same time, so one HBM fetch serves them through
// L1/L2 (cached loads here, not the skinny kernel's non-temporal stream).
// Pairing of A and B k-positions inside an MFMA is as in the skinny kernel
// (lane l of both operands holds k = 64*step + 16*(l>>4) .. +15).
//
// The workgroups that share a set of weight tiles (the row tiles) are given
// ids that the dispatcher sends to the same XCD back to back (ids differ by
// multiples of 8), so the later reads of a weight block come from that
// XCD's L2 rather than HBM.
#include "common.h"

#include <climits>

namespace w8a8 {

struct BatchedArgs {
  const int8_t* xq;
  const float* xs;
  const int8_t* wq;
  const float* ws;
  int M, N, K;
  int steps;    // ceil(K / 64)
  int tiles16;  // ceil(N / 16)
  int ngroups;  // ceil(tiles16 / TN): workgroup channel groups
  int mtiles;   // ceil(M / (16*MB*WR)): workgroup row tiles
  uint16_t* y_bf16;
  float* y_f32;
  int32_t* acc;
  unsigned long long* keys;  // fused argmax sub-keys (as in the skinny kernel), or null
  int subkeys, key_stride;
};

template <int MB, int TN, int WR, int KW, int U, bool kTiled, bool kArgmax, bool kTiledA>
__global__ __launch_bounds__(WR * KW * kWave) void gemm_w8a8_batched(BatchedArgs g) {
  // workgroup id -> (row tile, channel group), XCD-aware (see header)
  const int b = blockIdx.x;
  const int xcd = b % kXcds;
  const int slot = b / kXcds;
  const int mt = slot % g.mtiles;
  const int ng = (slot / g.mtiles) * kXcds + xcd;
  if (ng >= g.ngroups) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wr = wave % WR, wk = wave / WR;
  const int mb0 = (mt * WR + wr) * MB;          // this wave's first row block
  const bool live = mb0 * 16 < g.M;             // some of its rows are real
  if (!live && KW == 1) return;                 // (with KW > 1 it still meets the barrier)
  const int K = g.K;
  const int steps = g.steps;
  const int col = lane & 15, grp = lane >> 4;
  // this wave's k steps [k0, k0 + nk)
  const int k0 = (int)(((int64_t)steps * wk) / KW);
  const int nk = live ? (int)(((int64_t)steps * (wk + 1)) / KW) - k0 : 0;

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
    if constexpr (kTiledA) {
      // the activations' tiled layout (as the weights'): one 1 KiB block per
      // 16-row block and k step, padding rows zero
      return ((mb0 + i) * 16 < g.M)
                 ? *reinterpret_cast<const v4i*>(
                       g.xq + (((size_t)(mb0 + i) * (size_t)steps + (size_t)s) << 10) + (lane << 4))
                 : zero;
    } else {
      const int k = s * 64 + grp * 16;
      return (a_ok[i] && k < K) ? *reinterpret_cast<const v4i*>(a_ptr[i] + (size_t)s * 64) : zero;
    }
  };
  // Each channel group walks its k steps from its own starting point (int32
  // sums are exact in any order).  Row-major activations put every row's
  // fragment of a given k step at the same address modulo the row pitch, so
  // groups marching in lockstep would all hit the same memory channel.  The
  // row tiles of one channel group keep the same start, so they read each
  // weight block at about the same time and share one fetch of it in L2.
  const int rot = (int)(((int64_t)ng * 4) % (nk > 0 ? nk : 1));
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

  if constexpr (KW > 1) {
    // the k slices of each row group meet in LDS: waves wk > 0 store their
    // partial tiles (lane-contiguous 16-byte rows), the wk = 0 wave adds them
    __shared__ v4i red[KW - 1][WR][MB * TN][kWave];
    if (wk > 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) red[wk - 1][wr][i * TN + t][lane] = acc[i][t];
    }
    __syncthreads();
    if (wk > 0 || !live) return;
#pragma unroll
    for (int j = 0; j < KW - 1; ++j)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) acc[i][t] += red[j][wr][i * TN + t][lane];
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
            __hip_atomic_fetch_max(&g.keys[sub * g.key_stride], argmax_key(v, idx),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  }
}

// Launch shapes, measured on MI355X at 288 rows over the Qwen3-8B linears
// (tiled weights):
//  * row-major activations: 48 rows x 64 channels per workgroup with K in 4
//    slices; 48 x 32 with K in 8 slices when that leaves CUs idle (fewer
//    than 256 workgroups, e.g. N = 1024);
//  * tiled activations (each 16-row block's 64-wide k step one contiguous
//    KiB, as for the weights; 30% faster): 48 x 32 with K in 4 slices, or 8
//    slices below 256 workgroups.
struct BatchedShape {
  int mb, tn, wr, kw, u;
};
constexpr BatchedShape kWide{3, 4, 1, 4, 4};
constexpr BatchedShape kNarrow{3, 2, 1, 8, 2};
constexpr BatchedShape kTiledAWide{3, 2, 1, 4, 4};
constexpr int64_t kMinWorkgroups = 256;

static int64_t batched_workgroups(const BatchedShape& c, int64_t M, int64_t N) {
  const int64_t ngroups = ((N + 15) / 16 + c.tn - 1) / c.tn;
  const int64_t mtiles = (M + 16 * c.mb * c.wr - 1) / (16 * c.mb * c.wr);
  return ngroups * mtiles;
}

template <int MB, int TN, int WR, int KW, int U, bool TA>
static hipError_t launch_batched(BatchedArgs g, bool tiled, bool argmax, hipStream_t stream) {
  static_assert((KW - 1) * WR * MB * TN * 1024 <= 65536, "LDS reduction buffer");
  g.ngroups = (g.tiles16 + TN - 1) / TN;
  g.mtiles = (g.M + 16 * MB * WR - 1) / (16 * MB * WR);
  // grid: channel groups rounded up to a multiple of the XCD count, times row tiles
  const int64_t ng_padded = ((int64_t)g.ngroups + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)(ng_padded * g.mtiles)), block(WR * KW * kWave);
#define W8A8_B(TL, AM) \
  hipLaunchKernelGGL((gemm_w8a8_batched<MB, TN, WR, KW, U, TL, AM, TA>), grid, block, 0, stream, g)
  if (argmax) {
    if (tiled) W8A8_B(true, true);
    else W8A8_B(false, true);
  } else {
    if (tiled) W8A8_B(true, false);
    else W8A8_B(false, false);
  }
#undef W8A8_B
  return hipGetLastError();
}

}  // namespace w8a8

hipError_t w8a8_launch_gemm_batched(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, int64_t M, int64_t N, int64_t K,
                                    bool tiled, uint16_t* y_bf16, float* y_f32, int32_t* acc,
                                    void* keys, int subkeys, int key_stride, hipStream_t stream,
                                    bool a_tiled) {
  using namespace w8a8;
  if (M == 0 || N == 0) return hipSuccess;
  BatchedArgs g{};
  g.xq = xq; g.xs = x_scale; g.wq = wq; g.ws = w_scale;
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.steps = (int)((K + 63) / 64);
  g.tiles16 = (int)((N + 15) / 16);
  g.y_bf16 = y_bf16; g.y_f32 = y_f32; g.acc = acc;
  g.keys = reinterpret_cast<unsigned long long*>(keys);
  g.subkeys = subkeys; g.key_stride = key_stride;
  const bool argmax = keys != nullptr;
  if (a_tiled) {
    if (batched_workgroups(kTiledAWide, M, N) >= kMinWorkgroups)
      return launch_batched<kTiledAWide.mb, kTiledAWide.tn, kTiledAWide.wr, kTiledAWide.kw,
                            kTiledAWide.u, true>(g, tiled, argmax, stream);
    return launch_batched<kNarrow.mb, kNarrow.tn, kNarrow.wr, kNarrow.kw, kNarrow.u, true>(
        g, tiled, argmax, stream);
  }
  if (batched_workgroups(kWide, M, N) >= kMinWorkgroups)
    return launch_batched<kWide.mb, kWide.tn, kWide.wr, kWide.kw, kWide.u, false>(g, tiled, argmax,
                                                                                 stream);
  return launch_batched<kNarrow.mb, kNarrow.tn, kNarrow.wr, kNarrow.kw, kNarrow.u, false>(
      g, tiled, argmax, stream);
}
