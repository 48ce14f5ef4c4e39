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
  // k split across workgroups (gemm_w8a8_lds32 with KS > 1): per-wave int32
  // partials and arrival counters in the caller's workspace (zero between
  // calls; every call leaves them zero)
  int32_t* part;
  uint32_t* count;
  int part_bytes;
};

// Epilogue of one wave's MB x TN accumulator tiles: rows (mb0+i)*16 + 4*grp
// + r, columns (t0 + t)*16 + col.  y32 = (acc * x_scale[m]) * w_scale[n],
// written as fp32 / bf16 / int32 as requested, and the fused argmax fold.
// The lane's scales are all loaded first, in one batch: a load placed
// after an output store would wait for its own memory round trip (the
// store may alias it).
template <int MB, int TN, bool kArgmax>
__device__ __forceinline__ void batched_epilogue(const BatchedArgs& g, const v4i (&acc)[MB][TN],
                                                 int mb0, int t0, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  float wsv[TN], xsv[MB][4];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = (t0 + t) * 16 + col;
    wsv[t] = n < g.N ? g.ws[n] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = (mb0 + i) * 16 + 4 * grp + r;
      xsv[i][r] = m < g.M ? g.xs[m] : 0.0f;
    }
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int t16 = t0 + t;
    const int n = t16 * 16 + col;
    const bool n_ok = n < g.N;
    const float wsn = wsv[t];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = (mb0 + i) * 16 + 4 * grp + r;
        float v = -INFINITY;
        int idx = INT_MAX;
        if (m < g.M && n_ok) {
          const int32_t a = acc[i][t][r];
          const float y = (static_cast<float>(a) * xsv[i][r]) * wsn;
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

  batched_epilogue<MB, TN, kArgmax>(g, acc, mb0, ng * TN, lane);
}

// The LDS-pipelined kernel (tiled activations and tiled weights).  A
// workgroup of 2 x 2 waves computes 2*MB row blocks x 2*TN channel tiles;
// wave (wr, wc) owns row blocks wr*MB .. +MB-1 and tiles wc*TN .. +TN-1 of
// it, so each activation fragment feeds two waves and each weight fragment
// two.  Both operands are 1 KiB per (16-row block or 16-channel tile, k
// step) in lane order, so one direct-to-LDS load per wave instruction
// (global_load_lds_dwordx4: lane l's 16 bytes land at l*16) copies a whole
// fragment, and a lane's ds_read_b128 at l*16 gets its MFMA operand back.
// P stages of LDS, one k step each: steps s+1 .. s+P-2 are in flight while
// step s is multiplied.  Each wave issues a quarter of a step's fragments
// and waits for its own with an explicit vmcnt; one barrier per step then
// makes the step visible to all four waves and frees the stage of step s-1
// for step s + P - 1.  Fragments past the last row block or channel tile
// are fetched from block / tile 0 (in bounds) and their results dropped by
// the epilogue; the steps past the end are fetched again from the last one,
// and the step's fragment count is padded to a multiple of four (so every
// wave issues the same number of loads per step).  With KH > 1 the
// workgroup holds KH such groups of four waves, each with its own stages
// over one of KH equal slices of the k steps; their int32 tiles meet in
// LDS at the end (exact in any order) and the first group applies the
// epilogue.
constexpr int kLdsWaves = 4;

__device__ __forceinline__ void lds_dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// keeps the compiler from moving LDS reads across the explicit waits and
// barriers (the direct-to-LDS loads are not ordinary stores to it)
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// s_waitcnt with vmcnt = n and the other counters at their maxima (gfx9
// encoding: vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int MB, int TN, int P, int KH, bool kArgmax, bool kRowA = false>
__global__ __launch_bounds__(KH * kLdsWaves * kWave) void gemm_w8a8_lds(BatchedArgs g) {
  constexpr int FA = 2 * MB, FB = 2 * TN, F = FA + FB;   // fragments per k step
  // each wave issues FW loads per k step; the F..4*FW-1 padding loads fetch
  // fragment 0 again into LDS nobody reads, so that all waves wait alike
  constexpr int FW = (F + kLdsWaves - 1) / kLdsWaves;
  constexpr int STAGE = FW * kLdsWaves * 1024;
  static_assert(P >= 3, "one stage read, one refilled, at least one in flight");
  static_assert((KH - 1) * kLdsWaves * MB * TN * 1024 <= KH * P * STAGE, "k-half tiles fit the stages");
  __shared__ __attribute__((aligned(1024))) int8_t stage[KH][P][STAGE];

  // workgroup id -> (row tile, channel group), XCD-aware as above
  const int b = blockIdx.x;
  const int xcd = b % kXcds;
  const int slot = b / kXcds;
  const int mt = slot % g.mtiles;
  const int ng = (slot / g.mtiles) * kXcds + xcd;
  if (ng >= g.ngroups) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = (threadIdx.x / kWave) % kLdsWaves;   // position in its k half
  const int kh = threadIdx.x / (kWave * kLdsWaves);     // k half
  const int wr = wave & 1, wc = wave >> 1;
  const int steps = g.steps;             // >= 1 (the launcher routes K = 0 elsewhere)
  const int mblocks = (g.M + 15) / 16;
  // k slice kh takes steps [s0, s0 + nmax) (the launcher keeps steps % KH
  // == 0, so every slice runs the same iterations and the barriers match)
  const int nmax = steps / KH;
  const int s0 = kh * nmax;

  // this wave's fragment loads of every k step: fragment f = wave + 4 j
  const int8_t* src[FW];
#pragma unroll
  for (int j = 0; j < FW; ++j) {
    const int f = wave + kLdsWaves * j;
    if (f >= F) {
      src[j] = g.xq + (lane << 4);
    } else if (f < FA) {
      const int rb = mt * FA + f;
      if constexpr (kRowA) {
        // row-major activations, fetched into the tiled lane order (see
        // gemm_w8a8_lds32)
        const int row = min(rb * 16 + (lane & 15), g.M - 1);
        src[j] = g.xq + (size_t)row * (size_t)g.K + ((lane >> 4) << 4);
      } else {
        src[j] = g.xq + ((size_t)(rb < mblocks ? rb : 0) * (size_t)steps << 10) + (lane << 4);
      }
    } else {
      const int t16 = ng * FB + (f - FA);
      src[j] = g.wq + ((size_t)(t16 < g.tiles16 ? t16 : 0) * (size_t)steps << 10) + (lane << 4);
    }
  }
  // stage p of this slice <- its k step s (clamped to the slice's last)
  auto issue = [&](int p, int s) {
    s = s0 + min(s, nmax - 1);
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int f = wave + kLdsWaves * j;
      const size_t off = (kRowA && f < FA) ? (size_t)s * 64 : ((size_t)s << 10);
      lds_dma16(src[j] + off, &stage[kh][p][f * 1024]);
    }
  };

  v4i acc[MB][TN];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = v4i{0, 0, 0, 0};

  // steps 0 .. P-2 in flight; at step s, after the barrier (every wave is
  // past step s-1's reads), step s-1's stage is refilled with step s + P - 1
#pragma unroll
  for (int u = 0; u < P - 1; ++u) issue(u, u);
  for (int s = 0; s < nmax; ++s) {
    wait_vmcnt<(P - 2) * FW>();     // this wave's loads of step s are in LDS
    __builtin_amdgcn_s_barrier();   // ... and every wave's; step s-1's stage is free
    compiler_fence();
    issue((s + P - 1) % P, s + P - 1);
    const int8_t* st = stage[kh][s % P];
    v4i a[MB], bb[TN];
#pragma unroll
    for (int i = 0; i < MB; ++i)
      a[i] = *reinterpret_cast<const v4i*>(st + (wr * MB + i) * 1024 + (lane << 4));
#pragma unroll
    for (int t = 0; t < TN; ++t)
      bb[t] = *reinterpret_cast<const v4i*>(st + (FA + wc * TN + t) * 1024 + (lane << 4));
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bb[t], acc[i][t], 0, 0, 0);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this step's LDS reads are done
  }
  wait_vmcnt<0>();   // the redundant tail loads land before the LDS is reused

  if constexpr (KH > 1) {
    // the k halves' int32 tiles meet in LDS (exact in any order): halves
    // 1.. store theirs over their stages, half 0 adds them
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    v4i* red = reinterpret_cast<v4i*>(&stage[0][0][0]);
    if (kh > 0) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          red[((((kh - 1) * kLdsWaves + wave) * MB + i) * TN + t) * kWave + lane] = acc[i][t];
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int h = 1; h < KH; ++h)
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          acc[i][t] += red[((((h - 1) * kLdsWaves + wave) * MB + i) * TN + t) * kWave + lane];
  }

  batched_epilogue<MB, TN, kArgmax>(g, acc, mt * FA + wr * MB, ng * FB + wc * TN, lane);
}

typedef int v16i __attribute__((ext_vector_type(16)));

// 64-bit argmax keys held as two 32-bit lanes' words.
__device__ __forceinline__ unsigned long long key_max(unsigned long long a, unsigned long long b) {
  return b > a ? b : a;
}

// DPP move of a 64-bit value (both words with the same lane pattern).
template <int kCtrl>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, kCtrl, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), kCtrl, 0xF, 0xF, false);
  return ((unsigned long long)hi << 32) | lo;
}

// One butterfly level: a lane and its DPP partner (kCtrl) hold keys lo and
// hi for the same two rows; the lane with `upper` set keeps the row of hi,
// the other the row of lo, each the larger of its own and the partner's
// key.  The key to send is selected before the DPP move, so the move runs
// with every lane active (a DPP read from a lane that is off in EXEC
// returns 0, and a select of two DPP results can be compiled into exactly
// such a branch).
template <int kCtrl>
__device__ __forceinline__ unsigned long long keep_max(unsigned long long lo, unsigned long long hi,
                                                       bool upper) {
  const unsigned long long keep = upper ? hi : lo, send = upper ? lo : hi;
  return key_max(keep, dpp64<kCtrl>(send));
}
constexpr int kDppMirror = 0x140;       // lane j <-> 15 - j in each 16
constexpr int kDppHalfMirror = 0x141;   // lane j <-> 7 - j in each 8
constexpr int kDppXor3 = 0x1B;          // quad_perm [3,2,1,0]
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]

// Epilogue of the 32 x 32 kernels: y32 = (acc * x_scale[m]) * w_scale[n]
// for wave `wave`'s RB x CW accumulator blocks (rows (mt*RB + i)*32 + 8 (v
// / 4) + 4 g + v % 4, column (ng*4*CW + wave*CW + j)*32 + l % 32), written
// as requested (kStores) and folded into the argmax keys (kArgmax).  xs_sh
// holds the activation scales of the workgroup's RB*32 rows (written to
// LDS before the k loop, so a lane reads the 16 it needs with four 16-byte
// loads) and ws_lane[j] the weight scale of the lane's column of block j
// (registers loaded before the k loop); no global load sits between the
// epilogue's stores.  `stage_mem` is the workgroup's staging memory (at
// least lds32_row_key_bytes(RB)), free once every wave is past its last k
// step.
//
// Argmax fold, per row block i: lane l holds, for each of the 16 rows
// 8 (v / 4) + 4 g + v % 4 of its half-wave, the argmax keys (value, then
// lower index first; 0 outside M x N) of its CW columns, and keeps their
// maximum.  The maximum over the half-wave's 32 lanes is found for all 16
// rows at once by a transposed butterfly: at each of five levels a lane
// pairs with lane l ^ 16 (permlane16 swap), l ^ 15, l ^ 7, l ^ 3 and l ^ 1
// (DPP) and keeps the larger key of each pair for half of its remaining
// rows, so the even lane 2v of each half ends with row v's key and writes
// it to LDS.  The four waves' keys meet there and wave 0 folds each of the
// workgroup's rows with one device-scope atomic max.
constexpr int lds32_row_key_bytes(int RB) { return kLdsWaves * RB * 32 * 8; }

template <int RB, int CW, bool kArgmax, bool kStores>
__device__ __forceinline__ void lds32_epilogue(const BatchedArgs& g, const v16i (&acc)[RB][CW],
                                               const float* xs_sh, const float (&ws_lane)[CW],
                                               int8_t* stage_mem, int mt, int ng, int wave,
                                               int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
  const int c0 = (ng * kLdsWaves + wave) * CW;   // this wave's first 32-channel block
  unsigned long long* rows = reinterpret_cast<unsigned long long*>(stage_mem);
  // the row keys go to the stages: every wave must be past its last k step
  if constexpr (kArgmax) __syncthreads();

#pragma unroll
  for (int i = 0; i < RB; ++i) {
    // rows 8 q + 4 g .. +3 of this block for q = 0..3
    v4f xsq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xsq[q] = *reinterpret_cast<const v4f*>(xs_sh + i * 32 + 8 * q + 4 * hi);
    const int rows_left = g.M - (mt * RB + i) * 32;   // rows of this block below M
    unsigned long long m[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) m[v] = 0ull;
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int n = (c0 + j) * 32 + r32;
      const bool n_ok = n < g.N;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = 8 * (v >> 2) + (v & 3) + 4 * hi;   // row inside the 32-block
        const bool ok = rr < rows_left && n_ok;
        const int32_t a = acc[i][j][v];
        const float y = (static_cast<float>(a) * xsq[v >> 2][v & 3]) * ws_lane[j];
        if constexpr (kStores) {
          if (ok) {
            const size_t off = (size_t)((mt * RB + i) * 32 + rr) * (size_t)g.N + (size_t)n;
            if (g.y_f32) g.y_f32[off] = y;
            if (g.y_bf16) g.y_bf16[off] = f32_to_bf16_rne(y);
            if (g.acc) g.acc[off] = a;
          }
        }
        if constexpr (kArgmax) {
          // (no branch: the key is masked to 0 outside M x N)
          const unsigned long long key = argmax_key(y, n) & (0ull - (unsigned long long)ok);
          m[v] = key_max(m[v], key);   // blocks in increasing column order
        }
      }
    }
    if constexpr (kArgmax) {
      // level 1 (l ^ 16): rows 0..7 stay in lanes with bit 4 clear, 8..15 in the others
      unsigned long long m1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)m[k], (uint32_t)m[k + 8], false, false);
        const auto hw = __builtin_amdgcn_permlane16_swap((uint32_t)(m[k] >> 32),
                                                         (uint32_t)(m[k + 8] >> 32), false, false);
        m1[k] = key_max(((unsigned long long)(uint32_t)hw[0] << 32) | (uint32_t)lo[0],
                        ((unsigned long long)(uint32_t)hw[1] << 32) | (uint32_t)lo[1]);
      }
      // levels 2..4 (l ^ 15, l ^ 7, l ^ 3): bit 3, 2, 1 of the lane picks the rows kept
      unsigned long long m2[4], m3[2];
#pragma unroll
      for (int k = 0; k < 4; ++k) m2[k] = keep_max<kDppMirror>(m1[k], m1[k + 4], (lane & 8) != 0);
#pragma unroll
      for (int k = 0; k < 2; ++k) m3[k] = keep_max<kDppHalfMirror>(m2[k], m2[k + 2], (lane & 4) != 0);
      unsigned long long x = keep_max<kDppXor3>(m3[0], m3[1], (lane & 2) != 0);
      // level 5 (l ^ 1): lanes 2v and 2v + 1 of each half hold row v's key
      x = key_max(x, dpp64<kDppXor1>(x));
      if ((lane & 1) == 0) {
        const int v = (lane >> 1) & 15;
        const int rr = 8 * (v >> 2) + (v & 3) + 4 * hi;
        rows[(wave * RB + i) * 32 + rr] = x;
      }
    }
  }
  if constexpr (kArgmax) {
    __syncthreads();
    if (wave == 0) {
      for (int r = lane; r < RB * 32; r += kWave) {
        unsigned long long k = rows[r];
#pragma unroll
        for (int w = 1; w < kLdsWaves; ++w) k = key_max(k, rows[w * RB * 32 + r]);
        const int m = mt * RB * 32 + r;
        if (k != 0ull && m < g.M) {
          const size_t sub = (size_t)m * g.subkeys + (ng % g.subkeys);
          __hip_atomic_fetch_max(&g.keys[sub * g.key_stride], k, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// Hand-off of a k split across workgroups, per wave (wslot: the wave's
// (tile, wave) slot).  Each of the KS slices writes its int32 partial tile
// (16 bytes per lane per 4 accumulators, stores that go through to the
// device's coherence point), waits until they have completed, and counts its
// arrival with a device-scope atomic add; the last to arrive reads the other
// partials (loads from the coherence point, issued after its count
// returned), adds them, zeroes every partial of the slot and the counter
// (the workspace is left as it was found) and returns true: it runs the
// epilogue.  The sums are exact, so which slice is last does not matter.
// Partial layout: slot-major, then slice, then (block, quarter, lane).
constexpr int kScDevice = 16;   // cache policy of the buffer accesses: sc1 (device scope)

template <int RB, int CW, int KS>
__device__ __forceinline__ bool lds32_split_handoff(const BatchedArgs& g, v16i (&acc)[RB][CW],
                                                    size_t wslot, int ks, int lane) {
  constexpr int kBlk = RB * CW * 16 * kWave;   // int32 per wave partial
  const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(g.part, 0, g.part_bytes, 0x00020000);
  auto offset = [&](int slice, int i, int j, int q) {
    return (int)((((wslot * KS + slice) * kBlk) + (((i * CW + j) * 4 + q) * kWave + lane) * 4) * 4);
  };
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CW; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4i v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, part, offset(ks, i, j, q), 0, kScDevice);
      }
  // the partial has reached the coherence point before the arrival is counted
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  uint32_t old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(&g.count[wslot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, kWave);
  if (old != (uint32_t)(KS - 1)) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const v4i zero = {0, 0, 0, 0};
#pragma unroll
  for (int o = 1; o < KS; ++o) {
    const int other = ks + o < KS ? ks + o : ks + o - KS;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4i t = __builtin_amdgcn_raw_buffer_load_b128(part, offset(other, i, j, q), 0, kScDevice);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] += t[e];
        }
  }
#pragma unroll
  for (int sl = 0; sl < KS; ++sl)
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CW; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __builtin_amdgcn_raw_buffer_store_b128(zero, part, offset(sl, i, j, q), 0, kScDevice);
  if (lane == 0) __hip_atomic_exchange(&g.count[wslot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The bf16-only epilogue: each 32 x 32 block goes through the wave's own LDS
// tile (row stride lds32_tile_row halfwords; 80 bytes puts the two half-waves'
// rows in different banks) and leaves it as 16-byte row pieces, two stores
// per lane instead of sixteen 2-byte ones.  The block's rows are
// 8 (v / 4) + 4 g + v % 4 of column l % 32 as in lds32_epilogue; lane l then
// stores row (64 k + l) / 4, columns 8 ((64 k + l) % 4) .. +7.  Requires
// N % 8 == 0 and a 16-byte aligned y_bf16 (the kernel checks both and takes
// lds32_epilogue otherwise).  A wave's LDS writes and reads complete in
// order, so the tile needs no barrier; the values are those of
// lds32_epilogue.
constexpr int lds32_tile_row = 40;
constexpr int lds32_tile_bytes = 32 * lds32_tile_row * 2;

template <int RB, int CW>
__device__ __forceinline__ void lds32_store_bf16(const BatchedArgs& g, const v16i (&acc)[RB][CW],
                                                 const float* xs_sh, const float (&ws_lane)[CW],
                                                 uint16_t* tile, int mt, int ng, int wave, int lane) {
  const int r32 = lane & 31, hi = lane >> 5;
  const int c0 = (ng * kLdsWaves + wave) * CW;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    v4f xsq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xsq[q] = *reinterpret_cast<const v4f*>(xs_sh + i * 32 + 8 * q + 4 * hi);
    const int rows_left = g.M - (mt * RB + i) * 32;
    const size_t row0 = (size_t)(mt * RB + i) * 32;
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int n0 = (c0 + j) * 32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = 8 * (v >> 2) + (v & 3) + 4 * hi;
        const float y = (static_cast<float>(acc[i][j][v]) * xsq[v >> 2][v & 3]) * ws_lane[j];
        tile[rr * lds32_tile_row + r32] = f32_to_bf16_rne(y);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = k * kWave + lane, row = c >> 2, n = n0 + 8 * (c & 3);
        const v4i piece = *reinterpret_cast<const v4i*>(tile + row * lds32_tile_row + 8 * (c & 3));
        // (N % 8 == 0 and n % 8 == 0: a piece that starts below N ends there)
        if (row < rows_left && n < g.N)
          *reinterpret_cast<v4i*>(g.y_bf16 + (row0 + row) * (size_t)g.N + n) = piece;
      }
    }
  }
}

// The pipeline on v_mfma_i32_32x32x32_i8, which does twice the work of the
// 16 x 16 x 64 instruction for the same two operand KiB: a workgroup of
// four waves computes RB blocks of 32 rows x 4*CW blocks of 32 channels;
// wave w owns channel blocks w*CW .. +CW-1 over all RB row blocks.  The
// operands are the same 1 KiB (16-row block or 16-channel tile, k step)
// units; for the 32-wide half h of a step, lane l (r = l % 32, g = l / 32)
// takes unit 2*b + r/16 of its 32-block b at tile lane (r % 16) + 16 (2h +
// g), for both operands, so A and B pair the same k.  Lane l gets rows
// 8 (v / 4) + 4 g + v % 4 of column r in accumulator v.
//
// A wave's weight fragments feed that wave alone, so only the activation
// fragments, which all four waves read, go through LDS.  Per k step a wave
// loads, for each of its blocks, its two 16-byte pieces per lane straight
// into registers, P - 1 steps ahead, in a ring of P register slots (the
// loop is unrolled P times so that every slot index is static); the
// activation fragments of the same step go to LDS stage s % P with
// direct-to-LDS loads, and one barrier per step publishes them.  Against
// staging both operands in LDS this takes the weight bytes out of the LDS
// (their DMA writes and the waves' LDS reads of them) and gives P - 1 steps
// of lookahead for the same LDS; with CW = 2 each activation fragment read
// from LDS feeds two MFMAs.
//
// Every wave issues the same loads per step, with no wave-dependent branch
// in the k loop (a branch there makes the compiler drain all loads before
// the next MFMA): when the FA = 2*RB activation fragments do not split
// evenly over the four waves (FA % 4 == 2), waves 2w and 2w+1 both copy
// fragment 4*(FA/4) + w, the same bytes to the same LDS, so each wave
// issues FA/4 + 1 of them.  Fragments past the last row block or channel
// tile are fetched from block / tile 0 (in bounds) and their results
// dropped by the epilogue; the steps past the end are fetched again from
// the last one.
template <int RB, int CW, int P, bool kArgmax, bool kStores, bool kRowA = false, bool kRot = false,
          int KS = 1>
__global__ __launch_bounds__(kLdsWaves * kWave, P <= 4 ? (CW == 1 ? 4 : 2) : 2) void gemm_w8a8_lds32(BatchedArgs g) {
  static_assert(KS == 1 || (!kArgmax && kStores), "a k split hands int32 partials over, no argmax fold");
  constexpr int FA = 2 * RB;                               // activation fragments per step
  constexpr int FAF = FA / kLdsWaves;                      // whole share per wave
  constexpr bool kDup = FA % kLdsWaves != 0;               // (FA even: then FA % 4 == 2)
  constexpr int LA = FAF + (kDup ? 1 : 0);                 // activation loads per wave per step
  constexpr int LW = LA + 2 * CW;                          // loads per wave per step
  constexpr int STAGE = FA * 1024;
  constexpr int D = P - 1;                                 // steps of lookahead
  static_assert(P >= 2, "one stage read while the next one fills");
  constexpr int kTrBytes = kArgmax ? lds32_row_key_bytes(RB) : 0;
  constexpr int kStageBytes = P * STAGE >= kTrBytes ? P * STAGE : kTrBytes;
  // (one LDS array: the stages, then the workgroup's row scales; a second
  // LDS object makes the compiler wait for the direct-to-LDS loads before
  // every LDS read)
  // (with stores and no argmax fold, each wave also gets a 32 x 32 bf16
  // tile after the row scales for the vectorized epilogue)
  constexpr bool kVecEpi = kStores && !kArgmax;
  constexpr int kEpiBytes = kVecEpi ? kLdsWaves * lds32_tile_bytes : 0;
  __shared__ __attribute__((aligned(1024))) int8_t stage_mem[kStageBytes + RB * 32 * 4 + kEpiBytes];

  const int b = blockIdx.x;
  const int xcd = b % kXcds;
  const int slot = b / kXcds;
  const int mt = slot % g.mtiles;
  const int ks = (slot / g.mtiles) % KS;   // k slice (the slices of a tile are KS slots apart)
  const int ng = (slot / g.mtiles / KS) * kXcds + xcd;
  if (ng >= g.ngroups) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // this workgroup's k steps: [kbase, kbase + steps) of the g.steps
  const int kbase = (int)(((int64_t)g.steps * ks) / KS);
  const int steps = (int)(((int64_t)g.steps * (ks + 1)) / KS) - kbase;
  const int mblocks = (g.M + 15) / 16;
  const int r32 = lane & 31, hi = lane >> 5;
  const int lane_off = ((r32 & 15) + 16 * hi) << 4;

  // the epilogue's scales: the workgroup's row scales into LDS after the
  // stages (visible after the k loop's first barrier), the lane's column
  // scales in registers
  float* xs_sh = reinterpret_cast<float*>(stage_mem + kStageBytes);
  if (threadIdx.x < RB * 32) {
    const int m = mt * RB * 32 + threadIdx.x;
    xs_sh[threadIdx.x] = m < g.M ? g.xs[m] : 0.0f;
  }
  float ws_lane[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int n = ((ng * kLdsWaves + wave) * CW + j) * 32 + r32;
    ws_lane[j] = n < g.N ? g.ws[n] : 0.0f;
  }

  // activation fragments of every step: wave w copies fragments w, w+4, ...
  // (FAF of them) and, when FA % 4 == 2, fragment 4 FAF + w / 2
  const int8_t* src[LA];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int f = j < FAF ? wave + kLdsWaves * j : kLdsWaves * FAF + (wave >> 1);
    const int rb = mt * FA + f;
    if constexpr (kRowA) {
      const int row = min(rb * 16 + (lane & 15), g.M - 1);
      src[j] = g.xq + (size_t)row * (size_t)g.K + ((lane >> 4) << 4);
    } else {
      src[j] = g.xq + ((size_t)(rb < mblocks ? rb : 0) * (size_t)g.steps << 10) + (lane << 4);
    }
  }
  // k steps in a rotated order (kRot): the workgroups that read one weight
  // tile (same ng) or one activation tile (same mt) start at different k,
  // so that one of them misses in L2 while the others hit; the int32 sums do
  // not depend on the order
  int kstart = 0;
  if constexpr (kRot) {
    const int nq = (g.ngroups + kXcds - 1) / kXcds;
    kstart = (int)(((int64_t)(mt + g.mtiles * (ng / kXcds)) * steps) / ((int64_t)g.mtiles * nq));
  }
  auto kstep = [&](int s) {
    s = min(s, steps - 1);   // (steps past the end fetch the last one again)
    if constexpr (kRot) {
      s += kstart;
      if (s >= steps) s -= steps;
    }
    return kbase + s;
  };
  auto issue_a = [&](int p, int s) {
    s = kstep(s);
    const size_t off = kRowA ? (size_t)s * 64 : ((size_t)s << 10);
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int f = j < FAF ? wave + kLdsWaves * j : kLdsWaves * FAF + (wave >> 1);
      lds_dma16(src[j] + off, stage_mem + p * STAGE + f * 1024);
    }
  };
  // this lane's weight units (tiles past the last are fetched from tile 0;
  // their columns are dropped by the epilogue)
  const int8_t* wsrc[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int t16 = ((ng * kLdsWaves + wave) * CW + j) * 2 + (r32 >> 4);
    wsrc[j] = g.wq + ((size_t)(t16 < g.tiles16 ? t16 : 0) * (size_t)g.steps << 10) + lane_off;
  }
  auto load_b = [&](v4i (&dst)[CW][2], int s) {
    s = kstep(s);
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      dst[j][0] = *reinterpret_cast<const v4i*>(wsrc[j] + ((size_t)s << 10));
      dst[j][1] = *reinterpret_cast<const v4i*>(wsrc[j] + ((size_t)s << 10) + 512);
    }
  };

  v16i acc[RB][CW];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  v4i bq[P][CW][2];
#pragma unroll
  for (int u = 0; u < D; ++u) {
    issue_a(u, u);
    load_b(bq[u], u);
  }
  // one k step: ring slot u = s % P holds step s's weights, stage u its
  // activations
  auto step = [&](int u, int s) {
    // step s's loads (issued D steps ago) are in; steps s+1 .. s+D-1 may
    // still be in flight (loads complete in issue order)
    wait_vmcnt<(D - 1) * LW>();
    __builtin_amdgcn_s_barrier();   // every wave's activations of step s are in LDS
    compiler_fence();
    issue_a((u + D) % P, s + D);    // the stage step s-1 used (every wave is past it)
    load_b(bq[(u + D) % P], s + D);
    const int8_t* st = stage_mem + u * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i a[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i)
        a[i] = *reinterpret_cast<const v4i*>(st + (2 * i + (r32 >> 4)) * 1024 + (h << 9) + lane_off);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bq[u][j][h], acc[i][j], 0, 0, 0);
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this step's LDS reads are done
  };
  // whole rounds of P steps with no branch inside (so the ring stays in the
  // same registers), then the last steps % P
  int s0 = 0;
  for (; s0 + P <= steps; s0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) step(u, s0 + u);
  }
#pragma unroll
  for (int u = 0; u < P - 1; ++u)
    if (s0 + u < steps) step(u, s0 + u);
  wait_vmcnt<0>();

  if constexpr (KS > 1) {
    if (!lds32_split_handoff<RB, CW, KS>(g, acc, ((size_t)ng * g.mtiles + mt) * kLdsWaves + wave, ks, lane))
      return;   // another slice of this tile finishes it
  }
  if constexpr (kVecEpi) {
    if (g.y_bf16 && !g.y_f32 && !g.acc && g.N % 8 == 0 && (reinterpret_cast<uintptr_t>(g.y_bf16) & 15) == 0) {
      uint16_t* tile = reinterpret_cast<uint16_t*>(stage_mem + kStageBytes + RB * 32 * 4 + wave * lds32_tile_bytes);
      lds32_store_bf16<RB, CW>(g, acc, xs_sh, ws_lane, tile, mt, ng, wave, lane);
      return;
    }
  }
  lds32_epilogue<RB, CW, kArgmax, kStores>(g, acc, xs_sh, ws_lane, stage_mem, mt, ng, wave, lane);
}

template <int RB, int CW, int P, bool kRowA = false, bool kRot = false, int KS = 1>
static hipError_t launch_lds32(BatchedArgs g, bool argmax, hipStream_t stream) {
  g.ngroups = (g.tiles16 + 2 * kLdsWaves * CW - 1) / (2 * kLdsWaves * CW);
  g.mtiles = (g.M + 32 * RB - 1) / (32 * RB);
  const int64_t ng_padded = ((int64_t)g.ngroups + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)(ng_padded * g.mtiles * KS)), block(kLdsWaves * kWave);
  if constexpr (KS > 1) {
    (void)argmax;   // (the dispatcher never splits an argmax fold)
    hipLaunchKernelGGL((gemm_w8a8_lds32<RB, CW, P, false, true, kRowA, kRot, KS>), grid, block, 0, stream, g);
  } else {
    const bool stores = g.y_bf16 || g.y_f32 || g.acc;
    if (argmax && !stores)
      hipLaunchKernelGGL((gemm_w8a8_lds32<RB, CW, P, true, false, kRowA, kRot>), grid, block, 0, stream, g);
    else if (argmax)
      hipLaunchKernelGGL((gemm_w8a8_lds32<RB, CW, P, true, true, kRowA, kRot>), grid, block, 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_w8a8_lds32<RB, CW, P, false, true, kRowA, kRot>), grid, block, 0, stream, g);
  }
  return hipGetLastError();
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

// (no fused argmax: the LM-head argmax path passes row-major activations,
// which take the register-fragment kernel)
template <int MB, int TN, int P, int KH, bool kRowA = false>
static hipError_t launch_lds(BatchedArgs g, hipStream_t stream) {
  g.ngroups = (g.tiles16 + 2 * TN - 1) / (2 * TN);
  g.mtiles = (g.M + 32 * MB - 1) / (32 * MB);
  const int64_t ng_padded = ((int64_t)g.ngroups + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)(ng_padded * g.mtiles)), block(KH * kLdsWaves * kWave);
  hipLaunchKernelGGL((gemm_w8a8_lds<MB, TN, P, KH, false, kRowA>), grid, block, 0, stream, g);
  return hipGetLastError();
}
constexpr BatchedShape kWide{3, 4, 1, 4, 4};
constexpr BatchedShape kNarrow{3, 2, 1, 8, 2};
constexpr BatchedShape kTiledAWide{3, 2, 1, 4, 4};
constexpr int64_t kMinWorkgroups = 256;

// The LDS-pipelined kernel (tiled activations and weights): 96 rows x 64
// channels per workgroup.  Measured at 288 rows, weights rotated past the
// Infinity Cache, against the register-fragment kernel above:
//  * 4 stages, whole K per workgroup, once the grid is wide enough to keep
//    ~2 workgroups per CU busy: gate/up 4096 -> 12288 40.2 vs 49.8 us;
//  * K cut into 4 slices of 4 waves each (3 stages each, tiles summed in
//    LDS) on narrower grids, where one workgroup's chain of k steps would
//    be too long: down 12288 -> 4096 41.8 vs 46.6 us, q 19.7 vs 20.5 us;
//  * below ~128 workgroups (k/v, 1024 channels) the register-fragment
//    kernel stays faster.
struct LdsShape {
  int mb, tn, p;
};
constexpr LdsShape kLdsShape{3, 2, 4};
constexpr int64_t kLdsMinWorkgroups = 512;
constexpr int kLdsSplit = 4, kLdsSplitStages = 3;
constexpr int64_t kLdsSplitMinWorkgroups = 128;

// The 32 x 32 kernel where its grid fills the chip (counted in 64-row x
// 128-channel workgroups), measured at 288 rows against the 16 x 16
// pipeline: q/k/v fused 4096 -> 6144 (240 workgroups) 22.8 vs 35.5 us,
// gate 4096 -> 12288 (480) 33.3 vs 39.1 us, gate/up fused 4096 -> 24576
// (960) 55-59 vs 67 us.  With the bf16 outputs stored through the wave's
// LDS tile (16-byte pieces: the per-workgroup epilogue went from ~3.4 us to
// well under 1 us), the k order rotated per workgroup and 5 steps of
// lookahead for the 64 x 128 tile, A/B on one box: o 4096 -> 4096 (160
// workgroups) 15.3 us against 19.0 for the k-sliced 16 x 16 form, q/k/v
// 16.0-16.4 (21.1), gate 27.5-28.2 (31.0), gate/up 48.1 (51.6-57).  At 160
// workgroups every CU holds one workgroup; its loads, not the MFMAs or the
// barrier, set the step time (without the MFMAs the loop is no faster;
// deeper lookahead, more waves per workgroup or activations staged through
// registers instead of direct-to-LDS loads gave no more).  Tiles and lookahead by grid width, measured at 288 rows
// (A/B on one box, weights streamed into registers against the earlier
// form that staged them in LDS): q/k/v 64 x 128 with 3 steps of lookahead
// 20.9 us (staged: 22-23), gate the same 30.5-30.9 us (33.6-34.5), gate/up
// 64 x 256 with 2 steps 51.9-52.2 us (57-60); the 4096 -> 151936 LM head
// with the argmax folded in, 96 x 256 with 2 steps (each weight block read
// once per 96 rows, three workgroups per CU): 213-219 us per verify step
// against 252-265 us for the staged 96 x 128 form.
constexpr int64_t kLds32MinWorkgroups = 160;
constexpr int64_t kLds32WideTileMinWorkgroups = 768;
constexpr int64_t kLds32TallTileMinWorkgroups = 2048;

static int64_t lds32_workgroups(int64_t M, int64_t N) {
  return ((N + 15) / 16 + 2 * kLdsWaves - 1) / (2 * kLdsWaves) * ((M + 63) / 64);
}

// the same count for 96-row workgroups
static int64_t lds32_wide_workgroups(int64_t M, int64_t N) {
  return ((N + 15) / 16 + 2 * kLdsWaves - 1) / (2 * kLdsWaves) * ((M + 95) / 96);
}

// k split across two workgroups for long reductions on the 64 x 128 grids
// (down 12288 -> 4096 at 288 rows: 96 x 128 tiles in 2 slices, 192
// workgroups, 33-34 us against 39.5-41 unsplit; at K = 4096 the handoff ate
// the gain: o 15.0-15.3 either way): at least kLds32SplitMinSteps k steps,
// and every workgroup of the split grid resident at once.
constexpr int kLds32Split = 2;
constexpr int64_t kLds32SplitMinSteps = 128;
constexpr int64_t kLds32SplitMaxWorkgroups = 256;

static bool lds32_split(int64_t M, int64_t N, int64_t steps) {
  const int64_t wg32 = lds32_workgroups(M, N);
  return wg32 >= kLds32MinWorkgroups && wg32 < kLds32WideTileMinWorkgroups &&
         steps >= kLds32SplitMinSteps &&
         lds32_wide_workgroups(M, N) * kLds32Split <= kLds32SplitMaxWorkgroups;
}

// workspace of the split: arrival counters (one per wave and tile, padded to
// 256 bytes), then the partials (per wave and slice, 96 x 32 int32 tiles)
static int64_t lds32_split_slots(int64_t M, int64_t N) {
  return lds32_wide_workgroups(M, N) * kLdsWaves;
}
static size_t lds32_split_count_bytes(int64_t M, int64_t N) {
  return ((size_t)lds32_split_slots(M, N) * sizeof(uint32_t) + 255) & ~(size_t)255;
}
static size_t lds32_split_part_bytes(int64_t M, int64_t N) {
  return (size_t)lds32_split_slots(M, N) * kLds32Split * (3 * 1 * 16 * kWave) * sizeof(int32_t);
}

static int64_t lds_workgroups(int64_t M, int64_t N) {
  const int64_t ngroups = ((N + 15) / 16 + 2 * kLdsShape.tn - 1) / (2 * kLdsShape.tn);
  const int64_t mtiles = (M + 32 * kLdsShape.mb - 1) / (32 * kLdsShape.mb);
  return ngroups * mtiles;
}

static int64_t batched_workgroups(const BatchedShape& c, int64_t M, int64_t N) {
  const int64_t ngroups = ((N + 15) / 16 + c.tn - 1) / c.tn;
  const int64_t mtiles = (M + 16 * c.mb * c.wr - 1) / (16 * c.mb * c.wr);
  return ngroups * mtiles;
}

// The LDS-pipelined kernels where the grid suits them (returns false to
// leave the shape to the register-fragment kernel).
template <bool kRowA>
static bool launch_lds_path(const BatchedArgs& g, int64_t M, int64_t N, bool argmax,
                            hipStream_t stream, hipError_t* err) {
  if (lds32_wide_workgroups(M, N) >= kLds32TallTileMinWorkgroups) {
    *err = launch_lds32<3, 2, 3, kRowA>(g, argmax, stream);
    return true;
  }
  const int64_t wg32 = lds32_workgroups(M, N);
  if (!argmax && g.part && lds32_split(M, N, g.steps)) {
    // (k order not rotated: with 96-row tiles the rotated starts lie ~8 steps
    // apart, too far for the L2 to keep the shared weight and activation
    // steps, and the HBM traffic of 288 x 4096 x 12288 went 1.5 -> 3.5x the
    // algorithmic bytes for no gain in time)
    *err = launch_lds32<3, 1, 6, kRowA, false, kLds32Split>(g, argmax, stream);
    return true;
  }
  if (wg32 >= kLds32WideTileMinWorkgroups) {
    *err = launch_lds32<2, 2, 3, kRowA, true>(g, argmax, stream);
    return true;
  }
  if (wg32 >= kLds32MinWorkgroups) {
    *err = launch_lds32<2, 1, 6, kRowA, true>(g, argmax, stream);
    return true;
  }
  if (argmax) return false;   // (the 16 x 16 pipeline has no argmax fold)
  const int64_t lwg = lds_workgroups(M, N);
  if (lwg >= kLdsMinWorkgroups) {
    *err = launch_lds<kLdsShape.mb, kLdsShape.tn, kLdsShape.p, 1, kRowA>(g, stream);
    return true;
  }
  if (lwg >= kLdsSplitMinWorkgroups && g.steps % kLdsSplit == 0) {
    *err = launch_lds<kLdsShape.mb, kLdsShape.tn, kLdsSplitStages, kLdsSplit, kRowA>(g, stream);
    return true;
  }
  return false;
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

size_t w8a8_batched_workspace_bytes(int64_t M, int64_t N, int64_t K, bool a_tiled) {
  using namespace w8a8;
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (!a_tiled && K % 64 != 0) return 0;   // (row-major activations: the LDS path needs K % 64 == 0)
  if (!lds32_split(M, N, (K + 63) / 64)) return 0;
  return lds32_split_count_bytes(M, N) + lds32_split_part_bytes(M, N);
}

hipError_t w8a8_launch_gemm_batched(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, int64_t M, int64_t N, int64_t K,
                                    bool tiled, uint16_t* y_bf16, float* y_f32, int32_t* acc,
                                    void* keys, int subkeys, int key_stride, hipStream_t stream,
                                    bool a_tiled, void* workspace) {
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
  if (workspace && tiled && w8a8_batched_workspace_bytes(M, N, K, a_tiled) > 0) {
    g.count = reinterpret_cast<uint32_t*>(workspace);
    g.part = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + lds32_split_count_bytes(M, N));
    g.part_bytes = (int)lds32_split_part_bytes(M, N);
  }
  // The LDS-pipelined kernels take tiled activations, or row-major ones
  // when K is a multiple of 64 (each fragment then gathered from 16 rows
  // into the same lane order)
  if (tiled && g.steps > 0) {
    hipError_t e = hipSuccess;
    if (a_tiled && launch_lds_path<false>(g, M, N, argmax, stream, &e)) return e;
    if (!a_tiled && K % 64 == 0 && launch_lds_path<true>(g, M, N, argmax, stream, &e)) return e;
  }
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
