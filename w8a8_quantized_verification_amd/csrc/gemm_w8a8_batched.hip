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

// Epilogue of one wave's MB x TN accumulator tiles: rows (mb0+i)*16 + 4*grp
// + r, columns (t0 + t)*16 + col.  y32 = (acc * x_scale[m]) * w_scale[n],
// written as fp32 / bf16 / int32 as requested, and the fused argmax fold.
template <int MB, int TN, bool kArgmax>
__device__ __forceinline__ void batched_epilogue(const BatchedArgs& g, const v4i (&acc)[MB][TN],
                                                 int mb0, int t0, int lane) {
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int t16 = t0 + t;
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

// The same pipeline on v_mfma_i32_32x32x32_i8: a workgroup of four waves
// computes RB blocks of 32 rows x 4*CW blocks of 32 channels; wave w owns
// channel blocks w*CW .. +CW-1 over all RB row blocks.  The staged
// fragments are the same 1 KiB (16-row block or 16-channel tile, k step)
// units; for the 32-wide half h of a step, lane l (r = l % 32, g = l / 32)
// reads unit 2*b + r/16 of its 32-block b at tile lane (r % 16) + 16 (2h +
// g), for both operands, so A and B pair the same k.  Lane l gets rows
// 8 (v / 4) + 4 g + v % 4 of column r in accumulator v.  The launch bound
// holds every form to 128 registers (at least four workgroups per CU).
// With the argmax fold's transpose and row maxima inside the stages, the
// 96-row form (90 registers, 32 KB of LDS) runs five per CU: 288 rows x
// 151936 channels ~288 us, against ~309 at four per CU and 362-384 at
// three (the transpose padded, in LDS of its own).
typedef int v16i __attribute__((ext_vector_type(16)));

template <int RB, int CW, int P, bool kArgmax, bool kRowA = false>
__global__ __launch_bounds__(kLdsWaves * kWave, 4) void gemm_w8a8_lds32(BatchedArgs g) {
  constexpr int FA = 2 * RB, FB = 2 * kLdsWaves * CW, F = FA + FB;
  constexpr int FW = (F + kLdsWaves - 1) / kLdsWaves;
  constexpr int STAGE = FW * kLdsWaves * 1024;
  static_assert(P >= 2, "one stage read while the next one fills");
  // the stages, also the argmax fold's transpose buffer once the k loop is done
  constexpr int kTrBytes = kArgmax ? kLdsWaves * 32 * 32 * 8 : 0;
  constexpr int kStages = P * STAGE >= kTrBytes ? P : (kTrBytes + STAGE - 1) / STAGE;
  __shared__ __attribute__((aligned(1024))) int8_t stage[kStages][STAGE];

  const int b = blockIdx.x;
  const int xcd = b % kXcds;
  const int slot = b / kXcds;
  const int mt = slot % g.mtiles;
  const int ng = (slot / g.mtiles) * kXcds + xcd;
  if (ng >= g.ngroups) return;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int steps = g.steps;
  const int mblocks = (g.M + 15) / 16;

  const int8_t* src[FW];
#pragma unroll
  for (int j = 0; j < FW; ++j) {
    const int f = wave + kLdsWaves * j;
    if (f >= F) {
      src[j] = g.xq + (lane << 4);
    } else if (f < FA) {
      const int rb = mt * FA + f;
      if constexpr (kRowA) {
        // row-major activations (K a multiple of 64): lane l fetches row
        // 16 rb + l % 16, bytes 16 (l / 16) .. +15 of the step, landing at
        // l * 16 as in the tiled layout; rows past M repeat row M - 1 (they
        // only feed accumulator rows the epilogue drops)
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
  auto issue = [&](int p, int s) {
    s = min(s, steps - 1);
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int f = wave + kLdsWaves * j;
      const size_t off = (kRowA && f < FA) ? (size_t)s * 64 : ((size_t)s << 10);
      lds_dma16(src[j] + off, &stage[p][f * 1024]);
    }
  };

  const int r32 = lane & 31, hi = lane >> 5;
  const int lane_off = ((r32 & 15) + 16 * hi) << 4;
  v16i acc[RB][CW];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CW; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

#pragma unroll
  for (int u = 0; u < P - 1; ++u) issue(u, u);
  for (int s = 0; s < steps; ++s) {
    wait_vmcnt<(P - 2) * FW>();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    issue((s + P - 1) % P, s + P - 1);
    const int8_t* st = stage[s % P];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i a[RB], bb[CW];
#pragma unroll
      for (int i = 0; i < RB; ++i)
        a[i] = *reinterpret_cast<const v4i*>(st + (2 * i + (r32 >> 4)) * 1024 + (h << 9) + lane_off);
#pragma unroll
      for (int j = 0; j < CW; ++j)
        bb[j] = *reinterpret_cast<const v4i*>(st + (FA + 2 * (wave * CW + j) + (r32 >> 4)) * 1024 +
                                              (h << 9) + lane_off);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < CW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this step's LDS reads are done
  }
  wait_vmcnt<0>();

  // argmax fold: each wave transposes its (row, column) keys of one 32 x 32
  // block at a time through LDS (the stages, free once every wave is past
  // its last step) so that lane r < 32 reduces row r over the block's 32
  // columns; the waves' row maxima meet in LDS and wave 0 folds each of the
  // workgroup's rows with one device-scope atomic max.  Keys order by value
  // and then by lower index, so their maximum is the row's argmax.
  // 32 u64 per transposed row, column c of row r stored at c ^ r: the
  // half-wave's writes of one row and each lane's reads of its own row
  // across the columns both touch 32 distinct bank pairs, with no padding
  // (so the transpose fits in the stages of the 96-row form)
  constexpr int kTrStride = 32;
  static_assert(!kArgmax || kLdsWaves * 32 * kTrStride * 8 <= kStages * STAGE,
                "transpose fits the stages");
  // each wave's RB * 32 row maxima go to the start of its own transpose
  // region once its last transpose has been read (no LDS beyond the stages)
  static_assert(RB * 32 <= 32 * kTrStride, "row maxima fit a transpose region");
  unsigned long long* tr = reinterpret_cast<unsigned long long*>(&stage[0][0]) +
                           (size_t)wave * 32 * kTrStride;
  if constexpr (kArgmax) __syncthreads();
  unsigned long long rk[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) rk[i] = 0ull;

#pragma unroll
  for (int j = 0; j < CW; ++j) {
    const int c32 = ng * kLdsWaves * CW + wave * CW + j;   // 32-channel block
    const int n = c32 * 32 + r32;
    const bool n_ok = n < g.N;
    const float wsn = n_ok ? g.ws[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = 8 * (v >> 2) + 4 * hi + (v & 3);     // row inside the 32-block
        const int m = (mt * RB + i) * 32 + rr;
        unsigned long long key = 0ull;
        if (m < g.M && n_ok) {
          const int32_t a = acc[i][j][v];
          const float y = (static_cast<float>(a) * g.xs[m]) * wsn;
          const size_t o = (size_t)m * (size_t)g.N + (size_t)n;
          if (g.y_f32) g.y_f32[o] = y;
          if (g.y_bf16) g.y_bf16[o] = f32_to_bf16_rne(y);
          if (g.acc) g.acc[o] = a;
          key = argmax_key(y, n);
        }
        if constexpr (kArgmax) tr[rr * kTrStride + (r32 ^ rr)] = key;
      }
      if constexpr (kArgmax) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes landed
        __builtin_amdgcn_wave_barrier();
        if (lane < 32) {
          unsigned long long k = rk[i];
#pragma unroll 8
          for (int c = 0; c < 32; ++c) {
            const unsigned long long o = tr[lane * kTrStride + (c ^ lane)];
            k = o > k ? o : k;
          }
          rk[i] = k;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  if constexpr (kArgmax) {
    if (lane < 32) {
#pragma unroll
      for (int i = 0; i < RB; ++i) tr[i * 32 + lane] = rk[i];
    }
    __syncthreads();
    if (wave == 0) {
      for (int r = lane; r < RB * 32; r += kWave) {
        const unsigned long long* rows0 = reinterpret_cast<const unsigned long long*>(&stage[0][0]);
        unsigned long long k = rows0[r];
#pragma unroll
        for (int w = 1; w < kLdsWaves; ++w) {
          const unsigned long long o = rows0[(size_t)w * 32 * kTrStride + r];
          k = o > k ? o : k;
        }
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

template <int RB, int CW, int P, bool kRowA = false>
static hipError_t launch_lds32(BatchedArgs g, bool argmax, hipStream_t stream) {
  g.ngroups = (g.tiles16 + 2 * kLdsWaves * CW - 1) / (2 * kLdsWaves * CW);
  g.mtiles = (g.M + 32 * RB - 1) / (32 * RB);
  const int64_t ng_padded = ((int64_t)g.ngroups + kXcds - 1) / kXcds * kXcds;
  const dim3 grid((unsigned)(ng_padded * g.mtiles)), block(kLdsWaves * kWave);
  if (argmax)
    hipLaunchKernelGGL((gemm_w8a8_lds32<RB, CW, P, true, kRowA>), grid, block, 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_w8a8_lds32<RB, CW, P, false, kRowA>), grid, block, 0, stream, g);
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

// The 32 x 32 form (64 rows x 128 channels per workgroup) where its grid
// fills the chip, measured at 288 rows against the 16 x 16 pipeline:
// q/k/v fused 4096 -> 6144 (240 workgroups) 22.8 vs 35.5 us, gate 4096 ->
// 12288 (480) 33.3 vs 39.1 us, gate/up fused 4096 -> 24576 (960) 55-59 vs
// 67 us; with 160 workgroups (o, down at 4096 channels) it is slower (22.1
// vs 19.3 us, 50.1 vs 41.6 us), so those keep the k-sliced 16 x 16 form.
// Stage count and tile by grid width, measured at 288 rows (A/B on one
// box): wider grids keep more workgroups per CU with fewer stages, which
// pays more than deeper prefetch (stages beyond these were slower
// everywhere).  q/k/v 4096 -> 6144 (240 workgroups of 64 x 128): 4 stages,
// 22.9 us (3: 27.8, 2: 44.1); gate 4096 -> 12288 (480): 3-4 stages, 32.4-33.0
// us (2: 46.6); gate/up 4096 -> 24576 (960): 2 stages, 55.3 us (3: 58.0);
// the 4096 -> 151936 LM head: 96 x 128 workgroups (each weight block read
// once per 96 rows), 2 stages, ~288 us with the argmax folded in (64 x
// 128, 3 stages: ~447 us).
constexpr int64_t kLds32MinWorkgroups = 224;
constexpr int64_t kLds32DeepMinWorkgroups = 512;
constexpr int64_t kLds32DoubleBufferMinWorkgroups = 768;
constexpr int64_t kLds32WideMinWorkgroups = 2048;

static int64_t lds32_workgroups(int64_t M, int64_t N) {
  return ((N + 15) / 16 + 2 * kLdsWaves - 1) / (2 * kLdsWaves) * ((M + 63) / 64);
}

// the 96-row form's grid
static int64_t lds32_wide_workgroups(int64_t M, int64_t N) {
  return ((N + 15) / 16 + 2 * kLdsWaves - 1) / (2 * kLdsWaves) * ((M + 95) / 96);
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
  if (lds32_wide_workgroups(M, N) >= kLds32WideMinWorkgroups) {
    *err = launch_lds32<3, 1, 2, kRowA>(g, argmax, stream);
    return true;
  }
  const int64_t wg32 = lds32_workgroups(M, N);
  if (wg32 >= kLds32DoubleBufferMinWorkgroups) {
    *err = launch_lds32<2, 1, 2, kRowA>(g, argmax, stream);
    return true;
  }
  if (wg32 >= kLds32DeepMinWorkgroups) {
    *err = launch_lds32<2, 1, 3, kRowA>(g, argmax, stream);
    return true;
  }
  if (wg32 >= kLds32MinWorkgroups) {
    *err = launch_lds32<2, 1, 4, kRowA>(g, argmax, stream);
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
