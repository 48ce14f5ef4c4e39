// Chained skinny verification step for gfx950: one persistent launch runs a
// sequence of steps over the same few token rows (M <= 16):
//   QUANTIZE  bf16 rows -> int8 codes + per-row scales (per-token symmetric
//             quantization, optional smoothing multiply),
//   LINEAR    W8A8 linear on tiled weights with the dequant fused (bf16 and/or
//             fp32 out),
//   LM_HEAD   the same linear with the argmax folded into the epilogue,
//   ACCEPT    greedy acceptance from the folded argmax keys.
//
// Pages: verification time is the weight bytes over the memory bandwidth
// (gist.science German summary, Technische Zusammenfassung §3 item 4;
// Japanese summary, 技術的サマリー §2.3).  A verify step with a handful of
// token rows is one long weight stream, cut into a few hundred linears; as
// separate launches each one pays a ramp (the first loads' round trip) and a
// tail (the last workgroups finishing alone) in which HBM idles.  Here the
// workgroups stay resident for the whole sequence and meet at a device-wide
// barrier between consecutive steps, so step i+1 sees every output of steps
// 0..i (any dependency between steps is honoured); before waiting at a
// barrier each workgroup already issues the weight loads of its first share
// of the next linear (weights never depend on earlier steps), so the weight
// stream continues through the barrier and through the quantization steps.
//
// The arithmetic of every step is that of the separate calls, bit for bit:
//   codes:  amax = max|v|, scale = amax/127, inv = 127/amax (0 if amax == 0),
//           q = 0 where v == 0 else clamp(rint(v*inv), -127, 127)
//   linear: acc = exact int32 sum, y32 = fp32(fp32(fp32(acc)*xs[m])*ws[n]),
//           y = bf16_rne(y32) (Japanese summary §2.2 items 1-3)
//   argmax: lowest index among equal maxima; acceptance: the longest draft
//           prefix equal to the target's argmax, then the target's token.
//
// Linear work split ("stream-K"): the weight of a linear is cut into
// blocks of two 16-channel tiles x 64 k (2 KiB, two MFMA operands that share
// one activation operand, contiguous per tile in the tiled layout); T =
// ceil(tiles16/2) * steps blocks.  Workgroup w of G takes the blocks
// [w*T/G, (w+1)*T/G) in (pair, k) order (one block each if T < G), so every
// workgroup streams the same number of bytes whatever the shape; its eight
// waves take the k steps of each pair segment round-robin (adjacent KiB) and
// reduce through LDS.  A pair covered by one workgroup is stored directly;
// a pair shared by several adds its int32 partials into a zeroed workspace
// with device-scope atomics (exact, order-free), and the last of its
// contributors (found by a per-pair arrival counter; the contributor count
// follows from the block ranges) applies the epilogue and zeroes the
// workspace and counter behind it.
//
// Barrier: everything a step hands to a later step is written and read with
// device-scope accesses (served at the device's coherence point, not from
// one XCD's L2), so each workgroup only waits for its stores to complete
// (vmcnt), adds one to a device-scope arrival counter and spins on it until
// all workgroups of the launch have arrived for that step.  The launch size
// is the number of workgroups that fit on the device at once (the occupancy
// query times the CU count), so on an otherwise idle device all of them are
// resident; every wait is also bounded by a wall-clock limit: past it the
// launch records a status word and every workgroup leaves, so a launch
// always terminates.  The last workgroup to leave resets the counters.
#include "../../include/w8a8.h"
#include "common.h"

#include <algorithm>
#include <climits>
#include <cstring>
#include <vector>

namespace w8a8 {

constexpr int kChainWaves = 8;
constexpr int kChainThreads = kChainWaves * kWave;
constexpr int kChainUnroll = 4;  // k steps per batch (two batches in flight per wave)
constexpr int kChainSegSlots = 32;  // pair segments per chunk of a linear (LDS slots)
constexpr int kChainSegWords = 2 * 4 * kWave;  // int32 per slot: two 16x16 int32 tiles
constexpr int kChainPerCu = 1;   // workgroups per CU (8 waves: two per SIMD, up to 256 VGPRs)
constexpr int kChainWavesPerSimd = kChainPerCu * kChainWaves / 4;
constexpr int kChainCache = 4;   // quantization: groups of 8 kept in registers
constexpr uint32_t kChainMagic = 0x31613877u;
constexpr int kChainMaxRows = 16;

struct ChainStep {  // 128 bytes, read with scalar loads
  int32_t kind, N, K, steps;
  int32_t tiles16, B, G, tpb;  // tpb: 16-channel tiles per block (1 or 2)
  int32_t blocks;  // tile pairs * steps (< 2^20: tiled weights are < 2 GiB)
  int32_t aligned; // 1: workgroup shares are whole tile groups (one contributor each)
  const void* in;
  const float* in_scale;  // LINEAR / LM_HEAD: x_scale; QUANTIZE: smoothing factors or null
  const int8_t* wq;
  const float* ws;
  void* out;
  float* out_f32;
  const int32_t* draft;
  int32_t* argmax;
  int32_t* accept_len;
  int32_t* next_token;
  int32_t wbytes;  // bytes of the tiled weights (< 2^31)
  int32_t pad2;
};
static_assert(sizeof(ChainStep) == 128, "ChainStep layout");

struct ChainHeader {
  uint32_t magic, n_steps, M, nwg;  // nwg: the launch size the plan was made for
  const ChainStep* steps;
  int32_t* part;
  uint32_t* count;
  unsigned long long* keys;
  uint32_t* sync;  // barrier words, one per 256-byte line (kSync*)
};

// The step table and header never change during a launch: they are read
// through the constant address space, so the loads are scalar and every
// field is wave-uniform.
template <class T>
__device__ __forceinline__ T chain_const_load(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "dword-sized");
  T v;
#if defined(__HIP_DEVICE_COMPILE__)
  typedef const uint32_t __attribute__((address_space(4)))* KWords;
  const KWords src = (KWords)p;
  uint32_t* dst = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) dst[i] = src[i];
#else
  v = *p;
#endif
  return v;
}

// plan layout (byte offsets)
// Barrier words (uint32), each on a 256-byte line of its own: per XCD group
// (workgroups w with w % 8 == x) an arrival and a leave counter and a release
// word, plus the global arrival and leave counters and the status word.
constexpr int kSyncLine = 64;
constexpr int kSyncArrive = 0, kSyncGlobalArrive = 8, kSyncRelease = 9, kSyncLeave = 17,
              kSyncGlobalLeave = 25, kSyncStatus = 26, kSyncLines = 27;
constexpr size_t kPlanSync = 256;
constexpr size_t kPlanSteps = kPlanSync + kSyncLines * 256;


// Blocks of a linear split over G workgroups: workgroup w starts at
// floor(w*T/G) when T >= G (every range then holds at least one block), else
// at min(w, T) (one block each, the rest idle), so no range in the middle
// is empty and the contributors of a tile are the owners of its first and
// last block and every workgroup between them.
// (All of it fits 32 bits: T < 2^20 and G <= 2048.)  The results are
// wave-uniform and moved to scalar registers.
__device__ __forceinline__ int chain_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int chain_split(int w, int T, int G) {
  return chain_uniform(T >= G ? (int)((unsigned)(w * T) / (unsigned)G) : min(w, T));
}
// Start of workgroup w's share.  An aligned step cuts at whole pairs (the
// same rule over the pairs), so every pair has one contributor.
__device__ __forceinline__ int chain_start(const ChainStep& st, int w, int G) {
  if (st.aligned) return chain_split(w, st.blocks / st.steps, G) * st.steps;
  return chain_split(w, st.blocks, G);
}
// The workgroup whose (block-granular) share holds block x.
__device__ __forceinline__ int chain_owner(int x, int T, int G) {
  return chain_uniform(T >= G ? (int)((unsigned)((x + 1) * G - 1) / (unsigned)T) : x);
}
// Contributors of pair p: the owners of its first and last block and every
// workgroup between them.
__device__ __forceinline__ int chain_contributors(const ChainStep& st, int p, int G) {
  if (st.aligned) return 1;
  const int x0 = p * st.steps;
  return chain_owner(x0 + st.steps - 1, st.blocks, G) - chain_owner(x0, st.blocks, G) + 1;
}

__device__ __forceinline__ bool chain_is_linear(int kind) {
  return kind == W8A8_CHAIN_LINEAR || kind == W8A8_CHAIN_LM_HEAD;
}

// Weight stream of a linear as a buffer resource: one VGPR offset per lane
// and segment, the block offsets in SGPRs; accesses past the end (none are
// made) would read zeros.  Non-temporal: each block is read once.
constexpr int kChainNt = 2;
constexpr int kChainSc1 = 16;  // device-scope access (served by the coherence point)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chain_weights(const ChainStep& st) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(st.wq), 0, st.wbytes, 0x00020000);
}

// Block x of a linear = (pair p, k step s) with x = p * steps + s: the two
// 16-channel tiles 2p and 2p+1 at k step s (the second absent past the last
// tile).  One batch: this wave's k steps s0 + wave + kChainWaves * (j + u),
// u < kChainUnroll, of the segment [s0, s0 + n) of pair p.  The loads carry
// no branches: a load that must read nothing gets an offset past the end of
// its buffer, which the hardware answers with zeros.
constexpr int kChainOob = 0x7ffffff0;
__device__ __forceinline__ void chain_load_batch(const ChainStep& st,
                                                 const __amdgpu_buffer_rsrc_t w, int p, int s0,
                                                 int J, int j, int wave, int lane,
                                                 v4i (&b)[kChainUnroll][2]) {
  const int steps = st.steps;
  const bool two = st.tpb == 2 && 2 * p + 1 < st.tiles16;
  const int voff = ((st.tpb * p * steps + s0 + wave) << 10) + (lane << 4);
#pragma unroll
  for (int u = 0; u < kChainUnroll; ++u) {
    const bool live = j + u < J;
    const int soff = (j + u) * (kChainWaves << 10);
    b[u][0] = __builtin_amdgcn_raw_buffer_load_b128(w, live ? voff : kChainOob, soff, kChainNt);
    b[u][1] = __builtin_amdgcn_raw_buffer_load_b128(w, (live && two) ? voff : kChainOob,
                                                     soff + (steps << 10), kChainNt);
  }
}

// Position of a wave in its workgroup's share of a linear: the segment of
// pair p at k steps [s0, s0 + n) (starting at block x), the wave's J steps
// in it, and the batch that starts at its j-th step.  A wave with no step in
// a segment still has one (empty) batch there, so every wave ends every
// segment exactly once (the reduction below waits for all of them).
struct ChainCursor {
  int x, p, s0, n, J, j;
};

__device__ __forceinline__ void chain_segment(ChainCursor& c, int steps, int b1, int wave) {
  c.p = chain_uniform((unsigned)c.x / (unsigned)steps);
  c.s0 = c.x - c.p * steps;
  c.n = min(steps - c.s0, b1 - c.x);
  c.J = c.n > wave ? (c.n - wave + kChainWaves - 1) / kChainWaves : 0;
  c.j = 0;
}

// Next batch; false past the end of the share.
__device__ __forceinline__ bool chain_advance(ChainCursor& c, int steps, int b1, int wave) {
  c.j += kChainUnroll;
  if (c.j < c.J) return true;
  c.x += c.n;
  if (c.x >= b1) return false;
  chain_segment(c, steps, b1, wave);
  return true;
}

// This wave's first batch in its workgroup's share of a linear (the batch
// chain_linear starts with).
__device__ __forceinline__ void chain_prefetch(const ChainStep& st, int wg, int nwg, int wave,
                                               int lane, v4i (&b)[kChainUnroll][2]) {
  const int b0 = chain_start(st, wg, nwg), b1 = chain_start(st, wg + 1, nwg);
  const int steps = st.steps;
  const int p = chain_uniform((unsigned)b0 / (unsigned)steps);
  const int s0 = b0 - p * steps;
  const int n = b0 < b1 ? min(steps - s0, b1 - b0) : 0;
  const int J = n > wave ? (n - wave + kChainWaves - 1) / kChainWaves : 0;
  chain_load_batch(st, chain_weights(st), p, s0, J, 0, wave, lane, b);
}

__device__ __forceinline__ unsigned long long chain_wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)(v & 0xffffffffull), off, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// Output of one tile pair, by one wave: `slot` points at this lane's words
// of the pair's LDS slot, element (tt, r) at slot[(tt * 4 + r) * 64]: rows
// 4*grp + r of channel 16*(2p+tt) + col; xsr[r] and wsr[tt] are the scales
// of those rows and channels.
__device__ __forceinline__ void chain_pair_out(const ChainStep& st, const ChainHeader& h, int M,
                                               int p, int32_t* slot, int contributors,
                                               const float (&xsr)[4], const float (&wsr)[2],
                                               int lane) {
  const bool argmax = st.kind == W8A8_CHAIN_LM_HEAD;
  const int col = lane & 15, grp = lane >> 4;
  const int N = st.N;
  if (contributors > 1) {
    // partial of a shared pair: exchanged through device-scope atomics, which
    // the hardware performs at one coherence point per address; the last
    // contributor takes the totals back into the slot
#pragma unroll 1
    for (int tt = 0; tt < 2; ++tt) {
      const int n = tt < st.tpb ? 16 * (st.tpb * p + tt) + col : N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * grp + r;
        if (m < M && n < N)
          __hip_atomic_fetch_add(&h.part[(size_t)m * N + n], slot[(tt * 4 + r) * kWave],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    uint32_t old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&h.count[p], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, kWave);
    if (old != (uint32_t)(contributors - 1)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll 1
    for (int tt = 0; tt < 2; ++tt) {
      const int n = tt < st.tpb ? 16 * (st.tpb * p + tt) + col : N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * grp + r;
        if (m < M && n < N)
          slot[(tt * 4 + r) * kWave] = __hip_atomic_exchange(
              &h.part[(size_t)m * N + n], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (lane == 0) __hip_atomic_exchange(&h.count[p], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = st.tpb * p + tt;
    const int n = tt < st.tpb ? 16 * t + col : N;
    float bv[4];
    int bi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * grp + r;
      bv[r] = -INFINITY;
      bi[r] = INT_MAX;
      if (m < M && n < N) {
        const float y = (static_cast<float>(slot[(tt * 4 + r) * kWave]) * xsr[r]) * wsr[tt];
        const size_t o = (size_t)m * (size_t)N + (size_t)n;
        if (st.out_f32)
          __hip_atomic_store(&st.out_f32[o], y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (st.out)
          __hip_atomic_store(&static_cast<uint16_t*>(st.out)[o], f32_to_bf16_rne(y),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bv[r] = y;
        bi[r] = n;
      }
    }
    if (argmax) {
      // (max, lowest index) over the tile's 16 channels, then one device-scope
      // atomic max into one of the row's sub-keys
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float ov = __shfl_xor(bv[r], off, kWave);
          const int oi = __shfl_xor(bi[r], off, kWave);
          if (ov > bv[r] || (ov == bv[r] && oi < bi[r])) { bv[r] = ov; bi[r] = oi; }
        }
        const int m = 4 * grp + r;
        if (col == 0 && m < M && bi[r] != INT_MAX) {
          const size_t sub = (size_t)m * kArgmaxSubkeys + (size_t)(t % kArgmaxSubkeys);
          __hip_atomic_fetch_max(&h.keys[sub * kArgmaxKeyStride], argmax_key(bv[r], bi[r]),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

// Activation operand of one batch: row `col` of xq (rows >= M lie past the
// buffer's end and read as zeros), the 16 k of lane group `grp` at this
// wave's k steps; k >= K (a ragged last step) and steps past the wave's
// share read zero.
__device__ __forceinline__ void chain_load_act(const __amdgpu_buffer_rsrc_t x, int K, int col,
                                               int grp, int s0, int J, int j, int wave,
                                               v4i (&a)[kChainUnroll]) {
  const int voff = col * K + grp * 16 + (s0 + wave) * 64;
#pragma unroll
  for (int u = 0; u < kChainUnroll; ++u) {
    const int s = s0 + wave + kChainWaves * (j + u);
    const bool ok = j + u < J && s * 64 + grp * 16 < K;
    a[u] = __builtin_amdgcn_raw_buffer_load_b128(x, ok ? voff : kChainOob,
                                                 (j + u) * kChainWaves * 64, kChainSc1);
  }
}

// One linear: this workgroup's blocks [b0, b1), in chunks of at most
// kChainSegSlots pair segments.  Each wave walks its batches with two
// register sets in turn: the loads of batch i+1 are issued before the MFMAs
// of batch i, across segment ends, so a wave keeps two batches in flight and
// never waits for the other waves while it streams; at the end of each of
// its segments it adds its partial tiles into the segment's LDS slot (LDS
// atomics).  After the chunk, the waves share out its pairs and store or
// hand off each one (only the first and last pair of a workgroup's share can
// have other contributors).  With use_pre, `pb` already holds the weights of
// the first batch (issued by chain_prefetch before the barrier).
__device__ __forceinline__ void chain_linear(const ChainStep& st, const ChainHeader& h, int M,
                                             int wg, int nwg, int32_t* seg,
                                             v4i (&pb)[kChainUnroll][2], bool use_pre) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = lane & 15, grp = lane >> 4;
  const int steps = st.steps, K = st.K;
  const int b0 = chain_start(st, wg, nwg), b1 = chain_start(st, wg + 1, nwg);
  const __amdgpu_buffer_rsrc_t w = chain_weights(st);
  const __amdgpu_buffer_rsrc_t xa =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(st.in), 0, M * K, 0x00020000);
  const v4i zero = v4i{0, 0, 0, 0};
  // the activation scales of this lane's output rows, loaded once: they
  // arrive while the weights stream
  float xsr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    xsr[r] = 4 * grp + r < M ? __hip_atomic_load(&st.in_scale[4 * grp + r], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT)
                             : 0.0f;
  bool pre = use_pre;
#pragma unroll 1
  for (int cx = b0; cx < b1;) {
    const int p_first = chain_uniform((unsigned)cx / (unsigned)steps);
    const int ce = min(b1, (p_first + kChainSegSlots) * steps);
    const int nseg = chain_uniform((unsigned)(ce - 1) / (unsigned)steps) - p_first + 1;
    for (int i = threadIdx.x; i < nseg * kChainSegWords; i += kChainThreads) seg[i] = 0;
    // the weight scales of the (up to four) pairs this wave stores after the
    // chunk, loaded now so that they arrive while the weights stream
    float wsr[kChainSegSlots / kChainWaves][2];
#pragma unroll
    for (int i = 0; i < kChainSegSlots / kChainWaves; ++i)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int n = tt < st.tpb ? 16 * (st.tpb * (p_first + wave + kChainWaves * i) + tt) + col
                                  : st.N;
        wsr[i][tt] = (wave + kChainWaves * i < nseg && n < st.N) ? st.ws[n] : 0.0f;
      }
    __syncthreads();
    v4i acc[2] = {zero, zero};
    auto mfma = [&](const v4i (&a)[kChainUnroll], const v4i (&b)[kChainUnroll][2]) {
#pragma unroll
      for (int u = 0; u < kChainUnroll; ++u) {
        acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][0], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[u][1], acc[1], 0, 0, 0);
      }
    };
    // end of this wave's part of a segment: add it into the segment's slot
    auto flush = [&](int p) {
      int32_t* slot = seg + (p - p_first) * kChainSegWords + lane;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) atomicAdd(slot + (tt * 4 + r) * kWave, acc[tt][r]);
      acc[0] = zero;
      acc[1] = zero;
    };
    ChainCursor c;
    c.x = cx;
    chain_segment(c, steps, ce, wave);
    v4i pa[kChainUnroll], qa[kChainUnroll], qb[kChainUnroll][2];
    chain_load_act(xa, K, col, grp, c.s0, c.J, c.j, wave, pa);
    if (!pre) chain_load_batch(st, w, c.p, c.s0, c.J, c.j, wave, lane, pb);
    pre = false;
    ChainCursor cur = c;
    bool more = chain_advance(c, steps, ce, wave);
#pragma unroll 1
    while (true) {
      // batch `cur` is in (pa, pb); `c` is the next one
      if (more) {
        chain_load_act(xa, K, col, grp, c.s0, c.J, c.j, wave, qa);
        chain_load_batch(st, w, c.p, c.s0, c.J, c.j, wave, lane, qb);
      }
      mfma(pa, pb);
      if (cur.j + kChainUnroll >= cur.J) flush(cur.p);
      if (!more) break;
      cur = c;
      more = chain_advance(c, steps, ce, wave);
      // batch `cur` is in (qa, qb)
      if (more) {
        chain_load_act(xa, K, col, grp, c.s0, c.J, c.j, wave, pa);
        chain_load_batch(st, w, c.p, c.s0, c.J, c.j, wave, lane, pb);
      }
      mfma(qa, qb);
      if (cur.j + kChainUnroll >= cur.J) flush(cur.p);
      if (!more) break;
      cur = c;
      more = chain_advance(c, steps, ce, wave);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kChainSegSlots / kChainWaves; ++i) {
      const int k = wave + kChainWaves * i;
      if (k < nseg) {
        const int p = p_first + k;
        chain_pair_out(st, h, M, p, seg + k * kChainSegWords + lane,
                       chain_contributors(st, p, nwg), xsr, wsr[i], lane);
      }
    }
    __syncthreads();
    cx = ce;
  }
}

// One row of QUANTIZE (all threads of the workgroup).
__device__ __forceinline__ void chain_quant_row(const ChainStep& st, int row, float* red_f) {
  const int tid = threadIdx.x;
  const int K = st.K;
  const uint16_t* in_row = static_cast<const uint16_t*>(st.in) + (size_t)row * (size_t)K;
  const float* smooth = st.in_scale;
  constexpr int kStride = kChainThreads * 8;
  auto load8 = [&](int k, float v[8]) {
    const uint64_t* src = reinterpret_cast<const uint64_t*>(in_row + k);
    const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t w[4] = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    if (smooth) {
      const float4 s0 = *reinterpret_cast<const float4*>(smooth + k);
      const float4 s1 = *reinterpret_cast<const float4*>(smooth + k + 4);
      const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = v[i] * s[i];
    }
  };
  float cache[kChainCache][8];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < kChainCache; ++c) {
    const int k = tid * 8 + c * kStride;
    if (k < K) {
      load8(k, cache[c]);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(cache[c][i]));
    }
  }
#pragma unroll 1
  for (int k = tid * 8 + kChainCache * kStride; k < K; k += kStride) {
    float v[8];
    load8(k, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  if ((tid & (kWave - 1)) == 0) red_f[tid / kWave] = amax;
  __syncthreads();
  amax = red_f[0];
#pragma unroll
  for (int w = 1; w < kChainWaves; ++w) amax = fmaxf(amax, red_f[w]);
  const float s = amax / 127.0f;
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (tid == 0)
    __hip_atomic_store(&st.out_f32[row], amax > 0.0f ? s : 0.0f, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  int8_t* q = static_cast<int8_t*>(st.out) + (size_t)row * (size_t)K;
  auto emit = [&](int k, const float v[8]) {
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float r = __builtin_rintf(v[i] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      const int qi = (v[i] == 0.0f) ? 0 : (int)r;
      packed[i >> 2] |= ((uint32_t)(qi & 0xff)) << (8 * (i & 3));
    }
    __hip_atomic_store(reinterpret_cast<uint64_t*>(q + k),
                       ((uint64_t)packed[1] << 32) | packed[0], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  };
#pragma unroll
  for (int c = 0; c < kChainCache; ++c) {
    const int k = tid * 8 + c * kStride;
    if (k < K) emit(k, cache[c]);
  }
#pragma unroll 1
  for (int k = tid * 8 + kChainCache * kStride; k < K; k += kStride) {
    float v[8];
    load8(k, v);
    emit(k, v);
  }
}

// ACCEPT (workgroup 0): per row the maximum of its sub-keys (each exchanged
// with zero, leaving the keys zero for the next LM head), then per sequence
// the walk along the draft.
__device__ __forceinline__ void chain_accept(const ChainStep& st, const ChainHeader& h, int M,
                                             int* s_arg) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll 1
  for (int i = wave; i < M; i += kChainWaves) {
    unsigned long long k = 0;
    if (lane < kArgmaxSubkeys)
      k = __hip_atomic_exchange(&h.keys[((size_t)i * kArgmaxSubkeys + lane) * kArgmaxKeyStride],
                                0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    k = chain_wave_max_u64(k);
    if (lane == 0) {
      const int a = k ? (int)(~(uint32_t)(k & 0xffffffffull)) : 0;
      s_arg[i] = a;
      if (st.argmax) st.argmax[i] = a;
    }
  }
  __syncthreads();
  const int G = st.G;
  if ((int)threadIdx.x < st.B) {
    const int b = threadIdx.x;
    const int* row = s_arg + b * (G + 1);
    int n = 0;
    while (n < G && st.draft[(size_t)b * G + n] == row[n]) ++n;
    st.accept_len[b] = n;
    st.next_token[b] = row[n];
  }
}

__device__ __forceinline__ uint32_t* chain_sync(const ChainHeader& h, int line) {
  return h.sync + line * kSyncLine;
}

// The barrier is a two-level tree: the workgroups of one XCD group (w % 8)
// count into their group's counter, the last of a group into the global
// counter, and the last group writes every group's release word, on which
// that group's workgroups spin.  Same-address device-scope atomics are
// serialized at the coherence point, so no address sees more than one
// group's workgroups.  Counters only grow during a launch; the last
// workgroup to leave resets them all.
//
// Arrival at the barrier that ends step `step`.  Everything one step hands
// to a later one (linear outputs, codes, scales, partial sums, argmax keys)
// is written and read with device-scope accesses, which the hardware serves
// at the device's coherence point rather than in one XCD's L2, so the
// barrier needs no cache write-back or invalidate: each wave waits until its
// stores have completed before the workgroup is counted.
__device__ __forceinline__ void chain_arrive(const ChainHeader& h, int step, int wg, int nwg) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int x = wg % kXcds;
    const uint32_t groups = (uint32_t)min(nwg, kXcds);
    const uint32_t gx = (uint32_t)((nwg - x + kXcds - 1) / kXcds);
    const uint32_t n = (uint32_t)step + 1;
    const uint32_t old = __hip_atomic_fetch_add(chain_sync(h, kSyncArrive + x), 1u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == n * gx - 1) {
      const uint32_t o2 = __hip_atomic_fetch_add(chain_sync(h, kSyncGlobalArrive), 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 == n * groups - 1)
        for (uint32_t y = 0; y < groups; ++y)
          __hip_atomic_store(chain_sync(h, kSyncRelease + y), n, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Wait until steps 0..step-1 are complete; false if the launch was aborted
// (the wall-clock limit passed here or in another workgroup).
__device__ __forceinline__ bool chain_wait(const ChainHeader& h, int step, int wg,
                                           uint64_t tick_limit, int* s_ok) {
  if (threadIdx.x == 0) {
    const uint32_t* rel = chain_sync(h, kSyncRelease + wg % kXcds);
    uint32_t* status = chain_sync(h, kSyncStatus);
    int ok = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
    const uint64_t t0 = wall_clock64();
    for (uint32_t it = 1; ok && __hip_atomic_load(rel, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                                    (uint32_t)step; ++it) {
      if ((it & 255u) == 0u &&
          __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
        ok = 0;
      else if (wall_clock64() - t0 > tick_limit) {
        __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
      } else {
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    *s_ok = ok;
  }
  __syncthreads();
  return *s_ok != 0;
}

// Leave: the same tree; the last workgroup out (every other one has finished
// all its waits by then) resets every counter and release word.
__device__ __forceinline__ void chain_leave(const ChainHeader& h, int wg, int nwg) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int x = wg % kXcds;
    const uint32_t groups = (uint32_t)min(nwg, kXcds);
    const uint32_t gx = (uint32_t)((nwg - x + kXcds - 1) / kXcds);
    const uint32_t old = __hip_atomic_fetch_add(chain_sync(h, kSyncLeave + x), 1u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gx - 1) {
      const uint32_t o2 = __hip_atomic_fetch_add(chain_sync(h, kSyncGlobalLeave), 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (o2 == groups - 1) {
        for (int line = 0; line < kSyncStatus; ++line)
          __hip_atomic_store(chain_sync(h, line), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__global__ __launch_bounds__(kChainThreads, kChainWavesPerSimd) void chain_kernel(
    const ChainHeader* __restrict__ hp, uint64_t tick_limit) {
  __shared__ int32_t seg[kChainSegSlots * kChainSegWords];
  __shared__ float red_f[kChainWaves];
  __shared__ int s_arg[kChainMaxRows];
  __shared__ int s_ok;
  // the header and the step table are read in parallel (the table sits at
  // a fixed offset in the plan)
  const ChainHeader h = chain_const_load(hp);
  const ChainStep* steps =
      reinterpret_cast<const ChainStep*>(reinterpret_cast<const char*>(hp) + kPlanSteps);
  if (h.magic != kChainMagic) return;
  const int nwg = gridDim.x, wg = blockIdx.x;
  if ((uint32_t)nwg != h.nwg) {  // prepared for another launch size: nothing runs
    if (wg == 0 && threadIdx.x == 0)
      __hip_atomic_store(chain_sync(h, kSyncStatus), 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int M = (int)h.M;
  const int n_steps = (int)h.n_steps;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  v4i pre[kChainUnroll][2];
  int pre_step = -1;  // step whose first batch `pre` holds
  // Work of this workgroup in a step other than a linear.
  auto busy = [&](int kind) {
    return (kind == W8A8_CHAIN_QUANTIZE && wg < M) || (kind == W8A8_CHAIN_ACCEPT && wg == 0);
  };
#pragma unroll 1
  for (int i = 0; i < n_steps; ++i) {
    const ChainStep st = chain_const_load(steps + i);
    if (i > 0) {
      // before waiting, issue the first weight loads of the next linear this
      // workgroup will stream, unless it has other work before it (its own
      // loads would queue behind them)
      if (pre_step < i) {
#pragma unroll 1
        for (int j = i; j < n_steps; ++j) {
          const int kind = chain_const_load(steps + j).kind;
          if (chain_is_linear(kind)) {
            const ChainStep sj = chain_const_load(steps + j);
            chain_prefetch(sj, wg, nwg, wave, lane, pre);
            pre_step = j;
            break;
          }
          if (busy(kind)) break;
        }
      }
      if (!chain_wait(h, i, wg, tick_limit, &s_ok)) break;
    }
    if (chain_is_linear(st.kind)) {
      chain_linear(st, h, M, wg, nwg, seg, pre, pre_step == i);
    } else if (st.kind == W8A8_CHAIN_QUANTIZE) {
      if (wg < M) chain_quant_row(st, wg, red_f);
    } else if (st.kind == W8A8_CHAIN_ACCEPT) {
      if (wg == 0) chain_accept(st, h, M, s_arg);
    }
    if (i + 1 < n_steps) chain_arrive(h, i, wg, nwg);
  }
  chain_leave(h, wg, nwg);
}

struct ChainSizes {
  size_t steps_end, count_off, part_off, keys_off, total;
};

static ChainSizes chain_sizes(const w8a8_chain_op* ops, int n, int64_t M) {
  int64_t max_tiles = 0, max_mn = 0;
  bool head = false;
  for (int i = 0; i < n; ++i) {
    if (ops[i].kind == W8A8_CHAIN_LINEAR || ops[i].kind == W8A8_CHAIN_LM_HEAD) {
      max_tiles = std::max(max_tiles, (ops[i].N + 15) / 16);
      max_mn = std::max(max_mn, M * ops[i].N);
    }
    head = head || ops[i].kind == W8A8_CHAIN_LM_HEAD;
  }
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  ChainSizes s;
  s.steps_end = kPlanSteps + (size_t)n * sizeof(ChainStep);
  s.count_off = up(s.steps_end);
  s.part_off = up(s.count_off + (size_t)max_tiles * sizeof(uint32_t));
  s.keys_off = up(s.part_off + (size_t)max_mn * sizeof(int32_t));
  s.total = s.keys_off + (head ? (size_t)M * kArgmaxSubkeys * kArgmaxKeyStride * 8 : 0);
  return s;
}

}  // namespace w8a8

// Launch size: the workgroups that fit on the device at once.
static hipError_t chain_grid(int* grid, uint64_t* ticks) {
  using namespace w8a8;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = 0, per_cu = 0, khz = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chain_kernel, kChainThreads, 0);
  if (e != hipSuccess) return e;
  if (cus <= 0 || per_cu <= 0 || khz <= 0) return hipErrorInvalidConfiguration;
  *grid = cus * std::min(per_cu, kChainPerCu);
  *ticks = (uint64_t)khz * 1000ull;  // one second of wall clock per wait
  return hipSuccess;
}

size_t w8a8_chain_plan_bytes_impl(const w8a8_chain_op* ops, int n_ops, int64_t M) {
  return w8a8::chain_sizes(ops, n_ops, M).total;
}

hipError_t w8a8_chain_prepare_impl(const w8a8_chain_op* ops, int n_ops, int64_t M, void* plan,
                                   hipStream_t stream) {
  using namespace w8a8;
  const ChainSizes sz = chain_sizes(ops, n_ops, M);
  int nwg = 0;
  uint64_t ticks = 0;
  hipError_t ge = chain_grid(&nwg, &ticks);
  if (ge != hipSuccess) return ge;
  char* base = static_cast<char*>(plan);
  std::vector<char> host(sz.steps_end, 0);
  ChainHeader hd{};
  hd.magic = kChainMagic;
  hd.n_steps = (uint32_t)n_ops;
  hd.M = (uint32_t)M;
  hd.nwg = (uint32_t)nwg;
  hd.steps = reinterpret_cast<const ChainStep*>(base + kPlanSteps);
  hd.count = reinterpret_cast<uint32_t*>(base + sz.count_off);
  hd.part = reinterpret_cast<int32_t*>(base + sz.part_off);
  hd.keys = reinterpret_cast<unsigned long long*>(base + sz.keys_off);
  hd.sync = reinterpret_cast<uint32_t*>(base + kPlanSync);
  std::memcpy(host.data(), &hd, sizeof(hd));
  for (int i = 0; i < n_ops; ++i) {
    const w8a8_chain_op& o = ops[i];
    ChainStep s{};
    s.kind = o.kind;
    s.N = (int32_t)o.N;
    s.K = (int32_t)o.K;
    s.steps = (int32_t)((o.K + 63) / 64);
    s.tiles16 = (int32_t)((o.N + 15) / 16);
    // Blocks of one or two tiles x one k step, and whole groups per
    // workgroup or an even split (stream-K): the choice with the least
    // streaming for the busiest workgroup, a shared group's hand-off (a few
    // device-scope round trips under load) counted as ~100 KiB.  One CU
    // cannot pull much more than its share of HBM, so a CU left idle is not
    // made up by the others.
    {
      const int64_t kib = s.steps, handoff = 100;
      const int64_t u1 = s.tiles16, u2 = (s.tiles16 + 1) / 2;
      const int64_t a2 = (u2 + nwg - 1) / nwg * 2 * kib, a1 = (u1 + nwg - 1) / nwg * kib;
      const int64_t sk = (int64_t)s.tiles16 * kib / nwg + handoff;
      s.tpb = a1 < a2 && a1 <= sk ? 1 : 2;
      s.aligned = std::min(a1, a2) <= sk ? 1 : 0;
    }
    s.blocks = (s.tiles16 + s.tpb - 1) / s.tpb * s.steps;  // tile groups x k steps
    s.wbytes = (int32_t)std::min<int64_t>((int64_t)s.tiles16 * s.steps * 1024, INT32_MAX);
    s.B = (int32_t)o.B;
    s.G = (int32_t)o.G;
    s.in = o.in;
    s.in_scale = o.kind == W8A8_CHAIN_QUANTIZE ? o.smooth : o.in_scale;
    s.wq = o.wq_tiled;
    s.ws = o.w_scale;
    s.out = o.out;
    s.out_f32 = o.out_f32;
    s.draft = o.draft;
    s.argmax = o.argmax;
    s.accept_len = o.accept_len;
    s.next_token = o.next_token;
    std::memcpy(host.data() + kPlanSteps + (size_t)i * sizeof(ChainStep), &s, sizeof(s));
  }
  hipError_t e = hipMemsetAsync(base + sz.steps_end, 0, sz.total - sz.steps_end, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(base, host.data(), sz.steps_end, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e;
}

hipError_t w8a8_launch_chain(const void* plan, hipStream_t stream) {
  using namespace w8a8;
  int grid = 0;
  uint64_t ticks = 0;
  hipError_t e = chain_grid(&grid, &ticks);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chain_kernel, dim3((unsigned)grid), dim3(kChainThreads), 0, stream,
                     reinterpret_cast<const ChainHeader*>(plan), ticks);
  return hipGetLastError();
}

hipError_t w8a8_chain_read_status(const void* plan, int32_t* status, hipStream_t stream) {
  using namespace w8a8;
  hipError_t e = hipMemcpyAsync(status, static_cast<const char*>(plan) + kPlanSync +
                                    (size_t)kSyncStatus * kSyncLine * sizeof(uint32_t),
                                sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return e;
}

int w8a8_chain_grid_size() {
  int grid = 0;
  uint64_t ticks = 0;
  return chain_grid(&grid, &ticks) == hipSuccess ? grid : 0;
}
