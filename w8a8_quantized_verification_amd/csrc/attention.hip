// Attention of the verified block over the KV cache (gfx950): the softmax
// part of the verifier, kept in high precision after the dequant step
// (gist.science German summary, Technische Zusammenfassung §2
// "De-Quantisierung"; Italian summary §2 pipeline; Japanese summary §2.2
// item 3).  For each sequence b the T = G + 1 verified positions attend,
// causally, to the first L_b cache positions (the last T of them are the
// block's own keys): query i reads keys j <= L_b - T + i; grouped-query
// heads (query head h reads kv head h / (Hq / Hkv)); head dimension 128;
// fp32 softmax, bf16 output.
//
// Split over the keys (flash-decoding): a workgroup of four waves per
// (split, kv head, b); each wave streams its quarter of the split's cache
// positions in blocks of 16, with every query row that reads its kv head
// (T x Hq/Hkv rows, <= 64) held in registers, an online softmax per row,
// and its blocks requested in bursts of 2-6 before they are multiplied.
// Both products run on the bf16 MFMA straight from registers (no LDS
// staging), blocks taken in pairs:
//   S^T = K Q^T  (v_mfma_f32_16x16x32_bf16 per block; A = 16 keys,
//                 B = 16 query rows),
//   O^T += V^T P^T (v_mfma_f32_16x16x32_bf16 over the pair's 32 positions;
//                   A = 16 dims, B = P^T in exactly the lanes S^T left it).
// The four waves' states merge in LDS into one partial result per
// workgroup; a second kernel merges the splits of each row.  Bound by
// reading the cache: 2 * 128 * 2 bytes per position and kv head.
//
// Cache layouts.  K: [B][Hkv][Lmax][128], one row per position.  The MFMA
// sums over the 128 dims in any order, so lane (c, g) = (lane % 16, lane /
// 16) takes dims 32g .. 32g+31 of key row c (64 contiguous bytes) as its 4
// k-steps, and the query operand uses the same order.  V: blocked, 16
// positions x 128 dims per 4 KiB block, ordered so that lane (c, g) reads
// 64 contiguous bytes that hold, for each dim block db, the values of dim
// 16 db + c at the 4 positions 4g .. 4g+3 of the block: position p, dim d
// of (b, h) is element
//   (p / 16) * 2048 + ((p % 16 / 4) * 16 + d % 16) * 32 + (d / 16) * 4 + p % 4
// of its [Lmax * 128] slab (Lmax a multiple of 16).
#include "common.h"

#include <algorithm>
#include <cmath>

namespace w8a8 {

constexpr int kDh = 128;
constexpr int kVBlk = 16;               // cache positions per block
constexpr int kAttnMaxRows = 64;        // T * Hq / Hkv
constexpr int kTargetWaves = 1024;      // 1 wave per SIMD
constexpr int kAttnWaves = 4;           // waves per workgroup (merged in LDS)

// Most blocks requested together by one wave (its register buffers), by
// the number of 16-row query blocks: as many as fit beside Q and O.
constexpr int attn_max_burst(int qb) { return qb == 1 ? 4 : qb == 2 ? 6 : qb == 3 ? 4 : 2; }

// element index of (position p, dim d) inside one (b, kv head) V slab
__host__ __device__ inline size_t v_blocked_index(int p, int d) {
  const int in = p % kVBlk;
  return (size_t)(p / kVBlk) * (kVBlk * kDh) +
         (size_t)(((in / 4) * 16 + (d % 16)) * 32 + (d / 16) * 4 + (in % 4));
}

struct AttnArgs {
  const uint16_t* q;      // [B][T][Hq][128]
  const uint16_t* k;      // [B][Hkv][Lmax][128]
  const uint16_t* v;      // [B][Hkv][Lmax/16] blocks of 16 x 128 (v_blocked_index)
  const int32_t* len;     // [B]
  int B, T, Hq, Hkv, Lmax, nsplit, split_keys;
  float* part_o;          // [B][Hkv][nsplit][rows][128]
  float* part_ml;         // [B][Hkv][nsplit][rows][2]: running max (log2 units), sum
  uint16_t* out;          // [B][T][Hq][128]
};

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

// 1/sqrt(128) * log2(e): scores go straight to the base-2 exponent
constexpr float kScoreToLog2 = 0.08838834764831845f * 1.4426950408889634f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

// v op v' where v' is the value of lane ^ 16 (resp. ^ 32), for a commutative
// op: the swap instructions return both halves of the pair {own, partner}
// (the order differs between the two rows of the pair, which a commutative
// op does not see)
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void attn_load_block(const uint16_t* kp, const uint16_t* vp,
                                                uint4 (&kr)[4], uint4 (&vr)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    kr[u] = reinterpret_cast<const uint4*>(kp)[u];
    vr[u] = reinterpret_cast<const uint4*>(vp)[u];
  }
}

template <int QB>
struct AttnState {
  v4f o[QB][kDh / 16];   // O^T: lane (c, g) holds query row 16 qb + c, dims 16 db + 4 g .. +3
  float m[QB];           // running row max (log2 units; equal across the 4 lanes of a row)
  float l[QB];           // running partial row sum (this lane's keys)
};

// Two blocks of 16 positions, starting at p0 (a multiple of 32 from the
// wave's start) and p0 + 16; positions >= p_hi (the end of this wave's
// range) or past a row's last visible position get zero weight.
//
// S^T of each block on v_mfma_f32_16x16x32_bf16 (4 k-steps over the dims);
// then O^T += V^T P^T over the 32 positions on the same instruction: lane
// (c, g)'s 8 k-slots are positions 4g .. 4g+3 of the first block, then of
// the second, in both operands (the V bytes of both blocks side by side,
// and P exactly as the two S^T results hold it).
//
// Lazy rescaling: a row's reference maximum m moves only when a pair's
// maximum exceeds it by more than kRescaleSlack (log2 units), so the
// weights exp2(s - m) stay <= 2^kRescaleSlack and O and l are rescaled
// rarely (the result is the same for any reference; only the rounding of
// the partial sums moves).
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ void attn_mask_v(uint4 (&vr)[4], const uint4 (&vr_in)[4], int pg, int L) {
  // positions >= L hold arbitrary bits: their weights are zero, and their
  // values must be too (0 * NaN)
  const uint32_t m01 = (pg + 0 < L ? 0x0000ffffu : 0u) | (pg + 1 < L ? 0xffff0000u : 0u);
  const uint32_t m23 = (pg + 2 < L ? 0x0000ffffu : 0u) | (pg + 3 < L ? 0xffff0000u : 0u);
#pragma unroll
  for (int u = 0; u < 4; ++u)
    vr[u] = make_uint4(vr_in[u].x & m01, vr_in[u].y & m23, vr_in[u].z & m01, vr_in[u].w & m23);
}

template <int QB>
__device__ __forceinline__ void attn_pair(AttnState<QB>& st, const uint4 (&qf)[QB][4],
                                          const int (&lim)[QB], const uint4 (&ka)[4],
                                          const uint4 (&va_in)[4], const uint4 (&kb)[4],
                                          const uint4 (&vb_in)[4], int p0, int p_hi, int L,
                                          int grp) {
  const int pg = p0 + 4 * grp;           // this lane's positions: pg + r, pg + 16 + r
  uint4 va[4], vb[4];
  attn_mask_v(va, va_in, pg, L);
  attn_mask_v(vb, vb_in, pg + kVBlk, L);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    v4f sa = v4f{0.f, 0.f, 0.f, 0.f}, sb = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ka[ks]),
                                                    __builtin_bit_cast(v8bf, qf[qb][ks]), sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, kb[ks]),
                                                    __builtin_bit_cast(v8bf, qf[qb][ks]), sb, 0, 0, 0);
    }
    // lane holds query row 16 qb + c
    const int vis_end = min(lim[qb] + 1, p_hi);
    float sv[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = (pg + r < vis_end) ? sa[r] * kScoreToLog2 : -INFINITY;
      sv[4 + r] = (pg + kVBlk + r < vis_end) ? sb[r] * kScoreToLog2 : -INFINITY;
    }
    float bm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    bm = max_xor32(max_xor16(bm));
    // the row's reference moves up to bm when bm exceeds it by the slack
    // (always on its first visible pair, where m = -inf)
    const bool move = bm > st.m[qb] + kRescaleSlack;
    if (__any(move)) {
      // 1 for a row that keeps its reference (also one with no visible key
      // yet, m = -inf); 0 for a row's first visible pair
      const float alpha = move ? exp2_hw(st.m[qb] - bm) : 1.0f;
      st.m[qb] = move ? bm : st.m[qb];
      st.l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < kDh / 16; ++db) st.o[qb][db] *= alpha;
    }
    const float mu = (st.m[qb] == -INFINITY) ? 0.0f : st.m[qb];
    // P as the sum of two bf16 values (hi + lo carries ~16 significant bits),
    // so that the product keeps the softmax weights at fp32-like precision
    // (hardware fp32 -> bf16 conversion, round to nearest even; P is finite)
    float pf[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) pf[r] = exp2_hw(sv[r] - mu);
    st.l[qb] += ((pf[0] + pf[1]) + (pf[2] + pf[3])) + ((pf[4] + pf[5]) + (pf[6] + pf[7]));
    v8bf hb, lb;
#pragma unroll
    for (int r = 0; r < 8; ++r) hb[r] = (__bf16)pf[r];
#pragma unroll
    for (int r = 0; r < 8; ++r) lb[r] = (__bf16)(pf[r] - (float)hb[r]);
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) {
      const uint4 wa = va[db / 2], wb = vb[db / 2];
      const uint4 w = (db & 1) ? make_uint4(wa.z, wa.w, wb.z, wb.w) : make_uint4(wa.x, wa.y, wb.x, wb.y);
      const v8bf vop = __builtin_bit_cast(v8bf, w);
      v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, hb, st.o[qb][db], 0, 0, 0);
      st.o[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, lb, acc, 0, 0, 0);
    }
  }
}

// A wave's state in LDS for the merge, lane-ordered (conflict-free 16-byte
// accesses).
template <int QB>
struct AttnSlot {
  v4f o[QB][kDh / 16][kWave];
  float m[QB][kWave];
  float l[QB][kWave];
};

template <int QB>
__device__ __forceinline__ void attn_store(AttnSlot<QB>& sl, const AttnState<QB>& st, int lane) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    sl.m[qb][lane] = st.m[qb];
    sl.l[qb][lane] = st.l[qb];
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) sl.o[qb][db][lane] = st.o[qb][db];
  }
}

// st <- st merged with the state in sl (the same rows and dims per lane)
template <int QB>
__device__ __forceinline__ void attn_merge(AttnState<QB>& st, const AttnSlot<QB>& sl, int lane) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float mo = sl.m[qb][lane];
    const float M = fmaxf(st.m[qb], mo);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    const float fa = exp2_hw(st.m[qb] - Ms), fb = exp2_hw(mo - Ms);   // 0 for m = -inf
    st.m[qb] = M;
    st.l[qb] = fa * st.l[qb] + fb * sl.l[qb][lane];
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) st.o[qb][db] = fa * st.o[qb][db] + fb * sl.o[qb][db][lane];
  }
}

// Workgroup (split, kv head, b): kAttnWaves waves, wave w on positions
// [split * split_keys + w * split_keys / kAttnWaves, + split_keys / kAttnWaves),
// each with its own online softmax; their states are merged in LDS (a
// two-level tree over two slots), and wave 0 writes one partial result per
// row.
template <int QB, int NB>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_split_kernel(AttnArgs a) {
  __shared__ AttnSlot<QB> slot[2];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int c = lane & 15, grp = lane >> 4;
  const int group = a.Hq / a.Hkv;
  const int rows = a.T * group;
  int L = a.len[b];
  L = L < a.T ? a.T : (L > a.Lmax ? a.Lmax : L);
  if (split * a.split_keys >= L) return;   // whole workgroup; the combine reads splits below L only
  const int wkeys = a.split_keys / kAttnWaves;
  const int p_begin = split * a.split_keys + wave * wkeys;
  const int p_end = min(p_begin + wkeys, L);
  const int nb = p_end > p_begin ? (p_end - p_begin + kVBlk - 1) / kVBlk : 0;

  // query rows j = 16 qb + c (row j is query position j / group, head
  // kvh * group + j % group), dims 32 grp .. +31; lim = last visible position
  uint4 qf[QB][4];
  int lim[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int j = qb * 16 + c;
    lim[qb] = -1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[qb][ks] = make_uint4(0u, 0u, 0u, 0u);
    if (j < rows && nb > 0) {
      const int i = j / group, h = kvh * group + (j - i * group);
      const uint4* src = reinterpret_cast<const uint4*>(
          a.q + (((size_t)b * a.T + i) * a.Hq + h) * kDh + grp * 32);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qf[qb][ks] = src[ks];
      lim[qb] = L - a.T + i;
    }
  }

  AttnState<QB> st;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    st.m[qb] = -INFINITY;
    st.l[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < kDh / 16; ++db) st.o[qb][db] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  const size_t slab = ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * kDh;
  const uint16_t* kp = a.k + slab + (size_t)c * kDh + grp * 32;   // + p0 * 128
  const uint16_t* vp = a.v + slab + (size_t)lane * 32;            // + p0 * 128 (block p0 / 16)
  // Bursts of NB blocks (NB even: pairs): each iteration requests its NB
  // blocks at once and computes them in order as they arrive, so that nothing is in flight
  // across the loop's back edge (the buffers are fixed registers, and the
  // waits stay exact).  Loads past the range are clamped to the last block;
  // blocks past the range compute with zero weight.
  for (int n = 0; n < nb; n += NB) {
    uint4 kbuf[NB][4], vbuf[NB][4];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const size_t pu = (size_t)p_begin + (size_t)min(n + u, nb - 1) * kVBlk;
      attn_load_block(kp + pu * kDh, vp + pu * kDh, kbuf[u], vbuf[u]);
    }
#pragma unroll
    for (int u = 0; u < NB; u += 2)
      attn_pair<QB>(st, qf, lim, kbuf[u], vbuf[u], kbuf[u + 1], vbuf[u + 1],
                    p_begin + (n + u) * kVBlk, p_end, L, grp);
  }
  // row sums over the row's 4 lanes (each of them then holds the total)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) st.l[qb] = sum_xor32(sum_xor16(st.l[qb]));

  static_assert(kAttnWaves == 4, "two-level merge of four waves");
  if (wave >= 2) attn_store<QB>(slot[wave - 2], st, lane);
  __syncthreads();
  if (wave < 2) attn_merge<QB>(st, slot[wave], lane);
  __syncthreads();
  if (wave == 1) attn_store<QB>(slot[0], st, lane);
  __syncthreads();
  if (wave != 0) return;
  attn_merge<QB>(st, slot[0], lane);

  const size_t base = (((size_t)b * a.Hkv + kvh) * a.nsplit + split) * rows;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int j = qb * 16 + c;
    if (j < rows) {
      if (grp == 0) {
        a.part_ml[(base + j) * 2] = st.m[qb];
        a.part_ml[(base + j) * 2 + 1] = st.l[qb];
      }
      float* dst = a.part_o + (base + j) * kDh + 4 * grp;
#pragma unroll
      for (int db = 0; db < kDh / 16; ++db)
        *reinterpret_cast<float4*>(dst + 16 * db) =
            make_float4(st.o[qb][db][0], st.o[qb][db][1], st.o[qb][db][2], st.o[qb][db][3]);
    }
  }
}

// One workgroup per output row (b, i, h): the weights of the splits that
// saw keys, exp2(m_s - max m), then sum_s w_s O_s / sum_s w_s l_s.  Thread
// t takes dims 2 (t % 64) .. +1 of the splits s = t / 64 (mod 4); the first
// kCombineUnroll of its splits have their (m, l) and partial O loaded in
// one round (longer rows loop over the rest).
constexpr int kCombineThreads = 256;
constexpr int kCombineGroups = kCombineThreads / kWave;
constexpr int kCombineUnroll = 8;
static_assert(kCombineGroups == 4, "the sums below take four groups");

__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
  __shared__ float red[2][kCombineGroups];
  __shared__ float2 part[kCombineGroups - 1][kWave];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, dp = t & (kWave - 1), g = t / kWave;
  const int group = a.Hq / a.Hkv;
  const int kvh = h / group, j = i * group + h % group, rows = a.T * group;
  int L = a.len[b];
  L = L < a.T ? a.T : (L > a.Lmax ? a.Lmax : L);
  const int ns = (L + a.split_keys - 1) / a.split_keys;        // splits that saw keys
  const size_t row0 = ((size_t)b * a.Hkv + kvh) * a.nsplit;    // split s: (row0 + s) * rows + j
  const size_t sstride = (size_t)rows * kDh;
  const float2* ml = reinterpret_cast<const float2*>(a.part_ml) + row0 * rows + j;   // + s * rows
  const float* po = a.part_o + (row0 * rows + j) * kDh + 2 * dp;                    // + s * sstride
  float2 mlv[kCombineUnroll], ov[kCombineUnroll];
#pragma unroll
  for (int u = 0; u < kCombineUnroll; ++u) {
    const int s = g + u * kCombineGroups;
    mlv[u] = make_float2(-INFINITY, 0.0f);
    ov[u] = make_float2(0.0f, 0.0f);
    if (s < ns) {
      mlv[u] = ml[(size_t)s * rows];
      ov[u] = *reinterpret_cast<const float2*>(po + (size_t)s * sstride);
    }
  }
  float mmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < kCombineUnroll; ++u) mmax = fmaxf(mmax, mlv[u].x);
  for (int s = g + kCombineUnroll * kCombineGroups; s < ns; s += kCombineGroups)
    mmax = fmaxf(mmax, ml[(size_t)s * rows].x);
  if (dp == 0) red[0][g] = mmax;     // equal across the group's lanes
  __syncthreads();
  // finite: split 0 holds position 0, visible to every row
  mmax = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float lsum = 0.0f;
  float2 o = make_float2(0.0f, 0.0f);
#pragma unroll
  for (int u = 0; u < kCombineUnroll; ++u) {
    const float w = exp2_hw(mlv[u].x - mmax);     // 0 for a split with no visible key (or none)
    lsum += w * mlv[u].y;
    o.x += w * ov[u].x;
    o.y += w * ov[u].y;
  }
  for (int s = g + kCombineUnroll * kCombineGroups; s < ns; s += kCombineGroups) {
    const float2 m2 = ml[(size_t)s * rows];
    const float2 v = *reinterpret_cast<const float2*>(po + (size_t)s * sstride);
    const float w = exp2_hw(m2.x - mmax);
    lsum += w * m2.y;
    o.x += w * v.x;
    o.y += w * v.y;
  }
  if (dp == 0) red[1][g] = lsum;
  if (g > 0) part[g - 1][dp] = o;
  __syncthreads();
  if (g != 0) return;
  const float l = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
#pragma unroll
  for (int u = 0; u < kCombineGroups - 1; ++u) {
    o.x += part[u][dp].x;
    o.y += part[u][dp].y;
  }
  uint16_t* dst = a.out + (((size_t)b * a.T + i) * a.Hq + h) * kDh + 2 * dp;
  *reinterpret_cast<uint32_t*>(dst) =
      (uint32_t)f32_to_bf16_rne(o.x / l) | ((uint32_t)f32_to_bf16_rne(o.y / l) << 16);
}

// Row-major V [B*Hkv][Lmax][128] into the blocked layout: one wave per
// block of 16 positions; lane (c, g) gathers its 32 values and writes its
// 64 contiguous bytes.
__global__ __launch_bounds__(kWave) void pack_v_kernel(const uint16_t* v, int Lmax, uint16_t* out) {
  const int blk = blockIdx.x;
  const size_t slab = (size_t)blockIdx.y * Lmax * kDh;
  const int lane = threadIdx.x, c = lane & 15, grp = lane >> 4;
  const uint16_t* src = v + slab + ((size_t)blk * kVBlk + 4 * grp) * kDh + c;
  uint32_t w[16];
#pragma unroll
  for (int db = 0; db < kDh / 16; ++db) {
    w[2 * db] = (uint32_t)src[0 * kDh + 16 * db] | ((uint32_t)src[1 * kDh + 16 * db] << 16);
    w[2 * db + 1] = (uint32_t)src[2 * kDh + 16 * db] | ((uint32_t)src[3 * kDh + 16 * db] << 16);
  }
  uint4* dst = reinterpret_cast<uint4*>(out + slab + (size_t)blk * kVBlk * kDh + (size_t)lane * 32);
#pragma unroll
  for (int u = 0; u < 4; ++u) dst[u] = make_uint4(w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]);
}

// Between the [q;k;v] linear and attention (Qwen3's attention block; the
// pages do not describe it): per-head RMSNorm of q and k over their 128 dims
// with bf16 gammas, rotate-half rotary embedding at position p = L_b - T + i
// (dim pairs (d, d+64) turned by p * base^(-d/64)), and the append of k and
// v to the cache at that position.  One wave per (token row, head); lane l
// holds dims l and l + 64, i.e. exactly one rotation pair.
struct RopeFreqs {
  float f[64];   // fp32(base^(-d/64)), computed on the host in double and rounded
};

__global__ __launch_bounds__(kWave) void qk_norm_rope_append_kernel(
    const uint16_t* qkv, int T, int Hq, int Hkv, const uint16_t* q_gamma,
    const uint16_t* k_gamma, float eps, RopeFreqs freqs, const int32_t* len, int Lmax,
    uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache) {
  const int row = blockIdx.x;          // b * T + i
  const int h = blockIdx.y;            // 0..Hq+2Hkv-1
  const int b = row / T, i = row % T;
  const int lane = threadIdx.x;
  const int heads = Hq + 2 * Hkv;
  int L = len[b];
  L = L < T ? T : (L > Lmax ? Lmax : L);
  const int pos = L - T + i;
  const uint16_t* x = qkv + ((size_t)row * heads + h) * kDh;
  float x1 = bf16_to_f32(x[lane]), x2 = bf16_to_f32(x[lane + 64]);
  if (h >= Hq + Hkv) {                 // v: appended as is, into the blocked layout
    const int kvh = h - Hq - Hkv;
    uint16_t* slab = v_cache + ((size_t)b * Hkv + kvh) * (size_t)Lmax * kDh;
    slab[v_blocked_index(pos, lane)] = x[lane];
    slab[v_blocked_index(pos, lane + 64)] = x[lane + 64];
    return;
  }
  float ss = x1 * x1 + x2 * x2;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  const float r = 1.0f / sqrtf(ss / 128.0f + eps);
  const uint16_t* g = h < Hq ? q_gamma : k_gamma;
  const float n1 = bf16_to_f32(f32_to_bf16_rne(bf16_to_f32(f32_to_bf16_rne(x1 * r)) * bf16_to_f32(g[lane])));
  const float n2 = bf16_to_f32(f32_to_bf16_rne(bf16_to_f32(f32_to_bf16_rne(x2 * r)) * bf16_to_f32(g[lane + 64])));
  // the angle is one fp32 product, as in fp32 inference
  float sn, cs;
  sincosf((float)pos * freqs.f[lane], &sn, &cs);
  const uint16_t o1 = f32_to_bf16_rne(n1 * cs - n2 * sn);
  const uint16_t o2 = f32_to_bf16_rne(n2 * cs + n1 * sn);
  uint16_t* dst;
  if (h < Hq) dst = q_out + ((size_t)row * Hq + h) * kDh;
  else dst = k_cache + (((size_t)b * Hkv + (h - Hq)) * Lmax + pos) * kDh;
  dst[lane] = o1;
  dst[lane + 64] = o2;
}

}  // namespace w8a8

namespace {

// Blocks per wave: enough that the grid holds about kTargetWaves waves,
// even (the kernel takes blocks in pairs), and a multiple of the burst the
// launch uses: 2 or 4 blocks when a wave has that few, else the largest
// burst its registers allow.  A split is the kAttnWaves waves of a
// workgroup.
struct AttnSplit {
  int nsplit, split_keys, burst;
};

AttnSplit attn_split(int64_t B, int64_t Hkv, int64_t Lmax, int qb) {
  using namespace w8a8;
  const int64_t blocks = (Lmax + kVBlk - 1) / kVBlk;
  int64_t bpw = (blocks * B * Hkv + kTargetWaves - 1) / kTargetWaves;
  bpw = std::max<int64_t>((bpw + 1) / 2 * 2, 2);
  int burst = 2;
  if (qb > 0 && bpw > 2) {   // qb = 0: the smallest split any launch uses (workspace size)
    burst = bpw <= 4 ? std::min(4, attn_max_burst(qb)) : attn_max_burst(qb);
    bpw = (bpw + burst - 1) / burst * burst;
  }
  const int64_t bps = bpw * kAttnWaves;
  const int64_t nsplit = (blocks + bps - 1) / bps;   // <= 131072 / 128
  return AttnSplit{(int)nsplit, (int)(bps * kVBlk), burst};
}

}  // namespace

size_t w8a8_attention_workspace_bytes_impl(int64_t B, int64_t Hkv, int64_t Lmax) {
  using namespace w8a8;
  const AttnSplit sp = attn_split(B, Hkv, Lmax, 0);
  const size_t rows = (size_t)B * Hkv * sp.nsplit * kAttnMaxRows;
  const size_t o = (rows * kDh * sizeof(float) + 255) & ~(size_t)255;
  return o + rows * 2 * sizeof(float);
}

hipError_t w8a8_launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const int32_t* lengths, int64_t B, int64_t T,
                                        int64_t Hq, int64_t Hkv, int64_t Lmax, uint16_t* out,
                                        void* workspace, hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  const int qb = (int)((T * (Hq / Hkv) + 15) / 16);
  const AttnSplit sp = attn_split(B, Hkv, Lmax, qb);
  const size_t ws_rows = (size_t)B * Hkv * attn_split(B, Hkv, Lmax, 0).nsplit * kAttnMaxRows;
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.len = lengths;
  a.B = (int)B; a.T = (int)T; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.Lmax = (int)Lmax;
  a.nsplit = sp.nsplit;
  a.split_keys = sp.split_keys;
  // the partial sums sit where the workspace size puts them (its split
  // count is an upper bound of this launch's)
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                       ((ws_rows * kDh * sizeof(float) + 255) & ~(size_t)255));
  a.out = out;
  const dim3 grid((unsigned)a.nsplit, (unsigned)Hkv, (unsigned)B);
  const dim3 block(kAttnWaves * kWave);
#define W8A8_ATTN_LAUNCH(QB, NB) hipLaunchKernelGGL((attn_split_kernel<QB, NB>), grid, block, 0, stream, a)
  if (qb == 1) {
    if (sp.burst == 2) W8A8_ATTN_LAUNCH(1, 2); else W8A8_ATTN_LAUNCH(1, attn_max_burst(1));
  } else if (qb == 2) {
    if (sp.burst == 2) W8A8_ATTN_LAUNCH(2, 2);
    else if (sp.burst == 4) W8A8_ATTN_LAUNCH(2, 4);
    else W8A8_ATTN_LAUNCH(2, attn_max_burst(2));
  } else if (qb == 3) {
    if (sp.burst == 2) W8A8_ATTN_LAUNCH(3, 2); else W8A8_ATTN_LAUNCH(3, attn_max_burst(3));
  } else {
    W8A8_ATTN_LAUNCH(4, attn_max_burst(4));
  }
#undef W8A8_ATTN_LAUNCH
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)T, (unsigned)Hq, (unsigned)B),
                     dim3(kCombineThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t w8a8_launch_pack_v_cache(const uint16_t* v, int64_t BH, int64_t Lmax, uint16_t* out,
                                    hipStream_t stream) {
  using namespace w8a8;
  if (BH == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_v_kernel, dim3((unsigned)(Lmax / kVBlk), (unsigned)BH), dim3(kWave), 0,
                     stream, v, (int)Lmax, out);
  return hipGetLastError();
}

hipError_t w8a8_launch_qk_norm_rope_append(const uint16_t* qkv, int64_t B, int64_t T, int64_t Hq,
                                           int64_t Hkv, const uint16_t* q_gamma,
                                           const uint16_t* k_gamma, float eps, float rope_base,
                                           const int32_t* lengths, int64_t Lmax, uint16_t* q_out,
                                           uint16_t* k_cache, uint16_t* v_cache,
                                           hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  RopeFreqs freqs;
  for (int d = 0; d < 64; ++d) freqs.f[d] = (float)std::pow((double)rope_base, -(double)d / 64.0);
  hipLaunchKernelGGL(qk_norm_rope_append_kernel, dim3((unsigned)(B * T), (unsigned)(Hq + 2 * Hkv)),
                     dim3(kWave), 0, stream, qkv, (int)T, (int)Hq, (int)Hkv, q_gamma, k_gamma, eps,
                     freqs, lengths, (int)Lmax, q_out, k_cache, v_cache);
  return hipGetLastError();
}
