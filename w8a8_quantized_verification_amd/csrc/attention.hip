// Attention of the verified block over the KV cache (gfx950): the softmax
// part of the verifier, kept in high precision after the dequant step
// (gist.science German summary, Technische Zusammenfassung §2
// "De-Quantisierung"; Italian summary §2 pipeline; Japanese summary §2.2
// item 3).  For each sequence b the T = G + 1 verified positions attend,
// causally, to the first L_b cache positions (the last T of them are the
// block's own keys): query i reads keys j <= L_b - T + i; grouped-query
// heads (query head h reads kv head h / (Hq / Hkv)); head dimension 128;
// fp32 arithmetic, bf16 output.
//
// Split over the keys (flash-decoding): workgroup (split, kv head, b) takes
// 64 cache positions and every query row that reads its kv head (T x
// Hq/Hkv rows, <= 64, a contiguous run of them per wave); the 64-key tile of
// K and V goes through LDS, and each wave keeps an online softmax (running max,
// sum, unnormalised output) for its rows, one key per lane for the scores
// and two output dimensions per lane for the value sum, all of its rows at
// once so that each LDS value feeds several independent accumulations.  A second kernel merges the splits of each row.  Bound
// by reading the cache (2 * 128 * 2 bytes per position and kv head).
#include "common.h"

#include <cmath>

namespace w8a8 {

constexpr int kDh = 128;
constexpr int kAttnChunk = 64;      // cache positions per workgroup (one LDS tile)
constexpr int kAttnTile = 64;       // keys per LDS tile
constexpr int kAttnThreads = 256;
constexpr int kAttnMaxRows = 64;    // T * Hq / Hkv
constexpr int kAttnMaxSplits = 2048; // cache positions up to 2048 * 64 = 131072

struct AttnArgs {
  const uint16_t* q;      // [B][T][Hq][128]
  const uint16_t* k;      // [B][Hkv][Lmax][128]
  const uint16_t* v;
  const int32_t* len;     // [B]
  int B, T, Hq, Hkv, Lmax, nsplit;
  float* part_o;          // [B][Hkv][nsplit][rows][128]
  float* part_ml;         // [B][Hkv][nsplit][rows][2]
  uint16_t* out;          // [B][T][Hq][128]
};

// RW: query rows per wave (rows r = wave * RW + jr); the rows of a wave are
// processed together so that every K or V value read from LDS feeds RW
// independent accumulations.
template <int RW>
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(AttnArgs a) {
  __shared__ uint32_t qs[kAttnMaxRows][kDh / 2];   // bf16 pairs
  // K rows as bf16 pairs with word w of row j stored at word w ^ j (a
  // lane-per-row read of one word is then conflict-free); V rows plain (a
  // row is read across the lanes)
  __shared__ uint32_t ks[kAttnTile][kDh / 2];
  __shared__ uint32_t vs[kAttnTile][kDh / 2];
  __shared__ float ps[kAttnThreads / kWave][RW][kAttnTile];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int group = a.Hq / a.Hkv;
  const int rows = a.T * group;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int L = a.len[b];
  L = L < a.T ? a.T : (L > a.Lmax ? a.Lmax : L);
  const int c0 = split * kAttnChunk;
  const int c1 = min(c0 + kAttnChunk, L);
  const float scale = 0.08838834764831845f;   // 1/sqrt(128)

  // query rows r = i * group + g (position i, head kvh * group + g), bf16 pairs in LDS
  for (int e = tid; e < rows * (kDh / 2); e += kAttnThreads) {
    const int r = e / (kDh / 2), d2 = e % (kDh / 2);
    const int i = r / group, h = kvh * group + r % group;
    qs[r][d2] = *reinterpret_cast<const uint32_t*>(
        a.q + (((size_t)b * a.T + i) * a.Hq + h) * kDh + 2 * d2);
  }

  const int r0 = wave * RW;
  float m[RW], l[RW], o0[RW], o1[RW];
#pragma unroll
  for (int jr = 0; jr < RW; ++jr) { m[jr] = -INFINITY; l[jr] = 0.0f; o0[jr] = 0.0f; o1[jr] = 0.0f; }

  const uint16_t* kb = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * kDh;
  const uint16_t* vb = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * kDh;
  for (int t0 = c0; t0 < c1; t0 += kAttnTile) {
    __syncthreads();   // previous tile's reads (and the q fill) done
    // 64 rows x 128 bf16 of K and V, 16 bytes per load: all loads first, then
    // the LDS stores (the loads of one tile are independent)
    constexpr int kLoads = kAttnTile * (kDh / 8) / kAttnThreads;
    uint4 kk[kLoads], vv[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = tid + u * kAttnThreads;
      const int j = e / (kDh / 8), d8 = (e % (kDh / 8)) * 8;
      kk[u] = make_uint4(0u, 0u, 0u, 0u);
      vv[u] = make_uint4(0u, 0u, 0u, 0u);
      if (t0 + j < c1) {
        kk[u] = *reinterpret_cast<const uint4*>(kb + (size_t)(t0 + j) * kDh + d8);
        vv[u] = *reinterpret_cast<const uint4*>(vb + (size_t)(t0 + j) * kDh + d8);
      }
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e = tid + u * kAttnThreads;
      const int j = e / (kDh / 8), w0 = (e % (kDh / 8)) * 4;
      const uint32_t kw[4] = {kk[u].x, kk[u].y, kk[u].z, kk[u].w};
      const uint32_t vw[4] = {vv[u].x, vv[u].y, vv[u].z, vv[u].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        ks[j][(w0 + w) ^ j] = kw[w];
        vs[j][w0 + w] = vw[w];
      }
    }
    __syncthreads();
    if (r0 >= rows) continue;      // (every wave still meets both barriers)

    // scores of key t0 + lane against the wave's rows
    float acc[RW];
#pragma unroll
    for (int jr = 0; jr < RW; ++jr) acc[jr] = 0.0f;
#pragma unroll 4
    for (int d2 = 0; d2 < kDh / 2; ++d2) {
      const uint32_t kw = ks[lane][d2 ^ lane];
      const float k0 = __uint_as_float(kw << 16), k1 = __uint_as_float(kw & 0xffff0000u);
#pragma unroll
      for (int jr = 0; jr < RW; ++jr) {
        const uint32_t qw = qs[r0 + jr < rows ? r0 + jr : 0][d2];
        acc[jr] += __uint_as_float(qw << 16) * k0;
        acc[jr] += __uint_as_float(qw & 0xffff0000u) * k1;
      }
    }
    const int p = t0 + lane;
    float alpha[RW];
#pragma unroll
    for (int jr = 0; jr < RW; ++jr) {
      const int last = L - a.T + (r0 + jr) / group;          // inclusive
      const bool vis = r0 + jr < rows && p < c1 && p <= last;
      const float s = vis ? acc[jr] * scale : -INFINITY;
      const float mnew = fmaxf(m[jr], wave_max(s));
      float pj = 0.0f;
      alpha[jr] = 1.0f;
      if (mnew != -INFINITY) {
        alpha[jr] = expf(m[jr] - mnew);                     // 0 when m was -inf
        pj = vis ? expf(s - mnew) : 0.0f;
        m[jr] = mnew;
      }
      float psum = pj;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off, kWave);
      l[jr] = l[jr] * alpha[jr] + psum;
      ps[wave][jr][lane] = pj;
    }
    // (the wave's own LDS rows: written and read by the same wave, in order)
    float a0[RW], a1[RW];
#pragma unroll
    for (int jr = 0; jr < RW; ++jr) { a0[jr] = o0[jr] * alpha[jr]; a1[jr] = o1[jr] * alpha[jr]; }
#pragma unroll 4
    for (int j = 0; j < kAttnTile; ++j) {
      const uint32_t vw = vs[j][lane];
      const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
#pragma unroll
      for (int jr = 0; jr < RW; ++jr) {
        const float pk = ps[wave][jr][j];
        a0[jr] += pk * v0;
        a1[jr] += pk * v1;
      }
    }
#pragma unroll
    for (int jr = 0; jr < RW; ++jr) { o0[jr] = a0[jr]; o1[jr] = a1[jr]; }
  }
  // partial results of this split
  const size_t base = (((size_t)b * a.Hkv + kvh) * a.nsplit + split) * kAttnMaxRows;
#pragma unroll
  for (int jr = 0; jr < RW; ++jr) {
    const int r = r0 + jr;
    if (r >= rows) break;
    float* po = a.part_o + (base + r) * kDh;
    po[2 * lane] = o0[jr];
    po[2 * lane + 1] = o1[jr];
    if (lane == 0) {
      a.part_ml[(base + r) * 2] = m[jr];
      a.part_ml[(base + r) * 2 + 1] = l[jr];
    }
  }
}

__global__ __launch_bounds__(kDh) void attn_combine_kernel(AttnArgs a) {
  __shared__ float wts[kAttnMaxSplits];
  __shared__ float red[kDh / kWave];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int d = threadIdx.x;
  const int group = a.Hq / a.Hkv;
  const int kvh = h / group, r = i * group + h % group;
  const size_t row0 = ((size_t)b * a.Hkv + kvh) * a.nsplit;   // split s: (row0 + s) * rows + r
  // each thread reads the (max, sum) of its splits; block max, then weights
  float ms[kAttnMaxSplits / kDh], lsn[kAttnMaxSplits / kDh];
  float mmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < kAttnMaxSplits / kDh; ++u) {
    const int s = d + u * kDh;
    ms[u] = -INFINITY;
    lsn[u] = 0.0f;
    if (s < a.nsplit) {
      const size_t idx = (row0 + s) * kAttnMaxRows + r;
      ms[u] = a.part_ml[idx * 2];
      lsn[u] = a.part_ml[idx * 2 + 1];
    }
    mmax = fmaxf(mmax, ms[u]);
  }
  mmax = wave_max(mmax);
  if ((d & (kWave - 1)) == 0) red[d / kWave] = mmax;
  __syncthreads();
  mmax = fmaxf(red[0], red[1]);
  float lpart = 0.0f;
#pragma unroll
  for (int u = 0; u < kAttnMaxSplits / kDh; ++u) {
    const int s = d + u * kDh;
    const float w = (ms[u] == -INFINITY) ? 0.0f : expf(ms[u] - mmax);
    if (s < a.nsplit) wts[s] = w;
    lpart += lsn[u] * w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lpart += __shfl_xor(lpart, off, kWave);
  __syncthreads();   // wts complete; red[] reused below
  if ((d & (kWave - 1)) == 0) red[d / kWave] = lpart;
  __syncthreads();
  const float lsum = red[0] + red[1];
  // (a split with no visible key has weight 0 and a zero partial output)
  float o = 0.0f;
  int s = 0;
  for (; s + 8 <= a.nsplit; s += 8) {
    float po[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) po[u] = a.part_o[((row0 + s + u) * kAttnMaxRows + r) * kDh + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) o += po[u] * wts[s + u];
  }
  for (; s < a.nsplit; ++s) o += a.part_o[((row0 + s) * kAttnMaxRows + r) * kDh + d] * wts[s];
  const float y = lsum > 0.0f ? o / lsum : 0.0f;
  a.out[(((size_t)b * a.T + i) * a.Hq + h) * kDh + d] = f32_to_bf16_rne(y);
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
  if (h >= Hq + Hkv) {                 // v: appended as is
    const int kvh = h - Hq - Hkv;
    uint16_t* dst = v_cache + (((size_t)b * Hkv + kvh) * Lmax + pos) * kDh;
    dst[lane] = x[lane];
    dst[lane + 64] = x[lane + 64];
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

size_t w8a8_attention_workspace_bytes_impl(int64_t B, int64_t Hkv, int64_t Lmax) {
  using namespace w8a8;
  const int64_t nsplit = (Lmax + kAttnChunk - 1) / kAttnChunk;
  const size_t rows = (size_t)B * Hkv * nsplit * kAttnMaxRows;
  const size_t o = (rows * kDh * sizeof(float) + 255) & ~(size_t)255;
  return o + rows * 2 * sizeof(float);
}

hipError_t w8a8_launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const int32_t* lengths, int64_t B, int64_t T,
                                        int64_t Hq, int64_t Hkv, int64_t Lmax, uint16_t* out,
                                        void* workspace, hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.len = lengths;
  a.B = (int)B; a.T = (int)T; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.Lmax = (int)Lmax;
  a.nsplit = (int)((Lmax + kAttnChunk - 1) / kAttnChunk);
  const size_t rows = (size_t)B * Hkv * a.nsplit * kAttnMaxRows;
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                       ((rows * kDh * sizeof(float) + 255) & ~(size_t)255));
  a.out = out;
  const dim3 grid((unsigned)a.nsplit, (unsigned)Hkv, (unsigned)B);
  const int rw = (int)((T * (Hq / Hkv) + 3) / 4);   // rows per wave, 4 waves
#define W8A8_ATT(RW) hipLaunchKernelGGL(attn_partial_kernel<RW>, grid, dim3(kAttnThreads), 0, stream, a)
  switch (rw) {
    case 1: W8A8_ATT(1); break;
    case 2: W8A8_ATT(2); break;
    case 3: W8A8_ATT(3); break;
    case 4: W8A8_ATT(4); break;
    case 5: W8A8_ATT(5); break;
    case 6: W8A8_ATT(6); break;
    case 7: case 8: W8A8_ATT(8); break;
    case 9: case 10: W8A8_ATT(10); break;
    case 11: case 12: W8A8_ATT(12); break;
    default: W8A8_ATT(16); break;
  }
#undef W8A8_ATT
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)T, (unsigned)Hq, (unsigned)B), dim3(kDh),
                     0, stream, a);
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
