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
// Hq/Hkv rows, <= 64); the tile's K and V go through LDS and both products
// run on the bf16 MFMA (details at the kernel).  A second kernel merges the splits of each row.  Bound
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

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// The partial kernel on v_mfma_f32_16x16x32_bf16 (one 64-key tile per
// workgroup).  S = Q K^T: wave w takes the 16 keys of key block w against
// every 16-row query block (4 steps of 32 dims).  The row maxima and sums
// over the 64 keys meet in LDS; P = exp(S - m) goes to LDS as two bf16
// parts (hi = bf16(P), lo = bf16(P - hi)), each multiplied by V, which keeps
// the weights to ~16 significant bits.  O = P V: wave w takes
// dims 32w .. 32w+31 (2 dim blocks) against every query block (2 steps of
// 32 keys); each lane gathers its 8 keys' values of one dim from the
// row-major V tile (2-byte LDS reads).  LDS rows are padded so that the 16
// rows a wave reads at once fall in distinct banks.
constexpr int kQRow = kDh + 8;         // bf16 per padded Q / K row (272 bytes)
constexpr int kVtRow = kAttnTile + 8;  // bf16 per padded P row (144 bytes)

__global__ __launch_bounds__(kAttnThreads) void attn_partial_mfma_kernel(AttnArgs a) {
  // Q rows; after the scores, the same bytes hold the low parts of P
  __shared__ __attribute__((aligned(16))) uint16_t qs[kAttnMaxRows][kQRow];
  static_assert(sizeof(uint16_t) * kAttnMaxRows * kVtRow <= sizeof(qs), "P low parts fit");
  uint16_t(*ps_lo)[kVtRow] = reinterpret_cast<uint16_t(*)[kVtRow]>(&qs[0][0]);
  __shared__ __attribute__((aligned(16))) uint16_t ks[kAttnTile][kQRow];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kAttnTile][kQRow];
  __shared__ __attribute__((aligned(16))) uint16_t ps[kAttnMaxRows][kVtRow];
  __shared__ float red[kAttnThreads / kWave][kAttnMaxRows];
  __shared__ float rowm[kAttnMaxRows];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int group = a.Hq / a.Hkv;
  const int rows = a.T * group;
  const int rblocks = (rows + 15) / 16;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  int L = a.len[b];
  L = L < a.T ? a.T : (L > a.Lmax ? a.Lmax : L);
  const int t0 = split * kAttnTile;
  const int c1 = min(t0 + kAttnTile, L);
  const float scale = 0.08838834764831845f;   // 1/sqrt(128)
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);

  // Q rows (zero beyond `rows`), K rows, V transposed: every global load is
  // issued before the first LDS store
  constexpr int kQLoads = kAttnMaxRows * (kDh / 8) / kAttnThreads;
  constexpr int kLoads = kAttnTile * (kDh / 8) / kAttnThreads;
  const uint16_t* kb = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * kDh;
  const uint16_t* vb = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * kDh;
  uint4 qq[kQLoads], kk[kLoads], vv[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int e = tid + u * kAttnThreads;
    const int j = e / (kDh / 8), d8 = (e % (kDh / 8)) * 8;
    kk[u] = z4;
    vv[u] = z4;
    if (t0 + j < c1) {
      kk[u] = *reinterpret_cast<const uint4*>(kb + (size_t)(t0 + j) * kDh + d8);
      vv[u] = *reinterpret_cast<const uint4*>(vb + (size_t)(t0 + j) * kDh + d8);
    }
  }
#pragma unroll
  for (int u = 0; u < kQLoads; ++u) {
    const int e = tid + u * kAttnThreads;
    const int r = e / (kDh / 8), d8 = (e % (kDh / 8)) * 8;
    qq[u] = z4;
    if (r < rows) {
      const int i = r / group, h = kvh * group + r % group;
      qq[u] = *reinterpret_cast<const uint4*>(a.q + (((size_t)b * a.T + i) * a.Hq + h) * kDh + d8);
    }
  }
#pragma unroll
  for (int u = 0; u < kQLoads; ++u) {
    const int e = tid + u * kAttnThreads;
    const int r = e / (kDh / 8), d8 = (e % (kDh / 8)) * 8;
    if (r < rblocks * 16) *reinterpret_cast<uint4*>(&qs[r][d8]) = qq[u];
  }
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int e = tid + u * kAttnThreads;
    const int j = e / (kDh / 8), d8 = (e % (kDh / 8)) * 8;
    *reinterpret_cast<uint4*>(&ks[j][d8]) = kk[u];
    *reinterpret_cast<uint4*>(&vs[j][d8]) = vv[u];
  }
  __syncthreads();

  // S for key block `wave`: lane holds rows 16*qb + 4*grp + r, key 16*wave + col
  v4f sacc[kAttnMaxRows / 16];
#pragma unroll
  for (int qb = 0; qb < kAttnMaxRows / 16; ++qb) {
    sacc[qb] = v4f{0.f, 0.f, 0.f, 0.f};
    if (qb < rblocks) {
#pragma unroll
      for (int st = 0; st < kDh / 32; ++st) {
        const v4i qa = *reinterpret_cast<const v4i*>(&qs[qb * 16 + col][st * 32 + grp * 8]);
        const v4i kb4 = *reinterpret_cast<const v4i*>(&ks[wave * 16 + col][st * 32 + grp * 8]);
        sacc[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qa),
                                                            __builtin_bit_cast(v8bf, kb4),
                                                            sacc[qb], 0, 0, 0);
      }
    }
  }
  const int p = t0 + wave * 16 + col;
  // scale and mask; row maxima over this wave's 16 keys, then over the 4 waves
#pragma unroll
  for (int qb = 0; qb < kAttnMaxRows / 16; ++qb) {
    if (qb >= rblocks) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qr = qb * 16 + 4 * grp + r;
      const bool vis = qr < rows && p < c1 && p <= L - a.T + qr / group;
      float s = vis ? sacc[qb][r] * scale : -INFINITY;
      sacc[qb][r] = s;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) s = fmaxf(s, __shfl_xor(s, off, kWave));
      if (col == 0) red[wave][qr] = s;
    }
  }
  __syncthreads();
  // P = exp(S - m) as bf16 into LDS; partial row sums of the rounded values
#pragma unroll
  for (int qb = 0; qb < kAttnMaxRows / 16; ++qb) {
    if (qb >= rblocks) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qr = qb * 16 + 4 * grp + r;
      const float m = fmaxf(fmaxf(red[0][qr], red[1][qr]), fmaxf(red[2][qr], red[3][qr]));
      if (wave == 0 && col == 0) rowm[qr] = m;
      const float s = sacc[qb][r];
      // P as the sum of two bf16 values (hi + lo carries ~16 significant
      // bits), so that the product keeps the softmax weights at fp32-like
      // precision through the bf16 MFMA
      const float pf = (s == -INFINITY) ? 0.0f : expf(s - m);
      const uint16_t hi = f32_to_bf16_rne(pf);
      const uint16_t lo = f32_to_bf16_rne(pf - bf16_to_f32(hi));
      ps[qr][wave * 16 + col] = hi;
      ps_lo[qr][wave * 16 + col] = lo;
      sacc[qb][r] = pf;
    }
  }
  __syncthreads();   // all maxima read before red is reused; P complete
#pragma unroll
  for (int qb = 0; qb < kAttnMaxRows / 16; ++qb) {
    if (qb >= rblocks) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qr = qb * 16 + 4 * grp + r;
      float l = sacc[qb][r];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) l += __shfl_xor(l, off, kWave);
      if (col == 0) red[wave][qr] = l;
    }
  }

  // O = P V for dims 32*wave .. +31; lane holds rows 16*qb + 4*grp + r, dim 16*db + col
  const size_t base = (((size_t)b * a.Hkv + kvh) * a.nsplit + split) * kAttnMaxRows;
#pragma unroll
  for (int qb = 0; qb < kAttnMaxRows / 16; ++qb) {
    if (qb >= rblocks) break;
#pragma unroll
    for (int dbi = 0; dbi < 2; ++dbi) {
      const int db = wave * 2 + dbi;
      v4f o = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < kAttnTile / 32; ++st) {
        const v4i ph = *reinterpret_cast<const v4i*>(&ps[qb * 16 + col][st * 32 + grp * 8]);
        const v4i pl = *reinterpret_cast<const v4i*>(&ps_lo[qb * 16 + col][st * 32 + grp * 8]);
        // the B operand: dim 16*db + col of keys 32*st + 8*grp .. +7, gathered
        // from the row-major V tile
        uint32_t vw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = st * 32 + grp * 8 + 2 * q;
          vw[q] = (uint32_t)vs[j][db * 16 + col] | ((uint32_t)vs[j + 1][db * 16 + col] << 16);
        }
        const v4i vb4 = v4i{(int)vw[0], (int)vw[1], (int)vw[2], (int)vw[3]};
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ph),
                                                     __builtin_bit_cast(v8bf, vb4), o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, pl),
                                                     __builtin_bit_cast(v8bf, vb4), o, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qr = qb * 16 + 4 * grp + r;
        if (qr < rows) a.part_o[(base + qr) * kDh + db * 16 + col] = o[r];
      }
    }
  }
  __syncthreads();   // the partial sums in red and the maxima in rowm are complete
  if (tid < rows) {
    a.part_ml[(base + tid) * 2] = rowm[tid];
    a.part_ml[(base + tid) * 2 + 1] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
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
  for (; s + 32 <= a.nsplit; s += 32) {
    float po[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) po[u] = a.part_o[((row0 + s + u) * kAttnMaxRows + r) * kDh + d];
#pragma unroll
    for (int u = 0; u < 32; ++u) o += po[u] * wts[s + u];
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
  hipLaunchKernelGGL(attn_partial_mfma_kernel, grid, dim3(kAttnThreads), 0, stream, a);
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
