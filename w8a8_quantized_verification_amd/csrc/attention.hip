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
// 256 cache positions and every query row that reads its kv head (T x
// Hq/Hkv rows, <= 64); 64-key tiles of K and V go through LDS, each wave
// keeps an online softmax (running max, sum, unnormalised output) for its
// rows, one key per lane for the scores and two output dimensions per lane
// for the value sum.  A second kernel merges the splits of each row.  Bound
// by reading the cache (2 * 128 * 2 bytes per position and kv head).
#include "common.h"

#include <cmath>

namespace w8a8 {

constexpr int kDh = 128;
constexpr int kAttnChunk = 256;     // cache positions per workgroup
constexpr int kAttnTile = 64;       // keys per LDS tile
constexpr int kAttnThreads = 256;
constexpr int kAttnMaxRows = 64;    // T * Hq / Hkv
constexpr int kKRow = kDh + 2;      // padded LDS row (bf16): row j starts at bank j

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

__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(AttnArgs a) {
  __shared__ uint32_t qs[kAttnMaxRows][kDh / 2];   // bf16 pairs
  __shared__ uint16_t ks[kAttnTile][kKRow];
  __shared__ uint16_t vs[kAttnTile][kKRow];
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

  // this wave's rows: r = wave + 4 * jr
  constexpr int kMaxR = kAttnMaxRows / (kAttnThreads / kWave);
  float m[kMaxR], l[kMaxR], o0[kMaxR], o1[kMaxR];
#pragma unroll
  for (int jr = 0; jr < kMaxR; ++jr) { m[jr] = -INFINITY; l[jr] = 0.0f; o0[jr] = 0.0f; o1[jr] = 0.0f; }

  const uint16_t* kb = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * kDh;
  const uint16_t* vb = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * kDh;
  for (int t0 = c0; t0 < c1; t0 += kAttnTile) {
    __syncthreads();   // previous tile's reads (and the q fill) done
    // 64 rows x 128 bf16 of K and V: 16 bytes per thread per pass
    for (int e = tid; e < kAttnTile * (kDh / 8); e += kAttnThreads) {
      const int j = e / (kDh / 8), d8 = (e % (kDh / 8)) * 8;
      uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
      if (t0 + j < c1) {
        kk = *reinterpret_cast<const uint4*>(kb + (size_t)(t0 + j) * kDh + d8);
        vv = *reinterpret_cast<const uint4*>(vb + (size_t)(t0 + j) * kDh + d8);
      }
      const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // padded rows are 4-byte aligned: store 32-bit pairs
        *reinterpret_cast<uint32_t*>(&ks[j][d8 + 2 * w]) = kw[w];
        *reinterpret_cast<uint32_t*>(&vs[j][d8 + 2 * w]) = vw[w];
      }
    }
    __syncthreads();
#pragma unroll
    for (int jr = 0; jr < kMaxR; ++jr) {
      const int r = wave + 4 * jr;
      if (r >= rows) break;
      const int i = r / group;
      const int last = L - a.T + i;                 // inclusive
      // score of key t0 + lane
      const int p = t0 + lane;
      float s = -INFINITY;
      if (p < c1 && p <= last) {
        float acc = 0.0f;
#pragma unroll 8
        for (int d = 0; d < kDh; d += 2) {
          const uint32_t kw = *reinterpret_cast<const uint32_t*>(&ks[lane][d]);
          const uint32_t qw = qs[r][d / 2];
          acc += __uint_as_float(qw << 16) * __uint_as_float(kw << 16);
          acc += __uint_as_float(qw & 0xffff0000u) * __uint_as_float(kw & 0xffff0000u);
        }
        s = acc * scale;
      }
      const float tmax = wave_max(s);
      const float mnew = fmaxf(m[jr], tmax);
      if (mnew == -INFINITY) continue;              // nothing visible yet
      const float alpha = expf(m[jr] - mnew);       // 0 when m was -inf
      const float pj = (s == -INFINITY) ? 0.0f : expf(s - mnew);
      float psum = pj;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off, kWave);
      l[jr] = l[jr] * alpha + psum;
      float a0 = o0[jr] * alpha, a1 = o1[jr] * alpha;
      for (int j = 0; j < kAttnTile; ++j) {
        const float pk = __shfl(pj, j, kWave);
        const uint32_t vw = *reinterpret_cast<const uint32_t*>(&vs[j][2 * lane]);
        a0 += pk * __uint_as_float(vw << 16);
        a1 += pk * __uint_as_float(vw & 0xffff0000u);
      }
      o0[jr] = a0; o1[jr] = a1;
      m[jr] = mnew;
    }
  }
  // partial results of this split
  const size_t base = (((size_t)b * a.Hkv + kvh) * a.nsplit + split) * kAttnMaxRows;
#pragma unroll
  for (int jr = 0; jr < kMaxR; ++jr) {
    const int r = wave + 4 * jr;
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
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int d = threadIdx.x;
  const int group = a.Hq / a.Hkv;
  const int kvh = h / group, r = i * group + h % group;
  float mmax = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) {
    const size_t idx = (((size_t)b * a.Hkv + kvh) * a.nsplit + s) * kAttnMaxRows + r;
    mmax = fmaxf(mmax, a.part_ml[idx * 2]);
  }
  float lsum = 0.0f, o = 0.0f;
  if (mmax != -INFINITY) {
    for (int s = 0; s < a.nsplit; ++s) {
      const size_t idx = (((size_t)b * a.Hkv + kvh) * a.nsplit + s) * kAttnMaxRows + r;
      const float ms = a.part_ml[idx * 2];
      if (ms == -INFINITY) continue;
      const float w = expf(ms - mmax);
      lsum += a.part_ml[idx * 2 + 1] * w;
      o += a.part_o[idx * kDh + d] * w;
    }
  }
  const float y = lsum > 0.0f ? o / lsum : 0.0f;
  a.out[(((size_t)b * a.T + i) * a.Hq + h) * kDh + d] = f32_to_bf16_rne(y);
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
  hipLaunchKernelGGL(attn_partial_kernel, dim3((unsigned)a.nsplit, (unsigned)Hkv, (unsigned)B),
                     dim3(kAttnThreads), 0, stream, a);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)T, (unsigned)Hq, (unsigned)B), dim3(kDh),
                     0, stream, a);
  return hipGetLastError();
}
