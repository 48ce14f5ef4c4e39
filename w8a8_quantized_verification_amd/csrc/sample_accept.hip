// Stochastic verification at temperature T > 0 (gfx950): speculative
// sampling of single-token drafts on the fp32 dequantized logits.
//
// The pages: the dequantized logits are high precision before softmax and
// the rejection-sampling test, which keeps the lossless guarantee of
// speculative decoding (gist.science German summary, Technische
// Zusammenfassung §2 "De-Quantisierung"; Italian summary, Sommario tecnico
// §2 item 3; French summary §2 "Échantillonnage de rejet"; Japanese summary
// §2.2 item 4), from T = 0 to T = 1 (German §3; Japanese §4).
//
// Per sequence b with drafts d[0..G-1] and rows r_i = b*(G+1)+i:
//   p_i = softmax(y[r_i] / T); accept d_i with probability p_i(d_i), in order,
//   stopping at the first rejection (n accepted); the next token is drawn
//   from p_n with d_n removed (rejection) or from p_G (all accepted).
// Every decision is exact and order-free:
//   x_j = max(fp32(fp32(y_j - m) * inv_t), -32), m = row max, inv_t = fp32(1/T)
//   w_j = exp_f32(x_j)        (fixed fp32 steps, below)
//   W_j = floor(w_j * 2^40)   (uint64; sums are exact in any order)
//   accept iff u_accept * Z < W(d) * 2^32        (Z = sum_j W_j)
//   token = first j with S_j > floor(u_sample * Z' / 2^64)  (inverse CDF)
//
// Three kernels, all bound by reading the logits (4 bytes per element):
//   1. chunk maxima      grid R*C, one 2048-element chunk per workgroup;
//   2. chunk weight sums grid R*C: row max from the chunk maxima, then the
//      chunk's sum of W (and the row max, stored by chunk 0);
//   3. accept + sample   one workgroup per sequence: the sequential
//      acceptance over the rows' totals, then the chunk holding the target
//      (block scan over chunk sums) and the element inside it (block scan).
#include "common.h"

#include <climits>

namespace w8a8 {

constexpr int kSThreads = 256;
constexpr int kSPerThread = 8;
constexpr int kSChunk = kSThreads * kSPerThread;   // logits per chunk
constexpr int kSWaves = kSThreads / kWave;

// e^x for x in [-32, 0], every step one IEEE fp32 operation (the file is
// built without floating-point contraction):
//   k = rint(x * log2(e)); r = (x - k*ln2_hi) - k*ln2_lo   (Cody-Waite)
//   p = Horner over the Taylor coefficients 1/7!, ..., 1/2!, 1, 1 at r
//   e^x = p * 2^k
__device__ __forceinline__ float exp_f32(float x) {
  const float log2e = __uint_as_float(0x3fb8aa3bu);
  const float ln2_hi = __uint_as_float(0x3f317200u);   // 15 significant bits
  const float ln2_lo = __uint_as_float(0x35bfbe8eu);
  const float k = rintf(x * log2e);
  const float r = (x - k * ln2_hi) - k * ln2_lo;
  float p = __uint_as_float(0x39500d01u);              // 1/7!
  p = p * r + __uint_as_float(0x3ab60b61u);            // 1/6!
  p = p * r + __uint_as_float(0x3c088889u);            // 1/5!
  p = p * r + __uint_as_float(0x3d2aaaabu);            // 1/4!
  p = p * r + __uint_as_float(0x3e2aaaabu);            // 1/3!
  p = p * r + __uint_as_float(0x3f000000u);            // 1/2!
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  return ldexpf(p, (int)k);
}

// Fixed-point softmax numerator of one logit.
__device__ __forceinline__ unsigned long long fixed_weight(float y, float m, float inv_t) {
  float x = (y - m) * inv_t;
  x = x < -32.0f ? -32.0f : x;
  const float w = exp_f32(x);
  return (unsigned long long)ldexpf(w, 40);   // exact: an integer-valued float
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

struct SampleArgs {
  const float* logits;      // [R][V]
  int64_t V;
  int R, C;                 // rows, chunks per row
  float inv_t;
  float* chunk_max;         // [R][C]
  unsigned long long* chunk_sum;  // [R][C]
  float* row_max;           // [R]
  unsigned long long* weights;    // [R][V] output of the weights-only entry, or null
};

__global__ __launch_bounds__(kSThreads) void sample_chunk_max_kernel(SampleArgs a) {
  const int c = blockIdx.x % a.C;
  const int r = blockIdx.x / a.C;
  const float* row = a.logits + (size_t)r * (size_t)a.V;
  const int64_t base = (int64_t)c * kSChunk;
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kSPerThread; ++k) {
    const int64_t j = base + k * kSThreads + threadIdx.x;
    if (j < a.V) m = fmaxf(m, row[j]);
  }
  m = wave_max(m);
  __shared__ float part[kSWaves];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = part[0];
#pragma unroll
    for (int w = 1; w < kSWaves; ++w) v = fmaxf(v, part[w]);
    a.chunk_max[(size_t)r * a.C + c] = v;
  }
}

__device__ __forceinline__ float block_row_max(const SampleArgs& a, int r) {
  float m = -INFINITY;
  for (int c = threadIdx.x; c < a.C; c += kSThreads) m = fmaxf(m, a.chunk_max[(size_t)r * a.C + c]);
  m = wave_max(m);
  __shared__ float part[kSWaves];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = m;
  __syncthreads();
  float v = part[0];
#pragma unroll
  for (int w = 1; w < kSWaves; ++w) v = fmaxf(v, part[w]);
  return v;
}

__global__ __launch_bounds__(kSThreads) void sample_chunk_sum_kernel(SampleArgs a) {
  const int c = blockIdx.x % a.C;
  const int r = blockIdx.x / a.C;
  const float m = block_row_max(a, r);
  const float* row = a.logits + (size_t)r * (size_t)a.V;
  const int64_t base = (int64_t)c * kSChunk;
  unsigned long long s = 0;
#pragma unroll
  for (int k = 0; k < kSPerThread; ++k) {
    const int64_t j = base + k * kSThreads + threadIdx.x;
    if (j < a.V) {
      const unsigned long long w = fixed_weight(row[j], m, a.inv_t);
      s += w;
      if (a.weights) a.weights[(size_t)r * (size_t)a.V + j] = w;
    }
  }
  s = wave_sum_u64(s);
  __shared__ unsigned long long part[kSWaves];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long v = 0;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) v += part[w];
    if (a.chunk_sum) a.chunk_sum[(size_t)r * a.C + c] = v;
    if (c == 0 && a.row_max) a.row_max[r] = m;
  }
}

// Inclusive scan of one uint64 per thread over the block (Hillis-Steele in
// LDS).  Every thread must call it.
__device__ __forceinline__ unsigned long long block_inclusive_scan(unsigned long long v,
                                                                  unsigned long long* buf) {
  buf[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < kSThreads; off <<= 1) {
    const unsigned long long add = threadIdx.x >= (unsigned)off ? buf[threadIdx.x - off] : 0ull;
    __syncthreads();
    buf[threadIdx.x] += add;
    __syncthreads();
  }
  return buf[threadIdx.x];
}

struct AcceptArgs {
  SampleArgs s;
  const int32_t* draft;          // [B][G]
  const uint32_t* u_accept;      // [B][G]
  const unsigned long long* u_sample;  // [B]
  int G;
  int32_t* accept_len;
  int32_t* next_token;
};

__global__ __launch_bounds__(kSThreads) void sample_accept_kernel(AcceptArgs a) {
  const int b = blockIdx.x;
  const SampleArgs& s = a.s;
  const int G = a.G;
  const int64_t V = s.V;
  __shared__ unsigned long long part[kSWaves];
  __shared__ unsigned long long scan_buf[kSThreads];
  __shared__ int s_n, s_found;
  __shared__ unsigned long long s_z;

  // 1. acceptance, position by position
  int n = 0;
  unsigned long long z = 0;
  for (;; ++n) {
    const int r = b * (G + 1) + n;
    unsigned long long t = 0;
    for (int c = threadIdx.x; c < s.C; c += kSThreads) t += s.chunk_sum[(size_t)r * s.C + c];
    t = wave_sum_u64(t);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long zz = 0;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) zz += part[w];
      s_z = zz;
      int next = n;
      if (n < G) {
        const int d = a.draft[(size_t)b * G + n];
        const unsigned long long wd =
            (d >= 0 && d < V) ? fixed_weight(s.logits[(size_t)r * V + d], s.row_max[r], s.inv_t) : 0ull;
        // u * Z < W(d) * 2^32, compared exactly in 96 bits
        const unsigned long long u = a.u_accept[(size_t)b * G + n];
        const unsigned long long lo = u * zz;
        const unsigned long long hi = __umul64hi(u, zz);
        const unsigned long long rhs_hi = wd >> 32, rhs_lo = wd << 32;
        const bool acc = hi < rhs_hi || (hi == rhs_hi && lo < rhs_lo);
        if (acc) next = n + 1;
      }
      s_n = next;
    }
    __syncthreads();
    z = s_z;
    const int next = s_n;
    __syncthreads();
    if (next == n) break;     // rejected at n, or n == G
  }

  // 2. the row to sample and its excluded token
  const int r = b * (G + 1) + n;
  const float m = s.row_max[r];
  int excl = -1;
  unsigned long long w_excl = 0;
  if (n < G) {
    const int d = a.draft[(size_t)b * G + n];
    if (d >= 0 && d < V) {
      excl = d;
      w_excl = fixed_weight(s.logits[(size_t)r * V + d], m, s.inv_t);
    }
  }
  const unsigned long long zr = z - w_excl;                  // > 0 (see header)
  const unsigned long long target = __umul64hi(a.u_sample[b], zr);   // floor(u * Z' / 2^64)
  const int excl_chunk = excl >= 0 ? excl / kSChunk : -1;

  // 3. the chunk whose inclusive prefix first exceeds the target
  unsigned long long carry = 0;
  int chunk = -1;
  unsigned long long chunk_base = 0;
  for (int c0 = 0; c0 < s.C && chunk < 0; c0 += kSThreads) {
    const int c = c0 + threadIdx.x;
    unsigned long long v = 0;
    if (c < s.C) {
      v = s.chunk_sum[(size_t)r * s.C + c];
      if (c == excl_chunk) v -= w_excl;
    }
    const unsigned long long inc = block_inclusive_scan(v, scan_buf) + carry;
    if (threadIdx.x == 0) s_found = INT_MAX;
    __syncthreads();
    if (c < s.C && inc > target) atomicMin(&s_found, c);
    __syncthreads();
    const int f = s_found;
    if (f != INT_MAX) {
      chunk = f;
      // exclusive prefix of the found chunk
      chunk_base = scan_buf[f - c0] + carry;
      const unsigned long long fv = s.chunk_sum[(size_t)r * s.C + f] - (f == excl_chunk ? w_excl : 0ull);
      chunk_base -= fv;
    }
    carry += scan_buf[kSThreads - 1];
    __syncthreads();
  }

  // (a chunk is always found: the chunk totals add up to Z' > target; the
  // guard keeps every read in bounds regardless)
  if (chunk < 0) {
    if (threadIdx.x == 0) {
      a.accept_len[b] = n;
      a.next_token[b] = -1;
    }
    return;
  }

  // 4. the element inside that chunk: thread t owns elements 8t .. 8t+7
  const float* row = s.logits + (size_t)r * (size_t)V;
  const int64_t e0 = (int64_t)chunk * kSChunk + (int64_t)threadIdx.x * kSPerThread;
  unsigned long long w[kSPerThread];
  unsigned long long tot = 0;
#pragma unroll
  for (int k = 0; k < kSPerThread; ++k) {
    const int64_t j = e0 + k;
    w[k] = (j < V && j != excl) ? fixed_weight(row[j], m, s.inv_t) : 0ull;
    tot += w[k];
  }
  const unsigned long long inc = block_inclusive_scan(tot, scan_buf);
  if (threadIdx.x == 0) s_found = INT_MAX;
  __syncthreads();
  unsigned long long acc = chunk_base + inc - tot;   // exclusive prefix before element e0
#pragma unroll
  for (int k = 0; k < kSPerThread; ++k) {
    acc += w[k];
    if (acc > target) {
      atomicMin(&s_found, (int)(e0 + k));
      break;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.accept_len[b] = n;
    a.next_token[b] = s_found;
  }
}

}  // namespace w8a8

size_t w8a8_sample_workspace_bytes_impl(int64_t R, int64_t V) {
  using namespace w8a8;
  const int64_t C = (V + kSChunk - 1) / kSChunk;
  const size_t sums = (size_t)R * C * sizeof(unsigned long long);
  const size_t maxes = ((size_t)R * C * sizeof(float) + 255) & ~(size_t)255;
  const size_t rows = ((size_t)R * sizeof(float) + 255) & ~(size_t)255;
  return ((sums + 255) & ~(size_t)255) + maxes + rows;
}

static w8a8::SampleArgs sample_args(const float* logits, int64_t R, int64_t V, float inv_t,
                                    void* workspace) {
  using namespace w8a8;
  SampleArgs s{};
  s.logits = logits;
  s.V = V;
  s.R = (int)R;
  s.C = (int)((V + kSChunk - 1) / kSChunk);
  s.inv_t = inv_t;
  char* p = reinterpret_cast<char*>(workspace);
  const size_t sums = (((size_t)R * s.C * sizeof(unsigned long long)) + 255) & ~(size_t)255;
  const size_t maxes = ((size_t)R * s.C * sizeof(float) + 255) & ~(size_t)255;
  s.chunk_sum = reinterpret_cast<unsigned long long*>(p);
  s.chunk_max = reinterpret_cast<float*>(p + sums);
  s.row_max = reinterpret_cast<float*>(p + sums + maxes);
  return s;
}

hipError_t w8a8_launch_sample_weights(const float* logits, int64_t R, int64_t V, float inv_t,
                                      uint64_t* weights, void* workspace, hipStream_t stream) {
  using namespace w8a8;
  if (R == 0) return hipSuccess;
  SampleArgs s = sample_args(logits, R, V, inv_t, workspace);
  s.weights = reinterpret_cast<unsigned long long*>(weights);
  const dim3 grid((unsigned)(R * s.C));
  hipLaunchKernelGGL(sample_chunk_max_kernel, grid, dim3(kSThreads), 0, stream, s);
  hipLaunchKernelGGL(sample_chunk_sum_kernel, grid, dim3(kSThreads), 0, stream, s);
  return hipGetLastError();
}

hipError_t w8a8_launch_verify_sample(const float* logits, int64_t V, const int32_t* draft,
                                     int64_t B, int64_t G, float inv_t, const uint32_t* u_accept,
                                     const uint64_t* u_sample, int32_t* accept_len,
                                     int32_t* next_token, void* workspace, hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  const int64_t R = B * (G + 1);
  AcceptArgs a{};
  a.s = sample_args(logits, R, V, inv_t, workspace);
  a.draft = draft;
  a.u_accept = u_accept;
  a.u_sample = reinterpret_cast<const unsigned long long*>(u_sample);
  a.G = (int)G;
  a.accept_len = accept_len;
  a.next_token = next_token;
  const dim3 grid((unsigned)(R * a.s.C));
  hipLaunchKernelGGL(sample_chunk_max_kernel, grid, dim3(kSThreads), 0, stream, a.s);
  hipLaunchKernelGGL(sample_chunk_sum_kernel, grid, dim3(kSThreads), 0, stream, a.s);
  hipLaunchKernelGGL(sample_accept_kernel, dim3((unsigned)B), dim3(kSThreads), 0, stream, a);
  return hipGetLastError();
}
