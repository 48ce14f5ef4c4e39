// LM-head argmax and greedy acceptance of the draft block, for gfx950.
//
// Pages: the target checks the whole drafted block in one pass, and the
// acceptance reads the dequantized logits kept in high precision
// (gist.science Japanese summary, 技術的サマリー §2.2 item 4; gist.science
// Italian summary, Sommario tecnico §2 "Campionamento di rifiuto"); correct
// drafts are accepted together and decoding restarts at the first wrong one
// (gist.science French summary, lay section "Le Double Chef"); results are
// for greedy decoding, T = 0 (Japanese summary §4).
//
// Pass 1 (one workgroup of 256 threads per (row, 4096-logit chunk)): each
// thread keeps a (max, index) over its strided elements, then the wave
// (shuffles) and the workgroup (LDS) reduce it; ties keep the lower index.
// Pass 2 (one workgroup of 16 waves per sequence): the partials of each of
// the sequence's G+1 rows are reduced by a group of waves with 8
// independent 8-byte loads in flight per lane, then thread 0 walks the
// draft to its first mismatch.
// The W8A8 LM-head kernel can instead fold each row's maximum into packed
// (value, index) sub-keys in its epilogue; accept_keys_kernel then only
// reads, combines and resets those.
#include "common.h"

#include <climits>

namespace w8a8 {

constexpr int kArgThreads = 256;
constexpr int kArgChunk = 4096;      // logits per pass-1 workgroup
constexpr int kAcceptWaves = 16;     // pass-2 workgroup: 1024 threads
constexpr int kMaxDraftRows = 256;   // G + 1 <= 256
constexpr int kAcceptUnroll = 8;

__device__ __forceinline__ void take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ void take(float& bv, int& bi, int2 p) {
  take(bv, bi, __int_as_float(p.x), p.y);
}

__global__ __launch_bounds__(kArgThreads) void argmax_chunks_kernel(
    const float* __restrict__ logits, int V, int nchunks, int2* __restrict__ parts) {
  const int64_t row = blockIdx.x / nchunks;
  const int c = blockIdx.x % nchunks;
  const float* lrow = logits + (size_t)row * (size_t)V;
  const int beg = c * kArgChunk;
  const int end = min(V, beg + kArgChunk);
  float bv = -INFINITY;
  int bi = INT_MAX;
  // 4 independent loads in flight per thread; each thread walks increasing
  // indices, so a strict '>' keeps its first maximum.
  int i = beg + threadIdx.x;
  for (; i + 3 * kArgThreads < end; i += 4 * kArgThreads) {
    const float v0 = lrow[i], v1 = lrow[i + kArgThreads];
    const float v2 = lrow[i + 2 * kArgThreads], v3 = lrow[i + 3 * kArgThreads];
    take(bv, bi, v0, i);
    take(bv, bi, v1, i + kArgThreads);
    take(bv, bi, v2, i + 2 * kArgThreads);
    take(bv, bi, v3, i + 3 * kArgThreads);
  }
  for (; i < end; i += kArgThreads) take(bv, bi, lrow[i], i);

  wave_argmax(bv, bi);
  __shared__ float sv[kArgThreads / kWave];
  __shared__ int si[kArgThreads / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgThreads / kWave; ++w) take(bv, bi, sv[w], si[w]);
    parts[(size_t)row * nchunks + c] = make_int2(__float_as_int(bv), bi);
  }
}

__global__ __launch_bounds__(kAcceptWaves * kWave) void accept_kernel(
    const int2* __restrict__ parts, int nparts, const int32_t* __restrict__ draft, int G,
    int32_t* __restrict__ argmax, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ next_token) {
  __shared__ float sv[kAcceptWaves];
  __shared__ int si[kAcceptWaves];
  __shared__ int row_arg[kMaxDraftRows];
  __shared__ int s_draft[kMaxDraftRows];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rows = G + 1;
  // the draft is read in parallel up front, so the walk below is LDS-only
  for (int i = threadIdx.x; i < G; i += blockDim.x) s_draft[i] = draft[(size_t)b * G + i];
  const int wpr = rows >= kAcceptWaves ? 1 : kAcceptWaves / rows;  // waves per row
  const int rows_per_pass = kAcceptWaves / wpr;
  const int sub = wave % wpr;
  for (int r0 = 0; r0 < rows; r0 += rows_per_pass) {
    const int i = r0 + wave / wpr;
    const bool live = (wave / wpr) < rows_per_pass && i < rows;
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (live) {
      const int2* p = parts + ((size_t)b * rows + i) * (size_t)nparts;
      const int stride = wpr * kWave;
      int c = sub * kWave + lane;
      for (; c + (kAcceptUnroll - 1) * stride < nparts; c += kAcceptUnroll * stride) {
        int2 v[kAcceptUnroll];
#pragma unroll
        for (int u = 0; u < kAcceptUnroll; ++u) v[u] = p[c + u * stride];
#pragma unroll
        for (int u = 0; u < kAcceptUnroll; ++u) take(bv, bi, v[u]);
      }
      for (; c < nparts; c += stride) take(bv, bi, p[c]);
    }
    wave_argmax(bv, bi);
    if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
    __syncthreads();
    if (live && sub == 0 && lane == 0) {
      for (int w = 1; w < wpr; ++w) take(bv, bi, sv[wave + w], si[wave + w]);
      const int a = (bi == INT_MAX) ? 0 : bi;  // only for rows without a comparable value
      row_arg[i] = a;
      if (argmax) argmax[(size_t)b * rows + i] = a;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < G && s_draft[n] == row_arg[n]) ++n;
    accept_len[b] = n;
    next_token[b] = row_arg[n];
  }
}

// Acceptance from the LM-head kernel's fused argmax sub-keys: one workgroup
// of 4 waves per sequence; each wave takes one row at a time, lane s taking
// (and zeroing) sub-key s with an atomic exchange at the coherence point, a
// 64-bit wave maximum combining them; then thread 0 walks the draft.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

constexpr int kAcceptKeyWaves = 4;

__global__ __launch_bounds__(kAcceptKeyWaves * kWave) void accept_keys_kernel(
    unsigned long long* __restrict__ keys, int subkeys, int key_stride,
    const int32_t* __restrict__ draft, int G, int32_t* __restrict__ argmax,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ next_token) {
  __shared__ int row_arg[kMaxDraftRows];
  __shared__ int s_draft[kMaxDraftRows];
  const int b = blockIdx.x;
  const int rows = G + 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  // the draft is read in parallel with the key exchanges, so the walk below
  // is LDS-only (no chain of dependent global loads)
  for (int i = threadIdx.x; i < G; i += blockDim.x) s_draft[i] = draft[(size_t)b * G + i];
  // up to 8 rows' sub-key exchanges per wave are issued before any is reduced
  unsigned long long k[8];
  for (int i0 = wave; i0 < rows; i0 += 8 * kAcceptKeyWaves) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kAcceptKeyWaves;
      k[u] = 0;
      if (i < rows && lane < subkeys) {
        const size_t sub = ((size_t)b * rows + i) * subkeys + lane;
        k[u] = __hip_atomic_exchange(&keys[sub * key_stride], 0ull, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kAcceptKeyWaves;
      const unsigned long long key = wave_max_u64(k[u]);
      if (i < rows && lane == 0) {
        const int a = key ? (int)(~(uint32_t)(key & 0xffffffffull)) : 0;
        row_arg[i] = a;
        if (argmax) argmax[(size_t)b * rows + i] = a;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < G && s_draft[n] == row_arg[n]) ++n;
    accept_len[b] = n;
    next_token[b] = row_arg[n];
  }
}

static int argmax_chunks(int64_t V) { return (int)((V + kArgChunk - 1) / kArgChunk); }

}  // namespace w8a8

size_t w8a8_argmax_workspace_bytes(int64_t R, int64_t V) {
  using namespace w8a8;
  if (R <= 0 || V <= 0) return 0;
  return (size_t)R * (size_t)argmax_chunks(V) * sizeof(int2);
}

hipError_t w8a8_launch_accept(const void* parts, int nparts, const int32_t* draft, int64_t B,
                              int64_t G, int32_t* argmax, int32_t* accept_len,
                              int32_t* next_token, hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)B), dim3(kAcceptWaves * kWave), 0, stream,
                     reinterpret_cast<const int2*>(parts), nparts, draft, (int)G, argmax,
                     accept_len, next_token);
  return hipGetLastError();
}

hipError_t w8a8_launch_accept_keys(unsigned long long* keys, int subkeys, int key_stride,
                                   const int32_t* draft, int64_t B, int64_t G, int32_t* argmax,
                                   int32_t* accept_len, int32_t* next_token, hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(accept_keys_kernel, dim3((unsigned)B), dim3(kAcceptKeyWaves * kWave), 0,
                     stream, keys, subkeys, key_stride, draft, (int)G, argmax, accept_len,
                     next_token);
  return hipGetLastError();
}

hipError_t w8a8_launch_verify_accept(const float* logits, int64_t V, const int32_t* draft,
                                     int64_t B, int64_t G, int32_t* argmax,
                                     int32_t* accept_len, int32_t* next_token,
                                     void* workspace, hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  const int64_t R = B * (G + 1);
  const int nchunks = argmax_chunks(V);
  int2* parts = reinterpret_cast<int2*>(workspace);
  hipLaunchKernelGGL(argmax_chunks_kernel, dim3((unsigned)(R * nchunks)), dim3(kArgThreads), 0,
                     stream, logits, (int)V, nchunks, parts);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return w8a8_launch_accept(parts, nchunks, draft, B, G, argmax, accept_len, next_token, stream);
}
