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
// Pass 1 (one workgroup of 256 threads per (row, chunk)): each workgroup scans one chunk
// of one logits row with coalesced loads, keeps a per-thread (max, index),
// and reduces it over the wave with shuffles and over the 4 waves through
// LDS; ties keep the lower index.  Pass 2 (one wave per sequence): reduces
// the chunk results of the sequence's G+1 rows the same way, then finds the
// first draft position that differs from the target's argmax.
#include "common.h"

#include <climits>

namespace w8a8 {

constexpr int kArgThreads = 256;
constexpr int kArgChunk = 4096;  // logits per pass-1 workgroup

__device__ __forceinline__ void take(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__global__ __launch_bounds__(kArgThreads) void argmax_chunks_kernel(
    const float* __restrict__ logits, int V, int nchunks, float* __restrict__ pmax,
    int* __restrict__ pidx) {
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
    pmax[(size_t)row * nchunks + c] = bv;
    pidx[(size_t)row * nchunks + c] = bi;
  }
}

__global__ __launch_bounds__(kWave) void accept_kernel(
    const float* __restrict__ pmax, const int* __restrict__ pidx, int nchunks,
    const int32_t* __restrict__ draft, int G, int32_t* __restrict__ argmax,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ next_token) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  int n_acc = -1;   // first mismatch position, found in order
  int next = 0;
  for (int i = 0; i <= G; ++i) {
    const size_t row = (size_t)b * (G + 1) + i;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int c = lane; c < nchunks; c += kWave) take(bv, bi, pmax[row * nchunks + c], pidx[row * nchunks + c]);
    wave_argmax(bv, bi);
    const int a = (bi == INT_MAX) ? 0 : bi;  // only reachable for rows without a comparable value
    if (lane == 0 && argmax) argmax[row] = a;
    if (n_acc < 0) {
      const bool match = (i < G) && (draft[(size_t)b * G + i] == a);
      if (!match) { n_acc = i; next = a; }
    }
  }
  if (lane == 0) {
    accept_len[b] = n_acc;
    next_token[b] = next;
  }
}

static int argmax_chunks(int64_t V) { return (int)((V + kArgChunk - 1) / kArgChunk); }

}  // namespace w8a8

size_t w8a8_argmax_workspace_bytes(int64_t R, int64_t V) {
  using namespace w8a8;
  if (R <= 0 || V <= 0) return 0;
  const size_t n = (size_t)R * (size_t)argmax_chunks(V);
  const size_t fbytes = (n * sizeof(float) + 255) & ~(size_t)255;
  return fbytes + n * sizeof(int);
}

hipError_t w8a8_launch_verify_accept(const float* logits, int64_t V, const int32_t* draft,
                                     int64_t B, int64_t G, int32_t* argmax,
                                     int32_t* accept_len, int32_t* next_token,
                                     void* workspace, hipStream_t stream) {
  using namespace w8a8;
  if (B == 0) return hipSuccess;
  const int64_t R = B * (G + 1);
  const int nchunks = argmax_chunks(V);
  const size_t n = (size_t)R * (size_t)nchunks;
  float* pmax = reinterpret_cast<float*>(workspace);
  int* pidx = reinterpret_cast<int*>(reinterpret_cast<char*>(workspace) +
                                     ((n * sizeof(float) + 255) & ~(size_t)255));
  hipLaunchKernelGGL(argmax_chunks_kernel, dim3((unsigned)(R * nchunks)), dim3(kArgThreads),
                     0, stream, logits, (int)V, nchunks, pmax, pidx);
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)B), dim3(kWave), 0, stream, pmax, pidx,
                     nchunks, draft, (int)G, argmax, accept_len, next_token);
  return hipGetLastError();
}
