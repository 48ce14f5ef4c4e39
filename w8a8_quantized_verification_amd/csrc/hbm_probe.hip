// Streaming-read probe: the HBM read bandwidth this chip sustains for a
// plain stream of 16-byte loads, measured in the same process as the
// kernels it is compared with.
//
// The verify step's cost is the weight bytes it reads over the memory
// bandwidth (gist.science German summary, Technische Zusammenfassung §3
// item 4; Japanese summary, 技術的サマリー §2.3), so the useful ceiling for
// the weight-streaming GEMM is what a pure read of the same bytes achieves,
// beside the nominal 8 TB/s.
//
// Each thread XORs 16-byte non-temporal loads in a grid-stride walk: at any
// moment every wave reads inside one sliding window of the buffer, and one
// wave instruction covers 1 KiB of consecutive bytes.  Eight loads per
// thread are in flight before any is consumed.  Each workgroup writes one
// word (the fold of its lanes) so the loads cannot be dropped; those 8 KiB
// of writes are the probe's only stores.
#include "common.h"

#include <hip/hip_ext.h>

namespace w8a8 {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const v4i* __restrict__ buf,
                                                                  int64_t units,
                                                                  uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  v4i x = v4i{0, 0, 0, 0};
  for (; i + (kProbeUnroll - 1) * stride < units; i += kProbeUnroll * stride) {
    v4i v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) x ^= v[u];
  }
  for (; i < units; i += stride) x ^= __builtin_nontemporal_load(buf + i);
  uint32_t f = (uint32_t)(x[0] ^ x[1] ^ x[2] ^ x[3]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) f ^= (uint32_t)__shfl_xor((int)f, off, kWave);
  __shared__ uint32_t part[kProbeThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = f;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / kWave; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

}  // namespace w8a8

hipError_t w8a8_launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  using namespace w8a8;
  const int64_t units = (int64_t)(bytes / 16);
  const dim3 grid((unsigned)blocks), block(kProbeThreads);
  if (ev0)
    hipExtLaunchKernelGGL(hbm_read_kernel, grid, block, 0, stream, ev0, ev1, 0,
                          reinterpret_cast<const v4i*>(buf), units, sink);
  else
    hipLaunchKernelGGL(hbm_read_kernel, grid, block, 0, stream,
                       reinterpret_cast<const v4i*>(buf), units, sink);
  return hipGetLastError();
}
