// w8a8_lm_head_verify without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The LM-head argmax keys (64 sub-keys of 8 bytes, 256 bytes apart, per
// verified row: 16 KiB per row) live in `scratch`, a file-scope device array
// sized for W8A8_NOALLOC_MAX_ROWS rows (4.5 MiB).  Each GPU the library runs
// on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel: its device address is looked up once per device
// with hipGetSymbolAddress (with that device current) and kept in
// g_scratch[device].
//
// Every call first clears the sub-keys its rows use with a small fill kernel
// (no hipMemsetAsync: the call may be captured into a graph), then runs the
// same two kernels as w8a8_lm_head_verify; the acceptance kernel leaves the
// keys zero again.  All calls on one GPU share the array: calls that overlap
// in time on one GPU (two streams, two threads) race on it.
#include "../../include/w8a8.h"

#include <mutex>
#include <string>

#include "common.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kScratchWords =
    (size_t)W8A8_NOALLOC_MAX_ROWS * w8a8::kArgmaxSubkeys * w8a8::kArgmaxKeyStride;

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned long long scratch[kScratchWords];

namespace w8a8 {

// zero sub-key s of row m (word (m * subkeys + s) * stride) for m < rows
__global__ __launch_bounds__(256) void clear_keys_kernel(unsigned long long* keys, int rows) {
  const int n = rows * kArgmaxSubkeys;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    keys[(size_t)i * kArgmaxKeyStride] = 0ull;
}

}  // namespace w8a8

// The device address of this GPU's copy of `scratch` (looked up on the first
// call on each device, with that device current).
static hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t w8a8_launch_lm_head_verify_noalloc(const int8_t* xq, const float* x_scale,
                                              const int8_t* wq_tiled, const float* w_scale,
                                              int64_t V, int64_t K, const int32_t* draft,
                                              int64_t B, int64_t G, float* logits,
                                              int32_t* argmax, int32_t* accept_len,
                                              int32_t* next_token, hipStream_t stream) {
  using namespace w8a8;
  void* keys = nullptr;
  hipError_t e = scratch_address(&keys);
  if (e != hipSuccess) return e;
  const int rows = (int)(B * (G + 1));
  const int blocks = (rows * kArgmaxSubkeys + 255) / 256;
  hipLaunchKernelGGL(clear_keys_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<unsigned long long*>(keys), rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = w8a8_launch_lm_head_argmax(xq, x_scale, wq_tiled, w_scale, rows, V, K, logits, keys, stream);
  if (e != hipSuccess) return e;
  return w8a8_launch_accept_from_keys(keys, draft, B, G, argmax, accept_len, next_token, stream);
}
