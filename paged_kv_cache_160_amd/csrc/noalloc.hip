// Fixed device scratch for the decode call that allocates nothing
// (paged_attention_decode_append_noalloc): the partition states and counters
// that other decode calls keep in a caller's workspace live here instead, in
// one file-scope device array per GPU, held until the process ends.
//
// The array's host-side name is not a device address: its address on the
// current GPU comes from hipGetSymbolAddress, taken once per device and kept,
// and only that address is handed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace pkv {

static __device__ __align__(256) unsigned char scratch[PKV_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];    // scratch's device address on each GPU, once set up

__global__ void zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

int scratch_workspace(hipStream_t stream, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PKV_ERR_HIP;
    // The decode counters must start at zero (every call leaves them zero).
    // A fill kernel on the caller's stream, ahead of the call's own kernels,
    // rather than a memset, so that the first call may be captured in a graph.
    constexpr int kWords = PKV_WS_COUNTER_BYTES / 4;
    hipLaunchKernelGGL(zero_words, dim3((kWords + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       kWords);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PKV_OK;
}

}  // namespace pkv
