// Split-K workspace for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): a file-scope
// static device array that every GPU the library runs on holds until the process ends.
//
// In host code `scratch` is only a host-side stand-in for the array; its device address
// on the current GPU comes from hipGetSymbolAddress, once per device, and only that
// address is ever handed to kernels.  Layout as any awq_gemm workspace: the arrival
// counters first (cleared by a fill kernel at the first use on a device, and left zero
// by every completed call), then the fp32 partial sums.
#include <mutex>

#include "kernels.hpp"

namespace w4 {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(clear_words_kernel, dim3(kMaxCounters / 256), dim3(256), 0, stream, (uint32_t*)p,
                       kMaxCounters);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace w4
