// static_scratch.hip -- the scratch memory of skinny_mm_run_static, the run
// call for callers that cannot allocate device memory.
//
// The scratch is one file-scope device array of fixed size.  Every GPU the
// library runs on holds its own copy (at its own address) until the process
// ends.  In host code the array's name is only a host-side handle: the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current and kept per device; nothing else uses the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

static __device__ __align__(256) unsigned char scratch[skinny::kStaticScratchBytes];

namespace skinny {

namespace {

// the counter region must start at zero (every run leaves it at zero); a
// kernel rather than a memset, so a first call under stream capture records
// an ordinary kernel node
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

constexpr int kMaxDevices = 64;

std::mutex g_mutex;
char* g_base[kMaxDevices];  // device address of `scratch` per device, null until looked up

}  // namespace

hipError_t static_scratch(hipStream_t stream, char** base) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // the stream must belong to the current device, whose copy is used
  int sdev = dev;
  e = hipStreamGetDevice(stream, &sdev);
  if (e != hipSuccess) return e;
  if (sdev != dev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_base[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    const int64_t words = (int64_t)(kStaticCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       (uint32_t*)ptr, words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_base[dev] = (char*)ptr;
  }
  *base = g_base[dev];
  return hipSuccess;
}

}  // namespace skinny
