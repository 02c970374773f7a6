// pa_noalloc.hip - the static device scratch of pa_decode_step_noalloc, for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that must not call hipMalloc). The entry point itself is in
// pa_api.cpp; its contract is in include/pagedattn.h.
//
// The array lives in the code object: every GPU the library runs on holds its
// own copy, at its own address, until the process ends. Host code never uses
// the array's name as an address (on the host it only stands for the symbol):
// the device address is looked up once per device, with that device current,
// by hipGetSymbolAddress, and kept; that address is what the kernels get.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"
#include "pagedattn.h"

namespace pa {
namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Clears n int32 words (the arrival counters at the start of the scratch). A
// kernel rather than hipMemsetAsync, so that a captured graph holds no memset
// node.
__global__ __launch_bounds__(256) void clear_words_kernel(int32_t *c, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) c[i] = 0;
}

}  // namespace

void *noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

hipError_t launch_clear_words(void *words, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_words_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<int32_t *>(words), n);
  return hipGetLastError();
}

}  // namespace pa
