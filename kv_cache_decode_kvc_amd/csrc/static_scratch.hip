// Library-owned scratch for the no-allocation entry point
// (kvc_append_decode_attn_noalloc): a file-scope device array, one copy per
// GPU, held until the process ends.  Its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that
// address is handed to kernels or host code: the array's name in host code
// is a host-side stand-in, not a device address.
//
// Layout (kvc_internal.h): three counter arrays of kStaticCounterWords
// int32 each (split tickets, per-sequence arrivals, per-unit arrivals), the
// persistent form's two scheduling counters, then the split partials (lse,
// outputs) from kStaticPartialOff.  Each call
// clears the counter words it will use before its main kernel (a small fill
// kernel, so the call stays capturable in a HIP graph); the partials are
// written before they are read.

#include <mutex>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up)

__global__ __launch_bounds__(256) void clear_counters_kernel(int32_t* tickets, int32_t* seq_arrivals,
                                                             int32_t* unit_arrivals, int32_t* sched,
                                                             int units, int B) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < units) {
    tickets[i] = 0;
    unit_arrivals[i] = 0;
  }
  if (i < B) seq_arrivals[i] = 0;
  if (i < 2) sched[i] = 0;
}

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = a;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

hipError_t launch_clear_static_counters(void* base, int units, int B, hipStream_t s) {
  int32_t* w = static_cast<int32_t*>(base);
  const int n = units > B ? units : B;
  hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     w, w + kStaticCounterWords, w + 2 * kStaticCounterWords,
                     w + kStaticSchedOff / sizeof(int32_t), units, B);
  return hipGetLastError();
}

}  // namespace kvc
