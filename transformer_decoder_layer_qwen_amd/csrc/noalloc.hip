// Device memory of the allocation-free decode entry point
// (qlayer_decode_noalloc): one file-scope device array, present on every GPU
// the library runs on from module load until the process ends, and a kernel
// that writes the RoPE frequency table into it (a kernel node, not a copy,
// so the call stays usable under stream capture).
//
// Host code never uses the array's name as a device address: the name is a
// host-side stand-in there. Each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address reaches kernels.
#include <mutex>

#include "../../include/qlayer.h"
#include "common.h"
#include "kernels.h"

static __device__ __align__(256) char scratch[QLAYER_NOALLOC_MAX_WORKSPACE];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // per-device address of `scratch`

struct RopeTable {
  double w[64];
};

__global__ __launch_bounds__(64) void fill_rope_kernel(const RopeTable t, int n, double* dst) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = t.w[i];
}

}  // namespace

hipError_t ql_noalloc_scratch(void** ptr) {
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
  *ptr = g_scratch[dev];
  return hipSuccess;
}

hipError_t ql_fill_rope_table(const double* w, int n, double* dst, hipStream_t s) {
  if (n < 0 || n > 64) return hipErrorInvalidValue;
  RopeTable t{};
  for (int i = 0; i < n; ++i) t.w[i] = w[i];
  hipLaunchKernelGGL(fill_rope_kernel, dim3(1), dim3(64), 0, s, t, n, dst);
  return hipGetLastError();
}
