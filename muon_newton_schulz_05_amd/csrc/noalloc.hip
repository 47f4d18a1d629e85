// noalloc.hip -- the fixed device scratch of muon_step_noalloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid it) run a step in this
// file-scope array instead of a plan's workspace.  Each GPU the library runs
// on holds its own copy of the array until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address.  Its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and kept; host code uses
// only that address (kernel arguments, fills, copies).
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
char* g_scratch_ptr[kMaxDevices] = {};

// Zero n bytes (n a multiple of 16) with 16-byte vector stores: a kernel,
// not a memset, so that a caller's stream capture records only kernels.
__global__ __launch_bounds__(256) void k_fill_zero(u32x4_t* p, uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t scratch_address(int device, char** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != device) hipSetDevice(cur);
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

hipError_t launch_fill_zero(void* p, uint64_t bytes, hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  uint64_t blocks = (n16 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<u32x4_t*>(p), n16);
  return hipGetLastError();
}

}  // namespace muon
