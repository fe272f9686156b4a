// Device scratch of loka_gemm_fp8_ln_noalloc: the forward's workspace (the
// tensor recipe's amax partials and a row-major weight rearranged into the
// fragment-interleaved layout) held in a fixed file-scope device array, so
// the entry point needs no allocation by the caller or the library.
//
// Every GPU the library runs on holds its own copy of the array until the
// process ends.  Its address on a device comes from hipGetSymbolAddress,
// looked up once per device on the first call made with that device
// current; host code uses only that address, never the array's name (which
// in host code is a stand-in, not a device address).  Calls on one GPU share
// its array: calls that overlap in time on one GPU race.  The kernels that
// use it write every byte they later read within the same call (each
// partials block writes its own entry; the rearrangement writes every
// packed byte including the zero padding), so nothing has to be cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/loka_fp8.h"
#include "launch.hpp"

namespace loka {
namespace {

constexpr size_t kScratchBytes = LOKA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

// The device address of the current device's array (looked up on first use).
// A non-null stream must belong to the current device.
hipError_t noalloc_scratch(hipStream_t s, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (s != nullptr) {
    hipDevice_t sd = -1;
    if ((e = hipStreamGetDevice(s, &sd)) != hipSuccess) return e;
    if (sd != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace loka
