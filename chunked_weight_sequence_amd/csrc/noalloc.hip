// Device-resident scratch for ttt_chunk_scan_noalloc: the scan's workspace taken from a
// file-scope device array instead of a caller allocation, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// Each GPU the library runs on holds its own copy of `scratch` (TTT_SCAN_SCRATCH_BYTES) for the
// life of the process. In host code the array's name is only a host-side stand-in: its device
// address, different on every device, comes from hipGetSymbolAddress, called once per device
// with that device current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ttt_mi355x.h"
#include "launch.hpp"

namespace ttt {
namespace {

static __device__ __align__(256) unsigned char scratch[TTT_SCAN_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scan_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    void* p = nullptr;
    // the caller made `device` current; the symbol resolves to that device's copy
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[device] = p;
  }
  *ptr = g_ptr[device];
  return hipSuccess;
}

}  // namespace ttt
