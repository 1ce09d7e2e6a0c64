// Library-owned decode scratch, for callers that cannot allocate device
// memory during a call (code under graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The decode kernels keep their split partials (m, l, O) and the batch's unit
// offsets in a workspace.  kvc_attn_decode takes it from the caller;
// kvc_attn_decode_noalloc uses `scratch`, a fixed array in device memory that
// the code object itself carries, so nothing is allocated at call time.  Each
// device the library runs on holds its own copy of the array (kScratchBytes)
// from the moment the code object is loaded there until the process ends.
//
// In host code the name `scratch` is only a host-side stand-in for the
// symbol, never a device address.  Its device address is looked up once per
// device, with that device current, by hipGetSymbolAddress, and only that
// address is handed to kernels.
#include <mutex>

#include "kvfa_internal.h"

namespace kvfa {

namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** addr) {
  *addr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  return hipSuccess;
}

}  // namespace kvfa
