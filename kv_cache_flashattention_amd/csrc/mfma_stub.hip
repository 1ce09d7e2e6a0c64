// The matrix-core prefill kernel is not wired in yet: prefill takes the VALU path.
#include "kvfa_internal.h"

namespace kvfa {

hipError_t launch_prefill_mfma(const CacheView&, int, int, const void*, const void*, const void*,
                               void*, float, hipStream_t, bool* handled) {
  *handled = false;
  return hipSuccess;
}

}  // namespace kvfa
