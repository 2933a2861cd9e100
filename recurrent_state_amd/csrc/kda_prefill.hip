// Chunked (WY / UT-transform) prefill for gfx950.  Placeholder until the MFMA
// kernel lands: reports "not supported" so that no caller mistakes another
// kernel for it.

#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace kda {

hipError_t launch_prefill_chunked(const kda_shape&, int32_t, int32_t, float*, int64_t*, TokenInputs, float*, int32_t,
                                  const int32_t*, float*, int64_t*, int32_t, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kda
