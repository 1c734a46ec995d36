// Causal prefill (un-absorbed form).  Not built yet: the entry point reports
// hipErrorNotSupported, which the C ABI maps to MLA_ERR_UNSUPPORTED.
#include "mla_common.h"

extern "C" hipError_t mla_launch_prefill(const uint16_t*, const uint16_t*, const uint16_t*,
                                         const int32_t*, const int32_t*, const uint16_t*,
                                         const uint16_t*, uint16_t*, void*, int, int, int, float,
                                         hipStream_t) {
  return hipErrorNotSupported;
}
