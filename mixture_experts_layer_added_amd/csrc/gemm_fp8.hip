// FP8 E4M3 expert FFN (not built yet).
#include "common.h"

namespace moe {

hipError_t launch_fp8_ffn(const Dims&, const void*, const float*, const int32_t*, const int32_t*,
                          const void*, const float*, const void*, const float*, void*, void*,
                          float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
