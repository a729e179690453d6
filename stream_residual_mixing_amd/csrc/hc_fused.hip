// Fast paths for n = 4 bfloat16 streams (placeholder: not yet enabled).
#include "hc_device.h"
#include "hc_fast.h"

namespace hc {

int64_t fast_coeffs_packed_bytes(int, int64_t, int) { return 0; }
bool fast_coeffs_supported(int, int, int64_t, const void*) { return false; }
hipError_t launch_fast_coeffs_pre(const void*, int64_t, int64_t, const float*, const float*, float,
                                  float, float, int, float*, float*, float*, void*, void*,
                                  hipStream_t) {
  return hipErrorInvalidValue;
}
bool fast_post_supported(int, int, int64_t, const void*, const void*, const void*) { return false; }
hipError_t launch_fast_post(const void*, int64_t, int64_t, const float*, const float*, const void*,
                            void*, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace hc
