// Specialised fast paths of libhc (internal). Each has a predicate saying
// whether it covers a call; otherwise the generic kernels run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

// Bytes of the packed phi used by the fused coefficient kernel (0 if unused).
int64_t fast_coeffs_packed_bytes(int n, int64_t C, int dtype);
bool fast_coeffs_supported(int dtype, int n, int64_t C, const void* X);
// Fused coefficients (+ pre-read when F_in != nullptr) for n = 4 bfloat16 streams.
hipError_t launch_fast_coeffs_pre(const void* X, int64_t T, int64_t C, const float* phi,
                                  const float* bias, float a_pre, float a_post, float a_res,
                                  int iters, float* h_pre, float* h_post, float* h_res, void* F_in,
                                  void* packed, hipStream_t st);

bool fast_post_supported(int dtype, int n, int64_t C, const void* X, const void* F, const void* Y);
hipError_t launch_fast_post(const void* X, int64_t T, int64_t C, const float* h_res,
                            const float* h_post, const void* F, void* Y, hipStream_t st);

}  // namespace hc
