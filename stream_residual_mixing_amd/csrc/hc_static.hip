// Static mHC ("mHC-SSM" abstract): one set of maps per layer, shared by every
// token. Pre- and post-mixing lie on the simplex (softmax of n logits), residual
// mixing is Sinkhorn-projected as in mHC ([mHC] Eq. 9). The apply kernels are
// the mHC pre-read and post/res write with coefficients that are the same for
// every thread, so they come through scalar loads.
#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

namespace {

// One workgroup of 256 threads. Thread e < n*n owns entry (e / n, e % n) of the
// residual map; every sum is taken by each thread over LDS in a fixed order.
__global__ __launch_bounds__(256) void static_maps_kernel(const float* __restrict__ z, int n, int iters,
                                                          float* __restrict__ h_pre, float* __restrict__ h_post,
                                                          float* __restrict__ h_res) {
  __shared__ float M[256];
  const int e = threadIdx.x, nn = n * n;
  const int i = e / n, j = e - (e / n) * n;
  if (e < 2) {  // softmax of the pre (e = 0) or post (e = 1) logits
    const float* l = z + e * n;
    float mx = l[0];
    for (int k = 1; k < n; ++k) mx = fmaxf(mx, l[k]);
    float s = 0.f;
    for (int k = 0; k < n; ++k) s += expf(l[k] - mx);
    float* out = e == 0 ? h_pre : h_post;
    for (int k = 0; k < n; ++k) out[k] = expf(l[k] - mx) / s;
  }
  // exp of the residual logits less their maximum (a common factor, removed by
  // the first normalisation)
  float mx = z[2 * n];
  for (int k = 1; k < nn; ++k) mx = fmaxf(mx, z[2 * n + k]);
  if (e < nn) M[e] = expf(z[2 * n + e] - mx);
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    float v = 0.f;
    if (e < nn) {
      float cs = 0.f;
      for (int r = 0; r < n; ++r) cs += M[r * n + j];
      v = M[e] / cs;
    }
    __syncthreads();
    if (e < nn) M[e] = v;
    __syncthreads();
    if (e < nn) {
      float rs = 0.f;
      for (int c = 0; c < n; ++c) rs += M[i * n + c];
      v = M[e] / rs;
    }
    __syncthreads();
    if (e < nn) M[e] = v;
    __syncthreads();
  }
  if (e < nn) h_res[e] = M[e];
}

// F_in[t, c] = sum_i h_pre[i] X[t, i, c]; one thread per (token, 8 channels), all
// NS rows in flight.
template <typename T, int NS, bool VEC>
__global__ __launch_bounds__(256) void static_pre_kernel(const T* __restrict__ X, int64_t T_, int64_t C,
                                                         const float* __restrict__ h_pre, T* __restrict__ F_in) {
  const int64_t nch = (C + 7) / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T_ * nch) return;
  const int64_t t = g / nch, c0 = (g - t * nch) * 8;
  const int cnt = (int)min((int64_t)8, C - c0);
  float x[NS][8];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const T* p = X + (t * NS + i) * C + c0;
    if (VEC) load8_nt(p, x[i]); else load8_tail(p, cnt, x[i]);
  }
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const float w = h_pre[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += w * x[i][e];
  }
  T* q = F_in + t * C + c0;
  if (VEC) store8_nt(q, o); else store8_tail(q, cnt, o);
}

// X_next[t, i] = sum_j h_res[i, j] X[t, j] + h_post[i] F_out[t]; all rows of a
// chunk are read before any is written, so X_next may equal X.
template <typename T, int NS, bool VEC>
__global__ __launch_bounds__(256) void static_post_kernel(const T* X, int64_t T_, int64_t C,
                                                          const float* __restrict__ h_res,
                                                          const float* __restrict__ h_post,
                                                          const T* __restrict__ F, T* Y) {
  const int64_t nch = (C + 7) / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T_ * nch) return;
  const int64_t t = g / nch, c0 = (g - t * nch) * 8;
  const int cnt = (int)min((int64_t)8, C - c0);
  float x[NS][8], f[8];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const T* p = X + (t * NS + j) * C + c0;
    if (VEC) load8_nt(p, x[j]); else load8_tail(p, cnt, x[j]);
  }
  if (VEC) load8_nt(F + t * C + c0, f); else load8_tail(F + t * C + c0, cnt, f);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    float y[8];
    const float wp = h_post[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = wp * f[e];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float w = h_res[i * NS + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] += w * x[j][e];
    }
    T* q = Y + (t * NS + i) * C + c0;
    if (VEC) store8_nt(q, y); else store8_tail(q, cnt, y);
  }
}

template <typename T, int NS>
void static_dispatch(bool post, bool vec, const void* X, int64_t T_, int64_t C, const float* h_pre_or_res,
                     const float* h_post, const void* F, void* Y, hipStream_t st) {
  const int64_t work = T_ * ((C + 7) / 8);
  const dim3 g((unsigned)((work + 255) / 256)), b(256);
  if (post) {
    if (vec)
      hipLaunchKernelGGL((static_post_kernel<T, NS, true>), g, b, 0, st, (const T*)X, T_, C, h_pre_or_res, h_post,
                         (const T*)F, (T*)Y);
    else
      hipLaunchKernelGGL((static_post_kernel<T, NS, false>), g, b, 0, st, (const T*)X, T_, C, h_pre_or_res, h_post,
                         (const T*)F, (T*)Y);
  } else {
    if (vec)
      hipLaunchKernelGGL((static_pre_kernel<T, NS, true>), g, b, 0, st, (const T*)X, T_, C, h_pre_or_res, (T*)Y);
    else
      hipLaunchKernelGGL((static_pre_kernel<T, NS, false>), g, b, 0, st, (const T*)X, T_, C, h_pre_or_res, (T*)Y);
  }
}

template <typename T>
void static_dispatch_n(int n, bool post, bool vec, const void* X, int64_t T_, int64_t C, const float* h1,
                       const float* h2, const void* F, void* Y, hipStream_t st) {
  switch (n) {
#define HC_STATIC_CASE(NS) \
  case NS: static_dispatch<T, NS>(post, vec, X, T_, C, h1, h2, F, Y, st); break;
    HC_STATIC_CASE(1) HC_STATIC_CASE(2) HC_STATIC_CASE(3) HC_STATIC_CASE(4)
    HC_STATIC_CASE(5) HC_STATIC_CASE(6) HC_STATIC_CASE(7) HC_STATIC_CASE(8)
    HC_STATIC_CASE(9) HC_STATIC_CASE(10) HC_STATIC_CASE(11) HC_STATIC_CASE(12)
    HC_STATIC_CASE(13) HC_STATIC_CASE(14) HC_STATIC_CASE(15) HC_STATIC_CASE(16)
#undef HC_STATIC_CASE
    default: break;
  }
}

}  // namespace

hipError_t launch_static_maps(const float* logits, int n, int iters, float* h_pre, float* h_post, float* h_res,
                              hipStream_t st) {
  hipLaunchKernelGGL(static_maps_kernel, dim3(1), dim3(256), 0, st, logits, n, iters, h_pre, h_post, h_res);
  return hipGetLastError();
}

hipError_t launch_static_apply(int dtype, bool post, bool vec, const void* X, int64_t T_, int n, int64_t C,
                               const float* h1, const float* h2, const void* F, void* Y, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  if (dtype == 0) static_dispatch_n<float>(n, post, vec, X, T_, C, h1, h2, F, Y, st);
  else static_dispatch_n<bf16_t>(n, post, vec, X, T_, C, h1, h2, F, Y, st);
  return hipGetLastError();
}

}  // namespace hc
