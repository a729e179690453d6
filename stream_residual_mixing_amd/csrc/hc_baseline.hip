// The unconstrained Hyper-Connections baseline and the gain diagnostic of the
// mHC notes, on the stream state layout of the mHC calls:
//   - HC's maps ([mHC] section 3 Preliminary, Eq. 5): each stream row of a token
//     is RMS-normalised over its C channels on its own, projected by theta
//     [n + 2, C] (pre, post, res_0 .. res_{n-1}) and mapped through
//     alpha * tanh(.) + b, unconstrained. The maps are applied with the mHC
//     pre-read and post kernels (hc_pre, hc_post): only the coefficients differ.
//   - the Amax gain ([mHC] section 3.1): the largest absolute row and column
//     sums of the composite residual map H_{L-1} ... H_0 of each token.
#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

namespace {

// stream rows per wave: theta is read from L2 once for that many rows
template <int NS>
constexpr int rows_per_wave() { return NS <= 8 ? 8 : 4; }

// Sum over the 64 lanes of a wave (a fixed butterfly, every lane gets the sum).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// One wave per RW consecutive stream rows (row = t * n + i). Each lane adds
// its channels' products with the n + 2 theta rows and the row's sum of
// squares; the wave sums them; lane r then forms row r's maps:
// x~ . theta_k = (x . theta_k) / r with r = sqrt(sum x^2 / C) (0 for a zero row).
template <typename T, int NS, bool VEC>
__global__ __launch_bounds__(256) void hc_tanh_kernel(const T* __restrict__ X, int64_t T_, int64_t C,
                                                      const float* __restrict__ theta,
                                                      const float* __restrict__ bias, float a_pre, float a_post,
                                                      float a_res, float* __restrict__ h_pre,
                                                      float* __restrict__ h_post, float* __restrict__ h_res) {
  constexpr int NK = NS + 2, HROWS = rows_per_wave<NS>();
  const int lane = threadIdx.x & 63;
  const int64_t nrows = T_ * NS;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * HROWS;
  if (r0 >= nrows) return;  // uniform over the wave; the kernel has no barrier
  int64_t rows[HROWS];
#pragma unroll
  for (int r = 0; r < HROWS; ++r) rows[r] = r0 + r < nrows ? r0 + r : nrows - 1;
  float acc[HROWS][NK + 1];
#pragma unroll
  for (int r = 0; r < HROWS; ++r)
#pragma unroll
    for (int k = 0; k <= NK; ++k) acc[r][k] = 0.f;
  if (VEC) {
    for (int64_t c0 = (int64_t)lane * 8; c0 < C; c0 += 512) {
      float x[HROWS][8];
#pragma unroll
      for (int r = 0; r < HROWS; ++r) load8_nt(X + rows[r] * C + c0, x[r]);
#pragma unroll
      for (int r = 0; r < HROWS; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][NK] += x[r][e] * x[r][e];
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        float th[8];
        load8(theta + (int64_t)k * C + c0, th);
#pragma unroll
        for (int r = 0; r < HROWS; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][k] += th[e] * x[r][e];
      }
    }
  } else {
    for (int64_t c = lane; c < C; c += 64) {
      float x[HROWS];
#pragma unroll
      for (int r = 0; r < HROWS; ++r) {
        x[r] = Elem<T>::ld(X + rows[r] * C + c);
        acc[r][NK] += x[r] * x[r];
      }
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        const float th = theta[(int64_t)k * C + c];
#pragma unroll
        for (int r = 0; r < HROWS; ++r) acc[r][k] += th * x[r];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < HROWS; ++r)
#pragma unroll
    for (int k = 0; k <= NK; ++k) acc[r][k] = wave_sum(acc[r][k]);
  if (lane >= HROWS || r0 + lane >= nrows) return;
  float v[NK + 1];
#pragma unroll
  for (int k = 0; k <= NK; ++k) {
    float s = acc[0][k];
#pragma unroll
    for (int r = 1; r < HROWS; ++r) s = lane == r ? acc[r][k] : s;
    v[k] = s;
  }
  const int64_t row = r0 + lane, t = row / NS;
  const int i = (int)(row - t * NS);
  const float rms = sqrtf(v[NK] / (float)C);
  const float invr = rms > 0.f ? 1.0f / rms : 0.f;
  h_pre[t * NS + i] = a_pre * tanhf(v[0] * invr) + bias[i];
  h_post[t * NS + i] = a_post * tanhf(v[1] * invr) + bias[NS + i];
#pragma unroll
  for (int j = 0; j < NS; ++j)
    h_res[(t * NS + j) * NS + i] = a_res * tanhf(v[2 + j] * invr) + bias[2 * NS + j * NS + i];
}

// One thread per token: M = H_{L-1} ... H_0 (n x n, float32), then the largest
// absolute row sum (forward gain) and column sum (backward gain).
template <int NS>
__global__ __launch_bounds__(256) void amax_gain_kernel(const float* __restrict__ H, int64_t L, int64_t T_,
                                                        float* __restrict__ fwd, float* __restrict__ bwd) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T_) return;
  float M[NS][NS];
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) M[i][j] = i == j ? 1.f : 0.f;
  for (int64_t l = 0; l < L; ++l) {
    const float* A = H + (l * T_ + t) * NS * NS;
    float R[NS][NS];
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < NS; ++k) s += A[i * NS + k] * M[k][j];
        R[i][j] = s;
      }
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int j = 0; j < NS; ++j) M[i][j] = R[i][j];
  }
  float gf = 0.f, gb = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    float rs = 0.f, cs = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      rs += M[i][j];
      cs += M[j][i];
    }
    gf = fmaxf(gf, fabsf(rs));
    gb = fmaxf(gb, fabsf(cs));
  }
  fwd[t] = gf;
  bwd[t] = gb;
}

template <typename T, int NS>
void tanh_dispatch_vec(bool vec, const void* X, int64_t T_, int64_t C, const float* theta, const float* bias,
                       float a_pre, float a_post, float a_res, float* h_pre, float* h_post, float* h_res,
                       hipStream_t st) {
  const int64_t waves = (T_ * NS + rows_per_wave<NS>() - 1) / rows_per_wave<NS>();
  const dim3 g((unsigned)((waves + 3) / 4)), b(256);
  if (vec)
    hipLaunchKernelGGL((hc_tanh_kernel<T, NS, true>), g, b, 0, st, (const T*)X, T_, C, theta, bias, a_pre, a_post,
                       a_res, h_pre, h_post, h_res);
  else
    hipLaunchKernelGGL((hc_tanh_kernel<T, NS, false>), g, b, 0, st, (const T*)X, T_, C, theta, bias, a_pre,
                       a_post, a_res, h_pre, h_post, h_res);
}

template <typename T>
void tanh_dispatch_n(int n, bool vec, const void* X, int64_t T_, int64_t C, const float* theta, const float* bias,
                     float a_pre, float a_post, float a_res, float* h_pre, float* h_post, float* h_res,
                     hipStream_t st) {
  switch (n) {
#define HC_TANH_CASE(NS) \
  case NS: tanh_dispatch_vec<T, NS>(vec, X, T_, C, theta, bias, a_pre, a_post, a_res, h_pre, h_post, h_res, st); break;
    HC_TANH_CASE(1) HC_TANH_CASE(2) HC_TANH_CASE(3) HC_TANH_CASE(4)
    HC_TANH_CASE(5) HC_TANH_CASE(6) HC_TANH_CASE(7) HC_TANH_CASE(8)
    HC_TANH_CASE(9) HC_TANH_CASE(10) HC_TANH_CASE(11) HC_TANH_CASE(12)
    HC_TANH_CASE(13) HC_TANH_CASE(14) HC_TANH_CASE(15) HC_TANH_CASE(16)
#undef HC_TANH_CASE
    default: break;
  }
}

}  // namespace

hipError_t launch_hc_tanh(int dtype, bool vec, const void* X, int64_t T_, int n, int64_t C, const float* theta,
                          const float* bias, float a_pre, float a_post, float a_res, float* h_pre, float* h_post,
                          float* h_res, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  if (dtype == 0)
    tanh_dispatch_n<float>(n, vec, X, T_, C, theta, bias, a_pre, a_post, a_res, h_pre, h_post, h_res, st);
  else
    tanh_dispatch_n<bf16_t>(n, vec, X, T_, C, theta, bias, a_pre, a_post, a_res, h_pre, h_post, h_res, st);
  return hipGetLastError();
}

hipError_t launch_amax_gain(const float* H, int64_t L, int64_t T_, int n, float* fwd, float* bwd, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  const dim3 g((unsigned)((T_ + 255) / 256)), b(256);
  switch (n) {
#define HC_GAIN_CASE(NS) \
  case NS: hipLaunchKernelGGL(amax_gain_kernel<NS>, g, b, 0, st, H, L, T_, fwd, bwd); break;
    HC_GAIN_CASE(1) HC_GAIN_CASE(2) HC_GAIN_CASE(3) HC_GAIN_CASE(4)
    HC_GAIN_CASE(5) HC_GAIN_CASE(6) HC_GAIN_CASE(7) HC_GAIN_CASE(8)
    HC_GAIN_CASE(9) HC_GAIN_CASE(10) HC_GAIN_CASE(11) HC_GAIN_CASE(12)
    HC_GAIN_CASE(13) HC_GAIN_CASE(14) HC_GAIN_CASE(15) HC_GAIN_CASE(16)
#undef HC_GAIN_CASE
    default: break;
  }
  return hipGetLastError();
}

}  // namespace hc
