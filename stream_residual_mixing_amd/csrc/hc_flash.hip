// xHC-Flash pieces on gfx950: a block of L consecutive sublayers that shares one
// routing decision and the block-entry state's full-state read.
//
// "xHC: Expanded Hyper-Connections" (paper summary, memory efficiency and the
// xHC-Flash variant; repository README, method and memory-efficiency table):
// routing shared across the block, the sublayers' pre maps
// formed from the block-entry state, residual mixing deferred to the block's
// last sublayer, and a light correction that rebuilds the later sublayers'
// inputs without reading the state again. Within the block the sublayers before
// the last only add H_post[:, j] F_out^(j) to the active rows, so sublayer l's
// dense read is F_pre^(l) + sum_{j<l} c_j F_out^(j) with the per-token scalars
// c_j = sum_a h_pre^(l)[idx_a] H_post[a, j].
//  * pre_multi_kernel: the L dense reads F_pre^(l) = sum_i h_pre^(l)_i X_0,i from
//    one pass over the entry state (bfloat16, N a multiple of 4 up to 16);
//  * flash_input_kernel: the correction, F_in^(l) from F_pre^(l) and F_out^(0..l-1);
//  * flash_post_maps_kernel: the block end as one mix of the entry state's
//    active rows, X_L,A = H_res X_0,A + sum_j E[:, j] F_out^(j), with E[:, j] =
//    H_res H_post[:, j] for j < L-1 and H_post[:, L-1] for the last sublayer.
#include "hc.h"
#include "hc_device.h"
#include "hc_launch.h"

namespace hc {
namespace {

__device__ __forceinline__ void unpack8f(const uint4& q, float v[8]) {
  v[0] = bf2f(q.x & 0xffffu); v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = bf2f(q.y & 0xffffu); v[3] = __uint_as_float(q.y & 0xffff0000u);
  v[4] = bf2f(q.z & 0xffffu); v[5] = __uint_as_float(q.z & 0xffff0000u);
  v[6] = bf2f(q.w & 0xffffu); v[7] = __uint_as_float(q.w & 0xffff0000u);
}

// F_pre[l, t, c] = sum_i h_pre[l, t, i] X[t, i, c], l < L, from one read of X: 8
// channels per thread, all NS stream rows in flight at once, the L outputs
// rounded once to bfloat16.
template <int NS, int L>
__global__ __launch_bounds__(256) void pre_multi_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t C,
                                                        const float* __restrict__ h_pre, uint16_t* __restrict__ F) {
  const int64_t nch = C / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  const uint16_t* p = X + t * NS * C + c0;
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  uint4 x[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p + i * C));
    x[i] = make_uint4(v.x, v.y, v.z, v.w);
  }
  float o[L][8];
#pragma unroll
  for (int l = 0; l < L; ++l)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[l][e] = 0.f;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    float xv[8];
    unpack8f(x[i], xv);
#pragma unroll
    for (int l = 0; l < L; ++l) {
      const float w = h_pre[((int64_t)l * T + t) * NS + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[l][e] += w * xv[e];
    }
  }
#pragma unroll
  for (int l = 0; l < L; ++l)
    __builtin_nontemporal_store(
        u4{pack_bf2_hw(o[l][0], o[l][1]), pack_bf2_hw(o[l][2], o[l][3]), pack_bf2_hw(o[l][4], o[l][5]),
           pack_bf2_hw(o[l][6], o[l][7])},
        reinterpret_cast<u4*>(F + ((int64_t)l * T + t) * C + c0));
}

// F_in[t, c] = F_pre_l[t, c] + sum_{j<l} c_j[t] F_outs[t, j, c], c_j[t] = sum_a
// h_pre_l[t, idx[t, a]] H_post[t, a, j] (H_post [T, k, L]). Workgroup (x, t)
// takes token t's channels [x * 256 V, (x + 1) * 256 V), V per thread (V = 8
// needs C % 8 == 0 and 16-byte aligned rows): the first l lanes form the
// token's c_j into LDS while every thread's row loads are in flight. Indices
// are clamped into [0, N). Workgroup (t, x): blockIdx.x = t, blockIdx.y = x.
constexpr int FI_THR = 256;
constexpr int FI_MAXL = 3;  // l < L <= HC_MAX_FLASH_SUBLAYERS
static_assert(HC_MAX_FLASH_SUBLAYERS - 1 <= FI_MAXL, "earlier outputs a corrected input can take");
template <typename TE, int V>
__global__ __launch_bounds__(FI_THR) void flash_input_kernel(int64_t T, int N, int64_t C, int k, int L, int l,
                                                             const TE* F_pre, const float* __restrict__ h_pre,
                                                             const int32_t* __restrict__ idx,
                                                             const float* __restrict__ H_post,
                                                             const TE* __restrict__ F_outs, TE* F_in) {  // F_in may be F_pre
  __shared__ float cs[FI_MAXL];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t c0 = ((int64_t)blockIdx.y * FI_THR + tid) * V;
  const bool ok = c0 < C;
  const int64_t cc = ok ? c0 : 0;
  float acc[V], f[FI_MAXL][V];
  if constexpr (V == 8) {
    load8(F_pre + t * C + cc, acc);
#pragma unroll
    for (int j = 0; j < FI_MAXL; ++j)
      if (j < l) load8(F_outs + (t * L + j) * C + cc, f[j]);
  } else {
    acc[0] = Elem<TE>::ld(F_pre + t * C + cc);
#pragma unroll
    for (int j = 0; j < FI_MAXL; ++j)
      if (j < l) f[j][0] = Elem<TE>::ld(F_outs + (t * L + j) * C + cc);
  }
  if (tid < l) {
    float cj = 0.f;
    for (int a = 0; a < k; ++a) {
      int s = idx[t * k + a];
      s = s < 0 ? 0 : (s >= N ? N - 1 : s);
      cj += h_pre[t * N + s] * H_post[(t * k + a) * L + tid];
    }
    cs[tid] = cj;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < FI_MAXL; ++j) {
    if (j < l) {
      const float cj = cs[j];
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += cj * f[j][e];
    }
  }
  if (ok) {
    TE* out = F_in + t * C + c0;
#pragma unroll
    for (int e = 0; e < V; ++e) Elem<TE>::st(out + e, acc[e]);
  }
}

// E[t, a, j] = sum_b H_res[t, a, b] H_post[t, b, j] for the components of the
// sublayers before the last (j < L - 1) and H_post[t, a, j] for the last
// sublayer's components (L - 1 <= j < Kb): one thread per (t, a, j).
__global__ __launch_bounds__(256) void flash_post_maps_kernel(int64_t T, int k, int L, int Kb,
                                                              const float* __restrict__ H_post,
                                                              const float* __restrict__ H_res, float* __restrict__ E) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T * k * Kb) return;
  const int64_t t = g / (k * Kb);
  const int r = (int)(g - t * k * Kb);
  const int a = r / Kb, j = r - a * Kb;
  float v;
  if (j >= L - 1) {
    v = H_post[(t * k + a) * Kb + j];
  } else {
    v = 0.f;
    for (int b = 0; b < k; ++b) v += H_res[(t * k + a) * k + b] * H_post[(t * k + b) * Kb + j];
  }
  E[g] = v;
}

}  // namespace

bool fast_pre_multi_supported(int dtype, int N, int64_t C, int L, const void* X, const void* F) {
  return dtype == 1 && N % 4 == 0 && N >= 4 && N <= 16 && L >= 1 && L <= 4 && C % 8 == 0 &&
         reinterpret_cast<uintptr_t>(X) % 16 == 0 && reinterpret_cast<uintptr_t>(F) % 16 == 0;
}

hipError_t launch_fast_pre_multi(const void* X, int64_t T, int N, int64_t C, int L, const float* h_pre, void* F,
                                 hipStream_t st) {
  const dim3 grid((unsigned)((T * (C / 8) + 255) / 256)), blk(256);
  const uint16_t* x = (const uint16_t*)X;
  uint16_t* f = (uint16_t*)F;
#define HC_PM(NS, LL) hipLaunchKernelGGL((pre_multi_kernel<NS, LL>), grid, blk, 0, st, x, T, C, h_pre, f)
#define HC_PM_L(NS)        \
  switch (L) {             \
    case 1: HC_PM(NS, 1); break; \
    case 2: HC_PM(NS, 2); break; \
    case 3: HC_PM(NS, 3); break; \
    default: HC_PM(NS, 4); break; \
  }
  switch (N) {
    case 4: HC_PM_L(4) break;
    case 8: HC_PM_L(8) break;
    case 12: HC_PM_L(12) break;
    default: HC_PM_L(16) break;
  }
#undef HC_PM_L
#undef HC_PM
  return hipGetLastError();
}

hipError_t launch_flash_input(int dtype, bool vec, int64_t T, int N, int64_t C, int k, int L, int l,
                              const void* F_pre, const float* h_pre, const int32_t* idx, const float* H_post,
                              const void* F_outs, void* F_in, hipStream_t st) {
  const int V = vec ? 8 : 1;
  const dim3 grid((unsigned)T, (unsigned)((C / V + FI_THR - 1) / FI_THR)), blk(FI_THR);
#define HC_FI(TE, VV)                                                                                        \
  hipLaunchKernelGGL((flash_input_kernel<TE, VV>), grid, blk, 0, st, T, N, C, k, L, l, (const TE*)F_pre, h_pre, \
                     idx, H_post, (const TE*)F_outs, (TE*)F_in)
  if (dtype == 1) {
    if (vec) HC_FI(bf16_t, 8);
    else HC_FI(bf16_t, 1);
  } else {
    if (vec) HC_FI(float, 8);
    else HC_FI(float, 1);
  }
#undef HC_FI
  return hipGetLastError();
}

hipError_t launch_flash_post_maps(int64_t T, int k, int L, int Kb, const float* H_post, const float* H_res, float* E,
                                  hipStream_t st) {
  const int64_t n = T * k * Kb;
  hipLaunchKernelGGL(flash_post_maps_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, T, k, L, Kb, H_post,
                     H_res, E);
  return hipGetLastError();
}

}  // namespace hc
