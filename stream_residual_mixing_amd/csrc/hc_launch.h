// Host-side launch functions of libhc's kernels (internal; the public ABI is include/hc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define HC_MAX_COMPONENTS_DEV 8

namespace hc {

// Causal depthwise convolution set: r kernels of sizes kappa[j]; the weights of
// kernel j start `offset[j]` floats into the concatenated weight array.
struct ConvSpec {
  int r;
  int kappa[HC_MAX_COMPONENTS_DEV - 1];
  int64_t offset[HC_MAX_COMPONENTS_DEV - 1];
};

// ---- generic kernels (hc_generic.hip)
hipError_t launch_proj_generic(int dtype, const void* X, int64_t tok_stride, int64_t T, int64_t C,
                               int nvec, const int32_t* idx, int Nstreams, const float* phiA,
                               int colsA, const float* phiB, int colsB, float* P, float* ss,
                               hipStream_t st);
hipError_t launch_coeff_epilogue(const float* P, const float* ss, float len, int64_t T, int npre,
                                 int npost, int nres, float a_pre, float a_post, float a_res,
                                 const float* bias, int iters, float* h_pre, float* h_post,
                                 float* h_res, hipStream_t st);
hipError_t launch_xhc_select(const float* P, int pcols, int pre_off, int router_off, const float* ss,
                             float len, int64_t T, int N, int k, int m, float a_pre,
                             const float* b_pre, float* h_pre, float* score, int32_t* idx,
                             hipStream_t st);
hipError_t launch_pre_generic(int dtype, bool vec, const void* X, int64_t T, int n, int64_t C,
                              const float* h, void* F_in, hipStream_t st);
hipError_t launch_post_generic(int dtype, bool vec, const void* X, int64_t T, int n, int64_t C,
                               const float* h_res, const float* h_post, const void* F, void* Y,
                               hipStream_t st);
hipError_t launch_mix_generic(int dtype, bool vec, void* X, int64_t T, int N, int64_t C, int k,
                              const int32_t* idx, const float* H_res, const float* H_post,
                              const void* Wb, int K, hipStream_t st, const void* Wb2 = nullptr, int j0 = 0);
int64_t augment_generic_lds_bytes(int r, int64_t C);
hipError_t launch_augment_generic(int dtype, int vdtype, const void* F, int64_t B, int64_t S,
                                  int64_t C, const float* w, const ConvSpec& spec, void* V,
                                  hipStream_t st);

// ---- HC baseline and the gain diagnostic (hc_baseline.hip)
// vec: C % 8 == 0 with X and theta 16-byte aligned.
hipError_t launch_hc_tanh(int dtype, bool vec, const void* X, int64_t T, int n, int64_t C, const float* theta,
                          const float* bias, float a_pre, float a_post, float a_res, float* h_pre, float* h_post,
                          float* h_res, hipStream_t st);
hipError_t launch_amax_gain(const float* H, int64_t L, int64_t T, int n, float* fwd, float* bwd, hipStream_t st);

// ---- static mHC (hc_static.hip)
hipError_t launch_static_maps(const float* logits, int n, int iters, float* h_pre, float* h_post, float* h_res,
                              hipStream_t st);
// post: X_next from (h_res = h1, h_post = h2, F); else F_in (into Y) from h_pre = h1.
// vec: C % 8 == 0 with X, F and Y 16-byte aligned.
hipError_t launch_static_apply(int dtype, bool post, bool vec, const void* X, int64_t T, int n, int64_t C,
                               const float* h1, const float* h2, const void* F, void* Y, hipStream_t st);

// ---- xHC-Flash (hc_flash.hip)
// The L dense reads of the block-entry state from one pass: h_pre [L, T, N], F [L, T, C]
// (bfloat16, N % 4 == 0, N <= 16, L <= 4, C % 8 == 0, 16-byte aligned X and F).
bool fast_pre_multi_supported(int dtype, int N, int64_t C, int L, const void* X, const void* F);
hipError_t launch_fast_pre_multi(const void* X, int64_t T, int N, int64_t C, int L, const float* h_pre, void* F,
                                 hipStream_t st);
// F_in = F_pre_l + sum_{j<l} c_j F_outs[:, j] (h_pre_l [T, N], H_post [T, k, L], F_outs [T, L, C]);
// vec: C % 8 == 0 with the three stream arrays 16-byte aligned.
hipError_t launch_flash_input(int dtype, bool vec, int64_t T, int N, int64_t C, int k, int L, int l,
                              const void* F_pre, const float* h_pre, const int32_t* idx, const float* H_post,
                              const void* F_outs, void* F_in, hipStream_t st);
// E [T, k, L]: the block end's write maps (H_res H_post[:, j] for j < L - 1, H_post[:, L - 1]).
hipError_t launch_flash_post_maps(int64_t T, int k, int L, int Kb, const float* H_post, const float* H_res, float* E,
                                  hipStream_t st);

}  // namespace hc
