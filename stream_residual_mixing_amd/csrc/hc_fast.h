// Specialised fast paths of libhc (internal). Each has a predicate saying
// whether it covers a call; otherwise the generic kernels run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hc {

// Bytes of the packed phi used by the fused coefficient kernel (0 if unused).
int64_t fast_coeffs_packed_bytes(int n, int64_t C, int dtype);
// Bytes of the per-item partial projections of the fused kernels (0 if unused).
int64_t fast_coeffs_partial_bytes(int64_t T, int n, int64_t C, int dtype);
bool fast_coeffs_supported(int dtype, int n, int64_t T, int64_t C, const void* X);
// Coefficients (+ pre-read when F_in != nullptr) for n = 4 bfloat16 streams.
// h_pre may be nullptr when F_in is given (the pre-read forms h_pre itself).
hipError_t launch_fast_coeffs_pre(const void* X, int64_t T, int64_t C, const float* phi,
                                  const float* bias, float a_pre, float a_post, float a_res,
                                  int iters, float* h_pre, float* h_post, float* h_res, void* F_in,
                                  void* packed, float* partial, hipStream_t st);
// phi [4C, 24] float32 -> the packed bf16 hi/lo B-operand layout (fast_coeffs_packed_bytes).
hipError_t launch_fast_pack(const float* phi, int64_t C, void* packed, hipStream_t st);
// Pre-read for n = 4 bfloat16 streams (C % 8 == 0, 16-byte aligned).
hipError_t launch_fast_pre(const void* X, int64_t T, int64_t C, const float* h_pre, void* F_in,
                           hipStream_t st);
// Post/res write fused with the coefficients of the state it writes (phi, bias, gates of
// the next sublayer) and, when F_in_n != nullptr, its pre-read (h_pre_n may then be
// nullptr). phi_packed (may be nullptr) holds phi already packed; otherwise phi is
// packed into `packed`.
hipError_t launch_fast_post_coeffs(const void* X, int64_t T, int64_t C, const float* h_res,
                                   const float* h_post, const void* F, void* Y, const float* phi,
                                   const void* phi_packed, const float* bias, float a_pre, float a_post,
                                   float a_res, int iters, float* h_pre_n, float* h_post_n, float* h_res_n,
                                   void* F_in_n, void* packed, float* partial, hipStream_t st);

bool fast_post_supported(int dtype, int n, int64_t C, const void* X, const void* F, const void* Y);

// mHC sublayer backward for n = 4 bfloat16 streams (hc_backward.hip), in two
// stages (all device pointers; the bfloat16 arrays 16-byte aligned):
//  post: dF_out = H_post dX_next and dh[:, 4:24] = [dH_post | dH_res] from X,
//    F_out, dX_next and the forward's h_post;
//  main: dh[:, 0:4] = dH_pre from X and dF_in, then dX, dphi, dbias, dalpha.
bool fast_backward_supported(int dtype, int n, int64_t T, int64_t C, int iters);
int64_t fast_backward_ws_bytes(int64_t T, int64_t C);
hipError_t launch_fast_backward_post(const void* X, int64_t T, int64_t C, const float* h_post, const void* F_out,
                                     const void* dX_next, void* dF_out, float* dh, hipStream_t st);
hipError_t launch_fast_backward(const void* X, int64_t T, int64_t C, const float* phi, const float* bias,
                                float a_pre, float a_post, float a_res, int iters, const void* dX_next,
                                const void* dF_in, float* dh, void* dX, float* dphi, float* dbias, float* dalpha,
                                void* ws, hipStream_t st);
// xHC routed-step backward (N % 4 == 0, N <= 16, k = 4, K = 1 or 4, bfloat16, C %
// 32 == 0; the bfloat16 arrays 16-byte aligned), both calls sharing one workspace
// size:
//  route: dX holds dX_next on entry and the route's gradient on exit (only the
//    active rows change); dWb (K = 1: dF_out [T, C] bfloat16; K = 4: dV [T, 4, C]
//    float32), dphi_act [4C, 4K + 16], db_act, dalpha [2] (post, res), dh
//    [T, 4K + 16] = [dH_post | dH_res];
//  pre: dX += the dense read's gradient; dphi_pre [NC, N], db_pre [N],
//    dalpha [1], dh_pre [T, N].
bool fast_xhc_backward_supported(int dtype, int N, int k, int K, int64_t T, int64_t C, int iters);
int64_t fast_xhc_backward_ws_bytes(int64_t T, int N, int64_t C);
hipError_t launch_fast_xroute_backward(const void* X, int64_t T, int N, int64_t C, const int32_t* idx,
                                       const float* phi_act, const float* b_act, float a_post, float a_res, int iters,
                                       const void* Wb, int K, void* dX, void* dWb, float* dphi_act, float* db_act,
                                       float* dalpha, float* dh, void* ws, hipStream_t st);
hipError_t launch_fast_xpre_backward(const void* X, int64_t T, int N, int64_t C, const float* phi_pre,
                                     const float* b_pre, float a_pre, const void* dF_in, void* dX, float* dphi_pre,
                                     float* db_pre, float* dalpha, float* dh_pre, void* ws, hipStream_t st);
// Backward of the temporal augmentation for r = 3 convs of sizes (4, 8, 12): dV
// [T, 4, C] float32 in; dF_out [T, C] (F_out's dtype, bfloat16 or float32) and
// dconv_w (conv_w's layout) out; any C.
bool fast_augment_backward_supported(int dtype, int64_t B, int64_t S, int64_t C, const int* kappa, int r);
int64_t fast_augment_backward_ws_bytes(int64_t B, int64_t S, int64_t C);
hipError_t launch_fast_augment_backward(const void* F_out, int dtype, int64_t B, int64_t S, int64_t C,
                                        const float* conv_w, const float* dV, void* dF_out, float* dconv_w, void* ws,
                                        hipStream_t st);
// Pieces of the backward in hc_fused.hip, beside the partial layout they read:
//  front: phi packed for the projection (packed) and in the row form of the
//    dP phi^T operand (phi_rows, 4C x 128 bytes), then the projection partials
//    of X on 64-token items, which also carry the partial sums of
//    dH_pre = <dF_in, x_i> taken from the same read of X;
//  coeffs: gates' and Sinkhorn's backward from dh [T, 24] (dH_pre, columns 0..3,
//    written here from the front's partials; dH_post and dH_res read from the
//    post stage): dP [T, 32], g2 [T],
//    the sums red [ceil(T / 16), 36] over groups of 16 tokens, and the
//    forward's h_pre [T, 4] and h_res [T, 16]; dynamic LDS of iters * 1 KB
//    (iters <= 64).
int64_t fast_bwd_packed_bytes(int64_t C);
int64_t fast_bwd_partial_bytes(int64_t T, int64_t C);
hipError_t launch_fast_bwd_front(const void* X, int64_t T, int64_t C, const float* phi, void* packed,
                                 uint4* phi_rows, float* partial, const void* dF_in, hipStream_t st);
// xHC routed-step backward pieces: the gathered active set's coefficient
// backward for K = 1 or 4 (partials of launch_fast_xhc_active, dh [T, 4K + 16] =
// [dH_post | dH_res], h_res out), and the pre map's: the full-state projection of
// the pre columns with the sums <dF_in, x_i> from the same read of the state
// (pack + proj_wide on stream groups), and its backward (dh_pre [T, N], dP, g2,
// red, h_pre [T, N] out). Partial buffer sizes of each.
hipError_t launch_fast_xroute_bwd_coeffs(const float* partial, int64_t T, int64_t C, int K, const float* b_act,
                                         float a_post, float a_res, int iters, const float* dh, float* dP, float* g2,
                                         float* red, float* h_res, hipStream_t st);
hipError_t launch_fast_xpre_bwd_front(const void* X, int64_t T, int N, int64_t C, const float* phi_pre,
                                      const void* dF_in, void* packed, uint4* phi_rows, float* partial,
                                      hipStream_t st);
hipError_t launch_fast_xpre_bwd_coeffs(const float* partial, int64_t T, int N, int64_t C, const float* b_pre,
                                       float a_pre, float* dh_pre, float* dP, float* g2, float* red, float* h_pre,
                                       hipStream_t st);
int64_t fast_xroute_partial_bytes(int64_t T, int64_t C, int K);
int64_t fast_xpre_partial_bytes(int64_t T, int N, int64_t C);
hipError_t launch_fast_bwd_coeffs(const float* partial, int64_t T, int64_t C, const float* bias, float a_pre,
                                  float a_post, float a_res, int iters, float* dh, float* dP, float* g2,
                                  float* red, float* h_pre, float* h_res, hipStream_t st);

// xHC fast paths (bfloat16 streams, C % 32 == 0). Workspace needs of each (all zero
// when the shape has no fast path): the packed phi and the per-item partials.
struct XhcFastWs {
  int64_t packed, partial;
};
// full-state projection (pre columns N and/or router columns N - m): N % 4 == 0, N <= 16
XhcFastWs xhc_pre_fast_ws(int64_t T, int N, int64_t C, int m, bool with_router, int dtype);
XhcFastWs xhc_router_fast_ws(int64_t T, int N, int64_t C, int m, int dtype);
// xHC-Flash block entry (L >= 2) as one projection pass of the router and the L pre
// maps: workspace need ({0, 0} when not covered).
XhcFastWs flash_entry_fast_ws(int64_t T, int N, int64_t C, int m, int L, int dtype);
hipError_t launch_fast_flash_entry(const void* X, int64_t T, int N, int64_t C, int k, int m, int L,
                                   const float* phi_pre, const float* b_pre, float a_pre, const float* w_router,
                                   float* h_pre, float* score, int32_t* idx, void* packed, float* partial,
                                   hipStream_t st);
// active-set projection: k == 4, k*K + k*k <= 32
XhcFastWs xhc_route_fast_ws(int64_t T, int64_t C, int k, int K, int dtype);
// Full-state pass: h_pre (phi_pre != nullptr) and/or router scores + selection
// (w_router != nullptr) from one MFMA projection over all N streams, and when
// F_in != nullptr the pre-read (h_pre then required).
hipError_t launch_fast_xhc_full(const void* X, int64_t T, int N, int64_t C, int k, int m, const float* phi_pre,
                                const float* b_pre, float a_pre, const float* w_router, float* h_pre, float* score,
                                int32_t* idx, void* F_in, void* packed, float* partial, hipStream_t st);
// Active coefficients H_post [T, 4, K], H_res [T, 4, 4] of the streams idx[t, 0..3].
// Streaming copy of `bytes` (a multiple of 16; 16-byte aligned pointers).
hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t st);
// xHC mix + scatter in place for k = 4 bfloat16 active streams, 1 <= K <= 4
// (C % 8 == 0, X and Wb 16-byte aligned).
bool fast_mix_supported(int dtype, int k, int K, int64_t C, const void* X, const void* Wb);
hipError_t launch_fast_mix(void* X, int64_t T, int N, int64_t C, const int32_t* idx, const float* H_res,
                           const float* H_post, const void* Wb, int K, hipStream_t st,
                           const void* Wb2 = nullptr, int j0 = 0);
// The active set's coefficients (H_post [T, 4, K], H_res [T, 4, 4]) for k = 4:
// phi_act packed (and, with phi_rows, also in the backward's row form), the
// gathered projection (64-token items up to K = 4, 32-token ones beyond) and
// the finish. nt_rows: the gathered rows with nontemporal loads, for a caller
// whose next pass gains less from finding them in the last-level cache.
hipError_t launch_fast_xhc_active(const void* X, int64_t T, int N, int64_t C, const int32_t* idx, int K,
                                  const float* phi_act, const float* b_act, float a_post, float a_res, int iters,
                                  float* Hp, float* Hr, void* packed, float* partial, hipStream_t st,
                                  uint4* phi_rows = nullptr, bool nt_rows = false);

// xHC chained step (the route of sublayer l, then sublayer l + 1's maps and dense
// read with one read of the full state): bfloat16, N = 16, k = 4, m <= k, C %
// 512 == 0, 16-byte aligned state, h_pre [T, 16] and idx [T, 4].
//  carry: per-item partials [pre N | router N - m] of sublayer l + 1's maps over
//    the rows outside route l's active set (the first xhc_chain_carry_part_bytes),
//    then those maps packed (xhc_chain_carry_bytes in all);
//  pack_full: [phi_pre | w_router] of one sublayer in the projection's packed form;
//  dense: F_in = sum_i h_pre_i x_i and the carry of the packed maps over the rows
//    not in idx, one pass over the state;
//  chain_maps: the active rows (idx_prev) after the mix grouped by stream and
//    projected, added to the carry, then h_pre, score and idx of the next sublayer.
struct XhcChainWs {
  int64_t packed, pair_part, ptok, pos, tile_off, sort;
};
bool xhc_chain_supported(int dtype, int64_t T, int N, int64_t C, int k, int m);
int64_t xhc_chain_carry_part_bytes(int64_t T, int N, int64_t C);
int64_t xhc_chain_carry_bytes(int64_t T, int N, int64_t C);
XhcChainWs xhc_chain_ws(int64_t T, int N, int64_t C, int k);
// the full-state pre-read alone (N % 4 == 0, N <= 16, C % 8 == 0, 16-byte aligned X, F_in)
hipError_t launch_fast_pre_wide(const void* X, int64_t T, int N, int64_t C, const float* h_pre, void* F_in,
                               hipStream_t st);
hipError_t launch_fast_xhc_pack_full(const float* phi_pre, const float* w_router, int N, int m, int64_t C,
                                     void* packed, hipStream_t st);
hipError_t launch_fast_xhc_dense(const void* X, int64_t T, int N, int64_t C, const float* h_pre, const int32_t* idx,
                                 const void* packed, void* F_in, float* carry, hipStream_t st);
hipError_t launch_fast_xhc_chain_maps(const void* X, int64_t T, int N, int64_t C, int k, int m,
                                      const int32_t* idx_prev, const void* packed, const float* carry,
                                      const float* b_pre, float a_pre, float* h_pre, float* score, int32_t* idx,
                                      int32_t* ptok, int32_t* tile_off, int32_t* pos, int32_t* sortw,
                                      float* pair_part, hipStream_t st);

// Temporal augmentation for kappa = {4, 8, 12} (C % 4 == 0; F_out and V aligned to 4
// elements): conv + Gram pass, then Gram-Schmidt from the Gram matrices.
bool fast_augment_supported(int dtype, int vdtype, int64_t S, int64_t C, const int* kappa, int r, const void* F,
                            const void* V);
int64_t fast_augment_workspace_bytes(int64_t B, int64_t S, int64_t C);
hipError_t launch_fast_augment(int dtype, int vdtype, const void* F, int64_t B, int64_t S, int64_t C,
                               const float* w, void* V, float* gram, hipStream_t st);

}  // namespace hc
