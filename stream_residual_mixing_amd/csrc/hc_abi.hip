// extern "C" entry points of libhc (declared in include/hc.h): argument
// validation on the host, workspace carving and kernel dispatch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "hc.h"
#include "hc_launch.h"
#include "hc_fast.h"

namespace {

inline int64_t align256(int64_t b) { return (b + 255) & ~(int64_t)255; }

inline bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t esize(int dtype) { return dtype == HC_F32 ? 4 : 2; }

// True when [a, a+na) and [b, b+nb) share a byte.
inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa < pb + (uintptr_t)nb && pb < pa + (uintptr_t)na;
}

int device_status() {
  static const int status = [] {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return HC_ERR_DEVICE;
    return HC_OK;
  }();
  return status;
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? HC_OK : HC_ERR_LAUNCH; }

inline bool dtype_ok(int d) { return d == HC_F32 || d == HC_BF16; }

// Vector (16-byte) paths need C % 8 == 0 and 16-byte aligned stream pointers.
inline bool vec_ok(int64_t C, std::initializer_list<const void*> ps) {
  if (C % 8 != 0) return false;
  for (const void* p : ps)
    if (p && !aligned_to(p, 16)) return false;
  return true;
}

// Workspace of the mHC coefficient calls: projection rows P [T, n*n+2n],
// squared norms ss [T], a private h_pre [T, n] (used when the caller passes
// none), and for the fast path the packed phi and the per-item partial
// projections.
struct CoeffWs {
  float* P;
  float* ss;
  float* h_pre;
  void* packed;
  float* partial;
};

int64_t mhc_ws_bytes(int64_t T, int n, int64_t C, int dtype) {
  const int ncols = n * n + 2 * n;
  int64_t b = align256(T * ncols * 4) + align256(T * 4) + align256(T * n * 4);
  b += align256(hc::fast_coeffs_packed_bytes(n, C, dtype));
  b += align256(hc::fast_coeffs_partial_bytes(T, n, C, dtype));
  return b;
}

CoeffWs carve_mhc(void* ws, int64_t T, int n, int64_t C, int dtype) {
  const int ncols = n * n + 2 * n;
  char* p = (char*)ws;
  CoeffWs w;
  w.P = (float*)p;
  p += align256(T * ncols * 4);
  w.ss = (float*)p;
  p += align256(T * 4);
  w.h_pre = (float*)p;
  p += align256(T * n * 4);
  w.packed = p;
  p += align256(hc::fast_coeffs_packed_bytes(n, C, dtype));
  w.partial = (float*)p;
  return w;
}

int check_mhc_common(const void* X, int dtype, int64_t T, int n, int64_t C) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (T < 0 || C < 1 || C > (1ll << 26) || n < 1 || n > HC_MAX_MHC_STREAMS) return HC_ERR_SHAPE;
  if (T > 0 && !X) return HC_ERR_NULL;
  if (X && !aligned_to(X, esize(dtype))) return HC_ERR_ALIGN;
  return HC_OK;
}

int check_coeff_args(const void* X, int dtype, int64_t T, int n, int64_t C, const float* phi,
                     const float* bias, int iters, const float* h_pre, const float* h_post,
                     const float* h_res, bool h_pre_optional, void* ws, int64_t ws_bytes) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK) return s;
  if (iters < 1 || iters > HC_MAX_ITERS) return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!phi || !bias || !h_post || !h_res || (!h_pre && !h_pre_optional)) return HC_ERR_NULL;
  for (const void* p : {(const void*)phi, (const void*)bias, (const void*)h_pre, (const void*)h_post,
                        (const void*)h_res})
    if (p && !aligned_to(p, 4)) return HC_ERR_ALIGN;
  if (!ws || !aligned_to(ws, 256) || ws_bytes < mhc_ws_bytes(T, n, C, dtype)) return HC_ERR_WORKSPACE;
  const int64_t xb = T * n * C * (int64_t)esize(dtype);
  const int64_t wsb = mhc_ws_bytes(T, n, C, dtype);
  const void* outs[3] = {h_pre, h_post, h_res};
  const int64_t ob[3] = {T * n * 4, T * n * 4, T * n * n * 4};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(outs[i], ob[i], X, xb) || overlaps(outs[i], ob[i], phi, (int64_t)n * C * (n * n + 2 * n) * 4) ||
        overlaps(outs[i], ob[i], bias, (n * n + 2 * n) * 4) || overlaps(outs[i], ob[i], ws, wsb))
      return HC_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return HC_ERR_ALIAS;
  }
  if (overlaps(ws, wsb, X, xb) || overlaps(ws, wsb, phi, (int64_t)n * C * (n * n + 2 * n) * 4) ||
      overlaps(ws, wsb, bias, (n * n + 2 * n) * 4))
    return HC_ERR_ALIAS;
  return HC_OK;
}

// Generic coefficient path: projection, then the per-token epilogue.
int run_coeffs_generic(const void* X, int dtype, int64_t T, int n, int64_t C, const float* phi,
                       const float* bias, float a_pre, float a_post, float a_res, int iters,
                       float* h_pre, float* h_post, float* h_res, const CoeffWs& w,
                       hipStream_t st) {
  const int ncols = n * n + 2 * n;
  hipError_t e = hc::launch_proj_generic(dtype, X, (int64_t)n * C, T, C, n, nullptr, n, phi, ncols,
                                         nullptr, 0, w.P, w.ss, st);
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  e = hc::launch_coeff_epilogue(w.P, w.ss, (float)((double)n * (double)C), T, n, n, n, a_pre, a_post,
                                a_res, bias, iters, h_pre, h_post, h_res, st);
  return launch_status(e);
}

}  // namespace

extern "C" {

const char* hc_status_string(int status) {
  switch (status) {
    case HC_OK: return "ok";
    case HC_ERR_NULL: return "a required pointer is NULL";
    case HC_ERR_SHAPE: return "a size or count is out of range";
    case HC_ERR_DTYPE: return "unknown dtype code";
    case HC_ERR_ALIGN: return "a pointer is not aligned to its element size";
    case HC_ERR_ALIAS: return "an output overlaps an input it must not";
    case HC_ERR_DEVICE: return "no usable HIP device";
    case HC_ERR_LAUNCH: return "a kernel launch failed";
    case HC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case HC_ERR_SCRATCH: return "the sizes need more than the library's fixed scratch (HC_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int hc_version(void) { return 102; }

int64_t hc_coeffs_workspace_bytes(int64_t T, int n, int64_t C, int dtype) {
  if (T < 0 || n < 1 || n > HC_MAX_MHC_STREAMS || C < 1 || !dtype_ok(dtype)) return -1;
  return mhc_ws_bytes(T, n, C, dtype);
}

int hc_coeffs(const void* X, int dtype, int64_t T, int n, int64_t C, const float* phi,
              const float* bias, float alpha_pre, float alpha_post, float alpha_res,
              int sinkhorn_iters, float* h_pre, float* h_post, float* h_res, void* workspace,
              int64_t workspace_bytes, void* stream) {
  int s = check_coeff_args(X, dtype, T, n, C, phi, bias, sinkhorn_iters, h_pre, h_post, h_res,
                           false, workspace, workspace_bytes);
  if (s != HC_OK || T == 0) return s;
  if ((s = device_status()) != HC_OK) return s;
  const CoeffWs w = carve_mhc(workspace, T, n, C, dtype);
  hipStream_t st = (hipStream_t)stream;
  if (hc::fast_coeffs_supported(dtype, n, T, C, X)) {
    return launch_status(hc::launch_fast_coeffs_pre(X, T, C, phi, bias, alpha_pre, alpha_post,
                                                    alpha_res, sinkhorn_iters, h_pre, h_post,
                                                    h_res, nullptr, w.packed, w.partial, st));
  }
  return run_coeffs_generic(X, dtype, T, n, C, phi, bias, alpha_pre, alpha_post, alpha_res,
                            sinkhorn_iters, h_pre, h_post, h_res, w, st);
}

int hc_pre(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_pre, void* F_in,
           void* stream) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK || T == 0) return s;
  if (!h_pre || !F_in) return HC_ERR_NULL;
  if (!aligned_to(h_pre, 4) || !aligned_to(F_in, esize(dtype))) return HC_ERR_ALIGN;
  const int64_t xb = T * n * C * (int64_t)esize(dtype), fb = T * C * (int64_t)esize(dtype);
  if (overlaps(F_in, fb, X, xb) || overlaps(F_in, fb, h_pre, T * n * 4)) return HC_ERR_ALIAS;
  if ((s = device_status()) != HC_OK) return s;
  if (dtype == HC_BF16 && n == 4 && vec_ok(C, {X, F_in}))
    return launch_status(hc::launch_fast_pre(X, T, C, h_pre, F_in, (hipStream_t)stream));
  return launch_status(hc::launch_pre_generic(dtype, vec_ok(C, {X, F_in}), X, T, n, C, h_pre, F_in,
                                              (hipStream_t)stream));
}

int hc_coeffs_pre(const void* X, int dtype, int64_t T, int n, int64_t C, const float* phi,
                  const float* bias, float alpha_pre, float alpha_post, float alpha_res,
                  int sinkhorn_iters, float* h_pre, float* h_post, float* h_res, void* F_in,
                  void* workspace, int64_t workspace_bytes, void* stream) {
  int s = check_coeff_args(X, dtype, T, n, C, phi, bias, sinkhorn_iters, h_pre, h_post, h_res,
                           true, workspace, workspace_bytes);
  if (s != HC_OK || T == 0) return s;
  if (!F_in) return HC_ERR_NULL;
  if (!aligned_to(F_in, esize(dtype))) return HC_ERR_ALIGN;
  {
    const int64_t xb = T * n * C * (int64_t)esize(dtype), fb = T * C * (int64_t)esize(dtype);
    const int64_t wsb = mhc_ws_bytes(T, n, C, dtype);
    if (overlaps(F_in, fb, X, xb) || overlaps(F_in, fb, workspace, wsb) ||
        overlaps(F_in, fb, h_pre, T * n * 4) || overlaps(F_in, fb, h_post, T * n * 4) ||
        overlaps(F_in, fb, h_res, T * n * n * 4) ||
        overlaps(F_in, fb, phi, (int64_t)n * C * (n * n + 2 * n) * 4) ||
        overlaps(F_in, fb, bias, (n * n + 2 * n) * 4))
      return HC_ERR_ALIAS;
  }
  if ((s = device_status()) != HC_OK) return s;
  const CoeffWs w = carve_mhc(workspace, T, n, C, dtype);
  hipStream_t st = (hipStream_t)stream;
  if (hc::fast_coeffs_supported(dtype, n, T, C, X) && aligned_to(F_in, 16)) {
    return launch_status(hc::launch_fast_coeffs_pre(X, T, C, phi, bias, alpha_pre, alpha_post,
                                                    alpha_res, sinkhorn_iters, h_pre, h_post, h_res, F_in,
                                                    w.packed, w.partial, st));
  }
  // Generic: the pre-read needs h_pre, kept in the workspace when the caller
  // does not ask for it.
  float* hp = h_pre ? h_pre : w.h_pre;
  s = run_coeffs_generic(X, dtype, T, n, C, phi, bias, alpha_pre, alpha_post, alpha_res,
                         sinkhorn_iters, hp, h_post, h_res, w, st);
  if (s != HC_OK) return s;
  return launch_status(hc::launch_pre_generic(dtype, vec_ok(C, {X, F_in}), X, T, n, C, hp, F_in, st));
}

int64_t hc_backward_workspace_bytes(int64_t T, int n, int64_t C, int dtype) {
  if (T < 0) return -1;
  if (T == 0) return 0;
  if (!hc::fast_backward_supported(dtype, n, T, C, 1)) return -1;
  return hc::fast_backward_ws_bytes(T, C);
}

// the shapes and dtype both backward stages cover (T >= 0)
static int check_backward_shape(int dtype, int64_t T, int n, int64_t C) {
  if (!dtype_ok(dtype) || dtype != HC_BF16) return HC_ERR_DTYPE;
  if (T < 0 || n != 4 || C < 32 || C % 32 != 0 || C > (1ll << 26)) return HC_ERR_SHAPE;
  return HC_OK;
}

// pairwise overlap of outputs with every input and with each other
static bool any_overlap(const void* const* outs, const int64_t* ob, int no, const void* const* ins,
                        const int64_t* ib, int ni) {
  for (int i = 0; i < no; ++i) {
    for (int j = 0; j < ni; ++j)
      if (overlaps(outs[i], ob[i], ins[j], ib[j])) return true;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return true;
  }
  return false;
}

int hc_backward_post(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_post, const void* F_out,
                     const void* dX_next, void* dF_out, float* dh, void* stream) {
  int s = check_backward_shape(dtype, T, n, C);
  if (s != HC_OK || T == 0) return s;
  if (!hc::fast_backward_supported(dtype, n, T, C, 1)) return HC_ERR_SHAPE;
  if (!X || !h_post || !F_out || !dX_next || !dF_out || !dh) return HC_ERR_NULL;
  for (const void* p : {X, (const void*)h_post, F_out, dX_next, (const void*)dF_out})
    if (!aligned_to(p, 16)) return HC_ERR_ALIGN;
  if (!aligned_to(dh, 4)) return HC_ERR_ALIGN;
  const int64_t xb = T * 4 * C * 2, fb = T * C * 2;
  const void* ins[4] = {X, h_post, F_out, dX_next};
  const int64_t ib[4] = {xb, T * 16, fb, xb};
  const void* outs[2] = {dF_out, dh};
  const int64_t ob[2] = {fb, T * 24 * 4};
  if (any_overlap(outs, ob, 2, ins, ib, 4)) return HC_ERR_ALIAS;
  if ((s = device_status()) != HC_OK) return s;
  return launch_status(
      hc::launch_fast_backward_post(X, T, C, h_post, F_out, dX_next, dF_out, dh, (hipStream_t)stream));
}

int hc_backward(const void* X, int dtype, int64_t T, int n, int64_t C, const float* phi, const float* bias,
                float alpha_pre, float alpha_post, float alpha_res, int sinkhorn_iters, const void* dX_next,
                const void* dF_in, float* dh, void* dX, float* dphi, float* dbias, float* dalpha, void* workspace,
                int64_t workspace_bytes, void* stream) {
  int s = check_backward_shape(dtype, T, n, C);
  if (s != HC_OK) return s;
  if (sinkhorn_iters < 1 || sinkhorn_iters > HC_MAX_BWD_ITERS) return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!hc::fast_backward_supported(dtype, n, T, C, sinkhorn_iters)) return HC_ERR_SHAPE;
  if (!X || !phi || !bias || !dX_next || !dF_in || !dh || !dX || !dphi || !dbias || !dalpha) return HC_ERR_NULL;
  for (const void* p : {X, dX_next, dF_in, (const void*)dX})
    if (!aligned_to(p, 16)) return HC_ERR_ALIGN;
  for (const void* p : {(const void*)phi, (const void*)bias, (const void*)dh, (const void*)dphi,
                        (const void*)dbias, (const void*)dalpha})
    if (!aligned_to(p, 4)) return HC_ERR_ALIGN;
  const int64_t wsb = hc::fast_backward_ws_bytes(T, C);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int64_t xb = T * 4 * C * 2, fb = T * C * 2, pb = 4 * C * 24 * 4, hb = T * 24 * 4;
  // dh is read and written: it may overlap nothing else
  const void* ins[6] = {X, phi, bias, dX_next, dF_in, dh};
  const int64_t ib[6] = {xb, pb, 24 * 4, xb, fb, hb};
  const void* outs[5] = {dX, dphi, dbias, dalpha, workspace};
  const int64_t ob[5] = {xb, pb, 24 * 4, 3 * 4, wsb};
  if (any_overlap(outs, ob, 5, ins, ib, 6)) return HC_ERR_ALIAS;
  {
    const void* ins2[5] = {X, phi, bias, dX_next, dF_in};
    const int64_t ib2[5] = {xb, pb, 24 * 4, xb, fb};
    const void* outs2[1] = {dh};
    const int64_t ob2[1] = {hb};
    if (any_overlap(outs2, ob2, 1, ins2, ib2, 5)) return HC_ERR_ALIAS;
  }
  if ((s = device_status()) != HC_OK) return s;
  return launch_status(hc::launch_fast_backward(X, T, C, phi, bias, alpha_pre, alpha_post, alpha_res,
                                                sinkhorn_iters, dX_next, dF_in, dh, dX, dphi, dbias, dalpha,
                                                workspace, (hipStream_t)stream));
}

int64_t xhc_backward_workspace_bytes(int64_t T, int N, int64_t C, int k, int K, int dtype) {
  if (T < 0) return -1;
  if (T == 0) return 0;
  if (!hc::fast_xhc_backward_supported(dtype, N, k, K, T, C, 1)) return -1;
  return hc::fast_xhc_backward_ws_bytes(T, N, C);
}

// the shapes both xHC backward calls cover (T >= 0)
static int check_xhc_backward_shape(int dtype, int64_t T, int N, int64_t C) {
  if (!dtype_ok(dtype) || dtype != HC_BF16) return HC_ERR_DTYPE;
  if (T < 0 || N < 4 || N > 16 || N % 4 != 0 || C < 32 || C % 32 != 0 || C > (1ll << 26)) return HC_ERR_SHAPE;
  return HC_OK;
}

int xhc_route_backward(const void* X, int dtype, int64_t T, int N, int64_t C, int k, const int32_t* idx,
                       const float* phi_act, const float* b_act, float alpha_post, float alpha_res,
                       int sinkhorn_iters, const void* Wb, int K, void* dX, void* dWb, float* dphi_act,
                       float* db_act, float* dalpha, float* dh, void* workspace, int64_t workspace_bytes,
                       void* stream) {
  int s = check_xhc_backward_shape(dtype, T, N, C);
  if (s != HC_OK) return s;
  if (k != 4 || (K != 1 && K != 4) || sinkhorn_iters < 1 || sinkhorn_iters > HC_MAX_BWD_ITERS)
    return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!hc::fast_xhc_backward_supported(dtype, N, k, K, T, C, sinkhorn_iters)) return HC_ERR_SHAPE;
  if (!X || !idx || !phi_act || !b_act || !Wb || !dX || !dWb || !dphi_act || !db_act || !dalpha || !dh)
    return HC_ERR_NULL;
  for (const void* p : {X, Wb, (const void*)dX, (const void*)dWb, (const void*)idx})
    if (!aligned_to(p, 16)) return HC_ERR_ALIGN;
  for (const void* p : {(const void*)phi_act, (const void*)b_act, (const void*)dphi_act, (const void*)db_act,
                        (const void*)dalpha, (const void*)dh})
    if (!aligned_to(p, 4)) return HC_ERR_ALIGN;
  const int64_t wsb = hc::fast_xhc_backward_ws_bytes(T, N, C);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int ncol = 4 * K + 16;
  // Wb: K bfloat16 rows per token; dWb: bfloat16 for K = 1, float32 for K = 4
  const int64_t xb = T * N * C * 2, wb = T * K * C * 2, dwb = K == 1 ? T * C * 2 : T * K * C * 4;
  const int64_t pb = 4 * C * ncol * 4;
  // dX is read and written: it may overlap nothing else
  const void* ins[6] = {X, idx, phi_act, b_act, Wb, dX};
  const int64_t ib[6] = {xb, T * 4 * 4, pb, ncol * 4, wb, xb};
  const void* outs[6] = {dWb, dphi_act, db_act, dalpha, dh, workspace};
  const int64_t ob[6] = {dwb, pb, ncol * 4, 2 * 4, T * ncol * 4, wsb};
  if (any_overlap(outs, ob, 6, ins, ib, 6)) return HC_ERR_ALIAS;
  {
    const void* i2[5] = {X, idx, phi_act, b_act, Wb};
    const int64_t b2[5] = {xb, T * 4 * 4, pb, ncol * 4, wb};
    const void* o2[1] = {dX};
    const int64_t ob2[1] = {xb};
    if (any_overlap(o2, ob2, 1, i2, b2, 5)) return HC_ERR_ALIAS;
  }
  if ((s = device_status()) != HC_OK) return s;
  return launch_status(hc::launch_fast_xroute_backward(X, T, N, C, idx, phi_act, b_act, alpha_post, alpha_res,
                                                       sinkhorn_iters, Wb, K, dX, dWb, dphi_act, db_act, dalpha,
                                                       dh, workspace, (hipStream_t)stream));
}

int xhc_pre_backward(const void* X, int dtype, int64_t T, int N, int64_t C, const float* phi_pre, const float* b_pre,
                     float alpha_pre, const void* dF_in, void* dX, float* dphi_pre, float* db_pre, float* dalpha,
                     float* dh_pre, void* workspace, int64_t workspace_bytes, void* stream) {
  int s = check_xhc_backward_shape(dtype, T, N, C);
  if (s != HC_OK || T == 0) return s;
  if (!hc::fast_xhc_backward_supported(dtype, N, 4, 1, T, C, 1)) return HC_ERR_SHAPE;
  if (!X || !phi_pre || !b_pre || !dF_in || !dX || !dphi_pre || !db_pre || !dalpha || !dh_pre) return HC_ERR_NULL;
  for (const void* p : {X, dF_in, (const void*)dX, (const void*)dh_pre})
    if (!aligned_to(p, 16)) return HC_ERR_ALIGN;
  for (const void* p : {(const void*)phi_pre, (const void*)b_pre, (const void*)dphi_pre, (const void*)db_pre,
                        (const void*)dalpha})
    if (!aligned_to(p, 4)) return HC_ERR_ALIGN;
  const int64_t wsb = hc::fast_xhc_backward_ws_bytes(T, N, C);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int64_t xb = T * N * C * 2, fb = T * C * 2, pb = (int64_t)N * C * N * 4;
  const void* ins[5] = {X, phi_pre, b_pre, dF_in, dX};
  const int64_t ib[5] = {xb, pb, N * 4, fb, xb};
  const void* outs[5] = {dphi_pre, db_pre, dalpha, dh_pre, workspace};
  const int64_t ob[5] = {pb, N * 4, 4, T * N * 4, wsb};
  if (any_overlap(outs, ob, 5, ins, ib, 5)) return HC_ERR_ALIAS;
  {
    const void* i2[4] = {X, phi_pre, b_pre, dF_in};
    const int64_t b2[4] = {xb, pb, N * 4, fb};
    const void* o2[1] = {dX};
    const int64_t ob2[1] = {xb};
    if (any_overlap(o2, ob2, 1, i2, b2, 4)) return HC_ERR_ALIAS;
  }
  if ((s = device_status()) != HC_OK) return s;
  return launch_status(hc::launch_fast_xpre_backward(X, T, N, C, phi_pre, b_pre, alpha_pre, dF_in, dX, dphi_pre,
                                                     db_pre, dalpha, dh_pre, workspace, (hipStream_t)stream));
}

int64_t xhc_augment_backward_workspace_bytes(int64_t B, int64_t S, int64_t C, const int* kappa, int r, int dtype) {
  if (B < 0 || S < 0 || C < 1) return -1;
  if (B == 0 || S == 0) return 0;
  if (!hc::fast_augment_backward_supported(dtype, B, S, C, kappa, r)) return -1;
  return hc::fast_augment_backward_ws_bytes(B, S, C);
}

int xhc_augment_backward(const void* F_out, int dtype, int64_t B, int64_t S, int64_t C, const float* conv_w,
                         const int* kappa, int r, const float* dV, void* dF_out, float* dconv_w, void* workspace,
                         int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (B < 0 || S < 0 || C < 1 || C > (1ll << 26) || r != 3 || !kappa) return HC_ERR_SHAPE;
  if (B == 0 || S == 0) return HC_OK;
  if (!hc::fast_augment_backward_supported(dtype, B, S, C, kappa, r)) return HC_ERR_SHAPE;
  if (!F_out || !conv_w || !dV || !dF_out || !dconv_w) return HC_ERR_NULL;
  if (!aligned_to(F_out, esize(dtype)) || !aligned_to(dF_out, esize(dtype)) || !aligned_to(conv_w, 4) ||
      !aligned_to(dV, 4) || !aligned_to(dconv_w, 4))
    return HC_ERR_ALIGN;
  const int64_t wsb = hc::fast_augment_backward_ws_bytes(B, S, C);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int64_t T = B * S, fb = T * C * esize(dtype), wb = C * 24 * 4;
  const void* ins[3] = {F_out, conv_w, dV};
  const int64_t ib[3] = {fb, wb, T * 4 * C * 4};
  const void* outs[3] = {dF_out, dconv_w, workspace};
  const int64_t ob[3] = {fb, wb, wsb};
  if (any_overlap(outs, ob, 3, ins, ib, 3)) return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  return launch_status(hc::launch_fast_augment_backward(F_out, dtype, B, S, C, conv_w, dV, dF_out, dconv_w,
                                                        workspace, (hipStream_t)stream));
}

int hc_post(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res,
            const float* h_post, const void* F_out, void* X_next, void* stream) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK || T == 0) return s;
  if (!h_res || !h_post || !F_out || !X_next) return HC_ERR_NULL;
  if (!aligned_to(h_res, 4) || !aligned_to(h_post, 4) || !aligned_to(F_out, esize(dtype)) ||
      !aligned_to(X_next, esize(dtype)))
    return HC_ERR_ALIGN;
  const int64_t xb = T * n * C * (int64_t)esize(dtype), fb = T * C * (int64_t)esize(dtype);
  if (X_next != X && overlaps(X_next, xb, X, xb)) return HC_ERR_ALIAS;
  if (overlaps(X_next, xb, F_out, fb) || overlaps(X_next, xb, h_res, T * n * n * 4) ||
      overlaps(X_next, xb, h_post, T * n * 4))
    return HC_ERR_ALIAS;
  if ((s = device_status()) != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  return launch_status(hc::launch_post_generic(dtype, vec_ok(C, {X, F_out, X_next}), X, T, n, C,
                                               h_res, h_post, F_out, X_next, st));
}

}  // extern "C"

namespace {

// Validation shared by hc_post_coeffs and hc_post_pre: hc_post's arguments, then
// hc_coeffs' arguments on X_next, then the new coefficients against the inputs.
int check_post_coeffs(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res,
                      const float* h_post, const void* F_out, void* X_next, const float* phi_next,
                      const float* bias_next, int sinkhorn_iters, float* h_pre_next, bool h_pre_optional,
                      float* h_post_next, float* h_res_next, void* workspace, int64_t workspace_bytes) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK) return s;
  if (sinkhorn_iters < 1 || sinkhorn_iters > HC_MAX_ITERS) return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!h_res || !h_post || !F_out || !X_next) return HC_ERR_NULL;
  if (!aligned_to(h_res, 4) || !aligned_to(h_post, 4) || !aligned_to(F_out, esize(dtype)) ||
      !aligned_to(X_next, esize(dtype)))
    return HC_ERR_ALIGN;
  const int64_t xb = T * n * C * (int64_t)esize(dtype), fb = T * C * (int64_t)esize(dtype);
  if (X_next != X && overlaps(X_next, xb, X, xb)) return HC_ERR_ALIAS;
  if (overlaps(X_next, xb, F_out, fb) || overlaps(X_next, xb, h_res, T * n * n * 4) ||
      overlaps(X_next, xb, h_post, T * n * 4))
    return HC_ERR_ALIAS;
  s = check_coeff_args(X_next, dtype, T, n, C, phi_next, bias_next, sinkhorn_iters, h_pre_next,
                       h_post_next, h_res_next, h_pre_optional, workspace, workspace_bytes);
  if (s != HC_OK) return s;
  // the new coefficients must not overlap the coefficients being read
  const void* outs[3] = {h_pre_next, h_post_next, h_res_next};
  const int64_t ob[3] = {T * n * 4, T * n * 4, T * n * n * 4};
  for (int i = 0; i < 3; ++i)
    if (overlaps(outs[i], ob[i], h_res, T * n * n * 4) || overlaps(outs[i], ob[i], h_post, T * n * 4) ||
        overlaps(outs[i], ob[i], F_out, fb) || overlaps(outs[i], ob[i], X, xb))
      return HC_ERR_ALIAS;
  return HC_OK;
}

}  // namespace

extern "C" {

int hc_post_coeffs(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res,
                   const float* h_post, const void* F_out, void* X_next, const float* phi_next,
                   const float* bias_next, float alpha_pre, float alpha_post, float alpha_res,
                   int sinkhorn_iters, float* h_pre_next, float* h_post_next, float* h_res_next,
                   void* workspace, int64_t workspace_bytes, void* stream) {
  int s = check_post_coeffs(X, dtype, T, n, C, h_res, h_post, F_out, X_next, phi_next, bias_next, sinkhorn_iters,
                            h_pre_next, false, h_post_next, h_res_next, workspace, workspace_bytes);
  if (s != HC_OK || T == 0) return s;
  if ((s = device_status()) != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const CoeffWs w = carve_mhc(workspace, T, n, C, dtype);
  if (hc::fast_post_supported(dtype, n, C, X, F_out, X_next) && hc::fast_coeffs_supported(dtype, n, T, C, X_next))
    return launch_status(hc::launch_fast_post_coeffs(X, T, C, h_res, h_post, F_out, X_next, phi_next, nullptr,
                                                     bias_next, alpha_pre, alpha_post, alpha_res, sinkhorn_iters,
                                                     h_pre_next, h_post_next, h_res_next, nullptr, w.packed,
                                                     w.partial, st));
  hipError_t e = hc::launch_post_generic(dtype, vec_ok(C, {X, F_out, X_next}), X, T, n, C, h_res, h_post,
                                         F_out, X_next, st);
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  return run_coeffs_generic(X_next, dtype, T, n, C, phi_next, bias_next, alpha_pre, alpha_post, alpha_res,
                            sinkhorn_iters, h_pre_next, h_post_next, h_res_next, w, st);
}

int64_t hc_phi_packed_bytes(int n, int64_t C, int dtype) {
  if (n < 1 || n > HC_MAX_MHC_STREAMS || C < 1 || !dtype_ok(dtype)) return -1;
  return hc::fast_coeffs_packed_bytes(n, C, dtype);
}

int hc_phi_pack(const float* phi, int n, int64_t C, int dtype, void* packed, int64_t packed_bytes, void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (n < 1 || n > HC_MAX_MHC_STREAMS || C < 1 || C > (1ll << 26)) return HC_ERR_SHAPE;
  const int64_t pb = hc::fast_coeffs_packed_bytes(n, C, dtype);
  if (pb == 0) return HC_OK;  // no packed form for this shape: the calls use phi itself
  if (!phi || !packed) return HC_ERR_NULL;
  if (!aligned_to(phi, 4) || !aligned_to(packed, 256)) return HC_ERR_ALIGN;
  if (packed_bytes < pb) return HC_ERR_SHAPE;
  if (overlaps(packed, pb, phi, (int64_t)n * C * (n * n + 2 * n) * 4)) return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  return launch_status(hc::launch_fast_pack(phi, C, packed, (hipStream_t)stream));
}

int hc_post_pre(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res,
                const float* h_post, const void* F_out, void* X_next, const float* phi_next,
                const void* phi_next_packed, const float* bias_next, float alpha_pre, float alpha_post,
                float alpha_res, int sinkhorn_iters, float* h_pre_next, float* h_post_next,
                float* h_res_next, void* F_in_next, void* workspace, int64_t workspace_bytes,
                void* stream) {
  int s = check_post_coeffs(X, dtype, T, n, C, h_res, h_post, F_out, X_next, phi_next, bias_next, sinkhorn_iters,
                            h_pre_next, true, h_post_next, h_res_next, workspace, workspace_bytes);
  if (s != HC_OK || T == 0) return s;
  if (!F_in_next) return HC_ERR_NULL;
  if (!aligned_to(F_in_next, esize(dtype))) return HC_ERR_ALIGN;
  {
    const int64_t xb = T * n * C * (int64_t)esize(dtype), fb = T * C * (int64_t)esize(dtype);
    const int64_t wsb = mhc_ws_bytes(T, n, C, dtype);
    const int64_t pb = hc::fast_coeffs_packed_bytes(n, C, dtype);
    if (overlaps(F_in_next, fb, X, xb) || overlaps(F_in_next, fb, X_next, xb) ||
        overlaps(F_in_next, fb, F_out, fb) || overlaps(F_in_next, fb, workspace, wsb) ||
        overlaps(F_in_next, fb, h_res, T * n * n * 4) || overlaps(F_in_next, fb, h_post, T * n * 4) ||
        overlaps(F_in_next, fb, h_pre_next, T * n * 4) || overlaps(F_in_next, fb, h_post_next, T * n * 4) ||
        overlaps(F_in_next, fb, h_res_next, T * n * n * 4) ||
        overlaps(F_in_next, fb, phi_next, (int64_t)n * C * (n * n + 2 * n) * 4) ||
        overlaps(F_in_next, fb, bias_next, (n * n + 2 * n) * 4) ||
        (phi_next_packed && pb > 0 && overlaps(F_in_next, fb, phi_next_packed, pb)))
      return HC_ERR_ALIAS;
    if (phi_next_packed && pb > 0 &&
        (!aligned_to(phi_next_packed, 16) || overlaps(phi_next_packed, pb, X_next, xb) ||
         overlaps(phi_next_packed, pb, workspace, wsb)))
      return phi_next_packed && !aligned_to(phi_next_packed, 16) ? HC_ERR_ALIGN : HC_ERR_ALIAS;
  }
  if ((s = device_status()) != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const CoeffWs w = carve_mhc(workspace, T, n, C, dtype);
  if (hc::fast_post_supported(dtype, n, C, X, F_out, X_next) && hc::fast_coeffs_supported(dtype, n, T, C, X_next) &&
      aligned_to(F_in_next, 16))
    return launch_status(hc::launch_fast_post_coeffs(X, T, C, h_res, h_post, F_out, X_next, phi_next,
                                                     phi_next_packed, bias_next, alpha_pre, alpha_post, alpha_res,
                                                     sinkhorn_iters, h_pre_next, h_post_next, h_res_next, F_in_next,
                                                     w.packed, w.partial, st));
  // generic: post, coefficients of X_next (h_pre kept in the workspace when not
  // requested), pre-read of X_next
  hipError_t e = hc::launch_post_generic(dtype, vec_ok(C, {X, F_out, X_next}), X, T, n, C, h_res, h_post,
                                         F_out, X_next, st);
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  float* hp = h_pre_next ? h_pre_next : w.h_pre;
  s = run_coeffs_generic(X_next, dtype, T, n, C, phi_next, bias_next, alpha_pre, alpha_post, alpha_res,
                         sinkhorn_iters, hp, h_post_next, h_res_next, w, st);
  if (s != HC_OK) return s;
  return launch_status(hc::launch_pre_generic(dtype, vec_ok(C, {X_next, F_in_next}), X_next, T, n, C, hp,
                                              F_in_next, st));
}

// ------------------------------------------------------------- no-alloc --

}  // extern "C"

// The workspace of hc_post_pre_noalloc: a file-scope device array, one copy per
// GPU. In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever passed on.
static __device__ __align__(256) unsigned char scratch[HC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HC_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return HC_ERR_DEVICE;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HC_OK;
}

}  // namespace

extern "C" {

int hc_post_pre_noalloc(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res,
                        const float* h_post, const void* F_out, void* X_next, const float* phi_next,
                        const void* phi_next_packed, const float* bias_next, float alpha_pre, float alpha_post,
                        float alpha_res, int sinkhorn_iters, float* h_pre_next, float* h_post_next,
                        float* h_res_next, void* F_in_next, void* stream) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK) return s;
  if (sinkhorn_iters < 1 || sinkhorn_iters > HC_MAX_ITERS) return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (mhc_ws_bytes(T, n, C, dtype) > HC_NOALLOC_SCRATCH_BYTES) return HC_ERR_SCRATCH;
  void* ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != HC_OK) return s;
  return hc_post_pre(X, dtype, T, n, C, h_res, h_post, F_out, X_next, phi_next, phi_next_packed, bias_next,
                     alpha_pre, alpha_post, alpha_res, sinkhorn_iters, h_pre_next, h_post_next, h_res_next,
                     F_in_next, ws, HC_NOALLOC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------------------ xHC --

// xhc_pre workspace: projection rows P [T, N + router columns], ss [T], a private
// h_pre [T, N]; then the fast path's packed phi and per-item partials.
static int64_t xhc_pre_ws(int64_t T, int N, int64_t C, int m, int with_router, int dtype) {
  const int pcols = N + (with_router ? N - m : 0);
  const hc::XhcFastWs f = hc::xhc_pre_fast_ws(T, N, C, m, with_router, dtype);
  return align256(T * pcols * 4) + align256(T * 4) + align256(T * N * 4) + align256(f.packed) +
         align256(f.partial);
}

int64_t xhc_pre_workspace_bytes(int64_t T, int N, int64_t C, int m, int with_router, int dtype) {
  if (T < 0 || N < 1 || N > HC_MAX_STREAMS || m < 1 || m > N || C < 1 || !dtype_ok(dtype)) return -1;
  return xhc_pre_ws(T, N, C, m, with_router, dtype);
}

int xhc_pre(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int m,
            const float* phi_pre, const float* b_pre, float alpha_pre, const float* w_router,
            float* h_pre, void* F_in, int32_t* idx, float* score, void* workspace,
            int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (T < 0 || C < 1 || C > (1ll << 26) || N < 1 || N > HC_MAX_STREAMS || m < 1 || k < m ||
      k > N || k > HC_MAX_ACTIVE)
    return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!X || !phi_pre || !b_pre || !F_in) return HC_ERR_NULL;
  if (w_router && (!idx || !score)) return HC_ERR_NULL;
  const size_t es = esize(dtype);
  if (!aligned_to(X, es) || !aligned_to(F_in, es) || !aligned_to(phi_pre, 4) || !aligned_to(b_pre, 4) ||
      (w_router && !aligned_to(w_router, 4)) || (h_pre && !aligned_to(h_pre, 4)) ||
      (idx && !aligned_to(idx, 4)) || (score && !aligned_to(score, 4)))
    return HC_ERR_ALIGN;
  const int with_router = w_router != nullptr;
  const int64_t wsb = xhc_pre_ws(T, N, C, m, with_router, dtype);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int64_t xb = T * N * C * (int64_t)es, fb = T * C * (int64_t)es;
  const void* outs[4] = {F_in, h_pre, with_router ? idx : nullptr, with_router ? score : nullptr};
  const int64_t ob[4] = {fb, T * N * 4, T * k * 4, T * (N - m) * 4};
  const void* ins[5] = {X, phi_pre, b_pre, w_router, workspace};
  const int64_t ib[5] = {xb, (int64_t)N * C * N * 4, N * 4, (int64_t)N * C * (N - m) * 4, wsb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], ob[i], ins[j], ib[j])) return HC_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return HC_ERR_ALIAS;
  }
  int s = device_status();
  if (s != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* p = (char*)workspace;
  const int pcols = N + (with_router ? N - m : 0);
  float* P = (float*)p;
  p += align256(T * pcols * 4);
  float* ss = (float*)p;
  p += align256(T * 4);
  float* hp = h_pre ? h_pre : (float*)p;
  p += align256(T * N * 4);
  hipError_t e;
  const hc::XhcFastWs f = hc::xhc_pre_fast_ws(T, N, C, m, with_router, dtype);
  if (f.packed > 0 && aligned_to(X, 16) && aligned_to(F_in, 16)) {
    void* packed = p;
    float* partial = (float*)(p + align256(f.packed));
    e = hc::launch_fast_xhc_full(X, T, N, C, k, m, phi_pre, b_pre, alpha_pre, w_router, hp, score, idx, F_in,
                                 packed, partial, st);
    return launch_status(e);
  } else {
    e = hc::launch_proj_generic(dtype, X, (int64_t)N * C, T, C, N, nullptr, N, phi_pre, N, w_router,
                                with_router ? N - m : 0, P, ss, st);
    if (e != hipSuccess) return HC_ERR_LAUNCH;
    e = hc::launch_xhc_select(P, pcols, 0, N, ss, (float)((double)N * (double)C), T, N, k, m, alpha_pre,
                              b_pre, hp, with_router ? score : nullptr, with_router ? idx : nullptr, st);
  }
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  return launch_status(hc::launch_pre_generic(dtype, vec_ok(C, {X, F_in}), X, T, N, C, hp, F_in, st));
}

// xhc_route workspace: projection rows P [T, k*K + k*k], ss [T], H_post, H_res, and
// with the router its rows and ss; then the fast paths' packed phi and per-item
// partials (the router pass and the active pass run one after the other and
// share them).
static hc::XhcFastWs xhc_route_fast(int64_t T, int N, int64_t C, int k, int m, int K, int with_router,
                                    int dtype) {
  hc::XhcFastWs f = hc::xhc_route_fast_ws(T, C, k, K, dtype);
  if (with_router) {
    const hc::XhcFastWs r = hc::xhc_router_fast_ws(T, N, C, m, dtype);
    f.packed = f.packed > r.packed ? f.packed : r.packed;
    f.partial = f.partial > r.partial ? f.partial : r.partial;
  }
  return f;
}

static int64_t xhc_route_ws(int64_t T, int N, int64_t C, int k, int m, int K, int with_router, int dtype) {
  const int acols = k * K + k * k;
  int64_t b = align256(T * acols * 4) + align256(T * 4) + align256(T * k * K * 4) + align256(T * k * k * 4);
  if (with_router) b += align256(T * (N - m) * 4) + align256(T * 4);
  const hc::XhcFastWs f = xhc_route_fast(T, N, C, k, m, K, with_router, dtype);
  return b + align256(f.packed) + align256(f.partial);
}

int64_t xhc_route_workspace_bytes(int64_t T, int N, int64_t C, int k, int m, int K, int with_router,
                                  int dtype) {
  if (T < 0 || N < 1 || N > HC_MAX_STREAMS || m < 1 || k < m || k > N || k > HC_MAX_ACTIVE || K < 1 ||
      K > HC_MAX_COMPONENTS || C < 1 || !dtype_ok(dtype))
    return -1;
  return xhc_route_ws(T, N, C, k, m, K, with_router, dtype);
}

int xhc_route(void* X, int dtype, int64_t T, int N, int64_t C, int k, int m, const float* w_router,
              const int32_t* idx_in, const float* phi_act, const float* b_act, float alpha_post,
              float alpha_res, int sinkhorn_iters, const void* Wb, int K, int32_t* idx_out,
              float* score_out, float* h_post_out, float* h_res_out, void* workspace,
              int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (T < 0 || C < 1 || C > (1ll << 26) || N < 1 || N > HC_MAX_STREAMS || m < 1 || k < m || k > N ||
      k > HC_MAX_ACTIVE || K < 1 || K > HC_MAX_COMPONENTS || sinkhorn_iters < 1 ||
      sinkhorn_iters > HC_MAX_ITERS)
    return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!X || !phi_act || !b_act || !Wb || !idx_out) return HC_ERR_NULL;
  if (!idx_in && !w_router) return HC_ERR_NULL;
  const size_t es = esize(dtype);
  if (!aligned_to(X, es) || !aligned_to(Wb, es) || !aligned_to(phi_act, 4) || !aligned_to(b_act, 4) ||
      !aligned_to(idx_out, 4) || (idx_in && !aligned_to(idx_in, 4)) ||
      (w_router && !aligned_to(w_router, 4)) || (score_out && !aligned_to(score_out, 4)) ||
      (h_post_out && !aligned_to(h_post_out, 4)) || (h_res_out && !aligned_to(h_res_out, 4)))
    return HC_ERR_ALIGN;
  const int with_router = idx_in == nullptr;
  const int64_t wsb = xhc_route_ws(T, N, C, k, m, K, with_router, dtype);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int acols = k * K + k * k;
  const int64_t xb = T * N * C * (int64_t)es;
  // X is updated in place; the other outputs must not overlap anything.
  const void* outs[5] = {X, idx_out, with_router ? score_out : nullptr, h_post_out, h_res_out};
  const int64_t ob[5] = {xb, T * k * 4, T * (N - m) * 4, T * k * K * 4, T * k * k * 4};
  const void* ins[6] = {Wb, phi_act, b_act, w_router, idx_in, workspace};
  const int64_t ib[6] = {T * K * C * (int64_t)es, (int64_t)k * C * acols * 4, acols * 4,
                         w_router ? (int64_t)N * C * (N - m) * 4 : 0, T * k * 4, wsb};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 6; ++j) {
      if (i == 1 && j == 4 && outs[i] == ins[j]) continue;  // idx_out may equal idx_in
      if (overlaps(outs[i], ob[i], ins[j], ib[j])) return HC_ERR_ALIAS;
    }
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return HC_ERR_ALIAS;
  }
  int s = device_status();
  if (s != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* p = (char*)workspace;
  float* P = (float*)p;
  p += align256(T * acols * 4);
  float* ss = (float*)p;
  p += align256(T * 4);
  float* Hp = h_post_out ? h_post_out : (float*)p;
  p += align256(T * k * K * 4);
  float* Hr = h_res_out ? h_res_out : (float*)p;
  p += align256(T * k * k * 4);
  float* Pr = nullptr;
  float* ssf = nullptr;
  if (with_router) {
    Pr = (float*)p;
    p += align256(T * (N - m) * 4);
    ssf = (float*)p;
    p += align256(T * 4);
  }
  const hc::XhcFastWs fw = xhc_route_fast(T, N, C, k, m, K, with_router, dtype);
  void* packed = p;
  float* partial = (float*)(p + align256(fw.packed));
  const bool x16 = aligned_to(X, 16);
  hipError_t e;
  if (with_router) {
    if (x16 && hc::xhc_router_fast_ws(T, N, C, m, dtype).packed > 0) {
      e = hc::launch_fast_xhc_full(X, T, N, C, k, m, nullptr, nullptr, 0.f, w_router, nullptr, score_out, idx_out,
                                   nullptr, packed, partial, st);
    } else {
      e = hc::launch_proj_generic(dtype, X, (int64_t)N * C, T, C, N, nullptr, N, w_router, N - m, nullptr, 0,
                                  Pr, ssf, st);
      if (e != hipSuccess) return HC_ERR_LAUNCH;
      e = hc::launch_xhc_select(Pr, N - m, 0, 0, ssf, (float)((double)N * (double)C), T, N, k, m, 0.f,
                                nullptr, nullptr, score_out, idx_out, st);
    }
    if (e != hipSuccess) return HC_ERR_LAUNCH;
  } else if (idx_out != idx_in) {
    e = hipMemcpyAsync(idx_out, idx_in, (size_t)(T * k * 4), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return HC_ERR_LAUNCH;
  }
  if (x16 && hc::xhc_route_fast_ws(T, C, k, K, dtype).packed > 0) {
    e = hc::launch_fast_xhc_active(X, T, N, C, idx_out, K, phi_act, b_act, alpha_post, alpha_res, sinkhorn_iters,
                                   Hp, Hr, packed, partial, st, nullptr, K > 1);
  } else {
    e = hc::launch_proj_generic(dtype, X, (int64_t)N * C, T, C, k, idx_out, N, phi_act, acols, nullptr, 0,
                                P, ss, st);
    if (e != hipSuccess) return HC_ERR_LAUNCH;
    e = hc::launch_coeff_epilogue(P, ss, (float)((double)k * (double)C), T, 0, k * K, k, 0.f, alpha_post,
                                  alpha_res, b_act, sinkhorn_iters, nullptr, Hp, Hr, st);
  }
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  if (hc::fast_mix_supported(dtype, k, K, C, X, Wb))
    return launch_status(hc::launch_fast_mix(X, T, N, C, idx_out, Hr, Hp, Wb, K, st));
  return launch_status(hc::launch_mix_generic(dtype, vec_ok(C, {X, Wb}), X, T, N, C, k, idx_out, Hr, Hp,
                                              Wb, K, st));
}

// ------------------------------------------------------ xHC chained step

// Workspace of the chained calls: the packed maps (route, and each sublayer's
// full-state maps in turn), the partials (route, projection, pairs in turn),
// H_post, H_res, h_pre and score scratch, and the pair tables.
struct ChainWs {
  void* packed;
  float *partial, *Hp, *Hr, *hp, *sc;
  int32_t *ptok, *pos, *toff, *sortw;
};

static int64_t chain_ws(int64_t T, int N, int64_t C, int k, int m, int K, void* base, ChainWs* w) {
  const hc::XhcChainWs c = hc::xhc_chain_ws(T, N, C, k);
  const hc::XhcFastWs r = hc::xhc_route_fast_ws(T, C, k, K, HC_BF16);
  const hc::XhcFastWs f = hc::xhc_pre_fast_ws(T, N, C, m, true, HC_BF16);
  int64_t pk = c.packed, pt = c.pair_part;
  pk = r.packed > pk ? r.packed : pk;
  pk = f.packed > pk ? f.packed : pk;
  pt = r.partial > pt ? r.partial : pt;
  pt = f.partial > pt ? f.partial : pt;
  const int64_t sz[10] = {pk, pt, T * k * K * 4, T * k * k * 4, T * N * 4, T * (N - m) * 4, c.ptok, c.pos,
                          c.tile_off, c.sort};
  char* p = (char*)base;
  int64_t off = 0;
  void* ptrs[10];
  for (int i = 0; i < 10; ++i) {
    ptrs[i] = p ? p + off : nullptr;
    off += align256(sz[i]);
  }
  if (w) {
    w->packed = ptrs[0];
    w->partial = (float*)ptrs[1];
    w->Hp = (float*)ptrs[2];
    w->Hr = (float*)ptrs[3];
    w->hp = (float*)ptrs[4];
    w->sc = (float*)ptrs[5];
    w->ptok = (int32_t*)ptrs[6];
    w->pos = (int32_t*)ptrs[7];
    w->toff = (int32_t*)ptrs[8];
    w->sortw = (int32_t*)ptrs[9];
  }
  return off;
}

int64_t xhc_chain_carry_bytes(int64_t T, int N, int64_t C, int k, int m, int dtype) {
  if (!dtype_ok(dtype) || !hc::xhc_chain_supported(dtype, T < 1 ? 1 : T, N, C, k, m)) return -1;
  return hc::xhc_chain_carry_bytes(T, N, C);
}

int64_t xhc_chain_workspace_bytes(int64_t T, int N, int64_t C, int k, int m, int K, int dtype) {
  if (!dtype_ok(dtype) || K < 1 || K > HC_MAX_COMPONENTS || !hc::xhc_chain_supported(dtype, T < 1 ? 1 : T, N, C, k, m))
    return -1;
  return chain_ws(T, N, C, k, m, K, nullptr, nullptr);
}

int xhc_pre_chain(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int m,
                  const float* phi_pre, const float* b_pre, float alpha_pre, const float* w_router,
                  const float* phi_pre_next, const float* w_router_next,
                  float* h_pre, void* F_in, int32_t* idx, float* score, void* carry_out,
                  void* workspace, int64_t workspace_bytes, void* stream) {
  if (dtype != HC_BF16) return HC_ERR_DTYPE;
  if (T < 0 || !hc::xhc_chain_supported(dtype, T < 1 ? 1 : T, N, C, k, m)) return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!X || !phi_pre || !b_pre || !w_router || !phi_pre_next || !w_router_next || !F_in || !idx || !carry_out)
    return HC_ERR_NULL;
  if (!aligned_to(X, 16) || !aligned_to(F_in, 16) || !aligned_to(idx, 16) || !aligned_to(carry_out, 256) ||
      !aligned_to(phi_pre, 4) || !aligned_to(b_pre, 4) || !aligned_to(w_router, 4) || !aligned_to(phi_pre_next, 4) ||
      !aligned_to(w_router_next, 4) || (h_pre && !aligned_to(h_pre, 16)) || (score && !aligned_to(score, 4)))
    return HC_ERR_ALIGN;
  const int64_t wsb = chain_ws(T, N, C, k, m, 1, nullptr, nullptr);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int64_t NC = (int64_t)N * C, xb = T * NC * 2, cb = hc::xhc_chain_carry_bytes(T, N, C);
  const void* outs[5] = {F_in, h_pre, idx, score, carry_out};
  const int64_t ob[5] = {T * C * 2, T * N * 4, T * k * 4, T * (N - m) * 4, cb};
  const void* ins[7] = {X, phi_pre, b_pre, w_router, phi_pre_next, w_router_next, workspace};
  const int64_t ib[7] = {xb, NC * N * 4, N * 4, NC * (N - m) * 4, NC * N * 4, NC * (N - m) * 4, wsb};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], ob[i], ins[j], ib[j])) return HC_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return HC_ERR_ALIAS;
  }
  int s = device_status();
  if (s != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  ChainWs w;
  chain_ws(T, N, C, k, m, 1, workspace, &w);
  float* hp = h_pre ? h_pre : w.hp;
  float* sc = score ? score : w.sc;
  hipError_t e = hc::launch_fast_xhc_full(X, T, N, C, k, m, phi_pre, b_pre, alpha_pre, w_router, hp, sc, idx,
                                          nullptr, w.packed, w.partial, st);
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  // the next sublayer's maps, packed into the carry beside the partials the pre-read forms
  void* cpk = (char*)carry_out + hc::xhc_chain_carry_part_bytes(T, N, C);
  if ((e = hc::launch_fast_xhc_pack_full(phi_pre_next, w_router_next, N, m, C, cpk, st)) != hipSuccess)
    return HC_ERR_LAUNCH;
  return launch_status(hc::launch_fast_xhc_dense(X, T, N, C, hp, idx, cpk, F_in, (float*)carry_out, st));
}

int xhc_route_pre(void* X, int dtype, int64_t T, int N, int64_t C, int k, int m,
                  const int32_t* idx_in, const float* phi_act, const float* b_act, float alpha_post,
                  float alpha_res, int sinkhorn_iters, const void* Wb, int K,
                  const float* b_pre, float alpha_pre, const void* carry_in,
                  const float* phi_pre_next, const float* w_router_next, void* carry_out,
                  float* h_post_out, float* h_res_out, int32_t* idx_out, float* score_out, float* h_pre_out,
                  void* F_in, void* workspace, int64_t workspace_bytes, void* stream) {
  if (dtype != HC_BF16) return HC_ERR_DTYPE;
  if (T < 0 || K < 1 || K > HC_MAX_COMPONENTS || sinkhorn_iters < 1 || sinkhorn_iters > HC_MAX_ITERS ||
      !hc::xhc_chain_supported(dtype, T < 1 ? 1 : T, N, C, k, m) || hc::xhc_route_fast_ws(T < 1 ? 1 : T, C, k, K, dtype).packed == 0)
    return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  const bool next = phi_pre_next || w_router_next || carry_out;
  if (!X || !idx_in || !phi_act || !b_act || !Wb || !b_pre || !carry_in || !idx_out || !F_in ||
      (next && (!phi_pre_next || !w_router_next || !carry_out)))
    return HC_ERR_NULL;
  if (!aligned_to(X, 16) || !aligned_to(Wb, 16) || !aligned_to(F_in, 16) || !aligned_to(idx_in, 16) ||
      !aligned_to(idx_out, 16) || !aligned_to(carry_in, 256) || (carry_out && !aligned_to(carry_out, 256)) ||
      !aligned_to(phi_act, 4) || !aligned_to(b_act, 4) || !aligned_to(b_pre, 4) ||
      (phi_pre_next && !aligned_to(phi_pre_next, 4)) ||
      (w_router_next && !aligned_to(w_router_next, 4)) || (h_post_out && !aligned_to(h_post_out, 4)) ||
      (h_res_out && !aligned_to(h_res_out, 4)) || (score_out && !aligned_to(score_out, 4)) ||
      (h_pre_out && !aligned_to(h_pre_out, 16)))
    return HC_ERR_ALIGN;
  const int64_t wsb = chain_ws(T, N, C, k, m, K, nullptr, nullptr);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int acols = k * K + k * k;
  const int64_t NC = (int64_t)N * C, xb = T * NC * 2, cb = hc::xhc_chain_carry_bytes(T, N, C);
  // X is updated in place; carry_out may be carry_in and idx_out may be idx_in.
  const void* outs[8] = {X, carry_out, h_post_out, h_res_out, idx_out, score_out, h_pre_out, F_in};
  const int64_t ob[8] = {xb, cb, T * k * K * 4, T * k * k * 4, T * k * 4, T * (N - m) * 4, T * N * 4, T * C * 2};
  const void* ins[9] = {idx_in, phi_act, b_act, Wb, b_pre, carry_in, phi_pre_next, w_router_next, workspace};
  const int64_t ib[9] = {T * k * 4, (int64_t)k * C * acols * 4, acols * 4, T * K * C * 2, N * 4, cb,
                         NC * N * 4, NC * (N - m) * 4, wsb};
  for (int i = 0; i < 8; ++i) {
    for (int j = 0; j < 9; ++j) {
      if (i == 1 && j == 5 && outs[i] == ins[j]) continue;  // carry_out == carry_in
      if (i == 4 && j == 0 && outs[i] == ins[j]) continue;  // idx_out == idx_in
      if (overlaps(outs[i], ob[i], ins[j], ib[j])) return HC_ERR_ALIAS;
    }
    for (int j = 0; j < i; ++j)
      if (overlaps(outs[i], ob[i], outs[j], ob[j])) return HC_ERR_ALIAS;
  }
  int s = device_status();
  if (s != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  ChainWs w;
  chain_ws(T, N, C, k, m, K, workspace, &w);
  float* Hp = h_post_out ? h_post_out : w.Hp;
  float* Hr = h_res_out ? h_res_out : w.Hr;
  float* hp = h_pre_out ? h_pre_out : w.hp;
  float* sc = score_out ? score_out : w.sc;
  // route l: the active set's maps from its rows, then the mix in place
  hipError_t e = hc::launch_fast_xhc_active(X, T, N, C, idx_in, K, phi_act, b_act, alpha_post, alpha_res,
                                            sinkhorn_iters, Hp, Hr, w.packed, w.partial, st, nullptr, K > 1);
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  if ((e = hc::launch_fast_mix(X, T, N, C, idx_in, Hr, Hp, Wb, K, st)) != hipSuccess) return HC_ERR_LAUNCH;
  // sublayer l + 1's maps (packed in the carry): the carry's partials plus the rewritten rows
  const int64_t cpb = hc::xhc_chain_carry_part_bytes(T, N, C);
  const void* pk1 = (const char*)carry_in + cpb;
  if ((e = hc::launch_fast_xhc_chain_maps(X, T, N, C, k, m, idx_in, pk1, (const float*)carry_in, b_pre,
                                          alpha_pre, hp, sc, idx_out, w.ptok, w.toff, w.pos, w.sortw, w.partial,
                                          st)) !=
      hipSuccess)
    return HC_ERR_LAUNCH;
  if (!next) return launch_status(hc::launch_fast_pre_wide(X, T, N, C, hp, F_in, st));
  // the pre-read of sublayer l + 1, which also forms the carry of sublayer l + 2 (its maps
  // packed first; in place, after the rewritten rows' pass has read the carried ones)
  void* pk2 = (char*)carry_out + cpb;
  if ((e = hc::launch_fast_xhc_pack_full(phi_pre_next, w_router_next, N, m, C, pk2, st)) != hipSuccess)
    return HC_ERR_LAUNCH;
  return launch_status(hc::launch_fast_xhc_dense(X, T, N, C, hp, idx_out, pk2, F_in, (float*)carry_out, st));
}

// ---------------------------------------------------------------- xHC-Flash

// xhc_flash_pre workspace: xhc_pre's (one pass per pre map), a score scratch, and
// the one-pass block entry's packed phi and partials (L >= 2 on the fast path).
static int64_t flash_pre_ws(int64_t T, int N, int64_t C, int m, int L, int dtype) {
  const hc::XhcFastWs f = hc::flash_entry_fast_ws(T, N, C, m, L, dtype);
  return xhc_pre_ws(T, N, C, m, 1, dtype) + align256(T * (N - m) * 4) + align256(f.packed) + align256(f.partial);
}

int64_t xhc_flash_pre_workspace_bytes(int64_t T, int N, int64_t C, int m, int L, int dtype) {
  if (T < 0 || N < 2 || N > HC_MAX_STREAMS || m < 1 || m >= N || C < 1 || L < 1 || L > HC_MAX_FLASH_SUBLAYERS ||
      !dtype_ok(dtype))
    return -1;
  return flash_pre_ws(T, N, C, m, L, dtype);
}

int xhc_flash_pre(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int m, int L, const float* phi_pre,
                  const float* b_pre, float alpha_pre, const float* w_router, int32_t* idx, float* score,
                  float* h_pre, void* F_pre, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (T < 0 || C < 1 || C > (1ll << 26) || N < 2 || N > HC_MAX_STREAMS || m < 1 || k < m || k > N ||
      m >= N || k > HC_MAX_ACTIVE || L < 1 || L > HC_MAX_FLASH_SUBLAYERS)
    return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if (!X || !phi_pre || !b_pre || !w_router || !idx || !h_pre || !F_pre) return HC_ERR_NULL;
  const size_t es = esize(dtype);
  if (!aligned_to(X, es) || !aligned_to(F_pre, es) || !aligned_to(phi_pre, 4) || !aligned_to(b_pre, 4) ||
      !aligned_to(w_router, 4) || !aligned_to(h_pre, 4) || !aligned_to(idx, 4) || (score && !aligned_to(score, 4)))
    return HC_ERR_ALIGN;
  const int64_t wsb = flash_pre_ws(T, N, C, m, L, dtype);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int64_t NC = (int64_t)N * C;
  const void* outs[4] = {F_pre, h_pre, idx, score};
  const int64_t ob[4] = {L * T * C * (int64_t)es, L * T * N * 4, T * k * 4, T * (N - m) * 4};
  const void* ins[5] = {X, phi_pre, b_pre, w_router, workspace};
  const int64_t ib[5] = {T * NC * (int64_t)es, L * NC * N * 4, (int64_t)L * N * 4, NC * (N - m) * 4, wsb};
  if (any_overlap(outs, ob, 4, ins, ib, 5)) return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* p = (char*)workspace;
  const int pcols = N + (N - m);
  float* P = (float*)p;
  p += align256(T * pcols * 4);
  float* ss = (float*)p;
  p += align256(T * 4);
  p += align256(T * N * 4);  // (xhc_pre's h_pre scratch; h_pre is an output here)
  const hc::XhcFastWs f = hc::xhc_pre_fast_ws(T, N, C, m, 1, dtype);
  void* packed = p;
  float* partial = (float*)(p + align256(f.packed));
  p += align256(f.packed) + align256(f.partial);
  float* sc = score ? score : (float*)p;
  p += align256(T * (N - m) * 4);
  const bool fast = f.packed > 0 && aligned_to(X, 16);
  const hc::XhcFastWs fe = hc::flash_entry_fast_ws(T, N, C, m, L, dtype);
  hipError_t e = hipSuccess;
  // the router and all L pre maps from one projection pass over the entry state,
  // else sublayer l's pre map from its own phi_pre^(l), b_pre^(l) (the router with the first)
  const bool one_pass = fe.packed > 0 && aligned_to(X, 16);
  if (one_pass)
    e = hc::launch_fast_flash_entry(X, T, N, C, k, m, L, phi_pre, b_pre, alpha_pre, w_router, h_pre, sc, idx, p,
                                    (float*)(p + align256(fe.packed)), st);
  for (int l = 0; l < (one_pass ? 0 : L) && e == hipSuccess; ++l) {
    const float* phl = phi_pre + (int64_t)l * NC * N;
    const float* bl = b_pre + (int64_t)l * N;
    float* hl = h_pre + (int64_t)l * T * N;
    const float* wr = l == 0 ? w_router : nullptr;
    if (fast) {
      e = hc::launch_fast_xhc_full(X, T, N, C, k, m, phl, bl, alpha_pre, wr, hl, l == 0 ? sc : nullptr,
                                   l == 0 ? idx : nullptr, nullptr, packed, partial, st);
    } else {
      e = hc::launch_proj_generic(dtype, X, NC, T, C, N, nullptr, N, phl, N, wr, wr ? N - m : 0, P, ss, st);
      if (e == hipSuccess)
        e = hc::launch_xhc_select(P, wr ? pcols : N, 0, N, ss, (float)((double)N * (double)C), T, N, k, m,
                                  alpha_pre, bl, hl, wr ? sc : nullptr, wr ? idx : nullptr, st);
    }
  }
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  // the L dense reads of the entry state
  if (hc::fast_pre_multi_supported(dtype, N, C, L, X, F_pre))
    return launch_status(hc::launch_fast_pre_multi(X, T, N, C, L, h_pre, F_pre, st));
  for (int l = 0; l < L; ++l) {
    void* Fl = (char*)F_pre + (int64_t)l * T * C * (int64_t)es;
    e = hc::launch_pre_generic(dtype, vec_ok(C, {X, Fl}), X, T, N, C, h_pre + (int64_t)l * T * N, Fl, st);
    if (e != hipSuccess) return HC_ERR_LAUNCH;
  }
  return HC_OK;
}

// write-back components of a block: L - 1 earlier outputs and the last sublayer's K_last
static bool flash_components_ok(int L, int K_last) {
  return L >= 1 && L <= HC_MAX_FLASH_SUBLAYERS && K_last >= 1 && L - 1 + K_last <= HC_MAX_COMPONENTS;
}

static int64_t flash_maps_ws(int64_t T, int64_t C, int k, int Kb, int dtype) {
  const hc::XhcFastWs f = hc::xhc_route_fast_ws(T, C, k, Kb, dtype);
  return align256(T * (k * Kb + k * k) * 4) + align256(T * 4) + align256(f.packed) + align256(f.partial);
}

int64_t xhc_flash_maps_workspace_bytes(int64_t T, int N, int64_t C, int k, int L, int K_last, int dtype) {
  if (T < 0 || N < 1 || N > HC_MAX_STREAMS || k < 1 || k > N || k > HC_MAX_ACTIVE || C < 1 ||
      !flash_components_ok(L, K_last) || !dtype_ok(dtype))
    return -1;
  return flash_maps_ws(T, C, k, L - 1 + K_last, dtype);
}

int xhc_flash_maps(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int L, int K_last,
                   const int32_t* idx, const float* phi_act, const float* b_act, float alpha_post, float alpha_res,
                   int sinkhorn_iters, float* H_post, float* H_res, void* workspace, int64_t workspace_bytes,
                   void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (T < 0 || C < 1 || C > (1ll << 26) || N < 1 || N > HC_MAX_STREAMS || k < 1 || k > N || k > HC_MAX_ACTIVE ||
      !flash_components_ok(L, K_last) || sinkhorn_iters < 1 || sinkhorn_iters > HC_MAX_ITERS)
    return HC_ERR_SHAPE;
  L = L - 1 + K_last;  // from here on: the write-back columns Kb
  if (T == 0) return HC_OK;
  if (!X || !idx || !phi_act || !b_act || !H_post || !H_res) return HC_ERR_NULL;
  if (!aligned_to(X, esize(dtype)) || !aligned_to(idx, 4) || !aligned_to(phi_act, 4) || !aligned_to(b_act, 4) ||
      !aligned_to(H_post, 4) || !aligned_to(H_res, 4))
    return HC_ERR_ALIGN;
  const int64_t wsb = flash_maps_ws(T, C, k, L, dtype);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const int acols = k * L + k * k;
  const void* outs[2] = {H_post, H_res};
  const int64_t ob[2] = {T * k * L * 4, T * k * k * 4};
  const void* ins[5] = {X, idx, phi_act, b_act, workspace};
  const int64_t ib[5] = {T * N * C * (int64_t)esize(dtype), T * k * 4, (int64_t)k * C * acols * 4, acols * 4, wsb};
  if (any_overlap(outs, ob, 2, ins, ib, 5)) return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  char* p = (char*)workspace;
  float* P = (float*)p;
  p += align256(T * acols * 4);
  float* ss = (float*)p;
  p += align256(T * 4);
  const hc::XhcFastWs f = hc::xhc_route_fast_ws(T, C, k, L, dtype);
  void* packed = p;
  float* partial = (float*)(p + align256(f.packed));
  hipError_t e;
  if (aligned_to(X, 16) && f.packed > 0) {
    e = hc::launch_fast_xhc_active(X, T, N, C, idx, L, phi_act, b_act, alpha_post, alpha_res, sinkhorn_iters,
                                   H_post, H_res, packed, partial, st, nullptr, L > 1);
  } else {
    e = hc::launch_proj_generic(dtype, X, (int64_t)N * C, T, C, k, idx, N, phi_act, acols, nullptr, 0, P, ss, st);
    if (e != hipSuccess) return HC_ERR_LAUNCH;
    e = hc::launch_coeff_epilogue(P, ss, (float)((double)k * (double)C), T, 0, k * L, k, 0.f, alpha_post,
                                  alpha_res, b_act, sinkhorn_iters, nullptr, H_post, H_res, st);
  }
  return launch_status(e);
}

int xhc_flash_input(int dtype, int64_t T, int N, int64_t C, int k, int L, int K_last, int l, const void* F_pre_l,
                    const float* h_pre_l, const int32_t* idx, const float* H_post, const void* F_outs, void* F_in,
                    void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (T < 0 || C < 1 || C > (1ll << 26) || N < 1 || N > HC_MAX_STREAMS || k < 1 || k > N || k > HC_MAX_ACTIVE ||
      !flash_components_ok(L, K_last) || l < 0 || l >= L)
    return HC_ERR_SHAPE;
  L = L - 1 + K_last;  // H_post's and F_outs' row length Kb (only components j < l are read)
  if (T == 0) return HC_OK;
  if (!F_pre_l || !h_pre_l || !idx || !H_post || !F_in || (l > 0 && !F_outs)) return HC_ERR_NULL;
  const size_t es = esize(dtype);
  if (!aligned_to(F_pre_l, es) || !aligned_to(F_in, es) || (F_outs && !aligned_to(F_outs, es)) ||
      !aligned_to(h_pre_l, 4) || !aligned_to(idx, 4) || !aligned_to(H_post, 4))
    return HC_ERR_ALIGN;
  const int64_t fb = T * C * (int64_t)es;
  // F_in may be F_pre_l itself (each element is read before it is written); no other overlap
  const void* outs[1] = {F_in};
  const int64_t ob[1] = {fb};
  const void* ins[5] = {F_in == F_pre_l ? nullptr : F_pre_l, h_pre_l, idx, H_post, l > 0 ? F_outs : nullptr};
  const int64_t ib[5] = {fb, T * N * 4, T * k * 4, T * k * L * 4, T * L * C * (int64_t)es};
  if (any_overlap(outs, ob, 1, ins, ib, 5)) return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  return launch_status(hc::launch_flash_input(dtype, vec_ok(C, {F_pre_l, F_outs, F_in}), T, N, C, k, L, l, F_pre_l,
                                              h_pre_l, idx, H_post, F_outs, F_in, (hipStream_t)stream));
}

int64_t xhc_flash_post_workspace_bytes(int64_t T, int k, int L, int K_last) {
  if (T < 0 || k < 1 || k > HC_MAX_ACTIVE || !flash_components_ok(L, K_last)) return -1;
  return align256(T * k * (L - 1 + K_last) * 4);
}

int xhc_flash_post(void* X, int dtype, int64_t T, int N, int64_t C, int k, int L, int K_last, const int32_t* idx,
                   const float* H_post, const float* H_res, const void* F_outs, const void* W_last, void* workspace,
                   int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return HC_ERR_DTYPE;
  if (T < 0 || C < 1 || C > (1ll << 26) || N < 1 || N > HC_MAX_STREAMS || k < 1 || k > N || k > HC_MAX_ACTIVE ||
      !flash_components_ok(L, K_last))
    return HC_ERR_SHAPE;
  const int Lsub = L;
  L = L - 1 + K_last;  // from here on: the write-back components Kb
  if (T == 0) return HC_OK;
  if (!X || !idx || !H_post || !H_res || !F_outs) return HC_ERR_NULL;
  const size_t es = esize(dtype);
  if (!aligned_to(X, es) || !aligned_to(F_outs, es) || (W_last && !aligned_to(W_last, es)) || !aligned_to(idx, 4) ||
      !aligned_to(H_post, 4) || !aligned_to(H_res, 4))
    return HC_ERR_ALIGN;
  const int64_t wsb = align256(T * k * L * 4);
  if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
  const void* outs[2] = {X, workspace};
  const int64_t ob[2] = {T * N * C * (int64_t)es, wsb};
  const void* ins[5] = {idx, H_post, H_res, F_outs, W_last};
  const int64_t ib[5] = {T * k * 4, T * k * L * 4, T * k * k * 4, T * L * C * (int64_t)es,
                         T * K_last * C * (int64_t)es};
  if (any_overlap(outs, ob, 2, ins, ib, 5)) return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  float* E = (float*)workspace;
  hipError_t e = hc::launch_flash_post_maps(T, k, Lsub, L, H_post, H_res, E, st);
  if (e != hipSuccess) return HC_ERR_LAUNCH;
  // the last sublayer's components from W_last when given (component rows Lsub - 1 ..)
  const int j0 = W_last ? Lsub - 1 : L;
  if (hc::fast_mix_supported(dtype, k, L, C, X, F_outs) && (!W_last || hc::fast_mix_supported(dtype, k, L, C, X, W_last)))
    return launch_status(hc::launch_fast_mix(X, T, N, C, idx, H_res, E, F_outs, L, st, W_last, j0));
  return launch_status(hc::launch_mix_generic(dtype, vec_ok(C, {X, F_outs, W_last}), X, T, N, C, k, idx, H_res, E,
                                              F_outs, L, st, W_last, j0));
}

static int augment_spec(int64_t B, int64_t S, int64_t C, const int* kappa, int r, hc::ConvSpec& spec,
                        int64_t& wtot) {
  if (B < 0 || S < 0 || C < 1 || C > (1ll << 26) || r < 0 || r > HC_MAX_COMPONENTS - 1) return HC_ERR_SHAPE;
  if (r > 0 && !kappa) return HC_ERR_NULL;
  wtot = 0;
  spec = hc::ConvSpec{};
  spec.r = r;
  for (int j = 0; j < r; ++j) {
    if (kappa[j] < 1 || kappa[j] > HC_MAX_KAPPA) return HC_ERR_SHAPE;
    spec.kappa[j] = kappa[j];
    spec.offset[j] = wtot;
    wtot += C * kappa[j];
  }
  return HC_OK;
}

static bool augment_fast_shape(int64_t C, const int* kappa, int r) {
  return r == 3 && kappa[0] == 4 && kappa[1] == 8 && kappa[2] == 12 && C % 4 == 0;
}

int64_t xhc_augment_workspace_bytes(int64_t B, int64_t S, int64_t C, const int* kappa, int r, int dtype,
                                    int v_dtype) {
  if (!dtype_ok(dtype) || !dtype_ok(v_dtype)) return -1;
  hc::ConvSpec spec;
  int64_t wtot;
  if (augment_spec(B, S, C, kappa, r, spec, wtot) != HC_OK) return -1;
  return augment_fast_shape(C, kappa, r) ? hc::fast_augment_workspace_bytes(B, S, C) : 0;
}

int xhc_augment(const void* F_out, int dtype, int64_t B, int64_t S, int64_t C, const float* conv_w,
                const int* kappa, int r, void* V, int v_dtype, void* workspace, int64_t workspace_bytes,
                void* stream) {
  if (!dtype_ok(dtype) || !dtype_ok(v_dtype)) return HC_ERR_DTYPE;
  hc::ConvSpec spec;
  int64_t wtot;
  int s = augment_spec(B, S, C, kappa, r, spec, wtot);
  if (s != HC_OK) return s;
  const bool fast_shape = augment_fast_shape(C, kappa, r);
  if (!fast_shape && hc::augment_generic_lds_bytes(r, C) > 160 * 1024 - 1024) return HC_ERR_SHAPE;
  const int64_t T = B * S;
  if (T == 0) return HC_OK;
  if (!F_out || !V || (r > 0 && !conv_w)) return HC_ERR_NULL;
  if (!aligned_to(F_out, esize(dtype)) || !aligned_to(V, esize(v_dtype)) || (conv_w && !aligned_to(conv_w, 4)))
    return HC_ERR_ALIGN;
  const int64_t vb = T * (r + 1) * C * (int64_t)esize(v_dtype);
  const int64_t fb = T * C * (int64_t)esize(dtype);
  if (overlaps(V, vb, F_out, fb) || overlaps(V, vb, conv_w, wtot * 4)) return HC_ERR_ALIAS;
  const int64_t wsb = fast_shape ? hc::fast_augment_workspace_bytes(B, S, C) : 0;
  if (wsb > 0) {
    if (!workspace || !aligned_to(workspace, 256) || workspace_bytes < wsb) return HC_ERR_WORKSPACE;
    if (overlaps(workspace, wsb, V, vb) || overlaps(workspace, wsb, F_out, fb) ||
        overlaps(workspace, wsb, conv_w, wtot * 4))
      return HC_ERR_ALIAS;
  }
  if ((s = device_status()) != HC_OK) return s;
  if (fast_shape && hc::fast_augment_supported(dtype, v_dtype, S, C, kappa, r, F_out, V))
    return launch_status(hc::launch_fast_augment(dtype, v_dtype, F_out, B, S, C, conv_w, V, (float*)workspace,
                                                 (hipStream_t)stream));
  if (hc::augment_generic_lds_bytes(r, C) > 160 * 1024 - 1024) return HC_ERR_SHAPE;
  return launch_status(hc::launch_augment_generic(dtype, v_dtype, F_out, B, S, C, conv_w, spec, V,
                                                  (hipStream_t)stream));
}

int hc_tanh_coeffs(const void* X, int dtype, int64_t T, int n, int64_t C, const float* theta,
                   const float* bias, float alpha_pre, float alpha_post, float alpha_res, float* h_pre,
                   float* h_post, float* h_res, void* stream) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK || T == 0) return s;
  if (!theta || !bias || !h_pre || !h_post || !h_res) return HC_ERR_NULL;
  for (const void* p : {(const void*)theta, (const void*)bias, (const void*)h_pre, (const void*)h_post,
                        (const void*)h_res})
    if (!aligned_to(p, 4)) return HC_ERR_ALIGN;
  const int64_t xb = T * n * C * (int64_t)esize(dtype), thb = (int64_t)(n + 2) * C * 4, bb = (n * n + 2 * n) * 4;
  const void* outs[3] = {h_pre, h_post, h_res};
  const int64_t ob[3] = {T * n * 4, T * n * 4, T * n * n * 4};
  for (int a = 0; a < 3; ++a) {
    if (overlaps(outs[a], ob[a], X, xb) || overlaps(outs[a], ob[a], theta, thb) || overlaps(outs[a], ob[a], bias, bb))
      return HC_ERR_ALIAS;
    for (int b = 0; b < a; ++b)
      if (overlaps(outs[a], ob[a], outs[b], ob[b])) return HC_ERR_ALIAS;
  }
  if ((s = device_status()) != HC_OK) return s;
  const bool vec = C % 8 == 0 && aligned_to(X, 16) && aligned_to(theta, 16);
  return launch_status(hc::launch_hc_tanh(dtype, vec, X, T, n, C, theta, bias, alpha_pre, alpha_post, alpha_res,
                                          h_pre, h_post, h_res, (hipStream_t)stream));
}

int hc_amax_gain(const float* h_res, int64_t L, int64_t T, int n, float* gain_fwd, float* gain_bwd, void* stream) {
  if (L < 0 || T < 0 || n < 1 || n > HC_MAX_MHC_STREAMS) return HC_ERR_SHAPE;
  if (T == 0) return HC_OK;
  if ((L > 0 && !h_res) || !gain_fwd || !gain_bwd) return HC_ERR_NULL;
  if (!aligned_to(h_res, 4) || !aligned_to(gain_fwd, 4) || !aligned_to(gain_bwd, 4)) return HC_ERR_ALIGN;
  const int64_t hb = L * T * n * n * 4;
  if (overlaps(gain_fwd, T * 4, gain_bwd, T * 4) || overlaps(gain_fwd, T * 4, h_res, hb) ||
      overlaps(gain_bwd, T * 4, h_res, hb))
    return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  return launch_status(hc::launch_amax_gain(h_res, L, T, n, gain_fwd, gain_bwd, (hipStream_t)stream));
}

int hc_static_maps(const float* logits, int n, int sinkhorn_iters, float* h_pre, float* h_post, float* h_res,
                   void* stream) {
  if (n < 1 || n > HC_MAX_MHC_STREAMS || sinkhorn_iters < 1 || sinkhorn_iters > HC_MAX_ITERS) return HC_ERR_SHAPE;
  if (!logits || !h_pre || !h_post || !h_res) return HC_ERR_NULL;
  for (const void* p : {(const void*)logits, (const void*)h_pre, (const void*)h_post, (const void*)h_res})
    if (!aligned_to(p, 4)) return HC_ERR_ALIGN;
  const void* outs[3] = {h_pre, h_post, h_res};
  const int64_t ob[3] = {(int64_t)n * 4, (int64_t)n * 4, (int64_t)n * n * 4};
  for (int a = 0; a < 3; ++a) {
    if (overlaps(outs[a], ob[a], logits, (int64_t)(n * n + 2 * n) * 4)) return HC_ERR_ALIAS;
    for (int b = 0; b < a; ++b)
      if (overlaps(outs[a], ob[a], outs[b], ob[b])) return HC_ERR_ALIAS;
  }
  int s = device_status();
  if (s != HC_OK) return s;
  return launch_status(hc::launch_static_maps(logits, n, sinkhorn_iters, h_pre, h_post, h_res, (hipStream_t)stream));
}

int hc_static_pre(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_pre, void* F_in,
                  void* stream) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK || T == 0) return s;
  if (!h_pre || !F_in) return HC_ERR_NULL;
  if (!aligned_to(h_pre, 4) || !aligned_to(F_in, esize(dtype))) return HC_ERR_ALIGN;
  const int64_t xb = T * n * C * (int64_t)esize(dtype), fb = T * C * (int64_t)esize(dtype);
  if (overlaps(F_in, fb, X, xb) || overlaps(F_in, fb, h_pre, (int64_t)n * 4)) return HC_ERR_ALIAS;
  if ((s = device_status()) != HC_OK) return s;
  return launch_status(hc::launch_static_apply(dtype, false, vec_ok(C, {X, F_in}), X, T, n, C, h_pre, nullptr,
                                               nullptr, F_in, (hipStream_t)stream));
}

int hc_static_post(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res, const float* h_post,
                   const void* F_out, void* X_next, void* stream) {
  int s = check_mhc_common(X, dtype, T, n, C);
  if (s != HC_OK || T == 0) return s;
  if (!h_res || !h_post || !F_out || !X_next) return HC_ERR_NULL;
  if (!aligned_to(h_res, 4) || !aligned_to(h_post, 4) || !aligned_to(F_out, esize(dtype)) ||
      !aligned_to(X_next, esize(dtype)))
    return HC_ERR_ALIGN;
  const int64_t xb = T * n * C * (int64_t)esize(dtype), fb = T * C * (int64_t)esize(dtype);
  if (X_next != X && overlaps(X_next, xb, X, xb)) return HC_ERR_ALIAS;
  if (overlaps(X_next, xb, F_out, fb) || overlaps(X_next, xb, h_res, (int64_t)n * n * 4) ||
      overlaps(X_next, xb, h_post, (int64_t)n * 4))
    return HC_ERR_ALIAS;
  if ((s = device_status()) != HC_OK) return s;
  return launch_status(hc::launch_static_apply(dtype, true, vec_ok(C, {X, F_out, X_next}), X, T, n, C, h_res, h_post,
                                               F_out, X_next, (hipStream_t)stream));
}

int hc_copy_probe(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0) return HC_ERR_SHAPE;
  if (bytes == 0) return HC_OK;
  if (!src || !dst) return HC_ERR_NULL;
  if (bytes % 16 != 0 || !aligned_to(src, 16) || !aligned_to(dst, 16)) return HC_ERR_ALIGN;
  if (overlaps(src, bytes, dst, bytes)) return HC_ERR_ALIAS;
  int s = device_status();
  if (s != HC_OK) return s;
  return launch_status(hc::launch_copy_probe(src, dst, bytes, (hipStream_t)stream));
}

}  // extern "C"
