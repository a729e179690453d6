"""Python binding of libhc, the gfx950 hyper-connection sublayer library.

Every function here has the name of a C entry point in include/hc.h and only
marshals arguments: it checks tensor devices/dtypes/contiguity, allocates the
outputs and the workspace with torch (device memory only), and calls the C ABI
with raw device pointers and the current HIP stream. All arithmetic runs in the
HIP kernels of libhc.so. If the library is missing, every call raises.

Stream tensors are torch.float32 or torch.bfloat16 on a HIP device; coefficient
tensors, phi, biases and conv weights are torch.float32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhc.so")

HC_F32, HC_BF16 = 0, 1
_DT = {torch.float32: HC_F32, torch.bfloat16: HC_BF16}

_c_i64, _c_int, _c_float, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p

_SIGS = {
    "hc_status_string": (ctypes.c_char_p, [_c_int]),
    "hc_version": (_c_int, []),
    "hc_coeffs_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int]),
    "hc_coeffs": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _c_float, _c_float, _c_float,
                           _c_int, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "hc_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp]),
    "hc_coeffs_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _c_float, _c_float,
                               _c_float, _c_int, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "hc_post": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "hc_backward_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int]),
    "hc_backward_post": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "hc_backward": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _c_float, _c_float, _c_float, _c_int,
                             _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "hc_post_coeffs": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _c_float,
                                _c_float, _c_float, _c_int, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "hc_phi_packed_bytes": (_c_i64, [_c_int, _c_i64, _c_int]),
    "hc_phi_pack": (_c_int, [_vp, _c_int, _c_i64, _c_int, _vp, _c_i64, _vp]),
    "hc_post_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_float,
                             _c_float, _c_float, _c_int, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_pre_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int]),
    "xhc_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _c_float, _vp,
                         _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_route_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int,
                                           _c_int]),
    "xhc_route": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _vp, _vp,
                           _c_float, _c_float, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_i64,
                           _vp]),
    "xhc_augment_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _vp, _c_int, _c_int, _c_int]),
    "xhc_flash_pre_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int]),
    "xhc_flash_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _vp, _vp, _c_float,
                               _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_flash_maps_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int]),
    "xhc_flash_maps": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _vp, _c_float,
                                _c_float, _c_int, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_flash_input": (_c_int, [_c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp]),
    "xhc_flash_post_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_int]),
    "xhc_flash_post": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp,
                                _c_i64, _vp]),
    "xhc_augment": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_i64, _vp]),
    "xhc_backward_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int]),
    "xhc_route_backward": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _vp, _vp, _vp, _c_float, _c_float,
                                    _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_pre_backward": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _c_float, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _c_i64, _vp]),
    "xhc_augment_backward_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _vp, _c_int, _c_int]),
    "xhc_augment_backward": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int, _vp, _vp, _vp, _vp,
                                      _c_i64, _vp]),
    "hc_copy_probe": (_c_int, [_vp, _vp, _c_i64, _vp]),
    "hc_tanh_coeffs": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _c_float, _c_float, _c_float,
                                _vp, _vp, _vp, _vp]),
    "hc_amax_gain": (_c_int, [_vp, _c_i64, _c_i64, _c_int, _vp, _vp, _vp]),
    "hc_static_maps": (_c_int, [_vp, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "hc_static_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp]),
    "hc_static_post": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp]),
}

_lib = None


class HCError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


def lib() -> ctypes.CDLL:
    """The loaded libhc.so with argument types set (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m stream_residual_mixing_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().hc_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise HCError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev_tensor(t, name, dtypes=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a tensor on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def _f32(t, name):
    return _dev_tensor(t, name, (torch.float32,))


def _workspace(nbytes: int, device, workspace):
    if nbytes < 0:
        raise ValueError("invalid sizes for the workspace query")
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------- mHC


def hc_coeffs_workspace_bytes(T: int, n: int, C: int, dtype) -> int:
    return int(lib().hc_coeffs_workspace_bytes(T, n, C, _DT[dtype]))


def hc_coeffs(X, phi, bias, alpha, sinkhorn_iters=20, *, out=None, workspace=None, stream=None):
    """(h_pre [T,n], h_post [T,n], h_res [T,n,n]) of X [T,n,C]; alpha = (pre, post, res)."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    phi, bias = _f32(phi, "phi"), _f32(bias, "bias")
    if out is None:
        out = (torch.empty(T, n, device=X.device), torch.empty(T, n, device=X.device),
               torch.empty(T, n, n, device=X.device))
    h_pre, h_post, h_res = out
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), X.device, workspace)
    a = [float(v) for v in alpha]
    _check("hc_coeffs", lib().hc_coeffs(_ptr(X), _DT[X.dtype], T, n, C, _ptr(phi), _ptr(bias), a[0], a[1],
                                        a[2], int(sinkhorn_iters), _ptr(h_pre), _ptr(h_post), _ptr(h_res),
                                        _ptr(ws), ws.numel(), _stream(X.device, stream)))
    return h_pre, h_post, h_res


def hc_pre(X, h_pre, *, out=None, stream=None):
    """F_in [T,C] = sum_i h_pre[:, i] X[:, i, :]."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    h_pre = _f32(h_pre, "h_pre")
    F_in = torch.empty(T, C, dtype=X.dtype, device=X.device) if out is None else out
    _check("hc_pre", lib().hc_pre(_ptr(X), _DT[X.dtype], T, n, C, _ptr(h_pre), _ptr(F_in),
                                  _stream(X.device, stream)))
    return F_in


def hc_coeffs_pre(X, phi, bias, alpha, sinkhorn_iters=20, *, out=None, workspace=None, stream=None,
                  want_h_pre=True):
    """Fused coefficients + pre-read: (h_pre or None, h_post, h_res, F_in)."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    phi, bias = _f32(phi, "phi"), _f32(bias, "bias")
    if out is None:
        out = (torch.empty(T, n, device=X.device) if want_h_pre else None,
               torch.empty(T, n, device=X.device), torch.empty(T, n, n, device=X.device),
               torch.empty(T, C, dtype=X.dtype, device=X.device))
    h_pre, h_post, h_res, F_in = out
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), X.device, workspace)
    a = [float(v) for v in alpha]
    _check("hc_coeffs_pre", lib().hc_coeffs_pre(_ptr(X), _DT[X.dtype], T, n, C, _ptr(phi), _ptr(bias), a[0],
                                                a[1], a[2], int(sinkhorn_iters), _ptr(h_pre), _ptr(h_post),
                                                _ptr(h_res), _ptr(F_in), _ptr(ws), ws.numel(),
                                                _stream(X.device, stream)))
    return h_pre, h_post, h_res, F_in


def hc_post(X, h_res, h_post, F_out, *, out=None, stream=None):
    """X_next [T,n,C] = h_res @ X + h_post^T F_out (out may be X itself)."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,))
    X_next = torch.empty_like(X) if out is None else out
    _check("hc_post", lib().hc_post(_ptr(X), _DT[X.dtype], T, n, C, _ptr(_f32(h_res, "h_res")),
                                    _ptr(_f32(h_post, "h_post")), _ptr(F_out), _ptr(X_next),
                                    _stream(X.device, stream)))
    return X_next


def hc_backward_workspace_bytes(T: int, n: int, C: int, dtype) -> int:
    return int(lib().hc_backward_workspace_bytes(T, n, C, _DT[dtype]))


def hc_backward_post(X, h_post, F_out, dX_next, *, out=None, stream=None):
    """Backward, post stage (n = 4, bfloat16): (dF_out, dh) with dF_out = H_post dX_next
    and dh [T, 24] float32 holding dH_post (columns 4..7) and dH_res (8..23)."""
    X = _dev_tensor(X, "X", (torch.bfloat16,))
    T, n, C = X.shape
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,))
    dX_next = _dev_tensor(dX_next, "dX_next", (X.dtype,))
    if out is None:
        out = (torch.empty(T, C, dtype=X.dtype, device=X.device), torch.empty(T, n * n + 2 * n, device=X.device))
    dF_out, dh = out
    _check("hc_backward_post", lib().hc_backward_post(_ptr(X), _DT[X.dtype], T, n, C, _ptr(_f32(h_post, "h_post")),
                                                      _ptr(F_out), _ptr(dX_next), _ptr(dF_out),
                                                      _ptr(_f32(dh, "dh")), _stream(X.device, stream)))
    return dF_out, dh


def hc_backward(X, phi, bias, alpha, dX_next, dF_in, dh, sinkhorn_iters=20, *, out=None, workspace=None,
                stream=None):
    """Backward, main stage (n = 4, bfloat16): fills dh[:, 0:4] (dH_pre), reads the rest of
    dh from hc_backward_post, returns (dX, dphi, dbias, dalpha)."""
    X = _dev_tensor(X, "X", (torch.bfloat16,))
    T, n, C = X.shape
    dX_next = _dev_tensor(dX_next, "dX_next", (X.dtype,))
    dF_in = _dev_tensor(dF_in, "dF_in", (X.dtype,))
    phi, bias, dh = _f32(phi, "phi"), _f32(bias, "bias"), _f32(dh, "dh")
    if out is None:
        dev = X.device
        out = (torch.empty_like(X), torch.empty(n * C, n * n + 2 * n, device=dev),
               torch.empty(n * n + 2 * n, device=dev), torch.empty(3, device=dev))
    dX, dphi, dbias, dalpha = out
    ws = _workspace(hc_backward_workspace_bytes(T, n, C, X.dtype), X.device, workspace)
    a = [float(v) for v in alpha]
    _check("hc_backward", lib().hc_backward(_ptr(X), _DT[X.dtype], T, n, C, _ptr(phi), _ptr(bias), a[0], a[1], a[2],
                                            int(sinkhorn_iters), _ptr(dX_next), _ptr(dF_in), _ptr(dh), _ptr(dX),
                                            _ptr(dphi), _ptr(dbias), _ptr(dalpha), _ptr(ws), ws.numel(),
                                            _stream(X.device, stream)))
    return dX, dphi, dbias, dalpha


def hc_post_coeffs(X, h_res, h_post, F_out, phi_next, bias_next, alpha_next, sinkhorn_iters=20, *, out=None,
                   coeffs_out=None, workspace=None, stream=None):
    """X_next = h_res @ X + h_post^T F_out, plus the coefficients of X_next under the next
    sublayer's phi/bias/alpha. Returns (X_next, (h_pre', h_post', h_res'))."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,))
    X_next = torch.empty_like(X) if out is None else out
    if coeffs_out is None:
        coeffs_out = (torch.empty(T, n, device=X.device), torch.empty(T, n, device=X.device),
                      torch.empty(T, n, n, device=X.device))
    hp, hq, hr = coeffs_out
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), X.device, workspace)
    a = [float(v) for v in alpha_next]
    _check("hc_post_coeffs", lib().hc_post_coeffs(
        _ptr(X), _DT[X.dtype], T, n, C, _ptr(_f32(h_res, "h_res")), _ptr(_f32(h_post, "h_post")), _ptr(F_out),
        _ptr(X_next), _ptr(_f32(phi_next, "phi_next")), _ptr(_f32(bias_next, "bias_next")), a[0], a[1], a[2],
        int(sinkhorn_iters), _ptr(hp), _ptr(hq), _ptr(hr), _ptr(ws), ws.numel(), _stream(X.device, stream)))
    return X_next, coeffs_out


def hc_phi_packed_bytes(n: int, C: int, dtype) -> int:
    return int(lib().hc_phi_packed_bytes(n, C, _DT[dtype]))


def hc_phi_pack(phi, n, C, dtype=torch.bfloat16, *, out=None, stream=None):
    """phi [n*C, n*n+2n] float32 in the packed form of the fast path (a uint8 tensor), or
    None when (n, C, dtype) has no packed form."""
    phi = _f32(phi, "phi")
    nbytes = hc_phi_packed_bytes(n, C, dtype)
    if nbytes < 0:
        raise ValueError("invalid sizes for hc_phi_packed_bytes")
    if nbytes == 0:
        return None
    packed = torch.empty(nbytes, dtype=torch.uint8, device=phi.device) if out is None else out
    _check("hc_phi_pack", lib().hc_phi_pack(_ptr(phi), n, C, _DT[dtype], _ptr(packed),
                                            packed.numel() * packed.element_size(), _stream(phi.device, stream)))
    return packed


def hc_post_pre(X, h_res, h_post, F_out, phi_next, bias_next, alpha_next, sinkhorn_iters=20, *,
                phi_next_packed=None, out=None, coeffs_out=None, F_in_out=None, want_h_pre=True,
                workspace=None, stream=None):
    """hc_post_coeffs followed by the pre-read of X_next.
    Returns (X_next, (h_pre' or None, h_post', h_res'), F_in')."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,))
    X_next = torch.empty_like(X) if out is None else out
    if coeffs_out is None:
        coeffs_out = (torch.empty(T, n, device=X.device) if want_h_pre else None,
                      torch.empty(T, n, device=X.device), torch.empty(T, n, n, device=X.device))
    hp, hq, hr = coeffs_out
    F_in = torch.empty(T, C, dtype=X.dtype, device=X.device) if F_in_out is None else F_in_out
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), X.device, workspace)
    a = [float(v) for v in alpha_next]
    _check("hc_post_pre", lib().hc_post_pre(
        _ptr(X), _DT[X.dtype], T, n, C, _ptr(_f32(h_res, "h_res")), _ptr(_f32(h_post, "h_post")), _ptr(F_out),
        _ptr(X_next), _ptr(_f32(phi_next, "phi_next")), _ptr(phi_next_packed),
        _ptr(_f32(bias_next, "bias_next")), a[0], a[1], a[2], int(sinkhorn_iters), _ptr(hp), _ptr(hq), _ptr(hr),
        _ptr(F_in), _ptr(ws), ws.numel(), _stream(X.device, stream)))
    return X_next, coeffs_out, F_in


# ------------------------------------------------------------------- xHC


def xhc_pre_workspace_bytes(T, N, C, m, with_router, dtype) -> int:
    return int(lib().xhc_pre_workspace_bytes(T, N, C, m, int(bool(with_router)), _DT[dtype]))


def xhc_pre(X, phi_pre, b_pre, alpha_pre, w_router=None, k=4, m=2, *, want_h_pre=True, out=None,
            workspace=None, stream=None):
    """Full-state pass: dict(h_pre, F_in[, idx, score]). out = (h_pre or None, F_in)
    writes into given tensors."""
    X = _dev_tensor(X, "X", _DT)
    T, N, C = X.shape
    dev = X.device
    if out is not None:
        h_pre, F_in = out
    else:
        h_pre = torch.empty(T, N, device=dev) if want_h_pre else None
        F_in = torch.empty(T, C, dtype=X.dtype, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev) if w_router is not None else None
    score = torch.empty(T, N - m, device=dev) if w_router is not None else None
    ws = _workspace(xhc_pre_workspace_bytes(T, N, C, m, w_router is not None, X.dtype), dev, workspace)
    _check("xhc_pre", lib().xhc_pre(_ptr(X), _DT[X.dtype], T, N, C, k, m, _ptr(_f32(phi_pre, "phi_pre")),
                                    _ptr(_f32(b_pre, "b_pre")), float(alpha_pre),
                                    _ptr(None if w_router is None else _f32(w_router, "w_router")),
                                    _ptr(h_pre), _ptr(F_in), _ptr(idx), _ptr(score), _ptr(ws), ws.numel(),
                                    _stream(dev, stream)))
    out = dict(h_pre=h_pre, F_in=F_in)
    if w_router is not None:
        out.update(idx=idx, score=score)
    return out


def xhc_route_workspace_bytes(T, N, C, k, m, K, with_router, dtype) -> int:
    return int(lib().xhc_route_workspace_bytes(T, N, C, k, m, K, int(bool(with_router)), _DT[dtype]))


def xhc_route(X, Wb, phi_act, b_act, alpha_post, alpha_res, *, k=4, m=2, idx=None, w_router=None,
              sinkhorn_iters=20, want_coeffs=False, workspace=None, stream=None):
    """In-place sparse update of X [T,N,C] with write-back components Wb [T,K,C] (or [T,C]).

    Returns dict(idx[, score][, h_post, h_res])."""
    X = _dev_tensor(X, "X", _DT)
    T, N, C = X.shape
    dev = X.device
    Wb = _dev_tensor(Wb, "Wb", (X.dtype,))
    K = 1 if Wb.dim() == 2 else Wb.shape[1]
    idx_in = None if idx is None else _dev_tensor(idx, "idx", (torch.int32,))
    idx_out = torch.empty(T, k, dtype=torch.int32, device=dev)
    score = torch.empty(T, N - m, device=dev) if idx_in is None else None
    hp = torch.empty(T, k, K, device=dev) if want_coeffs else None
    hr = torch.empty(T, k, k, device=dev) if want_coeffs else None
    ws = _workspace(xhc_route_workspace_bytes(T, N, C, k, m, K, idx_in is None, X.dtype), dev, workspace)
    _check("xhc_route", lib().xhc_route(_ptr(X), _DT[X.dtype], T, N, C, k, m,
                                        _ptr(None if w_router is None else _f32(w_router, "w_router")),
                                        _ptr(idx_in), _ptr(_f32(phi_act, "phi_act")), _ptr(_f32(b_act, "b_act")),
                                        float(alpha_post), float(alpha_res), int(sinkhorn_iters), _ptr(Wb), K,
                                        _ptr(idx_out), _ptr(score), _ptr(hp), _ptr(hr), _ptr(ws), ws.numel(),
                                        _stream(dev, stream)))
    out = dict(idx=idx_out)
    if score is not None:
        out["score"] = score
    if want_coeffs:
        out.update(h_post=hp, h_res=hr)
    return out


def xhc_flash_pre_workspace_bytes(T: int, N: int, C: int, m: int, L: int, dtype) -> int:
    return int(lib().xhc_flash_pre_workspace_bytes(T, N, C, m, L, _DT[dtype]))


def xhc_flash_pre(X, phi_pre, b_pre, alpha_pre, w_router, *, k=4, m=2, out=None, workspace=None, stream=None):
    """xHC-Flash block entry: phi_pre [L, N*C, N], b_pre [L, N]. Returns (idx [T, k],
    score [T, N-m], h_pre [L, T, N], F_pre [L, T, C])."""
    X = _dev_tensor(X, "X", _DT)
    T, N, C = X.shape
    dev = X.device
    phi_pre = _f32(phi_pre, "phi_pre")
    L = phi_pre.shape[0]
    if out is None:
        out = (torch.empty(T, k, dtype=torch.int32, device=dev), torch.empty(T, N - m, device=dev),
               torch.empty(L, T, N, device=dev), torch.empty(L, T, C, dtype=X.dtype, device=dev))
    idx, score, h_pre, F_pre = out
    ws = _workspace(xhc_flash_pre_workspace_bytes(T, N, C, m, L, X.dtype), dev, workspace)
    _check("xhc_flash_pre", lib().xhc_flash_pre(_ptr(X), _DT[X.dtype], T, N, C, k, m, L, _ptr(phi_pre),
                                                _ptr(_f32(b_pre, "b_pre")), float(alpha_pre),
                                                _ptr(_f32(w_router, "w_router")), _ptr(idx), _ptr(score),
                                                _ptr(h_pre), _ptr(F_pre), _ptr(ws), ws.numel(), _stream(dev, stream)))
    return idx, score, h_pre, F_pre


def xhc_flash_maps_workspace_bytes(T: int, N: int, C: int, k: int, L: int, dtype) -> int:
    return int(lib().xhc_flash_maps_workspace_bytes(T, N, C, k, L, _DT[dtype]))


def xhc_flash_maps(X, idx, phi_act, b_act, alpha_post, alpha_res, L, *, sinkhorn_iters=20, out=None,
                   workspace=None, stream=None):
    """The block's maps from X's active rows: returns (H_post [T, k, L], H_res [T, k, k])."""
    X = _dev_tensor(X, "X", _DT)
    T, N, C = X.shape
    idx = _dev_tensor(idx, "idx", (torch.int32,))
    k = idx.shape[1]
    dev = X.device
    if out is None:
        out = (torch.empty(T, k, L, device=dev), torch.empty(T, k, k, device=dev))
    Hp, Hr = out
    ws = _workspace(xhc_flash_maps_workspace_bytes(T, N, C, k, L, X.dtype), dev, workspace)
    _check("xhc_flash_maps", lib().xhc_flash_maps(_ptr(X), _DT[X.dtype], T, N, C, k, L, _ptr(idx),
                                                  _ptr(_f32(phi_act, "phi_act")), _ptr(_f32(b_act, "b_act")),
                                                  float(alpha_post), float(alpha_res), int(sinkhorn_iters), _ptr(Hp),
                                                  _ptr(Hr), _ptr(ws), ws.numel(), _stream(dev, stream)))
    return Hp, Hr


def xhc_flash_input(l, F_pre_l, h_pre_l, idx, H_post, F_outs, *, N=None, out=None, stream=None):
    """Sublayer l's input from the entry-state read F_pre_l [T, C] and the earlier
    outputs F_outs [T, L, C] (rows j < l read). Returns F_in [T, C]."""
    F_pre_l = _dev_tensor(F_pre_l, "F_pre_l", _DT)
    T, C = F_pre_l.shape
    h_pre_l = _f32(h_pre_l, "h_pre_l")
    N = h_pre_l.shape[1] if N is None else N
    idx = _dev_tensor(idx, "idx", (torch.int32,))
    H_post = _f32(H_post, "H_post")
    k, L = H_post.shape[1], H_post.shape[2]
    F_outs = None if F_outs is None else _dev_tensor(F_outs, "F_outs", (F_pre_l.dtype,))
    F_in = torch.empty_like(F_pre_l) if out is None else out
    _check("xhc_flash_input", lib().xhc_flash_input(_DT[F_pre_l.dtype], T, N, C, k, L, int(l), _ptr(F_pre_l),
                                                    _ptr(h_pre_l), _ptr(idx), _ptr(H_post), _ptr(F_outs), _ptr(F_in),
                                                    _stream(F_pre_l.device, stream)))
    return F_in


def xhc_flash_post_workspace_bytes(T: int, k: int, L: int) -> int:
    return int(lib().xhc_flash_post_workspace_bytes(T, k, L))


def xhc_flash_post(X, idx, H_post, H_res, F_outs, *, workspace=None, stream=None):
    """Block end in place on X [T, N, C] from the entry state's active rows and
    F_outs [T, L, C]. Returns X."""
    X = _dev_tensor(X, "X", _DT)
    T, N, C = X.shape
    idx = _dev_tensor(idx, "idx", (torch.int32,))
    H_post = _f32(H_post, "H_post")
    k, L = H_post.shape[1], H_post.shape[2]
    F_outs = _dev_tensor(F_outs, "F_outs", (X.dtype,))
    ws = _workspace(xhc_flash_post_workspace_bytes(T, k, L), X.device, workspace)
    _check("xhc_flash_post", lib().xhc_flash_post(_ptr(X), _DT[X.dtype], T, N, C, k, L, _ptr(idx), _ptr(H_post),
                                                  _ptr(_f32(H_res, "H_res")), _ptr(F_outs), _ptr(ws), ws.numel(),
                                                  _stream(X.device, stream)))
    return X


def xhc_augment_workspace_bytes(batch, seq, C, kappas, dtype, v_dtype=None) -> int:
    karr = (ctypes.c_int * max(len(kappas), 1))(*[int(x) for x in kappas])
    vdt = dtype if v_dtype is None else v_dtype
    return int(lib().xhc_augment_workspace_bytes(batch, seq, C, karr, len(kappas), _DT[dtype], _DT[vdt]))


def xhc_augment(F_out, conv_w, kappas, batch, seq, *, v_dtype=None, workspace=None, stream=None):
    """V [T, r+1, C] = Gram-Schmidt([F_out; causal depthwise convs]); conv_w concatenated fp32."""
    F_out = _dev_tensor(F_out, "F_out", _DT)
    T, C = F_out.shape
    if T != batch * seq:
        raise ValueError("F_out rows must equal batch * seq")
    r = len(kappas)
    vdt = F_out.dtype if v_dtype is None else v_dtype
    V = torch.empty(T, r + 1, C, dtype=vdt, device=F_out.device)
    karr = (ctypes.c_int * max(r, 1))(*[int(x) for x in kappas])
    w = _f32(conv_w, "conv_w") if r > 0 else None
    nbytes = int(lib().xhc_augment_workspace_bytes(batch, seq, C, karr, r, _DT[F_out.dtype], _DT[vdt]))
    ws = _workspace(nbytes, F_out.device, workspace) if nbytes > 0 else None
    _check("xhc_augment", lib().xhc_augment(_ptr(F_out), _DT[F_out.dtype], batch, seq, C, _ptr(w), karr, r,
                                            _ptr(V), _DT[vdt], _ptr(ws), 0 if ws is None else ws.numel(),
                                            _stream(F_out.device, stream)))
    return V


def hc_tanh_coeffs(X, theta, bias, alpha, *, out=None, stream=None):
    """HC's unconstrained maps (h_pre [T,n], h_post [T,n], h_res [T,n,n]) of X [T,n,C];
    theta [n+2, C] float32, bias [n*n+2n], alpha = (pre, post, res)."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    if out is None:
        out = (torch.empty(T, n, device=X.device), torch.empty(T, n, device=X.device),
               torch.empty(T, n, n, device=X.device))
    h_pre, h_post, h_res = out
    a = [float(v) for v in alpha]
    _check("hc_tanh_coeffs", lib().hc_tanh_coeffs(_ptr(X), _DT[X.dtype], T, n, C, _ptr(_f32(theta, "theta")),
                                                  _ptr(_f32(bias, "bias")), a[0], a[1], a[2], _ptr(h_pre),
                                                  _ptr(h_post), _ptr(h_res), _stream(X.device, stream)))
    return h_pre, h_post, h_res


def hc_amax_gain(h_res_layers, *, stream=None):
    """(forward gain [T], backward gain [T]) of the chain h_res_layers [L, T, n, n] (layer 0 first)."""
    H = _f32(h_res_layers, "h_res_layers")
    L, T, n, _ = H.shape
    fwd = torch.empty(T, device=H.device)
    bwd = torch.empty(T, device=H.device)
    _check("hc_amax_gain", lib().hc_amax_gain(_ptr(H), L, T, n, _ptr(fwd), _ptr(bwd), _stream(H.device, stream)))
    return fwd, bwd


def hc_static_maps(logits, n, sinkhorn_iters=20, *, stream=None):
    """Static mHC maps (h_pre [n], h_post [n], h_res [n, n]) from logits [n*n + 2n] float32."""
    z = _f32(logits, "logits")
    h_pre = torch.empty(n, device=z.device)
    h_post = torch.empty(n, device=z.device)
    h_res = torch.empty(n, n, device=z.device)
    _check("hc_static_maps", lib().hc_static_maps(_ptr(z), n, int(sinkhorn_iters), _ptr(h_pre), _ptr(h_post),
                                                  _ptr(h_res), _stream(z.device, stream)))
    return h_pre, h_post, h_res


def hc_static_pre(X, h_pre, *, out=None, stream=None):
    """F_in [T, C] = sum_i h_pre[i] X[:, i, :] with one h_pre [n] for every token."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    F_in = torch.empty(T, C, dtype=X.dtype, device=X.device) if out is None else out
    _check("hc_static_pre", lib().hc_static_pre(_ptr(X), _DT[X.dtype], T, n, C, _ptr(_f32(h_pre, "h_pre")),
                                                _ptr(F_in), _stream(X.device, stream)))
    return F_in


def hc_static_post(X, h_res, h_post, F_out, *, out=None, stream=None):
    """X_next [T, n, C] = h_res X[t] + h_post^T F_out[t] with maps shared by every token."""
    X = _dev_tensor(X, "X", _DT)
    T, n, C = X.shape
    Y = torch.empty_like(X) if out is None else out
    _check("hc_static_post", lib().hc_static_post(_ptr(X), _DT[X.dtype], T, n, C, _ptr(_f32(h_res, "h_res")),
                                                  _ptr(_f32(h_post, "h_post")),
                                                  _ptr(_dev_tensor(F_out, "F_out", _DT)), _ptr(Y),
                                                  _stream(X.device, stream)))
    return Y


def xhc_backward_workspace_bytes(T: int, N: int, C: int, k: int, K: int, dtype) -> int:
    return int(lib().xhc_backward_workspace_bytes(T, N, C, k, K, _DT[dtype]))


def xhc_route_backward(X, idx, phi_act, b_act, alpha_post, alpha_res, Wb, dX, sinkhorn_iters=20, *, out=None,
                       workspace=None, stream=None):
    """Backward of xhc_route (k = 4, bfloat16). X: the state before the route; Wb: F_out
    [T, C] (K = 1) or the augmentation's V [T, 4, C] (K = 4); dX holds dX_next and is
    updated in place to the route's gradient. Returns (dX, dWb, dphi_act, db_act,
    dalpha [post, res], dh [T, 4K + 16]); dWb is bfloat16 [T, C] for K = 1 and
    float32 [T, 4, C] for K = 4."""
    X = _dev_tensor(X, "X", (torch.bfloat16,))
    T, N, C = X.shape
    idx = _dev_tensor(idx, "idx", (torch.int32,))
    k = idx.shape[1]
    Wb = _dev_tensor(Wb, "Wb", (X.dtype,))
    K = 1 if Wb.dim() == 2 else Wb.shape[1]
    dX = _dev_tensor(dX, "dX", (X.dtype,))
    nc = k * K + k * k
    if out is None:
        dev = X.device
        dWb = (torch.empty(T, C, dtype=X.dtype, device=dev) if K == 1 else
               torch.empty(T, K, C, dtype=torch.float32, device=dev))
        out = (dWb, torch.empty(k * C, nc, device=dev), torch.empty(nc, device=dev), torch.empty(2, device=dev),
               torch.empty(T, nc, device=dev))
    dWb, dphi, db, dalpha, dh = out
    ws = _workspace(xhc_backward_workspace_bytes(T, N, C, k, K, X.dtype), X.device, workspace)
    _check("xhc_route_backward", lib().xhc_route_backward(
        _ptr(X), _DT[X.dtype], T, N, C, k, _ptr(idx), _ptr(_f32(phi_act, "phi_act")), _ptr(_f32(b_act, "b_act")),
        float(alpha_post), float(alpha_res), int(sinkhorn_iters), _ptr(Wb), K, _ptr(dX), _ptr(dWb), _ptr(dphi),
        _ptr(db), _ptr(dalpha), _ptr(dh), _ptr(ws), ws.numel(), _stream(X.device, stream)))
    return dX, dWb, dphi, db, dalpha, dh


def xhc_pre_backward(X, phi_pre, b_pre, alpha_pre, dF_in, dX, *, out=None, workspace=None, stream=None):
    """Backward of xhc_pre's dense read (bfloat16): dX += its gradient (in place).
    Returns (dX, dphi_pre, db_pre, dalpha [1], dh_pre [T, N])."""
    X = _dev_tensor(X, "X", (torch.bfloat16,))
    T, N, C = X.shape
    dF_in = _dev_tensor(dF_in, "dF_in", (X.dtype,))
    dX = _dev_tensor(dX, "dX", (X.dtype,))
    if out is None:
        dev = X.device
        out = (torch.empty(N * C, N, device=dev), torch.empty(N, device=dev), torch.empty(1, device=dev),
               torch.empty(T, N, device=dev))
    dphi, db, dalpha, dh = out
    ws = _workspace(xhc_backward_workspace_bytes(T, N, C, 4, 1, X.dtype), X.device, workspace)
    _check("xhc_pre_backward", lib().xhc_pre_backward(
        _ptr(X), _DT[X.dtype], T, N, C, _ptr(_f32(phi_pre, "phi_pre")), _ptr(_f32(b_pre, "b_pre")), float(alpha_pre),
        _ptr(dF_in), _ptr(dX), _ptr(dphi), _ptr(db), _ptr(dalpha), _ptr(dh), _ptr(ws), ws.numel(),
        _stream(X.device, stream)))
    return dX, dphi, db, dalpha, dh


def xhc_augment_backward_workspace_bytes(B: int, S: int, C: int, kappas, dtype) -> int:
    k = (ctypes.c_int * len(kappas))(*[int(x) for x in kappas])
    return int(lib().xhc_augment_backward_workspace_bytes(B, S, C, k, len(kappas), _DT[dtype]))


def xhc_augment_backward(F_out, conv_w, kappas, B, S, dV, *, out=None, workspace=None, stream=None):
    """Backward of xhc_augment (kappas (4, 8, 12)): dV [T, 4, C] float32 in; returns
    (dF_out [T, C] in F_out's dtype, dconv_w in conv_w's layout)."""
    F_out = _dev_tensor(F_out, "F_out", _DT)
    T, C = F_out.shape
    dV = _f32(dV, "dV")
    conv_w = _f32(conv_w, "conv_w")
    if out is None:
        out = (torch.empty_like(F_out), torch.empty_like(conv_w))
    dF, dw = out
    k = (ctypes.c_int * len(kappas))(*[int(x) for x in kappas])
    ws = _workspace(xhc_augment_backward_workspace_bytes(B, S, C, kappas, F_out.dtype), F_out.device, workspace)
    _check("xhc_augment_backward", lib().xhc_augment_backward(
        _ptr(F_out), _DT[F_out.dtype], B, S, C, _ptr(conv_w), k, len(kappas), _ptr(dV), _ptr(dF), _ptr(dw),
        _ptr(ws), ws.numel(), _stream(F_out.device, stream)))
    return dF, dw


def hc_copy_probe(src, dst, *, stream=None):
    """Copy src into dst (same byte size, 16-byte aligned) with the library's streaming
    copy: a measurement probe of the device's streaming rate, not part of the method."""
    src = _dev_tensor(src, "src")
    dst = _dev_tensor(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not src.is_contiguous() or not dst.is_contiguous():
        raise ValueError("hc_copy_probe needs contiguous tensors of the same byte size")
    _check("hc_copy_probe", lib().hc_copy_probe(_ptr(src), _ptr(dst), nbytes, _stream(src.device, stream)))
    return dst


__all__ = [
    "LIB_PATH", "HCError", "lib", "status_string", "hc_coeffs_workspace_bytes", "hc_coeffs", "hc_pre",
    "hc_coeffs_pre", "hc_post", "hc_backward_workspace_bytes", "hc_backward_post", "hc_backward", "xhc_backward_workspace_bytes",
    "xhc_route_backward", "xhc_pre_backward", "xhc_augment_backward_workspace_bytes", "xhc_augment_backward", "hc_post_coeffs", "hc_phi_packed_bytes", "hc_phi_pack", "hc_post_pre",
    "xhc_pre_workspace_bytes", "xhc_pre", "xhc_route_workspace_bytes",
    "xhc_route", "xhc_augment_workspace_bytes", "xhc_augment", "xhc_flash_pre_workspace_bytes", "xhc_flash_pre",
    "xhc_flash_maps_workspace_bytes", "xhc_flash_maps", "xhc_flash_input", "xhc_flash_post_workspace_bytes",
    "xhc_flash_post", "hc_tanh_coeffs", "hc_amax_gain",
    "hc_static_maps", "hc_static_pre", "hc_static_post", "hc_copy_probe",
]
