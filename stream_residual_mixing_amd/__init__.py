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
    "hc_post_pre_noalloc": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _c_float, _c_float, _c_float, _c_int, _vp, _vp, _vp, _vp, _vp]),
    "xhc_pre_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int]),
    "xhc_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _c_float, _vp,
                         _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_route_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int,
                                           _c_int]),
    "xhc_route": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _vp, _vp,
                           _c_float, _c_float, _c_int, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _c_i64,
                           _vp]),
    "xhc_chain_carry_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int]),
    "xhc_chain_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int]),
    "xhc_pre_chain": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _c_float, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_route_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _vp, _vp, _vp, _c_float,
                               _c_float, _c_int, _vp, _c_int, _vp, _c_float, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_augment_workspace_bytes": (_c_i64, [_c_i64, _c_i64, _c_i64, _vp, _c_int, _c_int, _c_int]),
    "xhc_flash_pre_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int]),
    "xhc_flash_pre": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _vp, _vp, _c_float,
                               _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_flash_maps_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int]),
    "xhc_flash_maps": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                _c_float, _c_float, _c_int, _vp, _vp, _vp, _c_i64, _vp]),
    "xhc_flash_input": (_c_int, [_c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp]),
    "xhc_flash_post_workspace_bytes": (_c_i64, [_c_i64, _c_int, _c_int, _c_int]),
    "xhc_flash_post": (_c_int, [_vp, _c_int, _c_i64, _c_int, _c_i64, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                _vp, _vp, _c_i64, _vp]),
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


def _dev_tensor(t, name, dtypes=None, shape=None, device=None):
    """t checked before any launch: a contiguous tensor on a HIP device (the given
    one if any), of one of `dtypes` and exactly `shape`. The C ABI takes raw
    pointers, so a wrong size would reach the kernels; here it raises instead."""
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a tensor on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")
    return t


def _f32(t, name, shape=None, device=None):
    return _dev_tensor(t, name, (torch.float32,), shape, device)


def _i32(t, name, shape=None, device=None):
    return _dev_tensor(t, name, (torch.int32,), shape, device)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _workspace(nbytes: int, device, workspace):
    """The caller's workspace if it is large enough (checked like any argument), else
    a new one; the byte count passed to the C call is the tensor's true size."""
    if nbytes < 0:
        raise ValueError("invalid sizes for the workspace query")
    if workspace is not None:
        _dev_tensor(workspace, "workspace", device=device)
        if _nbytes(workspace) >= nbytes:
            return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _state(X, name="X", dtypes=None):
    X = _dev_tensor(X, name, _DT if dtypes is None else dtypes)
    if X.dim() != 3:
        raise ValueError(f"{name} must be [T, streams, C], got shape {tuple(X.shape)}")
    return X


# ------------------------------------------------------------------- mHC


def hc_coeffs_workspace_bytes(T: int, n: int, C: int, dtype) -> int:
    return int(lib().hc_coeffs_workspace_bytes(T, n, C, _DT[dtype]))


def _coeff_outs(out, T, n, dev, want_h_pre=True):
    if out is None:
        return (torch.empty(T, n, device=dev) if want_h_pre else None, torch.empty(T, n, device=dev),
                torch.empty(T, n, n, device=dev))
    h_pre, h_post, h_res = out
    return (None if h_pre is None else _f32(h_pre, "h_pre out", (T, n), dev), _f32(h_post, "h_post out", (T, n), dev),
            _f32(h_res, "h_res out", (T, n, n), dev))


def _phi_bias(phi, bias, n, C, dev, name="phi", bname="bias"):
    nc = n * n + 2 * n
    return _f32(phi, name, (n * C, nc), dev), _f32(bias, bname, (nc,), dev)


def _stream_out(out, name, shape, dtype, dev):
    if out is None:
        return torch.empty(*shape, dtype=dtype, device=dev)
    return _dev_tensor(out, name, (dtype,), shape, dev)


def hc_coeffs(X, phi, bias, alpha, sinkhorn_iters=20, *, out=None, workspace=None, stream=None):
    """(h_pre [T,n], h_post [T,n], h_res [T,n,n]) of X [T,n,C]; alpha = (pre, post, res)."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    phi, bias = _phi_bias(phi, bias, n, C, dev)
    h_pre, h_post, h_res = _coeff_outs(out, T, n, dev)
    if h_pre is None:
        raise ValueError("hc_coeffs needs an h_pre output")
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), dev, workspace)
    a = [float(v) for v in alpha]
    _check("hc_coeffs", lib().hc_coeffs(_ptr(X), _DT[X.dtype], T, n, C, _ptr(phi), _ptr(bias), a[0], a[1],
                                        a[2], int(sinkhorn_iters), _ptr(h_pre), _ptr(h_post), _ptr(h_res),
                                        _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    return h_pre, h_post, h_res


def hc_pre(X, h_pre, *, out=None, stream=None):
    """F_in [T,C] = sum_i h_pre[:, i] X[:, i, :]."""
    X = _state(X)
    T, n, C = X.shape
    h_pre = _f32(h_pre, "h_pre", (T, n), X.device)
    F_in = _stream_out(out, "F_in out", (T, C), X.dtype, X.device)
    _check("hc_pre", lib().hc_pre(_ptr(X), _DT[X.dtype], T, n, C, _ptr(h_pre), _ptr(F_in),
                                  _stream(X.device, stream)))
    return F_in


def hc_coeffs_pre(X, phi, bias, alpha, sinkhorn_iters=20, *, out=None, workspace=None, stream=None,
                  want_h_pre=True):
    """Fused coefficients + pre-read: (h_pre or None, h_post, h_res, F_in)."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    phi, bias = _phi_bias(phi, bias, n, C, dev)
    if out is None:
        h_pre, h_post, h_res = _coeff_outs(None, T, n, dev, want_h_pre)
        F_in = _stream_out(None, "F_in out", (T, C), X.dtype, dev)
    else:
        h_pre, h_post, h_res = _coeff_outs(out[:3], T, n, dev)
        F_in = _stream_out(out[3], "F_in out", (T, C), X.dtype, dev)
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), dev, workspace)
    a = [float(v) for v in alpha]
    _check("hc_coeffs_pre", lib().hc_coeffs_pre(_ptr(X), _DT[X.dtype], T, n, C, _ptr(phi), _ptr(bias), a[0],
                                                a[1], a[2], int(sinkhorn_iters), _ptr(h_pre), _ptr(h_post),
                                                _ptr(h_res), _ptr(F_in), _ptr(ws), _nbytes(ws),
                                                _stream(dev, stream)))
    return h_pre, h_post, h_res, F_in


def hc_post(X, h_res, h_post, F_out, *, out=None, stream=None):
    """X_next [T,n,C] = h_res @ X + h_post^T F_out (out may be X itself)."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,), (T, C), dev)
    h_res = _f32(h_res, "h_res", (T, n, n), dev)
    h_post = _f32(h_post, "h_post", (T, n), dev)
    X_next = _stream_out(out, "X_next out", (T, n, C), X.dtype, dev)
    _check("hc_post", lib().hc_post(_ptr(X), _DT[X.dtype], T, n, C, _ptr(h_res), _ptr(h_post), _ptr(F_out),
                                    _ptr(X_next), _stream(dev, stream)))
    return X_next


def hc_backward_workspace_bytes(T: int, n: int, C: int, dtype) -> int:
    return int(lib().hc_backward_workspace_bytes(T, n, C, _DT[dtype]))


def hc_backward_post(X, h_post, F_out, dX_next, *, out=None, stream=None):
    """Backward, post stage (n = 4, bfloat16): (dF_out, dh) with dF_out = H_post dX_next
    and dh [T, 24] float32 holding dH_post (columns 4..7) and dH_res (8..23)."""
    X = _state(X, dtypes=(torch.bfloat16,))
    T, n, C = X.shape
    dev = X.device
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,), (T, C), dev)
    dX_next = _dev_tensor(dX_next, "dX_next", (X.dtype,), (T, n, C), dev)
    h_post = _f32(h_post, "h_post", (T, n), dev)
    nc = n * n + 2 * n
    if out is None:
        out = (None, None)
    dF_out = _stream_out(out[0], "dF_out out", (T, C), X.dtype, dev)
    dh = torch.empty(T, nc, device=dev) if out[1] is None else _f32(out[1], "dh out", (T, nc), dev)
    _check("hc_backward_post", lib().hc_backward_post(_ptr(X), _DT[X.dtype], T, n, C, _ptr(h_post), _ptr(F_out),
                                                      _ptr(dX_next), _ptr(dF_out), _ptr(dh), _stream(dev, stream)))
    return dF_out, dh


def hc_backward(X, phi, bias, alpha, dX_next, dF_in, dh, sinkhorn_iters=20, *, out=None, workspace=None,
                stream=None):
    """Backward, main stage (n = 4, bfloat16): fills dh[:, 0:4] (dH_pre), reads the rest of
    dh from hc_backward_post, returns (dX, dphi, dbias, dalpha)."""
    X = _state(X, dtypes=(torch.bfloat16,))
    T, n, C = X.shape
    dev = X.device
    nc = n * n + 2 * n
    dX_next = _dev_tensor(dX_next, "dX_next", (X.dtype,), (T, n, C), dev)
    dF_in = _dev_tensor(dF_in, "dF_in", (X.dtype,), (T, C), dev)
    phi, bias = _phi_bias(phi, bias, n, C, dev)
    dh = _f32(dh, "dh", (T, nc), dev)
    if out is None:
        out = (torch.empty_like(X), torch.empty(n * C, nc, device=dev), torch.empty(nc, device=dev),
               torch.empty(3, device=dev))
    dX = _dev_tensor(out[0], "dX out", (X.dtype,), (T, n, C), dev)
    dphi = _f32(out[1], "dphi out", (n * C, nc), dev)
    dbias = _f32(out[2], "dbias out", (nc,), dev)
    dalpha = _f32(out[3], "dalpha out", (3,), dev)
    ws = _workspace(hc_backward_workspace_bytes(T, n, C, X.dtype), dev, workspace)
    a = [float(v) for v in alpha]
    _check("hc_backward", lib().hc_backward(_ptr(X), _DT[X.dtype], T, n, C, _ptr(phi), _ptr(bias), a[0], a[1], a[2],
                                            int(sinkhorn_iters), _ptr(dX_next), _ptr(dF_in), _ptr(dh), _ptr(dX),
                                            _ptr(dphi), _ptr(dbias), _ptr(dalpha), _ptr(ws), _nbytes(ws),
                                            _stream(dev, stream)))
    return dX, dphi, dbias, dalpha


def hc_post_coeffs(X, h_res, h_post, F_out, phi_next, bias_next, alpha_next, sinkhorn_iters=20, *, out=None,
                   coeffs_out=None, workspace=None, stream=None):
    """X_next = h_res @ X + h_post^T F_out, plus the coefficients of X_next under the next
    sublayer's phi/bias/alpha. Returns (X_next, (h_pre', h_post', h_res'))."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,), (T, C), dev)
    h_res = _f32(h_res, "h_res", (T, n, n), dev)
    h_post = _f32(h_post, "h_post", (T, n), dev)
    phi_next, bias_next = _phi_bias(phi_next, bias_next, n, C, dev, "phi_next", "bias_next")
    X_next = _stream_out(out, "X_next out", (T, n, C), X.dtype, dev)
    hp, hq, hr = _coeff_outs(coeffs_out, T, n, dev)
    if hp is None:
        raise ValueError("hc_post_coeffs needs an h_pre output")
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), dev, workspace)
    a = [float(v) for v in alpha_next]
    _check("hc_post_coeffs", lib().hc_post_coeffs(
        _ptr(X), _DT[X.dtype], T, n, C, _ptr(h_res), _ptr(h_post), _ptr(F_out), _ptr(X_next), _ptr(phi_next),
        _ptr(bias_next), a[0], a[1], a[2], int(sinkhorn_iters), _ptr(hp), _ptr(hq), _ptr(hr), _ptr(ws), _nbytes(ws),
        _stream(dev, stream)))
    return X_next, (hp, hq, hr)


def hc_phi_packed_bytes(n: int, C: int, dtype) -> int:
    return int(lib().hc_phi_packed_bytes(n, C, _DT[dtype]))


def _packed(t, name, n, C, dtype, dev):
    nbytes = hc_phi_packed_bytes(n, C, dtype)
    t = _dev_tensor(t, name, device=dev)
    if nbytes <= 0 or _nbytes(t) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes; the packed form of these sizes needs {nbytes}")
    return t


def hc_phi_pack(phi, n, C, dtype=torch.bfloat16, *, out=None, stream=None):
    """phi [n*C, n*n+2n] float32 in the packed form of the fast path (a uint8 tensor), or
    None when (n, C, dtype) has no packed form."""
    phi = _f32(phi, "phi", (n * C, n * n + 2 * n))
    nbytes = hc_phi_packed_bytes(n, C, dtype)
    if nbytes < 0:
        raise ValueError("invalid sizes for hc_phi_packed_bytes")
    if nbytes == 0:
        return None
    packed = (torch.empty(nbytes, dtype=torch.uint8, device=phi.device) if out is None
              else _packed(out, "packed out", n, C, dtype, phi.device))
    _check("hc_phi_pack", lib().hc_phi_pack(_ptr(phi), n, C, _DT[dtype], _ptr(packed), _nbytes(packed),
                                            _stream(phi.device, stream)))
    return packed


def hc_post_pre(X, h_res, h_post, F_out, phi_next, bias_next, alpha_next, sinkhorn_iters=20, *,
                phi_next_packed=None, out=None, coeffs_out=None, F_in_out=None, want_h_pre=True,
                workspace=None, stream=None):
    """hc_post_coeffs followed by the pre-read of X_next.
    Returns (X_next, (h_pre' or None, h_post', h_res'), F_in')."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,), (T, C), dev)
    h_res = _f32(h_res, "h_res", (T, n, n), dev)
    h_post = _f32(h_post, "h_post", (T, n), dev)
    phi_next, bias_next = _phi_bias(phi_next, bias_next, n, C, dev, "phi_next", "bias_next")
    pk = None if phi_next_packed is None else _packed(phi_next_packed, "phi_next_packed", n, C, X.dtype, dev)
    X_next = _stream_out(out, "X_next out", (T, n, C), X.dtype, dev)
    hp, hq, hr = _coeff_outs(coeffs_out, T, n, dev, want_h_pre)
    F_in = _stream_out(F_in_out, "F_in out", (T, C), X.dtype, dev)
    ws = _workspace(hc_coeffs_workspace_bytes(T, n, C, X.dtype), dev, workspace)
    a = [float(v) for v in alpha_next]
    _check("hc_post_pre", lib().hc_post_pre(
        _ptr(X), _DT[X.dtype], T, n, C, _ptr(h_res), _ptr(h_post), _ptr(F_out), _ptr(X_next), _ptr(phi_next),
        _ptr(pk), _ptr(bias_next), a[0], a[1], a[2], int(sinkhorn_iters), _ptr(hp), _ptr(hq), _ptr(hr),
        _ptr(F_in), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    return X_next, (hp, hq, hr), F_in


# The fixed per-GPU scratch of hc_post_pre_noalloc (HC_NOALLOC_SCRATCH_BYTES in hc.h).
HC_NOALLOC_SCRATCH_BYTES = 32 << 20


def hc_post_pre_noalloc(X, h_res, h_post, F_out, phi_next, bias_next, alpha_next, sinkhorn_iters=20, *,
                        phi_next_packed=None, out=None, coeffs_out=None, F_in_out=None, want_h_pre=True,
                        stream=None):
    """hc_post_pre with the library's fixed scratch as its workspace (no device memory is
    allocated by the C call; pass every output to allocate nothing here either).
    Returns (X_next, (h_pre' or None, h_post', h_res'), F_in')."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,), (T, C), dev)
    h_res = _f32(h_res, "h_res", (T, n, n), dev)
    h_post = _f32(h_post, "h_post", (T, n), dev)
    phi_next, bias_next = _phi_bias(phi_next, bias_next, n, C, dev, "phi_next", "bias_next")
    pk = None if phi_next_packed is None else _packed(phi_next_packed, "phi_next_packed", n, C, X.dtype, dev)
    X_next = _stream_out(out, "X_next out", (T, n, C), X.dtype, dev)
    hp, hq, hr = _coeff_outs(coeffs_out, T, n, dev, want_h_pre)
    F_in = _stream_out(F_in_out, "F_in out", (T, C), X.dtype, dev)
    a = [float(v) for v in alpha_next]
    _check("hc_post_pre_noalloc", lib().hc_post_pre_noalloc(
        _ptr(X), _DT[X.dtype], T, n, C, _ptr(h_res), _ptr(h_post), _ptr(F_out), _ptr(X_next), _ptr(phi_next),
        _ptr(pk), _ptr(bias_next), a[0], a[1], a[2], int(sinkhorn_iters), _ptr(hp), _ptr(hq), _ptr(hr),
        _ptr(F_in), _stream(dev, stream)))
    return X_next, (hp, hq, hr), F_in


# ------------------------------------------------------------------- xHC


def xhc_pre_workspace_bytes(T, N, C, m, with_router, dtype) -> int:
    return int(lib().xhc_pre_workspace_bytes(T, N, C, m, int(bool(with_router)), _DT[dtype]))


def xhc_pre(X, phi_pre, b_pre, alpha_pre, w_router=None, k=4, m=2, *, want_h_pre=True, out=None,
            workspace=None, stream=None):
    """Full-state pass: dict(h_pre, F_in[, idx, score]). out = (h_pre or None, F_in)
    writes into given tensors."""
    X = _state(X)
    T, N, C = X.shape
    dev = X.device
    phi_pre = _f32(phi_pre, "phi_pre", (N * C, N), dev)
    b_pre = _f32(b_pre, "b_pre", (N,), dev)
    if w_router is not None:
        if not 1 <= m <= k <= N:
            raise ValueError(f"need 1 <= m <= k <= N, got m={m} k={k} N={N}")
        w_router = _f32(w_router, "w_router", (N * C, N - m), dev)
    if out is not None:
        h_pre = None if out[0] is None else _f32(out[0], "h_pre out", (T, N), dev)
        F_in = _stream_out(out[1], "F_in out", (T, C), X.dtype, dev)
    else:
        h_pre = torch.empty(T, N, device=dev) if want_h_pre else None
        F_in = torch.empty(T, C, dtype=X.dtype, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev) if w_router is not None else None
    score = torch.empty(T, N - m, device=dev) if w_router is not None else None
    ws = _workspace(xhc_pre_workspace_bytes(T, N, C, m, w_router is not None, X.dtype), dev, workspace)
    _check("xhc_pre", lib().xhc_pre(_ptr(X), _DT[X.dtype], T, N, C, k, m, _ptr(phi_pre), _ptr(b_pre),
                                    float(alpha_pre), _ptr(w_router), _ptr(h_pre), _ptr(F_in), _ptr(idx),
                                    _ptr(score), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    res = dict(h_pre=h_pre, F_in=F_in)
    if w_router is not None:
        res.update(idx=idx, score=score)
    return res


def xhc_route_workspace_bytes(T, N, C, k, m, K, with_router, dtype) -> int:
    return int(lib().xhc_route_workspace_bytes(T, N, C, k, m, K, int(bool(with_router)), _DT[dtype]))


def _write_back(Wb, T, C, dtypes, dev):
    """Wb [T, C] (one component) or [T, K, C]; returns (Wb, K)."""
    Wb = _dev_tensor(Wb, "Wb", dtypes, device=dev)
    if Wb.dim() == 2:
        _dev_tensor(Wb, "Wb", shape=(T, C))
        return Wb, 1
    if Wb.dim() != 3 or tuple(Wb.shape[::2]) != (T, C):
        raise ValueError(f"Wb has shape {tuple(Wb.shape)}, expected ({T}, {C}) or ({T}, K, {C})")
    return Wb, Wb.shape[1]


def xhc_route(X, Wb, phi_act, b_act, alpha_post, alpha_res, *, k=4, m=2, idx=None, w_router=None,
              sinkhorn_iters=20, want_coeffs=False, workspace=None, stream=None):
    """In-place sparse update of X [T,N,C] with write-back components Wb [T,K,C] (or [T,C]).

    Returns dict(idx[, score][, h_post, h_res])."""
    X = _state(X)
    T, N, C = X.shape
    dev = X.device
    Wb, K = _write_back(Wb, T, C, (X.dtype,), dev)
    nc = k * K + k * k
    phi_act = _f32(phi_act, "phi_act", (k * C, nc), dev)
    b_act = _f32(b_act, "b_act", (nc,), dev)
    idx_in = None if idx is None else _i32(idx, "idx", (T, k), dev)
    if idx_in is None:
        if w_router is None:
            raise ValueError("xhc_route needs idx or w_router")
        if not 1 <= m <= k <= N:
            raise ValueError(f"need 1 <= m <= k <= N, got m={m} k={k} N={N}")
        w_router = _f32(w_router, "w_router", (N * C, N - m), dev)
    else:
        w_router = None
    idx_out = torch.empty(T, k, dtype=torch.int32, device=dev)
    score = torch.empty(T, N - m, device=dev) if idx_in is None else None
    hp = torch.empty(T, k, K, device=dev) if want_coeffs else None
    hr = torch.empty(T, k, k, device=dev) if want_coeffs else None
    ws = _workspace(xhc_route_workspace_bytes(T, N, C, k, m, K, idx_in is None, X.dtype), dev, workspace)
    _check("xhc_route", lib().xhc_route(_ptr(X), _DT[X.dtype], T, N, C, k, m, _ptr(w_router), _ptr(idx_in),
                                        _ptr(phi_act), _ptr(b_act), float(alpha_post), float(alpha_res),
                                        int(sinkhorn_iters), _ptr(Wb), K, _ptr(idx_out), _ptr(score), _ptr(hp),
                                        _ptr(hr), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    res = dict(idx=idx_out)
    if score is not None:
        res["score"] = score
    if want_coeffs:
        res.update(h_post=hp, h_res=hr)
    return res


def xhc_chain_carry_bytes(T: int, N: int, C: int, k: int, m: int, dtype) -> int:
    """Bytes of the carry of the chained xHC calls, or -1 for a shape they do not cover."""
    return int(lib().xhc_chain_carry_bytes(T, N, C, k, m, _DT[dtype]))


def xhc_chain_workspace_bytes(T: int, N: int, C: int, k: int, m: int, K: int, dtype) -> int:
    return int(lib().xhc_chain_workspace_bytes(T, N, C, k, m, K, _DT[dtype]))


def _carry(t, name, nbytes, dev):
    if nbytes < 0:
        raise ValueError("the chained xHC calls do not cover this shape (bfloat16, N = 16, k = 4, m <= 4, "
                         "C a multiple of 512)")
    if t is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev)
    t = _dev_tensor(t, name, (torch.uint8,), device=dev)
    if _nbytes(t) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, needs {nbytes}")
    return t


def xhc_pre_chain(X, phi_pre, b_pre, alpha_pre, w_router, phi_pre_next, w_router_next, *, k=4, m=2,
                  carry_out=None, out=None, workspace=None, stream=None):
    """xhc_pre of the first sublayer of a chain, whose pre-read also forms the carry of
    the next sublayer's maps (phi_pre_next, w_router_next). out = (h_pre or None, F_in).
    Returns dict(h_pre, F_in, idx, score, carry)."""
    X = _state(X, dtypes=(torch.bfloat16,))
    T, N, C = X.shape
    dev = X.device
    if not 1 <= m <= k <= N:
        raise ValueError(f"need 1 <= m <= k <= N, got m={m} k={k} N={N}")
    phi_pre = _f32(phi_pre, "phi_pre", (N * C, N), dev)
    b_pre = _f32(b_pre, "b_pre", (N,), dev)
    w_router = _f32(w_router, "w_router", (N * C, N - m), dev)
    phi_pre_next = _f32(phi_pre_next, "phi_pre_next", (N * C, N), dev)
    w_router_next = _f32(w_router_next, "w_router_next", (N * C, N - m), dev)
    if out is not None:
        h_pre = None if out[0] is None else _f32(out[0], "h_pre out", (T, N), dev)
        F_in = _stream_out(out[1], "F_in out", (T, C), X.dtype, dev)
    else:
        h_pre = torch.empty(T, N, device=dev)
        F_in = torch.empty(T, C, dtype=X.dtype, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    score = torch.empty(T, N - m, device=dev)
    carry_out = _carry(carry_out, "carry_out", xhc_chain_carry_bytes(T, N, C, k, m, X.dtype), dev)
    ws = _workspace(xhc_chain_workspace_bytes(T, N, C, k, m, 1, X.dtype), dev, workspace)
    _check("xhc_pre_chain", lib().xhc_pre_chain(_ptr(X), _DT[X.dtype], T, N, C, k, m, _ptr(phi_pre), _ptr(b_pre),
                                                float(alpha_pre), _ptr(w_router), _ptr(phi_pre_next),
                                                _ptr(w_router_next), _ptr(h_pre), _ptr(F_in), _ptr(idx), _ptr(score),
                                                _ptr(carry_out), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    return dict(h_pre=h_pre, F_in=F_in, idx=idx, score=score, carry=carry_out)


def xhc_route_pre(X, Wb, phi_act, b_act, alpha_post, alpha_res, idx, carry, b_pre, alpha_pre,
                  *, phi_pre_next=None, w_router_next=None, carry_out=None, k=4, m=2, sinkhorn_iters=20,
                  want_coeffs=False, out=None, workspace=None, stream=None):
    """One chained step: xhc_route of sublayer l in place on X (active set idx, the
    carry written with it), then xhc_pre of sublayer l + 1 (b_pre, alpha_pre; its
    phi_pre and w_router came with the carry); with phi_pre_next and w_router_next
    (sublayer l + 2's maps) also the carry for the next call (carry_out may be `carry`
    itself). out = (h_pre or None, F_in). Returns dict(idx, score, h_pre, F_in,
    carry[, h_post, h_res])."""
    X = _state(X, dtypes=(torch.bfloat16,))
    T, N, C = X.shape
    dev = X.device
    if not 1 <= m <= k <= N:
        raise ValueError(f"need 1 <= m <= k <= N, got m={m} k={k} N={N}")
    Wb, K = _write_back(Wb, T, C, (X.dtype,), dev)
    nc = k * K + k * k
    phi_act = _f32(phi_act, "phi_act", (k * C, nc), dev)
    b_act = _f32(b_act, "b_act", (nc,), dev)
    idx = _i32(idx, "idx", (T, k), dev)
    b_pre = _f32(b_pre, "b_pre", (N,), dev)
    nbytes = xhc_chain_carry_bytes(T, N, C, k, m, X.dtype)
    if carry is None:
        raise ValueError("xhc_route_pre needs the carry written with idx (xhc_pre_chain or the previous call)")
    carry = _carry(carry, "carry", nbytes, dev)
    nxt = phi_pre_next is not None or w_router_next is not None
    if nxt:
        if phi_pre_next is None or w_router_next is None:
            raise ValueError("phi_pre_next and w_router_next go together")
        phi_pre_next = _f32(phi_pre_next, "phi_pre_next", (N * C, N), dev)
        w_router_next = _f32(w_router_next, "w_router_next", (N * C, N - m), dev)
        carry_out = _carry(carry_out, "carry_out", nbytes, dev)
    elif carry_out is not None:
        raise ValueError("carry_out needs the next sublayer's maps (phi_pre_next, w_router_next)")
    if out is not None:
        h_pre = None if out[0] is None else _f32(out[0], "h_pre out", (T, N), dev)
        F_in = _stream_out(out[1], "F_in out", (T, C), X.dtype, dev)
    else:
        h_pre = torch.empty(T, N, device=dev)
        F_in = torch.empty(T, C, dtype=X.dtype, device=dev)
    idx_out = torch.empty(T, k, dtype=torch.int32, device=dev)
    score = torch.empty(T, N - m, device=dev)
    hp = torch.empty(T, k, K, device=dev) if want_coeffs else None
    hr = torch.empty(T, k, k, device=dev) if want_coeffs else None
    ws = _workspace(xhc_chain_workspace_bytes(T, N, C, k, m, K, X.dtype), dev, workspace)
    _check("xhc_route_pre", lib().xhc_route_pre(
        _ptr(X), _DT[X.dtype], T, N, C, k, m, _ptr(idx), _ptr(phi_act), _ptr(b_act), float(alpha_post),
        float(alpha_res), int(sinkhorn_iters), _ptr(Wb), K, _ptr(b_pre), float(alpha_pre), _ptr(carry),
        _ptr(phi_pre_next), _ptr(w_router_next), _ptr(carry_out), _ptr(hp), _ptr(hr),
        _ptr(idx_out), _ptr(score), _ptr(h_pre), _ptr(F_in), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    res = dict(idx=idx_out, score=score, h_pre=h_pre, F_in=F_in, carry=carry_out)
    if want_coeffs:
        res.update(h_post=hp, h_res=hr)
    return res


def xhc_flash_pre_workspace_bytes(T: int, N: int, C: int, m: int, L: int, dtype) -> int:
    return int(lib().xhc_flash_pre_workspace_bytes(T, N, C, m, L, _DT[dtype]))


def xhc_flash_pre(X, phi_pre, b_pre, alpha_pre, w_router, *, k=4, m=2, out=None, workspace=None, stream=None):
    """xHC-Flash block entry: phi_pre [L, N*C, N], b_pre [L, N]. Returns (idx [T, k],
    score [T, N-m], h_pre [L, T, N], F_pre [L, T, C])."""
    X = _state(X)
    T, N, C = X.shape
    dev = X.device
    phi_pre = _f32(phi_pre, "phi_pre", device=dev)
    if phi_pre.dim() != 3 or tuple(phi_pre.shape[1:]) != (N * C, N):
        raise ValueError(f"phi_pre has shape {tuple(phi_pre.shape)}, expected (L, {N * C}, {N})")
    L = phi_pre.shape[0]
    b_pre = _f32(b_pre, "b_pre", (L, N), dev)
    if not 1 <= m <= k <= N:
        raise ValueError(f"need 1 <= m <= k <= N, got m={m} k={k} N={N}")
    w_router = _f32(w_router, "w_router", (N * C, N - m), dev)
    if out is None:
        out = (torch.empty(T, k, dtype=torch.int32, device=dev), torch.empty(T, N - m, device=dev),
               torch.empty(L, T, N, device=dev), torch.empty(L, T, C, dtype=X.dtype, device=dev))
    idx = _i32(out[0], "idx out", (T, k), dev)
    score = None if out[1] is None else _f32(out[1], "score out", (T, N - m), dev)
    h_pre = _f32(out[2], "h_pre out", (L, T, N), dev)
    F_pre = _stream_out(out[3], "F_pre out", (L, T, C), X.dtype, dev)
    ws = _workspace(xhc_flash_pre_workspace_bytes(T, N, C, m, L, X.dtype), dev, workspace)
    _check("xhc_flash_pre", lib().xhc_flash_pre(_ptr(X), _DT[X.dtype], T, N, C, k, m, L, _ptr(phi_pre),
                                                _ptr(b_pre), float(alpha_pre), _ptr(w_router), _ptr(idx), _ptr(score),
                                                _ptr(h_pre), _ptr(F_pre), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    return idx, score, h_pre, F_pre


def xhc_flash_maps_workspace_bytes(T: int, N: int, C: int, k: int, L: int, dtype, K_last: int = 1) -> int:
    return int(lib().xhc_flash_maps_workspace_bytes(T, N, C, k, L, K_last, _DT[dtype]))


def xhc_flash_maps(X, idx, phi_act, b_act, alpha_post, alpha_res, L, *, K_last=1, sinkhorn_iters=20, out=None,
                   workspace=None, stream=None):
    """The block's maps from X's active rows: returns (H_post [T, k, Kb], H_res [T, k, k]),
    Kb = L - 1 + K_last write-back components (K_last: the last sublayer's)."""
    X = _state(X)
    T, N, C = X.shape
    dev = X.device
    idx = _i32(idx, "idx", device=dev)
    if idx.dim() != 2 or idx.shape[0] != T:
        raise ValueError(f"idx has shape {tuple(idx.shape)}, expected ({T}, k)")
    k = idx.shape[1]
    Kb = L - 1 + K_last
    nc = k * Kb + k * k
    phi_act = _f32(phi_act, "phi_act", (k * C, nc), dev)
    b_act = _f32(b_act, "b_act", (nc,), dev)
    if out is None:
        out = (torch.empty(T, k, Kb, device=dev), torch.empty(T, k, k, device=dev))
    Hp = _f32(out[0], "H_post out", (T, k, Kb), dev)
    Hr = _f32(out[1], "H_res out", (T, k, k), dev)
    ws = _workspace(xhc_flash_maps_workspace_bytes(T, N, C, k, L, X.dtype, K_last), dev, workspace)
    _check("xhc_flash_maps", lib().xhc_flash_maps(_ptr(X), _DT[X.dtype], T, N, C, k, L, K_last, _ptr(idx),
                                                  _ptr(phi_act), _ptr(b_act), float(alpha_post), float(alpha_res),
                                                  int(sinkhorn_iters), _ptr(Hp), _ptr(Hr), _ptr(ws), _nbytes(ws),
                                                  _stream(dev, stream)))
    return Hp, Hr


def xhc_flash_input(l, F_pre_l, h_pre_l, idx, H_post, F_outs, *, K_last=1, N=None, out=None, stream=None):
    """Sublayer l's input from the entry-state read F_pre_l [T, C] and the block's
    write-back components F_outs [T, Kb, C] (rows j < l read; Kb = L - 1 + K_last, the
    width of H_post [T, k, Kb]). Returns F_in [T, C]."""
    F_pre_l = _dev_tensor(F_pre_l, "F_pre_l", _DT)
    if F_pre_l.dim() != 2:
        raise ValueError(f"F_pre_l must be [T, C], got shape {tuple(F_pre_l.shape)}")
    T, C = F_pre_l.shape
    dev = F_pre_l.device
    h_pre_l = _f32(h_pre_l, "h_pre_l", device=dev)
    if h_pre_l.dim() != 2 or h_pre_l.shape[0] != T:
        raise ValueError(f"h_pre_l has shape {tuple(h_pre_l.shape)}, expected ({T}, N)")
    if N is not None and h_pre_l.shape[1] != N:
        raise ValueError(f"h_pre_l has {h_pre_l.shape[1]} streams, expected N = {N}")
    N = h_pre_l.shape[1]
    H_post = _f32(H_post, "H_post", device=dev)
    if H_post.dim() != 3 or H_post.shape[0] != T:
        raise ValueError(f"H_post has shape {tuple(H_post.shape)}, expected ({T}, k, Kb)")
    k, Kb = H_post.shape[1], H_post.shape[2]
    L = Kb - K_last + 1
    idx = _i32(idx, "idx", (T, k), dev)
    F_outs = None if F_outs is None else _dev_tensor(F_outs, "F_outs", (F_pre_l.dtype,), (T, Kb, C), dev)
    F_in = _stream_out(out, "F_in out", (T, C), F_pre_l.dtype, dev)
    _check("xhc_flash_input", lib().xhc_flash_input(_DT[F_pre_l.dtype], T, N, C, k, L, K_last, int(l), _ptr(F_pre_l),
                                                    _ptr(h_pre_l), _ptr(idx), _ptr(H_post), _ptr(F_outs), _ptr(F_in),
                                                    _stream(dev, stream)))
    return F_in


def xhc_flash_post_workspace_bytes(T: int, k: int, L: int, K_last: int = 1) -> int:
    return int(lib().xhc_flash_post_workspace_bytes(T, k, L, K_last))


def xhc_flash_post(X, idx, H_post, H_res, F_outs, *, K_last=1, W_last=None, workspace=None, stream=None):
    """Block end in place on X [T, N, C] from the entry state's active rows and the
    write-back components F_outs [T, Kb, C] (the earlier sublayers' outputs, then the
    last sublayer's K_last components; Kb = H_post.shape[2]), or with the last
    sublayer's components in W_last [T, K_last, C] (F_outs' last K_last rows then
    unread). Returns X."""
    X = _state(X)
    T, N, C = X.shape
    dev = X.device
    H_post = _f32(H_post, "H_post", device=dev)
    if H_post.dim() != 3 or H_post.shape[0] != T:
        raise ValueError(f"H_post has shape {tuple(H_post.shape)}, expected ({T}, k, Kb)")
    k, Kb = H_post.shape[1], H_post.shape[2]
    L = Kb - K_last + 1
    idx = _i32(idx, "idx", (T, k), dev)
    H_res = _f32(H_res, "H_res", (T, k, k), dev)
    F_outs = _dev_tensor(F_outs, "F_outs", (X.dtype,), (T, Kb, C), dev)
    W_last = None if W_last is None else _dev_tensor(W_last, "W_last", (X.dtype,), (T, K_last, C), dev)
    ws = _workspace(xhc_flash_post_workspace_bytes(T, k, L, K_last), dev, workspace)
    _check("xhc_flash_post", lib().xhc_flash_post(_ptr(X), _DT[X.dtype], T, N, C, k, L, K_last, _ptr(idx),
                                                  _ptr(H_post), _ptr(H_res), _ptr(F_outs), _ptr(W_last), _ptr(ws),
                                                  _nbytes(ws), _stream(dev, stream)))
    return X


def xhc_augment_workspace_bytes(batch, seq, C, kappas, dtype, v_dtype=None) -> int:
    karr = (ctypes.c_int * max(len(kappas), 1))(*[int(x) for x in kappas])
    vdt = dtype if v_dtype is None else v_dtype
    return int(lib().xhc_augment_workspace_bytes(batch, seq, C, karr, len(kappas), _DT[dtype], _DT[vdt]))


def _conv_w(conv_w, kappas, C, dev):
    """The concatenated conv taps [C, kappa_1] | [C, kappa_2] | ... as one float32 vector."""
    w = _f32(conv_w, "conv_w", device=dev)
    need = C * sum(int(x) for x in kappas)
    if w.numel() != need:
        raise ValueError(f"conv_w has {w.numel()} values, expected C * sum(kappas) = {need}")
    return w


def xhc_augment(F_out, conv_w, kappas, batch, seq, *, v_dtype=None, out=None, workspace=None, stream=None):
    """V [T, r+1, C] = Gram-Schmidt([F_out; causal depthwise convs]); conv_w concatenated fp32."""
    F_out = _dev_tensor(F_out, "F_out", _DT)
    if F_out.dim() != 2:
        raise ValueError(f"F_out must be [T, C], got shape {tuple(F_out.shape)}")
    T, C = F_out.shape
    dev = F_out.device
    if T != batch * seq:
        raise ValueError("F_out rows must equal batch * seq")
    r = len(kappas)
    vdt = F_out.dtype if v_dtype is None else v_dtype
    if vdt not in _DT:
        raise TypeError(f"v_dtype {vdt} is not a stream dtype")
    V = _stream_out(out, "V out", (T, r + 1, C), vdt, dev)
    karr = (ctypes.c_int * max(r, 1))(*[int(x) for x in kappas])
    w = _conv_w(conv_w, kappas, C, dev) if r > 0 else None
    nbytes = int(lib().xhc_augment_workspace_bytes(batch, seq, C, karr, r, _DT[F_out.dtype], _DT[vdt]))
    if nbytes < 0:
        raise ValueError("invalid sizes for xhc_augment")
    ws = _workspace(nbytes, dev, workspace) if nbytes > 0 else None
    _check("xhc_augment", lib().xhc_augment(_ptr(F_out), _DT[F_out.dtype], batch, seq, C, _ptr(w), karr, r,
                                            _ptr(V), _DT[vdt], _ptr(ws), 0 if ws is None else _nbytes(ws),
                                            _stream(dev, stream)))
    return V


def hc_tanh_coeffs(X, theta, bias, alpha, *, out=None, stream=None):
    """HC's unconstrained maps (h_pre [T,n], h_post [T,n], h_res [T,n,n]) of X [T,n,C];
    theta [n+2, C] float32, bias [n*n+2n], alpha = (pre, post, res)."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    theta = _f32(theta, "theta", (n + 2, C), dev)
    bias = _f32(bias, "bias", (n * n + 2 * n,), dev)
    h_pre, h_post, h_res = _coeff_outs(out, T, n, dev)
    if h_pre is None:
        raise ValueError("hc_tanh_coeffs needs an h_pre output")
    a = [float(v) for v in alpha]
    _check("hc_tanh_coeffs", lib().hc_tanh_coeffs(_ptr(X), _DT[X.dtype], T, n, C, _ptr(theta), _ptr(bias), a[0],
                                                  a[1], a[2], _ptr(h_pre), _ptr(h_post), _ptr(h_res),
                                                  _stream(dev, stream)))
    return h_pre, h_post, h_res


def hc_amax_gain(h_res_layers, *, stream=None):
    """(forward gain [T], backward gain [T]) of the chain h_res_layers [L, T, n, n] (layer 0 first)."""
    H = _f32(h_res_layers, "h_res_layers")
    if H.dim() != 4 or H.shape[2] != H.shape[3]:
        raise ValueError(f"h_res_layers must be [L, T, n, n], got shape {tuple(H.shape)}")
    L, T, n, _ = H.shape
    fwd = torch.empty(T, device=H.device)
    bwd = torch.empty(T, device=H.device)
    _check("hc_amax_gain", lib().hc_amax_gain(_ptr(H), L, T, n, _ptr(fwd), _ptr(bwd), _stream(H.device, stream)))
    return fwd, bwd


def hc_static_maps(logits, n, sinkhorn_iters=20, *, stream=None):
    """Static mHC maps (h_pre [n], h_post [n], h_res [n, n]) from logits [n*n + 2n] float32."""
    z = _f32(logits, "logits", (n * n + 2 * n,))
    h_pre = torch.empty(n, device=z.device)
    h_post = torch.empty(n, device=z.device)
    h_res = torch.empty(n, n, device=z.device)
    _check("hc_static_maps", lib().hc_static_maps(_ptr(z), n, int(sinkhorn_iters), _ptr(h_pre), _ptr(h_post),
                                                  _ptr(h_res), _stream(z.device, stream)))
    return h_pre, h_post, h_res


def hc_static_pre(X, h_pre, *, out=None, stream=None):
    """F_in [T, C] = sum_i h_pre[i] X[:, i, :] with one h_pre [n] for every token."""
    X = _state(X)
    T, n, C = X.shape
    h_pre = _f32(h_pre, "h_pre", (n,), X.device)
    F_in = _stream_out(out, "F_in out", (T, C), X.dtype, X.device)
    _check("hc_static_pre", lib().hc_static_pre(_ptr(X), _DT[X.dtype], T, n, C, _ptr(h_pre), _ptr(F_in),
                                                _stream(X.device, stream)))
    return F_in


def hc_static_post(X, h_res, h_post, F_out, *, out=None, stream=None):
    """X_next [T, n, C] = h_res X[t] + h_post^T F_out[t] with maps shared by every token."""
    X = _state(X)
    T, n, C = X.shape
    dev = X.device
    h_res = _f32(h_res, "h_res", (n, n), dev)
    h_post = _f32(h_post, "h_post", (n,), dev)
    F_out = _dev_tensor(F_out, "F_out", (X.dtype,), (T, C), dev)
    Y = _stream_out(out, "X_next out", (T, n, C), X.dtype, dev)
    _check("hc_static_post", lib().hc_static_post(_ptr(X), _DT[X.dtype], T, n, C, _ptr(h_res), _ptr(h_post),
                                                  _ptr(F_out), _ptr(Y), _stream(dev, stream)))
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
    X = _state(X, dtypes=(torch.bfloat16,))
    T, N, C = X.shape
    dev = X.device
    idx = _i32(idx, "idx", device=dev)
    if idx.dim() != 2 or idx.shape[0] != T:
        raise ValueError(f"idx has shape {tuple(idx.shape)}, expected ({T}, k)")
    k = idx.shape[1]
    Wb, K = _write_back(Wb, T, C, (X.dtype,), dev)
    dX = _dev_tensor(dX, "dX", (X.dtype,), (T, N, C), dev)
    nc = k * K + k * k
    phi_act = _f32(phi_act, "phi_act", (k * C, nc), dev)
    b_act = _f32(b_act, "b_act", (nc,), dev)
    if out is None:
        dWb = (torch.empty(T, C, dtype=X.dtype, device=dev) if K == 1 else
               torch.empty(T, K, C, dtype=torch.float32, device=dev))
        out = (dWb, torch.empty(k * C, nc, device=dev), torch.empty(nc, device=dev), torch.empty(2, device=dev),
               torch.empty(T, nc, device=dev))
    if K == 1:
        dWb = _dev_tensor(out[0], "dWb out", (X.dtype,), (T, C), dev)
    else:
        dWb = _f32(out[0], "dWb out", (T, K, C), dev)
    dphi = _f32(out[1], "dphi out", (k * C, nc), dev)
    db = _f32(out[2], "db out", (nc,), dev)
    dalpha = _f32(out[3], "dalpha out", (2,), dev)
    dh = _f32(out[4], "dh out", (T, nc), dev)
    ws = _workspace(xhc_backward_workspace_bytes(T, N, C, k, K, X.dtype), dev, workspace)
    _check("xhc_route_backward", lib().xhc_route_backward(
        _ptr(X), _DT[X.dtype], T, N, C, k, _ptr(idx), _ptr(phi_act), _ptr(b_act), float(alpha_post),
        float(alpha_res), int(sinkhorn_iters), _ptr(Wb), K, _ptr(dX), _ptr(dWb), _ptr(dphi), _ptr(db), _ptr(dalpha),
        _ptr(dh), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    return dX, dWb, dphi, db, dalpha, dh


def xhc_pre_backward(X, phi_pre, b_pre, alpha_pre, dF_in, dX, *, out=None, workspace=None, stream=None):
    """Backward of xhc_pre's dense read (bfloat16): dX += its gradient (in place).
    Returns (dX, dphi_pre, db_pre, dalpha [1], dh_pre [T, N])."""
    X = _state(X, dtypes=(torch.bfloat16,))
    T, N, C = X.shape
    dev = X.device
    dF_in = _dev_tensor(dF_in, "dF_in", (X.dtype,), (T, C), dev)
    dX = _dev_tensor(dX, "dX", (X.dtype,), (T, N, C), dev)
    phi_pre = _f32(phi_pre, "phi_pre", (N * C, N), dev)
    b_pre = _f32(b_pre, "b_pre", (N,), dev)
    if out is None:
        out = (torch.empty(N * C, N, device=dev), torch.empty(N, device=dev), torch.empty(1, device=dev),
               torch.empty(T, N, device=dev))
    dphi = _f32(out[0], "dphi out", (N * C, N), dev)
    db = _f32(out[1], "db out", (N,), dev)
    dalpha = _f32(out[2], "dalpha out", (1,), dev)
    dh = _f32(out[3], "dh out", (T, N), dev)
    ws = _workspace(xhc_backward_workspace_bytes(T, N, C, 4, 1, X.dtype), dev, workspace)
    _check("xhc_pre_backward", lib().xhc_pre_backward(
        _ptr(X), _DT[X.dtype], T, N, C, _ptr(phi_pre), _ptr(b_pre), float(alpha_pre), _ptr(dF_in), _ptr(dX),
        _ptr(dphi), _ptr(db), _ptr(dalpha), _ptr(dh), _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    return dX, dphi, db, dalpha, dh


def xhc_augment_backward_workspace_bytes(B: int, S: int, C: int, kappas, dtype) -> int:
    k = (ctypes.c_int * len(kappas))(*[int(x) for x in kappas])
    return int(lib().xhc_augment_backward_workspace_bytes(B, S, C, k, len(kappas), _DT[dtype]))


def xhc_augment_backward(F_out, conv_w, kappas, B, S, dV, *, out=None, workspace=None, stream=None):
    """Backward of xhc_augment (kappas (4, 8, 12)): dV [T, 4, C] float32 in; returns
    (dF_out [T, C] in F_out's dtype, dconv_w in conv_w's layout)."""
    F_out = _dev_tensor(F_out, "F_out", _DT)
    if F_out.dim() != 2 or F_out.shape[0] != B * S:
        raise ValueError(f"F_out has shape {tuple(F_out.shape)}, expected ({B * S}, C)")
    T, C = F_out.shape
    dev = F_out.device
    r = len(kappas)
    dV = _f32(dV, "dV", (T, r + 1, C), dev)
    conv_w = _conv_w(conv_w, kappas, C, dev)
    if out is None:
        out = (torch.empty_like(F_out), torch.empty_like(conv_w))
    dF = _stream_out(out[0], "dF_out out", (T, C), F_out.dtype, dev)
    dw = _f32(out[1], "dconv_w out", tuple(conv_w.shape), dev)
    k = (ctypes.c_int * max(r, 1))(*[int(x) for x in kappas])
    nbytes = xhc_augment_backward_workspace_bytes(B, S, C, kappas, F_out.dtype)
    if nbytes < 0:
        raise ValueError("invalid sizes for xhc_augment_backward")
    ws = _workspace(nbytes, dev, workspace)
    _check("xhc_augment_backward", lib().xhc_augment_backward(
        _ptr(F_out), _DT[F_out.dtype], B, S, C, _ptr(conv_w), k, r, _ptr(dV), _ptr(dF), _ptr(dw),
        _ptr(ws), _nbytes(ws), _stream(dev, stream)))
    return dF, dw


def hc_copy_probe(src, dst, *, stream=None):
    """Copy src into dst (same byte size, 16-byte aligned) with the library's streaming
    copy: a measurement probe of the device's streaming rate, not part of the method."""
    src = _dev_tensor(src, "src")
    dst = _dev_tensor(dst, "dst", device=src.device)
    if _nbytes(dst) != _nbytes(src):
        raise ValueError("hc_copy_probe needs contiguous tensors of the same byte size")
    _check("hc_copy_probe", lib().hc_copy_probe(_ptr(src), _ptr(dst), _nbytes(src), _stream(src.device, stream)))
    return dst


__all__ = [
    "LIB_PATH", "HCError", "lib", "status_string", "hc_coeffs_workspace_bytes", "hc_coeffs", "hc_pre",
    "hc_coeffs_pre", "hc_post", "hc_backward_workspace_bytes", "hc_backward_post", "hc_backward", "xhc_backward_workspace_bytes",
    "xhc_route_backward", "xhc_pre_backward", "xhc_augment_backward_workspace_bytes", "xhc_augment_backward", "hc_post_coeffs", "hc_phi_packed_bytes", "hc_phi_pack", "hc_post_pre",
    "hc_post_pre_noalloc", "HC_NOALLOC_SCRATCH_BYTES",
    "xhc_pre_workspace_bytes", "xhc_pre", "xhc_route_workspace_bytes",
    "xhc_route", "xhc_chain_carry_bytes", "xhc_chain_workspace_bytes", "xhc_pre_chain", "xhc_route_pre",
    "xhc_augment_workspace_bytes", "xhc_augment", "xhc_flash_pre_workspace_bytes", "xhc_flash_pre",
    "xhc_flash_maps_workspace_bytes", "xhc_flash_maps", "xhc_flash_input", "xhc_flash_post_workspace_bytes",
    "xhc_flash_post", "hc_tanh_coeffs", "hc_amax_gain",
    "hc_static_maps", "hc_static_pre", "hc_static_post", "hc_copy_probe",
]
