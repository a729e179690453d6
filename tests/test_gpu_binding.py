"""The Python binding checks every tensor it hands to the C ABI (device,
contiguity, dtype and exact shape, including caller-supplied outputs and
workspaces) and raises before any launch: an undersized buffer must never reach
a kernel as a raw pointer. Each case passes one wrong argument; the library is
loaded but no kernel runs."""
import numpy as np
import pytest

from hc_testutil import have_gpu, note

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc


def _mhc(T=8, n=4, C=64, dtype=None):
    dev = "cuda"
    dtype = dtype or torch.bfloat16
    return dict(X=torch.zeros(T, n, C, dtype=dtype, device=dev), phi=torch.zeros(n * C, n * n + 2 * n, device=dev),
                bias=torch.zeros(n * n + 2 * n, device=dev), h_pre=torch.zeros(T, n, device=dev),
                h_post=torch.zeros(T, n, device=dev), h_res=torch.zeros(T, n, n, device=dev),
                F=torch.zeros(T, C, dtype=dtype, device=dev))


def _raises(exc, fn, *a, **k):
    torch.cuda.synchronize()
    with pytest.raises(exc):
        fn(*a, **k)


def test_mhc_calls_reject_wrong_shapes_and_outputs():
    note("binding validation: mHC calls")
    d = _mhc()
    X, phi, bias, F = d["X"], d["phi"], d["bias"], d["F"]
    a = [0.01] * 3
    _raises(ValueError, hc.hc_post, X, d["h_res"], d["h_post"], F[:, :32].contiguous())  # F_out [T, C/2]
    _raises(ValueError, hc.hc_post, X, d["h_res"][:, :2].contiguous(), d["h_post"], F)
    _raises(ValueError, hc.hc_post, X, d["h_res"], d["h_post"][:4], F)
    _raises(ValueError, hc.hc_post, X, d["h_res"], d["h_post"], F, out=torch.empty_like(X)[:4])
    _raises(TypeError, hc.hc_post, X, d["h_res"], d["h_post"], F, out=torch.empty(X.shape, device="cuda"))
    _raises(ValueError, hc.hc_coeffs, X, phi[:-1], bias, a)
    _raises(ValueError, hc.hc_coeffs, X, phi, bias[:-1], a)
    _raises(ValueError, hc.hc_coeffs, X, phi, bias, a, out=(d["h_pre"], d["h_post"], d["h_res"][:1]))
    _raises(TypeError, hc.hc_pre, X, d["h_pre"], out=torch.empty(8, 64, device="cuda"))  # F_in of the wrong dtype
    _raises(ValueError, hc.hc_pre, X, d["h_pre"].t().contiguous())
    _raises(ValueError, hc.hc_pre, X.transpose(0, 1), d["h_pre"])  # not contiguous
    _raises(ValueError, hc.hc_coeffs_pre, X, phi, bias, a,
            out=(d["h_pre"], d["h_post"], d["h_res"], torch.empty(8, 32, dtype=X.dtype, device="cuda")))
    _raises(ValueError, hc.hc_post_coeffs, X, d["h_res"], d["h_post"], F, phi[:, :20].contiguous(), bias, a)
    _raises(ValueError, hc.hc_post_pre, X, d["h_res"], d["h_post"], F, phi, bias, a,
            F_in_out=torch.empty(8, 63, dtype=X.dtype, device="cuda"))
    _raises(ValueError, hc.hc_post_pre, X, d["h_res"], d["h_post"], F, phi, bias, a,
            phi_next_packed=torch.empty(16, dtype=torch.uint8, device="cuda"))
    _raises(ValueError, hc.hc_phi_pack, phi[:10], 4, 64)
    _raises(ValueError, hc.hc_coeffs, torch.zeros(8, 256, dtype=torch.bfloat16, device="cuda"), phi, bias, a)
    _raises(TypeError, hc.hc_coeffs, X.cpu(), phi, bias, a)


def test_backward_and_static_calls_reject_wrong_shapes():
    note("binding validation: backward and static calls")
    d = _mhc(C=64)
    X, F = d["X"], d["F"]
    dXn = torch.zeros_like(X)
    _raises(ValueError, hc.hc_backward_post, X, d["h_post"], F, dXn[:4])
    dh = torch.zeros(8, 24, device="cuda")
    _raises(ValueError, hc.hc_backward, X, d["phi"], d["bias"], [0.01] * 3, dXn, F, dh[:, :20].contiguous())
    _raises(ValueError, hc.hc_backward, X, d["phi"], d["bias"], [0.01] * 3, dXn, F[:, :8].contiguous(), dh)
    _raises(ValueError, hc.hc_static_pre, X, torch.zeros(5, device="cuda"))
    _raises(ValueError, hc.hc_static_post, X, torch.zeros(4, 3, device="cuda"), torch.zeros(4, device="cuda"), F)
    _raises(ValueError, hc.hc_tanh_coeffs, X, torch.zeros(6, 32, device="cuda"), d["bias"], [0.01] * 3)
    _raises(ValueError, hc.hc_static_maps, torch.zeros(23, device="cuda"), 4)
    _raises(ValueError, hc.hc_amax_gain, torch.zeros(2, 8, 4, 3, device="cuda"))
    _raises(ValueError, hc.hc_copy_probe, torch.zeros(64, device="cuda"), torch.zeros(32, device="cuda"))


def test_xhc_calls_reject_wrong_shapes():
    note("binding validation: xHC calls")
    T, N, C, k, m = 8, 8, 64, 4, 2
    X = torch.zeros(T, N, C, dtype=torch.bfloat16, device="cuda")
    phi_pre = torch.zeros(N * C, N, device="cuda")
    b_pre = torch.zeros(N, device="cuda")
    W = torch.zeros(N * C, N - m, device="cuda")
    _raises(ValueError, hc.xhc_pre, X, phi_pre[:, :4].contiguous(), b_pre, 0.01, W, k, m)
    _raises(ValueError, hc.xhc_pre, X, phi_pre, b_pre, 0.01, W[:, :3].contiguous(), k, m)
    _raises(ValueError, hc.xhc_pre, X, phi_pre, b_pre, 0.01, W, k, m,
            out=(None, torch.empty(T, C // 2, dtype=X.dtype, device="cuda")))
    F = torch.zeros(T, C, dtype=X.dtype, device="cuda")
    phi_act = torch.zeros(k * C, k + k * k, device="cuda")
    b_act = torch.zeros(k + k * k, device="cuda")
    idx = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    _raises(ValueError, hc.xhc_route, X, F[:, :32].contiguous(), phi_act, b_act, 0.01, 0.01, k=k, m=m, idx=idx)
    _raises(ValueError, hc.xhc_route, X, F, phi_act, b_act, 0.01, 0.01, k=k, m=m, idx=idx[:, :3].contiguous())
    _raises(TypeError, hc.xhc_route, X, F, phi_act, b_act, 0.01, 0.01, k=k, m=m, idx=idx.long())
    _raises(ValueError, hc.xhc_route, X, torch.zeros(T, 4, C, dtype=X.dtype, device="cuda"), phi_act, b_act, 0.01,
            0.01, k=k, m=m, idx=idx)  # K = 4 components against phi_act for K = 1
    _raises(ValueError, hc.xhc_route, X, F, phi_act, b_act, 0.01, 0.01, k=k, m=m)  # neither idx nor router
    w = torch.zeros(C * 24, device="cuda")
    _raises(ValueError, hc.xhc_augment, F, w[:-1], (4, 8, 12), 2, 4)
    _raises(ValueError, hc.xhc_augment, F, w, (4, 8, 12), 3, 4)
    _raises(ValueError, hc.xhc_augment, F, w, (4, 8, 12), 2, 4,
            out=torch.empty(T, 3, C, dtype=X.dtype, device="cuda"))
    _raises(ValueError, hc.xhc_augment_backward, F, w, (4, 8, 12), 2, 4, torch.zeros(T, 4, C - 1, device="cuda"))
    Hp = torch.zeros(T, k, 2, device="cuda")
    Hr = torch.zeros(T, k, k, device="cuda")
    Fo = torch.zeros(T, 2, C, dtype=X.dtype, device="cuda")
    _raises(ValueError, hc.xhc_flash_post, X, idx, Hp, Hr, Fo[:, :1].contiguous())
    _raises(ValueError, hc.xhc_flash_post, X, idx, Hp, Hr[:, :3].contiguous(), Fo)
    _raises(ValueError, hc.xhc_flash_input, 1, F, torch.zeros(T, N, device="cuda"), idx, Hp, Fo[:4])
    _raises(ValueError, hc.xhc_flash_pre, X, phi_pre, b_pre, 0.01, W)  # phi_pre without the L axis
    _raises(ValueError, hc.xhc_flash_maps, X, idx, torch.zeros(k * C, k, device="cuda"),
            torch.zeros(k * 2 + k * k, device="cuda"), 0.01, 0.01, 2)


def test_valid_call_still_runs_after_rejections():
    note("binding validation: a valid call after the rejections")
    d = _mhc(T=3, C=64, dtype=torch.float32)
    X = torch.randn(3, 4, 64, device="cuda")
    Y = hc.hc_post(X, torch.eye(4, device="cuda").expand(3, 4, 4).contiguous(), torch.zeros(3, 4, device="cuda"),
                   torch.zeros(3, 64, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(Y, X)
    ws = torch.empty(4, dtype=torch.uint8, device="cuda")  # too small: the binding allocates its own
    h = hc.hc_coeffs(X, d["phi"], d["bias"], [0.01] * 3, workspace=ws)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(h[2].cpu().numpy()))
