"""GPU parity of the HC baseline maps (mHC notes Eq. 5), the Amax gain
diagnostic (section 3.1) and static mHC (the mHC-SSM abstract) against the fp64
oracle, through the C ABI; the HC maps applied with the mHC pre-read and post
calls."""
import numpy as np
import pytest

import oracle as O
import synth
from hc_testutil import check_bf16, check_fp32, check_stream, dev, have_gpu, host64, note

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc


def _hc_inputs(seed, T, n, C, dtype):
    rng = np.random.default_rng(seed)
    X = synth.Tensor(rng.standard_normal((T, n, C)).astype(np.float32), dtype)
    theta = (0.02 * rng.standard_normal((n + 2, C))).astype(np.float32)
    bias = rng.standard_normal(n * n + 2 * n).astype(np.float32)
    F = synth.Tensor(rng.standard_normal((T, C)).astype(np.float32), dtype)
    return X, theta, bias, F


@pytest.mark.parametrize("n,C,T,dtype", [(4, 256, 512, synth.F32), (4, 4096, 133, synth.BF16),
                                         (1, 64, 7, synth.F32), (3, 100, 19, synth.BF16),
                                         (16, 96, 5, synth.F32), (8, 4096, 30, synth.BF16)])
def test_hc_tanh_coeffs_and_apply(n, C, T, dtype):
    note(f"HC tanh maps n={n} C={C} T={T} dtype={dtype}")
    X, theta, bias, F = _hc_inputs(300 + n, T, n, C, dtype)
    Xv = X.values.copy()
    Xv[T // 2, n - 1] = 0.0  # a zero stream row: its maps are the biases
    X = synth.Tensor(Xv, dtype)
    alpha = (0.6, 0.8, 1.2)
    hp, hq, hr = hc.hc_tanh_coeffs(dev(X), dev(theta), dev(bias), alpha)
    torch.cuda.synchronize()
    rp, rq, rr = O.hc_tanh_coeffs(X.values, theta, bias, alpha)
    check_fp32("h_pre", host64(hp), rp)
    check_fp32("h_post", host64(hq), rq)
    check_fp32("h_res", host64(hr), rr)
    np.testing.assert_array_equal(host64(hr)[T // 2, :, n - 1], bias[2 * n:].reshape(n, n)[:, n - 1])
    # applied with the mHC kernels: pre-read and post/res write of the HC maps
    F_in = hc.hc_pre(dev(X), hp)
    Xn = hc.hc_post(dev(X), hr, hq, dev(F))
    torch.cuda.synchronize()
    check_stream("F_in", dtype, host64(F_in), O.hc_pre(X.values, host64(hp)))
    check_stream("X_next", dtype, host64(Xn), O.hc_post(X.values, host64(hr), host64(hq), F.values))


@pytest.mark.parametrize("L,T,n", [(8, 300, 4), (1, 17, 1), (3, 65, 7), (5, 40, 16), (0, 9, 4)])
def test_amax_gain_parity(L, T, n):
    note(f"Amax gain L={L} T={T} n={n}")
    rng = np.random.default_rng(400 + L * 17 + n)
    H = (np.eye(n) + 0.3 * rng.standard_normal((L, T, n, n))).astype(np.float32)
    f, g = hc.hc_amax_gain(torch.from_numpy(H).cuda())
    torch.cuda.synchronize()
    rf, rg = O.amax_gain(H) if L > 0 else (np.ones(T), np.ones(T))
    check_fp32("gain_fwd", host64(f), rf)
    check_fp32("gain_bwd", host64(g), rg)


def test_gain_of_mhc_chain_is_one_and_hc_chain_drifts():
    """The diagnostic on chains of maps the library computes: 8 layers of mHC
    h_res (Sinkhorn, rows normalised last) keep the forward gain at 1; HC's
    unconstrained tanh maps of the same states do not."""
    T, n, C, L = 256, 4, 512, 8
    rng = np.random.default_rng(500)
    hs_m, hs_h = [], []
    for layer in range(L):
        inp = synth.mhc_layer(600 + layer, 0, T, n, C, synth.F32)
        X = dev(inp["X"])
        hs_m.append(hc.hc_coeffs(X, dev(inp["phi"]), dev(inp["bias"]), [0.5, 0.5, 2.0])[2])
        theta = (0.05 * rng.standard_normal((n + 2, C))).astype(np.float32)
        bias = np.concatenate([np.zeros(2 * n), np.eye(n).reshape(-1)]).astype(np.float32)
        hs_h.append(hc.hc_tanh_coeffs(X, dev(theta), dev(bias), (0.5, 0.5, 0.5))[2])
    fm, bm = hc.hc_amax_gain(torch.stack(hs_m))
    fh, bh = hc.hc_amax_gain(torch.stack(hs_h))
    torch.cuda.synchronize()
    rf, rb = O.amax_gain(np.stack([host64(h) for h in hs_m]))
    check_fp32("mHC gain_fwd", host64(fm), rf)
    assert np.abs(host64(fm) - 1.0).max() < 1e-5
    note(f"HC forward gain: max {float(fh.max()):.3f}, mHC forward gain: max {float(fm.max()):.6f}")
    assert float(fh.max()) > 1.05


@pytest.mark.parametrize("n,C,T,dtype", [(4, 4096, 133, synth.BF16), (4, 256, 512, synth.F32),
                                         (1, 64, 9, synth.F32), (7, 100, 21, synth.BF16), (16, 64, 5, synth.F32)])
def test_static_mhc_maps_and_apply(n, C, T, dtype):
    note(f"static mHC n={n} C={C} T={T} dtype={dtype}")
    rng = np.random.default_rng(700 + n)
    z = (2.0 * rng.standard_normal(n * n + 2 * n)).astype(np.float32)
    hp, hq, hr = hc.hc_static_maps(torch.from_numpy(z).cuda(), n, 20)
    torch.cuda.synchronize()
    rp, rq, rr = O.static_mhc_maps(z, n, 20)
    check_fp32("static h_pre", host64(hp), rp)
    check_fp32("static h_post", host64(hq), rq)
    check_fp32("static h_res", host64(hr), rr)
    X = synth.Tensor(rng.standard_normal((T, n, C)).astype(np.float32), dtype)
    F = synth.Tensor(rng.standard_normal((T, C)).astype(np.float32), dtype)
    F_in = hc.hc_static_pre(dev(X), hp)
    Xn = hc.hc_static_post(dev(X), hr, hq, dev(F))
    Xd = dev(X)
    hc.hc_static_post(Xd, hr, hq, dev(F), out=Xd)  # in place
    torch.cuda.synchronize()
    check_stream("static F_in", dtype, host64(F_in), O.static_pre(X.values, host64(hp)))
    ref = O.static_post(X.values, host64(hr), host64(hq), F.values)
    check_stream("static X_next", dtype, host64(Xn), ref)
    np.testing.assert_array_equal(host64(Xd), host64(Xn))
