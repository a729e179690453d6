"""GPU parity of hc_backward (gradients of one mHC sublayer, n = 4 bfloat16)
against the fp64 oracle's mhc_sublayer_backward, through the C ABI, on the synth
recipe's inputs and upstream gradients.

The two stages run as a training step runs them: hc_backward_post (dF_out and
the map gradients dH_post, dH_res, with the forward's h_post) and then
hc_backward with dF_in.

Tolerances. dX and dF_out are bfloat16 outputs rounded once from float32: the
stream bound of the forward tests (relative L2 1e-2, per element max(2e-2, one
bf16 ulp)). The map gradients dh are float32 sums over the channels (relative
L2 1e-4 as below). dphi, dbias and dalpha are float32 sums over the tokens of
per-token gradients. Each of those carries float32 sums over the 4C channels,
20 Sinkhorn steps in reverse and, for dphi, dP split into two bfloat16 parts on
the matrix cores (16 significant bits, 2^-17 relative per element). That gives
relative L2 errors of order 1e-5; the bound is 1e-4.
"""
import numpy as np
import pytest

import oracle as O
import synth
from hc_testutil import check_bf16, check_fp32, dev, have_gpu, host64, note

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc

BWD_REL = 1e-4


def _inputs(seed, T, C, alpha=None, phi_scale=1.0):
    inp = synth.mhc_layer(seed, 0, T, 4, C, synth.BF16)
    g = synth.mhc_grads(seed, 0, T, 4, C, synth.BF16)
    if alpha is not None:
        inp["alpha"] = np.array(alpha, np.float32)
    if phi_scale != 1.0:
        inp["phi"] = (inp["phi"] * np.float32(phi_scale)).astype(np.float32)
    return inp, g


def _gpu(inp, g, iters=20):
    """Forward coefficients, then the two backward stages as a training step runs
    them: the post stage (dF_out, dH_post, dH_res), then the main stage with dF_in."""
    X = dev(inp["X"])
    phi, bias = dev(inp["phi"]), dev(inp["bias"])
    alpha = [float(a) for a in inp["alpha"]]
    _, h_post, _ = hc.hc_coeffs(X, phi, bias, alpha, iters)
    dXn = dev(g["dX_next"])
    dF_out, dh = hc.hc_backward_post(X, h_post, dev(inp["F_out"]), dXn)
    dX, dphi, dbias, dalpha = hc.hc_backward(X, phi, bias, alpha, dXn, dev(g["dF_in"]), dh, iters)
    torch.cuda.synchronize()
    return dict(dX=host64(dX), dF_out=host64(dF_out), dphi=host64(dphi), dbias=host64(dbias), dalpha=host64(dalpha),
                dh=host64(dh))


def _oracle(inp, g, iters=20, rows=None, chunk=None):
    """The oracle on all tokens (chunk: that many at a time, the token sums added
    over the chunks); rows: the tokens whose dX and dF_out are kept."""
    T = inp["X"].values.shape[0]
    chunk = chunk or T
    keep = np.arange(T) if rows is None else np.asarray(rows)
    out = dict(dphi=0.0, dbias=0.0, dalpha=0.0, dX=[], dF_out=[], dh=[])
    for s in range(0, T, chunk):
        sl = slice(s, min(T, s + chunk))
        r = O.mhc_sublayer_backward(inp["X"].values[sl], inp["phi"], inp["bias"], inp["alpha"],
                                    inp["F_out"].values[sl], g["dX_next"].values[sl], g["dF_in"].values[sl],
                                    iters)
        for k in ("dphi", "dbias", "dalpha"):
            out[k] = out[k] + r[k]
        sel = keep[(keep >= sl.start) & (keep < sl.stop)] - sl.start
        for k in ("dX", "dF_out", "dh"):
            out[k].append(r[k][sel])
    for k in ("dX", "dF_out", "dh"):
        out[k] = np.concatenate(out[k])
    return out


def _compare(got, ref, rows=None):
    sel = slice(None) if rows is None else np.asarray(rows)
    check_bf16("dX", got["dX"][sel], ref["dX"])
    check_bf16("dF_out", got["dF_out"][sel], ref["dF_out"])
    check_fp32("dh", got["dh"][sel], ref["dh"], BWD_REL)
    errs = {k: check_fp32(k, got[k], ref[k], BWD_REL) for k in ("dphi", "dbias", "dalpha")}
    note(f"relative L2: {', '.join(f'{k} {v:.2e}' for k, v in errs.items())}")


@pytest.mark.parametrize("T,C", [(70, 256), (33, 96), (64, 4096), (1, 32), (129, 160), (32 * 700 + 5, 256)])
def test_backward_shapes(T, C):
    """Ragged T (not a multiple of the 32-token tiles and 64-token items), C not a
    multiple of the 128-channel chunks, one token, the workload's C; at 22,405
    tokens each workgroup of the dX pass walks several tiles (its dphi partial
    summing them) and ends on the ragged one."""
    note(f"hc_backward n=4 C={C} T={T} bf16")
    inp, g = _inputs(400 + T, T, C)
    _compare(_gpu(inp, g), _oracle(inp, g))


@pytest.mark.parametrize("iters", [1, 5, 64])
def test_backward_sinkhorn_iterations(iters):
    """The on-chip Sinkhorn recompute for 1, 5 and the largest supported count."""
    note(f"hc_backward iters={iters} C=128 T=40")
    inp, g = _inputs(410 + iters, 40, 128, alpha=(0.3, 0.4, 0.5), phi_scale=5.0)
    _compare(_gpu(inp, g, iters), _oracle(inp, g, iters))


def test_backward_strong_gates():
    """Gates and phi large enough that the sigmoids and Sinkhorn are far from their
    values at z = b, so every gradient path carries weight."""
    note("hc_backward strong gates C=512 T=96")
    inp, g = _inputs(420, 96, 512, alpha=(0.8, 0.6, 1.0), phi_scale=10.0)
    _compare(_gpu(inp, g), _oracle(inp, g))


def test_backward_zero_state_tokens():
    """All-zero states (1/r taken as 0) next to ordinary ones."""
    note("hc_backward zero-state tokens C=256 T=50")
    inp, g = _inputs(430, 50, 256)
    z = np.array([0, 7, 31, 32, 49])
    vals = inp["X"].values.copy()
    vals[z] = 0.0
    inp["X"] = synth.Tensor(vals, synth.BF16)
    _compare(_gpu(inp, g), _oracle(inp, g))


def test_backward_deterministic():
    """Every sum runs in a fixed order: two runs give the same bits."""
    note("hc_backward determinism C=1024 T=300")
    inp, g = _inputs(440, 300, 1024)
    a, b = _gpu(inp, g), _gpu(inp, g)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_backward_full_size():
    """The n = 4, C = 4096, T = 8192 workload in one call: dphi, dbias and dalpha
    against the oracle over every token (in chunks of 512), dX and dF_out on
    sampled tokens."""
    w = synth.WORKLOADS["mhc_n4_C4096_T8192_bf16"]
    T, C = w["T"], w["C"]
    note(f"hc_backward full size n=4 C={C} T={T} bf16")
    inp = synth.mhc_layer(w["seed"], 0, T, 4, C, synth.BF16)
    g = synth.mhc_grads(w["seed"], 0, T, 4, C, synth.BF16)
    got = _gpu(inp, g)
    rng = np.random.default_rng(450)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 254, replace=False)]))
    _compare(got, _oracle(inp, g, rows=rows, chunk=512), rows=rows)
