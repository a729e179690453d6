"""GPU parity of the mHC calls (hc_coeffs, hc_pre, hc_coeffs_pre, hc_post) against
the fp64 oracle, through the C ABI. Inputs come from the seeded synth recipe;
the oracle always sees the same (stream-dtype rounded) values as the GPU."""
import numpy as np
import pytest

import oracle as O
import synth
from hc_testutil import (check_bf16, check_fp32, check_stream, dev, have_gpu, host64, note,
                         rel_l2)

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc


def _run_sublayer(inp, fused=True, iters=20):
    X = dev(inp["X"])
    phi, bias = dev(inp["phi"]), dev(inp["bias"])
    alpha = [float(a) for a in inp["alpha"]]
    if fused:
        h_pre, h_post, h_res, F_in = hc.hc_coeffs_pre(X, phi, bias, alpha, iters)
    else:
        h_pre, h_post, h_res = hc.hc_coeffs(X, phi, bias, alpha, iters)
        F_in = hc.hc_pre(X, h_pre)
    X_next = hc.hc_post(X, h_res, h_post, dev(inp["F_out"]))
    torch.cuda.synchronize()
    return dict(h_pre=host64(h_pre), h_post=host64(h_post), h_res=host64(h_res), F_in=host64(F_in),
                X_next=host64(X_next))


def _compare_all(got, ref, dtype, literal=False):
    for k in ("h_pre", "h_post", "h_res"):
        check_fp32(k, got[k], ref[k])
    check_stream("F_in", dtype, got["F_in"], ref["F_in"], literal)
    check_stream("X_next", dtype, got["X_next"], ref["X_next"], literal)
    # Sinkhorn sums of the GPU coefficients
    assert np.max(np.abs(got["h_res"].sum(-1) - 1)) < 1e-6
    assert np.max(np.abs(got["h_res"].sum(-2) - 1)) < 1e-6


def _oracle(inp, iters=20):
    return O.mhc_sublayer(inp["X"].values, inp["phi"], inp["bias"], inp["alpha"], inp["F_out"].values, iters)


@pytest.mark.parametrize("fused", [True, False])
def test_mhc_n4_C256_T512_fp32_full(fused):
    w = synth.WORKLOADS["mhc_n4_C256_T512_f32"]
    note(f"mHC n=4 C=256 T=512 fp32 fused={fused}")
    inp = synth.mhc_layer(0, 0, w["T"], w["n"], w["C"], w["dtype"])
    _compare_all(_run_sublayer(inp, fused), _oracle(inp), synth.F32)


@pytest.mark.parametrize("T", [1, 7, 133])
@pytest.mark.parametrize("fused", [True, False])
def test_mhc_n4_C4096_bf16_ragged_T(T, fused):
    note(f"mHC n=4 C=4096 bf16 T={T} fused={fused}")
    inp = synth.mhc_layer(1, 0, T, 4, 4096, synth.BF16)
    _compare_all(_run_sublayer(inp, fused), _oracle(inp), synth.BF16, literal=True)


def test_mhc_n4_C4096_T8192_bf16_full_size_sampled():
    """Full-size run (T=8192, the benchmarked launch); oracle on sampled tokens,
    invariants on every token."""
    w = synth.WORKLOADS["mhc_n4_C4096_T8192_bf16"]
    note("mHC full size (n=4 C=4096 T=8192 bf16)")
    inp = synth.mhc_layer(1, 0, w["T"], w["n"], w["C"], w["dtype"])
    got = _run_sublayer(inp, fused=True)
    rng = np.random.default_rng(101)
    sample = np.unique(np.concatenate([[0, w["T"] - 1], rng.choice(w["T"], 254, replace=False)]))
    sub = dict(inp)
    sub["X"] = synth.Tensor(inp["X"].values[sample], synth.BF16)
    sub["F_out"] = synth.Tensor(inp["F_out"].values[sample], synth.BF16)
    ref = _oracle(sub)
    _compare_all({k: v[sample] for k, v in got.items()}, ref, synth.BF16, literal=True)
    h = got["h_res"]
    assert np.all(h >= 0)
    assert np.max(np.abs(h.sum(-1) - 1)) < 1e-6 and np.max(np.abs(h.sum(-2) - 1)) < 1e-6
    assert np.all((got["h_pre"] > 0) & (got["h_pre"] < 1))
    assert np.all((got["h_post"] > 0) & (got["h_post"] < 2))


@pytest.mark.parametrize("n,C,dtype", [(1, 64, synth.F32), (2, 100, synth.BF16), (3, 40, synth.F32),
                                       (4, 100, synth.BF16), (4, 24, synth.F32), (8, 96, synth.BF16),
                                       (16, 33, synth.F32), (5, 512, synth.BF16)])
def test_other_stream_counts_and_ragged_channels(n, C, dtype):
    note(f"mHC n={n} C={C} {dtype} T=37")
    inp = synth.mhc_layer(7, n, 37, n, C, dtype)
    _compare_all(_run_sublayer(inp, fused=True), _oracle(inp), dtype)
    _compare_all(_run_sublayer(inp, fused=False), _oracle(inp), dtype)


def test_n1_is_plain_residual_bit_exact():
    # n = 1: H_res = [1]; with supplied h_post = 1 the post write is x + F_out (Eq. 1).
    note("mHC n=1 plain residual fp32")
    rng = np.random.default_rng(5)
    X = rng.standard_normal((9, 1, 64)).astype(np.float32)
    F = rng.standard_normal((9, 64)).astype(np.float32)
    Y = hc.hc_post(dev(X), dev(np.ones((9, 1, 1))), dev(np.ones((9, 1))), dev(F))
    np.testing.assert_array_equal(Y.cpu().numpy(), (X.astype(np.float64) + F[:, None, :]).astype(np.float32))
    inp = synth.mhc_layer(8, 0, 9, 1, 64, synth.F32)
    _, _, h_res = hc.hc_coeffs(dev(inp["X"]), dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    assert np.all(h_res.cpu().numpy() == 1.0)


def test_post_in_place():
    note("mHC post in place bf16")
    inp = synth.mhc_layer(9, 0, 21, 4, 4096, synth.BF16)
    ref = _oracle(inp)
    X = dev(inp["X"])
    _, h_post, h_res, _ = hc.hc_coeffs_pre(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    hc.hc_post(X, h_res, h_post, dev(inp["F_out"]), out=X)
    torch.cuda.synchronize()
    check_bf16("X_next in place", host64(X), ref["X_next"])


def test_empty_input():
    note("mHC T=0")
    X = torch.empty(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    phi = torch.zeros(256, 24, device="cuda")
    out = hc.hc_coeffs_pre(X, phi, torch.zeros(24, device="cuda"), [0.01] * 3)
    assert out[3].shape == (0, 64)
    Y = hc.hc_post(X, out[2], out[1], torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"))
    assert Y.shape == (0, 4, 64)


def test_scale_invariance_power_of_two_bit_exact():
    # coeffs(2^k X) == coeffs(X): sums and products scale exactly by powers of two
    # and r = sqrt(ss/len) is correctly rounded, so the logits are bit-identical.
    note("mHC scale invariance bf16 n=4 C=4096")
    inp = synth.mhc_layer(10, 0, 40, 4, 4096, synth.BF16)
    X = dev(inp["X"])
    a = hc.hc_coeffs(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    b = hc.hc_coeffs(X * 4, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_phi_zero_closed_form_on_gpu(golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "sinkhorn_phi0_n4.json")))
    note("mHC phi=0 closed form")
    inp = synth.mhc_layer(11, 0, 16, 4, 4096, synth.BF16)
    phi = torch.zeros(4 * 4096, 24, device="cuda")
    h_pre, h_post, h_res, F_in = hc.hc_coeffs_pre(dev(inp["X"]), phi, dev(inp["bias"]), [0.01] * 3)
    np.testing.assert_allclose(h_pre.cpu().numpy(), g["h_pre"], atol=1e-7)
    np.testing.assert_allclose(h_post.cpu().numpy(), g["h_post"], atol=1e-7)
    expect = np.full((4, 4), g["h_res_offdiag"]) + np.eye(4) * (g["h_res_diag"] - g["h_res_offdiag"])
    np.testing.assert_allclose(h_res.cpu().numpy(), np.broadcast_to(expect, (16, 4, 4)), atol=1e-6)
    check_bf16("F_in = sum/2", host64(F_in), 0.5 * inp["X"].values.astype(np.float64).sum(1))


def test_wide_logits_follow_twenty_iterations():
    # Far from convergence the output is M^(20), not the limit: compare with the
    # oracle's 20-iteration result (rows exact, columns off by >1e-4).
    note("mHC wide Sinkhorn logits")
    inp = synth.mhc_layer(12, 0, 33, 4, 256, synth.F32)
    inp["bias"] = inp["bias"].copy()
    inp["bias"][8:] = np.random.default_rng(3).standard_normal(16).astype(np.float32) * 3.0
    inp["alpha"] = np.array([0.5, 0.5, 2.0], np.float32)
    got = _run_sublayer(inp, fused=True)
    ref = _oracle(inp)
    check_fp32("h_res wide", got["h_res"], ref["h_res"])
    assert np.max(np.abs(ref["h_res"].sum(-2) - 1)) > 1e-4


@pytest.mark.slow
def test_mhc_n4_C7168_T16384_chain_per_layer_and_conservation():
    """8 chained sublayers at full size: per layer the oracle runs on the GPU's
    bf16 X_l for sampled tokens; the stream-sum conservation holds on all tokens."""
    w = synth.WORKLOADS["mhc_n4_C7168_T16384_bf16_8layers"]
    T, n, C = w["T"], w["n"], w["C"]
    rng = np.random.default_rng(202)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 62, replace=False)]))
    first = synth.mhc_layer(2, 0, T, n, C, w["dtype"])
    X = dev(first["X"])
    del first["X"]
    for layer in range(w["layers"]):
        note(f"mHC chain layer {layer} (n=4 C=7168 T=16384 bf16)")
        inp = first if layer == 0 else synth.mhc_layer(2, layer, T, n, C, w["dtype"], draw_x=False)
        F = dev(inp["F_out"])
        h_pre, h_post, h_res, F_in = hc.hc_coeffs_pre(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
        Xn = hc.hc_post(X, h_res, h_post, F)
        torch.cuda.synchronize()
        Xs = host64(X[torch.from_numpy(sample).cuda()])
        ref = O.mhc_sublayer(Xs, inp["phi"], inp["bias"], inp["alpha"], inp["F_out"].values[sample])
        got = dict(h_pre=host64(h_pre)[sample], h_post=host64(h_post)[sample], h_res=host64(h_res)[sample],
                   F_in=host64(F_in[torch.from_numpy(sample).cuda()]),
                   X_next=host64(Xn[torch.from_numpy(sample).cuda()]))
        _compare_all(got, ref, synth.BF16)
        # conservation over every token: sum_i X_next = sum_i X + (sum_i h_post) F
        lhs = Xn.float().sum(1)
        rhs = X.float().sum(1) + h_post.sum(1, keepdim=True) * F.float()
        e = (torch.linalg.vector_norm(lhs - rhs) / torch.linalg.vector_norm(rhs)).item()
        assert e < 1e-2, f"layer {layer}: conservation rel err {e}"
        X = Xn
        del F, F_in


def test_mhc_n4_C7168_chain_end_to_end():
    """Reduced-T chain of 8 layers at C=7168: each layer against the oracle on the
    GPU's input, and the independent oracle chain (bf16 rounding between layers)
    against the GPU's last state."""
    T, n, C = 45, 4, 7168
    first = synth.mhc_layer(2, 0, T, n, C, synth.BF16)
    X = dev(first["X"])
    Xo = first["X"].values.astype(np.float64)
    for layer in range(8):
        note(f"mHC 8-layer chain C=7168 T=45 layer {layer}")
        inp = first if layer == 0 else synth.mhc_layer(2, layer, T, n, C, synth.BF16, draw_x=False)
        h_pre, h_post, h_res, F_in = hc.hc_coeffs_pre(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
        Xn = hc.hc_post(X, h_res, h_post, dev(inp["F_out"]))
        torch.cuda.synchronize()
        ref = O.mhc_sublayer(host64(X), inp["phi"], inp["bias"], inp["alpha"], inp["F_out"].values)
        _compare_all(dict(h_pre=host64(h_pre), h_post=host64(h_post), h_res=host64(h_res),
                          F_in=host64(F_in), X_next=host64(Xn)), ref, synth.BF16)
        chain = O.mhc_sublayer(Xo, inp["phi"], inp["bias"], inp["alpha"], inp["F_out"].values)
        Xo = synth.round_to_bf16(chain["X_next"].astype(np.float32))[0].astype(np.float64)
        X = Xn
    assert rel_l2(host64(X), Xo) < 1e-2


# ------------------------------------------------ post fused with next coefficients

def _post_coeffs_case(T, C, seed, in_place=False):
    inp = synth.mhc_layer(seed, 0, T, 4, C, synth.BF16)
    nxt = synth.mhc_layer(seed, 1, T, 4, C, synth.BF16, draw_x=False)
    X = dev(inp["X"])
    h_pre, h_post, h_res = hc.hc_coeffs(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    ref = _oracle(inp)
    out = X if in_place else None
    Xn, (hp2, hq2, hr2) = hc.hc_post_coeffs(X, h_res, h_post, dev(inp["F_out"]), dev(nxt["phi"]), dev(nxt["bias"]),
                                            [0.01] * 3, out=out)
    torch.cuda.synchronize()
    check_bf16("X_next", host64(Xn), ref["X_next"], literal_max_abs=True)
    # coefficients of the state actually written (the GPU's bf16 X_next)
    r2 = O.hc_coeffs(host64(Xn), nxt["phi"], nxt["bias"], nxt["alpha"])
    for name, g, r in zip(("h_pre'", "h_post'", "h_res'"), (hp2, hq2, hr2), r2):
        check_fp32(name, host64(g), r)


@pytest.mark.parametrize("T", [1, 16, 133])
def test_post_coeffs_matches_post_then_coeffs(T):
    note(f"mHC hc_post_coeffs n=4 C=4096 bf16 T={T}")
    _post_coeffs_case(T, 4096, 20 + T)


def test_post_coeffs_in_place_and_small_C():
    note("mHC hc_post_coeffs in place, C=64 and C=7168")
    _post_coeffs_case(37, 64, 31, in_place=True)
    _post_coeffs_case(19, 7168, 32)
    note("mHC hc_post_coeffs generic shapes (C=40 bf16)")
    _post_coeffs_case(11, 40, 33)


def test_chain_with_post_coeffs_C7168():
    """The chained path (pre-read + post fused with the next coefficients) over 8
    layers at C=7168: each layer against the oracle on the GPU's own input state."""
    T, n, C = 45, 4, 7168
    layers = [synth.mhc_layer(2, 0, T, n, C, synth.BF16)] + [
        synth.mhc_layer(2, l, T, n, C, synth.BF16, draw_x=False) for l in range(1, 9)]
    X = dev(layers[0]["X"])
    h_pre, h_post, h_res = hc.hc_coeffs(X, dev(layers[0]["phi"]), dev(layers[0]["bias"]), [0.01] * 3)
    for l in range(8):
        note(f"mHC chained path C=7168 T=45 layer {l}")
        inp = layers[l]
        F_in = hc.hc_pre(X, h_pre)
        Xn, (h_pre, h_post_n, h_res_n) = hc.hc_post_coeffs(X, h_res, h_post, dev(inp["F_out"]),
                                                         dev(layers[l + 1]["phi"]), dev(layers[l + 1]["bias"]),
                                                         [0.01] * 3)
        torch.cuda.synchronize()
        ref = O.mhc_sublayer(host64(X), inp["phi"], inp["bias"], inp["alpha"], inp["F_out"].values)
        check_bf16("F_in", host64(F_in), ref["F_in"])
        check_bf16("X_next", host64(Xn), ref["X_next"])
        r2 = O.hc_coeffs(host64(Xn), layers[l + 1]["phi"], layers[l + 1]["bias"], layers[l + 1]["alpha"])
        for name, g, r in zip(("h_pre'", "h_post'", "h_res'"), (h_pre, h_post_n, h_res_n), r2):
            check_fp32(name, host64(g), r)
        X, h_post, h_res = Xn, h_post_n, h_res_n


# ------------------------------------------- the whole step: post, next coefficients, next pre-read

def _post_pre_case(T, C, seed, dtype=synth.BF16, in_place=False, packed=False, want_h_pre=True):
    inp = synth.mhc_layer(seed, 0, T, 4, C, dtype)
    nxt = synth.mhc_layer(seed, 1, T, 4, C, dtype, draw_x=False)
    X = dev(inp["X"])
    h_pre, h_post, h_res = hc.hc_coeffs(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    ref = _oracle(inp)
    phi_n = dev(nxt["phi"])
    pk = hc.hc_phi_pack(phi_n, 4, C, X.dtype) if packed else None
    out = X if in_place else None
    Xn, (hp2, hq2, hr2), F_in = hc.hc_post_pre(X, h_res, h_post, dev(inp["F_out"]), phi_n, dev(nxt["bias"]),
                                               [0.01] * 3, phi_next_packed=pk, out=out, want_h_pre=want_h_pre)
    torch.cuda.synchronize()
    if dtype == synth.BF16:
        check_bf16("X_next", host64(Xn), ref["X_next"], literal_max_abs=True)
    else:
        check_fp32("X_next", host64(Xn), ref["X_next"])
    # coefficients and pre-read of the state actually written (the GPU's X_next)
    r2 = O.hc_coeffs(host64(Xn), nxt["phi"], nxt["bias"], nxt["alpha"])
    got = (hp2, hq2, hr2) if want_h_pre else (None, hq2, hr2)
    for name, g, r in zip(("h_pre'", "h_post'", "h_res'"), got, r2):
        if g is not None:
            check_fp32(name, host64(g), r)
    F_ref = O.hc_pre(host64(Xn), r2[0])
    if dtype == synth.BF16:
        check_bf16("F_in'", host64(F_in), F_ref)
    else:
        check_fp32("F_in'", host64(F_in), F_ref)
    return Xn, hq2, hr2, F_in


@pytest.mark.parametrize("T", [1, 16, 133])
def test_post_pre_matches_post_then_coeffs_pre(T):
    note(f"mHC hc_post_pre n=4 C=4096 bf16 T={T}")
    _post_pre_case(T, 4096, 40 + T)


def test_post_pre_in_place_small_C_generic_and_no_h_pre():
    note("mHC hc_post_pre in place C=64, C=7168 without h_pre, C=32")
    _post_pre_case(37, 64, 51, in_place=True)
    _post_pre_case(19, 7168, 52, want_h_pre=False)
    _post_pre_case(70, 32, 53)
    note("mHC hc_post_pre generic shapes (C=40 bf16, C=256 fp32)")
    _post_pre_case(11, 40, 54)
    _post_pre_case(23, 256, 55, dtype=synth.F32)


def test_post_pre_packed_phi_is_identical():
    """hc_phi_pack once + hc_post_pre(phi_next_packed) gives the same bits as
    letting the call pack phi itself."""
    note("mHC hc_post_pre with phi packed by hc_phi_pack, C=4096 T=77")
    a = _post_pre_case(77, 4096, 61, packed=False)
    b = _post_pre_case(77, 4096, 61, packed=True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(host64(x), host64(y))


@pytest.mark.parametrize("T,C", [(133, 4096), (300, 7168), (40, 32)])
def test_pre_read_h_pre_matches_returned_coefficients_bit_exact(T, C):
    """The fused pre-read forms each token's h_pre from the partial projections
    itself; its F_in must be exactly hc_pre(X_next, h_pre') with the h_pre' the
    same call returns, and the same whether or not h_pre' is requested (also
    for hc_coeffs_pre, whose projection adds the channels in another order than
    hc_post_pre's, so its h_pre' may differ from that one in the last bits)."""
    note(f"mHC pre-read h_pre consistency n=4 C={C} T={T}")
    inp = synth.mhc_layer(80 + T, 0, T, 4, C, synth.BF16)
    nxt = synth.mhc_layer(80 + T, 1, T, 4, C, synth.BF16, draw_x=False)
    X = dev(inp["X"])
    h_pre, h_post, h_res = hc.hc_coeffs(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    args = (X, h_res, h_post, dev(inp["F_out"]), dev(nxt["phi"]), dev(nxt["bias"]), [0.01] * 3)
    Xn, (hp2, _, _), F_a = hc.hc_post_pre(*args)
    _, (none, _, _), F_b = hc.hc_post_pre(*args, want_h_pre=False)
    assert none is None
    F_ref = hc.hc_pre(Xn, hp2)
    hq, _, _, F_c = hc.hc_coeffs_pre(Xn, dev(nxt["phi"]), dev(nxt["bias"]), [0.01] * 3)
    _, _, _, F_d = hc.hc_coeffs_pre(Xn, dev(nxt["phi"]), dev(nxt["bias"]), [0.01] * 3, want_h_pre=False)
    F_q = hc.hc_pre(Xn, hq)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu().numpy()
    np.testing.assert_allclose(hq.cpu().numpy(), hp2.cpu().numpy(), rtol=1e-6, atol=0)
    for F in (F_a, F_b):
        np.testing.assert_array_equal(bits(F), bits(F_ref))
    for F in (F_c, F_d):
        np.testing.assert_array_equal(bits(F), bits(F_q))


def test_phi_pack_layout_pin():
    """The packed form: per group of 8 rows, columns 0..23 hi = bf16(phi), 24..47
    lo = bf16(phi - hi), 8 consecutive rows of one column contiguous."""
    note("hc_phi_pack layout, C=64")
    C = 64
    rng = np.random.default_rng(7)
    phi = rng.standard_normal((4 * C, 24)).astype(np.float32) * 0.02
    pk = hc.hc_phi_pack(torch.from_numpy(phi).cuda(), 4, C, torch.bfloat16)
    torch.cuda.synchronize()
    got = pk.cpu().numpy().view(np.uint16).reshape(4 * C // 8, 48, 8)
    hi, hi_bits = synth.round_to_bf16(phi)
    _, lo_bits = synth.round_to_bf16(phi - hi)  # phi - hi is exact in float32
    want = np.concatenate([hi_bits.reshape(4 * C // 8, 8, 24), lo_bits.reshape(4 * C // 8, 8, 24)], axis=2)
    np.testing.assert_array_equal(got, want.transpose(0, 2, 1))


def test_chain_with_post_pre_C7168():
    """The chained path as one call per step over 8 layers at C=7168, each layer
    against the oracle on the GPU's own input state."""
    T, n, C = 45, 4, 7168
    layers = [synth.mhc_layer(2, 0, T, n, C, synth.BF16)] + [
        synth.mhc_layer(2, l, T, n, C, synth.BF16, draw_x=False) for l in range(1, 9)]
    X = dev(layers[0]["X"])
    h_pre, h_post, h_res, F_in = hc.hc_coeffs_pre(X, dev(layers[0]["phi"]), dev(layers[0]["bias"]), [0.01] * 3)
    for l in range(8):
        note(f"mHC hc_post_pre chain C=7168 T=45 layer {l}")
        inp = layers[l]
        ref = O.mhc_sublayer(host64(X), inp["phi"], inp["bias"], inp["alpha"], inp["F_out"].values)
        check_bf16("F_in", host64(F_in), ref["F_in"])
        Xn, (h_pre, h_post_n, h_res_n), F_in = hc.hc_post_pre(
            X, h_res, h_post, dev(inp["F_out"]), dev(layers[l + 1]["phi"]), dev(layers[l + 1]["bias"]), [0.01] * 3)
        torch.cuda.synchronize()
        check_bf16("X_next", host64(Xn), ref["X_next"])
        r2 = O.hc_coeffs(host64(Xn), layers[l + 1]["phi"], layers[l + 1]["bias"], layers[l + 1]["alpha"])
        for name, g, r in zip(("h_pre'", "h_post'", "h_res'"), (h_pre, h_post_n, h_res_n), r2):
            check_fp32(name, host64(g), r)
        X, h_post, h_res = Xn, h_post_n, h_res_n


# ------------------------------- the benchmarked launch: several items per workgroup

def _round_sample(T, rounds=4, per_round=64, seed=303):
    """Tokens from every round of items a persistent workgroup takes (at T = 8192,
    C = 4096 the 1,024 items are tile-major over 256 workgroups, so round r covers
    tokens 2048 r .. 2048 r + 2047), plus the round boundaries and both ends."""
    rng = np.random.default_rng(seed)
    q = T // rounds
    parts = [np.array([0, T - 1])]
    for r in range(rounds):
        parts.append(rng.choice(np.arange(r * q, (r + 1) * q), per_round, replace=False))
        parts.append(np.array([r * q, min(T - 1, (r + 1) * q - 1)]))
    return np.unique(np.concatenate(parts))


def _bf16_ulp_dev(v):
    """One bfloat16 ulp at |v| on the device (0 where v == 0), float64."""
    m, e = torch.frexp(v.double())
    return torch.where(v == 0, torch.zeros_like(m), torch.ldexp(torch.ones_like(m), e - 8))


def _check_conservation_all_tokens(X0, Xn, h_res, h_post, F):
    """sum_i X_next = sum_i X + (sum_i h_post) F on every token and channel (Eq. 6:
    H_res has unit column sums), within the column-sum error, fp32 accumulation and
    the bf16 rounding of the four stored streams; in float64 on the device."""
    cs = (h_res.double().sum(-2) - 1).abs().max().item()
    assert cs < 1e-6, f"column sums off by {cs:.2e}"
    for s in range(0, X0.shape[0], 2048):
        x = X0[s:s + 2048].double()
        xn = Xn[s:s + 2048].double()
        f = F[s:s + 2048].double()
        hp = h_post[s:s + 2048].double()
        lhs = xn.sum(1)
        rhs = x.sum(1) + hp.sum(1, keepdim=True) * f
        bound = 0.5 * _bf16_ulp_dev(xn).sum(1) + 1e-5 * (x.abs().sum(1) + hp.abs().sum(1, keepdim=True) * f.abs())
        bad = int(((lhs - rhs).abs() > bound).sum().item())
        assert bad == 0, f"stream-sum conservation fails on {bad} elements (tokens {s}..)"


def _full_size_post_case(fused_pre, in_place):
    w = synth.WORKLOADS["mhc_n4_C4096_T8192_bf16"]
    T, n, C = w["T"], w["n"], w["C"]
    note(f"mHC {'hc_post_pre' if fused_pre else 'hc_post_coeffs'} full size n=4 C=4096 T=8192 bf16 "
         f"in_place={in_place}")
    inp = synth.mhc_layer(1, 0, T, n, C, synth.BF16)
    nxt = synth.mhc_layer(1, 1, T, n, C, synth.BF16, draw_x=False)
    X = dev(inp["X"])
    X0 = X.clone()
    F = dev(inp["F_out"])
    h_pre, h_post, h_res = hc.hc_coeffs(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    args = (X, h_res, h_post, F, dev(nxt["phi"]), dev(nxt["bias"]), [0.01] * 3)
    out = X if in_place else None
    if fused_pre:
        Xn, (hp2, hq2, hr2), F_in = hc.hc_post_pre(*args, out=out)
    else:
        Xn, (hp2, hq2, hr2) = hc.hc_post_coeffs(*args, out=out)
    torch.cuda.synchronize()
    sample = _round_sample(T)
    st = torch.from_numpy(sample).cuda()
    sub = dict(inp)
    sub["X"] = synth.Tensor(inp["X"].values[sample], synth.BF16)
    sub["F_out"] = synth.Tensor(inp["F_out"].values[sample], synth.BF16)
    ref = _oracle(sub)
    check_bf16("X_next (sampled)", host64(Xn[st]), ref["X_next"], literal_max_abs=True)
    Xs = host64(Xn[st])
    r2 = O.hc_coeffs(Xs, nxt["phi"], nxt["bias"], nxt["alpha"])
    for name, g, r in zip(("h_pre'", "h_post'", "h_res'"), (hp2, hq2, hr2), r2):
        check_fp32(name + " (sampled)", host64(g[st]), r)
    if fused_pre:
        check_bf16("F_in' (sampled)", host64(F_in[st]), O.hc_pre(Xs, r2[0]), literal_below=8.0)
        # every token: the pre-read equals hc_pre(X_next, h_pre') bit for bit
        F_ref = hc.hc_pre(Xn, hp2)
        torch.cuda.synchronize()
        assert torch.equal(F_in.view(torch.int16), F_ref.view(torch.int16))
    # every token: Sinkhorn sums, gate ranges, stream-sum conservation of the write
    hr = hr2.double()
    assert (hr >= 0).all().item()
    assert (hr.sum(-1) - 1).abs().max().item() < 1e-6 and (hr.sum(-2) - 1).abs().max().item() < 1e-6
    assert ((hp2 > 0) & (hp2 < 1)).all().item() and ((hq2 > 0) & (hq2 < 2)).all().item()
    _check_conservation_all_tokens(X0, Xn, h_res, h_post, F)


@pytest.mark.parametrize("in_place", [False, True])
def test_post_pre_n4_C4096_T8192_full_size(in_place):
    _full_size_post_case(True, in_place)


@pytest.mark.parametrize("in_place", [False, True])
def test_post_coeffs_n4_C4096_T8192_full_size(in_place):
    _full_size_post_case(False, in_place)


@pytest.mark.slow
def test_post_pre_chain_n4_C7168_T16384_full_size():
    """The 8-layer C = 7168, T = 16384 chain through hc_post_pre (14 items per
    workgroup): per layer the oracle on sampled tokens of the GPU's own input
    state, the pre-read bit-exact against hc_pre on every token, and stream-sum
    conservation on every token."""
    w = synth.WORKLOADS["mhc_n4_C7168_T16384_bf16_8layers"]
    T, n, C, layers = w["T"], w["n"], w["C"], w["layers"]
    sample = _round_sample(T, rounds=8, per_round=16, seed=404)
    st = torch.from_numpy(sample).cuda()
    first = synth.mhc_layer(2, 0, T, n, C, w["dtype"])
    X = dev(first["X"])
    del first["X"]
    h_pre, h_post, h_res, F_in = hc.hc_coeffs_pre(X, dev(first["phi"]), dev(first["bias"]), [0.01] * 3)
    cur = first
    ping = torch.empty_like(X)
    for layer in range(layers):
        note(f"mHC hc_post_pre chain layer {layer} (n=4 C=7168 T=16384 bf16)")
        nxt = synth.mhc_layer(2, layer + 1, T, n, C, w["dtype"], draw_x=False)
        F = dev(cur["F_out"])
        Xs = host64(X[st])
        ref = O.mhc_sublayer(Xs, cur["phi"], cur["bias"], cur["alpha"], cur["F_out"].values[sample])
        check_bf16(f"F_in layer {layer}", host64(F_in[st]), ref["F_in"])
        Xn, (h_pre, h_post_n, h_res_n), F_in = hc.hc_post_pre(X, h_res, h_post, F, dev(nxt["phi"]),
                                                              dev(nxt["bias"]), [0.01] * 3, out=ping)
        F_ref = hc.hc_pre(Xn, h_pre)
        torch.cuda.synchronize()
        check_bf16(f"X_next layer {layer}", host64(Xn[st]), ref["X_next"])
        r2 = O.hc_coeffs(host64(Xn[st]), nxt["phi"], nxt["bias"], nxt["alpha"])
        for name, g, r in zip(("h_pre'", "h_post'", "h_res'"), (h_pre, h_post_n, h_res_n), r2):
            check_fp32(f"{name} layer {layer}", host64(g[st]), r)
        assert torch.equal(F_in.view(torch.int16), F_ref.view(torch.int16))
        _check_conservation_all_tokens(X, Xn, h_res, h_post, F)
        ping, X = X, Xn
        h_post, h_res, cur = h_post_n, h_res_n, nxt
        del F, F_ref
