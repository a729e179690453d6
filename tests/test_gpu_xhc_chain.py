"""GPU parity of the chained xHC calls (xhc_pre_chain, xhc_route_pre) through the C
ABI: a chain of sublayers, each call's outputs compared with the fp64 oracle on
the state the GPU holds at that point (xhc_route of sublayer l, then xhc_pre of
sublayer l + 1), and with the unchained calls (xhc_pre, xhc_route) on the same
state. The chained calls add the projection's sums in another order, so a token
whose candidate scores are within rounding of each other may pick either: there
the choice is checked to be a valid top-(k - m) (each chosen score at least each
passed-over one, to within 1e-5), elsewhere the indices are compared exactly."""
import numpy as np
import pytest

import oracle as O
import synth
from hc_testutil import bf16_ulp, check_bf16, check_fp32, dev, have_gpu, host64, note

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc

N, K_ACT, M_FIX = 16, 4, 2
SCORE_TOL = 1e-5   # fp32 scores against fp64, well above their rounding
GAP = 1e-4         # tokens whose deciding scores are closer than this may go either way


def _maps(inp):
    return dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], dev(inp["w_router"])


def _check_selection(name, got_idx, X_host, inp, sample=None):
    """got_idx [t, k] against the oracle's scores of X_host: equal where the k - m
    chosen candidates are clear of the rest, a valid top-(k - m) elsewhere."""
    k, m = K_ACT, M_FIX
    sc = O.xhc_router_scores(X_host, inp["w_router"])  # [t, N - m]
    ref = O.xhc_pre(X_host, inp["phi_pre"], inp["b_pre"], inp["alpha_pre"], inp["w_router"], k, m)["idx"]
    srt = -np.sort(-sc, axis=1)
    clear = srt[:, k - m - 1] - srt[:, k - m] > GAP
    got = np.asarray(got_idx, np.int64)
    np.testing.assert_array_equal(got[clear], ref[clear], err_msg=f"{name}: indices of clear tokens")
    for t in np.nonzero(~clear)[0]:
        g = got[t]
        assert list(g[:m]) == list(range(m)) and np.all(np.diff(g) > 0), f"{name}: token {t} idx {g}"
        chosen = g[m:] - m
        rest = np.setdiff1d(np.arange(N - m), chosen)
        assert sc[t, chosen].min() >= sc[t, rest].max() - SCORE_TOL, f"{name}: token {t} is not a top-{k - m}"
    note(f"{name}: {int((~clear).sum())} of {len(clear)} tokens within {GAP} of a tie")
    return clear


def _rows(Xd, sample):
    """The state's rows (all, or the sampled tokens) in float64 on the host."""
    return host64(Xd if sample is None else Xd[torch.as_tensor(sample, device=Xd.device)])


def _check_pre_outputs(name, got, Xd, inp, sample):
    """h_pre, F_in, score, idx of a chained call against the oracle's xhc_pre of the
    state (the sampled tokens)."""
    sl = (lambda a: a) if sample is None else (lambda a: a[sample])
    Xs = _rows(Xd, sample)
    ref = O.xhc_pre(Xs, inp["phi_pre"], inp["b_pre"], inp["alpha_pre"], inp["w_router"], K_ACT, M_FIX)
    check_fp32(f"{name} h_pre", sl(host64(got["h_pre"])), ref["h_pre"])
    check_bf16(f"{name} F_in", sl(host64(got["F_in"])), ref["F_in"])
    check_fp32(f"{name} score", sl(host64(got["score"])), ref["score"])
    _check_selection(f"{name} idx", sl(got["idx"].cpu().numpy()), Xs, inp)


def _check_against_unchained(name, got, X_state, inp):
    """The same sublayer by xhc_pre on a copy of the state, on every token."""
    k, m = K_ACT, M_FIX
    ref = hc.xhc_pre(X_state.clone(), *_maps(inp), k=k, m=m)
    torch.cuda.synchronize()
    check_fp32(f"{name} h_pre vs xhc_pre", host64(got["h_pre"]), host64(ref["h_pre"]), tol=1e-6)
    a, b = host64(got["F_in"]), host64(ref["F_in"])
    # Both are RNE roundings of float32 sums of 16 terms h_i x_i whose h_i differ by
    # float32 rounding (|x| < 8 here): the sums differ by well under 1e-4, so the
    # rounded values by at most that plus one bf16 step of the larger.
    excess = np.abs(a - b) - bf16_ulp(np.maximum(np.abs(a), np.abs(b))) - 1e-4
    assert float(excess.max()) <= 0.0, f"{name}: F_in differs from xhc_pre's by {float(np.abs(a - b).max()):.3g}"
    same = (got["idx"] == ref["idx"]).all(dim=1)
    note(f"{name}: idx equal to xhc_pre's on {int(same.sum().item())} of {same.numel()} tokens")
    return same


def _check_inactive_unchanged(name, X_before, X_after, idx):
    """On the device, every token: rows outside the active set are bit for bit the input."""
    T = X_before.shape[0]
    act = torch.zeros(T, N, dtype=torch.bool, device=X_before.device)
    act.scatter_(1, idx.long(), True)
    assert int(act.sum().item()) == T * idx.shape[1], f"{name}: active indices repeat within a token"
    same = (X_before.view(torch.int16) == X_after.view(torch.int16)).all(dim=2)
    assert bool(same[~act].all().item()), f"{name}: {int((~same[~act]).sum().item())} inactive rows changed"


def _write_back(layer, seed, l, K):
    """The route's write-back components: F_out (K = 1), else K seeded N(0, 1)
    components [T, K, C] standing in for the augmentation's output."""
    if K == 1:
        return layer["F_out"]
    T, C = layer["F_out"].values.shape
    return synth.Tensor(synth.normal(synth.make_rng(seed, l, stream=2), (T, K, C)), synth.BF16)


def _run_chain(seed, T, C, L, carry_in_place, sample=None, K=1):
    """L sublayers: xhc_pre_chain, L - 1 calls of xhc_route_pre, the last route by
    xhc_route; every call checked against the oracle on the GPU's state. K: the
    routes' write-back components."""
    k, m = K_ACT, M_FIX
    layers = [synth.xhc_layer(seed, l, T, N, C, k, m, K, synth.BF16) for l in range(L)]
    wbs = [_write_back(layers[l], seed, l, K) for l in range(L)]
    X = dev(layers[0]["X"])
    note(f"xhc_pre_chain T={T} C={C} seed={seed}")
    res = hc.xhc_pre_chain(X, *_maps(layers[0]), dev(layers[1]["phi_pre"]), dev(layers[1]["w_router"]), k=k, m=m)
    torch.cuda.synchronize()
    _check_pre_outputs("sublayer 0", res, X, layers[0], sample)
    _check_against_unchained("sublayer 0", res, X, layers[0])
    carry, idx = res["carry"], res["idx"]
    sl = (lambda a: a) if sample is None else (lambda a: a[sample])
    for l in range(L - 1):
        nxt = layers[l + 2] if l + 2 < L else None
        X_before = X.clone()
        idx_host = idx.cpu().numpy().astype(np.int64)
        note(f"xhc_route_pre sublayer {l} -> {l + 1} T={T} C={C} next={nxt is not None}")
        out = hc.xhc_route_pre(
            X, dev(wbs[l]), dev(layers[l]["phi_act"]), dev(layers[l]["b_act"]), layers[l]["alpha_post"],
            layers[l]["alpha_res"], idx, carry, dev(layers[l + 1]["b_pre"]), layers[l + 1]["alpha_pre"],
            phi_pre_next=None if nxt is None else dev(nxt["phi_pre"]),
            w_router_next=None if nxt is None else dev(nxt["w_router"]),
            carry_out=(carry if carry_in_place else None) if nxt is not None else None,
            k=k, m=m, want_coeffs=True)
        torch.cuda.synchronize()
        # route l on the state before the call
        Xb = _rows(X_before, sample)
        ref_X, ref_hp, ref_hr = O.xhc_route(Xb, sl(idx_host), layers[l]["phi_act"], layers[l]["b_act"],
                                            layers[l]["alpha_post"], layers[l]["alpha_res"],
                                            sl(wbs[l].values.astype(np.float64)))
        check_fp32(f"route {l} H_post", sl(host64(out["h_post"])), ref_hp)
        check_fp32(f"route {l} H_res", sl(host64(out["h_res"])), ref_hr)
        _check_inactive_unchanged(f"route {l}", X_before, X, idx)
        act = np.zeros((Xb.shape[0], N), bool)
        act[np.arange(Xb.shape[0])[:, None], sl(idx_host)] = True
        check_bf16(f"route {l} X_active", _rows(X, sample)[act], ref_X[act])
        del X_before
        # pre of sublayer l + 1 on the state the route wrote
        _check_pre_outputs(f"sublayer {l + 1}", out, X, layers[l + 1], sample)
        _check_against_unchained(f"sublayer {l + 1}", out, X, layers[l + 1])
        idx = out["idx"]
        if nxt is not None:
            carry = out["carry"]
    # the chain's last route, unchained
    last = layers[L - 1]
    hc.xhc_route(X, dev(wbs[L - 1]), dev(last["phi_act"]), dev(last["b_act"]), last["alpha_post"],
                 last["alpha_res"], k=k, m=m, idx=idx)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 64, 300])
def test_chain_small(T):
    """Ragged and whole 64-token tiles (the carry's items and the pair tiles)."""
    _run_chain(11, T, 1024, 3, carry_in_place=True)


def test_chain_separate_carries_C2048():
    _run_chain(12, 200, 2048, 4, carry_in_place=False)


@pytest.mark.parametrize("T", [45, 300])
def test_chain_augmented_K4(T):
    """The routes write back K = 4 components (the augmented step's route)."""
    _run_chain(14, T, 1024, 3, carry_in_place=True, K=4)


def test_chain_augmented_K4_full_size_N16_C4096_T8192():
    """The benchmarked augmented shape (2 sequences of 4096 tokens): oracle on 256
    sampled tokens per call, the unchained calls on every token."""
    rng = np.random.default_rng(6)
    sample = np.sort(rng.choice(8192, 256, replace=False))
    _run_chain(15, 8192, 4096, 3, carry_in_place=True, sample=sample, K=4)


def test_chain_full_size_N16_C4096_T8192():
    """The benchmarked shape: oracle on 256 sampled tokens per call, the unchained
    calls on every token."""
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(8192, 256, replace=False))
    _run_chain(13, 8192, 4096, 3, carry_in_place=True, sample=sample)


def test_chain_uncovered_shape_is_rejected():
    """Shapes outside the chained path's cover give HC_ERR_SHAPE (-1 from the size
    query), before any launch."""
    assert hc.xhc_chain_carry_bytes(64, 8, 1024, 4, 2, torch.bfloat16) == -1
    assert hc.xhc_chain_carry_bytes(64, 16, 1000, 4, 2, torch.bfloat16) == -1
    assert hc.xhc_chain_carry_bytes(64, 16, 1024, 4, 2, torch.bfloat16) > 0
    X = torch.zeros(64, 8, 1024, dtype=torch.bfloat16, device="cuda")
    z = lambda *s: torch.zeros(*s, device="cuda")
    with pytest.raises(ValueError):
        hc.xhc_pre_chain(X, z(8 * 1024, 8), z(8), 0.01, z(8 * 1024, 6), z(8 * 1024, 8), z(8 * 1024, 6))
