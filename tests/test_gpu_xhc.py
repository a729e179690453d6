"""GPU parity of the xHC calls (xhc_pre, xhc_route, xhc_augment) against the fp64
oracle, through the C ABI. Routing indices and scatter placement are compared
bit-exactly; values with the fp32 / bf16 tolerances."""
import numpy as np
import pytest

import oracle as O
import synth
from hc_testutil import check_bf16, check_fp32, check_stream, dev, have_gpu, host64, note

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc

GAP = 1e-3


def _router_scores_chunked(Xv, w_router, chunk=256):
    out = []
    for s in range(0, Xv.shape[0], chunk):
        out.append(O.xhc_router_scores(Xv[s:s + chunk], w_router))
    return np.concatenate(out)


def enforce_score_gaps(inp, k, m, seed):
    """Redraw (seeded) every token whose top-(k-m+1) candidate scores are closer than
    1e-3 to each other, so the selection does not hinge on rounding."""
    rng = synth.make_rng(seed, 0, stream=7)
    X = inp["X"]
    todo = np.arange(X.shape[0])
    for _ in range(50):
        s = _router_scores_chunked(X.values[todo], inp["w_router"])
        top = -np.sort(-s, axis=1)[:, : k - m + 1]
        bad = todo[np.any(top[:, :-1] - top[:, 1:] <= GAP, axis=1)]
        if bad.size == 0:
            return
        synth.redraw_rows(rng, X, bad)
        todo = bad
    raise AssertionError("could not enforce score gaps")


def _xhc_inputs(seed, T, N, k, m, C, K, batch=None, seq=None):
    inp = synth.xhc_layer(seed, 0, T, N, C, k, m, K, synth.BF16,
                          kappas=(4, 8, 12)[: K - 1] if K > 1 else ())
    enforce_score_gaps(inp, k, m, seed)
    return inp


def _check_pre(inp, k, m, got, sample=None):
    Xv = inp["X"].values if sample is None else inp["X"].values[sample]
    ref = O.xhc_pre(Xv, inp["phi_pre"], inp["b_pre"], inp["alpha_pre"], inp["w_router"], k, m)
    sl = (lambda a: a) if sample is None else (lambda a: a[sample])
    check_fp32("h_pre", sl(host64(got["h_pre"])), ref["h_pre"])
    # |F_in| reaches ~10 over 16 streams, where one bf16 rounding step is 0.031:
    # the per-element bound is max(2e-2, one bf16 ulp of the oracle value).
    _, worst = check_bf16("F_in", sl(host64(got["F_in"])), ref["F_in"])
    note(f"F_in literal max abs error {worst:.4f}")
    check_fp32("score", sl(host64(got["score"])), ref["score"])
    np.testing.assert_array_equal(sl(got["idx"].cpu().numpy()), ref["idx"])
    return ref


def _check_route(X_before, inp, idx, Wb_host, got_X, got_coeffs, sample=None):
    sl = (lambda a: a) if sample is None else (lambda a: a[sample])
    ref_X, ref_hp, ref_hr = O.xhc_route(sl(X_before), sl(idx), inp["phi_act"], inp["b_act"], inp["alpha_post"],
                                        inp["alpha_res"], sl(Wb_host))
    gX = sl(host64(got_X))
    check_fp32("H_post_A", sl(host64(got_coeffs["h_post"])), ref_hp)
    check_fp32("H_res_A", sl(host64(got_coeffs["h_res"])), ref_hr)
    # inactive streams are bit-identical; active rows within the bf16 rule
    T, N = gX.shape[:2]
    act = np.zeros((T, N), bool)
    act[np.arange(T)[:, None], sl(idx)] = True
    assert np.array_equal(gX[~act], sl(X_before)[~act])
    check_bf16("X_active", gX[act], ref_X[act])


def _check_inactive_bit_identical_all_tokens(X_before, X_after, idx):
    """On the device, every token: the rows outside the active set are bit for bit
    the input rows (in-place scatter, inactive streams never written)."""
    T, N = X_before.shape[:2]
    act = torch.zeros(T, N, dtype=torch.bool, device=X_before.device)
    act.scatter_(1, idx.long(), True)
    assert int(act.sum().item()) == T * idx.shape[1], "active indices repeat within a token"
    ib = X_before.view(torch.int16) if X_before.dtype == torch.bfloat16 else X_before.view(torch.int32)
    ia = X_after.view(torch.int16) if X_after.dtype == torch.bfloat16 else X_after.view(torch.int32)
    same = (ib == ia).all(dim=2)
    assert bool(same[~act].all().item()), f"{int((~same[~act]).sum().item())} inactive rows changed"


@pytest.mark.parametrize("T", [1, 77])
def test_xhc_N16_C4096_pre_and_route(T):
    N, k, m, C = 16, 4, 2, 4096
    note(f"xHC N=16 k=4 m=2 C=4096 bf16 K=1 T={T}")
    inp = _xhc_inputs(3, T, N, k, m, C, 1)
    X = dev(inp["X"])
    pre = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], dev(inp["w_router"]), k, m)
    torch.cuda.synchronize()
    _check_pre(inp, k, m, pre)
    idx = pre["idx"].cpu().numpy().astype(np.int64)
    X_before = inp["X"].values.astype(np.float64)
    # route with the supplied active set
    out = hc.xhc_route(X, dev(inp["F_out"]), dev(inp["phi_act"]), dev(inp["b_act"]), inp["alpha_post"],
                       inp["alpha_res"], k=k, m=m, idx=pre["idx"], want_coeffs=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["idx"].cpu().numpy(), idx)
    _check_route(X_before, inp, idx, inp["F_out"].values.astype(np.float64), X, out)
    # route selecting by itself from the (original) state gives the same set
    X2 = dev(inp["X"])
    out2 = hc.xhc_route(X2, dev(inp["F_out"]), dev(inp["phi_act"]), dev(inp["b_act"]), inp["alpha_post"],
                        inp["alpha_res"], k=k, m=m, w_router=dev(inp["w_router"]), want_coeffs=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out2["idx"].cpu().numpy(), idx)
    check_fp32("route score", host64(out2["score"]), O.xhc_router_scores(inp["X"].values, inp["w_router"]))
    assert torch.equal(X, X2)


@pytest.mark.slow
def test_xhc_N16_C4096_T8192_full_size():
    w = synth.WORKLOADS["xhc_N16_k4_m2_C4096_T8192_bf16_K1"]
    T, N, k, m, C = w["T"], w["N"], w["k"], w["m"], w["C"]
    note("xHC full size (N=16 k=4 C=4096 T=8192 bf16)")
    inp = _xhc_inputs(3, T, N, k, m, C, 1)
    X = dev(inp["X"])
    pre = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], dev(inp["w_router"]), k, m)
    torch.cuda.synchronize()
    # indices on every token
    s_all = _router_scores_chunked(inp["X"].values, inp["w_router"])
    np.testing.assert_array_equal(pre["idx"].cpu().numpy(), O.xhc_select(s_all, k, m))
    rng = np.random.default_rng(303)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 126, replace=False)]))
    _check_pre(inp, k, m, pre, sample)
    idx = pre["idx"].cpu().numpy().astype(np.int64)
    X0 = X.clone()
    out = hc.xhc_route(X, dev(inp["F_out"]), dev(inp["phi_act"]), dev(inp["b_act"]), inp["alpha_post"],
                       inp["alpha_res"], k=k, m=m, idx=pre["idx"], want_coeffs=True)
    torch.cuda.synchronize()
    _check_inactive_bit_identical_all_tokens(X0, X, pre["idx"])
    del X0
    _check_route(inp["X"].values, inp, idx, inp["F_out"].values, X, out, sample)


@pytest.mark.parametrize("vdt", ["bf16", "f32"])
def test_xhc_N16_C4096_augment_and_route(vdt):
    B, S, N, k, m, C = 2, 40, 16, 4, 2, 4096
    note(f"xHC augmented K=4 B=2 S=40 C=4096 V={vdt}")
    inp = _xhc_inputs(4, B * S, N, k, m, C, 4)
    F = dev(inp["F_out"])
    w = dev(np.concatenate([wj.reshape(-1) for wj in inp["conv_w"]]))
    V = hc.xhc_augment(F, w, inp["kappas"], B, S, v_dtype=torch.bfloat16 if vdt == "bf16" else torch.float32)
    torch.cuda.synchronize()
    refV = O.xhc_augment(inp["F_out"].values, inp["conv_w"], B, S)
    if vdt == "bf16":
        check_bf16("V", host64(V), refV)
    else:
        check_fp32("V", host64(V), refV)
    np.testing.assert_array_equal(host64(V[:, 0]), inp["F_out"].values)  # v_1 = out
    if vdt != "bf16":
        return
    X = dev(inp["X"])
    pre = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], dev(inp["w_router"]), k, m)
    torch.cuda.synchronize()
    _check_pre(inp, k, m, pre)
    idx = pre["idx"].cpu().numpy().astype(np.int64)
    out = hc.xhc_route(X, V, dev(inp["phi_act"]), dev(inp["b_act"]), inp["alpha_post"], inp["alpha_res"],
                       k=k, m=m, idx=pre["idx"], want_coeffs=True)
    torch.cuda.synchronize()
    _check_route(inp["X"].values, inp, idx, host64(V), X, out)


@pytest.mark.slow
def test_xhc_N16_C4096_T8192_K4_full_size():
    wl = synth.WORKLOADS["xhc_N16_k4_m2_C4096_T8192_bf16_K4"]
    B, S, N, k, m, C = wl["batch"], wl["seq"], wl["N"], wl["k"], wl["m"], wl["C"]
    T = B * S
    note("xHC full size (K=4, B=2 S=4096 C=4096 bf16)")
    inp = _xhc_inputs(4, T, N, k, m, C, 4)
    F = dev(inp["F_out"])
    w = dev(np.concatenate([wj.reshape(-1) for wj in inp["conv_w"]]))
    V = hc.xhc_augment(F, w, inp["kappas"], B, S)
    X = dev(inp["X"])
    X0 = X.clone()
    pre = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], dev(inp["w_router"]), k, m)
    out = hc.xhc_route(X, V, dev(inp["phi_act"]), dev(inp["b_act"]), inp["alpha_post"], inp["alpha_res"],
                       k=k, m=m, idx=pre["idx"], want_coeffs=True)
    torch.cuda.synchronize()
    _check_inactive_bit_identical_all_tokens(X0, X, pre["idx"])
    del X0
    s_all = _router_scores_chunked(inp["X"].values, inp["w_router"])
    np.testing.assert_array_equal(pre["idx"].cpu().numpy(), O.xhc_select(s_all, k, m))
    rng = np.random.default_rng(404)
    # sample includes sequence starts (zero padding) and the boundary between sequences
    sample = np.unique(np.concatenate([[0, 1, S - 1, S, S + 1, T - 1], rng.choice(T, 90, replace=False)]))
    refV = O.xhc_augment(inp["F_out"].values, inp["conv_w"], B, S)[sample]
    check_bf16("V", host64(V)[sample], refV)
    _check_pre(inp, k, m, pre, sample)
    idx = pre["idx"].cpu().numpy().astype(np.int64)
    _check_route(inp["X"].values, inp, idx, host64(V), X, out, sample)


def test_k_equals_N_is_dense_mhc():
    note("xHC k=N=4 m=1 vs mHC")
    N, C, T = 4, 256, 50
    rng = np.random.default_rng(31)
    Xt = synth.Tensor(rng.standard_normal((T, N, C)).astype(np.float32), synth.BF16)
    phi_pre = (0.02 * rng.standard_normal((N * C, N))).astype(np.float32)
    phi_act = (0.02 * rng.standard_normal((N * C, N + N * N))).astype(np.float32)
    b_pre = np.zeros(N, np.float32)
    b_act = synth.mhc_bias(N)[N:]
    W = rng.standard_normal((N * C, N - 1)).astype(np.float32)
    F = synth.Tensor(rng.standard_normal((T, C)).astype(np.float32), synth.BF16)
    X = dev(Xt)
    pre = hc.xhc_pre(X, dev(phi_pre), dev(b_pre), 0.01, dev(W), N, 1)
    hc.xhc_route(X, dev(F), dev(phi_act), dev(b_act), 0.01, 0.01, k=N, m=1, idx=pre["idx"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pre["idx"].cpu().numpy(), np.tile(np.arange(N), (T, 1)))
    ref = O.mhc_sublayer(Xt.values, np.concatenate([phi_pre, phi_act], 1), np.concatenate([b_pre, b_act]),
                         [0.01] * 3, F.values)
    check_bf16("F_in", host64(pre["F_in"]), ref["F_in"], literal_max_abs=True)
    check_bf16("X_next", host64(X), ref["X_next"], literal_max_abs=True)


def test_fixed_only_and_ties_and_invalid_indices():
    N, C, T = 8, 64, 64
    rng = np.random.default_rng(32)
    Xt = synth.Tensor(rng.standard_normal((T, N, C)).astype(np.float32), synth.F32)
    phi_pre = (0.02 * rng.standard_normal((N * C, N))).astype(np.float32)
    W = rng.standard_normal((N * C, N - 2)).astype(np.float32)
    W[:, 4] = W[:, 1]  # candidate streams 3 and 6 tie exactly
    note("xHC m=k fixed-only selection")
    pre = hc.xhc_pre(dev(Xt), dev(phi_pre), dev(np.zeros(N)), 0.01, dev(W), 2, 2)
    np.testing.assert_array_equal(pre["idx"].cpu().numpy(), np.tile([0, 1], (T, 1)))
    note("xHC exact ties go to the lower stream")
    pre = hc.xhc_pre(dev(Xt), dev(phi_pre), dev(np.zeros(N)), 0.01, dev(W), 3, 2)
    got = pre["idx"].cpu().numpy()
    s = host64(pre["score"])
    assert np.array_equal(s[:, 1], s[:, 4])
    ref = O.xhc_select(s, 3, 2)  # selection on the GPU's own fp32 scores
    np.testing.assert_array_equal(got, ref)
    assert np.any(got[:, 2] == 3)
    assert not np.any(got == 6)  # one routed slot: the tie with stream 3 always goes to 3
    note("xHC invalid supplied indices leave the token unchanged")
    X = dev(Xt)
    idx = np.tile(np.array([0, 2, 5], np.int32), (T, 1))
    idx[3] = [0, 2, 99]
    idx[5] = [-1, 2, 5]
    phi_act = (0.02 * rng.standard_normal((3 * C, 3 + 9))).astype(np.float32)
    b_act = np.concatenate([np.zeros(3), np.eye(3).reshape(-1)]).astype(np.float32)
    Fv = rng.standard_normal((T, C)).astype(np.float32)
    hc.xhc_route(X, dev(Fv), dev(phi_act), dev(b_act), 0.01, 0.01, k=3, m=1, idx=dev(idx))
    torch.cuda.synchronize()
    Y = X.cpu().numpy()
    assert np.array_equal(Y[3], Xt.values[3]) and np.array_equal(Y[5], Xt.values[5])
    ok = [t for t in range(T) if t not in (3, 5)]
    ref_X, _, _ = O.xhc_route(Xt.values[ok], idx[ok].astype(np.int64), phi_act, b_act, 0.01, 0.01, Fv[ok])
    check_fp32("X valid tokens", Y[ok], ref_X)


@pytest.mark.parametrize("K", [1, 4])
def test_fast_mix_invalid_indices_leave_token_unchanged(K):
    """k = 4 bf16 (the MFMA route path and its mix kernel): a token with an index
    outside [0, N) keeps all its streams bit for bit; the other tokens follow the
    oracle."""
    N, k, C, T = 8, 4, 64, 40
    note(f"xHC fast route k=4 K={K} with invalid supplied indices")
    rng = np.random.default_rng(100 + K)
    Xt = synth.Tensor(rng.standard_normal((T, N, C)).astype(np.float32), synth.BF16)
    idx = np.array([sorted(rng.choice(N, k, replace=False)) for _ in range(T)], np.int32)
    idx[3, 3] = 99
    idx[7, 0] = -1
    idx[T - 1, 2] = N
    Wb = synth.Tensor(rng.standard_normal((T, K, C)).astype(np.float32), synth.BF16)
    phi_act = (0.02 * rng.standard_normal((k * C, k * K + k * k))).astype(np.float32)
    b_act = np.concatenate([np.zeros(k * K), np.eye(k).reshape(-1)]).astype(np.float32)
    X = dev(Xt)
    hc.xhc_route(X, dev(Wb), dev(phi_act), dev(b_act), 0.01, 0.01, k=k, m=1, idx=dev(idx))
    torch.cuda.synchronize()
    Y = host64(X)
    bad = (3, 7, T - 1)
    for t in bad:
        np.testing.assert_array_equal(Y[t], Xt.values[t])
    ok = [t for t in range(T) if t not in bad]
    ref_X, _, _ = O.xhc_route(Xt.values[ok], idx[ok].astype(np.int64), phi_act, b_act, 0.01, 0.01,
                              Wb.values[ok])
    act = np.zeros((len(ok), N), bool)
    act[np.arange(len(ok))[:, None], idx[ok]] = True
    assert np.array_equal(Y[ok][~act], Xt.values[ok][~act])
    check_bf16("X_active valid tokens", Y[ok][act], ref_X[act])


@pytest.mark.parametrize("k,m,K,C,dtype", [(2, 1, 1, 100, synth.F32), (3, 2, 2, 64, synth.BF16),
                                           (4, 2, 3, 72, synth.F32), (5, 1, 4, 96, synth.BF16)])
def test_route_other_active_counts(k, m, K, C, dtype):
    N, T = 9, 29
    note(f"xHC route k={k} m={m} K={K} C={C} {dtype}")
    rng = np.random.default_rng(40 + k)
    Xt = synth.Tensor(rng.standard_normal((T, N, C)).astype(np.float32), dtype)
    Wb = synth.Tensor(rng.standard_normal((T, K, C)).astype(np.float32), dtype)
    idx = np.array([sorted(rng.choice(N, k, replace=False)) for _ in range(T)], np.int32)
    phi_act = (0.02 * rng.standard_normal((k * C, k * K + k * k))).astype(np.float32)
    b_act = np.concatenate([np.zeros(k * K), np.eye(k).reshape(-1)]).astype(np.float32)
    X = dev(Xt)
    out = hc.xhc_route(X, dev(Wb), dev(phi_act), dev(b_act), 0.01, 0.01, k=k, m=m, idx=dev(idx),
                       want_coeffs=True)
    torch.cuda.synchronize()
    ref_X, ref_hp, ref_hr = O.xhc_route(Xt.values, idx.astype(np.int64), phi_act, b_act, 0.01, 0.01, Wb.values)
    check_fp32("H_post_A", host64(out["h_post"]), ref_hp)
    check_fp32("H_res_A", host64(out["h_res"]), ref_hr)
    if dtype == synth.F32:
        check_fp32("X", host64(X), ref_X)
    else:
        check_bf16("X", host64(X), ref_X)


@pytest.mark.parametrize("r,C,S", [(0, 64, 5), (3, 100, 17), (2, 48, 1), (3, 4096, 13)])
def test_augment_edges(r, C, S):
    note(f"xHC augment r={r} C={C} S={S}")
    B = 3
    rng = np.random.default_rng(50 + r)
    F = synth.Tensor(rng.standard_normal((B * S, C)).astype(np.float32), synth.F32)
    kap = (4, 8, 12)[:r]
    ws = [rng.standard_normal((C, kk)).astype(np.float32) / np.sqrt(kk) for kk in kap]
    w = dev(np.concatenate([x.reshape(-1) for x in ws])) if r else torch.zeros(1, device="cuda")
    V = hc.xhc_augment(dev(F), w, kap, B, S)
    torch.cuda.synchronize()
    check_fp32("V", host64(V), O.xhc_augment(F.values, ws, B, S))


def test_augment_one_hot_taps_pin_order_and_padding():
    note("xHC augment one-hot taps")
    B, S, C = 2, 20, 32
    rng = np.random.default_rng(60)
    F = rng.standard_normal((B * S, C)).astype(np.float32)
    w = np.zeros((C, 4), np.float32)
    w[:, 0] = 1.0  # delay by 3 with zero fill
    V = hc.xhc_augment(dev(F), dev(w), (4,), B, S)
    torch.cuda.synchronize()
    ref = O.xhc_augment(F, [w], B, S)
    check_fp32("V one-hot", host64(V), ref)


@pytest.mark.parametrize("dtype", [synth.F32, synth.BF16])
def test_augment_fast_strips_one_hot_delays(dtype):
    """kappa = 4, 8, 12 (the strip-walking kernels): one-hot taps turn the three
    convs into delays of 3, 7 and 11 rows, across 36-token strip boundaries, a
    ragged last strip and two sequences (zero fill at each start); then random
    taps on the same shape. With the delays, the first 11 positions of a
    sequence have an all-zero component, which the unregularised Gram-Schmidt
    turns into 0/0 on both sides, so those positions are left out of that case."""
    B, S, C = 2, 80, 64
    rng = np.random.default_rng(61)
    F = synth.Tensor(rng.standard_normal((B * S, C)).astype(np.float32), dtype)
    kap = (4, 8, 12)
    one_hot = [np.zeros((C, kk), np.float32) for kk in kap]
    for w in one_hot:
        w[:, 0] = 1.0
    rand = [rng.standard_normal((C, kk)).astype(np.float32) / np.sqrt(kk) for kk in kap]
    pos = np.tile(np.arange(S), B)
    for name, ws, keep in (("one-hot", one_hot, pos >= 11), ("random", rand, pos >= 0)):
        note(f"xHC augment strips {name} taps B={B} S={S} C={C} dtype={dtype}")
        V = hc.xhc_augment(dev(F), dev(np.concatenate([x.reshape(-1) for x in ws])), kap, B, S)
        torch.cuda.synchronize()
        check_stream(f"V {name}", dtype, host64(V)[keep], O.xhc_augment(F.values, ws, B, S)[keep])


# ------------------------------------ shapes of the MFMA paths (bf16, C % 32 == 0)

@pytest.mark.parametrize("N,m,C,T", [(8, 2, 96, 45), (12, 3, 288, 33), (16, 2, 1024, 70), (4, 1, 32, 64)])
def test_fast_full_state_pass_shapes(N, m, C, T):
    """xhc_pre over stream groups of 4: several N, ragged T, C not a multiple of the
    256-channel super-chunk; h_pre, scores, indices (bit-exact) and F_in."""
    k = min(4, N)
    note(f"xHC xhc_pre N={N} k={k} m={m} C={C} T={T} bf16")
    inp = _xhc_inputs(50 + N, T, N, k, m, C, 1)
    X = dev(inp["X"])
    pre = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], dev(inp["w_router"]), k, m)
    torch.cuda.synchronize()
    _check_pre(inp, k, m, pre)
    note(f"xHC xhc_pre N={N} without router")
    pre2 = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], None, k, m)
    torch.cuda.synchronize()
    assert torch.equal(pre2["h_pre"], pre["h_pre"]) and torch.equal(pre2["F_in"], pre["F_in"])


@pytest.mark.parametrize("N", [4, 16])
def test_fast_full_state_pre_read_h_pre_alignment(N):
    """The pre-read reads h_pre as float4 when it is 16-byte aligned and one float at
    a time otherwise: an h_pre given at a 4-byte offset gives the same bits."""
    T, C, k, m = 70, 256, min(4, N), 1
    note(f"xHC xhc_pre N={N} C={C} T={T} with h_pre at a 4-byte offset")
    inp = _xhc_inputs(90 + N, T, N, k, m, C, 1)
    X = dev(inp["X"])
    a = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], None, k, m)
    buf = torch.empty(T * N + 1, device=X.device)
    h_off = buf[1:].view(T, N)
    F_off = torch.empty(T, C, dtype=X.dtype, device=X.device)
    b = hc.xhc_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], None, k, m, out=(h_off, F_off))
    torch.cuda.synchronize()
    assert h_off.data_ptr() % 16 == 4
    assert torch.equal(a["h_pre"], b["h_pre"]) and torch.equal(a["F_in"], b["F_in"])
    ref = O.xhc_pre(inp["X"].values, inp["phi_pre"], inp["b_pre"], inp["alpha_pre"], inp["w_router"], k, m)
    check_fp32("h_pre", host64(b["h_pre"]), ref["h_pre"])
    check_bf16("F_in", host64(b["F_in"]), ref["F_in"])


@pytest.mark.parametrize("K,C,T", [(1, 96, 29), (2, 64, 40), (3, 320, 17), (4, 4096, 33),
                                   (1, 96, 64 * 600 + 17), (4, 1024, 64 * 520 + 33)])
def test_fast_route_shapes(K, C, T):
    """xhc_route with k = 4 gathered streams for K = 1..4 write-back components, with
    supplied indices and with the router inside. The last two shapes give the
    gathered 64-token pass 601 and 521 items, so a workgroup streams up to 3 of them
    (each next item's index table prefetched while the current one runs) and the
    last tile is ragged."""
    N, k, m = 8, 4, 1
    note(f"xHC xhc_route N={N} k=4 K={K} C={C} T={T} bf16")
    inp = _xhc_inputs(60 + K, T, N, k, m, C, 1)
    rng = np.random.default_rng(70 + K)
    Wb = synth.Tensor(rng.standard_normal((T, K, C)).astype(np.float32), synth.BF16)
    phi_act = (0.02 * rng.standard_normal((k * C, k * K + k * k))).astype(np.float32)
    b_act = np.concatenate([np.zeros(k * K), np.eye(k).reshape(-1)]).astype(np.float32)
    inp = dict(inp, phi_act=phi_act, b_act=b_act)
    idx = np.array([sorted(rng.choice(N, k, replace=False)) for _ in range(T)], np.int32)
    X = dev(inp["X"])
    out = hc.xhc_route(X, dev(Wb), dev(phi_act), dev(b_act), 0.01, 0.01, k=k, m=m, idx=dev(idx),
                       want_coeffs=True)
    torch.cuda.synchronize()
    _check_route(inp["X"].values.astype(np.float64), inp, idx.astype(np.int64), Wb.values.astype(np.float64),
                 X, out)
    note(f"xHC xhc_route N={N} K={K} with the router inside")
    X2 = dev(inp["X"])
    out2 = hc.xhc_route(X2, dev(Wb), dev(phi_act), dev(b_act), 0.01, 0.01, k=k, m=m, w_router=dev(inp["w_router"]),
                        want_coeffs=True)
    torch.cuda.synchronize()
    s_ref = O.xhc_router_scores(inp["X"].values, inp["w_router"])
    np.testing.assert_array_equal(out2["idx"].cpu().numpy(), O.xhc_select(s_ref, k, m))
    check_fp32("route score", host64(out2["score"]), s_ref)
    _check_route(inp["X"].values.astype(np.float64), inp, out2["idx"].cpu().numpy().astype(np.int64),
                 Wb.values.astype(np.float64), X2, out2)


# ------------------------------- Gram-Schmidt on nearly dependent components

def _near_dependent_case(kind, B, S, C, rng):
    """F_out and conv taps whose components are close to linearly dependent:
    'current': each conv puts weight 1 on the current token and eps * N(0, 1/kappa)
    on the others, so every g_j is F_out plus an eps-sized part; 'smooth': F_out
    varies slowly along the sequence (a sine per channel of period P plus 1% noise)
    and the taps are shared by all channels, so the convs are close to multiples
    of F_out and its first differences."""
    name, par = kind.split(":")
    if name == "current":
        eps = float(par)
        F = rng.standard_normal((B * S, C)).astype(np.float32)
        ws = []
        for kk in (4, 8, 12):
            w = (eps * rng.standard_normal((C, kk)) / np.sqrt(kk)).astype(np.float32)
            w[:, kk - 1] = 1.0
            ws.append(w)
    else:
        P = float(par)
        t = np.tile(np.arange(S), B)[:, None]
        th = rng.uniform(0, 2 * np.pi, (1, C))
        amp = rng.uniform(0.5, 2.0, (1, C))
        F = (amp * np.sin(2 * np.pi * t / P + th) + 0.01 * rng.standard_normal((B * S, C))).astype(np.float32)
        ws = [np.tile((rng.standard_normal(kk) / np.sqrt(kk)).astype(np.float32), (C, 1)) for kk in (4, 8, 12)]
    return F, ws


@pytest.mark.parametrize("kind", ["current:1e-1", "current:1e-2", "current:1e-3", "smooth:64", "smooth:4096"])
@pytest.mark.parametrize("fdt,vdt", [(synth.F32, "f32"), (synth.BF16, "f32"), (synth.BF16, "bf16")])
def test_augment_nearly_dependent_components(kind, fdt, vdt):
    """The fast augmentation (kappa = 4, 8, 12, C = 4096) on nearly dependent
    components, against the float64 modified Gram-Schmidt. The float32 modified
    form errs on v_j by about u ||a_j|| / ||v_j|| (u = 2^-24: the rounding of the
    conv output, amplified by the cancellation), a Gram-matrix form by its square;
    per token and component the error must stay within 64 u ||a_j|| / ||v_j||
    (float32 V; bfloat16 V: the stream bound). Positions with a full 11-token
    window only: nearer a sequence start the components are exactly dependent for
    the 'current' taps (the modified form divides 0 by 0 there)."""
    B, S, C = 2, 96, 4096
    seeds = {"current:1e-1": 71, "current:1e-2": 72, "current:1e-3": 73, "smooth:64": 74, "smooth:4096": 75}
    rng = np.random.default_rng(seeds[kind])
    F, ws = _near_dependent_case(kind, B, S, C, rng)
    Ft = synth.Tensor(F, fdt)
    note(f"xHC augment nearly dependent components {kind} F={fdt} V={vdt} B={B} S={S} C={C}")
    V = hc.xhc_augment(dev(Ft), dev(np.concatenate([w.reshape(-1) for w in ws])), (4, 8, 12), B, S,
                       v_dtype=torch.bfloat16 if vdt == "bf16" else torch.float32)
    torch.cuda.synchronize()
    got = host64(V)
    ref = O.xhc_augment(Ft.values, ws, B, S)
    keep = np.tile(np.arange(S), B) >= 11
    assert np.all(np.isfinite(ref[keep])) and np.all(np.isfinite(got[keep]))
    np.testing.assert_array_equal(got[:, 0], Ft.values)  # v_1 = F_out exactly
    if vdt == "bf16":
        check_bf16("V nearly dependent", got[keep], ref[keep])
        return
    u = 2.0 ** -24
    for j, w in enumerate(ws, start=1):
        a = O.causal_dwconv(Ft.values, w, B, S)[keep]
        r, g = ref[keep, j], got[keep, j]
        err = np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)
        amp = np.linalg.norm(a, axis=1) / np.linalg.norm(r, axis=1)
        worst = float(np.max(err / (u * amp)))
        note(f"  v_{j + 1}: worst error {worst:.1f} u ||a||/||v||, largest ||a||/||v|| {amp.max():.1f}")
        assert worst <= 64.0, f"v_{j + 1}: error {worst:.1f} u ||a_j||/||v_j|| > 64"
