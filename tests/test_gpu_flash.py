"""GPU parity of the xHC-Flash calls (xhc_flash_pre, xhc_flash_maps,
xhc_flash_input, xhc_flash_post) against the fp64 oracle, through the C ABI.

Each stage is checked against the oracle on the GPU's own inputs to that stage
(the GPU's idx, h_pre, F_pre, H_post, H_res), so every bfloat16 output is
rounded once and the stream bound holds: relative L2 1e-2 and per element
max(2e-2, one bf16 ulp). Float32 outputs (h_pre, H_post, H_res, scores) carry
float32 sums over N*C or k*C products and 20 Sinkhorn steps: relative L2 1e-5
(the default float32 bound of these tests). The active set is compared bit-exactly on
inputs whose top router scores are at least 1e-3 apart.
"""
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


def _gaps(X, w_r, k, m, seed):
    """Redraw (seeded) the tokens whose top-(k-m+1) candidate scores are within GAP."""
    rng = synth.make_rng(seed, 0, stream=7)
    todo = np.arange(X.shape[0])
    for _ in range(50):
        s = np.concatenate([O.xhc_router_scores(X.values[todo[i:i + 256]], w_r) for i in range(0, todo.size, 256)])
        top = -np.sort(-s, axis=1)[:, : k - m + 1]
        bad = todo[np.any(top[:, :-1] - top[:, 1:] <= GAP, axis=1)]
        if bad.size == 0:
            return
        synth.redraw_rows(rng, X, bad)
        todo = bad
    raise AssertionError("could not enforce score gaps")


def _inputs(seed, T, N, C, k, m, L, dtype, alpha=0.01, phi_std=synth.PHI_STD, K_last=1):
    """Block-entry state, L pre maps, the router, the active maps' weights (identity
    res logits, as the xHC recipe) for L - 1 + K_last write-back components, L
    sublayer outputs and (K_last = 4) the last sublayer's conv taps, all seeded."""
    rng = synth.make_rng(seed, 0)
    X = synth.Tensor(synth.normal(rng, (T, N, C)), dtype)
    Kb = L - 1 + K_last
    inp = dict(X=X, phi_pre=synth.normal(rng, (L, N * C, N), phi_std),
               b_pre=synth.normal(rng, (L, N), 0.1),
               w_router=synth.normal(rng, (N * C, N - m), float(np.sqrt(1.0 / (N * C)))),
               phi_act=synth.normal(rng, (k * C, k * Kb + k * k), phi_std))
    b_act = np.zeros(k * Kb + k * k, np.float32)
    b_act[k * Kb:] = np.eye(k, dtype=np.float32).reshape(-1)
    inp["b_act"] = b_act
    inp["F_outs"] = synth.Tensor(synth.normal(rng, (T, L, C)), dtype)
    if K_last > 1:
        inp["conv_w"] = [synth.normal(rng, (C, kk), float(np.sqrt(1.0 / kk))) for kk in (4, 8, 12)[:K_last - 1]]
    inp["alpha"] = alpha
    _gaps(X, inp["w_router"], k, m, seed)
    return inp


def _run_and_check(inp, k, m, L, sample=None, K_last=1, seqs=1):
    X = dev(inp["X"])
    T, N, C = X.shape
    sl = (lambda a: a) if sample is None else (lambda a: a[sample])
    a = inp["alpha"]
    idx, score, h_pre, F_pre = hc.xhc_flash_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), a, dev(inp["w_router"]),
                                                k=k, m=m)
    Hp, Hr = hc.xhc_flash_maps(X, idx, dev(inp["phi_act"]), dev(inp["b_act"]), a, a, L, K_last=K_last)
    F_outs = dev(inp["F_outs"])
    if K_last > 1:  # the last sublayer (the MLP) writes back its augmentation
        kap = (4, 8, 12)[:K_last - 1]
        V = hc.xhc_augment(F_outs[:, L - 1].contiguous(), dev(np.concatenate([w.reshape(-1) for w in inp["conv_w"]])),
                           kap, seqs, T // seqs)
        W = torch.cat([F_outs[:, :L - 1], V], 1).contiguous()
    else:
        W = F_outs
    F_in = [hc.xhc_flash_input(l, F_pre[l], h_pre[l], idx, Hp, W, K_last=K_last) for l in range(L)]
    Xp = X.clone()
    hc.xhc_flash_post(Xp, idx, Hp, Hr, W, K_last=K_last)
    torch.cuda.synchronize()
    if K_last > 1:
        refV = O.xhc_augment(inp["F_outs"].values[:, L - 1], inp["conv_w"], seqs, T // seqs)
        check_stream("V of the last sublayer", inp["X"].dtype, sl(host64(V)), sl(refV))
        # the same block end with the last sublayer's components kept apart (W_last): the
        # rows of W they replace are not read, and the state is bit-identical
        Wz = W.clone()
        Wz[:, L - 1:] = float("nan")
        Xq = X.clone()
        hc.xhc_flash_post(Xq, idx, Hp, Hr, Wz, K_last=K_last, W_last=V)
        torch.cuda.synchronize()
        assert torch.equal(Xq, Xp)
    dt = inp["X"].dtype
    Xv = sl(inp["X"].values)
    pre = O.xhc_flash_pre(Xv, list(inp["phi_pre"]), list(inp["b_pre"]), a, inp["w_router"], k, m)
    gidx = sl(idx.cpu().numpy()).astype(np.int64)
    np.testing.assert_array_equal(gidx, pre["idx"])
    check_fp32("score", sl(host64(score)), pre["score"])
    check_fp32("h_pre", host64(h_pre)[:, sample] if sample is not None else host64(h_pre), pre["h_pre"])
    gF = host64(F_pre)
    for l in range(L):
        check_stream(f"F_pre[{l}]", dt, sl(gF[l]), pre["F_pre"][l])
    ref_hp, ref_hr = O.xhc_flash_maps(Xv, gidx, inp["phi_act"], inp["b_act"], a, a, L, K_last=K_last)
    check_fp32("H_post", sl(host64(Hp)), ref_hp)
    check_fp32("H_res", sl(host64(Hr)), ref_hr)
    gh, gHp, gHr = host64(h_pre), sl(host64(Hp)), sl(host64(Hr))
    Fo = sl(host64(W))  # the block's components as the GPU holds them (V from the GPU's augmentation)
    for l in range(L):  # the correction on the GPU's own F_pre, h_pre and H_post
        ref = O.xhc_flash_input(l, sl(gF[l]), sl(gh[l]), gidx, gHp, Fo)
        check_stream(f"F_in[{l}]", dt, sl(host64(F_in[l])), ref)
    ref_X = O.xhc_flash_post(Xv, gidx, gHp, gHr, Fo, K_last=K_last)
    gX = sl(host64(Xp))
    act = np.zeros(gX.shape[:2], bool)
    act[np.arange(gX.shape[0])[:, None], gidx] = True
    assert np.array_equal(gX[~act], Xv[~act]), "rows outside the active set changed"
    check_stream("X_L active rows", dt, gX[act], ref_X[act])
    return dict(idx=idx, h_pre=h_pre, F_pre=F_pre, Hp=Hp, Hr=Hr, F_outs=W)


@pytest.mark.parametrize("L,N,C,T,k,m,dtype", [
    (2, 16, 256, 70, 4, 2, synth.BF16),   # attention + MLP, the fast paths, ragged T
    (4, 16, 128, 33, 4, 2, synth.BF16),   # the four-sublayer block
    (3, 8, 96, 40, 4, 1, synth.BF16),     # C not a multiple of 128, N = 8
    (1, 16, 256, 5, 4, 2, synth.BF16),    # one sublayer: plain xHC
    (2, 6, 40, 29, 3, 1, synth.F32),      # float32 and shapes only the generic kernels take
    (4, 12, 64, 1, 4, 2, synth.BF16),     # one token
    (2, 16, 40, 20, 4, 2, synth.BF16),    # C % 32 != 0: generic projections beside the 16-byte kernels
    (2, 16, 96, 50, 4, 2, synth.BF16),    # the 46-column entry pass with a partial 128-channel step
    (4, 16, 160, 20, 4, 2, synth.BF16),   # the 78-column entry pass with a partial 128-channel step
])
def test_flash_block(L, N, C, T, k, m, dtype):
    note(f"xhc_flash L={L} N={N} C={C} T={T} k={k} m={m} {dtype}")
    _run_and_check(_inputs(800 + 7 * L + N + T, T, N, C, k, m, L, dtype), k, m, L)


def test_flash_strong_maps():
    """Gates and weights large enough that h_pre, H_post and H_res are far from
    their values at the bias, so the correction scalars vary per token."""
    note("xhc_flash strong maps L=2 N=16 C=256 T=64")
    _run_and_check(_inputs(830, 64, 16, 256, 4, 2, 2, synth.BF16, alpha=0.8, phi_std=0.3), 4, 2, 2)


def test_flash_input_in_place():
    """F_in may be written over F_pre_l itself: same values as into a fresh buffer."""
    note("xhc_flash_input in place L=3 N=16 C=256 T=40")
    inp = _inputs(840, 40, 16, 256, 4, 2, 3, synth.BF16)
    r = _run_and_check(inp, 4, 2, 3)
    fresh = hc.xhc_flash_input(2, r["F_pre"][2], r["h_pre"][2], r["idx"], r["Hp"], r["F_outs"])
    buf = r["F_pre"][2].clone()
    hc.xhc_flash_input(2, buf, r["h_pre"][2], r["idx"], r["Hp"], r["F_outs"], out=buf)
    torch.cuda.synchronize()
    assert torch.equal(fresh, buf)


@pytest.mark.parametrize("L", [2, 4])
def test_flash_full_size(L):
    """N = 16, k = 4, m = 2, C = 4096, T = 8192 (the xHC workload's shape) in one
    block; every call on all tokens, the oracle on 256 sampled tokens (each token's
    block is independent of the others)."""
    note(f"xhc_flash full size L={L} N=16 C=4096 T=8192 bf16")
    T, N, C = 8192, 16, 4096
    inp = _inputs(850 + L, T, N, C, 4, 2, L, synth.BF16)
    rng = np.random.default_rng(860 + L)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 254, replace=False)]))
    _run_and_check(inp, 4, 2, L, sample=sample)


def test_flash_single_sublayer_matches_xhc_calls():
    """A block of one sublayer is one plain xHC sublayer: xhc_flash_pre +
    xhc_flash_maps + xhc_flash_post give the same active set, h_pre, dense read,
    maps and state, bit for bit, as xhc_pre + xhc_route on the same inputs."""
    note("xhc_flash L=1 against xhc_pre + xhc_route N=16 C=256 T=50")
    k, m = 4, 2
    inp = _inputs(870, 50, 16, 256, k, m, 1, synth.BF16, alpha=0.5, phi_std=0.2)
    X = dev(inp["X"])
    a = inp["alpha"]
    idx, score, h_pre, F_pre = hc.xhc_flash_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), a, dev(inp["w_router"]),
                                                k=k, m=m)
    Hp, Hr = hc.xhc_flash_maps(X, idx, dev(inp["phi_act"]), dev(inp["b_act"]), a, a, 1)
    F_outs = dev(inp["F_outs"])
    Xf = X.clone()
    hc.xhc_flash_post(Xf, idx, Hp, Hr, F_outs)
    pre = hc.xhc_pre(X, dev(inp["phi_pre"][0]), dev(inp["b_pre"][0]), a, w_router=dev(inp["w_router"]), k=k, m=m)
    Xr = X.clone()
    out = hc.xhc_route(Xr, F_outs[:, 0].contiguous(), dev(inp["phi_act"]), dev(inp["b_act"]), a, a, k=k, m=m,
                       idx=pre["idx"], want_coeffs=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, pre["idx"])
    assert torch.equal(h_pre[0], pre["h_pre"])
    assert torch.equal(F_pre[0], pre["F_in"])
    assert torch.equal(Hp, out["h_post"]) and torch.equal(Hr, out["h_res"])
    assert torch.equal(Xf, Xr)


@pytest.mark.parametrize("L,N,C,T,seqs,dtype", [
    (2, 16, 256, 70, 2, synth.BF16),   # attention + augmented MLP: 5 components
    (4, 16, 128, 36, 3, synth.BF16),   # four sublayers, the last augmented: 7 components
    (2, 8, 40, 26, 2, synth.F32),      # float32 and shapes only the generic kernels take
])
def test_flash_block_augmented_mlp(L, N, C, T, seqs, dtype):
    """The block's last sublayer writes back K_r = 4 augmented components (the
    README's default configuration augments the MLP side): maps with L - 1 + 4
    post columns, corrected inputs, and the block end against the oracle."""
    note(f"xhc_flash augmented MLP L={L} N={N} C={C} T={T} {dtype}")
    inp = _inputs(880 + 7 * L + N + T, T, N, C, 4, 2 if N > 8 else 1, L, dtype, K_last=4)
    _run_and_check(inp, 4, 2 if N > 8 else 1, L, K_last=4, seqs=seqs)


def test_flash_augmented_full_size():
    """Attention + augmented MLP at N = 16, k = 4, m = 2, C = 4096, T = 8192 (2
    sequences of 4096): every call on all tokens, the oracle on sampled tokens."""
    note("xhc_flash augmented MLP full size L=2 N=16 C=4096 T=8192 bf16")
    T, N, C = 8192, 16, 4096
    inp = _inputs(890, T, N, C, 4, 2, 2, synth.BF16, K_last=4)
    rng = np.random.default_rng(891)
    sample = np.unique(np.concatenate([[0, 1, 4095, 4096, 4097, T - 1], rng.choice(T, 250, replace=False)]))
    _run_and_check(inp, 4, 2, 2, sample=sample, K_last=4, seqs=2)


def test_flash_single_augmented_sublayer_matches_route():
    """A block of one augmented sublayer is xhc_route with its K = 4 components:
    the same maps and state, bit for bit."""
    note("xhc_flash L=1 K_last=4 against xhc_route K=4 N=16 C=256 T=48")
    k, m = 4, 2
    inp = _inputs(895, 48, 16, 256, k, m, 1, synth.BF16, alpha=0.5, phi_std=0.2, K_last=4)
    X = dev(inp["X"])
    a = inp["alpha"]
    idx, _, _, _ = hc.xhc_flash_pre(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), a, dev(inp["w_router"]), k=k, m=m)
    F = dev(inp["F_outs"])[:, 0].contiguous()
    V = hc.xhc_augment(F, dev(np.concatenate([w.reshape(-1) for w in inp["conv_w"]])), (4, 8, 12), 2, 24)
    Hp, Hr = hc.xhc_flash_maps(X, idx, dev(inp["phi_act"]), dev(inp["b_act"]), a, a, 1, K_last=4)
    Xf = X.clone()
    hc.xhc_flash_post(Xf, idx, Hp, Hr, V, K_last=4)
    Xr = X.clone()
    out = hc.xhc_route(Xr, V, dev(inp["phi_act"]), dev(inp["b_act"]), a, a, k=k, m=m, idx=idx, want_coeffs=True)
    torch.cuda.synchronize()
    assert torch.equal(Hp, out["h_post"]) and torch.equal(Hr, out["h_res"])
    assert torch.equal(Xf, Xr)
