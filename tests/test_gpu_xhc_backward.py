"""GPU parity of the xHC routed-step backward (xhc_route_backward, then
xhc_pre_backward; k = 4, K = 1, bfloat16) against the fp64 oracle's
xhc_route_backward and xhc_pre_backward, through the C ABI, on the synth
recipe's xHC inputs and upstream gradients.

Tolerances as for the mHC backward: the route's dX and dF_out are bfloat16
outputs rounded once from float32 (the route's pass-through rows are compared
bit for bit); the map gradients and dphi, db, dalpha are float32 sums (relative
L2 1e-4, from the float32 channel sums, 20 reverse Sinkhorn steps and dP split
into two bfloat16 parts on the matrix cores). The final dX is rounded twice: the
route's gradient is stored in bfloat16, and the pre call adds its own term to
it and rounds again. So per element it may be off by up to half a bfloat16 ulp
of the route's value plus half an ulp of the sum; the bound is max(2e-2, one
ulp of each), with relative L2 1e-2.
"""
import numpy as np
import pytest

import oracle as O
import synth
from hc_testutil import BF16_MAX_ABS, BF16_REL_L2, bf16_ulp, check_bf16, check_fp32, dev, have_gpu, host64, note, rel_l2

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc

BWD_REL = 1e-4


def _inputs(seed, T, N, C, m=1, strong=False):
    inp = synth.xhc_layer(seed, 0, T, N, C, 4, m, 1, synth.BF16)
    g = synth.mhc_grads(seed, 0, T, N, C, synth.BF16)  # dX_next [T, N, C], dF_in [T, C]
    if strong:  # gates and maps far from their values at z = b
        inp["phi_act"] = (inp["phi_act"] * np.float32(10.0)).astype(np.float32)
        inp["phi_pre"] = (inp["phi_pre"] * np.float32(10.0)).astype(np.float32)
        inp["alpha_post"], inp["alpha_res"], inp["alpha_pre"] = 0.6, 0.9, 0.7
    # the active set the forward chose
    idx = O.xhc_pre(inp["X"].values, inp["phi_pre"], inp["b_pre"], inp["alpha_pre"], inp["w_router"], 4, m)["idx"]
    return inp, g, idx.astype(np.int32)


def _gpu(inp, g, idx, iters=20):
    X = dev(inp["X"])
    dX = dev(g["dX_next"]).clone()
    r = hc.xhc_route_backward(X, dev(idx), dev(inp["phi_act"]), dev(inp["b_act"]), inp["alpha_post"],
                              inp["alpha_res"], dev(inp["F_out"]), dX, iters)
    torch.cuda.synchronize()
    route = dict(zip(("dX", "dWb", "dphi_act", "db_act", "dalpha", "dh"), (host64(t) for t in r)))
    p = hc.xhc_pre_backward(X, dev(inp["phi_pre"]), dev(inp["b_pre"]), inp["alpha_pre"], dev(g["dF_in"]), dX)
    torch.cuda.synchronize()
    pre = dict(zip(("dX", "dphi_pre", "db_pre", "dalpha", "dh_pre"), (host64(t) for t in p)))
    return route, pre


def _oracle(inp, g, idx, iters=20, chunk=None, rows=None):
    T = inp["X"].values.shape[0]
    chunk = chunk or T
    keep = np.arange(T) if rows is None else np.asarray(rows)
    acc = {}
    per = {"dX_route": [], "dX": [], "dWb": [], "dh": [], "dh_pre": []}
    for s in range(0, T, chunk):
        sl = slice(s, min(T, s + chunk))
        X = inp["X"].values[sl]
        r = O.xhc_route_backward(X, idx[sl], inp["phi_act"], inp["b_act"], inp["alpha_post"], inp["alpha_res"],
                                 inp["F_out"].values[sl], g["dX_next"].values[sl], iters)
        p = O.xhc_pre_backward(X, inp["phi_pre"], inp["b_pre"], inp["alpha_pre"], g["dF_in"].values[sl])
        for k, v in (("dphi_act", r["dphi_act"]), ("db_act", r["db_act"]),
                     ("dalpha", np.array([r["dalpha_post"], r["dalpha_res"]])), ("dphi_pre", p["dphi_pre"]),
                     ("db_pre", p["db_pre"]), ("dalpha_pre", np.array([p["dalpha_pre"]]))):
            acc[k] = acc.get(k, 0.0) + v
        sel = keep[(keep >= sl.start) & (keep < sl.stop)] - sl.start
        per["dX_route"].append(r["dX"][sel])
        per["dX"].append(r["dX"][sel] + p["dX"][sel])
        per["dWb"].append(r["dWb"][sel, 0])
        per["dh"].append(r["dh"][sel])
        per["dh_pre"].append(p["dh_pre"][sel])
    return {**acc, **{k: np.concatenate(v) for k, v in per.items()}}


def _check_two_roundings(name, got, ref, got_first, ref_first):
    """bfloat16 output rounded twice: the route stores got_first = rnd(a) (a the float32
    route gradient), the pre call then stores got = rnd(got_first + b) (b its float32
    gradient). Round to nearest even moves a value by at most half an ulp of the
    rounded result, so |got - ref| <= ulp(got_first)/2 + ulp(got)/2 + |a - ref_first| +
    |b - (ref - ref_first)|; the float32 errors of a and b are bounded here by 2e-5 of
    the magnitudes plus 1e-6. Per element: within max(2e-2, that bound)."""
    e = rel_l2(got, ref)
    assert e <= BF16_REL_L2, f"{name}: relative L2 {e:.3e} > {BF16_REL_L2}"
    err = np.abs(got - ref)
    fp32 = 2e-5 * (np.abs(ref_first) + np.abs(ref - ref_first)) + 1e-6
    bound = np.maximum(BF16_MAX_ABS, 0.5 * bf16_ulp(got_first) + 0.5 * bf16_ulp(got) + fp32)
    bad = int(np.sum(err > bound))
    assert bad == 0, (f"{name}: {bad} elements exceed max(2e-2, ulp(first)/2 + ulp(sum)/2 + float32 error); "
                      f"worst {err.max():.3e}")


def _compare(route, pre, ref, g, idx, rows=None):
    sel = slice(None) if rows is None else np.asarray(rows)
    T = route["dX"].shape[0]
    # rows outside the active set pass dX_next through unchanged (bit for bit)
    inactive = np.ones(route["dX"].shape[:2], bool)
    inactive[np.arange(T)[:, None], idx] = False
    dXn = g["dX_next"].values.astype(np.float64)
    np.testing.assert_array_equal(route["dX"][inactive], dXn[inactive])
    check_bf16("route dX", route["dX"][sel], ref["dX_route"])
    check_bf16("dF_out", route["dWb"][sel], ref["dWb"])
    check_fp32("dh", route["dh"][sel], ref["dh"], BWD_REL)
    _check_two_roundings("dX", pre["dX"][sel], ref["dX"], route["dX"][sel], ref["dX_route"])
    check_fp32("dh_pre", pre["dh_pre"][sel], ref["dh_pre"], BWD_REL)
    errs = {k: check_fp32(k, route[k], ref[k], BWD_REL) for k in ("dphi_act", "db_act", "dalpha")}
    errs.update({k: check_fp32(k, pre[k], ref[k], BWD_REL) for k in ("dphi_pre", "db_pre")})
    errs["dalpha_pre"] = check_fp32("dalpha_pre", pre["dalpha"], ref["dalpha_pre"], BWD_REL)
    note(f"relative L2: {', '.join(f'{k} {v:.2e}' for k, v in errs.items())}")


@pytest.mark.parametrize("N,C,T,m", [(16, 256, 70, 2), (8, 96, 33, 1), (4, 128, 40, 1), (12, 4096, 20, 2),
                                     (16, 256, 64 * 300 + 9, 2)])
def test_xhc_backward_shapes(N, C, T, m):
    """Several N (k = 4 active), ragged T, C not a multiple of the 128-channel
    chunks, the workload's C; N = 4 is the dense case (every stream active). At
    19,209 tokens the gathered projection's workgroups take 2 items and the dX
    passes' workgroups several tiles each, ending on a ragged one."""
    note(f"xHC backward N={N} C={C} T={T} m={m} bf16")
    inp, g, idx = _inputs(500 + N + T, T, N, C, m)
    route, pre = _gpu(inp, g, idx)
    _compare(route, pre, _oracle(inp, g, idx, chunk=4096), g, idx)


def test_xhc_backward_strong_gates():
    note("xHC backward strong gates N=16 C=512 T=64")
    inp, g, idx = _inputs(530, 64, 16, 512, 2, strong=True)
    route, pre = _gpu(inp, g, idx)
    _compare(route, pre, _oracle(inp, g, idx), g, idx)


def test_xhc_backward_deterministic():
    note("xHC backward determinism N=16 C=1024 T=100")
    inp, g, idx = _inputs(540, 100, 16, 1024, 2)
    a, b = _gpu(inp, g, idx), _gpu(inp, g, idx)
    for x, y in zip(a, b):
        for k in x:
            np.testing.assert_array_equal(x[k], y[k], err_msg=k)


def test_xhc_backward_full_size():
    """The N = 16, k = 4, m = 2, C = 4096, T = 8192 workload: dphi, db, dalpha against
    the oracle over every token (chunks of 256), dX, dF_out and the map gradients
    on sampled tokens, the pass-through rows on every token."""
    w = synth.WORKLOADS["xhc_N16_k4_m2_C4096_T8192_bf16_K1"]
    T, N, C = w["T"], w["N"], w["C"]
    note(f"xHC backward full size N={N} C={C} T={T} bf16")
    inp, g, idx = _inputs(w["seed"], T, N, C, w["m"])
    route, pre = _gpu(inp, g, idx)
    rng = np.random.default_rng(550)
    rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 126, replace=False)]))
    _compare(route, pre, _oracle(inp, g, idx, chunk=256, rows=rows), g, idx, rows=rows)


# ------------------------------------------------ augmented step (K = 4)

def _aug_inputs(seed, B, S, N, C, m=2):
    inp = synth.xhc_layer(seed, 0, B * S, N, C, 4, m, 4, synth.BF16)
    g = synth.mhc_grads(seed, 0, B * S, N, C, synth.BF16)
    idx = O.xhc_pre(inp["X"].values, inp["phi_pre"], inp["b_pre"], inp["alpha_pre"], inp["w_router"], 4, m)["idx"]
    return inp, g, idx.astype(np.int32)


@pytest.mark.parametrize("B,S,N,C", [(2, 200, 16, 96), (3, 7, 8, 512), (1, 300, 16, 4096)])
def test_augmented_step_backward(B, S, N, C):
    """K = 4: the GPU forward's V feeds xhc_route_backward (dV in float32), whose dV
    feeds xhc_augment_backward (dF_out, the conv taps); each stage against the
    oracle on the same inputs: several strips of 128 tokens with sequence starts
    inside them, sequences shorter than the longest kernel, C past whole
    channel blocks."""
    note(f"xHC augmented backward B={B} S={S} N={N} C={C} bf16")
    inp, g, idx = _aug_inputs(560 + S, B, S, N, C)
    kap = inp["kappas"]
    w = np.concatenate([x.reshape(-1) for x in inp["conv_w"]])
    V = hc.xhc_augment(dev(inp["F_out"]), dev(w), kap, B, S)
    torch.cuda.synchronize()
    Vh = host64(V)
    X = dev(inp["X"])
    dX = dev(g["dX_next"]).clone()
    dXo, dV, dphi, db, dal, dh = hc.xhc_route_backward(X, dev(idx), dev(inp["phi_act"]), dev(inp["b_act"]),
                                                       inp["alpha_post"], inp["alpha_res"], V, dX)
    dF, dw = hc.xhc_augment_backward(dev(inp["F_out"]), dev(w), kap, B, S, dV)
    torch.cuda.synchronize()
    r = O.xhc_route_backward(inp["X"].values, idx, inp["phi_act"], inp["b_act"], inp["alpha_post"],
                             inp["alpha_res"], Vh, g["dX_next"].values, 20)
    check_bf16("route dX", host64(dXo), r["dX"])
    check_fp32("dV", host64(dV), r["dWb"], BWD_REL)
    check_fp32("dh", host64(dh), r["dh"], BWD_REL)
    errs = {"dphi_act": check_fp32("dphi_act", host64(dphi), r["dphi_act"], BWD_REL),
            "db_act": check_fp32("db_act", host64(db), r["db_act"], BWD_REL),
            "dalpha": check_fp32("dalpha", host64(dal), np.array([r["dalpha_post"], r["dalpha_res"]]), BWD_REL)}
    # the augmentation backward on the GPU's own dV (its stage on its own input)
    a = O.xhc_augment_backward(inp["F_out"].values, inp["conv_w"], B, S, host64(dV))
    check_bf16("dF_out", host64(dF), a["dF_out"])
    ref_w = np.concatenate([x.reshape(-1) for x in a["dconv_ws"]])
    errs["dconv"] = check_fp32("dconv", host64(dw), ref_w, BWD_REL)
    note(f"relative L2: {', '.join(f'{k} {v:.2e}' for k, v in errs.items())}")


def test_augment_backward_deterministic():
    note("xhc_augment_backward determinism B=2 S=300 C=256")
    B, S, C = 2, 300, 256
    inp = synth.xhc_layer(590, 0, B * S, 4, C, 4, 1, 4, synth.BF16)
    w = np.concatenate([x.reshape(-1) for x in inp["conv_w"]])
    dV = torch.randn(B * S, 4, C, device="cuda", generator=torch.Generator(device="cuda").manual_seed(5))
    a = hc.xhc_augment_backward(dev(inp["F_out"]), dev(w), inp["kappas"], B, S, dV)
    b = hc.xhc_augment_backward(dev(inp["F_out"]), dev(w), inp["kappas"], B, S, dV)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _aug_only(seed, B, S, C, dtype):
    """F_out, conv taps (as the xHC recipe draws them) and a seeded upstream dV."""
    rng = synth.make_rng(seed, 0)
    F = synth.Tensor(synth.normal(rng, (B * S, C)), dtype)
    ws = [synth.normal(rng, (C, k), float(np.sqrt(1.0 / k))) for k in (4, 8, 12)]
    dV = synth.normal(synth.make_rng(seed, 0, stream=2), (B * S, 4, C))
    return F, ws, dV


def _aug_only_check(F, ws, dV, B, S):
    w = np.concatenate([x.reshape(-1) for x in ws])
    dF, dw = hc.xhc_augment_backward(dev(F), dev(w), (4, 8, 12), B, S, torch.from_numpy(dV).cuda())
    torch.cuda.synchronize()
    a = O.xhc_augment_backward(F.values, ws, B, S, dV.astype(np.float64))
    if F.dtype == synth.BF16:
        check_bf16("dF_out", host64(dF), a["dF_out"])
        e = rel_l2(host64(dF), a["dF_out"])
    else:
        e = check_fp32("dF_out", host64(dF), a["dF_out"], BWD_REL)
    ed = check_fp32("dconv", host64(dw), np.concatenate([x.reshape(-1) for x in a["dconv_ws"]]), BWD_REL)
    note(f"relative L2: dF_out {e:.2e}, dconv {ed:.2e}")


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 11, 12, 13])
def test_augment_backward_short_sequences(S):
    """Sequences no longer than the convs' reach: every token near a sequence
    start (masked windows, the transpose's sums cleared at each start, the
    position wrapping inside one load group); C = 200 leaves part of the last
    channel block idle."""
    B = 37
    note(f"xhc_augment_backward short sequences B={B} S={S} C=200 bf16")
    _aug_only_check(*_aug_only(600 + S, B, S, 200, synth.BF16), B, S)


@pytest.mark.parametrize("B,S,C", [(3, 100, 300), (1, 517, 64)])
def test_augment_backward_float32(B, S, C):
    """F_out and dF_out in float32: the same kernels on float32 rows."""
    note(f"xhc_augment_backward float32 B={B} S={S} C={C}")
    _aug_only_check(*_aug_only(620 + S, B, S, C, synth.F32), B, S)


def test_augment_backward_full_size():
    """The augmented workload's shape, B = 2 sequences of S = 4096, C = 4096, in one
    call: dF_out over every element and the conv taps summed over all tokens."""
    B, S, C = 2, 4096, 4096
    note(f"xhc_augment_backward full size B={B} S={S} C={C} bf16")
    _aug_only_check(*_aug_only(640, B, S, C, synth.BF16), B, S)


def test_augment_backward_long_strips():
    """A shape that takes the 256-token strips (at least two workgroups per CU)
    with sequence starts inside strips (every 3000 tokens) and a ragged last strip
    (9000 = 35 * 256 + 40)."""
    B, S, C = 3, 3000, 4096
    note(f"xhc_augment_backward long strips B={B} S={S} C={C} bf16")
    _aug_only_check(*_aug_only(650, B, S, C, synth.BF16), B, S)


def test_augment_backward_odd_channels():
    """C odd: the Gram pass takes one channel per thread (the pair path needs even C)."""
    B, S, C = 5, 37, 201
    note(f"xhc_augment_backward odd C B={B} S={S} C={C} bf16")
    _aug_only_check(*_aug_only(660, B, S, C, synth.BF16), B, S)
