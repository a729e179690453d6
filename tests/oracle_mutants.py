"""Plausible mistakes planted in the fp64 oracle, on the CPU, to show that its
pins (tests/test_oracle_pins.py) catch them. Each mutant replaces one oracle
function with a variant that carries one mistake a reader could make from the
pages (a swapped normalisation order, a missing factor, a transposed operand,
an off-by-one range, a dropped mask ...). apply(name) patches the oracle module
and package in the running process; tests/test_oracle_mutants.py runs the pin
suite under each mutant in a subprocess and requires it to fail."""
import numpy as np

import oracle
import oracle.hc_oracle as H

_orig = {}


def _keep(name):
    if name not in _orig:
        _orig[name] = getattr(H, name)
    return _orig[name]


def _sinkhorn_rows_first(logits, iters):
    M = np.exp(np.asarray(logits, np.float64))
    for _ in range(int(iters)):
        M = M / M.sum(axis=-1, keepdims=True)  # rows first (the pages normalise columns first)
        M = M / M.sum(axis=-2, keepdims=True)
    return M


def _coeffs_post_sigma(X, phi, bias, alpha, sinkhorn_iters=20):
    h_pre, h_post, h_res = _keep("hc_coeffs")(X, phi, bias, alpha, sinkhorn_iters)
    return h_pre, h_post / 2.0, h_res  # sigma instead of 2 sigma


def _rms_sum(xflat):
    u, r = _keep("rms_normalise")(xflat)
    n = np.asarray(xflat).shape[-1]
    return u / np.sqrt(n), r * np.sqrt(n)  # the 2-norm instead of the RMS


def _post_res_transposed(X, h_res, h_post, F_out):
    return _keep("hc_post")(X, np.swapaxes(np.asarray(h_res, np.float64), -1, -2), h_post, F_out)


def _select_bottom(score, k, m):
    score = np.asarray(score, np.float64)
    T, ncand = score.shape
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(ncand), key=lambda j: (score[t, j], j))[: k - m]  # lowest scores
        idx[t] = sorted(list(range(m)) + [m + j for j in order])
    return idx


def _conv_taps_reversed(F_out, w, batch, seq):
    return _keep("causal_dwconv")(F_out, np.asarray(w, np.float64)[:, ::-1], batch, seq)


def _gs_on_inputs(comps):
    G = np.asarray(comps, np.float64)
    V = G.copy()
    for j in range(1, G.shape[1]):
        v = G[:, j].copy()
        for i in range(j):  # projections on the raw components instead of the orthogonalised ones
            v = v - (np.sum(v * G[:, i], axis=1) / np.sum(G[:, i] * G[:, i], axis=1))[:, None] * G[:, i]
        V[:, j] = v
    return V


def _flash_input_inclusive(l, F_pre_l, h_pre_l, idx, H_post, F_outs):
    L = np.asarray(H_post).shape[2]
    return _keep("xhc_flash_input")(min(l + 1, L), F_pre_l, h_pre_l, idx, H_post, F_outs)  # j <= l


def _flash_post_mix_all(X, idx, H_post, H_res, F_outs):
    X = np.asarray(X, np.float64).copy()
    idx = np.asarray(idx)
    F = np.asarray(F_outs, np.float64)
    T = F.shape[0]
    X_A = H.xhc_gather(X, idx) + np.einsum("taj,tjc->tac", np.asarray(H_post, np.float64), F)
    X[np.arange(T)[:, None], idx] = np.einsum("tab,tbc->tac", np.asarray(H_res, np.float64), X_A)  # mixes its own write
    return X


def _sinkhorn_bwd_sign(logits, grad, iters):
    return -_keep("sinkhorn_knopp_backward")(logits, grad, iters)


def _route_zero_inactive(X, idx, phi_act, b_act, alpha_post, alpha_res, Wb, sinkhorn_iters=20):
    Xn, hp, hr = _keep("xhc_route")(X, idx, phi_act, b_act, alpha_post, alpha_res, Wb, sinkhorn_iters)
    keep = np.zeros(Xn.shape[:2], bool)
    keep[np.arange(Xn.shape[0])[:, None], np.asarray(idx)] = True
    return np.where(keep[:, :, None], Xn, 0.0), hp, hr  # inactive streams lost


def _logits_no_bias(X, phi, bias, alpha):
    return _keep("mhc_logits")(X, phi, np.zeros_like(np.asarray(bias, np.float64)), alpha)


def _gates_backward_no_rms(dz, P, rho, gate, x, phi, N):
    dP = dz * gate[None, :] * rho[:, None]
    dx = dP @ phi.T  # the gradient through the RMS factor forgotten
    return dx, x.T @ dP, dz.sum(axis=0), (dz * P * rho[:, None]).sum(axis=0)


def _conv_backward_causal(F_out, w, batch, seq, dg):
    dF, dw = _keep("causal_dwconv_backward")(F_out, w, batch, seq, dg)
    return _keep("causal_dwconv")(dg, w, batch, seq), dw  # the forward direction instead of the transpose


def _mgs_backward_sign(comps, dV):
    return -_keep("modified_gram_schmidt_backward")(comps, dV)


def _route_backward_drops_passthrough(X, idx, phi_act, b_act, alpha_post, alpha_res, Wb, dX_next, sinkhorn_iters=20):
    r = dict(_keep("xhc_route_backward")(X, idx, phi_act, b_act, alpha_post, alpha_res, Wb, dX_next, sinkhorn_iters))
    keep = np.zeros(r["dX"].shape[:2], bool)
    keep[np.arange(keep.shape[0])[:, None], np.asarray(idx)] = True
    r["dX"] = np.where(keep[:, :, None], r["dX"], 0.0)  # inactive rows get no gradient
    return r


def _router_without_rms(X, w_router):
    X = np.asarray(X, np.float64)
    return H.sigmoid(X.reshape(X.shape[0], -1) @ np.asarray(w_router, np.float64))  # state not normalised


def _router_without_sigmoid(X, w_router):
    u, _ = H.rms_normalise(H.flatten_state(X))
    return u @ np.asarray(w_router, np.float64)  # raw logits instead of sigma(logits)


MUTANTS = {
    "router_without_rms": ("xhc_router_scores", _router_without_rms),
    "router_without_sigmoid": ("xhc_router_scores", _router_without_sigmoid),
    "sinkhorn_rows_first": ("sinkhorn_knopp", _sinkhorn_rows_first),
    "post_gate_sigma": ("hc_coeffs", _coeffs_post_sigma),
    "rms_is_two_norm": ("rms_normalise", _rms_sum),
    "post_res_transposed": ("hc_post", _post_res_transposed),
    "select_lowest_scores": ("xhc_select", _select_bottom),
    "conv_taps_reversed": ("causal_dwconv", _conv_taps_reversed),
    "gram_schmidt_on_inputs": ("modified_gram_schmidt", _gs_on_inputs),
    "flash_input_own_output": ("xhc_flash_input", _flash_input_inclusive),
    "flash_post_mixes_last_write": ("xhc_flash_post", _flash_post_mix_all),
    "sinkhorn_backward_sign": ("sinkhorn_knopp_backward", _sinkhorn_bwd_sign),
    "route_drops_inactive": ("xhc_route", _route_zero_inactive),
    "logits_without_bias": ("mhc_logits", _logits_no_bias),
    "gates_backward_without_rms_term": ("_gates_backward", _gates_backward_no_rms),
    "conv_backward_forward_direction": ("causal_dwconv_backward", _conv_backward_causal),
    "gram_schmidt_backward_sign": ("modified_gram_schmidt_backward", _mgs_backward_sign),
    "route_backward_drops_passthrough": ("xhc_route_backward", _route_backward_drops_passthrough),
}


def apply(name):
    fn, repl = MUTANTS[name]
    _keep(fn)
    setattr(H, fn, repl)
    if hasattr(oracle, fn):  # names with a leading underscore stay in the module
        setattr(oracle, fn, repl)
