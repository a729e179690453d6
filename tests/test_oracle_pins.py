"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: hand-derived
fixtures (tests/golden), closed forms, invariants stated on the pages, brute
force over tiny inputs, or an independent library routine. The tests are
chosen so that a dropped term, a wrong sign or index, a transposed operand or
a swapped normalisation order fails at least one of them.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch

import oracle as O
import synth


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _frac_matrix(d):
    return np.array([[float(Fraction(n, q)) for n, q in zip(rn, rq)]
                     for rn, rq in zip(d["num"], d["den"])])


def _cfg_like_res_logits(rng, T, n, spread=0.03):
    """Logits shaped like the workloads': identity bias plus small noise."""
    return np.eye(n)[None] + spread * rng.standard_normal((T, n, n))


# ---------------------------------------------------------------- sigmoid

def test_sigmoid_closed_forms_and_library():
    z = np.linspace(-30, 30, 1001)
    assert O.sigmoid(0.0) == 0.5
    np.testing.assert_allclose(O.sigmoid(z), scipy.special.expit(z), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(O.sigmoid(-z), 1.0 - O.sigmoid(z), atol=1e-15)
    s = O.sigmoid(z)
    assert np.all(s > 0) and np.all(s < 1)


# ---------------------------------------------------------------- Sinkhorn

def test_sinkhorn_hand_derived_2x2(golden_dir):
    g = _load(golden_dir, "sinkhorn_2x2.json")
    L = np.log(np.array(g["M0"], dtype=np.float64))
    np.testing.assert_allclose(O.sinkhorn_knopp(L, 1), _frac_matrix(g["after_1_iteration"]),
                               rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.sinkhorn_knopp(L, 2), _frac_matrix(g["after_2_iterations"]),
                               rtol=0, atol=1e-15)


def test_sinkhorn_2x2_limit_closed_form():
    # Diagonal scaling keeps the cross ratio ad/bc, so the doubly stochastic limit
    # of a positive 2x2 matrix is [[p, 1-p], [1-p, p]] with p = sqrt(ad)/(sqrt(ad)+sqrt(bc)).
    rng = np.random.default_rng(1)
    for _ in range(20):
        a, b, c, d = rng.uniform(0.2, 5.0, 4)
        p = math.sqrt(a * d) / (math.sqrt(a * d) + math.sqrt(b * c))
        H = O.sinkhorn_knopp(np.log([[a, b], [c, d]]), 400)
        np.testing.assert_allclose(H, [[p, 1 - p], [1 - p, p]], atol=1e-12)


def test_sinkhorn_uniqueness_of_scaling():
    # A doubly stochastic A: convex combination of permutation matrices (Birkhoff).
    rng = np.random.default_rng(2)
    n = 5
    perms = [np.eye(n)[list(p)] for p in itertools.permutations(range(n))]
    w = rng.dirichlet(np.ones(8))
    A = sum(wi * perms[j] for wi, j in zip(w, rng.choice(len(perms), 8, replace=False)))
    A = 0.9 * A + 0.1 / n  # strictly positive, still doubly stochastic
    u, v = rng.standard_normal(n), rng.standard_normal(n)
    L = np.log(A) + u[:, None] + v[None, :]
    np.testing.assert_allclose(O.sinkhorn_knopp(L, 500), A, atol=1e-12)
    # A constant offset is a global factor e^0.7: the first T_c removes it, so one
    # iteration returns A itself.
    L2 = np.log(A) + 0.7
    np.testing.assert_allclose(O.sinkhorn_knopp(L2, 1), A, atol=1e-14)


def test_sinkhorn_n1_is_identity():
    for z in (-3.0, 0.0, 2.5):
        assert O.sinkhorn_knopp(np.array([[z]]), 20)[0, 0] == 1.0


def test_sinkhorn_permutation_equivariance():
    rng = np.random.default_rng(3)
    n = 4
    L = rng.standard_normal((n, n))
    P = np.eye(n)[[2, 0, 3, 1]]
    Q = np.eye(n)[[1, 3, 0, 2]]
    np.testing.assert_allclose(O.sinkhorn_knopp(P @ L @ Q, 20), P @ O.sinkhorn_knopp(L, 20) @ Q,
                               atol=1e-14)


def test_sinkhorn_rows_exact_columns_converged_at_workload_logits():
    rng = np.random.default_rng(4)
    H = O.sinkhorn_knopp(_cfg_like_res_logits(rng, 512, 4), 20)
    assert np.all(H >= 0)
    assert np.max(np.abs(H.sum(-1) - 1)) < 1e-13
    assert np.max(np.abs(H.sum(-2) - 1)) < 1e-6


def test_sinkhorn_order_rows_last():
    # Wide logits are far from converged after 20 iterations. Because T_r runs
    # last, rows sum to 1 to rounding while columns visibly do not.
    rng = np.random.default_rng(5)
    H = O.sinkhorn_knopp(4.0 * rng.standard_normal((64, 4, 4)), 20)
    assert np.max(np.abs(H.sum(-1) - 1)) < 1e-13
    assert np.max(np.abs(H.sum(-2) - 1)) > 1e-4


def test_sinkhorn_norm_and_closure():
    # Eq. 6 properties: ||H||_2 <= 1 (doubly stochastic), products stay doubly stochastic.
    rng = np.random.default_rng(6)
    Hs = O.sinkhorn_knopp(_cfg_like_res_logits(rng, 8, 4, spread=0.5), 60)
    for H in Hs:
        assert np.linalg.norm(H, 2) <= 1 + 1e-12
    prod = np.eye(4)
    for H in Hs:
        prod = H @ prod
    np.testing.assert_allclose(prod.sum(0), 1, atol=1e-12)
    np.testing.assert_allclose(prod.sum(1), 1, atol=1e-12)
    assert np.all(prod >= 0)
    assert np.linalg.norm(prod, 2) <= 1 + 1e-12


def test_sinkhorn_near_permutation_pins_mat_order():
    # A large logit on (i, (i+1) % n) drives H_res to that permutation; mat() is
    # row-major so z_res[i*n + j] lands on H_res[i, j].
    n = 4
    T = 1
    bias = np.zeros(n * n + 2 * n)
    for i in range(n):
        bias[2 * n + i * n + (i + 1) % n] = 25.0
    X = np.random.default_rng(7).standard_normal((T, n, 8))
    phi = np.zeros((n * 8, n * n + 2 * n))
    _, _, h_res = O.hc_coeffs(X, phi, bias, [0.01] * 3, 20)
    target = np.zeros((n, n))
    for i in range(n):
        target[i, (i + 1) % n] = 1.0
    np.testing.assert_allclose(h_res[0], target, atol=1e-9)


# -------------------------------------------------- projection, norm and gates

def test_phi_zero_closed_form(golden_dir):
    g = _load(golden_dir, "sinkhorn_phi0_n4.json")
    n, C, T = 4, 16, 5
    X = np.random.default_rng(8).standard_normal((T, n, C))
    h_pre, h_post, h_res = O.hc_coeffs(X, np.zeros((n * C, n * n + 2 * n)), synth.mhc_bias(n),
                                       [0.01] * 3, 20)
    np.testing.assert_allclose(h_pre, g["h_pre"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(h_post, g["h_post"], rtol=0, atol=1e-15)
    expect = np.full((n, n), g["h_res_offdiag"]) + np.eye(n) * (g["h_res_diag"] - g["h_res_offdiag"])
    np.testing.assert_allclose(h_res, np.broadcast_to(expect, h_res.shape), atol=1e-15)


def test_single_entry_state_closed_form():
    # One nonzero entry a at (stream i, channel c): r = |a|/sqrt(nC), so the
    # normalised flat vector is sign(a)*sqrt(nC) at index i*C + c and 0 elsewhere.
    # One-hot phi columns then make every logit a closed form; distinct gates per
    # block pin which alpha multiplies which block, and the row of phi that is
    # hit pins the stream-major flattening.
    n, C = 3, 5
    ncol = n * n + 2 * n
    i0, c0, a = 2, 3, -0.37
    X = np.zeros((1, n, C))
    X[0, i0, c0] = a
    flat = i0 * C + c0
    phi = np.zeros((n * C, ncol))
    phi[flat, :] = np.arange(1, ncol + 1) / ncol       # every column reads the entry
    phi[(flat + 1) % (n * C), :] = 100.0                # a wrong flattening would read this row
    alpha = np.array([0.011, 0.023, 0.037])
    bias = np.linspace(-0.5, 0.5, ncol)
    val = -math.sqrt(n * C)
    P = val * np.arange(1, ncol + 1) / ncol
    z = np.concatenate([alpha[0] * P[:n], alpha[1] * P[n:2 * n], alpha[2] * P[2 * n:]]) + bias
    h_pre, h_post, h_res = O.hc_coeffs(X, phi, bias, alpha, 20)
    np.testing.assert_allclose(h_pre[0], 1 / (1 + np.exp(-z[:n])), rtol=1e-14)
    np.testing.assert_allclose(h_post[0], 2 / (1 + np.exp(-z[n:2 * n])), rtol=1e-14)
    np.testing.assert_allclose(h_res[0], O.sinkhorn_knopp(z[2 * n:].reshape(n, n), 20), rtol=1e-14)


def test_projection_brute_force_tiny():
    rng = np.random.default_rng(9)
    n, C, T = 2, 3, 4
    X = rng.standard_normal((T, n, C))
    phi = rng.standard_normal((n * C, n * n + 2 * n))
    bias = rng.standard_normal(n * n + 2 * n)
    alpha = [0.3, 0.5, 0.7]
    z = O.mhc_logits(X, phi, bias, alpha)
    for t in range(T):
        ss = 0.0
        for i in range(n):
            for c in range(C):
                ss += X[t, i, c] ** 2
        r = math.sqrt(ss / (n * C))
        for j in range(n * n + 2 * n):
            acc = 0.0
            for i in range(n):
                for c in range(C):
                    acc += X[t, i, c] / r * phi[i * C + c, j]
            a = alpha[0] if j < n else alpha[1] if j < 2 * n else alpha[2]
            assert abs(z[t, j] - (a * acc + bias[j])) < 1e-12


def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((7, 96)) * 3.0
    u, r = O.rms_normalise(x)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), eps=0.0).numpy()
    np.testing.assert_allclose(u, ref, rtol=1e-13)


def test_coeffs_scale_invariant_and_zero_state():
    rng = np.random.default_rng(11)
    n, C = 4, 32
    X = rng.standard_normal((6, n, C))
    phi = 0.02 * rng.standard_normal((n * C, n * n + 2 * n))
    bias = synth.mhc_bias(n)
    a = [0.01] * 3
    for got, ref in zip(O.hc_coeffs(3.7 * X, phi, bias, a), O.hc_coeffs(X, phi, bias, a)):
        np.testing.assert_allclose(got, ref, rtol=1e-13)
    h_pre, h_post, h_res = O.hc_coeffs(np.zeros((1, n, C)), phi, bias, a)
    np.testing.assert_allclose(h_pre, 0.5)
    np.testing.assert_allclose(h_post, 1.0)
    np.testing.assert_allclose(h_res[0], O.sinkhorn_knopp(np.eye(n), 20))


# ---------------------------------------------------------------- pre / post

def test_pre_post_closed_forms_phi_zero():
    rng = np.random.default_rng(12)
    n, C, T = 4, 24, 3
    X = rng.standard_normal((T, n, C))
    F = rng.standard_normal((T, C))
    out = O.mhc_sublayer(X, np.zeros((n * C, n * n + 2 * n)), synth.mhc_bias(n), [0.01] * 3, F)
    np.testing.assert_allclose(out["F_in"], 0.5 * X.sum(1), rtol=1e-14)
    H0 = O.sinkhorn_knopp(np.eye(n), 20)
    np.testing.assert_allclose(out["X_next"], np.einsum("ij,tjc->tic", H0, X) + F[:, None, :],
                               rtol=1e-13, atol=1e-14)


def test_pre_picks_weighted_streams():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((2, 3, 5))
    h = np.array([[0.0, 1.0, 0.0], [0.0, 0.0, 2.0]])
    np.testing.assert_array_equal(O.hc_pre(X, h), np.stack([X[0, 1], 2 * X[1, 2]]))


def test_post_n1_is_plain_residual():
    # n = 1 with H_res = [1], H_pre = H_post = 1: x_{l+1} = x_l + F (Eq. 1).
    rng = np.random.default_rng(14)
    x = rng.standard_normal((4, 1, 9))
    F = rng.standard_normal((4, 9))
    np.testing.assert_array_equal(O.hc_post(x, np.ones((4, 1, 1)), np.ones((4, 1)), F),
                                  x + F[:, None, :])
    np.testing.assert_array_equal(O.hc_pre(x, np.ones((4, 1))), x[:, 0])


def test_post_cyclic_permutation_pins_row_column_roles():
    rng = np.random.default_rng(15)
    n = 4
    X = rng.standard_normal((2, n, 6))
    H = np.zeros((2, n, n))
    for i in range(n):
        H[:, i, (i + 1) % n] = 1.0
    Y = O.hc_post(X, H, np.zeros((2, n)), np.zeros((2, 6)))
    np.testing.assert_array_equal(Y, X[:, [(i + 1) % n for i in range(n)]])
    hp = np.array([[1.0, 2.0, 3.0, 4.0], [0.5, 0, 0, 0]])
    F = rng.standard_normal((2, 6))
    Y2 = O.hc_post(np.zeros_like(X), H, hp, F)
    np.testing.assert_allclose(Y2, hp[:, :, None] * F[:, None, :], rtol=0, atol=0)


def test_post_conserves_stream_sum():
    # Column sums of a doubly stochastic H_res are 1, so sum_i X_next[i] =
    # sum_i X[i] + (sum_i h_post_i) F_out (feature mean kept; mHC notes section 1).
    rng = np.random.default_rng(16)
    n, C, T = 4, 64, 32
    X = rng.standard_normal((T, n, C))
    phi = 0.02 * rng.standard_normal((n * C, n * n + 2 * n))
    F = rng.standard_normal((T, C))
    out = O.mhc_sublayer(X, phi, synth.mhc_bias(n), [0.01] * 3, F)
    lhs = out["X_next"].sum(1)
    rhs = X.sum(1) + out["h_post"].sum(1)[:, None] * F
    assert np.max(np.abs(lhs - rhs)) < 1e-6 * np.max(np.abs(rhs))


def test_post_linear_in_state_and_output():
    rng = np.random.default_rng(17)
    n, C, T = 3, 7, 2
    H = rng.uniform(size=(T, n, n))
    hp = rng.uniform(size=(T, n))
    X1, X2 = rng.standard_normal((2, T, n, C))
    F1, F2 = rng.standard_normal((2, T, C))
    lhs = O.hc_post(2 * X1 - X2, H, hp, 2 * F1 - F2)
    rhs = 2 * O.hc_post(X1, H, hp, F1) - O.hc_post(X2, H, hp, F2)
    np.testing.assert_allclose(lhs, rhs, atol=1e-13)


# ---------------------------------------------------------------- routing

def test_select_brute_force_tiny():
    # Brute force over every (k-m)-subset of the candidates: the routed set is the
    # unique subset S in which every member beats every non-member, where j beats
    # j' if s_j > s_j', or s_j == s_j' and j < j' (ties to the lower index).
    rng = np.random.default_rng(18)
    N, k, m = 7, 4, 1
    s = np.round(rng.uniform(size=(200, N - m)), 2)  # coarse values: many exact ties
    idx = O.xhc_select(s, k, m)

    def beats(t, j, jj):
        return s[t, j] > s[t, jj] or (s[t, j] == s[t, jj] and j < jj)

    for t in range(s.shape[0]):
        ok = [comb for comb in itertools.combinations(range(N - m), k - m)
              if all(beats(t, j, jj) for j in comb for jj in range(N - m) if jj not in comb)]
        assert len(ok) == 1
        expect = sorted(list(range(m)) + [m + j for j in ok[0]])
        assert list(idx[t]) == expect, (t, s[t], idx[t], expect)


def test_select_fixed_only_and_candidate_offset():
    s = np.random.default_rng(19).uniform(size=(10, 6))
    np.testing.assert_array_equal(O.xhc_select(s, 3, 3), np.tile([0, 1, 2], (10, 1)))
    s2 = np.zeros((1, 6))
    s2[0, 4] = 1.0  # candidate column 4 is stream m + 4
    assert list(O.xhc_select(s2, 3, 2)[0]) == [0, 1, 6]


def test_router_duplicate_columns_tie_to_lower_index():
    rng = np.random.default_rng(20)
    N, C, m, k = 6, 4, 2, 3
    X = rng.standard_normal((50, N, C))
    W = rng.standard_normal((N * C, N - m))
    W[:, 3] = W[:, 1]  # streams m+1 and m+3 always tie exactly
    s = O.xhc_router_scores(X, W)
    assert np.array_equal(s[:, 1], s[:, 3])
    idx = O.xhc_select(s, k, m)  # one routed slot
    hits = 0
    for t in range(50):
        if s[t, 1] == s[t].max():
            hits += 1
            assert m + 1 in idx[t] and m + 3 not in idx[t]
    assert hits > 0


def test_router_scores_single_nonzero_entry_closed_form():
    # One nonzero entry a at (stream i, channel c): r = |a| / sqrt(N C), so the
    # normalised state is sign(a) sqrt(N C) at row i*C + c and zero elsewhere, and
    # each candidate's score is 1 / (1 + exp(-sign(a) sqrt(N C) W_r[i*C + c, j]))
    # (xHC summary, sparse residual streams, step 1; reading: sigma of a linear
    # router on the RMS-normalised flattened state). Scalar math.exp, no matmul.
    rng = np.random.default_rng(23)
    N, C, m = 5, 3, 2
    W = 0.4 * rng.standard_normal((N * C, N - m))
    cases = [(0, 0, 2.5), (3, 1, -0.75), (4, 2, 1e-3), (2, 0, -40.0)]
    X = np.zeros((len(cases), N, C))
    for t, (i, c, a) in enumerate(cases):
        X[t, i, c] = a
    s = O.xhc_router_scores(X, W)
    assert s.shape == (len(cases), N - m)
    for t, (i, c, a) in enumerate(cases):
        for j in range(N - m):
            logit = math.copysign(math.sqrt(N * C), a) * W[i * C + c, j]
            assert abs(s[t, j] - 1.0 / (1.0 + math.exp(-logit))) < 1e-15, (t, j)
    # The score does not depend on |a| (the RMS factor cancels it), only on its sign.
    np.testing.assert_array_equal(O.xhc_router_scores(7.0 * X, W), s)


def test_router_scores_brute_force_loops():
    # Every score from scalar loops: the token's sum of squares, r, each logit as
    # an exactly rounded sum over the N*C flattened entries in stream-major order,
    # then the logistic function.
    rng = np.random.default_rng(24)
    T, N, C, m = 4, 4, 3, 1
    X = rng.standard_normal((T, N, C))
    W = rng.standard_normal((N * C, N - m))
    s = O.xhc_router_scores(X, W)
    for t in range(T):
        vals = [X[t, i, c] for i in range(N) for c in range(C)]
        r = math.sqrt(math.fsum(v * v for v in vals) / (N * C))
        for j in range(N - m):
            logit = math.fsum(vals[q] / r * W[q, j] for q in range(N * C))
            assert abs(s[t, j] - 1.0 / (1.0 + math.exp(-logit))) < 1e-13, (t, j)


def test_router_selection_independent_of_normalisation():
    # No bias and r > 0: ordering of u @ W equals ordering of x @ W.
    rng = np.random.default_rng(21)
    N, C, m, k = 8, 6, 2, 4
    X = rng.standard_normal((40, N, C))
    W = rng.standard_normal((N * C, N - m))
    raw = O.sigmoid(X.reshape(40, -1) @ W)
    np.testing.assert_array_equal(O.xhc_select(raw, k, m),
                                  O.xhc_select(O.xhc_router_scores(X, W), k, m))


def test_route_k_equals_N_is_dense_mhc():
    # With every stream active (k = N, any m), the sparse update is mHC's.
    rng = np.random.default_rng(22)
    N, C, T = 4, 16, 6
    X = rng.standard_normal((T, N, C))
    phi_pre = 0.3 * rng.standard_normal((N * C, N))
    phi_act = 0.3 * rng.standard_normal((N * C, N + N * N))
    b_pre = 0.1 * rng.standard_normal(N)
    b_act = 0.1 * rng.standard_normal(N + N * N)
    F = rng.standard_normal((T, C))
    W = rng.standard_normal((N * C, N - 1))
    a_pre, a_post, a_res = 0.2, 0.3, 0.4
    pre = O.xhc_pre(X, phi_pre, b_pre, a_pre, W, k=N, m=1)
    np.testing.assert_array_equal(pre["idx"], np.tile(np.arange(N), (T, 1)))
    Xn, _, _ = O.xhc_route(X, pre["idx"], phi_act, b_act, a_post, a_res, F)
    ref = O.mhc_sublayer(X, np.concatenate([phi_pre, phi_act], 1),
                         np.concatenate([b_pre, b_act]), [a_pre, a_post, a_res], F)
    np.testing.assert_allclose(pre["F_in"], ref["F_in"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Xn, ref["X_next"], rtol=1e-13, atol=1e-13)


def test_route_passes_inactive_streams_and_identity_maps():
    rng = np.random.default_rng(23)
    N, C, T, k = 8, 5, 9, 3
    X = rng.standard_normal((T, N, C))
    idx = np.array([sorted(rng.choice(N, k, replace=False)) for _ in range(T)])
    phi_act = rng.standard_normal((k * C, k + k * k))
    b_act = rng.standard_normal(k + k * k)
    Xn, _, _ = O.xhc_route(X, idx, phi_act, b_act, 0.01, 0.01, rng.standard_normal((T, C)))
    for t in range(T):
        for i in range(N):
            if i not in idx[t]:
                assert np.array_equal(Xn[t, i], X[t, i])
    # alpha = 0, res bias 40*I and post bias -40: H_res ~ I, H_post ~ 0 -> X unchanged.
    b_id = np.concatenate([np.full(k, -40.0), (40.0 * np.eye(k)).reshape(-1)])
    Xi, Hp, Hr = O.xhc_route(X, idx, phi_act, b_id, 0.0, 0.0, rng.standard_normal((T, C)))
    np.testing.assert_allclose(Xi, X, atol=1e-15)


def test_route_gather_order_and_slot_semantics():
    # Slot a of the active set is stream idx[a]; a cyclic H_res_A moves slot a+1 into slot a.
    rng = np.random.default_rng(24)
    N, C, k = 6, 4, 3
    X = rng.standard_normal((1, N, C))
    idx = np.array([[1, 3, 4]])
    b = np.concatenate([np.full(k, -60.0),
                        (60.0 * np.eye(k)[[1, 2, 0]]).reshape(-1)])  # H[a, a+1] large
    Xn, _, _ = O.xhc_route(X, idx, np.zeros((k * C, k + k * k)), b, 0.0, 0.0, np.zeros((1, C)))
    np.testing.assert_allclose(Xn[0, 1], X[0, 3], atol=1e-12)
    np.testing.assert_allclose(Xn[0, 3], X[0, 4], atol=1e-12)
    np.testing.assert_allclose(Xn[0, 4], X[0, 1], atol=1e-12)


# ---------------------------------------------------------------- augmentation

def test_conv_one_hot_taps():
    rng = np.random.default_rng(25)
    B, S, C, kap = 2, 10, 3, 4
    F = rng.standard_normal((B * S, C))
    w_last = np.zeros((C, kap))
    w_last[:, kap - 1] = 1.0
    np.testing.assert_array_equal(O.causal_dwconv(F, w_last, B, S), F)
    w_first = np.zeros((C, kap))
    w_first[:, 0] = 1.0
    g = O.causal_dwconv(F, w_first, B, S).reshape(B, S, C)
    Fb = F.reshape(B, S, C)
    np.testing.assert_array_equal(g[:, kap - 1:], Fb[:, :S - kap + 1])
    assert np.all(g[:, :kap - 1] == 0)


def test_conv_matches_fir_filter_per_sequence():
    rng = np.random.default_rng(26)
    B, S, C = 3, 40, 5
    F = rng.standard_normal((B * S, C))
    for kap in (4, 8, 12):
        w = rng.standard_normal((C, kap))
        g = O.causal_dwconv(F, w, B, S).reshape(B, S, C)
        for b in range(B):
            for c in range(C):
                ref = scipy.signal.lfilter(w[c, ::-1], [1.0], F.reshape(B, S, C)[b, :, c])
                np.testing.assert_allclose(g[b, :, c], ref, rtol=1e-12, atol=1e-12)


def test_mgs_orthogonal_first_exact_and_qr():
    rng = np.random.default_rng(27)
    T, Kr, C = 6, 4, 50
    G = rng.standard_normal((T, Kr, C))
    G[:, 1:] += 0.8 * G[:, :1]  # correlated, as the conv outputs are
    V = O.modified_gram_schmidt(G)
    np.testing.assert_array_equal(V[:, 0], G[:, 0])
    for t in range(T):
        for i in range(Kr):
            for j in range(i):
                cos = V[t, i] @ V[t, j] / (np.linalg.norm(V[t, i]) * np.linalg.norm(V[t, j]))
                assert abs(cos) < 1e-12
        Q, R = np.linalg.qr(G[t].T)
        for j in range(Kr):
            np.testing.assert_allclose(V[t, j], Q[:, j] * R[j, j], rtol=1e-10, atol=1e-12)


def test_mgs_keeps_orthogonal_components():
    rng = np.random.default_rng(28)
    Q, _ = np.linalg.qr(rng.standard_normal((30, 4)))
    G = (Q * np.array([2.0, 0.5, 3.0, 1.5])).T[None]
    np.testing.assert_allclose(O.modified_gram_schmidt(G), G, atol=1e-14)


def test_augment_components_order():
    # V[:, 0] is the raw output; V[:, 1] is the kappa_1 conv minus its projection.
    rng = np.random.default_rng(29)
    B, S, C = 1, 16, 6
    F = rng.standard_normal((B * S, C))
    ws = [rng.standard_normal((C, k)) for k in (4, 8, 12)]
    V = O.xhc_augment(F, ws, B, S)
    g1 = O.causal_dwconv(F, ws[0], B, S)
    coef = np.sum(g1 * F, 1) / np.sum(F * F, 1)
    np.testing.assert_allclose(V[:, 1], g1 - coef[:, None] * F, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(V[:, 0], F)


# ------------------------------------------------------------ synth recipe

def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    r, bits = synth.round_to_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(r, ref)
    assert bits.dtype == np.uint16


# ----------------------------------- HC baseline (Eq. 5) and the Amax gain (section 3.1)

def test_hc_tanh_zero_projection_gives_the_static_maps():
    """theta = 0: every tanh is 0, so the maps are the biases (the static part)."""
    rng = np.random.default_rng(200)
    T, n, C = 3, 4, 16
    X = rng.standard_normal((T, n, C))
    b = rng.standard_normal(n * n + 2 * n)
    hp, hq, hr = O.hc_tanh_coeffs(X, np.zeros((n + 2, C)), b, (0.7, -1.3, 2.0))
    np.testing.assert_array_equal(hp, np.tile(b[:n], (T, 1)))
    np.testing.assert_array_equal(hq, np.tile(b[n:2 * n], (T, 1)))
    np.testing.assert_array_equal(hr, np.tile(b[2 * n:].reshape(n, n), (T, 1, 1)))


def test_hc_tanh_single_nonzero_entry_closed_form():
    """A stream row with one nonzero entry v at channel c normalises to
    sign(v) sqrt(C) e_c, so theta_k . x~ = sign(v) sqrt(C) theta[k, c]; the row
    index of H_res is the theta row, the column the stream."""
    n, C = 3, 9
    rng = np.random.default_rng(201)
    theta = rng.standard_normal((n + 2, C)) * 0.3
    b = rng.standard_normal(n * n + 2 * n)
    a = (0.5, 1.5, -0.25)
    X = np.zeros((1, n, C))
    cols, vals = [2, 7, 0], [-3.0, 0.5, 11.0]
    for i in range(n):
        X[0, i, cols[i]] = vals[i]
    hp, hq, hr = O.hc_tanh_coeffs(X, theta, b, a)
    for i in range(n):
        s = math.copysign(math.sqrt(C), vals[i])
        assert math.isclose(hp[0, i], a[0] * math.tanh(s * theta[0, cols[i]]) + b[i], rel_tol=1e-14)
        assert math.isclose(hq[0, i], a[1] * math.tanh(s * theta[1, cols[i]]) + b[n + i], rel_tol=1e-14)
        for j in range(n):
            want = a[2] * math.tanh(s * theta[2 + j, cols[i]]) + b[2 * n + j * n + i]
            assert math.isclose(hr[0, j, i], want, rel_tol=1e-14, abs_tol=1e-15)


def test_hc_tanh_brute_force_and_per_stream_scale_invariance():
    rng = np.random.default_rng(202)
    T, n, C = 2, 3, 5
    X = rng.standard_normal((T, n, C))
    X[1, 2] = 0.0  # an all-zero row: x~ = 0
    theta = rng.standard_normal((n + 2, C))
    b = rng.standard_normal(n * n + 2 * n)
    a = (0.9, 0.4, 1.1)
    hp, hq, hr = O.hc_tanh_coeffs(X, theta, b, a)
    for t in range(T):
        for i in range(n):
            row = [float(v) for v in X[t, i]]
            r = math.sqrt(sum(v * v for v in row) / C)
            xt = [v / r if r > 0 else 0.0 for v in row]
            dot = lambda k: sum(theta[k, c] * xt[c] for c in range(C))
            assert math.isclose(hp[t, i], a[0] * math.tanh(dot(0)) + b[i], rel_tol=1e-12, abs_tol=1e-14)
            assert math.isclose(hq[t, i], a[1] * math.tanh(dot(1)) + b[n + i], rel_tol=1e-12, abs_tol=1e-14)
            for j in range(n):
                assert math.isclose(hr[t, j, i], a[2] * math.tanh(dot(2 + j)) + b[2 * n + j * n + i],
                                    rel_tol=1e-12, abs_tol=1e-14)
    # each stream is normalised on its own: scaling one stream by 2^k changes nothing
    Xs = X.copy()
    Xs[:, 0] *= 8.0
    Xs[:, 1] *= 0.25
    for u, v in zip(O.hc_tanh_coeffs(Xs, theta, b, a), (hp, hq, hr)):
        np.testing.assert_array_equal(u, v)


def test_amax_gain_closed_forms():
    T, n = 4, 3
    eye = np.broadcast_to(np.eye(n), (5, T, n, n))
    f, g = O.amax_gain(eye)
    np.testing.assert_array_equal(f, np.ones(T))
    np.testing.assert_array_equal(g, np.ones(T))
    # permutations keep every row and column sum at 1
    perms = np.stack([np.stack([np.eye(n)[list(p)] for p in itertools.islice(itertools.permutations(range(n)),
                                                                             T)]) for _ in range(3)])
    f, g = O.amax_gain(perms)
    np.testing.assert_array_equal(f, np.ones(T))
    # diagonal maps multiply: gain = max_i |prod_l d_l[i]|
    rng = np.random.default_rng(203)
    d = rng.uniform(-2, 2, (4, T, n))
    f, g = O.amax_gain(np.einsum("ltn,nm->ltnm", d, np.eye(n)))
    want = np.abs(np.prod(d, axis=0)).max(axis=1)
    np.testing.assert_allclose(f, want, rtol=1e-14)
    np.testing.assert_allclose(g, want, rtol=1e-14)
    # Sinkhorn outputs end with a row normalisation: a chain of them has row sums
    # exactly 1 (to rounding), so the forward gain is 1
    Hs = np.stack([O.sinkhorn_knopp(rng.standard_normal((T, n, n)), 20) for _ in range(6)])
    f, _ = O.amax_gain(Hs)
    np.testing.assert_allclose(f, 1.0, rtol=0, atol=1e-13)


def test_amax_gain_brute_force_order():
    """M = H_{L-1} ... H_0 (a transposed or reversed product fails this)."""
    rng = np.random.default_rng(204)
    L, T, n = 3, 2, 3
    H = rng.standard_normal((L, T, n, n))
    f, g = O.amax_gain(H)
    for t in range(T):
        M = [[1.0 if i == j else 0.0 for j in range(n)] for i in range(n)]
        for layer in range(L):
            A = H[layer, t]
            M = [[sum(A[i][k] * M[k][j] for k in range(n)) for j in range(n)] for i in range(n)]
        rows = [abs(sum(M[i][j] for j in range(n))) for i in range(n)]
        cols = [abs(sum(M[i][j] for i in range(n))) for j in range(n)]
        assert math.isclose(f[t], max(rows), rel_tol=1e-12)
        assert math.isclose(g[t], max(cols), rel_tol=1e-12)


# ------------------------------------------------ static mHC (the mHC-SSM abstract)

def test_static_maps_simplex_and_sinkhorn():
    rng = np.random.default_rng(210)
    n = 4
    z = rng.standard_normal(n * n + 2 * n) * 2.0
    hp, hq, hr = O.static_mhc_maps(z, n, 20)
    np.testing.assert_allclose(hp, scipy.special.softmax(z[:n]), rtol=1e-14)
    np.testing.assert_allclose(hq, scipy.special.softmax(z[n:2 * n]), rtol=1e-14)
    np.testing.assert_allclose(hr, O.sinkhorn_knopp(z[2 * n:].reshape(n, n), 20), rtol=0, atol=0)
    assert math.isclose(hp.sum(), 1.0, rel_tol=1e-15) and (hp > 0).all()
    np.testing.assert_allclose(hr.sum(axis=1), 1.0, rtol=1e-14)  # rows normalised last
    # equal logits: the uniform point of the simplex; a shift changes nothing
    hp0, _, _ = O.static_mhc_maps(np.zeros(n * n + 2 * n), n)
    np.testing.assert_array_equal(hp0, np.full(n, 0.25))
    hp1, hq1, _ = O.static_mhc_maps(z + 3.0, n, 20)
    np.testing.assert_allclose(hp1, hp, rtol=1e-14)


def test_static_apply_is_the_broadcast_mhc_apply():
    """The static maps applied to every token equal the per-token formulas written
    out with explicit loops."""
    rng = np.random.default_rng(211)
    T, n, C = 3, 3, 5
    X = rng.standard_normal((T, n, C))
    F = rng.standard_normal((T, C))
    hp, hq, hr = O.static_mhc_maps(rng.standard_normal(n * n + 2 * n), n, 20)
    Fin = O.static_pre(X, hp)
    Xn = O.static_post(X, hr, hq, F)
    for t in range(T):
        for c in range(C):
            assert math.isclose(Fin[t, c], sum(hp[i] * X[t, i, c] for i in range(n)), rel_tol=1e-13, abs_tol=1e-14)
            for i in range(n):
                want = sum(hr[i, j] * X[t, j, c] for j in range(n)) + hq[i] * F[t, c]
                assert math.isclose(Xn[t, i, c], want, rel_tol=1e-13, abs_tol=1e-14)


# ---------------------------------------------------------------- backward

def _central_difference(f, arr, h=1e-6):
    """Brute-force gradient of the scalar f at arr by central differences."""
    out = np.zeros_like(arr)
    for idx in np.ndindex(arr.shape):
        a = arr.copy()
        a[idx] += h
        up = f(a)
        a[idx] -= 2 * h
        out[idx] = (up - f(a)) / (2 * h)
    return out


@pytest.mark.parametrize("n,iters", [(4, 20), (3, 5), (2, 1)])
def test_sinkhorn_backward_finite_differences(n, iters):
    """The Sinkhorn backward is the gradient of sum(G * SK(z)): central
    differences of the forward oracle, entry by entry."""
    rng = np.random.default_rng(300 + n)
    z = rng.standard_normal((2, n, n))
    G = rng.standard_normal((2, n, n))
    got = O.sinkhorn_knopp_backward(z, G, iters)
    want = _central_difference(lambda a: np.sum(G * O.sinkhorn_knopp(a, iters)), z)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-8 * np.abs(want).max())


def test_sinkhorn_backward_invariances_and_zero_iterations():
    """The first step normalises columns, so SK(exp(z + v_j)) = SK(exp(z)) for any
    column shift v: the gradient sums to zero down every column, exactly. Row shifts
    only cancel in the limit: row sums shrink as the iterations grow. With no
    iteration SK is exp, whose gradient is G * exp(z)."""
    rng = np.random.default_rng(310)
    z = rng.standard_normal((3, 4, 4))
    G = rng.standard_normal((3, 4, 4))
    for iters in (1, 5, 20):
        g = O.sinkhorn_knopp_backward(z, G, iters)
        np.testing.assert_allclose(g.sum(axis=-2), 0.0, atol=1e-14)
    row5 = np.abs(O.sinkhorn_knopp_backward(z, G, 5).sum(axis=-1)).max()
    row40 = np.abs(O.sinkhorn_knopp_backward(z, G, 40).sum(axis=-1)).max()
    assert row40 < 1e-3 * row5
    np.testing.assert_allclose(O.sinkhorn_knopp_backward(z, G, 0), G * np.exp(z), rtol=1e-15)


def _sublayer_loss(dXn, dFi, iters):
    def L(X, phi, b, al, Fo):
        o = O.mhc_sublayer(X, phi, b, al, Fo, iters)
        return np.sum(dXn * o["X_next"]) + np.sum(dFi * o["F_in"])
    return L


@pytest.mark.parametrize("T,n,C,iters", [(2, 4, 3, 20), (3, 2, 5, 7), (1, 1, 4, 3)])
def test_sublayer_backward_finite_differences(T, n, C, iters):
    """Every gradient of mhc_sublayer_backward (state, phi, bias, the three gates,
    F_out) against central differences of L = <dX_next, X_next> + <dF_in, F_in>
    through the forward oracle. Gates and phi are large enough that no sigmoid
    saturates and Sinkhorn is far from its fixed point."""
    rng = np.random.default_rng(320 + 10 * n + C)
    X = rng.standard_normal((T, n, C))
    phi = 0.3 * rng.standard_normal((n * C, n * n + 2 * n))
    b = 0.5 * rng.standard_normal(n * n + 2 * n)
    al = np.array([0.7, 0.9, 1.3])
    Fo = rng.standard_normal((T, C))
    dXn = rng.standard_normal((T, n, C))
    dFi = rng.standard_normal((T, C))
    L = _sublayer_loss(dXn, dFi, iters)
    g = O.mhc_sublayer_backward(X, phi, b, al, Fo, dXn, dFi, iters)
    cases = [("dX", X, lambda a: L(a, phi, b, al, Fo)), ("dphi", phi, lambda a: L(X, a, b, al, Fo)),
             ("dbias", b, lambda a: L(X, phi, a, al, Fo)), ("dalpha", al, lambda a: L(X, phi, b, a, Fo)),
             ("dF_out", Fo, lambda a: L(X, phi, b, al, a))]
    for name, arr, f in cases:
        want = _central_difference(f, arr)
        np.testing.assert_allclose(g[name], want, rtol=0, atol=1e-7 * np.abs(want).max(), err_msg=name)


def test_sublayer_backward_zero_state_and_bias_gradient():
    """The all-zero state: the forward's z is the bias alone (1/r taken as 0), so
    the gradient reaching x is the plain transpose of the apply, H_res^T dX_next +
    H_pre dF_in, with the maps of z = b; dphi is zero (vec x = 0) and the bias
    gradient is the logit gradient itself."""
    rng = np.random.default_rng(330)
    T, n, C = 2, 4, 6
    X = np.zeros((T, n, C))
    phi = rng.standard_normal((n * C, n * n + 2 * n))
    b = rng.standard_normal(n * n + 2 * n)
    dXn = rng.standard_normal((T, n, C))
    dFi = rng.standard_normal((T, C))
    g = O.mhc_sublayer_backward(X, phi, b, (0.5, 0.5, 0.5), rng.standard_normal((T, C)), dXn, dFi, 20)
    hp = 1.0 / (1.0 + np.exp(-b[:n]))
    hr = O.sinkhorn_knopp(b[2 * n:].reshape(n, n), 20)
    want = np.einsum("ij,tic->tjc", hr, dXn) + hp[None, :, None] * dFi[:, None, :]
    np.testing.assert_allclose(g["dX"], want, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(g["dphi"], 0.0)
    np.testing.assert_allclose(g["dbias"], g["dz"].sum(axis=0), rtol=1e-15)
    np.testing.assert_array_equal(g["dalpha"], 0.0)


@pytest.mark.parametrize("N,k,K,C", [(6, 3, 1, 3), (5, 2, 2, 4)])
def test_route_backward_finite_differences(N, k, K, C):
    """xhc_route_backward against central differences of L = <dX_next, X_next>
    through xhc_route with the active set held fixed (a discrete choice): state,
    phi_act, b_act, both gates and the write-back components."""
    rng = np.random.default_rng(340 + N + K)
    T = 2
    X = rng.standard_normal((T, N, C))
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(T)])
    phi = 0.3 * rng.standard_normal((k * C, k * K + k * k))
    b = 0.5 * rng.standard_normal(k * K + k * k)
    ap, ar = 0.8, 1.1
    Wb = rng.standard_normal((T, K, C))
    dXn = rng.standard_normal((T, N, C))
    g = O.xhc_route_backward(X, idx, phi, b, ap, ar, Wb, dXn, 20)

    def L(X, phi, b, ap, ar, Wb):
        return np.sum(dXn * O.xhc_route(X, idx, phi, b, ap, ar, Wb, 20)[0])
    cases = [("dX", X, lambda a: L(a, phi, b, ap, ar, Wb)), ("dphi_act", phi, lambda a: L(X, a, b, ap, ar, Wb)),
             ("db_act", b, lambda a: L(X, phi, a, ap, ar, Wb)), ("dWb", Wb, lambda a: L(X, phi, b, ap, ar, a))]
    for name, arr, f in cases:
        want = _central_difference(f, arr)
        np.testing.assert_allclose(g[name], want, rtol=0, atol=1e-7 * np.abs(want).max(), err_msg=name)
    for name, v, f in (("dalpha_post", ap, lambda a: L(X, phi, b, a[0], ar, Wb)),
                       ("dalpha_res", ar, lambda a: L(X, phi, b, ap, a[0], Wb))):
        want = _central_difference(f, np.array([v]))[0]
        assert math.isclose(g[name], want, rel_tol=1e-6), name
    # the rows the route does not touch pass the upstream gradient through unchanged
    inactive = np.ones((T, N), bool)
    inactive[np.arange(T)[:, None], idx] = False
    np.testing.assert_array_equal(g["dX"][inactive], dXn[inactive])


def test_pre_backward_finite_differences_and_router():
    """xhc_pre_backward against central differences of L = <dF_in, F_in> through
    xhc_pre (state, phi_pre, b_pre, the gate); the router's weights change F_in
    not at all while the active set stays the same, so they get no gradient."""
    rng = np.random.default_rng(350)
    T, N, C = 2, 6, 3
    X = rng.standard_normal((T, N, C))
    phi = 0.3 * rng.standard_normal((N * C, N))
    b = 0.5 * rng.standard_normal(N)
    a0 = 0.9
    dFi = rng.standard_normal((T, C))
    g = O.xhc_pre_backward(X, phi, b, a0, dFi)

    def L(X, phi, b, a0):
        return np.sum(dFi * O.xhc_pre(X, phi, b, a0)["F_in"])
    for name, arr, f in (("dX", X, lambda a: L(a, phi, b, a0)), ("dphi_pre", phi, lambda a: L(X, a, b, a0)),
                         ("db_pre", b, lambda a: L(X, phi, a, a0))):
        want = _central_difference(f, arr)
        np.testing.assert_allclose(g[name], want, rtol=0, atol=1e-7 * np.abs(want).max(), err_msg=name)
    assert math.isclose(g["dalpha_pre"], _central_difference(lambda a: L(X, phi, b, a[0]), np.array([a0]))[0],
                        rel_tol=1e-6)
    W = rng.standard_normal((N * C, N - 2))
    F0 = O.xhc_pre(X, phi, b, a0, W, 3, 2)["F_in"]
    F1 = O.xhc_pre(X, phi, b, a0, W + 1e-3 * rng.standard_normal(W.shape), 3, 2)["F_in"]
    np.testing.assert_array_equal(F0, F1)


def test_route_backward_with_every_stream_active_is_the_mhc_backward():
    """k = N with the identity active set: the route is the mHC post/res write, so
    its gradients equal mhc_sublayer_backward's with a zero pre map, dF_in = 0 and
    phi = [any pre columns | phi_act]."""
    rng = np.random.default_rng(360)
    T, n, C = 3, 4, 5
    X = rng.standard_normal((T, n, C))
    phi_act = 0.3 * rng.standard_normal((n * C, n + n * n))
    b_act = 0.5 * rng.standard_normal(n + n * n)
    F = rng.standard_normal((T, C))
    dXn = rng.standard_normal((T, n, C))
    idx = np.tile(np.arange(n), (T, 1))
    g = O.xhc_route_backward(X, idx, phi_act, b_act, 0.7, 1.2, F, dXn, 20)
    phi = np.concatenate([rng.standard_normal((n * C, n)), phi_act], axis=1)
    bias = np.concatenate([np.zeros(n), b_act])
    ref = O.mhc_sublayer_backward(X, phi, bias, (0.5, 0.7, 1.2), F, dXn, np.zeros((T, C)), 20)
    np.testing.assert_allclose(g["dX"], ref["dX"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dWb"][:, 0], ref["dF_out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dphi_act"], ref["dphi"][:, n:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["db_act"], ref["dbias"][n:], rtol=1e-12, atol=1e-12)
    assert math.isclose(g["dalpha_post"], ref["dalpha"][1], rel_tol=1e-12)
    assert math.isclose(g["dalpha_res"], ref["dalpha"][2], rel_tol=1e-12)


@pytest.mark.parametrize("B,S,C,kappas", [(2, 5, 6, (2, 3, 4)), (1, 7, 5, (4, 8, 12))])
def test_augment_backward_finite_differences(B, S, C, kappas):
    """xhc_augment_backward against central differences of L = <dV, V> through
    xhc_augment: F_out and every conv kernel (kernels longer than the sequence
    included). C >= K_r keeps the components independent."""
    rng = np.random.default_rng(370 + S)
    F = rng.standard_normal((B * S, C))
    ws = [0.5 * rng.standard_normal((C, k)) for k in kappas]
    dV = rng.standard_normal((B * S, 4, C))
    g = O.xhc_augment_backward(F, ws, B, S, dV)

    def L(F, ws):
        return np.sum(dV * O.xhc_augment(F, ws, B, S))
    want = _central_difference(lambda a: L(a, ws), F)
    np.testing.assert_allclose(g["dF_out"], want, rtol=0, atol=1e-7 * np.abs(want).max())
    for j in range(len(ws)):
        want = _central_difference(lambda a: L(F, [a if q == j else ws[q] for q in range(len(ws))]), ws[j])
        np.testing.assert_allclose(g["dconv_ws"][j], want, rtol=0, atol=1e-7 * np.abs(want).max(), err_msg=str(j))


def test_conv_backward_adjoint_identities():
    """The conv is linear in F_out and in w, so <dg, conv(F, w)> equals <dF, F>
    and <dw, w> exactly (up to rounding) for the backward's dF and dw."""
    rng = np.random.default_rng(380)
    B, S, C, k = 3, 9, 4, 5
    F = rng.standard_normal((B * S, C))
    w = rng.standard_normal((C, k))
    dg = rng.standard_normal((B * S, C))
    dF, dw = O.causal_dwconv_backward(F, w, B, S, dg)
    val = np.sum(dg * O.causal_dwconv(F, w, B, S))
    assert math.isclose(np.sum(dF * F), val, rel_tol=1e-12)
    assert math.isclose(np.sum(dw * w), val, rel_tol=1e-12)


# ------------------------------------------------------------------ xHC-Flash

def _flash_case(seed, T=6, N=8, C=5, k=4, m=2, L=2, K_last=1):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, N, C))
    phis = [rng.standard_normal((N * C, N)) * 0.3 for _ in range(L)]
    bs = [rng.standard_normal(N) * 0.2 for _ in range(L)]
    w_r = rng.standard_normal((N * C, N - m)) * 0.3
    Kb = L - 1 + K_last
    phi_act = rng.standard_normal((k * C, k * Kb + k * k)) * 0.3
    b_act = rng.standard_normal(k * Kb + k * k) * 0.2
    F_outs = rng.standard_normal((T, L, C))
    return X, phis, bs, w_r, phi_act, b_act, F_outs


@pytest.mark.parametrize("L,K_last", [(1, 1), (2, 1), (3, 1), (4, 1), (2, 4), (3, 4), (1, 4)])
def test_flash_matches_materialised_block(L, K_last):
    """The block run sublayer by sublayer with the state written out after each
    one (sublayers before the last add their post write to the active rows, the
    last mixes with H_res and adds its own, every sublayer's input is the dense
    read of the state as it then is) gives the inputs xhc_flash_input rebuilds
    from the entry-state reads and the state xhc_flash_post writes. With
    K_last = 4 the last sublayer (the MLP) writes back its augmentation: the
    Gram-Schmidt components of causal convs of its own output, each through its
    own post-map column, as xhc_route adds K components."""
    T, C = 8, 5
    X0, phis, bs, w_r, phi_act, b_act, F_outs = _flash_case(700 + 10 * L + K_last, T=T, C=C, L=L, K_last=K_last)
    k, m = 4, 2
    pre = O.xhc_flash_pre(X0, phis, bs, 0.7, w_r, k, m)
    idx = pre["idx"]
    H_post, H_res = O.xhc_flash_maps(X0, idx, phi_act, b_act, 0.6, 0.9, L, 20, K_last=K_last)
    assert H_post.shape == (T, k, L - 1 + K_last)
    if K_last == 1:
        last = F_outs[:, L - 1:L]
    else:  # 2 sequences of 4 tokens, kernels 2, 3, 4 (any sizes: the block end is linear in them)
        rng = np.random.default_rng(33)
        ws = [rng.standard_normal((C, kk)) / np.sqrt(kk) for kk in (2, 3, 4)[:K_last - 1]]
        last = O.xhc_augment(F_outs[:, L - 1], ws, 2, T // 2)
    W = np.concatenate([F_outs[:, :L - 1], last], axis=1)
    rows = np.arange(T)[:, None]
    Xs = X0.copy()
    for l in range(L):
        want = np.einsum("ti,tic->tc", pre["h_pre"][l], Xs)  # dense read of the current state
        got = O.xhc_flash_input(l, pre["F_pre"][l], pre["h_pre"][l], idx, H_post, W)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
        XA = Xs[rows, idx]
        if l < L - 1:
            for a in range(k):
                XA[:, a] = XA[:, a] + H_post[:, a, l, None] * F_outs[:, l]
        else:
            mixed = np.zeros_like(XA)
            for a in range(k):
                for b in range(k):
                    mixed[:, a] += H_res[:, a, b, None] * XA[:, b]
                for r in range(K_last):
                    mixed[:, a] += H_post[:, a, L - 1 + r, None] * last[:, r]
            XA = mixed
        Xs[rows, idx] = XA
    got_X = O.xhc_flash_post(X0, idx, H_post, H_res, W, K_last=K_last)
    np.testing.assert_allclose(got_X, Xs, rtol=1e-12, atol=1e-12)
    # rows outside the active set are the entry state's
    act = np.zeros((T, X0.shape[1]), bool)
    act[rows, idx] = True
    np.testing.assert_array_equal(got_X[~act], X0[~act])
    if L == 1:  # one augmented sublayer is xhc_route with the K_last components
        X1, hp, hr = O.xhc_route(X0, idx, phi_act, b_act, 0.6, 0.9, last, 20)
        np.testing.assert_allclose(got_X, X1, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(H_post, hp, rtol=1e-14)


def test_flash_single_sublayer_is_xhc():
    """L = 1 is one plain xHC sublayer: the same h_pre, dense read and active set
    as xhc_pre, and the block end equals xhc_route with Wb = F_out."""
    X0, phis, bs, w_r, phi_act, b_act, F_outs = _flash_case(720, L=1)
    pre = O.xhc_flash_pre(X0, phis, bs, 0.7, w_r, 4, 2)
    ref = O.xhc_pre(X0, phis[0], bs[0], 0.7, w_r, 4, 2)
    np.testing.assert_array_equal(pre["idx"], ref["idx"])
    np.testing.assert_allclose(pre["h_pre"][0], ref["h_pre"], rtol=1e-14)
    np.testing.assert_allclose(pre["F_pre"][0], ref["F_in"], rtol=1e-14)
    H_post, H_res = O.xhc_flash_maps(X0, pre["idx"], phi_act, b_act, 0.6, 0.9, 1, 20)
    X1, hp, hr = O.xhc_route(X0, pre["idx"], phi_act, b_act, 0.6, 0.9, F_outs[:, 0], 20)
    np.testing.assert_allclose(O.xhc_flash_post(X0, pre["idx"], H_post, H_res, F_outs), X1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(H_post, hp, rtol=1e-14)


def test_flash_correction_coefficient_by_hand():
    """One token, N = 6, k = 4 active streams idx = (0, 1, 3, 5), L = 2: the
    correction of sublayer 1 is c = sum_a h_pre^(1)[idx_a] H_post[a, 0] (here
    0.5*1 + 0.25*2 + 1*0 + 2*0.5 = 2), so F_in^(1) = F_pre^(1) + 2 F_out^(0)."""
    h1 = np.array([[0.5, 0.25, 9.0, 1.0, 9.0, 2.0]])
    idx = np.array([[0, 1, 3, 5]])
    H_post = np.zeros((1, 4, 2))
    H_post[0, :, 0] = [1.0, 2.0, 0.0, 0.5]
    H_post[0, :, 1] = [7.0, 7.0, 7.0, 7.0]  # sublayer 1's own map plays no part in its input
    F_pre1 = np.array([[1.0, -1.0, 3.0]])
    F_outs = np.array([[[2.0, 0.0, -1.0], [100.0, 100.0, 100.0]]])
    got = O.xhc_flash_input(1, F_pre1, h1, idx, H_post, F_outs)
    np.testing.assert_allclose(got, [[5.0, -1.0, 1.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.xhc_flash_input(0, F_pre1, h1, idx, H_post, F_outs), F_pre1, rtol=0, atol=0)
