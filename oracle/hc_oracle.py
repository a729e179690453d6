"""Plain fp64 CPU oracle for the hyper-connection sublayer (mHC and xHC).

TEST INFRASTRUCTURE. Only the test suite, the smoke check in __graft_entry__ and
the cpu_baseline leg of bench.py may import or run this module. The product path
(the HIP library and its Python binding) never calls it, and this module imports
nothing from the product package: the two share no kernels, helpers, tables or
constants. Inputs come from the seeded generators in
synth/__init__.py, which hold no arithmetic of the method.

Everything is evaluated in float64 straight from the definitions on the pages:

* "mHC: Manifold-Constrained Hyper-Connections" (paper notes), Eq. 3 (layer
  update), Eq. 6 (Birkhoff polytope), section 4.2 Eq. 7-9 (parameterisation,
  sigmoid / 2*sigmoid activations, Sinkhorn-Knopp with t_max = 20), section
  4.3.1 Eq. 10-19 (merged phi and b, RMS factor r) and the F_pre / F_post,res
  definitions that close section 4.3.1.
* "xHC: Expanded Hyper-Connections" (paper summary), Method: temporal feature
  augmentation (causal depthwise convolutions, Gram-Schmidt over the K_r
  components), sparse residual stream architecture (steps 1-3: fixed + routed
  streams, dense read, sparse update with inactive streams passed through), and
  parameterisation (alpha gate, Sinkhorn on the active streams, 2*sigmoid post).
* "xHC" repository README, default configuration table (N=16, k=4, 2 fixed /
  2 routed, kernels {4,8,12}, augmentation on the MLP side only).

Readings where the pages are silent or garbled (flattening order, column order
of phi, no RMSNorm epsilon, routed scores used for selection only, ascending
slot order, causal padding per sequence, ...) are stated at each function.

Parity pins: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (closed forms, invariants, brute force, library
routines, hand-derived fixtures under tests/golden/).
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Elementary maps
# ---------------------------------------------------------------------------

def sigmoid(z):
    """sigma(z) = 1 / (1 + e^-z)  (mHC notes, Eq. 8 and Eq. 17)."""
    z = _f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def sinkhorn_knopp(logits, iters: int):
    """Sinkhorn-Knopp of mHC notes section 4.2, Eq. 8-9.

    M^(0) = exp(logits); each iteration first normalises every column to sum 1
    (T_c) and then every row to sum 1 (T_r): M^(t) = T_r(T_c(M^(t-1))). The
    result is M^(iters); no epsilon, no temperature. Works on [..., n, n].
    """
    M = np.exp(_f64(logits))
    for _ in range(int(iters)):
        M = M / M.sum(axis=-2, keepdims=True)  # T_c: column sums -> 1
        M = M / M.sum(axis=-1, keepdims=True)  # T_r: row sums -> 1
    return M


def flatten_state(X):
    """vec(x_l): the n x C state of each token as one 1 x nC row (mHC notes, 4.2).

    Reading: row-major, stream-major order (index i*C + c), i.e. the contiguous
    slice of X[T, n, C].
    """
    X = _f64(X)
    return X.reshape(X.shape[0], -1)


def rms_normalise(xflat):
    """RMSNorm of the flattened state without epsilon and without a gain.

    Eq. 15 of mHC notes 4.3.1 gives r = ||x||_2 / sqrt(nC); the RMSNorm weight is
    folded into phi (4.3.1), and no epsilon appears on the page. Reading for the
    all-zero state: u = 0 (the limit of RMSNorm(0) as epsilon -> 0+).
    Returns (u, r) with u = x / r.
    """
    xflat = _f64(xflat)
    r = np.sqrt(np.mean(xflat * xflat, axis=-1))
    safe = np.where(r > 0.0, r, 1.0)
    u = np.where((r > 0.0)[:, None], xflat / safe[:, None], 0.0)
    return u, r


# ---------------------------------------------------------------------------
# mHC (dense n-stream) sublayer
# ---------------------------------------------------------------------------

def mhc_logits(X, phi, bias, alpha):
    """Gated logits [H~pre | H~post | H~res] per token (mHC notes Eq. 7, 14-16).

    X: [T, n, C]; phi: [nC, n*n + 2n] with columns [pre n | post n | res n*n];
    bias: [n*n + 2n] in the same order; alpha = (alpha_pre, alpha_post, alpha_res).
    z = alpha_block * (RMSNorm(vec x) @ phi) + b. (Eq. 16 divides by r after the
    product; that is the same number in exact arithmetic.)
    """
    X = _f64(X)
    T, n, C = X.shape
    phi = _f64(phi)
    assert phi.shape == (n * C, n * n + 2 * n)
    u, _ = rms_normalise(flatten_state(X))
    P = u @ phi
    a = _f64(alpha)
    gate = np.concatenate([np.full(n, a[0]), np.full(n, a[1]), np.full(n * n, a[2])])
    return gate[None, :] * P + _f64(bias)[None, :]


def hc_coeffs(X, phi, bias, alpha, sinkhorn_iters: int = 20):
    """H_pre = sigma, H_post = 2 sigma, H_res = Sinkhorn-Knopp (mHC notes Eq. 8, 17-19).

    Returns h_pre [T, n], h_post [T, n], h_res [T, n, n]; mat() is row-major:
    H_res[i, j] = z_res[i*n + j].
    """
    X = _f64(X)
    T, n, _ = X.shape
    z = mhc_logits(X, phi, bias, alpha)
    h_pre = sigmoid(z[:, :n])
    h_post = 2.0 * sigmoid(z[:, n:2 * n])
    h_res = sinkhorn_knopp(z[:, 2 * n:].reshape(T, n, n), sinkhorn_iters)
    return h_pre, h_post, h_res


def hc_pre(X, h_pre):
    """F_pre = H_pre x_l: F_in[t, c] = sum_i h_pre[t, i] X[t, i, c] (mHC notes 4.3.1)."""
    X = _f64(X)
    return np.einsum("ti,tic->tc", _f64(h_pre), X)


def hc_post(X, h_res, h_post, F_out):
    """F_post,res = H_res x_l + H_post^T F (mHC notes Eq. 3 and 4.3.1).

    X_next[t, i, c] = sum_j h_res[t, i, j] X[t, j, c] + h_post[t, i] F_out[t, c].
    H_post^T F is the outer product of the 1 x n row H_post with the C-vector F
    (the only product the dimensions allow).
    """
    X = _f64(X)
    return (np.einsum("tij,tjc->tic", _f64(h_res), X)
            + _f64(h_post)[:, :, None] * _f64(F_out)[:, None, :])


def mhc_sublayer(X, phi, bias, alpha, F_out, sinkhorn_iters: int = 20):
    """One forward sublayer: coefficients, pre-read, post/res write.

    F_out is supplied (it stands in for F(F_in)). Returns dict with every output.
    """
    h_pre, h_post, h_res = hc_coeffs(X, phi, bias, alpha, sinkhorn_iters)
    F_in = hc_pre(X, h_pre)
    X_next = hc_post(X, h_res, h_post, F_out)
    return dict(h_pre=h_pre, h_post=h_post, h_res=h_res, F_in=F_in, X_next=X_next)


# ---------------------------------------------------------------------------
# xHC (N streams, k active) sublayer
# ---------------------------------------------------------------------------

def xhc_router_scores(X, w_router):
    """Sigmoid router scores over the candidate streams m..N-1.

    xHC summary, sparse residual stream architecture, step 1: scores are sigmoid
    of a score derived from the full N-stream state. Reading: a linear router
    on the RMS-normalised flattened state, no bias, no gate:
    s = sigma(u_full @ W_r), W_r: [N*C, N-m].
    """
    u, _ = rms_normalise(flatten_state(X))
    return sigmoid(u @ _f64(w_router))


def xhc_select(score, k: int, m: int):
    """Active set: m fixed streams plus the top-(k-m) candidates by score.

    xHC summary step 1 (fixed + routed). Readings: candidates are streams
    m..N-1 (score column j belongs to stream m+j); ties go to the lower stream
    index; the k slots are listed in ascending stream order.
    Returns idx [T, k] int64.
    """
    score = _f64(score)
    T, ncand = score.shape
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(ncand), key=lambda j: (-score[t, j], j))[: k - m]
        chosen = list(range(m)) + [m + j for j in order]
        idx[t] = sorted(chosen)
    return idx


def xhc_pre(X, phi_pre, b_pre, alpha_pre, w_router=None, k=None, m=None):
    """Full-state pass: dense read over all N streams (+ router and selection).

    xHC summary step 2: input_l = sum_{i<N} h_pre_i x_i, with h_pre from the
    shared gated-projection pattern (reading: as mHC, h_pre = sigma(alpha_pre *
    (RMSNorm(vec X) @ phi_pre) + b_pre)).
    Returns dict(h_pre, F_in[, score, idx]).
    """
    X = _f64(X)
    u, _ = rms_normalise(flatten_state(X))
    h_pre = sigmoid(float(alpha_pre) * (u @ _f64(phi_pre)) + _f64(b_pre)[None, :])
    out = dict(h_pre=h_pre, F_in=hc_pre(X, h_pre))
    if w_router is not None:
        s = xhc_router_scores(X, w_router)
        out["score"] = s
        out["idx"] = xhc_select(s, k, m)
    return out


def xhc_gather(X, idx):
    """X_active: the k active stream rows of each token, in slot order."""
    X = _f64(X)
    T = X.shape[0]
    return X[np.arange(T)[:, None], np.asarray(idx)]


def xhc_active_coeffs(X_A, phi_act, b_act, alpha_post, alpha_res, K: int,
                      sinkhorn_iters: int = 20):
    """H_post_A [k, K] = 2 sigma(.), H_res_A [k, k] = Sinkhorn-Knopp(.) from X_active.

    xHC summary step 3 (maps generated only from the active state) and
    parameterisation (alpha gate, 2*sigmoid post map, Sinkhorn on the active
    streams). Readings: X_active is flattened in slot order and RMS-normalised
    on its own (r_A = ||vec X_A|| / sqrt(kC)); phi_act: [k*C, k*K + k*k] with
    columns [post (a*K + j) | res (a*k + b)], b_act in the same order.
    """
    X_A = _f64(X_A)
    T, k, _ = X_A.shape
    u, _ = rms_normalise(flatten_state(X_A))
    P = u @ _f64(phi_act)
    z = np.concatenate([float(alpha_post) * P[:, :k * K],
                        float(alpha_res) * P[:, k * K:]], axis=1) + _f64(b_act)[None, :]
    H_post = 2.0 * sigmoid(z[:, :k * K]).reshape(T, k, K)
    H_res = sinkhorn_knopp(z[:, k * K:].reshape(T, k, k), sinkhorn_iters)
    return H_post, H_res


def xhc_route(X, idx, phi_act, b_act, alpha_post, alpha_res, Wb, sinkhorn_iters: int = 20):
    """Sparse residual update, scattered back (xHC summary step 3).

    X_A_new = H_res_A X_A + H_post_A Wb, where Wb[t] is the K x C stack of
    write-back components (K = 1: F_out; K = r+1: the augmented components).
    The rows idx[t] of X[t] are replaced; every other stream passes through.
    Returns (X_new [T, N, C] fp64, H_post [T, k, K], H_res [T, k, k]).
    """
    X = _f64(X).copy()
    idx = np.asarray(idx)
    Wb = _f64(Wb)
    if Wb.ndim == 2:
        Wb = Wb[:, None, :]
    T = X.shape[0]
    K = Wb.shape[1]
    X_A = xhc_gather(X, idx)
    H_post, H_res = xhc_active_coeffs(X_A, phi_act, b_act, alpha_post, alpha_res, K,
                                      sinkhorn_iters)
    X_A_new = np.einsum("tab,tbc->tac", H_res, X_A) + np.einsum("taj,tjc->tac", H_post, Wb)
    X[np.arange(T)[:, None], idx] = X_A_new
    return X, H_post, H_res


def causal_dwconv(F_out, w, batch: int, seq: int):
    """Causal depthwise 1-D convolution along each sequence (xHC summary, temporal
    feature augmentation; kernel sizes from the README's default configuration).

    F_out: [batch*seq, C] (tokens of each sequence contiguous), w: [C, kappa].
    Readings: cross-correlation with w[c, kappa-1] on the current token,
    g[t, c] = sum_s w[c, s] * F_out[t - kappa + 1 + s, c], zero before the start
    of each sequence, no bias, no activation.
    """
    F = _f64(F_out).reshape(batch, seq, -1)
    w = _f64(w)
    kappa = w.shape[1]
    C = F.shape[2]
    pad = np.concatenate([np.zeros((batch, kappa - 1, C)), F], axis=1)
    g = np.zeros_like(F)
    for s in range(kappa):
        g += w[None, None, :, s] * pad[:, s:s + seq, :]
    return g.reshape(batch * seq, C)


def modified_gram_schmidt(comps):
    """Gram-Schmidt over the K_r components of each token (xHC summary).

    comps: [T, K_r, C] = [out; g_1; ...; g_r]. v_1 = out; for j = 1..r the
    component g_j has its projections on v_1..v_j removed one after the other
    (the modified form: each coefficient uses the partially updated vector).
    The components are not normalised and no epsilon is used.
    """
    G = _f64(comps)
    T, Kr, C = G.shape
    V = np.empty_like(G)
    V[:, 0] = G[:, 0]
    for j in range(1, Kr):
        v = G[:, j].copy()
        for i in range(j):
            num = np.sum(v * V[:, i], axis=1)
            den = np.sum(V[:, i] * V[:, i], axis=1)
            v = v - (num / den)[:, None] * V[:, i]
        V[:, j] = v
    return V


def xhc_augment(F_out, conv_ws, batch: int, seq: int):
    """out_aug = [out; DWConv_k1(out); ...] followed by Gram-Schmidt -> V [T, K_r, C]."""
    F = _f64(F_out)
    comps = [F] + [causal_dwconv(F, w, batch, seq) for w in conv_ws]
    return modified_gram_schmidt(np.stack(comps, axis=1))


# ---------------------------------------------------------------------------
# The unconstrained HC baseline and the gain of a chain of residual maps
# ---------------------------------------------------------------------------

def hc_tanh_coeffs(X, theta, bias, alpha):
    """Hyper-Connections' maps (mHC notes, section 3 Preliminary, Eq. 5).

    Each stream row x_i (length C) of a token is RMS-normalised on its own (the
    last dimension; reading: no learnable gain and no epsilon, and an all-zero
    row gives x~ = 0), then
        H_pre[i]     = a_pre  * tanh(theta_pre    . x~_i) + b_pre[i]
        H_post[i]    = a_post * tanh(theta_post   . x~_i) + b_post[i]
        H_res[j, i]  = a_res  * tanh(theta_res[j] . x~_i) + b_res[j, i]
    (H_res = a tanh(theta_res x~^T) + b: row j, column i; row j is output stream j
    of the residual update, as in the mHC calls).
    theta: [n + 2, C] rows (pre, post, res_0 .. res_{n-1}); bias: [n*n + 2n]
    (pre n | post n | res n*n row-major); alpha = (pre, post, res).
    Returns h_pre [T, n], h_post [T, n], h_res [T, n, n].
    """
    X = _f64(X)
    T, n, C = X.shape
    th = _f64(theta)
    b = _f64(bias)
    r = np.sqrt(np.mean(X * X, axis=2, keepdims=True))
    xt = np.divide(X, r, out=np.zeros_like(X), where=r > 0)
    P = xt @ th.T  # [T, n, n + 2]: P[t, i, k] = theta_k . x~_i
    h_pre = alpha[0] * np.tanh(P[:, :, 0]) + b[:n]
    h_post = alpha[1] * np.tanh(P[:, :, 1]) + b[n:2 * n]
    h_res = alpha[2] * np.tanh(np.transpose(P[:, :, 2:], (0, 2, 1))) + b[2 * n:].reshape(n, n)
    return h_pre, h_post, h_res


def amax_gain(h_res_layers):
    """Amax gain magnitude of a chain of residual maps (mHC notes, section 3.1).

    h_res_layers: [L, T, n, n], layer 0 first. Per token the composite map is
    M = H_{L-1} ... H_1 H_0, the product that carries x_0 to x_L through the
    residual terms of Eq. 3. The forward gain is the largest absolute row sum,
    max_i |sum_j M[i, j]|; the backward gain the largest absolute column sum,
    max_j |sum_i M[i, j]|. Returns (forward [T], backward [T]).
    """
    H = _f64(h_res_layers)
    L, T, n, _ = H.shape
    M = np.broadcast_to(np.eye(n), (T, n, n)).copy()
    for layer in range(L):
        M = H[layer] @ M
    return np.abs(M.sum(axis=2)).max(axis=1), np.abs(M.sum(axis=1)).max(axis=1)


# ---------------------------------------------------------------------------
# Static mHC (the mHC-SSM abstract): per-layer maps that do not depend on the input
# ---------------------------------------------------------------------------

def softmax(z):
    """exp(z_i) / sum_j exp(z_j) over the last axis (the max is subtracted first;
    the result is the same in exact arithmetic)."""
    z = _f64(z)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def static_mhc_maps(logits, n: int, sinkhorn_iters: int = 20):
    """Maps of static mHC ("mHC-SSM" abstract): one set per layer, shared by all
    tokens. Pre-mixing and post-mixing are simplex-constrained; reading: each is
    the softmax of its n logits (nonnegative, summing to 1). Residual mixing is
    Sinkhorn-projected as in mHC (exp of the n x n logits, then sinkhorn_iters
    alternating column / row normalisations, mHC notes Eq. 9).
    logits: [n*n + 2n] (pre n | post n | res n*n row-major, the layout of the mHC
    bias). Returns h_pre [n], h_post [n], h_res [n, n]."""
    z = _f64(logits)
    return (softmax(z[:n]), softmax(z[n:2 * n]),
            sinkhorn_knopp(z[2 * n:].reshape(n, n), sinkhorn_iters))


def static_pre(X, h_pre):
    """F_in[t] = sum_i h_pre[i] X[t, i]: the mHC pre-read with one h_pre for every token."""
    X = _f64(X)
    return hc_pre(X, np.broadcast_to(_f64(h_pre), X.shape[:2]))


def static_post(X, h_res, h_post, F_out):
    """X_next[t] = h_res X[t] + h_post^T F_out[t]: the mHC post with maps shared by every token."""
    X = _f64(X)
    T, n, _ = X.shape
    return hc_post(X, np.broadcast_to(_f64(h_res), (T, n, n)), np.broadcast_to(_f64(h_post), (T, n)), F_out)


# ---------------------------------------------------------------------------
# mHC backward (gradients of one sublayer)
# ---------------------------------------------------------------------------

def sinkhorn_knopp_backward(logits, grad, iters: int):
    """Gradient of sum(grad * SK(logits)) with respect to the logits.

    mHC notes 4.3.1, on Eq. 19: the backward recomputes the iterates and walks the
    iterations in reverse. The forward is sinkhorn_knopp: M^(0) = exp(logits);
    each iteration A = T_c(M) (A_ij = M_ij / s_j, s_j the column sum), then
    B = T_r(A) (B_ij = A_ij / q_i, q_i the row sum). For Y = M / s with s the sum
    along one axis and upstream G, dM = (G - sum_axis(G * Y)) / s. The last step is
    the derivative of exp: d logits = dM^(0) * M^(0). Works on [..., n, n].
    """
    z = _f64(logits)
    M = np.exp(z)
    saved = []
    for _ in range(int(iters)):
        s = M.sum(axis=-2, keepdims=True)
        A = M / s
        q = A.sum(axis=-1, keepdims=True)
        B = A / q
        saved.append((s, A, q, B))
        M = B
    g = _f64(grad)
    for s, A, q, B in reversed(saved):
        g = (g - (g * B).sum(axis=-1, keepdims=True)) / q  # through T_r
        g = (g - (g * A).sum(axis=-2, keepdims=True)) / s  # through T_c
    return g * np.exp(z)


def mhc_sublayer_backward(X, phi, bias, alpha, F_out, dX_next, dF_in, sinkhorn_iters: int = 20):
    """Gradients of one mHC sublayer (mhc_sublayer) for the upstream gradients
    dX_next [T, n, C] of X_next and dF_in [T, C] of F_in.

    The forward is recomputed from X (mHC notes 4.3: the intermediates of the mHC
    kernels are recomputed in the backward rather than kept), in the form of Eq.
    14-16: P = vec(x) phi, r = ||vec x|| / sqrt(nC), z = alpha_block * P / r + b.
    Then the chain rule in reverse order:
      F_post,res (Eq. 3): dF_out = H_post dX_next, dH_res[i, j] = <dX_next_i, x_j>,
        dH_post[i] = <dX_next_i, F_out>, dx_j += sum_i H_res[i, j] dX_next_i;
      F_pre: dH_pre[i] = <dF_in, x_i>, dx_i += H_pre[i] dF_in;
      Eq. 17-19: dz = dH_pre sigma', dH_post 2 sigma', Sinkhorn backward;
      Eq. 16: db = dz, dalpha_block = sum over the block of dz P / r,
        dP = alpha_block dz / r, d(1/r) = sum alpha_block dz P;
      Eq. 15: with 1/r = (ss / nC)^(-1/2), ss = ||vec x||^2,
        dss = -(1/2) d(1/r) (1/r)^3 / nC, and d vec x += 2 dss vec x;
      Eq. 14: d vec x += dP phi^T, dphi = vec(x)^T dP.
    Reading for the all-zero state: 1/r is taken as 0 there (as in the forward)
    and contributes no gradient.
    Returns dict(dX [T, n, C], dF_out [T, C], dphi [nC, n*n + 2n], dbias
    [n*n + 2n], dalpha [3], dz [T, n*n + 2n], dh [T, n*n + 2n]); dh holds the
    gradients of the maps [dH_pre | dH_post | dH_res (row-major)] per token;
    dbias and dalpha sum over tokens.
    """
    X = _f64(X)
    T, n, C = X.shape
    N = n * C
    x = X.reshape(T, N)
    phi = _f64(phi)
    assert phi.shape == (N, n * n + 2 * n)
    a = _f64(alpha)
    gate = np.concatenate([np.full(n, a[0]), np.full(n, a[1]), np.full(n * n, a[2])])
    ss = np.sum(x * x, axis=-1)
    r = np.sqrt(ss / N)
    rho = np.where(r > 0.0, 1.0 / np.where(r > 0.0, r, 1.0), 0.0)
    P = x @ phi
    z = gate[None, :] * P * rho[:, None] + _f64(bias)[None, :]
    h_pre = sigmoid(z[:, :n])
    s_post = sigmoid(z[:, n:2 * n])
    h_post = 2.0 * s_post
    z_res = z[:, 2 * n:].reshape(T, n, n)
    h_res = sinkhorn_knopp(z_res, sinkhorn_iters)

    dXn = _f64(dX_next)
    dFi = _f64(dF_in)
    Fo = _f64(F_out)
    # post/res write
    dF_out = np.einsum("ti,tic->tc", h_post, dXn)
    dh_res = np.einsum("tic,tjc->tij", dXn, X)
    dh_post = np.einsum("tic,tc->ti", dXn, Fo)
    dX = np.einsum("tij,tic->tjc", h_res, dXn)
    # pre-read
    dh_pre = np.einsum("tc,tic->ti", dFi, X)
    dX = dX + h_pre[:, :, None] * dFi[:, None, :]
    # activations and Sinkhorn
    dz = np.empty_like(z)
    dz[:, :n] = dh_pre * h_pre * (1.0 - h_pre)
    dz[:, n:2 * n] = dh_post * 2.0 * s_post * (1.0 - s_post)
    dz[:, 2 * n:] = sinkhorn_knopp_backward(z_res, dh_res, sinkhorn_iters).reshape(T, n * n)
    # gates and bias
    dbias = dz.sum(axis=0)
    u = dz * P * rho[:, None]
    dalpha = np.array([u[:, :n].sum(), u[:, n:2 * n].sum(), u[:, 2 * n:].sum()])
    dP = dz * gate[None, :] * rho[:, None]
    drho = np.sum(dz * gate[None, :] * P, axis=-1)
    dss = np.where(ss > 0.0, -0.5 * drho * rho ** 3 / N, 0.0)
    # RMS factor and projection
    dx = dP @ phi.T + 2.0 * dss[:, None] * x
    dphi = x.T @ dP
    dX = dX + dx.reshape(T, n, C)
    dh = np.concatenate([dh_pre, dh_post, dh_res.reshape(T, n * n)], axis=1)
    return dict(dX=dX, dF_out=dF_out, dphi=dphi, dbias=dbias, dalpha=dalpha, dz=dz, dh=dh)


# ---------------------------------------------------------------------------
# xHC backward (gradients of the routed step)
# ---------------------------------------------------------------------------

def _gates_backward(dz, P, rho, gate, x, phi, N):
    """The shared tail of the gated-projection backward (Eq. 14-16 pattern):
    z = gate * P * rho + b with P = x phi and rho = 1/r = (||x||^2 / N)^(-1/2).
    Returns (d x [T, N], dphi, dbias, per-column dz P rho summed over tokens)."""
    ss = np.sum(x * x, axis=-1)
    dP = dz * gate[None, :] * rho[:, None]
    drho = np.sum(dz * gate[None, :] * P, axis=-1)
    dss = np.where(ss > 0.0, -0.5 * drho * rho ** 3 / N, 0.0)
    dx = dP @ phi.T + 2.0 * dss[:, None] * x
    return dx, x.T @ dP, dz.sum(axis=0), (dz * P * rho[:, None]).sum(axis=0)


def _rho(x):
    r = np.sqrt(np.mean(x * x, axis=-1))
    return np.where(r > 0.0, 1.0 / np.where(r > 0.0, r, 1.0), 0.0)


def xhc_route_backward(X, idx, phi_act, b_act, alpha_post, alpha_res, Wb, dX_next, sinkhorn_iters: int = 20):
    """Gradients of xhc_route for the upstream gradient dX_next [T, N, C].

    xHC summary step 3 with the parameterisation: on the active rows (slot order)
    the route is the mHC post/res write X_A_new = H_res_A X_A + H_post_A Wb with
    maps formed from the active state alone (r_A over k C), so its backward is
    the chain rule of mhc_sublayer_backward without the pre map: dWb = H_post_A^T
    dX_next_A, dH_post_A[a, j] = <dX_next_a, Wb_j>, dH_res_A[a, b] = <dX_next_a,
    x_b>, dx_A = H_res_A^T dX_next_A, then 2 sigma' and the Sinkhorn backward, the
    gates, the RMS factor and the projection. Rows not in idx pass through, so
    their gradient is dX_next itself; the active rows are replaced, so theirs is
    dx_A alone. idx is a constant (a discrete choice).
    Returns dict(dX [T, N, C], dWb [T, K, C], dphi_act, db_act, dalpha_post,
    dalpha_res, dh [T, k*K + k*k] = [dH_post (a*K + j) | dH_res (a*k + b)]).
    """
    X = _f64(X)
    idx = np.asarray(idx)
    Wb = _f64(Wb)
    if Wb.ndim == 2:
        Wb = Wb[:, None, :]
    T, N, C = X.shape
    k, K = idx.shape[1], Wb.shape[1]
    X_A = xhc_gather(X, idx)
    x = X_A.reshape(T, k * C)
    phi = _f64(phi_act)
    rho = _rho(x)
    P = x @ phi
    gate = np.concatenate([np.full(k * K, float(alpha_post)), np.full(k * k, float(alpha_res))])
    z = gate[None, :] * P * rho[:, None] + _f64(b_act)[None, :]
    s_post = sigmoid(z[:, :k * K]).reshape(T, k, K)
    H_post = 2.0 * s_post
    z_res = z[:, k * K:].reshape(T, k, k)
    H_res = sinkhorn_knopp(z_res, sinkhorn_iters)
    dXn_A = xhc_gather(dX_next, idx)
    dWb = np.einsum("taj,tac->tjc", H_post, dXn_A)
    dH_post = np.einsum("tac,tjc->taj", dXn_A, Wb)
    dH_res = np.einsum("tac,tbc->tab", dXn_A, X_A)
    dX_A = np.einsum("tab,tac->tbc", H_res, dXn_A)
    dz = np.concatenate([(dH_post * 2.0 * s_post * (1.0 - s_post)).reshape(T, k * K),
                         sinkhorn_knopp_backward(z_res, dH_res, sinkhorn_iters).reshape(T, k * k)], axis=1)
    dx, dphi, dbias, u = _gates_backward(dz, P, rho, gate, x, phi, k * C)
    dX_A = dX_A + dx.reshape(T, k, C)
    dX = _f64(dX_next).copy()
    dX[np.arange(T)[:, None], idx] = dX_A
    dh = np.concatenate([dH_post.reshape(T, k * K), dH_res.reshape(T, k * k)], axis=1)
    return dict(dX=dX, dWb=dWb, dphi_act=dphi, db_act=dbias, dalpha_post=u[:k * K].sum(),
                dalpha_res=u[k * K:].sum(), dh=dh)


def xhc_pre_backward(X, phi_pre, b_pre, alpha_pre, dF_in):
    """Gradients of xhc_pre's dense read F_in = sum_i h_pre_i x_i for the upstream
    gradient dF_in [T, C].

    xHC summary step 2 with h_pre = sigma(alpha_pre (vec X) phi_pre / r + b_pre),
    r over the whole N C state (as xhc_pre). dH_pre[i] = <dF_in, x_i>, dx_i +=
    H_pre[i] dF_in, then sigma', the gate, the RMS factor and the projection.
    Reading: the router's scores only choose the active set (they scale nothing),
    and the choice is discrete, so the router weights receive no gradient.
    Returns dict(dX [T, N, C], dphi_pre [NC, N], db_pre [N], dalpha_pre,
    dh_pre [T, N]).
    """
    X = _f64(X)
    T, N, C = X.shape
    x = X.reshape(T, N * C)
    phi = _f64(phi_pre)
    rho = _rho(x)
    P = x @ phi
    gate = np.full(N, float(alpha_pre))
    h = sigmoid(gate[None, :] * P * rho[:, None] + _f64(b_pre)[None, :])
    dFi = _f64(dF_in)
    dh_pre = np.einsum("tc,tic->ti", dFi, X)
    dX = h[:, :, None] * dFi[:, None, :]
    dz = dh_pre * h * (1.0 - h)
    dx, dphi, dbias, u = _gates_backward(dz, P, rho, gate, x, phi, N * C)
    return dict(dX=dX + dx.reshape(T, N, C), dphi_pre=dphi, db_pre=dbias, dalpha_pre=u.sum(), dh_pre=dh_pre)


def causal_dwconv_backward(F_out, w, batch: int, seq: int, dg):
    """Gradients of causal_dwconv (g = conv(F_out, w)) for the upstream dg [T, C]:
    dF[t, c] = sum_s w[c, s] dg[t + kappa - 1 - s, c] (within the sequence: the
    conv read F[t'] for the outputs t' .. t' + kappa - 1), dw[c, s] = sum over the
    tokens t of dg[t, c] F[t - kappa + 1 + s, c] (zero before the sequence start).
    Returns (dF [T, C], dw [C, kappa])."""
    F = _f64(F_out).reshape(batch, seq, -1)
    w = _f64(w)
    G = _f64(dg).reshape(batch, seq, -1)
    kappa = w.shape[1]
    C = F.shape[2]
    padF = np.concatenate([np.zeros((batch, kappa - 1, C)), F], axis=1)
    padG = np.concatenate([G, np.zeros((batch, kappa - 1, C))], axis=1)
    dF = np.zeros_like(F)
    dw = np.zeros_like(w)
    for s in range(kappa):
        dF += w[None, None, :, s] * padG[:, kappa - 1 - s:kappa - 1 - s + seq, :]
        dw[:, s] = np.sum(G * padF[:, s:s + seq, :], axis=(0, 1))
    return dF.reshape(batch * seq, C), dw


def modified_gram_schmidt_backward(comps, dV):
    """Gradient of modified_gram_schmidt for the upstream dV [T, K_r, C].

    The forward steps are recomputed and walked in reverse. Step (j, i) replaces
    v by v - (n / d) V_i with n = <v, V_i>, d = <V_i, V_i>; for upstream gv:
      d v_old = gv - (<V_i, gv> / d) V_i,
      d V_i  += -(n / d) gv - <V_i, gv> (v_old / d - 2 n V_i / d^2).
    The steps of component j run after those of every earlier component, so
    walking j from the last down collects every term of dV_i before V_i's own
    steps are walked. Returns d comps [T, K_r, C]."""
    G = _f64(comps)
    T, Kr, C = G.shape
    V = np.empty_like(G)
    V[:, 0] = G[:, 0]
    steps = {}
    for j in range(1, Kr):
        v = G[:, j].copy()
        for i in range(j):
            steps[j, i] = v.copy()
            n = np.sum(v * V[:, i], axis=1)
            d = np.sum(V[:, i] * V[:, i], axis=1)
            v = v - (n / d)[:, None] * V[:, i]
        V[:, j] = v
    gV = _f64(dV).copy()
    dU = np.zeros_like(G)
    for j in range(Kr - 1, 0, -1):
        gv = gV[:, j].copy()
        for i in range(j - 1, -1, -1):
            v_old = steps[j, i]
            Vi = V[:, i]
            n = np.sum(v_old * Vi, axis=1)[:, None]
            d = np.sum(Vi * Vi, axis=1)[:, None]
            p = np.sum(Vi * gv, axis=1)[:, None]
            gV[:, i] += -(n / d) * gv - p * (v_old / d - 2.0 * n * Vi / d ** 2)
            gv = gv - (p / d) * Vi
        dU[:, j] = gv
    dU[:, 0] = gV[:, 0]
    return dU


def xhc_augment_backward(F_out, conv_ws, batch: int, seq: int, dV):
    """Gradients of xhc_augment for the upstream dV [T, K_r, C]: Gram-Schmidt
    backward, then component 0 (F_out itself) plus each causal conv's backward.
    Returns dict(dF_out [T, C], dconv_ws [list of [C, kappa]])."""
    F = _f64(F_out)
    comps = [F] + [causal_dwconv(F, w, batch, seq) for w in conv_ws]
    dU = modified_gram_schmidt_backward(np.stack(comps, axis=1), dV)
    dF = dU[:, 0].copy()
    dws = []
    for j, w in enumerate(conv_ws):
        df, dw = causal_dwconv_backward(F, w, batch, seq, dU[:, j + 1])
        dF += df
        dws.append(dw)
    return dict(dF_out=dF, dconv_ws=dws)


# ------------------------------------------------------------------ xHC-Flash
#
# "xHC: Expanded Hyper-Connections" (paper summary, memory efficiency and the
# xHC-Flash variant; repository README, method and memory-efficiency table): a block of L consecutive sublayers shares one routing
# decision, forms every sublayer's pre map from the block-entry state, and
# defers the residual mixing to the block's last sublayer (attention + MLP: L =
# 2; the four-sublayer variant: L = 4); a light correction rebuilds the later
# sublayers' inputs without reading the state again. The pages give no
# formulas; the readings taken here:
#  * sublayer l has its own phi_pre^(l), b_pre^(l) (alpha_pre shared) applied to
#    the RMS-normalised flattening of the entry state X_0, as xhc_pre forms h_pre;
#  * the router runs once on X_0; its active set idx serves all L sublayers;
#  * the active maps come from X_0's active rows: a post map per sublayer (one
#    write-back component each) and one H_res for the block, i.e.
#    xhc_active_coeffs with K = L (post columns a*L + l);
#  * sublayers l < L-1 add H_post[:, l] F_out^(l) to the active rows with no
#    mixing; the last one mixes with H_res and adds its own write, as xhc_route.
# Under these readings the later dense reads are exact functions of the entry
# state's dense reads and the earlier outputs (xhc_flash_input).


def xhc_flash_pre(X, phi_pres, b_pres, alpha_pre, w_router, k: int, m: int):
    """Block entry: the shared active set and the L pre maps and dense reads of X_0.
    Returns dict(idx [T, k], score, h_pre [L, T, N], F_pre [L, T, C])."""
    first = xhc_pre(X, phi_pres[0], b_pres[0], alpha_pre, w_router, k, m)
    hs, fs = [first["h_pre"]], [first["F_in"]]
    for l in range(1, len(phi_pres)):
        r = xhc_pre(X, phi_pres[l], b_pres[l], alpha_pre)
        hs.append(r["h_pre"])
        fs.append(r["F_in"])
    return dict(idx=first["idx"], score=first["score"], h_pre=np.stack(hs), F_pre=np.stack(fs))


def xhc_flash_maps(X, idx, phi_act, b_act, alpha_post, alpha_res, L: int, sinkhorn_iters: int = 20,
                   K_last: int = 1):
    """The block's maps from X_0's active rows: H_post [T, k, L - 1 + K_last] (column
    l < L - 1: sublayer l's post map; columns L - 1 ..: one per write-back component
    of the last sublayer, which the README's configuration augments on the MLP
    side, K_last = K_r = 4) and the block's H_res [T, k, k]; phi_act has
    k (L - 1 + K_last) + k*k columns in xhc_active_coeffs' order."""
    return xhc_active_coeffs(xhc_gather(X, idx), phi_act, b_act, alpha_post, alpha_res, L - 1 + K_last,
                             sinkhorn_iters)


def xhc_flash_input(l: int, F_pre_l, h_pre_l, idx, H_post, F_outs):
    """Sublayer l's input without a second read of the state. Before l the block
    only added H_post[:, j] F_out^(j) to the active rows, so its dense read is
      F_in^(l) = F_pre^(l) + sum_{j<l} c_j F_out^(j),
      c_j[t] = sum_a h_pre^(l)[t, idx[t, a]] H_post[t, a, j].
    F_outs: [T, L, C] or a list (only j < l used)."""
    F = _f64(F_pre_l).copy()
    T = F.shape[0]
    idx = np.asarray(idx)
    h_act = _f64(h_pre_l)[np.arange(T)[:, None], idx]  # [T, k]
    H_post = _f64(H_post)
    for j in range(l):
        c = np.sum(h_act * H_post[:, :, j], axis=1)
        F += c[:, None] * _f64(F_outs[:, j] if not isinstance(F_outs, list) else F_outs[j])
    return F


def xhc_flash_post(X, idx, H_post, H_res, F_outs, K_last: int = 1):
    """Block end: the active rows after all L sublayers,
      X_L,A = H_res (X_0,A + sum_{j<L-1} H_post[:, j] W_j) + sum_{j>=L-1} H_post[:, j] W_j;
    the other rows pass through. F_outs = W [T, L - 1 + K_last, C]: the outputs
    F_out^(0..L-2) of the sublayers before the last, then the last sublayer's K_last
    write-back components (F_out^(L-1) itself when K_last = 1, the augmentation's
    V with K_last = K_r). Returns X_L [T, N, C] fp64."""
    X = _f64(X).copy()
    idx = np.asarray(idx)
    F = _f64(F_outs)
    T, Kb = F.shape[0], F.shape[1]
    L = Kb - K_last + 1
    H_post = _f64(H_post)
    X_A = xhc_gather(X, idx)
    if L > 1:
        X_A = X_A + np.einsum("taj,tjc->tac", H_post[:, :, :L - 1], F[:, :L - 1])
    X_A = np.einsum("tab,tbc->tac", _f64(H_res), X_A) + np.einsum("taj,tjc->tac", H_post[:, :, L - 1:], F[:, L - 1:])
    X[np.arange(T)[:, None], idx] = X_A
    return X
