"""Throughput of the fused mHC n=4, C=4096 sublayer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one forward hyper-connection sublayer over T = 8192 tokens
(batch 4 x seq 2048) of a bfloat16 n=4, C=4096 stream state, F_out supplied:
RMS factor, skinny projection nC -> 24, gates, sigmoid / 2*sigmoid, 20
Sinkhorn iterations, pre-read F_in and post/res write X_next.

Headline (steady state of a chain of sublayers): one hc_post_pre call per step,
the work between two sublayer functions: the post/res write of sublayer l, the
coefficients of the state it writes under sublayer l+1's parameters, and sublayer
l+1's pre-read. Every step thus computes one sublayer's coefficients, pre-read and
post write. phi is a weight: it is packed once (hc_phi_pack) before timing; the
same chain with phi packed inside every step is reported too. The state
ping-pongs between two buffers; F_out rotates over three.

Also reported: the chain as two calls per step (hc_pre + hc_post_coeffs) with
each call's duration, and the isolated sublayer (hc_coeffs_pre + hc_post) on
three rotated input sets.

Prints one JSON line: tokens/s of the whole job, achieved algorithmic HBM
bandwidth, a roofline entry for the dominant call (duration from HIP events
recorded around its launches inside the timed region) and the fp64 CPU oracle
timed on the host cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s + achieved HBM GB/s (% peak), fused mHC n=4 C=4096 sublayer, 1 GPU"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
WORKLOAD = "mhc_n4_C4096_T8192_bf16"
SINKHORN_ITERS = 20


def source_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "stream_residual_mixing_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(T: int, n: int, C: int, esize: int = 2) -> dict:
    """Bytes each call must move at least (counted once per launch).

    hc_coeffs_pre: read X (nC per token), read phi and bias once, write F_in (C)
    and the n + n*n post/res coefficients (h_pre is not requested).
    hc_post: read X (nC), F_out (C) and the n*n + n coefficients, write X_next
    (nC): the (n+1)C reads and nC writes of the fused post/res kernel.
    hc_pre: read X (nC) and h_pre (n), write F_in (C).
    hc_post_coeffs: hc_post plus phi and bias once, and the n*n + 2n
    coefficients of X_next written.
    hc_post_pre: hc_post plus phi and bias once, the n*n + n post/res
    coefficients of X_next written, and the pre-read of X_next (read nC, write
    C); h_pre of X_next is used on chip and not stored."""
    ncols = n * n + 2 * n
    coef = (n + n * n) * 4
    par = n * C * ncols * 4 + ncols * 4
    cp = T * (n * C * esize + C * esize + coef) + par
    post = T * (n * C * esize + C * esize + coef + n * C * esize)
    pre = T * (n * C * esize + n * 4 + C * esize)
    pc = post + T * ncols * 4 + par
    # hc_post_pre: hc_post_coeffs without storing h_pre, plus the pre-read of X_next
    pp = post + T * (n + n * n) * 4 + par + T * (n * C * esize + C * esize)
    return {"hc_coeffs_pre": cp, "hc_post": post, "hc_pre": pre, "hc_post_coeffs": pc, "hc_post_pre": pp}


def xhc_algorithmic_bytes(T: int, N: int, C: int, k: int, m: int, K: int, esize: int = 2) -> dict:
    """Minimum bytes of each xHC call (counted once per launch; weights once).

    xhc_pre: read the full state X (N C per token) once, write F_in (C) and the
    k indices + N - m scores; phi_pre and W_r once.
    xhc_route (indices given): read the k active rows and the K write-back
    components, write the k active rows back; the k indices; phi_act once.
    xhc_augment: read F_out (C), write V (K C)."""
    pre = T * (N * C * esize + C * esize + k * 4 + (N - m) * 4) + N * C * (N + N - m) * 4
    route = T * (2 * k * C * esize + K * C * esize + k * 4) + k * C * (k * K + k * k) * 4
    aug = T * (C * esize + K * C * esize) + C * (4 + 8 + 12) * 4
    return {"xhc_pre": pre, "xhc_route": route, "xhc_augment": aug}


def hc_baseline_bench(torch, hc, dev, reps: int = 20) -> dict:
    """The HC baseline maps (hc_tanh_coeffs) and the static mHC pre-read and post on
    the n=4 C=4096 T=8192 bf16 state, three rotating state sets; and the Amax gain
    of an 8-layer chain of n=4 maps over T=16384 tokens. HIP events around the
    repeated calls."""
    T, n, C = 8192, 4, 4096
    g = torch.Generator(device=dev)
    g.manual_seed(4000)
    Xs = [torch.randn(T, n, C, device=dev, generator=g).to(torch.bfloat16) for _ in range(3)]
    theta = torch.randn(n + 2, C, device=dev, generator=g) * 0.02
    bias = torch.zeros(n * n + 2 * n, device=dev)
    out = (torch.empty(T, n, device=dev), torch.empty(T, n, device=dev), torch.empty(T, n, n, device=dev))

    def timeit(fn):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    t_tanh = timeit(lambda i: hc.hc_tanh_coeffs(Xs[i % 3], theta, bias, (0.1, 0.1, 0.1), out=out))
    tanh_bytes = T * n * C * 2 + T * (n * n + 2 * n) * 4
    L, T2 = 8, 16384
    H = (torch.eye(n, device=dev) + 0.1 * torch.randn(L, T2, n, n, device=dev, generator=g)).contiguous()
    t_gain = timeit(lambda i: hc.hc_amax_gain(H))
    gain_bytes = L * T2 * n * n * 4 + 2 * T2 * 4
    Fs = [torch.randn(T, C, device=dev, generator=g).to(torch.bfloat16) for _ in range(3)]
    z = torch.randn(n * n + 2 * n, device=dev, generator=g)
    sp, sq, sr = hc.hc_static_maps(z, n, SINKHORN_ITERS)
    F_in = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
    Xn = torch.empty(T, n, C, dtype=torch.bfloat16, device=dev)
    t_spre = timeit(lambda i: hc.hc_static_pre(Xs[i % 3], sp, out=F_in))
    t_spost = timeit(lambda i: hc.hc_static_post(Xs[i % 3], sr, sq, Fs[i % 3], out=Xn))
    spre_bytes = T * n * C * 2 + T * C * 2
    spost_bytes = T * n * C * 2 * 2 + T * C * 2
    stat = {name: {"workload": "static mHC n=4 C=4096 T=8192 bf16", "us": t * 1e6, "algorithmic_bytes": nb,
                   "achieved_GBps": nb / t / 1e9, "pct_hbm_peak": 100.0 * nb / t / 1e9 / HBM_PEAK_GBPS}
            for name, t, nb in (("hc_static_pre", t_spre, spre_bytes), ("hc_static_post", t_spost, spost_bytes))}
    return {**stat,
            "hc_tanh_coeffs": {"workload": "HC maps n=4 C=4096 T=8192 bf16", "us": t_tanh * 1e6,
                               "algorithmic_bytes": tanh_bytes, "achieved_GBps": tanh_bytes / t_tanh / 1e9,
                               "pct_hbm_peak": 100.0 * tanh_bytes / t_tanh / 1e9 / HBM_PEAK_GBPS},
            "hc_amax_gain": {"workload": "8-layer chain of n=4 maps, T=16384", "us": t_gain * 1e6,
                             "algorithmic_bytes": gain_bytes, "achieved_GBps": gain_bytes / t_gain / 1e9}}


def backward_algorithmic_bytes(T: int, n: int, C: int, esize: int = 2) -> dict:
    """Bytes of one mHC backward (both stages; n*n + 2n phi columns, float32 phi and
    dphi, float32 map gradients dh [T, n*n + 2n]): 'one_pass': read x, dX_next,
    F_out, dF_in and write dX, dF_out once, phi read and dphi written once;
    'by_design': what the launches move (post stage: x, dX_next, F_out read, dF_out
    written; main stage: x read by the projection (which also forms the dH_pre
    sums) and by the dX pass (which also forms the dphi partials), dF_in by both,
    dX_next by the dX pass, dX written)."""
    s, f = n * C * esize, C * esize
    phi_b = n * C * (n * n + 2 * n) * 4
    dh_b = (n * n + 2 * n) * 4
    post = s + s + f + f + dh_b
    main = 2 * s + 2 * f + s + s + dh_b
    return {"one_pass": T * (3 * s + 3 * f) + 2 * phi_b,
            "by_design": T * (post + main) + 2 * phi_b,
            "post_stage": T * post, "main_stage": T * main + 2 * phi_b}


def backward_bench(torch, hc, dev, reps: int = 10) -> dict:
    """The mHC sublayer backward (n=4 C=4096 T=8192 bf16): hc_backward_post then
    hc_backward, on three rotating sets of state and upstream gradients; HIP
    events around each stage of each repetition (median reported)."""
    T, n, C = 8192, 4, 4096
    g = torch.Generator(device=dev)
    g.manual_seed(5000)
    rn = lambda *shape, std=1.0: torch.randn(*shape, device=dev, generator=g) * std
    Xs = [rn(T, n, C).to(torch.bfloat16) for _ in range(3)]
    dXs = [rn(T, n, C).to(torch.bfloat16) for _ in range(3)]
    Fs = [rn(T, C).to(torch.bfloat16) for _ in range(3)]
    dFs = [rn(T, C).to(torch.bfloat16) for _ in range(3)]
    phi = rn(n * C, n * n + 2 * n, std=0.02)
    bias = torch.zeros(n * n + 2 * n, device=dev)
    bias[2 * n:] = torch.eye(n, device=dev).flatten()
    h_post = torch.rand(T, n, device=dev, generator=g) * 2.0
    dF_out = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
    dh = torch.empty(T, n * n + 2 * n, device=dev)
    out = (torch.empty(T, n, C, dtype=torch.bfloat16, device=dev), torch.empty(n * C, n * n + 2 * n, device=dev),
           torch.empty(n * n + 2 * n, device=dev), torch.empty(3, device=dev))
    ws = torch.empty(hc.hc_backward_workspace_bytes(T, n, C, torch.bfloat16), dtype=torch.uint8, device=dev)
    post = lambda i: hc.hc_backward_post(Xs[i % 3], h_post, Fs[i % 3], dXs[i % 3], out=(dF_out, dh))
    main = lambda i: hc.hc_backward(Xs[i % 3], phi, bias, (0.01, 0.01, 0.01), dXs[i % 3], dFs[i % 3], dh,
                                    SINKHORN_ITERS, out=out, workspace=ws)
    for i in range(3):
        post(i)
        main(i)
    torch.cuda.synchronize()
    tp, tm = [], []
    for r in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        post(r)
        ev[1].record()
        main(r)
        ev[2].record()
        torch.cuda.synchronize()
        tp.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        tm.append(ev[1].elapsed_time(ev[2]) * 1e-3)
    med = lambda v: sorted(v)[len(v) // 2]
    t_post, t_main = med(tp), med(tm)
    t = t_post + t_main
    bb = backward_algorithmic_bytes(T, n, C)
    return {"workload": "mHC backward n=4 C=4096 T=8192 bf16 (20 Sinkhorn iterations recomputed)",
            "us": t * 1e6, "post_stage_us": t_post * 1e6, "main_stage_us": t_main * 1e6, "tokens_per_s": T / t,
            "algorithmic_bytes": bb["one_pass"], "achieved_GBps": bb["one_pass"] / t / 1e9,
            "pct_hbm_peak": 100.0 * bb["one_pass"] / t / 1e9 / HBM_PEAK_GBPS,
            "by_design_bytes": bb["by_design"], "by_design_GBps": bb["by_design"] / t / 1e9,
            "post_stage_GBps": bb["post_stage"] / t_post / 1e9, "main_stage_GBps": bb["main_stage"] / t_main / 1e9,
            "counters": {"hc_backward_post": counter_summary(load_counters("hc_backward_post", source_digest()),
                                                             t_post),
                         "hc_backward": counter_summary(load_counters("hc_backward", source_digest()), t_main)}}


def xhc_backward_bench(torch, hc, dev, reps: int = 10) -> dict:
    """The xHC routed-step backward (N=16, k=4, m=2, C=4096, T=8192, bf16, K=1):
    xhc_route_backward then xhc_pre_backward on three rotating state sets (dX
    updated in place, as a training step does); HIP events around each call of
    each repetition (median reported). algorithmic_bytes is the one-pass
    minimum: the route reads x and dX_next on the active rows and F_out and
    writes dX on the active rows and dF_out; the pre call reads x, dF_in and dX
    and writes dX over the whole state."""
    N, k, m, C, T = 16, 4, 2, 4096, 8192
    g = torch.Generator(device=dev)
    g.manual_seed(6000)
    rn = lambda *shape, std=1.0: torch.randn(*shape, device=dev, generator=g) * std
    Xs = [rn(T, N, C).to(torch.bfloat16) for _ in range(3)]
    dXs = [rn(T, N, C).to(torch.bfloat16) for _ in range(3)]
    Fs = [rn(T, C).to(torch.bfloat16) for _ in range(3)]
    dFs = [rn(T, C).to(torch.bfloat16) for _ in range(3)]
    # an active set of m fixed and k - m routed streams per token, ascending
    r = torch.rand(T, N - m, device=dev, generator=g).argsort(dim=1)[:, :k - m] + m
    idx = torch.cat([torch.arange(m, device=dev).expand(T, m), r], 1).sort(dim=1).values.to(torch.int32).contiguous()
    phi_act = rn(k * C, k + k * k, std=0.02)
    b_act = torch.zeros(k + k * k, device=dev)
    b_act[k:] = torch.eye(k, device=dev).flatten()
    phi_pre, b_pre = rn(N * C, N, std=0.02), torch.zeros(N, device=dev)
    ws = torch.empty(hc.xhc_backward_workspace_bytes(T, N, C, k, 1, torch.bfloat16), dtype=torch.uint8, device=dev)
    ro = (torch.empty(T, C, dtype=torch.bfloat16, device=dev), torch.empty(k * C, k + k * k, device=dev),
          torch.empty(k + k * k, device=dev), torch.empty(2, device=dev), torch.empty(T, k + k * k, device=dev))
    po = (torch.empty(N * C, N, device=dev), torch.empty(N, device=dev), torch.empty(1, device=dev),
          torch.empty(T, N, device=dev))
    route = lambda i: hc.xhc_route_backward(Xs[i % 3], idx, phi_act, b_act, 0.01, 0.01, Fs[i % 3], dXs[i % 3],
                                            SINKHORN_ITERS, out=ro, workspace=ws)
    pre = lambda i: hc.xhc_pre_backward(Xs[i % 3], phi_pre, b_pre, 0.01, dFs[i % 3], dXs[i % 3], out=po, workspace=ws)
    for i in range(3):
        route(i)
        pre(i)
    torch.cuda.synchronize()
    tr, tp = [], []
    for i in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        route(i)
        ev[1].record()
        pre(i)
        ev[2].record()
        torch.cuda.synchronize()
        tr.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        tp.append(ev[1].elapsed_time(ev[2]) * 1e-3)
    med = lambda v: sorted(v)[len(v) // 2]
    t_r, t_p = med(tr), med(tp)
    s_a, s_f, f = k * C * 2, N * C * 2, C * 2
    alg_r = T * (2 * s_a + f + s_a + f) + 2 * k * C * (k + k * k) * 4
    alg_p = T * (s_f + f + s_f + s_f) + 2 * N * C * N * 4
    rate = lambda b, t: {"us": t * 1e6, "algorithmic_bytes": b, "achieved_GBps": b / t / 1e9,
                         "pct_hbm_peak": 100.0 * b / t / 1e9 / HBM_PEAK_GBPS}
    # augmented step (K = 4, B = 2 sequences of S = 4096): route backward with the
    # components V, then the augmentation backward of dV
    B, S = 2, 4096
    conv = torch.cat([rn(C, kk, std=(1.0 / kk) ** 0.5) for kk in (4, 8, 12)], 1).contiguous()
    Vs = [hc.xhc_augment(Fs[i], conv, (4, 8, 12), B, S) for i in range(3)]
    phi4 = rn(k * C, 4 * k + k * k, std=0.02)
    b4 = torch.zeros(4 * k + k * k, device=dev)
    b4[4 * k:] = torch.eye(k, device=dev).flatten()
    ro4 = (torch.empty(T, 4, C, device=dev), torch.empty(k * C, 4 * k + k * k, device=dev),
           torch.empty(4 * k + k * k, device=dev), torch.empty(2, device=dev), torch.empty(T, 4 * k + k * k, device=dev))
    ao = (torch.empty(T, C, dtype=torch.bfloat16, device=dev), torch.empty_like(conv))
    ws_a = torch.empty(hc.xhc_augment_backward_workspace_bytes(B, S, C, (4, 8, 12), torch.bfloat16), dtype=torch.uint8,
                       device=dev)
    route4 = lambda i: hc.xhc_route_backward(Xs[i % 3], idx, phi4, b4, 0.01, 0.01, Vs[i % 3], dXs[i % 3],
                                             SINKHORN_ITERS, out=ro4, workspace=ws)
    aug = lambda i: hc.xhc_augment_backward(Fs[i % 3], conv, (4, 8, 12), B, S, ro4[0], out=ao, workspace=ws_a)
    for i in range(3):
        route4(i)
        aug(i)
    torch.cuda.synchronize()
    t4, ta = [], []
    for i in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record()
        route4(i)
        ev[1].record()
        aug(i)
        ev[2].record()
        torch.cuda.synchronize()
        t4.append(ev[0].elapsed_time(ev[1]) * 1e-3)
        ta.append(ev[1].elapsed_time(ev[2]) * 1e-3)
    t_4, t_a = med(t4), med(ta)
    # route K = 4: x and dX_next on the active rows and V read, dX and dV (float32) written
    alg_4 = T * (2 * s_a + 4 * f + s_a + 4 * C * 4) + 2 * k * C * (4 * k + k * k) * 4
    # augmentation: F_out and dV read, dF_out written (taps once)
    alg_a = T * (f + 4 * C * 4 + f) + 2 * C * 24 * 4
    return {"workload": "xHC backward N=16 k=4 m=2 C=4096 T=8192 bf16: routed step (K=1) and augmented step (K=4, "
                        "B=2 S=4096, kappa 4,8,12); 20 Sinkhorn iterations recomputed",
            "tokens_per_s": T / (t_r + t_p), "us": (t_r + t_p) * 1e6,
            "xhc_route_backward": dict(rate(alg_r, t_r), counters=counter_summary(
                load_counters("xhc_route_backward", source_digest()), t_r)),
            "xhc_pre_backward": dict(rate(alg_p, t_p), counters=counter_summary(
                load_counters("xhc_pre_backward", source_digest()), t_p)),
            "augmented_us": (t_4 + t_a + t_p) * 1e6,
            "xhc_route_backward_K4": rate(alg_4, t_4), "xhc_augment_backward": rate(alg_a, t_a)}


def flash_bench(torch, hc, dev, reps: int = 10) -> dict:
    """xHC-Flash blocks of L = 2 (attention + MLP) and L = 4 sublayers at N=16, k=4,
    m=2, C=4096, T=8192 bf16, on three rotating entry states: xhc_flash_pre (routing,
    L pre maps, the L dense reads), xhc_flash_maps, xhc_flash_input for l = 1..L-1
    (sublayer 0 reads F_pre[0] as is), xhc_flash_post; HIP events around the block
    (median). algorithmic_bytes: the entry state read once, F_pre written, the
    active rows read for the maps, each corrected input's reads and write, and the
    block end's active rows read and written with the L outputs read."""
    N, k, m, C, T = 16, 4, 2, 4096, 8192
    g = torch.Generator(device=dev)
    g.manual_seed(7000)
    rn = lambda *shape, std=1.0: torch.randn(*shape, device=dev, generator=g) * std
    Xs = [rn(T, N, C).to(torch.bfloat16) for _ in range(3)]
    w_r = rn(N * C, N - m, std=(1.0 / (N * C)) ** 0.5)
    out = {}
    B, S = 2, 4096
    conv = torch.cat([rn(C, kk, std=(1.0 / kk) ** 0.5) for kk in (4, 8, 12)], 1).contiguous()
    for L, K_last in ((2, 1), (4, 1), (2, 4)):
        Kb = L - 1 + K_last
        phi_pre, b_pre = rn(L, N * C, N, std=0.02), torch.zeros(L, N, device=dev)
        phi_act = rn(k * C, k * Kb + k * k, std=0.02)
        b_act = torch.zeros(k * Kb + k * k, device=dev)
        b_act[k * Kb:] = torch.eye(k, device=dev).flatten()
        F_outs = rn(T, L, C).to(torch.bfloat16)
        W = F_outs if K_last == 1 else torch.cat([F_outs[:, :L - 1], F_outs[:, :1].expand(T, K_last, C)], 1).contiguous()
        V = torch.empty(T, K_last, C, dtype=torch.bfloat16, device=dev)
        F_last = F_outs[:, L - 1].contiguous()
        wsa = (torch.empty(max(hc.xhc_augment_workspace_bytes(B, S, C, (4, 8, 12), torch.bfloat16), 1),
                           dtype=torch.uint8, device=dev) if K_last > 1 else None)
        po = (torch.empty(T, k, dtype=torch.int32, device=dev), torch.empty(T, N - m, device=dev),
              torch.empty(L, T, N, device=dev), torch.empty(L, T, C, dtype=torch.bfloat16, device=dev))
        mo = (torch.empty(T, k, Kb, device=dev), torch.empty(T, k, k, device=dev))
        F_in = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(hc.xhc_flash_pre_workspace_bytes(T, N, C, m, L, torch.bfloat16), dtype=torch.uint8,
                          device=dev)
        wsm = torch.empty(hc.xhc_flash_maps_workspace_bytes(T, N, C, k, L, torch.bfloat16, K_last), dtype=torch.uint8,
                          device=dev)
        wsq = torch.empty(hc.xhc_flash_post_workspace_bytes(T, k, L, K_last), dtype=torch.uint8, device=dev)

        def block(i, ev=None):
            X = Xs[i % 3]
            idx, _, h_pre, F_pre = hc.xhc_flash_pre(X, phi_pre, b_pre, 0.01, w_r, k=k, m=m, out=po, workspace=wsp)
            if ev:
                ev[1].record()
            Hp, Hr = hc.xhc_flash_maps(X, idx, phi_act, b_act, 0.01, 0.01, L, K_last=K_last, out=mo, workspace=wsm)
            if ev:
                ev[2].record()
            for l in range(1, L):
                hc.xhc_flash_input(l, F_pre[l], h_pre[l], idx, Hp, W, K_last=K_last, out=F_in)
            if ev:
                ev[3].record()
            if K_last > 1:  # the last sublayer's augmentation, read by the block end where it is written
                hc.xhc_augment(F_last, conv, (4, 8, 12), B, S, out=V, workspace=wsa)
                hc.xhc_flash_post(X, idx, Hp, Hr, W, K_last=K_last, W_last=V, workspace=wsq)
            else:
                hc.xhc_flash_post(X, idx, Hp, Hr, W, K_last=K_last, workspace=wsq)

        for i in range(3):
            block(i)
        torch.cuda.synchronize()
        tt = [[], [], [], [], []]
        for i in range(reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record()
            block(i, ev)
            ev[4].record()
            torch.cuda.synchronize()
            for j in range(4):
                tt[j].append(ev[j].elapsed_time(ev[j + 1]) * 1e-3)
            tt[4].append(ev[0].elapsed_time(ev[4]) * 1e-3)
        md = [sorted(v)[len(v) // 2] for v in tt]
        e = 2
        alg = (T * N * C * e + L * T * C * e + T * k * C * e
               + sum((2 + l) * T * C * e for l in range(1, L))
               + 2 * T * k * C * e + Kb * T * C * e)
        if K_last > 1:  # the augmentation reads the MLP output and writes its components
            alg += T * C * e + K_last * T * C * e
        out[f"L{L}" + ("_augmented_mlp" if K_last > 1 else "")] = {
            "block_us": md[4] * 1e6, "per_sublayer_us": md[4] * 1e6 / L,
                        "xhc_flash_pre_us": md[0] * 1e6, "xhc_flash_maps_us": md[1] * 1e6,
                        "xhc_flash_input_us": md[2] * 1e6, "xhc_flash_post_us": md[3] * 1e6,
                        "algorithmic_bytes": alg, "achieved_GBps": alg / md[4] / 1e9,
                        "tokens_per_s_per_sublayer": T * L / md[4]}
    return {"workload": "xHC-Flash N=16 k=4 m=2 C=4096 T=8192 bf16, blocks of L = 2 and 4 sublayers (K = 1 each), "
                        "and L = 2 with the MLP's K_r = 4 augmentation (2 sequences of 4096, kappa 4, 8, 12; the "
                        "block end's time includes xhc_augment, whose output the block end reads as W_last)",
            **out}


def xhc_bench(torch, hc, dev, steps: int, warmup: int) -> dict:
    """Throughput of the xHC sublayer (N=16, k=4, m=2, C=4096, T=8192, bf16) on
    seeded synthetic device data: the routed step xhc_pre + xhc_route (K=1, F_out
    written back) and the augmented step xhc_pre + xhc_augment + xhc_route (K=4,
    B=2 S=4096), each also chained (xhc_route_pre per step), three rotating state
    sets, HIP events around every call."""
    N, k, m, C, T = 16, 4, 2, 4096, 8192
    B, S = 2, 4096
    g = torch.Generator(device=dev)
    g.manual_seed(3000)
    rn = lambda *shape, std=1.0: torch.randn(*shape, device=dev, generator=g) * std
    Xs = [rn(T, N, C).to(torch.bfloat16) for _ in range(3)]
    Fs = [rn(T, C).to(torch.bfloat16) for _ in range(3)]
    phi_pre, b_pre = rn(N * C, N, std=0.02), torch.zeros(N, device=dev)
    w_r = rn(N * C, N - m, std=(1.0 / (N * C)) ** 0.5)

    def act(K):
        b = torch.zeros(k * K + k * k, device=dev)
        b[k * K:] = torch.eye(k, device=dev).flatten()
        return rn(k * C, k * K + k * k, std=0.02), b

    phi1, b1 = act(1)
    phi4, b4 = act(4)
    conv = torch.cat([rn(C, kk, std=(1.0 / kk) ** 0.5) for kk in (4, 8, 12)], 1).contiguous()
    ab1 = xhc_algorithmic_bytes(T, N, C, k, m, 1)
    ab4 = xhc_algorithmic_bytes(T, N, C, k, m, 4)
    ws_pre = torch.empty(hc.xhc_pre_workspace_bytes(T, N, C, m, True, torch.bfloat16), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(max(hc.xhc_route_workspace_bytes(T, N, C, k, m, K, False, torch.bfloat16) for K in (1, 4)),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.empty(hc.xhc_augment_workspace_bytes(B, S, C, (4, 8, 12), torch.bfloat16), dtype=torch.uint8,
                       device=dev)

    def run(step, names):
        for i in range(warmup):
            step(i, None)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            step(warmup + i, evs[i])
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        return wall, {nm: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e-3 for j, nm in
                      enumerate(names)}

    def routed(i, evs):
        X = Xs[i % 3]
        if evs:
            evs[0].record()
        pre = hc.xhc_pre(X, phi_pre, b_pre, 0.01, w_r, k, m, want_h_pre=False, workspace=ws_pre)
        if evs:
            evs[1].record()
        hc.xhc_route(X, Fs[i % 3], phi1, b1, 0.01, 0.01, k=k, m=m, idx=pre["idx"], workspace=ws_r)
        if evs:
            evs[2].record()

    def augmented(i, evs):
        X = Xs[i % 3]
        if evs:
            evs[0].record()
        pre = hc.xhc_pre(X, phi_pre, b_pre, 0.01, w_r, k, m, want_h_pre=False, workspace=ws_pre)
        if evs:
            evs[1].record()
        V = hc.xhc_augment(Fs[i % 3], conv, (4, 8, 12), B, S, workspace=ws_a)
        if evs:
            evs[2].record()
        hc.xhc_route(X, V, phi4, b4, 0.01, 0.01, k=k, m=m, idx=pre["idx"], workspace=ws_r)
        if evs:
            evs[3].record()

    out = {}
    for name, fn, calls, ab in (("routed_K1", routed, ["xhc_pre", "xhc_route"], ab1),
                                ("augmented_K4", augmented, ["xhc_pre", "xhc_augment", "xhc_route"], ab4)):
        wall, kern = run(fn, calls)
        step_bytes = sum(ab[c] for c in calls)
        total = sum(kern.values())
        out[name] = {
            "tokens_per_s": T / total, "us_per_step": total * 1e6, "wall_us_per_step": wall * 1e6,
            "algorithmic_bytes_per_step": step_bytes,
            "achieved_GBps": step_bytes / total / 1e9, "pct_hbm_peak": 100.0 * step_bytes / total / 1e9 / HBM_PEAK_GBPS,
            "calls": {c: {"us": kern[c] * 1e6, "algorithmic_bytes": ab[c], "achieved_GBps": ab[c] / kern[c] / 1e9,
                          "pct_hbm_peak": 100.0 * ab[c] / kern[c] / 1e9 / HBM_PEAK_GBPS} for c in calls},
        }
        if name == "routed_K1":
            for c in calls:
                out[name]["calls"][c]["counters"] = counter_summary(load_counters(c, source_digest()), kern[c])
    # The chained form of the routed step: one xhc_route_pre call per sublayer (route
    # of sublayer l, maps and pre-read of sublayer l + 1, the carry of l + 2), each
    # state set carrying its own active set and carry from its previous step.
    ws_c = torch.empty(hc.xhc_chain_workspace_bytes(T, N, C, k, m, 1, torch.bfloat16), dtype=torch.uint8, device=dev)
    chain = []
    for i in range(3):
        r = hc.xhc_pre_chain(Xs[i], phi_pre, b_pre, 0.01, w_r, phi_pre, w_r, k=k, m=m, workspace=ws_c)
        chain.append([r["idx"], r["carry"]])
    fin_c = (torch.empty(T, N, device=dev), torch.empty(T, C, dtype=torch.bfloat16, device=dev))

    def chained(i, evs):
        st = chain[i % 3]
        if evs:
            evs[0].record()
        r = hc.xhc_route_pre(Xs[i % 3], Fs[i % 3], phi1, b1, 0.01, 0.01, st[0], st[1], b_pre, 0.01,
                             phi_pre_next=phi_pre, w_router_next=w_r, carry_out=st[1], k=k, m=m, out=fin_c,
                             workspace=ws_c)
        if evs:
            evs[1].record()
        st[0] = r["idx"]

    wall, kern = run(chained, ["xhc_route_pre"])
    step_bytes = ab1["xhc_pre"] + ab1["xhc_route"]
    total = kern["xhc_route_pre"]
    out["routed_K1_chained"] = {
        "tokens_per_s": T / total, "us_per_step": total * 1e6, "wall_us_per_step": wall * 1e6,
        "algorithmic_bytes_per_step": step_bytes, "achieved_GBps": step_bytes / total / 1e9,
        "pct_hbm_peak": 100.0 * step_bytes / total / 1e9 / HBM_PEAK_GBPS,
        "note": "xhc_route_pre per step (the same work as xhc_pre + xhc_route, the full state read once)",
        "counters": counter_summary(load_counters("xhc_route_pre", source_digest()), total)}

    # The augmented step chained: xhc_augment of the sublayer's F_out, then
    # xhc_route_pre with its K = 4 components (route l, pre-read of l + 1).
    ws_c4 = torch.empty(hc.xhc_chain_workspace_bytes(T, N, C, k, m, 4, torch.bfloat16), dtype=torch.uint8,
                        device=dev)
    for i in range(3):
        r = hc.xhc_pre_chain(Xs[i], phi_pre, b_pre, 0.01, w_r, phi_pre, w_r, k=k, m=m, workspace=ws_c4)
        chain[i] = [r["idx"], r["carry"]]

    def chained_aug(i, evs):
        st = chain[i % 3]
        if evs:
            evs[0].record()
        V = hc.xhc_augment(Fs[i % 3], conv, (4, 8, 12), B, S, workspace=ws_a)
        if evs:
            evs[1].record()
        r = hc.xhc_route_pre(Xs[i % 3], V, phi4, b4, 0.01, 0.01, st[0], st[1], b_pre, 0.01,
                             phi_pre_next=phi_pre, w_router_next=w_r, carry_out=st[1], k=k, m=m, out=fin_c,
                             workspace=ws_c4)
        if evs:
            evs[2].record()
        st[0] = r["idx"]

    wall, kern = run(chained_aug, ["xhc_augment", "xhc_route_pre"])
    step_bytes = ab4["xhc_pre"] + ab4["xhc_augment"] + ab4["xhc_route"]
    total = sum(kern.values())
    out["augmented_K4_chained"] = {
        "tokens_per_s": T / total, "us_per_step": total * 1e6, "wall_us_per_step": wall * 1e6,
        "algorithmic_bytes_per_step": step_bytes, "achieved_GBps": step_bytes / total / 1e9,
        "pct_hbm_peak": 100.0 * step_bytes / total / 1e9 / HBM_PEAK_GBPS,
        "calls_us": {c: v * 1e6 for c, v in kern.items()},
        "note": "xhc_augment + xhc_route_pre (K = 4) per step: the augmented step with the full state read once"}
    out["workload"] = ("xHC N=16 k=4 m=2 C=4096 T=8192 bf16 (K=1: F_out written back; K=4: B=2 S=4096 "
                       "augmentation, kappa 4,8,12); seeded synthetic device data; durations from HIP events")
    return out


def chain_c7168_bench(torch, hc, dev, layers: int = 8, rounds: int = 3) -> dict:
    """The 8-layer chain of mHC n=4, C=7168, T=16384 (batch 8 x seq 2048) bf16
    sublayers, each with its own phi (packed once, a weight) and F_out: the chain
    starts with hc_coeffs_pre, then one hc_post_pre call per layer (post/res write
    of layer l, coefficients and pre-read of layer l+1), the state ping-ponging
    between two buffers. HIP events around every call; `rounds` passes over the
    chain, median per layer reported."""
    T, n, C = 16384, 4, 7168
    g = torch.Generator(device=dev)
    g.manual_seed(2000)
    X = [(torch.randn(T, n, C, device=dev, generator=g)).to(torch.bfloat16), torch.empty(T, n, C, dtype=torch.bfloat16,
                                                                                       device=dev)]
    Fs = [torch.randn(T, C, device=dev, generator=g).to(torch.bfloat16) for _ in range(3)]
    phis = [torch.randn(n * C, n * n + 2 * n, device=dev, generator=g) * 0.02 for _ in range(layers + 1)]
    packs = [hc.hc_phi_pack(p, n, C, torch.bfloat16) for p in phis]
    bias = torch.zeros(n * n + 2 * n, device=dev)
    bias[2 * n:] = torch.eye(n, device=dev).flatten()
    alpha = [0.01] * 3
    ws = torch.empty(hc.hc_coeffs_workspace_bytes(T, n, C, torch.bfloat16), dtype=torch.uint8, device=dev)
    coef = [(None, torch.empty(T, n, device=dev), torch.empty(T, n, n, device=dev)) for _ in range(2)]
    F_in = [torch.empty(T, C, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    per = []
    for r in range(rounds + 1):
        hc.hc_coeffs_pre(X[0], phis[0], bias, alpha, SINKHORN_ITERS, out=(None, coef[0][1], coef[0][2], F_in[0]),
                         workspace=ws)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(layers + 1)]
        evs[0].record()
        for l in range(layers):
            cur, nxt = l % 2, (l + 1) % 2
            hc.hc_post_pre(X[cur], coef[cur][2], coef[cur][1], Fs[l % 3], phis[l + 1], bias, alpha, SINKHORN_ITERS,
                           phi_next_packed=packs[l + 1], out=X[nxt], coeffs_out=coef[nxt], F_in_out=F_in[nxt],
                           workspace=ws)
            evs[l + 1].record()
        torch.cuda.synchronize()
        if r > 0:  # the first pass warms up
            per += [evs[l].elapsed_time(evs[l + 1]) * 1e-3 for l in range(layers)]
        if layers % 2:
            X.reverse()  # the next pass starts from the last state
    t = float(np.median(per))
    nb = algorithmic_bytes(T, n, C)["hc_post_pre"]
    return {"workload": "mHC n=4 C=7168 T=16384 (batch 8 x seq 2048) bf16, 8 chained sublayers, one hc_post_pre "
                        "per layer (phi packed once per layer)",
            "per_layer_us": t * 1e6, "p10_us": float(np.percentile(per, 10)) * 1e6,
            "p90_us": float(np.percentile(per, 90)) * 1e6, "tokens_per_s_per_layer": T / t,
            "chain_us": t * layers * 1e6, "algorithmic_bytes_per_layer": nb, "achieved_GBps": nb / t / 1e9,
            "pct_hbm_peak": 100.0 * nb / t / 1e9 / HBM_PEAK_GBPS,
            "counters": counter_summary(load_counters("hc_post_pre_C7168", source_digest()), t)}


def small_latency_bench(torch, hc, dev, reps: int = 50) -> dict:
    """Latency of the smallest workload, mHC n=4 C=256 T=512 float32 (launch-bound):
    the isolated sublayer (hc_coeffs_pre + hc_post) and the chained step (hc_post_pre),
    each with HIP events around the calls (median), plus host wall time per step."""
    T, n, C = 512, 4, 256
    g = torch.Generator(device=dev)
    g.manual_seed(1000)
    X = torch.randn(T, n, C, device=dev, generator=g)
    F = torch.randn(T, C, device=dev, generator=g)
    phi = torch.randn(n * C, n * n + 2 * n, device=dev, generator=g) * 0.02
    bias = torch.zeros(n * n + 2 * n, device=dev)
    bias[2 * n:] = torch.eye(n, device=dev).flatten()
    alpha = [0.01] * 3
    ws = torch.empty(hc.hc_coeffs_workspace_bytes(T, n, C, torch.float32), dtype=torch.uint8, device=dev)
    co = (None, torch.empty(T, n, device=dev), torch.empty(T, n, n, device=dev), torch.empty(T, C, device=dev))
    co2 = (None, torch.empty(T, n, device=dev), torch.empty(T, n, n, device=dev))
    Xn = torch.empty_like(X)
    Fi = torch.empty(T, C, device=dev)

    def iso():
        hc.hc_coeffs_pre(X, phi, bias, alpha, SINKHORN_ITERS, out=co, workspace=ws)
        hc.hc_post(X, co[2], co[1], F, out=Xn)

    def chain():
        hc.hc_post_pre(X, co[2], co[1], F, phi, bias, alpha, SINKHORN_ITERS, out=Xn, coeffs_out=co2, F_in_out=Fi,
                       workspace=ws)

    out = {}
    for name, fn in (("isolated_sublayer", iso), ("chained_step", chain)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out[name] = {"gpu_median_us": float(np.median(ts)), "gpu_p90_us": float(np.percentile(ts, 90)),
                     "wall_us_per_step": (time.perf_counter() - t0) / reps * 1e6}
    out["workload"] = "mHC n=4 C=256 T=512 float32 (launch-latency bound)"
    return out


def device_copy_rate(torch, hc, dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Read + write GB/s of the library's streaming copy probe (16-byte nontemporal
    loads and stores) over three rotating buffer pairs of `nbytes`: the practical
    streaming ceiling of this device, measured on the same box."""
    src = [torch.full((nbytes // 4,), float(i), dtype=torch.float32, device=dev) for i in range(3)]
    dst = [torch.empty(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(3)]
    for i in range(3):
        hc.hc_copy_probe(src[i], dst[i])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        hc.hc_copy_probe(src[i % 3], dst[i % 3])
    b.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9


def torch_copy_rate(torch, dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Read + write GB/s of torch's own device-to-device copy of `nbytes` (three
    rotating buffer pairs) on the same box: context for the streaming rate of this
    GPU, not a ceiling (a copy kernel with nontemporal 16-byte loads and stores
    streams faster than torch's)."""
    src = [torch.full((nbytes // 4,), float(i), dtype=torch.float32, device=dev) for i in range(3)]
    dst = [torch.empty(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(3)]
    for i in range(3):
        dst[i].copy_(src[i])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        dst[i % 3].copy_(src[i % 3])
    b.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9


def load_counters(entry: str, digest: str):
    """The rocprofv3 counter figures of one entry point (profiles/traffic.json),
    or None when they were taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(entry)
    if not ent or ent.get("source_digest") != digest:
        return None
    return ent


def counter_summary(ent, launch_s: float):
    """HBM bytes by the two counter pairs and MFMA figures of one call, the rate
    of its MFMA work taken over the live duration `launch_s`."""
    if ent is None:
        return None
    return {"fetch_write_bytes": ent["bytes_per_launch"], "dram_bytes": ent["dram_bytes_per_launch"],
            "dram_read_bytes": ent["dram_read_bytes"], "dram_write_bytes": ent["dram_write_bytes"],
            "dram_over_algorithmic": ent["dram_bytes_per_launch"] / ent["algorithmic_bytes"],
            "mfma_flops": ent["mfma_flops"], "mfma_tflops": ent["mfma_flops"] / launch_s / 1e12,
            "mfma_frac_bf16_peak": ent["mfma_flops"] / launch_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "mfma_busy_frac": ent["mfma_busy_frac"], "kernels": ent["kernels"],
            "source": "profiles/traffic.json (rocprofv3 --pmc runs named there)"}


def cpu_baseline(min_seconds: float = 10.0, max_seconds: float = 30.0, single_seconds: float = 3.0) -> dict:
    """The fp64 oracle (as is) over 512-token chunks of the same workload, cycling
    through the 8192 tokens until at least `min_seconds` of work has run with the
    host's BLAS threads, then for `single_seconds` with one thread."""
    import synth
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits

    w = synth.WORKLOADS[WORKLOAD]
    T, n, C = w["T"], w["n"], w["C"]
    inp = synth.mhc_layer(w["seed"], 0, T, n, C, w["dtype"])
    Xv, Fv = inp["X"].values, inp["F_out"].values
    chunk = 512

    def run(seconds, cap):
        done, start, elapsed = 0, time.perf_counter(), 0.0
        while elapsed < seconds:
            s = done % T
            O.mhc_sublayer(Xv[s:s + chunk], inp["phi"], inp["bias"], inp["alpha"], Fv[s:s + chunk],
                           SINKHORN_ITERS)
            done += chunk
            elapsed = time.perf_counter() - start
            if elapsed > cap:
                break
        return done, elapsed

    done, elapsed = run(min_seconds, max_seconds)
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    with threadpool_limits(limits=1):
        done1, elapsed1 = run(single_seconds, 3 * single_seconds)
    return {"value": done / elapsed, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} tokens ({done // chunk} chunks of {chunk}) of the n=4 C=4096 bf16 workload, "
                      f"{elapsed:.1f} s, numpy fp64 with {threads} BLAS threads",
            "single_thread": {"value": done1 / elapsed1, "unit": "tokens/s", "cores": 1,
                              "sample": f"{done1} tokens, {elapsed1:.1f} s, one BLAS thread"}}


# The measurements besides the headline, by name (--only runs one of them alone).
SECTIONS = {
    "small_latency": lambda torch, hc, dev, args: small_latency_bench(torch, hc, dev),
    "chain_C7168": lambda torch, hc, dev, args: chain_c7168_bench(torch, hc, dev),
    "xhc": lambda torch, hc, dev, args: xhc_bench(torch, hc, dev, max(3, min(args.steps, 20)), 3),
    "hc_baseline": lambda torch, hc, dev, args: hc_baseline_bench(torch, hc, dev),
    "backward": lambda torch, hc, dev, args: backward_bench(torch, hc, dev),
    "xhc_backward": lambda torch, hc, dev, args: xhc_backward_bench(torch, hc, dev),
    "flash": lambda torch, hc, dev, args: flash_bench(torch, hc, dev),
}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-xhc", action="store_true", help="skip the xHC measurements")
    ap.add_argument("--only", choices=sorted(SECTIONS) + ["mhc"], default=None,
                    help="run one section only (for profiling one workload): mhc is the headline and its "
                         "variants; the others print their own JSON object")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sublayer is token-parallel: each GPU would run its own token shard)", file=sys.stderr)
        return 2

    import torch
    import synth
    import stream_residual_mixing_amd as hc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only is not None and args.only != "mhc":
        print(json.dumps({"section": args.only, args.only: SECTIONS[args.only](torch, hc, dev, args)}), flush=True)
        return 0
    w = synth.WORKLOADS[WORKLOAD]
    T, n, C = w["T"], w["n"], w["C"]
    inp = synth.mhc_layer(w["seed"], 0, T, n, C, w["dtype"])

    def up_bf16(t):
        return torch.from_numpy(t.bits.view(np.int16)).to(dev).view(torch.bfloat16)

    X0, F0 = up_bf16(inp["X"]), up_bf16(inp["F_out"])
    phi = torch.from_numpy(inp["phi"]).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev)
    alpha = [float(a) for a in inp["alpha"]]
    ws = torch.empty(hc.hc_coeffs_workspace_bytes(T, n, C, torch.bfloat16), dtype=torch.uint8, device=dev)
    F_in = torch.empty(T, C, dtype=torch.bfloat16, device=dev)
    ab = algorithmic_bytes(T, n, C)

    def timed(step_fn, names, steps, warmup, label):
        """Warm up, then time `steps` steps twice: once bare (events only at both
        ends, so no marker sits between kernels), once with HIP events around every
        call on the launch stream (per-call durations)."""
        for i in range(warmup):
            step_fn(i, None)
        torch.cuda.synchronize()
        e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e_start.record()
        for i in range(steps):
            step_fn(warmup + i, None)
        e_end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu = e_start.elapsed_time(e_end) * 1e-3
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            step_fn(warmup + steps + i, evs[i])
        torch.cuda.synchronize()
        kern = {nm: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e-3 for j, nm in enumerate(names)}
        dist[label] = {
            nm: {q: float(np.percentile([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs], p))
                 for q, p in (("p10_us", 10), ("median_us", 50), ("p90_us", 90))} for j, nm in enumerate(names)}
        # the median step period of the evented run: first event of step i to that
        # of step i + 1, the gaps between the steps' launches included
        period = (float(np.median([evs[i][0].elapsed_time(evs[i + 1][0]) for i in range(steps - 1)])) * 1e-3
                  if steps > 1 else gpu / steps)
        periods[label] = period
        return wall, gpu, kern

    dist = {}
    periods = {}

    Fs = [F0] + [F0.clone() for _ in range(2)]
    phi_packed = hc.hc_phi_pack(phi, n, C, torch.bfloat16)

    # --- chained sublayer, one call per step (headline)
    Xs = [X0.clone(), torch.empty_like(X0)]
    coef = [(None, torch.empty(T, n, device=dev), torch.empty(T, n, n, device=dev)) for _ in range(2)]
    F_ins = [torch.empty(T, C, dtype=torch.bfloat16, device=dev) for _ in range(2)]

    def make_chain_step(packed):
        def step(i, evs):
            cur, nxt = i % 2, (i + 1) % 2
            _, h_post, h_res = coef[cur]
            if evs is not None:
                evs[0].record()
            hc.hc_post_pre(Xs[cur], h_res, h_post, Fs[i % 3], phi, bias, alpha, SINKHORN_ITERS,
                           phi_next_packed=packed, out=Xs[nxt], coeffs_out=coef[nxt], F_in_out=F_ins[nxt],
                           workspace=ws)
            if evs is not None:
                evs[1].record()
        return step

    def chain_start():
        _, h_post, h_res, _ = hc.hc_coeffs_pre(Xs[0], phi, bias, alpha, SINKHORN_ITERS,
                                               out=(None, coef[0][1], coef[0][2], F_ins[0]), workspace=ws)

    chain_start()
    wall_pk, gpu_pk, kern_pk = timed(make_chain_step(None), ["hc_post_pre"], args.steps, args.warmup,
                                     "chain_phi_packed_each_step")

    # --- the same chain as two calls per step: pre-read, then post fused with the next coefficients
    coef2 = [(torch.empty(T, n, device=dev), torch.empty(T, n, device=dev), torch.empty(T, n, n, device=dev))
             for _ in range(2)]
    hc.hc_coeffs(Xs[0], phi, bias, alpha, SINKHORN_ITERS, out=coef2[0], workspace=ws)

    def two_call_step(i, evs):
        cur, nxt = i % 2, (i + 1) % 2
        h_pre, h_post, h_res = coef2[cur]
        if evs is not None:
            evs[0].record()
        hc.hc_pre(Xs[cur], h_pre, out=F_in)
        if evs is not None:
            evs[1].record()
        hc.hc_post_coeffs(Xs[cur], h_res, h_post, Fs[i % 3], phi, bias, alpha, SINKHORN_ITERS, out=Xs[nxt],
                          coeffs_out=coef2[nxt], workspace=ws)
        if evs is not None:
            evs[2].record()

    wall2, gpu2, kern2 = timed(two_call_step, ["hc_pre", "hc_post_coeffs"], args.steps, args.warmup,
                                "chain_two_calls")

    # --- isolated sublayer on rotated input sets
    h_post_i = torch.empty(T, n, device=dev)
    h_res_i = torch.empty(T, n, n, device=dev)
    X_next = torch.empty(T, n, C, dtype=torch.bfloat16, device=dev)
    iso_sets = [(X0, F0)] + [(X0.clone(), F0.clone()) for _ in range(2)]

    def iso_step(i, evs):
        X, F = iso_sets[i % 3]
        if evs is not None:
            evs[0].record()
        hc.hc_coeffs_pre(X, phi, bias, alpha, SINKHORN_ITERS, out=(None, h_post_i, h_res_i, F_in), workspace=ws)
        if evs is not None:
            evs[1].record()
        hc.hc_post(X, h_res_i, h_post_i, F, out=X_next)
        if evs is not None:
            evs[2].record()

    iso_wall, iso_gpu, iso_kern = timed(iso_step, ["hc_coeffs_pre", "hc_post"], args.steps, args.warmup,
                                        "isolated_sublayer")
    iso_bytes = ab["hc_coeffs_pre"] + ab["hc_post"]

    # headline last, once the clocks have settled under the variants above
    chain_start()
    wall, gpu_s, kern = timed(make_chain_step(phi_packed), ["hc_post_pre"], args.steps, args.warmup, "headline")
    step_bytes = ab["hc_post_pre"]

    # cache-cold variant of the headline call: 1 GiB of unrelated streaming (the copy
    # probe over 512 MiB, more than the memory-side cache) before every call, the call
    # timed alone by events around it
    flush = [torch.zeros(1 << 27, dtype=torch.float32, device=dev) for _ in range(2)]
    cold_step = make_chain_step(phi_packed)
    cold = []
    for i in range(args.steps + 2):
        hc.hc_copy_probe(flush[0], flush[1])
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        cold_step(i, evs)
        torch.cuda.synchronize()
        if i >= 2:
            cold.append(evs[0].elapsed_time(evs[1]) * 1e-3)
    del flush
    t_cold = float(np.median(cold))

    def rate(label, gpu_s, wall_s, nbytes):
        # The variants' rates come from the median step period of the evented run:
        # in some runs right after another GPU process, the bare run of the two-call
        # chain held one long stall in issuing (about 35 ms over 50 steps, on the
        # host's clock and the GPU's alike) that the per-step periods do not
        # show. The bare run's wall clock and GPU time per step are reported beside.
        per = periods[label]
        return {"tokens_per_s": T / per, "ms_per_step": per * 1e3, "achieved_GBps": nbytes / per / 1e9,
                "pct_hbm_peak": 100.0 * nbytes / per / 1e9 / HBM_PEAK_GBPS,
                "bare_wall_ms_per_step": wall_s / args.steps * 1e3,
                "bare_gpu_ms_per_step": gpu_s / args.steps * 1e3}

    one_pass = T * (n * C * 2 + C * 2 + n * C * 2 + C * 2 + (n + n * n) * 4 * 2)
    ms_per_step = wall / args.steps * 1e3
    tokens_per_s = T * args.steps / wall
    achieved = step_bytes / (wall / args.steps) / 1e9
    dom = "hc_post_pre"
    dom_gbps = ab[dom] / kern[dom] / 1e9
    digest = source_digest()
    cnt = load_counters(dom, digest)
    traffic = cnt["bytes_per_launch"] if cnt else None
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "mHC sublayer n=4 C=4096 T=8192 (batch 4 x seq 2048), bf16 streams, fp32 "
                               "coefficients, 20 Sinkhorn iterations, forward; steady state of a chain: post/res "
                               "write + next coefficients + next pre-read in one call per step, phi packed once",
                   "n": n, "C": C, "T": T, "sinkhorn_iters": SINKHORN_ITERS, "parallelism": "single GPU"},
        "achieved_GBps": achieved,
        "pct_hbm_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "gpu_ms_per_step": gpu_s / args.steps * 1e3,
        "roofline": {"kernel": "hc_post_pre (mhc_split_kernel<true> + finish_pre4_kernel)",
                     "bound": "hbm",
                     "achieved": dom_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dom_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": ab[dom],
                     "launch_us": kern[dom] * 1e6, "counters": counter_summary(cnt, kern[dom])},
        "headline_one_pass": {
            "bytes_per_step": one_pass, "achieved_GBps": one_pass / (wall / args.steps) / 1e9,
            "pct_hbm_peak": 100.0 * one_pass / (wall / args.steps) / 1e9 / HBM_PEAK_GBPS,
            "note": "the step's bytes counting the state X_next once (read X and F_out, write X_next and F_in, "
                    "coefficients): the pre-read of X_next, which the algorithmic count includes as the second "
                    "state read of a sublayer, left out"},
        "headline_cache_cold": {
            "call_us": t_cold * 1e6, "tokens_per_s": T / t_cold, "achieved_GBps": step_bytes / t_cold / 1e9,
            "pct_hbm_peak": 100.0 * step_bytes / t_cold / 1e9 / HBM_PEAK_GBPS,
            "note": "hc_post_pre timed alone after 1 GiB of unrelated streaming (hc_copy_probe over 512 MiB) before "
                    "every call, so nothing of its inputs is left in the caches when it starts"},
        "chain_phi_packed_each_step": dict(rate("chain_phi_packed_each_step", gpu_pk, wall_pk, step_bytes),
                                           call_us=dist["chain_phi_packed_each_step"][dom]["median_us"]),
        "chain_two_calls": dict(rate("chain_two_calls", gpu2, wall2, ab["hc_pre"] + ab["hc_post_coeffs"]),
                                calls_us={k: v * 1e6 for k, v in kern2.items()},
                                calls_GBps={k: ab[k] / v / 1e9 for k, v in kern2.items()}),
        "isolated_sublayer": dict(rate("isolated_sublayer", iso_gpu, iso_wall, iso_bytes), calls_us={k: v * 1e6 for k, v in iso_kern.items()},
                                  algorithmic_bytes_per_step=iso_bytes),
        "call_durations": dist,
        "device_copy_ceiling_GBps": device_copy_rate(torch, hc, dev),
        "torch_copy_GBps": torch_copy_rate(torch, dev),
        "source_digest": digest,
    }
    if args.only is None:
        for name in ("small_latency",) + (() if args.no_xhc else
                                           ("chain_C7168", "xhc", "hc_baseline", "backward", "xhc_backward", "flash")):
            result[name] = SECTIONS[name](torch, hc, dev, args)
    if not args.no_cpu_baseline and args.only is None:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
