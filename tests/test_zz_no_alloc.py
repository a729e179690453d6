"""hc_post_pre_noalloc (the entry point for callers that cannot allocate: its
workspace is the library's fixed per-GPU scratch) against hc_post_pre with a
caller workspace, through the C ABI: the same kernels run, so every output must
be identical bit for bit; two calls in a row, the second on a smaller input, so
the scratch's leftovers from the first call cannot leak into the second; and the
sizes beyond the scratch are rejected before any work."""
import numpy as np
import pytest

import synth
from hc_testutil import dev, have_gpu, note

pytestmark = pytest.mark.gpu

if have_gpu():
    import torch
    import stream_residual_mixing_amd as hc


def _case(T, C, seed, packed):
    inp = synth.mhc_layer(seed, 0, T, 4, C, synth.BF16)
    nxt = synth.mhc_layer(seed, 1, T, 4, C, synth.BF16, draw_x=False)
    X = dev(inp["X"])
    _, h_post, h_res = hc.hc_coeffs(X, dev(inp["phi"]), dev(inp["bias"]), [0.01] * 3)
    phi_n, b_n = dev(nxt["phi"]), dev(nxt["bias"])
    pk = hc.hc_phi_pack(phi_n, 4, C, torch.bfloat16) if packed else None
    return X, h_res, h_post, dev(inp["F_out"]), phi_n, b_n, pk


def _outputs(T, C, dev_):
    return (torch.full((T, 4, C), float("nan"), dtype=torch.bfloat16, device=dev_),
            (torch.full((T, 4), float("nan"), device=dev_), torch.full((T, 4), float("nan"), device=dev_),
             torch.full((T, 4, 4), float("nan"), device=dev_)),
            torch.full((T, C), float("nan"), dtype=torch.bfloat16, device=dev_))


def _same(a, b):
    Xa, ca, Fa = a
    Xb, cb, Fb = b
    assert torch.equal(Xa.view(torch.int16), Xb.view(torch.int16))
    assert torch.equal(Fa.view(torch.int16), Fb.view(torch.int16))
    for u, v in zip(ca, cb):
        assert torch.equal(u, v)


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_matches_post_pre_two_calls_second_smaller(packed):
    for T, C, seed in ((8192, 4096, 901), (300, 1024, 902)):
        note(f"hc_post_pre_noalloc vs hc_post_pre T={T} C={C} packed={packed}")
        X, h_res, h_post, F, phi_n, b_n, pk = _case(T, C, seed, packed)
        ref = _outputs(T, C, X.device)
        got = _outputs(T, C, X.device)
        hc.hc_post_pre(X, h_res, h_post, F, phi_n, b_n, [0.01] * 3, phi_next_packed=pk, out=ref[0],
                       coeffs_out=ref[1], F_in_out=ref[2])
        hc.hc_post_pre_noalloc(X, h_res, h_post, F, phi_n, b_n, [0.01] * 3, phi_next_packed=pk, out=got[0],
                               coeffs_out=got[1], F_in_out=got[2])
        torch.cuda.synchronize()
        _same(ref, got)


def test_noalloc_generic_shape_and_in_place():
    note("hc_post_pre_noalloc generic shape (C=40) and in place (C=256)")
    X, h_res, h_post, F, phi_n, b_n, _ = _case(37, 40, 903, False)
    ref = hc.hc_post_pre(X, h_res, h_post, F, phi_n, b_n, [0.01] * 3)
    got = hc.hc_post_pre_noalloc(X, h_res, h_post, F, phi_n, b_n, [0.01] * 3)
    torch.cuda.synchronize()
    _same(ref, got)
    X, h_res, h_post, F, phi_n, b_n, _ = _case(50, 256, 904, False)
    X2 = X.clone()
    ref = hc.hc_post_pre(X, h_res, h_post, F, phi_n, b_n, [0.01] * 3, out=X)
    got = hc.hc_post_pre_noalloc(X2, h_res, h_post, F, phi_n, b_n, [0.01] * 3, out=X2)
    torch.cuda.synchronize()
    _same(ref, got)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    note("hc_post_pre_noalloc: a workspace larger than the scratch is rejected before any work")
    T, C = 70000, 4096  # hc_coeffs_workspace_bytes > 32 MiB
    assert hc.hc_coeffs_workspace_bytes(T, 4, C, torch.bfloat16) > hc.HC_NOALLOC_SCRATCH_BYTES
    L = hc.lib()
    fake = 0x10000  # never dereferenced: the size check comes first
    st = L.hc_post_pre_noalloc(fake, 1, T, 4, C, fake, fake, fake, fake, fake, None, fake, 0.01, 0.01, 0.01, 20,
                               None, fake, fake, fake, None)
    assert st == -9 and "scratch" in hc.status_string(st)
