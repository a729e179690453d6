"""CPU tests of the C-ABI boundary: libhc.so loads, exports every symbol that
include/hc.h declares, and rejects bad arguments on the host before any device
work (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from hc_testutil import have_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def hc():
    import stream_residual_mixing_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libhc.so is not built (run __graft_entry__.build())")
    return m


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ("hc_coeffs", "hc_pre", "hc_coeffs_pre", "hc_post", "hc_post_coeffs", "hc_post_pre",
                 "hc_phi_pack", "hc_phi_packed_bytes", "xhc_pre", "xhc_route", "xhc_augment",
                 "xhc_pre_chain", "xhc_route_pre", "xhc_chain_carry_bytes", "xhc_chain_workspace_bytes",
                 "hc_status_string"):
        assert want in names


def test_library_exports_every_declared_symbol(hc):
    raw = ctypes.CDLL(hc.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(raw, n)]
    assert not missing, missing


def test_binding_names_match_c_entry_points(hc):
    for n in _declared_functions():
        if n in ("hc_status_string", "hc_version"):
            continue
        assert hasattr(hc, n), n


def test_status_strings(hc):
    L = hc.lib()
    for code in range(0, -10, -1):
        assert L.hc_status_string(code)
    assert L.hc_version() >= 100


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


def test_validation_rejects_bad_arguments_before_device_work(hc):
    L = hc.lib()
    ws = hc.lib().hc_coeffs_workspace_bytes(8, 4, 64, 1)
    assert ws > 0
    args = lambda **kw: dict(dict(X=FAKE, dt=1, T=8, n=4, C=64), **kw)

    def coeffs(X=FAKE, dt=1, T=8, n=4, C=64, phi=FAKE, bias=FAKE, iters=20, hpre=FAKE,
               wsp=ctypes.c_void_p(0x20000), wsb=ws):
        return L.hc_coeffs(X, dt, T, n, C, phi, bias, 0.01, 0.01, 0.01, iters, hpre,
                           ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000), wsp, wsb, None)

    assert coeffs(dt=7) == -3
    assert coeffs(n=0) == -2
    assert coeffs(n=17) == -2
    assert coeffs(C=0) == -2
    assert coeffs(T=-1) == -2
    assert coeffs(iters=0) == -2
    assert coeffs(X=None) == -1
    assert coeffs(phi=None) == -1
    assert coeffs(hpre=None) == -1
    assert coeffs(X=ctypes.c_void_p(0x10001)) == -4
    assert coeffs(wsb=ws - 1) == -8
    assert coeffs(wsp=ctypes.c_void_p(0x20010)) == -8
    # overlapping output and input
    assert coeffs(hpre=ctypes.c_void_p(0x10000)) == -5
    # empty input is valid and does nothing
    assert coeffs(T=0, X=None, phi=None, hpre=None, wsp=None, wsb=0) == 0

    post = lambda X=FAKE, Y=ctypes.c_void_p(0x90000), F=ctypes.c_void_p(0x50000): L.hc_post(
        X, 1, 8, 4, 64, ctypes.c_void_p(0x60000), ctypes.c_void_p(0x70000), F, Y, None)
    assert post(Y=None) == -1
    assert post(Y=ctypes.c_void_p(0x10002)) == -5       # partial overlap with X
    assert post(F=ctypes.c_void_p(0x90010)) == -5       # F_out inside X_next
    assert L.hc_pre(FAKE, 1, 8, 4, 64, FAKE, ctypes.c_void_p(0x10010), None) == -5

    # hc_post_pre: hc_post_coeffs' checks plus F_in_next
    def post_pre(Fin=ctypes.c_void_p(0xA0000), Y=ctypes.c_void_p(0x90000), hpre=ctypes.c_void_p(0xB0000),
                 packed=None, iters=20):
        return L.hc_post_pre(FAKE, 1, 8, 4, 64, ctypes.c_void_p(0x60000), ctypes.c_void_p(0x70000),
                             ctypes.c_void_p(0x50000), Y, ctypes.c_void_p(0xC0000), packed,
                             ctypes.c_void_p(0xD0000), 0.01, 0.01, 0.01, iters, hpre, ctypes.c_void_p(0xB1000),
                             ctypes.c_void_p(0xB2000), Fin, ctypes.c_void_p(0x100000), ws, None)
    assert post_pre(Fin=None) == -1
    assert post_pre(iters=0) == -2
    assert post_pre(Fin=ctypes.c_void_p(0xA0001)) == -4   # misaligned for bf16
    assert post_pre(Fin=ctypes.c_void_p(0x90010)) == -5   # F_in_next inside X_next
    assert post_pre(Fin=ctypes.c_void_p(0x10020)) == -5   # F_in_next inside X
    assert post_pre(Y=ctypes.c_void_p(0x10002)) == -5     # X_next partially over X
    assert post_pre(packed=ctypes.c_void_p(0x90100)) == -5  # packed phi inside X_next
    assert post_pre(packed=ctypes.c_void_p(0xE0008)) == -4  # packed phi not 16-byte aligned
    # hc_phi_pack: packed form exists for n = 4 bf16 with C % 32 == 0 only
    assert L.hc_phi_packed_bytes(4, 64, 1) == 4 * 64 // 8 * 48 * 16
    assert L.hc_phi_packed_bytes(4, 40, 1) == 0
    assert L.hc_phi_packed_bytes(4, 64, 0) == 0
    assert L.hc_phi_packed_bytes(0, 64, 1) == -1
    assert L.hc_phi_pack(FAKE, 4, 40, 1, None, 0, None) == 0  # nothing to pack
    assert L.hc_phi_pack(None, 4, 64, 1, ctypes.c_void_p(0x200000), 1 << 20, None) == -1
    assert L.hc_phi_pack(FAKE, 4, 64, 1, ctypes.c_void_p(0x200010), 1 << 20, None) == -4
    assert L.hc_phi_pack(FAKE, 4, 64, 1, ctypes.c_void_p(0x200000), 100, None) == -2
    assert L.hc_phi_pack(FAKE, 4, 64, 1, ctypes.c_void_p(0x10000), 1 << 20, None) == -5
    assert L.hc_phi_pack(FAKE, 4, 64, 9, ctypes.c_void_p(0x200000), 1 << 20, None) == -3

    # xHC shape rules: 1 <= m <= k <= N, k <= 16, K <= 8
    def xpre(N=16, k=4, m=2):
        return L.xhc_pre(FAKE, 1, 8, N, 64, k, m, FAKE, FAKE, 0.01, None, None,
                         ctypes.c_void_p(0x80000), None, None, ctypes.c_void_p(0x100000), 1 << 20, None)
    assert xpre(m=0) == -2
    assert xpre(k=1, m=2) == -2
    assert xpre(N=3, k=4) == -2
    assert xpre(N=65) == -2
    assert xpre(N=32, k=17) == -2

    def xroute(K=1, idx=FAKE, w=None):
        return L.xhc_route(ctypes.c_void_p(0x200000), 1, 8, 16, 64, 4, 2, w, idx, FAKE, FAKE, 0.01, 0.01,
                           20, ctypes.c_void_p(0x300000), K, ctypes.c_void_p(0x400000), None, None, None,
                           ctypes.c_void_p(0x500000), 1 << 20, None)
    assert xroute(K=0) == -2
    assert xroute(K=9) == -2
    assert xroute(idx=None, w=None) == -1

    karr = (ctypes.c_int * 3)(4, 8, 40)
    aug = lambda karr, r, dt=1, ws=ctypes.c_void_p(0x700000), wsb=1 << 20: L.xhc_augment(
        FAKE, dt, 2, 16, 64, FAKE, karr, r, ctypes.c_void_p(0x600000), 1, ws, wsb, None)
    assert aug(karr, 3) == -2
    karr = (ctypes.c_int * 3)(4, 8, 12)
    assert aug(karr, 8) == -2
    assert aug(karr, 3, dt=5) == -3
    # kappa = {4, 8, 12} takes a workspace of per-token Gram matrices
    wsa = L.xhc_augment_workspace_bytes(2, 16, 64, karr, 3, 1, 1)
    assert wsa == 2 * 16 * 1 * 10 * 4
    assert aug(karr, 3, ws=None, wsb=0) == -8
    assert aug(karr, 3, wsb=wsa - 1) == -8
    assert aug(karr, 3, ws=ctypes.c_void_p(0x600100)) == -5  # workspace inside V
    assert L.xhc_augment_workspace_bytes(2, 16, 64, karr, 2, 1, 1) == 0
    assert L.xhc_augment_workspace_bytes(2, 16, 64, karr, 3, 9, 1) == -1


def test_hc_tanh_and_gain_validation(hc):
    L = hc.lib()
    A, B, Cc = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    o1, o2, o3 = ctypes.c_void_p(0x400000), ctypes.c_void_p(0x410000), ctypes.c_void_p(0x420000)

    def tanh(X=A, dt=1, T=8, n=4, C=64, th=B, b=Cc, p=o1, q=o2, r=o3):
        return L.hc_tanh_coeffs(X, dt, T, n, C, th, b, 0.1, 0.1, 0.1, p, q, r, None)
    assert tanh(dt=7) == -3
    assert tanh(n=0) == -2 and tanh(n=17) == -2 and tanh(C=0) == -2 and tanh(T=-1) == -2
    assert tanh(T=0, X=None, th=None) == 0
    assert tanh(th=None) == -1 and tanh(r=None) == -1
    assert tanh(p=ctypes.c_void_p(0x400002)) == -4
    assert tanh(q=ctypes.c_void_p(0x400010)) == -5  # h_post inside h_pre
    assert tanh(p=ctypes.c_void_p(0x100010)) == -5  # h_pre inside X

    def gain(H=A, Ln=3, T=8, n=4, f=o1, g=o2):
        return L.hc_amax_gain(H, Ln, T, n, f, g, None)
    assert gain(n=0) == -2 and gain(n=17) == -2 and gain(Ln=-1) == -2 and gain(T=-1) == -2
    assert gain(T=0, H=None, f=None, g=None) == 0
    assert gain(H=None) == -1 and gain(f=None) == -1
    assert gain(g=ctypes.c_void_p(0x410002)) == -4
    assert gain(g=ctypes.c_void_p(0x400010)) == -5
    assert gain(f=ctypes.c_void_p(0x100010)) == -5


def test_static_mhc_validation(hc):
    L = hc.lib()
    z, a, b, c = (ctypes.c_void_p(v) for v in (0x100000, 0x200000, 0x210000, 0x220000))
    assert L.hc_static_maps(z, 0, 20, a, b, c, None) == -2
    assert L.hc_static_maps(z, 4, 0, a, b, c, None) == -2
    assert L.hc_static_maps(None, 4, 20, a, b, c, None) == -1
    assert L.hc_static_maps(z, 4, 20, ctypes.c_void_p(0x200002), b, c, None) == -4
    assert L.hc_static_maps(z, 4, 20, a, ctypes.c_void_p(0x200008), c, None) == -5
    assert L.hc_static_maps(z, 4, 20, ctypes.c_void_p(0x100010), b, c, None) == -5
    X, F, Y = ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), ctypes.c_void_p(0x3000000)
    assert L.hc_static_pre(X, 5, 8, 4, 64, a, F, None) == -3
    assert L.hc_static_pre(X, 1, 8, 4, 64, None, F, None) == -1
    assert L.hc_static_pre(X, 1, 8, 4, 64, a, ctypes.c_void_p(0x1000010), None) == -5
    assert L.hc_static_pre(X, 1, 0, 4, 64, None, None, None) == 0
    assert L.hc_static_post(X, 1, 8, 4, 64, a, b, F, ctypes.c_void_p(0x1000010), None) == -5
    assert L.hc_static_post(X, 1, 8, 4, 64, a, b, None, Y, None) == -1
    assert L.hc_static_post(X, 1, 8, 4, 64, a, b, F, ctypes.c_void_p(0x3000001), None) == -4


def test_copy_probe_validation(hc):
    L = hc.lib()
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert L.hc_copy_probe(a, b, 0, None) == 0
    assert L.hc_copy_probe(None, None, 0, None) == 0
    assert L.hc_copy_probe(a, b, -16, None) == -2
    assert L.hc_copy_probe(None, b, 64, None) == -1
    assert L.hc_copy_probe(a, b, 24, None) == -4
    assert L.hc_copy_probe(ctypes.c_void_p(0x100008), b, 64, None) == -4
    assert L.hc_copy_probe(a, ctypes.c_void_p(0x100010), 64, None) == -5


@pytest.mark.skipif(have_gpu(), reason="checks the no-device status; on a GPU box the call would run")
def test_valid_call_without_device_reports_device_error(hc):
    L = hc.lib()
    ws = L.hc_coeffs_workspace_bytes(8, 4, 64, 1)
    s = L.hc_coeffs(FAKE, 1, 8, 4, 64, ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), 0.01, 0.01,
                    0.01, 20, ctypes.c_void_p(0x300000), ctypes.c_void_p(0x310000),
                    ctypes.c_void_p(0x320000), ctypes.c_void_p(0x400000), ws, None)
    assert s == -6


def test_workspace_queries(hc):
    L = hc.lib()
    assert L.hc_coeffs_workspace_bytes(0, 4, 64, 1) >= 0
    assert L.hc_coeffs_workspace_bytes(8, 0, 64, 1) == -1
    assert L.xhc_pre_workspace_bytes(8, 16, 64, 2, 1, 1) > L.xhc_pre_workspace_bytes(8, 16, 64, 2, 0, 1)
    assert L.xhc_route_workspace_bytes(8, 16, 64, 4, 2, 4, 1, 1) > 0
    assert L.xhc_route_workspace_bytes(8, 16, 64, 4, 2, 9, 1, 1) == -1


def test_backward_validation(hc):
    L = hc.lib()
    T, C = 8, 64
    wsb = L.hc_backward_workspace_bytes(T, 4, C, 1)
    assert wsb > 0
    assert L.hc_backward_workspace_bytes(0, 4, C, 1) == 0
    assert L.hc_backward_workspace_bytes(T, 3, C, 1) == -1
    assert L.hc_backward_workspace_bytes(T, 4, 48, 1) == -1
    assert L.hc_backward_workspace_bytes(T, 4, C, 0) == -1
    assert L.hc_backward_workspace_bytes(-1, 4, C, 1) == -1
    P = lambda k: ctypes.c_void_p(0x1000000 * (k + 1))  # distinct, far apart, 256-byte aligned

    names = ["X", "phi", "bias", "dXn", "dFi", "dh", "dX", "dphi", "dbias", "dalpha", "ws"]

    def bwd(dt=1, T=T, n=4, C=C, iters=20, wsb=wsb, **kw):
        p = {nm: kw.get(nm, P(k)) for k, nm in enumerate(names)}
        return L.hc_backward(p["X"], dt, T, n, C, p["phi"], p["bias"], 0.01, 0.01, 0.01, iters, p["dXn"], p["dFi"],
                             p["dh"], p["dX"], p["dphi"], p["dbias"], p["dalpha"], p["ws"], wsb, None)
    assert bwd(dt=7) == -3 and bwd(dt=0) == -3
    assert bwd(n=3) == -2 and bwd(C=48) == -2 and bwd(C=0) == -2 and bwd(T=-1) == -2
    assert bwd(iters=0) == -2 and bwd(iters=65) == -2
    assert bwd(T=0, X=None, dX=None) == 0
    for nm in names[:-1]:
        assert bwd(**{nm: None}) == -1, nm
    assert bwd(X=ctypes.c_void_p(0x1000008)) == -4
    assert bwd(dX=ctypes.c_void_p(0x7000004)) == -4
    assert bwd(dphi=ctypes.c_void_p(0x8000002)) == -4
    assert bwd(ws=None) == -8 and bwd(wsb=wsb - 1) == -8 and bwd(ws=ctypes.c_void_p(0xb000010)) == -8
    assert bwd(dX=ctypes.c_void_p(0x4000000)) == -5  # dX over dX_next
    assert bwd(dh=ctypes.c_void_p(0x1000000)) == -5  # dh over X
    assert bwd(dbias=ctypes.c_void_p(0x8000010)) == -5  # dbias inside dphi
    assert bwd(ws=ctypes.c_void_p(0x7000000)) == -5  # workspace over dX

    pn = ["X", "hp", "Fo", "dXn", "dFo", "dh"]

    def post(dt=1, T=T, n=4, C=C, **kw):
        p = {nm: kw.get(nm, P(k)) for k, nm in enumerate(pn)}
        return L.hc_backward_post(p["X"], dt, T, n, C, p["hp"], p["Fo"], p["dXn"], p["dFo"], p["dh"], None)
    assert post(dt=0) == -3 and post(n=2) == -2 and post(C=40) == -2 and post(T=-2) == -2
    assert post(T=0, X=None) == 0
    for nm in pn:
        assert post(**{nm: None}) == -1, nm
    assert post(hp=ctypes.c_void_p(0x2000004)) == -4  # h_post is read 16 bytes at a time
    assert post(dh=ctypes.c_void_p(0x6000002)) == -4
    assert post(dFo=ctypes.c_void_p(0x3000000)) == -5  # dF_out over F_out
    assert post(dh=ctypes.c_void_p(0x5000010)) == -5  # dh inside dF_out


def test_xhc_backward_validation(hc):
    L = hc.lib()
    T, N, C = 8, 16, 64
    wsb = L.xhc_backward_workspace_bytes(T, N, C, 4, 1, 1)
    assert wsb > 0
    assert L.xhc_backward_workspace_bytes(0, N, C, 4, 1, 1) == 0
    assert L.xhc_backward_workspace_bytes(T, 6, C, 4, 1, 1) == -1
    assert L.xhc_backward_workspace_bytes(T, N, C, 3, 1, 1) == -1
    assert L.xhc_backward_workspace_bytes(T, N, C, 4, 2, 1) == -1
    assert L.xhc_backward_workspace_bytes(T, N, 40, 4, 1, 1) == -1
    assert L.xhc_backward_workspace_bytes(T, N, C, 4, 1, 0) == -1
    P = lambda k: ctypes.c_void_p(0x1000000 * (k + 1))  # distinct, far apart, 256-byte aligned
    rn = ["X", "idx", "phi", "b", "Wb", "dX", "dWb", "dphi", "db", "da", "dh", "ws"]

    def route(dt=1, T=T, N=N, C=C, k=4, K=1, iters=20, wsb=wsb, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(rn)}
        return L.xhc_route_backward(p["X"], dt, T, N, C, k, p["idx"], p["phi"], p["b"], 0.01, 0.01, iters, p["Wb"],
                                    K, p["dX"], p["dWb"], p["dphi"], p["db"], p["da"], p["dh"], p["ws"], wsb, None)
    assert route(dt=0) == -3 and route(dt=5) == -3
    assert route(N=6) == -2 and route(N=20) == -2 and route(k=3) == -2 and route(K=2) == -2 and route(C=48) == -2
    assert route(iters=0) == -2 and route(iters=65) == -2 and route(T=-1) == -2
    assert route(T=0, X=None) == 0
    for nm in rn[:-1]:
        assert route(**{nm: None}) == -1, nm
    assert route(idx=ctypes.c_void_p(0x2000004)) == -4  # idx is read 16 bytes per token
    assert route(dX=ctypes.c_void_p(0x6000008)) == -4
    assert route(ws=None) == -8 and route(wsb=wsb - 1) == -8
    assert route(dX=ctypes.c_void_p(0x1000000)) == -5  # dX over X
    assert route(dh=ctypes.c_void_p(0x6000100)) == -5  # dh inside dX
    assert route(dWb=ctypes.c_void_p(0x5000000)) == -5  # dF_out over F_out

    pn = ["X", "phi", "b", "dFi", "dX", "dphi", "db", "da", "dh", "ws"]

    def pre(dt=1, T=T, N=N, C=C, wsb=wsb, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(pn)}
        return L.xhc_pre_backward(p["X"], dt, T, N, C, p["phi"], p["b"], 0.01, p["dFi"], p["dX"], p["dphi"], p["db"],
                                  p["da"], p["dh"], p["ws"], wsb, None)
    assert pre(dt=0) == -3 and pre(N=2) == -2 and pre(C=40) == -2 and pre(T=-3) == -2
    assert pre(T=0, X=None) == 0
    for nm in pn[:-1]:
        assert pre(**{nm: None}) == -1, nm
    assert pre(dh=ctypes.c_void_p(0x9000004)) == -4
    assert pre(ws=None) == -8
    assert pre(dX=ctypes.c_void_p(0x4000000)) == -5  # dX over dF_in
    assert pre(dphi=ctypes.c_void_p(0x5000040)) == -5  # dphi inside dX


def test_xhc_chain_validation(hc):
    """xhc_pre_chain / xhc_route_pre: the covered shapes, required pointers, alignment,
    workspace and overlap rules, all rejected before any device work."""
    L = hc.lib()
    T, N, C = 8, 16, 512
    cb = L.xhc_chain_carry_bytes(T, N, C, 4, 2, 1)
    wsb = L.xhc_chain_workspace_bytes(T, N, C, 4, 2, 1, 1)
    assert cb > 0 and wsb > 0
    assert L.xhc_chain_carry_bytes(T, 8, C, 4, 2, 1) == -1       # N = 16 only
    assert L.xhc_chain_carry_bytes(T, N, 256, 4, 2, 1) == -1     # C % 512
    assert L.xhc_chain_carry_bytes(T, N, C, 3, 2, 1) == -1       # k = 4
    assert L.xhc_chain_carry_bytes(T, N, C, 4, 5, 1) == -1       # m <= k
    assert L.xhc_chain_carry_bytes(T, N, C, 4, 2, 0) == -1       # bfloat16
    assert L.xhc_chain_workspace_bytes(T, N, C, 4, 2, 9, 1) == -1
    P = lambda j: ctypes.c_void_p(0x1000000 * (j + 1))  # distinct, far apart, 256-byte aligned
    pn = ["X", "phi", "b", "w", "phin", "wn", "hp", "Fin", "idx", "sc", "carry", "ws"]

    def pre(dt=1, T=T, N=N, C=C, k=4, m=2, wsb=wsb, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(pn)}
        return L.xhc_pre_chain(p["X"], dt, T, N, C, k, m, p["phi"], p["b"], 0.01, p["w"], p["phin"], p["wn"], p["hp"],
                               p["Fin"], p["idx"], p["sc"], p["carry"], p["ws"], wsb, None)
    assert pre(dt=0) == -3 and pre(dt=7) == -3
    assert pre(N=8) == -2 and pre(C=1000) == -2 and pre(k=2) == -2 and pre(T=-1) == -2
    assert pre(T=0, X=None) == 0
    for nm in ["X", "phi", "b", "w", "phin", "wn", "Fin", "idx", "carry"]:
        assert pre(**{nm: None}) == -1, nm
    assert pre(idx=ctypes.c_void_p(0x9000004)) == -4    # idx rows are read 16 bytes at a time
    assert pre(carry=ctypes.c_void_p(0xB000010)) == -4  # the carry is 256-byte aligned
    assert pre(hp=ctypes.c_void_p(0x7000008)) == -4
    assert pre(ws=None) == -8 and pre(wsb=wsb - 1) == -8
    assert pre(Fin=ctypes.c_void_p(0x1000000)) == -5    # F_in over X
    assert pre(carry=ctypes.c_void_p(0xC000000 - 256)) == -5  # carry runs into the workspace

    rn = ["X", "idx", "pa", "ba", "Wb", "phi", "b", "w", "cin", "phin", "wn", "cout", "hpo", "hro", "idxo", "sc",
          "hp", "Fin", "ws"]

    def route(dt=1, T=T, N=N, C=C, k=4, m=2, K=1, iters=20, wsb=wsb, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(rn)}
        return L.xhc_route_pre(p["X"], dt, T, N, C, k, m, p["idx"], p["pa"], p["ba"], 0.01, 0.01, iters, p["Wb"], K,
                               p["b"], 0.01, p["cin"], p["phin"], p["wn"], p["cout"], p["hpo"],
                               p["hro"], p["idxo"], p["sc"], p["hp"], p["Fin"], p["ws"], wsb, None)
    assert route(dt=0) == -3
    assert route(N=12) == -2 and route(C=768) == -2 and route(K=0) == -2 and route(K=9) == -2
    assert route(iters=0) == -2 and route(T=-2) == -2
    assert route(T=0, X=None) == 0
    for nm in ["X", "idx", "pa", "ba", "Wb", "b", "cin", "idxo", "Fin"]:
        assert route(**{nm: None}) == -1, nm
    # the next sublayer's maps and carry_out go together
    assert route(cout=None) == -1 and route(phin=None) == -1
    assert route(idx=ctypes.c_void_p(0x2000008)) == -4
    assert route(idxo=ctypes.c_void_p(0xF000004)) == -4
    assert route(cin=ctypes.c_void_p(0x9000080)) == -4
    assert route(ws=None) == -8 and route(wsb=wsb - 1) == -8
    assert route(Fin=ctypes.c_void_p(0x1000000)) == -5          # F_in over X
    assert route(cout=ctypes.c_void_p(0x9000000 + 256)) == -5   # carry_out partly over carry_in
    assert route(hp=ctypes.c_void_p(0x13000000 - 256)) == -5    # h_pre runs into the workspace


def test_augment_backward_validation(hc):
    L = hc.lib()
    B, S, C = 2, 16, 64
    k = (ctypes.c_int * 3)(4, 8, 12)
    kbad = (ctypes.c_int * 3)(4, 8, 10)
    wsb = L.xhc_augment_backward_workspace_bytes(B, S, C, k, 3, 1)
    assert wsb > 0
    assert L.xhc_augment_backward_workspace_bytes(0, S, C, k, 3, 1) == 0
    assert L.xhc_augment_backward_workspace_bytes(B, S, C, kbad, 3, 1) == -1
    assert L.xhc_augment_backward_workspace_bytes(B, S, C, k, 2, 1) == -1
    P = lambda j: ctypes.c_void_p(0x1000000 * (j + 1))

    def aug(dt=1, B=B, S=S, C=C, kk=k, r=3, wsb=wsb, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(["F", "w", "dV", "dF", "dw", "ws"])}
        return L.xhc_augment_backward(p["F"], dt, B, S, C, p["w"], kk, r, p["dV"], p["dF"], p["dw"], p["ws"], wsb,
                                      None)
    assert aug(dt=4) == -3
    assert aug(r=2) == -2 and aug(kk=kbad) == -2 and aug(C=0) == -2 and aug(B=-1) == -2
    assert aug(B=0, F=None) == 0
    for nm in ("F", "w", "dV", "dF", "dw"):
        assert aug(**{nm: None}) == -1, nm
    assert aug(dF=ctypes.c_void_p(0x4000001)) == -4
    assert aug(ws=None) == -8 and aug(wsb=wsb - 1) == -8
    assert aug(dF=ctypes.c_void_p(0x1000000)) == -5  # dF_out over F_out
    assert aug(dw=ctypes.c_void_p(0x3000100)) == -5  # dconv inside dV


def test_flash_validation(hc):
    L = hc.lib()
    T, N, C, k, m, Ls = 8, 16, 64, 4, 2, 2
    assert L.xhc_flash_pre_workspace_bytes(T, N, C, m, Ls, 1) > 0
    assert L.xhc_flash_pre_workspace_bytes(T, N, C, m, 5, 1) == -1
    assert L.xhc_flash_pre_workspace_bytes(T, N, C, N, Ls, 1) == -1  # m = N leaves nothing to route
    assert L.xhc_flash_maps_workspace_bytes(T, N, C, k, 0, 1, 1) == -1
    assert L.xhc_flash_maps_workspace_bytes(T, N, C, k, Ls, 0, 1) == -1  # no component for the last sublayer
    assert L.xhc_flash_maps_workspace_bytes(T, N, C, k, 4, 6, 1) == -1  # 9 components > HC_MAX_COMPONENTS
    assert L.xhc_flash_post_workspace_bytes(T, k, Ls, 1) >= T * k * Ls * 4
    assert L.xhc_flash_post_workspace_bytes(T, k, Ls, 4) >= T * k * (Ls + 3) * 4
    assert L.xhc_flash_post_workspace_bytes(T, k, 5, 1) == -1
    P = lambda j: ctypes.c_void_p(0x1000000 * (j + 1))
    wsp = L.xhc_flash_pre_workspace_bytes(T, N, C, m, Ls, 1)

    def pre(dt=1, T=T, k=k, m=m, Lb=Ls, wsb=wsp, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(["X", "phi", "b", "w", "idx", "sc", "h", "F", "ws"])}
        return L.xhc_flash_pre(p["X"], dt, T, N, C, k, m, Lb, p["phi"], p["b"], ctypes.c_float(0.01), p["w"],
                               p["idx"], p["sc"], p["h"], p["F"], p["ws"], wsb, None)
    assert pre(dt=5) == -3
    assert pre(Lb=0) == -2 and pre(Lb=5) == -2 and pre(k=1) == -2 and pre(m=N) == -2
    assert pre(T=0, X=None) == 0
    for nm in ("X", "phi", "b", "w", "idx", "h", "F"):
        assert pre(**{nm: None}) == -1, nm
    assert pre(F=ctypes.c_void_p(0x8000001)) == -4
    assert pre(ws=None) == -8 and pre(wsb=wsp - 1) == -8
    assert pre(F=ctypes.c_void_p(0x1000000)) == -5  # F_pre over X
    assert pre(idx=ctypes.c_void_p(0x7000000)) == -5  # idx over h_pre

    wsm = L.xhc_flash_maps_workspace_bytes(T, N, C, k, Ls, 1, 1)

    def maps(Lb=Ls, Kl=1, iters=20, wsb=wsm, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(["X", "idx", "phi", "b", "Hp", "Hr", "ws"])}
        return L.xhc_flash_maps(p["X"], 1, T, N, C, k, Lb, Kl, p["idx"], p["phi"], p["b"], ctypes.c_float(0.01),
                                ctypes.c_float(0.01), iters, p["Hp"], p["Hr"], p["ws"], wsb, None)
    assert maps(Lb=5) == -2 and maps(iters=0) == -2 and maps(Kl=0) == -2 and maps(Kl=8) == -2
    for nm in ("X", "idx", "phi", "b", "Hp", "Hr"):
        assert maps(**{nm: None}) == -1, nm
    assert maps(wsb=wsm - 1) == -8
    assert maps(Hr=ctypes.c_void_p(0x5000000)) == -5  # H_res over H_post

    def inp(l=1, Lb=Ls, Kl=1, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(["Fp", "h", "idx", "Hp", "Fo", "Fi"])}
        return L.xhc_flash_input(1, T, N, C, k, Lb, Kl, l, p["Fp"], p["h"], p["idx"], p["Hp"], p["Fo"], p["Fi"],
                                 None)
    assert inp(l=2) == -2 and inp(l=-1) == -2 and inp(Lb=0) == -2 and inp(Kl=0) == -2
    assert inp(l=2, Kl=4) == -2  # l counts sublayers, not components
    for nm in ("Fp", "h", "idx", "Hp", "Fo", "Fi"):
        assert inp(**{nm: None}) == -1, nm
    assert inp(Fi=ctypes.c_void_p(0x6000001)) == -4
    assert inp(Fi=ctypes.c_void_p(0x5000000)) == -5  # F_in over F_outs

    wsq = L.xhc_flash_post_workspace_bytes(T, k, Ls, 1)

    def post(Lb=Ls, Kl=1, wsb=wsq, **kw):
        p = {nm: kw.get(nm, P(j)) for j, nm in enumerate(["X", "idx", "Hp", "Hr", "Fo", "ws"])}
        return L.xhc_flash_post(p["X"], 1, T, N, C, k, Lb, Kl, p["idx"], p["Hp"], p["Hr"], p["Fo"],
                                kw.get("Wl"), p["ws"], wsb, None)
    assert post(Lb=5) == -2 and post(Kl=0) == -2
    assert post(Kl=4) == -8  # the workspace holds T k (L - 1 + K_last) maps
    for nm in ("X", "idx", "Hp", "Hr", "Fo"):
        assert post(**{nm: None}) == -1, nm
    assert post(ws=None) == -8 and post(wsb=wsq - 1) == -8
    assert post(ws=ctypes.c_void_p(0x1000000)) == -5  # workspace inside X
    assert post(Wl=ctypes.c_void_p(0x9000001)) == -4  # W_last misaligned
    assert post(Wl=ctypes.c_void_p(0x1000000)) == -5  # W_last inside X
