"""Shared helpers of the GPU parity tests: upload synth tensors, compare to the oracle."""
from __future__ import annotations

import sys

import numpy as np

import synth


def have_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash log still says which."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def dev(x, device="cuda"):
    """A synth.Tensor or float32 numpy array as a device tensor in its dtype."""
    import torch
    if isinstance(x, synth.Tensor):
        if x.dtype == synth.BF16:
            return torch.from_numpy(np.ascontiguousarray(x.bits).view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x.values)).to(device)
    a = np.asarray(x)
    if a.dtype == np.int64 or a.dtype == np.int32:
        return torch.from_numpy(a.astype(np.int32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def bf16_ulp(v) -> np.ndarray:
    """Spacing of bfloat16 numbers at |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, np.float64))
    a = np.where(a < 2.0 ** -126, 2.0 ** -126, a)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


FP32_REL_L2 = 1e-5
BF16_REL_L2 = 1e-2
BF16_MAX_ABS = 2e-2


def check_fp32(name, got, ref, tol=FP32_REL_L2):
    e = rel_l2(got, ref)
    assert e <= tol, f"{name}: relative L2 {e:.3e} > {tol:.1e}"
    return e


def check_bf16(name, got, ref, literal_max_abs=False, literal_below=None):
    """bf16 stream outputs: rel-L2 <= 1e-2 and |err| <= max(2e-2, one bf16 ulp of the
    oracle value) per element; with literal_max_abs the plain 2e-2 bound must hold on
    every element, with literal_below=v on the elements whose oracle value is below v
    in magnitude (at 8 and above one RNE step of the stored value is 0.031)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    e = rel_l2(got, ref)
    assert e <= BF16_REL_L2, f"{name}: relative L2 {e:.3e} > {BF16_REL_L2}"
    err = np.abs(got - ref)
    bound = np.maximum(BF16_MAX_ABS, bf16_ulp(ref))
    bad = int(np.sum(err > bound))
    assert bad == 0, f"{name}: {bad} elements exceed max(2e-2, 1 ulp); worst {err.max():.3e}"
    if literal_max_abs:
        assert err.max() <= BF16_MAX_ABS, f"{name}: max abs error {err.max():.3e} > 2e-2"
    if literal_below is not None:
        small = np.abs(ref) < literal_below
        if small.any():
            w = float(err[small].max())
            assert w <= BF16_MAX_ABS, f"{name}: max abs error {w:.3e} > 2e-2 where |value| < {literal_below}"
    return e, float(err.max())


def check_stream(name, dtype, got, ref, literal_max_abs=False):
    if dtype == synth.F32:
        return check_fp32(name, got, ref)
    return check_bf16(name, got, ref, literal_max_abs)
