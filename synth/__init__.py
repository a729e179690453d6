"""Seeded synthetic inputs for the hyper-connection sublayer.

This module only draws random numbers and rounds them to the stream dtype. It
holds none of the method's arithmetic, so both the fp64 oracle and the HIP path
can take their inputs from it without sharing any computation.

Recipe (one numpy PCG64 generator per (seed, layer), entropy 1000*seed +
layer; draws are float32 standard normals scaled in float32, then rounded to the
stream dtype with round-to-nearest-even when the stream is bfloat16):

* mHC layer: X[T,n,C] ~ N(0,1), phi[nC, n*n+2n] ~ N(0, 0.02^2), F_out[T,C] ~ N(0,1),
  bias = [0]*n (pre) + [0]*n (post) + vec(I_n) (res), alpha = 0.01 for all three
  gates. Draw order: X, phi, F_out.
* xHC sublayer: X[T,N,C] ~ N(0,1), phi_pre[NC, N] ~ N(0, 0.02^2),
  w_router[NC, N-m] ~ N(0, 1/(NC)), phi_act[kC, k*K + k*k] ~ N(0, 0.02^2),
  F_out[T,C] ~ N(0,1), conv weights w_kappa[C, kappa] ~ N(0, 1/kappa) for the
  augmented (K > 1) case. b_pre = 0, b_act = [0]*(k*K) + vec(I_k), alpha = 0.01.
  Draw order: X, phi_pre, w_router, phi_act, F_out, conv weights.
* mHC upstream gradients (the backward's inputs): dX_next[T,n,C] ~ N(0,1) and
  dF_in[T,C] ~ N(0,1) in the stream dtype, from the side stream 1 of (seed,
  layer). Draw order: dX_next, dF_in.

Arrays are returned as host numpy float32 arrays whose values are exactly
representable in the stream dtype, plus (for bfloat16 streams) the raw uint16
bit patterns that are uploaded to the device.
"""
from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"

# The workloads, by shape: sizes, dtypes, and the seed their draws start from.
WORKLOADS = {
    "mhc_n4_C256_T512_f32": dict(seed=0, kind="mhc", n=4, C=256, T=512, dtype=F32, layers=1),
    "mhc_n4_C4096_T8192_bf16": dict(seed=1, kind="mhc", n=4, C=4096, T=8192, dtype=BF16, layers=1, batch=4,
                                    seq=2048),
    "mhc_n4_C7168_T16384_bf16_8layers": dict(seed=2, kind="mhc", n=4, C=7168, T=16384, dtype=BF16, layers=8,
                                             batch=8, seq=2048),
    "xhc_N16_k4_m2_C4096_T8192_bf16_K1": dict(seed=3, kind="xhc", N=16, k=4, m=2, C=4096, T=8192, dtype=BF16, K=1),
    "xhc_N16_k4_m2_C4096_T8192_bf16_K4": dict(seed=4, kind="xhc", N=16, k=4, m=2, C=4096, T=8192, dtype=BF16, K=4,
                                              batch=2, seq=4096, kappas=(4, 8, 12)),
}

PHI_STD = 0.02
ALPHA = 0.01
SINKHORN_ITERS = 20


def make_rng(seed: int, layer: int = 0, stream: int = 0) -> np.random.Generator:
    """Generator for (seed, layer); `stream` > 0 gives independent side streams."""
    return np.random.Generator(np.random.PCG64([1000 * seed + layer, stream]))


def round_to_bf16(a: np.ndarray):
    """Round float32 values to bfloat16 (nearest-even). Returns (values_f32, bits_u16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    bits = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, flat.size, step):
        u = flat[s:s + step].view(np.uint32)
        bump = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
        bits[s:s + step] = ((u + bump) >> 16).astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32).reshape(a.shape)
    return vals, bits.reshape(a.shape)


class Tensor:
    """A host tensor in its stream dtype: float32 values plus bf16 bits if any."""

    __slots__ = ("values", "bits", "dtype")

    def __init__(self, values: np.ndarray, dtype: str):
        if dtype == BF16:
            self.values, self.bits = round_to_bf16(values)
        elif dtype == F32:
            self.values, self.bits = np.ascontiguousarray(values, np.float32), None
        else:
            raise ValueError(dtype)
        self.dtype = dtype

    @property
    def shape(self):
        return self.values.shape


def normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def mhc_bias(n: int) -> np.ndarray:
    """[pre n | post n | res n*n]: pre/post logits 0, res logits vec(I_n)."""
    b = np.zeros(n * n + 2 * n, np.float32)
    b[2 * n:] = np.eye(n, dtype=np.float32).reshape(-1)
    return b


def mhc_layer(seed: int, layer: int, T: int, n: int, C: int, dtype: str,
              draw_x: bool = True) -> dict:
    """Inputs of one mHC sublayer. With draw_x=False the X draw is skipped (chains)."""
    rng = make_rng(seed, layer)
    out = {}
    if draw_x:
        out["X"] = Tensor(normal(rng, (T, n, C)), dtype)
    out["phi"] = normal(rng, (n * C, n * n + 2 * n), PHI_STD)
    out["F_out"] = Tensor(normal(rng, (T, C)), dtype)
    out["bias"] = mhc_bias(n)
    out["alpha"] = np.array([ALPHA, ALPHA, ALPHA], np.float32)
    return out


def mhc_grads(seed: int, layer: int, T: int, n: int, C: int, dtype: str) -> dict:
    """Upstream gradients of one mHC sublayer: dX_next [T, n, C] and dF_in [T, C]."""
    rng = make_rng(seed, layer, stream=1)
    return {"dX_next": Tensor(normal(rng, (T, n, C)), dtype), "dF_in": Tensor(normal(rng, (T, C)), dtype)}


def xhc_layer(seed: int, layer: int, T: int, N: int, C: int, k: int, m: int,
              K: int, dtype: str, kappas=(4, 8, 12)) -> dict:
    """Inputs of one xHC sublayer (K=1: plain write-back; K>1: augmented)."""
    rng = make_rng(seed, layer)
    out = {}
    out["X"] = Tensor(normal(rng, (T, N, C)), dtype)
    out["phi_pre"] = normal(rng, (N * C, N), PHI_STD)
    out["w_router"] = normal(rng, (N * C, N - m), float(np.sqrt(1.0 / (N * C))))
    out["phi_act"] = normal(rng, (k * C, k * K + k * k), PHI_STD)
    out["F_out"] = Tensor(normal(rng, (T, C)), dtype)
    if K > 1:
        assert len(kappas) == K - 1
        out["conv_w"] = [normal(rng, (C, kap), float(np.sqrt(1.0 / kap))) for kap in kappas]
        out["kappas"] = tuple(int(x) for x in kappas)
    out["b_pre"] = np.zeros(N, np.float32)
    b_act = np.zeros(k * K + k * k, np.float32)
    b_act[k * K:] = np.eye(k, dtype=np.float32).reshape(-1)
    out["b_act"] = b_act
    out["alpha_pre"] = ALPHA
    out["alpha_post"] = ALPHA
    out["alpha_res"] = ALPHA
    return out


def redraw_rows(rng: np.random.Generator, X: Tensor, tokens: np.ndarray) -> None:
    """Replace the state of the given tokens with fresh N(0,1) draws (in place)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size == 0:
        return
    fresh = Tensor(normal(rng, (tokens.size,) + X.values.shape[1:]), X.dtype)
    X.values[tokens] = fresh.values
    if X.bits is not None:
        X.bits[tokens] = fresh.bits
