"""Seeded synthetic inputs for the Sparse Delta Memory (SDM) layer forward.

This module is shared by the CPU oracle (``oracle/``) and the HIP path's tests and
benchmark. It holds no arithmetic of the method itself: it only draws random inputs with
the distributions of the five workload shapes and casts them to the dtype the device
receives. Both sides consume exactly the arrays produced here.

Workloads (a tiny case, a small layer, 1.4B- and 8B-scale layers, and a decode step):

=================  ==========================================================================
name               shape
=================  ==========================================================================
tiny_fp32          B=1 H=1 T=64, N=256 (16x16), d_k=32 d_v=32, kappa=W=R=4, fp32 everywhere
small              B=4 H=8 T=2048, N=65536 (256x256), d_k=d_v=128, kappa=W=R=16, bf16 in, fp32 table
layer_1p4b         B=8 H=16 T=4096, N=262144 (512x512), d_k=128 d_v=64, kappa=W=R=32, bf16 in + table
layer_8b_long      B=1 H=8 T=131072, N=262144, d_k=d_v=128, kappa=W=R=32, bf16, 10% repeated keys
decode             B=64 H=16 T=1, N=65536, d_k=d_v=128, kappa=W=R=16, bf16; 4096-token prefill
=================  ==========================================================================

Draw order for one workload (one ``numpy.random.default_rng(seed)``, float32 draws):
sub-keys [H,2,s,h] ~ N(0, 1/h); M0 [H,N,d_v] ~ N(0, 0.02^2); q [B,H,T,d_k] ~ N(0,1) then
L2-normalised over d_k; k likewise; v [B,H,T,d_v] ~ N(0,1); g [B,H,T] ~ N(3,1) and
alpha = sigmoid(g); beta [B,H,T] ~ U(0,1); then (layer_8b_long only) the repeated-key
positions. Every tensor is then cast to its dtype with round-to-nearest-even.

bf16 tensors are carried as ``uint16`` bit patterns; :func:`widen` turns any carried tensor
back into float32/float64 values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    B: int
    H: int
    T: int
    N: int
    d_k: int
    d_v: int
    kappa: int
    W: int
    R: int
    in_dtype: str   # "f32" | "bf16"  (q, k, v, sub-keys)
    mem_dtype: str  # "f32" | "bf16"  (M0 and the memory table)
    seed: int
    repeat_frac: float = 0.0  # fraction of key positions that repeat an earlier key
    prefill: int = 0          # prior tokens written into each sequence's table (decode)

    @property
    def s(self) -> int:
        r = math.isqrt(self.N)
        assert r * r == self.N
        return r

    @property
    def h(self) -> int:
        return self.d_k // 2

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Shape] = {
    "tiny_fp32": Shape("tiny_fp32", 1, 1, 64, 256, 32, 32, 4, 4, 4, "f32", "f32", 0),
    "small": Shape("small", 4, 8, 2048, 65536, 128, 128, 16, 16, 16, "bf16", "f32", 1),
    "layer_1p4b": Shape("layer_1p4b", 8, 16, 4096, 262144, 128, 64, 32, 32, 32, "bf16", "bf16", 2),
    "layer_8b_long": Shape("layer_8b_long", 1, 8, 131072, 262144, 128, 128, 32, 32, 32, "bf16", "bf16", 3,
                           repeat_frac=0.1),
    "decode": Shape("decode", 64, 16, 1, 65536, 128, 128, 16, 16, 16, "bf16", "bf16", 4, prefill=4096),
}

# Order used when a workload is referred to by position.
WORKLOAD_ORDER = ["tiny_fp32", "small", "layer_1p4b", "layer_8b_long", "decode"]


# ----------------------------------------------------------------------------- casting
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def widen(x: np.ndarray, dtype: str, to=np.float64) -> np.ndarray:
    """Values of a carried tensor (float32 array, or uint16 bf16 bits) as ``to``."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(to, copy=False)
    return np.asarray(x, dtype=np.float32).astype(to, copy=False)


# ----------------------------------------------------------------------------- drawing
def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _repeat_keys(rng: np.random.Generator, k: np.ndarray, frac: float) -> np.ndarray:
    """For each sequence, floor(frac*(T-1)) positions t>=1 (without replacement) copy the key
    of a uniformly chosen earlier position t' < t, in every head. Applied in increasing t,
    so a repeated position can itself be the source of a later repeat."""
    B, H, T, _ = k.shape
    nrep = int(math.floor(frac * (T - 1)))
    info = []
    for b in range(B):
        pos = np.sort(rng.choice(T - 1, size=nrep, replace=False) + 1)
        src = np.floor(rng.random(nrep) * pos).astype(np.int64)
        for t, t0 in zip(pos.tolist(), src.tolist()):
            k[b, :, t, :] = k[b, :, t0, :]
        info.append((pos, src))
    return info


def draw_params(shape: Shape, rng: np.random.Generator) -> Dict[str, np.ndarray]:
    s, h = shape.s, shape.h
    subkeys = (rng.standard_normal((shape.H, 2, s, h), dtype=np.float32) * np.float32(1.0 / math.sqrt(h)))
    M0 = rng.standard_normal((shape.H, shape.N, shape.d_v), dtype=np.float32) * np.float32(0.02)
    return {"subkeys": cast(subkeys, shape.in_dtype), "M0": cast(M0, shape.mem_dtype)}


def draw_tokens(shape: Shape, rng: np.random.Generator, B: int, T: int, repeat_frac: float = 0.0):
    H = shape.H
    q = _l2_normalise(rng.standard_normal((B, H, T, shape.d_k), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal((B, H, T, shape.d_k), dtype=np.float32))
    v = rng.standard_normal((B, H, T, shape.d_v), dtype=np.float32)
    g = rng.standard_normal((B, H, T), dtype=np.float32) + np.float32(3.0)
    alpha = _sigmoid(g)
    beta = rng.random((B, H, T), dtype=np.float32)
    rep = None
    if repeat_frac > 0:
        rep = _repeat_keys(rng, k, repeat_frac)
    out = {
        "q": cast(q, shape.in_dtype),
        "k": cast(k, shape.in_dtype),
        "v": cast(v, shape.in_dtype),
        "alpha": alpha,
        "beta": beta,
    }
    if rep is not None:
        out["repeats"] = rep
    return out


def make_inputs(shape: Shape, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All inputs of one workload: parameters (sub-keys, M0) and the token stream."""
    rng = np.random.default_rng(shape.seed if seed is None else seed)
    out = draw_params(shape, rng)
    out.update(draw_tokens(shape, rng, shape.B, shape.T, shape.repeat_frac))
    return out


def make_prefill(shape: Shape, b: int, T: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Prior tokens for sequence ``b`` of a decode workload (its own generator, seeded
    with (workload seed, b)), shaped [1, H, T, .]."""
    rng = np.random.default_rng([shape.seed, b])
    return draw_tokens(shape, rng, 1, shape.prefill if T is None else T)


def make_decode_bank(shape: Shape, n: int) -> Dict[str, np.ndarray]:
    """n successive decode tokens for every sequence of a decode workload (own generator,
    seeded with (workload seed, 2**20); the same distributions as every other token),
    shaped [n, B, H, 1, .] so that step i's tokens form one contiguous [B, H, 1, .] block."""
    rng = np.random.default_rng([shape.seed, 1 << 20])
    tk = draw_tokens(shape, rng, shape.B, n)
    return {k: np.ascontiguousarray(np.moveaxis(v, 2, 0)[:, :, :, None]) for k, v in tk.items()}


def adversarial(shape: Shape, kind: str, seed: int = 99) -> Dict[str, np.ndarray]:
    """Address-reuse stress inputs (same distributions, structured keys):

    * ``same_key``  every token of a sequence uses one key (all writes hit the same slots)
    * ``q_is_k``    q_t = k_t (each token reads the slots it just wrote)
    * ``period``    keys repeat with periods 1..40 tokens (reuse at every window distance)
    """
    out = make_inputs(shape, seed=seed)
    k = widen(out["k"], shape.in_dtype, np.float32).copy()
    q = widen(out["q"], shape.in_dtype, np.float32).copy()
    T = shape.T
    if kind == "same_key":
        k[:, :, :, :] = k[:, :, :1, :]
    elif kind == "q_is_k":
        q = k.copy()
    elif kind == "period":
        rng = np.random.default_rng(seed + 1)
        t = 0
        while t < T:
            p = int(rng.integers(1, 41))
            src = max(0, t - p)
            k[:, :, t, :] = k[:, :, src, :]
            if rng.random() < 0.5:
                q[:, :, t, :] = k[:, :, max(0, t - int(rng.integers(0, 41))), :]
            t += 1
    else:
        raise ValueError(kind)
    out["k"] = cast(k, shape.in_dtype)
    out["q"] = cast(q, shape.in_dtype)
    return out


def make_epilogue_inputs(shape: Shape, d_model: int, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Synthetic inputs of the steps around the recurrence, from their own generator
    (seeded with (workload seed, 7)): gate pre-activations a, b [B,H,T] ~ N(0, 1); per-head
    A_log ~ U(log 1, log 16) and dt_bias ~ N(-2, 0.5) (the ranges of Gated DeltaNet's
    initialisation); output gate pre-activation z [B,T,H,d_v] ~ N(0, 1) in the input dtype;
    norm weight w [d_v] ~ 1 + N(0, 0.1^2); head mixing weight Wo [d_model, H*d_v] ~
    N(0, 1/(H*d_v)) in bf16 (uint16 bits)."""
    rng = np.random.default_rng([shape.seed if seed is None else seed, 7])
    B, H, T, dv = shape.B, shape.H, shape.T, shape.d_v
    out = {
        "a": rng.standard_normal((B, H, T), dtype=np.float32),
        "b": rng.standard_normal((B, H, T), dtype=np.float32),
        "A_log": np.log(rng.uniform(1.0, 16.0, H)).astype(np.float32),
        "dt_bias": (rng.standard_normal(H) * 0.5 - 2.0).astype(np.float32),
        "w": (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32),
    }
    out["z"] = cast(rng.standard_normal((B, T, H, dv), dtype=np.float32), shape.in_dtype)
    out["Wo"] = cast((rng.standard_normal((d_model, H * dv)) / np.sqrt(H * dv)).astype(np.float32), "bf16")
    return out
