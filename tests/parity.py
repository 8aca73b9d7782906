"""Helpers for comparing the HIP path with the CPU oracle (index-exact up to counted ties,
float outputs within a relative tolerance)."""
from __future__ import annotations

import sys

import numpy as np

import sdm_inputs as SI

TIE_REL = 1e-5  # two slots whose exact scores differ by less than this (relative) are a tie


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x, y) -> float:
    """max |x - y| / max |y| over the whole tensor."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = float(np.max(np.abs(x - y))) if x.size else 0.0
    return d / max(float(np.max(np.abs(y))) if y.size else 0.0, 1e-30)


# ----------------------------------------------------------------------------- torch glue
def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "i32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_dev(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def empty_mem(shape, dtype, device="cuda"):
    import torch
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=device)


# ----------------------------------------------------------------------------- indices
def exact_slot_scores(x: np.ndarray, C1: np.ndarray, C2: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """float64 scores sigma1[i] + sigma2[j] of the given slots (n = i*s + j) for each row."""
    s, h = C1.shape
    s1 = x[:, :h] @ C1.T
    s2 = x[:, h:] @ C2.T
    i = slots // s
    j = slots % s
    return np.take_along_axis(s1, i, 1) + np.take_along_axis(s2, j, 1)


def compare_indices(gpu: np.ndarray, ora: np.ndarray, x: np.ndarray, C1, C2, N: int):
    """Position-by-position comparison of [T, n] slot lists. A mismatch is a counted tie when
    the two slots' exact scores differ by less than TIE_REL (relative); otherwise it is a
    failure. Returns (n_tie_positions, set_change_tokens, failures)."""
    assert gpu.shape == ora.shape
    bad_range = (gpu < 0) | (gpu >= N)
    fails = []
    if bad_range.any():
        fails.append(("out_of_range", int(bad_range.sum())))
        return 0, [], fails
    for t in range(gpu.shape[0]):
        if len(set(gpu[t].tolist())) != gpu.shape[1]:
            fails.append(("duplicate", t))
    mism = gpu != ora
    ties = 0
    set_change = []
    if mism.any():
        rows = np.nonzero(mism.any(1))[0]
        sg = exact_slot_scores(x[rows], C1, C2, gpu[rows])
        so = exact_slot_scores(x[rows], C1, C2, ora[rows])
        for k, t in enumerate(rows):
            pos = np.nonzero(mism[t])[0]
            a, b = sg[k, pos], so[k, pos]
            rel = np.abs(a - b) / np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-300)
            if np.all(rel < TIE_REL):
                ties += len(pos)
            else:
                fails.append(("mismatch", int(t), pos.tolist(), gpu[t, pos].tolist(), ora[t, pos].tolist(),
                              float(rel.max())))
            if set(gpu[t].tolist()) != set(ora[t].tolist()):
                set_change.append(int(t))
    return ties, set_change, fails


# ----------------------------------------------------------------------------- shapes
def lib_shape(sh: SI.Shape, **over):
    import sparse_memory_linear_amd as S
    d = dict(B=sh.B, H=sh.H, T=sh.T, N=sh.N, d_k=sh.d_k, d_v=sh.d_v, kappa=sh.kappa, W=sh.W, R=sh.R,
             in_dtype=sh.in_dtype, mem_dtype=sh.mem_dtype)
    d.update(over)
    return S.make_shape(**d)


def tolerance(sh: SI.Shape) -> float:
    """1e-4 relative with float32 inputs and table, 2e-2 with bf16 inputs."""
    return 1e-4 if (sh.in_dtype == "f32" and sh.mem_dtype == "f32") else 2e-2
