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


# ----------------------------------------------------------------------------- oracle pool
# Units are independent, so full-size parity runs the oracle one unit per task in a pool of
# worker processes. The pool is forked when the test session starts, before any test
# touches the GPU, so the workers never hold GPU state; they read their inputs and the
# device's results from .npy files in a shared directory (memory-mapped).
_POOL = None
_POOL_SIZE = 0


def start_pool(n: int = None):
    import multiprocessing as mp
    import os
    global _POOL, _POOL_SIZE
    if _POOL is None:
        n = n or max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = mp.get_context("fork").Pool(n)
        _POOL_SIZE = n
    return _POOL


def stop_pool():
    global _POOL
    if _POOL is not None:
        _POOL.close()
        _POOL.join()
        _POOL = None


def pool():
    assert _POOL is not None, "the oracle pool is started at collection time, before the GPU is touched"
    return _POOL


def pool_size() -> int:
    return _POOL_SIZE


class SharedDir:
    """A scratch directory (in /dev/shm when it has room) holding .npy files that the pool's
    workers map; removed on exit."""

    def __init__(self, need_bytes: int = 0):
        import shutil
        import tempfile
        base = None
        try:
            if shutil.disk_usage("/dev/shm").free > 2 * need_bytes + (1 << 30):
                base = "/dev/shm"
        except OSError:
            pass
        self.path = tempfile.mkdtemp(prefix="sdm_parity_", dir=base)

    def save(self, name: str, arr) -> None:
        import os
        np.save(os.path.join(self.path, name + ".npy"), np.ascontiguousarray(arr))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        import shutil
        shutil.rmtree(self.path, ignore_errors=True)


def _load(d: str, name: str):
    import os
    return np.load(os.path.join(d, name + ".npy"), mmap_mode="r")


def unit_parity(task) -> dict:
    """Parity procedure for one (batch, head) unit (runs in a pool worker):

    1. slot lists of keys and queries against the oracle's addressing, position by
       position; a mismatch must be a tie (exact scores within TIE_REL), else it fails;
    2. the oracle recurrence is run on the device's slot lists, with weights from the
       oracle's own float64 scores of those slots (so a tie that picked another, equally
       scored slot does not cascade into the rest of the sequence; where no tie occurred
       these are the oracle's own lists);
    3. o over every token and the whole final table against that run (relative error);
    4. rows that no token writes are bit-identical to the starting table.

    task: dir (shared directory), shape (sdm_inputs.Shape), b, h, and optional names of
    the arrays: start table ("M0", indexed [h]; or a per-unit table [b, h]), chunk (run
    the oracle's chunkwise form with that chunk length instead of the token rule) and
    token_rule (with chunk: also report the errors against the token-by-token rule)."""
    import time
    import oracle.sdm_oracle as O
    t0 = time.perf_counter()
    d, sh, b, h = task["dir"], task["shape"], task["b"], task["h"]
    ind, md = sh.in_dtype, sh.mem_dtype
    L = lambda n: _load(d, n)
    q = SI.widen(np.asarray(L("q")[b, h]), ind)
    k = SI.widen(np.asarray(L("k")[b, h]), ind)
    v = SI.widen(np.asarray(L("v")[b, h]), ind)
    alpha = np.asarray(L("alpha")[b, h], dtype=np.float64)
    beta = np.asarray(L("beta")[b, h], dtype=np.float64)
    sk = SI.widen(np.asarray(L("subkeys")[h]), ind)
    C1, C2 = sk[0], sk[1]
    start = task.get("start", "M0")
    Ms = SI.widen(np.asarray(L(start)[h] if start == "M0" else L(start)[b, h]), md)
    gw = np.asarray(L("widx")[b, h]).astype(np.int64)
    gr = np.asarray(L("ridx")[b, h]).astype(np.int64)
    out = {"b": b, "h": h, "tokens": int(len(gw))}
    oi_w, _, _ = O.address(k, C1, C2, sh.kappa, sh.W)
    oi_r, _, _ = O.address(q, C1, C2, sh.kappa, sh.R)
    tw, cw, fw = compare_indices(gw, oi_w, k, C1, C2, sh.N)
    tr, cr, fr = compare_indices(gr, oi_r, q, C1, C2, sh.N)
    out.update(ties=tw + tr, set_changes=len(set(cw) | set(cr)),
               tie_tokens=sorted(set(cw) | set(cr))[:16],
               differs=bool((gw != oi_w).any() or (gr != oi_r).any()), fails=(fw + fr)[:5])
    if fw or fr:
        return out
    ww, _ = O.slot_weights(k, C1, C2, gw)
    rw, _ = O.slot_weights(q, C1, C2, gr)
    go = np.asarray(L("o")[b, h], dtype=np.float64)
    gM = SI.widen(np.asarray(L("M")[b, h]), md)
    if task.get("chunk"):
        o_ref, M_ref = O.chunkwise_recurrence(Ms, gw, ww, gr, rw, v, alpha, beta, task["chunk"], md)
        if task.get("token_rule"):
            o_tok, M_tok = O.recurrence(Ms, gw, ww, gr, rw, v, alpha, beta, md)
            out.update(err_o_token_rule=rel_err(go, o_tok), err_M_token_rule=rel_err(gM, M_tok))
            del o_tok, M_tok
    else:
        o_ref, M_ref = O.recurrence(Ms, gw, ww, gr, rw, v, alpha, beta, md)
    touched = np.zeros(sh.N, bool)
    touched[gw.ravel()] = True
    out.update(err_o=rel_err(go, o_ref), err_M=rel_err(gM, M_ref),
               untouched_ok=bool(np.array_equal(gM[~touched], Ms[~touched])),
               rows_written=int(touched.sum()), oracle_s=time.perf_counter() - t0)
    return out


def summarise(name: str, sh, results, tol: float, extra=None) -> dict:
    """One record per workload: units and tokens compared, tie counts, worst errors."""
    rec = {
        "workload": name,
        "shape": {k: getattr(sh, k) for k in ("B", "H", "T", "N", "d_k", "d_v", "kappa", "W", "R", "in_dtype",
                                              "mem_dtype")},
        "units_compared": len(results),
        "token_heads_compared": int(sum(r["tokens"] for r in results)),
        "tie_positions": int(sum(r["ties"] for r in results)),
        "set_changing_tie_tokens": int(sum(r["set_changes"] for r in results)),
        "units_with_ties": int(sum(r["differs"] for r in results)),
        "max_rel_err_o": max((r.get("err_o", float("inf")) for r in results), default=0.0),
        "max_rel_err_table": max((r.get("err_M", float("inf")) for r in results), default=0.0),
        "untouched_rows_bit_identical": all(r.get("untouched_ok", False) for r in results),
        "tolerance": tol,
        "oracle_workers": pool_size(),
    }
    if extra:
        rec.update(extra)
    return rec


def write_record(rec: dict, fname: str = "parity_fullsize.json") -> None:
    """Adds the workload's record to <dir>/<fname>, dir = $SDM_PARITY_RECORD_DIR (else a
    directory under the system's temporary directory)."""
    import json
    import os
    import tempfile
    out = os.environ.get("SDM_PARITY_RECORD_DIR") or os.path.join(tempfile.gettempdir(), "sdm_parity_records")
    os.makedirs(out, exist_ok=True)
    path = os.path.join(out, fname)
    data = {}
    if os.path.exists(path):
        try:
            with open(path) as f:
                data = json.load(f)
        except ValueError:
            data = {}
    data[rec["workload"]] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)


def unit_backward_parity(task) -> dict:
    """Full-size parity of the recurrence backward for one unit (runs in a pool worker): the
    device's slot lists are checked against the oracle's addressing (ties counted), then the
    oracle's forward, log of pre-update rows and reverse walk run on the device's slot lists
    and float32 weights (the inputs the device's backward took), and every gradient is
    compared: dv, dalpha, dbeta, the write and read weight gradients and the table's
    gradient at the start (dM0)."""
    import time
    import oracle.sdm_oracle as O
    t0 = time.perf_counter()
    d, sh, b, h = task["dir"], task["shape"], task["b"], task["h"]
    ind, md = sh.in_dtype, sh.mem_dtype
    L = lambda n: _load(d, n)
    q = SI.widen(np.asarray(L("q")[b, h]), ind)
    k = SI.widen(np.asarray(L("k")[b, h]), ind)
    v = SI.widen(np.asarray(L("v")[b, h]), ind)
    alpha = np.asarray(L("alpha")[b, h], dtype=np.float64)
    beta = np.asarray(L("beta")[b, h], dtype=np.float64)
    sk = SI.widen(np.asarray(L("subkeys")[h]), ind)
    M0 = SI.widen(np.asarray(L("M0")[h]), md)
    gw = np.asarray(L("widx")[b, h]).astype(np.int64)
    gr = np.asarray(L("ridx")[b, h]).astype(np.int64)
    ww = np.asarray(L("wgt")[b, h], dtype=np.float64)
    rw = np.asarray(L("rgt")[b, h], dtype=np.float64)
    go = np.asarray(L("go")[b, h], dtype=np.float64)
    out = {"b": b, "h": h, "tokens": int(len(gw))}
    oi_w, _, _ = O.address(k, sk[0], sk[1], sh.kappa, sh.W)
    oi_r, _, _ = O.address(q, sk[0], sk[1], sh.kappa, sh.R)
    tw, cw, fw = compare_indices(gw, oi_w, k, sk[0], sk[1], sh.N)
    tr, cr, fr = compare_indices(gr, oi_r, q, sk[0], sk[1], sh.N)
    out.update(ties=tw + tr, set_changes=len(set(cw) | set(cr)), differs=bool(tw + tr), fails=(fw + fr)[:5])
    if fw or fr:
        return out
    _, MT = O.recurrence(M0, gw, ww, gr, rw, v, alpha, beta, md)
    xlog = O.recurrence_log(M0, gw, ww, v, alpha, beta, md)
    g = O.recurrence_backward(MT, xlog, gw, ww, gr, rw, v, alpha, beta, go)
    del xlog, MT
    dev = {"dv": L("dv")[b, h], "dalpha": L("dalpha")[b, h], "dbeta": L("dbeta")[b, h], "dwgt": L("dwgt")[b, h],
           "drgt": L("drgt")[b, h], "dM0": L("G")[b, h]}
    out["errs"] = {n: rel_err(np.asarray(a, dtype=np.float64), g[n]) for n, a in dev.items()}
    out["oracle_s"] = time.perf_counter() - t0
    return out
