"""Plain float64 oracle of the Sparse Delta Memory (SDM) layer forward.

TEST INFRASTRUCTURE. This module is the checker, not the product: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg import it. It shares
no code with the HIP path (``sparse_memory_linear_amd``) and imports nothing from it; the
only common module is the seeded input generator ``sdm_inputs`` (no method arithmetic).

Sources. "PL" is the paperlayer.ai source-linked summary of arXiv:2607.07386v1,
*Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity*; "Atlas" is the
atlas.scime.ai summary of the same paper. Citations give the page and its section:

* PL §2 Background, "Gated DeltaNet": a gated delta rule reads the value currently stored
  for a key, subtracts it from the new value, and writes the difference, with a decay gate
  alpha in (0, 1) and an input gate beta in [0, 1].
* PL §2 Background, "Product Key Memory": k slots out of N are found with sub-linear work,
  without forming all N scores.
* PL §3 Method, "Sparse memory updates" / "Sparse addressing" / "Sparse retrieval": an
  N-slot table; the gated delta update touches only the W slots selected from the key;
  R slots selected from the query are read as a weighted sum.
* PL §3 Method, "Connection to GDN": with N = d_qk, W = R = d_qk and dense key values the
  update is exactly Gated DeltaNet's.
* PL §3 Method, "Learned initial state": the table starts from a learned M0.
* PL §4 Experimental Setup, "SDM Configuration": read and write activations are
  softmax-normalised.
* PL App. B, "Gate dynamics": slots that are overwritten can be fully decayed (alpha -> 0).
* Atlas, "Approach": the W write and R read slots come from product-key top-k selection.

The pages give no equation, listing or worked example. The steps below are the plainest
reading of that prose; each point the pages leave open is marked READING and is listed,
with the same labels, in the design notes of the repository.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
brute force, closed forms and an independent dense Gated DeltaNet; absolute output
values on realistic inputs have no pin beyond those (the pages print none).
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "round_bf16",
    "round_mem",
    "half_scores",
    "top_order",
    "product_key_select",
    "softmax",
    "address",
    "slot_weights",
    "recurrence",
    "forward_unit",
    "forward",
    "decode_step_unit",
    "gates",
    "output_gate",
    "head_mix",
    "recurrence_log",
    "recurrence_backward",
]

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ----------------------------------------------------------------------------- rounding
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even, directly from
    float64 (no intermediate float32). bfloat16 keeps 8 significant bits and float32's
    exponent range; its smallest subnormal is 2**-133."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2**e with 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)              # exponent of one unit in the last place
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)  # np.rint: round half to even
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, x), y)
    return y


def round_mem(x: np.ndarray, mem_dtype: str) -> np.ndarray:
    """READING R10: the table is stored in its dtype, so every value written to it is
    rounded (nearest-even) to that dtype when it is written, i.e. after every token.
    "f64" (no rounding) exists for the closed-form pins only."""
    if mem_dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if mem_dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if mem_dtype == "bf16":
        return round_bf16(x)
    raise ValueError(mem_dtype)


# ----------------------------------------------------------------------------- addressing
def half_scores(x: np.ndarray, C1: np.ndarray, C2: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Product-key scores of the two halves of x (PL §2 "Product Key Memory"; Atlas
    "Approach"). x: [..., d_k]; C1, C2: [s, h] with h = d_k/2.

    READING R5: the first half x[:h] is scored against C1 and the second half x[h:]
    against C2 (plain dot products, no scale: READING R6)."""
    h = C1.shape[1]
    x = np.asarray(x, dtype=np.float64)
    s1 = x[..., :h] @ np.asarray(C1, dtype=np.float64).T
    s2 = x[..., h:] @ np.asarray(C2, dtype=np.float64).T
    return s1, s2


def top_order(scores: np.ndarray, ids: np.ndarray, count: int) -> np.ndarray:
    """Positions of the first ``count`` entries of each row ordered by (score descending,
    id ascending) -- READING R7, the tie rule used at every selection step."""
    order = np.lexsort((ids, -scores), axis=-1)
    return order[..., :count]


def product_key_select(x: np.ndarray, C1: np.ndarray, C2: np.ndarray, kappa: int, n_sel: int):
    """Select n_sel slots for each row of x by product keys.

    1. score each half against its sub-key set (``half_scores``);
    2. keep the top ``kappa`` sub-keys of each half (READING R7 order);
    3. form the kappa*kappa candidate slots n = i*s + j (READING R5) with score
       sigma1[i] + sigma2[j];
    4. keep the first n_sel candidates by (score desc, slot asc).

    Returns (slots [.., n_sel] int64, scores [.., n_sel] float64) in rank order. Every
    decision compares the float64 scores (READING R18: the plain reading, exact arithmetic
    up to float64 rounding; a device deciding in a narrower precision can order two slots
    differently only where their scores agree to within that precision, which the parity
    comparison counts as a tie, READING R17)."""
    x2 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    s = C1.shape[0]
    s1, s2 = half_scores(x2, C1, C2)
    sub = np.broadcast_to(np.arange(s), s1.shape)
    I1 = np.take_along_axis(sub, top_order(s1, sub, kappa), axis=-1)   # [T, kappa]
    I2 = np.take_along_axis(sub, top_order(s2, sub, kappa), axis=-1)
    T = x2.shape[0]
    slots = (I1[:, :, None] * s + I2[:, None, :]).reshape(T, kappa * kappa)
    cand = (np.take_along_axis(s1, I1, -1)[:, :, None] + np.take_along_axis(s2, I2, -1)[:, None, :]).reshape(T, -1)
    pick = top_order(cand, slots, n_sel)
    sel = np.take_along_axis(slots, pick, -1)
    sc = np.take_along_axis(cand, pick, -1)
    if np.ndim(x) == 1:
        return sel[0], sc[0]
    return sel, sc


def softmax(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, max-subtracted, temperature 1 (PL §4 "SDM
    Configuration": normalised read and write activations; READING R6)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - np.max(z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def address(x, C1, C2, kappa: int, n_sel: int, block: int = 4096):
    """(slots, weights, scores) for every row of x: product-key selection followed by a
    softmax over the selected scores (PL §3 "Sparse addressing", PL §4). Rows are
    processed in blocks only to bound memory; rows are independent."""
    x2 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    outs_i, outs_s = [], []
    for lo in range(0, x2.shape[0], block):
        i, sc = product_key_select(x2[lo:lo + block], C1, C2, kappa, n_sel)
        outs_i.append(i)
        outs_s.append(sc)
    idx = np.concatenate(outs_i, 0) if outs_i else np.zeros((0, n_sel), np.int64)
    sc = np.concatenate(outs_s, 0) if outs_s else np.zeros((0, n_sel))
    return idx, softmax(sc) if sc.size else sc, sc


def slot_weights(x, C1, C2, slots):
    """Weights and scores of given slot lists: slot n = i*s + j of row t scores
    x_t[:h].C1[i] + x_t[h:].C2[j] (READING R5), and the weights are the softmax over the
    listed slots' scores (PL §4 "SDM Configuration"; READING R6). x [T, d_k], slots [T, n].
    This is the last step of ``address`` applied to slot lists chosen elsewhere (where a
    tie let another ranking pick a different but equally scored slot). Returns
    (weights [T, n], scores [T, n]) in float64."""
    x2 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    sl = np.atleast_2d(np.asarray(slots, dtype=np.int64))
    s = C1.shape[0]
    s1, s2 = half_scores(x2, C1, C2)
    sc = np.take_along_axis(s1, sl // s, -1) + np.take_along_axis(s2, sl % s, -1)
    return softmax(sc), sc


# ----------------------------------------------------------------------------- recurrence
def recurrence(M0: np.ndarray, widx, wgt, ridx, rgt, v, alpha, beta, mem_dtype: str, decay: str = "written"):
    """Sparse gated delta write and weighted read, token by token, for one (batch, head).

    For token t with write slots n (weights a) and read slots m (weights u):

    * rho   = alpha_t * sum_j a_j M[n_j]        (READING R2: the read of the write slots
                                               is decayed, as in Gated DeltaNet, PL §2)
    * delta = beta_t * (v_t - rho)
    * M[n_j] <- round(alpha_t * M[n_j] + a_j * delta)   for the W slots only, from the
      values before this token's write (PL §3 "Sparse memory updates"; READING R1: no
      other row is decayed; READING R10: rounding to the table dtype)
    * o_t   = sum_r u_r M[m_r]                  after the write (READING R3; PL §3
                                               "Sparse retrieval", before the output norm)

    M0: [N, d_v] values of the initial table (PL §3 "Learned initial state").

    decay="table" is the other reading of R1: alpha_t decays every row of the table (then
    the rule is Gated DeltaNet's S_t = alpha_t (I - beta_t k k^T) S + beta_t k v^T with the
    sparse key k = sum_j a_j e_{n_j}). Rows are rounded to the table dtype only when they
    are written (READING R19): an untouched row holds its last written value times the
    exact product of the gates since.

    Returns o [T, d_v] float64 and the final table [N, d_v] float64."""
    if decay not in ("written", "table"):
        raise ValueError(decay)
    M = np.array(M0, dtype=np.float64, copy=True)
    T = len(widx)
    d_v = M.shape[1]
    o = np.zeros((T, d_v))
    for t in range(T):
        n = np.asarray(widx[t])
        a = np.asarray(wgt[t], dtype=np.float64)
        old = M[n]
        rho = alpha[t] * (a @ old)
        delta = beta[t] * (v[t] - rho)
        if decay == "table":
            M *= alpha[t]
        M[n] = round_mem(alpha[t] * old + a[:, None] * delta[None, :], mem_dtype)
        m = np.asarray(ridx[t])
        o[t] = np.asarray(rgt[t], dtype=np.float64) @ M[m]
    return o, M


def forward_unit(q, k, v, alpha, beta, C1, C2, M0, kappa: int, W: int, R: int, mem_dtype: str,
                 decay: str = "written") -> Dict:
    """One (batch, head) of the SDM layer forward: addresses from keys (writes) and
    queries (reads) (PL §3 "Sparse addressing"; READING R4: one sub-key pair per head
    serves both), then the recurrence from M0. All arguments are float64 values."""
    widx, wgt, wsc = address(k, C1, C2, kappa, W)
    ridx, rgt, rsc = address(q, C1, C2, kappa, R)
    o, M = recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, mem_dtype, decay)
    return {"o": o, "M": M, "widx": widx, "wgt": wgt, "wscore": wsc, "ridx": ridx, "rgt": rgt, "rscore": rsc}


def forward(inputs: Dict[str, np.ndarray], shape, units=None, columns=None, decay: str = "written") -> Dict:
    """Run ``forward_unit`` over the (b, h) units of a generated workload (``sdm_inputs``).

    ``units``: optional list of (b, h); ``columns``: optional slice of d_v columns (the
    columns of the table evolve independently, so a column subset is exact)."""
    from sdm_inputs import widen

    ind, md = shape.in_dtype, shape.mem_dtype
    if units is None:
        units = [(b, h) for b in range(shape.B) for h in range(shape.H)]
    cols = slice(None) if columns is None else columns
    out = {}
    for (b, h) in units:
        sk = widen(inputs["subkeys"][h], ind)
        M0 = widen(inputs["M0"][h][:, cols], md)
        out[(b, h)] = forward_unit(
            widen(inputs["q"][b, h], ind), widen(inputs["k"][b, h], ind), widen(inputs["v"][b, h][:, cols], ind),
            inputs["alpha"][b, h].astype(np.float64), inputs["beta"][b, h].astype(np.float64),
            sk[0], sk[1], M0, shape.kappa, shape.W, shape.R, md, decay)
    return out


def decode_step_unit(M, q, k, v, alpha, beta, C1, C2, kappa: int, W: int, R: int, mem_dtype: str,
                     decay: str = "written"):
    """One token of one unit on a table M that already holds earlier tokens' writes: the
    same rule as ``forward_unit`` with T = 1. Returns (o [d_v], new M)."""
    r = forward_unit(q[None], k[None], v[None], np.array([alpha]), np.array([beta]), C1, C2, M,
                     kappa, W, R, mem_dtype, decay)
    return r["o"][0], r["M"], r


# ----------------------------------------------------------------------------- gates and output
def _softplus(x):
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gates(a, b, A_log, dt_bias):
    """Decay and input gates from their pre-activations (PL App. B "Gate dynamics": the
    forget gate is exp(g), the input gate sigma(b); PL §4 "SDM Configuration": the forget
    gate and time-step bias follow Gated DeltaNet's conventions). READING R20:
    g = -exp(A_log[h]) * softplus(a + dt_bias[h]) <= 0, alpha = exp(g), beta = sigmoid(b).
    a, b: [..., H, T] per token-head pre-activations; A_log, dt_bias: [H]."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    A = np.exp(np.asarray(A_log, dtype=np.float64))[:, None]
    g = -A * _softplus(a + np.asarray(dt_bias, dtype=np.float64)[:, None])
    return np.exp(g), 1.0 / (1.0 + np.exp(-b))


def output_gate(o, z, w, eps: float):
    """Output of one token-head after the read (PL §3 "Sparse retrieval": RMS-normalised,
    then elementwise gated). READING R21: RMS over d_v with one weight vector w [d_v]
    shared by the heads; READING R22: the gate is SiLU(z), z from its own projection.
    o, z: [..., d_v]."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * np.asarray(w, dtype=np.float64) * (z / (1.0 + np.exp(-z)))


def head_mix(x, Wo):
    """Mixing of the heads into the layer output (PL §3 "Sparse retrieval": projected into
    the layer output). READING R23: y = x Wo^T, no bias; x [M, H*d_v] (heads concatenated
    per token), Wo [d_model, H*d_v]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(Wo, dtype=np.float64).T


# ----------------------------------------------------------------------------- backward
def recurrence_log(M0, widx, wgt, v, alpha, beta, mem_dtype: str):
    """The forward's record for the memory-efficient backward (PL App. A.3: sparse updates
    are applied in place and undone in the backward, keeping O(N d + T W d) memory): the
    pre-update values of each token's W write rows, xlog [T, W, d_v], as the token read
    them. The reads do not change the table, so only the write slots are needed."""
    M = np.array(M0, dtype=np.float64, copy=True)
    T, d_v = len(widx), M.shape[1]
    W = len(widx[0]) if T else 0
    xlog = np.zeros((T, W, d_v))
    for t in range(T):
        n = np.asarray(widx[t])
        a = np.asarray(wgt[t], dtype=np.float64)
        prev = M[n]
        xlog[t] = prev
        dl = beta[t] * (v[t] - alpha[t] * (a @ prev))
        M[n] = round_mem(alpha[t] * prev + a[:, None] * dl[None, :], mem_dtype)
    return xlog


def recurrence_backward(MT, xlog, widx, wgt, ridx, rgt, v, alpha, beta, go, dMT=None):
    """Gradients of L = sum_t <go_t, o_t> + <dMT, M_T> through ``recurrence`` (written-rows
    rule, R1), walking the tokens in reverse and restoring the table in place from the
    forward's log (PL App. A.3). The rounding of written rows is passed through unchanged.

    For token t (x_j = xlog[t, j], rho = alpha sum_j a_j x_j, delta = beta (v - rho)),
    with G the gradient of L with respect to the table after token t:
      read:   du_r = <go_t, M_t[m_r]>;  G[m_r] += u_r go_t
      write:  dy_j = G[n_j];  d delta = sum_j a_j dy_j;  da_j = <dy_j, delta>
              dalpha = sum_j <dy_j, x_j>;  dx_j = alpha dy_j
              dv_t = beta d delta;  dbeta = <d delta, v_t - rho>;  d rho = -beta d delta
              dalpha += <d rho, sum_j a_j x_j>;  da_j += alpha <d rho, x_j>
              dx_j += alpha a_j d rho;  G[n_j] = dx_j
      undo:   M[n_j] = x_j
    Returns a dict: dv [T, d_v], dalpha [T], dbeta [T], dwgt [T, W], drgt [T, R],
    dM0 [N, d_v] (G after token 0) and M0 (the table after every undo)."""
    M = np.array(MT, dtype=np.float64, copy=True)
    G = np.zeros_like(M) if dMT is None else np.array(dMT, dtype=np.float64, copy=True)
    T, d_v = len(widx), M.shape[1]
    W, R = (len(widx[0]), len(ridx[0])) if T else (0, 0)
    dv, dal, dbe = np.zeros((T, d_v)), np.zeros(T), np.zeros(T)
    dw, du = np.zeros((T, W)), np.zeros((T, R))
    for t in reversed(range(T)):
        n, m = np.asarray(widx[t]), np.asarray(ridx[t])
        a, u = np.asarray(wgt[t], dtype=np.float64), np.asarray(rgt[t], dtype=np.float64)
        x = np.asarray(xlog[t], dtype=np.float64)
        g = np.asarray(go[t], dtype=np.float64)
        # read after the write: o_t = sum_r u_r M_t[m_r]
        du[t] = M[m] @ g
        np.add.at(G, m, u[:, None] * g[None, :])
        # write
        s = a @ x
        rho = alpha[t] * s
        resid = v[t] - rho
        delta = beta[t] * resid
        dy = G[n].copy()
        ddelta = a @ dy
        dw[t] = dy @ delta
        dal[t] = np.sum(dy * x)
        dx = alpha[t] * dy
        dv[t] = beta[t] * ddelta
        dbe[t] = ddelta @ resid
        drho = -beta[t] * ddelta
        dal[t] += drho @ s
        dw[t] += alpha[t] * (x @ drho)
        dx += alpha[t] * a[:, None] * drho[None, :]
        G[n] = dx
        M[n] = x
    return {"dv": dv, "dalpha": dal, "dbeta": dbe, "dwgt": dw, "drgt": du, "dM0": G, "M0": M}



def address_backward(x, C1, C2, idx, weight, dweight):
    """Gradients of L = sum <dweight, weight> through the addressing of x with the selected
    slots held fixed (the selection itself carries no gradient): the weights are the softmax
    of the selected scores (PL §4 "SDM Configuration"; READING R6) and slot n = i*s + j
    scores x[:h].C1[i] + x[h:].C2[j] (PL §2 "Product Key Memory"; READING R5).

      dscore_k = weight_k (dweight_k - sum_l weight_l dweight_l)     (softmax Jacobian)
      dx[:h]   = sum_k dscore_k C1[i_k];   dx[h:] = sum_k dscore_k C2[j_k]
      dC1[i]  += dscore_k x[:h] for every k with i_k = i;  dC2[j] likewise with x[h:]

    x [T, d_k]; C1, C2 [s, h]; idx, weight, dweight [T, n_sel].
    Returns dx [T, d_k], dC1 [s, h], dC2 [s, h] (float64)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    C1 = np.asarray(C1, dtype=np.float64)
    C2 = np.asarray(C2, dtype=np.float64)
    s, h = C1.shape
    idx = np.atleast_2d(np.asarray(idx, dtype=np.int64))
    w = np.atleast_2d(np.asarray(weight, dtype=np.float64))
    dw = np.atleast_2d(np.asarray(dweight, dtype=np.float64))
    dsc = w * (dw - np.sum(w * dw, axis=-1, keepdims=True))
    i1, i2 = idx // s, idx % s
    dx = np.zeros_like(x)
    dx[:, :h] = np.einsum("tk,tkc->tc", dsc, C1[i1])
    dx[:, h:] = np.einsum("tk,tkc->tc", dsc, C2[i2])
    dC1 = np.zeros_like(C1)
    dC2 = np.zeros_like(C2)
    np.add.at(dC1, i1.ravel(), (dsc[:, :, None] * x[:, None, :h]).reshape(-1, h))
    np.add.at(dC2, i2.ravel(), (dsc[:, :, None] * x[:, None, h:]).reshape(-1, h))
    return dx, dC1, dC2


def chunkwise_recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, chunk: int, mem_dtype: str):
    """The chunkwise two-phase form of ``recurrence`` (written-rows rule, R1; PL App. A.1,
    "Phase 1" / "Phase 2", and App. A.2's sparse inner products between tokens' slot lists).

    Inside a chunk a row changes only at the tokens that write it, so with delta_t the write
    residual of token t (delta_t = beta_t (v_t - rho_t)) every quantity is the chunk-start
    table M0 plus a linear combination of the chunk's deltas. For a slot n and tokens
    tau < t, let dec(n; tau, t) be the product of alpha over the chunk's writers of n
    strictly between tau and t (tau = -1: from the chunk start). Then

      rho_t = alpha_t sum_j a_tj dec(n_tj; -1, t) M0[n_tj] + sum_{tau<t} K[t,tau] delta_tau
      K[t,tau] = alpha_t sum_{j: n_tj written by tau} a_tj dec(n_tj; tau, t) a_{tau,n_tj}
      o_t = sum_r u_tr dec(m_tr; -1, t+1) M0[m_tr] + sum_{tau<=t} Q[t,tau] delta_tau
      Q[t,tau] = sum_{r: m_tr written by tau} u_tr dec(m_tr; tau, t+1) a_{tau,m_tr}

    so (I + diag(beta) K) delta = beta (v - P), a unit lower-triangular system. Phase 1 needs
    only slots, weights and gates (parallel across chunks); Phase 2 gathers the chunk's rows,
    solves for delta, forms o, and writes each written row once:
      M[n] <- dec(n; -1, end) M0[n] + sum_{writers tau of n} dec(n; tau, end) a_{tau,n} delta_tau

    READING R26: rows are rounded to the table dtype once per chunk, when written back (the
    token-by-token rule rounds at every write; with a float64 or float32 table the two agree
    up to summation order). Returns o [T, d_v] and the final table [N, d_v] (float64)."""
    M = np.array(M0, dtype=np.float64, copy=True)
    T, d_v = len(widx), M.shape[1]
    o = np.zeros((T, d_v))
    for c0 in range(0, T, chunk):
        tok = list(range(c0, min(c0 + chunk, T)))
        L = len(tok)
        n = [np.asarray(widx[t]) for t in tok]
        a = [np.asarray(wgt[t], dtype=np.float64) for t in tok]
        m = [np.asarray(ridx[t]) for t in tok]
        u = [np.asarray(rgt[t], dtype=np.float64) for t in tok]
        al = np.array([alpha[t] for t in tok], dtype=np.float64)
        be = np.array([beta[t] for t in tok], dtype=np.float64)
        # writers of each slot in the chunk, in token order: slot -> [(local token, weight)]
        writers = {}
        for i in range(L):
            for slot, w in zip(n[i].tolist(), a[i].tolist()):
                writers.setdefault(slot, []).append((i, w))

        def dec(slot, lo, hi):
            """Product of alpha over the chunk's writers of slot strictly between lo and hi."""
            p = 1.0
            for i, _ in writers.get(slot, []):
                if lo < i < hi:
                    p *= al[i]
            return p

        # Phase 1: interactions and coefficients (no table values)
        K = np.zeros((L, L))
        Q = np.zeros((L, L))
        for i in range(L):
            for slot, w in zip(n[i].tolist(), a[i].tolist()):
                for k, wk in writers[slot]:
                    if k < i:
                        K[i, k] += al[i] * w * dec(slot, k, i) * wk
            for slot, w in zip(m[i].tolist(), u[i].tolist()):
                for k, wk in writers.get(slot, []):
                    if k <= i:
                        Q[i, k] += w * dec(slot, k, i + 1) * wk
        # Phase 2: gather, solve, read, write back
        P = np.zeros((L, d_v))
        O0 = np.zeros((L, d_v))
        for i in range(L):
            for slot, w in zip(n[i].tolist(), a[i].tolist()):
                P[i] += al[i] * w * dec(slot, -1, i) * M[slot]
            for slot, w in zip(m[i].tolist(), u[i].tolist()):
                O0[i] += w * dec(slot, -1, i + 1) * M[slot]
        V = np.asarray([v[t] for t in tok], dtype=np.float64)
        delta = np.linalg.solve(np.eye(L) + be[:, None] * K, be[:, None] * (V - P))
        o[tok] = O0 + Q @ delta
        new = {}
        for slot, ws in writers.items():
            row = dec(slot, -1, L) * M[slot]
            for k, wk in ws:
                row = row + dec(slot, k, L) * wk * delta[k]
            new[slot] = row
        for slot, row in new.items():
            M[slot] = round_mem(row, mem_dtype)
    return o, M
