"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes the oracle module (so that the same checks can be run against
deliberately broken copies of it, see ``test_oracle_mutations.py``) and raises
``AssertionError`` when the oracle disagrees with

* brute force over all N slots on tiny tables (product-key selection),
* closed forms of special cases of the update rule,
* an independent dense Gated DeltaNet written in its textbook matrix form,
* structural invariants (sparsity, state carry, column and unit independence),
* a hand-worked example.

Sources (the method is described in prose only): the paperlayer.ai summary of
arXiv:2607.07386v1 -- §2 Background ("Gated DeltaNet", "Product Key Memory"), §3 Method
("Sparse memory updates", "Sparse addressing", "Sparse retrieval", "Connection to GDN",
"Learned initial state"), §4 ("SDM Configuration"), App. B ("Gate dynamics").
"""
from __future__ import annotations

import math

import numpy as np

RNG = np.random.default_rng(20260711)


# ----------------------------------------------------------------------------- helpers
def _rand_unit(rng, T, d_k, d_v, s, quantised=False):
    h = d_k // 2
    if quantised:
        # small integers * 2^-3: all products and sums exact, many exact score ties
        x = rng.integers(-2, 3, size=(T, d_k)).astype(np.float64) / 8
        C1 = rng.integers(-2, 3, size=(s, h)).astype(np.float64) / 8
        C2 = rng.integers(-2, 3, size=(s, h)).astype(np.float64) / 8
    else:
        x = rng.standard_normal((T, d_k))
        C1 = rng.standard_normal((s, h)) / math.sqrt(h)
        C2 = rng.standard_normal((s, h)) / math.sqrt(h)
    v = rng.standard_normal((T, d_v))
    alpha = 1 / (1 + np.exp(-(rng.standard_normal(T) + 3)))
    beta = rng.random(T)
    return x, C1, C2, v, alpha, beta


def brute_force_top(x, C1, C2, n_sel):
    """Score every slot n = i*s + j as sigma1[i] + sigma2[j] (each half a correctly rounded
    float64 dot product, the two halves added in float64) and take the first n_sel by
    (score desc, slot asc). Written independently of the oracle: explicit loops over all N
    slots."""
    s, h = C1.shape
    sig1 = [math.fsum(float(x[c]) * float(C1[i, c]) for c in range(h)) for i in range(s)]
    sig2 = [math.fsum(float(x[h + c]) * float(C2[j, c]) for c in range(h)) for j in range(s)]
    cands = []
    for i in range(s):
        for j in range(s):
            cands.append((-(sig1[i] + sig2[j]), i * s + j))
    cands.sort()
    return [n for _, n in cands[:n_sel]]


def dense_gdn(S0, K, V, Q, alpha, beta):
    """Gated DeltaNet in matrix form (rows of S indexed by key dimension):
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T ;  o_t = S_t^T q_t."""
    S = S0.copy()
    d = S.shape[0]
    I = np.eye(d)
    outs = []
    for t in range(len(V)):
        k = K[t][:, None]
        S = alpha[t] * (I - beta[t] * (k @ k.T)) @ S + beta[t] * (k @ V[t][None, :])
        outs.append(S.T @ Q[t])
    return np.array(outs), S


# ----------------------------------------------------------------------------- pins
def pin_round_bf16(O):
    """bf16 rounding: agrees with IEEE round-to-nearest-even from float32 (computed here by
    integer arithmetic on the bit pattern) for float32 inputs, rounds directly from float64
    (no double rounding), and keeps ties-to-even."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    bits = x.view(np.uint32).astype(np.int64)
    lo = bits & 0xFFFF
    hi = bits >> 16
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & 1) == 1))
    ref = ((hi + up.astype(np.int64)) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 rounding of float32 values"
    # direct from float64: 1 + 2^-8 + 2^-30 lies just above the midpoint between 1 and 1+2^-7.
    assert O.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    # exact midpoints go to the even neighbour
    assert O.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert O.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2 * 2.0 ** -7
    assert O.round_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2 * 2.0 ** -7)


def pin_pk_equals_brute_force(O, cases=300):
    """PL §2 "Product Key Memory": product-key top-k returns the top slots without scoring
    all N. With kappa >= n_sel the result must equal brute force over all N (ties broken by
    slot index), including exact ties."""
    rng = np.random.default_rng(7)
    for c in range(cases):
        s = int(rng.choice([2, 3, 4, 5, 8]))
        d_k = int(rng.choice([2, 4, 6]))
        n_sel = int(rng.integers(1, min(s * s, 6) + 1))
        # kappa >= n_sel (or kappa = s, when every candidate is kept)
        kappa = int(rng.integers(min(n_sel, s), s + 1))
        x, C1, C2, *_ = _rand_unit(rng, 1, d_k, 1, s, quantised=(c % 2 == 0))
        got, _ = O.product_key_select(x[0], C1, C2, kappa, n_sel)
        ref = brute_force_top(x[0], C1, C2, n_sel)
        assert list(map(int, got)) == ref, (c, s, kappa, n_sel, list(got), ref)


def pin_softmax(O):
    """PL §4 "SDM Configuration": weights are a softmax over the selected scores."""
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 7)) * 4
    w = O.softmax(z)
    assert np.allclose(w.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(O.softmax(z + 123.25), w, rtol=1e-12, atol=0)
    assert O.softmax(np.array([[0.7]]))[0, 0] == 1.0
    # two scores differing by ln 3 -> weights 3/4 and 1/4
    w2 = O.softmax(np.array([[math.log(3.0), 0.0]]))[0]
    assert abs(w2[0] - 0.75) < 1e-15 and abs(w2[1] - 0.25) < 1e-15
    # the address call attaches softmax weights to the selected slots in rank order
    rng = np.random.default_rng(4)
    x, C1, C2, *_ = _rand_unit(rng, 3, 4, 1, 4)
    idx, wgt, sc = O.address(x, C1, C2, 4, 5)
    for t in range(3):
        s1, s2 = C1 @ x[t, :2], C2 @ x[t, 2:]
        exact = np.array([s1[n // 4] + s2[n % 4] for n in idx[t]])
        e = np.exp(exact - exact.max())
        assert np.allclose(wgt[t], e / e.sum(), rtol=1e-12, atol=0)
        assert np.all(np.diff(wgt[t]) <= 1e-15)  # rank order: non-increasing weights


def pin_dense_limit_softmax(O):
    """kappa = s and W = R = N (every slot selected): the sparse rule must equal the dense
    gated delta rule S_t = a S + b w (v - a S^T w)^T with w the softmax over all N scores,
    o_t = S_t^T u_t (matrix form, computed here without any slot bookkeeping)."""
    rng = np.random.default_rng(11)
    s, d_k, d_v, T = 3, 4, 5, 12
    N = s * s
    x_k, C1, C2, v, alpha, beta = _rand_unit(rng, T, d_k, d_v, s)
    x_q = rng.standard_normal((T, d_k))
    M0 = rng.standard_normal((N, d_v)) * 0.1
    r = O.forward_unit(x_q, x_k, v, alpha, beta, C1, C2, M0, s, N, N, "f64")

    def dense_weights(x):
        h = d_k // 2
        sc = np.array([[x[t, :h] @ C1[n // s] + x[t, h:] @ C2[n % s] for n in range(N)] for t in range(T)])
        e = np.exp(sc - sc.max(1, keepdims=True))
        return e / e.sum(1, keepdims=True)

    A, U = dense_weights(x_k), dense_weights(x_q)
    S = M0.copy()
    outs = []
    for t in range(T):
        a = A[t][:, None]
        S = alpha[t] * S + beta[t] * a @ (v[t][None, :] - alpha[t] * (a.T @ S))
        outs.append(S.T @ U[t])
    assert np.allclose(r["o"], np.array(outs), rtol=0, atol=1e-12)
    assert np.allclose(r["M"], S, rtol=0, atol=1e-12)


def pin_gdn_exact(O):
    """PL §3 "Connection to GDN": N = d_qk, W = R = N, identity addressing and raw
    (dense) key / query components as weights reproduce Gated DeltaNet exactly."""
    rng = np.random.default_rng(12)
    d, d_v, T = 6, 4, 20
    K = rng.standard_normal((T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d_v))
    alpha = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    S0 = rng.standard_normal((d, d_v)) * 0.3
    ident = np.tile(np.arange(d), (T, 1))
    o, M = O.recurrence(S0, ident, K, ident, Q, V, alpha, beta, "f64")
    o_ref, S_ref = dense_gdn(S0, K, V, Q, alpha, beta)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(M, S_ref, rtol=0, atol=1e-12)


def pin_identity(O):
    """alpha = 1, beta = 0: the table stays M0 bit for bit and reads return the weighted
    sums of M0 rows (closed form)."""
    rng = np.random.default_rng(13)
    s, d_k, d_v, T = 6, 8, 5, 30
    x_k, C1, C2, v, _, _ = _rand_unit(rng, T, d_k, d_v, s)
    x_q = rng.standard_normal((T, d_k))
    for md in ("f32", "bf16"):
        M0 = O.round_mem(rng.standard_normal((s * s, d_v)) * 0.02, md)
        r = O.forward_unit(x_q, x_k, v, np.ones(T), np.zeros(T), C1, C2, M0, 4, 5, 3, md)
        assert np.array_equal(r["M"], M0)
        ref = np.array([r["rgt"][t] @ M0[r["ridx"][t]] for t in range(T)])
        assert np.allclose(r["o"], ref, rtol=1e-14, atol=0)


def pin_overwrite(O):
    """W = 1, beta = 1: the selected slot becomes exactly v_t for any alpha; with R = 1 and
    q_t = k_t the read returns v_t."""
    rng = np.random.default_rng(14)
    s, d_k, d_v, T = 5, 4, 6, 25
    x, C1, C2, v, alpha, _ = _rand_unit(rng, T, d_k, d_v, s)
    for md in ("f32", "bf16"):
        vv = O.round_mem(v, md)
        M0 = O.round_mem(rng.standard_normal((s * s, d_v)), md)
        r = O.forward_unit(x, x, vv, alpha, np.ones(T), C1, C2, M0, 3, 1, 1, md)
        for t in range(T):
            assert r["ridx"][t][0] == r["widx"][t][0]
            assert np.array_equal(r["o"][t], vv[t])
        last = {}
        for t in range(T):
            last[int(r["widx"][t][0])] = t
        for n, t in last.items():
            assert np.array_equal(r["M"][n], vv[t])


def pin_erase(O):
    """PL App. B "Gate dynamics": alpha = 0 fully decays a written slot, leaving only the
    new contribution: M[n_j] = a_j * beta * v_t."""
    rng = np.random.default_rng(15)
    s, d_k, d_v, T = 4, 4, 3, 10
    x, C1, C2, v, _, beta = _rand_unit(rng, T, d_k, d_v, s)
    M0 = rng.standard_normal((s * s, d_v))
    r = O.forward_unit(x, x, v, np.zeros(T), beta, C1, C2, M0, 4, 3, 2, "f64")
    t = T - 1
    for j, n in enumerate(r["widx"][t]):
        assert np.allclose(r["M"][n], r["wgt"][t][j] * beta[t] * v[t], rtol=1e-15, atol=0)


def pin_sparsity_and_decay_scope(O):
    """PL §3 "Sparse memory updates": only the W selected rows change; every other row is
    bit-identical to M0 -- no row outside the write sets decays."""
    rng = np.random.default_rng(16)
    s, d_k, d_v, T = 8, 6, 4, 20
    x, C1, C2, v, alpha, beta = _rand_unit(rng, T, d_k, d_v, s)
    M0 = O.round_mem(rng.standard_normal((s * s, d_v)), "bf16")
    r = O.forward_unit(rng.standard_normal((T, d_k)), x, v, alpha, beta, C1, C2, M0, 3, 2, 2, "bf16")
    assert np.array_equal(O.round_bf16(r["M"]), r["M"]), "table values must stay bf16 values"
    touched = set(int(n) for row in r["widx"] for n in row)
    for n in range(s * s):
        if n not in touched:
            assert np.array_equal(r["M"][n], M0[n]), n
    assert len(touched) < s * s


def pin_decayed_residual_small(O):
    """Hand-worked example (PL §2 "Gated DeltaNet"; PL §3): s = 2, h = 1, one token.

    k = (1, 2), C1 = [[1], [-1]], C2 = [[1], [0.5]]  ->  sigma1 = (1, -1), sigma2 = (2, 1).
    Slot n = 2i + j scores: n0 = 3, n1 = 2, n2 = 1, n3 = 0. Top-2 write slots: (0, 1) with
    weights (e/(1+e), 1/(1+e)). M0 rows: M[0] = (1, 0), M[1] = (0, 2), others (5, 5).
    alpha = 1/2, beta = 1/2, v = (1, 1):
      rho   = 1/2 * (a0*(1,0) + a1*(0,2)) = (a0/2, a1)
      delta = 1/2 * ((1,1) - rho)        = ((1 - a0/2)/2, (1 - a1)/2)
      M[0]  = 1/2*(1,0) + a0*delta ;  M[1] = 1/2*(0,2) + a1*delta
    Read with q = k, R = 1: slot 0, o = M[0]."""
    e = math.e
    a0, a1 = e / (1 + e), 1 / (1 + e)
    k = np.array([[1.0, 2.0]])
    C1 = np.array([[1.0], [-1.0]])
    C2 = np.array([[1.0], [0.5]])
    M0 = np.array([[1.0, 0.0], [0.0, 2.0], [5.0, 5.0], [5.0, 5.0]])
    r = O.forward_unit(k, k, np.array([[1.0, 1.0]]), np.array([0.5]), np.array([0.5]), C1, C2, M0, 2, 2, 1, "f64")
    assert list(r["widx"][0]) == [0, 1]
    assert np.allclose(r["wgt"][0], [a0, a1], rtol=1e-15, atol=0)
    delta = np.array([(1 - a0 / 2) / 2, (1 - a1) / 2])
    M_0 = 0.5 * np.array([1.0, 0.0]) + a0 * delta
    M_1 = 0.5 * np.array([0.0, 2.0]) + a1 * delta
    assert np.allclose(r["M"][0], M_0, rtol=1e-15, atol=1e-16)
    assert np.allclose(r["M"][1], M_1, rtol=1e-15, atol=1e-16)
    assert np.array_equal(r["M"][2:], M0[2:])
    assert list(r["ridx"][0]) == [0]
    assert np.allclose(r["o"][0], M_0, rtol=1e-15, atol=1e-16)


def pin_read_after_write_two_tokens(O):
    """Two tokens writing the same slot: the second token's residual uses the first
    token's written value, and its read sees its own write (closed form, W = R = 1)."""
    C1 = np.array([[1.0], [0.0]])
    C2 = np.array([[1.0], [0.0]])
    k = np.array([[1.0, 1.0], [1.0, 1.0]])           # both tokens select slot 0 only
    M0 = np.zeros((4, 1))
    M0[0, 0] = 4.0
    v = np.array([[2.0], [8.0]])
    al = np.array([0.5, 0.25])
    be = np.array([0.5, 1.0])
    r = O.forward_unit(k, k, v, al, be, C1, C2, M0, 1, 1, 1, "f64")
    # t0: rho = 0.5*4 = 2, delta = 0.5*(2-2) = 0, M = 0.5*4 + 0 = 2 ; o0 = 2
    # t1: rho = 0.25*2 = 0.5, delta = 1*(8-0.5) = 7.5, M = 0.25*2 + 7.5 = 8 ; o1 = 8
    assert r["o"][0, 0] == 2.0 and r["o"][1, 0] == 8.0 and r["M"][0, 0] == 8.0


def pin_state_carry(O):
    """Running tokens [0, T) equals running [0, T1) and then [T1, T) from the carried
    table, bit for bit (the table is the whole state)."""
    rng = np.random.default_rng(17)
    s, d_k, d_v, T = 6, 6, 3, 40
    x, C1, C2, v, alpha, beta = _rand_unit(rng, T, d_k, d_v, s)
    q = rng.standard_normal((T, d_k))
    M0 = O.round_mem(rng.standard_normal((s * s, d_v)), "bf16")
    full = O.forward_unit(q, x, v, alpha, beta, C1, C2, M0, 4, 4, 3, "bf16")
    T1 = 17
    a = O.forward_unit(q[:T1], x[:T1], v[:T1], alpha[:T1], beta[:T1], C1, C2, M0, 4, 4, 3, "bf16")
    b = O.forward_unit(q[T1:], x[T1:], v[T1:], alpha[T1:], beta[T1:], C1, C2, a["M"], 4, 4, 3, "bf16")
    assert np.array_equal(np.concatenate([a["o"], b["o"]]), full["o"])
    assert np.array_equal(b["M"], full["M"])


def pin_columns_independent(O):
    """Each value column of the table evolves on its own: running a subset of columns
    gives exactly those columns of the full run."""
    rng = np.random.default_rng(18)
    s, d_k, d_v, T = 5, 4, 6, 25
    x, C1, C2, v, alpha, beta = _rand_unit(rng, T, d_k, d_v, s)
    q = rng.standard_normal((T, d_k))
    M0 = rng.standard_normal((s * s, d_v))
    full = O.forward_unit(q, x, v, alpha, beta, C1, C2, M0, 3, 4, 2, "f64")
    part = O.forward_unit(q, x, v[:, 2:5], alpha, beta, C1, C2, M0[:, 2:5], 3, 4, 2, "f64")
    # equal up to the summation order a matrix-vector product may use for other widths
    assert np.allclose(part["o"], full["o"][:, 2:5], rtol=1e-13, atol=1e-15)
    assert np.allclose(part["M"], full["M"][:, 2:5], rtol=1e-13, atol=1e-15)


def pin_read_uses_queries_write_uses_keys(O):
    """PL §3 "Sparse addressing": write slots come from keys and read slots from queries."""
    rng = np.random.default_rng(19)
    s, d_k, d_v, T = 6, 4, 2, 5
    x, C1, C2, v, alpha, beta = _rand_unit(rng, T, d_k, d_v, s)
    q = rng.standard_normal((T, d_k))
    r = O.forward_unit(q, x, v, alpha, beta, C1, C2, np.zeros((s * s, d_v)), 6, 3, 2, "f64")
    for t in range(T):
        assert list(r["widx"][t]) == brute_force_top(x[t], C1, C2, 3)
        assert list(r["ridx"][t]) == brute_force_top(q[t], C1, C2, 2)


# ----------------------------------------------------------------------------- whole-table decay
def _sparse_slots(rng, T, N, n_sel):
    """T rows of n_sel distinct slots in [0, N) with positive weights summing to 1."""
    idx = np.array([rng.choice(N, n_sel, replace=False) for _ in range(T)])
    w = rng.random((T, n_sel)) + 0.1
    return idx, w / w.sum(1, keepdims=True)


def pin_table_decay_is_sparse_gdn(O):
    """The other reading of whether alpha decays the whole table (decay="table"): the
    recurrence is then Gated DeltaNet in its textbook matrix form over all N slots, with key
    and query vectors k_t = sum_j a_j e_{n_j}, q_t = sum_r u_r e_{m_r} (PL §2 "Gated
    DeltaNet"; PL §3 "Connection to GDN")."""
    rng = np.random.default_rng(21)
    N, d_v, T, W, R = 20, 3, 40, 4, 3
    widx, wgt = _sparse_slots(rng, T, N, W)
    ridx, rgt = _sparse_slots(rng, T, N, R)
    V = rng.standard_normal((T, d_v))
    alpha = rng.uniform(0.3, 1.0, T)
    beta = rng.random(T)
    S0 = rng.standard_normal((N, d_v))
    K, Q = np.zeros((T, N)), np.zeros((T, N))
    for t in range(T):
        K[t, widx[t]] = wgt[t]
        Q[t, ridx[t]] = rgt[t]
    o, M = O.recurrence(S0, widx, wgt, ridx, rgt, V, alpha, beta, "f64", decay="table")
    o_ref, S_ref = dense_gdn(S0, K, V, Q, alpha, beta)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(M, S_ref, rtol=0, atol=1e-12)


def pin_table_decay_rows(O):
    """decay="table" with a bf16 table: a row no token writes ends as M0 times the product
    of all gates (not rounded: READING R19); rows the last token writes are bf16 values."""
    rng = np.random.default_rng(22)
    N, d_v, T, W, R = 64, 4, 30, 3, 2
    widx, wgt = _sparse_slots(rng, T, N, W)
    ridx, rgt = _sparse_slots(rng, T, N, R)
    V = O.round_mem(rng.standard_normal((T, d_v)), "bf16")
    alpha = 1 / (1 + np.exp(-(rng.standard_normal(T) + 3)))
    beta = rng.random(T)
    M0 = O.round_mem(rng.standard_normal((N, d_v)) * 0.02, "bf16")
    _, M = O.recurrence(M0, widx, wgt, ridx, rgt, V, alpha, beta, "bf16", decay="table")
    touched = set(int(n) for row in widx for n in row)
    untouched = [n for n in range(N) if n not in touched]
    assert untouched
    assert np.allclose(M[untouched], M0[untouched] * np.prod(alpha), rtol=1e-13, atol=0)
    last = widx[-1]
    assert np.array_equal(O.round_bf16(M[last]), M[last])


def pin_table_decay_alpha_one(O):
    """With alpha = 1 nothing decays, so both readings of the decay scope give the same
    result bit for bit (float32 and bf16 tables)."""
    rng = np.random.default_rng(23)
    s, d_k, d_v, T = 6, 6, 4, 25
    x, C1, C2, v, _, beta = _rand_unit(rng, T, d_k, d_v, s)
    q = rng.standard_normal((T, d_k))
    for md in ("f32", "bf16"):
        M0 = O.round_mem(rng.standard_normal((s * s, d_v)) * 0.02, md)
        a = O.forward_unit(q, x, v, np.ones(T), beta, C1, C2, M0, 4, 3, 3, md)
        b = O.forward_unit(q, x, v, np.ones(T), beta, C1, C2, M0, 4, 3, 3, md, decay="table")
        assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["M"], b["M"])


# ----------------------------------------------------------------------------- gates and output
def pin_gates_closed_forms(O):
    """PL App. B: alpha = exp(g), beta = sigmoid(b). With A_log = log c and a + dt_bias = 0,
    softplus(0) = ln 2 gives alpha = 2^-c; a -> -inf gives alpha -> 1; b = 0 gives 1/2 and
    beta(b) + beta(-b) = 1."""
    A_log = np.log(np.array([1.0, 2.0, 0.5]))
    dt = np.array([0.3, -1.0, 2.0])
    a = -dt[:, None] * np.ones((3, 4))
    b = np.array([[0.0, 1.0, -1.0, 3.0]] * 3)
    al, be = O.gates(a, b, A_log, dt)
    assert np.allclose(al, (2.0 ** -np.array([1.0, 2.0, 0.5]))[:, None] * np.ones((3, 4)), rtol=1e-15, atol=0)
    assert np.array_equal(be[:, 0], np.full(3, 0.5))
    assert np.allclose(be[:, 1] + be[:, 2], 1.0, rtol=0, atol=1e-15)
    al2, _ = O.gates(np.full((3, 1), -800.0), np.zeros((3, 1)), A_log, dt)
    assert np.all(al2 == 1.0)
    al3, _ = O.gates(np.full((3, 1), 50.0), np.zeros((3, 1)), A_log, dt)  # softplus(x) = x for large x
    assert np.allclose(al3[:, 0], np.exp(-np.exp(A_log) * (50.0 + dt)), rtol=1e-13, atol=0)


def pin_output_gate(O):
    """RMS normalisation then SiLU gate: a hand-worked token (o = (3, 4): RMS = sqrt(12.5);
    z = (1, -2): SiLU = 1/(1+e^-1), -2/(1+e^2)), invariance under a positive scale of o
    (eps = 0), and a zero gate where z = 0."""
    o = np.array([3.0, 4.0])
    w = np.array([1.0, 2.0])
    z = np.array([1.0, -2.0])
    y = O.output_gate(o, z, w, 0.0)
    r = math.sqrt(12.5)
    ref = np.array([3.0 / r * 1.0 / (1 + math.exp(-1.0)), 4.0 / r * 2.0 * (-2.0) / (1 + math.exp(2.0))])
    assert np.allclose(y, ref, rtol=1e-15, atol=0)
    rng = np.random.default_rng(31)
    o = rng.standard_normal((5, 8))
    z = rng.standard_normal((5, 8))
    w = rng.standard_normal(8)
    assert np.allclose(O.output_gate(o * 7.5, z, w, 0.0), O.output_gate(o, z, w, 0.0), rtol=1e-14, atol=0)
    z[:, 3] = 0.0
    assert np.all(O.output_gate(o, z, w, 1e-6)[:, 3] == 0.0)


def pin_head_mix(O):
    """The head mixing equals the explicit sum over heads and value columns."""
    rng = np.random.default_rng(32)
    M, H, dv, dm = 3, 2, 4, 5
    x = rng.standard_normal((M, H * dv))
    Wo = rng.standard_normal((dm, H * dv))
    y = O.head_mix(x, Wo)
    for m in range(M):
        for j in range(dm):
            ref = sum(x[m, h * dv + c] * Wo[j, h * dv + c] for h in range(H) for c in range(dv))
            assert abs(y[m, j] - ref) <= 1e-12 * max(1.0, abs(ref))


# ----------------------------------------------------------------------------- backward
def pin_backward_finite_differences(O):
    """The reverse recurrence's gradients equal central finite differences of the forward
    oracle (float64, no rounding) for every input: v, alpha, beta, write and read weights,
    M0; and the undo restores M0 exactly."""
    rng = np.random.default_rng(41)
    N, d_v, T, W, R = 12, 3, 9, 3, 2
    widx, wgt = _sparse_slots(rng, T, N, W)
    ridx = np.array([np.concatenate([[widx[t][0]], rng.choice(np.setdiff1d(np.arange(N), [widx[t][0]]), R - 1,
                                                                 replace=False)]) for t in range(T)])
    rgt = rng.random((T, R)) + 0.1
    v = rng.standard_normal((T, d_v))
    alpha = rng.uniform(0.4, 0.95, T)
    beta = rng.uniform(0.1, 0.9, T)
    M0 = rng.standard_normal((N, d_v))
    go = rng.standard_normal((T, d_v))
    dMT = rng.standard_normal((N, d_v))

    def loss(M0_, v_, al_, be_, w_, u_):
        o, M = O.recurrence(M0_, widx, w_, ridx, u_, v_, al_, be_, "f64")
        return float(np.sum(go * o) + np.sum(dMT * M))

    o, MT = O.recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, "f64")
    xlog = O.recurrence_log(M0, widx, wgt, v, alpha, beta, "f64")
    g = O.recurrence_backward(MT, xlog, widx, wgt, ridx, rgt, v, alpha, beta, go, dMT)
    assert np.array_equal(g["M0"], M0)
    args = [M0, v, alpha, beta, wgt, rgt]
    names = ["dM0", "dv", "dalpha", "dbeta", "dwgt", "drgt"]
    h = 1e-6
    for k, name in enumerate(names):
        base = args[k]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus = [np.array(a_, dtype=np.float64, copy=True) for a_ in args]
            minus = [np.array(a_, dtype=np.float64, copy=True) for a_ in args]
            plus[k][idx] += h
            minus[k][idx] -= h
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        assert np.allclose(g[name], num, rtol=1e-6, atol=1e-7), name


def pin_address_backward_finite_differences(O):
    """The addressing's gradients with the selection held fixed equal central finite
    differences of the forward oracle's own addressing (its softmax weights at unchanged
    slots) for the input rows and both sub-key sets; several selected slots share a sub-key
    of a half (the kappa x kappa staircase), so the scatter-add into the sub-key gradients
    is exercised."""
    rng = np.random.default_rng(43)
    s, h, T, kappa, n_sel = 6, 3, 5, 3, 4
    C1, C2 = rng.standard_normal((s, h)), rng.standard_normal((s, h))
    x = rng.standard_normal((T, 2 * h))
    idx, w, _ = O.address(x, C1, C2, kappa, n_sel)
    assert len(np.unique(idx // s)) < idx.size  # shared first-half sub-keys
    dw = rng.standard_normal(w.shape)
    dx, dC1, dC2 = O.address_backward(x, C1, C2, idx, w, dw)

    def loss(x_, C1_, C2_):
        i, ww, _ = O.address(x_, C1_, C2_, kappa, n_sel)
        assert np.array_equal(i, idx), "a perturbation changed the selection"
        return float(np.sum(dw * ww))

    args = [x, C1, C2]
    hstep = 1e-6
    for k, g in enumerate([dx, dC1, dC2]):
        num = np.zeros_like(args[k])
        for ii in np.ndindex(args[k].shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[k][ii] += hstep
            minus[k][ii] -= hstep
            num[ii] = (loss(*plus) - loss(*minus)) / (2 * hstep)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-8), ["dx", "dC1", "dC2"][k]


def pin_chunkwise_equals_sequential(O):
    """The chunkwise two-phase form (PL App. A.1-A.2) gives the token-by-token rule's output
    and final table (float64, no rounding) for any chunk length: many tokens per slot so
    that rows are written several times inside a chunk and read after, gates at 0 and 1,
    chunk lengths that do and do not divide T."""
    rng = np.random.default_rng(47)
    for trial in range(12):
        N, d_v = int(rng.integers(5, 11)), 3
        T = int(rng.integers(2, 13))
        W, R = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        widx = [rng.choice(N, W, replace=False) for _ in range(T)]
        ridx = [rng.choice(N, R, replace=False) for _ in range(T)]
        wgt, rgt = rng.random((T, W)) + 0.05, rng.random((T, R)) + 0.05
        v = rng.standard_normal((T, d_v))
        alpha = rng.uniform(0.2, 0.99, T)
        alpha[rng.random(T) < 0.15] = 0.0
        alpha[rng.random(T) < 0.15] = 1.0
        beta = rng.uniform(0.05, 1.0, T)
        M0 = rng.standard_normal((N, d_v))
        o1, M1 = O.recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, "f64")
        for C in (1, 2, 3, T):
            o2, M2 = O.chunkwise_recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, C, "f64")
            assert np.allclose(o1, o2, rtol=1e-10, atol=1e-10), (trial, C)
            assert np.allclose(M1, M2, rtol=1e-10, atol=1e-10), (trial, C)


def pin_chunkwise_bf16_rounding_point(O):
    """Where the chunkwise form rounds a bf16 table (READING R26; PL App. A.1: Phase 2 writes
    the state back once per chunk). Worked by hand on one slot, d_v = 1, W = R = 1 with
    weight 1, two tokens that both write and then read slot 0; every value is a short
    dyadic fraction, so float64 holds each one exactly and the only rounding is to bf16
    (8 significant bits, nearest-even):

      M0 = 97/64; token 0: alpha 1, beta 3/4, v 1; token 1: alpha 3/4, beta 1/4, v 1.
      delta_0 = 3/4 (1 - 97/64) = -99/256, new row y_0 = 97/64 - 99/256 = 289/256.
      Token by token: 289/256 is the midpoint of 288/256 and 290/256, so it rounds to the
        even 9/8; o_0 = 9/8. Token 1: delta_1 = 1/4 (1 - 3/4 * 9/8) = 5/128,
        y_1 = 27/32 + 5/128 = 113/128 (exact in bf16); o_1 = final row = 113/128.
      One chunk of two tokens: token 1 sees the unrounded 289/256, so
        delta_1 = 1/4 (1 - 867/1024) = 157/4096 and o_0 = 289/256,
        o_1 = 867/1024 + 157/4096 = 3625/4096; the write-back rounds once:
        3625/4096 = 226.5625/256 -> 227/256.
      Rounding the chunk-start row after its decay but before adding the deltas would give
        round(3/4 * 97/64) = round(291/256) = 292/256 (the even neighbour), then
        292/256 - 297/1024 + 157/4096 = 3641/4096 -> 228/256, not 227/256.
      With chunk length 1 every chunk writes its rows back at once: the table equals the
        token-by-token table (113/128), and o_0 is the unrounded 289/256 (a token reading a
        row it writes sees it before the write-back rounds it).
    """
    M0 = np.array([[97 / 64], [0.0]])
    widx = [np.array([0]), np.array([0])]
    one = [np.array([1.0]), np.array([1.0])]
    v = np.array([[1.0], [1.0]])
    alpha = np.array([1.0, 0.75])
    beta = np.array([0.75, 0.25])
    o, M = O.recurrence(M0, widx, one, widx, one, v, alpha, beta, "bf16")
    assert o[0, 0] == 9 / 8 and o[1, 0] == 113 / 128 and M[0, 0] == 113 / 128, (o, M)
    o, M = O.chunkwise_recurrence(M0, widx, one, widx, one, v, alpha, beta, 2, "bf16")
    assert o[0, 0] == 289 / 256 and o[1, 0] == 3625 / 4096 and M[0, 0] == 227 / 256, (o, M)
    o, M = O.chunkwise_recurrence(M0, widx, one, widx, one, v, alpha, beta, 1, "bf16")
    assert o[0, 0] == 289 / 256 and o[1, 0] == 113 / 128 and M[0, 0] == 113 / 128, (o, M)
    assert M[1, 0] == 0.0


def pin_chunkwise_chunk1_bf16_is_token_rule(O):
    """Chunk length 1 with a bf16 table is the token-by-token bf16 rule (READING R26 rounds
    at each chunk's write-back, and a chunk of one token writes back at its own write, where
    READING R10 rounds): the final table bit for bit, and every output up to float64
    summation order, on tables where rows are rewritten often and no token reads a slot it
    writes itself (that case is worked by hand in ``pin_chunkwise_bf16_rounding_point``)."""
    rng = np.random.default_rng(53)
    for trial in range(10):
        N, d_v = int(rng.integers(8, 14)), 4
        T = int(rng.integers(3, 40))
        W, R = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        widx, ridx = [], []
        for _ in range(T):
            perm = rng.permutation(N)
            widx.append(perm[:W])
            ridx.append(perm[W:W + R])
        wgt, rgt = rng.random((T, W)) + 0.05, rng.random((T, R)) + 0.05
        v = rng.standard_normal((T, d_v))
        alpha = rng.uniform(0.2, 0.99, T)
        beta = rng.uniform(0.05, 1.0, T)
        M0 = O.round_bf16(rng.standard_normal((N, d_v)))
        o1, M1 = O.recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, "bf16")
        o2, M2 = O.chunkwise_recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, 1, "bf16")
        assert np.array_equal(M1, M2), trial
        assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12), trial
        # longer chunks differ from the token rule by the rounding they skip, no more
        o3, M3 = O.chunkwise_recurrence(M0, widx, wgt, ridx, rgt, v, alpha, beta, 8, "bf16")
        scale = np.max(np.abs(M1))
        assert np.max(np.abs(M3 - M1)) <= 0.05 * scale, trial


ALL_PINS = [
    pin_round_bf16,
    pin_pk_equals_brute_force,
    pin_softmax,
    pin_dense_limit_softmax,
    pin_gdn_exact,
    pin_identity,
    pin_overwrite,
    pin_erase,
    pin_sparsity_and_decay_scope,
    pin_decayed_residual_small,
    pin_read_after_write_two_tokens,
    pin_state_carry,
    pin_columns_independent,
    pin_read_uses_queries_write_uses_keys,
    pin_table_decay_is_sparse_gdn,
    pin_table_decay_rows,
    pin_table_decay_alpha_one,
    pin_gates_closed_forms,
    pin_output_gate,
    pin_head_mix,
    pin_backward_finite_differences,
    pin_address_backward_finite_differences,
    pin_chunkwise_equals_sequential,
    pin_chunkwise_bf16_rounding_point,
    pin_chunkwise_chunk1_bf16_is_token_rule,
]
