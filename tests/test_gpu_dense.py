"""The dense limits of the sparse rule on the GPU (PL §3 "Connection to GDN"; PL §3
"Sparse addressing" with every slot selected).

* Gated DeltaNet exactly: N = d_k slots, every token writes and reads all of them in
  identity order with the raw key / query components as weights. The device recurrence
  (pipeline, and the chunkwise form) must give the textbook matrix-form Gated DeltaNet
  S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t, written
  out here in float64 with no slot bookkeeping.
* kappa = s and W = R = N through the whole forward (addressing included): the result must
  equal the dense gated delta rule with softmax weights over all N product-key scores.

Beside them, the other boundary of the slot lists: indices outside [0, N) are skipped and
counted.
"""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import empty_mem, from_dev, lib_shape, log, rel_err, to_dev
from pins import dense_gdn

pytestmark = pytest.mark.gpu

W_ = SI.WORKLOADS
TOL_F32 = 1e-4  # float32 table and sums over T <= 64 tokens of O(1) values


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()
    return S


def _gdn_inputs(B, H, T, d, d_v, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, H, T, d))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    Q = rng.standard_normal((B, H, T, d))
    V = rng.standard_normal((B, H, T, d_v))
    alpha = rng.uniform(0.5, 1.0, (B, H, T))
    beta = rng.uniform(0.0, 1.0, (B, H, T))
    S0 = rng.standard_normal((B, H, d, d_v)) * 0.3
    # the device sees float32 copies; the reference starts from the same values
    f = lambda a: a.astype(np.float32).astype(np.float64)
    return f(K), f(Q), f(V), f(alpha), f(beta), f(S0)


@pytest.mark.parametrize("path", ["pipeline", "chunked"])
@pytest.mark.parametrize("B,H,T", [(2, 3, 50), (4, 8, 33)])
def test_gdn_exact(sdm, path, B, H, T):
    import torch
    d, d_v = 16, 8  # N = d = 16 = 4 x 4 sub-key pairs; rows of 32 bytes
    K, Q, V, alpha, beta, S0 = _gdn_inputs(B, H, T, d, d_v, seed=B * 100 + H * 10 + T)
    sh = W_["tiny_fp32"].replace(B=B, H=H, T=T, N=d, d_k=d, d_v=d_v, kappa=4, W=d, R=d, in_dtype="f32",
                                 mem_dtype="f32")
    S = lib_shape(sh)
    ident = np.broadcast_to(np.arange(d, dtype=np.int32), (B, H, T, d))
    widx, ridx = to_dev(ident, "i32"), to_dev(ident, "i32")
    M = to_dev(S0, "f32")
    o = torch.empty((B, H, T, d_v), dtype=torch.float32, device="cuda")
    args = (widx, to_dev(K, "f32"), ridx, to_dev(Q, "f32"), to_dev(V, "f32"), to_dev(alpha, "f32"),
            to_dev(beta, "f32"), M, o)
    if path == "pipeline":
        ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
        sdm.recurrent(S, *args, ws)
    else:
        ws = torch.empty(sdm.workspace_bytes_chunked(S), dtype=torch.uint8, device="cuda")
        sdm.recurrent_chunked(S, *args, ws)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    go, gM = o.cpu().numpy(), M.cpu().numpy()
    eo = em = 0.0
    for b in range(B):
        for h in range(H):
            o_ref, S_ref = dense_gdn(S0[b, h], K[b, h], V[b, h], Q[b, h], alpha[b, h], beta[b, h])
            eo = max(eo, rel_err(go[b, h], o_ref))
            em = max(em, rel_err(gM[b, h], S_ref))
    log(f"[gdn exact] {path} B={B} H={H} T={T}: rel err o {eo:.2e}, table {em:.2e}")
    assert eo < TOL_F32 and em < TOL_F32


def test_gdn_exact_bf16_table(sdm):
    """The same identity addressing with a bf16 table: equals the oracle's token rule (every
    written row rounded once per token), which the dense case pins to Gated DeltaNet."""
    import torch
    B, H, T, d, d_v = 2, 2, 40, 16, 16
    K, Q, V, alpha, beta, S0 = _gdn_inputs(B, H, T, d, d_v, seed=77)
    S0 = SI.widen(SI.cast(S0, "bf16"), "bf16")
    sh = W_["tiny_fp32"].replace(B=B, H=H, T=T, N=d, d_k=d, d_v=d_v, kappa=4, W=d, R=d, in_dtype="f32",
                                 mem_dtype="bf16")
    S = lib_shape(sh)
    ident = np.broadcast_to(np.arange(d, dtype=np.int32), (B, H, T, d))
    M = to_dev(SI.cast(S0, "bf16"), "bf16")
    o = torch.empty((B, H, T, d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    sdm.recurrent(S, to_dev(ident, "i32"), to_dev(K, "f32"), to_dev(ident, "i32"), to_dev(Q, "f32"),
                  to_dev(V, "f32"), to_dev(alpha, "f32"), to_dev(beta, "f32"), M, o, ws)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    go, gM = o.cpu().numpy(), SI.widen(from_dev(M, "bf16"), "bf16")
    eo = em = 0.0
    for b in range(B):
        for h in range(H):
            ro, rM = O.recurrence(S0[b, h], ident[b, h], K[b, h], ident[b, h], Q[b, h], V[b, h], alpha[b, h],
                                  beta[b, h], "bf16")
            eo = max(eo, rel_err(go[b, h], ro))
            em = max(em, rel_err(gM[b, h], rM))
    log(f"[gdn exact] bf16 table: rel err o {eo:.2e}, table {em:.2e}")
    assert eo < 2e-2 and em < 2e-2


def _dense_softmax_rule(x_q, x_k, v, alpha, beta, C1, C2, M0):
    """Dense gated delta rule with softmax weights over all N = s^2 product-key scores,
    matrix form: S_t = a S + b w (v - a S^T w)^T, o_t = S_t^T u."""
    s, h = C1.shape

    def weights(x):
        sc = (x[:, :h] @ C1.T)[:, :, None] + (x[:, h:] @ C2.T)[:, None, :]  # [T, s, s], n = i*s + j
        sc = sc.reshape(len(x), s * s)
        e = np.exp(sc - sc.max(1, keepdims=True))
        return e / e.sum(1, keepdims=True)

    A, U = weights(x_k), weights(x_q)
    S = M0.copy()
    outs = []
    for t in range(len(v)):
        a = A[t][:, None]
        S = alpha[t] * S + beta[t] * a @ (v[t][None, :] - alpha[t] * (a.T @ S))
        outs.append(S.T @ U[t])
    return np.array(outs), S


@pytest.mark.parametrize("B,H,T,s,d_k,d_v", [(2, 2, 40, 4, 8, 8), (4, 8, 24, 4, 8, 16), (1, 2, 30, 8, 16, 8)])
def test_dense_softmax_limit(sdm, B, H, T, s, d_k, d_v):
    """kappa = s, W = R = N: every slot is selected by the addressing, so the order of the
    slot lists is free but the set and the softmax weights are fixed."""
    import torch
    N = s * s
    rng = np.random.default_rng(N + B * H + T)
    f = lambda a: a.astype(np.float32).astype(np.float64)
    q = f(rng.standard_normal((B, H, T, d_k)) * 0.5)
    k = f(rng.standard_normal((B, H, T, d_k)) * 0.5)
    v = f(rng.standard_normal((B, H, T, d_v)))
    alpha = f(rng.uniform(0.6, 1.0, (B, H, T)))
    beta = f(rng.uniform(0.0, 1.0, (B, H, T)))
    sub = f(rng.standard_normal((H, 2, s, d_k // 2)) * 0.5)
    M0 = f(rng.standard_normal((H, N, d_v)) * 0.2)
    sh = W_["tiny_fp32"].replace(B=B, H=H, T=T, N=N, d_k=d_k, d_v=d_v, kappa=s, W=N, R=N, in_dtype="f32",
                                 mem_dtype="f32")
    S = lib_shape(sh)
    M = empty_mem((B, H, N, d_v), "f32")
    sdm.init_from_M0(S, to_dev(M0, "f32"), M)
    o = torch.empty((B, H, T, d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    wout = torch.empty((B, H, T, N), dtype=torch.int32, device="cuda")
    rout = torch.empty_like(wout)
    sdm.forward(S, to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), to_dev(alpha, "f32"),
                to_dev(beta, "f32"), to_dev(sub, "f32"), M, o, ws, wout, rout)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    # every token selects every slot exactly once
    full = np.arange(N)
    assert np.array_equal(np.sort(wout.cpu().numpy(), axis=-1), np.broadcast_to(full, (B, H, T, N)))
    assert np.array_equal(np.sort(rout.cpu().numpy(), axis=-1), np.broadcast_to(full, (B, H, T, N)))
    go, gM = o.cpu().numpy(), M.cpu().numpy()
    eo = em = 0.0
    for b in range(B):
        for h in range(H):
            ro, rM = _dense_softmax_rule(q[b, h], k[b, h], v[b, h], alpha[b, h], beta[b, h], sub[h, 0], sub[h, 1],
                                         M0[h])
            eo = max(eo, rel_err(go[b, h], ro))
            em = max(em, rel_err(gM[b, h], rM))
    chunk = sdm.forward_uses_chunkwise(S)
    log(f"[dense limit] B={B} H={H} T={T} N={N} ({'chunkwise' if chunk else 'pipeline'}): "
        f"rel err o {eo:.2e}, table {em:.2e}")
    assert eo < TOL_F32 and em < TOL_F32


@pytest.mark.parametrize("W", [8, 6])  # 8: the pipelined recurrence; 6: the sequential path
def test_out_of_range_slots_are_skipped_and_counted(sdm, W):
    """Slot indices outside [0, N) in the lists passed to sdm_recurrent touch nothing and
    carry no weight; the workspace's error word counts them. Reference: the oracle's rule
    applied token by token to each token's valid slots only."""
    import torch
    B, H, T, N, d_v = 1, 2, 40, 256, 32
    rng = np.random.default_rng(W)
    widx = np.stack([np.stack([rng.permutation(N)[:W] for _ in range(T)]) for _ in range(B * H)]).reshape(B, H, T, W)
    ridx = rng.integers(0, N, (B, H, T, W))
    bad_w = rng.random((B, H, T, W)) < 0.15
    bad_r = rng.random((B, H, T, W)) < 0.15
    widx = np.where(bad_w, np.where(rng.random(widx.shape) < 0.5, -1, N + 3), widx).astype(np.int32)
    ridx = np.where(bad_r, np.where(rng.random(ridx.shape) < 0.5, -7, N), ridx).astype(np.int32)
    f = lambda a: a.astype(np.float32).astype(np.float64)
    wgt = f(rng.dirichlet(np.ones(W), (B, H, T)))
    rgt = f(rng.dirichlet(np.ones(W), (B, H, T)))
    v = f(rng.standard_normal((B, H, T, d_v)))
    alpha = f(rng.uniform(0.6, 1.0, (B, H, T)))
    beta = f(rng.uniform(0.0, 1.0, (B, H, T)))
    M0 = f(rng.standard_normal((B, H, N, d_v)) * 0.2)
    sh = W_["tiny_fp32"].replace(B=B, H=H, T=T, N=N, d_k=32, d_v=d_v, kappa=4, W=W, R=W)
    S = lib_shape(sh)
    M = to_dev(M0, "f32")
    o = torch.empty((B, H, T, d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    sdm.recurrent(S, to_dev(widx, "i32"), to_dev(wgt, "f32"), to_dev(ridx, "i32"), to_dev(rgt, "f32"), to_dev(v, "f32"),
                  to_dev(alpha, "f32"), to_dev(beta, "f32"), M, o, ws)
    torch.cuda.synchronize()
    n_bad = int(bad_w.sum() + bad_r.sum())
    assert sdm.workspace_error(ws) == n_bad
    go, gM = o.cpu().numpy(), M.cpu().numpy()
    eo = em = 0.0
    for b in range(B):
        for h in range(H):
            Mr = M0[b, h].copy()
            outs = []
            for t in range(T):
                kw, kr = ~bad_w[b, h, t], ~bad_r[b, h, t]
                ro, Mr = O.recurrence(Mr, widx[b, h, t][kw][None], wgt[b, h, t][kw][None], ridx[b, h, t][kr][None],
                                      rgt[b, h, t][kr][None], v[b, h, t][None], alpha[b, h, t:t + 1],
                                      beta[b, h, t:t + 1], "f32")
                outs.append(ro[0])
            eo = max(eo, rel_err(go[b, h], np.array(outs)))
            em = max(em, rel_err(gM[b, h], Mr))
    log(f"[out-of-range slots] W={W}: {n_bad} skipped and counted; rel err o {eo:.2e}, table {em:.2e}")
    assert eo < TOL_F32 and em < TOL_F32
