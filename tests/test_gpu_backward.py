"""Memory-efficient backward on the GPU against the oracle: the forward's log of pre-update
write rows, the reverse walk's gradients (v, alpha, beta, write and read weights, M0) and the
in-place undo that restores M0. The oracle runs its own forward and backward on the same
inputs (slots and weights from the oracle's addressing). The coupled case edits the read
lists so that reads hit the token's own write slots, repeat a slot, or share a slot's low
16 bits without being equal: the kernel's exact coupling path and its bitmap test."""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import empty_mem, from_dev, lib_shape, log, rel_err, to_dev, tolerance

pytestmark = pytest.mark.gpu

W_ = SI.WORKLOADS
CASES = {
    "tiny_fp32": W_["tiny_fp32"],
    "small_T128": W_["small"].replace(B=1, H=2, T=128),
    "layer_8b_T100": W_["layer_8b_long"].replace(B=1, H=2, T=100),
    "coupled_T96": W_["layer_8b_long"].replace(B=1, H=2, T=96),
    # every head of the 1.4B shape: the launch picks the configuration the full size uses
    # (32-column blocks, two columns per lane, 8 rows per group); the oracle checks three units
    "layer_1p4b_allheads_T40": W_["layer_1p4b"].replace(T=40),
    # 128 units of the small shape (float32 table): two columns per lane, 4 rows per group
    "small_128units_T24": W_["small"].replace(B=8, H=16, T=24),
    # edges: one token; fewer tokens than waves, lists that leave padding rows in the last
    # row group (float32 table, bf16 inputs); a d_v that leaves the last 16-column block
    # half empty
    "edge_T1": W_["small"].replace(B=1, H=2, T=1),
    "edge_T5_W3_R5": W_["small"].replace(B=2, H=1, T=5, W=3, R=5),
    "ragged_dv40_allheads_T24": W_["layer_1p4b"].replace(T=24, d_v=40),
}
SAMPLED = {"layer_1p4b_allheads_T40": [(0, 0), (3, 7), (7, 15)], "ragged_dv40_allheads_T24": [(0, 0), (7, 15)],
           "small_128units_T24": [(0, 0), (5, 11), (7, 15)]}


def couple(wi, ri, N):
    """Reads that hit their token's write slots (t % 3 == 0), repeat a read slot (1), or
    collide with a write or read slot in the low 16 bits only (2). Returns a new ridx."""
    ri = ri.copy()
    for t in range(len(ri)):
        if t % 3 == 0:
            ri[t, 0:4] = wi[t, 5:9]
        elif t % 3 == 1:
            ri[t, 10] = ri[t, 3]
            ri[t, 11] = ri[t, 3]
        else:
            ri[t, 7] = (wi[t, 2] + 65536) % N
            ri[t, 8] = (ri[t, 9] + 131072) % N
    return ri


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()
    return S


@pytest.mark.parametrize("name", list(CASES))
def test_log_and_backward(sdm, name):
    import torch
    sh = CASES[name]
    log(f"[backward] {name}")
    inp = SI.make_inputs(sh)
    S = lib_shape(sh)
    rng = np.random.default_rng(17)
    go = rng.standard_normal((sh.B, sh.H, sh.T, sh.d_v)).astype(np.float32)
    dMT = np.zeros((sh.B, sh.H, sh.N, sh.d_v), np.float32)
    shp_w, shp_r = (sh.B, sh.H, sh.T, sh.W), (sh.B, sh.H, sh.T, sh.R)
    widx, wgt = np.zeros(shp_w, np.int32), np.zeros(shp_w, np.float32)
    ridx, rgt = np.zeros(shp_r, np.int32), np.zeros(shp_r, np.float32)
    ref = {}
    check = set(SAMPLED.get(name, [(b, h) for b in range(sh.B) for h in range(sh.H)]))
    for b in range(sh.B):
        for h in range(sh.H):
            sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
            k = SI.widen(inp["k"][b, h], sh.in_dtype)
            q = SI.widen(inp["q"][b, h], sh.in_dtype)
            v = SI.widen(inp["v"][b, h], sh.in_dtype)
            al, be = inp["alpha"][b, h].astype(np.float64), inp["beta"][b, h].astype(np.float64)
            M0 = SI.widen(inp["M0"][h], sh.mem_dtype)
            wi, ww, _ = O.address(k, sk[0], sk[1], sh.kappa, sh.W)
            ri, rw, _ = O.address(q, sk[0], sk[1], sh.kappa, sh.R)
            if name.startswith("coupled"):
                ri = couple(wi, ri, sh.N)
            ww, rw = ww.astype(np.float32), rw.astype(np.float32)
            widx[b, h], wgt[b, h], ridx[b, h], rgt[b, h] = wi, ww, ri, rw
            if (b, h) not in check:
                continue
            o, MT = O.recurrence(M0, wi, ww.astype(np.float64), ri, rw.astype(np.float64), v, al, be, sh.mem_dtype)
            xl = O.recurrence_log(M0, wi, ww.astype(np.float64), v, al, be, sh.mem_dtype)
            g = O.recurrence_backward(MT, xl, wi, ww.astype(np.float64), ri, rw.astype(np.float64), v, al, be,
                                      go[b, h].astype(np.float64))
            ref[(b, h)] = (o, MT, xl, g)
    dev = {n: to_dev(inp[n], sh.in_dtype) for n in ("v",)}
    alpha, beta = to_dev(inp["alpha"], "f32"), to_dev(inp["beta"], "f32")
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, to_dev(inp["M0"], sh.mem_dtype), M)
    M0_dev = M.clone()
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    xlog = empty_mem((sh.B, sh.H, sh.T, sh.W, sh.d_v), sh.mem_dtype)
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    dW, dR = to_dev(widx, "i32"), to_dev(ridx, "i32")
    aW, aR = to_dev(wgt, "f32"), to_dev(rgt, "f32")
    sdm.recurrent_log(S, dW, aW, dR, aR, dev["v"], alpha, beta, M, o, xlog, ws)
    torch.cuda.synchronize()
    tol = tolerance(sh)
    gx = SI.widen(from_dev(xlog, sh.mem_dtype), sh.mem_dtype)
    go_o = o.cpu().numpy()
    for (b, h), (ro, rMT, rxl, _) in ref.items():
        eo, ex = rel_err(go_o[b, h], ro), rel_err(gx[b, h], rxl)
        log(f"[backward] {name} forward ({b},{h}): o {eo:.2e} log {ex:.2e}")
        assert eo < tol and ex < tol
    # backward from the GPU's own final table and log
    G = to_dev(dMT, "f32")
    dv = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    dal = torch.empty((sh.B, sh.H, sh.T), dtype=torch.float32, device="cuda")
    dbe = torch.empty_like(dal)
    dwg = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.float32, device="cuda")
    drg = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.float32, device="cuda")
    bws = torch.empty(sdm.backward_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    sdm.recurrent_backward(S, dW, aW, dR, aR, dev["v"], alpha, beta, M, xlog, to_dev(go, "f32"), G, dv, dal, dbe,
                           dwg, drg, bws)
    torch.cuda.synchronize()
    assert sdm.workspace_error(bws) == 0, "a workgroup of the backward gave up waiting"
    assert torch.equal(M, M0_dev), "the undo did not restore M0 bit for bit"
    out = {"dv": dv, "dalpha": dal, "dbeta": dbe, "dwgt": dwg, "drgt": drg, "dM0": G}
    for (b, h), (_, _, _, g) in ref.items():
        errs = {k: rel_err(t[b, h].cpu().numpy(), g[k]) for k, t in out.items()}
        log(f"[backward] {name} grads ({b},{h}): " + " ".join(f"{k} {e:.1e}" for k, e in errs.items()) + f" (tol {tol})")
        for k, e in errs.items():
            assert e < tol, k
    # the chain continues through the addressing: dk from dwgt, dq from drgt, both into the
    # sub-key gradient; the oracle does the same with its own weight gradients
    s = int(round(sh.N ** 0.5))
    dsub = torch.zeros((sh.H, 2, s, sh.d_k // 2), dtype=torch.float32, device="cuda")
    ref_dsub = np.zeros((sh.H, 2, s, sh.d_k // 2))
    sub = to_dev(inp["subkeys"], sh.in_dtype)
    for xname, n_sel, didx, dwt, dgrad, key, hidx, hwt in (("k", sh.W, dW, aW, dwg, "dwgt", widx, wgt),
                                                           ("q", sh.R, dR, aR, drg, "drgt", ridx, rgt)):
        dx = torch.empty((sh.B, sh.H, sh.T, sh.d_k), dtype=torch.float32, device="cuda")
        sdm.address_backward(S, to_dev(inp[xname], sh.in_dtype), sub, n_sel, didx, dwt, dgrad, dx, dsub)
        torch.cuda.synchronize()
        for (b, h), (_, _, _, g) in ref.items():
            sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
            rdx, dC1, dC2 = O.address_backward(SI.widen(inp[xname][b, h], sh.in_dtype), sk[0], sk[1], hidx[b, h],
                                               hwt[b, h].astype(np.float64), g[key])
            ref_dsub[h, 0] += dC1
            ref_dsub[h, 1] += dC2
            e = rel_err(dx[b, h].cpu().numpy(), rdx)
            log(f"[backward] {name} d{xname} ({b},{h}): {e:.1e}")
            assert e < tol, f"d{xname}"
    if name not in SAMPLED:  # the sub-key gradient sums over every unit
        e = rel_err(dsub.cpu().numpy(), ref_dsub)
        log(f"[backward] {name} dsubkeys: {e:.1e}")
        assert e < tol


@pytest.mark.parametrize("name", ["coupled_T96", "layer_8b_T100", "layer_1p4b_allheads_T40"])
def test_backward_repeatable(sdm, name):
    """Every run restores M0 bit for bit and gives the same G and dv bit for bit (no atomics
    there); the sums over columns added with atomics agree to rounding. Covers the start-up
    of the workgroups' control words and the completion ring."""
    import torch
    sh = CASES[name]
    log(f"[backward] repeat {name}")
    inp = SI.make_inputs(sh)
    S = lib_shape(sh)
    shp_w, shp_r = (sh.B, sh.H, sh.T, sh.W), (sh.B, sh.H, sh.T, sh.R)
    widx, wgt = np.zeros(shp_w, np.int32), np.zeros(shp_w, np.float32)
    ridx, rgt = np.zeros(shp_r, np.int32), np.zeros(shp_r, np.float32)
    for b in range(sh.B):
        for h in range(sh.H):
            sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
            wi, ww, _ = O.address(SI.widen(inp["k"][b, h], sh.in_dtype), sk[0], sk[1], sh.kappa, sh.W)
            ri, rw, _ = O.address(SI.widen(inp["q"][b, h], sh.in_dtype), sk[0], sk[1], sh.kappa, sh.R)
            if name.startswith("coupled"):
                ri = couple(wi, ri, sh.N)
            widx[b, h], wgt[b, h], ridx[b, h], rgt[b, h] = wi, ww, ri, rw
    v = to_dev(inp["v"], sh.in_dtype)
    alpha, beta = to_dev(inp["alpha"], "f32"), to_dev(inp["beta"], "f32")
    dW, dR, aW, aR = to_dev(widx, "i32"), to_dev(ridx, "i32"), to_dev(wgt, "f32"), to_dev(rgt, "f32")
    M0 = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, to_dev(inp["M0"], sh.mem_dtype), M0)
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    bws = torch.empty(sdm.backward_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(23)
    go = to_dev(rng.standard_normal((sh.B, sh.H, sh.T, sh.d_v)).astype(np.float32), "f32")
    first = None
    for it in range(4):
        M = M0.clone()
        o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
        xlog = empty_mem((sh.B, sh.H, sh.T, sh.W, sh.d_v), sh.mem_dtype)
        sdm.recurrent_log(S, dW, aW, dR, aR, v, alpha, beta, M, o, xlog, ws)
        G = torch.zeros((sh.B, sh.H, sh.N, sh.d_v), dtype=torch.float32, device="cuda")
        dv = torch.empty_like(go)
        dal = torch.empty((sh.B, sh.H, sh.T), dtype=torch.float32, device="cuda")
        dbe = torch.empty_like(dal)
        dwg = torch.empty(shp_w, dtype=torch.float32, device="cuda")
        drg = torch.empty(shp_r, dtype=torch.float32, device="cuda")
        sdm.recurrent_backward(S, dW, aW, dR, aR, v, alpha, beta, M, xlog, go, G, dv, dal, dbe, dwg, drg, bws)
        torch.cuda.synchronize()
        assert sdm.workspace_error(bws) == 0
        assert torch.equal(M, M0), f"run {it}: the undo did not restore M0"
        out = (G, dv, dal, dbe, dwg, drg)
        if first is None:
            first = out
            continue
        assert torch.equal(G, first[0]) and torch.equal(dv, first[1]), f"run {it}: G or dv changed"
        for a, b in zip(out[2:], first[2:]):
            assert rel_err(a.cpu().numpy(), b.cpu().numpy()) < 1e-5, f"run {it}: an atomic sum changed"
        log(f"[backward] repeat {name} run {it}: identical")
