"""Whole-table decay variant (alpha_t decays every row, applied lazily on the GPU) against
the oracle's dense definition (``recurrence(..., decay="table")``: every row multiplied by
alpha_t every token, rows rounded to the table dtype when written).

The GPU keeps, beside the table, the cumulative log-decay at each slot's last write (lam)
and of all tokens (lrun); ``sdm_materialize`` turns that state into the current table,
which is compared with the oracle's table. Tolerances as for the plain path."""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import compare_indices, empty_mem, from_dev, lib_shape, log, rel_err, to_dev, tolerance

pytestmark = pytest.mark.gpu

W_ = SI.WORKLOADS
CASES = {
    # float32 throughout, 16 x 16 product keys
    "tiny_fp32": W_["tiny_fp32"],
    # bf16 inputs, float32 table, s = 256, two units
    "small_T160": W_["small"].replace(B=1, H=2, T=160),
    # the 8B-scale shape (bf16 table, s = 512, repeated keys), ragged token count
    "layer_8b_T100": W_["layer_8b_long"].replace(B=1, H=2, T=100),
    # few units and long enough sequences for the order pass to cut each unit's tokens into
    # parallel segments (4 and 2 segments, the last one ragged): N = 4096 keeps the oracle's
    # dense decay of every row cheap
    "segments4_T8300": W_["small"].replace(B=1, H=2, T=8300, N=4096, d_k=64, d_v=32),
    "segments2_T4200_bf16": W_["layer_8b_long"].replace(B=1, H=2, T=4200, N=4096, d_k=64, d_v=32, kappa=16,
                                                         W=16, R=16),
}


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()
    return S


def upload(inp, sh):
    d = {k: to_dev(inp[k], sh.in_dtype) for k in ("q", "k", "v", "subkeys")}
    d["alpha"] = to_dev(inp["alpha"], "f32")
    d["beta"] = to_dev(inp["beta"], "f32")
    d["M0"] = to_dev(inp["M0"], sh.mem_dtype)
    return d


def unit_inputs(inp, sh, b, h, lo=0, hi=None):
    hi = sh.T if hi is None else hi
    sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
    return dict(q=SI.widen(inp["q"][b, h, lo:hi], sh.in_dtype), k=SI.widen(inp["k"][b, h, lo:hi], sh.in_dtype),
                v=SI.widen(inp["v"][b, h, lo:hi], sh.in_dtype), alpha=inp["alpha"][b, h, lo:hi].astype(np.float64),
                beta=inp["beta"][b, h, lo:hi].astype(np.float64), C1=sk[0], C2=sk[1],
                M0=SI.widen(inp["M0"][h], sh.mem_dtype))


def fresh_state(sdm, S, sh, dev):
    import torch
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M)
    lam = torch.empty((sh.B, sh.H, sh.N), dtype=torch.float64, device="cuda")
    lrun = torch.empty((sh.B, sh.H), dtype=torch.float64, device="cuda")
    sdm.decay_state_init(S, lam, lrun)
    return M, lam, lrun


def materialize(sdm, S, sh, M, lam, lrun):
    import torch
    out = torch.empty((sh.B, sh.H, sh.N, sh.d_v), dtype=torch.float32, device="cuda")
    sdm.materialize(S, M, lam, lrun, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_recurrent_decay_parity(sdm, name):
    """The recurrence alone on the oracle's slots and weights: outputs, the materialized
    table and the running log-decay."""
    import torch
    sh = CASES[name]
    log(f"[decay recurrent] {name}")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    shp_w, shp_r = (sh.B, sh.H, sh.T, sh.W), (sh.B, sh.H, sh.T, sh.R)
    widx, wgt = np.zeros(shp_w, np.int32), np.zeros(shp_w, np.float32)
    ridx, rgt = np.zeros(shp_r, np.int32), np.zeros(shp_r, np.float32)
    ref = {}
    for b in range(sh.B):
        for h in range(sh.H):
            U = unit_inputs(inp, sh, b, h)
            wi, ww, _ = O.address(U["k"], U["C1"], U["C2"], sh.kappa, sh.W)
            ri, rw, _ = O.address(U["q"], U["C1"], U["C2"], sh.kappa, sh.R)
            ww, rw = ww.astype(np.float32), rw.astype(np.float32)
            widx[b, h], wgt[b, h], ridx[b, h], rgt[b, h] = wi, ww, ri, rw
            ref[(b, h)] = O.recurrence(U["M0"], wi, ww.astype(np.float64), ri, rw.astype(np.float64), U["v"],
                                       U["alpha"], U["beta"], sh.mem_dtype, decay="table")
    M, lam, lrun = fresh_state(sdm, S, sh, dev)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes_decay(S), dtype=torch.uint8, device="cuda")
    sdm.recurrent_decay(S, to_dev(widx, "i32"), to_dev(wgt, "f32"), to_dev(ridx, "i32"), to_dev(rgt, "f32"),
                        dev["v"], dev["alpha"], dev["beta"], M, lam, lrun, o, ws)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    go = o.cpu().numpy()
    gM = materialize(sdm, S, sh, M, lam, lrun)
    tol = tolerance(sh)
    worst_o = worst_m = 0.0
    for (b, h), (ro, rM) in ref.items():
        worst_o = max(worst_o, rel_err(go[b, h], ro))
        worst_m = max(worst_m, rel_err(gM[b, h], rM))
        L = np.sum(np.log(inp["alpha"][b, h].astype(np.float64)))
        assert abs(float(lrun[b, h]) - L) <= 1e-9 * max(1.0, abs(L))
    log(f"[decay recurrent] {name}: rel err o {worst_o:.2e} table {worst_m:.2e} (tol {tol})")
    assert worst_o < tol and worst_m < tol


@pytest.mark.parametrize("name", ["tiny_fp32", "layer_8b_T100"])
def test_forward_decay_parity_and_state_carry(sdm, name):
    """The full forward with whole-table decay against the oracle, and the same tokens in
    two calls on the carried state (table, lam, lrun)."""
    import torch
    sh = CASES[name]
    log(f"[decay forward] {name}")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M, lam, lrun = fresh_state(sdm, S, sh, dev)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    wo = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.int32, device="cuda")
    ro = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.int32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes_decay(S), dtype=torch.uint8, device="cuda")
    sdm.forward_decay(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, lam, lrun, o, ws,
                      wo, ro)
    torch.cuda.synchronize()
    go, gw, gr = o.cpu().numpy(), wo.cpu().numpy(), ro.cpu().numpy()
    gM = materialize(sdm, S, sh, M, lam, lrun)
    tol = tolerance(sh)
    for b in range(sh.B):
        for h in range(sh.H):
            U = unit_inputs(inp, sh, b, h)
            oi_w, _, _ = O.address(U["k"], U["C1"], U["C2"], sh.kappa, sh.W)
            oi_r, _, _ = O.address(U["q"], U["C1"], U["C2"], sh.kappa, sh.R)
            _, _, fw = compare_indices(gw[b, h], oi_w, U["k"], U["C1"], U["C2"], sh.N)
            _, _, fr = compare_indices(gr[b, h], oi_r, U["q"], U["C1"], U["C2"], sh.N)
            assert not fw and not fr
            # the oracle on the device's slot lists (its own wherever no tie occurred)
            ww, _ = O.slot_weights(U["k"], U["C1"], U["C2"], gw[b, h])
            rw, _ = O.slot_weights(U["q"], U["C1"], U["C2"], gr[b, h])
            ro_, rM_ = O.recurrence(U["M0"], gw[b, h], ww, gr[b, h], rw, U["v"], U["alpha"], U["beta"], sh.mem_dtype,
                                    decay="table")
            eo = rel_err(go[b, h], ro_)
            em = rel_err(gM[b, h], rM_)
            log(f"[decay forward] {name} unit ({b},{h}): o {eo:.2e} table {em:.2e} (tol {tol})")
            assert eo < tol and em < tol
    # two calls on the carried state
    M2, lam2, lrun2 = fresh_state(sdm, S, sh, dev)
    T1 = sh.T // 2 + 3
    parts = []
    for lo, hi in ((0, T1), (T1, sh.T)):
        Sp = lib_shape(sh, T=hi - lo)
        sl = lambda t: t[:, :, lo:hi].clone()  # a fresh (aligned) buffer even where the slice is contiguous
        op = torch.empty((sh.B, sh.H, hi - lo, sh.d_v), dtype=torch.float32, device="cuda")
        wsp = torch.empty(sdm.workspace_bytes_decay(Sp), dtype=torch.uint8, device="cuda")
        sdm.forward_decay(Sp, sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["alpha"]), sl(dev["beta"]),
                          dev["subkeys"], M2, lam2, lrun2, op, wsp)
        parts.append(op)
    torch.cuda.synchronize()
    o2 = torch.cat(parts, 2).cpu().numpy()
    gM2 = materialize(sdm, S, sh, M2, lam2, lrun2)
    # the log-decay sums differ only in float64 summation order between the two runs
    assert rel_err(o2, go) < 1e-5 and rel_err(gM2, gM) < 1e-5
    assert np.allclose(lrun2.cpu().numpy(), lrun.cpu().numpy(), rtol=1e-12, atol=0)


def test_decode_decay_parity(sdm):
    """Prefill with the whole-table decay forward, then one fused decode step, against the
    oracle's prefill and decode step with the same rule."""
    import torch
    sh = W_["decode"].replace(B=3, H=2)
    P = 48
    log("[decay decode]")
    S_pre = lib_shape(sh, T=P)
    S_dec = lib_shape(sh, T=1)
    params = SI.make_inputs(sh)
    dev = upload(params, sh)
    M, lam, lrun = fresh_state(sdm, S_dec, sh, dev)
    pre = [SI.make_prefill(sh, b, T=P) for b in range(sh.B)]
    cat = {k: np.concatenate([p[k] for p in pre], 0) for k in ("q", "k", "v", "alpha", "beta")}
    dp = {k: to_dev(cat[k], sh.in_dtype if k in "qkv" else "f32") for k in cat}
    ws = torch.empty(sdm.workspace_bytes_decay(S_pre), dtype=torch.uint8, device="cuda")
    o_pre = torch.empty((sh.B, sh.H, P, sh.d_v), dtype=torch.float32, device="cuda")
    wo = torch.empty((sh.B, sh.H, P, sh.W), dtype=torch.int32, device="cuda")
    ro = torch.empty((sh.B, sh.H, P, sh.R), dtype=torch.int32, device="cuda")
    sdm.forward_decay(S_pre, dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], dev["subkeys"], M, lam, lrun, o_pre,
                      ws, wo, ro)
    o = torch.empty((sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    sdm.decode_step_decay(S_dec, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, lam,
                          lrun, o)
    torch.cuda.synchronize()
    go = o.cpu().numpy()
    gM = materialize(sdm, S_dec, sh, M, lam, lrun)
    gw, gr = wo.cpu().numpy(), ro.cpu().numpy()
    tol = tolerance(sh)
    worst, compared = 0.0, 0
    for b in range(sh.B):
        for h in range(sh.H):
            sk = SI.widen(params["subkeys"][h], sh.in_dtype)
            C1, C2 = sk[0], sk[1]
            M0 = SI.widen(params["M0"][h], sh.mem_dtype)
            U = {k: SI.widen(pre[b][k][0, h], sh.in_dtype) for k in ("q", "k", "v")}
            oi_w, _, _ = O.address(U["k"], C1, C2, sh.kappa, sh.W)
            oi_r, _, _ = O.address(U["q"], C1, C2, sh.kappa, sh.R)
            _, _, fw = compare_indices(gw[b, h], oi_w, U["k"], C1, C2, sh.N)
            _, _, fr = compare_indices(gr[b, h], oi_r, U["q"], C1, C2, sh.N)
            assert not fw and not fr
            # the oracle's prefill on the device's slot lists (its own wherever no tie occurred)
            ww, _ = O.slot_weights(U["k"], C1, C2, gw[b, h])
            rw, _ = O.slot_weights(U["q"], C1, C2, gr[b, h])
            _, Mpre = O.recurrence(M0, gw[b, h], ww, gr[b, h], rw, U["v"], pre[b]["alpha"][0, h].astype(np.float64),
                                   pre[b]["beta"][0, h].astype(np.float64), sh.mem_dtype, decay="table")
            r = {"M": Mpre}
            od, Md, _ = O.decode_step_unit(r["M"], SI.widen(params["q"][b, h, 0], sh.in_dtype),
                                           SI.widen(params["k"][b, h, 0], sh.in_dtype),
                                           SI.widen(params["v"][b, h, 0], sh.in_dtype), float(params["alpha"][b, h, 0]),
                                           float(params["beta"][b, h, 0]), C1, C2, sh.kappa, sh.W, sh.R, sh.mem_dtype,
                                           decay="table")
            worst = max(worst, rel_err(go[b, h, 0], od), rel_err(gM[b, h], Md))
            compared += 1
    log(f"[decay decode] rel err {worst:.2e} over {compared} units (tol {tol})")
    assert compared > 0 and worst < tol
