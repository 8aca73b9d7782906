"""HIP path against the CPU oracle, through the C ABI, on seeded inputs.

Slot indices must match position by position except counted ties (exact scores within
1e-5 relative); o and the final table must match within 1e-4 relative (float32 inputs and
table) or 2e-2 (bf16 inputs). Rows no token writes must stay bit-identical to M0."""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import (compare_indices, empty_mem, from_dev, lib_shape, log, rel_err, to_dev, tolerance)

pytestmark = pytest.mark.gpu

W_ = SI.WORKLOADS
CASES = {
    # full tiny workload: fp32 everywhere
    "tiny_fp32": W_["tiny_fp32"],
    # fp32 inputs with s = 64: vector-ALU scoring into the swizzled score tile
    "fp32_s64_T100": W_["tiny_fp32"].replace(B=1, H=2, T=100, N=4096, kappa=8, W=8, R=8),
    # the small layer's shape with fewer tokens (8 tiles of 32 tokens per head)
    "small_T256": W_["small"].replace(B=1, H=2, T=256),
    # 1.4B-scale layer shape (s = 512, d_v = 64, bf16 table), ragged token count
    "layer_1p4b_T100": W_["layer_1p4b"].replace(B=2, H=2, T=100),
    # 8B-scale layer shape with repeated keys
    "layer_8b_T300": W_["layer_8b_long"].replace(B=1, H=2, T=300),
}
# Shapes with enough (batch, head) units that the recurrence takes 16-byte lanes (the small
# cases above take 8-byte lanes): one pass per half wave with a float32 table, two passes
# with 32-byte blocks, and 16-byte blocks. name -> (shape, units compared with the oracle)
LANE_CASES = {
    "small_lanes16": (W_["small"].replace(B=4, H=8, T=96), None),
    "layer_1p4b_lanes16": (W_["layer_1p4b"].replace(B=32, H=4, T=24), [(0, 0), (5, 1), (17, 2), (31, 3)]),
    "layer_8b_lanes16": (W_["layer_8b_long"].replace(B=2, H=8, T=80), None),
}


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()  # fails loudly if the library is missing
    return S


def upload(inp, sh):
    d = {k: to_dev(inp[k], sh.in_dtype) for k in ("q", "k", "v", "subkeys")}
    d["alpha"] = to_dev(inp["alpha"], "f32")
    d["beta"] = to_dev(inp["beta"], "f32")
    d["M0"] = to_dev(inp["M0"], sh.mem_dtype)
    return d


def fresh_table(sdm, S, sh, dev):
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M)
    return M


def unit_inputs(inp, sh, b, h):
    sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
    return dict(q=SI.widen(inp["q"][b, h], sh.in_dtype), k=SI.widen(inp["k"][b, h], sh.in_dtype),
                v=SI.widen(inp["v"][b, h], sh.in_dtype), alpha=inp["alpha"][b, h].astype(np.float64),
                beta=inp["beta"][b, h].astype(np.float64), C1=sk[0], C2=sk[1],
                M0=SI.widen(inp["M0"][h], sh.mem_dtype))


# ----------------------------------------------------------------------------- init
@pytest.mark.parametrize("name", ["tiny_fp32", "layer_1p4b_T100"])
def test_init_from_M0_bit_exact(sdm, name):
    import torch
    sh = CASES[name]
    log(f"[init] {name}")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M = fresh_table(sdm, S, sh, dev)
    torch.cuda.synchronize()
    got = from_dev(M, sh.mem_dtype)
    for b in range(sh.B):
        assert np.array_equal(got[b], inp["M0"]), f"sequence {b} differs from M0"


# ----------------------------------------------------------------------------- addressing
@pytest.mark.parametrize("name", list(CASES))
def test_address_parity(sdm, name):
    import torch
    sh = CASES[name]
    log(f"[address] {name}")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    total_ties = 0
    for which, n_sel in (("k", sh.W), ("q", sh.R)):
        idx = torch.empty((sh.B, sh.H, sh.T, n_sel), dtype=torch.int32, device="cuda")
        wgt = torch.empty((sh.B, sh.H, sh.T, n_sel), dtype=torch.float32, device="cuda")
        sc = torch.empty_like(wgt)
        sdm.address(S, dev[which], dev["subkeys"], n_sel, idx, wgt, sc)
        torch.cuda.synchronize()
        gi, gw, gs = idx.cpu().numpy(), wgt.cpu().numpy(), sc.cpu().numpy()
        for b in range(sh.B):
            for h in range(sh.H):
                U = unit_inputs(inp, sh, b, h)
                x = U[which]
                oi, ow, osc = O.address(x, U["C1"], U["C2"], sh.kappa, n_sel)
                ties, changed, fails = compare_indices(gi[b, h], oi, x, U["C1"], U["C2"], sh.N)
                assert not fails, f"{name} {which} unit ({b},{h}): {fails[:3]}"
                total_ties += ties
                same = gi[b, h] == oi
                assert rel_err(gw[b, h][same], ow[same]) < 1e-4
                assert rel_err(gs[b, h][same], osc[same]) < 1e-4
                assert np.allclose(gw[b, h].sum(-1), 1.0, atol=1e-5)
    log(f"[address] {name}: tie positions {total_ties}")


# ----------------------------------------------------------------------------- addressing + init
@pytest.mark.parametrize("name,nparts", [("tiny_fp32", 1), ("small_T256", 2), ("layer_1p4b_T100", 3),
                                         ("layer_8b_T300", 2)])
def test_address_init_equals_separate_calls(sdm, name, nparts):
    """sdm_address_init: slot lists, weights and scores bit-identical to sdm_address, and once
    every part has run the table is M0 in every sequence, bit for bit (M starts as a byte
    pattern no copy of M0 holds)."""
    import torch
    sh = CASES[name]
    log(f"[address_init] {name} nparts={nparts}")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    M.view(torch.uint8).fill_(0xA5)
    for part in range(nparts):
        which, n_sel = (("k", sh.W), ("q", sh.R))[part % 2]
        outs = []
        for fused in (False, True):
            idx = torch.empty((sh.B, sh.H, sh.T, n_sel), dtype=torch.int32, device="cuda")
            wgt = torch.empty((sh.B, sh.H, sh.T, n_sel), dtype=torch.float32, device="cuda")
            sc = torch.empty_like(wgt)
            if fused:
                sdm.address_init(S, dev[which], dev["subkeys"], n_sel, idx, wgt, dev["M0"], M, part, nparts, score=sc)
            else:
                sdm.address(S, dev[which], dev["subkeys"], n_sel, idx, wgt, sc)
            outs.append((idx, wgt, sc))
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name} part {part}: outputs differ"
    torch.cuda.synchronize()
    got = from_dev(M, sh.mem_dtype)
    for b in range(sh.B):
        assert np.array_equal(got[b], inp["M0"]), f"{name}: sequence {b} differs from M0 after {nparts} parts"


# ----------------------------------------------------------------------------- recurrence
@pytest.mark.parametrize("name", list(CASES))
def test_recurrent_parity(sdm, name):
    """The recurrence alone, fed the oracle's slots and weights (no tie can cascade)."""
    import torch
    sh = CASES[name]
    log(f"[recurrent] {name}")
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
            # the device takes float32 weights: the oracle runs on exactly those values
            ww = ww.astype(np.float32)
            rw = rw.astype(np.float32)
            widx[b, h], wgt[b, h], ridx[b, h], rgt[b, h] = wi, ww, ri, rw
            ref[(b, h)] = O.recurrence(U["M0"], wi, ww.astype(np.float64), ri, rw.astype(np.float64), U["v"],
                                       U["alpha"], U["beta"], sh.mem_dtype)
    M = fresh_table(sdm, S, sh, dev)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    sdm.recurrent(S, to_dev(widx, "i32"), to_dev(wgt, "f32"), to_dev(ridx, "i32"), to_dev(rgt, "f32"), dev["v"],
                  dev["alpha"], dev["beta"], M, o, ws)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    go, gM = o.cpu().numpy(), SI.widen(from_dev(M, sh.mem_dtype), sh.mem_dtype)
    tol = tolerance(sh)
    worst_o = worst_m = 0.0
    for (b, h), (ro, rM) in ref.items():
        eo, em = rel_err(go[b, h], ro), rel_err(gM[b, h], rM)
        worst_o, worst_m = max(worst_o, eo), max(worst_m, em)
        touched = np.zeros(sh.N, bool)
        touched[widx[b, h].ravel()] = True
        assert np.array_equal(gM[b, h][~touched], SI.widen(inp["M0"][h], sh.mem_dtype)[~touched])
    log(f"[recurrent] {name}: rel err o {worst_o:.2e} table {worst_m:.2e} (tol {tol})")
    assert worst_o < tol and worst_m < tol


# ----------------------------------------------------------------------------- forward
def run_forward_and_compare(sdm, sh, inp, name, units=None):
    import torch
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M = fresh_table(sdm, S, sh, dev)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    wo = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.int32, device="cuda")
    ro = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.int32, device="cuda")
    sdm.forward(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, o, ws, wo, ro)
    torch.cuda.synchronize()
    go = o.cpu().numpy()
    gM = SI.widen(from_dev(M, sh.mem_dtype), sh.mem_dtype)
    gw, gr = wo.cpu().numpy(), ro.cpu().numpy()
    assert sdm.workspace_error(ws) == 0
    tol = tolerance(sh)
    worst_o = worst_m = 0.0
    ties = rerun = 0
    if units is None:
        units = [(b, h) for b in range(sh.B) for h in range(sh.H)]
    for (b, h) in units:
        U = unit_inputs(inp, sh, b, h)
        oi_w, _, _ = O.address(U["k"], U["C1"], U["C2"], sh.kappa, sh.W)
        oi_r, _, _ = O.address(U["q"], U["C1"], U["C2"], sh.kappa, sh.R)
        tw, cw, fw = compare_indices(gw[b, h], oi_w, U["k"], U["C1"], U["C2"], sh.N)
        tr, cr, fr = compare_indices(gr[b, h], oi_r, U["q"], U["C1"], U["C2"], sh.N)
        assert not fw and not fr, f"{name} unit ({b},{h}): {(fw + fr)[:3]}"
        ties += tw + tr
        rerun += bool(tw + tr)
        # the oracle on the device's slot lists with its own float64 weights (the oracle's own
        # lists wherever no tie occurred), so a tie does not cascade
        ww, _ = O.slot_weights(U["k"], U["C1"], U["C2"], gw[b, h])
        rw, _ = O.slot_weights(U["q"], U["C1"], U["C2"], gr[b, h])
        o_ref, M_ref = O.recurrence(U["M0"], gw[b, h], ww, gr[b, h], rw, U["v"], U["alpha"], U["beta"], sh.mem_dtype)
        worst_o = max(worst_o, rel_err(go[b, h], o_ref))
        worst_m = max(worst_m, rel_err(gM[b, h], M_ref))
        touched = np.zeros(sh.N, bool)
        touched[gw[b, h].ravel()] = True
        assert np.array_equal(gM[b, h][~touched], U["M0"][~touched])
    log(f"[forward] {name}: rel err o {worst_o:.2e} table {worst_m:.2e} (tol {tol}); tie positions {ties}, "
        f"units with ties (oracle run on the device's slot lists): {rerun}")
    assert worst_o < tol and worst_m < tol


@pytest.mark.parametrize("name", list(CASES))
def test_forward_parity(sdm, name):
    sh = CASES[name]
    log(f"[forward] {name}")
    run_forward_and_compare(sdm, sh, SI.make_inputs(sh), name)


@pytest.mark.parametrize("name", list(LANE_CASES))
def test_forward_parity_lanes(sdm, name):
    sh, units = LANE_CASES[name]
    log(f"[forward] {name}")
    run_forward_and_compare(sdm, sh, SI.make_inputs(sh), name, units)


@pytest.mark.parametrize("kind", ["same_key", "q_is_k", "period"])
def test_forward_address_reuse(sdm, kind):
    """Every token writing the same slots, reads of the slots just written, and reuse at
    every distance up to 40 tokens."""
    sh = W_["layer_8b_long"].replace(B=1, H=2, T=160, repeat_frac=0.0)
    log(f"[reuse] {kind}")
    run_forward_and_compare(sdm, sh, SI.adversarial(sh, kind), f"reuse-{kind}")


def test_forward_state_carry(sdm):
    """forward over [0, T) equals forward over [0, T1) then [T1, T) on the carried table."""
    import torch
    sh = CASES["small_T256"]
    log("[carry]")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    M1 = fresh_table(sdm, S, sh, dev)
    o1 = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    sdm.forward(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M1, o1, ws)
    M2 = fresh_table(sdm, S, sh, dev)
    T1 = 100
    parts = []
    for lo, hi in ((0, T1), (T1, sh.T)):
        Sp = lib_shape(sh, T=hi - lo)
        sl = lambda t: t[:, :, lo:hi].contiguous()
        op = torch.empty((sh.B, sh.H, hi - lo, sh.d_v), dtype=torch.float32, device="cuda")
        wsp = torch.empty(sdm.workspace_bytes(Sp), dtype=torch.uint8, device="cuda")
        sdm.forward(Sp, sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["alpha"]), sl(dev["beta"]), dev["subkeys"],
                    M2, op, wsp)
        parts.append(op)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(parts, 2), o1)
    assert torch.equal(M1, M2)


# ----------------------------------------------------------------------------- decode
def test_decode_step_parity(sdm):
    """Decode after a prefill: the prefill runs through sdm_forward, the oracle computes its
    own prefill; then one fused decode step is compared."""
    import torch
    sh = W_["decode"].replace(B=3, H=2)
    P = 48
    log("[decode]")
    S_pre = lib_shape(sh, T=P)
    S_dec = lib_shape(sh, T=1)
    params = SI.make_inputs(sh)  # sub-keys, M0 and the decode token
    dev = upload(params, sh)
    M = fresh_table(sdm, S_dec, sh, dev)
    pre = [SI.make_prefill(sh, b, T=P) for b in range(sh.B)]
    cat = {k: np.concatenate([p[k] for p in pre], 0) for k in ("q", "k", "v", "alpha", "beta")}
    dp = {k: to_dev(cat[k], sh.in_dtype if k in "qkv" else "f32") for k in cat}
    ws = torch.empty(sdm.workspace_bytes(S_pre), dtype=torch.uint8, device="cuda")
    o_pre = torch.empty((sh.B, sh.H, P, sh.d_v), dtype=torch.float32, device="cuda")
    wo = torch.empty((sh.B, sh.H, P, sh.W), dtype=torch.int32, device="cuda")
    ro = torch.empty((sh.B, sh.H, P, sh.R), dtype=torch.int32, device="cuda")
    sdm.forward(S_pre, dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta"], dev["subkeys"], M, o_pre, ws, wo, ro)
    o = torch.empty((sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    sdm.decode_step(S_dec, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, o)
    torch.cuda.synchronize()
    go = o.cpu().numpy()
    gM = SI.widen(from_dev(M, sh.mem_dtype), sh.mem_dtype)
    gw, gr = wo.cpu().numpy(), ro.cpu().numpy()
    tol = tolerance(sh)
    worst = 0.0
    compared = 0
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
                                   pre[b]["beta"][0, h].astype(np.float64), sh.mem_dtype)
            r = {"M": Mpre}
            qd = SI.widen(params["q"][b, h, 0], sh.in_dtype)
            kd = SI.widen(params["k"][b, h, 0], sh.in_dtype)
            vd = SI.widen(params["v"][b, h, 0], sh.in_dtype)
            od, Md, rd = O.decode_step_unit(r["M"], qd, kd, vd, float(params["alpha"][b, h, 0]),
                                            float(params["beta"][b, h, 0]), C1, C2, sh.kappa, sh.W, sh.R,
                                            sh.mem_dtype)
            worst = max(worst, rel_err(go[b, h, 0], od), rel_err(gM[b, h], Md))
            compared += 1
    log(f"[decode] rel err {worst:.2e} over {compared} units (tol {tol})")
    assert compared > 0 and worst < tol


@pytest.mark.parametrize("name,mem", [("decode", "bf16"), ("decode", "f32"), ("small", "f32")])
def test_decode_step_equals_forward_T1(sdm, name, mem):
    """State carry, decode form: one sdm_decode_step on a table equals one sdm_forward with
    T = 1 on a copy of the same table -- the same rows written (so the same slots) and the
    same values up to the order of the float32 sums; every other row untouched by both."""
    import torch
    sh = W_[name].replace(B=3, H=4, T=1, mem_dtype=mem)
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S1 = lib_shape(sh, T=1)
    Md = fresh_table(sdm, S1, sh, dev)
    Mf = Md.clone()
    od = torch.empty((sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    of = torch.empty_like(od)
    sdm.decode_step(S1, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], Md, od)
    ws = torch.empty(sdm.workspace_bytes(S1), dtype=torch.uint8, device="cuda")
    sdm.forward(S1, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], Mf, of, ws)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    M0 = fresh_table(sdm, S1, sh, dev)
    torch.cuda.synchronize()
    changed_d = (Md != M0).any(-1)
    changed_f = (Mf != M0).any(-1)
    assert torch.equal(changed_d, changed_f), "the decode step and the forward wrote different rows"
    tol = 1e-5 if mem == "f32" else 1e-2  # bf16 rows: one rounding of sums taken in another order
    eo = rel_err(od.cpu().numpy(), of.cpu().numpy())
    em = rel_err(SI.widen(from_dev(Md, mem), mem), SI.widen(from_dev(Mf, mem), mem))
    log(f"[decode = forward T=1] {name} {mem}: rel diff o {eo:.2e}, table {em:.2e}, "
        f"{int(changed_d.sum())} rows written")
    assert eo < tol and em < tol
