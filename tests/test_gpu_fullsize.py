"""The HIP path at full workload sizes, in the launch configuration the benchmark times,
checked where the oracle can follow it:

* slot indices of tokens sampled over the whole sequence (addressing is per token) are
  compared position by position, ties counted;
* outputs over a long prefix of sampled units are compared with the oracle run on that
  prefix (o_t depends only on tokens up to t), up to the first tie that changes a slot set;
* table rows that no token writes stay bit-identical to M0, in every checked unit;
* the whole sequence in two calls on the carried table equals one call, bit for bit;
* the chunkwise two-phase recurrence likewise: sampled units' outputs over a prefix against
  the oracle's chunkwise form, untouched rows still M0;
* decode: one step over all B x H tables, sampled units checked against the oracle after
  the oracle's own prefill (other tables hold M0 only; units are independent);
* the backward: with the output gradient nonzero only on a window of leading tokens, every
  gradient of a sampled unit against the oracle's backward over that window, exact zeros
  past it, and M0 restored bit for bit by the walk back over the whole sequence.
"""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import compare_indices, empty_mem, from_dev, lib_shape, log, rel_err, to_dev, tolerance

pytestmark = pytest.mark.gpu

W_ = SI.WORKLOADS
# workload -> (units checked against the oracle, prefix length, sampled tokens per unit)
PLAN = {
    "small": ([(0, 0), (3, 7)], 2048, 256),
    "layer_1p4b": ([(0, 0), (7, 15)], 4096, 256),
    "layer_8b_long": ([(0, 0), (0, 7)], 4096, 512),
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


def unit_inputs(inp, sh, b, h, T=None):
    T = sh.T if T is None else T
    sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
    return dict(q=SI.widen(inp["q"][b, h, :T], sh.in_dtype), k=SI.widen(inp["k"][b, h, :T], sh.in_dtype),
                v=SI.widen(inp["v"][b, h, :T], sh.in_dtype), alpha=inp["alpha"][b, h, :T].astype(np.float64),
                beta=inp["beta"][b, h, :T].astype(np.float64), C1=sk[0], C2=sk[1],
                M0=SI.widen(inp["M0"][h], sh.mem_dtype))


def forward(sdm, sh, dev, S, M, T_lo=0, T_hi=None):
    import torch
    T_hi = sh.T if T_hi is None else T_hi
    Sp = lib_shape(sh, T=T_hi - T_lo)
    sl = lambda t: t[:, :, T_lo:T_hi].contiguous()
    o = torch.empty((sh.B, sh.H, T_hi - T_lo, sh.d_v), dtype=torch.float32, device="cuda")
    wo = torch.empty((sh.B, sh.H, T_hi - T_lo, sh.W), dtype=torch.int32, device="cuda")
    ro = torch.empty((sh.B, sh.H, T_hi - T_lo, sh.R), dtype=torch.int32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(Sp), dtype=torch.uint8, device="cuda")
    sdm.forward(Sp, sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["alpha"]), sl(dev["beta"]), dev["subkeys"], M,
                o, ws, wo, ro)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    return o, wo, ro


@pytest.mark.parametrize("name", list(PLAN))
def test_fullsize_forward(sdm, name):
    import torch
    sh = W_[name]
    units, prefix, nsamp = PLAN[name]
    log(f"[full] {name}: generating inputs")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M)
    log(f"[full] {name}: forward B={sh.B} H={sh.H} T={sh.T}")
    o, wo, ro = forward(sdm, sh, dev, S, M)
    tol = tolerance(sh)
    rng = np.random.default_rng(7)
    ties = 0
    for (b, h) in units:
        U = unit_inputs(inp, sh, b, h)
        gw, gr = wo[b, h].cpu().numpy(), ro[b, h].cpu().numpy()
        # indices of tokens sampled over the whole sequence (always including the last)
        ts = np.unique(np.concatenate([rng.choice(sh.T, nsamp, replace=False), [sh.T - 1]]))
        for which, g, n_sel in (("k", gw, sh.W), ("q", gr, sh.R)):
            oi, _, _ = O.address(U[which][ts], U["C1"], U["C2"], sh.kappa, n_sel)
            t_, _, fails = compare_indices(g[ts], oi, U[which][ts], U["C1"], U["C2"], sh.N)
            assert not fails, f"{name} unit ({b},{h}) {which}: {fails[:3]}"
            ties += t_
        # outputs over the prefix, up to the first slot-set change caused by a tie
        P = min(prefix, sh.T)
        Up = unit_inputs(inp, sh, b, h, T=P)
        r = O.forward_unit(Up["q"], Up["k"], Up["v"], Up["alpha"], Up["beta"], Up["C1"], Up["C2"], Up["M0"],
                           sh.kappa, sh.W, sh.R, sh.mem_dtype)
        tw, cw, fw = compare_indices(gw[:P], r["widx"], Up["k"], Up["C1"], Up["C2"], sh.N)
        tr, cr, fr = compare_indices(gr[:P], r["ridx"], Up["q"], Up["C1"], Up["C2"], sh.N)
        assert not fw and not fr
        first = min(cw + cr) if (cw or cr) else P
        assert first >= P // 2, f"{name} unit ({b},{h}): slot sets diverge at token {first}"
        eo = rel_err(o[b, h, :first].cpu().numpy(), r["o"][:first])
        log(f"[full] {name} unit ({b},{h}): o over {first} tokens rel err {eo:.2e} (tol {tol}); "
            f"tie positions {tw + tr}")
        assert eo < tol
        # rows no token wrote are still M0
        Mh = SI.widen(from_dev(M[b, h], sh.mem_dtype), sh.mem_dtype)
        touched = np.zeros(sh.N, bool)
        touched[gw.ravel()] = True
        assert np.array_equal(Mh[~touched], U["M0"][~touched])
    log(f"[full] {name}: sampled tie positions {ties}")
    # the same sequence in two calls on the carried table: bit for bit
    M2 = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M2)
    T1 = sh.T // 2 + 3
    o1, _, _ = forward(sdm, sh, dev, S, M2, 0, T1)
    o2, _, _ = forward(sdm, sh, dev, S, M2, T1, sh.T)
    assert torch.equal(torch.cat([o1, o2], 2), o), "split call differs from the single call"
    assert torch.equal(M2, M), "carried table differs"


@pytest.mark.parametrize("name", list(PLAN))
def test_fullsize_chunked(sdm, name):
    """The chunkwise two-phase recurrence at full size, launched as ``bench.py --chunked``
    launches it (addressing of keys and queries, then one sdm_recurrent_chunked call over all
    units): in sampled units the device's slots are checked against the oracle's addressing
    of a prefix, and the outputs up to the first slot-set change caused by a tie against the
    oracle's chunkwise form on the oracle's own slots (o_t depends only on tokens up to t);
    rows no token writes stay M0."""
    import torch
    sh = W_[name]
    units, prefix, _ = PLAN[name]
    log(f"[full] chunked {name}: generating inputs")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M)
    wi = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.int32, device="cuda")
    wg = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.float32, device="cuda")
    ri = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.int32, device="cuda")
    rg = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.float32, device="cuda")
    sdm.address(S, dev["k"], dev["subkeys"], sh.W, wi, wg)
    sdm.address(S, dev["q"], dev["subkeys"], sh.R, ri, rg)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes_chunked(S), dtype=torch.uint8, device="cuda")
    log(f"[full] chunked {name}: B={sh.B} H={sh.H} T={sh.T}")
    sdm.recurrent_chunked(S, wi, wg, ri, rg, dev["v"], dev["alpha"], dev["beta"], M, o, ws)
    torch.cuda.synchronize()
    tol = tolerance(sh)
    for (b, h) in units:
        P = min(prefix, sh.T)
        Up = unit_inputs(inp, sh, b, h, T=P)
        owi, oww, _ = O.address(Up["k"], Up["C1"], Up["C2"], sh.kappa, sh.W)
        ori, orw, _ = O.address(Up["q"], Up["C1"], Up["C2"], sh.kappa, sh.R)
        gw, gr = wi[b, h, :P].cpu().numpy(), ri[b, h, :P].cpu().numpy()
        tw, cw, fw = compare_indices(gw, owi, Up["k"], Up["C1"], Up["C2"], sh.N)
        tr, cr, fr = compare_indices(gr, ori, Up["q"], Up["C1"], Up["C2"], sh.N)
        assert not fw and not fr
        first = min(cw + cr) if (cw or cr) else P
        assert first >= P // 2, f"{name} unit ({b},{h}): slot sets diverge at token {first}"
        oc, _ = O.chunkwise_recurrence(Up["M0"], owi, oww, ori, orw, Up["v"], Up["alpha"], Up["beta"], 64,
                                       sh.mem_dtype)
        eo = rel_err(o[b, h, :first].cpu().numpy(), oc[:first])
        log(f"[full] chunked {name} unit ({b},{h}): o over {first} tokens rel err {eo:.2e} (tol {tol}); "
            f"tie positions {tw + tr}")
        assert eo < tol
        Mh = SI.widen(from_dev(M[b, h], sh.mem_dtype), sh.mem_dtype)
        touched = np.zeros(sh.N, bool)
        touched[wi[b, h].cpu().numpy().ravel()] = True
        assert np.array_equal(Mh[~touched], Up["M0"][~touched])


def test_fullsize_decode(sdm):
    """One decode step over the full 64 x 16 tables (launch of the benchmark); sequences 0 and
    37 are prefilled with their 4096 prior tokens, the others hold M0."""
    import torch
    sh = W_["decode"]
    P = sh.prefill
    log(f"[full] decode: B={sh.B} H={sh.H} N={sh.N}, prefill {P} on sampled sequences")
    params = SI.make_inputs(sh)
    dev = upload(params, sh)
    S1 = lib_shape(sh, T=1)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S1, dev["M0"], M)
    Sp = lib_shape(sh, B=1, T=P)
    ws = torch.empty(sdm.workspace_bytes(Sp), dtype=torch.uint8, device="cuda")
    o_pre = torch.empty((1, sh.H, P, sh.d_v), dtype=torch.float32, device="cuda")
    pre = {}
    for b in (0, 37):
        pre[b] = SI.make_prefill(sh, b)
        t = {n: to_dev(pre[b][n], sh.in_dtype if n in ("q", "k", "v") else "f32")
             for n in ("q", "k", "v", "alpha", "beta")}
        sdm.forward(Sp, t["q"], t["k"], t["v"], t["alpha"], t["beta"], dev["subkeys"], M[b:b + 1], o_pre, ws)
    o = torch.empty((sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    sdm.decode_step(S1, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, o)
    torch.cuda.synchronize()
    tol = tolerance(sh)
    for b, h in ((0, 0), (37, 15), (5, 3)):
        sk = SI.widen(params["subkeys"][h], sh.in_dtype)
        M0h = SI.widen(params["M0"][h], sh.mem_dtype)
        if b in pre:
            pb = pre[b]
            r = O.forward_unit(SI.widen(pb["q"][0, h], sh.in_dtype), SI.widen(pb["k"][0, h], sh.in_dtype),
                               SI.widen(pb["v"][0, h], sh.in_dtype), pb["alpha"][0, h].astype(np.float64),
                               pb["beta"][0, h].astype(np.float64), sk[0], sk[1], M0h, sh.kappa, sh.W, sh.R,
                               sh.mem_dtype)
            Mstart = r["M"]
        else:
            Mstart = M0h
        o_ref, M_ref, _ = O.decode_step_unit(Mstart, SI.widen(params["q"][b, h, 0], sh.in_dtype),
                               SI.widen(params["k"][b, h, 0], sh.in_dtype), SI.widen(params["v"][b, h, 0], sh.in_dtype),
                               float(params["alpha"][b, h, 0]), float(params["beta"][b, h, 0]), sk[0], sk[1],
                               sh.kappa, sh.W, sh.R, sh.mem_dtype)
        eo = rel_err(o[b, h, 0].cpu().numpy(), o_ref)
        Mh = SI.widen(from_dev(M[b, h], sh.mem_dtype), sh.mem_dtype)
        em = rel_err(Mh, M_ref)
        log(f"[full] decode unit ({b},{h}): o rel err {eo:.2e}, table rel err {em:.2e} (tol {tol})")
        assert eo < tol and em < tol


def test_fullsize_decay_variant(sdm):
    """The whole-table decay variant at the full 8B-scale shape (131072 tokens, 8 units):
    with every gate alpha = 1 it decays nothing, so it must equal the written-rows path bit
    for bit; with the workload's gates the running log-decay equals sum(log alpha), two
    calls on the carried state match one call, and untouched slots keep lam = 0."""
    import torch
    sh = W_["layer_8b_long"]
    log("[full] decay variant: generating inputs")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    wsd = torch.empty(sdm.workspace_bytes_decay(S), dtype=torch.uint8, device="cuda")

    def run_decay(alpha, lo=0, hi=None, M=None, lam=None, lrun=None, wo=None):
        hi = sh.T if hi is None else hi
        Sp = lib_shape(sh, T=hi - lo)
        if M is None:
            M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
            sdm.init_from_M0(S, dev["M0"], M)
            lam = torch.empty((sh.B, sh.H, sh.N), dtype=torch.float64, device="cuda")
            lrun = torch.empty((sh.B, sh.H), dtype=torch.float64, device="cuda")
            sdm.decay_state_init(S, lam, lrun)
        sl = lambda t: t[:, :, lo:hi].clone()
        o = torch.empty((sh.B, sh.H, hi - lo, sh.d_v), dtype=torch.float32, device="cuda")
        sdm.forward_decay(Sp, sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(alpha), sl(dev["beta"]), dev["subkeys"],
                          M, lam, lrun, o, wsd, wo)
        return o, M, lam, lrun

    ones = torch.ones_like(dev["alpha"])
    log("[full] decay variant, alpha = 1")
    o1, M1, lam1, lrun1 = run_decay(ones)
    M2 = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M2)
    o2 = torch.empty_like(o1)
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    sdm.forward(S, dev["q"], dev["k"], dev["v"], ones, dev["beta"], dev["subkeys"], M2, o2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(M1, M2), "alpha = 1: decay variant differs from the plain path"
    assert float(lrun1.abs().max()) == 0.0
    log("[full] decay variant, workload gates, one call and two calls")
    wo = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.int32, device="cuda")
    oa, Ma, lama, lruna = run_decay(dev["alpha"], wo=wo)
    T1 = sh.T // 2 + 5
    ob1, Mb, lamb, lrunb = run_decay(dev["alpha"], 0, T1)
    ob2, Mb, lamb, lrunb = run_decay(dev["alpha"], T1, sh.T, Mb, lamb, lrunb)
    torch.cuda.synchronize()
    L = np.log(inp["alpha"].astype(np.float64)).sum(-1)
    assert np.allclose(lruna.cpu().numpy(), L, rtol=1e-9, atol=0)
    assert np.allclose(lrunb.cpu().numpy(), L, rtol=1e-9, atol=0)
    ob = torch.cat([ob1, ob2], 2).cpu().numpy()
    assert rel_err(ob, oa.cpu().numpy()) < 1e-5
    assert rel_err(SI.widen(from_dev(Mb, sh.mem_dtype), sh.mem_dtype),
                   SI.widen(from_dev(Ma, sh.mem_dtype), sh.mem_dtype)) < 1e-2
    # slots no token wrote keep lam = 0 (their value is still M0 times the whole decay);
    # written ones hold the (negative) log-decay after their last writer
    # (the order pass runs this shape in four parallel token segments: each written slot's
    # lam must be the cumulative log-decay through its latest writer over the whole call)
    gw = wo.cpu().numpy()
    for b, h in ((0, 0), (0, 7)):
        touched = np.zeros(sh.N, bool)
        touched[gw[b, h].ravel()] = True
        lam_h = lama[b, h].cpu().numpy()
        assert np.all(lam_h[~touched] == 0.0) and np.all(lam_h[touched] < 0.0)
        last = np.full(sh.N, -1, np.int64)
        np.maximum.at(last, gw[b, h].ravel(), np.repeat(np.arange(sh.T), sh.W))
        Lc = np.cumsum(np.maximum(np.log(inp["alpha"][b, h].astype(np.float64)), -1000.0))
        assert np.allclose(lam_h[touched], Lc[last[touched]], rtol=1e-9, atol=1e-9), \
            "lam of a written slot is not the log-decay through its latest writer"


@pytest.mark.parametrize("name", list(PLAN))
def test_fullsize_backward(sdm, name):
    """The forward with its log and the recurrence backward at full size, launched as
    ``bench.py --backward`` launches them (addressing of keys and queries, one
    sdm_recurrent_log call, one sdm_recurrent_backward call over all units and tokens). The
    output gradient go is nonzero only on a window [0, P) of every unit: the loss then depends
    only on those tokens, so the oracle's forward, log and backward over the window give every
    gradient of a sampled unit (dv, dalpha, dbeta, both weight gradients and dM0), while past
    the window every token gradient is exactly zero. The walk back over all T tokens must
    restore M0 bit for bit in every unit. P is cut at the first token where the device's slot
    lists differ from the oracle's (a tie), so that both sides differentiate the same slots."""
    import torch
    sh = W_[name]
    units, _, _ = PLAN[name]
    P = min(1024, sh.T)
    log(f"[full] backward {name}: generating inputs")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M)
    M0_dev = M.clone()
    shp_w, shp_r = (sh.B, sh.H, sh.T, sh.W), (sh.B, sh.H, sh.T, sh.R)
    wi = torch.empty(shp_w, dtype=torch.int32, device="cuda")
    wg = torch.empty(shp_w, dtype=torch.float32, device="cuda")
    ri = torch.empty(shp_r, dtype=torch.int32, device="cuda")
    rg = torch.empty(shp_r, dtype=torch.float32, device="cuda")
    sdm.address(S, dev["k"], dev["subkeys"], sh.W, wi, wg)
    sdm.address(S, dev["q"], dev["subkeys"], sh.R, ri, rg)
    torch.cuda.synchronize()
    ref = {}
    for (b, h) in units:
        Up = unit_inputs(inp, sh, b, h, T=P)
        owi, oww, _ = O.address(Up["k"], Up["C1"], Up["C2"], sh.kappa, sh.W)
        ori, orw, _ = O.address(Up["q"], Up["C1"], Up["C2"], sh.kappa, sh.R)
        gw, gr = wi[b, h, :P].cpu().numpy(), ri[b, h, :P].cpu().numpy()
        _, _, fw = compare_indices(gw, owi, Up["k"], Up["C1"], Up["C2"], sh.N)
        _, _, fr = compare_indices(gr, ori, Up["q"], Up["C1"], Up["C2"], sh.N)
        assert not fw and not fr
        diff = np.nonzero((gw != owi).any(1) | (gr != ori).any(1))[0]
        if len(diff):
            P = min(P, int(diff[0]))
        ref[(b, h)] = (Up, owi, oww, ori, orw)
    assert P >= 256, f"{name}: slot lists differ from the oracle's at token {P}"
    rng = np.random.default_rng(29)
    go_h = np.zeros((sh.B, sh.H, sh.T, sh.d_v), np.float32)
    go_h[:, :, :P] = rng.standard_normal((sh.B, sh.H, P, sh.d_v)).astype(np.float32)
    go = to_dev(go_h, "f32")
    del go_h
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    xlog = empty_mem((sh.B, sh.H, sh.T, sh.W, sh.d_v), sh.mem_dtype)
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    log(f"[full] backward {name}: log and backward B={sh.B} H={sh.H} T={sh.T}, go window {P}")
    sdm.recurrent_log(S, wi, wg, ri, rg, dev["v"], dev["alpha"], dev["beta"], M, o, xlog, ws)
    G = torch.zeros((sh.B, sh.H, sh.N, sh.d_v), dtype=torch.float32, device="cuda")
    dv = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    dal = torch.empty((sh.B, sh.H, sh.T), dtype=torch.float32, device="cuda")
    dbe = torch.empty_like(dal)
    dwg = torch.empty(shp_w, dtype=torch.float32, device="cuda")
    drg = torch.empty(shp_r, dtype=torch.float32, device="cuda")
    bws = torch.empty(sdm.backward_workspace_bytes(S), dtype=torch.uint8, device="cuda")
    sdm.recurrent_backward(S, wi, wg, ri, rg, dev["v"], dev["alpha"], dev["beta"], M, xlog, go, G, dv, dal, dbe,
                           dwg, drg, bws)
    torch.cuda.synchronize()
    assert sdm.workspace_error(bws) == 0, "a workgroup of the backward gave up waiting"
    assert torch.equal(M, M0_dev), "the undo over the whole sequence did not restore M0 bit for bit"
    for nm, t in (("dv", dv), ("dalpha", dal), ("dbeta", dbe), ("dwgt", dwg), ("drgt", drg)):
        nz = int(torch.count_nonzero(t[:, :, P:]))
        assert nz == 0, f"{nm}: {nz} nonzero entries past the go window"
    tol = tolerance(sh)
    for (b, h), (Up, owi, oww, ori, orw) in ref.items():
        wwp, rwp = oww[:P].astype(np.float32).astype(np.float64), orw[:P].astype(np.float32).astype(np.float64)
        v, al, be = Up["v"][:P], Up["alpha"][:P], Up["beta"][:P]
        _, MT = O.recurrence(Up["M0"], owi[:P], wwp, ori[:P], rwp, v, al, be, sh.mem_dtype)
        xl = O.recurrence_log(Up["M0"], owi[:P], wwp, v, al, be, sh.mem_dtype)
        g = O.recurrence_backward(MT, xl, owi[:P], wwp, ori[:P], rwp, v, al, be, go[b, h, :P].cpu().numpy()
                                  .astype(np.float64))
        out = {"dv": dv[b, h, :P], "dalpha": dal[b, h, :P], "dbeta": dbe[b, h, :P], "dwgt": dwg[b, h, :P],
               "drgt": drg[b, h, :P], "dM0": G[b, h]}
        errs = {k: rel_err(t.cpu().numpy(), g[k]) for k, t in out.items()}
        log(f"[full] backward {name} unit ({b},{h}): " + " ".join(f"{k} {e:.1e}" for k, e in errs.items()) +
            f" (tol {tol})")
        for k, e in errs.items():
            assert e < tol, k
