"""The HIP path at full workload sizes, in the launch configuration the benchmark times,
checked against the oracle (one unit per task in a pool of worker processes):

* forward, every workload but decode: every unit over the whole sequence -- slot lists
  position by position with ties counted, then o at every token and the whole final table
  against the oracle run on the device's slot lists with the oracle's own float64 weights
  (a tie that picked an equally scored slot does not cascade), rows no token writes
  bit-identical to M0; the same sequence in two calls equals one call bit for bit;
* the chunkwise two-phase recurrence: the same procedure for every unit against the
  oracle's chunkwise form, and against the token-by-token rule within the tolerance;
* decode: one step over all 64 x 16 tables, every unit checked, after a prefill of four
  sequences that is itself checked in full;
* the whole-table decay variant at the 8B-scale shape: bit-identical to the written-rows
  path when no gate decays, the running log-decay and the carried state consistent;
* the backward, with an output gradient on every token: in every unit every gradient
  against the oracle's forward, log and reverse walk on the device's slots and weights,
  and M0 restored bit for bit by the walk back over the whole sequence.

Per-workload records (units and token-heads compared, tie counts, worst errors) are
written to parity_fullsize.json in $SDM_PARITY_RECORD_DIR.
"""
import time

import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import (SharedDir, compare_indices, empty_mem, from_dev, lib_shape, log, pool, pool_size, rel_err,
                    summarise, to_dev, tolerance, unit_backward_parity, unit_parity, write_record)

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
    sl = lambda t: t[:, :, T_lo:T_hi].clone()  # a fresh (aligned) buffer even where the slice is contiguous
    o = torch.empty((sh.B, sh.H, T_hi - T_lo, sh.d_v), dtype=torch.float32, device="cuda")
    wo = torch.empty((sh.B, sh.H, T_hi - T_lo, sh.W), dtype=torch.int32, device="cuda")
    ro = torch.empty((sh.B, sh.H, T_hi - T_lo, sh.R), dtype=torch.int32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(Sp), dtype=torch.uint8, device="cuda")
    sdm.forward(Sp, sl(dev["q"]), sl(dev["k"]), sl(dev["v"]), sl(dev["alpha"]), sl(dev["beta"]), dev["subkeys"], M,
                o, ws, wo, ro)
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    return o, wo, ro


def run_pool(tasks, label):
    """Runs unit_parity over the tasks in the oracle pool, logging each finished unit."""
    results = []
    t0 = time.time()
    for r in pool().imap_unordered(unit_parity, tasks, chunksize=1):
        results.append(r)
        if len(results) % max(1, len(tasks) // 8) == 0 or len(results) == len(tasks):
            log(f"[full] {label}: {len(results)}/{len(tasks)} units checked ({time.time() - t0:.0f} s)")
    return sorted(results, key=lambda r: (r["b"], r["h"]))


def check_results(name, sh, results, tol, extra=None):
    fails = [(r["b"], r["h"], r["fails"]) for r in results if r["fails"]]
    assert not fails, f"{name}: slot lists differ from the oracle's beyond ties: {fails[:3]}"
    rec = summarise(name, sh, results, tol, extra)
    write_record(rec)
    log(f"[full] {name}: {rec['units_compared']} units, {rec['token_heads_compared']} token-heads, "
        f"tie positions {rec['tie_positions']} ({rec['set_changing_tie_tokens']} tokens with a changed slot set, "
        f"{rec['units_with_ties']} units re-run on the device's slots); rel err o {rec['max_rel_err_o']:.2e}, "
        f"table {rec['max_rel_err_table']:.2e} (tol {tol})")
    assert rec["untouched_rows_bit_identical"], f"{name}: a row no token wrote differs from the start table"
    assert rec["max_rel_err_o"] < tol and rec["max_rel_err_table"] < tol
    return rec


@pytest.mark.oracle_pool
@pytest.mark.parametrize("name", ["tiny_fp32"] + list(PLAN))
def test_fullsize_forward(sdm, name):
    """Every unit over the whole sequence, in the launch the benchmark times (one
    sdm_forward call over all units): slot lists position by position (ties counted), then
    o at every token and the whole final table against the oracle run on the device's slot
    lists (the oracle's own lists wherever no tie occurred), rows no token writes bit-equal
    to M0. The per-workload record (tie counts, worst errors) goes to
    parity_fullsize.json in $SDM_PARITY_RECORD_DIR."""
    import torch
    sh = W_[name]
    log(f"[full] {name}: generating inputs")
    inp = SI.make_inputs(sh)
    dev = upload(inp, sh)
    S = lib_shape(sh)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M)
    log(f"[full] {name}: forward B={sh.B} H={sh.H} T={sh.T}")
    o, wo, ro = forward(sdm, sh, dev, S, M)
    tol = tolerance(sh)
    need = M.numel() * M.element_size() + o.numel() * 4
    with SharedDir(need) as sd:
        for n in ("q", "k", "v", "alpha", "beta", "subkeys", "M0"):
            sd.save(n, inp[n])
        sd.save("o", o.cpu().numpy())
        sd.save("M", from_dev(M, sh.mem_dtype))
        sd.save("widx", wo.cpu().numpy())
        sd.save("ridx", ro.cpu().numpy())
        tasks = [dict(dir=sd.path, shape=sh, b=b, h=h) for b in range(sh.B) for h in range(sh.H)]
        log(f"[full] {name}: oracle over {len(tasks)} units in {pool_size()} workers")
        results = run_pool(tasks, name)
    check_results(name, sh, results, tol)
    # the same sequence in two calls on the carried table: bit for bit on the pipeline; where
    # the forward runs the chunkwise form (float32 tables, many units) the float32 sums of
    # its first phase can be ordered differently from run to run, so up to that order
    M2 = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, dev["M0"], M2)
    T1 = sh.T // 2 + 3
    o1, _, _ = forward(sdm, sh, dev, S, M2, 0, T1)
    o2, _, _ = forward(sdm, sh, dev, S, M2, T1, sh.T)
    if sdm.forward_uses_chunkwise(S):
        e_o = rel_err(torch.cat([o1, o2], 2).cpu().numpy(), o.cpu().numpy())
        e_m = rel_err(M2.float().cpu().numpy(), M.float().cpu().numpy())
        log(f"[full] {name}: split call against one call (chunkwise form): o {e_o:.1e}, table {e_m:.1e}")
        assert e_o < 1e-5 and e_m < 1e-5, "split call differs from the single call beyond float32 summation order"
    else:
        assert torch.equal(torch.cat([o1, o2], 2), o), "split call differs from the single call"
        assert torch.equal(M2, M), "carried table differs"


@pytest.mark.oracle_pool
@pytest.mark.parametrize("name", list(PLAN))
def test_fullsize_chunked(sdm, name):
    """The chunkwise two-phase recurrence at full size, launched as ``bench.py --chunked``
    launches it (addressing of keys and queries, then one sdm_recurrent_chunked call over all
    units): every unit over the whole sequence by the full-size parity procedure against the
    oracle's chunkwise form at chunk length 64 (READING R26 fixes where it rounds a bf16
    table), and its outputs and table also against the token-by-token rule within the
    tolerance."""
    import torch
    sh = W_[name]
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
    with SharedDir(M.numel() * M.element_size() + o.numel() * 4) as sd:
        for n in ("q", "k", "v", "alpha", "beta", "subkeys", "M0"):
            sd.save(n, inp[n])
        sd.save("o", o.cpu().numpy())
        sd.save("M", from_dev(M, sh.mem_dtype))
        sd.save("widx", wi.cpu().numpy())
        sd.save("ridx", ri.cpu().numpy())
        tasks = [dict(dir=sd.path, shape=sh, b=b, h=h, chunk=64, token_rule=True) for b in range(sh.B)
                 for h in range(sh.H)]
        log(f"[full] chunked {name}: oracle over {len(tasks)} units in {pool_size()} workers")
        results = run_pool(tasks, f"chunked {name}")
    tok_o = max(r["err_o_token_rule"] for r in results)
    tok_m = max(r["err_M_token_rule"] for r in results)
    check_results(f"{name}_chunked", sh, results, tol,
                  {"form": "chunkwise, chunk 64", "max_rel_err_o_vs_token_rule": tok_o,
                   "max_rel_err_table_vs_token_rule": tok_m})
    log(f"[full] chunked {name}: against the token-by-token rule: o {tok_o:.2e}, table {tok_m:.2e}")
    assert tok_o < tol and tok_m < tol


@pytest.mark.oracle_pool
def test_fullsize_decode(sdm):
    """One decode step over all 64 x 16 tables of the decode workload (the launch the
    benchmark times). Sequences 0, 21, 42 and 63 are first prefilled with their 4096 prior
    tokens (one sdm_forward call each); the others hold M0. Checked against the oracle:

    * the prefill of those 4 sequences (64 units): slot lists, every output and the whole
      table after the prefill, by the full-size parity procedure;
    * the decode step in every one of the 1024 units: the device's slot lists of the decode
      token (sdm_address, the selection the fused step uses) against the oracle's, then the
      oracle's decode step on the rows those lists name, taken from a copy of the table made
      just before the step: o and every written row; every row the step changed is one of
      the token's write slots (so the rest of each table is untouched)."""
    import torch
    sh = W_["decode"]
    P = sh.prefill
    PRE = (0, 21, 42, 63)
    log(f"[full] decode: B={sh.B} H={sh.H} N={sh.N}, prefill {P} tokens on sequences {PRE}")
    params = SI.make_inputs(sh)
    dev = upload(params, sh)
    S1 = lib_shape(sh, T=1)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S1, dev["M0"], M)
    Sp = lib_shape(sh, B=1, T=P)
    ws = torch.empty(sdm.workspace_bytes(Sp), dtype=torch.uint8, device="cuda")
    pre = {b: SI.make_prefill(sh, b) for b in PRE}
    o_pre = torch.empty((len(PRE), sh.H, P, sh.d_v), dtype=torch.float32, device="cuda")
    w_pre = torch.empty((len(PRE), sh.H, P, sh.W), dtype=torch.int32, device="cuda")
    r_pre = torch.empty((len(PRE), sh.H, P, sh.R), dtype=torch.int32, device="cuda")
    for i, b in enumerate(PRE):
        t = {n: to_dev(pre[b][n], sh.in_dtype if n in ("q", "k", "v") else "f32")
             for n in ("q", "k", "v", "alpha", "beta")}
        sdm.forward(Sp, t["q"], t["k"], t["v"], t["alpha"], t["beta"], dev["subkeys"], M[b:b + 1], o_pre[i:i + 1],
                    ws, w_pre[i:i + 1], r_pre[i:i + 1])
    torch.cuda.synchronize()
    assert sdm.workspace_error(ws) == 0
    snap = M.clone()
    o = torch.empty((sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    log("[full] decode: one step over all units")
    sdm.decode_step(S1, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, o)
    wi = torch.empty((sh.B, sh.H, 1, sh.W), dtype=torch.int32, device="cuda")
    wg = torch.empty((sh.B, sh.H, 1, sh.W), dtype=torch.float32, device="cuda")
    ri = torch.empty((sh.B, sh.H, 1, sh.R), dtype=torch.int32, device="cuda")
    rg = torch.empty((sh.B, sh.H, 1, sh.R), dtype=torch.float32, device="cuda")
    sdm.address(S1, dev["k"], dev["subkeys"], sh.W, wi, wg)
    sdm.address(S1, dev["q"], dev["subkeys"], sh.R, ri, rg)
    torch.cuda.synchronize()
    tol = tolerance(sh)
    # 1. the prefill of the four sequences, every unit in full
    with SharedDir(len(PRE) * sh.H * sh.N * sh.d_v * 2) as sd:
        for n in ("q", "k", "v", "alpha", "beta"):
            sd.save(n, np.concatenate([pre[b][n] for b in PRE], 0))
        sd.save("subkeys", params["subkeys"])
        sd.save("M0", params["M0"])
        sd.save("o", o_pre.cpu().numpy())
        sd.save("M", from_dev(snap[list(PRE)], sh.mem_dtype))
        sd.save("widx", w_pre.cpu().numpy())
        sd.save("ridx", r_pre.cpu().numpy())
        tasks = [dict(dir=sd.path, shape=sh.replace(B=len(PRE), T=P), b=i, h=h) for i in range(len(PRE))
                 for h in range(sh.H)]
        log(f"[full] decode: oracle prefill over {len(tasks)} units in {pool_size()} workers")
        res_pre = run_pool(tasks, "decode prefill")
    fails = [(r["b"], r["h"], r["fails"]) for r in res_pre if r["fails"]]
    assert not fails, fails[:3]
    # 2. the decode step in every unit, on the rows its slot lists name
    gw = wi[:, :, 0].cpu().numpy().astype(np.int64)
    gr = ri[:, :, 0].cpu().numpy().astype(np.int64)
    slots = torch.from_numpy(np.concatenate([gw, gr], -1)).cuda()            # [B, H, W + R]
    idx = slots[..., None].expand(-1, -1, -1, sh.d_v)
    before = SI.widen(from_dev(torch.gather(snap, 2, idx).contiguous(), sh.mem_dtype), sh.mem_dtype)
    after = SI.widen(from_dev(torch.gather(M, 2, idx).contiguous(), sh.mem_dtype), sh.mem_dtype)
    changed_ok = True
    for b in range(sh.B):
        ch = (M[b] != snap[b]).any(-1)                                         # [H, N]
        for h in range(sh.H):
            rows = torch.nonzero(ch[h]).flatten().cpu().numpy()
            changed_ok &= bool(np.isin(rows, gw[b, h]).all())
    assert changed_ok, "the decode step changed a row outside the token's write slots"
    go = o[:, :, 0].cpu().numpy()
    ties = set_changes = differs = 0
    worst_o = worst_m = 0.0
    for b in range(sh.B):
        for h in range(sh.H):
            sk = SI.widen(params["subkeys"][h], sh.in_dtype)
            C1, C2 = sk[0], sk[1]
            q1 = SI.widen(params["q"][b, h], sh.in_dtype)
            k1 = SI.widen(params["k"][b, h], sh.in_dtype)
            v1 = SI.widen(params["v"][b, h], sh.in_dtype)
            oi_w, _, _ = O.address(k1, C1, C2, sh.kappa, sh.W)
            oi_r, _, _ = O.address(q1, C1, C2, sh.kappa, sh.R)
            tw, cw, fw = compare_indices(gw[b, h][None], oi_w, k1, C1, C2, sh.N)
            tr, cr, fr = compare_indices(gr[b, h][None], oi_r, q1, C1, C2, sh.N)
            assert not fw and not fr, (b, h, fw + fr)
            ties += tw + tr
            set_changes += bool(cw or cr)
            differs += bool((gw[b, h] != oi_w[0]).any() or (gr[b, h] != oi_r[0]).any())
            # the rule touches only the listed rows: run it on a table of just those rows
            lst = np.concatenate([gw[b, h], gr[b, h]])
            uniq, first = np.unique(lst, return_index=True)
            sub = before[b, h][first]
            loc = {int(n): i for i, n in enumerate(uniq)}
            lw = np.array([[loc[int(n)] for n in gw[b, h]]])
            lr = np.array([[loc[int(n)] for n in gr[b, h]]])
            ww, _ = O.slot_weights(k1, C1, C2, gw[b, h][None])
            rw, _ = O.slot_weights(q1, C1, C2, gr[b, h][None])
            o_ref, sub_ref = O.recurrence(sub, lw, ww, lr, rw, v1, np.array([float(params["alpha"][b, h, 0])]),
                                          np.array([float(params["beta"][b, h, 0])]), sh.mem_dtype)
            worst_o = max(worst_o, rel_err(go[b, h], o_ref[0]))
            worst_m = max(worst_m, rel_err(after[b, h][first], sub_ref))
    rec = summarise("decode", sh, res_pre, tol, {
        "prefill_sequences_checked": list(PRE),
        "decode_units_compared": sh.B * sh.H,
        "decode_tie_positions": ties,
        "decode_units_with_set_changing_ties": set_changes,
        "decode_units_with_ties": differs,
        "decode_max_rel_err_o": worst_o,
        "decode_max_rel_err_written_rows": worst_m,
    })
    write_record(rec)
    log(f"[full] decode: prefill of {len(PRE)} sequences: rel err o {rec['max_rel_err_o']:.2e}, table "
        f"{rec['max_rel_err_table']:.2e}, tie positions {rec['tie_positions']}; decode step over {sh.B * sh.H} "
        f"units: rel err o {worst_o:.2e}, written rows {worst_m:.2e}, tie positions {ties} (tol {tol})")
    assert rec["untouched_rows_bit_identical"]
    assert rec["max_rel_err_o"] < tol and rec["max_rel_err_table"] < tol
    assert worst_o < tol and worst_m < tol


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


@pytest.mark.oracle_pool
@pytest.mark.parametrize("name", list(PLAN))
def test_fullsize_backward(sdm, name):
    """The forward with its log and the recurrence backward at full size, launched as
    ``bench.py --backward`` launches them (addressing of keys and queries, one
    sdm_recurrent_log call, one sdm_recurrent_backward call over all units and tokens), with
    an output gradient over every token: in every unit, the device's slot lists against the
    oracle's addressing (ties counted), then every gradient (dv, dalpha, dbeta, the weight
    gradients and dM0) against the oracle's forward, log and reverse walk on the device's
    slots and weights; the walk back over all T tokens must restore M0 bit for bit."""
    import torch
    sh = W_[name]
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
    go = torch.randn((sh.B, sh.H, sh.T, sh.d_v), device="cuda", generator=torch.Generator("cuda").manual_seed(29))
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    xlog = empty_mem((sh.B, sh.H, sh.T, sh.W, sh.d_v), sh.mem_dtype)
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    log(f"[full] backward {name}: log and backward B={sh.B} H={sh.H} T={sh.T}")
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
    del xlog
    assert sdm.workspace_error(bws) == 0, "a workgroup of the backward gave up waiting"
    assert torch.equal(M, M0_dev), "the undo over the whole sequence did not restore M0 bit for bit"
    del M, M0_dev
    tol = tolerance(sh)
    need = G.numel() * 4 + 2 * go.numel() * 4
    with SharedDir(need) as sd:
        for n in ("q", "k", "v", "alpha", "beta", "subkeys", "M0"):
            sd.save(n, inp[n])
        for n, t in (("widx", wi), ("wgt", wg), ("ridx", ri), ("rgt", rg), ("go", go), ("dv", dv), ("dalpha", dal),
                     ("dbeta", dbe), ("dwgt", dwg), ("drgt", drg), ("G", G)):
            sd.save(n, t.cpu().numpy())
        del G
        tasks = [dict(dir=sd.path, shape=sh, b=b, h=h) for b in range(sh.B) for h in range(sh.H)]
        log(f"[full] backward {name}: oracle over {len(tasks)} units in {pool_size()} workers")
        results = []
        t0 = time.time()
        for r in pool().imap_unordered(unit_backward_parity, tasks, chunksize=1):
            results.append(r)
            if len(results) % max(1, len(tasks) // 8) == 0 or len(results) == len(tasks):
                log(f"[full] backward {name}: {len(results)}/{len(tasks)} units checked ({time.time() - t0:.0f} s)")
    fails = [(r["b"], r["h"], r["fails"]) for r in results if r["fails"]]
    assert not fails, f"{name}: slot lists differ from the oracle's beyond ties: {fails[:3]}"
    worst = {}
    for r in results:
        for n, e in r["errs"].items():
            worst[n] = max(worst.get(n, 0.0), e)
    rec = {"workload": f"{name}_backward", "units_compared": len(results),
           "token_heads_compared": int(sum(r["tokens"] for r in results)),
           "tie_positions": int(sum(r["ties"] for r in results)),
           "max_rel_err": worst, "tolerance": tol, "m0_restored_bit_for_bit": True,
           "oracle_workers": pool_size(),
           "form": "recurrence backward on the device's slots and float32 weights, output gradient on every token"}
    write_record(rec)
    log(f"[full] backward {name}: {len(results)} units, every token: " +
        " ".join(f"{n} {e:.1e}" for n, e in worst.items()) + f" (tol {tol}); tie positions {rec['tie_positions']}")
    for n, e in worst.items():
        assert e < tol, n
