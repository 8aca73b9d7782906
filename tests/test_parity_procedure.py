"""The full-size parity procedure (``parity.unit_parity``) on the CPU, with the oracle's own
results standing in for the device's: it must pass them, count a planted tie and follow the
tied slot lists without a cascade, and fail a wrong slot or a wrong output."""
import numpy as np

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import SharedDir, rel_err, unit_parity

SH = SI.WORKLOADS["small"].replace(B=1, H=2, T=96, N=1024, kappa=8, W=8, R=8, mem_dtype="bf16")


def _device_like(inp, sh, swap=None):
    """The oracle's slots, outputs and table as a device would return them (o float32, the
    table in its dtype). swap = (token, a, b): the write list of unit (0, 0) at that token
    takes positions a and b in the other order (a tie broken the other way)."""
    o = np.zeros((sh.B, sh.H, sh.T, sh.d_v), np.float32)
    M = np.zeros((sh.B, sh.H, sh.N, sh.d_v), np.uint16)
    wi = np.zeros((sh.B, sh.H, sh.T, sh.W), np.int32)
    ri = np.zeros((sh.B, sh.H, sh.T, sh.R), np.int32)
    for h in range(sh.H):
        sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
        k = SI.widen(inp["k"][0, h], sh.in_dtype)
        q = SI.widen(inp["q"][0, h], sh.in_dtype)
        w_i, _, _ = O.address(k, sk[0], sk[1], sh.kappa, sh.W)
        r_i, _, _ = O.address(q, sk[0], sk[1], sh.kappa, sh.R)
        if swap and h == 0:
            t, a, b = swap
            w_i[t, [a, b]] = w_i[t, [b, a]]
        ww, _ = O.slot_weights(k, sk[0], sk[1], w_i)
        rw, _ = O.slot_weights(q, sk[0], sk[1], r_i)
        oo, MM = O.recurrence(SI.widen(inp["M0"][h], sh.mem_dtype), w_i, ww, r_i, rw,
                              SI.widen(inp["v"][0, h], sh.in_dtype), inp["alpha"][0, h].astype(np.float64),
                              inp["beta"][0, h].astype(np.float64), sh.mem_dtype)
        o[0, h], M[0, h] = oo, SI.cast(MM.astype(np.float32), "bf16")
        wi[0, h], ri[0, h] = w_i, r_i
    return o, M, wi, ri


def _run(inp, sh, o, M, wi, ri):
    with SharedDir() as sd:
        for n in ("q", "k", "v", "alpha", "beta", "subkeys", "M0"):
            sd.save(n, inp[n])
        sd.save("o", o)
        sd.save("M", M)
        sd.save("widx", wi)
        sd.save("ridx", ri)
        return [unit_parity(dict(dir=sd.path, shape=sh, b=0, h=h)) for h in range(sh.H)]


def test_procedure_passes_the_oracle_itself():
    inp = SI.make_inputs(SH)
    res = _run(inp, SH, *_device_like(inp, SH))
    for r in res:
        assert not r["fails"] and r["ties"] == 0 and r["untouched_ok"]
        assert r["err_o"] < 1e-6 and r["err_M"] == 0.0


def test_procedure_follows_a_tie():
    """Sub-keys 0 and 1 of the second half made equal: slots i*s + 0 and i*s + 1 then score
    exactly alike, the oracle ranks the lower slot first, and a device that ranked them the
    other way is counted as a tie and checked on its own lists."""
    inp = SI.make_inputs(SH)
    inp["subkeys"][0, 1, 1] = inp["subkeys"][0, 1, 0]
    sk = SI.widen(inp["subkeys"][0], SH.in_dtype)
    k = SI.widen(inp["k"][0, 0], SH.in_dtype)
    wi, _, _ = O.address(k, sk[0], sk[1], SH.kappa, SH.W)
    s = SH.s
    hit = None
    for t in range(SH.T):
        row = wi[t].tolist()
        for a, n in enumerate(row):
            if n % s == 0 and n + 1 in row:
                hit = (t, a, row.index(n + 1))
                break
        if hit:
            break
    assert hit, "no token selects both tied slots"
    res = _run(inp, SH, *_device_like(inp, SH, swap=hit))
    assert not res[0]["fails"] and res[0]["ties"] == 2 and res[0]["differs"]
    assert res[0]["err_o"] < 1e-6 and res[0]["err_M"] == 0.0


def test_procedure_fails_a_wrong_slot_and_a_wrong_output():
    inp = SI.make_inputs(SH)
    o, M, wi, ri = _device_like(inp, SH)
    bad = wi.copy()
    bad[0, 1, 10, 3] = (bad[0, 1, 10, 3] + 517) % SH.N
    res = _run(inp, SH, o, M, bad, ri)
    assert res[1]["fails"] and not res[0]["fails"]
    o2 = o.copy()
    o2[0, 0, 50] *= 1.5
    res = _run(inp, SH, o2, M, wi, ri)
    assert res[0]["err_o"] > 2e-2 and res[1]["err_o"] < 1e-6
    assert rel_err(o2[0, 1], o[0, 1]) == 0.0
