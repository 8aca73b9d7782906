"""Decode steps captured as a HIP graph (the launch-bound loop of a serving engine) give, on
every replay, bit for bit what the same steps give launched one call at a time:
sdm_decode_step records a single kernel launch on the caller's stream, no allocation and
no memory fill."""
import numpy as np
import pytest

import sdm_inputs as SI
from parity import from_dev, lib_shape, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()
    return S


@pytest.mark.parametrize("mem_dtype", ["bf16", "f32"])
def test_decode_graph_replays(sdm, mem_dtype):
    import torch
    sh = SI.WORKLOADS["decode"].replace(B=4, H=4, N=4096, d_k=64, d_v=64, kappa=8, W=8, R=8, mem_dtype=mem_dtype,
                                        prefill=0)
    inp = SI.make_inputs(sh.replace(T=1))
    steps = 4
    bank = SI.make_decode_bank(sh, steps)
    S = lib_shape(sh, T=1)
    sub = to_dev(inp["subkeys"], sh.in_dtype)
    M0 = to_dev(inp["M0"], sh.mem_dtype)
    tok = [{k: to_dev(bank[k][i], sh.in_dtype if k in ("q", "k", "v") else "f32") for k in ("q", "k", "v", "alpha",
                                                                                           "beta")}
           for i in range(steps)]
    mdt = torch.bfloat16 if mem_dtype == "bf16" else torch.float32
    Me = torch.empty((sh.B, sh.H, sh.N, sh.d_v), dtype=mdt, device="cuda")
    Mg = torch.empty_like(Me)
    sdm.init_from_M0(S, M0, Me)
    sdm.init_from_M0(S, M0, Mg)
    oe = torch.empty((steps, sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    og = torch.empty_like(oe)

    def run(M, o, i):
        t = tok[i]
        sdm.decode_step(S, t["q"], t["k"], t["v"], t["alpha"], t["beta"], sub, M, o[i])

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            run(Mg, og, i)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between the replays: the same steps, one call at a time, on the other table
        for i in range(steps):
            run(Me, oe, i)
        torch.cuda.synchronize()
        og.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(og, oe), f"replay {rep}: outputs differ"
        assert torch.equal(Mg, Me), f"replay {rep}: tables differ"
        log(f"[decode graph] {mem_dtype} replay {rep}: outputs and table equal to the eager steps")
    assert np.isfinite(oe.cpu().numpy()).all()


@pytest.mark.parametrize("mem_dtype,d_v,W", [("bf16", 128, 16), ("f32", 256, 16), ("bf16", 64, 8), ("f32", 256, 64)])
def test_decode_reads_own_writes(sdm, mem_dtype, d_v, W):
    """q = k: every read slot is one of the token's write slots, so the output is the weighted
    read of the rows just written (the fused step's path for read rows it wrote itself).
    Checked against the oracle's rule on the device's slot lists (sdm_address of the same
    vectors), with the oracle's float64 weights of those slots."""
    import oracle.sdm_oracle as O
    import torch
    sh = SI.WORKLOADS["decode"].replace(B=2, H=4, N=4096, d_k=64, d_v=d_v, kappa=8, W=W, R=W, mem_dtype=mem_dtype,
                                        prefill=0)
    inp = SI.make_inputs(sh.replace(T=1))
    S = lib_shape(sh, T=1)
    dev = {k: to_dev(inp[k], sh.in_dtype) for k in ("k", "v", "subkeys")}
    dev["alpha"], dev["beta"] = to_dev(inp["alpha"], "f32"), to_dev(inp["beta"], "f32")
    mdt = torch.bfloat16 if mem_dtype == "bf16" else torch.float32
    M = torch.empty((sh.B, sh.H, sh.N, sh.d_v), dtype=mdt, device="cuda")
    sdm.init_from_M0(S, to_dev(inp["M0"], sh.mem_dtype), M)
    o = torch.empty((sh.B, sh.H, 1, sh.d_v), dtype=torch.float32, device="cuda")
    sdm.decode_step(S, dev["k"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, o)
    wi = torch.empty((sh.B, sh.H, 1, W), dtype=torch.int32, device="cuda")
    wg = torch.empty((sh.B, sh.H, 1, W), dtype=torch.float32, device="cuda")
    sdm.address(S, dev["k"], dev["subkeys"], W, wi, wg)
    torch.cuda.synchronize()
    go, gw = o.cpu().numpy(), wi.cpu().numpy()
    gM = SI.widen(from_dev(M, sh.mem_dtype), sh.mem_dtype)
    worst_o = worst_m = 0.0
    for b in range(sh.B):
        for h in range(sh.H):
            sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
            x = SI.widen(inp["k"][b, h], sh.in_dtype)  # [1, d_k]
            sl = gw[b, h]                                # [1, W]
            wts, _ = O.slot_weights(x, sk[0], sk[1], sl)
            M0 = SI.widen(inp["M0"][h], sh.mem_dtype)
            ro, rM = O.recurrence(M0, sl, wts, sl, wts, SI.widen(inp["v"][b, h], sh.in_dtype),
                                  inp["alpha"][b, h].astype(np.float64), inp["beta"][b, h].astype(np.float64),
                                  sh.mem_dtype)
            worst_o = max(worst_o, float(np.max(np.abs(go[b, h] - ro)) / max(np.max(np.abs(ro)), 1e-30)))
            worst_m = max(worst_m, float(np.max(np.abs(gM[b, h] - rM)) / max(np.max(np.abs(rM)), 1e-30)))
    log(f"[decode q=k] {mem_dtype} d_v={d_v} W={W}: rel err o {worst_o:.2e}, table {worst_m:.2e}")
    tol = 1e-4 if mem_dtype == "f32" else 2e-2
    assert worst_o < tol and worst_m < tol
