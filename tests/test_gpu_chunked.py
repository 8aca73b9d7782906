"""Chunkwise two-phase recurrence on the GPU against the oracle's chunkwise form (same
chunk length, same rounding point: written rows rounded once per chunk) and, for float32
tables, against the token-by-token rule. Slots and weights come from the oracle's
addressing; the crowded cases (256- and 1024-slot tables, 16 or 32 slots per token) write
every slot several times per chunk and again in the next chunk, so the per-slot chains and
the interactions are long and most rows gathered ahead of their chunk are replaced by the
previous chunk's write-back."""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import empty_mem, from_dev, lib_shape, log, rel_err, to_dev, tolerance

pytestmark = pytest.mark.gpu

CHUNK = 64
W_ = SI.WORKLOADS
CASES = {
    "tiny_fp32": W_["tiny_fp32"],
    "small_T200": W_["small"].replace(B=1, H=2, T=200),
    "layer_1p4b_T150": W_["layer_1p4b"].replace(B=1, H=2, T=150),
    "layer_8b_T300": W_["layer_8b_long"].replace(B=1, H=2, T=300),
    "crowded_N256": SI.Shape("crowded_N256", 1, 2, 160, 256, 32, 32, 16, 16, 16, "f32", "f32", 9),
    # consecutive chunks rewrite the same rows: the rows a chunk gathers early are mostly stale
    "crowded_N1024_bf16": SI.Shape("crowded_N1024_bf16", 1, 2, 300, 1024, 64, 128, 32, 32, 32, "bf16", "bf16", 10),
    "crowded_N1024_f32": SI.Shape("crowded_N1024_f32", 1, 3, 200, 1024, 64, 64, 32, 32, 32, "f32", "f32", 11),
    # edges: one token; a few tokens with lists that are not a multiple of four (the narrow
    # slot loads, two occurrences per lane); float32 inputs with a bf16 table
    "edge_T1": W_["small"].replace(B=1, H=2, T=1),
    "edge_T5_W3_R5": W_["small"].replace(B=2, H=1, T=5, W=3, R=5),
    "in_f32_table_bf16_T130": W_["layer_1p4b"].replace(B=1, H=2, T=130, in_dtype="f32"),
}


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()
    return S


@pytest.mark.parametrize("name", list(CASES))
def test_chunked(sdm, name):
    import torch
    sh = CASES[name]
    log(f"[chunked] {name}")
    inp = SI.make_inputs(sh)
    S = lib_shape(sh)
    shp_w, shp_r = (sh.B, sh.H, sh.T, sh.W), (sh.B, sh.H, sh.T, sh.R)
    widx, wgt = np.zeros(shp_w, np.int32), np.zeros(shp_w, np.float32)
    ridx, rgt = np.zeros(shp_r, np.int32), np.zeros(shp_r, np.float32)
    ref = {}
    for b in range(sh.B):
        for h in range(sh.H):
            sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
            wi, ww, _ = O.address(SI.widen(inp["k"][b, h], sh.in_dtype), sk[0], sk[1], sh.kappa, sh.W)
            ri, rw, _ = O.address(SI.widen(inp["q"][b, h], sh.in_dtype), sk[0], sk[1], sh.kappa, sh.R)
            ww, rw = ww.astype(np.float32), rw.astype(np.float32)
            widx[b, h], wgt[b, h], ridx[b, h], rgt[b, h] = wi, ww, ri, rw
            args = (SI.widen(inp["M0"][h], sh.mem_dtype), wi, ww.astype(np.float64), ri, rw.astype(np.float64),
                    SI.widen(inp["v"][b, h], sh.in_dtype), inp["alpha"][b, h].astype(np.float64),
                    inp["beta"][b, h].astype(np.float64))
            oc, Mc = O.chunkwise_recurrence(*args, CHUNK, sh.mem_dtype)
            seq = O.recurrence(*args, sh.mem_dtype) if sh.mem_dtype == "f32" else None
            ref[(b, h)] = (oc, Mc, seq)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, to_dev(inp["M0"], sh.mem_dtype), M)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes_chunked(S), dtype=torch.uint8, device="cuda")
    sdm.recurrent_chunked(S, to_dev(widx, "i32"), to_dev(wgt, "f32"), to_dev(ridx, "i32"), to_dev(rgt, "f32"),
                          to_dev(inp["v"], sh.in_dtype), to_dev(inp["alpha"], "f32"), to_dev(inp["beta"], "f32"),
                          M, o, ws)
    torch.cuda.synchronize()
    tol = tolerance(sh)
    go = o.cpu().numpy()
    gM = SI.widen(from_dev(M, sh.mem_dtype), sh.mem_dtype)
    for (b, h), (oc, Mc, seq) in ref.items():
        eo, eM = rel_err(go[b, h], oc), rel_err(gM[b, h], Mc)
        msg = f"[chunked] {name} ({b},{h}): o {eo:.2e} M {eM:.2e}"
        if seq is not None:
            es, eMs = rel_err(go[b, h], seq[0]), rel_err(gM[b, h], seq[1])
            msg += f"; against the token-by-token rule: o {es:.2e} M {eMs:.2e}"
            assert es < tol and eMs < tol
        log(msg + f" (tol {tol})")
        assert eo < tol and eM < tol
