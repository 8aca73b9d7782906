"""Addressing backward on the GPU against the oracle: gradients of the selected slots'
softmax weights with respect to the addressed rows (keys for the write slots, queries for
the read slots) and the sub-keys, the selection held fixed (the oracle's own). Both calls
add into one sub-key gradient, as a caller would."""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import from_dev, lib_shape, log, rel_err, to_dev

pytestmark = pytest.mark.gpu

W_ = SI.WORKLOADS
CASES = {
    "tiny_fp32": W_["tiny_fp32"],
    "small_T96": W_["small"].replace(B=2, H=2, T=96),
    "layer_1p4b_T80": W_["layer_1p4b"].replace(B=2, H=2, T=80),
    "layer_8b_T200": W_["layer_8b_long"].replace(B=1, H=2, T=200),
}


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()
    return S


@pytest.mark.parametrize("name", list(CASES))
def test_address_backward(sdm, name):
    import torch
    sh = CASES[name]
    log(f"[address backward] {name}")
    inp = SI.make_inputs(sh)
    S = lib_shape(sh)
    s = int(round(sh.N ** 0.5))
    hd = sh.d_k // 2
    rng = np.random.default_rng(29)
    ref_dsub = np.zeros((sh.H, 2, s, hd))
    calls = []
    for xname, n_sel in (("k", sh.W), ("q", sh.R)):
        idx = np.zeros((sh.B, sh.H, sh.T, n_sel), np.int32)
        w = np.zeros((sh.B, sh.H, sh.T, n_sel), np.float32)
        dw = rng.standard_normal((sh.B, sh.H, sh.T, n_sel)).astype(np.float32)
        ref_dx = np.zeros((sh.B, sh.H, sh.T, sh.d_k))
        for h in range(sh.H):
            sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
            for b in range(sh.B):
                x = SI.widen(inp[xname][b, h], sh.in_dtype)
                i, ww, _ = O.address(x, sk[0], sk[1], sh.kappa, n_sel)
                idx[b, h], w[b, h] = i, ww
                dx, dC1, dC2 = O.address_backward(x, sk[0], sk[1], i, w[b, h].astype(np.float64),
                                                  dw[b, h].astype(np.float64))
                ref_dx[b, h] = dx
                ref_dsub[h, 0] += dC1
                ref_dsub[h, 1] += dC2
        calls.append((xname, n_sel, idx, w, dw, ref_dx))
    dsub = torch.zeros((sh.H, 2, s, hd), dtype=torch.float32, device="cuda")
    sub = to_dev(inp["subkeys"], sh.in_dtype)
    for xname, n_sel, idx, w, dw, ref_dx in calls:
        dx = torch.empty((sh.B, sh.H, sh.T, sh.d_k), dtype=torch.float32, device="cuda")
        sdm.address_backward(S, to_dev(inp[xname], sh.in_dtype), sub, n_sel, to_dev(idx, "i32"), to_dev(w, "f32"),
                             to_dev(dw, "f32"), dx, dsub)
        torch.cuda.synchronize()
        e = rel_err(dx.cpu().numpy(), ref_dx)
        log(f"[address backward] {name} d{xname}: {e:.2e}")
        assert e < 1e-4, f"d{xname}"
    e = rel_err(dsub.cpu().numpy(), ref_dsub)
    log(f"[address backward] {name} dsubkeys: {e:.2e}")
    assert e < 1e-4
