"""sdm_forward_static (the forward with the library's own per-GPU scratch array instead of a
caller workspace) against sdm_forward, through the C ABI, on three calls in a row, each on a
smaller input than the one before: identical slot lists, and outputs and tables bit for bit
on the pipeline (within 1e-5 relative where the forward runs the chunkwise form, whose
float32 sums can be ordered differently from run to run); a shape whose workspace exceeds
the array is refused before anything runs."""
import pytest

import sdm_inputs as SI
from parity import empty_mem, lib_shape, log, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _run(S, sh, inp, static):
    import torch
    import sparse_memory_linear_amd as L
    dev = {k: to_dev(inp[k], sh.in_dtype) for k in ("q", "k", "v", "subkeys")}
    dev["alpha"] = to_dev(inp["alpha"], "f32")
    dev["beta"] = to_dev(inp["beta"], "f32")
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    L.init_from_M0(S, to_dev(inp["M0"], sh.mem_dtype), M)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    wi = torch.empty((sh.B, sh.H, sh.T, sh.W), dtype=torch.int32, device="cuda")
    ri = torch.empty((sh.B, sh.H, sh.T, sh.R), dtype=torch.int32, device="cuda")
    if static:
        L.forward_static(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, o, wi, ri)
    else:
        ws = torch.empty(L.workspace_bytes(S), dtype=torch.uint8, device="cuda")
        L.forward(S, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], M, o, ws, wi, ri)
        assert L.workspace_error(ws) == 0
    torch.cuda.synchronize()
    return o, M, wi, ri


def test_forward_static_equals_forward():
    import torch
    import sparse_memory_linear_amd as L
    L.lib()
    cases = [SI.WORKLOADS["small"].replace(B=4, H=8, T=300),           # 32 units: the chunkwise form
             SI.WORKLOADS["small"].replace(B=2, H=4, T=200),           # smaller: the pipeline
             SI.WORKLOADS["layer_8b_long"].replace(B=1, H=2, T=150)]   # smaller still, bf16 table
    for sh in cases:
        S = lib_shape(sh)
        assert L.workspace_bytes(S) <= L.STATIC_SCRATCH_BYTES
        log(f"[static] {sh.name} B={sh.B} H={sh.H} T={sh.T}: workspace {L.workspace_bytes(S)} bytes, "
            f"chunkwise form {L.forward_uses_chunkwise(S)}")
        inp = SI.make_inputs(sh)
        ref = _run(S, sh, inp, static=False)
        got = _run(S, sh, inp, static=True)
        for name, a, b in zip(("o", "M", "widx", "ridx"), ref, got):
            if name in ("o", "M") and L.forward_uses_chunkwise(S):
                # the chunkwise form orders some float32 sums differently from run to run
                err = rel_err(a.float().cpu().numpy(), b.float().cpu().numpy())
                assert err < 1e-5, f"{sh.name}: {name} differs from sdm_forward by {err:.1e}"
            else:
                assert torch.equal(a, b), f"{sh.name}: {name} differs from sdm_forward"


def test_forward_static_refuses_a_large_workspace():
    import torch
    import sparse_memory_linear_amd as L
    sh = SI.WORKLOADS["layer_8b_long"]
    S = lib_shape(sh)
    assert L.workspace_bytes(S) > L.STATIC_SCRATCH_BYTES
    t = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(L.SdmError) as e:
        L.forward_static(S, t, t, t, t, t, t, t, t)
    assert e.value.code == -3  # SDM_ERR_WORKSPACE
