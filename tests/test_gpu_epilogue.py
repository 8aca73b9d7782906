"""Gates, output normalisation and gate, and head mixing on the GPU against the oracle
(float64 on the same inputs the device received)."""
import numpy as np
import pytest

import oracle.sdm_oracle as O
import sdm_inputs as SI
from parity import empty_mem, from_dev, lib_shape, log, rel_err, to_dev, tolerance

pytestmark = pytest.mark.gpu

W_ = SI.WORKLOADS


@pytest.fixture(scope="module")
def sdm():
    import torch
    import sparse_memory_linear_amd as S
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    S.lib()
    return S


def test_gates(sdm):
    import torch
    sh = W_["small"].replace(B=2, H=8, T=300)
    ep = SI.make_epilogue_inputs(sh, d_model=64)
    S = lib_shape(sh)
    al = torch.empty((sh.B, sh.H, sh.T), dtype=torch.float32, device="cuda")
    be = torch.empty_like(al)
    sdm.gates(S, to_dev(ep["a"], "f32"), to_dev(ep["b"], "f32"), to_dev(ep["A_log"], "f32"),
              to_dev(ep["dt_bias"], "f32"), al, be)
    torch.cuda.synchronize()
    ra, rb = O.gates(ep["a"], ep["b"], ep["A_log"], ep["dt_bias"])  # [B, H, T]
    ea, eb = rel_err(al.cpu().numpy(), ra), rel_err(be.cpu().numpy(), rb)
    log(f"[gates] rel err alpha {ea:.2e} beta {eb:.2e}")
    assert ea < 1e-5 and eb < 1e-5
    assert float(al.max()) <= 1.0 and float(al.min()) > 0.0


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_output_gate(sdm, in_dtype):
    import torch
    sh = W_["small"].replace(B=2, H=3, T=70, in_dtype=in_dtype)
    ep = SI.make_epilogue_inputs(sh, d_model=64)
    rng = np.random.default_rng(5)
    o = rng.standard_normal((sh.B, sh.H, sh.T, sh.d_v)).astype(np.float32)
    S = lib_shape(sh)
    x = torch.empty((sh.B, sh.T, sh.H, sh.d_v), dtype=torch.bfloat16, device="cuda")
    sdm.output_gate(S, to_dev(o, "f32"), to_dev(ep["z"], in_dtype), to_dev(ep["w"], "f32"), 1e-5, x)
    torch.cuda.synchronize()
    z = SI.widen(ep["z"], in_dtype)
    ref = O.output_gate(o.transpose(0, 2, 1, 3), z, ep["w"], 1e-5)  # [B,T,H,d_v]
    got = SI.widen(from_dev(x, "bf16"), "bf16")
    e = rel_err(got, ref)
    log(f"[output gate] {in_dtype}: rel err {e:.2e}")
    assert e < 1e-2  # one bf16 rounding of the output


@pytest.mark.parametrize("M,K,N", [(300, 256, 200), (128, 32, 128), (1000, 1024, 384)])
def test_head_mix(sdm, M, K, N):
    import torch
    rng = np.random.default_rng(M + K + N)
    x = SI.cast(rng.standard_normal((M, K)).astype(np.float32), "bf16")
    Wo = SI.cast((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32), "bf16")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    sdm.head_mix(to_dev(x, "bf16"), to_dev(Wo, "bf16"), y, M, K, N)
    torch.cuda.synchronize()
    ref = O.head_mix(SI.widen(x, "bf16"), SI.widen(Wo, "bf16"))
    e = rel_err(y.cpu().numpy(), ref)
    log(f"[head mix] {M}x{K}x{N}: rel err {e:.2e}")
    assert e < 1e-5  # exact bf16 products, float32 sums


@pytest.mark.parametrize("in_dtype,B,H,T,d_v,d_model", [
    ("bf16", 2, 3, 70, 128, 200),   # ragged row tile across the batch boundary, ragged columns
    ("f32", 1, 4, 300, 64, 384),
    ("bf16", 3, 2, 129, 32, 128),
    ("bf16", 1, 2, 260, 256, 130),
    ("bf16", 1, 10, 100, 128, 256),  # K = 1280: 32 tokens per workgroup
    ("f32", 2, 8, 40, 256, 64),      # K = 2048
])
def test_output_project(sdm, in_dtype, B, H, T, d_v, d_model):
    """Normalisation, gate and head mixing in one pass: against the oracle's chain in float64
    and against the two separate calls on the same inputs."""
    import torch
    sh = W_["small"].replace(B=B, H=H, T=T, d_v=d_v, in_dtype=in_dtype, mem_dtype="f32")
    ep = SI.make_epilogue_inputs(sh, d_model=d_model)
    rng = np.random.default_rng(B * 1000 + T + d_v)
    o = rng.standard_normal((B, H, T, d_v)).astype(np.float32)
    S = lib_shape(sh)
    od, zd, wd, Wod = to_dev(o, "f32"), to_dev(ep["z"], in_dtype), to_dev(ep["w"], "f32"), to_dev(ep["Wo"], "bf16")
    y = torch.full((B * T, d_model), float("nan"), dtype=torch.float32, device="cuda")
    sdm.output_project(S, od, zd, wd, 1e-5, Wod, d_model, y)
    x = torch.empty((B, T, H, d_v), dtype=torch.bfloat16, device="cuda")
    sdm.output_gate(S, od, zd, wd, 1e-5, x)
    y2 = torch.empty((B * T, d_model), dtype=torch.float32, device="cuda")
    sdm.head_mix(x, Wod, y2, B * T, H * d_v, d_model)
    torch.cuda.synchronize()
    got, two = y.cpu().numpy(), y2.cpu().numpy()
    assert np.isfinite(got).all()
    xr = O.output_gate(o.transpose(0, 2, 1, 3), SI.widen(ep["z"], in_dtype), ep["w"], 1e-5)
    ref = O.head_mix(xr.reshape(B * T, H * d_v), SI.widen(ep["Wo"], "bf16"))
    e, e2 = rel_err(got, ref), rel_err(got, two)
    log(f"[output project] {in_dtype} B={B} H={H} T={T} d_v={d_v} d_model={d_model}: rel err {e:.2e} "
        f"(vs separate calls {e2:.2e})")
    assert e < 1e-2   # one bf16 rounding of x, float32 sums
    assert np.array_equal(got, two)  # same bf16 x, same products and sums


@pytest.mark.parametrize("fused", [False, True])
def test_layer_end_to_end(sdm, fused):
    """Gates -> forward -> output normalisation and gate -> head mixing (two calls, or the
    fused sdm_output_project), against the oracle's chain of the same steps on the same
    inputs."""
    import torch
    sh = W_["layer_1p4b"].replace(B=1, H=2, T=96)
    d_model = 256
    inp = SI.make_inputs(sh)
    ep = SI.make_epilogue_inputs(sh, d_model=d_model)
    S = lib_shape(sh)
    dev = {k: to_dev(inp[k], sh.in_dtype) for k in ("q", "k", "v", "subkeys")}
    al = torch.empty((sh.B, sh.H, sh.T), dtype=torch.float32, device="cuda")
    be = torch.empty_like(al)
    sdm.gates(S, to_dev(ep["a"], "f32"), to_dev(ep["b"], "f32"), to_dev(ep["A_log"], "f32"),
              to_dev(ep["dt_bias"], "f32"), al, be)
    M = empty_mem((sh.B, sh.H, sh.N, sh.d_v), sh.mem_dtype)
    sdm.init_from_M0(S, to_dev(inp["M0"], sh.mem_dtype), M)
    o = torch.empty((sh.B, sh.H, sh.T, sh.d_v), dtype=torch.float32, device="cuda")
    ws = torch.empty(sdm.workspace_bytes(S), dtype=torch.uint8, device="cuda")
    sdm.forward(S, dev["q"], dev["k"], dev["v"], al, be, dev["subkeys"], M, o, ws)
    y = torch.empty((sh.B * sh.T, d_model), dtype=torch.float32, device="cuda")
    if fused:
        sdm.output_project(S, o, to_dev(ep["z"], sh.in_dtype), to_dev(ep["w"], "f32"), 1e-5, to_dev(ep["Wo"], "bf16"),
                           d_model, y)
    else:
        x = torch.empty((sh.B, sh.T, sh.H, sh.d_v), dtype=torch.bfloat16, device="cuda")
        sdm.output_gate(S, o, to_dev(ep["z"], sh.in_dtype), to_dev(ep["w"], "f32"), 1e-5, x)
        sdm.head_mix(x, to_dev(ep["Wo"], "bf16"), y, sh.B * sh.T, sh.H * sh.d_v, d_model)
    torch.cuda.synchronize()
    # oracle chain; the gates the device computed in float32 drive both recurrences
    ga = al.cpu().numpy().astype(np.float64)
    gb = be.cpu().numpy().astype(np.float64)
    ra, rb = O.gates(ep["a"][0], ep["b"][0], ep["A_log"], ep["dt_bias"])
    assert rel_err(ga[0], ra) < 1e-5 and rel_err(gb[0], rb) < 1e-5
    oo = np.zeros((sh.B, sh.T, sh.H, sh.d_v))
    for h in range(sh.H):
        sk = SI.widen(inp["subkeys"][h], sh.in_dtype)
        r = O.forward_unit(SI.widen(inp["q"][0, h], sh.in_dtype), SI.widen(inp["k"][0, h], sh.in_dtype),
                           SI.widen(inp["v"][0, h], sh.in_dtype), ga[0, h], gb[0, h], sk[0], sk[1],
                           SI.widen(inp["M0"][h], sh.mem_dtype), sh.kappa, sh.W, sh.R, sh.mem_dtype)
        oo[0, :, h] = r["o"]
    xr = O.output_gate(oo, SI.widen(ep["z"], sh.in_dtype), ep["w"], 1e-5)
    yr = O.head_mix(xr.reshape(sh.B * sh.T, sh.H * sh.d_v), SI.widen(ep["Wo"], "bf16"))
    e = rel_err(y.cpu().numpy(), yr)
    log(f"[layer] end to end ({'fused' if fused else 'two calls'}) rel err {e:.2e} (tol {tolerance(sh)})")
    assert e < tolerance(sh)
