"""The C-ABI library on the host: it loads, exports every entry point the header declares,
and rejects bad arguments before any HIP call (no GPU needed; no compute is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")


@pytest.fixture(scope="module")
def sdm():
    import sparse_memory_linear_amd as S
    if not os.path.exists(S.lib_path):
        from sparse_memory_linear_amd import build
        build.build(verbose=False)
    return S


@pytest.fixture(scope="module")
def no_gpu():
    # every call below must fail validation; never hand fake pointers to a real device
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_[A-Za-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(sdm):
    names = declared_functions()
    assert len(names) >= 10
    L = ctypes.CDLL(sdm.lib_path)
    for n in names:
        assert hasattr(L, n), f"libsdm.so does not export {n}"


def test_abi_version_and_status_strings(sdm):
    assert sdm.abi_version() == 1
    assert sdm.status_string(0) == "SDM_OK"
    assert sdm.status_string(-1) == "SDM_ERR_INVALID_ARG"
    assert sdm.status_string(-3) == "SDM_ERR_WORKSPACE"


def base(**kw):
    import sparse_memory_linear_amd as S
    d = dict(B=2, H=2, T=64, N=65536, d_k=128, d_v=128, kappa=16, W=16, R=16, in_dtype=1, mem_dtype=1)
    d.update(kw)
    return S.make_shape(**d)


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    ({"N": 65535}, -1),          # not a perfect square
    ({"N": 1}, -1),
    ({"N": 1024 * 1024}, -2),    # s > 512: outside the kernels' limits
    ({"d_k": 127}, -1),          # odd key width
    ({"d_k": 512}, -2),
    ({"kappa": 0}, -1),
    ({"kappa": 257}, -1),        # more than s sub-keys
    ({"kappa": 128}, -2),        # beyond 64
    ({"W": 0}, -1),
    ({"W": 257, "kappa": 16}, -1),  # more than kappa^2
    ({"W": 65, "kappa": 16}, -2),
    ({"d_v": 3, "mem_dtype": 0}, -2),  # rows must be multiples of 16 bytes
    ({"in_dtype": 7}, -1),
    ({"B": 0}, -1),
    ({"T": 0}, 0),
])
def test_check_shape(sdm, kw, code):
    assert sdm.check_shape(base(**kw)) == code


def test_workspace_bytes(sdm):
    S = base()
    n = sdm.workspace_bytes(S)
    tok = 2 * 2 * 64
    assert n >= tok * (16 + 16) * 8
    assert sdm.workspace_bytes(base(N=65535)) == 0


FAKE = 1 << 40  # 16-byte aligned fake device addresses, never dereferenced


def test_null_and_misaligned_pointers(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    assert L.sdm_init_from_M0(sp, None, FAKE, None) == -1
    assert L.sdm_init_from_M0(sp, FAKE + 4, FAKE + (1 << 36), None) == -1
    assert L.sdm_address(sp, FAKE, FAKE + 2**30, 16, None, FAKE + 2**31, None, None) == -1
    assert L.sdm_address(sp, FAKE, FAKE + 2**30, 0, FAKE + 2**32, FAKE + 2**33, None, None) == -1
    assert L.sdm_address(sp, FAKE, FAKE + 2**30, 300, FAKE + 2**32, FAKE + 2**33, None, None) == -1
    args = [FAKE + i * (1 << 36) for i in range(9)]
    args[2] += 8  # misaligned ridx
    assert L.sdm_recurrent(sp, *args, FAKE + 10 * (1 << 36), 1 << 30, None) == -1


def test_address_init_validates(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    x, c, idx, w, M0, M = (FAKE + i * (1 << 36) for i in range(6))
    # part and nparts out of range
    for part, nparts in ((0, 0), (-1, 2), (2, 2), (0, 65)):
        assert L.sdm_address_init(sp, x, c, 16, idx, w, None, M0, M, part, nparts, None) == -1
    # null or misaligned tables
    assert L.sdm_address_init(sp, x, c, 16, idx, w, None, None, M, 0, 1, None) == -1
    assert L.sdm_address_init(sp, x, c, 16, idx, w, None, M0, M + 8, 0, 1, None) == -1
    # M0 inside M, M over the slot outputs, the query or the sub-keys
    assert L.sdm_address_init(sp, x, c, 16, idx, w, None, M + 4096, M, 0, 1, None) == -1
    assert L.sdm_address_init(sp, x, c, 16, M + 4096, w, None, M0, M, 0, 1, None) == -1
    assert L.sdm_address_init(sp, M + 1024, c, 16, idx, w, None, M0, M, 0, 1, None) == -1
    assert L.sdm_address_init(sp, x, M + 2048, 16, idx, w, None, M0, M, 0, 1, None) == -1
    # the addressing checks of sdm_address still apply
    assert L.sdm_address_init(sp, x, c, 0, idx, w, None, M0, M, 0, 1, None) == -1
    assert L.sdm_address_init(sp, x, c, 16, None, w, None, M0, M, 0, 1, None) == -1


def test_workspace_too_small(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    need = sdm.workspace_bytes(S)
    p = [FAKE + i * (1 << 36) for i in range(12)]
    assert L.sdm_forward(ctypes.byref(S), p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], None, None, p[8], need - 256,
                         None) == -3
    assert L.sdm_forward(ctypes.byref(S), p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], None, None, None, need,
                         None) == -3
    assert L.sdm_recurrent(ctypes.byref(S), *p[:9], p[9], 8, None) == -3


def test_overlapping_buffers_rejected(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    # M0 inside M
    assert L.sdm_init_from_M0(sp, FAKE + 4096, FAKE, None) == -1
    # o overlapping the table
    p = [FAKE + i * (1 << 36) for i in range(12)]
    need = sdm.workspace_bytes(S)
    assert L.sdm_forward(sp, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[6] + 1024, None, None, p[8], need, None) == -1
    # workspace inside the table
    assert L.sdm_forward(sp, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], None, None, p[6] + 4096, need, None) == -1


def test_decode_requires_single_token(sdm, no_gpu):
    L = sdm.lib()
    S = base(T=2)
    p = [FAKE + i * (1 << 36) for i in range(9)]
    assert L.sdm_decode_step(ctypes.byref(S), *p, None) == -1
    S0 = base(T=1)
    assert L.sdm_decode_step(ctypes.byref(S0), None, *p[1:], None) == -1


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import sparse_memory_linear_amd as S
    monkeypatch.setattr(S, "lib_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(S, "_lib", None)
    with pytest.raises(S.SdmLibraryMissing):
        S.lib()


# ----------------------------------------------------------------------------- whole-table decay
def test_workspace_bytes_decay(sdm):
    S = base()
    n, nd = sdm.workspace_bytes(S), sdm.workspace_bytes_decay(S)
    tok = 2 * 2 * 64
    # per token: the cumulative log-decay (8 B) and one factor per slot (4 B each); per slot
    # its latest writer (4 B)
    assert nd >= n + tok * 8 + tok * (16 + 16) * 4 + 2 * 2 * 65536 * 4
    assert sdm.workspace_bytes_decay(base(N=65535)) == 0


def test_decay_calls_validate(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    p = [FAKE + i * (1 << 36) for i in range(16)]
    need = sdm.workspace_bytes_decay(S)
    # recurrent: widx wgt ridx rgt v alpha beta M lam lrun o ws
    args = p[:12]
    assert L.sdm_recurrent_decay(sp, *args[:8], None, args[9], args[10], args[11], need, None) == -1
    assert L.sdm_recurrent_decay(sp, *args[:9], None, args[10], args[11], need, None) == -1
    assert L.sdm_recurrent_decay(sp, *args[:8], args[7] + 4096, *args[9:12], need, None) == -1  # lam inside M
    assert L.sdm_recurrent_decay(sp, *args[:12], sdm.workspace_bytes(S), None) == -3  # plain workspace too small
    assert L.sdm_recurrent_decay(sp, *args[:8], args[8] + 8, *args[9:12], need, None) == -1  # misaligned lam
    # forward: q k v alpha beta subkeys M lam lrun o widx_out ridx_out ws
    assert L.sdm_forward_decay(sp, *p[:7], None, p[8], p[9], None, None, p[12], need, None) == -1
    assert L.sdm_forward_decay(sp, *p[:7], p[8], p[8] + 8, p[9], None, None, p[12], need, None) == -1  # lam/lrun overlap
    # decode: T must be 1, state required
    S1 = base(T=1)
    assert L.sdm_decode_step_decay(ctypes.byref(S1), *p[:7], None, p[8], p[9], None) == -1
    assert L.sdm_decode_step_decay(ctypes.byref(base(T=2)), *p[:10], None) == -1
    # state init and materialize
    assert L.sdm_decay_state_init(sp, None, p[1], None) == -1
    assert L.sdm_decay_state_init(sp, p[0], p[0] + 16, None) == -1  # lrun inside lam
    assert L.sdm_materialize(sp, p[0], p[1], p[2], None, None) == -1
    assert L.sdm_materialize(sp, p[0], p[1], p[2], p[0] + 4096, None) == -1  # out overlaps M


def test_decay_needs_the_pipelined_recurrence(sdm, no_gpu):
    """Whole-table decay runs only on the pipelined recurrence: a shape it does not take
    (slot lists that are not a multiple of 4 long) is refused before any launch."""
    L = sdm.lib()
    S = base(W=6, R=6)
    p = [FAKE + i * (1 << 36) for i in range(16)]
    assert L.sdm_recurrent_decay(ctypes.byref(S), *p[:12], 1 << 34, None) == -2


# ----------------------------------------------------------------------------- gates and output
def test_epilogue_calls_validate(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    p = [FAKE + i * (1 << 36) for i in range(8)]
    assert L.sdm_gates(sp, None, *p[1:6], None) == -1
    assert L.sdm_gates(sp, p[0], p[1], p[2], p[3], p[0] + 256, p[5], None) == -1  # alpha overlaps a
    assert L.sdm_output_gate(sp, p[0], p[1], p[2], ctypes.c_float(-1.0), p[3], None) == -1  # negative eps
    assert L.sdm_output_gate(sp, p[0], p[1], p[2], ctypes.c_float(1e-5), p[0] + 512, None) == -1  # x overlaps o
    assert L.sdm_head_mix(p[0], p[1], p[2], 100, 48, 64, None) == -1    # K not a multiple of 32
    assert L.sdm_head_mix(p[0], p[1], p[2], 100, 64, 0, None) == -1     # no output columns
    assert L.sdm_head_mix(p[0], p[1], p[0] + 64, 100, 64, 64, None) == -1  # y overlaps x
    assert L.sdm_head_mix(p[0], p[1], p[2], 0, 64, 64, None) == 0       # nothing to do
    assert L.sdm_head_mix(p[0], p[1], p[2], 1 << 31, 64, 64, None) == -2  # grid beyond the launch limit
    f = ctypes.c_float
    assert L.sdm_output_project(sp, p[0], p[1], p[2], f(-1.0), p[3], 256, p[4], None) == -1  # negative eps
    assert L.sdm_output_project(sp, p[0], p[1], p[2], f(1e-5), p[3], 0, p[4], None) == -1    # no output columns
    assert L.sdm_output_project(sp, p[0], p[1], p[2], f(1e-5), p[3], 256, p[0] + 64, None) == -1  # y overlaps o
    assert L.sdm_output_project(sp, p[0], p[1], p[2], f(1e-5), p[3], 256, p[3] + 64, None) == -1  # y overlaps Wo
    assert L.sdm_output_project(sp, p[0], p[1] + 8, p[2], f(1e-5), p[3], 256, p[4], None) == -1  # misaligned z
    S96 = base(d_v=96)
    assert L.sdm_output_project(ctypes.byref(S96), p[0], p[1], p[2], f(1e-5), p[3], 256, p[4], None) == -2
    S20 = base(H=21)  # K = H*d_v = 2688: x of 32 tokens does not fit in LDS
    assert L.sdm_output_project(ctypes.byref(S20), p[0], p[1], p[2], f(1e-5), p[3], 256, p[4], None) == -2
    S0 = base(T=0)
    assert L.sdm_output_project(ctypes.byref(S0), p[0], p[1], p[2], f(1e-5), p[3], 256, p[4], None) == 0


# ----------------------------------------------------------------------------- backward
def test_backward_calls_validate(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    p = [FAKE + i * (1 << 36) for i in range(20)]
    need = sdm.workspace_bytes(S)
    assert L.sdm_recurrent_log(sp, *p[:9], None, p[10], need, None) == -1            # no log buffer
    assert L.sdm_recurrent_log(sp, *p[:9], p[7] + 4096, p[10], need, None) == -1     # log inside the table
    bneed = sdm.backward_workspace_bytes(S)
    assert bneed > 0
    args = list(p[:16]) + [p[16], bneed]
    args[10] = args[7] + 64                                                            # G overlaps M
    assert L.sdm_recurrent_backward(sp, *args, None) == -1
    args = list(p[:16]) + [p[16], bneed]
    args[11] = args[9]                                                                 # dv overlaps go
    assert L.sdm_recurrent_backward(sp, *args, None) == -1
    args = list(p[:16]) + [p[16], bneed]
    args[0] = None
    assert L.sdm_recurrent_backward(sp, *args, None) == -1
    args = list(p[:16]) + [p[10] + 128, bneed]                                         # workspace inside G
    assert L.sdm_recurrent_backward(sp, *args, None) == -1
    args = list(p[:16]) + [p[16], bneed - 1]                                           # workspace too small
    assert L.sdm_recurrent_backward(sp, *args, None) == -3


def test_address_backward_validates(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    p = [FAKE + i * (1 << 36) for i in range(10)]
    ok = [p[0], p[1], 16, p[2], p[3], p[4], p[5], p[6]]
    args = list(ok)
    args[2] = 0                                                # no slots
    assert L.sdm_address_backward(sp, *args, None) == -1
    args = list(ok)
    args[2] = 17 * 17                                          # more than kappa^2
    assert L.sdm_address_backward(sp, *args, None) == -1
    args = list(ok)
    args[6] = p[0] + 64                                        # dx inside x
    assert L.sdm_address_backward(sp, *args, None) == -1
    args = list(ok)
    args[7] = p[1] + 32                                        # dsub inside the sub-keys
    assert L.sdm_address_backward(sp, *args, None) == -1
    args = list(ok)
    args[7] = args[6] + 16                                     # dsub inside dx
    assert L.sdm_address_backward(sp, *args, None) == -1
    args = list(ok)
    args[3] = None
    assert L.sdm_address_backward(sp, *args, None) == -1
    Z = base(T=0)
    assert L.sdm_address_backward(ctypes.byref(Z), *ok, None) == 0   # nothing to do


def test_chunked_validates(sdm, no_gpu):
    L = sdm.lib()
    S = base()
    sp = ctypes.byref(S)
    need = sdm.workspace_bytes_chunked(S)
    assert need > 0
    assert sdm.workspace_bytes_chunked(base(W=40, kappa=16)) == 0                 # lists longer than 32
    p = [FAKE + i * (1 << 36) for i in range(12)]
    ok = list(p[:9]) + [p[9], need]
    args = list(ok)
    args[10] = need - 1                                                            # workspace too small
    assert L.sdm_recurrent_chunked(sp, *args, None) == -3
    args = list(ok)
    args[8] = args[7] + 64                                                         # o inside the table
    assert L.sdm_recurrent_chunked(sp, *args, None) == -1
    args = list(ok)
    args[9] = args[0]                                                              # workspace over widx
    assert L.sdm_recurrent_chunked(sp, *args, None) == -1
    args = list(ok)
    args[2] = None
    assert L.sdm_recurrent_chunked(sp, *args, None) == -1
    assert L.sdm_recurrent_chunked(ctypes.byref(base(W=40, kappa=16)), *ok, None) == -2   # unsupported



def test_forward_static_validates(sdm, no_gpu):
    """The allocation-free forward checks its arguments and its workspace limit on the host
    before any HIP call."""
    import sdm_inputs as SI
    from parity import lib_shape
    L = sdm.lib()
    big = lib_shape(SI.WORKLOADS["layer_8b_long"])
    p = [0x100000 * (i + 1) for i in range(10)]  # q, k, v, alpha, beta, subkeys, M, o, widx_out, ridx_out
    assert sdm.workspace_bytes(big) > sdm.STATIC_SCRATCH_BYTES
    assert L.sdm_forward_static(ctypes.byref(big), *p, None) == -3           # workspace past the array
    small = lib_shape(SI.WORKLOADS["small"].replace(B=1, H=2, T=64))
    q = list(p)
    q[0] = None
    assert L.sdm_forward_static(ctypes.byref(small), *q, None) == -1         # null q
    q = list(p)
    q[1] += 4
    assert L.sdm_forward_static(ctypes.byref(small), *q, None) == -1         # misaligned k
    q = list(p)
    q[7] = q[6]
    assert L.sdm_forward_static(ctypes.byref(small), *q, None) == -1         # o overlaps M
    bad = lib_shape(SI.WORKLOADS["small"].replace(N=1000))
    assert L.sdm_forward_static(ctypes.byref(bad), *p, None) == -1           # N not a square


def test_forward_form_query(sdm):
    """Which recurrence form sdm_forward takes: the chunkwise form for a float32 table with at
    least 32 units, the pipeline otherwise; -1 for an invalid shape (host only)."""
    import sdm_inputs as SI
    from parity import lib_shape
    L = sdm.lib()
    W_ = SI.WORKLOADS
    assert sdm.forward_uses_chunkwise(lib_shape(W_["small"]))                       # 32 units, f32 table
    assert not sdm.forward_uses_chunkwise(lib_shape(W_["small"].replace(B=2)))      # 16 units
    assert not sdm.forward_uses_chunkwise(lib_shape(W_["tiny_fp32"]))               # one unit
    assert not sdm.forward_uses_chunkwise(lib_shape(W_["layer_1p4b"]))              # bf16 table
    assert not sdm.forward_uses_chunkwise(lib_shape(W_["layer_8b_long"]))
    bad = lib_shape(W_["small"].replace(N=1000))
    assert L.sdm_forward_uses_chunkwise(ctypes.byref(bad)) == -1
    # the forward's workspace covers the chunkwise lists where it takes that form
    s = lib_shape(W_["small"])
    assert sdm.workspace_bytes(s) >= sdm.workspace_bytes_chunked(s)
