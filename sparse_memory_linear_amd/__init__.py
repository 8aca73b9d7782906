"""Python binding of ``libsdm.so``, the MI355X (gfx950) Sparse Delta Memory layer forward.

Argument marshalling only: every step of the computation runs in the library's HIP
kernels. Tensors are ``torch`` device tensors (contiguous); the call is enqueued on
``torch.cuda.current_stream()`` unless a stream is given. The names follow the C ABI in
``include/sdm.h`` (``sdm_init_from_M0`` -> :func:`init_from_M0`, ...).

If ``libsdm.so`` has not been built (``python -m sparse_memory_linear_amd.build``), every
call raises :class:`SdmLibraryMissing`; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "SDM_F32", "SDM_BF16", "SdmError", "SdmLibraryMissing", "Shape", "lib", "lib_path",
    "make_shape", "check_shape", "workspace_bytes", "init_from_M0", "address", "recurrent",
    "forward", "forward_static", "STATIC_SCRATCH_BYTES", "forward_uses_chunkwise", "decode_step", "workspace_error", "status_string", "abi_version",
    "decay_state_init", "workspace_bytes_decay", "recurrent_decay", "forward_decay", "decode_step_decay",
    "materialize", "gates", "output_gate", "head_mix", "output_project", "recurrent_log", "recurrent_backward",
    "backward_workspace_bytes", "address_backward", "workspace_bytes_chunked", "recurrent_chunked",
]

SDM_F32 = 0
SDM_BF16 = 1
STATIC_SCRATCH_BYTES = 64 << 20  # SDM_STATIC_SCRATCH_BYTES of the header

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libsdm.so")


class SdmError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


class SdmLibraryMissing(RuntimeError):
    pass


class Shape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
        ("N", ctypes.c_int64),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("kappa", ctypes.c_int32), ("W", ctypes.c_int32), ("R", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("mem_dtype", ctypes.c_int32),
    ]

    def __repr__(self):
        return "Shape(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None
_P = ctypes.c_void_p
_SP = ctypes.POINTER(Shape)
_SIGS = {
    "sdm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sdm_abi_version": (ctypes.c_int, []),
    "sdm_check_shape": (ctypes.c_int, [_SP]),
    "sdm_workspace_bytes": (ctypes.c_size_t, [_SP]),
    "sdm_init_from_M0": (ctypes.c_int, [_SP, _P, _P, _P]),
    "sdm_address": (ctypes.c_int, [_SP, _P, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "sdm_address_init": (ctypes.c_int, [_SP, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_int32,
                                        ctypes.c_int32, _P]),
    "sdm_recurrent": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sdm_forward": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sdm_forward_static": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sdm_forward_uses_chunkwise": (ctypes.c_int, [_SP]),
    "sdm_decode_step": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sdm_workspace_error": (ctypes.c_int, [_P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int64), _P]),
    "sdm_decay_state_init": (ctypes.c_int, [_SP, _P, _P, _P]),
    "sdm_workspace_bytes_decay": (ctypes.c_size_t, [_SP]),
    "sdm_recurrent_decay": (ctypes.c_int, [_SP] + [_P] * 12 + [ctypes.c_size_t, _P]),
    "sdm_forward_decay": (ctypes.c_int, [_SP] + [_P] * 13 + [ctypes.c_size_t, _P]),
    "sdm_decode_step_decay": (ctypes.c_int, [_SP] + [_P] * 11),
    "sdm_materialize": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P]),
    "sdm_gates": (ctypes.c_int, [_SP, _P, _P, _P, _P, _P, _P, _P]),
    "sdm_output_gate": (ctypes.c_int, [_SP, _P, _P, _P, ctypes.c_float, _P, _P]),
    "sdm_head_mix": (ctypes.c_int, [_P, _P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P]),
    "sdm_output_project": (ctypes.c_int, [_SP, _P, _P, _P, ctypes.c_float, _P, ctypes.c_int32, _P, _P]),
    "sdm_recurrent_log": (ctypes.c_int, [_SP] + [_P] * 11 + [ctypes.c_size_t, _P]),
    "sdm_backward_workspace_bytes": (ctypes.c_size_t, [_SP]),
    "sdm_workspace_bytes_chunked": (ctypes.c_size_t, [_SP]),
    "sdm_recurrent_chunked": (ctypes.c_int, [_SP] + [_P] * 10 + [ctypes.c_size_t, _P]),
    "sdm_address_backward": (ctypes.c_int, [_SP, _P, _P, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "sdm_recurrent_backward": (ctypes.c_int, [_SP] + [_P] * 17 + [ctypes.c_size_t, _P]),
}


def lib():
    """The loaded ``libsdm.so`` (ctypes CDLL). Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise SdmLibraryMissing(
                f"{lib_path} is not built; run `python -m sparse_memory_linear_amd.build` "
                "(no fallback implementation exists)")
        L = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(code: int) -> str:
    try:
        return lib().sdm_status_string(int(code)).decode()
    except SdmLibraryMissing:
        return str(code)


def abi_version() -> int:
    return lib().sdm_abi_version()


def make_shape(B, H, T, N, d_k, d_v, kappa, W, R, in_dtype=SDM_BF16, mem_dtype=SDM_BF16) -> Shape:
    def dt(x):
        if isinstance(x, str):
            return {"f32": SDM_F32, "bf16": SDM_BF16}[x]
        return int(x)
    return Shape(int(B), int(H), int(T), int(N), int(d_k), int(d_v), int(kappa), int(W), int(R), dt(in_dtype),
                 dt(mem_dtype))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libsdm must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(code: int, where: str):
    if code != 0:
        raise SdmError(code, where)


def check_shape(shape: Shape) -> int:
    return lib().sdm_check_shape(ctypes.byref(shape))


def workspace_bytes(shape: Shape) -> int:
    return lib().sdm_workspace_bytes(ctypes.byref(shape))


def init_from_M0(shape: Shape, M0, M, stream=None):
    _check(lib().sdm_init_from_M0(ctypes.byref(shape), _ptr(M0), _ptr(M), _stream(stream)), "sdm_init_from_M0")


def address(shape: Shape, x, subkeys, n_sel: int, idx, weight, score=None, stream=None):
    _check(lib().sdm_address(ctypes.byref(shape), _ptr(x), _ptr(subkeys), int(n_sel), _ptr(idx), _ptr(weight),
                             _ptr(score), _stream(stream)), "sdm_address")


def address_init(shape: Shape, x, subkeys, n_sel: int, idx, weight, M0, M, part: int, nparts: int, score=None,
                 stream=None):
    _check(lib().sdm_address_init(ctypes.byref(shape), _ptr(x), _ptr(subkeys), int(n_sel), _ptr(idx),
                                  _ptr(weight), _ptr(score), _ptr(M0), _ptr(M), int(part), int(nparts),
                                  _stream(stream)), "sdm_address_init")


def recurrent(shape: Shape, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, stream=None):
    _check(lib().sdm_recurrent(ctypes.byref(shape), _ptr(widx), _ptr(wgt), _ptr(ridx), _ptr(rgt), _ptr(v),
                               _ptr(alpha), _ptr(beta), _ptr(M), _ptr(o), _ptr(ws), ws.numel() * ws.element_size(),
                               _stream(stream)), "sdm_recurrent")


def forward(shape: Shape, q, k, v, alpha, beta, subkeys, M, o, ws, widx_out=None, ridx_out=None, stream=None):
    _check(lib().sdm_forward(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                             _ptr(subkeys), _ptr(M), _ptr(o), _ptr(widx_out), _ptr(ridx_out), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "sdm_forward")


def forward_uses_chunkwise(shape: Shape) -> bool:
    """True where sdm_forward runs the chunkwise form of the recurrence for this shape."""
    r = lib().sdm_forward_uses_chunkwise(ctypes.byref(shape))
    if r < 0:
        raise SdmError(-1, "sdm_forward_uses_chunkwise")
    return bool(r)


def forward_static(shape: Shape, q, k, v, alpha, beta, subkeys, M, o, widx_out=None, ridx_out=None, stream=None):
    _check(lib().sdm_forward_static(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                    _ptr(subkeys), _ptr(M), _ptr(o), _ptr(widx_out), _ptr(ridx_out),
                                    _stream(stream)), "sdm_forward_static")


def decode_step(shape: Shape, q, k, v, alpha, beta, subkeys, M, o, stream=None):
    _check(lib().sdm_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(subkeys), _ptr(M), _ptr(o), _stream(stream)), "sdm_decode_step")


def workspace_error(ws, stream=None) -> int:
    out = ctypes.c_int64(0)
    _check(lib().sdm_workspace_error(_ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(out), _stream(stream)),
           "sdm_workspace_error")
    return out.value


# ----------------------------------------------------------------------------- whole-table decay
def decay_state_init(shape: Shape, lam, lrun, stream=None):
    _check(lib().sdm_decay_state_init(ctypes.byref(shape), _ptr(lam), _ptr(lrun), _stream(stream)),
           "sdm_decay_state_init")


def workspace_bytes_decay(shape: Shape) -> int:
    return lib().sdm_workspace_bytes_decay(ctypes.byref(shape))


def recurrent_decay(shape: Shape, widx, wgt, ridx, rgt, v, alpha, beta, M, lam, lrun, o, ws, stream=None):
    _check(lib().sdm_recurrent_decay(ctypes.byref(shape), _ptr(widx), _ptr(wgt), _ptr(ridx), _ptr(rgt), _ptr(v),
                                     _ptr(alpha), _ptr(beta), _ptr(M), _ptr(lam), _ptr(lrun), _ptr(o), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "sdm_recurrent_decay")


def forward_decay(shape: Shape, q, k, v, alpha, beta, subkeys, M, lam, lrun, o, ws, widx_out=None, ridx_out=None,
                  stream=None):
    _check(lib().sdm_forward_decay(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(subkeys), _ptr(M), _ptr(lam), _ptr(lrun), _ptr(o), _ptr(widx_out),
                                   _ptr(ridx_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "sdm_forward_decay")


def decode_step_decay(shape: Shape, q, k, v, alpha, beta, subkeys, M, lam, lrun, o, stream=None):
    _check(lib().sdm_decode_step_decay(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                       _ptr(subkeys), _ptr(M), _ptr(lam), _ptr(lrun), _ptr(o), _stream(stream)),
           "sdm_decode_step_decay")


def materialize(shape: Shape, M, lam, lrun, out, stream=None):
    _check(lib().sdm_materialize(ctypes.byref(shape), _ptr(M), _ptr(lam), _ptr(lrun), _ptr(out), _stream(stream)),
           "sdm_materialize")


# ----------------------------------------------------------------------------- gates and output
def gates(shape: Shape, a, b, A_log, dt_bias, alpha, beta, stream=None):
    _check(lib().sdm_gates(ctypes.byref(shape), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(alpha), _ptr(beta),
                           _stream(stream)), "sdm_gates")


def output_gate(shape: Shape, o, z, w, eps: float, x, stream=None):
    _check(lib().sdm_output_gate(ctypes.byref(shape), _ptr(o), _ptr(z), _ptr(w), float(eps), _ptr(x),
                                 _stream(stream)), "sdm_output_gate")


def head_mix(x, Wo, y, M: int, K: int, N: int, stream=None):
    _check(lib().sdm_head_mix(_ptr(x), _ptr(Wo), _ptr(y), int(M), int(K), int(N), _stream(stream)), "sdm_head_mix")


# ----------------------------------------------------------------------------- backward
def output_project(shape: Shape, o, z, w, eps: float, Wo, d_model: int, y, stream=None):
    _check(lib().sdm_output_project(ctypes.byref(shape), _ptr(o), _ptr(z), _ptr(w), float(eps), _ptr(Wo),
                                    int(d_model), _ptr(y), _stream(stream)), "sdm_output_project")


def recurrent_log(shape: Shape, widx, wgt, ridx, rgt, v, alpha, beta, M, o, xlog, ws, stream=None):
    _check(lib().sdm_recurrent_log(ctypes.byref(shape), _ptr(widx), _ptr(wgt), _ptr(ridx), _ptr(rgt), _ptr(v),
                                   _ptr(alpha), _ptr(beta), _ptr(M), _ptr(o), _ptr(xlog), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "sdm_recurrent_log")


def backward_workspace_bytes(shape: Shape) -> int:
    return lib().sdm_backward_workspace_bytes(ctypes.byref(shape))


def recurrent_backward(shape: Shape, widx, wgt, ridx, rgt, v, alpha, beta, M, xlog, go, G, dv, dalpha, dbeta, dwgt,
                       drgt, ws, stream=None):
    _check(lib().sdm_recurrent_backward(ctypes.byref(shape), _ptr(widx), _ptr(wgt), _ptr(ridx), _ptr(rgt), _ptr(v),
                                        _ptr(alpha), _ptr(beta), _ptr(M), _ptr(xlog), _ptr(go), _ptr(G), _ptr(dv),
                                        _ptr(dalpha), _ptr(dbeta), _ptr(dwgt), _ptr(drgt), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream)), "sdm_recurrent_backward")


def address_backward(shape: Shape, x, subkeys, n_sel: int, idx, weight, dweight, dx, dsub, stream=None):
    _check(lib().sdm_address_backward(ctypes.byref(shape), _ptr(x), _ptr(subkeys), int(n_sel), _ptr(idx),
                                      _ptr(weight), _ptr(dweight), _ptr(dx), _ptr(dsub), _stream(stream)),
           "sdm_address_backward")


def workspace_bytes_chunked(shape: Shape) -> int:
    return lib().sdm_workspace_bytes_chunked(ctypes.byref(shape))


def recurrent_chunked(shape: Shape, widx, wgt, ridx, rgt, v, alpha, beta, M, o, ws, stream=None):
    _check(lib().sdm_recurrent_chunked(ctypes.byref(shape), _ptr(widx), _ptr(wgt), _ptr(ridx), _ptr(rgt), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(M), _ptr(o), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)), "sdm_recurrent_chunked")
