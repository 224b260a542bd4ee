"""ctypes binding of libttt.so: same entry points as ``include/ttt.h``.

Argument marshalling only.  Tensors (torch, on the GPU) are passed as raw
device pointers; ``None`` becomes NULL; a plain int is taken as a pointer.
Every computation happens in the library's HIP kernels.  A missing library
raises at load time: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from enum import IntEnum

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libttt.so")

EXPORTS = ("ttt_workspace_size", "ttt_saved_size", "ttt_chunk_fwd", "ttt_chunk_bwd", "inplace_ttt_workspace_size",
           "inplace_ttt_fwd", "inplace_ttt_guarded_workspace_size", "inplace_ttt_fwd_guarded",
           "inplace_ttt_bwd_workspace_size", "inplace_ttt_bwd", "inplace_ttt_bwd_guarded_workspace_size",
           "inplace_ttt_bwd_guarded", "ttt_mlp_workspace_size", "ttt_mlp_chunk_fwd",
           "ttt_mlp_bwd_workspace_size", "ttt_mlp_chunk_bwd", "ttt_mlp_saved_size",
           "ttt_last_error", "ttt_version", "ttt_timing_enable", "ttt_timing_read", "ttt_chunk_bwd_noalloc",
           "ttt_noalloc_scratch_bytes")


class Status(IntEnum):
    OK = 0
    INVALID_ARG = -1
    UNSUPPORTED = -2
    WORKSPACE = -3
    HIP = -4


class DType(IntEnum):
    F32 = 0
    BF16 = 1


class Loss(IntEnum):
    MSE = 0
    IP = 1
    L1 = 2
    RMSE = 3


class Act(IntEnum):
    NONE = 0
    SILU = 1
    GELU = 2
    NORM = 3


class Decay(IntEnum):
    NONE = 0
    SCALAR = 1
    VECTOR = 2


class Kernel(IntEnum):
    """Mirror of ``ttt_kernel`` (per-kernel timing ids)."""
    FWD = 0
    BWD_SEQ = 1
    BWD_CROSS = 2
    DGAMMA = 3
    GENERIC_FWD = 4
    GENERIC_BWD = 5
    DECAY_CUMSUM = 6
    INPLACE_APPLY = 7
    INPLACE_UPDATE = 8
    DECAY_PREP = 9
    INPLACE_NORM = 10
    LIN_STATE = 11
    LIN_SCAN = 12
    LIN_OUT = 13
    INPLACE_BWD_W = 14
    INPLACE_BWD_DZ = 15
    INPLACE_BWD_DV = 16
    INPLACE_BWD_DW = 17
    MLP_FWD = 18
    MLP_BWD = 19
    NORM_FWD = 20
    NORM_BWD = 21
    NORM_QUERY = 22
    NORM_BWD_PRE = 23
    MLP_QUERY = 24
    MLP_BWD_PRE = 25


ENTRY_FWD = 0
ENTRY_BWD = 1


class TTTDesc(ctypes.Structure):
    """Mirror of ``ttt_desc``."""
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("C", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("loss", ctypes.c_int32), ("act", ctypes.c_int32),
                ("decay", ctypes.c_int32), ("lr_bias", ctypes.c_float)]


class TTTMlpDesc(ctypes.Structure):
    """Mirror of ``ttt_mlp_desc``."""
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dh", ctypes.c_int32), ("dv", ctypes.c_int32), ("C", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("loss", ctypes.c_int32), ("act", ctypes.c_int32),
                ("decay", ctypes.c_int32), ("lr_bias", ctypes.c_float)]


class TTTError(RuntimeError):
    def __init__(self, status, message):
        self.status = Status(status) if status in Status._value2member_map_ else status
        super().__init__(f"{self.status!r}: {message}")


_lib = None


def lib():
    """Load libttt.so (once).  Raises OSError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is missing: build it with "
                      "`python -m chunkwise_weight_recurrence_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    dptr = ctypes.POINTER(TTTDesc)
    L.ttt_workspace_size.argtypes = [dptr, i32, ctypes.POINTER(sz)]
    L.ttt_workspace_size.restype = i32
    L.ttt_saved_size.argtypes = [dptr, ctypes.POINTER(sz)]
    L.ttt_saved_size.restype = i32
    L.ttt_chunk_fwd.argtypes = [dptr] + [vp] * 11 + [vp, sz, vp]
    L.ttt_chunk_fwd.restype = i32
    L.ttt_chunk_bwd.argtypes = [dptr] + [vp] * 18 + [vp, sz, vp]
    L.ttt_chunk_bwd.restype = i32
    L.ttt_chunk_bwd_noalloc.argtypes = [dptr] + [vp] * 18 + [vp]
    L.ttt_chunk_bwd_noalloc.restype = i32
    L.ttt_noalloc_scratch_bytes.argtypes = []
    L.ttt_noalloc_scratch_bytes.restype = sz
    L.inplace_ttt_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.inplace_ttt_workspace_size.restype = i32
    L.inplace_ttt_fwd.argtypes = [i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    L.inplace_ttt_fwd.restype = i32
    L.inplace_ttt_guarded_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.inplace_ttt_guarded_workspace_size.restype = i32
    L.inplace_ttt_fwd_guarded.argtypes = [i32, i32, i32, i32, i32, f32, f32, ctypes.POINTER(ctypes.c_int64), i32,
                                          vp, vp, vp, vp, vp, vp, sz, vp]
    L.inplace_ttt_fwd_guarded.restype = i32
    L.inplace_ttt_bwd_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.inplace_ttt_bwd_workspace_size.restype = i32
    L.inplace_ttt_bwd.argtypes = [i32, i32, i32, i32, i32, f32] + [vp] * 9 + [sz, vp]
    L.inplace_ttt_bwd.restype = i32
    L.inplace_ttt_bwd_guarded_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(sz)]
    L.inplace_ttt_bwd_guarded_workspace_size.restype = i32
    L.inplace_ttt_bwd_guarded.argtypes = [i32, i32, i32, i32, i32, f32, f32, ctypes.POINTER(ctypes.c_int64), i32] + \
        [vp] * 12 + [sz, vp]
    L.inplace_ttt_bwd_guarded.restype = i32
    mptr = ctypes.POINTER(TTTMlpDesc)
    L.ttt_mlp_workspace_size.argtypes = [mptr, ctypes.POINTER(sz)]
    L.ttt_mlp_workspace_size.restype = i32
    L.ttt_mlp_chunk_fwd.argtypes = [mptr] + [vp] * 13 + [vp, sz, vp]
    L.ttt_mlp_saved_size.argtypes = [mptr, ctypes.POINTER(sz)]
    L.ttt_mlp_saved_size.restype = i32
    L.ttt_mlp_chunk_fwd.restype = i32
    L.ttt_mlp_bwd_workspace_size.argtypes = [mptr, ctypes.POINTER(sz)]
    L.ttt_mlp_bwd_workspace_size.restype = i32
    L.ttt_mlp_chunk_bwd.argtypes = [mptr] + [vp] * 18 + [vp, sz, vp]
    L.ttt_mlp_chunk_bwd.restype = i32
    L.ttt_last_error.argtypes = []
    L.ttt_last_error.restype = ctypes.c_char_p
    L.ttt_version.argtypes = []
    L.ttt_version.restype = ctypes.c_char_p
    L.ttt_timing_enable.argtypes = [i32]
    L.ttt_timing_enable.restype = i32
    L.ttt_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    L.ttt_timing_read.restype = i32
    _lib = L
    return L


def _p(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if hasattr(x, "is_contiguous") and not x.is_contiguous():
            raise ValueError("tensors passed to libttt must be contiguous")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x)!r} as a device pointer")


def _stream(stream):
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available() and torch.cuda.is_initialized():
                return torch.cuda.current_stream().cuda_stream
        except Exception:  # pragma: no cover - torch is optional for this module
            pass
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != 0:
        raise TTTError(status, ttt_last_error())


def make_desc(B, H, T, dk, dv, C, dtype="bf16", loss="mse", act="none", decay="none", lr_bias=-4.0):
    """Build a TTTDesc from names ("bf16"/"f32", "mse"/"ip"/"l1", "none"/"silu"/"gelu"/"norm",
    "none"/"scalar"/"vector")."""
    def enum(cls, x):
        return int(cls[x.upper()]) if isinstance(x, str) else int(x)
    return TTTDesc(B, H, T, dk, dv, C, enum(DType, dtype), enum(Loss, loss), enum(Act, act),
                   enum(Decay, decay), float(lr_bias))


def make_mlp_desc(B, H, T, dk, dh, dv, C, dtype="bf16", loss="mse", act="gelu", decay="none", lr_bias=-4.0):
    """Build a TTTMlpDesc from names, as make_desc (decay "none" or "scalar")."""
    def enum(cls, x):
        return int(cls[x.upper()]) if isinstance(x, str) else int(x)
    return TTTMlpDesc(B, H, T, dk, dh, dv, C, enum(DType, dtype), enum(Loss, loss), enum(Act, act),
                      enum(Decay, decay), float(lr_bias))


def ttt_last_error() -> str:
    return lib().ttt_last_error().decode()


def ttt_version() -> str:
    return lib().ttt_version().decode()


def ttt_workspace_size(desc: TTTDesc, entry: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ttt_workspace_size(ctypes.byref(desc), int(entry), ctypes.byref(n)))
    return n.value


def ttt_saved_size(desc: TTTDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ttt_saved_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ttt_chunk_fwd(desc, q, k, v, beta, gamma, log_decay, w0, o, w_final, w_ckpt, saved, ws, ws_bytes=None,
                  stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().ttt_chunk_fwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(beta), _p(gamma),
                               _p(log_decay), _p(w0), _p(o), _p(w_final), _p(w_ckpt), _p(saved), _p(ws),
                               int(ws_bytes), _stream(stream)))


def ttt_chunk_bwd(desc, q, k, v, beta, gamma, log_decay, w0, w_ckpt, saved, d_o, d_wfinal, dq, dk, dv,
                  dbeta, dgamma, dlog_decay, dw0, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().ttt_chunk_bwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(beta), _p(gamma),
                               _p(log_decay), _p(w0), _p(w_ckpt), _p(saved), _p(d_o), _p(d_wfinal), _p(dq),
                               _p(dk), _p(dv), _p(dbeta), _p(dgamma), _p(dlog_decay), _p(dw0),
                               _p(ws), int(ws_bytes), _stream(stream)))


def ttt_chunk_bwd_noalloc(desc, q, k, v, beta, gamma, log_decay, w0, w_ckpt, saved, d_o, d_wfinal, dq, dk, dv,
                          dbeta, dgamma, dlog_decay, dw0, stream=None):
    _check(lib().ttt_chunk_bwd_noalloc(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(beta), _p(gamma),
                                       _p(log_decay), _p(w0), _p(w_ckpt), _p(saved), _p(d_o), _p(d_wfinal), _p(dq),
                                       _p(dk), _p(dv), _p(dbeta), _p(dgamma), _p(dlog_decay), _p(dw0),
                                       _stream(stream)))


def ttt_noalloc_scratch_bytes() -> int:
    return int(lib().ttt_noalloc_scratch_bytes())


def ttt_mlp_workspace_size(desc: TTTMlpDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ttt_mlp_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ttt_mlp_chunk_fwd(desc, q, k, v, beta, gamma, w1_0, w2_0, o, w1_final, w2_final, w1_ckpt, w2_ckpt, saved,
                      ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().ttt_mlp_chunk_fwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(beta), _p(gamma), _p(w1_0),
                                   _p(w2_0), _p(o), _p(w1_final), _p(w2_final), _p(w1_ckpt), _p(w2_ckpt),
                                   _p(saved), _p(ws), int(ws_bytes), _stream(stream)))


def ttt_mlp_saved_size(desc: TTTMlpDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ttt_mlp_saved_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ttt_mlp_bwd_workspace_size(desc: TTTMlpDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().ttt_mlp_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def ttt_mlp_chunk_bwd(desc, q, k, v, beta, gamma, w1_ckpt, w2_ckpt, saved, d_o, d_w1final, d_w2final, dq, dk, dv,
                      dbeta, dgamma, dw1_0, dw2_0, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().ttt_mlp_chunk_bwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(beta), _p(gamma), _p(w1_ckpt),
                                   _p(w2_ckpt), _p(saved), _p(d_o), _p(d_w1final), _p(d_w2final), _p(dq), _p(dk), _p(dv),
                                   _p(dbeta), _p(dgamma), _p(dw1_0), _p(dw2_0), _p(ws), int(ws_bytes),
                                   _stream(stream)))


def inplace_ttt_workspace_size(B, T, d_model, d_ff, C) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().inplace_ttt_workspace_size(int(B), int(T), int(d_model), int(d_ff), int(C), ctypes.byref(n)))
    return n.value


def inplace_ttt_fwd(B, T, d_model, d_ff, C, eta, z, vhat, w_down, o, ws=None, ws_bytes=0, stream=None):
    _check(lib().inplace_ttt_fwd(int(B), int(T), int(d_model), int(d_ff), int(C), float(eta),
                                 _p(z), _p(vhat), _p(w_down), _p(o), _p(ws), int(ws_bytes), _stream(stream)))


def inplace_ttt_guarded_workspace_size(B, T, d_model, d_ff, C) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().inplace_ttt_guarded_workspace_size(int(B), int(T), int(d_model), int(d_ff), int(C),
                                                    ctypes.byref(n)))
    return n.value


def inplace_ttt_fwd_guarded(B, T, d_model, d_ff, C, eta, clip_tau, doc_starts, z, vhat, w_init, w_down, o,
                            ws=None, ws_bytes=0, stream=None):
    """``doc_starts``: host sequence of flat positions b * T + t (0 < t < T), increasing."""
    starts = [int(p) for p in (doc_starts or [])]
    arr = (ctypes.c_int64 * len(starts))(*starts) if starts else None
    _check(lib().inplace_ttt_fwd_guarded(int(B), int(T), int(d_model), int(d_ff), int(C), float(eta),
                                         float(clip_tau), arr, len(starts), _p(z), _p(vhat), _p(w_init),
                                         _p(w_down), _p(o), _p(ws), int(ws_bytes), _stream(stream)))


def inplace_ttt_bwd_workspace_size(B, T, d_model, d_ff, C) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().inplace_ttt_bwd_workspace_size(int(B), int(T), int(d_model), int(d_ff), int(C), ctypes.byref(n)))
    return n.value


def inplace_ttt_bwd(B, T, d_model, d_ff, C, eta, z, vhat, w_final, d_o, d_wfinal, dz, dvhat, dw0, ws, ws_bytes,
                    stream=None):
    _check(lib().inplace_ttt_bwd(int(B), int(T), int(d_model), int(d_ff), int(C), float(eta), _p(z), _p(vhat),
                                 _p(w_final), _p(d_o), _p(d_wfinal), _p(dz), _p(dvhat), _p(dw0), _p(ws), int(ws_bytes),
                                 _stream(stream)))


def inplace_ttt_bwd_guarded_workspace_size(B, T, d_model, d_ff, C) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().inplace_ttt_bwd_guarded_workspace_size(int(B), int(T), int(d_model), int(d_ff), int(C),
                                                        ctypes.byref(n)))
    return n.value


def inplace_ttt_bwd_guarded(B, T, d_model, d_ff, C, eta, clip_tau, doc_starts, z, vhat, w0, w_init, w_final, d_o,
                            d_wfinal, dz, dvhat, dw0, dw_init, ws, ws_bytes, stream=None):
    """``doc_starts``: host sequence of flat positions b * T + t (0 < t < T), increasing."""
    starts = [int(p) for p in (doc_starts or [])]
    arr = (ctypes.c_int64 * len(starts))(*starts) if starts else None
    _check(lib().inplace_ttt_bwd_guarded(int(B), int(T), int(d_model), int(d_ff), int(C), float(eta),
                                         float(clip_tau), arr, len(starts), _p(z), _p(vhat), _p(w0), _p(w_init),
                                         _p(w_final), _p(d_o), _p(d_wfinal), _p(dz), _p(dvhat), _p(dw0),
                                         _p(dw_init), _p(ws), int(ws_bytes), _stream(stream)))


def ttt_timing_enable(on: bool) -> None:
    _check(lib().ttt_timing_enable(1 if on else 0))


def ttt_timing_read(kernel) -> tuple[float, int]:
    """(summed device milliseconds, launch count) of one kernel since the last enable."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    status = lib().ttt_timing_read(int(kernel), ctypes.byref(ms), ctypes.byref(n))
    if status != 0:
        raise TTTError(status, "ttt_timing_read failed")
    return ms.value, n.value
