"""ctypes binding of libadakv.so (include/adakv.h).  Argument marshalling only:
every step of the eviction path runs in the library's HIP kernels.

Functions keep the C names.  Buffer arguments are torch tensors on the GPU (or
None for NULL); `stream` defaults to torch's current stream.  A status other
than ADAKV_OK raises AdakvError.  When the built library is missing, load()
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libadakv.so")

ADAKV_OK, ADAKV_EINVAL, ADAKV_EUNSUPPORTED, ADAKV_ECAPACITY, ADAKV_EWORKSPACE, ADAKV_EHIP = range(6)
ADAKV_BF16, ADAKV_F32 = 0, 1
ADAKV_SCORE_SNAPKV, ADAKV_SCORE_LAVA, ADAKV_SCORE_CRITICALKV, ADAKV_SCORE_LAPROX = 0, 1, 2, 3
(ADAKV_ALLOC_ADA, ADAKV_ALLOC_LAVA_LAYERS, ADAKV_ALLOC_ADA_CRITICALKV, ADAKV_ALLOC_GLOBAL, ADAKV_ALLOC_ADA_FLOOR,
 ADAKV_ALLOC_STREAMING) = range(6)

EXPORTS = ("adakv_workspace_bytes", "adakv_score", "adakv_score_lse", "adakv_lse_from_causal", "adakv_allocate",
           "adakv_compact", "adakv_decode_attn", "adakv_decode_attn_noalloc", "adakv_strerror", "adakv_version",
           "adakv_lava_online_allocate", "adakv_lava_online_compact")


class AdakvShape(ctypes.Structure):
    _fields_ = [("n_inst", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("n", ctypes.c_int32), ("w", ctypes.c_int32),
                ("pool", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scorer", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("eps", ctypes.c_float), ("reserved0", ctypes.c_int32)]


class AdakvAlloc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("alpha_num", ctypes.c_int32), ("alpha_den", ctypes.c_int32),
                ("ck_num", ctypes.c_int32), ("ck_den", ctypes.c_int32), ("sinks", ctypes.c_int32),
                ("budget", ctypes.c_int64), ("inst_budget", ctypes.POINTER(ctypes.c_int64))]


class AdakvError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: status {status} ({strerror(status)})")


_lib = None
_vp = ctypes.c_void_p


def load(path: Optional[str] = None):
    """Load libadakv.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m adaptive_head_budget_amd.build`")
    lib = ctypes.CDLL(p)
    S, A = ctypes.POINTER(AdakvShape), ctypes.POINTER(AdakvAlloc)
    lib.adakv_workspace_bytes.argtypes = [S, A, ctypes.c_int32]
    lib.adakv_workspace_bytes.restype = ctypes.c_size_t
    lib.adakv_score.argtypes = [S, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.adakv_score.restype = ctypes.c_int
    lib.adakv_score_lse.argtypes = [S, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.adakv_score_lse.restype = ctypes.c_int
    lib.adakv_lse_from_causal.argtypes = [S, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.adakv_lse_from_causal.restype = ctypes.c_int
    lib.adakv_allocate.argtypes = [S, A, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.adakv_allocate.restype = ctypes.c_int
    lib.adakv_compact.argtypes = [S, A, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp]
    lib.adakv_compact.restype = ctypes.c_int
    lib.adakv_decode_attn.argtypes = [S, A, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_int32,
                                      _vp, _vp, ctypes.c_size_t, _vp]
    lib.adakv_decode_attn.restype = ctypes.c_int
    lib.adakv_decode_attn_noalloc.argtypes = [S, A, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32,
                                              ctypes.c_int32, _vp, _vp]
    lib.adakv_decode_attn_noalloc.restype = ctypes.c_int
    lib.adakv_lava_online_allocate.argtypes = [S, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               ctypes.c_size_t, _vp]
    lib.adakv_lava_online_allocate.restype = ctypes.c_int
    lib.adakv_lava_online_compact.argtypes = [S, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64,
                                              _vp, _vp, _vp, _vp, _vp]
    lib.adakv_lava_online_compact.restype = ctypes.c_int
    lib.adakv_strerror.argtypes = [ctypes.c_int]
    lib.adakv_strerror.restype = ctypes.c_char_p
    lib.adakv_version.argtypes = []
    lib.adakv_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().adakv_strerror(status).decode()


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("buffers must be contiguous")
    return t.data_ptr()


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(st: int, call: str):
    if st != ADAKV_OK:
        raise AdakvError(st, call)


def adakv_version() -> int:
    return load().adakv_version()


def adakv_workspace_bytes(shape: AdakvShape, alloc: Optional[AdakvAlloc], reserve: int) -> int:
    return load().adakv_workspace_bytes(ctypes.byref(shape), ctypes.byref(alloc) if alloc is not None else None,
                                        reserve)


def adakv_score(shape, q_win, k, v, w_o, score, score2, ws, stream=None):
    st = load().adakv_score(ctypes.byref(shape), _p(q_win), _p(k), _p(v), _p(w_o), _p(score), _p(score2),
                            _p(ws), _nbytes(ws), _stream(stream))
    _check(st, "adakv_score")


def adakv_score_lse(shape, q_win, k, v, w_o, row_lse, score, score2, ws, stream=None):
    st = load().adakv_score_lse(ctypes.byref(shape), _p(q_win), _p(k), _p(v), _p(w_o), _p(row_lse), _p(score),
                                _p(score2), _p(ws), _nbytes(ws), _stream(stream))
    _check(st, "adakv_score_lse")


def adakv_lse_from_causal(shape, q_win, k, lse_causal, lse_out, row_flag=None, stream=None):
    st = load().adakv_lse_from_causal(ctypes.byref(shape), _p(q_win), _p(k), _p(lse_causal), _p(lse_out),
                                      _p(row_flag), _stream(stream))
    _check(st, "adakv_lse_from_causal")


def adakv_allocate(shape, alloc, score, score2, budgets, sel, sel_off, ws, stream=None):
    st = load().adakv_allocate(ctypes.byref(shape), ctypes.byref(alloc), _p(score), _p(score2), _p(budgets),
                               _p(sel), _p(sel_off), _p(ws), _nbytes(ws), _stream(stream))
    _check(st, "adakv_allocate")


def adakv_compact(shape, alloc, k, v, budgets, sel, sel_off, reserve, k_flat, v_flat, seg_start, seg_len,
                  stream=None):
    st = load().adakv_compact(ctypes.byref(shape), ctypes.byref(alloc), _p(k), _p(v), _p(budgets), _p(sel),
                              _p(sel_off), reserve, _p(k_flat), _p(v_flat), _p(seg_start), _p(seg_len),
                              _stream(stream))
    _check(st, "adakv_compact")


def adakv_decode_attn(shape, alloc, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, reserve, step, out, ws,
                      stream=None):
    st = load().adakv_decode_attn(ctypes.byref(shape), ctypes.byref(alloc), _p(q), _p(k_new), _p(v_new),
                                  _p(k_flat), _p(v_flat), _p(seg_start), _p(seg_len), reserve, step, _p(out),
                                  _p(ws), _nbytes(ws), _stream(stream))
    _check(st, "adakv_decode_attn")


def adakv_decode_attn_noalloc(shape, alloc, q, k_new, v_new, k_flat, v_flat, seg_start, seg_len, reserve, step, out,
                              stream=None):
    st = load().adakv_decode_attn_noalloc(ctypes.byref(shape), ctypes.byref(alloc), _p(q), _p(k_new), _p(v_new),
                                          _p(k_flat), _p(v_flat), _p(seg_start), _p(seg_len), reserve, step, _p(out),
                                          _stream(stream))
    _check(st, "adakv_decode_attn_noalloc")


def adakv_lava_online_allocate(shape, total_budget, score, prev_sel_off, prev_budgets, prev_sel, layer_ent, budgets,
                               sel, sel_off, ws, stream=None):
    st = load().adakv_lava_online_allocate(ctypes.byref(shape), int(total_budget), _p(score), _p(prev_sel_off),
                                           _p(prev_budgets), _p(prev_sel), _p(layer_ent), _p(budgets), _p(sel),
                                           _p(sel_off), _p(ws), _nbytes(ws), _stream(stream))
    _check(st, "adakv_lava_online_allocate")


def adakv_lava_online_compact(shape, k_new, v_new, k_old, v_old, seg_start_old, sel_old, sel_off_old, budgets, sel,
                              sel_off, max_rows, k_flat, v_flat, seg_start, seg_len, stream=None):
    st = load().adakv_lava_online_compact(ctypes.byref(shape), _p(k_new), _p(v_new), _p(k_old), _p(v_old),
                                          _p(seg_start_old), _p(sel_old), _p(sel_off_old), _p(budgets), _p(sel),
                                          _p(sel_off), int(max_rows), _p(k_flat), _p(v_flat), _p(seg_start),
                                          _p(seg_len), _stream(stream))
    _check(st, "adakv_lava_online_compact")
