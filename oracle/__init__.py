"""CPU oracle for RTPurbo's head-split sparse attention -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU product path never does; it
shares no code with ``rtp_oracle.c``.

The arithmetic lives in ``rtp_oracle.c`` (plain C, fp32 fused-multiply-add
chains for the indexer, double precision for softmax mass and attention).
This module only marshals numpy arrays and composes the C steps in the order
the method runs them:

  indexer projection -> indexer scores -> top-p -> attention over the set
  (retrieval heads), window set -> attention (local heads), 0..pos ->
  attention (dense).

Method source: "Full Attention Strikes Back: Transferring Full Attention into
Sparse within Hundred Training Steps" (arXiv 2605.16928), abstract
observations (1)-(3); zhichai.net forum post "RTPurbo: Turning Dense LLMs into
Sparse Attention Models ...", sections "Three Key Insights" and "The RTPurbo
Method".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rtp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-mfma", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    """Compile rtp_oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i64, i32, f32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_double
            L.orc_project.argtypes = [P, i64, i64, i32, P, P]
            L.orc_project.restype = None
            L.orc_scores.argtypes = [P, P, i64, P]
            L.orc_scores.restype = ctypes.c_int
            L.orc_topp.argtypes = [P, i64, f64, f32, P, P, P]
            L.orc_topp.restype = i64
            L.orc_topk.argtypes = [P, i64, i64, P]
            L.orc_topk.restype = i64
            L.orc_attend.argtypes = [P, P, P, i64, i32, P, i64, f64, P]
            L.orc_attend.restype = None
            L.orc_window_set.argtypes = [i64, i64, i64, P]
            L.orc_window_set.restype = i64
            L.orc_f32_to_bf16.argtypes = [f32]
            L.orc_f32_to_bf16.restype = ctypes.c_uint16
            L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
            L.orc_bf16_to_f32.restype = f32
            L.orc_fp8e4m3_to_f32.argtypes = [ctypes.c_uint8]
            L.orc_fp8e4m3_to_f32.restype = f32
            L.orc_fp8_dequant.argtypes = [P, i64, f32, P]
            L.orc_fp8_dequant.restype = None
            _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def as_f32(x: np.ndarray) -> np.ndarray:
    """fp32 view of an input array: uint16 arrays hold bf16 bit patterns."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float32)


# --------------------------------------------------------------------------
# single steps
# --------------------------------------------------------------------------

def project(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """bf16 bits [rows,16] of the fp32 FMA chain x[i,:] . W[:,c] (d ascending)."""
    x = np.ascontiguousarray(as_f32(x))
    rows, D = x.shape
    Wf = np.ascontiguousarray(as_f32(W)).reshape(D, 16)
    out = np.empty((rows, 16), np.uint16)
    lib().orc_project(_p(x), rows, D, D, _p(Wf), _p(out))
    return out


def scores(q_low: np.ndarray, k_low: np.ndarray) -> np.ndarray:
    """fp32 indexer scores of one query row against k_low [L,16] (bf16 bits)."""
    q_low = np.ascontiguousarray(q_low, np.uint16).reshape(16)
    k_low = np.ascontiguousarray(k_low, np.uint16).reshape(-1, 16)
    d = np.empty(k_low.shape[0], np.float32)
    rc = lib().orc_scores(_p(q_low), _p(k_low), k_low.shape[0], _p(d))
    if rc != 0:
        raise ArithmeticError("an indexer product is not exact in fp32")
    return d


def topp(d: np.ndarray, s: float, p: float, want_order: bool = True):
    """(selected ascending int32, rank order int64 or None, C_k float64 or None)."""
    d = np.ascontiguousarray(d, np.float32)
    L = d.shape[0]
    sel = np.empty(L, np.int32)
    order = np.empty(L, np.int64) if want_order else None
    cum = np.empty(L, np.float64) if want_order else None
    k = lib().orc_topp(_p(d), L, float(s), float(np.float32(p)), _p(sel),
                       _p(order) if want_order else None,
                       _p(cum) if want_order else None)
    if k < 0:
        raise ValueError("top-p needs L >= 1 and p > 0")
    return sel[:k].copy(), order, cum


def topk(d: np.ndarray, k: int) -> np.ndarray:
    """Selected ascending int32: the first min(k, L) keys of the rank order
    (score descending, index ascending)."""
    d = np.ascontiguousarray(d, np.float32)
    L = d.shape[0]
    sel = np.empty(L, np.int32)
    n = lib().orc_topk(_p(d), L, int(k), _p(sel))
    if n < 0:
        raise ValueError("top-k needs L >= 1 and k >= 1")
    return sel[:n].copy()


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
           scale: float) -> np.ndarray:
    """double [D]: softmax(scale q.k_j) over idx, weighted sum of v_j.

    K and V are [L, D] fp32 (or bf16 bits); rows are addressed by idx.
    """
    q = np.ascontiguousarray(as_f32(q)).reshape(-1)
    K = np.ascontiguousarray(as_f32(K))
    V = np.ascontiguousarray(as_f32(V))
    D = q.shape[0]
    assert K.shape[1] == D and V.shape[1] == D
    idx = np.ascontiguousarray(idx, np.int32)
    if idx.size:
        assert idx.min() >= 0 and idx.max() < K.shape[0]
    out = np.empty(D, np.float64)
    lib().orc_attend(_p(q), _p(K), _p(V), D, D, _p(idx), idx.shape[0], float(scale), _p(out))
    return out


def window_set(pos: int, window: int, sinks: int) -> np.ndarray:
    out = np.empty(pos + 1, np.int32)
    n = lib().orc_window_set(pos, window, sinks, _p(out))
    return out[:n].copy()


def fp8_to_f32(code: int) -> float:
    """One FP8 E4M3 code as fp32."""
    return float(lib().orc_fp8e4m3_to_f32(int(code)))


def fp8_dequant(codes: np.ndarray, scale: float) -> np.ndarray:
    """fp32 values of FP8 E4M3 codes (uint8) times a scale (one fp32 rounding)."""
    c = np.ascontiguousarray(codes, np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().orc_fp8_dequant(_p(c), c.size, float(np.float32(scale)), _p(out))
    return out


def f32_to_bf16(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(x)))


# --------------------------------------------------------------------------
# composed rows
# --------------------------------------------------------------------------

def retrieval_row(q: np.ndarray, K: np.ndarray, V: np.ndarray, Wq: np.ndarray,
                  Wk: np.ndarray, pos: int, idx_scale: float, p: float,
                  attn_scale: float, k_low: np.ndarray | None = None,
                  want_order: bool = True, top_k: int = 0, k_max: int = 0) -> dict:
    """One retrieval-head query row at position pos (keys 0..pos).

    q: [D]; K, V: [>= pos+1, D] of this row's KV head; Wq, Wk: [D, 16].
    k_low may be passed when it is already known for the whole context.
    top_k > 0: fixed top-k selection instead of top-p (p is then unused).
    k_max > 0: the top-p set is capped at its first k_max keys in rank order.
    """
    L = pos + 1
    q_low = project(np.asarray(q).reshape(1, -1), Wq)[0]
    if k_low is None:
        k_low = project(np.asarray(K)[:L], Wk)
    d = scores(q_low, k_low[:L])
    if top_k > 0:
        sel = topk(d, top_k)
        _, order, cum = topp(d, idx_scale, 1.0, want_order) if want_order else (None, None, None)
    else:
        sel, order, cum = topp(d, idx_scale, p, want_order)
        if k_max > 0 and len(sel) > k_max:
            sel = topk(d, k_max)
    out = attend(q, np.asarray(K)[:L], np.asarray(V)[:L], sel, attn_scale)
    return dict(q_low=q_low, k_low=k_low, d=d, sel=sel, order=order, cum=cum, out=out)


def local_row(q, K, V, pos: int, window: int, sinks: int, attn_scale: float):
    idx = window_set(pos, window, sinks)
    return attend(q, np.asarray(K)[: pos + 1], np.asarray(V)[: pos + 1], idx, attn_scale)


def dense_row(q, K, V, pos: int, attn_scale: float):
    idx = np.arange(pos + 1, dtype=np.int32)
    return attend(q, np.asarray(K)[: pos + 1], np.asarray(V)[: pos + 1], idx, attn_scale)
