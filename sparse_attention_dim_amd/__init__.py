"""Python binding of librtp (the gfx950 HIP implementation of RTPurbo's
head-split sparse attention hot path).

Argument marshalling only: every function here fills the C structs of
``include/rtp.h`` from torch tensors (device pointers) and calls the entry
point of the same name on the current HIP stream.  All computation happens in
the HIP kernels of ``librtp.so``; there is no CPU fallback, and loading fails
loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librtp.so")

RTP_OK, RTP_EINVAL, RTP_EUNSUPPORTED, RTP_EHIP, RTP_EWORKSPACE = 0, 1, 2, 3, 4
RTP_F32, RTP_BF16 = 0, 1
RTP_DECODE, RTP_CHUNK = 0, 1
RTP_BLOCK = 256
RTP_MAX_RET = 64
RTP_MAX_LEN = 1 << 20
RTP_FLAG_EXACT_MASS = 1
RTP_FLAG_GQA_SHARED = 2
RTP_NOALLOC_SCRATCH_BYTES = 64 << 20
# selection status word
SEL_OK, SEL_OVERFLOW, SEL_UNCERTIFIED, SEL_BAD_TOP_P = 0, 1, 2, 3
# per-row path codes of rtp_topp_select_paths
PATH_ALL, PATH_TINY, PATH_ROW, PATH_LARGE, PATH_LEVEL, PATH_LIST, PATH_SCAN, PATH_LIST_G = 1, 2, 3, 4, 5, 6, 7, 8
PATH_BITMAP, PATH_MERGE, PATH_EXACT_Z, PATH_COUNT, PATH_FROM_SCORES = 16, 32, 64, 128, 256

ENTRY_POINTS = (
    "rtp_version", "rtp_last_error", "rtp_indexer_append", "rtp_kv_append", "rtp_topp_select_workspace",
    "rtp_topp_select_workspace_min",
    "rtp_topp_select", "rtp_topp_select_begin", "rtp_topp_select_end", "rtp_topp_select_noalloc",
    "rtp_topk_select",
    "rtp_topp_select_paths", "rtp_indexer_scores",
    "rtp_sparse_attn_workspace",
    "rtp_sparse_attn_decode", "rtp_sparse_attn_prefill", "rtp_decode_attn_workspace",
    "rtp_decode_attn", "rtp_window_attn_workspace",
    "rtp_dense_attn_workspace", "rtp_window_attn", "rtp_dense_attn",
)


class RtpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("rtp status %d: %s" % (code, msg))
        self.code = code


class Layer(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("num_ret", ctypes.c_int32), ("ret_heads", ctypes.c_int32 * RTP_MAX_RET),
                ("window", ctypes.c_int32), ("num_sinks", ctypes.c_int32),
                ("attn_scale", ctypes.c_float), ("idx_scale", ctypes.c_float),
                ("k_max", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("kv_fp8", ctypes.c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_low", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32),
                ("k_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p), ("ring_table", ctypes.c_void_p),
                ("ring_pages", ctypes.c_int32)]


class Query(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("n_tok", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("seq", ctypes.c_int32), ("pos0", ctypes.c_int32)]


class Sel(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("status", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librtp.so; raises if it is missing (build it with __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("librtp.so is not built (%s); run __graft_entry__.build()" % path)
    # PyTorch (the memory and stream provider) first, so that the library
    # binds to the HIP runtime torch has loaded: a second runtime loaded ahead
    # of it would not see the device memory torch hands out
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    P, S, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    pl, pc, pq, ps = (ctypes.POINTER(Layer), ctypes.POINTER(Cache), ctypes.POINTER(Query),
                      ctypes.POINTER(Sel))
    sig = {
        "rtp_version": ([], ctypes.c_int),
        "rtp_last_error": ([], ctypes.c_char_p),
        "rtp_indexer_append": ([pl, pc, P, P, P, i32, P], ctypes.c_int),
        "rtp_kv_append": ([pl, pc, P, P, P, P, P, i32, P], ctypes.c_int),
        "rtp_topp_select_workspace": ([pl, pc, pq], S),
        "rtp_topp_select_workspace_min": ([pl, pc, pq], S),
        "rtp_topp_select": ([pl, pc, pq, P, P, ps, P, S, P], ctypes.c_int),
        "rtp_topp_select_begin": ([pl, pc, pq, P, P, ps, P, S, P], ctypes.c_int),
        "rtp_topp_select_end": ([pl, pc, pq, P, P, ps, P, S, P], ctypes.c_int),
        "rtp_topp_select_noalloc": ([pl, pc, pq, P, P, ps, P], ctypes.c_int),
        "rtp_topk_select": ([pl, pc, pq, P, i32, ps, P, S, P], ctypes.c_int),
        "rtp_topp_select_paths": ([pl, pc, pq, P, S, P, P], ctypes.c_int),
        "rtp_indexer_scores": ([pl, pc, pq, P, P, P, i64, P], ctypes.c_int),
        "rtp_sparse_attn_workspace": ([pl, pc, pq, i64], S),
        "rtp_sparse_attn_decode": ([pl, pc, pq, ps, P, P, S, P], ctypes.c_int),
        "rtp_sparse_attn_prefill": ([pl, pc, pq, ps, P, P, S, P], ctypes.c_int),
        "rtp_decode_attn_workspace": ([pl, pc, pq, i64], S),
        "rtp_decode_attn": ([pl, pc, pq, P, P, P, ps, P, P, S, P], ctypes.c_int),
        "rtp_window_attn_workspace": ([pl, pc, pq], S),
        "rtp_dense_attn_workspace": ([pl, pc, pq], S),
        "rtp_window_attn": ([pl, pc, pq, P, P, S, P], ctypes.c_int),
        "rtp_dense_attn": ([pl, pc, pq, P, P, S, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _check(code: int) -> None:
    if code != RTP_OK:
        raise RtpError(code, load().rtp_last_error().decode())


class Call:
    """One library call with its arguments marshalled once: struct references,
    device pointer values, sizes and the stream handle.  Calling the object
    issues the call again with the same arguments (on the stream fixed when it
    was made), costing one ctypes call; errors raise RtpError.  The object keeps
    the argument structs alive; the tensors behind the pointers must outlive it."""

    __slots__ = ("fn", "args", "keep")

    def __init__(self, name: str, args: tuple, keep: tuple):
        self.fn = getattr(load(), name)
        self.args = args
        self.keep = keep

    def __call__(self) -> None:
        code = self.fn(*self.args)
        if code != RTP_OK:
            _check(code)


def _run(name: str, args: tuple, keep: tuple, prepare: bool):
    c = Call(name, args, keep)
    if prepare:
        return c
    c()
    return None


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_layer(num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: int, ret_heads,
               window: int, num_sinks: int, attn_scale: float, idx_scale: float, k_max: int = 0,
               flags: int = 0, kv_fp8: int = 0, k_scale: float = 1.0, v_scale: float = 1.0) -> Layer:
    L = Layer()
    L.num_q_heads, L.num_kv_heads, L.head_dim, L.dtype = num_q_heads, num_kv_heads, head_dim, dtype
    rh = list(ret_heads)
    L.num_ret = len(rh)
    for i, h in enumerate(rh):
        L.ret_heads[i] = int(h)
    L.window, L.num_sinks = window, num_sinks
    L.attn_scale, L.idx_scale = attn_scale, idx_scale
    L.k_max, L.flags = k_max, flags
    L.kv_fp8, L.k_scale, L.v_scale = kv_fp8, k_scale, v_scale
    return L


def make_cache(k, v, k_low, block_table, seq_lens, max_seq_len: int, k_ring=None, v_ring=None,
               ring_table=None) -> Cache:
    C = Cache()
    C.k, C.v, C.k_low = _ptr(k), _ptr(v), _ptr(k_low)
    C.block_table, C.seq_lens = _ptr(block_table), _ptr(seq_lens)
    C.batch = block_table.shape[0]
    C.max_blocks = block_table.shape[1]
    C.max_seq_len = int(max_seq_len)
    if k_ring is not None:
        C.k_ring, C.v_ring, C.ring_table = _ptr(k_ring), _ptr(v_ring), _ptr(ring_table)
        C.ring_pages = ring_table.shape[1]
    return C


def make_query(q, kind: int, seq: int = 0, pos0: int = 0) -> Query:
    Q = Query()
    Q.q, Q.n_tok, Q.kind, Q.seq, Q.pos0 = _ptr(q), q.shape[0], kind, seq, pos0
    return Q


def make_sel(row_ptr, idx, status) -> Sel:
    S = Sel()
    S.row_ptr, S.idx, S.status = _ptr(row_ptr), _ptr(idx), _ptr(status)
    S.capacity = 0 if idx is None else idx.numel()
    return S


def version() -> int:
    return load().rtp_version()


def indexer_append(layer, cache, w_k, seq_id, pos, stream=None, prepare=False):
    return _run("rtp_indexer_append", (ctypes.byref(layer), ctypes.byref(cache), _ptr(w_k), _ptr(seq_id),
                                       _ptr(pos), seq_id.numel(), _stream(stream)), (layer, cache), prepare)


def kv_append(layer, cache, k_new, v_new, w_k, seq_id, pos, stream=None, prepare=False):
    """K/V rows of new tokens into the cache (and the ring) with their indexer keys, one launch."""
    return _run("rtp_kv_append", (ctypes.byref(layer), ctypes.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(w_k),
                                  _ptr(seq_id), _ptr(pos), seq_id.numel(), _stream(stream)), (layer, cache), prepare)


def topp_select_workspace(layer, cache, query) -> int:
    return load().rtp_topp_select_workspace(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query))


def topp_select_workspace_min(layer, cache, query) -> int:
    return load().rtp_topp_select_workspace_min(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query))


def topp_select(layer, cache, query, w_q, top_p, sel, ws, stream=None, prepare=False):
    return _run("rtp_topp_select", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(w_q),
                            _ptr(top_p), ctypes.byref(sel), _ptr(ws), _nbytes(ws), _stream(stream)),
                (layer, cache, query, sel), prepare)


def topp_select_begin(layer, cache, query, w_q, top_p, sel, ws, stream=None, prepare=False):
    """First phase of topp_select (the pass over the indexer keys); same arguments."""
    return _run("rtp_topp_select_begin", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(w_q),
                            _ptr(top_p), ctypes.byref(sel), _ptr(ws), _nbytes(ws), _stream(stream)),
                (layer, cache, query, sel), prepare)


def topp_select_end(layer, cache, query, w_q, top_p, sel, ws, stream=None, prepare=False):
    """Second phase of topp_select (cut and selected sets); same arguments as the first."""
    return _run("rtp_topp_select_end", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(w_q),
                            _ptr(top_p), ctypes.byref(sel), _ptr(ws), _nbytes(ws), _stream(stream)),
                (layer, cache, query, sel), prepare)


def topp_select_noalloc(layer, cache, query, w_q, top_p, sel, stream=None, prepare=False):
    """topp_select with the library's static scratch array instead of a workspace."""
    return _run("rtp_topp_select_noalloc", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query),
                                            _ptr(w_q), _ptr(top_p), ctypes.byref(sel), _stream(stream)),
                (layer, cache, query, sel), prepare)


def topk_select(layer, cache, query, w_q, k: int, sel, ws, stream=None, prepare=False):
    """Fixed top-k selection (same workspace as topp_select)."""
    return _run("rtp_topk_select", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(w_q),
                                    int(k), ctypes.byref(sel), _ptr(ws), _nbytes(ws), _stream(stream)),
                (layer, cache, query, sel), prepare)


def topp_select_paths(layer, cache, query, ws, paths, stream=None, prepare=False):
    """Per-row path codes (int32 device tensor [rows]) of the last selection run on ws."""
    return _run("rtp_topp_select_paths", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(ws),
                                          _nbytes(ws), _ptr(paths), _stream(stream)), (layer, cache, query), prepare)


def indexer_scores(layer, cache, query, w_q, q_low, scores, stream=None, prepare=False):
    return _run("rtp_indexer_scores", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(w_q),
                                       _ptr(q_low), _ptr(scores), scores.shape[1], _stream(stream)),
                (layer, cache, query), prepare)


def sparse_attn_workspace(layer, cache, query, capacity: int) -> int:
    return load().rtp_sparse_attn_workspace(ctypes.byref(layer), ctypes.byref(cache),
                                            ctypes.byref(query), capacity)


def sparse_attn_decode(layer, cache, query, sel, out, ws, stream=None, prepare=False):
    return _run("rtp_sparse_attn_decode", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query),
                                           ctypes.byref(sel), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)),
                (layer, cache, query, sel), prepare)


def sparse_attn_prefill(layer, cache, query, sel, out, ws, stream=None, prepare=False):
    return _run("rtp_sparse_attn_prefill", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query),
                                            ctypes.byref(sel), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)),
                (layer, cache, query, sel), prepare)


def decode_attn_workspace(layer, cache, query, capacity: int) -> int:
    return load().rtp_decode_attn_workspace(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), capacity)


def decode_attn(layer, cache, query, w_q, top_p, sel, out, ws, w_k=None, stream=None, prepare=False):
    """The attention of one decode step in one call: selection and sparse
    attention of the retrieval heads, window attention of the local heads
    (with w_k: the step's indexer keys appended first)."""
    return _run("rtp_decode_attn", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(w_q),
                                    _ptr(w_k), _ptr(top_p), ctypes.byref(sel), _ptr(out), _ptr(ws), _nbytes(ws),
                                    _stream(stream)), (layer, cache, query, sel), prepare)


def window_attn_workspace(layer, cache, query) -> int:
    return load().rtp_window_attn_workspace(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query))


def dense_attn_workspace(layer, cache, query) -> int:
    return load().rtp_dense_attn_workspace(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query))


def window_attn(layer, cache, query, out, ws, stream=None, prepare=False):
    return _run("rtp_window_attn", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(out),
                                    _ptr(ws), _nbytes(ws), _stream(stream)), (layer, cache, query), prepare)


def dense_attn(layer, cache, query, out, ws, stream=None, prepare=False):
    return _run("rtp_dense_attn", (ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), _ptr(out),
                                   _ptr(ws), _nbytes(ws), _stream(stream)), (layer, cache, query), prepare)