"""The C ABI on the CPU: librtp.so loads, exports every entry point that
include/rtp.h declares, and rejects invalid arguments on the host before
anything is enqueued (no GPU needed: no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

import sparse_attention_dim_amd as rtp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtp.h")
FAKE = 0x1000          # a non-NULL pointer value that the host checks never dereference


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rtp_[a-z_]+)\s*\(", src)))


def test_header_declares_the_five_hot_path_calls():
    names = declared()
    for n in ("rtp_indexer_append", "rtp_topp_select", "rtp_sparse_attn_decode",
              "rtp_sparse_attn_prefill", "rtp_window_attn"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = rtp.load()
    for n in declared():
        assert hasattr(lib, n), n
    assert sorted(declared()) == sorted(rtp.ENTRY_POINTS)
    assert rtp.version() == 2


def test_no_cpu_fallback_when_library_missing(tmp_path):
    saved = rtp._lib
    rtp._lib = None
    try:
        with pytest.raises(RuntimeError):
            rtp.load(str(tmp_path / "missing.so"))
    finally:
        rtp._lib = saved


def _layer(**kw):
    a = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=rtp.RTP_BF16, ret_heads=[1, 5, 9],
             window=2048, num_sinks=64, attn_scale=0.088, idx_scale=0.25)
    a.update(kw)
    return rtp.make_layer(**a)


def _cache(batch=2, max_blocks=4, max_seq_len=1000, null=None):
    C = rtp.Cache()
    C.k = C.v = C.k_low = C.block_table = C.seq_lens = FAKE
    if null:
        setattr(C, null, None)
    C.batch, C.max_blocks, C.max_seq_len = batch, max_blocks, max_seq_len
    return C


def _query(n_tok=2, kind=rtp.RTP_DECODE, seq=0, pos0=0):
    Q = rtp.Query()
    Q.q, Q.n_tok, Q.kind, Q.seq, Q.pos0 = FAKE, n_tok, kind, seq, pos0
    return Q


def _sel(capacity=100):
    S = rtp.Sel()
    S.row_ptr, S.idx, S.status, S.capacity = FAKE, FAKE, FAKE, capacity
    return S


def _window(layer, cache, query, ws_bytes=1 << 30):
    lib = rtp.load()
    return lib.rtp_window_attn(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), FAKE, FAKE,
                               ws_bytes, None)


def _select(layer, cache, query, sel, ws_bytes=1 << 40, fn="rtp_topp_select"):
    lib = rtp.load()
    return getattr(lib, fn)(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), FAKE, FAKE,
                            ctypes.byref(sel), FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_kv_heads=7), rtp.RTP_EINVAL),            # Hq % Hkv != 0
    (dict(head_dim=96), rtp.RTP_EUNSUPPORTED),
    (dict(ret_heads=[]), rtp.RTP_EINVAL),
    (dict(ret_heads=[3, 3]), rtp.RTP_EINVAL),          # not strictly ascending
    (dict(ret_heads=[40]), rtp.RTP_EINVAL),            # out of range
    (dict(window=0), rtp.RTP_EINVAL),
    (dict(num_sinks=-1), rtp.RTP_EINVAL),
    (dict(attn_scale=0.0), rtp.RTP_EINVAL),
    (dict(idx_scale=float("nan")), rtp.RTP_EINVAL),
    (dict(dtype=5), rtp.RTP_EINVAL),
    (dict(num_q_heads=64, num_kv_heads=4), rtp.RTP_EUNSUPPORTED),   # 16 query heads per KV head
    (dict(k_max=-1), rtp.RTP_EINVAL),
    (dict(flags=4), rtp.RTP_EINVAL),                   # unknown flag
])
def test_layer_checks(kw, code):
    assert _window(_layer(**kw), _cache(), _query()) == code
    assert rtp.load().rtp_last_error()


@pytest.mark.parametrize("ckw,qkw,code", [
    (dict(null="k_low"), {}, rtp.RTP_EINVAL),
    (dict(batch=0), {}, rtp.RTP_EINVAL),
    (dict(max_blocks=3, max_seq_len=1000), {}, rtp.RTP_EINVAL),       # 3 pages < 1000 tokens
    (dict(max_seq_len=(1 << 20) + 1, max_blocks=20000), {}, rtp.RTP_EUNSUPPORTED),
    ({}, dict(n_tok=3), rtp.RTP_EINVAL),                               # decode n_tok != batch
    ({}, dict(kind=rtp.RTP_CHUNK, n_tok=10, seq=2), rtp.RTP_EINVAL),   # seq out of range
    ({}, dict(kind=rtp.RTP_CHUNK, n_tok=10, pos0=995), rtp.RTP_EINVAL),  # rows past max_seq_len
    ({}, dict(kind=7), rtp.RTP_EINVAL),
    ({}, dict(n_tok=0), rtp.RTP_EINVAL),
])
def test_cache_and_query_checks(ckw, qkw, code):
    assert _window(_layer(), _cache(**ckw), _query(**qkw)) == code


def test_workspace_too_small():
    L, C, Q = _layer(), _cache(), _query()
    need = rtp.load().rtp_window_attn_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    assert need > 0
    assert _window(L, C, Q, ws_bytes=need - 1) == rtp.RTP_EWORKSPACE
    sel_need = rtp.load().rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    assert sel_need > 0
    assert _select(L, C, Q, _sel(), ws_bytes=sel_need - 1) == rtp.RTP_EWORKSPACE


@pytest.mark.parametrize("fn", ["rtp_topp_select", "rtp_topp_select_begin", "rtp_topp_select_end"])
def test_select_checks(fn):
    L, C, Q = _layer(), _cache(), _query()
    bad = _sel()
    bad.status = None
    assert _select(L, C, Q, bad, fn=fn) == rtp.RTP_EINVAL
    bad = _sel(capacity=-1)
    assert _select(L, C, Q, bad, fn=fn) == rtp.RTP_EINVAL
    sel_need = rtp.load().rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    assert _select(L, C, Q, _sel(), ws_bytes=sel_need - 1, fn=fn) == rtp.RTP_EWORKSPACE


def test_prepared_call_reports_the_same_errors():
    # a prepared call checks its arguments on every call, like the direct one
    L, C, Q = _layer(), _cache(), _query()
    bad = _sel()
    bad.status = None
    call = rtp.topp_select(L, C, Q, None, None, bad, None, stream=0, prepare=True)
    assert isinstance(call, rtp.Call)
    for _ in range(2):
        with pytest.raises(rtp.RtpError) as e:
            call()
        assert e.value.code == rtp.RTP_EINVAL
    with pytest.raises(rtp.RtpError):
        rtp.topp_select(L, C, Q, None, None, bad, None, stream=0)


def test_sparse_entry_points_check_query_kind():
    lib = rtp.load()
    L, C = _layer(), _cache()
    S = _sel()
    chunk = _query(kind=rtp.RTP_CHUNK, n_tok=10, pos0=100)
    assert lib.rtp_sparse_attn_decode(ctypes.byref(L), ctypes.byref(C), ctypes.byref(chunk), ctypes.byref(S),
                                      FAKE, FAKE, 1 << 40, None) == rtp.RTP_EINVAL
    dec = _query()
    assert lib.rtp_sparse_attn_prefill(ctypes.byref(L), ctypes.byref(C), ctypes.byref(dec), ctypes.byref(S),
                                       FAKE, FAKE, 1 << 40, None) == rtp.RTP_EINVAL


def test_append_zero_tokens_is_a_noop_and_checks_pointers():
    lib = rtp.load()
    L, C = _layer(), _cache()
    assert lib.rtp_indexer_append(ctypes.byref(L), ctypes.byref(C), FAKE, FAKE, FAKE, 0, None) == rtp.RTP_OK
    assert lib.rtp_indexer_append(ctypes.byref(L), ctypes.byref(C), None, FAKE, FAKE, 5, None) == rtp.RTP_EINVAL
    assert lib.rtp_indexer_append(ctypes.byref(L), ctypes.byref(C), FAKE, FAKE, FAKE, -1, None) == rtp.RTP_EINVAL


def test_workspace_sizes_grow_with_context():
    lib = rtp.load()
    L = _layer()
    small = lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(_cache(max_seq_len=1000)),
                                          ctypes.byref(_query()))
    big = lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(_cache(max_blocks=512, max_seq_len=131072)),
                                        ctypes.byref(_query()))
    assert big > small > 0
    assert lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(_cache(batch=0)), ctypes.byref(_query())) == 0


def test_chunk_select_minimum_workspace():
    # a bf16 prefill chunk: the recommended size holds a candidate buffer per
    # row; anything down to the minimum is accepted, below it is rejected
    lib = rtp.load()
    L = _layer()
    C = _cache(max_blocks=64, max_seq_len=16384)
    Q = _query(kind=rtp.RTP_CHUNK, n_tok=300, pos0=5000)
    full = lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    low = lib.rtp_topp_select_workspace_min(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    rows = 300 * 3
    assert 0 < low < full and full - low == rows * 4096 * 8
    assert _select(L, C, Q, _sel(), ws_bytes=low - 1) == rtp.RTP_EWORKSPACE
    # decode queries: one size
    D = _query()
    assert (lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(D)) ==
            lib.rtp_topp_select_workspace_min(ctypes.byref(L), ctypes.byref(C), ctypes.byref(D)))


def test_topk_and_paths_checks():
    lib = rtp.load()
    L, C, Q = _layer(), _cache(), _query()
    need = lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    topk = lib.rtp_topk_select
    for k in (0, -3):
        assert topk(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), FAKE, k, ctypes.byref(_sel()), FAKE,
                    need, None) == rtp.RTP_EINVAL
    bad = _sel()
    bad.row_ptr = None
    assert topk(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), FAKE, 8, ctypes.byref(bad), FAKE, need,
                None) == rtp.RTP_EINVAL
    assert topk(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), FAKE, 8, ctypes.byref(_sel()), FAKE,
                need - 1, None) == rtp.RTP_EWORKSPACE
    # top-p needs its p array; top-k does not (checked before any launch)
    assert lib.rtp_topp_select(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), FAKE, None, ctypes.byref(_sel()),
                               FAKE, need, None) == rtp.RTP_EINVAL
    paths = lib.rtp_topp_select_paths
    assert paths(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), FAKE, need, None, None) == rtp.RTP_EINVAL
    assert paths(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), FAKE, need - 1, FAKE, None) == rtp.RTP_EWORKSPACE


def test_max_len_constant_matches_header():
    src = open(HEADER).read()
    assert "#define RTP_MAX_LEN (1 << 20)" in src and rtp.RTP_MAX_LEN == 1 << 20


def test_noalloc_select_rejects_queries_beyond_its_scratch():
    # 48 decode rows over 2^20 keys need ~200 MB of scores: more than the
    # static scratch array, so the call fails on the host (nothing enqueued);
    # bad arguments are reported as by rtp_topp_select
    lib = rtp.load()
    L = _layer()
    C = _cache(batch=16, max_blocks=4096, max_seq_len=1 << 20)
    Q = _query(n_tok=16)
    need = lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    assert need > rtp.RTP_NOALLOC_SCRATCH_BYTES
    fn = lib.rtp_topp_select_noalloc
    assert fn(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), FAKE, FAKE, ctypes.byref(_sel()),
              None) == rtp.RTP_EWORKSPACE
    assert b"scratch" in lib.rtp_last_error()
    assert fn(ctypes.byref(_layer(window=0)), ctypes.byref(C), ctypes.byref(Q), FAKE, FAKE, ctypes.byref(_sel()),
              None) == rtp.RTP_EINVAL


def test_decode_attn_checks():
    # the decode step's call checks its arguments on the host like the
    # calls it stands for (nothing is enqueued on an error)
    lib = rtp.load()
    L, C, Q = _layer(), _cache(), _query()
    need = lib.rtp_decode_attn_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), 100)
    sel_need = lib.rtp_topp_select_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    sp_need = lib.rtp_sparse_attn_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q), 100)
    win_need = lib.rtp_window_attn_workspace(ctypes.byref(L), ctypes.byref(C), ctypes.byref(Q))
    assert need == sel_need + sp_need + win_need
    fn = lib.rtp_decode_attn

    def call(layer=L, cache=C, query=Q, sel=None, out=FAKE, ws_bytes=need):
        return fn(ctypes.byref(layer), ctypes.byref(cache), ctypes.byref(query), FAKE, None, FAKE,
                  ctypes.byref(sel or _sel()), out, FAKE, ws_bytes, None)

    assert call(ws_bytes=need - 1) == rtp.RTP_EWORKSPACE
    assert call(out=None) == rtp.RTP_EINVAL
    assert call(layer=_layer(window=0)) == rtp.RTP_EINVAL
    assert call(query=_query(kind=rtp.RTP_CHUNK, n_tok=10)) == rtp.RTP_EINVAL
    assert call(sel=_sel(capacity=-1)) == rtp.RTP_EINVAL
    big = _cache(batch=1500, max_blocks=4, max_seq_len=1000)       # 4500 rows: more than the sparse kernel's 4096
    assert call(cache=big, query=_query(n_tok=1500), ws_bytes=1 << 40) == rtp.RTP_EUNSUPPORTED


def test_decode_attn_gqa_shared_checks():
    # shared gathers: more workspace (partials of every head slot, the unions),
    # and at most four retrieval heads per KV head
    lib = rtp.load()
    C, Q = _cache(), _query()
    L0 = _layer()
    L1 = _layer(flags=rtp.RTP_FLAG_GQA_SHARED)
    n0 = lib.rtp_decode_attn_workspace(ctypes.byref(L0), ctypes.byref(C), ctypes.byref(Q), 100)
    n1 = lib.rtp_decode_attn_workspace(ctypes.byref(L1), ctypes.byref(C), ctypes.byref(Q), 100)
    assert n1 > n0
    many = rtp.make_layer(16, 2, 128, rtp.RTP_BF16, [0, 1, 2, 3, 4], 64, 4, 0.088, 0.25,
                          flags=rtp.RTP_FLAG_GQA_SHARED)     # five retrieval heads on KV head 0
    need = lib.rtp_decode_attn_workspace(ctypes.byref(many), ctypes.byref(C), ctypes.byref(Q), 100)
    assert need > 0
    r = lib.rtp_decode_attn(ctypes.byref(many), ctypes.byref(C), ctypes.byref(Q), FAKE, None, FAKE,
                            ctypes.byref(_sel()), FAKE, FAKE, need, None)
    assert r == rtp.RTP_EUNSUPPORTED
    assert b"KV head" in lib.rtp_last_error()
    bad = _layer(flags=8)
    assert lib.rtp_decode_attn_workspace(ctypes.byref(bad), ctypes.byref(C), ctypes.byref(Q), 100) == 0
