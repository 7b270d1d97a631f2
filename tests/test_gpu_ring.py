"""GPU parity of the cache-side layout (the full KV cache only for the KV heads
that serve a retrieval head, a window-only ring for the rest) and of the fused
K/V + indexer-key append (rtp_kv_append), through the C ABI:

  * rtp_kv_append writes the same K, V and indexer keys as the plain page
    fill followed by rtp_indexer_append (indexer keys bit-exact against the
    oracle);
  * on a ring cache, window attention of the local heads (decode and prefill
    chunks) matches the oracle's window sets and equals the full cache's
    output bit for bit; selection and sparse attention of the retrieval heads
    are unchanged;
  * dense attention and rings too short for the window are rejected.

Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dim_amd as rtp
import synth
from gpu_util import Dev, check_out, oracle_k_low, out_f32, say
from sparse_attention_dim_amd.paged import BLOCK, RingCache, bf16_bits, rtp_dtype, to_device

pytestmark = pytest.mark.gpu


def _ring_dev(w, ring_pages):
    d = Dev(w)                                        # the full cache, filled by rtp_indexer_append
    rc = RingCache(w.Hkv, w.D, w.Hq // w.Hkv, w.ret_heads, w.n_ret, [int(x) for x in w.seq_lens], w.dtype,
                   ring_pages, permute_seed=23, spare_blocks=2)
    rc.fill(d.layer, w.k, w.v, d.w_k)
    torch.cuda.synchronize()
    return d, rc


def _rows_equal(a: torch.Tensor, b: torch.Tensor):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a, b)


@pytest.mark.parametrize("wl,ring_pages", [(2, 4), (1, 5)], ids=["decode_bf16", "decode_f32"])
def test_ring_decode_window_and_retrieval(wl, ring_pages):
    w = synth.small(wl)
    say("[gpu] ring cache decode", w.name, "ring pages", ring_pages)
    d, rc = _ring_dev(w, ring_pages)
    say("   KV bytes: full %d, ring layout %d" % (2 * d.pc.k.numel() * d.pc.k.element_size(), rc.nbytes()))
    cache = rc.cache()
    # indexer keys: bit-exact, written by the fused append
    for b in range(w.B):
        for r in range(w.n_ret):
            np.testing.assert_array_equal(rc.k_low_logical(b, r), oracle_k_low(w, b, r))
    # local heads from the ring: equal to the full cache's output, bit for bit
    ws = torch.empty(rtp.window_attn_workspace(d.layer, cache, d.query), dtype=torch.uint8, device="cuda")
    out_ring = torch.zeros_like(d.q)
    rtp.window_attn(d.layer, cache, d.query, out_ring, ws)
    d.out.zero_()
    d.window()
    torch.cuda.synchronize()
    _rows_equal(out_ring, d.out)
    o = out_f32(out_ring)
    for t in range(w.n_tok):
        b, pos = w.row_seq(t), w.row_pos(t)
        for h in w.local_heads():
            g = w.kv_head(h)
            ref = oracle.local_row(w.q[t, h], w.k[b][:, g, :], w.v[b][:, g, :], pos, w.window, w.sinks,
                                   w.attn_scale)
            assert check_out(o[t, h], ref, w.dtype) <= 1.0, (t, h)
    # retrieval heads: selection and sparse attention read the full pages
    rows = d.rows
    cap = sum(int(x) for x in w.seq_lens) * w.n_ret
    rp_ring = torch.zeros(rows + 1, dtype=torch.int64, device="cuda")
    idx_ring = torch.zeros(cap, dtype=torch.int32, device="cuda")
    st_ring = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(rp_ring, idx_ring, st_ring)
    wsel = torch.empty(rtp.topp_select_workspace(d.layer, cache, d.query), dtype=torch.uint8, device="cuda")
    rtp.topp_select(d.layer, cache, d.query, d.w_q, d.top_p, sel, wsel)
    wsp = torch.empty(rtp.sparse_attn_workspace(d.layer, cache, d.query, cap), dtype=torch.uint8, device="cuda")
    rtp.sparse_attn_decode(d.layer, cache, d.query, sel, out_ring, wsp)
    d.select(capacity=cap)
    d.sparse()
    torch.cuda.synchronize()
    assert int(st_ring.item()) == 0
    assert torch.equal(rp_ring, d.row_ptr)
    n = int(rp_ring[-1].item())
    assert torch.equal(idx_ring[:n], d.idx[:n])
    _rows_equal(out_ring, d.out)
    # dense attention needs every key
    wsd = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(rtp.RtpError):
        rtp.dense_attn(d.layer, cache, d.query, torch.zeros_like(d.q), wsd)


def test_ring_prefill_chunk_window():
    w = synth.small(3)                              # L = 5000, chunk 300, window 500
    say("[gpu] ring cache prefill", w.name)
    d, rc = _ring_dev(w, 6)                         # 5 * 256 >= 500 + 255 + 299
    cache = rc.cache()
    out_ring = torch.zeros_like(d.q)
    rtp.window_attn(d.layer, cache, d.query, out_ring, None)
    d.out.zero_()
    d.window()
    torch.cuda.synchronize()
    _rows_equal(out_ring, d.out)
    o = out_f32(out_ring)
    for t in range(0, w.n_tok, 5):
        pos = w.row_pos(t)
        for h in w.local_heads()[::3]:
            g = w.kv_head(h)
            ref = oracle.local_row(w.q[t, h], w.k[0][:, g, :], w.v[0][:, g, :], pos, w.window, w.sinks,
                                   w.attn_scale)
            assert check_out(o[t, h], ref, w.dtype) <= 1.0, (t, h)
    # sparse prefill of the retrieval heads from the full pages
    st, rp, sets = d.select()
    cap = d.sel.capacity
    wsp = torch.empty(rtp.sparse_attn_workspace(d.layer, cache, d.query, cap), dtype=torch.uint8, device="cuda")
    rtp.sparse_attn_prefill(d.layer, cache, d.query, d.sel, out_ring, wsp)
    d.sparse()
    torch.cuda.synchronize()
    _rows_equal(out_ring, d.out)
    # a ring too short for the chunk's window span is rejected on the host
    short = RingCache(w.Hkv, w.D, w.Hq // w.Hkv, w.ret_heads, w.n_ret, [int(x) for x in w.seq_lens], w.dtype, 4)
    with pytest.raises(rtp.RtpError):
        rtp.window_attn(d.layer, short.cache(), d.query, out_ring, None)


@pytest.mark.parametrize("wl", [2, 1], ids=["bf16", "f32"])
def test_kv_append_equals_page_fill_and_indexer_append(wl):
    # without a ring, rtp_kv_append writes exactly the pages of the plain
    # fill and the indexer keys of rtp_indexer_append
    w = synth.small(wl)
    say("[gpu] kv append vs page fill", w.name)
    d = Dev(w)
    k2 = torch.zeros_like(d.pc.k)
    v2 = torch.zeros_like(d.pc.v)
    kl2 = torch.zeros_like(d.pc.k_low)
    cache2 = rtp.make_cache(k2, v2, kl2, d.pc.block_table, d.pc.seq_lens, max(d.pc.lens))
    for b in range(w.B):
        L = d.pc.lens[b]
        for j0 in range(0, L, 1000):                 # several calls, ragged last one
            j1 = min(L, j0 + 1000)
            kn = to_device(np.ascontiguousarray(w.k[b][j0:j1]))
            vn = to_device(np.ascontiguousarray(w.v[b][j0:j1]))
            sid = torch.full((j1 - j0,), b, dtype=torch.int32, device="cuda")
            pos = torch.arange(j0, j1, dtype=torch.int32, device="cuda")
            rtp.kv_append(d.layer, cache2, kn, vn, d.w_k, sid, pos)
    torch.cuda.synchronize()
    _rows_equal(k2, d.pc.k)
    _rows_equal(v2, d.pc.v)
    _rows_equal(kl2, d.pc.k_low)
