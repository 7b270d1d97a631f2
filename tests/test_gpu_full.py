"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark uses, on sampled rows the oracle computes one by one:

  decode fp32 L=4096 (every row), decode bf16 B=8 L=131072, decode bf16 B=64
  ragged 32K..512K, prefill chunk 4096 at L=131072, prefill chunk 8192 at
  L=1048576.

Sampled rows cover the first/last sequence and row, the longest and shortest
contexts, and a seeded random choice.  The same acceptance rules as the small
tests apply (bit-exact indexer scores, band-accepted sets, attention within
tolerance).  Each case prints its name before touching the GPU.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Dev, band_accept, check_out, out_f32, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

THREADS = min(os.cpu_count() or 1, 16)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_rows(w, d, rows, sets, out, k_low_cache):
    """rows: list of (t, r); checks selection bands and sparse outputs."""
    def job(tr):
        t, r = tr
        b, pos = w.row_seq(t), w.row_pos(t)
        h = w.ret_heads[r]
        g = w.kv_head(h)
        key = (b, r)
        if key not in k_low_cache:
            k_low_cache[key] = oracle.project(w.k[b][:, g, :], w.w_k[r])
        K = synth.as_f32(w.k[b][:, g, :])
        V = synth.as_f32(w.v[b][:, g, :])
        res = oracle.retrieval_row(w.q[t, h], K, V, w.w_q[r], w.w_k[r], pos, w.idx_scale,
                                   float(w.top_p[b]), w.attn_scale, k_low=k_low_cache[key])
        gset = sets[t * w.n_ret + r]
        ok, ex = band_accept(gset, res["order"], res["cum"], float(w.top_p[b]))
        ref = oracle.attend(w.q[t, h], K, V, gset, w.attn_scale)
        return tr, ok, ex, check_out(out[t, h], ref, w.dtype), len(gset)

    # fill the indexer keys needed, in parallel, before the row jobs
    need = sorted({(w.row_seq(t), r) for t, r in rows})
    def fill(br):
        b, r = br
        g = w.kv_head(w.ret_heads[r])
        return br, oracle.project(w.k[b][:, g, :], w.w_k[r])
    with cf.ThreadPoolExecutor(THREADS) as ex:
        for br, kl in ex.map(fill, [x for x in need if x not in k_low_cache]):
            k_low_cache[br] = kl
        results = list(ex.map(job, rows))
    for tr, ok, exact, err, n in results:
        assert ok, ("selection outside the band", tr, n)
        assert err <= 1.0, ("sparse attention", tr, err)
    return results


def _check_local(w, out, pairs):
    def job(th):
        t, h = th
        b, pos = w.row_seq(t), w.row_pos(t)
        g = w.kv_head(h)
        ref = oracle.local_row(w.q[t, h], synth.as_f32(w.k[b][: pos + 1, g, :]),
                               synth.as_f32(w.v[b][: pos + 1, g, :]), pos, w.window, w.sinks, w.attn_scale)
        return th, check_out(out[t, h], ref, w.dtype)
    with cf.ThreadPoolExecutor(THREADS) as ex:
        for th, err in ex.map(job, pairs):
            assert err <= 1.0, ("window attention", th, err)


def _check_dense(w, out, pairs):
    def job(th):
        t, h = th
        b, pos = w.row_seq(t), w.row_pos(t)
        g = w.kv_head(h)
        ref = oracle.dense_row(w.q[t, h], synth.as_f32(w.k[b][: pos + 1, g, :]),
                               synth.as_f32(w.v[b][: pos + 1, g, :]), pos, w.attn_scale)
        return th, check_out(out[t, h], ref, w.dtype)
    with cf.ThreadPoolExecutor(THREADS) as ex:
        for th, err in ex.map(job, pairs):
            assert err <= 1.0, ("dense attention", th, err)


def _decode_case(i, seqs):
    w = synth.config(i)
    say("[gpu-full] %s: B=%d max L=%d" % (w.name, w.B, int(w.seq_lens.max())))
    d = Dev(w, permute_seed=5)
    say("[gpu-full] %s: select" % w.name)
    st, rp, sets = d.select(capacity=int(sum(int(l) for l in w.seq_lens) * w.n_ret))
    assert st == 0
    say("[gpu-full] %s: sparse + window" % w.name)
    d.out.zero_()
    d.sparse()
    d.window()
    out = out_f32(d.out)
    rows = [(t, r) for t in seqs for r in range(w.n_ret)]
    res = _check_rows(w, d, rows, sets, out, {})
    loc = w.local_heads()
    g = np.random.default_rng(i)
    _check_local(w, out, [(t, int(h)) for t in seqs for h in g.choice(loc, 6, replace=False)])
    say("[gpu-full] %s: dense" % w.name)
    dense = torch.zeros_like(d.q)
    d.dense(dense)
    _check_dense(w, out_f32(dense), [(t, int(h)) for t in seqs for h in g.choice(w.Hq, 3, replace=False)])
    sizes = [n for *_, n in res]
    say("   budgets of checked rows: min %d median %d max %d" % (min(sizes), int(np.median(sizes)), max(sizes)))
    del d
    _free()


def test_full_decode_fp32_needles():
    w = synth.config(1)
    say("[gpu-full] %s" % w.name)
    d = Dev(w, permute_seed=5)
    st, rp, sets = d.select()
    assert st == 0
    d.sparse()
    d.window()
    out = out_f32(d.out)
    _check_rows(w, d, [(0, r) for r in range(w.n_ret)], sets, out, {})
    _check_local(w, out, [(0, h) for h in w.local_heads()])
    dense = torch.zeros_like(d.q)
    d.dense(dense)
    _check_dense(w, out_f32(dense), [(0, h) for h in range(w.Hq)])
    del d
    _free()


def test_full_decode_bf16_128k():
    _decode_case(2, [0, 3, 7])


def test_full_decode_bf16_ragged():
    lens = synth.ragged_lens(1005, 64, 32768, 524288)
    order = np.argsort(lens)
    _decode_case(5, sorted({int(order[0]), int(order[-1]), int(order[32]), 0}))


def _prefill_case(i, rows_t):
    w = synth.config(i)
    say("[gpu-full] %s: L=%d chunk %d" % (w.name, int(w.seq_lens[0]), w.n_tok))
    d = Dev(w, permute_seed=5)
    say("[gpu-full] %s: window + dense prefill" % w.name)
    d.out.zero_()
    d.window()
    out = out_f32(d.out)
    loc = w.local_heads()
    g = np.random.default_rng(i)
    _check_local(w, out, [(t, int(h)) for t in rows_t for h in g.choice(loc, 4, replace=False)])
    dense = torch.zeros_like(d.q)
    d.dense(dense)
    _check_dense(w, out_f32(dense), [(t, int(h)) for t in rows_t[:3] for h in g.choice(w.Hq, 2, replace=False)])
    return w, d, out


def test_full_prefill_128k():
    rows_t = [0, 1, 2047, 4095] + [int(x) for x in np.random.default_rng(3).choice(4096, 3, replace=False)]
    w, d, out = _prefill_case(3, rows_t)
    say("[gpu-full] %s: select + sparse prefill" % w.name)
    st, rp, sets = d.select(capacity=int(w.n_tok * w.n_ret * 8192))
    assert st == 0
    d.sparse()
    out = out_f32(d.out)
    _check_rows(w, d, [(t, r) for t in rows_t for r in range(w.n_ret)], sets, out, {})
    del d
    _free()


def test_full_prefill_1m():
    rows_t = [0, 1, 4095, 8191] + [int(x) for x in np.random.default_rng(4).choice(8192, 3, replace=False)]
    w, d, out = _prefill_case(4, rows_t)
    say("[gpu-full] %s: select + sparse prefill" % w.name)
    cap = int(w.n_tok * w.n_ret * 16384)
    st, rp, sets = d.select(capacity=cap)
    if st == 1:
        # the selection did not fit: rerun with the exact total it reported
        cap = int(rp[-1])
        say("   capacity %d" % cap)
        st, rp, sets = d.select(capacity=cap)
    assert st == 0
    d.sparse()
    out = out_f32(d.out)
    res = _check_rows(w, d, [(t, r) for t in rows_t for r in range(w.n_ret)], sets, out, {})
    sizes = [n for *_, n in res]
    say("   budgets of checked rows: min %d median %d max %d" % (min(sizes), int(np.median(sizes)), max(sizes)))
    del d
    _free()
