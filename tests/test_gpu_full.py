"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark uses, on sampled rows the oracle computes one by one:

  decode fp32 L=4096 (every row), decode bf16 B=8 L=131072, decode bf16 B=64
  ragged 32K..512K, prefill chunk 4096 at L=131072, prefill chunk 8192 at
  L=1048576; and decode bf16 B=21 L=131072, whose seed sends one row's
  candidate set past the keys the scoring pass flags (the from-scores route).

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
import sparse_attention_dim_amd as rtp
from gpu_util import Dev, band_accept, check_out, out_f32, path_counts, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

THREADS = min(os.cpu_count() or 1, 16)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_rows(w, d, rows, sets, out, k_low_cache, p_override=None):
    """rows: list of (t, r); checks selection bands and sparse outputs.  Rows
    are grouped by sequence; each sequence's K/V heads are widened to fp32
    once and dropped after its rows."""
    by_b = {}
    for t, r in rows:
        by_b.setdefault(w.row_seq(t), []).append((t, r))
    results = []
    for b, brow in sorted(by_b.items()):
        heads = sorted({w.kv_head(w.ret_heads[r]) for _, r in brow})
        kv = {g: (synth.as_f32(w.k[b][:, g, :]), synth.as_f32(w.v[b][:, g, :])) for g in heads}
        need = sorted({r for _, r in brow if (b, r) not in k_low_cache})

        def fill(r):
            g = w.kv_head(w.ret_heads[r])
            return r, oracle.project(w.k[b][:, g, :], w.w_k[r])

        def job(tr):
            t, r = tr
            pos = w.row_pos(t)
            h = w.ret_heads[r]
            K, V = kv[w.kv_head(h)]
            p = float(w.top_p[b]) if p_override is None else p_override
            res = oracle.retrieval_row(w.q[t, h], K, V, w.w_q[r], w.w_k[r], pos, w.idx_scale, p,
                                       w.attn_scale, k_low=k_low_cache[(b, r)])
            gset = sets[t * w.n_ret + r]
            ok, ex = band_accept(gset, res["order"], res["cum"], p)
            ref = oracle.attend(w.q[t, h], K, V, gset, w.attn_scale)
            err = check_out(out[t, h], ref, w.dtype) if out is not None else 0.0
            return tr, ok, ex, err, len(gset)

        with cf.ThreadPoolExecutor(THREADS) as ex:
            for r, kl in ex.map(fill, need):
                k_low_cache[(b, r)] = kl
            results += list(ex.map(job, brow))
        del kv
    for tr, ok, exact, err, n in results:
        assert ok, ("selection outside the band", tr, n)
        assert err <= 1.0, ("sparse attention", tr, err)
    return results


def _route_rows(paths, n_ret, per_route, rng):
    """Up to per_route rows of every route and emit order seen in paths."""
    picks = set()
    for code in range(1, 9):
        idx = np.flatnonzero((paths & 15) == code)
        picks.update(int(i) for i in rng.choice(idx, min(per_route, len(idx)), replace=False))
    for bit in (16, 32, 64, 128):
        idx = np.flatnonzero((paths & bit) != 0)
        picks.update(int(i) for i in rng.choice(idx, min(per_route, len(idx)), replace=False))
    return [(i // n_ret, i % n_ret) for i in sorted(picks)]


def _assert_routes(paths_checked, need):
    pc = path_counts(np.asarray(paths_checked, np.int32))
    say("   oracle-checked rows per route", pc)
    for name in need:
        assert pc[name] >= 16, ("route checked on fewer than 16 rows", name, pc[name])


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
    st, rp, sets, paths = d.select_mode(capacity=int(sum(int(l) for l in w.seq_lens) * w.n_ret))
    assert st == 0
    say("[gpu-full] %s: sparse + window" % w.name)
    d.out.zero_()
    d.sparse()
    d.window()
    out = out_f32(d.out)
    # every row of the step
    rows = [(t, r) for t in range(w.n_tok) for r in range(w.n_ret)]
    res = _check_rows(w, d, rows, sets, out, {})
    say("   paths of the rows", path_counts(paths))
    if i == 5:
        _assert_routes(paths, ["list", "list_g"])
    loc = w.local_heads()
    g = np.random.default_rng(i)
    _check_local(w, out, [(t, int(h)) for t in seqs for h in g.choice(loc, 6, replace=False)])
    say("[gpu-full] %s: dense" % w.name)
    dense = torch.zeros_like(d.q)
    d.dense(dense)
    _check_dense(w, out_f32(dense), [(t, int(h)) for t in seqs for h in g.choice(w.Hq, 3, replace=False)])
    sizes = [n for *_, n in res]
    say("   budgets of checked rows: min %d median %d max %d" % (min(sizes), int(np.median(sizes)), max(sizes)))
    # the step's attention in one call (rtp_decode_attn, as the benchmark runs
    # it): the same sets and bit-identical outputs as the oracle-checked calls
    say("[gpu-full] %s: rtp_decode_attn" % w.name)
    cap = int(sum(int(l) for l in w.seq_lens) * w.n_ret)
    row_ptr = torch.zeros(d.rows + 1, dtype=torch.int64, device="cuda")
    idx = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(row_ptr, idx, status)
    fout = torch.zeros_like(d.q)
    ws = torch.empty(rtp.decode_attn_workspace(d.layer, d.cache, d.query, cap), dtype=torch.uint8, device="cuda")
    for _ in range(2):                                  # twice: a call leaves no state behind
        rtp.decode_attn(d.layer, d.cache, d.query, d.w_q, d.top_p, sel, fout, ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        np.testing.assert_array_equal(row_ptr.cpu().numpy(), rp)
        n = int(rp[-1])
        np.testing.assert_array_equal(idx[:n].cpu().numpy(), d.idx[:n].cpu().numpy())
        assert torch.equal(fout, d.out), "rtp_decode_attn outputs differ from the separate calls"
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


def test_full_decode_bf16_128k_gqa_shared():
    # the shared gathers at the 128K decode shapes, with the grouped heads
    # sharing their planted cluster (overlapping sets): every row's set and
    # attention against the oracle, the CSR identical to the call without the
    # flag, the local heads bit-identical
    w = synth.cluster_decode(seed=1002, shared_kv=True, name="decode_bf16_B8_L131072_shared_clusters")
    say("[gpu-full] %s: B=%d L=%d, RTP_FLAG_GQA_SHARED" % (w.name, w.B, int(w.seq_lens.max())))
    d = Dev(w, permute_seed=5)
    cap = int(sum(int(l) for l in w.seq_lens) * w.n_ret)

    def call(flags):
        lay = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp.RTP_BF16, w.ret_heads, w.window, w.sinks, w.attn_scale,
                             w.idx_scale, flags=flags)
        row_ptr = torch.zeros(d.rows + 1, dtype=torch.int64, device="cuda")
        idx = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
        status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        sel = rtp.make_sel(row_ptr, idx, status)
        out = torch.zeros_like(d.q)
        ws = torch.empty(rtp.decode_attn_workspace(lay, d.cache, d.query, cap), dtype=torch.uint8, device="cuda")
        rtp.decode_attn(lay, d.cache, d.query, d.w_q, d.top_p, sel, out, ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        return row_ptr.cpu().numpy(), idx.cpu().numpy(), out

    rp, ix, out = call(rtp.RTP_FLAG_GQA_SHARED)
    rp0, ix0, out0 = call(0)
    np.testing.assert_array_equal(rp, rp0)
    np.testing.assert_array_equal(ix[: rp[-1]], ix0[: rp[-1]])
    loc = w.local_heads()
    assert torch.equal(out[:, loc], out0[:, loc])
    sets = [ix[rp[i]: rp[i + 1]] for i in range(d.rows)]
    rows = [(t, r) for t in range(w.n_tok) for r in range(w.n_ret)]
    _check_rows(w, d, rows, sets, out_f32(out), {})
    shared = 0
    for t in range(w.n_tok):
        for r in range(w.n_ret):
            for r2 in range(r + 1, w.n_ret):
                if w.kv_head(w.ret_heads[r]) == w.kv_head(w.ret_heads[r2]):
                    shared += len(np.intersect1d(sets[t * w.n_ret + r], sets[t * w.n_ret + r2]))
    say("   keys selected by two retrieval heads of one KV head:", shared, "of", int(rp[-1]))
    assert shared > 0
    del d
    _free()


def test_full_decode_bf16_128k_from_scores():
    # 21 sequences of 131072 keys (126 rows, the one-call step): with this
    # seed one row's candidate set reaches past the keys the scoring pass
    # flags in a chunk, so its row pass re-scores the chunks and gathers U
    # from the row's scores; that row and a sample of the others against the
    # oracle, the one-call step identical to the separate calls
    w = synth.cluster_decode(seed=3021, lens=(131072,) * 21, name="decode_bf16_B21_L131072")
    say("[gpu-full] %s: B=%d L=%d" % (w.name, w.B, int(w.seq_lens.max())))
    d = Dev(w, permute_seed=5)
    cap = int(sum(int(l) for l in w.seq_lens) * w.n_ret)
    say("[gpu-full] %s: select" % w.name)
    st, rp, sets, paths = d.select_mode(capacity=cap)
    assert st == 0
    pc = path_counts(paths)
    say("   paths of the rows", pc)
    fs = [int(i) for i in np.flatnonzero((paths & 256) != 0)]
    assert len(fs) >= 1
    say("[gpu-full] %s: sparse + window" % w.name)
    d.out.zero_()
    d.sparse()
    d.window()
    out = out_f32(d.out)
    g = np.random.default_rng(21)
    pick = set(fs) | {0, d.rows - 1} | {int(i) for i in g.choice(d.rows, 14, replace=False)}
    rows = [(i // w.n_ret, i % w.n_ret) for i in sorted(pick)]
    _check_rows(w, d, rows, sets, out, {})
    say("   oracle-checked rows: %d (from-scores rows %s)" % (len(rows), fs))
    say("[gpu-full] %s: rtp_decode_attn" % w.name)
    row_ptr = torch.zeros(d.rows + 1, dtype=torch.int64, device="cuda")
    idx = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(row_ptr, idx, status)
    fout = torch.zeros_like(d.q)
    ws = torch.empty(rtp.decode_attn_workspace(d.layer, d.cache, d.query, cap), dtype=torch.uint8, device="cuda")
    rtp.decode_attn(d.layer, d.cache, d.query, d.w_q, d.top_p, sel, fout, ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    np.testing.assert_array_equal(row_ptr.cpu().numpy(), rp)
    n = int(rp[-1])
    np.testing.assert_array_equal(idx[:n].cpu().numpy(), d.idx[:n].cpu().numpy())
    assert torch.equal(fout, d.out), "rtp_decode_attn outputs differ from the separate calls"
    del d
    _free()


def test_full_decode_bf16_ragged():
    lens = synth.ragged_lens(1005, 64, 32768, 524288)
    order = np.argsort(lens)
    _decode_case(5, sorted({int(order[0]), int(order[-1]), int(order[32]), 0}))


def test_full_decode_bf16_128k_topk():
    # fixed top-k at the decode workload's full size: bit-exact on every row
    w = synth.config(2)
    say("[gpu-full] %s: top-k 512" % w.name)
    d = Dev(w, permute_seed=5)
    st, rp, sets, paths = d.select_mode(top_k=512)
    assert st == 0
    for b in range(w.B):
        for r in range(w.n_ret):
            h = w.ret_heads[r]
            g = w.kv_head(h)
            q_low = oracle.project(w.q[b, h].reshape(1, -1), w.w_q[r])[0]
            dsc = oracle.scores(q_low, oracle.project(w.k[b][:, g, :], w.w_k[r]))
            np.testing.assert_array_equal(sets[b * w.n_ret + r], oracle.topk(dsc, 512))
    del d
    _free()


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
    cap = int(w.n_tok * w.n_ret * 8192)
    st, rp, sets, paths = d.select_mode(capacity=cap)
    assert st == 0
    d.sparse()
    out = out_f32(d.out)
    say("   paths of the rows", path_counts(paths))
    # every row of the chunk against the oracle
    k_low = {}
    rows = [(t, r) for t in range(w.n_tok) for r in range(w.n_ret)]
    res = _check_rows(w, d, rows, sets, out, k_low)
    say("   rows checked %d, bit-exact sets %d" % (len(res), sum(1 for x in res if x[2])))
    _assert_routes(paths, ["tiny", "row", "bitmap", "merge"])
    rng = np.random.default_rng(31)
    # a workspace at its minimum: every row takes the radix levels
    say("[gpu-full] %s: select, minimum workspace" % w.name)
    low = rtp.topp_select_workspace_min(d.layer, d.cache, d.query)
    st, rp, sets2, paths2 = d.select_mode(capacity=cap, ws_bytes=low)
    assert st == 0
    pick = _route_rows(paths2, w.n_ret, 48, rng)
    _check_rows(w, d, pick, sets2, None, k_low)
    _assert_routes([paths2[t * w.n_ret + r] for t, r in pick], ["level"])
    # the exact normaliser on every row that has keys outside its candidates
    say("[gpu-full] %s: select, exact normaliser" % w.name)
    st, rp, sets3, paths3 = d.select_mode(capacity=cap, flags=rtp.RTP_FLAG_EXACT_MASS)
    assert st == 0
    say("   paths", path_counts(paths3))
    pick = _route_rows(paths3, w.n_ret, 48, rng)
    _check_rows(w, d, pick, sets3, None, k_low)
    _assert_routes([paths3[t * w.n_ret + r] for t, r in pick], ["exact_z"])
    del d
    _free()


def test_full_prefill_1m():
    rows_t = [0, 1, 4095, 8191] + [int(x) for x in np.random.default_rng(4).choice(8192, 3, replace=False)]
    w, d, out = _prefill_case(4, rows_t)
    say("[gpu-full] %s: select + sparse prefill" % w.name)
    cap = int(w.n_tok * w.n_ret * 16384)
    st, rp, sets, paths = d.select_mode(capacity=cap)
    if st == 1:
        # the selection did not fit: rerun with the exact total it reported
        cap = int(rp[-1])
        say("   capacity %d" % cap)
        st, rp, sets, paths = d.select_mode(capacity=cap)
    assert st == 0
    d.sparse()
    out = out_f32(d.out)
    say("   paths of the rows", path_counts(paths))
    # >= 1024 rows: the 64 largest sets, 32 rows of every route seen, the
    # chunk's first and last rows, then a seeded sample
    rng = np.random.default_rng(4)
    sizes = np.diff(rp)
    pick = {(int(i) // w.n_ret, int(i) % w.n_ret) for i in np.argsort(sizes, kind="stable")[-64:]}
    pick |= set(_route_rows(paths, w.n_ret, 32, rng))
    pick |= {(t, r) for t in rows_t for r in range(w.n_ret)}
    rest = rng.permutation(d.rows)
    for i in rest:
        if len(pick) >= 1024:
            break
        pick.add((int(i) // w.n_ret, int(i) % w.n_ret))
    pick = sorted(pick)
    res = _check_rows(w, d, pick, sets, out, {})
    n = [x[4] for x in res]
    say("   rows checked %d; budgets min %d median %d max %d" % (len(res), min(n), int(np.median(n)), max(n)))
    _assert_routes([paths[t * w.n_ret + r] for t, r in pick], ["tiny", "row", "large", "bitmap", "merge"])
    del d
    _free()
