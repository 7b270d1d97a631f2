"""GPU parity of the chunked-prefill path (indexer append of the whole context,
top-p selection of every chunk row, sparse prefill attention, window prefill
attention, dense prefill attention) against the oracle, on the small prefill
workloads (several 4096-key chunks and 128-row query tiles with ragged tails,
permuted pages)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dim_amd as rtp
import synth
from gpu_util import Dev, band_accept, check_out, oracle_k_low, out_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=[3, 4], ids=["chunk_L5000", "chunk_L12000"])
def dev(request):
    w = synth.small(request.param)
    say("[gpu] prefill workload", w.name, "L", int(w.seq_lens[0]), "rows", w.n_tok, "ret", w.ret_heads)
    return Dev(w)


@pytest.fixture(scope="module")
def orc(dev):
    w = dev.w
    K = {g: synth.as_f32(w.k[0][:, g, :]) for g in range(w.Hkv)}
    V = {g: synth.as_f32(w.v[0][:, g, :]) for g in range(w.Hkv)}
    k_low = {r: oracle_k_low(w, 0, r) for r in range(w.n_ret)}
    res = {}
    for t in range(w.n_tok):
        pos = w.row_pos(t)
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            res[(t, r)] = oracle.retrieval_row(w.q[t, h], K[g], V[g], w.w_q[r], w.w_k[r], pos, w.idx_scale,
                                               float(w.top_p[0]), w.attn_scale, k_low=k_low[r])
    return dict(rows=res, K=K, V=V)


def test_indexer_keys_bit_exact(dev):
    w = dev.w
    for r in range(w.n_ret):
        np.testing.assert_array_equal(dev.pc.k_low_logical(0, r), oracle_k_low(w, 0, r))


def test_indexer_scores_bit_exact(dev, orc):
    w = dev.w
    say("[gpu] prefill indexer scores", w.name)
    q_low, sc = dev.scores()
    for (t, r), res in orc["rows"].items():
        row = t * w.n_ret + r
        np.testing.assert_array_equal(q_low[row], res["q_low"])
        L = w.row_pos(t) + 1
        np.testing.assert_array_equal(sc[row, :L].view(np.uint32), res["d"].view(np.uint32))


def test_selection_matches_oracle(dev, orc):
    w = dev.w
    say("[gpu] prefill top-p select", w.name)
    st, rp, sets = dev.select()
    assert st == 0
    exact = 0
    for (t, r), res in orc["rows"].items():
        ok, ex = band_accept(sets[t * w.n_ret + r], res["order"], res["cum"], float(w.top_p[0]))
        assert ok, (t, r, len(sets[t * w.n_ret + r]), len(res["sel"]))
        exact += ex
    assert exact >= len(orc["rows"]) - 2


def test_two_phase_select_equals_single_call(dev):
    say("[gpu] prefill two-phase select", dev.w.name)
    _, rp1, s1 = dev.select()
    _, rp2, s2 = dev.select(phased=True)
    np.testing.assert_array_equal(rp1, rp2)
    for a, b in zip(s1, s2):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("frac", [0.0, 0.01])
def test_selection_radix_level_path(dev, orc, frac):
    # a workspace below the recommended size: the rows whose candidate set does
    # not fit the smaller per-row buffer are resolved by radix levels on the
    # exact score and emitted by a rescan (frac 0: every row); same sets
    w = dev.w
    say("[gpu] prefill top-p select, reduced workspace", frac, w.name)
    full = rtp.topp_select_workspace(dev.layer, dev.cache, dev.query)
    low = rtp.topp_select_workspace_min(dev.layer, dev.cache, dev.query)
    st, rp, ref_sets = dev.select()
    assert st == 0
    st, rp, sets = dev.select(ws_bytes=low + int((full - low) * frac))
    assert st == 0
    for i in range(dev.rows):
        np.testing.assert_array_equal(sets[i], ref_sets[i])
    for (t, r), res in orc["rows"].items():
        ok, _ = band_accept(sets[t * w.n_ret + r], res["order"], res["cum"], float(w.top_p[0]))
        assert ok, (t, r)


@pytest.mark.parametrize("p", [0.3, 0.999])
def test_flat_scores_ties_cut_by_lowest_index(p):
    # zero key projection: all indexer scores of a row are 0, one tie group;
    # the set is the lowest indices reaching mass p (every row resolves its
    # cut inside the tie group)
    w = synth.small(3)
    w.w_k = np.zeros_like(w.w_k)
    w.top_p = np.full_like(w.top_p, p)
    say("[gpu] prefill flat scores", p)
    d = Dev(w)
    st, rp, sets = d.select()
    assert st == 0
    K = {g: synth.as_f32(w.k[0][:, g, :]) for g in range(w.Hkv)}
    V = {g: synth.as_f32(w.v[0][:, g, :]) for g in range(w.Hkv)}
    k_low = {r: oracle_k_low(w, 0, r) for r in range(w.n_ret)}
    for t in list(range(0, w.n_tok, 7)) + [w.n_tok - 1]:
        pos = w.row_pos(t)
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            res = oracle.retrieval_row(w.q[t, h], K[g], V[g], w.w_q[r], w.w_k[r], pos, w.idx_scale, p,
                                       w.attn_scale, k_low=k_low[r])
            got = sets[t * w.n_ret + r]
            ok, _ = band_accept(got, res["order"], res["cum"], p)
            assert ok, (t, r, len(got))
            np.testing.assert_array_equal(got, np.arange(len(got)))


def test_sparse_prefill_matches_oracle(dev, orc):
    w = dev.w
    say("[gpu] sparse prefill", w.name)
    st, rp, sets = dev.select()
    dev.out.zero_()
    dev.sparse()
    out = out_f32(dev.out)
    worst = 0.0
    for (t, r), res in orc["rows"].items():
        h = w.ret_heads[r]
        g = w.kv_head(h)
        ref = oracle.attend(w.q[t, h], orc["K"][g], orc["V"][g], sets[t * w.n_ret + r], w.attn_scale)
        e = check_out(out[t, h], ref, w.dtype)
        worst = max(worst, e)
        assert e <= 1.0, (t, r)
    say("   worst error / tolerance", round(worst, 4))


def test_window_prefill_matches_oracle(dev, orc):
    w = dev.w
    say("[gpu] window prefill", w.name)
    dev.out.zero_()
    dev.window()
    out = out_f32(dev.out)
    worst = 0.0
    for t in range(w.n_tok):
        pos = w.row_pos(t)
        for h in w.local_heads():
            g = w.kv_head(h)
            ref = oracle.local_row(w.q[t, h], orc["K"][g], orc["V"][g], pos, w.window, w.sinks, w.attn_scale)
            e = check_out(out[t, h], ref, w.dtype)
            worst = max(worst, e)
            assert e <= 1.0, (t, h)
    for h in w.ret_heads:
        assert np.all(out[:, h] == 0)
    say("   worst error / tolerance", round(worst, 4))


def test_dense_prefill_matches_oracle(dev, orc):
    w = dev.w
    say("[gpu] dense prefill", w.name)
    out_t = torch.zeros_like(dev.q)
    dev.dense(out_t)
    out = out_f32(out_t)
    worst = 0.0
    for t in list(range(0, w.n_tok, 7)) + [w.n_tok - 1]:
        pos = w.row_pos(t)
        for h in range(w.Hq):
            g = w.kv_head(h)
            ref = oracle.dense_row(w.q[t, h], orc["K"][g], orc["V"][g], pos, w.attn_scale)
            e = check_out(out[t, h], ref, w.dtype)
            worst = max(worst, e)
            assert e <= 1.0, (t, h)
    say("   worst error / tolerance", round(worst, 4))


def test_prefill_last_row_equals_decode(dev):
    # the chunk's last row sees exactly the keys of a decode query at the same
    # position: both paths must give the same selection and outputs
    w = dev.w
    say("[gpu] prefill last row vs decode", w.name)
    st, rp, sets = dev.select()
    dev.out.zero_()
    dev.sparse()
    dev.window()
    pre = out_f32(dev.out)[w.n_tok - 1]
    q_dec = dev.q[w.n_tok - 1:].contiguous()
    qd = rtp.make_query(q_dec, rtp.RTP_DECODE)
    rows = w.n_ret
    row_ptr = torch.zeros(rows + 1, dtype=torch.int64, device="cuda")
    idx = torch.empty(rows * int(w.seq_lens[0]), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(row_ptr, idx, status)
    ws = torch.empty(rtp.topp_select_workspace(dev.layer, dev.cache, qd), dtype=torch.uint8, device="cuda")
    rtp.topp_select(dev.layer, dev.cache, qd, dev.w_q, dev.top_p, sel, ws)
    out_d = torch.zeros_like(q_dec)
    ws2 = torch.empty(rtp.sparse_attn_workspace(dev.layer, dev.cache, qd, idx.numel()), dtype=torch.uint8,
                      device="cuda")
    rtp.sparse_attn_decode(dev.layer, dev.cache, qd, sel, out_d, ws2)
    ws3 = torch.empty(rtp.window_attn_workspace(dev.layer, dev.cache, qd), dtype=torch.uint8, device="cuda")
    rtp.window_attn(dev.layer, dev.cache, qd, out_d, ws3)
    torch.cuda.synchronize()
    rpd = row_ptr.cpu().numpy()
    idd = idx[: int(rpd[-1])].cpu().numpy()
    for r in range(rows):
        np.testing.assert_array_equal(idd[rpd[r]: rpd[r + 1]], sets[(w.n_tok - 1) * w.n_ret + r])
    dec = out_f32(out_d)[0]
    for h in range(w.Hq):
        ref = pre[h].astype(np.float64)
        assert np.max(np.abs(dec[h] - ref)) <= 1e-2 * np.linalg.norm(ref), h
