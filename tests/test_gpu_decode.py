"""GPU parity of the decode path (indexer append, top-p select, sparse decode,
window decode, dense decode) against the oracle, on the small decode workloads
(several 4096-key chunks, ragged tails, permuted pages) and edge cases."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import Dev, band_accept, check_out, oracle_k_low, out_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=[1, 2, 5], ids=["needle_f32", "cluster_bf16", "ragged_bf16"])
def dev(request):
    w = synth.small(request.param)
    say("[gpu] decode workload", w.name, "lens", list(w.seq_lens), "ret", w.ret_heads)
    return Dev(w)


def _oracle_rows(w):
    res = {}
    for t in range(w.n_tok):
        b, pos = w.row_seq(t), w.row_pos(t)
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            res[(t, r)] = oracle.retrieval_row(w.q[t, h], w.k[b][:, g, :], w.v[b][:, g, :], w.w_q[r],
                                               w.w_k[r], pos, w.idx_scale, float(w.top_p[b]),
                                               w.attn_scale)
    return res


@pytest.fixture(scope="module")
def orc(dev):
    return _oracle_rows(dev.w)


def test_indexer_keys_bit_exact(dev):
    w = dev.w
    for b in range(w.B):
        for r in range(w.n_ret):
            np.testing.assert_array_equal(dev.pc.k_low_logical(b, r), oracle_k_low(w, b, r))


def test_indexer_queries_and_scores_bit_exact(dev, orc):
    w = dev.w
    say("[gpu] indexer scores", w.name)
    q_low, sc = dev.scores()
    for (t, r), res in orc.items():
        row = t * w.n_ret + r
        np.testing.assert_array_equal(q_low[row], res["q_low"])
        L = w.row_pos(t) + 1
        np.testing.assert_array_equal(sc[row, :L].view(np.uint32), res["d"].view(np.uint32))


def test_selection_matches_oracle(dev, orc):
    w = dev.w
    say("[gpu] top-p select", w.name)
    st, rp, sets = dev.select()
    assert st == 0
    exact = 0
    for (t, r), res in orc.items():
        row = t * w.n_ret + r
        ok, ex = band_accept(sets[row], res["order"], res["cum"], float(w.top_p[w.row_seq(t)]))
        assert ok, (t, r, len(sets[row]), len(res["sel"]))
        exact += ex
    assert exact >= len(orc) - 1


def test_sparse_decode_matches_oracle(dev, orc):
    w = dev.w
    say("[gpu] sparse decode", w.name)
    st, rp, sets = dev.select()
    dev.out.zero_()
    dev.sparse()
    out = out_f32(dev.out)
    for (t, r), res in orc.items():
        b, h = w.row_seq(t), w.ret_heads[r]
        g = w.kv_head(h)
        ref = oracle.attend(w.q[t, h], w.k[b][:, g, :], w.v[b][:, g, :], sets[t * w.n_ret + r],
                            w.attn_scale)
        assert check_out(out[t, h], ref, w.dtype) <= 1.0, (t, r)


def test_window_decode_matches_oracle(dev):
    w = dev.w
    say("[gpu] window decode", w.name)
    dev.out.zero_()
    dev.window()
    out = out_f32(dev.out)
    for t in range(w.n_tok):
        b, pos = w.row_seq(t), w.row_pos(t)
        for h in w.local_heads():
            g = w.kv_head(h)
            ref = oracle.local_row(w.q[t, h], w.k[b][:, g, :], w.v[b][:, g, :], pos, w.window, w.sinks,
                                   w.attn_scale)
            assert check_out(out[t, h], ref, w.dtype) <= 1.0, (t, h)
    for h in w.ret_heads:                 # retrieval-head slices untouched
        assert np.all(out[:, h] == 0)


def test_dense_decode_matches_oracle(dev):
    w = dev.w
    say("[gpu] dense decode", w.name)
    out_t = torch.zeros_like(dev.q)
    dev.dense(out_t)
    out = out_f32(out_t)
    for t in range(w.n_tok):
        b, pos = w.row_seq(t), w.row_pos(t)
        for h in range(0, w.Hq, max(1, w.Hq // 8)):
            g = w.kv_head(h)
            ref = oracle.dense_row(w.q[t, h], w.k[b][:, g, :], w.v[b][:, g, :], pos, w.attn_scale)
            assert check_out(out[t, h], ref, w.dtype) <= 1.0, (t, h)


def test_deterministic(dev):
    w = dev.w
    say("[gpu] determinism", w.name)
    _, rp1, s1 = dev.select()
    dev.sparse()
    o1 = dev.out.clone()
    _, rp2, s2 = dev.select()
    dev.sparse()
    np.testing.assert_array_equal(rp1, rp2)
    for a, b in zip(s1, s2):
        np.testing.assert_array_equal(a, b)
    assert torch.equal(o1, dev.out)


def test_two_phase_select_equals_single_call(dev):
    """topp_select_begin / _end with window attention on a second stream in
    between: the same row pointers and sets as one topp_select call."""
    say("[gpu] two-phase select", dev.w.name)
    _, rp1, s1 = dev.select()
    _, rp2, s2 = dev.select(phased=True)
    np.testing.assert_array_equal(rp1, rp2)
    for a, b in zip(s1, s2):
        np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _custom(lens, p=0.9, window=4, sinks=2, dtype="bf16", flat=False, seed=5, Hq=8, Hkv=4, D=64,
            ret=(1, 6)):
    w = synth.cluster_decode(seed=seed, lens=lens, Hq=Hq, Hkv=Hkv, D=D, n_ret=len(ret), p=p,
                             window=window, sinks=sinks, rope=1e4, dtype=dtype,
                             size_dist=("loguniform", 1, 4), ret_heads=list(ret), name="edge")
    if flat:   # zero key projection: every indexer score is 0, one tie group per row
        w.w_k = np.zeros_like(w.w_k)
    return w


@pytest.mark.parametrize("lens,p,flat", [
    ((1, 2, 3), 0.9, False),                 # single-key rows; window and sinks clip
    ((255, 256, 257), 0.9, False),           # page boundaries
    ((4095, 4096, 4097), 0.5, False),        # chunk boundaries
    ((700, 1300), 1.0, False),               # p = 1 keeps every key
    ((600, 9000), 0.3, True),                # all scores equal: ties cut by lowest index
    ((20000,), 0.999, True),                 # a tie group larger than the sort buffer
])
def test_edge_cases(lens, p, flat):
    w = _custom(lens, p=p, flat=flat)
    say("[gpu] edge decode", lens, p, "flat" if flat else "")
    d = Dev(w)
    st, rp, sets = d.select()
    assert st == 0
    orc = _oracle_rows(w)
    for (t, r), res in orc.items():
        ok, _ = band_accept(sets[t * w.n_ret + r], res["order"], res["cum"], p)
        assert ok, (t, r)
        if flat and p < 1:
            k = len(sets[t * w.n_ret + r])
            assert list(sets[t * w.n_ret + r]) == list(range(k))
    d.sparse()
    d.window()
    out = out_f32(d.out)
    for (t, r), res in orc.items():
        b, h = t, w.ret_heads[r]
        g = w.kv_head(h)
        ref = oracle.attend(w.q[t, h], w.k[b][:, g, :], w.v[b][:, g, :], sets[t * w.n_ret + r], w.attn_scale)
        assert check_out(out[t, h], ref, w.dtype) <= 1.0
    for t in range(w.n_tok):
        for h in w.local_heads():
            g = w.kv_head(h)
            ref = oracle.local_row(w.q[t, h], w.k[t][:, g, :], w.v[t][:, g, :], w.row_pos(t), w.window,
                                   w.sinks, w.attn_scale)
            assert check_out(out[t, h], ref, w.dtype) <= 1.0


@pytest.mark.parametrize("lens,window,sinks", [
    ((1, 2, 31, 32, 33), 100, 3),            # fewer keys than one 32-key block; block edges
    ((127, 128, 129, 300), 100, 3),          # one split of window + sinks, ragged last block
    ((1000, 700), 300, 8),                   # several 128-key splits, sink run then window run
])
def test_bf16_d128_window_and_dense_decode(lens, window, sinks):
    # the bf16 D = 128 local-head and dense decode run on MFMA (GQA 4:1, some
    # query heads of a group are retrieval heads and stay unwritten)
    w = _custom(lens, dtype="bf16", Hq=32, Hkv=8, D=128, ret=(0, 5, 9, 14, 22, 31), window=window, sinks=sinks)
    say("[gpu] bf16 D=128 window/dense decode", lens, window, sinks)
    d = Dev(w)
    d.window()
    out = out_f32(d.out)
    dense = torch.zeros_like(d.q)
    d.dense(dense)
    den = out_f32(dense)
    for t in range(w.n_tok):
        for h in range(w.Hq):
            g = w.kv_head(h)
            K, V = synth.as_f32(w.k[t][:, g, :]), synth.as_f32(w.v[t][:, g, :])
            ref_d = oracle.dense_row(w.q[t, h], K, V, w.row_pos(t), w.attn_scale)
            assert check_out(den[t, h], ref_d, w.dtype) <= 1.0, ("dense", t, h)
            if h in w.ret_heads:
                continue
            ref_w = oracle.local_row(w.q[t, h], K, V, w.row_pos(t), w.window, w.sinks, w.attn_scale)
            assert check_out(out[t, h], ref_w, w.dtype) <= 1.0, ("window", t, h)


def test_capacity_overflow_reports_needed_size():
    w = _custom((3000, 5000), p=0.99)
    say("[gpu] capacity overflow")
    d = Dev(w)
    st, rp, _ = d.select()
    need = int(rp[-1])
    st2, rp2, _ = d.select(capacity=need - 1)
    assert st2 == 1 and int(rp2[-1]) == need
    assert torch.all(d.idx == -1)
    st3, rp3, sets = d.select(capacity=need)
    assert st3 == 0 and int(rp3[-1]) == need


def test_fp32_long_window_equals_dense():
    w = _custom((500, 900), dtype="f32", window=5000, sinks=0)
    say("[gpu] window >= context equals dense")
    d = Dev(w)
    d.window()
    dense = torch.zeros_like(d.q)
    d.dense(dense)
    loc = w.local_heads()
    np.testing.assert_allclose(out_f32(d.out)[:, loc], out_f32(dense)[:, loc], rtol=0, atol=1e-6)
