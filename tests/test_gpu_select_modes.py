"""GPU parity of the selection rules beside plain top-p, on the small decode and
prefill workloads, through the C ABI:

  * fixed top-k (rtp_topk_select): the first min(k, L) keys of the exact rank
    order, bit-exact against the oracle's top-k;
  * the top-p budget cap (layer k_max): the first min(k, k_max) keys for a k
    the 1e-6 mass band accepts;
  * the exact-normaliser route of the bf16 chunk path (RTP_FLAG_EXACT_MASS):
    every row that has keys outside its candidate set is cut with the
    normaliser summed exactly over every key, and is band-accepted;
  * a NaN or non-positive top_p reported as status 3;
  * a candidate set above 8192 keys (the large-row resolve), forced by flat
    scores at p = 0.999.

Every case prints its name before touching the GPU.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dim_amd as rtp
import synth
from gpu_util import Dev, band_accept, band_accept_cap, oracle_k_low, path_counts, say

pytestmark = pytest.mark.gpu

THREADS = min(os.cpu_count() or 1, 16)


def _oracle_rows(w):
    """Per (t, r): the oracle's exact scores, rank order and cumulative masses."""
    k_low = {}
    for b in range(w.B):
        for r in range(w.n_ret):
            k_low[(b, r)] = oracle_k_low(w, b, r)

    def job(tr):
        t, r = tr
        b, pos = w.row_seq(t), w.row_pos(t)
        h = w.ret_heads[r]
        g = w.kv_head(h)
        res = oracle.retrieval_row(w.q[t, h], w.k[b][:, g, :], w.v[b][:, g, :], w.w_q[r], w.w_k[r], pos,
                                   w.idx_scale, float(w.top_p[b]), w.attn_scale, k_low=k_low[(b, r)])
        return tr, dict(d=res["d"], order=res["order"], cum=res["cum"])

    with cf.ThreadPoolExecutor(THREADS) as ex:
        return dict(ex.map(job, [(t, r) for t in range(w.n_tok) for r in range(w.n_ret)]))


WORKLOADS = {"decode_f32": 1, "decode_bf16": 2, "decode_ragged": 5, "chunk_L5000": 3, "chunk_L12000": 4}


@pytest.fixture(scope="module", params=list(WORKLOADS), ids=list(WORKLOADS))
def case(request):
    w = synth.small(WORKLOADS[request.param])
    say("[gpu] select modes: workload", w.name)
    return Dev(w), _oracle_rows(w)


@pytest.mark.parametrize("k", [1, 17, 300, 5000])
def test_topk_bit_exact(case, k):
    dev, orc = case
    w = dev.w
    say("[gpu] top-k", k, w.name)
    st, rp, sets, paths = dev.select_mode(top_k=k)
    assert st == 0
    for (t, r), o in orc.items():
        want = oracle.topk(o["d"], k)
        np.testing.assert_array_equal(sets[t * w.n_ret + r], want, err_msg=str((t, r, k)))
    pc = path_counts(paths)
    # every row that is not kept whole was cut by count
    assert pc["count"] == dev.rows - pc["all"]
    say("   paths", pc)


@pytest.mark.parametrize("k_max", [1, 12, 150])
def test_topp_budget_cap(case, k_max):
    dev, orc = case
    w = dev.w
    say("[gpu] top-p capped at", k_max, w.name)
    st, rp, sets, paths = dev.select_mode(k_max=k_max)
    assert st == 0
    capped = 0
    for (t, r), o in orc.items():
        got = sets[t * w.n_ret + r]
        p = float(w.top_p[w.row_seq(t)])
        assert band_accept_cap(got, o["order"], o["cum"], p, k_max), (t, r, len(got))
        capped += len(got) == k_max
    assert np.max(np.diff(rp)) <= k_max
    say("   rows at the cap", capped, "of", dev.rows, "paths", path_counts(paths))


def test_keep_all_rows_capped():
    # p = 1 keeps every key; with the cap a row keeps its first k_max keys
    w = synth.small(2)
    w.top_p = np.ones_like(w.top_p)
    say("[gpu] p = 1 capped", w.name)
    dev = Dev(w)
    orc = _oracle_rows(w)
    st, rp, sets, _ = dev.select_mode(k_max=40)
    assert st == 0
    for (t, r), o in orc.items():
        np.testing.assert_array_equal(sets[t * w.n_ret + r], np.sort(o["order"][:40]))


@pytest.mark.parametrize("wl", ["chunk_L5000", "chunk_L12000"])
def test_exact_normaliser_route(wl):
    w = synth.small(WORKLOADS[wl])
    say("[gpu] exact-normaliser route", w.name)
    dev = Dev(w)
    orc = _oracle_rows(w)
    st, rp, ref, _ = dev.select_mode()
    assert st == 0
    st, rp, sets, paths = dev.select_mode(flags=rtp.RTP_FLAG_EXACT_MASS)
    assert st == 0
    pc = path_counts(paths)
    say("   paths", pc)
    assert pc["exact_z"] > 0
    same = 0
    for (t, r), o in orc.items():
        got = sets[t * w.n_ret + r]
        ok, _ = band_accept(got, o["order"], o["cum"], float(w.top_p[0]))
        assert ok, (t, r)
        same += np.array_equal(got, ref[t * w.n_ret + r])
    assert same >= dev.rows - 2
    # with a reduced workspace the rows without a buffer take the radix levels
    # and the exact normaliser too
    low = rtp.topp_select_workspace_min(dev.layer, dev.cache, dev.query)
    st, rp, sets, paths = dev.select_mode(flags=rtp.RTP_FLAG_EXACT_MASS, ws_bytes=low)
    assert st == 0
    pc = path_counts(paths)
    say("   reduced workspace paths", pc)
    assert pc["level"] > 0 and pc["exact_z"] > 0
    for (t, r), o in orc.items():
        ok, _ = band_accept(sets[t * w.n_ret + r], o["order"], o["cum"], float(w.top_p[0]))
        assert ok, (t, r)


@pytest.mark.parametrize("wl,bad", [("decode_bf16", float("nan")), ("decode_bf16", 0.0),
                                    ("chunk_L5000", -0.5), ("chunk_L5000", float("nan"))])
def test_invalid_top_p_is_reported(wl, bad):
    w = synth.small(WORKLOADS[wl])
    say("[gpu] invalid top_p", bad, w.name)
    dev = Dev(w)
    p = w.top_p.astype(np.float32).copy()
    p[-1] = bad
    st, rp, sets, _ = dev.select_mode(top_p=p)
    assert st == 3
    # fixed top-k does not read top_p
    st, rp, sets, _ = dev.select_mode(top_k=5, top_p=p)
    assert st == 0


def test_large_candidate_set_resolve():
    # flat scores (zero key projection) and p = 0.999: every key of a row is a
    # candidate, so rows past position ~8192 of the 12000-key chunk hold more
    # than 8192 and take the large-row resolve; the set is the lowest indices
    w = synth.small(4)
    w.w_k = np.zeros_like(w.w_k)
    w.top_p = np.full_like(w.top_p, 0.999)
    say("[gpu] large candidate sets", w.name)
    dev = Dev(w)
    st, rp, sets, paths = dev.select_mode()
    assert st == 0
    pc = path_counts(paths)
    say("   paths", pc)
    assert pc["large"] >= 16
    L = {t: w.row_pos(t) + 1 for t in range(w.n_tok)}
    for t in range(w.n_tok):
        for r in range(w.n_ret):
            got = sets[t * w.n_ret + r]
            n = int(np.ceil(np.float64(np.float32(0.999)) * L[t]))
            np.testing.assert_array_equal(got, np.arange(n), err_msg=str((t, r)))
    # the oracle on a sample of the large rows
    big = [i for i in range(dev.rows) if (paths[i] & 15) == rtp.PATH_LARGE]
    orc_rows = [(i // w.n_ret, i % w.n_ret) for i in big[:: max(1, len(big) // 24)]]
    for t, r in orc_rows:
        h = w.ret_heads[r]
        g = w.kv_head(h)
        res = oracle.retrieval_row(w.q[t, h], w.k[0][:, g, :], w.v[0][:, g, :], w.w_q[r], w.w_k[r],
                                   w.row_pos(t), w.idx_scale, 0.999, w.attn_scale)
        ok, _ = band_accept(sets[t * w.n_ret + r], res["order"], res["cum"], 0.999)
        assert ok, (t, r)


def test_decode_long_candidate_sets():
    # flat scores and p = 0.999 on decode rows of 40000, 20000 and 9001 keys:
    # every key is a candidate, so the rows take the list cut from the
    # workspace (8192 < U <= 32768) or the cut over the scores (U > 32768);
    # the set is the lowest indices
    w = synth.cluster_decode(seed=77, lens=(40000, 20000, 9001), Hq=8, Hkv=2, D=128, n_ret=2, p=0.999,
                             window=256, sinks=8, rope=1e4, size_dist=("loguniform", 4, 64), name="flat_long")
    w.w_k = np.zeros_like(w.w_k)
    say("[gpu] decode long candidate sets")
    dev = Dev(w)
    st, rp, sets, paths = dev.select_mode()
    assert st == 0
    pc = path_counts(paths)
    say("   paths", pc)
    assert pc["scan"] == 2 and pc["list_g"] == 4
    for t in range(w.n_tok):
        L = w.row_pos(t) + 1
        n = int(np.ceil(np.float64(np.float32(0.999)) * L))
        for r in range(w.n_ret):
            np.testing.assert_array_equal(sets[t * w.n_ret + r], np.arange(n), err_msg=str((t, r)))
    # the same rows under the cap and top-k (count cuts on both long routes)
    st, rp, sets, paths = dev.select_mode(k_max=15000)
    assert st == 0
    for t in range(w.n_tok):
        L = w.row_pos(t) + 1
        n = min(15000, int(np.ceil(np.float64(np.float32(0.999)) * L)))
        for r in range(w.n_ret):
            np.testing.assert_array_equal(sets[t * w.n_ret + r], np.arange(n), err_msg=str(("cap", t, r)))
    st, rp, sets, paths = dev.select_mode(top_k=12345)
    for t in range(w.n_tok):
        L = w.row_pos(t) + 1
        for r in range(w.n_ret):
            np.testing.assert_array_equal(sets[t * w.n_ret + r], np.arange(min(12345, L)))
