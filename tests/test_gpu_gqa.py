"""GPU parity of rtp_decode_attn with RTP_FLAG_GQA_SHARED (the retrieval heads
of one KV head gather the union of their selected keys once): the same
status, row pointers and selected indices as without the flag, local-head
outputs bit-identical, retrieval-head outputs against the oracle over the
selected sets; on workloads whose grouped heads share their planted cluster
(overlapping sets) and on independent clusters (disjoint sets), with groups
of 1, 2 and 3 retrieval heads, a union too large to merge in LDS, capacity
overflow and repeated calls."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_dim_amd as rtp
from gpu_util import Dev, check_out, out_f32, say

pytestmark = pytest.mark.gpu

RET = [4, 5, 6, 12, 13, 20]          # KV heads 1 (3 heads), 3 (2 heads), 5 (1 head) at Hq = 32, Hkv = 8


def _work(shared, lens=(6000, 9001, 4097), size_dist=("loguniform", 4, 256), p=0.9, seed=31, dtype="bf16"):
    return synth.cluster_decode(seed=seed, lens=lens, Hq=32, Hkv=8, D=128, n_ret=len(RET), p=p, window=300,
                                sinks=8, rope=1e4, dtype=dtype, size_dist=size_dist, ret_heads=RET,
                                name="gqa_shared" if shared else "gqa_disjoint", shared_kv=shared)


def _call(d: Dev, flags, capacity=None):
    w = d.w
    layer = rtp.make_layer(w.Hq, w.Hkv, w.D, d.layer.dtype, w.ret_heads, w.window, w.sinks, w.attn_scale,
                           w.idx_scale, flags=flags)
    if capacity is None:
        capacity = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.n_ret
    row_ptr = torch.zeros(d.rows + 1, dtype=torch.int64, device="cuda")
    idx = torch.full((max(capacity, 1),), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(row_ptr, idx, status)
    out = torch.zeros_like(d.q)
    ws = torch.empty(rtp.decode_attn_workspace(layer, d.cache, d.query, sel.capacity), dtype=torch.uint8,
                     device="cuda")
    rtp.decode_attn(layer, d.cache, d.query, d.w_q, d.top_p, sel, out, ws)
    torch.cuda.synchronize()
    return int(status.item()), row_ptr.cpu().numpy(), idx.cpu().numpy(), out


def _check(d: Dev, shared_expected):
    w = d.w
    a = _call(d, 0)
    b = _call(d, rtp.RTP_FLAG_GQA_SHARED)
    st, rp, ix, out = b
    assert st == a[0] == 0
    np.testing.assert_array_equal(rp, a[1])
    n = int(rp[-1])
    np.testing.assert_array_equal(ix[:n], a[2][:n])
    loc = w.local_heads()
    assert torch.equal(out[:, loc], a[3][:, loc]), "local-head outputs differ"
    o = out_f32(out)
    overlap = 0
    for t in range(w.n_tok):
        bq = w.row_seq(t)
        sets = {r: ix[rp[t * w.n_ret + r]: rp[t * w.n_ret + r + 1]] for r in range(w.n_ret)}
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            ref = oracle.attend(w.q[t, h], w.k[bq][:, g, :], w.v[bq][:, g, :], sets[r], w.attn_scale)
            assert check_out(o[t, h], ref, w.dtype) <= 1.0, (t, r)
        for r in range(w.n_ret):
            for r2 in range(r + 1, w.n_ret):
                if w.kv_head(w.ret_heads[r]) == w.kv_head(w.ret_heads[r2]):
                    overlap += len(np.intersect1d(sets[r], sets[r2]))
    say("   keys selected by two heads of one KV head:", overlap)
    if shared_expected:
        assert overlap > 0, "the shared-cluster workload should give overlapping sets"


@pytest.mark.parametrize("shared", [True, False], ids=["shared_clusters", "independent_clusters"])
def test_gqa_shared_gathers(shared):
    w = _work(shared)
    say("[gpu] gqa shared gathers", w.name, "lens", list(w.seq_lens))
    _check(Dev(w), shared)


def test_gqa_shared_fp32():
    w = _work(True, dtype="f32")
    say("[gpu] gqa shared gathers fp32", w.name)
    _check(Dev(w), True)


def test_gqa_shared_large_union_concatenated():
    # sets of thousands of keys per head: a group's lists exceed the LDS merge
    # and are gathered one after another (same results)
    w = _work(True, lens=(20000, 16385), size_dist=("loguniform", 3000, 6000), p=0.999, seed=33)
    say("[gpu] gqa shared gathers, large unions", w.name)
    _check(Dev(w), True)


def test_gqa_shared_capacity_overflow_and_repeat():
    w = _work(True)
    d = Dev(w)
    ok = _call(d, rtp.RTP_FLAG_GQA_SHARED)
    need = int(ok[1][-1])
    st, rp, _, out = _call(d, rtp.RTP_FLAG_GQA_SHARED, capacity=need - 1)
    assert st == 1
    np.testing.assert_array_equal(rp, ok[1])      # the row pointers give the size needed
    loc = w.local_heads()
    assert torch.equal(out[:, loc], ok[3][:, loc])
    again = _call(d, rtp.RTP_FLAG_GQA_SHARED)
    assert again[0] == 0
    np.testing.assert_array_equal(again[1], ok[1])
    assert torch.equal(again[3], ok[3]), "a repeated call differs"
