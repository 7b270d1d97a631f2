"""GPU parity of rtp_decode_attn (the attention of a decode step in one call:
selection and sparse attention of the retrieval heads, window attention of
the local heads) against rtp_topp_select, rtp_sparse_attn_decode and
rtp_window_attn, and against the oracle: same status, row pointers, selected
indices and outputs of every head, on every selection route (every key,
candidate sets cut in LDS or from the workspace list, gathered from the key
flags or the scores, and the cut over the row's scores)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_attention_dim_amd as rtp
from gpu_util import Dev, band_accept, check_out, oracle_k_low, out_f32, path_counts, say

pytestmark = pytest.mark.gpu


def _fused(d: Dev, capacity=None, top_p=None, w_k=None):
    w = d.w
    if capacity is None:
        capacity = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.n_ret
    row_ptr = torch.zeros(d.rows + 1, dtype=torch.int64, device="cuda")
    idx = torch.full((max(capacity, 1),), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(row_ptr, idx, status)
    out = torch.zeros_like(d.q)
    ws = torch.empty(rtp.decode_attn_workspace(d.layer, d.cache, d.query, sel.capacity), dtype=torch.uint8,
                     device="cuda")
    tp = d.top_p if top_p is None else torch.as_tensor(np.asarray(top_p, np.float32)).cuda()
    rtp.decode_attn(d.layer, d.cache, d.query, d.w_q, tp, sel, out, ws, w_k=w_k)
    torch.cuda.synchronize()
    return int(status.item()), row_ptr.cpu().numpy(), idx.cpu().numpy(), out


def _two_calls(d: Dev, capacity=None):
    d.out.zero_()
    st, rp, sets = d.select(capacity=capacity)
    if st == 0:
        d.sparse()
    d.window()
    return st, rp, d.idx.cpu().numpy(), d.out.clone()


def _same(d: Dev, a, b):
    st1, rp1, ix1, o1 = a
    st2, rp2, ix2, o2 = b
    assert st1 == st2
    np.testing.assert_array_equal(rp1, rp2)
    n = int(rp1[-1]) if st1 == 0 else 0
    np.testing.assert_array_equal(ix1[:n], ix2[:n])
    if st1 == 0:
        assert torch.equal(o1, o2), "outputs differ"
    else:
        loc = d.w.local_heads()
        assert torch.equal(o1[:, loc], o2[:, loc]), "local-head outputs differ"


@pytest.fixture(scope="module", params=[1, 2, 5], ids=["needle_f32", "cluster_bf16", "ragged_bf16"])
def dev(request):
    w = synth.small(request.param)
    say("[gpu] decode step attention", w.name, "lens", list(w.seq_lens))
    return Dev(w)


def test_fused_equals_two_calls_and_oracle(dev):
    w = dev.w
    a = _fused(dev)
    b = _two_calls(dev)
    _same(dev, a, b)
    st, rp, ix, out = a
    assert st == 0
    o = out_f32(out)
    for t in range(w.n_tok):
        bq, pos = w.row_seq(t), w.row_pos(t)
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            res = oracle.retrieval_row(w.q[t, h], w.k[bq][:, g, :], w.v[bq][:, g, :], w.w_q[r], w.w_k[r], pos,
                                       w.idx_scale, float(w.top_p[bq]), w.attn_scale)
            row = t * w.n_ret + r
            got = ix[rp[row]: rp[row + 1]]
            ok, _ = band_accept(got, res["order"], res["cum"], float(w.top_p[bq]))
            assert ok, (t, r)
            ref = oracle.attend(w.q[t, h], w.k[bq][:, g, :], w.v[bq][:, g, :], got, w.attn_scale)
            assert check_out(o[t, h], ref, w.dtype) <= 1.0, (t, r)
        for h in w.local_heads():
            g = w.kv_head(h)
            ref = oracle.local_row(w.q[t, h], w.k[bq][:, g, :], w.v[bq][:, g, :], pos, w.window, w.sinks,
                                   w.attn_scale)
            assert check_out(o[t, h], ref, w.dtype) <= 1.0, ("local", t, h)


def test_fused_indexer_key_append(dev):
    # the step's own indexer keys (each sequence's last position) overwritten
    # with garbage, then written by the call itself (w_k given): bit-exact keys
    # and the same selection and outputs as with the keys appended beforehand
    w = dev.w
    a = _fused(dev)
    pc = dev.pc
    saved = []
    for b in range(w.B):
        j = int(pc.lens[b]) - 1
        page = int(pc.table[b, j // 256])
        saved.append(pc.k_low[page, :, j % 256, :].clone())
        pc.k_low[page, :, j % 256, :] = 7.0
    torch.cuda.synchronize()
    b_ = _fused(dev, w_k=dev.w_k)
    _same(dev, a, b_)
    for b in range(w.B):
        j = int(pc.lens[b]) - 1
        page = int(pc.table[b, j // 256])
        assert torch.equal(pc.k_low[page, :, j % 256, :], saved[b]), b
        for r in range(w.n_ret):
            want = oracle_k_low(w, b, r)[j]
            got = pc.k_low[page, r, j % 256, :].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            np.testing.assert_array_equal(got, want, err_msg=str((b, r)))


def test_lds_route_taken(dev):
    # the planted workloads' candidate sets are small: most rows are cut in LDS
    st, rp, sets, paths = dev.select_mode()
    assert st == 0
    pc = path_counts(paths)
    say("   paths", pc, "of", dev.rows)
    assert pc["list"] >= dev.rows // 2


def _flat(lens, p, seed=77):
    w = synth.cluster_decode(seed=seed, lens=lens, Hq=8, Hkv=2, D=128, n_ret=2, p=p, window=256, sinks=8,
                             rope=1e4, size_dist=("loguniform", 4, 64), name="flat")
    w.w_k = np.zeros_like(w.w_k)
    return w


def test_fused_long_rows_every_route():
    # flat scores (one tie group per row): rows of 40000 keys take the cut
    # over the scores (selected indices written over the scores), 20000 and
    # 9001 keys the workspace list, 5000 keys the list gathered from the
    # scores into LDS; p = 1 rows keep every key
    w = _flat((40000, 20000, 9001, 5000, 3000), 0.999)
    w.top_p[4] = 1.0
    say("[gpu] decode step attention, flat long rows")
    d = Dev(w)
    a = _fused(d)
    b = _two_calls(d)
    _same(d, a, b)
    st, rp, ix, out = a
    assert st == 0
    _, _, _, paths = d.select_mode()
    pc = path_counts(paths)
    say("   paths", pc)
    assert pc["scan"] == 2 and pc["list_g"] == 4 and pc["list"] == 2 and pc["all"] == 2
    for t in range(w.n_tok):
        L = w.row_pos(t) + 1
        n = L if w.top_p[t] >= 1 else int(np.ceil(np.float64(np.float32(0.999)) * L))
        for r in range(w.n_ret):
            row = t * w.n_ret + r
            np.testing.assert_array_equal(ix[rp[row]: rp[row + 1]], np.arange(n), err_msg=str((t, r)))
    o = out_f32(out)
    for t in range(w.n_tok):
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            row = t * w.n_ret + r
            ref = oracle.attend(w.q[t, h], w.k[t][:, g, :], w.v[t][:, g, :], ix[rp[row]: rp[row + 1]],
                                w.attn_scale)
            assert check_out(o[t, h], ref, w.dtype) <= 1.0, (t, r)


def test_fused_spread_rows_gather_from_scores():
    # indexer keys scaled x4 spread the scores: the top-p sets reach more than
    # 4 units below their chunk maxima, past the keys the scoring pass flags,
    # so U is gathered from the rows' scores
    w = synth.small(2)
    w.w_k = synth.to_storage(synth.as_f32(w.w_k) * np.float32(4.0), w.dtype)     # exact: a power of two
    w.top_p = np.full_like(w.top_p, 0.99)
    say("[gpu] decode step attention, spread scores")
    d = Dev(w)
    a = _fused(d)
    b = _two_calls(d)
    _same(d, a, b)
    st, rp, ix, out = a
    assert st == 0
    _, _, _, paths = d.select_mode()
    pc = path_counts(paths)
    say("   paths", pc)
    assert pc["from_scores"] >= 1
    o = out_f32(out)
    for t in range(w.n_tok):
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            res = oracle.retrieval_row(w.q[t, h], w.k[t][:, g, :], w.v[t][:, g, :], w.w_q[r], w.w_k[r],
                                       w.row_pos(t), w.idx_scale, float(w.top_p[t]), w.attn_scale)
            row = t * w.n_ret + r
            got = ix[rp[row]: rp[row + 1]]
            ok, _ = band_accept(got, res["order"], res["cum"], float(w.top_p[t]))
            assert ok, (t, r)
            ref = oracle.attend(w.q[t, h], w.k[t][:, g, :], w.v[t][:, g, :], got, w.attn_scale)
            assert check_out(o[t, h], ref, w.dtype) <= 1.0, (t, r)


def test_fused_capacity_overflow():
    w = synth.small(2)
    say("[gpu] decode step attention, capacity overflow")
    d = Dev(w)
    st, rp, ix, out = _fused(d)
    need = int(rp[-1])
    st2, rp2, ix2, out2 = _fused(d, capacity=need - 1)
    assert st2 == 1 and int(rp2[-1]) == need
    np.testing.assert_array_equal(rp2, rp)
    assert np.all(ix2 == -1)
    ret = list(w.ret_heads)
    assert not torch.any(out2[:, ret] != 0), "no retrieval-head output on overflow"
    loc = w.local_heads()
    assert torch.equal(out2[:, loc], out[:, loc]), "local heads are written regardless"
    st3, rp3, ix3, out3 = _fused(d, capacity=need)
    assert st3 == 0
    assert torch.equal(out3, out)


def test_fused_invalid_top_p():
    w = synth.small(2)
    say("[gpu] decode step attention, invalid top_p")
    d = Dev(w)
    p = w.top_p.astype(np.float32).copy()
    p[0] = float("nan")
    st, rp, ix, out = _fused(d, top_p=p)
    assert st == 3
    assert np.all(ix == -1)
    assert not torch.any(out[:, list(w.ret_heads)] != 0)


def test_fused_repeated_calls_identical():
    # every call rewrites the row records: calls with other top_p values in
    # between leave the result unchanged
    w = synth.small(5)
    say("[gpu] decode step attention, repeated calls")
    d = Dev(w)
    a = _fused(d)
    _fused(d, top_p=np.full_like(w.top_p, 0.5))
    b = _fused(d)
    _same(d, a, b)
