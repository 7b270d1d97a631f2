"""GPU parity of the FP8 K/V variant (K and V stored as FP8 E4M3 codes with one
scale each; queries, projections and outputs in bf16) against the oracle on
the dequantised K/V, through the C ABI:

  * indexer keys from FP8 K: bit-exact (the oracle dequantises, then runs the
    same projection chain);
  * rtp_kv_append with FP8 input writes the same pages and indexer keys as the
    page fill plus rtp_indexer_append, also into a window-only ring;
  * top-p selection (band rule), sparse decode, window decode and dense
    decode within the bf16 tolerance; the sparse attention of a prefill chunk;
  * chunked window attention with FP8 K/V is reported as unsupported.

Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dim_amd as rtp
import synth
from gpu_util import band_accept, check_out, out_f32, say
from sparse_attention_dim_amd.paged import PagedCache, RingCache, to_device

pytestmark = pytest.mark.gpu


class Fp8Dev:
    """A workload with FP8 K/V pages on the GPU (indexer pages filled)."""

    def __init__(self, w, fill=True):
        self.w = w
        self.kc, self.vc, self.ks, self.vs = synth.fp8_kv(w)
        # the oracle's view of the stored K/V
        self.kf = [oracle.fp8_dequant(c, self.ks) for c in self.kc]
        self.vf = [oracle.fp8_dequant(c, self.vs) for c in self.vc]
        self.pc = PagedCache(self.kc, self.vc, w.n_ret, "fp8", permute_seed=17, spare_blocks=2)
        self.layer = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp.RTP_BF16, w.ret_heads, w.window, w.sinks, w.attn_scale,
                                    w.idx_scale, kv_fp8=1, k_scale=self.ks, v_scale=self.vs)
        self.q = to_device(w.q)
        self.w_q, self.w_k = to_device(w.w_q), to_device(w.w_k)
        self.top_p = torch.from_numpy(w.top_p.astype(np.float32)).cuda()
        self.cache = self.pc.cache(max(self.pc.lens))
        kind = rtp.RTP_DECODE if w.kind == "decode" else rtp.RTP_CHUNK
        self.query = rtp.make_query(self.q, kind, w.chunk_seq, w.chunk_pos0)
        if fill:
            for b in range(w.B):
                sid, pos = self.pc.all_positions(b)
                rtp.indexer_append(self.layer, self.cache, self.w_k, sid, pos)
            torch.cuda.synchronize()

    @property
    def rows(self):
        return self.w.n_tok * self.w.n_ret

    def k_low_ref(self, b, r):
        g = self.w.kv_head(self.w.ret_heads[r])
        return oracle.project(self.kf[b][:, g, :], self.w.w_k[r])

    def select_sparse(self):
        w = self.w
        cap = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.n_ret
        rp = torch.zeros(self.rows + 1, dtype=torch.int64, device="cuda")
        idx = torch.zeros(cap, dtype=torch.int32, device="cuda")
        st = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        sel = rtp.make_sel(rp, idx, st)
        ws = torch.empty(rtp.topp_select_workspace(self.layer, self.cache, self.query), dtype=torch.uint8,
                         device="cuda")
        rtp.topp_select(self.layer, self.cache, self.query, self.w_q, self.top_p, sel, ws)
        out = torch.zeros_like(self.q)
        wsp = torch.empty(rtp.sparse_attn_workspace(self.layer, self.cache, self.query, cap), dtype=torch.uint8,
                          device="cuda")
        if w.kind == "decode":
            rtp.sparse_attn_decode(self.layer, self.cache, self.query, sel, out, wsp)
        else:
            rtp.sparse_attn_prefill(self.layer, self.cache, self.query, sel, out, wsp)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        rpn = rp.cpu().numpy()
        ix = idx[: int(rpn[-1])].cpu().numpy()
        return [ix[rpn[i]: rpn[i + 1]] for i in range(self.rows)], out


@pytest.fixture(scope="module", params=[2, 5], ids=["decode_bf16", "decode_ragged"])
def dev(request):
    w = synth.small(request.param)
    say("[gpu] FP8 K/V workload", w.name)
    return Fp8Dev(w)


def test_fp8_indexer_keys_bit_exact(dev):
    w = dev.w
    for b in range(w.B):
        for r in range(w.n_ret):
            np.testing.assert_array_equal(dev.pc.k_low_logical(b, r), dev.k_low_ref(b, r), err_msg=str((b, r)))


def test_fp8_decode_retrieval_and_local_heads(dev):
    w = dev.w
    say("[gpu] FP8 decode select + sparse + window", w.name)
    sets, out = dev.select_sparse()
    ws = torch.empty(rtp.window_attn_workspace(dev.layer, dev.cache, dev.query), dtype=torch.uint8, device="cuda")
    rtp.window_attn(dev.layer, dev.cache, dev.query, out, ws)
    torch.cuda.synchronize()
    o = out_f32(out)
    worst = 0.0
    for t in range(w.n_tok):
        b, pos = w.row_seq(t), w.row_pos(t)
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            res = oracle.retrieval_row(w.q[t, h], dev.kf[b][:, g, :], dev.vf[b][:, g, :], w.w_q[r], w.w_k[r], pos,
                                       w.idx_scale, float(w.top_p[b]), w.attn_scale, k_low=dev.k_low_ref(b, r))
            ok, _ = band_accept(sets[t * w.n_ret + r], res["order"], res["cum"], float(w.top_p[b]))
            assert ok, (t, r)
            ref = oracle.attend(w.q[t, h], dev.kf[b][:, g, :], dev.vf[b][:, g, :], sets[t * w.n_ret + r],
                                w.attn_scale)
            e = check_out(o[t, h], ref, "bf16")
            worst = max(worst, e)
            assert e <= 1.0, ("sparse", t, r, e)
        for h in w.local_heads():
            g = w.kv_head(h)
            ref = oracle.local_row(w.q[t, h], dev.kf[b][:, g, :], dev.vf[b][:, g, :], pos, w.window, w.sinks,
                                   w.attn_scale)
            e = check_out(o[t, h], ref, "bf16")
            worst = max(worst, e)
            assert e <= 1.0, ("window", t, h, e)
    say("   worst error / tolerance", round(worst, 4))


def test_fp8_dense_decode(dev):
    w = dev.w
    say("[gpu] FP8 dense decode", w.name)
    out = torch.zeros_like(dev.q)
    ws = torch.empty(rtp.dense_attn_workspace(dev.layer, dev.cache, dev.query), dtype=torch.uint8, device="cuda")
    rtp.dense_attn(dev.layer, dev.cache, dev.query, out, ws)
    torch.cuda.synchronize()
    o = out_f32(out)
    for t in range(w.n_tok):
        b, pos = w.row_seq(t), w.row_pos(t)
        for h in range(0, w.Hq, 5):
            g = w.kv_head(h)
            ref = oracle.dense_row(w.q[t, h], dev.kf[b][:, g, :], dev.vf[b][:, g, :], pos, w.attn_scale)
            assert check_out(o[t, h], ref, "bf16") <= 1.0, (t, h)


def test_fp8_kv_append_flat_and_ring(dev):
    w = dev.w
    say("[gpu] FP8 kv append", w.name)
    k2, v2, kl2 = torch.zeros_like(dev.pc.k), torch.zeros_like(dev.pc.v), torch.zeros_like(dev.pc.k_low)
    cache2 = rtp.make_cache(k2, v2, kl2, dev.pc.block_table, dev.pc.seq_lens, max(dev.pc.lens))
    for b in range(w.B):
        L = dev.pc.lens[b]
        for j0 in range(0, L, 1500):
            j1 = min(L, j0 + 1500)
            sid = torch.full((j1 - j0,), b, dtype=torch.int32, device="cuda")
            pos = torch.arange(j0, j1, dtype=torch.int32, device="cuda")
            rtp.kv_append(dev.layer, cache2, to_device(dev.kc[b][j0:j1]), to_device(dev.vc[b][j0:j1]), dev.w_k,
                          sid, pos)
    torch.cuda.synchronize()
    assert torch.equal(k2, dev.pc.k) and torch.equal(v2, dev.pc.v)
    assert torch.equal(kl2.view(torch.int16), dev.pc.k_low.view(torch.int16))
    # a window-only ring holding the FP8 codes of the all-local KV heads
    rc = RingCache(w.Hkv, w.D, w.Hq // w.Hkv, w.ret_heads, w.n_ret, [int(x) for x in w.seq_lens], "fp8", 4,
                   permute_seed=3)
    rc.fill(dev.layer, dev.kc, dev.vc, dev.w_k)
    ring = rc.cache()
    o_ring, o_flat = torch.zeros_like(dev.q), torch.zeros_like(dev.q)
    ws = torch.empty(rtp.window_attn_workspace(dev.layer, ring, dev.query), dtype=torch.uint8, device="cuda")
    rtp.window_attn(dev.layer, ring, dev.query, o_ring, ws)
    rtp.window_attn(dev.layer, dev.cache, dev.query, o_flat, ws)
    torch.cuda.synchronize()
    assert torch.equal(o_ring.view(torch.int16), o_flat.view(torch.int16))
    say("   K/V bytes: bf16 pages %d, FP8 pages %d, FP8 ring layout %d" %
        (2 * dev.pc.k.numel() * 2, 2 * dev.pc.k.numel(), rc.nbytes()))


def test_fp8_prefill_chunk_sparse():
    w = synth.small(3)
    say("[gpu] FP8 prefill chunk", w.name)
    dev = Fp8Dev(w)
    sets, out = dev.select_sparse()
    o = out_f32(out)
    for t in range(0, w.n_tok, 3):
        pos = w.row_pos(t)
        for r, h in enumerate(w.ret_heads):
            g = w.kv_head(h)
            res = oracle.retrieval_row(w.q[t, h], dev.kf[0][:, g, :], dev.vf[0][:, g, :], w.w_q[r], w.w_k[r], pos,
                                       w.idx_scale, float(w.top_p[0]), w.attn_scale, k_low=dev.k_low_ref(0, r))
            ok, _ = band_accept(sets[t * w.n_ret + r], res["order"], res["cum"], float(w.top_p[0]))
            assert ok, (t, r)
            ref = oracle.attend(w.q[t, h], dev.kf[0][:, g, :], dev.vf[0][:, g, :], sets[t * w.n_ret + r],
                                w.attn_scale)
            assert check_out(o[t, h], ref, "bf16") <= 1.0, (t, r)
    with pytest.raises(rtp.RtpError) as e:
        rtp.window_attn(dev.layer, dev.cache, dev.query, out, None)
    assert e.value.code == rtp.RTP_EUNSUPPORTED
