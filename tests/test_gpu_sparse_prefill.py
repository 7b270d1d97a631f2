"""GPU parity of the sparse prefill attention (rtp_sparse_attn_prefill) on
hand-built selected sets, against the oracle's attention over the same sets.

The sets are chosen to reach every branch of the union-tile kernels: a
context of three 2^16-key windows (the last one partial), a 64-row tile whose
rows share a union of more than two 1024-key groups inside one window, a tile
of disjoint per-row sets spread over every window, empty rows, a ragged last
tile, a CSR whose capacity ends exactly at the last entry (so the last pieces
are read element by element), and an idx pointer that is not 16-byte
aligned.  Inputs are seeded draws of the synthetic generator."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_dim_amd as rtp
import synth
from gpu_util import check_out, say
from sparse_attention_dim_amd.paged import PagedCache, to_device

pytestmark = pytest.mark.gpu

L, N_TOK, HQ, HKV, D = 140000, 150, 8, 2, 128
RET = [1, 6]
SEED = 4242


def _sets():
    pos0 = L - N_TOK
    sets = {}
    for r in range(len(RET)):
        g = synth.rng(SEED, 100 + r)
        shared = np.sort(g.choice(65536, 2600, replace=False)) if r == 0 else \
            np.sort(131072 + g.choice(L - N_TOK - 131072, 5000, replace=False))
        for t in range(N_TOK):
            pos = pos0 + t
            if t < 64:                                       # one large shared union plus a few own keys
                own = g.choice(pos + 1, 20, replace=False)
                s = np.union1d(shared, own)
            elif t < 128:                                    # disjoint sets over every window; some empty
                s = np.array([], np.int64) if t % 7 == 0 else g.choice(pos + 1, 60, replace=False)
            else:                                            # ragged tail: sinks and the keys just before
                s = np.concatenate([np.arange(4), np.arange(pos - 299, pos + 1)])
            sets[(t, r)] = np.unique(s).astype(np.int32)
    return sets


@pytest.fixture(scope="module")
def case():
    K = synth.normal_rope(SEED, 1, 0, 0, L, HKV, D, 0.0, 0, "bf16")
    V = synth.normal_rope(SEED, 2, 0, 0, L, HKV, D, 0.0, 0, "bf16")
    Q = synth.normal_rope(SEED, 3, 0, 0, N_TOK, HQ, D, 0.0, 0, "bf16")
    pc = PagedCache([K], [V], len(RET), "bf16", permute_seed=5, spare_blocks=2)
    layer = rtp.make_layer(HQ, HKV, D, rtp.RTP_BF16, RET, 64, 4, 1.0 / np.sqrt(D), 0.25)
    q = to_device(Q)
    query = rtp.make_query(q, rtp.RTP_CHUNK, 0, L - N_TOK)
    sets = _sets()
    rows = N_TOK * len(RET)
    sizes = np.array([len(sets[(t, r)]) for t in range(N_TOK) for r in range(len(RET))], np.int64)
    rp = np.zeros(rows + 1, np.int64)
    rp[1:] = np.cumsum(sizes)
    flat = np.concatenate([sets[(t, r)] for t in range(N_TOK) for r in range(len(RET))]).astype(np.int32)
    say("[gpu] sparse prefill sets: rows", rows, "entries", int(rp[-1]), "max", int(sizes.max()))
    return dict(K=K, V=V, Q=Q, pc=pc, cache=pc.cache(L), layer=layer, q=q, query=query, sets=sets,
                rp=torch.from_numpy(rp).cuda(), flat=flat)


def _run(case, idx_t):
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(case["rp"], idx_t, status)
    ws = torch.empty(rtp.sparse_attn_workspace(case["layer"], case["cache"], case["query"], idx_t.numel()),
                     dtype=torch.uint8, device="cuda")
    out = torch.full_like(case["q"], 7.0)
    for _ in range(2):                                       # the second call reuses the workspace
        rtp.sparse_attn_prefill(case["layer"], case["cache"], case["query"], sel, out, ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _check(case, out):
    worst = 0.0
    Kf = {g: synth.as_f32(case["K"][:, g, :]) for g in range(HKV)}
    Vf = {g: synth.as_f32(case["V"][:, g, :]) for g in range(HKV)}
    for (t, r), s in case["sets"].items():
        h = RET[r]
        if len(s) == 0:
            assert np.all(out[t, h] == 0.0), (t, r)
            continue
        ref = oracle.attend(case["Q"][t, h], Kf[h // (HQ // HKV)], Vf[h // (HQ // HKV)], s, 1.0 / np.sqrt(D))
        e = check_out(out[t, h], ref, "bf16")
        worst = max(worst, e)
        assert e <= 1.0, (t, r, e)
    local = [h for h in range(HQ) if h not in RET]
    assert np.all(out[:, local, :] == 7.0)                   # local heads are not written
    say("   worst error / tolerance", round(worst, 4))


def test_sparse_prefill_sets_exact_capacity(case):
    say("[gpu] sparse prefill, capacity = entries")
    idx_t = torch.from_numpy(case["flat"]).cuda()
    _check(case, _run(case, idx_t))


def test_sparse_prefill_sets_unaligned_idx(case):
    say("[gpu] sparse prefill, idx at a 4-byte offset")
    n = len(case["flat"])
    buf = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    buf[1:] = torch.from_numpy(case["flat"]).cuda()
    _check(case, _run(case, buf[1:]))
