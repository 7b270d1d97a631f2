"""The allocation-free selection (rtp_topp_select_noalloc) against the
workspace entry point (rtp_topp_select) through the C ABI: two calls in a
row on the library's static scratch array, the second on a smaller input,
each bit-identical (row pointers, indices, status) to rtp_topp_select given
a workspace of the same size on the same inputs."""
import numpy as np
import pytest
import torch

import sparse_attention_dim_amd as rtp
import synth
from gpu_util import Dev, say

pytestmark = pytest.mark.gpu


def _run(dev, noalloc: bool):
    w = dev.w
    cap = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.n_ret
    row_ptr = torch.full((dev.rows + 1,), -5, dtype=torch.int64, device="cuda")
    idx = torch.full((cap,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sel = rtp.make_sel(row_ptr, idx, status)
    if noalloc:
        rtp.topp_select_noalloc(dev.layer, dev.cache, dev.query, dev.w_q, dev.top_p, sel)
    else:
        # the workspace size the allocation-free call uses
        full = rtp.topp_select_workspace(dev.layer, dev.cache, dev.query)
        ws = torch.empty(min(full, rtp.RTP_NOALLOC_SCRATCH_BYTES), dtype=torch.uint8, device="cuda")
        rtp.topp_select(dev.layer, dev.cache, dev.query, dev.w_q, dev.top_p, sel, ws)
    torch.cuda.synchronize()
    rp = row_ptr.cpu().numpy()
    n = int(rp[-1]) if int(status.item()) == 0 else 0
    return int(status.item()), rp, idx[:n].cpu().numpy()


def test_noalloc_select_equals_workspace_select():
    # first call: a bf16 prefill chunk (4200 rows over 12000 keys); second, a
    # smaller decode step (18 rows) on the same, now stale, scratch
    for i in (4, 2):
        w = synth.small(i)
        say("[gpu] allocation-free select:", w.name, "rows", w.n_tok * w.n_ret)
        dev = Dev(w)
        st_a, rp_a, ix_a = _run(dev, noalloc=True)
        st_b, rp_b, ix_b = _run(dev, noalloc=False)
        assert st_a == 0 and st_b == 0
        np.testing.assert_array_equal(rp_a, rp_b)
        np.testing.assert_array_equal(ix_a, ix_b)
