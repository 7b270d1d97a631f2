"""Helpers of the GPU parity tests: upload a synthetic workload into librtp's
paged layout, run the hot-path entry points, and compare with the oracle.

Acceptance rules (the tests' bar):
  * indexer keys, indexer queries and indexer scores: bit-exact;
  * selected sets: equal to the oracle's rank prefix {sigma(1..k)} for a k
    with C_k >= p - 1e-6 and C_{k-1} < p + 1e-6 (bit-exact outside the band);
  * attention outputs, per (query, head) row, against the oracle recomputed
    over the GPU's accepted set: fp32 max|diff| <= 1e-5 * max|ref|, bf16
    max|diff| <= 1e-2 * ||ref||_2.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_attention_dim_amd as rtp
import synth
from sparse_attention_dim_amd.paged import PagedCache, bf16_bits, rtp_dtype, to_device

BAND = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Dev:
    """A synthetic workload resident on the GPU with its indexer pages filled."""

    def __init__(self, w: synth.Workload, permute_seed=11, fill=True):
        self.w = w
        self.pc = PagedCache(w.k, w.v, w.n_ret, w.dtype, permute_seed=permute_seed, spare_blocks=3)
        self.layer = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp_dtype(w.dtype), w.ret_heads, w.window,
                                    w.sinks, w.attn_scale, w.idx_scale)
        self.q = to_device(w.q)
        self.w_q = to_device(w.w_q)
        self.w_k = to_device(w.w_k)
        self.top_p = torch.from_numpy(w.top_p.astype(np.float32)).cuda()
        max_len = max(self.pc.lens)
        self.cache = self.pc.cache(max_len)
        kind = rtp.RTP_DECODE if w.kind == "decode" else rtp.RTP_CHUNK
        self.query = rtp.make_query(self.q, kind, w.chunk_seq, w.chunk_pos0)
        self.out = torch.zeros_like(self.q)
        if fill:
            for b in range(w.B):
                sid, pos = self.pc.all_positions(b)
                rtp.indexer_append(self.layer, self.cache, self.w_k, sid, pos)
            torch.cuda.synchronize()

    @property
    def rows(self) -> int:
        return self.w.n_tok * self.w.n_ret

    def select(self, capacity: int | None = None, ws_bytes: int | None = None, phased: bool = False):
        w = self.w
        if capacity is None:
            capacity = sum(min(w.row_pos(t) + 1, 1 << 30) for t in range(w.n_tok)) * w.n_ret
        self.row_ptr = torch.zeros(self.rows + 1, dtype=torch.int64, device="cuda")
        self.idx = torch.full((max(capacity, 1),), -1, dtype=torch.int32, device="cuda")
        self.status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        self.sel = rtp.make_sel(self.row_ptr, self.idx, self.status)
        if ws_bytes is None:
            ws_bytes = rtp.topp_select_workspace(self.layer, self.cache, self.query)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        if phased:
            # the two phases, with the local heads' window attention on a second
            # stream between them (started once the first phase is done)
            args = (self.layer, self.cache, self.query, self.w_q, self.top_p, self.sel, ws)
            main = torch.cuda.current_stream()
            side = torch.cuda.Stream()
            wsw = torch.empty(rtp.window_attn_workspace(self.layer, self.cache, self.query), dtype=torch.uint8,
                              device="cuda")
            # prepared calls (arguments marshalled once), as a serving loop would
            begin = rtp.topp_select_begin(*args, stream=main, prepare=True)
            end = rtp.topp_select_end(*args, stream=main, prepare=True)
            window = rtp.window_attn(self.layer, self.cache, self.query, self.out, wsw, stream=side, prepare=True)
            fork, join = torch.cuda.Event(), torch.cuda.Event()
            begin()
            fork.record(main)
            side.wait_event(fork)
            window()
            end()
            join.record(side)
            main.wait_event(join)
        else:
            rtp.topp_select(self.layer, self.cache, self.query, self.w_q, self.top_p, self.sel, ws)
        torch.cuda.synchronize()
        del ws
        return self.sets()

    def select_mode(self, top_k: int = 0, k_max: int = 0, flags: int = 0, capacity: int | None = None,
                    ws_bytes: int | None = None, top_p=None):
        """Selection with another rule: fixed top-k (top_k > 0), the top-p
        budget cap (k_max), layer flags, or other top_p values.  Returns
        (status, row_ptr, sets or None, path codes)."""
        w = self.w
        layer = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp_dtype(w.dtype), w.ret_heads, w.window, w.sinks,
                               w.attn_scale, w.idx_scale, k_max=k_max, flags=flags)
        if capacity is None:
            capacity = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.n_ret
        self.row_ptr = torch.zeros(self.rows + 1, dtype=torch.int64, device="cuda")
        self.idx = torch.full((max(capacity, 1),), -1, dtype=torch.int32, device="cuda")
        self.status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        self.sel = rtp.make_sel(self.row_ptr, self.idx, self.status)
        if ws_bytes is None:
            ws_bytes = rtp.topp_select_workspace(layer, self.cache, self.query)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        tp = self.top_p if top_p is None else torch.as_tensor(np.asarray(top_p, np.float32)).cuda()
        if top_k > 0:
            rtp.topk_select(layer, self.cache, self.query, self.w_q, top_k, self.sel, ws)
        else:
            rtp.topp_select(layer, self.cache, self.query, self.w_q, tp, self.sel, ws)
        paths = torch.full((self.rows,), -1, dtype=torch.int32, device="cuda")
        rtp.topp_select_paths(layer, self.cache, self.query, ws, paths)
        torch.cuda.synchronize()
        del ws
        st, rp, sets = self.sets()
        return st, rp, sets, paths.cpu().numpy()

    def sets(self):
        rp = self.row_ptr.cpu().numpy()
        st = int(self.status.cpu().item())
        if st != 0:
            return st, rp, None
        idx = self.idx[: int(rp[-1])].cpu().numpy()
        return st, rp, [idx[rp[i]: rp[i + 1]] for i in range(self.rows)]

    def sparse(self):
        ws_bytes = rtp.sparse_attn_workspace(self.layer, self.cache, self.query, self.sel.capacity)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        if self.w.kind == "decode":
            rtp.sparse_attn_decode(self.layer, self.cache, self.query, self.sel, self.out, ws)
        else:
            rtp.sparse_attn_prefill(self.layer, self.cache, self.query, self.sel, self.out, ws)
        torch.cuda.synchronize()

    def window(self):
        ws = torch.empty(rtp.window_attn_workspace(self.layer, self.cache, self.query), dtype=torch.uint8,
                         device="cuda")
        rtp.window_attn(self.layer, self.cache, self.query, self.out, ws)
        torch.cuda.synchronize()

    def dense(self, out):
        ws = torch.empty(rtp.dense_attn_workspace(self.layer, self.cache, self.query), dtype=torch.uint8,
                         device="cuda")
        rtp.dense_attn(self.layer, self.cache, self.query, out, ws)
        torch.cuda.synchronize()

    def scores(self):
        w = self.w
        L = max(w.row_pos(t) + 1 for t in range(w.n_tok))
        q_low = torch.zeros((self.rows, 16), dtype=torch.int16, device="cuda")
        sc = torch.full((self.rows, L), float("nan"), dtype=torch.float32, device="cuda")
        rtp.indexer_scores(self.layer, self.cache, self.query, self.w_q, q_low, sc)
        torch.cuda.synchronize()
        return q_low.cpu().numpy().view(np.uint16), sc.cpu().numpy()


def out_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def band_accept(gpu: np.ndarray, order: np.ndarray, cum: np.ndarray, p: float, band: float = BAND):
    """(accepted, exact) for a GPU set against the oracle's rank order and C_k."""
    n = len(order)
    k = len(gpu)
    if np.float32(p) >= 1.0:
        ok = k == n and np.array_equal(gpu, np.arange(n))
        return ok, ok
    if k < 1 or k > n:
        return False, False
    if not np.array_equal(np.sort(order[:k]), gpu):
        return False, False
    ck = cum[k - 1]
    ck1 = cum[k - 2] if k >= 2 else 0.0
    pp = float(np.float32(p))
    ok = ck >= pp - band and ck1 < pp + band
    exact = ck >= pp and ck1 < pp
    return ok, exact


def band_accept_cap(gpu: np.ndarray, order: np.ndarray, cum: np.ndarray, p: float, k_max: int,
                    band: float = BAND) -> bool:
    """A set under the top-p budget cap: the first min(k, k_max) keys of the
    rank order for a k the band accepts."""
    if len(gpu) < k_max:
        return band_accept(gpu, order, cum, p, band)[0]
    if len(gpu) != k_max or not np.array_equal(np.sort(order[:k_max]), gpu):
        return False
    # some k >= k_max is accepted: C_{k_max - 1} < p + band (C_0 = 0)
    ck1 = cum[k_max - 2] if k_max >= 2 else 0.0
    return np.float32(p) >= 1.0 or ck1 < float(np.float32(p)) + band


def path_counts(paths: np.ndarray) -> dict:
    """Histogram of route codes (low 4 bits) and flags over the rows."""
    out = {}
    for name, code in (("all", 1), ("tiny", 2), ("row", 3), ("large", 4), ("level", 5), ("list", 6),
                       ("scan", 7), ("list_g", 8)):
        out[name] = int(np.sum((paths & 15) == code))
    for name, bit in (("bitmap", 16), ("merge", 32), ("exact_z", 64), ("count", 128), ("from_scores", 256),
                      ("flag_list", 512)):
        out[name] = int(np.sum((paths & bit) != 0))
    return out


def check_out(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """Error ratio against the tolerance (<= 1 passes)."""
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    if dtype == "f32":
        return err / (1e-5 * float(np.max(np.abs(ref))))
    return err / (1e-2 * float(np.linalg.norm(ref)))


def oracle_k_low(w: synth.Workload, b: int, r: int) -> np.ndarray:
    g = w.kv_head(w.ret_heads[r])
    return oracle.project(w.k[b][:, g, :], w.w_k[r])
