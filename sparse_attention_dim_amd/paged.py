"""Paged KV-cache construction for librtp (plumbing: torch allocates and copies).

Turns per-sequence logical arrays [L_b, Hkv, D] into the page pools of
``include/rtp.h`` -- k, v as [num_blocks, Hkv, 256, D], k_low as bf16
[num_blocks, num_ret, 256, 16] -- with a block table whose page ids may be
permuted.  Arrays of dtype uint16 hold bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np
import torch

from . import RTP_BLOCK, RTP_BF16, RTP_F32, kv_append, make_cache

BLOCK = RTP_BLOCK


def torch_dtype(dtype: str):
    """Storage type of K/V pages: bf16, fp32, or FP8 E4M3 codes held as uint8."""
    return {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[dtype]


def rtp_dtype(dtype: str) -> int:
    return RTP_BF16 if dtype == "bf16" else RTP_F32


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays become bfloat16 with the same bits."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 device tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class PagedCache:
    """Device pages of K, V and K_low for a batch of sequences."""

    def __init__(self, k_list, v_list, n_ret: int, dtype: str, device="cuda", permute_seed=None,
                 spare_blocks: int = 0):
        B = len(k_list)
        Hkv, D = k_list[0].shape[1], k_list[0].shape[2]
        lens = [int(k.shape[0]) for k in k_list]
        nblk = [(L + BLOCK - 1) // BLOCK for L in lens]
        total = sum(nblk) + spare_blocks
        ids = np.arange(total, dtype=np.int64)
        if permute_seed is not None:
            ids = np.random.default_rng(permute_seed).permutation(total)
        self.max_blocks = max(nblk)
        table = np.zeros((B, self.max_blocks), np.int32)
        off = 0
        for b in range(B):
            table[b, :nblk[b]] = ids[off: off + nblk[b]]
            off += nblk[b]
        td = torch_dtype(dtype)
        self.k = torch.zeros((total, Hkv, BLOCK, D), dtype=td, device=device)
        self.v = torch.zeros((total, Hkv, BLOCK, D), dtype=td, device=device)
        self.k_low = torch.zeros((total, n_ret, BLOCK, 16), dtype=torch.bfloat16, device=device)
        for b in range(B):
            pages = torch.from_numpy(table[b, :nblk[b]].astype(np.int64)).to(device)
            for pool, src in ((self.k, k_list[b]), (self.v, v_list[b])):
                x = to_device(src, device)
                pad = nblk[b] * BLOCK - lens[b]
                if pad:
                    x = torch.cat([x, torch.zeros((pad, Hkv, D), dtype=td, device=device)])
                x = x.view(nblk[b], BLOCK, Hkv, D).permute(0, 2, 1, 3).contiguous()
                pool.index_copy_(0, pages, x)
                del x
        self.block_table = torch.from_numpy(table).to(device)
        self.seq_lens = torch.tensor(lens, dtype=torch.int32, device=device)
        self.lens = lens
        self.max_seq_len = max(lens)
        self.Hkv, self.D, self.n_ret, self.dtype = Hkv, D, n_ret, dtype
        self.table = table

    def cache(self, max_seq_len: int | None = None):
        return make_cache(self.k, self.v, self.k_low, self.block_table, self.seq_lens,
                          self.max_seq_len if max_seq_len is None else max_seq_len)

    def k_low_logical(self, b: int, r: int) -> np.ndarray:
        """bf16 bits [L_b, 16] of retrieval head r's indexer keys of sequence b."""
        L = self.lens[b]
        nb = (L + BLOCK - 1) // BLOCK
        pages = torch.from_numpy(self.table[b, :nb].astype(np.int64)).to(self.k_low.device)
        x = self.k_low.index_select(0, pages)[:, r]             # [nb, 256, 16]
        return bf16_bits(x.reshape(nb * BLOCK, 16))[:L]

    def all_positions(self, b: int, device="cuda"):
        L = self.lens[b]
        return (torch.full((L,), b, dtype=torch.int32, device=device),
                torch.arange(L, dtype=torch.int32, device=device))


class RingCache:
    """The cache-side layout: full K/V pages only for the KV heads that serve a
    retrieval head, a window-only ring of ring_pages pages per sequence for the
    other KV heads, and the indexer pages.  Filled in position order by
    rtp_kv_append (each call spans at most (ring_pages - 1) * 256 positions of
    a sequence, so no two of its tokens share a ring slot)."""

    def __init__(self, Hkv: int, D: int, group: int, ret_heads, n_ret: int, lens, dtype: str, ring_pages: int,
                 device="cuda", permute_seed=None, spare_blocks: int = 0):
        serves = sorted({int(h) // group for h in ret_heads})
        self.pool_heads = serves
        self.ring_heads = [g for g in range(Hkv) if g not in serves]
        B = len(lens)
        nblk = [(int(L) + BLOCK - 1) // BLOCK for L in lens]
        total = sum(nblk) + spare_blocks
        g = np.random.default_rng(permute_seed)
        ids = g.permutation(total) if permute_seed is not None else np.arange(total)
        self.max_blocks = max(nblk)
        table = np.zeros((B, self.max_blocks), np.int32)
        off = 0
        for b in range(B):
            table[b, :nblk[b]] = ids[off: off + nblk[b]]
            off += nblk[b]
        rids = g.permutation(B * ring_pages) if permute_seed is not None else np.arange(B * ring_pages)
        td = torch_dtype(dtype)
        self.k = torch.zeros((total, len(serves), BLOCK, D), dtype=td, device=device)
        self.v = torch.zeros_like(self.k)
        self.k_ring = torch.zeros((B * ring_pages, max(1, len(self.ring_heads)), BLOCK, D), dtype=td, device=device)
        self.v_ring = torch.zeros_like(self.k_ring)
        self.k_low = torch.zeros((total, n_ret, BLOCK, 16), dtype=torch.bfloat16, device=device)
        self.block_table = torch.from_numpy(table).to(device)
        self.ring_table = torch.from_numpy(rids.reshape(B, ring_pages).astype(np.int32)).to(device)
        self.seq_lens = torch.tensor([int(L) for L in lens], dtype=torch.int32, device=device)
        self.lens = [int(L) for L in lens]
        self.max_seq_len = max(self.lens)
        self.ring_pages = ring_pages
        self.table = table
        self.device = device

    def cache(self, max_seq_len: int | None = None):
        return make_cache(self.k, self.v, self.k_low, self.block_table, self.seq_lens,
                          self.max_seq_len if max_seq_len is None else max_seq_len,
                          k_ring=self.k_ring, v_ring=self.v_ring, ring_table=self.ring_table)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k, self.v, self.k_ring, self.v_ring))

    def fill(self, layer, k_list, v_list, w_k, upto=None):
        """Append every sequence's tokens [0, upto[b]) in position order."""
        cache = self.cache()
        step = (self.ring_pages - 1) * BLOCK
        for b, L in enumerate(self.lens):
            end = L if upto is None else upto[b]
            for j0 in range(0, end, step):
                j1 = min(end, j0 + step)
                kn = to_device(np.ascontiguousarray(k_list[b][j0:j1]), self.device)
                vn = to_device(np.ascontiguousarray(v_list[b][j0:j1]), self.device)
                sid = torch.full((j1 - j0,), b, dtype=torch.int32, device=self.device)
                pos = torch.arange(j0, j1, dtype=torch.int32, device=self.device)
                kv_append(layer, cache, kn, vn, w_k, sid, pos)

    def k_low_logical(self, b: int, r: int) -> np.ndarray:
        L = self.lens[b]
        nb = (L + BLOCK - 1) // BLOCK
        pages = torch.from_numpy(self.table[b, :nb].astype(np.int64)).to(self.k_low.device)
        x = self.k_low.index_select(0, pages)[:, r]
        return bf16_bits(x.reshape(nb * BLOCK, 16))[:L]
