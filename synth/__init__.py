"""Seeded synthetic workloads for the RTPurbo hot path (shared input generator).

This module only draws inputs; it holds none of the method's arithmetic.
Both the GPU tests/benchmark and the CPU oracle checks take their inputs from
here.  The bulk N(0,1) draws and the rotary embedding run in ``synth.c``
(Philox4x32-10 counter generator, Box-Muller, rotate-half RoPE in double);
the planted structure (needles, relevance clusters, budgets) is drawn with
numpy's Philox bit generator keyed by the workload seed.

Workload recipe (the pages measure retrieval on needle-in-a-haystack, RULER
and LongBench; none of those suites is used or reproduced here -- these
synthetic needle / cluster workloads stand in for them):

* Q, K, V: i.i.d. N(0,1) before RoPE, rotated by RoPE at their positions,
  then structure is planted post-RoPE, then rounded once to the storage type.
* Indexer projections W_q, W_k [D,16] per retrieval head: a 0/1 selector of
  the 8 lowest-frequency rotary pairs (column 2m -> dim D/2-8+m, column 2m+1
  -> dim D-8+m) plus N(0, 0.02^2) on every entry (the forum post's
  low-frequency RoPE projection, "Three Key Insights" item 2).
* needles (small fp32 decode): 8 distinct positions per retrieval head whose
  key is 3x the head's post-RoPE query; the needles form an exact tie group.
* clusters (bf16 decode/prefill): a relevant set of n keys per (sequence,
  retrieval head) whose 16 low-frequency coordinates are a*u + 0.1*N(0,1),
  with u a random unit vector; the query's coordinates are a*u + 0.1*N(0,1).
  a is set so that the expected cluster share of the indexer-softmax mass is
  0.999 for the smallest cluster at the workload's context length.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None
_lock = threading.Lock()

# Philox tensor ids
T_Q, T_K, T_V, T_WQ, T_WK = 1, 2, 3, 4, 5

DTYPES = {"f32": 0, "bf16": 1}


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            u64, u32, i64, i32, f64 = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_double)
            L.syn_normal_rope.argtypes = [u64, u32, u32, i64, i64, i32, i32, f64, f64, i64, i32, P, i32]
            L.syn_normal_rope.restype = None
            L.syn_normal.argtypes = [u64, u32, u32, i64, f64, P]
            L.syn_normal.restype = None
            L.syn_uniform.argtypes = [u64, u32, u32, i64, P]
            L.syn_uniform.restype = None
            L.syn_philox.argtypes = [P, P, P]
            L.syn_philox.restype = None
            _lib = L
    return _lib


def nthreads() -> int:
    n = os.cpu_count() or 1
    lim = os.environ.get("OMP_NUM_THREADS")
    if lim and lim.isdigit():
        n = min(n, int(lim))
    return max(1, min(n, 16))


# --------------------------------------------------------------------------
# dtype helpers (storage conversion only)
# --------------------------------------------------------------------------

def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns (nearest-even)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    return ((u + r) >> 16).astype(np.uint16)


def from_bf16(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def as_f32(x: np.ndarray) -> np.ndarray:
    return from_bf16(x) if x.dtype == np.uint16 else np.asarray(x, np.float32)


# --------------------------------------------------------------------------
# raw draws
# --------------------------------------------------------------------------

def normal_rope(seed: int, tensor: int, stream: int, tok0: int, n_tok: int, H: int,
                D: int, rope_base: float, pos0: int, dtype: str, scale: float = 1.0) -> np.ndarray:
    out = np.empty((n_tok, H, D), np.float32 if dtype == "f32" else np.uint16)
    lib().syn_normal_rope(seed, tensor, stream, tok0, n_tok, H, D, scale, rope_base, pos0,
                          DTYPES[dtype], out.ctypes.data_as(ctypes.c_void_p), nthreads())
    return out


def normals(seed: int, tensor: int, stream: int, n: int, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().syn_normal(seed, tensor, stream, n, scale, out.ctypes.data_as(ctypes.c_void_p))
    return out


def rng(seed: int, *stream: int) -> np.random.Generator:
    """numpy Philox generator for the discrete choices of one planting step."""
    key = (seed * 0x9E3779B97F4A7C15 + sum((s + 1) * 1000003 ** (i + 1) for i, s in enumerate(stream)))
    return np.random.Generator(np.random.Philox(key=key % (1 << 64)))


def low_freq_dims(D: int) -> np.ndarray:
    """Dims of the 8 lowest-frequency rotary pairs, in projection-column order."""
    half = D // 2
    i = np.arange(half - 8, half)
    dims = np.empty(16, np.int64)
    dims[0::2] = i
    dims[1::2] = i + half
    return dims


def projections(seed: int, n_ret: int, D: int, dtype: str, noise: float = 0.02):
    """(W_q, W_k), each [n_ret, D, 16] in storage dtype: selector + N(0, noise^2)."""
    dims = low_freq_dims(D)
    out = []
    for tensor in (T_WQ, T_WK):
        W = normals(seed, tensor, 0, n_ret * D * 16, noise).reshape(n_ret, D, 16)
        W[:, dims, np.arange(16)] += 1.0
        out.append(to_storage(W.astype(np.float32), dtype))
    return out[0], out[1]


def amplitude(n_min: int, L: int, idx_scale: float, share: float = 0.999) -> float:
    """Cluster amplitude a giving expected cluster mass share `share` for a
    cluster of n_min keys among L (background scores ~ N(0, a^2))."""
    s = idx_scale
    rhs = math.log(share / (1.0 - share)) + math.log(L / n_min)
    return math.sqrt(rhs / (s - s * s / 2.0))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    kind: str                     # "decode": one query per sequence at seq_lens-1
    dtype: str                    # "chunk": rows pos0..pos0+n-1 of sequence chunk_seq
    Hq: int
    Hkv: int
    D: int
    ret_heads: list
    window: int
    sinks: int
    idx_scale: float
    attn_scale: float
    rope_base: float
    seq_lens: np.ndarray          # int64 [B]
    top_p: np.ndarray             # float32 [B]
    q: np.ndarray                 # [n_tok, Hq, D] storage dtype
    k: list                       # per sequence [L_b, Hkv, D]
    v: list
    w_q: np.ndarray               # [n_ret, D, 16]
    w_k: np.ndarray
    chunk_seq: int = 0
    chunk_pos0: int = 0
    info: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return len(self.seq_lens)

    @property
    def n_ret(self) -> int:
        return len(self.ret_heads)

    @property
    def n_tok(self) -> int:
        return self.q.shape[0]

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def kv_head(self, h: int) -> int:
        return h // self.group

    def row_pos(self, t: int) -> int:
        """Position of query row t (keys 0..pos are visible)."""
        if self.kind == "decode":
            return int(self.seq_lens[t]) - 1
        return self.chunk_pos0 + t

    def row_seq(self, t: int) -> int:
        return t if self.kind == "decode" else self.chunk_seq

    def local_heads(self) -> list:
        return [h for h in range(self.Hq) if h not in set(self.ret_heads)]


def _base(name, kind, dtype, Hq, Hkv, D, ret_heads, window, sinks, rope, lens, p, seed):
    return dict(name=name, kind=kind, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D,
                ret_heads=sorted(int(h) for h in ret_heads), window=window, sinks=sinks,
                idx_scale=0.25, attn_scale=1.0 / math.sqrt(D), rope_base=rope,
                seq_lens=np.asarray(lens, np.int64), top_p=np.asarray(p, np.float32))


def _kv(seed, lens, Hkv, D, rope, dtype):
    K = [normal_rope(seed, T_K, b, 0, int(L), Hkv, D, rope, 0, dtype) for b, L in enumerate(lens)]
    V = [normal_rope(seed, T_V, b, 0, int(L), Hkv, D, 0.0, 0, dtype) for b, L in enumerate(lens)]
    return K, V


def sample_ret_heads(seed: int, Hq: int, n_ret: int) -> list:
    g = rng(seed, 7)
    return sorted(int(h) for h in g.choice(Hq, size=n_ret, replace=False))


def needle_decode(seed=1, B=1, L=4096, Hq=8, Hkv=8, D=64, ret_heads=(0, 1), p=0.9,
                  window=512, sinks=4, rope=1e4, dtype="f32", n_needles=8, lens=None,
                  name="needle_decode"):
    """Decode with planted needles: K := 3 x (post-RoPE query of the head)."""
    lens = np.full(B, L, np.int64) if lens is None else np.asarray(lens, np.int64)
    cfg = _base(name, "decode", dtype, Hq, Hkv, D, ret_heads, window, sinks, rope, lens,
                np.full(B, p, np.float32), seed)
    q = np.concatenate([normal_rope(seed, T_Q, b, 0, 1, Hq, D, rope, int(lens[b]) - 1, dtype)
                        for b in range(B)])
    K, V = _kv(seed, lens, Hkv, D, rope, dtype)
    needles = {}
    for b in range(B):
        for h in cfg["ret_heads"]:
            g = h // (Hq // Hkv)
            pos = rng(seed, 1, b, h).choice(int(lens[b]) - 1, size=n_needles, replace=False)
            key = 3.0 * as_f32(q[b, h])
            K[b][pos, g, :] = to_storage(key, dtype)
            needles[(b, h)] = np.sort(pos)
    w_q, w_k = projections(seed, len(cfg["ret_heads"]), D, dtype)
    return Workload(q=q, k=K, v=V, w_q=w_q, w_k=w_k, info=dict(needles=needles), **cfg)


def _plant(vec_f32: np.ndarray, dims: np.ndarray, a: float, u: np.ndarray,
           noise: np.ndarray) -> None:
    vec_f32[..., dims] = a * u + 0.1 * noise


def cluster_decode(seed=2, lens=(131072,) * 8, Hq=32, Hkv=8, D=128, n_ret=6, p=0.95,
                   window=2048, sinks=64, rope=5e5, dtype="bf16", size_dist=("loguniform", 16, 4096),
                   ret_heads=None, name="cluster_decode", shared_kv=False):
    """Decode with one planted relevance cluster per (sequence, retrieval head).
    shared_kv: retrieval heads that share a KV head share their cluster (the
    first head of the group draws its positions and direction, the others
    plant only their queries along it), so their selected sets overlap."""
    lens = np.asarray(lens, np.int64)
    B = len(lens)
    ret = sample_ret_heads(seed, Hq, n_ret) if ret_heads is None else list(ret_heads)
    pv = np.broadcast_to(np.asarray(p, np.float32), (B,)).copy()
    cfg = _base(name, "decode", dtype, Hq, Hkv, D, ret, window, sinks, rope, lens, pv, seed)
    q = np.concatenate([normal_rope(seed, T_Q, b, 0, 1, Hq, D, rope, int(lens[b]) - 1, dtype)
                        for b in range(B)])
    K, V = _kv(seed, lens, Hkv, D, rope, dtype)
    dims = low_freq_dims(D)
    n_min = size_dist[1] if size_dist[0] == "loguniform" else size_dist[2]
    sizes, amps = {}, {}
    for b in range(B):
        L = int(lens[b])
        a = amplitude(n_min, L, 0.25)
        amps[b] = a
        first = {}                                        # KV head -> the group's cluster (shared_kv)
        for r, h in enumerate(ret):
            gen = rng(seed, 2, b, h)
            g = h // (Hq // Hkv)
            if shared_kv and g in first:
                n, u = first[g]
                sizes[(b, h)] = n
            else:
                n = _draw_size(gen, size_dist, L)
                sizes[(b, h)] = n
                if n == 0:
                    continue
                pos = gen.choice(L - 1, size=n, replace=False)
                u = gen.standard_normal(16)
                u /= np.linalg.norm(u)
                first[g] = (n, u)
                kf = as_f32(K[b][pos, g, :]).copy()
                _plant(kf, dims, a, u, gen.standard_normal((n, 16)))
                K[b][pos, g, :] = to_storage(kf, dtype)
            qf = as_f32(q[b, h]).copy()
            _plant(qf, dims, a, u, gen.standard_normal(16))
            q[b, h] = to_storage(qf, dtype)
    w_q, w_k = projections(seed, len(ret), D, dtype)
    return Workload(q=q, k=K, v=V, w_q=w_q, w_k=w_k, info=dict(sizes=sizes, amplitude=amps), **cfg)


def _draw_size(gen, size_dist, L):
    if size_dist[0] == "loguniform":
        lo, hi = size_dist[1], size_dist[2]
        n = int(math.floor(math.exp(gen.uniform(math.log(lo), math.log(hi)))))
    else:  # ("zipf", exponent, lo, hi): P(n) ~ n^-exponent on [lo, hi]
        _, ex, lo, hi = size_dist
        support = np.arange(lo, hi + 1, dtype=np.float64)
        w = support ** (-ex)
        cdf = np.cumsum(w) / w.sum()
        n = int(support[min(np.searchsorted(cdf, gen.uniform()), len(support) - 1)])
    return min(n, L // 2)


def cluster_chunk(seed=3, L=131072, C=4096, Hq=32, Hkv=8, D=128, n_ret=6, p=0.95, window=2048,
                  sinks=64, rope=5e5, dtype="bf16", n_clusters=16, size_range=(16, 4096),
                  run_mean=256, ret_heads=None, name="cluster_chunk"):
    """Last causal prefill chunk (rows L-C..L-1) with 16 relevance clusters per
    retrieval head; consecutive query rows attend to one cluster in runs of
    geometric length (mean run_mean)."""
    ret = sample_ret_heads(seed, Hq, n_ret) if ret_heads is None else list(ret_heads)
    cfg = _base(name, "chunk", dtype, Hq, Hkv, D, ret, window, sinks, rope, [L], [p], seed)
    pos0 = L - C
    q = normal_rope(seed, T_Q, 0, pos0, C, Hq, D, rope, pos0, dtype)
    K, V = _kv(seed, [L], Hkv, D, rope, dtype)
    dims = low_freq_dims(D)
    a = amplitude(size_range[0], L, 0.25)
    assign = {}
    for h in ret:
        gen = rng(seed, 3, h)
        g = h // (Hq // Hkv)
        sizes = [int(math.floor(math.exp(gen.uniform(math.log(size_range[0]),
                                                       math.log(size_range[1])))))
                 for _ in range(n_clusters)]
        members = gen.choice(pos0, size=sum(sizes), replace=False)
        us = gen.standard_normal((n_clusters, 16))
        us /= np.linalg.norm(us, axis=1, keepdims=True)
        off = 0
        for c in range(n_clusters):
            pos = members[off: off + sizes[c]]
            off += sizes[c]
            kf = as_f32(K[0][pos, g, :]).copy()
            _plant(kf, dims, a, us[c], gen.standard_normal((len(pos), 16)))
            K[0][pos, g, :] = to_storage(kf, dtype)
        rows = np.empty(C, np.int64)
        i = 0
        while i < C:
            run = int(gen.geometric(1.0 / run_mean))
            rows[i: i + run] = gen.integers(n_clusters)
            i += run
        qf = as_f32(q[:, h, :]).copy()
        _plant(qf, dims, a, us[rows], gen.standard_normal((C, 16)))
        q[:, h, :] = to_storage(qf, dtype)
        assign[h] = (sizes, rows)
    w_q, w_k = projections(seed, len(ret), D, dtype)
    return Workload(q=q, k=K, v=V, w_q=w_q, w_k=w_k, chunk_seq=0, chunk_pos0=pos0,
                    info=dict(amplitude=a, clusters=assign), **cfg)


# --------------------------------------------------------------------------
# the five named workloads and their small parity-test versions
# --------------------------------------------------------------------------

def ragged_lens(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    gen = rng(seed, 5)
    return np.floor(np.exp(gen.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)


def ragged_p(seed: int, B: int) -> np.ndarray:
    gen = rng(seed, 6)
    return np.asarray(gen.choice([0.8, 0.9, 0.95, 0.99], size=B), np.float32)


CONFIG_NAMES = {
    1: "decode fp32 B=1 L=4096 Hq=Hkv=8 D=64 needles",
    2: "decode bf16 B=8 L=131072 Hq=32 Hkv=8 D=128",
    3: "prefill bf16 chunk 4096 at L=131072",
    4: "prefill bf16 chunk 8192 at L=1048576",
    5: "decode bf16 B=64 ragged L in [32768, 524288]",
}


def config(i: int, seed: int | None = None) -> Workload:
    """The five workloads at full size."""
    s = 1000 + i if seed is None else seed
    if i == 1:
        return needle_decode(seed=s, name="decode_f32_L4096_needles")
    if i == 2:
        return cluster_decode(seed=s, name="decode_bf16_B8_L131072")
    if i == 3:
        return cluster_chunk(seed=s, name="prefill_bf16_C4096_L131072")
    if i == 4:
        return cluster_chunk(seed=s, L=1048576, C=8192, window=4096, rope=1e6,
                             size_range=(64, 16384), run_mean=512,
                             name="prefill_bf16_C8192_L1048576")
    if i == 5:
        B = 64
        return cluster_decode(seed=s, lens=ragged_lens(s, B, 32768, 524288), p=ragged_p(s, B),
                              size_dist=("zipf", 1.1, 16, 32768), name="decode_bf16_B64_ragged")
    raise ValueError(i)


def small(i: int, seed: int | None = None) -> Workload:
    """Scaled-down versions the oracle finishes in seconds: several tiles,
    ragged tails, same head layout and value distributions."""
    s = 2000 + i if seed is None else seed
    if i == 1:
        return needle_decode(seed=s, name="decode_f32_small")
    if i == 2:
        return cluster_decode(seed=s, lens=(6000, 9001, 4097), size_dist=("loguniform", 4, 256),
                              window=300, sinks=8, name="decode_bf16_small")
    if i == 3:
        return cluster_chunk(seed=s, L=5000, C=300, size_range=(4, 200), run_mean=40,
                             window=500, sinks=16, name="prefill_bf16_small")
    if i == 4:
        return cluster_chunk(seed=s, L=12000, C=700, size_range=(8, 400), run_mean=80,
                             window=1000, sinks=64, rope=1e6, name="prefill_bf16_small_b")
    if i == 5:
        B = 6
        return cluster_decode(seed=s, lens=ragged_lens(s, B, 300, 9000), p=ragged_p(s, B),
                              size_dist=("zipf", 1.1, 4, 2048), window=400, sinks=8,
                              name="decode_bf16_ragged_small")
    raise ValueError(i)


def fp8_kv(w: "Workload"):
    """FP8 E4M3 storage of a workload's K and V (the FP8 K/V variant's input):
    one power-of-two scale per tensor, 2^ceil(log2(max|x| / 448)), and each
    value x / scale rounded to the nearest E4M3 code (ties to even; no value
    exceeds 448).  Returns (k_codes, v_codes, k_scale, v_scale), codes as
    uint8 arrays shaped like w.k[b] / w.v[b]."""
    import torch

    def quant(arrs):
        amax = max(float(np.max(np.abs(as_f32(a)))) for a in arrs)
        scale = float(2.0 ** math.ceil(math.log2(amax / 448.0)))
        codes = [torch.from_numpy(np.ascontiguousarray(as_f32(a) / np.float32(scale))).to(torch.float8_e4m3fn)
                 .view(torch.uint8).numpy() for a in arrs]
        return codes, scale

    kc, ks = quant(w.k)
    vc, vs = quant(w.v)
    return kc, vc, ks, vs
