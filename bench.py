"""Benchmark of the RTPurbo hot path on one MI355X.

One step = one decode step of one attention layer for the whole batch: the
indexer append of the new tokens, top-p selection for every retrieval head,
sparse attention over the selected rows, and window attention for the local
heads (on a second stream, overlapping the retrieval heads' work).

The prefill leg times one chunk of one layer the same way (top-p selection of
every chunk row, sparse prefill attention, window prefill attention on the
second stream) at two sizes: 4096 rows at context 131072 and 8192 rows at
context 1048576, next to dense causal attention of the same chunk on the same
GPU, and reports tokens/s/layer and the speedup, plus the share of the sparse
tiles' rows x union grid the rows' own sets fill; a third run of the 131072
workload with independent query rows (no runs on one cluster) is the stress
case of those union tiles.  The same
step captured as one HIP graph per layer instance is timed too and reported
beside it. (decode bf16, batch 8, context 131072, 32 query / 8 KV heads, head dim
128, 6 retrieval heads, top-p 0.95, window 2048 + 64 sinks).  Inputs are
synthetic and resident in HBM before timing; four independent layer instances
are rotated so that the 256 MB last-level cache cannot hold a layer's indexer
keys between its steps.

Prints one JSON line.  Extra fields: per-call times, the dense same-GPU
baseline and the speedup, the whole-step algorithmic bandwidth, and the oracle
timed on a bounded sample on the host (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0          # dense bf16
METRIC = "decode µs/step/layer + prefill tokens/s/layer at 128K–1M ctx; % HBM/MFMA peak"
COUNTERS = os.path.join(ROOT, "profiles", "k_sel_score_decode_bf16_B8_L131072_counters.json")
SCORE_SRC = os.path.join(ROOT, "sparse_attention_dim_amd", "csrc", "select.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_counters():
    """HBM bytes per launch of the score kernel from the committed rocprofv3
    counter summary, or None if the kernel source changed since."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except OSError:
        return None
    if c.get("source_sha256_16") != source_hash(SCORE_SRC):
        return None
    return c.get("hbm_bytes_per_launch")


def summarize(kind: str, paths, command: str, out: str):
    """Write a short profile summary under profiles/ from rocprofv3 CSV output.

    kind "stats":    paths = [kernel_stats.csv]; a table of per-kernel calls
                     and durations.
    kind "counters": paths = [FETCH_SIZE counter_collection.csv, WRITE_SIZE
                     counter_collection.csv]; the score kernel's HBM bytes per
                     launch, each counter scaled by what it reads for the
                     bench's 1 GiB calibration copy (the last dispatch)."""
    import csv
    import re

    if kind == "stats":
        rows = list(csv.DictReader(open(paths[0])))
        lines = ["# rocprofv3 kernel statistics", "", "Command (from the repository root):", "",
                 "    " + command, "", "| kernel | calls | avg us | min us | max us | total % |",
                 "|---|---|---|---|---|---|"]
        for r in rows[:25]:
            name = r["Name"].replace("rtp::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
            name = re.sub(r"\(.*", "", name)
            lines.append("| %s | %s | %.2f | %.2f | %.2f | %.1f |" % (
                name[:70], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        open(out, "w").write("\n".join(lines) + "\n")
        return
    res = {}
    for cname, path in zip(("FETCH_SIZE", "WRITE_SIZE"), paths):
        rows = list(csv.DictReader(open(path)))
        calib = float(rows[-1]["Counter_Value"])           # KiB for 1 GiB moved
        scale = (1 << 20) / calib
        ks = [float(r["Counter_Value"]) for r in rows if re.search(r"k_sel_score<unsigned short, 0>", r["Kernel_Name"])]
        res[cname] = {"calibration_kib_per_gib": calib, "scale": scale,
                      "score_kernel_kib_raw": sum(ks) / len(ks), "dispatches": len(ks),
                      "score_kernel_bytes": sum(ks) / len(ks) * scale * 1024}
    summary = {
        "kernel": "k_sel_score<bf16, scores only> (decode bf16 B=8 L=131072, 6 retrieval heads)",
        "command": command,
        "counters": res,
        "hbm_bytes_per_launch": int(res["FETCH_SIZE"]["score_kernel_bytes"] + res["WRITE_SIZE"]["score_kernel_bytes"]),
        "algorithmic_read_bytes": 8 * 131072 * 6 * 32,
        "source_sha256_16": source_hash(SCORE_SRC),
    }
    json.dump(summary, open(out, "w"), indent=1)


def cpu_baseline(w, n_seq: int, threads: int):
    """Time the oracle (as it stands) on the first n_seq sequences of one
    decode step; the indexer keys of the context are computed untimed."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    jobs_kl = [(b, r) for b in range(n_seq) for r in range(w.n_ret)]

    def fill(br):
        b, r = br
        g = w.kv_head(w.ret_heads[r])
        return br, oracle.project(w.k[b][:, g, :], w.w_k[r])

    with cf.ThreadPoolExecutor(threads) as ex:
        k_low = dict(ex.map(fill, jobs_kl))
    kf = {}
    for b in range(n_seq):
        for g in range(w.Hkv):
            kf[(b, g)] = (np.ascontiguousarray(oracle.as_f32(w.k[b][:, g, :])),
                          np.ascontiguousarray(oracle.as_f32(w.v[b][:, g, :])))

    def ret_job(br):
        b, r = br
        h = w.ret_heads[r]
        K, V = kf[(b, w.kv_head(h))]
        return oracle.retrieval_row(w.q[b, h], K, V, w.w_q[r], w.w_k[r], w.row_pos(b), w.idx_scale,
                                    float(w.top_p[b]), w.attn_scale, k_low=k_low[(b, r)],
                                    want_order=False)["sel"].size

    def loc_job(bh):
        b, h = bh
        K, V = kf[(b, w.kv_head(h))]
        return oracle.local_row(w.q[b, h], K, V, w.row_pos(b), w.window, w.sinks, w.attn_scale)[0]

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        sizes = list(ex.map(ret_job, jobs_kl))
        list(ex.map(loc_job, [(b, h) for b in range(n_seq) for h in w.local_heads()]))
    dt = time.perf_counter() - t0
    return dt, sizes


def union_useful(rp, ix, n_tok: int, n_ret: int, m: int = 64) -> float:
    """Share of the sparse prefill tiles' rows x union grid that the rows'
    own sets fill: sum |S_i| / sum over tiles of (rows x |union of S_i|),
    tiles of m consecutive rows of one retrieval head."""
    import numpy as np

    grid = 0
    for r in range(n_ret):
        for t0 in range(0, n_tok, m):
            rows = [t * n_ret + r for t in range(t0, min(n_tok, t0 + m))]
            parts = [ix[rp[i]: rp[i + 1]] for i in rows]
            grid += len(rows) * len(np.unique(np.concatenate(parts)))
    return float(rp[-1]) / grid if grid else 0.0


def prefill_leg(cfg: int, steps: int, run_mean: int | None = None, dense: bool = True):
    """One prefill chunk of one layer: eager select + sparse prefill on the
    main stream, window prefill on a second stream; dense causal attention of
    the same chunk for comparison.  run_mean: the workload's generator with
    another mean run length of query rows on one cluster (1: independent
    rows, the stress case of the union tiles)."""
    import numpy as np
    import torch

    import sparse_attention_dim_amd as rtp
    import synth
    from sparse_attention_dim_amd.paged import PagedCache, rtp_dtype, to_device

    dev = torch.device("cuda:0")
    t0 = time.time()
    if run_mean is None:
        w = synth.config(cfg)
    else:
        assert cfg == 3
        w = synth.cluster_chunk(seed=1003, run_mean=run_mean, name="prefill_bf16_C4096_L131072_run%d" % run_mean)
    L = int(w.seq_lens[0])
    log("[bench] prefill %s generated in %.1fs" % (w.name, time.time() - t0))
    layer = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp_dtype(w.dtype), w.ret_heads, w.window, w.sinks,
                           w.attn_scale, w.idx_scale)
    pc = PagedCache(w.k, w.v, w.n_ret, w.dtype, device=dev, permute_seed=100)
    cache = pc.cache(L)
    q = to_device(w.q, dev)
    w_q, w_k = to_device(w.w_q, dev), to_device(w.w_k, dev)
    top_p = torch.from_numpy(w.top_p).to(dev)
    query = rtp.make_query(q, rtp.RTP_CHUNK, w.chunk_seq, w.chunk_pos0)
    sid, pos = pc.all_positions(0, dev)
    rtp.indexer_append(layer, cache, w_k, sid, pos)
    rows = w.n_tok * w.n_ret
    cap = rows * 16384
    row_ptr = torch.zeros(rows + 1, dtype=torch.int64, device=dev)
    idx = torch.empty(cap, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sel = rtp.make_sel(row_ptr, idx, status)
    ws_sel = torch.empty(rtp.topp_select_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
    ws_sp = torch.empty(rtp.sparse_attn_workspace(layer, cache, query, cap), dtype=torch.uint8, device=dev)
    ws_win = torch.empty(rtp.window_attn_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
    out = torch.zeros_like(q)
    side = torch.cuda.Stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step(times=None):
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            if times is not None:
                ev[2].record(side)
            rtp.window_attn(layer, cache, query, out, ws_win, stream=side)
            if times is not None:
                ev[3].record(side)
        if times is not None:
            ev[0].record()
        rtp.topp_select(layer, cache, query, w_q, top_p, sel, ws_sel)
        if times is not None:
            ev[1].record()
        rtp.sparse_attn_prefill(layer, cache, query, sel, out, ws_sp)
        main.wait_stream(side)

    step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "selection status %d" % int(status.item())
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    step_ms = a.elapsed_time(b) / steps
    # per-call times, sequential
    sel_ms, sp_ms, win_ms = [], [], []
    for _ in range(2):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        rtp.topp_select(layer, cache, query, w_q, top_p, sel, ws_sel)
        e[1].record()
        rtp.sparse_attn_prefill(layer, cache, query, sel, out, ws_sp)
        e[2].record()
        rtp.window_attn(layer, cache, query, out, ws_win)
        e[3].record()
        torch.cuda.synchronize()
        sel_ms.append(e[0].elapsed_time(e[1]))
        sp_ms.append(e[1].elapsed_time(e[2]))
        win_ms.append(e[2].elapsed_time(e[3]))
    rp = row_ptr.cpu().numpy()
    sizes = np.diff(rp)
    n_sel = int(rp[-1])
    useful = union_useful(rp, idx[:n_sel].cpu().numpy(), w.n_tok, w.n_ret)
    dense_ms = None
    if dense:
        ws_d = torch.empty(rtp.dense_attn_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
        dout = torch.zeros_like(q)
        rtp.dense_attn(layer, cache, query, dout, ws_d)
        torch.cuda.synchronize()
        a.record()
        nd = 2
        for _ in range(nd):
            rtp.dense_attn(layer, cache, query, dout, ws_d)
        b.record()
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b) / nd
        del ws_d
    # algorithmic flops: QK and PV, 2 D flops each per (query head, key) pair
    f_pair = 4 * w.D
    sp_flops = n_sel * f_pair
    win_pairs = sum(min(w.window + w.sinks, w.row_pos(t) + 1) for t in range(w.n_tok)) * (w.Hq - w.n_ret)
    dense_pairs = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.Hq
    sp_t, win_t = float(np.median(sp_ms)), float(np.median(win_ms))
    res = {
        "workload": w.name, "chunk_rows": w.n_tok, "context": L, "top_p": float(w.top_p[0]),
        "tokens_per_s": round(w.n_tok / (step_ms * 1e-3), 1), "step_ms": round(step_ms, 3),
        "select_ms": round(float(np.median(sel_ms)), 3), "sparse_ms": round(sp_t, 3),
        "window_ms": round(win_t, 3),
        "selected_per_row": {"min": int(sizes.min()), "median": int(np.median(sizes)),
                             "mean": round(float(sizes.mean()), 1), "max": int(sizes.max())},
        "sparse_tflops": round(sp_flops / (sp_t * 1e-3) / 1e12, 2),
        "sparse_mfma_frac": round(sp_flops / (sp_t * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 5),
        "sparse_union_useful": round(useful, 4),
        "window_tflops": round(win_pairs * f_pair / (win_t * 1e-3) / 1e12, 2),
    }
    if dense_ms is not None:
        res.update({"dense_ms": round(dense_ms, 3),
                    "dense_tflops": round(dense_pairs * f_pair / (dense_ms * 1e-3) / 1e12, 2),
                    "speedup_vs_dense": round(dense_ms / step_ms, 3)})
    del pc, cache, idx, ws_sel, ws_sp, ws_win
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--contiguous", action="store_true", help="pages in order instead of permuted")
    ap.add_argument("--graph", action="store_true", help="time HIP graph replays instead of eager launches")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill leg")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="KIND OUT COMMAND CSV...: write a profile summary from rocprofv3 output and exit")
    args = ap.parse_args()
    if args.summarize:
        kind, out, command, *paths = args.summarize
        summarize(kind, paths, command, out)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_dim_amd as rtp
    import synth
    from sparse_attention_dim_amd.paged import PagedCache, rtp_dtype, to_device

    rtp.load()
    dev = torch.device("cuda:0")
    t0 = time.time()
    w = synth.config(2)
    log("[bench] generated %s in %.1fs" % (w.name, time.time() - t0))
    B, L = w.B, int(w.seq_lens.max())
    layer = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp_dtype(w.dtype), w.ret_heads, w.window, w.sinks,
                           w.attn_scale, w.idx_scale)

    inst = []
    for i in range(args.instances):
        pc = PagedCache(w.k, w.v, w.n_ret, w.dtype, device=dev,
                        permute_seed=None if args.contiguous else 100 + i)
        cache = pc.cache(L)
        q = to_device(w.q, dev)
        w_q, w_k = to_device(w.w_q, dev), to_device(w.w_k, dev)
        top_p = torch.from_numpy(w.top_p).to(dev)
        query = rtp.make_query(q, rtp.RTP_DECODE)
        for b in range(B):
            sid, pos = pc.all_positions(b, dev)
            rtp.indexer_append(layer, cache, w_k, sid, pos)
        new_sid = torch.arange(B, dtype=torch.int32, device=dev)
        new_pos = (pc.seq_lens - 1).to(torch.int32)
        rows = B * w.n_ret
        cap = rows * L
        row_ptr = torch.zeros(rows + 1, dtype=torch.int64, device=dev)
        idx = torch.empty(cap, dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        sel = rtp.make_sel(row_ptr, idx, status)
        ws_sel = torch.empty(rtp.topp_select_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
        ws_sp = torch.empty(rtp.sparse_attn_workspace(layer, cache, query, cap), dtype=torch.uint8, device=dev)
        ws_win = torch.empty(rtp.window_attn_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
        out = torch.zeros_like(q)
        inst.append(dict(pc=pc, cache=cache, q=q, w_q=w_q, w_k=w_k, top_p=top_p, query=query,
                         sid=new_sid, pos=new_pos, sel=sel, row_ptr=row_ptr, idx=idx, status=status,
                         ws_sel=ws_sel, ws_sp=ws_sp, ws_win=ws_win, out=out))
    torch.cuda.synchronize()
    log("[bench] %d layer instances resident (%.1f GB allocated)" %
        (args.instances, torch.cuda.memory_allocated() / 1e9))

    calls = ("append", "select", "sparse", "window")

    def step(I, ev=None):
        if ev is not None:
            ev[0].record()
        rtp.indexer_append(layer, I["cache"], I["w_k"], I["sid"], I["pos"])
        if ev is not None:
            ev[1].record()
        rtp.topp_select(layer, I["cache"], I["query"], I["w_q"], I["top_p"], I["sel"], I["ws_sel"])
        if ev is not None:
            ev[2].record()
        rtp.sparse_attn_decode(layer, I["cache"], I["query"], I["sel"], I["out"], I["ws_sp"])
        if ev is not None:
            ev[3].record()
        rtp.window_attn(layer, I["cache"], I["query"], I["out"], I["ws_win"])
        if ev is not None:
            ev[4].record()

    # The local heads do not depend on the retrieval heads' selection: they run
    # on a second stream, forked from the main stream once the selection's pass
    # over the indexer keys is done (so the two bandwidth-bound passes do not
    # share HBM, and the window overlaps the latency-bound rest of the
    # selection and the sparse attention), and joined back at the end.  The
    # library calls are prepared once per layer instance and stream (their
    # arguments marshalled once), so the host enqueues a step faster than the
    # GPU runs it.
    side = torch.cuda.Stream()

    def make_step(I, main):
        sel_args = (layer, I["cache"], I["query"], I["w_q"], I["top_p"], I["sel"], I["ws_sel"])
        append = rtp.indexer_append(layer, I["cache"], I["w_k"], I["sid"], I["pos"], stream=main, prepare=True)
        begin = rtp.topp_select_begin(*sel_args, stream=main, prepare=True)
        end = rtp.topp_select_end(*sel_args, stream=main, prepare=True)
        sparse = rtp.sparse_attn_decode(layer, I["cache"], I["query"], I["sel"], I["out"], I["ws_sp"], stream=main,
                                        prepare=True)
        window = rtp.window_attn(layer, I["cache"], I["query"], I["out"], I["ws_win"], stream=side, prepare=True)
        fork, join = torch.cuda.Event(), torch.cuda.Event()

        def run():
            append()
            begin()
            fork.record(main)
            side.wait_event(fork)
            window()
            end()
            sparse()
            join.record(side)
            main.wait_event(join)
        return run

    main_stream = torch.cuda.current_stream()
    steps_overlap = [make_step(I, main_stream) for I in inst]

    def step_overlap(I):
        steps_overlap[inst.index(I)]()

    for s in range(args.warmup):
        step(inst[s % len(inst)])
        step_overlap(inst[s % len(inst)])
    torch.cuda.synchronize()
    assert all(int(I["status"].item()) == 0 for I in inst), "selection capacity overflow"

    # per-call breakdown: sequential eager launches with events between calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for s in range(args.steps):
        step(inst[s % len(inst)], evs[s])
    torch.cuda.synchronize()
    per_call = {c: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e3
                for i, c in enumerate(calls)}

    def timed(fn):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for s in range(args.steps):
            fn(s)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    eager_ms = timed(lambda s: steps_overlap[s % len(inst)]())

    # one HIP graph per layer instance, replayed round-robin
    graphs = []
    for I in inst:
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            make_step(I, torch.cuda.current_stream())()
        graphs.append(gph)
    for s in range(len(graphs) * 2):
        graphs[s % len(graphs)].replay()
    torch.cuda.synchronize()
    graph_ms = timed(lambda s: graphs[s % len(graphs)].replay())
    ms = graph_ms if args.graph else eager_ms
    launch = "hip_graph" if args.graph else "eager, two streams"

    # --- algorithmic bytes of one step ---------------------------------------
    rp = inst[0]["row_ptr"].cpu().numpy()
    n_sel = int(rp[-1])
    sizes = np.diff(rp)
    lens = w.seq_lens.astype(np.int64)
    kv_row = w.D * 2 * 2                          # one K row + one V row, bf16
    bytes_klow = int(sum(lens[b] for b in range(B)) * w.n_ret * 32)
    bytes_sparse = n_sel * kv_row + n_sel * 8
    win_keys = [min(w.window + w.sinks, int(l)) for l in lens]
    bytes_win = int(sum(win_keys) * w.Hkv * kv_row)
    step_bytes = bytes_klow + bytes_sparse + bytes_win

    # --- the dominant kernel: the indexer score pass, timed on its own ------
    I = inst[0]
    rows = B * w.n_ret
    qlow_buf = torch.empty((rows, 16), dtype=torch.int16, device=dev)
    score_bufs = [torch.empty((rows, L), dtype=torch.float32, device=dev) for _ in inst]
    score_calls = [rtp.indexer_scores(layer, J["cache"], J["query"], J["w_q"], qlow_buf, score_bufs[i],
                                      prepare=True) for i, J in enumerate(inst)]
    for c in score_calls:
        c()
    # back-to-back launches between one pair of events: prepared calls enqueue
    # faster than a launch runs, so the span is the launches plus their gaps
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for s in range(args.steps):
        score_calls[s % len(inst)]()
    k1.record()
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / args.steps
    k_achieved = bytes_klow / (k_ms * 1e-3) / 1e9

    # --- dense baseline on the same GPU --------------------------------------
    ws_dense = torch.empty(rtp.dense_attn_workspace(layer, I["cache"], I["query"]), dtype=torch.uint8,
                           device=dev)
    dense_out = torch.zeros_like(I["q"])
    for s in range(3):
        rtp.dense_attn(layer, inst[s % len(inst)]["cache"], inst[s % len(inst)]["query"], dense_out, ws_dense)
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nd = 10
    d0.record()
    for s in range(nd):
        J = inst[s % len(inst)]
        rtp.dense_attn(layer, J["cache"], J["query"], dense_out, ws_dense)
    d1.record()
    torch.cuda.synchronize()
    dense_ms = d0.elapsed_time(d1) / nd
    dense_bytes = int(sum(int(l) for l in lens) * w.Hkv * kv_row)

    # calibration copy of known size for the HBM counter runs (1 GiB read, 1 GiB write)
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # --- the oracle on the host, on a bounded sample --------------------------
    cpu = None
    if not args.no_cpu:
        threads = min(os.cpu_count() or 1, 16)
        ns = min(args.cpu_seqs, B)
        dt, _ = cpu_baseline(w, ns, threads)
        cpu = {"value": dt / ns * B * 1e6, "unit": "µs/step/layer", "cores": threads, "kind": "oracle",
               "sample": "retrieval rows and local heads of %d of the %d sequences of one decode step "
                         "(indexer keys of the context precomputed untimed), scaled x%d to the batch"
                         % (ns, B, B // ns)}

    prefill = None
    if not args.no_prefill:
        prefill = {"128k": prefill_leg(3, args.prefill_steps), "1m": prefill_leg(4, max(1, args.prefill_steps // 2)),
                   "128k_independent_rows": prefill_leg(3, args.prefill_steps, run_mean=1, dense=False)}

    res = {
        "metric": METRIC,
        "value": round(ms * 1e3, 2),
        "unit": "µs/step/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "kind": "decode", "batch": B, "context": L, "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.D, "retrieval_heads": w.n_ret, "top_p": 0.95,
                   "window": w.window, "sinks": w.sinks, "layer_instances": args.instances},
        "roofline": {"kernel": "k_sel_score<bf16, scores only> (rtp_indexer_scores, decode)", "bound": "hbm",
                     "achieved": round(k_achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(k_achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_counters(),
                     "algorithmic_bytes": bytes_klow, "avg_launch_us": round(k_ms * 1e3, 2)},
        "cpu_baseline": cpu,
        "per_call_us": {k: round(v, 2) for k, v in per_call.items()},
        "launch": launch,
        "eager_overlap_us": round(eager_ms * 1e3, 2),
        "graph_overlap_us": round(graph_ms * 1e3, 2),
        "pages": "contiguous" if args.contiguous else "permuted",
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "selected_per_row": {"min": int(sizes.min()), "median": int(np.median(sizes)),
                             "max": int(sizes.max()), "total": n_sel},
        "dense_us": round(dense_ms * 1e3, 2),
        "dense_hbm_frac": round(dense_bytes / (dense_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "speedup_vs_dense": round(dense_ms / ms, 3),
        "prefill": prefill,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
