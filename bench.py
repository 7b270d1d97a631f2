"""Benchmark of the RTPurbo hot path on one MI355X.

Headline: one decode step of one attention layer for the whole batch at
decode bf16, B = 8, L = 131072 (32 query / 8 KV heads, head dim 128, 6
retrieval heads, top-p 0.95, window 2048 + 64 sinks): the indexer append of
the new tokens, top-p selection for every retrieval head, sparse attention over
the selected rows, and window attention of the local heads (on a second stream,
overlapping the retrieval heads' latency-bound selection tail).  Four
independent layer instances rotate so the 256 MB last-level cache cannot hold
a layer's indexer keys between its steps.  Inputs are synthetic and resident in
HBM before timing.

Beside it (extra keys of the same JSON line):
  * decode_ragged: decode bf16, B = 64, per-sequence contexts 32K..512K
    (paged), per-request top-p -- its step time against the 60 % HBM target;
  * decode_f32_needles: decode fp32, B = 1, L = 4096 (launch-bound);
  * decode variants at the headline shape: FP8 K/V, fixed top-k, the k_max
    budget cap, and the window-only ring layout's memory;
  * prefill: one chunk of one layer (4096 rows at L = 131072, 8192 rows at
    L = 1048576, and the 131072 chunk with independent query rows) -- the
    chunk's indexer append, selection, sparse prefill attention, and window
    prefill attention on the second stream; tokens/s/layer, next to dense
    causal attention of the same chunk;
  * per-step median / p10 / p90 over at least 50 steps for every leg;
  * the oracle timed on the host on bounded samples (cpu_baseline).

Prints one JSON line.
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
EXP_PEAK_PER_S = 256 * 2.4e9 * 16  # v_exp_f32: quarter rate, 16 lanes per CU per clock
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
                     bench's 1 GiB calibration copy (the last dispatch).
    kind "pmc":      paths = [counter_collection.csv of one counter pass,
                     FETCH_SIZE csv, WRITE_SIZE csv]; per kernel: mean counter
                     values per dispatch and the derived MFMA / transcendental
                     / LDS figures, HBM bytes scaled as above."""
    import csv
    import re

    def short(n):
        n = n.replace("rtp::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
        return re.sub(r"\(.*", "", n)

    if kind == "stats":
        rows = list(csv.DictReader(open(paths[0])))
        lines = ["# rocprofv3 kernel statistics", "", "Command (from the repository root):", "",
                 "    " + command, "", "| kernel | calls | avg us | min us | max us | total % |",
                 "|---|---|---|---|---|---|"]
        for r in rows[:60]:
            lines.append("| %s | %s | %.2f | %.2f | %.2f | %.1f |" % (
                short(r["Name"])[:70], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        open(out, "w").write("\n".join(lines) + "\n")
        return
    if kind == "counters":
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
            "algorithmic_write_bytes": 8 * 131072 * 6 * 4,
            "source_sha256_16": source_hash(SCORE_SRC),
        }
        json.dump(summary, open(out, "w"), indent=1)
        return
    # pmc: counters per kernel name, averaged over its dispatches; each pass's
    # last dispatch is the 1 GiB calibration copy
    per = {}
    scale = {"FETCH_SIZE": None, "WRITE_SIZE": None}
    for path in paths:
        rows = list(csv.DictReader(open(path)))
        last = rows[-1]["Dispatch_Id"]
        for r in rows:
            if r["Dispatch_Id"] == last:
                if r["Counter_Name"] in scale:
                    scale[r["Counter_Name"]] = (1 << 20) / float(r["Counter_Value"])
                continue
            k = short(r["Kernel_Name"])
            d = per.setdefault(k, {})
            d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# rocprofv3 counters per kernel (mean per dispatch)", "", "Command (from the repository root):", "",
             "    " + command, "",
             "HBM bytes: FETCH_SIZE / WRITE_SIZE (KiB) scaled by what each reads for a 1 GiB copy "
             "(the bench's last dispatch): %s." % json.dumps({k: round(v, 4) if v else None for k, v in scale.items()}),
             "MFMA util = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) (GRBM_GUI_ACTIVE "
             "is summed over the 8 XCDs); bf16 MFMA flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.", "",
             "| kernel | dispatches | MFMA bf16 GFLOP | MFMA util | VALU insts (M) | trans f32 insts (M) | "
             "LDS insts (M) | LDS bank-conflict cycles (M) | HBM read MB | HBM write MB |",
             "|---|---|---|---|---|---|---|---|---|---|"]

    def mean(d, c):
        v = d.get(c)
        return sum(v) / len(v) if v else None

    for k, d in sorted(per.items()):
        if "copyBuffer" in k or "elementwise" in k:
            continue
        n = max(len(v) for v in d.values())
        mops, busy, gui = mean(d, "SQ_INSTS_VALU_MFMA_MOPS_BF16"), mean(d, "SQ_VALU_MFMA_BUSY_CYCLES"), mean(d, "GRBM_GUI_ACTIVE")
        f = lambda x, s=1e6: "%.2f" % (x / s) if x is not None else "-"
        util = "%.3f" % (busy / (gui / 8 * 1024)) if busy is not None and gui else "-"
        rd = mean(d, "FETCH_SIZE")
        wr = mean(d, "WRITE_SIZE")
        lines.append("| %s | %d | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            k[:60], n, f(mops * 512 if mops is not None else None, 1e9), util, f(mean(d, "SQ_INSTS_VALU")),
            f(mean(d, "SQ_INSTS_VALU_TRANS_F32")), f(mean(d, "SQ_INSTS_LDS")), f(mean(d, "SQ_LDS_BANK_CONFLICT")),
            f(rd * 1024 * scale["FETCH_SIZE"] if rd is not None and scale["FETCH_SIZE"] else None),
            f(wr * 1024 * scale["WRITE_SIZE"] if wr is not None and scale["WRITE_SIZE"] else None)))
    open(out, "w").write("\n".join(lines) + "\n")


def stats(xs):
    import numpy as np
    a = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def union_useful(rp, ix, n_tok: int, n_ret: int, m: int = 64):
    """(share of the sparse prefill tiles' rows x union grid that the rows'
    own sets fill, union keys over all tiles)."""
    import numpy as np

    grid = 0
    ukeys = 0
    for r in range(n_ret):
        for t0 in range(0, n_tok, m):
            rows = [t * n_ret + r for t in range(t0, min(n_tok, t0 + m))]
            parts = [ix[rp[i]: rp[i + 1]] for i in rows]
            u = len(np.unique(np.concatenate(parts)))
            ukeys += u
            grid += len(rows) * u
    return (float(rp[-1]) / grid if grid else 0.0), ukeys


# ---------------------------------------------------------------------------
# the oracle on the host (cpu_baseline legs)
# ---------------------------------------------------------------------------

def cpu_decode(w, seqs, threads: int, kv=None):
    """Seconds of the oracle for the retrieval rows and local heads of the
    sequences `seqs` of one decode step (indexer keys of the context computed
    untimed).  kv(b, g) gives fp32 K/V of a KV head (default: the workload's)."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    kf = {}
    for b in seqs:
        for g in range(w.Hkv):
            kf[(b, g)] = kv(b, g) if kv else (np.ascontiguousarray(oracle.as_f32(w.k[b][:, g, :])),
                                              np.ascontiguousarray(oracle.as_f32(w.v[b][:, g, :])))
    jobs_kl = [(b, r) for b in seqs for r in range(w.n_ret)]

    def fill(br):
        b, r = br
        return br, oracle.project(kf[(b, w.kv_head(w.ret_heads[r]))][0], w.w_k[r])

    with cf.ThreadPoolExecutor(threads) as ex:
        k_low = dict(ex.map(fill, jobs_kl))

    def ret_job(br):
        b, r = br
        h = w.ret_heads[r]
        K, V = kf[(b, w.kv_head(h))]
        return oracle.retrieval_row(w.q[b, h], K, V, w.w_q[r], w.w_k[r], w.row_pos(b), w.idx_scale,
                                    float(w.top_p[b]), w.attn_scale, k_low=k_low[(b, r)], want_order=False)["sel"].size

    def loc_job(bh):
        b, h = bh
        K, V = kf[(b, w.kv_head(h))]
        return oracle.local_row(w.q[b, h], K, V, w.row_pos(b), w.window, w.sinks, w.attn_scale)[0]

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(ret_job, jobs_kl))
        list(ex.map(loc_job, [(b, h) for b in seqs for h in w.local_heads()]))
    return time.perf_counter() - t0


def cpu_prefill(w, n_rows: int, n_local: int, threads: int):
    """Oracle seconds per retrieval row and per local (row, head) pair of a
    prefill chunk, on seeded samples (rows are independent, so the chunk's
    time scales linearly).  Indexer keys of the context computed untimed."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    g_rng = np.random.default_rng(7)
    heads = sorted({w.kv_head(h) for h in range(w.Hq)})
    kf = {g: (np.ascontiguousarray(oracle.as_f32(w.k[0][:, g, :])),
              np.ascontiguousarray(oracle.as_f32(w.v[0][:, g, :]))) for g in heads}
    with cf.ThreadPoolExecutor(threads) as ex:
        k_low = dict(ex.map(lambda r: (r, oracle.project(kf[w.kv_head(w.ret_heads[r])][0], w.w_k[r])),
                            range(w.n_ret)))
    rows = [(int(t), int(r)) for t, r in zip(g_rng.choice(w.n_tok, n_rows), g_rng.choice(w.n_ret, n_rows))]
    loc = w.local_heads()
    lrows = [(int(t), int(loc[i])) for t, i in zip(g_rng.choice(w.n_tok, n_local), g_rng.choice(len(loc), n_local))]

    def ret_job(tr):
        t, r = tr
        h = w.ret_heads[r]
        K, V = kf[w.kv_head(h)]
        return oracle.retrieval_row(w.q[t, h], K, V, w.w_q[r], w.w_k[r], w.row_pos(t), w.idx_scale,
                                    float(w.top_p[0]), w.attn_scale, k_low=k_low[r], want_order=False)["sel"].size

    def loc_job(th):
        t, h = th
        K, V = kf[w.kv_head(h)]
        return oracle.local_row(w.q[t, h], K, V, w.row_pos(t), w.window, w.sinks, w.attn_scale)[0]

    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(ret_job, rows))
        t1 = time.perf_counter()
        list(ex.map(loc_job, lrows))
        t2 = time.perf_counter()
    return (t1 - t0) / n_rows, (t2 - t1) / n_local


# ---------------------------------------------------------------------------
# decode legs
# ---------------------------------------------------------------------------

def decode_leg(w, args, instances: int, steps: int, warmup: int, fp8: bool = False, dense: bool = True,
               graph: bool = True, tag: str = "", extras: bool = False):
    """One decode step of one layer for the whole batch, eager launches on two
    streams (window attention of the local heads forked after the selection's
    pass over the indexer keys).  Returns a dict of measured figures."""
    import numpy as np
    import torch

    import synth
    import sparse_attention_dim_amd as rtp
    from sparse_attention_dim_amd.paged import PagedCache, rtp_dtype, to_device

    dev = torch.device("cuda:0")
    B, L = w.B, int(w.seq_lens.max())
    lens = w.seq_lens.astype(np.int64)
    if fp8:
        kc, vc, ks, vs = synth.fp8_kv(w)
        k_src, v_src, kdt = kc, vc, "fp8"
        layer = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp.RTP_BF16, w.ret_heads, w.window, w.sinks, w.attn_scale,
                               w.idx_scale, kv_fp8=1, k_scale=ks, v_scale=vs)
    else:
        k_src, v_src, kdt = w.k, w.v, w.dtype
        layer = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp_dtype(w.dtype), w.ret_heads, w.window, w.sinks,
                               w.attn_scale, w.idx_scale)
    inst = []
    for i in range(instances):
        pc = PagedCache(k_src, v_src, w.n_ret, kdt, device=dev, permute_seed=100 + i)
        cache = pc.cache(L)
        q = to_device(w.q, dev)
        w_q, w_k = to_device(w.w_q, dev), to_device(w.w_k, dev)
        top_p = torch.from_numpy(w.top_p.astype(np.float32)).to(dev)
        query = rtp.make_query(q, rtp.RTP_DECODE)
        for b in range(B):
            sid, pos = pc.all_positions(b, dev)
            rtp.indexer_append(layer, cache, w_k, sid, pos)
        rows = B * w.n_ret
        cap = int(sum(int(x) for x in lens)) * w.n_ret
        row_ptr = torch.zeros(rows + 1, dtype=torch.int64, device=dev)
        idx = torch.empty(cap, dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        sel = rtp.make_sel(row_ptr, idx, status)
        ws_sel = torch.empty(rtp.topp_select_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
        ws_sp = torch.empty(rtp.sparse_attn_workspace(layer, cache, query, cap), dtype=torch.uint8, device=dev)
        ws_ret = torch.empty(rtp.decode_attn_workspace(layer, cache, query, cap), dtype=torch.uint8, device=dev)
        ws_win = torch.empty(rtp.window_attn_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
        out = torch.zeros_like(q)
        inst.append(dict(pc=pc, cache=cache, q=q, w_q=w_q, w_k=w_k, top_p=top_p, query=query,
                         sid=torch.arange(B, dtype=torch.int32, device=dev), pos=(pc.seq_lens - 1).to(torch.int32),
                         sel=sel, row_ptr=row_ptr, idx=idx, status=status, ws_sel=ws_sel, ws_sp=ws_sp,
                         ws_ret=ws_ret, ws_win=ws_win, out=out))
    torch.cuda.synchronize()
    log("[bench] %s: %d layer instances resident (%.1f GB allocated)" %
        (tag, instances, torch.cuda.memory_allocated() / 1e9))
    side = torch.cuda.Stream()

    # one call for the step's attention (rtp_decode_attn) for batches of at
    # most 128 retrieval rows with bf16 or fp32 K/V (with bf16, D = 128 its row
    # pass also runs the local heads' window items on its spare CUs); the
    # ragged batch of 64 (384 rows) and FP8 K/V run the separate calls, the
    # window on a second stream beside the selection (measured faster there)
    fused_ok = B * w.n_ret <= 128 and not fp8

    def make_step(I, main, fused=True, window_first=False):
        sel_args = (layer, I["cache"], I["query"], I["w_q"], I["top_p"], I["sel"], I["ws_sel"])
        append = rtp.indexer_append(layer, I["cache"], I["w_k"], I["sid"], I["pos"], stream=main, prepare=True)
        window = rtp.window_attn(layer, I["cache"], I["query"], I["out"], I["ws_win"], stream=side, prepare=True)
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        if fused and fused_ok:
            # the step's indexer-key append, the selection and sparse attention
            # of the retrieval heads and the window attention of the local
            # heads in one call, on one stream
            step_attn = rtp.decode_attn(layer, I["cache"], I["query"], I["w_q"], I["top_p"], I["sel"], I["out"],
                                        I["ws_ret"], w_k=I["w_k"], stream=main, prepare=True)
            return step_attn
        begin = rtp.topp_select_begin(*sel_args, stream=main, prepare=True)
        end = rtp.topp_select_end(*sel_args, stream=main, prepare=True)
        sparse = rtp.sparse_attn_decode(layer, I["cache"], I["query"], I["sel"], I["out"], I["ws_sp"], stream=main,
                                        prepare=True)

        def run():
            if window_first:                             # the window beside the whole selection
                fork.record(main)
                side.wait_event(fork)
                window()
            append()
            begin()
            if not window_first:                         # the window beside the cut and the sparse attention
                fork.record(main)
                side.wait_event(fork)
                window()
            end()
            sparse()
            join.record(side)
            main.wait_event(join)
        return run

    main_stream = torch.cuda.current_stream()
    runs = [make_step(I, main_stream) for I in inst]
    n_i = len(inst)
    for s in range(warmup):
        runs[s % n_i]()
    torch.cuda.synchronize()
    assert all(int(I["status"].item()) == 0 for I in inst), "selection status"

    # per-call breakdown: sequential launches with events between the calls
    calls = ("append", "select", "sparse", "window")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(max(8, steps // 4))]
    for s, e in enumerate(evs):
        I = inst[s % n_i]
        e[0].record()
        rtp.indexer_append(layer, I["cache"], I["w_k"], I["sid"], I["pos"])
        e[1].record()
        rtp.topp_select(layer, I["cache"], I["query"], I["w_q"], I["top_p"], I["sel"], I["ws_sel"])
        e[2].record()
        rtp.sparse_attn_decode(layer, I["cache"], I["query"], I["sel"], I["out"], I["ws_sp"])
        e[3].record()
        rtp.window_attn(layer, I["cache"], I["query"], I["out"], I["ws_win"])
        e[4].record()
    torch.cuda.synchronize()
    per_call = {c: round(float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e3, 2)
                for i, c in enumerate(calls)}
    # the step's attention in one call (rtp_decode_attn: every head)
    for s, e in enumerate(evs):
        I = inst[s % n_i]
        e[0].record()
        rtp.decode_attn(layer, I["cache"], I["query"], I["w_q"], I["top_p"], I["sel"], I["out"], I["ws_ret"],
                        w_k=I["w_k"])
        e[1].record()
    torch.cuda.synchronize()
    per_call["decode_attn"] = round(float(np.median([e[0].elapsed_time(e[1]) for e in evs])) * 1e3, 2)

    # the timed region: exactly `steps` steps between synchronisations
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for s in range(steps):
        runs[s % n_i]()
    b_.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b_) / steps
    # per-step distribution: an event pair around every step (>= 50 steps)
    n_st = max(50, steps)
    pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_st)]
    for s, (e0, e1) in enumerate(pe):
        e0.record()
        runs[s % n_i]()
        e1.record()
    torch.cuda.synchronize()
    step_us = stats([e0.elapsed_time(e1) * 1e3 for e0, e1 in pe])
    # the same step with the selection and the sparse attention as separate
    # calls (rtp_topp_select_begin / _end, rtp_sparse_attn_decode)
    runs2 = [make_step(I, main_stream, fused=False) for I in inst]
    for s in range(warmup):
        runs2[s % n_i]()
    torch.cuda.synchronize()
    a.record()
    for s in range(steps):
        runs2[s % n_i]()
    b_.record()
    torch.cuda.synchronize()
    two_call_us = round(a.elapsed_time(b_) / steps * 1e3, 2)
    window_first_us = None
    if not fused_ok:
        # the separate calls with the window forked before the scoring pass
        runs3 = [make_step(I, main_stream, fused=False, window_first=True) for I in inst]
        for s in range(warmup):
            runs3[s % n_i]()
        torch.cuda.synchronize()
        a.record()
        for s in range(steps):
            runs3[s % n_i]()
        b_.record()
        torch.cuda.synchronize()
        window_first_us = round(a.elapsed_time(b_) / steps * 1e3, 2)

    graph_ms = None
    if graph:
        graphs = []
        for I in inst:
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                make_step(I, torch.cuda.current_stream())()
            graphs.append(gph)
        for s in range(2 * n_i):
            graphs[s % n_i].replay()
        torch.cuda.synchronize()
        a.record()
        for s in range(steps):
            graphs[s % n_i].replay()
        b_.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b_) / steps

    rp = inst[0]["row_ptr"].cpu().numpy()
    n_sel = int(rp[-1])
    sizes = np.diff(rp)
    elt = 1 if fp8 else (2 if w.dtype == "bf16" else 4)
    kv_row = w.D * elt * 2                               # one K row + one V row
    bytes_klow = int(lens.sum()) * w.n_ret * 32
    bytes_sparse = n_sel * kv_row + n_sel * 8
    bytes_win = int(sum(min(w.window + w.sinks, int(l)) for l in lens)) * w.Hkv * kv_row
    step_bytes = bytes_klow + bytes_sparse + bytes_win
    res = {"workload": w.name + ("_fp8kv" if fp8 else ""), "batch": B, "max_context": L,
           "us_per_step": round(ms * 1e3, 2), "step_us": step_us, "two_call_step_us": two_call_us,
           "window_first_step_us": window_first_us,
           "per_call_us": per_call,
           "graph_us": round(graph_ms * 1e3, 2) if graph_ms else None,
           "step_algorithmic_bytes": step_bytes,
           "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "selected_per_row": {"min": int(sizes.min()), "median": int(np.median(sizes)), "max": int(sizes.max()),
                                "total": n_sel}}
    I = inst[0]
    if dense:
        ws_dense = torch.empty(rtp.dense_attn_workspace(layer, I["cache"], I["query"]), dtype=torch.uint8, device=dev)
        dense_out = torch.zeros_like(I["q"])
        for s in range(2):
            rtp.dense_attn(layer, inst[s % n_i]["cache"], inst[s % n_i]["query"], dense_out, ws_dense)
        torch.cuda.synchronize()
        nd = 6
        a.record()
        for s in range(nd):
            J = inst[s % n_i]
            rtp.dense_attn(layer, J["cache"], J["query"], dense_out, ws_dense)
        b_.record()
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b_) / nd
        dense_bytes = int(lens.sum()) * w.Hkv * kv_row
        res.update({"dense_us": round(dense_ms * 1e3, 2),
                    "dense_hbm_frac": round(dense_bytes / (dense_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "speedup_vs_dense": round(dense_ms / ms, 3)})
        del ws_dense
    if extras:
        res["_inst"] = inst
        res["_layer"] = layer
        res["_bytes_klow"] = bytes_klow
    else:
        del inst
        torch.cuda.empty_cache()
    return res


def select_variants(res, w, steps: int):
    """Fixed top-k and the k_max cap on the headline decode instances: the
    selection call's time and its set sizes."""
    import numpy as np
    import torch

    import sparse_attention_dim_amd as rtp

    layer, inst = res["_layer"], res["_inst"]
    out = {}
    for name, kw in (("topk_512", dict(top_k=512)), ("topp_cap_256", dict(k_max=256))):
        lay = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp.RTP_BF16, w.ret_heads, w.window, w.sinks, w.attn_scale,
                             w.idx_scale, k_max=kw.get("k_max", 0))
        calls = []
        for I in inst:
            if "top_k" in kw:
                calls.append(rtp.topk_select(lay, I["cache"], I["query"], I["w_q"], kw["top_k"], I["sel"],
                                             I["ws_sel"], prepare=True))
            else:
                calls.append(rtp.topp_select(lay, I["cache"], I["query"], I["w_q"], I["top_p"], I["sel"],
                                             I["ws_sel"], prepare=True))
        for c in calls:
            c()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for s, (e0, e1) in enumerate(ev):
            e0.record()
            calls[s % len(calls)]()
            e1.record()
        torch.cuda.synchronize()
        rp = inst[(steps - 1) % len(inst)]["row_ptr"].cpu().numpy()
        sz = np.diff(rp)
        out[name] = {"select_us": stats([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]),
                     "selected_per_row": {"min": int(sz.min()), "median": int(np.median(sz)), "max": int(sz.max())}}
    return out


def gqa_variant(res, w, steps: int):
    """The step's attention in one call with and without RTP_FLAG_GQA_SHARED
    (the retrieval heads of one KV head gather the union of their selected
    keys once) on a decode leg's instances: median step time of each, and the
    K/V rows the sparse attention gathers (the union of a group's sets when
    the group's lists together hold at most 8192 keys, which the union pass
    merges; otherwise the lists one after another)."""
    import numpy as np
    import torch

    import sparse_attention_dim_amd as rtp

    inst = res["_inst"]
    I = inst[0]
    out = {}
    for name, flags in (("separate", 0), ("shared", rtp.RTP_FLAG_GQA_SHARED)):
        lay = rtp.make_layer(w.Hq, w.Hkv, w.D, rtp.RTP_BF16, w.ret_heads, w.window, w.sinks, w.attn_scale,
                             w.idx_scale, flags=flags)
        calls = []
        for J in inst:
            ws = torch.empty(rtp.decode_attn_workspace(lay, J["cache"], J["query"], J["sel"].capacity),
                             dtype=torch.uint8, device="cuda")
            J["_ws_gqa"] = ws
            calls.append(rtp.decode_attn(lay, J["cache"], J["query"], J["w_q"], J["top_p"], J["sel"], J["out"], ws,
                                         prepare=True))
        for c in calls:
            c()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for s_, (e0, e1) in enumerate(ev):
            e0.record()
            calls[s_ % len(calls)]()
            e1.record()
        torch.cuda.synchronize()
        out[name + "_step_us"] = stats([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
        for J in inst:
            J.pop("_ws_gqa", None)
    rp = I["row_ptr"].cpu().numpy()
    ix = I["idx"].cpu().numpy()
    total = union = gathered = 0
    for t in range(w.B):
        groups = {}
        for r, h in enumerate(w.ret_heads):
            groups.setdefault(h // (w.Hq // w.Hkv), []).append(ix[rp[t * w.n_ret + r]: rp[t * w.n_ret + r + 1]])
        for sets in groups.values():
            n = sum(len(x) for x in sets)
            u = len(np.unique(np.concatenate(sets)))
            total += n
            union += u
            gathered += u if (len(sets) > 1 and n <= 8192) else n
    kv_row = w.D * 2 * 2
    out.update({"selected_keys": int(total), "union_keys": int(union), "gathered_keys": int(gathered),
                "sparse_kv_bytes_separate": int(total) * kv_row, "sparse_kv_bytes_shared": int(gathered) * kv_row})
    return out


def score_roofline(res, w, steps: int):
    """The dominant kernel: the indexer score pass (k_sel_score), timed live
    with HIP events around back-to-back rtp_indexer_scores calls on the
    stream they run on."""
    import torch

    import sparse_attention_dim_amd as rtp

    layer, inst = res["_layer"], res["_inst"]
    rows = w.B * w.n_ret
    L = int(w.seq_lens.max())
    qlow_buf = torch.empty((rows, 16), dtype=torch.int16, device="cuda")
    score_bufs = [torch.empty((rows, L), dtype=torch.float32, device="cuda") for _ in inst]
    score_calls = [rtp.indexer_scores(layer, J["cache"], J["query"], J["w_q"], qlow_buf, score_bufs[i], prepare=True)
                   for i, J in enumerate(inst)]
    for c in score_calls:
        c()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for s in range(steps):
        score_calls[s % len(inst)]()
    k1.record()
    torch.cuda.synchronize()
    k_ms = k0.elapsed_time(k1) / steps
    # algorithmic bytes of the call: the indexer keys read (32 B per (row,
    # key)) and the scores it returns (4 B per (row, key))
    alg = res["_bytes_klow"] + res["_bytes_klow"] // 8
    achieved = alg / (k_ms * 1e-3) / 1e9
    del score_bufs
    return {"kernel": "k_sel_score<bf16, scores only> (rtp_indexer_scores, decode)", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_counters(),
            "algorithmic_bytes": alg, "algorithmic_read_bytes": res["_bytes_klow"],
            "avg_launch_us": round(k_ms * 1e3, 2)}


# ---------------------------------------------------------------------------
# prefill legs
# ---------------------------------------------------------------------------

def prefill_leg(cfg: int, steps: int, run_mean: int | None = None, dense: bool = True, cpu_rows: int = 0):
    """One prefill chunk of one layer: the chunk's indexer append, selection
    and sparse prefill on the main stream, window prefill on a second stream;
    dense causal attention of the same chunk for comparison.  run_mean: the
    workload's generator with another mean run length of query rows on one
    cluster (1: independent rows, the stress case of the union tiles)."""
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
    c_sid = sid[w.chunk_pos0:].contiguous()
    c_pos = pos[w.chunk_pos0:].contiguous()
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
    main = torch.cuda.current_stream()
    append = rtp.indexer_append(layer, cache, w_k, c_sid, c_pos, stream=main, prepare=True)
    select = rtp.topp_select(layer, cache, query, w_q, top_p, sel, ws_sel, stream=main, prepare=True)
    sparse = rtp.sparse_attn_prefill(layer, cache, query, sel, out, ws_sp, stream=main, prepare=True)
    window = rtp.window_attn(layer, cache, query, out, ws_win, stream=side, prepare=True)

    def step():
        append()                                          # a1: the chunk's indexer keys
        side.wait_stream(main)
        window()                                          # a6 on the second stream
        select()                                          # a2-a4
        sparse()                                          # a5
        main.wait_stream(side)

    for _ in range(3):
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
    pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in pe:
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    step_stats = stats([e0.elapsed_time(e1) for e0, e1 in pe])
    # per-call times, sequential launches
    t_app, t_sel, t_sp, t_win = [], [], [], []
    for _ in range(max(5, steps // 5)):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record()
        rtp.indexer_append(layer, cache, w_k, c_sid, c_pos)
        e[1].record()
        rtp.topp_select(layer, cache, query, w_q, top_p, sel, ws_sel)
        e[2].record()
        rtp.sparse_attn_prefill(layer, cache, query, sel, out, ws_sp)
        e[3].record()
        rtp.window_attn(layer, cache, query, out, ws_win)
        e[4].record()
        torch.cuda.synchronize()
        for lst, i in ((t_app, 0), (t_sel, 1), (t_sp, 2), (t_win, 3)):
            lst.append(e[i].elapsed_time(e[i + 1]))
    rp = row_ptr.cpu().numpy()
    sizes = np.diff(rp)
    n_sel = int(rp[-1])
    useful, ukeys = union_useful(rp, idx[:n_sel].cpu().numpy(), w.n_tok, w.n_ret)
    dense_ms = None
    if dense:
        ws_d = torch.empty(rtp.dense_attn_workspace(layer, cache, query), dtype=torch.uint8, device=dev)
        dout = torch.zeros_like(q)
        rtp.dense_attn(layer, cache, query, dout, ws_d)
        torch.cuda.synchronize()
        nd = 2
        a.record()
        for _ in range(nd):
            rtp.dense_attn(layer, cache, query, dout, ws_d)
        b.record()
        torch.cuda.synchronize()
        dense_ms = a.elapsed_time(b) / nd
        del ws_d
    f_pair = 4 * w.D                                      # QK and PV, 2 D flops each per (query head, key)
    sp_flops = n_sel * f_pair
    win_pairs = sum(min(w.window + w.sinks, w.row_pos(t) + 1) for t in range(w.n_tok)) * (w.Hq - w.n_ret)
    dense_pairs = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.Hq
    sel_pairs = sum(w.row_pos(t) + 1 for t in range(w.n_tok)) * w.n_ret
    sel_t, sp_t, win_t = (float(np.median(x)) for x in (t_sel, t_sp, t_win))
    res = {
        "workload": w.name, "chunk_rows": w.n_tok, "context": L, "top_p": float(w.top_p[0]),
        "tokens_per_s": round(w.n_tok / (step_ms * 1e-3), 1), "step_ms": round(step_ms, 3),
        "step_ms_stats": step_stats,
        "append_ms": round(float(np.median(t_app)), 4), "select_ms": round(sel_t, 3), "sparse_ms": round(sp_t, 3),
        "window_ms": round(win_t, 3),
        "selected_per_row": {"min": int(sizes.min()), "median": int(np.median(sizes)),
                             "mean": round(float(sizes.mean()), 1), "max": int(sizes.max())},
        # selection: bound by the softmax weight of every (row, key) pair (one
        # transcendental each) at v_exp_f32's rate
        "select_roofline": {"bound": "alu", "pairs": sel_pairs,
                            "achieved": round(sel_pairs / (sel_t * 1e-3) / 1e12, 3),
                            "peak": round(EXP_PEAK_PER_S / 1e12, 3), "unit": "T exp/s",
                            "frac": round(sel_pairs / (sel_t * 1e-3) / EXP_PEAK_PER_S, 4)},
        # sparse tiles: bound by the K/V gather of the tiles' union keys
        "sparse_roofline": {"bound": "hbm", "union_keys": ukeys, "bytes": ukeys * w.D * 2 * 2,
                            "achieved": round(ukeys * w.D * 4 / (sp_t * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(ukeys * w.D * 4 / (sp_t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "sparse_tflops": round(sp_flops / (sp_t * 1e-3) / 1e12, 2),
        "sparse_mfma_frac": round(sp_flops / (sp_t * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 5),
        "sparse_union_useful": round(useful, 4),
        "window_tflops": round(win_pairs * f_pair / (win_t * 1e-3) / 1e12, 2),
        "window_mfma_frac": round(win_pairs * f_pair / (win_t * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
    }
    if dense_ms is not None:
        res.update({"dense_ms": round(dense_ms, 3),
                    "dense_tflops": round(dense_pairs * f_pair / (dense_ms * 1e-3) / 1e12, 2),
                    "speedup_vs_dense": round(dense_ms / step_ms, 3)})
    del pc, cache, idx, ws_sel, ws_sp, ws_win
    torch.cuda.empty_cache()
    if cpu_rows:
        threads = min(os.cpu_count() or 1, 16)
        t_row, t_loc = cpu_prefill(w, cpu_rows, cpu_rows * 4, threads)
        est = t_row * w.n_tok * w.n_ret + t_loc * w.n_tok * len(w.local_heads())
        res["cpu_baseline"] = {"value": round(w.n_tok / est, 2), "unit": "tokens/s/layer", "cores": threads,
                               "kind": "oracle",
                               "sample": "%d retrieval rows and %d local (row, head) pairs of the chunk, seeded; "
                                         "scaled linearly to its %d x %d retrieval rows and %d x %d local pairs"
                                         % (cpu_rows, cpu_rows * 4, w.n_tok, w.n_ret, w.n_tok,
                                            len(w.local_heads()))}
    return res


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--cpu-seqs", type=int, default=8)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true", help="report HIP graph replays as the headline value")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill legs")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged batch-64 decode leg")
    ap.add_argument("--no-variants", action="store_true", help="skip the FP8 / top-k / cap / fp32 decode legs")
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--only", choices=["decode", "prefill128k", "prefill1m", "ragged"],
                    help="run one leg only (profiling); prints its dict")
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

    rtp.load()
    threads = min(os.cpu_count() or 1, 16)

    def calibration_copy():
        # a copy of known size for the HBM counter runs (1 GiB read, 1 GiB
        # written): the last dispatch of every run
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    if args.only in ("prefill128k", "prefill1m"):
        r = prefill_leg(3 if args.only == "prefill128k" else 4, args.prefill_steps, dense=False)
        calibration_copy()
        print(json.dumps(r))
        return

    def ragged_leg():
        # about a minute of host time to draw (its numpy steps hold the
        # interpreter lock, which would slow the launches of a leg timed
        # beside it), so it runs on its own, first
        t0 = time.time()
        w5 = synth.config(5)
        log("[bench] generated %s in %.1fs" % (w5.name, time.time() - t0))
        r5 = decode_leg(w5, args, 1, max(20, args.steps // 2), 4, graph=False, tag="ragged")
        r5["target_us_60pct_hbm"] = round(r5["step_algorithmic_bytes"] / (0.6 * HBM_PEAK_GBS * 1e9) * 1e6, 1)
        if not args.no_cpu:
            seqs = [int(x) for x in np.random.default_rng(5).choice(w5.B, 4, replace=False)]
            dt = cpu_decode(w5, seqs, threads)
            share = sum(int(w5.seq_lens[b]) for b in seqs) / float(w5.seq_lens.sum())
            r5["cpu_baseline"] = {"value": round(dt / share * 1e6, 1), "unit": "µs/step/layer", "cores": threads,
                                  "kind": "oracle",
                                  "sample": "retrieval rows and local heads of 4 seeded sequences of the 64 "
                                            "(%.1f%% of the context keys), scaled by their share" % (100 * share)}
        del w5
        return r5

    if args.only == "ragged":
        r = ragged_leg()
        calibration_copy()
        print(json.dumps(r))
        return
    ragged_res = None if (args.no_ragged or args.only) else ragged_leg()

    t0 = time.time()
    w = synth.config(2)
    log("[bench] generated %s in %.1fs" % (w.name, time.time() - t0))
    head = decode_leg(w, args, args.instances, args.steps, args.warmup, extras=True, tag="decode")
    roof = score_roofline(head, w, args.steps)
    variants = {} if args.no_variants else select_variants(head, w, max(50, args.steps))
    if not args.no_variants:
        variants["gqa_shared_gathers"] = {"independent_clusters": gqa_variant(head, w, max(50, args.steps))}
    for k in ("_inst", "_layer", "_bytes_klow"):
        head.pop(k, None)
    torch.cuda.empty_cache()
    if not args.no_variants:
        # the same shapes with the retrieval heads of a KV head sharing their
        # planted cluster (overlapping sets): the bytes a shared gather saves
        ws_ = synth.cluster_decode(seed=1002, shared_kv=True, name="decode_bf16_B8_L131072_shared_clusters")
        rs = decode_leg(ws_, args, 2, args.steps, args.warmup, dense=False, graph=False, extras=True,
                        tag="decode shared clusters")
        variants["gqa_shared_gathers"]["shared_clusters"] = gqa_variant(rs, ws_, max(50, args.steps))
        del rs, ws_
        torch.cuda.empty_cache()
    if args.only == "decode":
        calibration_copy()
        print(json.dumps(dict(head, roofline=roof, variants=variants)))
        return

    cpu = None
    if not args.no_cpu:
        ns = min(args.cpu_seqs, w.B)
        dt = cpu_decode(w, list(range(ns)), threads)
        cpu = {"value": round(dt / ns * w.B * 1e6, 1), "unit": "µs/step/layer", "cores": threads, "kind": "oracle",
               "sample": "retrieval rows and local heads of %d of the %d sequences of one decode step "
                         "(indexer keys of the context precomputed untimed), scaled x%d to the batch"
                         % (ns, w.B, w.B // ns)}

    if not args.no_variants:
        variants["fp8_kv"] = decode_leg(w, args, args.instances, args.steps, args.warmup, fp8=True, dense=False,
                                        graph=False, tag="decode FP8 K/V")
        # window-only ring: KV heads none of whose query heads retrieve keep
        # sinks + window instead of the whole context
        serves = {h // (w.Hq // w.Hkv) for h in w.ret_heads}
        n_ring = w.Hkv - len(serves)
        per_head = int(w.seq_lens.sum()) * w.D * 2 * 2
        ring_keys = 256 * (1 + (w.window + 255 + 255) // 256)
        variants["ring_layout"] = {"kv_heads_full": len(serves), "kv_heads_ring": n_ring,
                                   "kv_bytes_full_cache": per_head * w.Hkv,
                                   "kv_bytes_ring_layout": per_head * len(serves) + w.B * ring_keys * w.D * 4 * n_ring}
        w1 = synth.config(1)
        variants["decode_f32_needles"] = decode_leg(w1, args, args.instances, args.steps, args.warmup, graph=False,
                                                    tag="decode fp32")
    del w

    prefill = None
    if not args.no_prefill:
        prefill = {"128k": prefill_leg(3, args.prefill_steps, cpu_rows=0 if args.no_cpu else 48),
                   "1m": prefill_leg(4, args.prefill_steps, cpu_rows=0 if args.no_cpu else 16),
                   "128k_independent_rows": prefill_leg(3, args.prefill_steps, run_mean=1, dense=False)}

    calibration_copy()
    ms = (head["graph_us"] if args.graph else head["us_per_step"]) / 1e3
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
        "config": {"workload": head["workload"], "kind": "decode", "batch": head["batch"],
                   "context": head["max_context"], "q_heads": 32, "kv_heads": 8, "head_dim": 128,
                   "retrieval_heads": 6, "top_p": 0.95, "window": 2048, "sinks": 64,
                   "layer_instances": args.instances},
        "roofline": roof,
        "cpu_baseline": cpu,
        "launch": "hip_graph" if args.graph else "eager, two streams",
        "pages": "permuted",
        "decode": head,
        "decode_ragged": ragged_res,
        "variants": variants,
        "prefill": prefill,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
