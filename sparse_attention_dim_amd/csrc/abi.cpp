// abi.cpp -- the extern "C" entry points of librtp: host-side argument checks,
// workspace layout and kernel launches on the caller's stream.  No entry point
// allocates device memory or synchronises the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/rtp.h"
#include "device.hpp"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

rtp_status fail(rtp_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

rtp_status ok() {
    g_err.clear();
    return RTP_OK;
}

rtp_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(RTP_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Scratch of rtp_topp_select_noalloc: a static device array, one copy per GPU
// (each GPU the library runs on holds it until the process ends).  In host
// code `scratch` only names the symbol; its device address on the current
// GPU comes from hipGetSymbolAddress, taken once per device and kept.
static __device__ __align__(256) unsigned char scratch[RTP_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

constexpr int kMaxLen = RTP_MAX_LEN;      // longest supported context: fixed-point masses of every key fit 2^63
constexpr int kMaxDecodeRows = 4096;      // decode rows (batch * num_ret) of the sparse kernel
constexpr int kWinSplit = 64;             // keys per workgroup, local-head decode (VALU kernel)
constexpr int kWinSplitMfma = 128;        // keys per workgroup, local-head decode (bf16 MFMA kernel, D = 128)
constexpr int kDenseSplit = 1024;         // keys per workgroup, dense decode

int win_split(const rtp_layer* L, int dense) {
    if (dense) return kDenseSplit;
    return (L->dtype == RTP_BF16 && L->head_dim == 128 && !L->kv_fp8) ? kWinSplitMfma : kWinSplit;
}

// bf16 D = 128 chunks whose K/V are bf16 run on the MFMA tile kernels
bool mfma_chunk(const rtp_layer* L) { return L->dtype == RTP_BF16 && L->head_dim == 128 && !L->kv_fp8; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

rtp_status check_layer(const rtp_layer* L) {
    if (!L) return fail(RTP_EINVAL, "layer is NULL");
    if (L->num_q_heads < 1 || L->num_kv_heads < 1 || L->num_q_heads % L->num_kv_heads)
        return fail(RTP_EINVAL, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    L->num_q_heads, L->num_kv_heads);
    if (L->num_q_heads > 256) return fail(RTP_EUNSUPPORTED, "num_q_heads > 256");
    if (L->num_q_heads / L->num_kv_heads > 8) return fail(RTP_EUNSUPPORTED, "more than 8 query heads per KV head");
    if (L->head_dim != 64 && L->head_dim != 128)
        return fail(RTP_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", L->head_dim);
    if (L->dtype != RTP_F32 && L->dtype != RTP_BF16) return fail(RTP_EINVAL, "dtype %d", L->dtype);
    if (L->num_ret < 1 || L->num_ret > RTP_MAX_RET)
        return fail(RTP_EINVAL, "num_ret %d out of [1, %d]", L->num_ret, RTP_MAX_RET);
    for (int r = 0; r < L->num_ret; ++r) {
        const int h = L->ret_heads[r];
        if (h < 0 || h >= L->num_q_heads) return fail(RTP_EINVAL, "ret_heads[%d] = %d out of range", r, h);
        if (r && h <= L->ret_heads[r - 1]) return fail(RTP_EINVAL, "ret_heads must be strictly ascending");
    }
    if (L->window < 1) return fail(RTP_EINVAL, "window %d < 1", L->window);
    if (L->num_sinks < 0) return fail(RTP_EINVAL, "num_sinks %d < 0", L->num_sinks);
    if (!(L->attn_scale > 0.0f) || !std::isfinite(L->attn_scale)) return fail(RTP_EINVAL, "attn_scale");
    if (!(L->idx_scale > 0.0f) || !std::isfinite(L->idx_scale)) return fail(RTP_EINVAL, "idx_scale");
    if (L->k_max < 0) return fail(RTP_EINVAL, "k_max %d < 0", L->k_max);
    if (L->flags & ~(RTP_FLAG_EXACT_MASS | RTP_FLAG_GQA_SHARED)) return fail(RTP_EINVAL, "unknown flags 0x%x", L->flags);
    if (L->kv_fp8 != 0 && L->kv_fp8 != 1) return fail(RTP_EINVAL, "kv_fp8 %d", L->kv_fp8);
    if (L->kv_fp8) {
        if (L->dtype != RTP_BF16) return fail(RTP_EUNSUPPORTED, "FP8 K/V needs dtype RTP_BF16");
        if (!(L->k_scale > 0.0f) || !std::isfinite(L->k_scale) || !(L->v_scale > 0.0f) || !std::isfinite(L->v_scale))
            return fail(RTP_EINVAL, "FP8 scales must be finite and > 0");
    }
    return RTP_OK;
}

rtp_status check_cache(const rtp_cache* C) {
    if (!C) return fail(RTP_EINVAL, "cache is NULL");
    if (!C->k || !C->v || !C->k_low || !C->block_table || !C->seq_lens)
        return fail(RTP_EINVAL, "cache has a NULL pointer");
    if (C->batch < 1) return fail(RTP_EINVAL, "batch %d < 1", C->batch);
    if (C->max_seq_len < 1 || C->max_seq_len > kMaxLen)
        return fail(RTP_EUNSUPPORTED, "max_seq_len %d out of [1, %d]", C->max_seq_len, kMaxLen);
    if (C->max_blocks < 1 || (int64_t)C->max_blocks * RTP_BLOCK < C->max_seq_len)
        return fail(RTP_EINVAL, "max_blocks %d cannot hold max_seq_len %d", C->max_blocks, C->max_seq_len);
    if (C->k_ring && (!C->v_ring || !C->ring_table || C->ring_pages < 2))
        return fail(RTP_EINVAL, "ring: needs v_ring, ring_table and ring_pages >= 2");
    return RTP_OK;
}

// The ring holds every key the call's local heads need.
rtp_status check_ring_window(const rtp_layer* L, const rtp_cache* C, const rtp_query* Q) {
    if (!C->k_ring) return RTP_OK;
    if (L->num_sinks > RTP_BLOCK) return fail(RTP_EINVAL, "ring: num_sinks %d > %d", L->num_sinks, RTP_BLOCK);
    const int64_t span = (int64_t)L->window + 255 + (Q->kind == RTP_CHUNK ? Q->n_tok - 1 : 0);
    if ((int64_t)(C->ring_pages - 1) * RTP_BLOCK < span)
        return fail(RTP_EINVAL, "ring of %d pages cannot hold a window span of %lld positions", C->ring_pages,
                    (long long)span);
    return RTP_OK;
}

rtp_status check_query(const rtp_cache* C, const rtp_query* Q) {
    if (!Q) return fail(RTP_EINVAL, "query is NULL");
    if (!Q->q) return fail(RTP_EINVAL, "query q is NULL");
    if (Q->n_tok < 1) return fail(RTP_EINVAL, "n_tok %d < 1", Q->n_tok);
    if (Q->kind == RTP_DECODE) {
        if (Q->n_tok != C->batch) return fail(RTP_EINVAL, "decode n_tok %d != batch %d", Q->n_tok, C->batch);
    } else if (Q->kind == RTP_CHUNK) {
        if (Q->seq < 0 || Q->seq >= C->batch) return fail(RTP_EINVAL, "chunk seq %d out of range", Q->seq);
        if (Q->pos0 < 0 || (int64_t)Q->pos0 + Q->n_tok > C->max_seq_len)
            return fail(RTP_EINVAL, "chunk rows [%d, %d) exceed max_seq_len %d", Q->pos0, Q->pos0 + Q->n_tok,
                        C->max_seq_len);
    } else {
        return fail(RTP_EINVAL, "query kind %d", Q->kind);
    }
    return RTP_OK;
}

rtp_status check_all(const rtp_layer* L, const rtp_cache* C, const rtp_query* Q) {
    rtp_status s = check_layer(L);
    if (s) return s;
    if ((s = check_cache(C))) return s;
    return check_query(C, Q);
}

rtp::Geo make_geo(const rtp_layer* L, const rtp_cache* C, const rtp_query* Q) {
    rtp::Geo g;
    std::memset(&g, 0, sizeof g);
    g.Hq = L->num_q_heads;
    g.Hkv = L->num_kv_heads;
    g.D = L->head_dim;
    g.group = g.Hq / g.Hkv;
    g.n_ret = L->num_ret;
    for (int r = 0; r < L->num_ret; ++r) {
        g.ret_heads[r] = L->ret_heads[r];
        g.is_ret[L->ret_heads[r]] = 1;
    }
    g.window = L->window;
    g.sinks = L->num_sinks;
    g.attn_scale = L->attn_scale;
    g.idx_scale = L->idx_scale;
    g.sel_k = 0;
    g.k_max = L->k_max;
    g.flags = L->flags;
    g.kv_fp8 = L->kv_fp8;
    g.k_scale = L->kv_fp8 ? L->k_scale : 1.0f;
    g.v_scale = L->kv_fp8 ? L->v_scale : 1.0f;
    if (Q) {
        g.kind = Q->kind;
        g.seq = Q->seq;
        g.pos0 = Q->pos0;
        g.n_tok = Q->n_tok;
    }
    g.batch = C->batch;
    g.max_blocks = C->max_blocks;
    g.max_seq_len = C->max_seq_len;
    g.block_table = C->block_table;
    g.seq_lens = C->seq_lens;
    // KV layout: with a ring, the KV heads none of whose query heads
    // retrieve live in it; the rest keep their pages in k/v
    int serves[256] = {0};
    for (int r = 0; r < L->num_ret; ++r) serves[L->ret_heads[r] / g.group] = 1;
    int n_pool = 0, n_ring = 0;
    for (int kv = 0; kv < g.Hkv; ++kv) {
        const bool ring = C->k_ring && !serves[kv];
        g.kv_ring[kv] = ring;
        g.kv_slot[kv] = (uint8_t)(ring ? n_ring++ : n_pool++);
    }
    g.pool_heads = n_pool;
    g.ring_heads = n_ring;
    g.ring_pages = C->k_ring ? C->ring_pages : 0;
    g.ring_table = C->ring_table;
    g.k_ring = C->k_ring;
    g.v_ring = C->v_ring;
    return g;
}

// keys of the longest row of the call
int64_t max_keys(const rtp_cache* C, const rtp_query* Q) {
    return Q->kind == RTP_DECODE ? C->max_seq_len : (int64_t)Q->pos0 + Q->n_tok;
}

// ---- selection workspace ----------------------------------------------------

constexpr size_t kScoreBudget = (size_t)4 << 30;   // bytes of scores per row group

struct SelPlan {
    int rows_total, group_rows, nchunk, ucap;
    int64_t lpad;
    size_t off_scores, off_cmax, off_qlow, off_chist, off_ccnt, off_st, off_sel, off_ubuf, off_kmask, off_flist, total;
};

// Prefill chunks in bf16 take the tiled selection (the rows of one retrieval
// head share every indexer-key tile); decode rows and fp32 chunks take the
// per-row passes.
bool tiled_select(const rtp_layer* L, const rtp_query* Q) {
    return Q->kind == RTP_CHUNK && L->dtype == RTP_BF16;
}

SelPlan plan_select(const rtp_layer* L, const rtp_cache* C, const rtp_query* Q) {
    SelPlan p;
    p.rows_total = Q->n_tok * L->num_ret;
    const int64_t keys = max_keys(C, Q);
    p.nchunk = (int)((keys + rtp::kChunk - 1) / rtp::kChunk);
    p.lpad = (int64_t)p.nchunk * rtp::kChunk;
    p.ucap = (int)std::min<int64_t>(rtp::kCandG, p.lpad);
    const size_t per_row =
        (size_t)p.lpad * 4 + (size_t)p.lpad / 8 + (size_t)p.nchunk * (4 + 4 + rtp::kCB * 12 + rtp::kFl * 8) +
        (size_t)p.ucap * 12 +
        1024;
    const int64_t by_budget = std::max<int64_t>(1, (int64_t)(kScoreBudget / per_row));
    p.group_rows = (int)std::min<int64_t>({(int64_t)p.rows_total, by_budget, (int64_t)65535});
    const size_t G = (size_t)p.group_rows;
    size_t o = 0;
    p.off_scores = o; o = align256(o + G * (size_t)p.lpad * 4);
    p.off_cmax = o; o = align256(o + G * (size_t)p.nchunk * 4);
    p.off_qlow = o; o = align256(o + G * 16 * 2);
    p.off_chist = o; o = align256(o + G * (size_t)p.nchunk * rtp::kCB * 8);
    p.off_ccnt = o; o = align256(o + G * (size_t)p.nchunk * rtp::kCB * 4);
    p.off_st = o; o = align256(o + G * sizeof(rtp::RowState));
    p.off_sel = o; o = align256(o + G * (size_t)p.ucap * 4);
    p.off_ubuf = o; o = align256(o + G * (size_t)p.ucap * 8);
    p.off_kmask = o; o = align256(o + G * (size_t)p.lpad / 8);
    p.off_flist = o; o = align256(o + G * (size_t)p.nchunk * rtp::kFl * 8);
    p.total = o;
    return p;
}

rtp::SelWs sel_ws(const SelPlan& p, char* base) {
    rtp::SelWs w;
    w.scores = (float*)(base + p.off_scores);
    w.score_ld = p.lpad;
    w.cmax = (uint32_t*)(base + p.off_cmax);
    w.qlow = (uint16_t*)(base + p.off_qlow);
    w.chist = (unsigned long long*)(base + p.off_chist);
    w.st = (rtp::RowState*)(base + p.off_st);
    w.sel = (uint32_t*)(base + p.off_sel);
    w.ubuf = (unsigned long long*)(base + p.off_ubuf);
    w.ccnt = (unsigned*)(base + p.off_ccnt);
    w.kmask = (unsigned long long*)(base + p.off_kmask);
    w.flist = (unsigned long long*)(base + p.off_flist);
    w.nchunk = p.nchunk;
    w.rows = p.group_rows;
    w.ucap = p.ucap;
    return w;
}

// ---- decode attention workspaces --------------------------------------------

int64_t sparse_max_items(const rtp_layer* L, const rtp_query* Q, int64_t capacity) {
    const int64_t rows = (int64_t)Q->n_tok * L->num_ret;
    return rows + capacity / rtp::kSparseItem + 1;
}

int win_keys(const rtp_layer* L, const rtp_cache* C, int dense) {
    if (dense) return C->max_seq_len;
    return (int)std::min<int64_t>((int64_t)L->window + L->num_sinks, C->max_seq_len);
}

size_t win_ws_bytes(const rtp_layer* L, const rtp_cache* C, const rtp_query* Q, int dense) {
    if (Q->kind == RTP_CHUNK) return 0;     // the prefill kernel needs no workspace
    const int split = win_split(L, dense);
    const int nsplit = (win_keys(L, C, dense) + split - 1) / split;
    return align256((size_t)C->batch * L->num_q_heads * nsplit * (L->head_dim + 2) * 4);
}

rtp_status window_like(const rtp_layer* L, const rtp_cache* C, const rtp_query* Q, void* out, void* ws,
                       size_t ws_bytes, void* stream, int dense) {
    rtp_status s = check_all(L, C, Q);
    if (s) return s;
    if (!out) return fail(RTP_EINVAL, "out is NULL");
    if (dense && C->k_ring) return fail(RTP_EINVAL, "dense attention needs every key: the cache has a ring");
    if ((s = check_ring_window(L, C, Q))) return s;
    if (Q->kind == RTP_CHUNK) {
        if (!mfma_chunk(L))
            return fail(RTP_EUNSUPPORTED, "chunked %s attention is built for bf16 K/V, head_dim 128",
                        dense ? "dense" : "window");
        rtp::Geo g = make_geo(L, C, Q);
        g.n_hlist = 0;
        for (int h = 0; h < L->num_q_heads; ++h)
            if (dense || !g.is_ret[h]) g.hlist[g.n_hlist++] = h;
        return hip_status(rtp::launch_prefill_attn(g, Q->q, C->k, C->v, out, dense, (hipStream_t)stream),
                          dense ? "dense prefill launch" : "window prefill launch");
    }
    const size_t need = win_ws_bytes(L, C, Q, dense);
    if (!ws || ws_bytes < need) return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
    const rtp::Geo g = make_geo(L, C, Q);
    const int split = win_split(L, dense);
    const int nsplit = (win_keys(L, C, dense) + split - 1) / split;
    return hip_status(rtp::launch_window_decode(g, Q->q, C->k, C->v, out, (float*)ws, nsplit, split, dense,
                                                L->dtype, (hipStream_t)stream),
                      dense ? "dense decode launch" : "window decode launch");
}

}  // namespace

extern "C" {

int rtp_version(void) { return RTP_VERSION; }

const char* rtp_last_error(void) { return g_err.c_str(); }

rtp_status rtp_indexer_append(const rtp_layer* layer, const rtp_cache* cache, const void* w_k,
                              const int32_t* seq_id, const int32_t* pos, int32_t n, void* stream) {
    rtp_status s = check_layer(layer);
    if (s) return s;
    if ((s = check_cache(cache))) return s;
    if (n < 0) return fail(RTP_EINVAL, "n %d < 0", n);
    if (n == 0) return ok();
    if (!w_k || !seq_id || !pos) return fail(RTP_EINVAL, "NULL w_k / seq_id / pos");
    const rtp::Geo g = make_geo(layer, cache, nullptr);
    return hip_status(rtp::launch_indexer_append(g, cache->k, cache->k_low, w_k, seq_id, pos, n, layer->dtype,
                                                 (hipStream_t)stream),
                      "indexer append launch");
}

rtp_status rtp_kv_append(const rtp_layer* layer, const rtp_cache* cache, const void* k_new, const void* v_new,
                         const void* w_k, const int32_t* seq_id, const int32_t* pos, int32_t n, void* stream) {
    rtp_status s = check_layer(layer);
    if (s) return s;
    if ((s = check_cache(cache))) return s;
    if (n < 0) return fail(RTP_EINVAL, "n %d < 0", n);
    if (n == 0) return ok();
    if (!k_new || !v_new || !w_k || !seq_id || !pos) return fail(RTP_EINVAL, "NULL k_new / v_new / w_k / seq_id / pos");
    if (((uintptr_t)k_new | (uintptr_t)v_new) & 15) return fail(RTP_EINVAL, "k_new / v_new not 16-byte aligned");
    const rtp::Geo g = make_geo(layer, cache, nullptr);
    return hip_status(rtp::launch_kv_append(g, k_new, v_new, const_cast<void*>(cache->k), const_cast<void*>(cache->v),
                                            cache->k_low, w_k, seq_id, pos, n, layer->dtype, (hipStream_t)stream),
                      "kv append launch");
}

size_t rtp_topp_select_workspace(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query) {
    if (check_all(layer, cache, query)) return 0;
    if (tiled_select(layer, query))
        return rtp::chunk_select_ws_bytes(query->n_tok * layer->num_ret, layer->num_ret, query->pos0 + query->n_tok);
    return plan_select(layer, cache, query).total;
}

size_t rtp_topp_select_workspace_min(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query) {
    if (check_all(layer, cache, query)) return 0;
    if (tiled_select(layer, query))
        return rtp::chunk_select_head_bytes(query->n_tok * layer->num_ret, layer->num_ret,
                                            query->pos0 + query->n_tok);
    return plan_select(layer, cache, query).total;
}

// Device address of the current GPU's scratch array (looked up on its first use).
rtp_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RTP_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(RTP_EUNSUPPORTED, "device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(RTP_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return RTP_OK;
}

// phase: 0 the whole selection, 1 the scoring pass of the first row group
// (when every row fits one group), 2 the rest.  top_k > 0: fixed top-k.
static rtp_status topp_select_phase(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                    const void* w_q, const float* top_p, const rtp_sel* sel, void* workspace,
                                    size_t workspace_bytes, void* stream, int phase, int top_k) {
    rtp_status s = check_all(layer, cache, query);
    if (s) return s;
    if (!w_q || (!top_p && top_k <= 0)) return fail(RTP_EINVAL, "NULL w_q / top_p");
    if (!sel || !sel->row_ptr || !sel->status || (sel->capacity > 0 && !sel->idx) || sel->capacity < 0)
        return fail(RTP_EINVAL, "bad selection buffers");
    rtp::Geo g = make_geo(layer, cache, query);
    g.sel_k = top_k;
    rtp::SelOut out{sel->row_ptr, sel->idx, sel->capacity, sel->status};
    if (tiled_select(layer, query)) {
        const size_t need = rtp::chunk_select_head_bytes(query->n_tok * layer->num_ret, layer->num_ret,
                                                         query->pos0 + query->n_tok);
        if (!workspace || workspace_bytes < need)
            return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
        if (phase == 1) return ok();
        return hip_status(rtp::launch_chunk_select(g, query->q, w_q, (const uint16_t*)cache->k_low, top_p,
                                                   workspace, workspace_bytes, out, (hipStream_t)stream),
                          "chunk select launch");
    }
    const SelPlan p = plan_select(layer, cache, query);
    if (!workspace || workspace_bytes < p.total)
        return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, p.total);
    rtp::SelWs w = sel_ws(p, (char*)workspace);
    const bool one_group = p.group_rows >= p.rows_total;
    for (int row0 = 0; row0 < p.rows_total; row0 += p.group_rows) {
        w.rows = std::min(p.group_rows, p.rows_total - row0);
        int stage = rtp::kSelAll;
        if (phase == 1) {
            if (!one_group) break;
            stage = rtp::kSelScorePass;
        } else if (phase == 2 && one_group) {
            stage = rtp::kSelFinish;
        }
        hipError_t e = rtp::launch_select(g, query->q, w_q, (const uint16_t*)cache->k_low, top_p, row0, w, out,
                                          p.rows_total, layer->dtype, stage, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e, "top-p select launch");
    }
    return ok();
}

rtp_status rtp_topp_select(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                           const void* w_q, const float* top_p, const rtp_sel* sel, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return topp_select_phase(layer, cache, query, w_q, top_p, sel, workspace, workspace_bytes, stream, 0, 0);
}

rtp_status rtp_topp_select_noalloc(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                   const void* w_q, const float* top_p, const rtp_sel* sel, void* stream) {
    rtp_status s = check_all(layer, cache, query);
    if (s) return s;
    constexpr size_t cap = (size_t)RTP_NOALLOC_SCRATCH_BYTES;
    size_t bytes;
    if (tiled_select(layer, query)) {
        // the chunk path takes any workspace from its minimum up: the rows
        // whose candidate set misses the smaller pool take the radix levels
        const int rows = query->n_tok * layer->num_ret, keys = query->pos0 + query->n_tok;
        const size_t low = rtp::chunk_select_head_bytes(rows, layer->num_ret, keys);
        if (low > cap)
            return fail(RTP_EWORKSPACE, "selection needs %zu bytes of scratch, more than the %zu of the static array",
                        low, cap);
        bytes = std::min(cap, rtp::chunk_select_ws_bytes(rows, layer->num_ret, keys));
    } else {
        bytes = plan_select(layer, cache, query).total;
        if (bytes > cap)
            return fail(RTP_EWORKSPACE, "selection needs %zu bytes of scratch, more than the %zu of the static array",
                        bytes, cap);
    }
    void* ws = nullptr;
    if ((s = scratch_of_current_device(&ws))) return s;
    return topp_select_phase(layer, cache, query, w_q, top_p, sel, ws, bytes, stream, 0, 0);
}

rtp_status rtp_topk_select(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query, const void* w_q,
                           int32_t k, const rtp_sel* sel, void* workspace, size_t workspace_bytes, void* stream) {
    if (k < 1) return fail(RTP_EINVAL, "top-k k %d < 1", k);
    return topp_select_phase(layer, cache, query, w_q, nullptr, sel, workspace, workspace_bytes, stream, 0, k);
}

rtp_status rtp_topp_select_paths(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                 const void* workspace, size_t workspace_bytes, int32_t* paths, void* stream) {
    rtp_status s = check_all(layer, cache, query);
    if (s) return s;
    if (!workspace || !paths) return fail(RTP_EINVAL, "NULL workspace / paths");
    const rtp::Geo g = make_geo(layer, cache, query);
    if (tiled_select(layer, query)) {
        const size_t need = rtp::chunk_select_head_bytes(query->n_tok * layer->num_ret, layer->num_ret,
                                                         query->pos0 + query->n_tok);
        if (workspace_bytes < need) return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
        return hip_status(rtp::launch_chunk_paths(g, workspace, paths, (hipStream_t)stream), "paths launch");
    }
    const SelPlan p = plan_select(layer, cache, query);
    if (workspace_bytes < p.total) return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, p.total);
    if (p.group_rows < p.rows_total) return fail(RTP_EUNSUPPORTED, "rows of the call span several workspace passes");
    const rtp::SelWs w = sel_ws(p, (char*)workspace);
    return hip_status(rtp::launch_select_paths(w, p.rows_total, paths, (hipStream_t)stream), "paths launch");
}

rtp_status rtp_topp_select_begin(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                 const void* w_q, const float* top_p, const rtp_sel* sel, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return topp_select_phase(layer, cache, query, w_q, top_p, sel, workspace, workspace_bytes, stream, 1, 0);
}

rtp_status rtp_topp_select_end(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                               const void* w_q, const float* top_p, const rtp_sel* sel, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return topp_select_phase(layer, cache, query, w_q, top_p, sel, workspace, workspace_bytes, stream, 2, 0);
}

rtp_status rtp_indexer_scores(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                              const void* w_q, uint16_t* q_low, float* scores, int64_t score_ld, void* stream) {
    rtp_status s = check_all(layer, cache, query);
    if (s) return s;
    if (!w_q || !q_low || !scores) return fail(RTP_EINVAL, "NULL w_q / q_low / scores");
    if (score_ld < max_keys(cache, query)) return fail(RTP_EINVAL, "score_ld %lld too small", (long long)score_ld);
    const SelPlan p = plan_select(layer, cache, query);
    rtp::SelWs w;
    std::memset(&w, 0, sizeof w);
    w.scores = scores;
    w.score_ld = score_ld;
    w.qlow = q_low;
    w.nchunk = p.nchunk;
    w.rows = p.rows_total;
    if (p.rows_total > 65535) return fail(RTP_EUNSUPPORTED, "more than 65535 rows");
    rtp::SelOut out{nullptr, nullptr, 0, nullptr};
    const rtp::Geo g = make_geo(layer, cache, query);
    return hip_status(rtp::launch_select(g, query->q, w_q, (const uint16_t*)cache->k_low, nullptr, 0, w, out,
                                         p.rows_total, layer->dtype, rtp::kSelScoresOnly, (hipStream_t)stream),
                      "indexer score launch");
}

size_t rtp_sparse_attn_workspace(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                 int64_t capacity) {
    if (check_all(layer, cache, query) || capacity < 0) return 0;
    if (query->kind == RTP_CHUNK && mfma_chunk(layer))
        return std::max<size_t>(256, rtp::sparse_prefill_ws_bytes(query->n_tok, layer->num_ret,
                                                                  query->pos0 + query->n_tok));
    const int64_t rows = (int64_t)query->n_tok * layer->num_ret;
    const int64_t items = sparse_max_items(layer, query, capacity);
    return align256((size_t)items * (layer->head_dim + 2) * 4) + align256((size_t)(rows + 1) * 4);
}

rtp_status rtp_sparse_attn_decode(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                  const rtp_sel* sel, void* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    rtp_status s = check_all(layer, cache, query);
    if (s) return s;
    if (query->kind != RTP_DECODE) return fail(RTP_EINVAL, "rtp_sparse_attn_decode needs RTP_DECODE queries");
    if (!sel || !sel->row_ptr || !sel->status || !out) return fail(RTP_EINVAL, "NULL selection / out");
    if (sel->capacity > 0 && !sel->idx) return fail(RTP_EINVAL, "NULL idx");
    const int rows = query->n_tok * layer->num_ret;
    if (rows > kMaxDecodeRows) return fail(RTP_EUNSUPPORTED, "batch * num_ret %d > %d", rows, kMaxDecodeRows);
    const size_t need = rtp_sparse_attn_workspace(layer, cache, query, sel->capacity);
    if (!workspace || workspace_bytes < need)
        return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    const int64_t items = sparse_max_items(layer, query, sel->capacity);
    rtp::AttnWs w{};
    w.part = (float*)workspace;
    w.item_start = (int32_t*)((char*)workspace + align256((size_t)items * (layer->head_dim + 2) * 4));
    w.max_items = items;
    const rtp::Geo g = make_geo(layer, cache, query);
    return hip_status(rtp::launch_sparse_decode(g, query->q, cache->k, cache->v, sel->row_ptr, sel->idx,
                                                sel->status, out, w, 0, rows, layer->dtype, (hipStream_t)stream),
                      "sparse decode launch");
}

rtp_status rtp_sparse_attn_prefill(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                   const rtp_sel* sel, void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    rtp_status s = check_all(layer, cache, query);
    if (s) return s;
    if (query->kind != RTP_CHUNK) return fail(RTP_EINVAL, "rtp_sparse_attn_prefill needs RTP_CHUNK queries");
    if (!sel || !sel->row_ptr || !sel->status || !out) return fail(RTP_EINVAL, "NULL selection / out");
    if (sel->capacity > 0 && !sel->idx) return fail(RTP_EINVAL, "NULL idx");
    const size_t need = rtp_sparse_attn_workspace(layer, cache, query, sel->capacity);
    if (!workspace || workspace_bytes < need)
        return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    if (mfma_chunk(layer)) {
        const rtp::Geo g = make_geo(layer, cache, query);
        return hip_status(rtp::launch_sparse_prefill(g, query->q, cache->k, cache->v, sel->row_ptr, sel->idx,
                                                     sel->capacity, sel->status, out, workspace,
                                                     (hipStream_t)stream),
                          "sparse prefill launch");
    }
    const int rows = query->n_tok * layer->num_ret;
    const int64_t items = sparse_max_items(layer, query, sel->capacity);
    rtp::AttnWs w{};
    w.part = (float*)workspace;
    w.item_start = (int32_t*)((char*)workspace + align256((size_t)items * (layer->head_dim + 2) * 4));
    w.max_items = items;
    const rtp::Geo g = make_geo(layer, cache, query);
    // rows are processed in groups of at most kMaxDecodeRows; groups run in
    // stream order and reuse the same partial buffer
    for (int row0 = 0; row0 < rows; row0 += kMaxDecodeRows) {
        const int nr = std::min(kMaxDecodeRows, rows - row0);
        hipError_t e = rtp::launch_sparse_decode(g, query->q, cache->k, cache->v, sel->row_ptr, sel->idx,
                                                 sel->status, out, w, row0, nr, layer->dtype, (hipStream_t)stream);
        if (e != hipSuccess) return hip_status(e, "sparse prefill launch");
    }
    return ok();
}

static size_t sparse_dec_ws_bytes(const rtp_layer* layer, const rtp_query* query, int64_t capacity) {
    const int64_t rows = (int64_t)query->n_tok * layer->num_ret;
    const int64_t items = sparse_max_items(layer, query, capacity);
    return align256((size_t)items * (layer->head_dim + 2) * 4) + align256((size_t)(rows + 1) * 4);
}

// Shared gathers: at most kGqaMax retrieval heads per KV head.
static int gqa_max_group(const rtp_layer* L) {
    int best = 0, run = 0;
    for (int r = 0; r < L->num_ret; ++r) {
        run = (r && L->ret_heads[r - 1] / (L->num_q_heads / L->num_kv_heads) ==
                        L->ret_heads[r] / (L->num_q_heads / L->num_kv_heads)) ? run + 1 : 1;
        best = std::max(best, run);
    }
    return best;
}

// Extra workspace of the shared gathers: kGqaMax partial slots per item, the
// unions' keys and membership bytes (one padded row of keys per row), counts.
static size_t gqa_ws_bytes(const rtp_layer* layer, const rtp_query* query, int64_t capacity, int64_t lpad) {
    const int64_t rows = (int64_t)query->n_tok * layer->num_ret;
    const int64_t items = sparse_max_items(layer, query, capacity);
    return align256((size_t)items * rtp::kGqaMax * (layer->head_dim + 2) * 4) +
           align256((size_t)rows * lpad * 4) + align256((size_t)rows * lpad) + align256((size_t)rows * 4);
}

static bool gqa_on(const rtp_layer* layer) { return (layer->flags & RTP_FLAG_GQA_SHARED) && layer->kv_fp8 == 0; }

size_t rtp_decode_attn_workspace(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query,
                                 int64_t capacity) {
    if (check_all(layer, cache, query) || capacity < 0 || query->kind != RTP_DECODE) return 0;
    const SelPlan p = plan_select(layer, cache, query);
    return p.total + sparse_dec_ws_bytes(layer, query, capacity) + win_ws_bytes(layer, cache, query, 0) +
           (gqa_on(layer) ? gqa_ws_bytes(layer, query, capacity, p.lpad) : 0);
}

// Rows of one decode step up to which the row pass runs the window items on
// its spare workgroups (each row takes a CU; the items need free CUs).
constexpr int kRowsWithWindow = 128;

rtp_status rtp_decode_attn(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query, const void* w_q,
                           const void* w_k, const float* top_p, const rtp_sel* sel, void* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    rtp_status s = check_all(layer, cache, query);
    if (s) return s;
    if (query->kind != RTP_DECODE) return fail(RTP_EINVAL, "rtp_decode_attn needs RTP_DECODE queries");
    if (!w_q || !top_p || !out) return fail(RTP_EINVAL, "NULL w_q / top_p / out");
    if (!sel || !sel->row_ptr || !sel->status || (sel->capacity > 0 && !sel->idx) || sel->capacity < 0)
        return fail(RTP_EINVAL, "bad selection buffers");
    if ((s = check_ring_window(layer, cache, query))) return s;
    const int rows = query->n_tok * layer->num_ret;
    if (rows > kMaxDecodeRows) return fail(RTP_EUNSUPPORTED, "batch * num_ret %d > %d", rows, kMaxDecodeRows);
    const SelPlan p = plan_select(layer, cache, query);
    const bool gqa = gqa_on(layer);
    if (gqa && gqa_max_group(layer) > rtp::kGqaMax)
        return fail(RTP_EUNSUPPORTED, "RTP_FLAG_GQA_SHARED serves at most %d retrieval heads per KV head", rtp::kGqaMax);
    const size_t sp_bytes = sparse_dec_ws_bytes(layer, query, sel->capacity);
    const size_t win_bytes = win_ws_bytes(layer, cache, query, 0);
    const size_t need = p.total + sp_bytes + win_bytes + (gqa ? gqa_ws_bytes(layer, query, sel->capacity, p.lpad) : 0);
    if (!workspace || workspace_bytes < need)
        return fail(RTP_EWORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
    const int64_t items = sparse_max_items(layer, query, sel->capacity);
    char* aw = (char*)workspace + p.total;
    rtp::AttnWs w{};
    w.part = (float*)aw;
    w.item_start = (int32_t*)(aw + align256((size_t)items * (layer->head_dim + 2) * 4));
    w.max_items = items;
    float* wpart = (float*)(aw + sp_bytes);
    const rtp::Geo g = make_geo(layer, cache, query);
    const hipStream_t st = (hipStream_t)stream;
    const int split = win_split(layer, 0);
    const int nsplit = (win_keys(layer, cache, 0) + split - 1) / split;
    if (p.group_rows < p.rows_total) {
        // rows beyond one workspace pass: the calls in sequence (the indexer
        // keys appended first, at each sequence's last position)
        if (w_k) {
            hipError_t e = rtp::launch_indexer_append_last(g, cache->k, cache->k_low, w_k, layer->dtype, st);
            if (e != hipSuccess) return hip_status(e, "indexer append launch");
        }
        if ((s = topp_select_phase(layer, cache, query, w_q, top_p, sel, workspace, p.total, stream, 0, 0))) return s;
        hipError_t e = rtp::launch_sparse_decode(g, query->q, cache->k, cache->v, sel->row_ptr, sel->idx,
                                                 sel->status, out, w, 0, rows, layer->dtype, st);
        if (e != hipSuccess) return hip_status(e, "sparse decode launch");
        return hip_status(rtp::launch_window_decode(g, query->q, cache->k, cache->v, out, wpart, nsplit, split, 0,
                                                    layer->dtype, st),
                          "window decode launch");
    }
    const rtp::SelWs sw = sel_ws(p, (char*)workspace);
    const rtp::SelOut so{sel->row_ptr, sel->idx, sel->capacity, sel->status};
    // the window items run inside the row pass when they are MFMA items (bf16
    // K/V, D = 128) and the rows leave CUs free
    const bool merged = split == kWinSplitMfma && g.group <= 32 && rows <= kRowsWithWindow;
    rtp::WinWork win{(const uint16_t*)query->q, (const uint16_t*)cache->k, (const uint16_t*)cache->v, wpart, nsplit,
                     split, nsplit * cache->batch * layer->num_kv_heads};
    const rtp::KeyAppend app{cache->k, w_k};
    hipError_t e = rtp::launch_select(g, query->q, w_q, (const uint16_t*)cache->k_low, top_p, 0, sw, so, rows,
                                      layer->dtype, rtp::kSelRows, st, merged ? &win : nullptr, &app);
    if (e != hipSuccess) return hip_status(e, "top-p select launch");
    if (gqa) {
        // the shared gathers' partials ([item][kGqaMax][D + 2]) and unions after the window's partials
        char* gw = aw + sp_bytes + win_bytes;
        const size_t part_bytes = align256((size_t)items * rtp::kGqaMax * (layer->head_dim + 2) * 4);
        w.part = (float*)gw;
        w.ukey = (uint32_t*)(gw + part_bytes);
        w.umask = (uint8_t*)(gw + part_bytes + align256((size_t)rows * p.lpad * 4));
        w.ucnt = (int32_t*)(gw + part_bytes + align256((size_t)rows * p.lpad * 4) + align256((size_t)rows * p.lpad));
        w.ulen = p.lpad;
        e = rtp::launch_sparse_decode_gqa(g, query->q, cache->k, cache->v, sw, so, out, w, rows, layer->dtype,
                                          merged ? &win : nullptr, st);
    } else {
        e = rtp::launch_sparse_decode_sel(g, query->q, cache->k, cache->v, sw, so, out, w, rows, layer->dtype,
                                          merged ? &win : nullptr, st);
    }
    if (e != hipSuccess) return hip_status(e, "sparse decode launch");
    if (merged) return ok();
    return hip_status(rtp::launch_window_decode(g, query->q, cache->k, cache->v, out, wpart, nsplit, split, 0,
                                                layer->dtype, st),
                      "window decode launch");
}

size_t rtp_window_attn_workspace(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query) {
    if (check_all(layer, cache, query)) return 0;
    return win_ws_bytes(layer, cache, query, 0);
}

size_t rtp_dense_attn_workspace(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query) {
    if (check_all(layer, cache, query)) return 0;
    return win_ws_bytes(layer, cache, query, 1);
}

rtp_status rtp_window_attn(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return window_like(layer, cache, query, out, workspace, workspace_bytes, stream, 0);
}

rtp_status rtp_dense_attn(const rtp_layer* layer, const rtp_cache* cache, const rtp_query* query, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return window_like(layer, cache, query, out, workspace, workspace_bytes, stream, 1);
}

}  // extern "C"
