/*
 * rtp.h -- C ABI of the MI355X (gfx950) RTPurbo head-split sparse-attention
 * hot path: retrieval heads select tokens with a 16-dimensional indexer and
 * per-query top-p, then attend exactly over the selected K/V rows; local heads
 * attend over a sliding window plus sink tokens.
 *
 * Method: "Full Attention Strikes Back: Transferring Full Attention into
 * Sparse within Hundred Training Steps" (arXiv 2605.16928), abstract,
 * observations (1)-(3); zhichai.net forum post "RTPurbo: Turning Dense LLMs
 * into Sparse Attention Models with Just a Few Hundred Training Steps",
 * sections "Three Key Insights" and "The RTPurbo Method".
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns all
 *    memory (KV pages, indexer pages, projections, outputs, workspace); the
 *    library never allocates or frees device memory and keeps no device
 *    state between calls.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the null stream).  No entry point synchronises the host, so a sequence
 *    of calls can be captured into a HIP graph.  Buffers must stay alive until
 *    the enqueued work completes.
 *  - Argument checks run on the host before anything is enqueued and return
 *    RTP_EINVAL / RTP_EUNSUPPORTED; a failed launch returns RTP_EHIP.  The
 *    text of the last error of the calling thread is in rtp_last_error().
 *    Nothing is enqueued when a call returns an error.
 *  - dtype RTP_F32 or RTP_BF16 applies to Q, K, V, W_q, W_k and the attention
 *    output; indexer keys and queries (K_low, q_low) are always bf16.
 *
 * Data layout
 *  - KV pages: k, v are [num_blocks][num_kv_heads][RTP_BLOCK][head_dim];
 *    token j of sequence b lives in page block_table[b*max_blocks + j/RTP_BLOCK]
 *    at slot j % RTP_BLOCK.  Keys are stored after RoPE.
 *  - Indexer pages: k_low is bf16 [num_blocks][num_ret][RTP_BLOCK][16], using
 *    the same page ids as k/v (one 8 KiB run per page and retrieval head).
 *  - Projections w_q, w_k: [num_ret][head_dim][16], row-major.
 *  - Queries q: [n_tok][num_q_heads][head_dim], after RoPE.
 *  - Output out: [n_tok][num_q_heads][head_dim]; the sparse calls write the
 *    retrieval heads' slices, rtp_window_attn writes the local heads' slices,
 *    rtp_dense_attn writes every head.
 *  - Selected sets (CSR): rows are (query token t, retrieval head r) in
 *    token-major order, row = t*num_ret + r; row_ptr has rows+1 entries and
 *    each row's indices are ascending token positions.
 */
#ifndef RTP_H
#define RTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RTP_VERSION 1
#define RTP_IDX_DIM 16      /* indexer width (the pages' 16-dimensional indexer) */
#define RTP_BLOCK 256       /* tokens per KV page */
#define RTP_MAX_RET 64      /* most retrieval heads per layer */

typedef enum {
    RTP_OK = 0,
    RTP_EINVAL = 1,        /* an argument is out of range or inconsistent */
    RTP_EUNSUPPORTED = 2,  /* valid but not implemented (e.g. head_dim 96) */
    RTP_EHIP = 3,          /* a HIP launch failed */
    RTP_EWORKSPACE = 4     /* workspace smaller than the *_workspace size */
} rtp_status;

typedef enum { RTP_F32 = 0, RTP_BF16 = 1 } rtp_dtype;

typedef enum {
    RTP_DECODE = 0,  /* one query per sequence b (n_tok == batch) at position seq_lens[b]-1 */
    RTP_CHUNK = 1    /* n_tok consecutive queries of sequence `seq` at positions pos0..pos0+n_tok-1 */
} rtp_query_kind;

/* [host] Per-layer constants. */
typedef struct rtp_layer {
    int32_t num_q_heads;            /* Hq */
    int32_t num_kv_heads;           /* Hkv; Hq % Hkv == 0; query head h reads KV head h/(Hq/Hkv) */
    int32_t head_dim;               /* D: 64 or 128 */
    int32_t dtype;                  /* rtp_dtype of Q, K, V, W, output */
    int32_t num_ret;                /* retrieval heads, 1..RTP_MAX_RET */
    int32_t ret_heads[RTP_MAX_RET]; /* strictly ascending query-head ids; every other head is local */
    int32_t window;                 /* local heads: last `window` positions (incl. the query's), >= 1 */
    int32_t num_sinks;              /* local heads: plus positions 0..num_sinks-1, >= 0 */
    float attn_scale;               /* softmax scale of attention, e.g. 1/sqrt(D) */
    float idx_scale;                /* softmax scale of the indexer, e.g. 1/sqrt(16) */
} rtp_layer;

/* [host] struct of device pointers: the paged KV cache of a batch. */
typedef struct rtp_cache {
    const void *k;                  /* [num_blocks][Hkv][RTP_BLOCK][D] */
    const void *v;                  /* same layout as k */
    void *k_low;                    /* bf16 [num_blocks][num_ret][RTP_BLOCK][16] */
    const int32_t *block_table;     /* [batch][max_blocks] page ids */
    const int32_t *seq_lens;        /* [batch] tokens in the cache, incl. those appended this step */
    int32_t batch;
    int32_t max_blocks;             /* row stride of block_table */
    int32_t max_seq_len;            /* [host] upper bound of every seq_lens[b], at most 2^20 (the exact
                                       fixed-point mass sums hold 2^20 keys); sizes grids and workspaces */
} rtp_cache;

/* [host] struct: the query rows of one call. */
typedef struct rtp_query {
    const void *q;                  /* [n_tok][Hq][D] */
    int32_t n_tok;
    int32_t kind;                   /* rtp_query_kind */
    int32_t seq;                    /* RTP_CHUNK: sequence index */
    int32_t pos0;                   /* RTP_CHUNK: position of row 0; needs pos0+n_tok <= seq_lens[seq] */
} rtp_query;

/* [host] struct of device pointers: the selected sets. */
typedef struct rtp_sel {
    int64_t *row_ptr;               /* [n_tok*num_ret + 1] */
    int32_t *idx;                   /* [capacity] */
    int64_t capacity;               /* [host] entries available in idx */
    int32_t *status;                /* one int: 0 = ok, 1 = capacity overflow (then idx is not written
                                       and row_ptr[rows] holds the capacity needed), 2 = selection not
                                       certified (nothing written) */
} rtp_sel;

/* Library version (RTP_VERSION). */
int rtp_version(void);

/* Text of the calling thread's last error ("" if none). */
const char *rtp_last_error(void);

/*
 * a1. Indexer key append (the indexer key cache is written when K is appended).
 * For i < n and every retrieval head r with KV head g = ret_heads[r]/(Hq/Hkv):
 *   k_low[page(seq_id[i], pos[i])][r][slot][c] =
 *       bf16_rne( fp32 FMA chain over d = 0..D-1 from +0 of K[seq_id[i], pos[i], g, d] * w_k[r][d][c] )
 * K is read from the cache, so the token's K must already be stored there.
 * seq_id, pos: device int32[n].  n == 0 is a no-op.
 */
rtp_status rtp_indexer_append(const rtp_layer *layer, const rtp_cache *cache, const void *w_k,
                              const int32_t *seq_id, const int32_t *pos, int32_t n, void *stream);

/* Workspace bytes needed by rtp_topp_select / rtp_indexer_scores for this query.
 * For a bf16 RTP_CHUNK query this size holds a candidate buffer of 8192 keys
 * per row; rtp_topp_select also accepts any workspace down to
 * rtp_topp_select_workspace_min, and then resolves the rows whose candidate
 * set does not fit the smaller buffer by extra passes over the keys (same
 * result, more time).  For other queries both functions return the same size. */
size_t rtp_topp_select_workspace(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query);
size_t rtp_topp_select_workspace_min(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query);

/*
 * a2-a4. Indexer query projection, indexer scores over every causal key, and
 * dynamic top-p selection (abstract obs. (2)-(3); forum "Three Key Insights"
 * items 2-3).  For row (t, r), query head h = ret_heads[r], position pos:
 *   q_low = bf16_rne(fp32 FMA chain over d of q[t][h][d] * w_q[r][d][c])
 *   d_j   = fp32 chain over c = 0..15 from +0 of q_low[c]*k_low[j][r][c], j = 0..pos
 *   w_j   = exp(idx_scale * (d_j - max d)),  Z = sum w_j
 *   the selected set is the shortest prefix of keys ranked by (d_j descending,
 *   j ascending) whose mass reaches top_p[seq] * Z (all keys if top_p >= 1),
 *   written ascending.  Scores and the ranking are exact (bit for bit the
 *   fixed-order fp32 chain); masses use fp32 exp with an exact argument and
 *   are summed exactly in 2^-43 fixed point, so the set can differ from an
 *   exact-arithmetic one only where a cumulative mass lies within 1e-6 of p.
 * top_p: device float[batch], each in (0, 1] (device values are not checked).
 * On overflow (total > sel->capacity) *status = 1, row_ptr is complete and
 * idx is untouched.  *status = 2 means the chunk selection could not certify
 * a row's cut (an internal error bound was violated): nothing is written and
 * row_ptr is not meaningful.
 */
rtp_status rtp_topp_select(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                           const void *w_q, const float *top_p, const rtp_sel *sel,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * rtp_topp_select in two phases, for callers that overlap other work with the
 * latency-bound second phase (e.g. the local heads' window attention on a
 * second stream, started once _begin's work on `stream` is done).
 *   _begin: q_low, the indexer scores and their per-chunk statistics (the pass
 *           over the indexer keys) into the workspace;
 *   _end:   the cut and the selected sets, from that workspace.
 * Both take the arguments of rtp_topp_select and must get the same ones, on
 * the same stream, _begin first; the workspace must not be touched in
 * between.  Together they launch exactly the kernels of rtp_topp_select and
 * give the same result.  When the rows do not fit one workspace pass (or for
 * bf16 RTP_CHUNK queries) _begin launches nothing and _end does all the work.
 * Errors as for rtp_topp_select.
 */
rtp_status rtp_topp_select_begin(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                                 const void *w_q, const float *top_p, const rtp_sel *sel,
                                 void *workspace, size_t workspace_bytes, void *stream);
rtp_status rtp_topp_select_end(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                               const void *w_q, const float *top_p, const rtp_sel *sel,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * a2-a3 only, for inspection: q_low (bf16 [rows][16]) and the fp32 indexer
 * scores [rows][score_ld] (entries beyond a row's pos are not written).
 * score_ld >= max position + 1 of the call.
 */
rtp_status rtp_indexer_scores(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                              const void *w_q, uint16_t *q_low, float *scores, int64_t score_ld,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for rtp_sparse_attn_decode / _prefill given the CSR capacity. */
size_t rtp_sparse_attn_workspace(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                                 int64_t capacity);

/*
 * a5. Exact attention of each retrieval head over its selected rows (abstract:
 * the full KV cache is kept for retrieval heads, which run sparse attention):
 *   out[t][h] = sum_{j in S(t,r)} softmax_S(attn_scale * q[t][h] . K[j][g]) V[j][g]
 * with the softmax renormalised over S.  _decode takes RTP_DECODE queries,
 * _prefill takes RTP_CHUNK queries.  If *sel->status != 0 nothing is written.
 */
rtp_status rtp_sparse_attn_decode(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                                  const rtp_sel *sel, void *out, void *workspace, size_t workspace_bytes,
                                  void *stream);
rtp_status rtp_sparse_attn_prefill(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                                   const rtp_sel *sel, void *out, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* Workspace bytes for rtp_window_attn / rtp_dense_attn. */
size_t rtp_window_attn_workspace(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query);
size_t rtp_dense_attn_workspace(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query);

/*
 * a6. Local heads (abstract obs. (1): the remaining heads use a restricted
 * window; forum "Three Key Insights" item 1): for every non-retrieval head h
 * and query at position pos, exact softmax attention over the keys
 *   {0 .. num_sinks-1} U {pos-window+1 .. pos}, clipped to [0, pos].
 */
rtp_status rtp_window_attn(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                           void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dense causal attention of every head over keys 0..pos: the same-GPU
 * baseline against which the sparse path's speedup is reported.
 */
rtp_status rtp_dense_attn(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                          void *out, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RTP_H */
