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
 *  - Window-only ring (optional; the cache-side half of the method: the full
 *    KV cache is kept only for the KV heads that serve a retrieval head).
 *    When cache->k_ring is set, KV heads none of whose query heads retrieve
 *    ("ring heads") live in k_ring/v_ring [num_ring_blocks][n_ring][RTP_BLOCK][D]
 *    in ascending KV-head order, and k/v pages hold only the other KV heads
 *    ([num_blocks][Hkv - n_ring][RTP_BLOCK][D], ascending).  A sequence's ring
 *    has ring_pages pages: entry 0 of its ring_table row holds positions
 *    0..255 (the sinks), entries 1..ring_pages-1 hold later positions in
 *    rotation (position j >= 256 in entry 1 + (j/256 - 1) % (ring_pages - 1)),
 *    so only the last (ring_pages - 1) * 256 positions past the first page are
 *    kept.
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

#define RTP_VERSION 2
#define RTP_IDX_DIM 16      /* indexer width (the pages' 16-dimensional indexer) */
#define RTP_BLOCK 256       /* tokens per KV page */
#define RTP_MAX_RET 64      /* most retrieval heads per layer */
#define RTP_MAX_LEN (1 << 20) /* longest context: the exact 2^-43 fixed-point mass sums hold 2^20 keys
                               (each weight <= 1, so a row's total stays below 2^63) */

/* rtp_layer.flags */
#define RTP_FLAG_EXACT_MASS 1  /* bf16 chunk selection: sum the indexer-softmax normaliser exactly over
                                  every key of every row (an extra pass over the indexer keys of each
                                  row; the selected sets are those of the default, certified route) */
#define RTP_FLAG_GQA_SHARED 2  /* rtp_decode_attn: the retrieval heads of one KV head (at most 4 per KV
                                  head) gather the union of their selected keys once, each key row
                                  read once and scored for every head whose set holds it (abstract:
                                  retrieval heads keep the full KV cache; grouped-query attention
                                  shares it between query heads).  Same sets, same CSR; outputs as
                                  rtp_sparse_attn_decode up to the order of the partial merges.
                                  bf16 or fp32 K/V, decode queries whose selection fits one
                                  workspace pass; ignored by the other calls */

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
    int32_t k_max;                  /* top-p budget cap: a row keeps at most the first k_max keys of its
                                       rank order (a bound on the CSR capacity); 0 = no cap */
    int32_t flags;                  /* RTP_FLAG_* */
    int32_t kv_fp8;                 /* 1: K and V (cache pages, ring, rtp_kv_append input) are FP8 E4M3
                                       codes (OCP: bias 7, no infinities), code c standing for
                                       fl32(f32(c) * k_scale) (V: v_scale); Q, W and outputs stay in
                                       dtype, which must be RTP_BF16.  Supported by the decode calls,
                                       rtp_indexer_append, rtp_kv_append and rtp_sparse_attn_prefill;
                                       chunked window / dense attention return RTP_EUNSUPPORTED.
                                       0: K/V in dtype */
    float k_scale, v_scale;         /* FP8 scales (> 0, finite); ignored when kv_fp8 == 0 */
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
    int32_t max_seq_len;            /* [host] upper bound of every seq_lens[b], at most RTP_MAX_LEN;
                                       sizes grids and workspaces */
    const void *k_ring;             /* NULL: no ring (every KV head in k/v); else ring K pages, see above */
    const void *v_ring;
    const int32_t *ring_table;      /* [batch][ring_pages] page ids of the ring pools */
    int32_t ring_pages;             /* [host] >= 2 when k_ring is set */
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
                                       certified (nothing written), 3 = a top_p value is NaN or <= 0
                                       (nothing written) */
} rtp_sel;

/* Library version (RTP_VERSION). */
int rtp_version(void);

/* Text of the calling thread's last error ("" if none). */
const char *rtp_last_error(void);

/*
 * a1. Indexer key append: the 16-dimensional indexer key of every retrieval
 * head, written when a token's K enters the cache (abstract, observation (2):
 * a lightweight 16-dimensional token indexer replaces full-rank similarity;
 * forum post, "Three Key Insights" item 2: the projection is built on the
 * low-frequency RoPE dimensions).  For i < n and every retrieval head r with
 * KV head g = ret_heads[r]/(Hq/Hkv):
 *   k_low[page(seq_id[i], pos[i])][r][slot][c] =
 *       bf16_rne( fp32 FMA chain over d = 0..D-1 from +0 of K[seq_id[i], pos[i], g, d] * w_k[r][d][c] )
 * K is read from the cache, so the token's K must already be stored there
 * (rtp_kv_append stores K and V and writes k_low in one launch).
 * seq_id, pos: device int32[n] (pos[i] < max_seq_len; not checked on the
 * device).  n == 0 is a no-op.  Errors: RTP_EINVAL for NULL pointers or n < 0.
 */
rtp_status rtp_indexer_append(const rtp_layer *layer, const rtp_cache *cache, const void *w_k,
                              const int32_t *seq_id, const int32_t *pos, int32_t n, void *stream);

/*
 * a1 fused with the K/V append (abstract: retrieval heads keep the full KV
 * cache, the others a restricted window; forum post, "Three Key Insights"
 * item 1): stores the K and V rows of n new tokens, k_new / v_new
 * [n][Hkv][D] (dtype of the layer, 16-byte aligned), at positions pos[i] of
 * sequences seq_id[i] -- in k/v, or in the ring for the ring heads -- and
 * writes their indexer keys k_low exactly as rtp_indexer_append would, from
 * the new K rows, all in one launch.  The cache's k, v, k_ring, v_ring and
 * k_low are written (the const of rtp_cache's k/v does not apply here).
 * seq_id, pos: device int32[n]; tokens with an out-of-range seq_id or pos are
 * skipped.  Two tokens of one call that land in the same ring slot (positions
 * of a sequence (ring_pages - 1) * 256 or more apart) race: append such
 * positions in separate calls, in position order.  n == 0 is a no-op.  Errors: RTP_EINVAL for NULL pointers, n < 0
 * or misaligned k_new / v_new.
 */
rtp_status rtp_kv_append(const rtp_layer *layer, const rtp_cache *cache, const void *k_new, const void *v_new,
                         const void *w_k, const int32_t *seq_id, const int32_t *pos, int32_t n, void *stream);

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
 *   cut to its first layer->k_max keys when k_max > 0, written ascending.
 *   Scores and the ranking are exact (bit for bit the fixed-order fp32
 *   chain); masses use fp32 exp with an exact argument and are summed exactly
 *   in 2^-43 fixed point.  The bf16 chunk path sums the mass of the keys far
 *   from the cut from MFMA scores, bounds the error of that sum, and accepts
 *   a cut only where the bound cannot move it past the band below; other rows
 *   are cut again with the normaliser summed exactly over every key.  So on
 *   every path the set can differ from an exact-arithmetic one only where a
 *   cumulative mass lies within 1e-6 of p.
 * top_p: device float[batch] in (0, 1]; a NaN or non-positive value sets
 * *status = 3.  On overflow (total > sel->capacity) *status = 1, row_ptr is
 * complete and idx is untouched.  *status = 2 means the chunk selection could
 * not certify a row's cut (an internal error bound was violated): nothing is
 * written and row_ptr is not meaningful.
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
 * rtp_topp_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus the workspace),
 * checks, result and errors as rtp_topp_select; the workspace is a static
 * device array of RTP_NOALLOC_SCRATCH_BYTES on the current GPU (the stream
 * must belong to it), which each GPU the library runs on holds until the
 * process ends.  A query whose selection needs more scratch than that (see
 * rtp_topp_select_workspace; for bf16 chunks rtp_topp_select_workspace_min)
 * is rejected with RTP_EWORKSPACE before anything is enqueued.  The call
 * itself allocates nothing.  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (e.g. on two streams) race and must be
 * serialised by the caller; the array keeps the last call's contents, and
 * the selection clears what it needs itself.
 */
#define RTP_NOALLOC_SCRATCH_BYTES (64u << 20)
rtp_status rtp_topp_select_noalloc(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                                   const void *w_q, const float *top_p, const rtp_sel *sel, void *stream);

/*
 * Fixed top-k selection: the fixed-budget rule that the method's dynamic
 * top-p replaces (abstract, observation (3); forum post, "Three Key Insights"
 * item 3).  Same arguments, scores, ranking, output and workspace as
 * rtp_topp_select, with a host count k >= 1 instead of top_p: each row keeps
 * the first min(k, pos + 1) keys of its rank order (d_j descending, j
 * ascending), written ascending.  The set is exact (no mass band).  The cut
 * runs through the same radix machinery with key counts in place of masses.
 * layer->k_max is not used.
 */
rtp_status rtp_topk_select(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                           const void *w_q, int32_t k, const rtp_sel *sel,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Inspection: after rtp_topp_select or rtp_topk_select with the same layer,
 * cache, query and workspace (and nothing else run on that workspace since),
 * writes one code per row (int32 [n_tok*num_ret], device) telling how its set
 * was formed: the low 4 bits name the route -- 1 every key, 2 / 3 / 4 the
 * bf16 chunk path's candidate buffer of at most 1024 / 8192 / 16384 keys, 5
 * the chunk path's radix levels over every key tile, 6 the decode path's
 * candidate list in LDS, 7 the decode path's cut over the row's scores, 8 the
 * decode path's candidate list of more than 8192 keys cut from the
 * workspace -- and the
 * flags 16 (ordered through a bitmap) / 32 (ordered by merging runs), 64 (the
 * normaliser summed exactly over every key), 128 (the cut counted keys: top-k
 * or the k_max cap), 256 (decode path: the candidate set was gathered from
 * the row's scores because it reaches past the keys the scoring pass flags,
 * those within 4 units of s * (chunk maximum - score)).  For the decode path and fp32 chunks only when every row
 * fits one pass of the workspace (RTP_EUNSUPPORTED otherwise).
 */
rtp_status rtp_topp_select_paths(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                                 const void *workspace, size_t workspace_bytes, int32_t *paths, void *stream);

/*
 * a2-a3 only, for inspection: q_low (bf16 [rows][16]) and the fp32 indexer
 * scores [rows][score_ld] (entries beyond a row's pos are not written).
 * score_ld >= max position + 1 of the call.  Needs no workspace.
 */
rtp_status rtp_indexer_scores(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                              const void *w_q, uint16_t *q_low, float *scores, int64_t score_ld, void *stream);

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

/*
 * a2-a6 of one decode step in one call: the selection of rtp_topp_select and
 * the attention of rtp_sparse_attn_decode over it for the retrieval heads, and
 * the window attention of rtp_window_attn for the local heads (abstract:
 * retrieval heads score every cached token with the lightweight indexer and
 * attend sparsely over the full KV cache, the other heads use a restricted
 * window; forum post, "Open Questions and Limitations": per-query token counts
 * vary, so here the attention reads each row's selected keys straight from the
 * selection's row records, with no host round trip and no pass that writes the
 * CSR before the attention reads it; with bf16 K/V and head_dim 128 the local
 * heads' window attention runs on the compute units the per-row selection
 * leaves free).  w_k: NULL, or the indexer projections: then the step's
 * tokens' indexer keys (position seq_lens[b]-1 of every sequence) are written
 * first, exactly as rtp_indexer_append would write them (a1; their K rows must
 * be in the cache), by the scoring pass itself.  Otherwise the same arguments
 * as rtp_topp_select plus `out`; the same
 * selection, CSR output and status codes as rtp_topp_select, the same
 * retrieval-head outputs as rtp_sparse_attn_decode with that sel, and the same
 * local-head outputs as rtp_window_attn.  On capacity overflow (*status = 1,
 * row_ptr complete, idx untouched) and for an invalid top_p (*status = 3) the
 * retrieval heads' outputs are not written; the local heads' always are.
 * RTP_DECODE queries only.  workspace: rtp_decode_attn_workspace(layer, cache,
 * query, sel->capacity) bytes.  Errors: as the three calls; RTP_EINVAL for
 * another query kind.
 */
size_t rtp_decode_attn_workspace(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                                 int64_t capacity);
rtp_status rtp_decode_attn(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                           const void *w_q, const void *w_k, const float *top_p, const rtp_sel *sel, void *out,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes for rtp_window_attn / rtp_dense_attn. */
size_t rtp_window_attn_workspace(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query);
size_t rtp_dense_attn_workspace(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query);

/*
 * a6. Local heads (abstract obs. (1): the remaining heads use a restricted
 * window; forum "Three Key Insights" item 1): for every non-retrieval head h
 * and query at position pos, exact softmax attention over the keys
 *   {0 .. num_sinks-1} U {pos-window+1 .. pos}, clipped to [0, pos].
 * With a ring the ring heads read it: it must hold every key a query of the
 * call needs, so num_sinks <= 256 and (ring_pages - 1) * 256 >= window + 255
 * (+ n_tok - 1 for chunks); RTP_EINVAL otherwise.
 */
rtp_status rtp_window_attn(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                           void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dense causal attention of every head over keys 0..pos: the same-GPU
 * baseline against which the sparse path's speedup is reported.  Needs every
 * key of every head: RTP_EINVAL for a cache with a ring.
 */
rtp_status rtp_dense_attn(const rtp_layer *layer, const rtp_cache *cache, const rtp_query *query,
                          void *out, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RTP_H */
