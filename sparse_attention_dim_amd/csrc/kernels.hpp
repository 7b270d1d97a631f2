// kernels.hpp -- launch parameters shared by the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rtp {

constexpr int kMaxRet = 64;

// Geometry of one call (host-filled, passed by value to kernels).
struct Geo {
    int Hq, Hkv, D, group;        // group = Hq / Hkv
    int n_ret;
    int ret_heads[kMaxRet];
    int is_ret[256];              // 1 if query head h retrieves (Hq <= 256)
    int window, sinks;
    float attn_scale, idx_scale;
    int kind, seq, pos0, n_tok;   // query rows
    int batch, max_blocks;
    int max_seq_len;              // host bound; device lengths are clamped to [1, max_seq_len]
    int n_hlist;                  // heads computed by a prefill attention launch
    int hlist[256];
    const int32_t* block_table;
    const int32_t* seq_lens;
};

// Position of query token t (keys 0..pos visible) and its sequence.
__device__ __forceinline__ int row_seq(const Geo& g, int t) { return g.kind == 0 ? t : g.seq; }
__device__ __forceinline__ int seq_len(const Geo& g, int b) {
    return min(max(g.seq_lens[b], 1), g.max_seq_len);
}
__device__ __forceinline__ int row_pos(const Geo& g, int t) {
    return g.kind == 0 ? seq_len(g, t) - 1 : g.pos0 + t;
}

// Per-row state of the top-p selection (device workspace).
struct RowState {
    float m;                      // row maximum score
    int32_t mode;                 // 0 every key, 1 ordered list in SelWs::sel, 2 threshold (Tkey, jT)
    uint32_t Tkey;                // threshold: keys with score key > Tkey, or == Tkey and index <= jT
    int32_t jT;
    int32_t L;                    // keys of the row
    int32_t count;                // selected keys
    unsigned long long target;    // ceil(p Z), fixed point
    float d_thr;                  // U = keys with score >= d_thr
};

constexpr int kChunk = 4096;      // keys per workgroup of the scoring pass
constexpr int kCB = 128;          // mass-histogram bins per chunk (1/4 unit of s (m_c - d) each)
constexpr int kCand = 8192;       // candidates ranked by one sort

// Device workspace of the selection, for `rows` rows of at most Lpad keys.
struct SelWs {
    float* scores;                // [rows][Lpad]
    int64_t score_ld;
    uint32_t* cmax;               // [rows][nchunk] ordered keys of chunk maxima
    uint16_t* qlow;               // [rows][16]
    unsigned long long* chist;    // [rows][nchunk][kCB] chunk mass histograms
    RowState* st;                 // [rows]
    uint32_t* sel;                // [rows][kCand] selected indices, ascending (mode 1)
    unsigned long long* ubuf;     // [rows][kCand] U in index order: (score key << 32) | ~index
    unsigned* ccnt;               // [rows][nchunk][kCB] cumulative key counts of the chunk bins
    uint32_t* row_n;              // [rows] size of U
    uint32_t* chunk_cnt;          // [rows][nchunk] output offsets per chunk (mode 2)
    int nchunk;
    int rows;                     // rows of this group
};

struct SelOut {
    int64_t* row_ptr;
    int32_t* idx;
    int64_t capacity;
    int32_t* status;
};

// Launchers (defined in the .hip files; return hipError_t of the launches).
hipError_t launch_indexer_append(const Geo& g, const void* k, void* k_low, const void* w_k,
                                 const int32_t* seq_id, const int32_t* pos, int n, int dtype,
                                 hipStream_t s);

// Selection of rows [row0, row0 + ws.rows) of the call, all of it or one stage.
enum SelStage {
    kSelAll = 0,                  // scoring pass with statistics, then gather, cut, emit
    kSelScoresOnly = 1,           // projection and scores only (rtp_indexer_scores)
    kSelScorePass = 2,            // the first part of kSelAll
    kSelFinish = 3,               // the rest of kSelAll
};
hipError_t launch_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                         const float* top_p, int row0, const SelWs& ws, const SelOut& out,
                         int total_rows, int dtype, int stage, hipStream_t s);

// Selected keys per work item (one wavefront) of the sparse decode: a row of
// n selected keys makes ceil(n / kSparseItem) partial results, so a call needs
// at most rows + capacity / kSparseItem + 1 of them.
constexpr int kSparseItem = 64;

// Split-K partial attention of retrieval rows over their selected sets and the combine.
struct AttnWs {
    float* part;                  // [items][D + 2]
    int32_t* item_start;          // [rows + 1]
    int64_t max_items;
};
// Rows [row0, row0 + rows) of the call (rows <= 4096); row_ptr is the full CSR array.
hipError_t launch_sparse_decode(const Geo& g, const void* q, const void* k, const void* v,
                                const int64_t* row_ptr, const int32_t* idx, const int32_t* status,
                                void* out, const AttnWs& ws, int row0, int rows, int dtype, hipStream_t s);

// Top-p selection of the rows of one prefill chunk (bf16, D <= 128): indexer
// scores of 32-row x 32-key tiles by MFMA as a filter, exact fixed-order
// scores only where they decide the set; same result as launch_select.
// Workspace: chunk_select_head_bytes at least; the rest is a pool of
// candidate entries, chunk_select_ws_bytes recommends 4096 per row.
size_t chunk_select_head_bytes(int rows, int n_ret, int n_keys);
size_t chunk_select_ws_bytes(int rows, int n_ret, int n_keys);
hipError_t launch_chunk_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                               const float* top_p, void* ws, size_t ws_bytes, const SelOut& out, hipStream_t s);

// Sparse attention of the retrieval heads of a prefill chunk (bf16, D = 128):
// MFMA over the union of 64 consecutive rows' selected sets, masked per row.
// Workspace: per-row window offsets, per (tile, window) union bitmaps and
// sizes, and the partial results of every row, window and split.  idx_n is
// the number of readable entries of idx (the CSR capacity).
size_t sparse_prefill_ws_bytes(int n_tok, int n_ret, int n_keys);
hipError_t launch_sparse_prefill(const Geo& g, const void* q, const void* k, const void* v, const int64_t* row_ptr,
                                 const int32_t* idx, int64_t idx_n, const int32_t* status, void* out, void* ws,
                                 hipStream_t s);

// Chunked-prefill attention (bf16, D = 128) of the heads g.hlist[0..n_hlist):
// sinks + causal window, or dense causal.
hipError_t launch_prefill_attn(const Geo& g, const void* q, const void* k, const void* v, void* out,
                               int dense, hipStream_t s);

// Local-head (window) or dense decode attention, split over keys, then combine.
hipError_t launch_window_decode(const Geo& g, const void* q, const void* k, const void* v, void* out,
                                float* part, int nsplit, int split_keys, int dense, int dtype,
                                hipStream_t s);

}  // namespace rtp
