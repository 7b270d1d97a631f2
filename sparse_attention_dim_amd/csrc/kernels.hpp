// kernels.hpp -- launch parameters shared by the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rtp {

constexpr int kMaxRet = 64;
constexpr int kFlagExactMass = 1; // RTP_FLAG_EXACT_MASS

// How a row's selected set was formed (the per-row record that
// rtp_topp_select_paths reports): low 4 bits the resolver, then flags.
constexpr int kPathAll = 1;       // every key of the row
constexpr int kPathTiny = 2;      // chunk path: candidate set of at most 1024 keys
constexpr int kPathRow = 3;       // chunk path: at most 8192 keys (per-row resolve)
constexpr int kPathLarge = 4;     // chunk path: at most 16384 keys (large-row resolve)
constexpr int kPathLevel = 5;     // chunk path: radix levels over every key tile (no buffer)
constexpr int kPathList = 6;      // decode path: candidate list cut in LDS
constexpr int kPathScan = 7;      // decode path: cut over the row's scores
constexpr int kPathListG = 8;     // decode path: candidate list cut from the workspace (above 8192 keys)
constexpr int kPathBitmap = 16;   // chunk path: ordered through a bitmap of the kept range
constexpr int kPathMerge = 32;    // chunk path: ordered by merging the writers' runs
constexpr int kPathExactZ = 64;   // the normaliser was summed exactly over every key
constexpr int kPathCount = 128;   // the cut counted keys (fixed top-k, or the budget cap)
constexpr int kPathFromScores = 256;  // decode path: U gathered from the row's scores (not from the key masks)
constexpr int kPathFlagList = 512;    // decode path: U taken from the scoring pass's per-chunk lists of flagged keys

// Geometry of one call (host-filled, passed by value to kernels).
struct Geo {
    int Hq, Hkv, D, group;        // group = Hq / Hkv
    int n_ret;
    // per-head tables as bytes: Geo is passed by value to every kernel, so its
    // size is kernel-argument traffic on every launch (Hq <= 256)
    uint8_t ret_heads[kMaxRet];
    uint8_t is_ret[256];          // 1 if query head h retrieves
    int window, sinks;
    float attn_scale, idx_scale;
    int kind, seq, pos0, n_tok;   // query rows
    int batch, max_blocks;
    int max_seq_len;              // host bound; device lengths are clamped to [1, max_seq_len]
    int n_hlist;                  // heads computed by a prefill attention launch
    uint8_t hlist[256];
    int sel_k;                    // selection: fixed top-k budget (0: top-p)
    int k_max;                    // top-p budget cap (0: none)
    int flags;                    // RTP_FLAG_* of the layer
    const int32_t* block_table;
    const int32_t* seq_lens;
    // KV layout.  k/v pages hold pool_heads KV heads (Hkv, or only the KV
    // heads that serve a retrieval head when a window-only ring holds the
    // rest); KV head g sits at slot kv_slot[g] of its pool, in the ring pool
    // (ring_heads per page, pages from ring_table) when kv_ring[g].
    int pool_heads, ring_heads, ring_pages;
    uint8_t kv_slot[256];
    uint8_t kv_ring[256];
    const int32_t* ring_table;    // [batch][ring_pages]
    const void* k_ring;
    const void* v_ring;
    int kv_fp8;                   // K/V stored as FP8 E4M3 codes
    float k_scale, v_scale;       // their scales (1 otherwise)
};

// Physical page of logical page lp (positions 256 lp ...) of sequence b for
// KV head g: the block table, or for a ring head entry 0 (positions 0..255,
// kept for the sinks) and entries 1..ring_pages-1 in rotation.
__device__ __forceinline__ int kv_page(const Geo& g, int b, int kvh, int lp) {
    if (g.kv_ring[kvh]) {
        const int e = lp == 0 ? 0 : 1 + (lp - 1) % (g.ring_pages - 1);
        return g.ring_table[(size_t)b * g.ring_pages + e];
    }
    return g.block_table[(size_t)b * g.max_blocks + lp];
}
// K/V row number (in units of D elements) of slot `slot` of `page` for KV head g.
__device__ __forceinline__ size_t kv_rowidx(const Geo& g, int page, int kvh, int slot) {
    return ((size_t)page * (g.kv_ring[kvh] ? g.ring_heads : g.pool_heads) + g.kv_slot[kvh]) * 256 + slot;
}

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
    int32_t mode;                 // 0 every key, 1 ordered list in SelWs::sel, 2 ordered list over the row's
                                  // scores (int32 indices written in place; the cut is (Tkey, jT))
    uint32_t Tkey;                // threshold: keys with score key > Tkey, or == Tkey and index <= jT
    int32_t jT;
    int32_t L;                    // keys of the row
    int32_t count;                // selected keys
    unsigned long long target;    // ceil(p Z), fixed point (a key count when unit)
    float d_thr;                  // U = keys with score >= d_thr
    int32_t unit;                 // the cut counts keys (fixed top-k, or the budget cap)
    int32_t path;                 // kPath* code of the row
    int32_t ks;                   // candidate threshold of the plan: U = keys with s (m - d) < ks / 4 (+ margin)
    int32_t has_jo;               // mode 1 cut in LDS: the K/V row numbers of the selected keys follow the
                                  // list, as uint32 in the row's SelWs::ubuf
};

constexpr int kChunk = 4096;      // keys per workgroup of the scoring pass
constexpr int kCB = 128;          // mass-histogram bins per chunk (1/4 unit of s (m_c - d) each)
constexpr int kCand = 8192;       // candidates ranked in LDS
constexpr int kCandG = 32768;     // candidates ranked from the workspace list (more: a cut over the scores)
constexpr int kLowBin = 15;       // chunk bins flagged per key by the scoring pass (x_c < 4 units)
constexpr int kFl = 512;         // entries of a chunk's list of flagged keys (more: the row takes the key masks)

// Device workspace of the selection, for `rows` rows of at most Lpad keys.
struct SelWs {
    float* scores;                // [rows][Lpad]
    int64_t score_ld;
    uint32_t* cmax;               // [rows][nchunk] ordered keys of chunk maxima
    uint16_t* qlow;               // [rows][16]
    unsigned long long* chist;    // [rows][nchunk][kCB] chunk mass histograms
    RowState* st;                 // [rows]
    uint32_t* sel;                // [rows][ucap] selected indices, ascending (mode 1)
    unsigned long long* ubuf;     // [rows][ucap] U in index order when it is gathered from the scores and
                                  // exceeds LDS: (score key << 32) | ~index
    unsigned* ccnt;               // [rows][nchunk][kCB] cumulative key counts of the chunk bins
    unsigned long long* kmask;    // [rows][Lpad / 64] bit j: key j lies in chunk bin <= kLowBin of its chunk
    unsigned long long* flist;    // [rows][nchunk][kFl] each chunk's flagged keys in index order,
                                  // (score key << 32) | ~index (its first kFl of them)
    int nchunk;
    int rows;                     // rows of this group
    int ucap;                     // row stride of ubuf / sel: min(kCandG, padded keys)
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
// The indexer keys of every sequence's last position (a decode step's tokens).
hipError_t launch_indexer_append_last(const Geo& g, const void* k, void* k_low, const void* w_k, int dtype,
                                      hipStream_t s);
// K and V of n new tokens ([n][Hkv][D]) into their pages (the ring for the
// ring heads) and their indexer keys, in one launch.
hipError_t launch_kv_append(const Geo& g, const void* k_new, const void* v_new, void* k, void* v, void* k_low,
                            const void* w_k, const int32_t* seq_id, const int32_t* pos, int n, int dtype,
                            hipStream_t s);

// Selection of rows [row0, row0 + ws.rows) of the call, all of it or one stage.
enum SelStage {
    kSelAll = 0,                  // scoring pass with statistics, then gather, cut, emit
    kSelScoresOnly = 1,           // projection and scores only (rtp_indexer_scores)
    kSelScorePass = 2,            // the first part of kSelAll
    kSelFinish = 3,               // the rest of kSelAll
    kSelRows = 4,                 // kSelAll without the emit: the row records hold the sets
};
// Local-head window work (bf16, D = 128, MFMA items) that the row pass of a
// decode step runs on its spare workgroups (kSelRows only): items = nsplit *
// batch * Hkv, partials [batch][Hq][nsplit][D + 2].
struct WinWork {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* part;
    int nsplit, split_keys, items;
};
constexpr int kWinCUs = 256;      // compute units of the part: the row pass and its window items fill them
// Indexer-key append fused into a decode step's scoring pass: the K cache
// (holding the new tokens' K rows) and W_k; w_k == nullptr: no append.
struct KeyAppend {
    const void* k;
    const void* w_k;
};
hipError_t launch_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                         const float* top_p, int row0, const SelWs& ws, const SelOut& out,
                         int total_rows, int dtype, int stage, hipStream_t s, const WinWork* win = nullptr,
                         const KeyAppend* app = nullptr);
// Path codes (kPath*) of the rows of the last selection, from its workspace.
hipError_t launch_select_paths(const SelWs& ws, int rows, int32_t* paths, hipStream_t s);

// Selected keys per work item (one wavefront) of the sparse decode: a row of
// n selected keys makes ceil(n / kSparseItem) partial results, so a call needs
// at most rows + capacity / kSparseItem + 1 of them.
constexpr int kSparseItem = 64;

// Split-K partial attention of retrieval rows over their selected sets and the combine.
struct AttnWs {
    float* part;                  // [items][D + 2] ([items][kGqaMax][D + 2] for shared gathers)
    int32_t* item_start;          // [rows + 1]
    int64_t max_items;
    // shared gathers of the retrieval heads of one KV head (a group of
    // consecutive retrieval rows of a token): the union of their selected keys
    // in the region of the group's first row
    uint32_t* ukey;               // [rows][ulen] union keys
    uint8_t* umask;               // [rows][ulen] bit i: key selected by the group's row i
    int32_t* ucnt;                // [rows] union size (first row of a group)
    int64_t ulen;
};
constexpr int kGqaMax = 4;        // retrieval heads per KV head served by one shared gather
// Rows [row0, row0 + rows) of the call (rows <= 4096); row_ptr is the full CSR array.
hipError_t launch_sparse_decode(const Geo& g, const void* q, const void* k, const void* v,
                                const int64_t* row_ptr, const int32_t* idx, const int32_t* status,
                                void* out, const AttnWs& ws, int row0, int rows, int dtype, hipStream_t s);

// The same from the selection's workspace (rows of one selection call, one
// group): each row's selected keys are read from its row record, and the
// items write the CSR output (row pointers, capacity check, indices).
// win (bf16 D = 128 only): the window partials written by the row pass are
// merged by the same combine launch.
hipError_t launch_sparse_decode_sel(const Geo& g, const void* q, const void* k, const void* v, const SelWs& sw,
                                    const SelOut& so, void* out, const AttnWs& ws, int rows, int dtype,
                                    const WinWork* win, hipStream_t s);
// The same with the retrieval heads of one KV head gathering the union of
// their selected keys once (bf16 or fp32 K/V): a union pass (which also writes
// the CSR), the sparse items over the unions, and the combine.
hipError_t launch_sparse_decode_gqa(const Geo& g, const void* q, const void* k, const void* v, const SelWs& sw,
                                    const SelOut& so, void* out, const AttnWs& ws, int rows, int dtype,
                                    const WinWork* win, hipStream_t s);

// Top-p selection of the rows of one prefill chunk (bf16, D <= 128): indexer
// scores of 32-row x 32-key tiles by MFMA as a filter, exact fixed-order
// scores only where they decide the set; same result as launch_select.
// Workspace: chunk_select_head_bytes at least; the rest is a pool of
// candidate entries, chunk_select_ws_bytes recommends 4096 per row.
size_t chunk_select_head_bytes(int rows, int n_ret, int n_keys);
size_t chunk_select_ws_bytes(int rows, int n_ret, int n_keys);
hipError_t launch_chunk_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                               const float* top_p, void* ws, size_t ws_bytes, const SelOut& out, hipStream_t s);
hipError_t launch_chunk_paths(const Geo& g, const void* ws, int32_t* paths, hipStream_t s);

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
