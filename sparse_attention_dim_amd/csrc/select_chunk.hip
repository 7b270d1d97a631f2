// select_chunk.hip -- top-p selection for a chunk of prefill rows on gfx950,
// with the indexer scores of every (row, key) pair formed by MFMA and exact
// fixed-order scores computed only where they decide the result.
//
// Method: arXiv 2605.16928 abstract obs. (2)-(3); zhichai.net forum post
// "RTPurbo: Turning Dense LLMs into Sparse Attention Models ...", "Three Key
// Insights" items 2-3.  The selected set is defined by the exact score
// d = fp32 chain over c = 0..15 of q_low[c] * k_low[c] (exact bf16 products),
// ranked by (d descending, index ascending), cut where the indexer-softmax mass
// reaches p.  Prefill rows of one retrieval head share every key, so the
// 16-wide contraction of a 32-key x 32-row tile is one
// v_mfma_f32_32x32x16_bf16.  The MFMA sum e is not the fixed-order chain, but
// |e - d| <= delta / 8 with delta = 2^-16 |q_low| max|k_low| (the chain's own
// rounding is at most ~2^-20 sum|q_c k_c| and the measured MFMA deviation is
// below 2^-21 sum|q_c k_c|).  Passes over the 32 rows x all keys of one head
// of a workgroup, one kernel each (so each runs at the occupancy its own
// registers and LDS allow):
//   P1  (k_csel_max) q_low and the row maxima of e: m' = max e + delta >=
//       max d (the largest key norm comes from a pre-pass over the head's
//       indexer keys);
//   P2  (k_csel_hist) mass histograms over x = s (m' - e) in bins of 1/4
//       (weights exp(-x) summed in fp64 LDS atomics); the cut bin with a
//       target raised by a margin that covers the approximation;
//       U = bins <= cut + 1.  Bins are far wider than s delta, so every key
//       ranked at or above the exact cut is in U.  Rows whose U is small
//       enough get a segment of a shared pool, sized by an upper bound of
//       U's size from the masses (a key of bin b weighs at least e^-(b+1)/4);
//   P3  (k_csel_rec) for those rows, the key indices of U into the segment.
//       The resolve pass forms U's exact scores and exact fixed-point
//       weights, U's exact mass (keys outside U enter the total with their
//       approximate fp64 weights: they hold at most the 1 - p tail, with a
//       relative error below s delta / 8), and the cut by radix selection;
//   levels (k_csel_main) a row without a segment (U too large, or the pool
//       full) scores U exactly in-lane and is narrowed by radix levels on the
//       exact score (extra passes behind the MFMA filter), then emitted by a
//       rescan.
// Every result is certified: the cut score must lie above every exact score
// that a key outside U can have, else the call reports status 2.
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTR = 32;          // rows per workgroup
constexpr int kProv = 40;        // P2 flags the key tiles holding a pair with x < kProv (U's tiles when ue < kProv)
constexpr int kHB = kProv + 1;   // P2 bins of x: one per unit below kProv, the last one open-ended
constexpr int kFlagWords = (1 << 20) / 1024;   // flag words of a row tile: one bit per 32-key tile, 2^20 keys
constexpr int kTileList = 16384; // flagged tiles the recording pass lists in LDS (more: it streams every tile)
constexpr float kBinsPerX = 4.0f;
constexpr int kNB = 64;          // radix buckets per level
constexpr int kNBP = kNB + 1;
constexpr int kCapC = 128;       // candidates of one cut bucket sorted in LDS
constexpr int kSmallU = 8192;    // U sorted by the per-row resolve kernel
constexpr int kTinyU = 1024;     // U sorted by the small-row resolve kernel
constexpr int kSegBlk = 4;       // segment slots reserved at a time by one lane of the third pass
constexpr int kSegPad = 8 * kSegBlk;   // 8 writers per row and run (4 waves x 2 halves): their last blocks' slack
// largest segment (U plus each run's padding), sorted by the large-row kernel:
// U of up to 16384 keys at the most runs, a multiple of its 512 threads
constexpr int kSegMax = 16384 + 512;
constexpr int kPoolPerRow = 4096;   // pool entries per row in the recommended workspace
constexpr int kNormKeys = 4096;  // keys per block of the key-norm pre-pass
constexpr float kLog2eF = 1.4426950408889634f;
constexpr unsigned long long kNoSeg = ~0ull;


// modes of a row
constexpr int kAll = 0;          // p >= 1: every key
constexpr int kLevel = 2;        // threshold found by radix levels (rescan emit)
constexpr int kBuf = 3;          // U held in the buffer (sorted by the resolve kernel)

// Per-row result of the main kernel (device workspace).
struct CRow {
    float mp;        // m' (upper bound of the row's exact maximum)
    float delta;     // 8x the |MFMA - exact| bound of the row
    float e_thr;     // a pair is in U iff its MFMA score e >= e_thr
    float T;         // exact score of the cut (kLevel)
    float d_edge;    // exact scores of keys outside U are <= d_edge
    int mode;
    int u_end;       // last P2 bin of U
    int n_tie;       // keys with d == T taken, lowest indices first (kLevel)
    int count;       // selected keys (kLevel) or used slots of the segment (kBuf)
    int bad;         // certification failed
    unsigned long long target;   // fixed-point mass to reach (kLevel)
    unsigned long long seg;      // pool offset of the row's segment (kBuf)
    unsigned long long light;    // approximate fixed-point mass of the keys outside U (kBuf)
    unsigned long long zex;      // exact fixed-point mass of every key of the row (retried rows), else 0
    int kcnt;        // > 0: the cut counts keys up to kcnt (fixed top-k or the budget cap); -3: invalid top_p
    int path;        // kPath* code (written by the resolvers)
};

// orders this wave's LDS writes before its following LDS reads (other lanes)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ void unpack8(uint4 a, float* f) {
    f[0] = __uint_as_float(a.x << 16); f[1] = __uint_as_float(a.x & 0xFFFF0000u);
    f[2] = __uint_as_float(a.y << 16); f[3] = __uint_as_float(a.y & 0xFFFF0000u);
    f[4] = __uint_as_float(a.z << 16); f[5] = __uint_as_float(a.z & 0xFFFF0000u);
    f[6] = __uint_as_float(a.w << 16); f[7] = __uint_as_float(a.w & 0xFFFF0000u);
}

// exact fixed-order score of one pair
__device__ __forceinline__ float exact_score(const float* q16, uint4 k0, uint4 k1) {
    float kf[16];
    unpack8(k0, kf);
    unpack8(k1, kf + 8);
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc = __builtin_fmaf(q16[c], kf[c], acc);
    return acc;
}

// P2 bin argument of an MFMA score, x = (m' - e) s kBinsPerX >= 0 (m' - e >=
// delta, far above the rounding of m' s kBinsPerX), and its bin.  The same
// operations run in every pass, so a pair's bin never changes.
__device__ __forceinline__ float bin_x(float e, float sB, float mpB) { return __builtin_fmaf(-e, sB, mpB); }
__device__ __forceinline__ int bin_of(float x) {
    return (int)__builtin_amdgcn_fmed3f(x, 0.0f, (float)(kHB - 1));
}

// Visits tiles first, first + stride, ... < ntile (a wave-uniform sequence)
// with D tile loads in flight: the A operand of tile it + D stride is
// requested before tile it is processed, and the page id that operand's
// address needs was requested D tiles earlier still (so waiting for it never
// waits for the operand loads issued since).  page(it) reads the page table;
// load(it, page) reads the tile's A operand.
template <int D, typename Page, typename Load, typename Body>
__device__ __forceinline__ void tile_loop(int first, int stride, int ntile, Page page, Load load, Body body) {
    // the loads run unconditionally on clamped tile numbers (the few past the
    // end repeat the last tile), so their waits count exactly.  The operands
    // sit in a ring of 2 D registers: tile t's operand is in slot t mod 2D
    // and the load of tile t + D goes to another slot, so no operand is ever
    // copied between registers (a copy would wait for its load).  The page
    // ids sit in a ring of 2 D as well, requested 2 D tiles ahead.
    const auto cl = [&](int it) { return min(it, ntile - 1); };
    constexpr int R = 2 * D;
    int pring[R];
    uint4 ring[R];
#pragma unroll
    for (int x = 0; x < R; ++x) pring[x] = page(cl(first + x * stride));
#pragma unroll
    for (int x = 0; x < D; ++x) {
        ring[x] = load(cl(first + x * stride), pring[x]);
        pring[x] = page(cl(first + (x + R) * stride));
    }
    for (int it0 = first; it0 < ntile; it0 += R * stride) {
#pragma unroll
        for (int x = 0; x < R; ++x) {
            const int it = it0 + x * stride;
            const int s = (x + D) % R;                  // the slot of tile it + D
            ring[s] = load(cl(it + D * stride), pring[s]);
            pring[s] = page(cl(it + (D + R) * stride));
            if (it < ntile) body(it, ring[x]);
        }
    }
}
constexpr int kPre = 8;          // tile loads requested ahead per wave
constexpr int kPreHist = 4;      // the same in the histogram, level and emit passes (registers set their occupancy)

// LDS of the radix levels: per-row bucket masses and counts and the gathered
// candidates of the last bucket.  (The P2 histograms are bin-major, [bin][row],
// so the bank of a lane's atomic depends on its row only.)
constexpr int kHmBytes = kTR * kNBP * 8;
constexpr int kHcBytes = kTR * kNBP * 4;
constexpr int kCandBytes = kTR * kCapC * 8;
constexpr int kLevelBytes = kHmBytes + kHcBytes + kCandBytes;
static_assert(kHmBytes % 16 == 0 && (kHmBytes + kHcBytes) % 8 == 0, "aligned level structures");

// Per-row state handed from the histogram pass to the later passes (device
// workspace, one record per row of the call).
struct CState {
    float mp;        // m' (upper bound of the row's exact maximum)
    float delta;     // 8x the |MFMA - exact| bound of the row
    float e_thr;     // a pair is in U iff its MFMA score e >= e_thr
    float edge;      // exact scores of keys outside U are <= edge
    uint32_t klo, khi, shift;   // exact-score key range of the level path and its first shift
    uint32_t ucount; // keys of U (exact: the runs' counts of pairs of bins <= uend)
    int mode;        // kAll or kLevel
    int uend;        // last P2 bin of U
    int kcnt;        // > 0: the cut counts keys (fixed top-k, or a keep-all row capped); -3: invalid top_p
    int pad1;
    unsigned long long seg;     // pool offset of the row's segment, kNoSeg if none
    unsigned long long light;   // approximate fixed-point mass of the keys outside U
};

// Coordinates (row tile, retrieval head, run of key tiles) of a workgroup
// of an (nt, n_ret, runs) grid, remapped so that the workgroups one XCD
// receives (the dispatcher deals consecutive workgroups out over the 8 XCDs
// in turn) share one (head, run) and walk its row tiles in order: they stream
// the same key tiles at about the same time, which that XCD's L2 then serves
// once (long contexts, where a head's indexer keys overflow what the L2s and
// the last-level cache keep between passes).  Grids whose size is not a
// multiple of 8, and short contexts, keep their order.
constexpr int kXcd = 8;
constexpr int kXcdMinKeys = 1 << 19;
struct Blk {
    int x, y, z;
};
__device__ __forceinline__ Blk xcd_blk(const Geo& g) {
    const int nx = gridDim.x, ny = gridDim.y, n = nx * ny * gridDim.z;
    Blk b{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
    if (n % kXcd || g.pos0 + g.n_tok < kXcdMinKeys) return b;
    const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const int lam = (lin % kXcd) * (n / kXcd) + lin / kXcd;
    b.x = lam % nx;
    b.y = (lam / nx) % ny;
    b.z = lam / (nx * ny);
    return b;
}

// The MFMA tile view of one workgroup: rows t0 .. t0 + 31 of retrieval head r,
// lane row lr = lane % 32 and half hh = lane / 32; tile `it` covers keys
// it*32 .. it*32 + 31 (A operand: k_low[key it*32 + lr][8 hh .. 8 hh + 7],
// B operand: q_low[lr][8 hh .. 8 hh + 7]).
struct TileCtx {
    int r, t0, n_valid, lr, hh, pos, L_max, ntile, nfull;
    bool row_ok;
    const int32_t* bt;
    const bf16_t* k_low;
    int n_ret;
    uint4 qb;
    __device__ int page(int it) const { return bt[min(it * 32 + lr, L_max - 1) >> 8]; }
    __device__ uint4 load(int it, int pg) const {
        const int kk = min(it * 32 + lr, L_max - 1);
        return *reinterpret_cast<const uint4*>(k_low + (((size_t)pg * n_ret + r) * kBlk + (kk & 255)) * 16 + 8 * hh);
    }
    __device__ f32x16_t mfma(const uint4& a) const {
        f32x16_t acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qb), acc, 0, 0, 0);
    }
    __device__ int key_of(int it, int i) const { return it * 32 + (i >> 2) * 8 + 4 * hh + (i & 3); }
};

// rows t0 .. t0 + n_valid - 1 with q_low in qs; keys below L_max are visited
__device__ TileCtx tile_ctx_at(const Geo& g, const bf16_t* k_low, const float (*qs)[16], int r, int t0, int n_valid,
                               int L_max) {
    TileCtx c;
    const int lane = threadIdx.x & 63;
    c.r = r;
    c.t0 = t0;
    c.n_valid = n_valid;
    c.lr = lane & 31;
    c.hh = lane >> 5;
    c.row_ok = c.lr < c.n_valid;
    c.pos = g.pos0 + c.t0 + c.lr;
    c.L_max = L_max;
    c.ntile = (c.L_max + 31) / 32;
    c.nfull = (g.pos0 + c.t0 + 1) / 32;
    c.bt = g.block_table + (size_t)g.seq * g.max_blocks;
    c.k_low = k_low;
    c.n_ret = g.n_ret;
    uint32_t w4[4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
        w4[x] = (__float_as_uint(qs[c.lr][8 * c.hh + 2 * x]) >> 16) |
                (__float_as_uint(qs[c.lr][8 * c.hh + 2 * x + 1]) & 0xFFFF0000u);
    c.qb = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    return c;
}

// the view of row tile rt (rows 32 rt ...) of retrieval head r
__device__ TileCtx tile_ctx(const Geo& g, const bf16_t* k_low, const float (*qs)[16], int rt, int r) {
    const int t0 = rt * kTR, n_valid = min(kTR, g.n_tok - t0);
    return tile_ctx_at(g, k_low, qs, r, t0, n_valid, g.pos0 + t0 + n_valid);
}

// q_low of row tile rt of retrieval head r as floats (zero for rows past the chunk)
__device__ void load_qs(const Geo& g, const uint16_t* __restrict__ qlow, float (*qs)[16], int rt, int r) {
    const int t0 = rt * kTR;
    const int n_valid = min(kTR, g.n_tok - t0);
    for (int o = threadIdx.x; o < kTR * 16; o += 256) {
        const int lr = o >> 4, c = o & 15;
        qs[lr][c] = lr < n_valid ? bf2f(qlow[((size_t)(t0 + lr) * g.n_ret + r) * 16 + c]) : 0.0f;
    }
}

// The histogram pass splits each row tile's key tiles over several
// workgroups: their histograms and tile flags meet in these device
// accumulators (zeroed by P1), and the last workgroup of a row tile to
// arrive takes the epilogue.
constexpr int kMaxSplit = 8;     // most runs of key tiles per row tile
static_assert(kSegMax >= 16384 + kMaxSplit * kSegPad, "a segment holds U of 16384 keys at the most runs");

struct HistAcc {
    double* hist;        // [rows][kHB], rows in result-record order
    uint32_t* cnt;       // [rows][nsplit][kProv]: pairs per bin below kProv, per run
    uint32_t* segoff;    // [rows][nsplit]: slot of each run's part of the row's segment
    uint32_t* tflags;    // [n_ret][nt32][nfw + 1]
    uint32_t* arrive;    // [n_ret][nt32]
    uint32_t* lrows;     // result records of the rows with U > kSmallU (the large-row resolve's list)
    uint32_t* mrows;     // result records of the rows with kTinyU < U <= kSmallU (the per-row resolve's list)
    uint32_t* zrows;     // rows whose cut is retried with the exact normaliser (or counted under the cap)
    unsigned long long* lctr;   // [0], [1]: entries of lrows and the next one taken; [2], [3]: the same of mrows;
                                // [4]: entries of zrows, [5], [6]: the next item of the exact-mass pass and
                                // of the retried resolve
    int nt32, nfw, nsplit;
};

// the run of key tiles [tb, te) of split z of a row tile with ntile tiles
__device__ __forceinline__ void split_run(int z, int nsplit, int ntile, int& tb, int& te) {
    const int ns = min(nsplit, ntile);
    tb = z < ns ? (int)((long long)z * ntile / ns) : 0;
    te = z < ns ? (int)((long long)(z + 1) * ntile / ns) : 0;
}

// ---------------------------------------------------------------------------
// P1.  grid (ceil(n_tok / 256), n_ret, runs), 256 threads: the row maxima of
// the MFMA scores over one run of key tiles, for 256 rows (eight 32-row
// slices): every key tile read feeds the eight slices' MFMAs, so the head's
// indexer keys are streamed once per 256 rows.  The runs' maxima meet in
// rmaxk by atomicMax (zeroed with q_low by the key-norm pass); the histogram
// pass forms m' = max e + delta >= max d from them.  The first run writes
// delta (the largest key norm comes from the key-norm pass) and zeroes the
// histogram pass's accumulators of its rows.
// ---------------------------------------------------------------------------
constexpr int kTRM = 256;                // rows per P1 workgroup
constexpr int kSlices = kTRM / kTR;
__global__ __launch_bounds__(256) void k_csel_max(Geo g, const bf16_t* __restrict__ k_low,
                                                  const uint16_t* __restrict__ qlow, const float* __restrict__ knorm,
                                                  int nblk, CState* __restrict__ st, uint32_t* __restrict__ rmaxk,
                                                  HistAcc acc, int nrun) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const Blk bk = xcd_blk(g);
    const int r = bk.y, t0 = bk.x * kTRM, z = bk.z;
    const int n_valid = min(kTRM, g.n_tok - t0);
    if (z == 0) {
        // the histogram pass's accumulators of these rows start at zero
        for (int x = tid; x < n_valid * kHB; x += 256)
            acc.hist[((size_t)(t0 + x / kHB) * g.n_ret + r) * kHB + x % kHB] = 0.0;
        for (int hf = 0; hf < kSlices && t0 + hf * kTR < g.n_tok; ++hf) {
            const size_t rt = (size_t)r * acc.nt32 + kSlices * bk.x + hf;
            for (int x = tid; x <= acc.nfw; x += 256) acc.tflags[rt * (acc.nfw + 1) + x] = 0u;
            if (tid == 0) acc.arrive[rt] = 0u;
        }
    }
    __shared__ float qs[kTRM][16];
    __shared__ uint32_t rmax[kTRM];
    __shared__ uint32_t kmax_bits;
    for (int o = tid; o < kTRM * 16; o += 256) {
        const int lr = o >> 4, c = o & 15;
        qs[lr][c] = lr < n_valid ? bf2f(qlow[((size_t)(t0 + lr) * g.n_ret + r) * 16 + c]) : 0.0f;
    }
    rmax[tid] = 0u;
    if (tid == 0) kmax_bits = 0u;
    __syncthreads();
    const int lr = lane & 31, hh = lane >> 5;
    uint4 qb[kSlices];
#pragma unroll
    for (int j = 0; j < kSlices; ++j) {
        uint32_t w4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
            w4[x] = (__float_as_uint(qs[kTR * j + lr][8 * hh + 2 * x]) >> 16) |
                    (__float_as_uint(qs[kTR * j + lr][8 * hh + 2 * x + 1]) & 0xFFFF0000u);
        qb[j] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    const int L_max = g.pos0 + t0 + n_valid;              // keys the group's rows see
    const int ntile = (L_max + 31) / 32;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;
    int tb, te;
    split_run(z, nrun, ntile, tb, te);
    float mx[kSlices];
#pragma unroll
    for (int j = 0; j < kSlices; ++j) mx[j] = -INFINITY;
    const auto page = [&](int it) { return bt[min(it * 32 + lr, L_max - 1) >> 8]; };
    const auto load = [&](int it, int pg) {
        const int kk = min(it * 32 + lr, L_max - 1);
        return *reinterpret_cast<const uint4*>(k_low + (((size_t)pg * g.n_ret + r) * kBlk + (kk & 255)) * 16 + 8 * hh);
    };
    tile_loop<kPreHist>(tb + wid, 4, te, page, load, [&](int it, const uint4& cur) {
#pragma unroll
        for (int j = 0; j < kSlices; ++j) {
            if (kTR * j >= n_valid) continue;                 // (uniform)
            f32x16_t sc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[i] = 0.0f;
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(qb[j]), sc, 0, 0, 0);
            // tiles below the slice's first row's position hold keys every
            // row of the slice sees
            if (it < (g.pos0 + t0 + kTR * j + 1) / 32) {
#pragma unroll
                for (int i = 0; i < 16; ++i) mx[j] = fmaxf(mx[j], sc[i]);
            } else {
                const int pos = g.pos0 + t0 + kTR * j + lr;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    mx[j] = fmaxf(mx[j], it * 32 + (i >> 2) * 8 + 4 * hh + (i & 3) <= pos ? sc[i] : -INFINITY);
            }
        }
    });
#pragma unroll
    for (int j = 0; j < kSlices; ++j) {
        const float m = fmaxf(mx[j], __shfl_xor(mx[j], 32));
        if (hh == 0 && kTR * j + lr < n_valid && m > -INFINITY) atomicMax(&rmax[kTR * j + lr], score_key(m));
    }
    if (z == 0) {
        float kn = 0.0f;
        for (int b = tid; b < nblk; b += 256) kn = fmaxf(kn, knorm[(size_t)r * nblk + b]);
        kn = wave_max(kn);
        if (lane == 0) atomicMax(&kmax_bits, __float_as_uint(kn));
    }
    __syncthreads();
    if (tid < n_valid) {
        if (rmax[tid]) atomicMax(&rmaxk[(size_t)(t0 + tid) * g.n_ret + r], rmax[tid]);
        if (z == 0) {
            float qn2 = 0.0f;
            for (int c = 0; c < 16; ++c) qn2 = __builtin_fmaf(qs[tid][c], qs[tid][c], qn2);
            // delta exceeds the true deviation bound by a factor >= 8, far more
            // than the rounding of this sum: m' >= every exact score of the row
            st[(size_t)(t0 + tid) * g.n_ret + r].delta =
                0x1.0p-16f * sqrtf(qn2) * sqrtf(__uint_as_float(kmax_bits)) * 1.0009765625f;
        }
    }
}

// ---------------------------------------------------------------------------
// P2.  grid (ceil(n_tok / 32), n_ret, nsplit), 256 threads: workgroup z takes
// the z-th of nsplit equal runs of the row tile's key tiles.  Mass histograms
// over x = s (m' - e) in bins of 1/4 (weights exp(-x) summed in fp64 LDS
// atomics, then added into the device accumulators); the last workgroup of
// the row tile: the cut bin with a target raised by a margin that covers the
// approximation; U = bins <= cut + 1; pool segments, sized exactly from the
// runs' counts of U's pairs (one part per run), and the result records of the
// rows whose U fits one.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_csel_hist(Geo g, const bf16_t* __restrict__ k_low,
                                                   const float* __restrict__ top_p,
                                                   const uint16_t* __restrict__ qlow, CState* __restrict__ st,
                                                   const uint32_t* __restrict__ rmaxk,
                                                   unsigned long long* __restrict__ pool_ctr,
                                                   unsigned long long pool_cap, HistAcc acc,
                                                   CRow* __restrict__ rows_out) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const float s = g.idx_scale;
    const float sB = s * kBinsPerX;
    const int nfw = acc.nfw;
    __shared__ double hist[kHB][kTR];
    __shared__ uint32_t hcnt[kProv][kTR];                // pairs per bin below kProv (this run)
    __shared__ int s_last;
    __shared__ uint32_t tflag[kFlagWords];              // key tiles holding a pair with x < kProv
    __shared__ int s_full;                              // a row's U reaches past kProv: no tile list
    __shared__ float qs[kTR][16];
    __shared__ float r_mp[kTR], r_delta[kTR];
    __shared__ uint32_t r_tot[kTR], r_cz[kTR][kMaxSplit];
    __shared__ unsigned long long r_seg[kTR];
    __shared__ int r_mode[kTR], r_uend[kTR];
    const Blk bk = xcd_blk(g);
    load_qs(g, qlow, qs, bk.x, bk.y);
    const int r = bk.y, t0 = bk.x * kTR;
    const int n_valid = min(kTR, g.n_tok - t0);
    if (tid < kTR) {
        // m' = max e + delta from the maximum pass
        const size_t row = (size_t)(t0 + min(tid, n_valid - 1)) * g.n_ret + r;
        r_delta[tid] = st[row].delta;
        r_mp[tid] = key_score(rmaxk[row]) + r_delta[tid];
    }
    for (int x = tid; x < kHB * kTR; x += 256) (&hist[0][0])[x] = 0.0;
    for (int x = tid; x < kProv * kTR; x += 256) (&hcnt[0][0])[x] = 0u;
    for (int x = tid; x < nfw; x += 256) tflag[x] = 0u;
    if (tid == 0) s_full = 0;
    __syncthreads();
    const TileCtx tc = tile_ctx(g, k_low, qs, bk.x, bk.y);
    const float mpB = r_mp[tc.lr] * sB;
    // this workgroup's run of key tiles (none when the row tile has fewer
    // tiles than splits)
    const int z = bk.z;
    int tb, te;
    split_run(z, acc.nsplit, tc.ntile, tb, te);
    if (te > tb) {
        constexpr float kW = -kLog2eF / kBinsPerX;       // exp(-x / 4) = 2^(x kW)
        // Pairs of the open-ended last bin (x >= kProv, weights below e^-10 of
        // the row maximum) are summed in registers: a float sum per tile (16
        // terms, relative error < 2^-20), added to a double per lane.  Only
        // the pairs below kProv take an LDS atomic of their bin.  In a full
        // tile the weights come first, each from one FMA and one exp2:
        // 2^(e cA + cB) with cA = -sB kW, cB = m' sB kW, whose argument is
        // within 2^-23 |arg| + 2^-24 s log2(e) (|e| + 2 |m'|) of the exact
        // s log2(e) (e - m') (the constants' and the FMA's roundings); a
        // pair with x < kProv weighs more than e^-10 on its own, so a wave
        // whose lanes all sum below kNearW holds none and skips the bins
        // and the exact test (the binned loop reuses the weights).
        const float cA = -sB * kW, cB = mpB * kW;
        constexpr float kNearW = 4.53e-05f;              // below e^-10 by more than the weights' error
        double* hrow = &hist[0][tc.lr];
        double far = 0.0;
        tile_loop<kPreHist>(tb + wid, 4, te, [&](int it) { return tc.page(it); },
                    [&](int it, int pg) { return tc.load(it, pg); }, [&](int it, const uint4& cur) {
            const f32x16_t sc = tc.mfma(cur);
            if (it < tc.nfull) {
                float w[16];
                float f = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    w[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cA, cB));
                    f += w[i];
                }
                if (__ballot(f >= kNearW) != 0ull) {
                    // a lane may hold a pair below kProv: the exact test per
                    // pair; those pairs take their bins with the weights
                    // above, the others are summed again without them
                    f = 0.0f;
                    bool any = false;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float x = bin_x(sc[i], sB, mpB);
                        const bool nr = x < (float)kProv;
                        any |= nr;
                        f += nr ? 0.0f : w[i];
                        if (nr) {
                            const int b = bin_of(x);
                            atomicAdd(&hrow[b * kTR], (double)w[i]);
                            atomicAdd(&hcnt[b][tc.lr], 1u);
                        }
                    }
                    if (__ballot(any) != 0ull && lane == 0) atomicOr(&tflag[it >> 5], 1u << (it & 31));
                }
                far += (double)f;
                return;
            }
            float mx = sc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
            if (__ballot(bin_x(mx, sB, mpB) < (float)kProv) != 0ull && lane == 0)
                atomicOr(&tflag[it >> 5], 1u << (it & 31));
            float f = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float x = bin_x(sc[i], sB, mpB);
                const float w = __builtin_amdgcn_exp2f(x * kW);
                if (tc.key_of(it, i) <= tc.pos) {
                    if (x < (float)kProv) {
                        const int b = bin_of(x);
                        atomicAdd(&hrow[b * kTR], (double)w);
                        atomicAdd(&hcnt[b][tc.lr], 1u);
                    } else {
                        f += w;
                    }
                }
            }
            far += (double)f;
        });
        atomicAdd(&hrow[(kHB - 1) * kTR], far);
    }
    __syncthreads();
    const size_t rt = (size_t)r * acc.nt32 + bk.x;          // the row tile
    uint32_t* tf = acc.tflags + rt * (nfw + 1);
    for (int x = tid; x < kProv * n_valid; x += 256) {
        const int row = x / kProv, b = x - row * kProv;
        acc.cnt[(((size_t)(t0 + row) * g.n_ret + r) * acc.nsplit + z) * kProv + b] = hcnt[b][row];
    }
    __syncthreads();                                     // (read back by the epilogue when nsplit == 1)
    if (acc.nsplit > 1) {
        // add this run's histograms and flags into the accumulators; the
        // last workgroup of the row tile to arrive reads them back
        for (int x = tid; x < kHB * n_valid; x += 256) {
            const int b = x / n_valid, row = x - b * n_valid;
            const double v = hist[b][row];
            if (v != 0.0) unsafeAtomicAdd(&acc.hist[((size_t)(t0 + row) * g.n_ret + r) * kHB + b], v);
        }
        for (int x = tid; x < nfw; x += 256)
            if (tflag[x]) atomicOr(&tf[x], tflag[x]);
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = atomicAdd(&acc.arrive[rt], 1u) == (uint32_t)(acc.nsplit - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        for (int x = tid; x < kHB * kTR; x += 256) {
            const int b = x / kTR, row = x - b * kTR;
            hist[b][row] = row < n_valid ? __hip_atomic_load(&acc.hist[((size_t)(t0 + row) * g.n_ret + r) * kHB + b],
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                         : 0.0;
        }
        __syncthreads();
    } else {
        for (int x = tid; x < nfw; x += 256) tf[x] = tflag[x];
    }
    // cut bin of the approximate masses, U = bins <= cut + 1.  The target
    // carries a margin eta that covers the relative error of the approximate
    // weights (<= s delta / 8 plus the exp2 rounding); U is every key when the
    // bins are not wide against delta.
    if (tid < n_valid) {
        const int row = tid;
        const float p = g.sel_k > 0 ? 1.0f : top_p[g.seq];
        const int pos = g.pos0 + t0 + row;
        // a count target: the fixed top-k budget, or the cap of a keep-all row
        const int kc = g.sel_k > 0 ? g.sel_k : (!(p < 1.0f) && g.k_max > 0 ? g.k_max : 0);
        CState o;
        o.mp = r_mp[row];
        o.delta = r_delta[row];
        o.mode = kLevel;
        o.uend = kHB - 1;
        o.edge = -INFINITY;
        o.light = 0ull;
        o.ucount = 0u;
        o.seg = kNoSeg;
        o.e_thr = -INFINITY;
        o.klo = 0u;
        o.khi = 0u;
        o.shift = 0u;
        o.kcnt = 0;
        o.pad1 = 0;
        if (g.sel_k <= 0 && !(p > 0.0f)) {
            o.mode = kAll;                               // NaN or p <= 0: reported, nothing selected
            o.kcnt = -3;
        } else if (kc > 0 ? kc >= pos + 1 : !(p < 1.0f)) {
            o.mode = kAll;
        } else {
            const double sd = (double)s * (double)r_delta[row];
            int bc = kHB - 1;
            if (kc > 0) {
                // count cut: the first bin whose cumulative pair count reaches
                // kc (pairs past kProv are not counted per bin: U is then
                // every key)
                o.kcnt = kc;
                uint32_t cum = 0u;
                for (int b = 0; b < kProv; ++b) {
                    for (int zz = 0; zz < acc.nsplit; ++zz)
                        cum += acc.cnt[(((size_t)(t0 + row) * g.n_ret + r) * acc.nsplit + zz) * kProv + b];
                    if (cum >= (uint32_t)kc) {
                        bc = b;
                        break;
                    }
                }
            } else {
                double Z = 0.0;
                for (int b = 0; b < kHB; ++b) Z += hist[b][row];
                const double tgt_a = (double)p * (1.0 + sd + 0x1.0p-16) * Z;
                double cum = 0.0;
                for (int b = 0; b < kHB; ++b) {
                    cum += hist[b][row];
                    if (cum >= tgt_a) {
                        bc = b;
                        break;
                    }
                }
            }
            const int ue = (sd < 1.0 / 64.0) ? min(bc + 1, kHB - 1) : kHB - 1;
            double light = 0.0;
            if (kc == 0)
                for (int b = ue + 1; b < kHB; ++b) light += hist[b][row];
            // the keys of U in each run of key tiles, exactly: the pairs of
            // bins <= ue counted by every run (every key of the run when U
            // is all of them); the row's segment holds run after run, each
            // with kSegPad slots of slack for its writers' last blocks
            uint32_t uc = 0u, tot = 0u;
            for (int zz = 0; zz < acc.nsplit; ++zz) {
                uint32_t c = 0u;
                if (ue < kHB - 1) {
                    const uint32_t* cr = acc.cnt + (((size_t)(t0 + row) * g.n_ret + r) * acc.nsplit + zz) * kProv;
                    for (int b = 0; b <= ue; ++b) c += cr[b];
                } else {
                    int rb, re;
                    split_run(zz, acc.nsplit, tc.ntile, rb, re);
                    c = (uint32_t)max(0, min(32 * re, pos + 1) - 32 * rb);
                }
                r_cz[row][zz] = c;
                uc += c;
                tot += c + kSegPad;
            }
            o.ucount = uc;
            r_tot[row] = tot;
            o.uend = ue;
            o.light = (unsigned long long)__double2ll_rn(light * kFix);
            const double mp = (double)o.mp;
            if (ue == kHB - 1) {
                o.klo = 0u;                               // every key is in U
            } else {
                // the smallest MFMA score whose bin is <= ue (the bin is
                // monotone in the score, so U is e >= e_thr)
                const float mpBr = o.mp * sB;
                uint32_t klo = score_key(-INFINITY), khi = score_key(o.mp);
                while (klo < khi) {
                    const uint32_t mid = klo + ((khi - klo) >> 1);
                    if (bin_of(bin_x(key_score(mid), sB, mpBr)) <= ue) khi = mid; else klo = mid + 1;
                }
                o.e_thr = key_score(khi);
                // keys of U: x < (ue + 1) / 4, so e > m' - (ue + 1) / (4 s);
                // keys outside: the reverse.  The margin covers the float
                // rounding of the bin argument and the MFMA deviation.
                const double span = (double)(ue + 1) / ((double)kBinsPerX * (double)s);
                const double marg = 0x1.0p-18 * (span + 2.0 * fabs(mp)) + 2.0 * (double)o.delta;
                o.klo = score_key(__double2float_rd(mp - span - marg));
                o.edge = __double2float_ru(mp - span + marg);
            }
            o.khi = score_key(o.mp);
            const uint32_t spn = o.khi - o.klo;
            const int bits = spn ? 32 - __clz(spn) : 0;
            o.shift = bits > 6 ? bits - 6 : 0;
        }
        r_mode[row] = o.mode;
        r_uend[row] = o.uend;
        r_seg[row] = kNoSeg;
        st[(size_t)(t0 + row) * g.n_ret + r] = o;
    }
    __syncthreads();
    // pool segments for the rows whose U fits the largest segment (one
    // allocation per workgroup; a full pool sends the rows to the radix levels)
    if (tid == 0) {
        unsigned long long tot = 0;
        for (int row = 0; row < n_valid; ++row)
            if (r_mode[row] == kLevel && r_tot[row] <= (uint32_t)kSegMax) tot += r_tot[row];
        if (tot) {
            const unsigned long long base = atomicAdd(pool_ctr, tot);
            if (base + tot <= pool_cap) {
                unsigned long long off = base;
                for (int row = 0; row < n_valid; ++row)
                    if (r_mode[row] == kLevel && r_tot[row] <= (uint32_t)kSegMax) {
                        r_seg[row] = off;
                        off += r_tot[row];
                        if (r_uend[row] >= kProv) s_full = 1;   // a recorded U past the flagged tiles
                    }
            }
        }
    }
    __syncthreads();
    // each pooled row: its segment, the runs' places in it, and its result
    // record (the recording pass fills the segment; the resolve reads it)
    if (tid < n_valid && r_seg[tid] != kNoSeg) {
        const size_t rg = (size_t)(t0 + tid) * g.n_ret + r;
        CState* c = st + rg;
        c->seg = r_seg[tid];
        uint32_t off = 0u;
        for (int zz = 0; zz < acc.nsplit; ++zz) {
            acc.segoff[rg * acc.nsplit + zz] = off;
            off += r_cz[tid][zz] + kSegPad;
        }
        CRow out;
        out.mp = c->mp;
        out.delta = c->delta;
        out.e_thr = c->e_thr;
        out.T = 0.0f;
        out.d_edge = c->edge;
        out.mode = kBuf;
        out.u_end = c->uend;
        out.n_tie = 0;
        out.count = (int)r_tot[tid];
        out.bad = 0;
        out.target = 0ull;
        out.seg = r_seg[tid];
        out.light = c->light;
        out.zex = 0ull;
        out.kcnt = c->kcnt;
        out.path = 0;
        rows_out[rg] = out;
        if (out.count > kSmallU)
            acc.lrows[atomicAdd(&acc.lctr[0], 1ull)] = (uint32_t)rg;
        else if (out.count > kTinyU)
            acc.mrows[atomicAdd(&acc.lctr[2], 1ull)] = (uint32_t)rg;
    }
    // whether the row tile's key-tile flags suffice (last word)
    if (tid == 0) tf[nfw] = (uint32_t)s_full;
}

// ---------------------------------------------------------------------------
// P3.  grid (ceil(n_tok / 32), n_ret, nsplit), 256 threads: workgroup z
// records, for the rows with a pool segment, the key indices of U (MFMA score
// >= e_thr) found in run z of the key tiles (the runs of P2) into that run's
// part of the segment, slots reserved kSegBlk at a time per lane; the slack
// of each lane's last block and the part's unused tail are marked empty.
// A writer (wave, half) visits its keys in increasing order and the runs'
// parts follow each other in key order, so each writer's entries, read in
// slot order, ascend.  The rows' result records were written by P2.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_csel_rec(Geo g, const bf16_t* __restrict__ k_low,
                                                  const uint16_t* __restrict__ qlow, CState* __restrict__ st,
                                                  unsigned long long* __restrict__ pool, HistAcc acc) {
    const int tid = threadIdx.x, wid = tid >> 6;
    const Blk bk = xcd_blk(g);
    const int r = bk.y, t0 = bk.x * kTR, z = bk.z;
    const int n_valid = min(kTR, g.n_tok - t0);
    const int nfw = acc.nfw;
    __shared__ float qs[kTR][16];
    __shared__ CState rs[kTR];
    __shared__ uint32_t ucnt[kTR], ucap[kTR];
    __shared__ unsigned long long ubase[kTR];
    __shared__ uint16_t tlist[kTileList];               // the flagged key tiles of the run, ascending
    __shared__ unsigned long long scan_sh[256 / 64 + 1];
    __shared__ int s_any;
    if (tid == 0) s_any = 0;
    __syncthreads();
    if (tid < n_valid) {
        const size_t rg = (size_t)(t0 + tid) * g.n_ret + r;
        rs[tid] = st[rg];
        ucnt[tid] = 0u;
        ucap[tid] = 0u;
        ubase[tid] = 0ull;
        if (rs[tid].mode == kLevel && rs[tid].seg != kNoSeg) {
            const uint32_t o0 = acc.segoff[rg * acc.nsplit + z];
            const uint32_t o1 = z + 1 < acc.nsplit ? acc.segoff[rg * acc.nsplit + z + 1]
                                                   : rs[tid].ucount + (uint32_t)(acc.nsplit * kSegPad);
            ubase[tid] = rs[tid].seg + o0;
            ucap[tid] = o1 - o0;
            s_any = 1;
        }
    }
    __syncthreads();
    if (!s_any) return;
    load_qs(g, qlow, qs, bk.x, bk.y);
    __syncthreads();                                     // qs complete before the tile view reads it
    const TileCtx tc = tile_ctx(g, k_low, qs, bk.x, bk.y);
    int tb, te;
    split_run(z, acc.nsplit, tc.ntile, tb, te);
    // The run's key tiles that can hold a key of U (flagged by the histogram
    // pass), listed in LDS; every tile of the run when a row's U reaches past
    // the flagged bins or the list does not fit.
    const uint32_t* tf = acc.tflags + ((size_t)r * acc.nt32 + bk.x) * (nfw + 1);
    int nlist = -1;                                      // -1: every tile of the run
    if (tf[nfw] == 0u) {
        constexpr int kPerT = kFlagWords / 256;          // flag words per thread
        const int wb = tid * kPerT, we = min(wb + kPerT, nfw);
        const auto bits_of = [&](int w) {
            uint32_t bits = tf[w];
            const int k0 = 32 * w;                       // keep tiles tb <= k < te
            if (k0 < tb) bits &= tb - k0 >= 32 ? 0u : ~0u << (tb - k0);
            if (k0 + 32 > te) bits &= te - k0 <= 0 ? 0u : ~0u >> (32 - (te - k0));
            return bits;
        };
        uint32_t c = 0u;
        for (int w = wb; w < we; ++w) c += __popc(bits_of(w));
        unsigned long long tot;
        uint32_t o = (uint32_t)block_excl_scan_u64<256>(c, &tot, scan_sh);
        if (tot <= (unsigned long long)kTileList) {
            for (int w = wb; w < we; ++w) {
                uint32_t bits = bits_of(w);
                while (bits) {
                    const int b = __ffs(bits) - 1;
                    bits &= bits - 1u;
                    tlist[o++] = (uint16_t)(32 * w + b);
                }
            }
            nlist = (int)tot;
        }
    }
    __syncthreads();
    const int lr = tc.lr;
    const bool pooled = tc.row_ok && rs[lr].mode == kLevel && rs[lr].seg != kNoSeg;
    const unsigned long long sg = pooled ? ubase[lr] : 0ull;
    const uint32_t scap = pooled ? ucap[lr] : 0u;
    const float e_fast = pooled ? rs[lr].e_thr : INFINITY;
    uint32_t bp = 0u, be = 0u;                          // the lane's reserved block [bp, be)
    // entry: (writer << 24) | key
    const unsigned long long wtag = (unsigned long long)(wid * 2 + tc.hh) << 24;
    const auto record = [&](int key) {
        if (bp == be) {
            bp = atomicAdd(&ucnt[lr], (uint32_t)kSegBlk);
            be = bp + kSegBlk;
        }
        if (bp < scap) pool[sg + bp] = wtag | (unsigned long long)(uint32_t)key;
        ++bp;
    };
    const auto body = [&](int it, const uint4& cur) {
        const f32x16_t sc = tc.mfma(cur);
        // U is a small part of the keys: one test of the lane's largest score
        // skips nearly every tile
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
        if (!__ballot(mx >= e_fast)) return;
        if (it < tc.nfull) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (sc[i] >= e_fast) record(tc.key_of(it, i));
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (sc[i] >= e_fast && tc.key_of(it, i) <= tc.pos) record(tc.key_of(it, i));
        }
    };
    // the listed tiles only (in increasing order per wave, so a writer's
    // entries still ascend), or every tile of the run
    const bool use_list = nlist >= 0;
    const int nvirt = use_list ? nlist : te - tb;
    const auto tile_of = [&](int k) { return use_list ? (int)tlist[min(k, kTileList - 1)] : tb + k; };
    if (nvirt > 0)
        tile_loop<kPre>(wid, 4, nvirt, [&](int k) { return tc.page(tile_of(k)); },
                        [&](int k, int pg) { return tc.load(tile_of(k), pg); },
                        [&](int k, const uint4& cur) { body(tile_of(k), cur); });
    for (uint32_t x = bp; x < be; ++x)
        if (x < scap) pool[sg + x] = ~0ull;               // unused slots of the last block
    __syncthreads();
    // the part's unreserved tail; a part that overflowed sends the row to the
    // radix levels (exact counts: a safeguard)
    for (int row = 0; row < n_valid; ++row) {
        if (rs[row].mode != kLevel || rs[row].seg == kNoSeg) continue;
        for (uint32_t x = ucnt[row] + tid; x < ucap[row]; x += 256) pool[ubase[row] + x] = ~0ull;
    }
    if (tid < n_valid && rs[tid].mode == kLevel && rs[tid].seg != kNoSeg && ucnt[tid] > ucap[tid])
        st[(size_t)(t0 + tid) * g.n_ret + r].seg = kNoSeg;
}

// The retry route: rows whose cut the approximate normaliser cannot certify
// are listed for the exact-mass pass and resolved again with the exact
// normaliser (their counts are written then).
__device__ __forceinline__ void list_retry(uint32_t* zrows, unsigned long long* zctr, int row) {
    zrows[atomicAdd(&zctr[0], 1ull)] = (uint32_t)row;
}

// Certification of a mass cut made with the normaliser Z' = zu + light, where
// zu is U's exact mass and light the mass of the keys outside U summed from
// their MFMA scores.  Each such weight carries a relative error of at most
// eta = s delta (1/8 + 1/80) + 2^-16: s delta / 8 from the score bound (with
// 1 % to spare), s delta / 80 from the roundings of the one-FMA exponent
// argument that scale with |e| and |m'| (both at most 2^16 delta: at most
// ln2 3 log2(e) 2^-8 s delta < s delta / 85), and 2^-16 from the rest of the
// argument's rounding, exp2 and the per-tile float sums, so
// the exact Z lies in [Z' - light eta, Z' + light eta].  The cut (mass P_k
// through the cut key, P_{k-1} before it) is kept when P_k / Z >= p - band
// and P_{k-1} / Z < p + band for every Z in that interval; band = 0.9e-6
// leaves 1e-7 of the 1e-6 acceptance band for the fp32 exp and fixed-point
// rounding of the exact weights.
constexpr double kBandCert = 0.9e-6;
__device__ __forceinline__ double light_eta(float s, float delta) {
    return (double)s * (double)delta * (0.125 * 1.01 + 0.0125) + 0x1.0p-16;
}
__device__ __forceinline__ bool mass_certified(double p, unsigned long long zu, unsigned long long light, double eta,
                                               unsigned long long pk, unsigned long long pk1) {
    const double zc = (double)zu + (double)light, dl = (double)light * eta;
    return (double)pk >= (p - kBandCert) * (zc + dl) && (double)pk1 < (p + kBandCert) * (zc - dl);
}

// ---------------------------------------------------------------------------
// Radix levels.  grid (ceil(n_tok / 32), n_ret), 256 threads: the rows that
// have no pool segment (and the keep-all rows' records).  A mass cut that the
// approximate normaliser cannot certify, or that keeps more than k_max keys,
// is marked (bad = 2) and listed for the retry route; retry != 0 resolves the
// marked rows again, with the exact normaliser or by count, and writes their
// counts.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_csel_main(Geo g, const bf16_t* __restrict__ k_low,
                                                   const float* __restrict__ top_p, const uint16_t* __restrict__ qlow,
                                                   const CState* __restrict__ st, CRow* __restrict__ rows_out,
                                                   int retry, int* __restrict__ counts, uint32_t* __restrict__ zrows,
                                                   unsigned long long* __restrict__ zctr) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r = blockIdx.y;
    const int t0 = blockIdx.x * kTR;
    const int n_valid = min(kTR, g.n_tok - t0);
    const float s = g.idx_scale;

    __shared__ __align__(16) unsigned char smem[kLevelBytes];
    unsigned long long(*hm)[kNBP] = reinterpret_cast<unsigned long long(*)[kNBP]>(smem);
    uint32_t(*hc)[kNBP] = reinterpret_cast<uint32_t(*)[kNBP]>(smem + kHmBytes);
    unsigned long long(*cand)[kCapC] = reinterpret_cast<unsigned long long(*)[kCapC]>(smem + kHmBytes + kHcBytes);

    __shared__ float qs[kTR][16];                        // q_low as floats
    __shared__ uint32_t cand_n[kTR];
    __shared__ unsigned long long zu[kTR];               // exact mass of U
    __shared__ float r_mp[kTR], r_delta[kTR], r_T[kTR], r_edge[kTR], r_ethr[kTR];
    __shared__ int r_mode[kTR], r_uend[kTR], r_ntie[kTR], r_done[kTR], r_gather[kTR], r_bad[kTR], r_pooled[kTR];
    __shared__ uint32_t r_klo[kTR], r_khi[kTR], r_shift[kTR], r_cnthi[kTR];
    __shared__ unsigned long long r_shi[kTR], r_target[kTR], r_light[kTR], r_zex[kTR];
    __shared__ int r_unit[kTR], r_kcnt[kTR], r_rec[kTR];
    __shared__ int s_any;
    __shared__ uint4 ktile[4][32][2];                    // per wave: the 32 keys of the current tile

    // the rows' state; pooled rows are finished by the recording pass
    if (tid == 0) s_any = 0;
    __syncthreads();
    if (tid < kTR) {
        const int row = tid;
        zu[row] = 0ull;
        cand_n[row] = 0u;
        r_target[row] = 0ull;
        r_gather[row] = 0;
        r_bad[row] = 0;
        r_ntie[row] = 0;
        r_T[row] = 0.0f;
        r_shi[row] = 0ull;
        r_cnthi[row] = 0u;
        r_pooled[row] = 0;
        r_done[row] = 1;
        r_mode[row] = kLevel;
        r_unit[row] = 0;
        r_kcnt[row] = 0;
        r_zex[row] = 0ull;
        r_rec[row] = 0;
        if (row < n_valid) {
            const CState c = st[(size_t)(t0 + row) * g.n_ret + r];
            r_kcnt[row] = c.kcnt;
            r_unit[row] = c.kcnt > 0;
            r_mp[row] = c.mp;
            r_delta[row] = c.delta;
            r_ethr[row] = c.e_thr;
            r_edge[row] = c.edge;
            r_klo[row] = c.klo;
            r_khi[row] = c.khi;
            r_shift[row] = c.shift;
            r_mode[row] = c.mode;
            r_uend[row] = c.uend;
            r_light[row] = c.light;
            r_pooled[row] = c.mode == kLevel && c.seg != kNoSeg;
            r_done[row] = c.mode != kLevel || r_pooled[row];
            r_rec[row] = !r_pooled[row];
            if (retry) {
                // only the rows marked for the retry route, from their records
                const CRow& cw = rows_out[(size_t)(t0 + row) * g.n_ret + r];
                const bool mine = !r_pooled[row] && cw.mode == kLevel && cw.bad == 2;
                r_rec[row] = mine;
                r_done[row] = !mine;
                if (mine) {
                    r_kcnt[row] = cw.kcnt;
                    r_unit[row] = cw.kcnt > 0;
                    r_zex[row] = cw.zex;
                }
            }
            if (r_rec[row]) s_any = 1;                    // a record to write here
        }
    }
    for (int x = tid; x < kTR * kNBP; x += 256) {
        (&hm[0][0])[x] = 0ull;
        (&hc[0][0])[x] = 0u;
    }
    __syncthreads();
    if (!s_any) return;
    load_qs(g, qlow, qs, blockIdx.x, blockIdx.y);
    __syncthreads();
    const TileCtx tc = tile_ctx(g, k_low, qs, blockIdx.x, blockIdx.y);
    const int lr = tc.lr, hh = tc.hh;
    const bool row_ok = tc.row_ok;
    const int pos = tc.pos;
    const int ntile = tc.ntile, nfull = tc.nfull;
    const auto page_a = [&](int it) { return tc.page(it); };
    const auto load_a = [&](int it, int pg) { return tc.load(it, pg); };
    const auto mfma_tile = [&](const uint4& a) { return tc.mfma(a); };
    const auto key_of = [&](int it, int i) { return tc.key_of(it, i); };

    // ---- P3 and the radix levels on the exact score for the rows without a
    // pool segment.  Level 0 computes the exact score and weight of every key
    // of U: the mass of U and the level-0 radix histogram; further levels
    // (64 buckets each, highest scores first) narrow the cut bucket, and its
    // keys are finally gathered for one sort.
    for (int level = 0; level < 8; ++level) {
        if (level > 0) {
            for (int x = tid; x < kTR * kNBP; x += 256) {
                (&hm[0][0])[x] = 0ull;
                (&hc[0][0])[x] = 0u;
            }
        }
        if (tid == 0) s_any = 0;
        __syncthreads();
        if (tid < kTR && !r_done[tid]) s_any = 1;
        __syncthreads();
        if (!s_any) break;

        // Each lane owns one row (lr) and scores its own pairs: the row's state
        // sits in registers, the tile's keys are copied to LDS when some lane
        // of the wave needs an exact score, U's mass accumulates per lane.
        const bool active = row_ok && !r_done[lr];
        const float e_thr = r_ethr[lr];
        const int gath = r_gather[lr];
        const bool ranged = active && (gath || level > 0);
        const float lo = ranged ? key_score(r_klo[lr]) : 0.0f, hi = ranged ? key_score(r_khi[lr]) : 0.0f;
        const float dl = r_delta[lr];
        const uint32_t klo = r_klo[lr], khi = r_khi[lr], shift = r_shift[lr];
        const float mp_row = r_mp[lr];
        const bool unit = r_unit[lr] != 0;
        float qv[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) qv[c] = qs[lr][c];
        unsigned long long zacc = 0ull;
        tile_loop<kPreHist>(wid, 4, ntile, page_a, load_a, [&](int it, const uint4& cur) {
            const f32x16_t sc = mfma_tile(cur);
            // which of this lane's pairs need an exact score
            uint32_t need = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                bool in = active && sc[i] >= e_thr;
                if (it >= nfull) in = in && key_of(it, i) <= pos;
                // only pairs whose exact score can fall inside [lo, hi]
                if (ranged) in = in && !(sc[i] + dl < lo) && !(sc[i] - dl > hi);
                need |= (uint32_t)in << i;
            }
            if (__ballot(need != 0u) == 0ull) return;
            ktile[wid][lr][hh] = cur;                     // key it*32 + lr, dims 8 hh .. 8 hh + 7
            wave_lds_sync();
            while (need) {
                const int i = __ffs(need) - 1;
                need &= need - 1u;
                const int kl = (i >> 2) * 8 + 4 * hh + (i & 3);
                const int key = it * 32 + kl;
                const float d = exact_score(qv, ktile[wid][kl][0], ktile[wid][kl][1]);
                const uint32_t kd = score_key(d);
                if (gath) {
                    if (kd >= klo && kd <= khi) {
                        const uint32_t cs = atomicAdd(&cand_n[lr], 1u);
                        if (cs < (uint32_t)kCapC)
                            cand[lr][cs] = ((unsigned long long)kd << 32) | (unsigned long long)(~(uint32_t)key);
                    }
                } else {
                    const unsigned long long w = unit ? 1ull : weight_bin(d, mp_row, s).w;
                    if (level == 0) zacc += w;
                    if (kd >= klo && kd <= khi) {
                        const uint32_t bk = min((khi - kd) >> shift, (uint32_t)(kNB - 1));
                        atomicAdd(&hm[lr][bk], w);
                        atomicAdd(&hc[lr][bk], 1u);
                    }
                    // above the range: counted by earlier levels; below: ranks below the cut
                }
            }
            wave_lds_sync();                              // the tile's keys are read before the next copy
        });
        if (level == 0) {
            zacc += __shfl_xor(zacc, 32);
            if (hh == 0 && zacc) atomicAdd(&zu[lr], zacc);
        }
        __syncthreads();

        // per-row step: resolve, narrow, or switch to gathering
        if (tid < kTR) {
            const int row = tid;
            if (!r_done[row]) {
                if (level == 0) {
                    if (r_unit[row]) {
                        r_target[row] = (unsigned long long)r_kcnt[row];
                    } else {
                        const float p = top_p[g.seq];
                        const unsigned long long Z = retry ? r_zex[row] : zu[row] + r_light[row];
                        unsigned long long tgt = (unsigned long long)ceil((double)p * (double)Z);
                        if (tgt > Z) tgt = Z;
                        if (tgt < 1ull) tgt = 1ull;
                        r_target[row] = tgt;
                    }
                }
                if (r_gather[row]) {
                    r_done[row] = 1;                     // final sort of the cut bucket's keys below
                } else {
                    unsigned long long cum = r_shi[row];
                    uint32_t ch = r_cnthi[row];
                    int bc = -1;
                    const uint32_t nbk = ((r_khi[row] - r_klo[row]) >> r_shift[row]) + 1u;
                    for (int b = 0; b < (int)min(nbk, (uint32_t)kNB); ++b) {
                        if (cum + hm[row][b] >= r_target[row] && hc[row][b]) {
                            bc = b;
                            break;
                        }
                        cum += hm[row][b];
                        ch += hc[row][b];
                    }
                    if (bc < 0) {
                        // U does not reach the target: the approximation bound failed
                        r_bad[row] = 1;
                        r_done[row] = 1;
                    } else {
                        r_shi[row] = cum;
                        r_cnthi[row] = ch;
                        const uint32_t khi = r_khi[row] - ((uint32_t)bc << r_shift[row]);
                        const uint32_t wdt = (1u << r_shift[row]) - 1u;
                        const uint32_t klo = (khi - r_klo[row] > wdt) ? khi - wdt : r_klo[row];
                        r_khi[row] = khi;
                        r_klo[row] = klo;
                        const uint32_t n_c = hc[row][bc];
                        if (klo == khi && n_c > (uint32_t)kCapC) {
                            // one score value with many keys: a tie group cut by index
                            const unsigned long long wT =
                                r_unit[row] ? 1ull : weight_bin(key_score(khi), r_mp[row], s).w;
                            const unsigned long long need = r_target[row] - cum;
                            r_T[row] = key_score(khi);
                            r_ntie[row] = (int)((need + wT - 1ull) / wT);
                            r_done[row] = 1;
                            r_gather[row] = 2;               // resolved without candidates
                        } else if (n_c <= (uint32_t)kCapC) {
                            r_gather[row] = 1;
                            cand_n[row] = 0u;
                        } else {
                            const uint32_t spn = khi - klo;
                            const int bits = spn ? 32 - __clz(spn) : 0;
                            r_shift[row] = bits > 6 ? bits - 6 : 0;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- per-row results; rows resolved by levels sort their candidates here
    if (wid == 0) {
        for (int row = 0; row < n_valid; ++row) {
            if (!r_rec[row]) continue;                   // pooled rows: written by the histogram pass
            const bool unit = r_unit[row] != 0;
            unsigned long long pk = 0ull, pk1 = 0ull;    // mass through the cut key and before it
            CRow out;
            out.mp = r_mp[row];
            out.delta = r_delta[row];
            out.e_thr = r_ethr[row];
            out.seg = kNoSeg;
            out.d_edge = r_edge[row];
            out.u_end = r_uend[row];
            out.mode = r_mode[row];
            out.T = 0.0f;
            out.n_tie = 0;
            out.count = 0;
            out.target = r_target[row];
            out.light = r_light[row];
            out.zex = r_zex[row];
            out.kcnt = r_kcnt[row];
            out.path = kPathLevel | (retry ? kPathExactZ : 0) | (unit ? kPathCount : 0);
            int bad = r_bad[row];
            if (out.mode == kLevel && !bad) {
                if (r_gather[row] == 2) {
                    out.T = r_T[row];
                    out.n_tie = r_ntie[row];
                    out.count = (int)r_cnthi[row] + r_ntie[row];
                    const unsigned long long wT = unit ? 1ull : weight_bin(out.T, r_mp[row], s).w;
                    pk = r_shi[row] + (unsigned long long)r_ntie[row] * wT;
                    pk1 = pk - wT;
                } else {
                    const int n = min((int)cand_n[row], kCapC);
                    if (n == 0 || r_gather[row] != 1 || !r_done[row]) {
                        bad = 1;
                    } else {
                        // bitonic sort (descending) of the candidates, two per lane
                        unsigned long long* cr = cand[row];
                        for (int x = lane + n; x < kCapC; x += 64) cr[x] = 0ull;
                        wave_lds_sync();
                        for (int k = 2; k <= kCapC; k <<= 1)
                            for (int j = k >> 1; j > 0; j >>= 1) {
                                for (int i = lane; i < kCapC; i += 64) {
                                    const int ixj = i ^ j;
                                    if (ixj > i) {
                                        const unsigned long long x = cr[i], y = cr[ixj];
                                        const bool desc = (i & k) == 0;
                                        if (desc ? (x < y) : (x > y)) {
                                            cr[i] = y;
                                            cr[ixj] = x;
                                        }
                                    }
                                }
                                wave_lds_sync();
                            }
                        // cumulative exact mass in rank order; the lane holds
                        // ranks 2 lane and 2 lane + 1
                        const int i0 = 2 * lane, i1 = 2 * lane + 1;
                        const float mpr = r_mp[row];
                        const unsigned long long w0 =
                            i0 < n ? (unit ? 1ull : weight_bin(key_score((uint32_t)(cr[i0] >> 32)), mpr, s).w) : 0ull;
                        const unsigned long long w1 =
                            i1 < n ? (unit ? 1ull : weight_bin(key_score((uint32_t)(cr[i1] >> 32)), mpr, s).w) : 0ull;
                        const unsigned long long incl = wave_incl_scan_u64(w0 + w1);
                        const unsigned long long c0 = r_shi[row] + incl - w1;   // through rank i0
                        const unsigned long long c1 = c0 + w1;                  // through rank i1
                        const unsigned long long tgt = r_target[row];
                        int first = 1 << 30;
                        if (i0 < n && c0 >= tgt) first = i0;
                        else if (i1 < n && c1 >= tgt) first = i1;
                        first = (int)wave_reduce32((uint32_t)first, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
                        if (first >= n) bad = 1;
                        const int ic = first < n ? first : n - 1;
                        {
                            // the masses at the cut, from the lane holding rank ic
                            unsigned long long a = 0ull, b = 0ull;
                            if (ic == i0) {
                                a = c0;
                                b = c0 - w0;
                            } else if (ic == i1) {
                                a = c1;
                                b = c0;
                            }
                            a = wave_sum_u64(a);
                            b = wave_sum_u64(b);
                            pk = a;
                            pk1 = b;
                        }
                        const uint32_t kT = (uint32_t)(cr[ic] >> 32);
                        int tie = 0, above = 0;
                        if (i0 <= ic) {
                            if ((uint32_t)(cr[i0] >> 32) == kT) ++tie; else ++above;
                        }
                        if (i1 <= ic) {
                            if ((uint32_t)(cr[i1] >> 32) == kT) ++tie; else ++above;
                        }
                        tie = (int)wave_sum_u32((uint32_t)tie);
                        above = (int)wave_sum_u32((uint32_t)above);
                        out.T = key_score(kT);
                        out.n_tie = tie;
                        out.count = (int)r_cnthi[row] + above + tie;
                    }
                }
                // certification: no key outside U can reach the cut
                if (!(out.T > out.d_edge)) bad = 1;
                if (!bad && !unit) {
                    const float p = top_p[g.seq];
                    const bool cap = g.k_max > 0 && out.count > g.k_max;
                    const bool unsure = !retry && out.light != 0ull &&
                                        ((g.flags & kFlagExactMass) ||
                                         !mass_certified((double)p, zu[row], out.light, light_eta(s, out.delta), pk,
                                                         pk1));
                    if (retry && cap) {
                        bad = 1;                         // capped after the exact normaliser: not handled
                    } else if (cap || unsure) {
                        bad = 2;                         // the retry route: exact normaliser, or by count
                        out.kcnt = cap ? g.k_max : 0;
                        out.zex = 0ull;
                        if (lane == 0) list_retry(zrows, zctr, (t0 + row) * g.n_ret + r);
                    }
                }
            }
            out.bad = bad;
            if (lane == 0) {
                rows_out[(size_t)(t0 + row) * g.n_ret + r] = out;
                if (retry) counts[(t0 + row) * g.n_ret + r] = bad ? -1 : out.count;
            }
            wave_lds_sync();
        }
    }
}

// ---------------------------------------------------------------------------
// Resolve of a row held in a pool segment (the key indices of U, empty slots
// marked ~0): the exact fixed-order score and exact fixed-point weight of
// every key of U, the target from U's exact mass plus the approximate mass of
// the keys outside U, the cut by radix selection over U's score keys (levels
// of kRB buckets with exact masses per bucket, highest scores first; once the
// cut bucket holds at most 64 keys one wavefront sorts them in registers;
// ties: lowest indices first), its certification, and the selected indices
// sorted ascending, stored over the segment.  Writes the row's count (-1 if
// certification failed).  NT threads, U of up to CAP keys in LDS.
// ---------------------------------------------------------------------------
constexpr int kRBits = 10;       // radix bits per level of the resolve (the small-row kernel: 8)

// Low word of a resolve entry (score key << 32 | low): larger for a smaller
// key index (ties rank lowest index first), with the writer of the entry in
// its low 3 bits.  Key indices are below 2^20.
__device__ __forceinline__ uint32_t lo_word(int key, int writer) {
    return ((0xFFFFFu - (uint32_t)key) << 3) | (uint32_t)writer;
}
__device__ __forceinline__ uint32_t lo_key(uint32_t lo) { return 0xFFFFFu - (lo >> 3); }

template <int RB>
struct ResolveSmem {
    unsigned long long hm[RB];
    uint32_t hc[RB];
    unsigned long long small_v[64], small_w[64];
    uint32_t kmin, kmax, s_u, tkey;
    int s_i, ntie, fail;
    unsigned long long s_S, s_C;
    unsigned long long pk, pk1, cnt;    // mass through the cut key and before it; keys taken
};

template <int CAP, int NT, int RBITS = kRBits>
__device__ void resolve_row(const Geo& g, const CRow& cr, int row, int rid, bool retry,
                            const bf16_t* __restrict__ k_low, const uint16_t* __restrict__ qlow,
                            const float* __restrict__ top_p, unsigned long long* __restrict__ pool,
                            int* __restrict__ count_out, int* __restrict__ path_out, uint32_t* __restrict__ zrows,
                            unsigned long long* __restrict__ zctr, unsigned long long* sk,
                            unsigned long long* scan_sh, ResolveSmem<1 << RBITS>& sm) {
    constexpr int kRB = 1 << RBITS;                      // radix buckets per level
    constexpr int PER = CAP / NT;
    static_assert(CAP % NT == 0, "whole slots per thread");
    const int tid = threadIdx.x, lane = tid & 63;
    const int slots = cr.count;
    const float s = g.idx_scale;
    const bool unit0 = cr.kcnt > 0;                      // count cut: fixed top-k (or a capped keep-all row)
    const float p = unit0 ? 1.0f : top_p[g.seq];
    if (!retry && !unit0 && cr.light != 0ull && (g.flags & kFlagExactMass)) {
        if (tid == 0) list_retry(zrows, zctr, row);      // the exact normaliser was asked for
        return;
    }
    unsigned long long* ub = pool + cr.seg;
    const int r = row % g.n_ret;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;
    float q16[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) q16[c] = bf2f(qlow[(size_t)row * 16 + c]);
    if (tid == 0) {
        sm.kmin = 0xFFFFFFFFu;
        sm.kmax = 0u;
        sm.fail = 0;
    }
    __syncthreads();
    // exact scores and weights; slot i of thread tid is tid + x NT; empty -> 0
    unsigned long long zl = 0ull, nl = 0ull;
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    for (int i = tid; i < slots; i += NT) {
        unsigned long long e = 0ull;
        const unsigned long long v = ub[i];
        if (v != ~0ull) {
            const int key = (int)(v & 0xFFFFFFull);
            const int page = bt[key >> 8];
            const uint4* kp = reinterpret_cast<const uint4*>(
                k_low + (((size_t)page * g.n_ret + r) * kBlk + (key & 255)) * 16);
            const float d = exact_score(q16, kp[0], kp[1]);
            zl += unit0 ? 1ull : weight_bin(d, cr.mp, s).w;
            ++nl;
            const uint32_t kd = score_key(d);
            kmn = min(kmn, kd);
            kmx = max(kmx, kd);
            e = ((unsigned long long)kd << 32) | (unsigned long long)lo_word(key, (int)(v >> 24) & 7);
        }
        sk[i] = e;
    }
    kmx = wave_max_u32(kmx);
    kmn = ~wave_max_u32(~kmn);
    if (lane == 0) {
        atomicMax(&sm.kmax, kmx);
        atomicMin(&sm.kmin, kmn);
    }
    unsigned long long zu, n64;
    block_excl_scan_u64<NT>(zl, &zu, scan_sh);
    block_excl_scan_u64<NT>(nl, &n64, scan_sh);
    unsigned long long target;
    if (unit0) {
        target = (unsigned long long)cr.kcnt;
    } else {
        const unsigned long long Z = retry ? cr.zex : zu + cr.light;
        target = (unsigned long long)ceil((double)p * (double)Z);
        if (target > Z) target = Z;
        if (target < 1ull) target = 1ull;
    }
    bool unit = unit0;
    const auto wkey = [&](uint32_t key) { return unit ? 1ull : weight_bin(key_score(key), cr.mp, s).w; };
    const uint32_t kmin0 = sm.kmin, kmax0 = sm.kmax;
    // ---- radix cut: Tkey and the number of ties at Tkey taken (lowest
    // indices).  A mass cut is certified against the approximate normaliser;
    // one that keeps more than k_max keys is cut again by count.
    for (int pass = 0; pass < 2; ++pass) {
    if (pass) __syncthreads();                           // every thread has read the first cut
    uint32_t klo = kmin0, khi = kmax0;
    unsigned long long S_hi = 0ull, C_hi = 0ull;
    bool done = n64 == 0ull || (unit ? n64 : zu) < target;   // U cannot reach the target: not certified
    if (tid == 0) sm.fail = done ? 1 : 0;
    for (int level = 0; level < 6 && !done; ++level) {
        const uint32_t span = khi - klo;
        const int bits = span ? 32 - __clz(span) : 0;
        const int shift = bits > RBITS ? bits - RBITS : 0;
        for (int b = tid; b < kRB; b += NT) {
            sm.hm[b] = 0ull;
            sm.hc[b] = 0u;
        }
        __syncthreads();
        for (int i = tid; i < slots; i += NT) {
            const unsigned long long v = sk[i];
            if (!v) continue;
            const uint32_t key = (uint32_t)(v >> 32);
            if (key < klo || key > khi) continue;
            const uint32_t bk = (khi - key) >> shift;      // bucket 0 holds the highest keys
            atomicAdd(&sm.hm[bk], wkey(key));
            atomicAdd(&sm.hc[bk], 1u);
        }
        __syncthreads();
        constexpr int BPT = kRB / NT;                       // buckets per thread (1 or 2)
        static_assert(BPT >= 1 && kRB % NT == 0, "whole buckets per thread");
        unsigned long long loc = 0ull, locc = 0ull;
#pragma unroll
        for (int x = 0; x < BPT; ++x) {
            loc += sm.hm[BPT * tid + x];
            locc += sm.hc[BPT * tid + x];
        }
        unsigned long long tot;
        const unsigned long long ex = S_hi + block_excl_scan_u64<NT>(loc, &tot, scan_sh);
        const unsigned long long exc = C_hi + block_excl_scan_u64<NT>(locc, &tot, scan_sh);
        if (tid == 0) sm.s_i = kRB;
        __syncthreads();
        {
            unsigned long long run = ex;
#pragma unroll
            for (int x = 0; x < BPT; ++x) {
                const int b = BPT * tid + x;
                run += sm.hm[b];
                if (run >= target && sm.hc[b]) {
                    atomicMin(&sm.s_i, b);
                    break;
                }
            }
        }
        __syncthreads();
        const int bk = sm.s_i;
        if (bk >= kRB) {                                     // rounding: U does not reach the target
            if (tid == 0) sm.fail = 1;
            done = true;
            break;
        }
        if (bk / BPT == tid) {
            unsigned long long run = ex, runc = exc;
            for (int b = BPT * tid; b < bk; ++b) {
                run += sm.hm[b];
                runc += sm.hc[b];
            }
            sm.s_S = run;
            sm.s_C = runc;
            sm.s_u = sm.hc[bk];
        }
        __syncthreads();
        S_hi = sm.s_S;
        C_hi = sm.s_C;
        const uint32_t n_b = sm.s_u;
        const uint32_t nkhi = khi - ((uint32_t)bk << shift);
        const uint32_t wdt = (1u << shift) - 1u;
        const uint32_t nklo = (nkhi - klo > wdt) ? nkhi - wdt : klo;
        klo = nklo;
        khi = nkhi;
        __syncthreads();
        if (n_b <= 64u) {
            // the bucket's keys into one wavefront, sorted in registers
            if (tid == 0) sm.s_u = 0u;
            __syncthreads();
            for (int i = tid; i < slots; i += NT) {
                const unsigned long long v = sk[i];
                if (!v) continue;
                const uint32_t key = (uint32_t)(v >> 32);
                if (key < klo || key > khi) continue;
                const uint32_t slot = atomicAdd(&sm.s_u, 1u);
                if (slot < 64u) {
                    sm.small_v[slot] = v;
                    sm.small_w[slot] = wkey(key);
                }
            }
            __syncthreads();
            if (tid < 64) {
                const int nbk = (int)min(sm.s_u, 64u);
                unsigned long long v = lane < nbk ? sm.small_v[lane] : 0ull;
                unsigned long long w = lane < nbk ? sm.small_w[lane] : 0ull;
#pragma unroll
                for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
                    for (int jj = k >> 1; jj > 0; jj >>= 1) {
                        const unsigned long long ov = __shfl_xor(v, jj), ow = __shfl_xor(w, jj);
                        const bool desc = (lane & k) == 0 || k == 64;
                        const bool lower = (lane & jj) == 0;
                        const bool take = desc == lower ? ov > v : ov < v;
                        if (take) {
                            v = ov;
                            w = ow;
                        }
                    }
                const unsigned long long incl = wave_incl_scan_u64(w);
                const unsigned long long reach = __ballot(lane < nbk && S_hi + incl >= target);
                const int ic = reach ? __ffsll((long long)reach) - 1 : nbk - 1;
                const uint32_t tk = (uint32_t)(lane_u64(v, ic) >> 32);
                const unsigned long long tie = __ballot(lane <= ic && lane < nbk && (uint32_t)(v >> 32) == tk);
                if (lane == 0) {
                    sm.tkey = tk;
                    sm.ntie = __popcll(tie);
                    if (!reach) sm.fail = 1;
                }
                if (lane == ic) {
                    sm.pk = S_hi + incl;
                    sm.pk1 = S_hi + incl - w;
                    sm.cnt = C_hi + (unsigned long long)ic + 1ull;
                }
            }
            __syncthreads();
            done = true;
            break;
        }
        if (klo == khi) {
            // one score value with more than 64 keys: its lowest indices first
            if (tid == 0) {
                const unsigned long long wT = wkey(klo);
                const unsigned long long need = target - S_hi;
                const unsigned long long nt = min((need + wT - 1ull) / wT, (unsigned long long)n_b);
                sm.tkey = klo;
                sm.ntie = (int)nt;
                sm.pk = S_hi + nt * wT;
                sm.pk1 = sm.pk - wT;
                sm.cnt = C_hi + nt;
            }
            __syncthreads();
            done = true;
            break;
        }
    }
    if (!done && tid == 0) sm.fail = 1;                  // no level isolated the cut
    __syncthreads();
    if (pass == 0 && !unit0 && !sm.fail) {
        if (!retry && cr.light != 0ull &&
            !mass_certified((double)p, zu, cr.light, light_eta(s, cr.delta), sm.pk, sm.pk1)) {
            if (tid == 0) list_retry(zrows, zctr, row);   // uniform: shared values after a barrier
            return;
        }
        if (g.k_max > 0 && sm.cnt > (unsigned long long)g.k_max) {
            unit = true;                                 // the budget cap: the first k_max keys by count
            target = (unsigned long long)g.k_max;
            continue;
        }
    }
    break;
    }
    const uint32_t Tkey = sm.tkey;
    const int ntie = sm.ntie;
    const bool ok = !sm.fail && key_score(Tkey) > cr.d_edge;
    const int pflags = (retry ? kPathExactZ : 0) | (unit ? kPathCount : 0);
    if (!ok) {
        if (tid == 0) {
            *count_out = -1;
            *path_out = rid | pflags;
        }
        __syncthreads();
        return;
    }
    // ---- the keys above the cut and the ties at it, as (index << 1 | tie),
    // sorted ascending; then the ties past the first ntie dropped.  Each
    // writer's entries ascend in slot order, so the kept keys are 8 sorted
    // runs (every thread takes a contiguous range of slots), merged by rank.
    uint32_t* sv = reinterpret_cast<uint32_t*>(sk);     // 2 CAP words
    const int sp = (slots + NT - 1) / NT;                // <= PER
    const int s0 = min(tid * sp, slots);
    uint32_t vals[PER];                                  // (index << 1 | tie) << 4 | writer (8: not kept)
    unsigned long long clo = 0ull, chi = 0ull;           // kept per writer, 16-bit fields
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int i = s0 + x;
        const unsigned long long v = (x < sp && i < slots) ? sk[i] : 0ull;
        const uint32_t key = (uint32_t)(v >> 32);
        const bool keep = v != 0ull && key >= Tkey;
        const uint32_t lo = (uint32_t)v;
        const int w = (int)(lo & 7u);
        vals[x] = (((lo_key(lo) << 1) | (key == Tkey ? 1u : 0u)) << 4) | (keep ? (uint32_t)w : 8u);
        if (keep) {
            if (w < 4) clo += 1ull << (16 * w);
            else chi += 1ull << (16 * (w - 4));
        }
    }
    unsigned long long tlo, thi;
    const unsigned long long elo = block_excl_scan_u64<NT>(clo, &tlo, scan_sh);
    const unsigned long long ehi = block_excl_scan_u64<NT>(chi, &thi, scan_sh);
    const auto field = [](unsigned long long a, unsigned long long b, int w) {
        return (int)(((w < 4 ? a : b) >> (16 * (w & 3))) & 0xFFFFull);
    };
    // Kept indices spanning at most 64 CAP: a bitmap over their range (the
    // slots are in registers now, so the area is free) gives the ascending
    // order without a merge; the ties past the first ntie are cut at the
    // index of the ntie-th tie, found the same way.
    {
        uint32_t imn = 0xFFFFFFFFu, imx = 0u, ntk = 0u;
#pragma unroll
        for (int x = 0; x < PER; ++x)
            if ((vals[x] & 15u) != 8u) {
                const uint32_t id = vals[x] >> 5;
                imn = min(imn, id);
                imx = max(imx, id);
                ntk += (vals[x] >> 4) & 1u;
            }
        imx = wave_max_u32(imx);
        imn = ~wave_max_u32(~imn);
        ntk = wave_sum_u32(ntk);
        if (tid == 0) {
            sm.kmin = 0xFFFFFFFFu;
            sm.kmax = 0u;
            sm.s_u = 0u;
        }
        __syncthreads();
        if (lane == 0) {
            atomicMin(&sm.kmin, imn);
            atomicMax(&sm.kmax, imx);
            atomicAdd(&sm.s_u, ntk);
        }
        __syncthreads();
        const uint32_t bmin = sm.kmin, bmax = sm.kmax, ties_all = sm.s_u;
        const int nwords = bmax >= bmin ? (int)((bmax - bmin) / 32u + 1u) : 0;
        if (nwords > 0 && nwords <= 2 * CAP) {
            uint32_t* bmp = sv;
            // word w of the bitmap sits at w + w / 64: a thread's run of
            // consecutive words then meets the other lanes' runs in distinct
            // banks (the area holds 2 CAP + 2 CAP / 64 words)
            const auto bw = [](int w) { return w + (w >> 6); };
            const int wper = (nwords + NT - 1) / NT;
            const int w0 = min(tid * wper, nwords), w1 = min(w0 + wper, nwords);
            // (tie mode) 0: no tie kept, 1: ties up to index jlim, 2: every tie
            int tmode = ntie <= 0 ? 0 : ((uint32_t)ntie >= ties_all ? 2 : 1);
            uint32_t jlim = 0u;
            if (tmode == 1) {
                for (int w = tid; w < nwords; w += NT) bmp[bw(w)] = 0u;
                __syncthreads();
#pragma unroll
                for (int x = 0; x < PER; ++x)
                    if ((vals[x] & 15u) != 8u && ((vals[x] >> 4) & 1u)) {
                        const uint32_t o = (vals[x] >> 5) - bmin;
                        atomicOr(&bmp[bw((int)(o >> 5))], 1u << (o & 31u));
                    }
                __syncthreads();
                unsigned long long c = 0ull;
                for (int w = w0; w < w1; ++w) c += __popc(bmp[bw(w)]);
                unsigned long long tt;
                unsigned long long rk = block_excl_scan_u64<NT>(c, &tt, scan_sh);
                const unsigned long long want = (unsigned long long)ntie - 1ull;   // rank of the last kept tie
                if (want >= rk && want < rk + c) {
                    for (int w = w0; w < w1; ++w) {
                        uint32_t bits = bmp[bw(w)];
                        const int n = __popc(bits);
                        if (rk + (unsigned long long)n > want) {
                            for (unsigned long long k = want - rk; k > 0; --k) bits &= bits - 1u;
                            sm.s_S = (unsigned long long)(bmin + 32u * (uint32_t)w + (uint32_t)(__ffs(bits) - 1));
                            break;
                        }
                        rk += (unsigned long long)n;
                    }
                }
                __syncthreads();
                jlim = (uint32_t)sm.s_S;
            }
            for (int w = tid; w < nwords; w += NT) bmp[bw(w)] = 0u;
            __syncthreads();
#pragma unroll
            for (int x = 0; x < PER; ++x) {
                if ((vals[x] & 15u) == 8u) continue;
                const uint32_t id = vals[x] >> 5;
                const bool tie = (vals[x] >> 4) & 1u;
                if (tie && (tmode == 0 || (tmode == 1 && id > jlim))) continue;
                const uint32_t o = id - bmin;
                atomicOr(&bmp[bw((int)(o >> 5))], 1u << (o & 31u));
            }
            __syncthreads();
            unsigned long long c = 0ull;
            for (int w = w0; w < w1; ++w) c += __popc(bmp[bw(w)]);
            unsigned long long cnt;
            unsigned long long o = block_excl_scan_u64<NT>(c, &cnt, scan_sh);
            uint32_t* ubi = reinterpret_cast<uint32_t*>(ub);
            for (int w = w0; w < w1; ++w) {
                uint32_t bits = bmp[bw(w)];
                while (bits) {
                    const int b = __ffs(bits) - 1;
                    bits &= bits - 1u;
                    ubi[o++] = bmin + 32u * (uint32_t)w + (uint32_t)b;
                }
            }
            if (tid == 0) {
                *count_out = (int)cnt;
                *path_out = rid | pflags | kPathBitmap;
            }
            __syncthreads();
            return;
        }
    }
    int nk = 0, cnt8[8], rb[8];                          // block-uniform: kept in scalar registers
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        cnt8[w] = __builtin_amdgcn_readfirstlane(field(tlo, thi, w));
        rb[w] = nk;                                      // run w at sv[rb[w] ..), contiguous
        nk += cnt8[w];
    }
    {
        int off[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) off[w] = field(elo, ehi, w);
#pragma unroll
        for (int x = 0; x < PER; ++x) {
            const int w = (int)(vals[x] & 15u);
            if (w == 8) continue;
            int q = 0, b = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (u == w) {
                    q = off[u]++;
                    b = rb[u];
                }
            sv[b + q] = vals[x] >> 4;
        }
    }
    __syncthreads();
    // the merged order: a value's place is the count of values below it in
    // the 8 runs (a binary search in each; the values are distinct indices,
    // so in its own run that count is its place there).  Written to the
    // second half of the area.
    // The searches run in lockstep: the same halving step for all 8 runs (read
    // positions clamped to each run), so their LDS reads overlap.
    uint32_t* so = sv + CAP;
    int top = 1;
    {
        int mc = 1;
#pragma unroll
        for (int u = 0; u < 8; ++u) mc = max(mc, cnt8[u]);
        while (2 * top <= mc) top <<= 1;
    }
    for (int i = tid; i < nk; i += NT) {
        const uint32_t v = sv[i];
        int lo[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) lo[u] = 0;
        for (int step = top; step > 0; step >>= 1) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = lo[u] + step;
                const int n = cnt8[u];
                const uint32_t y = n > 0 ? sv[rb[u] + min(t, n) - 1] : 0xFFFFFFFFu;
                lo[u] = (t <= n && y < v) ? t : lo[u];
            }
        }
        int P = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) P += lo[u];
        so[P] = v;
    }
    __syncthreads();
    // ties in index order: each thread a contiguous run of the sorted list
    const int per = (nk + NT - 1) / NT;
    const int r0 = min(tid * per, nk), r1 = min(r0 + per, nk);
    unsigned long long tl = 0ull;
    for (int i = r0; i < r1; ++i) tl += so[i] & 1u;
    unsigned long long ttot;
    const unsigned long long tbase = block_excl_scan_u64<NT>(tl, &ttot, scan_sh);
    unsigned long long kl = 0ull;
    {
        unsigned long long tr = tbase;
        for (int i = r0; i < r1; ++i) {
            const bool tie = so[i] & 1u;
            if (!tie || tr < (unsigned long long)ntie) ++kl;
            if (tie) ++tr;
        }
    }
    unsigned long long cnt;
    const unsigned long long obase = block_excl_scan_u64<NT>(kl, &cnt, scan_sh);
    uint32_t* ubi = reinterpret_cast<uint32_t*>(ub);
    {
        unsigned long long tr = tbase, o = obase;
        for (int i = r0; i < r1; ++i) {
            const uint32_t v = so[i];
            const bool tie = v & 1u;
            if (!tie || tr < (unsigned long long)ntie) ubi[o++] = v >> 1;
            if (tie) ++tr;
        }
    }
    if (tid == 0) {
        *count_out = (int)cnt;
        *path_out = rid | pflags | kPathMerge;
    }
    __syncthreads();
}

// Rows with U in (kTinyU, kSmallU]: two 512-thread workgroups per CU (their
// LDS fills it) take the rows the histogram pass listed from a shared
// counter, so no LDS is held by workgroups of rows that are not theirs.
constexpr int kRT = 512;
__global__ __launch_bounds__(kRT) __attribute__((amdgpu_waves_per_eu(4)))   // two workgroups per CU
void k_csel_resolve(Geo g, CRow* __restrict__ rows, int n_rows,
                                                      const uint32_t* __restrict__ mrows,
                                                      unsigned long long* __restrict__ mctr,
                                                      const bf16_t* __restrict__ k_low,
                                                      const uint16_t* __restrict__ qlow,
                                                      const float* __restrict__ top_p,
                                                      unsigned long long* __restrict__ pool,
                                                      int* __restrict__ counts, uint32_t* __restrict__ zrows,
                                                      unsigned long long* __restrict__ zctr) {
    __shared__ unsigned long long sk[kSmallU + kSmallU / 128];
    __shared__ unsigned long long scan_sh[kRT / 64 + 1];
    __shared__ ResolveSmem<1 << kRBits> sm;
    __shared__ unsigned long long s_next;
    const unsigned long long n_list = min(mctr[0], (unsigned long long)n_rows);
    for (;;) {
        __syncthreads();                                 // every thread has read the previous entry number
        if (threadIdx.x == 0) s_next = atomicAdd(&mctr[1], 1ull);
        __syncthreads();
        const unsigned long long e = s_next;
        if (e >= n_list) break;
        const int row = (int)mrows[e];
        const CRow cr = rows[row];
        if (cr.mode != kBuf || cr.bad || cr.count <= kTinyU || cr.count > kSmallU) continue;
        resolve_row<kSmallU, kRT>(g, cr, row, kPathRow, false, k_low, qlow, top_p, pool, &counts[row],
                                  &rows[row].path, zrows, zctr, sk, scan_sh, sm);
    }
}

// Rows with U of at most kTinyU keys: the same resolve on 128 threads with
// 256-bucket radix levels (12 KB of LDS), so that many rows share a CU; and
// the counts of the rows that have no segment.  grid (rows).
constexpr int kRTS = 128;
constexpr int kRBitsS = 8;
__global__ __launch_bounds__(kRTS) void k_csel_resolve_small(Geo g, CRow* __restrict__ rows,
                                                             const bf16_t* __restrict__ k_low,
                                                             const uint16_t* __restrict__ qlow,
                                                             const float* __restrict__ top_p,
                                                             unsigned long long* __restrict__ pool,
                                                             int* __restrict__ counts, uint32_t* __restrict__ zrows,
                                                             unsigned long long* __restrict__ zctr) {
    const int row = blockIdx.x;
    const CRow cr = rows[row];
    if (cr.mode != kBuf) {
        if (threadIdx.x == 0) {
            const int L = g.pos0 + row / g.n_ret + 1;
            counts[row] = cr.kcnt == -3 ? -3 : (cr.bad ? -1 : (cr.mode == kAll ? L : cr.count));
            if (cr.mode == kAll) rows[row].path = kPathAll;
        }
        return;
    }
    if (cr.bad) {
        if (threadIdx.x == 0) counts[row] = -1;
        return;
    }
    if (cr.count > kTinyU) return;
    __shared__ unsigned long long sk[kTinyU + kTinyU / 128];
    __shared__ unsigned long long scan_sh[kRTS / 64 + 1];
    __shared__ ResolveSmem<1 << kRBitsS> sm;
    resolve_row<kTinyU, kRTS, kRBitsS>(g, cr, row, kPathTiny, false, k_low, qlow, top_p, pool, &counts[row],
                                       &rows[row].path, zrows, zctr, sk, scan_sh, sm);
}

// Rows with U in (kSmallU, kSegMax]: one 512-thread workgroup per CU takes
// the rows the histogram pass listed, one at a time from a shared counter
// (rows differ several-fold in cost, so a fixed assignment leaves CUs idle).
// A listed row that the recording pass sent to the radix levels is skipped.
// retry: the listed rows are the retry route's (any segment size), resolved
// with their exact normaliser.  list_n[0] holds the entries, *next the next
// entry taken.
constexpr int kRTL = 512;      // threads of the large-row resolve (two waves per SIMD: room for its registers)
__global__ __launch_bounds__(kRTL) void k_csel_resolve_large(Geo g, CRow* __restrict__ rows, int n_rows,
                                                             const uint32_t* __restrict__ list,
                                                             const unsigned long long* __restrict__ list_n,
                                                             unsigned long long* __restrict__ next, int retry,
                                                             const bf16_t* __restrict__ k_low,
                                                             const uint16_t* __restrict__ qlow,
                                                             const float* __restrict__ top_p,
                                                             unsigned long long* __restrict__ pool,
                                                             int* __restrict__ counts, uint32_t* __restrict__ zrows,
                                                             unsigned long long* __restrict__ zctr) {
    __shared__ unsigned long long sk[kSegMax + kSegMax / 128];
    __shared__ unsigned long long scan_sh[kRTL / 64 + 1];
    __shared__ ResolveSmem<1 << kRBits> sm;
    __shared__ unsigned long long s_next;
    const unsigned long long n_list = min(list_n[0], (unsigned long long)n_rows);
    for (;;) {
        __syncthreads();                                 // every thread has read the previous entry number
        if (threadIdx.x == 0) s_next = atomicAdd(next, 1ull);
        __syncthreads();
        const unsigned long long e = s_next;
        if (e >= n_list) break;
        const int row = (int)list[e];
        const CRow cr = rows[row];
        if (cr.mode != kBuf || (!retry && cr.count <= kSmallU)) continue;
        if (cr.bad) {
            if (threadIdx.x == 0) counts[row] = -1;
            continue;
        }
        resolve_row<kSegMax, kRTL>(g, cr, row, kPathLarge, retry != 0, k_low, qlow, top_p, pool, &counts[row],
                                   &rows[row].path, zrows, zctr, sk, scan_sh, sm);
    }
}

// Exact mass of every key of the rows on the retry route: the fixed-order
// score and exact fixed-point weight of each key, summed per piece of
// kZPiece keys and added into the row's record (an exact, order-free sum).
// Items (listed row, piece) are taken from a shared counter.  256 threads.
constexpr int kZPiece = 32768;
__global__ __launch_bounds__(256) void k_csel_zexact(Geo g, CRow* __restrict__ rows, int n_rows,
                                                     const uint32_t* __restrict__ zrows,
                                                     unsigned long long* __restrict__ zctr,
                                                     const bf16_t* __restrict__ k_low,
                                                     const uint16_t* __restrict__ qlow) {
    __shared__ unsigned long long s_next;
    __shared__ unsigned long long red[4];
    const int tid = threadIdx.x;
    const unsigned long long n_list = min(zctr[0], (unsigned long long)n_rows);
    const int npiece = (g.pos0 + g.n_tok + kZPiece - 1) / kZPiece;
    const unsigned long long n_items = n_list * (unsigned long long)npiece;
    const float s = g.idx_scale;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;
    for (;;) {
        __syncthreads();
        if (tid == 0) s_next = atomicAdd(&zctr[1], 1ull);
        __syncthreads();
        const unsigned long long e = s_next;
        if (e >= n_items) break;
        const int row = (int)zrows[e / (unsigned long long)npiece];
        const int k0 = (int)(e % (unsigned long long)npiece) * kZPiece;
        const int L = g.pos0 + row / g.n_ret + 1;
        if (k0 >= L) continue;
        const int r = row % g.n_ret;
        const float mp = rows[row].mp;
        float q16[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) q16[c] = bf2f(qlow[(size_t)row * 16 + c]);
        unsigned long long acc = 0ull;
        const int k1 = min(L, k0 + kZPiece);
        for (int key = k0 + tid; key < k1; key += 256) {
            const int page = bt[key >> 8];
            const uint4* kp = reinterpret_cast<const uint4*>(
                k_low + (((size_t)page * g.n_ret + r) * kBlk + (key & 255)) * 16);
            acc += weight_bin(exact_score(q16, kp[0], kp[1]), mp, s).w;
        }
        acc = wave_sum_u64(acc);
        if ((tid & 63) == 0) red[tid >> 6] = acc;
        __syncthreads();
        if (tid == 0) atomicAdd(&rows[row].zex, red[0] + red[1] + red[2] + red[3]);
    }
}

// CSR row pointers over all rows of the call, the certification and the
// capacity check.
__global__ __launch_bounds__(1024) void k_csel_rowptr(const int* __restrict__ counts, int rows,
                                                      int64_t* __restrict__ row_ptr, int64_t capacity,
                                                      int32_t* __restrict__ status) {
    const int tid = threadIdx.x;
    __shared__ unsigned long long scan_sh[1024 / 64 + 1];
    __shared__ int s_bad;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    int64_t carry = 0;
    if (tid == 0) row_ptr[0] = 0;
    for (int i0 = 0; i0 < rows; i0 += 1024) {
        const int i = i0 + tid;
        const int c = i < rows ? counts[i] : 0;
        if (c == -3) atomicMax(&s_bad, 3);               // invalid top_p
        else if (c < 0) atomicMax(&s_bad, 2);            // a cut not certified
        const unsigned long long cu = c > 0 ? (unsigned long long)c : 0ull;
        unsigned long long tot;
        const unsigned long long ex = block_excl_scan_u64<1024>(cu, &tot, scan_sh);
        if (i < rows) row_ptr[i + 1] = carry + (int64_t)(ex + cu);
        carry += (int64_t)tot;
    }
    __syncthreads();
    if (tid == 0) *status = s_bad ? s_bad : (carry > capacity ? 1 : 0);
}

// Rows held in a segment and keep-all rows: copy into idx.  grid (rows), 256 threads.
__global__ __launch_bounds__(256) void k_csel_copy(const CRow* __restrict__ rows,
                                                   const unsigned long long* __restrict__ pool,
                                                   const int64_t* __restrict__ row_ptr, int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ status) {
    const int row = blockIdx.x;
    if (*status != 0) return;
    const int mode = rows[row].mode;
    if (mode == kLevel) return;
    const int64_t b = row_ptr[row], n = row_ptr[row + 1] - b;
    if (mode == kAll) {
        for (int64_t i = threadIdx.x; i < n; i += 256) idx[b + i] = (int32_t)i;
    } else {
        const uint32_t* ubi = reinterpret_cast<const uint32_t*>(pool + rows[row].seg);
        for (int64_t i = threadIdx.x; i < n; i += 256) idx[b + i] = (int32_t)ubi[i];
    }
}

// ---------------------------------------------------------------------------
// Rescan emit of the rows resolved by levels.  grid (ceil(n_tok / 32), n_ret),
// one wavefront: keys in index order, selected keys written ascending at
// row_ptr[row].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_csel_emit(Geo g, const bf16_t* __restrict__ k_low,
                                                  const uint16_t* __restrict__ qlow, const CRow* __restrict__ rows,
                                                  const int64_t* __restrict__ row_ptr, int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ status) {
    const int lane = threadIdx.x;
    const int r = blockIdx.y, t0 = blockIdx.x * kTR;
    const int n_valid = min(kTR, g.n_tok - t0);
    const int lr = lane & 31, hh = lane >> 5;
    const int row = (t0 + min(lr, n_valid - 1)) * g.n_ret + r;
    const int pos = g.pos0 + t0 + lr;
    if (*status != 0) return;
    const CRow cr = rows[row];
    const bool row_ok = lr < n_valid && cr.mode == kLevel;
    if (__ballot(row_ok) == 0ull) return;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;
    float q16[16];
    uint4 qb;
    {
        const uint4* qp = reinterpret_cast<const uint4*>(qlow + (size_t)row * 16);
        const uint4 a0 = qp[0], a1 = qp[1];
        unpack8(a0, q16);
        unpack8(a1, q16 + 8);
        qb = hh ? a1 : a0;
    }
    const int L_max = g.pos0 + t0 + n_valid;
    const int ntile = (L_max + 31) / 32;
    const int64_t wpos = row_ok ? row_ptr[row] : 0;
    const int64_t lim = row_ok ? row_ptr[row + 1] - wpos : 0;
    int run_sel = 0, run_tie = 0;
    auto page_a = [&](int it) { return bt[min(it * 32 + lr, L_max - 1) >> 8]; };
    auto load_a = [&](int it, int pg) {
        const int kk = min(it * 32 + lr, L_max - 1);
        return *reinterpret_cast<const uint4*>(
            k_low + (((size_t)pg * g.n_ret + r) * kBlk + (kk & 255)) * 16 + 8 * hh);
    };
    tile_loop<kPreHist>(0, 1, ntile, page_a, load_a, [&](int it, const uint4& cur) {
        f32x16_t sc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = 0.0f;
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(cur), as_bf16x8(qb), sc, 0, 0, 0);
        // certain selections, and the pairs whose exact score decides
        uint32_t sel = 0, amb = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int kj = it * 32 + (i >> 2) * 8 + 4 * hh + (i & 3);
            const bool in = row_ok && kj <= pos && sc[i] >= cr.e_thr;
            const bool hi = sc[i] - cr.delta > cr.T;
            const bool near = !hi && !(sc[i] + cr.delta < cr.T);
            sel |= (uint32_t)(in && hi) << i;
            amb |= (uint32_t)(in && near) << i;
        }
        uint32_t tie = 0;
        if (__ballot(amb != 0u) != 0ull) {
            uint32_t m = amb;
            while (m) {
                const int i = __ffs(m) - 1;
                m &= m - 1;
                const int kj = it * 32 + (i >> 2) * 8 + 4 * hh + (i & 3);
                const int pg = bt[kj >> 8];
                const uint4* kp = reinterpret_cast<const uint4*>(
                    k_low + (((size_t)pg * g.n_ret + r) * kBlk + (kj & 255)) * 16);
                const float d = exact_score(q16, kp[0], kp[1]);
                if (d > cr.T) sel |= 1u << i;
                else if (d == cr.T) tie |= 1u << i;
            }
        }
        // ties in index order: groups of four keys alternate between the halves
        if (__ballot(tie != 0u) != 0ull) {
            uint32_t tc[4], tp[4];
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) tc[gq] = __popc((tie >> (4 * gq)) & 0xFu);
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) tp[gq] = __shfl_xor(tc[gq], 32);
            int acc = run_tie;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                int o = acc + (hh ? (int)tp[gq] : 0);     // the partner's group comes first for hh = 1
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * gq + e;
                    if ((tie >> i) & 1u) {
                        if (o < cr.n_tie) sel |= 1u << i;
                        ++o;
                    }
                }
                acc += (int)tc[gq] + (int)tp[gq];
            }
            run_tie = acc;
        }
        // ordered write of the selected keys
        if (__ballot(sel != 0u) != 0ull) {
            // counts of the four groups of this half packed in 3-bit fields
            uint32_t pk = 0;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) pk |= (uint32_t)__popc((sel >> (4 * gq)) & 0xFu) << (3 * gq);
            const uint32_t pp = __shfl_xor(pk, 32);
            int acc = run_sel;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int c_m = (pk >> (3 * gq)) & 7, c_p = (pp >> (3 * gq)) & 7;
                int o = acc + (hh ? c_p : 0);
                uint32_t m = (sel >> (4 * gq)) & 0xFu;
                while (m) {
                    const int e = __ffs(m) - 1;
                    m &= m - 1;
                    if (o < lim) idx[wpos + o] = it * 32 + gq * 8 + 4 * hh + e;
                    ++o;
                }
                acc += c_m + c_p;
            }
            run_sel = acc;
        }
    });
}

// Largest squared indexer-key norm of each block of kNormKeys keys of the
// chunk's sequence, per retrieval head, and the resets of the pool counter and
// the large-row list; the workgroups past nblk form q_low of 16 rows each.
// grid (nblk + ceil(n_tok / 16), n_ret), 256 threads.
__global__ __launch_bounds__(256) void k_csel_knorm(Geo g, const bf16_t* __restrict__ k_low, int n_keys,
                                                    float* __restrict__ knorm, int nblk,
                                                    unsigned long long* __restrict__ pool_ctr,
                                                    const bf16_t* __restrict__ q, const bf16_t* __restrict__ w_q,
                                                    uint16_t* __restrict__ qlow_out, uint32_t* __restrict__ rmaxk) {
    const int r = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
    if (blk >= nblk) {
        // q_low of 16 rows (fixed-order fp32 chain over d, one bf16 rounding;
        // the query rows and W_q staged in LDS) and their P1 maxima zeroed
        __shared__ __align__(16) float wq[128 * 16];
        __shared__ __align__(16) float qr[16][128];
        const int t0 = (blk - nblk) * 16, nv = min(16, g.n_tok - t0);
        stage_f32(w_q + (size_t)r * g.D * 16, wq, g.D * 16, tid);
        for (int i = 0; i < nv; ++i)
            stage_f32(q + ((size_t)(t0 + i) * g.Hq + g.ret_heads[r]) * g.D, qr[i], g.D, tid);
        __syncthreads();
        const int i = tid >> 4, c = tid & 15;
        if (i >= nv) return;
        float acc = 0.0f;
#pragma unroll 16
        for (int d = 0; d < g.D; ++d) acc = __builtin_fmaf(qr[i][d], wq[d * 16 + c], acc);
        qlow_out[((size_t)(t0 + i) * g.n_ret + r) * 16 + c] = f2bf(acc);
        if (c == 0) rmaxk[(size_t)(t0 + i) * g.n_ret + r] = 0u;
        return;
    }
    if (blk == 0 && r == 0 && tid < 8) pool_ctr[tid] = 0ull;   // pool; the row lists and their queues
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;
    float kn = 0.0f;
    for (int i = tid; i < kNormKeys; i += 256) {
        const int key = blk * kNormKeys + i;
        if (key >= n_keys) break;
        const int page = bt[key >> 8];
        const uint4* kp = reinterpret_cast<const uint4*>(k_low + (((size_t)page * g.n_ret + r) * kBlk + (key & 255)) * 16);
        float kf[16];
        unpack8(kp[0], kf);
        unpack8(kp[1], kf + 8);
        float n2 = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) n2 = __builtin_fmaf(kf[c], kf[c], n2);
        kn = fmaxf(kn, n2);
    }
    __shared__ float red[4];
    kn = wave_max(kn);
    if ((tid & 63) == 0) red[tid >> 6] = kn;
    __syncthreads();
    if (tid == 0) knorm[(size_t)r * nblk + blk] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

struct ChunkWs {
    size_t crow, cst, qlow, counts, rmaxk, knorm, tflags, hacc, hcnt, segoff, arrive, lrows, mrows, zrows, ctr, pool, head;
    int nblk, nfw, nsplit;
};

// key-tile runs per row tile of the histogram and recording passes: about six
// waves of workgroups over the chip (four per CU), but runs of at least ~1024
// key tiles (each workgroup's fixed cost: q_low, LDS clears, the merge)
int hist_splits(int n_tok, int n_ret, int n_keys) {
    const int nwg = (n_tok + kTR - 1) / kTR * n_ret, max_tiles = (n_keys + 31) / 32;
    return std::max(1, std::min({kMaxSplit, (6144 + nwg - 1) / nwg, max_tiles / 1024}));
}

// key-tile runs per 256-row group of the maximum pass: about two waves of
// workgroups over the chip, runs of at least ~512 key tiles
int max_runs(int n_tok, int n_ret, int n_keys) {
    const int nwg = (n_tok + kTRM - 1) / kTRM * n_ret, max_tiles = (n_keys + 31) / 32;
    return std::max(1, std::min((2048 + nwg - 1) / nwg, max_tiles / 512));
}

ChunkWs chunk_ws(int rows, int n_ret, int n_keys) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    ChunkWs w;
    w.nblk = (n_keys + kNormKeys - 1) / kNormKeys;
    w.crow = 0;
    w.cst = w.crow + up((size_t)rows * sizeof(CRow));
    w.qlow = w.cst + up((size_t)rows * sizeof(CState));
    w.counts = w.qlow + up((size_t)rows * 16 * 2);
    w.rmaxk = w.counts + up((size_t)rows * 4);
    w.knorm = w.rmaxk + up((size_t)rows * 4);
    w.nfw = (n_keys + 1023) / 1024;                     // one bit per 32-key tile
    w.tflags = w.knorm + up((size_t)n_ret * w.nblk * 4);
    const size_t nrt = (size_t)((rows / n_ret + kTR - 1) / kTR) * n_ret;   // row tiles
    w.nsplit = hist_splits(rows / n_ret, n_ret, n_keys);
    w.hacc = w.tflags + up(nrt * (w.nfw + 1) * 4);
    w.hcnt = w.hacc + up((size_t)rows * kHB * 8);
    w.segoff = w.hcnt + up((size_t)rows * w.nsplit * kProv * 4);
    w.arrive = w.segoff + up((size_t)rows * w.nsplit * 4);
    w.lrows = w.arrive + up(nrt * 4);
    w.mrows = w.lrows + up((size_t)rows * 4);
    w.zrows = w.mrows + up((size_t)rows * 4);
    w.ctr = w.zrows + up((size_t)rows * 4);
    w.pool = w.ctr + 256;
    w.head = w.pool;
    return w;
}

// Per-row path codes of the last chunk selection (inspection).
__global__ void k_csel_paths(const CRow* __restrict__ rows, int n, int32_t* __restrict__ paths) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) paths[i] = rows[i].path;
}

}  // namespace

hipError_t launch_chunk_paths(const Geo& g, const void* ws, int32_t* paths, hipStream_t s) {
    const int rows = g.n_tok * g.n_ret;
    const CRow* crow = (const CRow*)((const char*)ws + chunk_ws(rows, g.n_ret, g.pos0 + g.n_tok).crow);
    hipLaunchKernelGGL(k_csel_paths, dim3((rows + 255) / 256), dim3(256), 0, s, crow, rows, paths);
    return hipGetLastError();
}

size_t chunk_select_head_bytes(int rows, int n_ret, int n_keys) { return chunk_ws(rows, n_ret, n_keys).head; }

size_t chunk_select_ws_bytes(int rows, int n_ret, int n_keys) {
    return chunk_select_head_bytes(rows, n_ret, n_keys) + (size_t)rows * kPoolPerRow * 8;
}

hipError_t launch_chunk_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                               const float* top_p, void* ws, size_t ws_bytes, const SelOut& out, hipStream_t s) {
    const int rows = g.n_tok * g.n_ret;
    const int n_keys = g.pos0 + g.n_tok;
    const ChunkWs w = chunk_ws(rows, g.n_ret, n_keys);
    if (g.D > 128 || ws_bytes < w.head) return hipErrorInvalidValue;
    char* base = (char*)ws;
    CRow* crow = (CRow*)(base + w.crow);
    CState* cst = (CState*)(base + w.cst);
    uint16_t* qlow = (uint16_t*)(base + w.qlow);
    int* counts = (int*)(base + w.counts);
    float* knorm = (float*)(base + w.knorm);
    unsigned long long* ctr = (unsigned long long*)(base + w.ctr);
    uint32_t* tflags = (uint32_t*)(base + w.tflags);
    unsigned long long* pool = (unsigned long long*)(base + w.pool);
    const unsigned long long pool_cap = (ws_bytes - w.head) / 8;
    const dim3 grid((g.n_tok + kTR - 1) / kTR, g.n_ret);
    HistAcc acc;
    acc.hist = (double*)(base + w.hacc);
    acc.cnt = (uint32_t*)(base + w.hcnt);
    acc.segoff = (uint32_t*)(base + w.segoff);
    acc.tflags = tflags;
    acc.arrive = (uint32_t*)(base + w.arrive);
    acc.nt32 = (int)grid.x;
    acc.nfw = w.nfw;
    acc.nsplit = w.nsplit;
    acc.lrows = (uint32_t*)(base + w.lrows);
    acc.mrows = (uint32_t*)(base + w.mrows);
    acc.zrows = (uint32_t*)(base + w.zrows);
    acc.lctr = ctr + 1;
    unsigned long long* zctr = acc.lctr + 4;
    uint32_t* rmaxk = (uint32_t*)(base + w.rmaxk);
    hipLaunchKernelGGL(k_csel_knorm, dim3(w.nblk + (g.n_tok + 15) / 16, g.n_ret), dim3(256), 0, s, g,
                       (const bf16_t*)k_low, n_keys, knorm, w.nblk, ctr, (const bf16_t*)q, (const bf16_t*)w_q, qlow,
                       rmaxk);
    const int nrun = max_runs(g.n_tok, g.n_ret, n_keys);
    hipLaunchKernelGGL(k_csel_max, dim3((g.n_tok + kTRM - 1) / kTRM, g.n_ret, nrun), dim3(256), 0, s, g,
                       (const bf16_t*)k_low, qlow, knorm, w.nblk, cst, rmaxk, acc, nrun);
    hipLaunchKernelGGL(k_csel_hist, dim3(grid.x, grid.y, acc.nsplit), dim3(256), 0, s, g, (const bf16_t*)k_low, top_p,
                       qlow, cst, rmaxk, ctr, pool_cap, acc, crow);
    hipLaunchKernelGGL(k_csel_rec, dim3(grid.x, grid.y, acc.nsplit), dim3(256), 0, s, g, (const bf16_t*)k_low, qlow,
                       cst, pool, acc);
    hipLaunchKernelGGL(k_csel_main, grid, dim3(256), 0, s, g, (const bf16_t*)k_low, top_p, qlow, cst, crow, 0, counts,
                       acc.zrows, zctr);
    hipLaunchKernelGGL(k_csel_resolve, dim3(std::min(rows, 512)), dim3(kRT), 0, s, g, crow, rows, acc.mrows,
                       acc.lctr + 2, (const bf16_t*)k_low, qlow, top_p, pool, counts, acc.zrows, zctr);
    hipLaunchKernelGGL(k_csel_resolve_small, dim3(rows), dim3(kRTS), 0, s, g, crow, (const bf16_t*)k_low, qlow,
                       top_p, pool, counts, acc.zrows, zctr);
    hipLaunchKernelGGL(k_csel_resolve_large, dim3(std::min(rows, 256)), dim3(kRTL), 0, s, g, crow, rows, acc.lrows,
                       acc.lctr, acc.lctr + 1, 0, (const bf16_t*)k_low, qlow, top_p, pool, counts, acc.zrows, zctr);
    // the retry route (rows listed above; each launch ends at once when none is)
    hipLaunchKernelGGL(k_csel_zexact, dim3(std::min(rows * ((n_keys + kZPiece - 1) / kZPiece), 1024)), dim3(256), 0,
                       s, g, crow, rows, acc.zrows, zctr, (const bf16_t*)k_low, qlow);
    hipLaunchKernelGGL(k_csel_main, grid, dim3(256), 0, s, g, (const bf16_t*)k_low, top_p, qlow, cst, crow, 1, counts,
                       acc.zrows, zctr);
    hipLaunchKernelGGL(k_csel_resolve_large, dim3(std::min(rows, 256)), dim3(kRTL), 0, s, g, crow, rows, acc.zrows,
                       zctr, zctr + 2, 1, (const bf16_t*)k_low, qlow, top_p, pool, counts, acc.zrows, zctr);
    hipLaunchKernelGGL(k_csel_rowptr, dim3(1), dim3(1024), 0, s, counts, rows, out.row_ptr, out.capacity,
                       out.status);
    hipLaunchKernelGGL(k_csel_copy, dim3(rows), dim3(256), 0, s, crow, pool, out.row_ptr, out.idx, out.status);
    hipLaunchKernelGGL(k_csel_emit, grid, dim3(64), 0, s, g, (const bf16_t*)k_low, qlow, crow, out.row_ptr,
                       out.idx, out.status);
    return hipGetLastError();
}

}  // namespace rtp
