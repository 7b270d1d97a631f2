// attn_sparse_prefill.hip -- sparse attention of the retrieval heads over their
// selected rows for a prefill chunk, on gfx950 bf16 MFMA.
//
// Method: arXiv 2605.16928 abstract (retrieval heads keep the full KV cache
// and attend to the rows their indexer selects); zhichai.net forum post
// "RTPurbo: Turning Dense LLMs into Sparse Attention Models ...", "Three Key
// Insights" items 2-3.  Every chunk row attends to its own selected set with
// the softmax renormalised over the set.
//
// Consecutive chunk rows of one head select largely the same keys (the
// selected sets of 64 neighbouring rows fill ~75% of their union at the
// clustered workloads), so the attention runs per tile of 64 rows of one
// retrieval head over the union of their sets, 64 union keys at a time, with
// each row's keys masked to its own set.  The key axis is cut into 2^16-key
// windows; a (tile, window) pair is a unit of work.
//   k_sp_winoff  where each row's sorted list enters every window
//   k_sp_union   one workgroup per (tile, window): the union as a bitmap over
//                the window's keys, built from the rows' entries read flat
//                (16-byte loads over the concatenated ranges, so the work
//                follows the entry count, not the longest row); writes the
//                bitmap, the union size, and empty partial results
//   k_sp_tile    one workgroup per (tile, window, split): the union's 1024-key
//                groups g = split, split + S, ... ; per group the union keys
//                (ranks from the bitmap's popcount prefix), their K/V row
//                offsets, and every row's 64-bit key masks of its 16 blocks
//                (one flat pass over the entries); then per 64-key block the
//                gathered K rows (row-major) and V^T (transposed) in LDS, the
//                next block's rows already loading into registers, and
//                S^T = K . Q^T, O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16.
//                Four waves: two 32-row halves x two 32-key halves of each
//                block, the key halves merged at the end.
//   k_sp_combine the partial results of a row (per window and split) merged
//                into its output.
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBM = 64;            // rows per tile
constexpr int kNT = 256;           // threads of the tile kernel
constexpr int kNTU = 512;          // threads of the union kernel (its entry scans take kNTU * kUL pieces a round)
constexpr int kBN = 64;            // union keys per block
constexpr int kD = 128;
constexpr int kKsLd = kD + 8;      // K row stride in LDS (bf16)
constexpr int kVtLd = kBN + 4;     // V^T row stride in LDS (bf16)
constexpr int kWinLog = 16;
constexpr int kWin = 1 << kWinLog; // keys per bitmap window
constexpr int kWords = kWin / 32;
constexpr int kMB = 16;            // blocks per group
constexpr int kGK = kMB * kBN;     // union keys per group
constexpr int kPS = kD + 4;        // floats per partial result: O[D], max, mass (16-byte rows)
constexpr int kMaxSplit = 8;
constexpr int kUL = 8;             // 4-entry pieces per thread and round of an entry scan
constexpr int kPoolG = 4;          // groups a (tile, window) may keep in the block pool
constexpr int kTargetWG = 2048;    // tile workgroups the split aims for

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// element e (0..7) of 8 packed bf16
__device__ __forceinline__ uint32_t bf_at(const uint4& u, int e) {
    const uint32_t w = (e >> 1) == 0 ? u.x : (e >> 1) == 1 ? u.y : (e >> 1) == 2 ? u.z : u.w;
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// The entries of a tile's rows inside one window, as one flat sequence of
// 4-entry pieces: row i covers idx[rb[i], re[i]) and is read from the
// 4-aligned position ra[i]; its pieces are cp[i] .. cp[i+1]-1.
struct Ranges {
    int64_t rb[kBM], re[kBM], ra[kBM];
    int cp[kBM + 1];
};

// Lanes 0..63: row i's range [b, e) (b <= e) into R and the piece prefix.
// The caller synchronises before R is read.
__device__ __forceinline__ void set_ranges(int64_t b, int64_t e, Ranges& R) {
    const int tid = threadIdx.x;
    const int64_t a = b & ~(int64_t)3;
    const int n = e > b ? (int)((e - a + 3) >> 2) : 0;
    R.rb[tid] = b;
    R.re[tid] = e;
    R.ra[tid] = a;
    const int x = (int)wave_incl_scan_u32((uint32_t)n);   // inclusive scan over the wave
    R.cp[tid + 1] = x;
    if (tid == 0) R.cp[0] = 0;
}

// Visit the tile's entries in the window: every thread takes kUL pieces per
// round (16-byte loads where idx is 16-byte aligned and the piece lies inside
// idx_n), and f(row, k[4], valid bits) runs per piece; a piece's keys ascend.
template <int NT, typename F>
__device__ __forceinline__ void for_pieces(const Ranges& R, const int32_t* __restrict__ idx, int64_t idx_n, F&& f) {
    const int tid = threadIdx.x;
    const int total = R.cp[kBM];
    const bool vec = (reinterpret_cast<uintptr_t>(idx) & 15) == 0;
    for (int base = 0; base < total; base += NT * kUL) {
        // the row whose pieces hold piece c: the last i with cp[i] <= c, by six
        // halving steps run for all kUL pieces together
        int lo[kUL];
#pragma unroll
        for (int u = 0; u < kUL; ++u) lo[u] = 0;
#pragma unroll
        for (int step = kBM / 2; step > 0; step >>= 1)
#pragma unroll
            for (int u = 0; u < kUL; ++u)
                if (R.cp[lo[u] + step] <= base + u * NT + tid) lo[u] += step;
        int k[kUL][4];
        uint32_t vm[kUL];
#pragma unroll
        for (int u = 0; u < kUL; ++u) {
            const int c = base + u * NT + tid;
            const int64_t p = R.ra[lo[u]] + 4 * (int64_t)(c - R.cp[lo[u]]);
            const int64_t b = R.rb[lo[u]], e = c < total ? R.re[lo[u]] : 0;
            vm[u] = 0u;
#pragma unroll
            for (int x = 0; x < 4; ++x) vm[u] |= (p + x >= b && p + x < e) ? 1u << x : 0u;
            if (vm[u] && vec && p + 4 <= idx_n) {
                const int4 v = *reinterpret_cast<const int4*>(idx + p);
                k[u][0] = v.x;
                k[u][1] = v.y;
                k[u][2] = v.z;
                k[u][3] = v.w;
            } else {
#pragma unroll
                for (int x = 0; x < 4; ++x) k[u][x] = (vm[u] >> x) & 1u ? idx[p + x] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kUL; ++u) f(lo[u], k[u], vm[u]);
    }
}

// OR bits into LDS words, one atomic per run of equal addresses (the caller's
// addresses come in runs: ascending keys of one row).
__device__ __forceinline__ void merged_or(uint32_t* base, const int (&a)[4], const uint32_t (&bit)[4], uint32_t ok) {
    int cur = -1;
    uint32_t acc = 0u;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (!((ok >> c) & 1u)) continue;
        if (a[c] != cur) {
            if (cur >= 0) atomicOr(&base[cur], acc);
            cur = a[c];
            acc = 0u;
        }
        acc |= bit[c];
    }
    if (cur >= 0) atomicOr(&base[cur], acc);
}

// union rank of a key of the window (its bit is set)
__device__ __forceinline__ int union_rank(const uint32_t* bm, const uint32_t* wpre, int off) {
    const int wd = off >> 5;
    return (int)(wpre[wd] + __popc(bm[wd] & ((1u << (off & 31)) - 1u)));
}

// Bitmap popcount prefix: wpre[w] = set bits of words 0..w-1; returns the total.
template <int NT>
__device__ __forceinline__ uint32_t bitmap_prefix(const uint32_t* bm, uint32_t* wpre, unsigned long long* scan) {
    const int tid = threadIdx.x;
    constexpr int per = kWords / NT;
    uint32_t loc = 0;
#pragma unroll
    for (int k = 0; k < per; ++k) loc += __popc(bm[tid * per + k]);
    unsigned long long tot;
    uint32_t ex = (uint32_t)block_excl_scan_u64<NT>(loc, &tot, scan);
#pragma unroll
    for (int k = 0; k < per; ++k) {
        wpre[tid * per + k] = ex;
        ex += __popc(bm[tid * per + k]);
    }
    return (uint32_t)tot;
}

// K/V row number (page * pool heads + slot of the kv head) * 256 + slot of a key
__device__ __forceinline__ uint32_t kv_row(const Geo& g, const int32_t* bt, int kvh, uint32_t key) {
    return ((uint32_t)bt[key >> 8] * (uint32_t)g.pool_heads + (uint32_t)g.kv_slot[kvh]) * (uint32_t)kBlk +
           (key & 255u);
}

__global__ void k_sp_reset(uint32_t* ctr) {
    if (threadIdx.x == 0) *ctr = 0u;
}

// One block of the pool: the K/V row numbers of its 64 union keys and every
// tile row's 64-bit key mask.
struct PoolBlock {
    uint32_t kvrow[kBN];
    uint32_t mask[kBM][2];
};

// grid (ntile * nwin, n_ret), kNTU threads.  A (tile, window) whose union has
// at most kPoolG groups takes its blocks from the pool (ctr counts the blocks
// handed out) and writes them whole; otherwise (or when the pool is full) it
// leaves the bitmap for the tile kernel, which then builds each group itself.
__global__ __launch_bounds__(kNTU) void k_sp_union(Geo g, const int64_t* __restrict__ row_ptr, int nwin, int nsplit,
                                                  const int32_t* __restrict__ idx, int64_t idx_n,
                                                  const int32_t* __restrict__ status, int64_t* __restrict__ wr,
                                                  uint32_t* __restrict__ tw_n, int32_t* __restrict__ tw_off,
                                                  uint32_t* __restrict__ tw_bm, uint32_t* __restrict__ ctr,
                                                  PoolBlock* __restrict__ pool, int pool_blocks,
                                                  float* __restrict__ part) {
    if (*status != 0) return;
    __shared__ Ranges R;
    __shared__ __attribute__((aligned(16))) uint32_t bm[kWords];
    __shared__ uint32_t wpre[kWords];
    __shared__ __attribute__((aligned(16))) uint32_t mk[kPoolG * kMB][kBM][2];
    __shared__ unsigned long long scan[kNTU / 64 + 1];
    __shared__ int64_t bnd[2][kBM];
    __shared__ int s_base;
    const int tid = threadIdx.x;
    const int r = blockIdx.y;
    const int ntile = (g.n_tok + kBM - 1) / kBM;
    const int tile = blockIdx.x / nwin, win = blockIdx.x - tile * nwin;
    const int t0 = tile * kBM, w0 = win * kWin;
    const int kvh = g.ret_heads[r] / g.group;
    const size_t tw = ((size_t)r * ntile + tile) * nwin + win;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;
    for (int x = tid; x < kWords; x += kNTU) bm[x] = 0u;
    // empty partial results of the tile's rows for this window
    for (int x = tid; x < kBM * nsplit; x += kNTU) {
        const int i = x / nsplit, sp = x - i * nsplit;
        const int t = t0 + i;
        if (t < g.n_tok) {
            float* pp = part + (((size_t)(t * g.n_ret + r) * nwin + win) * nsplit + sp) * kPS;
            pp[kD] = -INFINITY;
            pp[kD + 1] = 0.0f;
        }
    }
    // where each row's sorted list crosses the window's two edges (lanes 0..63
    // the lower edge, 64..127 the upper one)
    if (tid < 2 * kBM) {
        const int i = tid & (kBM - 1), side = tid >> 6;
        const int t = t0 + i;
        int64_t lo = 0, hi = 0;
        if (t < g.n_tok) {
            const int row = t * g.n_ret + r;
            hi = min(row_ptr[row + 1], idx_n);
            lo = min(row_ptr[row], hi);
        }
        const int64_t bound = (int64_t)w0 + (int64_t)side * kWin;
        while (lo < hi) {                              // first position with idx >= bound
            const int64_t mid = lo + ((hi - lo) >> 1);
            if (idx[mid] < bound) lo = mid + 1; else hi = mid;
        }
        bnd[side][i] = lo;
    }
    __syncthreads();
    if (tid < kBM) {
        const int64_t b = bnd[0][tid], e = max(bnd[1][tid], b);
        set_ranges(b, e, R);
        if (t0 + tid < g.n_tok) {
            int64_t* w = wr + ((size_t)(t0 + tid) * g.n_ret + r) * nwin * 2 + 2 * win;
            w[0] = b;
            w[1] = e;
        }
    }
    __syncthreads();
    // the union bitmap
    for_pieces<kNTU>(R, idx, idx_n, [&](int, const int (&k)[4], uint32_t vm) {
        int a[4];
        uint32_t bit[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int off = k[c] - w0;
            if ((unsigned)off >= (unsigned)kWin) vm &= ~(1u << c);
            a[c] = off >> 5;
            bit[c] = 1u << (off & 31);
        }
        merged_or(bm, a, bit, vm);
    });
    __syncthreads();
    const uint32_t nU = bitmap_prefix<kNTU>(bm, wpre, scan);
    const int nb = (int)((nU + kBN - 1) / kBN);
    if (tid == 0) {
        tw_n[tw] = nU;
        int base = -1;
        if (nb > 0 && nb <= kPoolG * kMB) {
            base = (int)atomicAdd(ctr, (uint32_t)nb);
            if (base + nb > pool_blocks) base = -1;
        }
        tw_off[tw] = base;
        s_base = base;
    }
    for (int x = tid; x < kPoolG * kMB * kBM * 2; x += kNTU) (&mk[0][0][0])[x] = 0u;
    __syncthreads();
    const int base = s_base;
    if (nU == 0) return;
    if (base < 0) {
        uint4* dst = reinterpret_cast<uint4*>(tw_bm + tw * kWords);
        for (int x = tid; x < kWords / 4; x += kNTU) dst[x] = *reinterpret_cast<const uint4*>(&bm[4 * x]);
        return;
    }
    // the blocks: every key's K/V row number, every row's masks
    {
        constexpr int per = kWords / kNTU;
#pragma unroll
        for (int k = 0; k < per; ++k) {
            const int wd = tid * per + k;
            uint32_t bits = bm[wd];
            uint32_t rank = wpre[wd];
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1u;
                pool[base + (rank >> 6)].kvrow[rank & 63] = kv_row(g, bt, kvh, (uint32_t)(w0 + wd * 32 + b));
                ++rank;
            }
        }
        if (tid < kBN) {                              // the last block's unused key slots
            const int u = (int)nU + tid;
            if (u < nb * kBN) pool[base + (u >> 6)].kvrow[u & 63] = 0u;
        }
    }
    for_pieces<kNTU>(R, idx, idx_n, [&](int row, const int (&k)[4], uint32_t vm) {
        int a[4];
        uint32_t bit[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            int off = k[c] - w0;
            if ((unsigned)off >= (unsigned)kWin) {
                vm &= ~(1u << c);
                off = 0;
            }
            const int lr = union_rank(bm, wpre, off);
            a[c] = ((lr >> 6) * kBM + row) * 2 + ((lr >> 5) & 1);
            bit[c] = 1u << (lr & 31);
        }
        merged_or(&mk[0][0][0], a, bit, vm);
    });
    __syncthreads();
    for (int x = tid; x < nb * kBM * 2; x += kNTU) {
        const int b = x / (kBM * 2), y = x - b * (kBM * 2);
        (&pool[base + b].mask[0][0])[y] = (&mk[b][0][0])[y];
    }
}

// LDS of the tile kernel.  The K / V^T staging area is reused at the end for
// the exchange of the key halves' accumulators.
struct TileSmem {
    union {
        struct {
            bf16_t Ks[kBN * kKsLd];
            bf16_t Vt[kD * kVtLd];
        } kv;
        float xo[2 * 64 * 64];                        // [row half][accumulator][lane]
    } u;
    uint32_t bm[kWords];                              // union bitmap of the window
    uint32_t wpre[kWords];                            // exclusive prefix of its word popcounts
    uint32_t memb[kMB][kBM][2];                       // per block and row: 64-bit key mask
    uint32_t roff[kGK];                               // the group's keys, then their K/V row numbers
    float xm[2][64], xl[2][64];
    unsigned long long scan[kNT / 64 + 1];
    int klo, khi;                                     // first and last union key of the group
    Ranges R;
};

// One group of a union the pool did not take, built in LDS from the bitmap and
// the rows' entries: the union keys of ranks [g0, g1) (their K/V row numbers
// in roff) and every row's 64-bit masks of the group's blocks (an entry whose
// key lies in the group's key range [klo, khi] has its rank in [g0, g1)).
template <typename S>
__device__ void build_group(const Geo& g, S& sm, const int32_t* __restrict__ idx, int64_t idx_n, const int32_t* bt,
                            int kvh, int w0, int g0, int g1) {
    const int tid = threadIdx.x;
    for (int x = tid; x < kMB * kBM * 2; x += kNT) (&sm.memb[0][0][0])[x] = 0u;
    {
        constexpr int per = kWords / kNT;
#pragma unroll
        for (int k = 0; k < per; ++k) {
            const int wd = tid * per + k;
            const uint32_t pre = sm.wpre[wd];
            uint32_t bits = sm.bm[wd];
            if (pre >= (uint32_t)g1 || pre + __popc(bits) <= (uint32_t)g0) continue;
            uint32_t rank = pre;
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1u;
                if (rank >= (uint32_t)g0 && rank < (uint32_t)g1) {
                    const uint32_t key = (uint32_t)(w0 + wd * 32 + b);
                    sm.roff[rank - g0] = kv_row(g, bt, kvh, key);
                    if (rank == (uint32_t)g0) sm.klo = (int)key;
                    if (rank == (uint32_t)(g1 - 1)) sm.khi = (int)key;
                }
                ++rank;
            }
        }
    }
    __syncthreads();
    const int klo = sm.klo, khi = sm.khi;
    for_pieces<kNT>(sm.R, idx, idx_n, [&](int row, const int (&k)[4], uint32_t vm) {
        int a[4];
        uint32_t bit[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool in = ((vm >> c) & 1u) && k[c] >= klo && k[c] <= khi;
            if (!in) vm &= ~(1u << c);
            const int lr = union_rank(sm.bm, sm.wpre, in ? k[c] - w0 : 0) - g0;
            a[c] = ((lr >> 6) * kBM + row) * 2 + ((lr >> 5) & 1);
            bit[c] = 1u << (lr & 31);
        }
        merged_or(&sm.memb[0][0][0], a, bit, vm);
    });
    __syncthreads();
}

// grid (ntile * nwin * nsplit, n_ret), kNT threads: tile, window, split.
__global__ __launch_bounds__(kNT) void k_sp_tile(Geo g, const bf16_t* __restrict__ q,
                                                 const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
                                                 const int64_t* __restrict__ wr, int nwin, int nsplit,
                                                 const int32_t* __restrict__ idx, int64_t idx_n,
                                                 const int32_t* __restrict__ status, const uint32_t* __restrict__ tw_n,
                                                 const int32_t* __restrict__ tw_off,
                                                 const uint32_t* __restrict__ tw_bm,
                                                 const PoolBlock* __restrict__ pool, float* __restrict__ part) {
    if (*status != 0) return;
    __shared__ __attribute__((aligned(16))) TileSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r = blockIdx.y;
    const int ntile = (g.n_tok + kBM - 1) / kBM;
    const int sp = blockIdx.x % nsplit;
    const int tw_x = blockIdx.x / nsplit;
    const int tile = tw_x / nwin, win = tw_x - tile * nwin;
    const size_t tw = ((size_t)r * ntile + tile) * nwin + win;
    const int nU = (int)tw_n[tw];
    const int ngroups = (nU + kGK - 1) / kGK;
    if (sp >= ngroups) return;
    const int hq = g.ret_heads[r], kvh = hq / g.group;
    const int t0 = tile * kBM, w0 = win * kWin;
    const int rh = wid & 1, kh = wid >> 1;           // row half, key half of this wave
    const int hh = lane >> 5, qi = lane & 31;
    const int t = t0 + rh * 32 + qi;                  // query row of this lane
    const bool qok = t < g.n_tok;
    const float sc = g.attn_scale * kLog2e;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;

    const int pbase = tw_off[tw];                     // >= 0: the union's blocks are in the pool
    if (pbase < 0) {
        // the bitmap, its popcount prefix and the rows' entry ranges
        const uint4* src = reinterpret_cast<const uint4*>(tw_bm + tw * kWords);
        for (int x = tid; x < kWords / 4; x += kNT) *reinterpret_cast<uint4*>(&sm.bm[4 * x]) = src[x];
        __syncthreads();
        bitmap_prefix<kNT>(sm.bm, sm.wpre, sm.scan);
        if (tid < kBM) {
            int64_t b = 0, e = 0;
            if (t0 + tid < g.n_tok) {
                const int64_t* w = wr + ((size_t)(t0 + tid) * g.n_ret + r) * nwin * 2 + 2 * win;
                b = w[0];
                e = w[1];
            }
            set_ranges(b, e, sm.R);
        }
    }

    // Q^T operand: lane holds Q[t][16 kk + 8 hh + 0..7] for kk = 0..7
    uint4 qreg[8];
    {
        const bf16_t* qp = q + ((size_t)min(t, g.n_tok - 1) * g.Hq + hq) * kD + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            qreg[kk] = qok ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
    }
    f32x16_t oacc[4];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dd][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    // staging of a block: thread = key pair kp (keys 2 kp, 2 kp + 1) x 16 dims
    const int kp = tid & 31, dq = tid >> 5;
    uint4 kr[4], vr[4];
    const auto load_blk = [&](int b0, int nk) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kl = b0 + 2 * kp + j;
            if (kl < nk) {
                const size_t base = (size_t)sm.roff[kl] * kD + 16 * dq;
                kr[2 * j] = *reinterpret_cast<const uint4*>(kc + base);
                kr[2 * j + 1] = *reinterpret_cast<const uint4*>(kc + base + 8);
                vr[2 * j] = *reinterpret_cast<const uint4*>(vc + base);
                vr[2 * j + 1] = *reinterpret_cast<const uint4*>(vc + base + 8);
            } else {
                kr[2 * j] = kr[2 * j + 1] = vr[2 * j] = vr[2 * j + 1] = make_uint4(0, 0, 0, 0);
            }
        }
    };

    for (int grp = sp; grp < ngroups; grp += nsplit) {
        const int g0 = grp * kGK, g1 = min(nU, g0 + kGK);
        const int nk = g1 - g0;
        __syncthreads();                              // the previous group is done with memb / roff
        if (pbase >= 0) {
            // the group's blocks from the pool: key rows and masks
            const PoolBlock* pb = pool + pbase + g0 / kBN;
            const int nbk = (nk + kBN - 1) / kBN;
            for (int x = tid; x < nbk * kBN; x += kNT) sm.roff[x] = pb[x >> 6].kvrow[x & 63];
            for (int x = tid; x < nbk * kBM * 2; x += kNT) {
                const int b = x / (kBM * 2), y = x - b * (kBM * 2);
                (&sm.memb[b][0][0])[y] = (&pb[b].mask[0][0])[y];
            }
            __syncthreads();
        } else {
            build_group(g, sm, idx, idx_n, bt, kvh, w0, g0, g1);
        }
        const int nb = (nk + kBN - 1) / kBN;
        load_blk(0, nk);
        for (int blk = 0; blk < nb; ++blk) {
            if (blk > 0) __syncthreads();             // the previous block's LDS reads are done
            // registers -> LDS: K rows, V^T as key pairs
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                bf16_t* kd = &sm.u.kv.Ks[(2 * kp + j) * kKsLd + 16 * dq];
                *reinterpret_cast<uint4*>(kd) = kr[2 * j];
                *reinterpret_cast<uint4*>(kd + 8) = kr[2 * j + 1];
            }
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const uint4& a = vr[x >> 3];
                const uint4& b = vr[2 + (x >> 3)];
                const uint32_t w = bf_at(a, x & 7) | (bf_at(b, x & 7) << 16);
                *reinterpret_cast<uint32_t*>(&sm.u.kv.Vt[(16 * dq + x) * kVtLd + 2 * kp]) = w;
            }
            if (blk + 1 < nb) load_blk((blk + 1) * kBN, nk);
            __syncthreads();
            const uint32_t mask = sm.memb[blk][rh * 32 + qi][kh];

            // S^T for this wave's 32 keys and 32 rows
            f32x16_t s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.0f;
            {
                const bf16_t* krow = &sm.u.kv.Ks[(32 * kh + qi) * kKsLd + 8 * hh];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const uint4 a = *reinterpret_cast<const uint4*>(krow + 16 * kk);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[kk]), s, 0, 0, 0);
                }
            }
            // scale, mask, block maximum of this lane's query
            float mt = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kq = (i >> 2) * 8 + 4 * hh + (i & 3);
                const bool ok = qok && ((mask >> kq) & 1u);
                const float v = ok ? s[i] * sc : -INFINITY;
                s[i] = v;
                mt = fmaxf(mt, v);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            uint32_t pb[8];                           // P^T as bf16 pairs
            if (m_new == -INFINITY) {
#pragma unroll
                for (int x = 0; x < 8; ++x) pb[x] = 0u;
            } else {
                // (raw v_exp_f32 below: its results under 2^-126 weigh nothing
                // against the running maximum's weight of 1)
                if (__ballot(m_new > m_run)) {        // rescale only when a maximum of the wave moved
                    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
                    l_run *= corr;
#pragma unroll
                    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[dd][i] *= corr;
                }
                m_run = m_new;
                float p[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
                    l_run += p[i];
                }
#pragma unroll
                for (int x = 0; x < 8; ++x) pb[x] = pack2(p[2 * x], p[2 * x + 1]);
            }
            // O^T += V^T P^T
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint4 bp = make_uint4(pb[4 * kk], pb[4 * kk + 1], pb[4 * kk + 2], pb[4 * kk + 3]);
                const int kc0 = 32 * kh + 16 * kk + 4 * hh;
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    const bf16_t* vrp = &sm.u.kv.Vt[(32 * dd + qi) * kVtLd + kc0];
                    const uint2 lo = *reinterpret_cast<const uint2*>(vrp);
                    const uint2 hi = *reinterpret_cast<const uint2*>(vrp + 8);
                    const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    oacc[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bp), oacc[dd], 0, 0, 0);
                }
            }
        }
    }
    // merge the key halves: the second half's waves hand over through LDS
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();
    if (kh == 1) {
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.u.xo[(rh * 64 + dd * 16 + i) * 64 + lane] = oacc[dd][i];
        sm.xm[rh][lane] = m_run;
        sm.xl[rh][lane] = l_run;
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = sm.xm[rh][lane], l1 = sm.xl[rh][lane];
    const float M = fmaxf(m_run, m1);
    const float f0 = m_run == -INFINITY ? 0.0f : exp2f(m_run - M);
    const float f1 = m1 == -INFINITY ? 0.0f : exp2f(m1 - M);
    const float l_tot = l_run * f0 + l1 * f1;
    if (!qok || !(l_tot > 0.0f)) return;
    // lane holds O[t][32 dd + 8 (i/4) + 4 hh + (i%4)]
    float* pp = part + (((size_t)(t * g.n_ret + r) * nwin + win) * nsplit + sp) * kPS;
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = 32 * dd + 8 * r4 + 4 * hh;
            float o[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o[c] = oacc[dd][4 * r4 + c] * f0 + sm.u.xo[(rh * 64 + dd * 16 + 4 * r4 + c) * 64 + lane] * f1;
            *reinterpret_cast<float4*>(pp + d0) = make_float4(o[0], o[1], o[2], o[3]);
        }
    if (hh == 0) {
        pp[kD] = M;
        pp[kD + 1] = l_tot;
    }
}

// Merge of a row's partial results (every window and split; empty ones hold
// mass 0).  grid (ceil(rows / 2)), 128 threads: a row per 64 lanes, lane w
// reading slot w's maximum and mass, then two output elements per lane.  A row
// with an empty set gets zeros.
__global__ __launch_bounds__(128) void k_sp_combine(Geo g, int nslot, const float* __restrict__ part,
                                                   const int32_t* __restrict__ status, bf16_t* __restrict__ out) {
    if (*status != 0) return;
    const int row = blockIdx.x * 2 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int rows = g.n_tok * g.n_ret;
    if (row >= rows) return;
    const int t = row / g.n_ret, r = row - t * g.n_ret;
    const float* pr = part + (size_t)row * nslot * kPS;
    // the largest maximum of the live slots, 64 slots per pass
    float M = -INFINITY;
    for (int w0 = 0; w0 < nslot; w0 += 64) {
        if (w0 + lane < nslot) {
            const float2 h = *reinterpret_cast<const float2*>(pr + (size_t)(w0 + lane) * kPS + kD);
            if (h.y > 0.0f) M = fmaxf(M, h.x);
        }
    }
    M = wave_max(M);
    float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int w0 = 0; w0 < nslot; w0 += 64) {
        float f = 0.0f, mass = 0.0f;
        if (w0 + lane < nslot) {
            const float2 h = *reinterpret_cast<const float2*>(pr + (size_t)(w0 + lane) * kPS + kD);
            if (h.y > 0.0f) {
                f = exp2f(h.x - M);
                mass = h.y;
            }
        }
        l += wave_sum(mass * f);
        unsigned long long todo = __ballot(mass > 0.0f);
        while (todo) {
            const int w = __ffsll((long long)todo) - 1;
            todo &= todo - 1ull;
            const float fw = __shfl(f, w);
            const float2 v = *reinterpret_cast<const float2*>(pr + (size_t)(w0 + w) * kPS + 2 * lane);
            o0 += v.x * fw;
            o1 += v.y * fw;
        }
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    *reinterpret_cast<uint32_t*>(out + ((size_t)t * g.Hq + g.ret_heads[r]) * kD + 2 * lane) = pack2(o0 * inv, o1 * inv);
}

struct SpPlan {
    int nwin, ntile, nsplit, pool_blocks;
    size_t n_tw, off_wr, off_twn, off_twoff, off_bm, off_pool, off_part, bytes;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

SpPlan sp_plan(int n_tok, int n_ret, int n_keys) {
    SpPlan p;
    p.nwin = (n_keys + kWin - 1) / kWin;
    p.ntile = (n_tok + kBM - 1) / kBM;
    p.n_tw = (size_t)p.ntile * n_ret * p.nwin;
    p.nsplit = (int)std::min<size_t>(kMaxSplit, std::max<size_t>(1, (kTargetWG + p.n_tw - 1) / p.n_tw));
    const size_t rows = (size_t)n_tok * n_ret;
    // pooled blocks: a quarter block per (row, window), at least 1024
    p.pool_blocks = (int)std::min<size_t>(1u << 30, std::max<size_t>(1024, rows * p.nwin / 4));
    size_t o = 256;                                   // the pool's block counter
    p.off_wr = o;
    o = align256(o + rows * p.nwin * 2 * 8);          // each row's entry range per window
    p.off_twn = o;
    o = align256(o + p.n_tw * 4);
    p.off_twoff = o;
    o = align256(o + p.n_tw * 4);
    p.off_bm = o;
    o = align256(o + p.n_tw * kWords * 4);
    p.off_pool = o;
    o = align256(o + (size_t)p.pool_blocks * sizeof(PoolBlock));
    p.off_part = o;
    o = align256(o + rows * p.nwin * p.nsplit * kPS * 4);
    p.bytes = o;
    return p;
}

}  // namespace

size_t sparse_prefill_ws_bytes(int n_tok, int n_ret, int n_keys) { return sp_plan(n_tok, n_ret, n_keys).bytes; }

hipError_t launch_sparse_prefill(const Geo& g, const void* q, const void* k, const void* v, const int64_t* row_ptr,
                                 const int32_t* idx, int64_t idx_n, const int32_t* status, void* out, void* ws,
                                 hipStream_t s) {
    const int rows = g.n_tok * g.n_ret;
    const SpPlan p = sp_plan(g.n_tok, g.n_ret, g.pos0 + g.n_tok);
    char* base = (char*)ws;
    uint32_t* ctr = (uint32_t*)base;
    int64_t* wr = (int64_t*)(base + p.off_wr);
    uint32_t* tw_n = (uint32_t*)(base + p.off_twn);
    int32_t* tw_off = (int32_t*)(base + p.off_twoff);
    uint32_t* tw_bm = (uint32_t*)(base + p.off_bm);
    PoolBlock* pool = (PoolBlock*)(base + p.off_pool);
    float* part = (float*)(base + p.off_part);
    hipLaunchKernelGGL(k_sp_reset, dim3(1), dim3(64), 0, s, ctr);
    hipLaunchKernelGGL(k_sp_union, dim3(p.ntile * p.nwin, g.n_ret), dim3(kNTU), 0, s, g, row_ptr, p.nwin, p.nsplit,
                       idx, idx_n, status, wr, tw_n, tw_off, tw_bm, ctr, pool, p.pool_blocks, part);
    hipLaunchKernelGGL(k_sp_tile, dim3(p.ntile * p.nwin * p.nsplit, g.n_ret), dim3(kNT), 0, s, g, (const bf16_t*)q,
                       (const bf16_t*)k, (const bf16_t*)v, wr, p.nwin, p.nsplit, idx, idx_n, status, tw_n, tw_off, tw_bm,
                       pool, part);
    hipLaunchKernelGGL(k_sp_combine, dim3((rows + 1) / 2), dim3(128), 0, s, g, p.nwin * p.nsplit, part, status,
                       (bf16_t*)out);
    return hipGetLastError();
}

}  // namespace rtp
