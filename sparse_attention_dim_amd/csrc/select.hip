// select.hip -- indexer query projection, indexer scores and dynamic top-p
// selection on gfx950 (VALU; the score is a K=16 contraction read once per key,
// so the scoring pass is bound by the HBM stream of the indexer key cache).
//
// Method: arXiv 2605.16928 abstract obs. (2)-(3) (16-dimensional indexer,
// dynamic top-p instead of fixed top-k); zhichai.net forum post "RTPurbo:
// Turning Dense LLMs into Sparse Attention Models ...", "Three Key Insights"
// items 2-3 (low-frequency projection; cumulative top-p).  The forum's
// "Open Questions and Limitations" notes that per-query token counts are
// unfriendly to GPU parallelism; here the scoring pass is split into fixed
// 4096-key chunks so variable budgets never change its launch shape.
//
// Passes (one row = one (query token, retrieval head) pair):
//   score:   q_low = bf16(fp32 chain over d of q . W_q) (every workgroup of the
//            row forms it while its first indexer-key loads are in flight),
//            fp32 chain scores of every key of a chunk, the chunk maximum m_c,
//            the chunk's cumulative mass histogram (exact fixed-point weights
//            exp(s (d - m_c)) summed over bins of x_c = s (m_c - d), 1/4 wide),
//            a bit per key flagging the lowest kLowBin + 1 bins, and the
//            chunk's list of those flagged keys (score key and index, index
//            order, the first kFl of them)
//   row:     one workgroup per row.  Row maximum m and total mass
//            Z = sum_c exp(s (m_c - m)) Z_c; every chunk bin whose upper edge
//            lies below a threshold X on the row's x axis certainly holds
//            keys with x < X, which gives a lower bound of the mass above
//            any X.  The smallest X whose bound reaches the target fixes the
//            candidate set U = {d >= m - X / s}: it holds every key ranked at
//            or above the cut.  U is taken from the chunks' flagged-key lists
//            when they hold it (else from the key flags and the stored
//            scores, or from the row's scores formed again) into LDS, and the
//            cut is found by radix selection over its score keys with exact
//            masses per bucket (ties: lowest indices first); when U does not
//            fit the workspace list the same selection runs over the row's
//            scores.  U is gathered in index order, so the selected keys are
//            its filter.
//   emit:    CSR row pointers, the capacity check, and the selected indices
//            of every row (the one-call decode step writes them from its
//            sparse attention items instead)
// Workgroups of one pass never wait on each other: every hand-off between
// workgroups is a kernel boundary (a device-scope fence per workgroup costs an
// L2 write-back and invalidate on this multi-XCD part).
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"
#include "win_mfma.hpp"

namespace rtp {

namespace {

constexpr float kCBPerUnit = 4.0f;   // chunk histogram bins per unit of x
constexpr int kGB = 256;             // row threshold grid (same width), X = k / 4
constexpr int kRT = 512;             // row workgroup
constexpr int kNR = 2048;            // radix buckets of the narrowing fallback
constexpr int kMaxChunks = 256;      // 2^20 keys

__device__ __forceinline__ void unpack8(uint4 a, float* f) {
    f[0] = __uint_as_float(a.x << 16); f[1] = __uint_as_float(a.x & 0xFFFF0000u);
    f[2] = __uint_as_float(a.y << 16); f[3] = __uint_as_float(a.y & 0xFFFF0000u);
    f[4] = __uint_as_float(a.z << 16); f[5] = __uint_as_float(a.z & 0xFFFF0000u);
    f[6] = __uint_as_float(a.w << 16); f[7] = __uint_as_float(a.w & 0xFFFF0000u);
}

struct RowInfo {
    int lrow, row, t, r, b, pos, L, nch;
};

__device__ __forceinline__ RowInfo row_info(const Geo& g, int row0, int lrow) {
    RowInfo ri;
    ri.lrow = lrow;
    ri.row = row0 + lrow;
    ri.t = ri.row / g.n_ret;
    ri.r = ri.row - ri.t * g.n_ret;
    ri.b = row_seq(g, ri.t);
    ri.pos = row_pos(g, ri.t);
    ri.L = ri.pos + 1;
    ri.nch = (ri.L + kChunk - 1) / kChunk;
    return ri;
}

// ---------------------------------------------------------------------------
// Scores.  grid (nchunk, rows), 256 threads.  Thread i of chunk c scores keys
// c*4096 + 256*k + i, k = 0..15, i.e. slot i of the chunk's 16 pages: every
// iteration reads one page's 8 KiB run of the head's indexer keys, coalesced.
// STATS: also the chunk maximum, the chunk's mass histogram and a bit per key
// flagging chunk bins <= kLowBin.
// ---------------------------------------------------------------------------
template <typename T, int STATS>
__global__ __launch_bounds__(256) void k_sel_score(Geo g, const T* __restrict__ q, const T* __restrict__ w_q,
                                                   bf16_t* __restrict__ k_low, int row0, SelWs ws, SelOut out,
                                                   KeyAppend ap) {
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    if (STATS && chunk == 0 && tid == 0 && ri.lrow == 0 && row0 == 0) {
        *out.status = 0;
        out.row_ptr[0] = 0;
    }
    if (chunk >= ri.nch) return;
    __shared__ float wmax[4];
    __shared__ unsigned long long hist[kCB];
    __shared__ unsigned hcnt[kCB];
    __shared__ uint32_t wcnt[STATS ? 64 : 1];            // flagged keys per 64-key word of the chunk
    __shared__ __align__(16) float qrow[128];
    __shared__ __align__(16) float wq[128 * kIdx];
    __shared__ float qs[kIdx];
    __shared__ float knew[kIdx];                          // the appended token's indexer key (fused append)
    __shared__ __align__(16) float krow[STATS ? 128 : 1];
    __shared__ __align__(16) float wkn[STATS ? 128 * kIdx : 1];
    const int32_t* bt = g.block_table + (size_t)ri.b * g.max_blocks;
    float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int jbase = chunk * kChunk;

    // The chunk's 16 page ids, one per lane (clamped to the row's last page;
    // slots past the row's end are read but never used), then read out by
    // lane number: the loads of a 4-page group wait on no scalar load.
    const int last_page = (ri.L - 1) >> 8;
    const int my_page = bt[min((jbase >> 8) + (tid & 15), last_page)];
    // q and W_q into registers first (16-byte pieces: W_q is at most 512 of
    // them, q at most 32), so that their wait does not cover the key loads
    const int h = g.ret_heads[ri.r];
    const T* qp = q + ((size_t)ri.t * g.Hq + h) * g.D;
    const T* wp = w_q + (size_t)ri.r * g.D * kIdx;
    constexpr int V = 16 / sizeof(T);
    const bool vec = ((reinterpret_cast<uintptr_t>(qp) | reinterpret_cast<uintptr_t>(wp)) & 15) == 0;
    uint4 wreg[2], qreg = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 2; ++k)
        wreg[k] = vec && (tid + 256 * k) * V < g.D * kIdx ? reinterpret_cast<const uint4*>(wp)[tid + 256 * k]
                                                           : make_uint4(0, 0, 0, 0);
    if (vec && tid * V < g.D) qreg = reinterpret_cast<const uint4*>(qp)[tid];
    // a decode step with the indexer-key append fused in: the workgroup of the
    // chunk holding the query's position forms that token's indexer key for
    // this row's head from its K row and W_k (the fixed-order chain of
    // rtp_indexer_append), stores it, and scores the position with it
    const bool app = STATS && ap.w_k != nullptr && g.kind == 0 && chunk == (ri.L - 1) / kChunk;
    const int jnew = app ? ri.L - 1 : -1;
    int new_page = 0;
    if (app) {
        // W_k and the K row straight into LDS (only this workgroup of the row waits on them)
        const T* wk = (const T*)ap.w_k + (size_t)ri.r * g.D * kIdx;
        for (int x = tid; x < g.D * kIdx; x += 256) wkn[x] = ld(wk + x);
        new_page = bt[jnew >> 8];
        if (tid < g.D) {
            const size_t ko = kv_rowidx(g, new_page, h / g.group, jnew & 255) * (size_t)g.D + tid;
            krow[tid] = g.kv_fp8 ? ldk((const fp8e4_t*)ap.k + ko, g.k_scale) : ldk((const T*)ap.k + ko, 1.0f);
        }
    }
    // all four groups of four pages in flight before the first is scored (32 x
    // 16-byte loads per thread outstanding)
    uint4 bufA[8], bufB[8];
    auto load_group = [&](int k0, uint4* buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int page = __builtin_amdgcn_readlane(my_page, k0 + u);
            const uint4* kp = reinterpret_cast<const uint4*>(
                k_low + (((size_t)page * g.n_ret + ri.r) * kBlk + tid) * kIdx);
            buf[2 * u] = kp[0];
            buf[2 * u + 1] = kp[1];
        }
    };
    load_group(0, bufA);
    load_group(4, bufB);
    // q_low: the query row and W_q staged through LDS, the fixed-order chain
    // over d run by 16 lanes while the first key loads are in flight
    if (vec) {
        const auto put = [&](const uint4& u, float* dst) {
            if (sizeof(T) == 4) {
                *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(u.x), __uint_as_float(u.y),
                                                              __uint_as_float(u.z), __uint_as_float(u.w));
            } else {
                float f[8];
                unpack8(u, f);
                *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
            }
        };
#pragma unroll
        for (int k = 0; k < 2; ++k)
            if ((tid + 256 * k) * V < g.D * kIdx) put(wreg[k], wq + (tid + 256 * k) * V);
        if (tid * V < g.D) put(qreg, qrow + tid * V);
    } else {
        stage_f32(qp, qrow, g.D, tid);
        stage_f32(wp, wq, g.D * kIdx, tid);
    }
    if (STATS && tid < kCB) {
        hist[tid] = 0ull;
        hcnt[tid] = 0u;
    }
    __syncthreads();
    if (tid < kIdx) {
        float acc = 0.0f;
#pragma unroll 16
        for (int d = 0; d < g.D; ++d) acc = __builtin_fmaf(qrow[d], wq[d * kIdx + tid], acc);
        const bf16_t qb = f2bf(acc);
        qs[tid] = bf2f(qb);
        if (chunk == 0) ws.qlow[(size_t)ri.lrow * kIdx + tid] = qb;
    } else if (app && tid >= 64 && tid < 64 + kIdx) {   // another wavefront: the two chains run side by side
        const int c = tid - 64;
        float acc = 0.0f;
#pragma unroll 16
        for (int d = 0; d < g.D; ++d) acc = __builtin_fmaf(krow[d], wkn[d * kIdx + c], acc);
        const bf16_t kb = f2bf(acc);
        knew[c] = bf2f(kb);
        k_low[(((size_t)new_page * g.n_ret + ri.r) * kBlk + (jnew & 255)) * kIdx + c] = kb;
    }
    __syncthreads();
    float qv[kIdx];
#pragma unroll
    for (int c = 0; c < kIdx; ++c) qv[c] = qs[c];

    float dv[16];
    float mx = -INFINITY;
    auto score_group = [&](int k0, const uint4* buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = jbase + (k0 + u) * 256 + tid;
            float kf[kIdx];
            unpack8(buf[2 * u], kf);
            unpack8(buf[2 * u + 1], kf + 8);
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < kIdx; ++c) acc = __builtin_fmaf(qv[c], kf[c], acc);
            dv[k0 + u] = acc;
            (void)j;
        }
    };
    uint4 bufC[8], bufD[8];
    load_group(8, bufC);
    load_group(12, bufD);
    score_group(0, bufA);
    score_group(4, bufB);
    score_group(8, bufC);
    score_group(12, bufD);
    if (app && (jnew & 255) == tid && jnew >= jbase) {
        // the appended position, scored with the key formed above
        const int k = (jnew - jbase) >> 8;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < kIdx; ++c) acc = __builtin_fmaf(qv[c], knew[c], acc);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk)
            if (kk == k) dv[kk] = acc;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k)
        if (jbase + k * 256 + tid < ri.L) mx = fmaxf(mx, dv[k]);
    if (!STATS) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int j = jbase + k * 256 + tid;
            if (j < ri.L) srow[j] = dv[k];
        }
        return;
    }
    mx = wave_max(mx);
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    const float mc = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    if (tid == 0) ws.cmax[(size_t)ri.lrow * ws.nchunk + chunk] = score_key(mc);
    const float s = g.idx_scale;
    // a bit per key for the row pass's gather of U: the key lies in chunk bin
    // <= kLowBin (the wave's 64 consecutive keys of step k are one 64-bit word);
    // only those keys' scores are stored (the row pass forms any other score
    // it needs again from the indexer keys) -- except under a fixed top-k
    // budget, whose cut usually lies below the flagged bins: then every score
    // is stored
    unsigned long long* km = ws.kmask + ((size_t)ri.lrow * ws.score_ld + jbase) / 64;
    uint32_t lowm = 0u;                                   // bit k: this thread's key of step k is flagged
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int j = jbase + k * 256 + tid;
        bool low = false;
        if (j < ri.L) {
            const WeightBin wb = weight_bin(dv[k], mc, s);
            const int b = wb.bin >> 4;                    // 64 level-1 bins per unit -> 4 per unit
            atomicAdd(&hist[b], wb.w);
            atomicAdd(&hcnt[b], 1u);
            low = b <= kLowBin;
            if (low || g.sel_k > 0) srow[j] = dv[k];
        }
        lowm |= low ? 1u << k : 0u;
        const unsigned long long bal = __ballot(low);
        if ((tid & 63) == 0) {
            km[4 * k + (tid >> 6)] = bal;
            wcnt[4 * k + (tid >> 6)] = (uint32_t)__popcll(bal);
        }
    }
    __syncthreads();
    // the chunk's flagged keys in index order (word 4k + w holds keys
    // jbase + 256 k + 64 w + lane): each key's place is the flagged count of
    // the words before its own plus the flagged lanes below it in its word;
    // the first kFl of them are listed (a chunk with more takes the masks)
    {
        const int lane = tid & 63, wv = tid >> 6;
        const uint32_t wc = wcnt[lane];
        const uint32_t wex = wave_incl_scan_u32(wc) - wc;
        unsigned long long* fl = ws.flist + ((size_t)ri.lrow * ws.nchunk + chunk) * kFl;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const bool low = (lowm >> k) & 1u;
            const unsigned long long bal = __ballot(low);
            const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            const uint32_t at = lane_u32(wex, 4 * k + wv) + below;
            if (low && at < (uint32_t)kFl)
                fl[at] = ((unsigned long long)score_key(dv[k]) << 32) | (unsigned long long)(~(uint32_t)(jbase + k * 256 + tid));
        }
    }
    // cumulative over bins (the mass of keys with x_c < (b + 1) / 4)
    if (tid < 64) {
        const unsigned long long a = hist[2 * tid], b = hist[2 * tid + 1];
        const unsigned long long incl = wave_incl_scan_u64(a + b);
        unsigned long long* ch = ws.chist + ((size_t)ri.lrow * ws.nchunk + chunk) * kCB;
        ch[2 * tid] = incl - b;
        ch[2 * tid + 1] = incl;
    } else if (tid < 128) {
        const int t = tid - 64;
        const unsigned a = hcnt[2 * t], b = hcnt[2 * t + 1];
        const unsigned incl = wave_incl_scan_u32(a + b);
        unsigned* cc = ws.ccnt + ((size_t)ri.lrow * ws.nchunk + chunk) * kCB;
        cc[2 * t] = incl - b;
        cc[2 * t + 1] = incl;
    }
}

// ---------------------------------------------------------------------------
// Resolve.  One 1024-thread workgroup per row.
// ---------------------------------------------------------------------------
// Radix selection of the cut among keys with score key in [klo, khi] (the
// candidate list cand[0..n) if n >= 0, else every key of the row): exact
// fixed-point masses per 2048-bucket level, the mass ranked above khi is S_hi.
// Returns the cut key Tkey and jT: a key is selected iff its score key >
// Tkey, or == Tkey and its index <= jT.
struct Cut {
    uint32_t Tkey;
    int32_t jT;
};

// One radix level's bucket search (kRT threads, kBPT buckets each; nb buckets
// in use): the first bucket, highest keys first, whose cumulative mass (or
// count) from S_hi reaches target and that holds a key -- or, when rounding
// leaves the target unreached, the last bucket.  Leaves the mass ranked above
// that bucket in *s_S and its key count in *s_u; returns its index.
constexpr int kBPT = kNR / kRT;

__device__ int bucket_search(const unsigned long long* hmb, const uint32_t* hcb, unsigned long long S_hi,
                             unsigned long long target, int nb, unsigned long long* scan_sh, int* s_i,
                             unsigned long long* s_S, uint32_t* s_u) {
    const int tid = threadIdx.x;
    unsigned long long loc = 0ull;
#pragma unroll
    for (int b = 0; b < kBPT; ++b) loc += hmb[kBPT * tid + b];
    unsigned long long tot;
    const unsigned long long ex = S_hi + block_excl_scan_u64<kRT>(loc, &tot, scan_sh);
    if (tid == 0) *s_i = kNR;
    __syncthreads();
    unsigned long long run = ex;
#pragma unroll
    for (int b = 0; b < kBPT; ++b) {
        const int i = kBPT * tid + b;
        if (run + hmb[i] >= target && hcb[i]) {
            atomicMin(s_i, i);
            break;
        }
        run += hmb[i];
    }
    __syncthreads();
    int bk = *s_i;
    // the mass ranked above the bucket, from the thread that holds it
    if (bk < kNR && bk / kBPT == tid) {
        unsigned long long above = ex;
        for (int b = 0; b < bk % kBPT; ++b) above += hmb[kBPT * tid + b];
        *s_S = above;
        *s_u = hcb[bk];
    }
    if (bk >= kNR && tid == 0) {
        // the target is not reached (rounding): the last bucket
        *s_S = S_hi + tot - hmb[nb - 1];
        *s_u = hcb[nb - 1];
    }
    if (bk >= kNR) bk = nb - 1;
    __syncthreads();
    return bk;
}

__device__ Cut radix_cut(const unsigned long long* cand, int n, const float* srow, int L, uint32_t klo,
                         uint32_t khi, unsigned long long S_hi, unsigned long long target, float m, float s,
                         bool unit, unsigned long long* hmb, uint32_t* hcb, unsigned long long* scan_sh,
                         uint32_t* s_u, unsigned long long* s_S, int* s_i) {
    const int tid = threadIdx.x;
    const bool from_list = n >= 0;
    const int cnt = from_list ? n : L;
    auto key_at = [&](int i, int* j) -> uint32_t {
        if (from_list) {
            *j = (int)~(uint32_t)cand[i];
            return (uint32_t)(cand[i] >> 32);
        }
        *j = i;
        return score_key(srow[i]);
    };
    for (int level = 0; level < 4; ++level) {
        const uint32_t span = khi - klo;
        const int bits = span ? 32 - __clz(span) : 0;
        const int shift = bits > 11 ? bits - 11 : 0;
        for (int i = tid; i < kNR; i += kRT) {
            hmb[i] = 0ull;
            hcb[i] = 0u;
        }
        __syncthreads();
        for (int i = tid; i < cnt; i += kRT) {
            int j;
            const uint32_t key = key_at(i, &j);
            if (key < klo || key > khi) continue;
            const uint32_t bk = (khi - key) >> shift;         // bucket 0 holds the highest keys
            atomicAdd(&hmb[bk], unit ? 1ull : weight_bin(key_score(key), m, s).w);
            atomicAdd(&hcb[bk], 1u);
        }
        __syncthreads();
        // first bucket (highest keys first) whose cumulative mass (or count) reaches target
        const int nb = (int)(span >> shift) + 1;
        const int bk = bucket_search(hmb, hcb, S_hi, target, nb, scan_sh, s_i, s_S, s_u);
        const unsigned long long S_b = *s_S;
        const uint32_t n_b = *s_u;
        const uint32_t nkhi = khi - ((uint32_t)bk << shift);
        const uint32_t wdt = shift >= 32 ? 0xFFFFFFFFu : ((1u << shift) - 1u);
        const uint32_t nklo = (nkhi - klo > wdt) ? nkhi - wdt : klo;
        __syncthreads();
        klo = nklo;
        khi = nkhi;
        S_hi = S_b;
        if (klo == khi) {
            // one score value: its tie group takes the lowest indices first
            const unsigned long long wT = unit ? 1ull : weight_bin(key_score(klo), m, s).w;
            const unsigned long long need = target - S_hi;
            const uint32_t ntie = (uint32_t)min((need + wT - 1ull) / wT, (unsigned long long)n_b);
            Cut c;
            c.Tkey = klo;
            if (ntie >= n_b) {
                // every tie is taken: jT = the largest tie index
                if (tid == 0) *s_i = -1;
                __syncthreads();
                for (int i = tid; i < cnt; i += kRT) {
                    int j;
                    if (key_at(i, &j) == klo) atomicMax(s_i, j);
                }
                __syncthreads();
                c.jT = *s_i;
            } else {
                // the ntie-th smallest tie index, by an ordered scan of the row
                if (tid == 0) {
                    *s_u = 0u;
                    *s_i = -1;
                }
                __syncthreads();
                for (int j0 = 0; j0 < L; j0 += kRT) {
                    const int j = j0 + tid;
                    const bool is_tie = j < L && score_key(srow[j]) == klo;
                    const uint32_t before_blk = *s_u;
                    unsigned long long t2;
                    const unsigned long long rank = block_excl_scan_u64<kRT>(is_tie ? 1ull : 0ull, &t2, scan_sh);
                    if (is_tie && before_blk + rank + 1ull == ntie) *s_i = j;
                    __syncthreads();
                    if (tid == 0) *s_u = before_blk + (uint32_t)t2;
                    __syncthreads();
                    if (*s_i >= 0) break;
                }
                c.jT = *s_i;
            }
            __syncthreads();
            return c;
        }
    }
    // unreachable for 32-bit keys (each level fixes at least 11 bits)
    Cut c;
    c.Tkey = khi;
    c.jT = L;
    return c;
}

// Plan of one row, formed by the row's workgroup: row maximum m, total mass Z = sum_c exp(s (m_c - m)) Z_c, the
// target, and the threshold d_thr of the candidate set U.  Every chunk bin
// whose upper edge, moved to the row's axis, lies below X = k / 4 certainly
// holds keys with s (m - d) < X: that gives a lower bound LB(k) of the mass
// above any k; the smallest k whose bound reaches the target (plus one unit
// of rounding per key) fixes U = {d >= m - X / s}.
struct Plan {
    float m, d_thr;
    unsigned long long target;                        // mass, or a key count when unit
    int all;                                          // every key (p >= 1, or a count >= L)
    int ks;                                           // X = ks / 4, or kGB if no grid point suffices
    int unit;                                         // count cut: fixed top-k, or a capped keep-all row
    int bad;                                          // top_p is NaN or <= 0
};

// NT threads (dred, ured: NT / 64 entries); chist, ccnt, cmax: the row's
// chunk statistics (device memory or an LDS copy).
template <int NT>
__device__ __forceinline__ Plan row_plan(const Geo& g, const RowInfo& ri, const unsigned long long* __restrict__ chist,
                         const unsigned* __restrict__ ccnt, const uint32_t* __restrict__ cmax, float p,
                         double* fch, double* dch, double* dred, uint32_t* ured, int* s_k) {
    const int tid = threadIdx.x;
    const int nch = ri.nch;
    const float s = g.idx_scale;
    // the chunk's maximum and total mass (one chunk per thread, nch <= 256);
    // p is the row's top_p (1 for a fixed top-k)
    const uint32_t cm = tid < nch ? cmax[tid] : 0u;
    const unsigned long long ztot = tid < nch ? chist[(size_t)tid * kCB + kCB - 1] : 0ull;
    // a count target: the fixed top-k budget, or the cap of a keep-all row
    const int kc = g.sel_k > 0 ? g.sel_k : (!(p < 1.0f) && g.k_max > 0 ? g.k_max : 0);
    uint32_t mk = wave_max_u32(cm);
    if ((tid & 63) == 0) ured[tid >> 6] = mk;
    if (tid == 0) {
        s_k[0] = kGB;
        s_k[1] = 16;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) mk = max(mk, ured[w]);
    Plan pl;
    pl.m = key_score(mk);
    double z = 0.0;
    if (tid < nch) {
        const double dc = (double)s * ((double)pl.m - (double)key_score(cm));
        const double f = exp(-dc);
        dch[tid] = dc;
        fch[tid] = f;
        z = f * (double)ztot;
    }
    z = wave_sum_f64(z);
    if ((tid & 63) == 0) dred[tid >> 6] = z;
    __syncthreads();
    double Z = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) Z += dred[w];
    pl.bad = g.sel_k <= 0 && !(p > 0.0f);
    pl.unit = kc > 0;
    pl.all = pl.bad || (kc > 0 ? kc >= ri.L : !(p < 1.0f));
    unsigned long long target = (unsigned long long)ceil((double)p * Z);
    if ((double)target > Z) target = (unsigned long long)Z;
    if (target < 1ull) target = 1ull;
    pl.target = kc > 0 ? (unsigned long long)kc : target;
    pl.d_thr = -INFINITY;
    pl.ks = kGB;
    if (pl.all) return pl;
    // LB(k) is non-decreasing in k: first at the 16 points k = 16 i + 15, then
    // at the 16 values up to the first point that reaches.  16 lanes share one
    // k (chunk bin b counts once (b + 1) / 4 + dc <= k / 4).  A count cut
    // bounds the number of keys the same way, from the cumulative counts.
    const double need = pl.unit ? (double)pl.target : (double)target * (1.0 + 0x1.0p-40) + (double)ri.L + 1.0;
    const int grp = tid >> 4, sub = tid & 15;
    const auto lb_reaches = [&](int k) {
        double lb = 0.0;
        for (int c = sub; c < nch; c += 16) {
            const double bmax = floor((double)(k - 1) - (double)kCBPerUnit * dch[c]);
            if (bmax >= 0.0) {
                const int b = (int)fmin(bmax, (double)(kCB - 1));
                lb += pl.unit ? (double)ccnt[(size_t)c * kCB + b] : fch[c] * (double)chist[(size_t)c * kCB + b];
            }
        }
        lb = row_sum_f64(lb);                             // the 16 lanes of k are one DPP row
        return sub == 0 && lb >= need;
    };
    if (tid < 256 && lb_reaches(16 * grp + 15)) atomicMin(&s_k[1], grp);
    __syncthreads();
    const int ic = s_k[1];
    if (tid < 256 && ic < 16 && lb_reaches(16 * ic + grp)) atomicMin(&s_k[0], 16 * ic + grp);
    __syncthreads();
    const int ks = s_k[0];
    pl.ks = ks;
    if (ks < kGB) {
        // the margin covers the float rounding of the chunk bins
        const double X = (double)ks / (double)kCBPerUnit;
        const double xm = X + 0x1.0p-18 * (X + 1.0);
        pl.d_thr = __double2float_rd((double)pl.m - xm / (double)s - 0x1.0p-20 * fabs((double)pl.m));
    }
    return pl;
}

// U: in chunk c, the keys whose chunk bin is at most bsel(c) = ks + 1 - 4 dc
// (a quarter unit beyond the bins that LB(ks) counts, so U holds every key
// with s (m - d) < ks / 4 and the cut lies inside it); dc = s (m - m_c).
__device__ __forceinline__ int chunk_bsel(int ks, double dc) {
    return ks >= kGB ? kCB - 1 : (int)fmin(floor((double)(ks + 1) - (double)kCBPerUnit * dc), (double)(kCB - 1));
}

// Cut among a candidate list held in LDS (cand = (score key << 32) | ~index,
// wgt = exact fixed-point weights): radix levels of 2048 buckets with exact
// masses; once the cut bucket holds at most 64 keys, one wavefront sorts them
// in registers (score key descending, index ascending) and finds the first
// whose cumulative mass reaches the target.
template <typename Wt>
__device__ Cut list_cut(const unsigned long long* cand, Wt wgt, int n, const float* srow,
                        int L, uint32_t klo, uint32_t khi, unsigned long long target, float m, float s, bool unit,
                        unsigned long long* hmb, uint32_t* hcb, unsigned long long* scan_sh, uint32_t* s_u,
                        unsigned long long* s_S, int* s_i, unsigned long long* small_v, unsigned long long* small_w,
                        Cut* s_cut) {
    const int tid = threadIdx.x, lane = tid & 63;
    unsigned long long S_hi = 0ull;
    for (int level = 0; level < 4; ++level) {
        const uint32_t span = khi - klo;
        const int bits = span ? 32 - __clz(span) : 0;
        const int shift = bits > 11 ? bits - 11 : 0;
        for (int i = tid; i < kNR; i += kRT) {
            hmb[i] = 0ull;
            hcb[i] = 0u;
        }
        __syncthreads();
        for (int i = tid; i < n; i += kRT) {
            const uint32_t key = (uint32_t)(cand[i] >> 32);
            if (key < klo || key > khi) continue;
            const uint32_t bk = (khi - key) >> shift;         // bucket 0 holds the highest keys
            atomicAdd(&hmb[bk], wgt(i));
            atomicAdd(&hcb[bk], 1u);
        }
        __syncthreads();
        const int nb = (int)(span >> shift) + 1;
        const int bk = bucket_search(hmb, hcb, S_hi, target, nb, scan_sh, s_i, s_S, s_u);
        S_hi = *s_S;
        const uint32_t n_b = *s_u;
        const uint32_t nkhi = khi - ((uint32_t)bk << shift);
        const uint32_t wdt = shift >= 32 ? 0xFFFFFFFFu : ((1u << shift) - 1u);
        const uint32_t nklo = (nkhi - klo > wdt) ? nkhi - wdt : klo;
        klo = nklo;
        khi = nkhi;
        __syncthreads();
        if (n_b <= 64u) {
            // the bucket's keys into a wavefront, sorted in registers
            if (tid == 0) *s_u = 0u;
            __syncthreads();
            for (int i = tid; i < n; i += kRT) {
                const uint32_t key = (uint32_t)(cand[i] >> 32);
                if (key < klo || key > khi) continue;
                const uint32_t slot = atomicAdd(s_u, 1u);
                if (slot < 64u) {
                    small_v[slot] = cand[i];
                    small_w[slot] = wgt(i);
                }
            }
            __syncthreads();
            if (tid < 64) {
                const int nbk = (int)min(*s_u, 64u);
                const unsigned long long v0 = lane < nbk ? small_v[lane] : 0ull;
                const unsigned long long w0 = lane < nbk ? small_w[lane] : 0ull;
                // each key's place in descending order: the keys above it (the
                // entries are distinct), counted from broadcast LDS reads
                int rank = 0;
                for (int j0 = 0; j0 < nbk; j0 += 16) {
                    unsigned long long c[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) c[u] = small_v[min(j0 + u, 63)];
#pragma unroll
                    for (int u = 0; u < 16; ++u) rank += (j0 + u < nbk && c[u] > v0) ? 1 : 0;
                }
                // (one wavefront: every lane's reads above precede the writes)
                if (lane < nbk) {
                    small_v[rank] = v0;
                    small_w[rank] = w0;
                }
                __builtin_amdgcn_wave_barrier();
                const unsigned long long v = lane < nbk ? small_v[lane] : 0ull;
                const unsigned long long w = lane < nbk ? small_w[lane] : 0ull;
                const unsigned long long incl = wave_incl_scan_u64(w);
                const unsigned long long reach = __ballot(lane < nbk && S_hi + incl >= target);
                const int ic = reach ? __ffsll((long long)reach) - 1 : nbk - 1;
                const unsigned long long vc = lane_u64(v, ic);
                if (lane == 0) {
                    s_cut->Tkey = (uint32_t)(vc >> 32);
                    s_cut->jT = (int32_t)~(uint32_t)vc;
                }
            }
            __syncthreads();
            return *s_cut;
        }
        if (klo == khi) {
            // one score value with more than 64 keys: its lowest indices first
            const unsigned long long wT = unit ? 1ull : weight_bin(key_score(klo), m, s).w;
            const unsigned long long need = target - S_hi;
            const uint32_t ntie = (uint32_t)min((need + wT - 1ull) / wT, (unsigned long long)n_b);
            Cut c;
            c.Tkey = klo;
            // the list is in index order: the ntie-th tie of the list
            if (tid == 0) {
                *s_u = 0u;
                *s_i = -1;
            }
            __syncthreads();
            for (int i0 = 0; i0 < n; i0 += kRT) {
                const int i = i0 + tid;
                const bool is_tie = i < n && (uint32_t)(cand[i] >> 32) == klo;
                const uint32_t before_blk = *s_u;
                unsigned long long t2;
                const unsigned long long rank = block_excl_scan_u64<kRT>(is_tie ? 1ull : 0ull, &t2, scan_sh);
                if (is_tie && before_blk + rank + 1ull == ntie) *s_i = (int)~(uint32_t)cand[i];
                __syncthreads();
                if (tid == 0) *s_u = before_blk + (uint32_t)t2;
                __syncthreads();
                if (*s_i >= 0) break;
            }
            c.jT = *s_i;
            __syncthreads();
            return c;
        }
    }
    Cut c;
    c.Tkey = khi;
    c.jT = L;
    return c;
}

// The row's cut (kRT threads).  U with its exact weights, the cut, and the
// selected indices in order.
constexpr int kBtCache = 1536;                        // page ids cached in LDS: rows of up to 393216 keys
// LDS of a row's cut.
struct ResolveSm {
    __align__(16) unsigned long long big[2 * kCand];   // U (index order) and its weights
    unsigned long long scan_sh[kRT / 64 + 1];
    union {
        struct {
            unsigned long long hmb[kNR];
            uint32_t hcb[kNR];
        } cut;
        struct {                                      // the plan, before any cut
            double fch[kMaxChunks], dch[kMaxChunks];
            int16_t bsel[kMaxChunks];                 // each chunk's last bin in U (-1: none)
            float mc[kMaxChunks];                     // each chunk's maximum score (the gather of U)
            int32_t fofs[kMaxChunks];                 // each chunk's first place in S0 (the flagged-key lists)
        } plan;
    };
    unsigned long long small_v[64], small_w[64];
    int32_t btc[kBtCache];                            // the row's page ids (rows of at most kBtCache pages)
    double dred[kRT / 64];
    uint32_t ured[kRT / 64];
    int s_k[2];
    Cut s_cut;
    int s_i;
    uint32_t s_n;
    unsigned long long s_S;
};

// The cut of one row with nU keys in U, from its plan st.  U is in LDS with
// its weights (nU <= kCand, `loaded`), in the workspace list (nU <= ucap: read
// into LDS, or read from there with weights formed as needed), or not
// gathered (nU > ucap: the cut over the row's scores).  Writes the row's state
// and its selected keys: the workspace list of the row (mode 1), or the
// row's score array overwritten in place by the indices (mode 2).
__device__ __forceinline__ void resolve_body(const Geo& g, const RowInfo& ri, const SelWs& ws, RowState st, int nU, bool loaded,
                             bool bt_cached, ResolveSm& sm) {
    const int tid = threadIdx.x;
    unsigned long long* cand = sm.big;
    unsigned long long* wgt = sm.big + kCand;
    unsigned long long* scan_sh = sm.scan_sh;
    unsigned long long* hmb = sm.cut.hmb;
    uint32_t* hcb = sm.cut.hcb;
    unsigned long long* small_v = sm.small_v;
    unsigned long long* small_w = sm.small_w;
    Cut& s_cut = sm.s_cut;
    int& s_i = sm.s_i;
    uint32_t& s_n = sm.s_n;
    unsigned long long& s_S = sm.s_S;
    const float s = g.idx_scale;
    float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const float m = st.m, d_thr = st.d_thr;
    unsigned long long target = st.target;
    bool unit = st.unit != 0;
    const uint32_t klo = d_thr == -INFINITY ? 0u : score_key(d_thr), khi = score_key(m);
    const auto selected_by = [](const Cut& c, uint32_t key, int j) { return key > c.Tkey || (key == c.Tkey && j <= c.jT); };
    if (nU <= ws.ucap) {
        const unsigned long long* ub = ws.ubuf + (size_t)ri.lrow * ws.ucap;
        const bool in_lds = nU <= kCand;
        if (in_lds && !loaded) {
            for (int i = tid; i < nU; i += kRT) {
                const unsigned long long e = ub[i];
                cand[i] = e;
                wgt[i] = unit ? 1ull : weight_bin(key_score((uint32_t)(e >> 32)), m, s).w;
            }
            __syncthreads();
        }
        // the candidate list: in LDS with its exact weights, or (more than
        // kCand keys) read from the workspace list, weights formed as needed
        const unsigned long long* cl = in_lds ? cand : ub;
        const auto w_lds = [&](int i) { return wgt[i]; };
        const auto w_list = [&](int i) {
            return unit ? 1ull : weight_bin(key_score((uint32_t)(cl[i] >> 32)), m, s).w;
        };
        const int per = (nU + kRT - 1) / kRT;              // contiguous entries per thread, index order
        Cut cut;
        unsigned long long tot2;
        uint32_t o;
        for (int pass = 0;; ++pass) {
            cut = in_lds ? list_cut(cl, w_lds, nU, srow, ri.L, klo, khi, target, m, s, unit, hmb, hcb, scan_sh, &s_n,
                                    &s_S, &s_i, small_v, small_w, &s_cut)
                         : list_cut(cl, w_list, nU, srow, ri.L, klo, khi, target, m, s, unit, hmb, hcb, scan_sh,
                                    &s_n, &s_S, &s_i, small_v, small_w, &s_cut);
            uint32_t c = 0;
            for (int x = 0; x < per; ++x) {
                const int i = tid * per + x;
                if (i < nU && selected_by(cut, (uint32_t)(cl[i] >> 32), (int)~(uint32_t)cl[i])) ++c;
            }
            o = (uint32_t)block_excl_scan_u64<kRT>(c, &tot2, scan_sh);
            // the budget cap: a top-p set of more than k_max keys is cut
            // again by count (U holds it, so it holds the first k_max keys)
            if (pass > 0 || unit || g.k_max <= 0 || tot2 <= (unsigned long long)g.k_max) break;
            unit = true;
            target = (unsigned long long)g.k_max;
            if (in_lds) {
                for (int i = tid; i < nU; i += kRT) wgt[i] = 1ull;
                __syncthreads();
            }
        }
        // U is in index order: its selected entries, in order, into the row's
        // list; a list cut in LDS also gets the K/V row numbers of its keys
        // (page ids from the LDS cache) in the row's unused workspace list
        uint32_t* sl = ws.sel + (size_t)ri.lrow * ws.ucap;
        uint32_t* jo = reinterpret_cast<uint32_t*>(ws.ubuf + (size_t)ri.lrow * ws.ucap);
        const bool with_jo = in_lds && bt_cached;
        const int kvh = g.ret_heads[ri.r] / g.group;
        for (int x = 0; x < per; ++x) {
            const int i = tid * per + x;
            if (i < nU) {
                const int j = (int)~(uint32_t)cl[i];
                if (selected_by(cut, (uint32_t)(cl[i] >> 32), j)) {
                    if (with_jo) jo[o] = (uint32_t)kv_rowidx(g, sm.btc[j >> 8], kvh, j & 255);
                    sl[o++] = (uint32_t)j;
                }
            }
        }
        if (tid == 0) {
            st.mode = 1;
            st.Tkey = cut.Tkey;
            st.jT = cut.jT;
            st.count = (int32_t)tot2;
            st.unit = unit;
            st.path = (in_lds ? kPathList : kPathListG) | (unit ? kPathCount : 0) | st.path;
            st.has_jo = with_jo;
            ws.st[ri.lrow] = st;
        }
        return;
    }
    // ---- U larger than the workspace list: the cut over the row's scores
    Cut cut;
    unsigned long long tot;
    for (int pass = 0;; ++pass) {
        cut = radix_cut(cand, -1, srow, ri.L, klo, khi, 0ull, target, m, s, unit, hmb, hcb, scan_sh, &s_n, &s_S,
                        &s_i);
        unsigned long long c = 0ull;
        for (int j = tid; j < ri.L; j += kRT) c += selected_by(cut, score_key(srow[j]), j) ? 1ull : 0ull;
        block_excl_scan_u64<kRT>(c, &tot, scan_sh);
        if (pass > 0 || unit || g.k_max <= 0 || tot <= (unsigned long long)g.k_max) break;
        unit = true;                                      // the budget cap, as above
        target = (unsigned long long)g.k_max;
    }
    // the selected indices, ascending, over the row's scores (int32): blocks
    // of 16 consecutive keys per thread; a block is read into registers before
    // the block scan, and its writes land below its end, so no later read
    // sees them
    int32_t* orow = reinterpret_cast<int32_t*>(srow);
    uint32_t base = 0u;
    for (int j0 = 0; j0 < ri.L; j0 += 16 * kRT) {
        const int jj = j0 + 16 * tid;
        float dv[16];
        if (jj < ri.L) {                                  // jj + 16 <= Lpad: the row is padded to whole chunks
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 v = *reinterpret_cast<const float4*>(srow + jj + 4 * u);
                dv[4 * u] = v.x;
                dv[4 * u + 1] = v.y;
                dv[4 * u + 2] = v.z;
                dv[4 * u + 3] = v.w;
            }
        }
        uint32_t msk = 0u, c = 0u;
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (jj + e < ri.L && selected_by(cut, score_key(dv[e]), jj + e)) {
                msk |= 1u << e;
                ++c;
            }
        unsigned long long t2;
        uint32_t o = base + (uint32_t)block_excl_scan_u64<kRT>(c, &t2, scan_sh);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (msk & (1u << e)) orow[o++] = jj + e;
        base += (uint32_t)t2;
    }
    if (tid == 0) {
        st.mode = 2;
        st.Tkey = cut.Tkey;
        st.jT = cut.jT;
        st.count = (int32_t)tot;
        st.unit = unit;
        st.path = kPathScan | (unit ? kPathCount : 0);
        ws.st[ri.lrow] = st;
    }
}

// The fixed-order chain scores of every key of chunks ca and cb (cb < 0: ca
// only) of a row, formed again from the indexer keys (q_low from the scoring
// pass) into the row's score array: the scoring pass stores only the keys it
// flags.  kRT threads, 8 keys per thread and chunk; both chunks' loads are in
// flight before the first is used.
__device__ __forceinline__ void rescore_chunks(const Geo& g, const RowInfo& ri, const SelWs& ws,
                                               const bf16_t* __restrict__ k_low, const int32_t* btc, bool bt_cached,
                                               int ca, int cb) {
    const int tid = threadIdx.x;
    float qv[kIdx];
#pragma unroll
    for (int x = 0; x < kIdx; ++x) qv[x] = bf2f(ws.qlow[(size_t)ri.lrow * kIdx + x]);
    float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int32_t* bt = g.block_table + (size_t)ri.b * g.max_blocks;
    constexpr int K = kChunk / kRT;
    uint4 kb[2][K][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = h == 0 || cb < 0 ? ca : cb;
#pragma unroll
        for (int x = 0; x < K; ++x) {
            const int j = min(c * kChunk + tid + kRT * x, ri.L - 1);
            const int page = bt_cached ? btc[j >> 8] : bt[j >> 8];
            const uint4* kp =
                reinterpret_cast<const uint4*>(k_low + (((size_t)page * g.n_ret + ri.r) * kBlk + (j & 255)) * kIdx);
            kb[h][x][0] = kp[0];
            kb[h][x][1] = kp[1];
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        if (h == 1 && cb < 0) break;
        const int c = h == 0 ? ca : cb;
#pragma unroll
        for (int x = 0; x < K; ++x) {
            const int j = c * kChunk + tid + kRT * x;
            float kf[kIdx];
            unpack8(kb[h][x][0], kf);
            unpack8(kb[h][x][1], kf + 8);
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < kIdx; ++i) acc = __builtin_fmaf(qv[i], kf[i], acc);
            if (j < ri.L) srow[j] = acc;
        }
    }
}

// Row pass.  One kRT-thread workgroup per row: the plan, from the scoring
// pass's chunk statistics (staged in LDS with the row's key masks when the
// row has at most kStageChunks chunks, so that the plan makes no dependent
// global round); U; the cut; the row's selected keys.  U is found without
// reading the row's scores when every chunk's part of U lies in its chunk bins
// <= kLowBin: the keys the masks flag in those chunks (S0, a superset of U)
// are compacted in index order, their scores read (all loads in flight), their
// chunk bins formed again and U kept in place.  Otherwise U comes from a pass
// over the row's scores.
constexpr int kStageChunks = 48;   // chist (48 KiB) + ccnt (24 KiB) + key masks (24 KiB) + cmax of 48 chunks

__device__ __forceinline__ void row_pass(const Geo& g, const float* __restrict__ top_p, const bf16_t* __restrict__ k_low,
                         const RowInfo& ri, const SelWs& ws, int32_t* __restrict__ status, ResolveSm& sm) {
    const int tid = threadIdx.x;
    const size_t crow = (size_t)ri.lrow * ws.nchunk;
    const unsigned long long* chist = ws.chist + crow * kCB;
    const unsigned* ccnt = ws.ccnt + crow * kCB;
    const uint32_t* cmax = ws.cmax + crow;
    const unsigned long long* kmask = ws.kmask + (size_t)ri.lrow * ws.score_ld / 64;
    const int nwd = (ri.L + 63) / 64;                     // mask words of the row
    const float p = g.sel_k > 0 ? 1.0f : top_p[ri.b];
    const int npg = (ri.L + kBlk - 1) / kBlk;
    const bool bt_cached = npg <= kBtCache;
    if (bt_cached) {
        const int32_t* bt = g.block_table + (size_t)ri.b * g.max_blocks;
        for (int i = tid; i < npg; i += kRT) sm.btc[i] = bt[i];
    }
    if (ri.nch <= kStageChunks) {
        // one round of loads: every chunk's histograms, maximum and key masks into LDS
        unsigned long long* hs = sm.big;
        unsigned* cs = reinterpret_cast<unsigned*>(sm.big + kStageChunks * kCB);
        unsigned long long* ks = sm.big + kStageChunks * kCB * 3 / 2;
        uint32_t* ms = reinterpret_cast<uint32_t*>(ks + kStageChunks * (kChunk / 64));
        constexpr int kPer = kStageChunks * kCB / kRT;
        constexpr int kPerM = kStageChunks * (kChunk / 64) / kRT;
        const int n = ri.nch * kCB;
        unsigned long long hv[kPer], kv[kPerM];
        unsigned cv[kPer];
        const uint32_t mv = tid < ri.nch ? cmax[tid] : 0u;
#pragma unroll
        for (int x = 0; x < kPer; ++x) {                  // every load in flight before the first store
            const int i = tid + kRT * x;
            hv[x] = i < n ? chist[i] : 0ull;
            cv[x] = i < n ? ccnt[i] : 0u;
        }
#pragma unroll
        for (int x = 0; x < kPerM; ++x) {
            const int i = tid + kRT * x;
            kv[x] = i < nwd ? kmask[i] : 0ull;
        }
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
            const int i = tid + kRT * x;
            if (i < n) {
                hs[i] = hv[x];
                cs[i] = cv[x];
            }
        }
#pragma unroll
        for (int x = 0; x < kPerM; ++x) {
            const int i = tid + kRT * x;
            if (i < nwd) ks[i] = kv[x];
        }
        if (tid < ri.nch) ms[tid] = mv;
        __syncthreads();
        chist = hs;
        ccnt = cs;
        cmax = ms;
        kmask = ks;
    }
    const Plan pl = row_plan<kRT>(g, ri, chist, ccnt, cmax, p, sm.plan.fch, sm.plan.dch, sm.dred, sm.ured, sm.s_k);
    RowState st;
    st.m = pl.m;
    st.L = ri.L;
    st.Tkey = 0u;
    st.jT = ri.L;
    st.target = pl.target;
    st.d_thr = pl.d_thr;
    st.ks = pl.ks;
    st.has_jo = 0;
    if (pl.all) {
        if (tid == 0) {
            st.mode = 0;
            st.count = ri.L;
            st.unit = 0;
            st.path = kPathAll;
            ws.st[ri.lrow] = st;
            if (pl.bad) *status = 3;                      // invalid top_p: reported, nothing emitted
        }
        return;
    }
    st.mode = 1;
    st.count = 0;
    st.unit = pl.unit;
    st.path = 0;
    const bool unit = pl.unit != 0;
    const float s = g.idx_scale;
    const float m = pl.m;
    // each chunk's part of U: its keys in chunk bins <= bsel; the masks hold
    // it when bsel <= kLowBin
    unsigned long long cnt_c = 0ull;
    int cov = 1, flok = 1;
    uint32_t nfl = 0u;                                    // the chunk's flagged keys, when it has a part of U
    if (tid < ri.nch) {
        const int b = chunk_bsel(pl.ks, sm.plan.dch[tid]);
        cnt_c = b >= 0 ? (unsigned long long)ccnt[(size_t)tid * kCB + b] : 0ull;
        cov = b <= kLowBin;
        if (b >= 0) {
            nfl = ccnt[(size_t)tid * kCB + kLowBin];      // keys of chunk bins <= kLowBin: the flagged ones
            flok = nfl <= (uint32_t)kFl;
        }
        sm.plan.bsel[tid] = (int16_t)b;
        sm.plan.mc[tid] = key_score(cmax[tid]);           // out of the staging area, which U overwrites
    }
    // one scan for both counts (each sum < 2^32): U's keys (low half) and the flagged keys (high half)
    unsigned long long both;
    const unsigned long long pre = block_excl_scan_u64<kRT>(cnt_c | ((unsigned long long)nfl << 32), &both, sm.scan_sh);
    if (tid < ri.nch) sm.plan.fofs[tid] = (int32_t)(pre >> 32);
    unsigned long long nU = both & 0xFFFFFFFFull;
    const bool covered = __syncthreads_and(cov) != 0;
    // every chunk with a part of U lists all its flagged keys: S0 is their lists, concatenated
    const bool fl_route = covered && __syncthreads_and(flok) != 0;
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    unsigned long long* gdst = ws.ubuf + (size_t)ri.lrow * ws.ucap;
    // S0: the flagged keys of the chunks with a part of U (covered rows)
    uint32_t nS0 = 0u;
    if (fl_route) {
        nS0 = (uint32_t)(both >> 32);
    } else if (covered) {
        uint32_t c = 0u;
        for (int wi = tid; wi < nwd; wi += kRT)
            if (sm.plan.bsel[wi / (kChunk / 64)] >= 0) c += (uint32_t)__popcll(kmask[wi]);
        nS0 = block_sum_u32<kRT>(c, sm.ured);
    }
    bool loaded = false;                                  // U and its weights in LDS
    const bool covered_path = covered && nS0 <= (uint32_t)ws.ucap;
    if (covered_path) {
      const bool to_lds = nS0 <= (uint32_t)kCand;
      if (fl_route) {
        // pass 1: S0 from the chunks' lists (entries carry their score keys);
        // entry i belongs to the last chunk whose first place is <= i (chunks
        // without a part of U list nothing here)
        const unsigned long long* flr = ws.flist + (size_t)ri.lrow * ws.nchunk * kFl;
        constexpr int F = 16;
        for (uint32_t i0 = 0; i0 < nS0; i0 += F * kRT) {
            unsigned long long e[F];
#pragma unroll
            for (int x = 0; x < F; ++x) {
                const uint32_t i = i0 + x * kRT + tid;
                e[x] = 0ull;
                if (i < nS0) {
                    int lo = 0;                           // fofs is non-decreasing, fofs[0] = 0
#pragma unroll
                    for (int step = kMaxChunks / 2; step > 0; step >>= 1)
                        if (lo + step < ri.nch && (uint32_t)sm.plan.fofs[lo + step] <= i) lo += step;
                    e[x] = flr[(size_t)lo * kFl + (i - (uint32_t)sm.plan.fofs[lo])];
                }
            }
#pragma unroll
            for (int x = 0; x < F; ++x) {
                const uint32_t i = i0 + x * kRT + tid;
                if (i < nS0) {
                    if (to_lds) sm.big[i] = e[x]; else gdst[i] = e[x];
                }
            }
        }
      } else {
        // pass 1: S0's indices in index order (4 mask words = 256 keys per thread and step)
        uint32_t base = 0u;
        for (int w0 = 0; w0 < nwd; w0 += 4 * kRT) {
            unsigned long long mw[4];
            uint32_t c = 0u;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int wi = w0 + 4 * tid + x;
                mw[x] = wi < nwd && sm.plan.bsel[wi / (kChunk / 64)] >= 0 ? kmask[wi] : 0ull;
                c += (uint32_t)__popcll(mw[x]);
            }
            unsigned long long t2;
            uint32_t o = base + (uint32_t)block_excl_scan_u64<kRT>(c, &t2, sm.scan_sh);
            // each lane expands its own words bit by bit, or (when fewer
            // steps: clustered flags, one thread's words holding hundreds of
            // them) the wavefront expands its non-zero words one at a time, a
            // lane per bit
            const int lane = tid & 63;
            const unsigned long long below = (1ull << lane) - 1ull;
            int nzw = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) nzw += __popcll(__ballot(mw[x] != 0ull));
            if ((uint32_t)nzw >= wave_max_u32(c)) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    unsigned long long mm = mw[x];
                    while (mm) {
                        const int e = __ffsll((long long)mm) - 1;
                        mm &= mm - 1ull;
                        const unsigned long long ent = (unsigned long long)(~(uint32_t)(64 * (w0 + 4 * tid + x) + e));
                        if (to_lds) sm.big[o] = ent; else gdst[o] = ent;
                        ++o;
                    }
                }
            } else {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    unsigned long long nz = __ballot(mw[x] != 0ull);
                    while (nz) {
                        const int l = __ffsll((long long)nz) - 1;
                        nz &= nz - 1ull;
                        const unsigned long long wv =
                            ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(mw[x] >> 32), l) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mw[x], l);
                        const uint32_t ow = (uint32_t)__builtin_amdgcn_readlane((int)o, l);
                        if ((wv >> lane) & 1ull) {
                            const uint32_t at = ow + (uint32_t)__popcll(wv & below);
                            const int wi = w0 + 4 * (tid - lane + l) + x;
                            const unsigned long long ent = (unsigned long long)(~(uint32_t)(64 * wi + lane));
                            if (to_lds) sm.big[at] = ent; else gdst[at] = ent;
                        }
                    }
                    o += (uint32_t)__popcll(mw[x]);
                }
            }
            base += (uint32_t)t2;
        }
      }
        __syncthreads();
        // pass 2: S0's scores (every load of a batch in flight together, or
        // the score keys of the listed entries), their
        // chunk bins formed again, U kept in place in index order (a batch's
        // entries are all read before the block scan that orders its writes)
        // per thread and batch: per <= 16 consecutive entries, spread evenly;
        // the loop is unrolled for the smallest R >= per (a row of a few
        // hundred keys does not step through 16 predicated slots)
        const uint32_t per = min((nS0 + kRT - 1) / kRT, 16u);
        uint32_t ubase = 0u;
        auto pass2 = [&](auto RC) {
          constexpr int R = decltype(RC)::value;
          for (uint32_t i0 = 0; i0 < nS0; i0 += per * kRT) {
            const uint32_t ib = i0 + per * tid;           // the thread's consecutive entries
            const uint32_t ie = min(ib + per, nS0);
            uint32_t jx[R];
            float dv[R];
#pragma unroll
            for (int x = 0; x < R; ++x) {
                const unsigned long long e = ib + x < ie ? (to_lds ? sm.big[ib + x] : gdst[ib + x]) : 0ull;
                jx[x] = ib + x < ie ? ~(uint32_t)e : 0u;
                dv[x] = key_score((uint32_t)(e >> 32));
            }
            if (!fl_route) {
#pragma unroll
                for (int x = 0; x < R; ++x) dv[x] = ib + x < ie ? srow[jx[x]] : 0.0f;
            }
            uint32_t keep = 0u;
#pragma unroll
            for (int x = 0; x < R; ++x) {
                if (ib + x >= ie) continue;
                const int ch = (int)(jx[x] / kChunk);
                if ((weight_bin(dv[x], sm.plan.mc[ch], s).bin >> 4) <= sm.plan.bsel[ch]) keep |= 1u << x;
            }
            unsigned long long t2;
            uint32_t o = ubase + (uint32_t)block_excl_scan_u64<kRT>((unsigned long long)__popc(keep), &t2, sm.scan_sh);
#pragma unroll
            for (int x = 0; x < R; ++x) {
                if (!((keep >> x) & 1u)) continue;
                const uint32_t key = score_key(dv[x]);
                const unsigned long long ent = ((unsigned long long)key << 32) | (unsigned long long)(~jx[x]);
                if (to_lds) {
                    sm.big[o] = ent;
                    sm.big[kCand + o] = unit ? 1ull : weight_bin(key_score(key), m, s).w;
                } else {
                    gdst[o] = ent;
                }
                ++o;
            }
            ubase += (uint32_t)t2;
          }
        };
        if (per <= 2) pass2(std::integral_constant<int, 2>{});
        else if (per <= 4) pass2(std::integral_constant<int, 4>{});
        else if (per <= 8) pass2(std::integral_constant<int, 8>{});
        else pass2(std::integral_constant<int, 16>{});
        nU = ubase;
        loaded = to_lds;
        if (fl_route) st.path = kPathFlagList;
    } else {
        // U is gathered from the scores, or the cut runs over the whole row:
        // every chunk it reads gets all its scores (the scoring pass stored
        // only the flagged keys', or every key's under a fixed top-k)
        const bool whole = nU > (unsigned long long)ws.ucap;
        if (g.sel_k <= 0) {
            int pend = -1;                                // chunks taken in pairs
            for (int c = 0; c < ri.nch; ++c)
                if (whole || sm.plan.bsel[c] >= 0) {
                    if (pend < 0) {
                        pend = c;
                    } else {
                        rescore_chunks(g, ri, ws, k_low, sm.btc, bt_cached, pend, c);
                        pend = -1;
                    }
                }
            if (pend >= 0) rescore_chunks(g, ri, ws, k_low, sm.btc, bt_cached, pend, -1);
            __syncthreads();
        }
    }
    if (!covered_path && nU <= (unsigned long long)ws.ucap) {
        st.path = kPathFromScores;
        // U from the row's scores, 16 consecutive keys per thread (one chunk),
        // compacted in index order into LDS (with weights) or the workspace list
        const bool to_lds = nU <= (unsigned long long)kCand;
        const uint32_t dcap = to_lds ? (uint32_t)kCand : (uint32_t)ws.ucap;
        uint32_t base = 0u;
        // the next step's scores are requested before this step's are used;
        // chunks without a part of U are not read
        float4 nx[4];
        const auto fetch = [&](int jj) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                nx[u] = jj < ri.L && sm.plan.bsel[jj / kChunk] >= 0
                            ? *reinterpret_cast<const float4*>(srow + jj + 4 * u)
                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        };
        fetch(16 * tid);
        for (int j0 = 0; j0 < ri.L; j0 += 16 * kRT) {
            const int jj = j0 + 16 * tid;
            uint32_t msk = 0u, c = 0u;
            float dv[16];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                dv[4 * u] = nx[u].x;
                dv[4 * u + 1] = nx[u].y;
                dv[4 * u + 2] = nx[u].z;
                dv[4 * u + 3] = nx[u].w;
            }
            fetch(jj + 16 * kRT);
            if (jj < ri.L) {
                const int ch = jj / kChunk;
                const int bs = sm.plan.bsel[ch];
                const float mc = sm.plan.mc[ch];
                if (bs >= 0) {
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (jj + e < ri.L && (weight_bin(dv[e], mc, s).bin >> 4) <= bs) {
                            msk |= 1u << e;
                            ++c;
                        }
                }
            }
            unsigned long long t2;
            uint32_t o = base + (uint32_t)block_excl_scan_u64<kRT>(c, &t2, sm.scan_sh);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if ((msk & (1u << e)) && o < dcap) {
                    const uint32_t key = score_key(dv[e]);
                    const unsigned long long ent = ((unsigned long long)key << 32) | (unsigned long long)(~(uint32_t)(jj + e));
                    if (to_lds) {
                        sm.big[o] = ent;
                        sm.big[kCand + o] = unit ? 1ull : weight_bin(key_score(key), m, s).w;
                    } else {
                        gdst[o] = ent;
                    }
                    ++o;
                }
            base += (uint32_t)t2;
        }
        loaded = to_lds;
    }
    __syncthreads();
    resolve_body(g, ri, ws, st, (int)nU, loaded, bt_cached, sm);
}

__global__ __launch_bounds__(kRT) void k_sel_row(Geo g, const float* __restrict__ top_p,
                                                 const bf16_t* __restrict__ k_low, int row0, SelWs ws,
                                                 int32_t* __restrict__ status) {
    __shared__ ResolveSm sm;
    row_pass(g, top_p, k_low, row_info(g, row0, blockIdx.x), ws, status, sm);
}

// The row pass with the decode step's local-head window attention on its
// spare workgroups: workgroups [0, rows) take the rows (one CU each, for their
// LDS), the others run window items of win_mfma.hpp, one per wavefront, on the
// CUs the rows leave free -- so the window's K/V stream overlaps the rows'
// latency-bound selection.  The window's partials are merged by the combine.
struct WinSm {
    int pgs[64];
    __align__(16) bf16_t Vs[32 * kWVsLd];
};

__global__ __launch_bounds__(kRT) void k_sel_row_win(Geo g, const float* __restrict__ top_p,
                                                     const bf16_t* __restrict__ k_low, int row0, SelWs ws,
                                                     int32_t* __restrict__ status, WinWork wa) {
    __shared__ union {
        ResolveSm rs;
        WinSm w[kRT / 64];
    } u;
    if ((int)blockIdx.x < ws.rows) {
        row_pass(g, top_p, k_low, row_info(g, row0, blockIdx.x), ws, status, u.rs);
        return;
    }
    const int wv = threadIdx.x >> 6;
    const int stride = ((int)gridDim.x - ws.rows) * (kRT / 64);
    for (int it = ((int)blockIdx.x - ws.rows) * (kRT / 64) + wv; it < wa.items; it += stride)
        win_mfma_item<true>(g, wa.q, wa.k, wa.v, wa.part, wa.nsplit, wa.split_keys, 0, it % wa.nsplit,
                            it / wa.nsplit, u.w[wv].pgs, u.w[wv].Vs);
}


// ---------------------------------------------------------------------------
// CSR row pointers of the group's rows and the capacity check (groups of more
// than kRowsInEmit rows; smaller groups are handled inside the emit pass).
// ---------------------------------------------------------------------------
constexpr int kRowsInEmit = 1024;

__global__ __launch_bounds__(kRT) void k_sel_rowptr(int row0, SelWs ws, SelOut out) {
    const int tid = threadIdx.x;
    __shared__ unsigned long long scan_sh[kRT / 64 + 1];
    int64_t carry = out.row_ptr[row0];
    for (int i0 = 0; i0 < ws.rows; i0 += kRT) {
        const int i = i0 + tid;
        const unsigned long long c = i < ws.rows ? (unsigned long long)ws.st[i].count : 0ull;
        unsigned long long tot;
        const unsigned long long ex = block_excl_scan_u64<kRT>(c, &tot, scan_sh);
        if (i < ws.rows) out.row_ptr[row0 + i + 1] = carry + (int64_t)(ex + c);
        carry += (int64_t)tot;
    }
    if (tid == 0 && carry > out.capacity && *out.status == 0) *out.status = 1;
}

// ---------------------------------------------------------------------------
// Emit.  grid (min(nchunk, kEmitWG), rows), 256 threads: workgroup x copies the
// 4096-entry slices x, x + kEmitWG, ... of a row's ordered selected list (the
// workspace list, the row's score array overwritten by indices, or every key).
// ROWPTR: the group is small, so every workgroup sums the counts before its
// row itself; the first one writes the row pointer and checks the capacity.
// ---------------------------------------------------------------------------
constexpr int kEmitWG = 4;

template <int ROWPTR>
__global__ __launch_bounds__(256) void k_sel_emit(Geo g, int row0, SelWs ws, SelOut out) {
    const int tid = threadIdx.x;
    const int first = blockIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    const RowState st = ws.st[ri.lrow];
    if (first >= ri.nch) return;
    if (first > 0 && first * kChunk >= st.count) return;   // nothing of this row here
    int64_t rbase;
    if (ROWPTR) {
        __shared__ unsigned long long red[8];
        unsigned long long before = 0, all = 0;
        for (int i = tid; i < ws.rows; i += 256) {
            const unsigned long long c = (unsigned long long)ws.st[i].count;
            all += c;
            if (i < ri.lrow) before += c;
        }
        before = wave_sum_u64(before);
        all = wave_sum_u64(all);
        if ((tid & 63) == 0) {
            red[tid >> 6] = before;
            red[4 + (tid >> 6)] = all;
        }
        __syncthreads();
        const int64_t carry = out.row_ptr[row0];
        rbase = carry + (int64_t)(red[0] + red[1] + red[2] + red[3]);
        const int64_t total = carry + (int64_t)(red[4] + red[5] + red[6] + red[7]);
        if (first == 0 && tid == 0) out.row_ptr[ri.row + 1] = rbase + st.count;
        if (total > out.capacity) {
            if (first == 0 && tid == 0 && ri.lrow == 0 && *out.status == 0) *out.status = 1;
            return;
        }
    } else {
        rbase = out.row_ptr[ri.row];
    }
    if (*out.status != 0) return;
    const uint32_t* src = st.mode == 1 ? ws.sel + (size_t)ri.lrow * ws.ucap
                                       : reinterpret_cast<const uint32_t*>(ws.scores + (size_t)ri.lrow * ws.score_ld);
    for (int chunk = first; chunk * kChunk < st.count; chunk += gridDim.x) {
        const int jbase = chunk * kChunk;
        for (int k = tid; k < kChunk && jbase + k < st.count; k += 256)
            out.idx[rbase + jbase + k] = st.mode == 0 ? jbase + k : (int32_t)src[jbase + k];
    }
}

// Per-row path codes of the last selection (inspection).  grid (rows / 256 + 1).
__global__ void k_sel_paths(const RowState* __restrict__ st, int rows, int32_t* __restrict__ paths) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < rows) paths[i] = st[i].path;
}

}  // namespace

hipError_t launch_select_paths(const SelWs& ws, int rows, int32_t* paths, hipStream_t s) {
    hipLaunchKernelGGL(k_sel_paths, dim3((rows + 255) / 256), dim3(256), 0, s, ws.st, rows, paths);
    return hipGetLastError();
}

hipError_t launch_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                         const float* top_p, int row0, const SelWs& ws, const SelOut& out,
                         int total_rows, int dtype, int stage, hipStream_t s, const WinWork* win,
                         const KeyAppend* app) {
    (void)total_rows;
    const dim3 grid(ws.nchunk, ws.rows);
    bf16_t* kl = (bf16_t*)const_cast<uint16_t*>(k_low);
    const KeyAppend ap = app && stage != kSelScoresOnly ? *app : KeyAppend{nullptr, nullptr};
    const bool scores_only = stage == kSelScoresOnly;
    if (stage != kSelFinish) {
        if (dtype == 0 && scores_only)
            hipLaunchKernelGGL((k_sel_score<float, 0>), grid, dim3(256), 0, s, g, (const float*)q, (const float*)w_q,
                               kl, row0, ws, out, ap);
        else if (dtype == 0)
            hipLaunchKernelGGL((k_sel_score<float, 1>), grid, dim3(256), 0, s, g, (const float*)q, (const float*)w_q,
                               kl, row0, ws, out, ap);
        else if (scores_only)
            hipLaunchKernelGGL((k_sel_score<bf16_t, 0>), grid, dim3(256), 0, s, g, (const bf16_t*)q,
                               (const bf16_t*)w_q, kl, row0, ws, out, ap);
        else
            hipLaunchKernelGGL((k_sel_score<bf16_t, 1>), grid, dim3(256), 0, s, g, (const bf16_t*)q,
                               (const bf16_t*)w_q, kl, row0, ws, out, ap);
    }
    if (scores_only || stage == kSelScorePass) return hipGetLastError();
    if (stage == kSelRows && win && win->items > 0) {
        const int nw = std::min((win->items + kRT / 64 - 1) / (kRT / 64), std::max(1, kWinCUs - ws.rows));
        hipLaunchKernelGGL(k_sel_row_win, dim3(ws.rows + nw), dim3(kRT), 0, s, g, top_p, kl, row0, ws, out.status,
                           *win);
    } else {
        hipLaunchKernelGGL(k_sel_row, dim3(ws.rows), dim3(kRT), 0, s, g, top_p, kl, row0, ws, out.status);
    }
    if (stage == kSelRows) return hipGetLastError();
    const dim3 egrid(std::min(ws.nchunk, kEmitWG), ws.rows);
    if (ws.rows <= kRowsInEmit) {
        hipLaunchKernelGGL(k_sel_emit<1>, egrid, dim3(256), 0, s, g, row0, ws, out);
    } else {
        hipLaunchKernelGGL(k_sel_rowptr, dim3(1), dim3(kRT), 0, s, row0, ws, out);
        hipLaunchKernelGGL(k_sel_emit<0>, egrid, dim3(256), 0, s, g, row0, ws, out);
    }
    return hipGetLastError();
}

}  // namespace rtp
