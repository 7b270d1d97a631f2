// select.hip -- indexer query projection, indexer scores and dynamic top-p
// selection on gfx950 (VALU; the score is a K=16 contraction read once per key,
// so the scoring pass is bound by the HBM stream of the indexer key cache).
//
// Method: arXiv 2605.16928 abstract obs. (2)-(3) (16-dimensional indexer,
// dynamic top-p instead of fixed top-k); zhichai.net forum post "RTPurbo:
// Turning Dense LLMs into Sparse Attention Models ...", "Three Key Insights"
// items 2-3 (low-frequency projection; cumulative top-p).  The forum's
// "Open Questions and Limitations" notes that per-query token counts are
// unfriendly to GPU parallelism; here every pass is split into fixed
// 4096-key chunks so variable budgets never change the launch shape.
//
// Passes (one row = one (query token, retrieval head) pair):
//   1 score:   q_low, fp32 chain scores of every key, chunk maxima
//   2 hist:    exact fixed-point mass per level-1 bin (device atomics)
//   2b cut:    per row, the bin b1 where the cumulative mass reaches p
//   3 refine:  per-chunk count of keys above b1; keys of bin b1 gathered
//   4 resolve: one workgroup per row ranks bin b1 exactly (score desc, index
//              asc), fixes the last selected key and the per-chunk offsets
//   4b rowptr: CSR row pointers and the capacity check
//   5 emit:    ordered compaction of the selected indices
// Workgroups of one pass never wait on each other: every hand-off between
// workgroups is a kernel boundary (a device-scope fence per workgroup costs an
// L2 write-back and invalidate on this multi-XCD part).
#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

// level-1 bin only: identical arithmetic to weight_bin's bin
__device__ __forceinline__ int bin_of(float d, float m, float s) {
    float t = d - m;
    float y = s * t;
    float x = -y * kBinsPerUnit;
    x = fminf(x, (float)(kNB1 - 1));
    return (int)x;
}

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
// Pass 1.  grid (nchunk, rows), 256 threads.  Thread i of chunk c scores keys
// c*4096 + 256*k + i, k = 0..15, i.e. slot i of the chunk's 16 pages: every
// iteration reads one page's 8 KiB run of the head's indexer keys, coalesced.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_sel_score(Geo g, const T* __restrict__ q,
                                                   const T* __restrict__ w_q,
                                                   const bf16_t* __restrict__ k_low, int row0,
                                                   SelWs ws, SelOut out, int scores_only) {
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    if (!scores_only) {
        const int nthr = gridDim.x * 256;
        for (int i = chunk * 256 + tid; i < kNB1; i += nthr) {
            ws.hmass[(size_t)ri.lrow * kNB1 + i] = 0ull;
            ws.hcnt[(size_t)ri.lrow * kNB1 + i] = 0u;
        }
        for (int i = chunk * 256 + tid; i < ws.nchunk; i += nthr)
            ws.chunk_cnt[(size_t)ri.lrow * ws.nchunk + i] = 0u;
        if (chunk == 0 && tid == 0) {
            ws.cand_n[ri.lrow] = 0u;
            if (ri.lrow == 0 && row0 == 0) {
                *out.status = 0;
                out.row_ptr[0] = 0;
            }
        }
    }
    if (chunk >= ri.nch) return;

    __shared__ float qs[kIdx];
    __shared__ float wmax[4];
    __shared__ float qrow[128];
    __shared__ float wq[128 * kIdx];
    const int32_t* bt = g.block_table + (size_t)ri.b * g.max_blocks;
    float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int jbase = chunk * kChunk;

    // Issue the first group of indexer-key loads, then build q_low while they
    // are in flight (the query row and W_q are staged through LDS so that the
    // fixed-order chain runs on LDS operands).
    uint4 buf[8];
    // Unconditional loads: page ids are uniform per 256-key step (clamped to the
    // row's last page) and slots past the row's end are read but never used.
    const int last_page = (ri.L - 1) >> 8;
    auto load_group = [&](int k0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pi = min((jbase >> 8) + k0 + u, last_page);
            const int page = bt[pi];
            const uint4* kp = reinterpret_cast<const uint4*>(
                k_low + (((size_t)page * g.n_ret + ri.r) * kBlk + tid) * kIdx);
            buf[2 * u] = kp[0];
            buf[2 * u + 1] = kp[1];
        }
    };
    load_group(0);
    {
        const int h = g.ret_heads[ri.r];
        const T* qp = q + ((size_t)ri.t * g.Hq + h) * g.D;
        const T* wp = w_q + (size_t)ri.r * g.D * kIdx;
        for (int x = tid; x < g.D; x += 256) qrow[x] = ld(qp + x);
        for (int x = tid; x < g.D * kIdx; x += 256) wq[x] = ld(wp + x);
    }
    __syncthreads();
    if (tid < kIdx) {
        float acc = 0.0f;
        for (int d = 0; d < g.D; ++d) acc = __builtin_fmaf(qrow[d], wq[d * kIdx + tid], acc);
        const bf16_t qb = f2bf(acc);
        qs[tid] = bf2f(qb);
        if (chunk == 0) ws.qlow[(size_t)ri.lrow * kIdx + tid] = qb;
    }
    __syncthreads();
    float qv[kIdx];
#pragma unroll
    for (int c = 0; c < kIdx; ++c) qv[c] = qs[c];

    float mx = -INFINITY;
#pragma unroll 1
    for (int k0 = 0; k0 < 16; k0 += 4) {
        if (k0) load_group(k0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = jbase + (k0 + u) * 256 + tid;
            float kf[kIdx];
            unpack8(buf[2 * u], kf);
            unpack8(buf[2 * u + 1], kf + 8);
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < kIdx; ++c) acc = __builtin_fmaf(qv[c], kf[c], acc);
            if (j < ri.L) {
                srow[j] = acc;
                mx = fmaxf(mx, acc);
            }
        }
    }
    if (scores_only) return;
    mx = wave_max(mx);
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
        float m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        ws.cmax[(size_t)ri.lrow * ws.nchunk + chunk] = score_key(m);
    }
}

// ---------------------------------------------------------------------------
// Pass 2.  Level-1 histogram of exact fixed-point mass.  grid (nhist, rows):
// a workgroup covers kHistKeys keys (four score chunks), accumulates in LDS and
// adds its non-empty bins to the row's histogram with device atomics (integer,
// so the result does not depend on their order).
// ---------------------------------------------------------------------------
constexpr int kHistKeys = 4 * kChunk;

__device__ __forceinline__ float row_max(const SelWs& ws, int lrow, int nch, uint32_t* red) {
    const int tid = threadIdx.x;
    uint32_t mk = 0u;
    for (int c = tid; c < nch; c += 256) {
        const uint32_t v = ws.cmax[(size_t)lrow * ws.nchunk + c];
        mk = v > mk ? v : mk;
    }
    mk = wave_max_u32(mk);
    if ((tid & 63) == 0) red[tid >> 6] = mk;
    __syncthreads();
    mk = red[0];
    for (int w = 1; w < 4; ++w) mk = red[w] > mk ? red[w] : mk;
    __syncthreads();
    return key_score(mk);
}

__global__ __launch_bounds__(256) void k_sel_hist(Geo g, int row0, SelWs ws) {
    const int tid = threadIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    const int jbase = blockIdx.x * kHistKeys;
    if (jbase >= ri.L) return;
    __shared__ unsigned long long hm[kNB1];
    __shared__ uint32_t hc[kNB1];
    __shared__ uint32_t red[4];
    for (int i = tid; i < kNB1; i += 256) {
        hm[i] = 0ull;
        hc[i] = 0u;
    }
    const float m = row_max(ws, ri.lrow, ri.nch, red);
    const float s = g.idx_scale;
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    for (int k0 = 0; k0 < kHistKeys / 256; k0 += 16) {
        float dv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) dv[k] = srow[min(jbase + (k0 + k) * 256 + tid, ri.L - 1)];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int j = jbase + (k0 + k) * 256 + tid;
            if (j < ri.L) {
                const WeightBin wb = weight_bin(dv[k], m, s);
                atomicAdd(&hm[wb.bin], wb.w);
                atomicAdd(&hc[wb.bin], 1u);
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < kNB1; i += 256) {
        if (hc[i]) {
            atomicAdd(&ws.hmass[(size_t)ri.lrow * kNB1 + i], hm[i]);
            atomicAdd(&ws.hcnt[(size_t)ri.lrow * kNB1 + i], hc[i]);
        }
    }
}

// ---------------------------------------------------------------------------
// Pass 2b.  One workgroup per row: total mass, target ceil(p Z) and the bin b1
// where the cumulative mass (highest scores first) reaches it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sel_cut(Geo g, const float* __restrict__ top_p, int row0, SelWs ws) {
    const int tid = threadIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.x);
    __shared__ uint32_t red[4], red2[4];
    __shared__ unsigned long long scan_sh[5];
    __shared__ int s_b1;
    const float m = row_max(ws, ri.lrow, ri.nch, red);
    unsigned long long lm[8];
    uint32_t lc[8];
    unsigned long long msum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        lm[i] = ws.hmass[(size_t)ri.lrow * kNB1 + tid * 8 + i];
        lc[i] = ws.hcnt[(size_t)ri.lrow * kNB1 + tid * 8 + i];
        msum += lm[i];
    }
    unsigned long long Z;
    const unsigned long long before = block_excl_scan_u64<256>(msum, &Z, scan_sh);
    const float p = top_p[ri.b];
    unsigned long long target = Z;
    const int keep_all = !(p < 1.0f);
    if (!keep_all) {
        const double pz = ceil((double)p * (double)Z);
        target = (unsigned long long)pz;
        if (target > Z) target = Z;
        if (target < 1ull) target = 1ull;
    }
    if (tid == 0) s_b1 = kNB1;
    __syncthreads();
    if (!keep_all) {
        unsigned long long run = before;
        for (int i = 0; i < 8; ++i) {
            run += lm[i];
            if (run >= target) {
                atomicMin(&s_b1, tid * 8 + i);
                break;
            }
        }
    }
    __syncthreads();
    const int b1 = s_b1;
    uint32_t ca = 0;
    unsigned long long sa = 0;
    for (int i = 0; i < 8; ++i) {
        if (tid * 8 + i < b1) {
            ca += lc[i];
            sa += lm[i];
        }
    }
    const uint32_t cnt_above = block_sum_u32<256>(ca, red2);
    unsigned long long S_above;
    (void)block_excl_scan_u64<256>(sa, &S_above, scan_sh);
    if (tid == 0) {
        RowState st;
        st.m = m;
        st.b1 = b1;
        st.Z = Z;
        st.target = target;
        st.S_above = S_above;
        st.cnt_above = cnt_above;
        st.cnt_b1 = b1 < kNB1 ? ws.hcnt[(size_t)ri.lrow * kNB1 + b1] : 0u;
        st.Tkey = 0u;
        st.jT = -1;
        st.L = ri.L;
        st.count = keep_all ? ri.L : 0;
        ws.st[ri.lrow] = st;
    }
}

// ---------------------------------------------------------------------------
// Pass 3.  Keys above the cut bin are counted per chunk; keys of the cut bin
// are gathered as (score key << 32 | ~index) for the exact ranking.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sel_refine(Geo g, int row0, SelWs ws) {
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    if (chunk >= ri.nch) return;
    __shared__ uint32_t red[4];
    const RowState st = ws.st[ri.lrow];
    const float s = g.idx_scale;
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int jbase = chunk * kChunk;
    uint32_t above = 0;
    if (st.b1 >= kNB1) {
        above = (uint32_t)min(kChunk, ri.L - jbase);
    } else {
        const bool gather = st.cnt_b1 <= (uint32_t)kCand;
        float dv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) dv[k] = srow[min(jbase + k * 256 + tid, ri.L - 1)];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int j = jbase + k * 256 + tid;
            if (j < ri.L) {
                const float d = dv[k];
                const int bn = bin_of(d, st.m, s);
                if (bn < st.b1) {
                    ++above;
                } else if (bn == st.b1 && gather) {
                    const uint32_t slot = atomicAdd(&ws.cand_n[ri.lrow], 1u);
                    if (slot < (uint32_t)kCand)
                        ws.cand[(size_t)ri.lrow * kCand + slot] =
                            ((unsigned long long)score_key(d) << 32) | (unsigned long long)(~(uint32_t)j);
                }
            }
        }
    }
    const uint32_t tot = block_sum_u32<256>(above, red);
    if (tid == 0) ws.chunk_cnt[(size_t)ri.lrow * ws.nchunk + chunk] = tot;
}

// ---------------------------------------------------------------------------
// Pass 4.  One 1024-thread workgroup per row: exact ranking inside bin b1.
// ---------------------------------------------------------------------------
constexpr int kRT = 1024;

__device__ void bitonic_desc(unsigned long long* a, int n) {
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n; i += kRT) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const unsigned long long x = a[i], y = a[ixj];
                    const bool desc = (i & k) == 0;
                    if (desc ? (x < y) : (x > y)) {
                        a[i] = y;
                        a[ixj] = x;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Given candidates cand[0..n) sorted by rank, the mass S0 ranked before them and
// the target, find the first candidate whose cumulative mass reaches target.
__device__ int first_reaching(const unsigned long long* cand, int n, float m, float s,
                              unsigned long long S0, unsigned long long target,
                              unsigned long long* scan_sh, int* s_idx) {
    constexpr int per = kCand / kRT;   // 8 candidates per thread
    unsigned long long wv[per];
    unsigned long long loc = 0;
    for (int i = 0; i < per; ++i) {
        const int c = threadIdx.x * per + i;
        wv[i] = 0;
        if (c < n) wv[i] = weight_bin(key_score((uint32_t)(cand[c] >> 32)), m, s).w;
        loc += wv[i];
    }
    unsigned long long tot;
    unsigned long long run = S0 + block_excl_scan_u64<kRT>(loc, &tot, scan_sh);
    if (threadIdx.x == 0) *s_idx = n - 1;   // mass of the bin reaches target by construction
    __syncthreads();
    for (int i = 0; i < per; ++i) {
        const int c = threadIdx.x * per + i;
        run += wv[i];
        if (c < n && run >= target) {
            atomicMin(s_idx, c);
            break;
        }
    }
    __syncthreads();
    return *s_idx;
}

__global__ __launch_bounds__(kRT) void k_sel_resolve(Geo g, int row0, SelWs ws, SelOut out,
                                                     int total_rows) {
    const int tid = threadIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.x);
    __shared__ unsigned long long cand[kCand];
    __shared__ unsigned long long scan_sh[kRT / 64 + 1];
    __shared__ uint32_t ccount[1024];          // per-chunk selected keys of bin b1
    __shared__ unsigned long long hmb[kNB1];
    __shared__ uint32_t hcb[kNB1];
    __shared__ int s_idx;
    __shared__ uint32_t s_klo, s_khi, s_n;
    __shared__ unsigned long long s_S;
    RowState st = ws.st[ri.lrow];
    const float s = g.idx_scale;
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int nch = ri.nch;

    for (int c = tid; c < 1024; c += kRT) ccount[c] = 0u;
    __syncthreads();

    if (st.b1 < kNB1) {
        uint32_t Tkey = 0u;
        int32_t jT = -1;
        bool have_cands = false;
        bool whole_bin = false;            // the candidates are every key of bin b1
        int n = 0, ic = -1;
        unsigned long long S0 = st.S_above;
        if (st.cnt_b1 <= (uint32_t)kCand) {
            n = (int)st.cnt_b1;
            for (int i = tid; i < n; i += kRT) cand[i] = ws.cand[(size_t)ri.lrow * kCand + i];
            have_cands = true;
            whole_bin = true;
        } else {
            // Many keys share bin b1: narrow the score-key range with 2048-bucket
            // histograms over the row until it fits the sort or is one tie group.
            uint32_t klo = 0u, khi = 0xFFFFFFFFu;
            unsigned long long S_hi = st.S_above;
            for (int iter = 0; iter < 4; ++iter) {
                const uint32_t span = khi - klo;
                const int bits = span ? 32 - __clz(span) : 0;
                const int shift = bits > 11 ? bits - 11 : 0;
                for (int i = tid; i < kNB1; i += kRT) {
                    hmb[i] = 0ull;
                    hcb[i] = 0u;
                }
                __syncthreads();
                for (int j = tid; j < ri.L; j += kRT) {
                    const float d = srow[j];
                    if (bin_of(d, st.m, s) != st.b1) continue;
                    const uint32_t key = score_key(d);
                    if (key < klo || key > khi) continue;
                    const uint32_t bk = (key - klo) >> shift;
                    atomicAdd(&hmb[bk], weight_bin(d, st.m, s).w);
                    atomicAdd(&hcb[bk], 1u);
                }
                __syncthreads();
                if (tid == 0) {
                    // buckets rank from the highest key down
                    const uint32_t nb = (span >> shift) + 1u;
                    unsigned long long run = S_hi;
                    uint32_t kb = 0;
                    for (int32_t bk = (int32_t)nb - 1; bk >= 0; --bk) {
                        if (run + hmb[bk] >= st.target && hcb[bk]) {
                            kb = (uint32_t)bk;
                            break;
                        }
                        run += hmb[bk];
                    }
                    s_S = run;
                    s_klo = klo + (kb << shift);
                    const uint32_t top = s_klo + ((1u << shift) - 1u);
                    s_khi = (shift == 32 || top < s_klo || top > khi) ? khi : top;
                    s_n = hcb[kb];
                }
                __syncthreads();
                klo = s_klo;
                khi = s_khi;
                S_hi = s_S;
                if (s_n <= (uint32_t)kCand) {
                    // gather the bucket's keys and rank them by sorting
                    if (tid == 0) s_n = 0u;
                    __syncthreads();
                    for (int j = tid; j < ri.L; j += kRT) {
                        const float d = srow[j];
                        if (bin_of(d, st.m, s) != st.b1) continue;
                        const uint32_t key = score_key(d);
                        if (key < klo || key > khi) continue;
                        const uint32_t slot = atomicAdd(&s_n, 1u);
                        if (slot < (uint32_t)kCand)
                            cand[slot] = ((unsigned long long)key << 32) | (unsigned long long)(~(uint32_t)j);
                    }
                    __syncthreads();
                    n = min((int)s_n, kCand);
                    S0 = S_hi;
                    have_cands = true;
                    break;
                }
                if (klo == khi) {
                    // one tie group: take its lowest-index members until the mass is reached
                    const unsigned long long wT = weight_bin(key_score(klo), st.m, s).w;
                    const unsigned long long need = st.target - S_hi;
                    const unsigned long long ntie = (need + wT - 1ull) / wT;
                    if (tid == 0) s_n = 0u;
                    if (tid == 0) s_idx = -1;
                    __syncthreads();
                    // ordered scan in index order, kRT keys at a time
                    for (int j0 = 0; j0 < ri.L; j0 += kRT) {
                        const int j = j0 + tid;
                        const bool is_tie = j < ri.L && score_key(srow[j]) == klo &&
                                            bin_of(srow[j], st.m, s) == st.b1;
                        const uint32_t before_blk = s_n;
                        unsigned long long tot;
                        const unsigned long long rank =
                            block_excl_scan_u64<kRT>(is_tie ? 1ull : 0ull, &tot, scan_sh);
                        if (is_tie && before_blk + rank + 1ull == ntie) s_idx = j;
                        __syncthreads();
                        if (tid == 0) s_n = before_blk + (uint32_t)tot;
                        __syncthreads();
                        if (s_idx >= 0) break;
                    }
                    Tkey = klo;
                    jT = s_idx;
                    break;
                }
            }
        }
        if (have_cands) {
            int np2 = 1;
            while (np2 < n) np2 <<= 1;
            for (int i = n + tid; i < np2; i += kRT) cand[i] = 0ull;
            __syncthreads();
            bitonic_desc(cand, np2);
            ic = first_reaching(cand, n, st.m, s, S0, st.target, scan_sh, &s_idx);
            Tkey = (uint32_t)(cand[ic] >> 32);
            jT = (int32_t)(~(uint32_t)cand[ic]);
        }
        // selected keys of bin b1 per chunk
        if (whole_bin) {
            for (int i = tid; i <= ic; i += kRT)
                atomicAdd(&ccount[(int)(~(uint32_t)cand[i]) / kChunk], 1u);
        } else {
            for (int j = tid; j < ri.L; j += kRT) {
                const float d = srow[j];
                if (bin_of(d, st.m, s) != st.b1) continue;
                const uint32_t key = score_key(d);
                if (key > Tkey || (key == Tkey && j <= jT)) atomicAdd(&ccount[j / kChunk], 1u);
            }
        }
        st.Tkey = Tkey;
        st.jT = jT;
    }
    __syncthreads();
    // per-chunk output offsets of this row (nch <= 1024 chunks)
    {
        unsigned long long n_c = 0;
        if (tid < nch) {
            if (st.b1 >= kNB1)
                n_c = (unsigned long long)min(kChunk, ri.L - tid * kChunk);
            else
                n_c = ws.chunk_cnt[(size_t)ri.lrow * ws.nchunk + tid] + ccount[tid];
        }
        unsigned long long tot;
        const unsigned long long ex = block_excl_scan_u64<kRT>(n_c, &tot, scan_sh);
        if (tid < nch) ws.chunk_cnt[(size_t)ri.lrow * ws.nchunk + tid] = (uint32_t)ex;
        if (tid == 0) {
            st.count = (int32_t)tot;
            ws.st[ri.lrow] = st;
        }
    }
    (void)total_rows;
}

// ---------------------------------------------------------------------------
// Pass 4b.  CSR row pointers of the group's rows and the capacity check.
// ---------------------------------------------------------------------------
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
    if (tid == 0 && carry > out.capacity) *out.status = 1;
}

// ---------------------------------------------------------------------------
// Pass 5.  Ordered compaction of the selected indices of each chunk.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sel_emit(Geo g, int row0, SelWs ws, SelOut out) {
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    if (chunk >= ri.nch) return;
    if (*out.status != 0) return;
    __shared__ uint32_t wcnt[4];
    const RowState st = ws.st[ri.lrow];
    const float s = g.idx_scale;
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    int64_t base = out.row_ptr[ri.row] + ws.chunk_cnt[(size_t)ri.lrow * ws.nchunk + chunk];
    const int jbase = chunk * kChunk;
    const int lane = tid & 63, wid = tid >> 6;
    float dv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) dv[k] = srow[min(jbase + k * 256 + tid, ri.L - 1)];
    for (int k = 0; k < 16; ++k) {
        if (jbase + k * 256 >= ri.L) break;
        const int j = jbase + k * 256 + tid;
        bool sel = false;
        if (j < ri.L) {
            if (st.b1 >= kNB1) {
                sel = true;
            } else {
                const float d = dv[k];
                const int bn = bin_of(d, st.m, s);
                if (bn < st.b1) {
                    sel = true;
                } else if (bn == st.b1) {
                    const uint32_t key = score_key(d);
                    sel = key > st.Tkey || (key == st.Tkey && j <= st.jT);
                }
            }
        }
        const unsigned long long bal = __ballot(sel);
        const uint32_t before = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wcnt[wid] = __popcll(bal);
        __syncthreads();
        uint32_t wbase = 0;
        for (int w = 0; w < wid; ++w) wbase += wcnt[w];
        const uint32_t tot = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        const int64_t o = base + wbase + before;
        if (sel && o < out.capacity) out.idx[o] = j;
        base += tot;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                         const float* top_p, int row0, const SelWs& ws, const SelOut& out,
                         int total_rows, int dtype, int scores_only, hipStream_t s) {
    const dim3 grid(ws.nchunk, ws.rows);
    if (dtype == 0)
        hipLaunchKernelGGL(k_sel_score<float>, grid, dim3(256), 0, s, g, (const float*)q,
                           (const float*)w_q, k_low, row0, ws, out, scores_only);
    else
        hipLaunchKernelGGL(k_sel_score<bf16_t>, grid, dim3(256), 0, s, g, (const bf16_t*)q,
                           (const bf16_t*)w_q, k_low, row0, ws, out, scores_only);
    if (scores_only) return hipGetLastError();
    const int nhist = (ws.nchunk + 3) / 4;
    hipLaunchKernelGGL(k_sel_hist, dim3(nhist, ws.rows), dim3(256), 0, s, g, row0, ws);
    hipLaunchKernelGGL(k_sel_cut, dim3(ws.rows), dim3(256), 0, s, g, top_p, row0, ws);
    hipLaunchKernelGGL(k_sel_refine, grid, dim3(256), 0, s, g, row0, ws);
    hipLaunchKernelGGL(k_sel_resolve, dim3(ws.rows), dim3(kRT), 0, s, g, row0, ws, out, total_rows);
    hipLaunchKernelGGL(k_sel_rowptr, dim3(1), dim3(kRT), 0, s, row0, ws, out);
    hipLaunchKernelGGL(k_sel_emit, grid, dim3(256), 0, s, g, row0, ws, out);
    return hipGetLastError();
}

}  // namespace rtp
