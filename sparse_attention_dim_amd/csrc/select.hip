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
//            and the chunk's cumulative mass histogram: exact fixed-point
//            weights exp(s (d - m_c)) summed over bins of x_c = s (m_c - d)
//            (1/4 wide)
//   gather / resolve: every workgroup of the gather pass forms its row's plan
//            (below) and gathers its chunk's part of U; one workgroup per row
//            then resolves the cut.  Row maximum m and total mass
//            Z = sum_c exp(s (m_c - m)) Z_c; every chunk bin whose upper edge
//            lies below a threshold X on the row's x axis certainly holds
//            keys with x < X, which gives a lower bound of the mass above
//            any X.  The smallest X whose bound reaches the target fixes the
//            candidate set U = {d >= m - X / s}: it holds every key ranked at
//            or above the cut.  U is gathered from the scores into LDS and the
//            cut is found by radix selection over its score keys with exact
//            masses per bucket (ties: lowest indices first); when U does not
//            fit LDS the same selection runs over the row's scores.  U is
//            gathered in index order, so the selected keys are its filter.
//   emit:    CSR row pointers, the capacity check, and the selected indices
//            of every row
// Workgroups of one pass never wait on each other: every hand-off between
// workgroups is a kernel boundary (a device-scope fence per workgroup costs an
// L2 write-back and invalidate on this multi-XCD part).
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

constexpr float kCBPerUnit = 4.0f;   // chunk histogram bins per unit of x
constexpr int kGB = 256;             // row threshold grid (same width), X = k / 4
constexpr int kRT = 1024;            // resolve workgroup
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
// STATS: also the chunk maximum and the chunk's mass histogram.
// ---------------------------------------------------------------------------
template <typename T, int STATS>
__global__ __launch_bounds__(256) void k_sel_score(Geo g, const T* __restrict__ q, const T* __restrict__ w_q,
                                                   const bf16_t* __restrict__ k_low, int row0, SelWs ws,
                                                   SelOut out) {
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
    __shared__ __align__(16) float qrow[128];
    __shared__ __align__(16) float wq[128 * kIdx];
    __shared__ float qs[kIdx];
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
    uint4 buf[8];
    auto load_group = [&](int k0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int page = __builtin_amdgcn_readlane(my_page, k0 + u);
            const uint4* kp = reinterpret_cast<const uint4*>(
                k_low + (((size_t)page * g.n_ret + ri.r) * kBlk + tid) * kIdx);
            buf[2 * u] = kp[0];
            buf[2 * u + 1] = kp[1];
        }
    };
    load_group(0);
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
    }
    __syncthreads();
    float qv[kIdx];
#pragma unroll
    for (int c = 0; c < kIdx; ++c) qv[c] = qs[c];

    float dv[16];
    float mx = -INFINITY;
#pragma unroll
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
            dv[k0 + u] = acc;
            if (j < ri.L) mx = fmaxf(mx, acc);
        }
    }
    // the scores, after every key load was issued
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int j = jbase + k * 256 + tid;
        if (j < ri.L) srow[j] = dv[k];
    }
    if (!STATS) return;
    mx = wave_max(mx);
    if ((tid & 63) == 0) wmax[tid >> 6] = mx;
    __syncthreads();
    const float mc = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    if (tid == 0) ws.cmax[(size_t)ri.lrow * ws.nchunk + chunk] = score_key(mc);
    const float s = g.idx_scale;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int j = jbase + k * 256 + tid;
        if (j < ri.L) {
            const WeightBin wb = weight_bin(dv[k], mc, s);
            atomicAdd(&hist[wb.bin >> 4], wb.w);         // 64 level-1 bins per unit -> 4 per unit
            atomicAdd(&hcnt[wb.bin >> 4], 1u);
        }
    }
    __syncthreads();
    // cumulative over bins (the mass of keys with x_c < (b + 1) / 4)
    if (tid < 64) {
        const unsigned long long a = hist[2 * tid], b = hist[2 * tid + 1];
        unsigned long long incl = a + b;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long y = __shfl_up(incl, o);
            if (tid >= o) incl += y;
        }
        unsigned long long* ch = ws.chist + ((size_t)ri.lrow * ws.nchunk + chunk) * kCB;
        ch[2 * tid] = incl - b;
        ch[2 * tid + 1] = incl;
    } else if (tid < 128) {
        const int t = tid - 64;
        const unsigned a = hcnt[2 * t], b = hcnt[2 * t + 1];
        unsigned incl = a + b;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned y = __shfl_up(incl, o);
            if (t >= o) incl += y;
        }
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

__device__ Cut radix_cut(const unsigned long long* cand, int n, const float* srow, int L, uint32_t klo,
                         uint32_t khi, unsigned long long S_hi, unsigned long long target, float m, float s,
                         unsigned long long* hmb, uint32_t* hcb, unsigned long long* scan_sh, uint32_t* s_u,
                         unsigned long long* s_S, int* s_i) {
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
            atomicAdd(&hmb[bk], weight_bin(key_score(key), m, s).w);
            atomicAdd(&hcb[bk], 1u);
        }
        __syncthreads();
        // first bucket (highest keys first) whose cumulative mass reaches target
        unsigned long long loc = hmb[2 * tid] + hmb[2 * tid + 1];
        unsigned long long tot;
        const unsigned long long ex = S_hi + block_excl_scan_u64<kRT>(loc, &tot, scan_sh);
        if (tid == 0) *s_i = kNR;
        __syncthreads();
        if (ex + hmb[2 * tid] >= target && hcb[2 * tid]) atomicMin(s_i, 2 * tid);
        else if (ex + loc >= target && hcb[2 * tid + 1]) atomicMin(s_i, 2 * tid + 1);
        __syncthreads();
        const int nb = (int)(span >> shift) + 1;
        int bk = *s_i;
        // the mass ranked above the bucket, from the thread that holds it
        if (bk < kNR && (bk >> 1) == tid) {
            *s_S = (bk & 1) ? ex + hmb[2 * tid] : ex;
            *s_u = hcb[bk];
        }
        if (bk >= kNR && tid == 0) {
            // the target is not reached (rounding): the last bucket
            *s_S = S_hi + tot - hmb[nb - 1];
            *s_u = hcb[nb - 1];
        }
        if (bk >= kNR) bk = nb - 1;
        __syncthreads();
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
            const unsigned long long wT = weight_bin(key_score(klo), m, s).w;
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

// Plan of one row, computed by every workgroup of the gather pass (256
// threads): row maximum m, total mass Z = sum_c exp(s (m_c - m)) Z_c, the
// target, and the threshold d_thr of the candidate set U.  Every chunk bin
// whose upper edge, moved to the row's axis, lies below X = k / 4 certainly
// holds keys with s (m - d) < X: that gives a lower bound LB(k) of the mass
// above any k; the smallest k whose bound reaches the target (plus one unit
// of rounding per key) fixes U = {d >= m - X / s}.
struct Plan {
    float m, d_thr;
    unsigned long long target;
    int all;                                          // p >= 1: every key
    int ks;                                           // X = ks / 4, or kGB if no grid point suffices
};

__device__ Plan row_plan(const Geo& g, const RowInfo& ri, const SelWs& ws, const float* __restrict__ top_p,
                         double* fch, double* dch, double* dred, uint32_t* ured, int* s_k) {
    const int tid = threadIdx.x;
    const int nch = ri.nch;
    const float s = g.idx_scale;
    const unsigned long long* chist = ws.chist + (size_t)ri.lrow * ws.nchunk * kCB;
    const uint32_t* cmax = ws.cmax + (size_t)ri.lrow * ws.nchunk;
    // one round of loads: the chunk's maximum and total mass (one chunk per
    // thread, nch <= 256) and p
    const uint32_t cm = tid < nch ? cmax[tid] : 0u;
    const unsigned long long ztot = tid < nch ? chist[(size_t)tid * kCB + kCB - 1] : 0ull;
    const float p = top_p[ri.b];
    uint32_t mk = wave_max_u32(cm);
    if ((tid & 63) == 0) ured[tid >> 6] = mk;
    if (tid == 0) {
        s_k[0] = kGB;
        s_k[1] = 16;
    }
    __syncthreads();
    mk = max(max(ured[0], ured[1]), max(ured[2], ured[3]));
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
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
    if ((tid & 63) == 0) dred[tid >> 6] = z;
    __syncthreads();
    const double Z = dred[0] + dred[1] + dred[2] + dred[3];
    pl.all = !(p < 1.0f);
    unsigned long long target = (unsigned long long)ceil((double)p * Z);
    if ((double)target > Z) target = (unsigned long long)Z;
    if (target < 1ull) target = 1ull;
    pl.target = target;
    pl.d_thr = -INFINITY;
    pl.ks = kGB;
    if (pl.all) return pl;
    // LB(k) is non-decreasing in k: first at the 16 points k = 16 i + 15, then
    // at the 16 values up to the first point that reaches.  16 lanes share one
    // k (chunk bin b counts once (b + 1) / 4 + dc <= k / 4).
    const double need = (double)target * (1.0 + 0x1.0p-40) + (double)ri.L + 1.0;
    const int grp = tid >> 4, sub = tid & 15;
    const auto lb_reaches = [&](int k) {
        double lb = 0.0;
        for (int c = sub; c < nch; c += 16) {
            const double bmax = floor((double)(k - 1) - (double)kCBPerUnit * dch[c]);
            if (bmax >= 0.0) lb += fch[c] * (double)chist[(size_t)c * kCB + (int)fmin(bmax, (double)(kCB - 1))];
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) lb += __shfl_xor(lb, o);
        return sub == 0 && lb >= need;
    };
    if (lb_reaches(16 * grp + 15)) atomicMin(&s_k[1], grp);
    __syncthreads();
    const int ic = s_k[1];
    if (ic < 16 && lb_reaches(16 * ic + grp)) atomicMin(&s_k[0], 16 * ic + grp);
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

// Gather.  grid (nchunk, rows), 256 threads: the row's plan, then the chunk's
// keys of U written at the chunk's place in the row's index-ordered list.
// The first chunk's workgroup records the plan and the size of U.
__global__ __launch_bounds__(256) void k_sel_gather(Geo g, const float* __restrict__ top_p, int row0, SelWs ws) {
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    if (chunk >= ri.nch) return;
    __shared__ double fch[kMaxChunks], dch[kMaxChunks];
    __shared__ double dred[4];
    __shared__ uint32_t ured[4];
    __shared__ int s_k[2];
    __shared__ unsigned long long scan_sh[256 / 64 + 1];
    __shared__ uint32_t s_base;
    // the chunk's scores, loaded while the plan is formed
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int j0 = chunk * kChunk + 16 * tid;             // 16 consecutive keys per thread
    float dv[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float4 v = *reinterpret_cast<const float4*>(srow + j0 + 4 * u);
        dv[4 * u] = v.x;
        dv[4 * u + 1] = v.y;
        dv[4 * u + 2] = v.z;
        dv[4 * u + 3] = v.w;
    }
    const Plan pl = row_plan(g, ri, ws, top_p, fch, dch, dred, ured, s_k);
    if (pl.all) {
        if (chunk == 0 && tid == 0) {
            RowState st;
            st.m = pl.m;
            st.L = ri.L;
            st.Tkey = 0u;
            st.jT = ri.L;
            st.target = pl.target;
            st.d_thr = pl.d_thr;
            st.mode = 0;
            st.count = ri.L;
            ws.st[ri.lrow] = st;
        }
        return;
    }
    // U: in chunk c, the keys whose chunk bin is at most bsel(c) = ks + 1 - 4 dc
    // (a quarter unit beyond the bins that LB(ks) counts, so U holds every key
    // with s (m - d) < ks / 4 and the cut lies inside it).  The cumulative
    // counts give every chunk's share of U, hence its place in the index-ordered
    // list, without atomics.
    const unsigned* ccnt = ws.ccnt + (size_t)ri.lrow * ws.nchunk * kCB;
    const auto bsel = [&](int c) {
        return pl.ks >= kGB ? kCB - 1 : (int)fmin(floor((double)(pl.ks + 1) - (double)kCBPerUnit * dch[c]), (double)(kCB - 1));
    };
    unsigned long long cnt_c = 0ull;
    if (tid < ri.nch) {
        const int b = bsel(tid);
        cnt_c = b >= 0 ? (unsigned long long)ccnt[(size_t)tid * kCB + b] : 0ull;
    }
    unsigned long long nU;
    const unsigned long long off_c = block_excl_scan_u64<256>(cnt_c, &nU, scan_sh);
    if (tid == chunk) s_base = (uint32_t)off_c;
    if (chunk == 0 && tid == 0) {
        RowState st;
        st.m = pl.m;
        st.L = ri.L;
        st.Tkey = 0u;
        st.jT = ri.L;
        st.target = pl.target;
        st.d_thr = pl.d_thr;
        st.mode = 1;
        st.count = 0;
        ws.st[ri.lrow] = st;
        ws.row_n[ri.lrow] = (uint32_t)nU;                 // at most 2^20
    }
    if (nU > (unsigned long long)kCand) return;           // the row takes the long path
    const int bmine = bsel(chunk);
    if (bmine < 0) return;
    const float mc = key_score(ws.cmax[(size_t)ri.lrow * ws.nchunk + chunk]);
    const float s = g.idx_scale;
    uint32_t inU = 0u, c = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const bool in = j0 + e < ri.L && (weight_bin(dv[e], mc, s).bin >> 4) <= bmine;
        inU |= in ? 1u << e : 0u;
        c += in ? 1u : 0u;
    }
    __syncthreads();
    unsigned long long tot;
    uint32_t o = s_base + (uint32_t)block_excl_scan_u64<256>(c, &tot, scan_sh);
    unsigned long long* ub = ws.ubuf + (size_t)ri.lrow * kCand;
#pragma unroll
    for (int e = 0; e < 16; ++e)
        if (inU & (1u << e))
            ub[o++] = ((unsigned long long)score_key(dv[e]) << 32) | (unsigned long long)(~(uint32_t)(j0 + e));
}

// Cut among a candidate list held in LDS (cand = (score key << 32) | ~index,
// wgt = exact fixed-point weights): radix levels of 2048 buckets with exact
// masses; once the cut bucket holds at most 64 keys, one wavefront sorts them
// in registers (score key descending, index ascending) and finds the first
// whose cumulative mass reaches the target.
__device__ Cut list_cut(const unsigned long long* cand, const unsigned long long* wgt, int n, const float* srow,
                        int L, uint32_t klo, uint32_t khi, unsigned long long target, float m, float s,
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
            atomicAdd(&hmb[bk], wgt[i]);
            atomicAdd(&hcb[bk], 1u);
        }
        __syncthreads();
        const unsigned long long loc = hmb[2 * tid] + hmb[2 * tid + 1];
        unsigned long long tot;
        const unsigned long long ex = S_hi + block_excl_scan_u64<kRT>(loc, &tot, scan_sh);
        if (tid == 0) *s_i = kNR;
        __syncthreads();
        if (ex + hmb[2 * tid] >= target && hcb[2 * tid]) atomicMin(s_i, 2 * tid);
        else if (ex + loc >= target && hcb[2 * tid + 1]) atomicMin(s_i, 2 * tid + 1);
        __syncthreads();
        const int nb = (int)(span >> shift) + 1;
        int bk = *s_i;
        if (bk < kNR && (bk >> 1) == tid) {
            *s_S = (bk & 1) ? ex + hmb[2 * tid] : ex;
            *s_u = hcb[bk];
        }
        if (bk >= kNR && tid == 0) {
            *s_S = S_hi + tot - hmb[nb - 1];
            *s_u = hcb[nb - 1];
        }
        if (bk >= kNR) bk = nb - 1;
        __syncthreads();
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
                    small_w[slot] = wgt[i];
                }
            }
            __syncthreads();
            if (tid < 64) {
                const int nbk = (int)min(*s_u, 64u);
                unsigned long long v = lane < nbk ? small_v[lane] : 0ull;
                unsigned long long w = lane < nbk ? small_w[lane] : 0ull;
#pragma unroll
                for (int k = 2; k <= 64; k <<= 1)
#pragma unroll
                    for (int j = k >> 1; j > 0; j >>= 1) {
                        const unsigned long long ov = __shfl_xor(v, j), ow = __shfl_xor(w, j);
                        const bool desc = (lane & k) == 0 || k == 64;
                        const bool lower = (lane & j) == 0;
                        const bool take = desc == lower ? ov > v : ov < v;
                        if (take) {
                            v = ov;
                            w = ow;
                        }
                    }
                unsigned long long incl = w;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const unsigned long long y = __shfl_up(incl, o);
                    if (lane >= o) incl += y;
                }
                const unsigned long long reach = __ballot(lane < nbk && S_hi + incl >= target);
                const int ic = reach ? __ffsll((long long)reach) - 1 : nbk - 1;
                const unsigned long long vc = __shfl(v, ic);
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
            const unsigned long long wT = weight_bin(key_score(klo), m, s).w;
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

// Resolve.  One 1024-thread workgroup per row: U with its exact weights, the
// cut, and the selected indices in order (a list that did not fit: the cut
// over the row's scores and per-chunk counts).
__global__ __launch_bounds__(kRT) void k_sel_resolve(Geo g, int row0, SelWs ws) {
    const int tid = threadIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.x);
    RowState st = ws.st[ri.lrow];
    if (st.mode == 0) return;
    __shared__ unsigned long long cand[kCand];
    __shared__ unsigned long long wgt[kCand];
    __shared__ unsigned long long scan_sh[kRT / 64 + 1];
    __shared__ unsigned long long hmb[kNR];
    __shared__ uint32_t hcb[kNR];
    __shared__ uint32_t ccount[kMaxChunks];
    __shared__ unsigned long long small_v[64], small_w[64];
    __shared__ Cut s_cut;
    __shared__ int s_i;
    __shared__ uint32_t s_n;
    __shared__ unsigned long long s_S;
    const float s = g.idx_scale;
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int nch = ri.nch;
    const float m = st.m, d_thr = st.d_thr;
    const unsigned long long target = st.target;
    const int lane = tid & 63;
    const int nU = (int)ws.row_n[ri.lrow];
    const uint32_t klo = d_thr == -INFINITY ? 0u : score_key(d_thr), khi = score_key(m);
    const auto selected_by = [](const Cut& c, uint32_t key, int j) { return key > c.Tkey || (key == c.Tkey && j <= c.jT); };
    if (nU <= kCand) {
        const unsigned long long* ub = ws.ubuf + (size_t)ri.lrow * kCand;
        for (int i = tid; i < nU; i += kRT) {
            const unsigned long long e = ub[i];
            cand[i] = e;
            wgt[i] = weight_bin(key_score((uint32_t)(e >> 32)), m, s).w;
        }
        __syncthreads();
        const Cut cut = list_cut(cand, wgt, nU, srow, ri.L, klo, khi, target, m, s, hmb, hcb, scan_sh, &s_n, &s_S,
                                 &s_i, small_v, small_w, &s_cut);
        // U is in index order: its selected entries, in order, into the row's list
        constexpr int per = kCand / kRT;
        uint32_t c = 0;
#pragma unroll
        for (int x = 0; x < per; ++x) {
            const int i = tid * per + x;
            if (i < nU && selected_by(cut, (uint32_t)(cand[i] >> 32), (int)~(uint32_t)cand[i])) ++c;
        }
        unsigned long long tot2;
        uint32_t o = (uint32_t)block_excl_scan_u64<kRT>(c, &tot2, scan_sh);
        uint32_t* sl = ws.sel + (size_t)ri.lrow * kCand;
#pragma unroll
        for (int x = 0; x < per; ++x) {
            const int i = tid * per + x;
            if (i < nU) {
                const int j = (int)~(uint32_t)cand[i];
                if (selected_by(cut, (uint32_t)(cand[i] >> 32), j)) sl[o++] = (uint32_t)j;
            }
        }
        if (tid == 0) {
            st.mode = 1;
            st.Tkey = cut.Tkey;
            st.jT = cut.jT;
            st.count = (int32_t)tot2;
            ws.st[ri.lrow] = st;
        }
        return;
    }
    // ---- U too large for LDS: the cut over the row's scores, selected keys per
    // chunk for the ordered compaction
    for (int c = tid; c < kMaxChunks; c += kRT) ccount[c] = 0u;
    const Cut cut = radix_cut(cand, -1, srow, ri.L, klo, khi, 0ull, target, m, s, hmb, hcb, scan_sh, &s_n, &s_S,
                              &s_i);
    for (int j = tid; j < ri.L; j += kRT) {
        const bool sel = selected_by(cut, score_key(srow[j]), j);
        const unsigned long long b = __ballot(sel);
        if (lane == 0 && b) atomicAdd(&ccount[j / kChunk], (uint32_t)__popcll(b));
    }
    __syncthreads();
    unsigned long long n_c = tid < nch ? ccount[tid] : 0ull;
    unsigned long long tot;
    const unsigned long long ex = block_excl_scan_u64<kRT>(n_c, &tot, scan_sh);
    if (tid < nch) ws.chunk_cnt[(size_t)ri.lrow * ws.nchunk + tid] = (uint32_t)ex;
    if (tid == 0) {
        st.mode = 2;
        st.Tkey = cut.Tkey;
        st.jT = cut.jT;
        st.count = (int32_t)tot;
        ws.st[ri.lrow] = st;
    }
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
    if (tid == 0 && carry > out.capacity) *out.status = 1;
}

// ---------------------------------------------------------------------------
// Emit.  grid (min(nchunk, kEmitWG), rows), 256 threads: workgroup x writes the
// parts of a row's output that belong to 4096-key chunks x, x + kEmitWG, ...
// (slices of the ordered list, or the ordered compaction of a chunk's selected
// keys).  ROWPTR: the group is small, so every workgroup sums the counts before
// its row itself; the first one writes the row pointer and checks the capacity.
// ---------------------------------------------------------------------------
constexpr int kEmitWG = 4;

template <int ROWPTR>
__global__ __launch_bounds__(256) void k_sel_emit(Geo g, int row0, SelWs ws, SelOut out) {
    const int tid = threadIdx.x;
    const int first = blockIdx.x;
    const RowInfo ri = row_info(g, row0, blockIdx.y);
    const RowState st = ws.st[ri.lrow];
    if (first >= ri.nch) return;
    if (first > 0 && st.mode == 1 && first * kChunk >= st.count) return;   // nothing of this row here
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
    __shared__ uint32_t wcnt[4];
    const float* srow = ws.scores + (size_t)ri.lrow * ws.score_ld;
    const int lane = tid & 63, wid = tid >> 6;
    for (int chunk = first; chunk < ri.nch; chunk += gridDim.x) {
        const int jbase = chunk * kChunk;
        if (st.mode == 0) {
            for (int k = tid; k < kChunk && jbase + k < ri.L; k += 256) out.idx[rbase + jbase + k] = jbase + k;
            continue;
        }
        if (st.mode == 1) {
            if (jbase >= st.count) break;
            const uint32_t* sl = ws.sel + (size_t)ri.lrow * kCand;
            for (int k = tid; k < kChunk && jbase + k < st.count; k += 256)
                out.idx[rbase + jbase + k] = (int32_t)sl[jbase + k];
            continue;
        }
        int64_t base = rbase + ws.chunk_cnt[(size_t)ri.lrow * ws.nchunk + chunk];
        float dv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) dv[k] = srow[min(jbase + k * 256 + tid, ri.L - 1)];
        for (int k = 0; k < 16; ++k) {
            if (jbase + k * 256 >= ri.L) break;
            const int j = jbase + k * 256 + tid;
            bool sel = false;
            if (j < ri.L) {
                const uint32_t key = score_key(dv[k]);
                sel = key > st.Tkey || (key == st.Tkey && j <= st.jT);
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
}

}  // namespace

hipError_t launch_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                         const float* top_p, int row0, const SelWs& ws, const SelOut& out,
                         int total_rows, int dtype, int stage, hipStream_t s) {
    (void)total_rows;
    const dim3 grid(ws.nchunk, ws.rows);
    const bf16_t* kl = (const bf16_t*)k_low;
    const bool scores_only = stage == kSelScoresOnly;
    if (stage != kSelFinish) {
        if (dtype == 0 && scores_only)
            hipLaunchKernelGGL((k_sel_score<float, 0>), grid, dim3(256), 0, s, g, (const float*)q, (const float*)w_q,
                               kl, row0, ws, out);
        else if (dtype == 0)
            hipLaunchKernelGGL((k_sel_score<float, 1>), grid, dim3(256), 0, s, g, (const float*)q, (const float*)w_q,
                               kl, row0, ws, out);
        else if (scores_only)
            hipLaunchKernelGGL((k_sel_score<bf16_t, 0>), grid, dim3(256), 0, s, g, (const bf16_t*)q,
                               (const bf16_t*)w_q, kl, row0, ws, out);
        else
            hipLaunchKernelGGL((k_sel_score<bf16_t, 1>), grid, dim3(256), 0, s, g, (const bf16_t*)q,
                               (const bf16_t*)w_q, kl, row0, ws, out);
    }
    if (scores_only || stage == kSelScorePass) return hipGetLastError();
    hipLaunchKernelGGL(k_sel_gather, grid, dim3(256), 0, s, g, top_p, row0, ws);
    hipLaunchKernelGGL(k_sel_resolve, dim3(ws.rows), dim3(kRT), 0, s, g, row0, ws);
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
