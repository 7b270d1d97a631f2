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
// 16-wide contraction of a 32-row x 32-key tile is one
// v_mfma_f32_32x32x16_bf16.  The MFMA sum is not the fixed-order chain, but
// it lies within delta = 2^-16 |q_low| max|k_low| of it (the chain's own
// rounding is at most ~2^-20 sum|q_c k_c| and the measured MFMA deviation is
// below 2^-21 sum|q_c k_c|), so
//   * the row maximum is bounded by m' = max(MFMA score) + delta;
//   * an approximate mass histogram over MFMA scores locates the cut, with the
//     target raised by a margin that covers the approximation; every key that
//     can rank above the exact cut lies in the set U of keys whose approximate
//     bin is at most one past that cut bin (bins are 1 / (2 s) wide in score,
//     far wider than delta);
//   * exact scores and exact fixed-point masses are computed for U only and
//     refined by radix levels on the exact score until the cut is resolved;
//   * keys outside U enter the total mass with their approximate weights
//     (they hold at most the 1 - p tail, so the relative error of the
//     cumulative mass stays far inside 1e-6).
// Kernels: main (passes + resolve, one workgroup per 32 rows of one head),
// row pointers, emit (ordered, exact near the cut, ties by lowest index).
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTR = 32;          // rows per workgroup
constexpr int kNB = 64;          // bins per histogram level
constexpr int kCapC = 128;       // exact candidates resolved by one sort per row
constexpr int kQ = 64;           // exact-work queue length per wave
constexpr float kBin1 = 2.0f;    // level-1 bins per unit of x = s (m' - e)
constexpr float kLog2eF = 1.4426950408889634f;

// Per-row result of the main kernel (device workspace).
struct CRow {
    float mp;        // m' (upper bound of the row's exact maximum)
    float delta;     // |MFMA - exact| bound of the row
    float T;         // exact score of the cut
    int mode;        // 0 keep all, 1 all of U, 2 threshold
    int u_end;       // last level-1 bin of U
    int n_tie;       // keys with d == T taken (lowest indices)
    int count;       // selected keys
    int pad;
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

// approximate weight in fixed point: exp(-x) * 2^43 (x >= 0), truncated
__device__ __forceinline__ unsigned long long approx_w(float x) {
    const float f = exp2f(-x * kLog2eF) * 8796093022208.0f;
    if (!(f >= 1.0f)) return 0ull;
    const uint32_t u = __float_as_uint(f);
    const int e = (int)(u >> 23) - 150;
    const unsigned long long m = (u & 0x7FFFFFu) | 0x800000u;
    return e >= 0 ? (m << e) : (m >> (-e));
}

__device__ __forceinline__ int bin1_of(float x) {
    return (int)fminf(x * kBin1, (float)(kNB - 1));
}

struct Tile {
    int page_off;    // element offset of the tile's first key row in k_low
};

// ---------------------------------------------------------------------------
// Main kernel.  grid (ceil(n_tok / 32), n_ret), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_csel_main(Geo g, const bf16_t* __restrict__ q,
                                                   const bf16_t* __restrict__ w_q,
                                                   const bf16_t* __restrict__ k_low,
                                                   const float* __restrict__ top_p, CRow* __restrict__ rows_out,
                                                   uint16_t* __restrict__ qlow_out) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r = blockIdx.y;
    const int t0 = blockIdx.x * kTR;
    const int n_valid = min(kTR, g.n_tok - t0);
    const int h_q = g.ret_heads[r];
    const float s = g.idx_scale;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;

    __shared__ float qs[kTR][16];                       // q_low as floats
    __shared__ unsigned long long hm[kTR][kNB];
    __shared__ uint32_t hc[kTR][kNB];
    __shared__ unsigned long long cand[kTR][kCapC];
    __shared__ uint32_t cand_n[kTR];
    __shared__ uint32_t rmax[kTR];                       // ordered keys of the row maxima
    __shared__ uint32_t kmax_bits;
    __shared__ unsigned long long zu[kTR];               // exact mass of U
    // per-row refinement state
    __shared__ float r_mp[kTR], r_delta[kTR], r_T[kTR];
    __shared__ int r_mode[kTR], r_uend[kTR], r_ntie[kTR], r_done[kTR], r_gather[kTR];
    __shared__ uint32_t r_klo[kTR], r_khi[kTR], r_shift[kTR], r_cnthi[kTR];
    __shared__ unsigned long long r_shi[kTR], r_target[kTR], r_zlight[kTR];
    __shared__ int s_any;
    __shared__ uint32_t qpair[4][kQ];                    // per-wave exact-work queue: (row << 26) | key

    // ---- q_low of the 32 rows: fixed-order fp32 chain over d, bf16 rounding
    {
        __shared__ float wq[128 * 16];
        const bf16_t* wp = w_q + (size_t)r * g.D * 16;
        for (int x = tid; x < g.D * 16; x += 256) wq[x] = bf2f(wp[x]);
        __syncthreads();
        for (int o = tid; o < kTR * 16; o += 256) {
            const int lr = o >> 4, c = o & 15;
            float acc = 0.0f;
            if (lr < n_valid) {
                const bf16_t* qp = q + ((size_t)(t0 + lr) * g.Hq + h_q) * g.D;
                for (int d = 0; d < g.D; ++d) acc = __builtin_fmaf(bf2f(qp[d]), wq[d * 16 + c], acc);
            }
            const bf16_t qb = f2bf(acc);
            qs[lr][c] = bf2f(qb);
            if (lr < n_valid) qlow_out[((size_t)(t0 + lr) * g.n_ret + r) * 16 + c] = qb;
        }
        for (int x = tid; x < kTR * kNB; x += 256) {
            (&hm[0][0])[x] = 0ull;
            (&hc[0][0])[x] = 0u;
        }
        if (tid < kTR) {
            rmax[tid] = 0u;
            zu[tid] = 0ull;
            cand_n[tid] = 0u;
        }
        if (tid == 0) kmax_bits = 0u;
        __syncthreads();
    }

    // lane roles in the MFMA tiles: row lr = lane % 32, half hh = lane / 32
    const int lr = lane & 31, hh = lane >> 5;
    const bool row_ok = lr < n_valid;
    const int pos = g.pos0 + t0 + lr;                    // the lane's row position
    uint4 qb;                                             // B operand: q_low[lr][8 hh .. 8 hh + 7]
    {
        uint32_t w4[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
            w4[x] = (__float_as_uint(qs[lr][8 * hh + 2 * x]) >> 16) | (__float_as_uint(qs[lr][8 * hh + 2 * x + 1]) & 0xFFFF0000u);
        qb = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    const int L_max = g.pos0 + t0 + n_valid;             // keys of the longest row
    const int ntile = (L_max + 31) / 32;

    // load the A operand of tile `it`: k_low[key it*32 + lr][8 hh .. 8 hh + 7]
    auto load_a = [&](int it) {
        const int key = it * 32 + lr;
        const int kk = min(key, L_max - 1);
        const int page = bt[kk >> 8];
        return *reinterpret_cast<const uint4*>(
            k_low + (((size_t)page * g.n_ret + r) * kBlk + (kk & 255)) * 16 + 8 * hh);
    };
    auto mfma_tile = [&](const uint4& a) {
        f32x16_t acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qb), acc, 0, 0, 0);
    };
    auto key_of = [&](int it, int i) { return it * 32 + (i >> 2) * 8 + 4 * hh + (i & 3); };

    // ---- pass 1: row maxima of the MFMA scores, largest key norm
    {
        float m_e = -INFINITY, kn = 0.0f;
        uint4 a = ntile > wid ? load_a(wid) : make_uint4(0, 0, 0, 0);
        for (int it = wid; it < ntile; it += 4) {
            const uint4 cur = a;
            if (it + 4 < ntile) a = load_a(it + 4);
            float kf[8];
            unpack8(cur, kf);
            float n2 = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) n2 = __builtin_fmaf(kf[e], kf[e], n2);
            n2 += __shfl_xor(n2, 32);
            kn = fmaxf(kn, n2);
            const f32x16_t sc = mfma_tile(cur);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key_of(it, i) <= pos) m_e = fmaxf(m_e, sc[i]);
        }
        m_e = fmaxf(m_e, __shfl_xor(m_e, 32));
        kn = wave_max(kn);
        if (row_ok && hh == 0 && m_e > -INFINITY) atomicMax(&rmax[lr], score_key(m_e));
        if (lane == 0) atomicMax(&kmax_bits, __float_as_uint(kn));
        __syncthreads();
        if (tid < kTR) {
            float qn2 = 0.0f;
            for (int c = 0; c < 16; ++c) qn2 = __builtin_fmaf(qs[tid][c], qs[tid][c], qn2);
            const float delta = 0x1.0p-16f * sqrtf(qn2) * sqrtf(__uint_as_float(kmax_bits)) * 1.0009765625f;
            // delta exceeds the true deviation bound by a factor >= 8, far more
            // than the rounding of this sum: m' >= every exact score of the row
            r_mp[tid] = key_score(rmax[tid]) + delta;
            r_delta[tid] = delta;
        }
        __syncthreads();
    }
    const float mp = r_mp[lr];
    const float delta = r_delta[lr];

    // ---- pass 2: approximate level-1 mass histogram (mass only)
    {
        uint4 a = ntile > wid ? load_a(wid) : make_uint4(0, 0, 0, 0);
        for (int it = wid; it < ntile; it += 4) {
            const uint4 cur = a;
            if (it + 4 < ntile) a = load_a(it + 4);
            const f32x16_t sc = mfma_tile(cur);
            if (row_ok) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (key_of(it, i) <= pos) {
                        const float x = s * (mp - sc[i]);
                        atomicAdd(&hm[lr][bin1_of(x)], approx_w(x));
                    }
                }
            }
        }
        __syncthreads();
        // cut bin of the approximate masses, U = bins <= cut + 1.  The target
        // carries a margin eta that covers the relative error of the
        // approximate weights (|s (MFMA - exact)| <= s delta / 8) and their
        // fixed-point truncation; U is everything when the bins are not wide
        // against delta.
        if (tid < kTR) {
            const int row = tid;
            const float p = top_p[g.seq];
            r_mode[row] = 2;
            r_done[row] = 0;
            r_gather[row] = 0;
            r_uend[row] = kNB - 1;
            if (row >= n_valid) {
                r_done[row] = 1;
            } else if (!(p < 1.0f)) {
                r_mode[row] = 0;
                r_done[row] = 1;
            } else {
                const double sd = (double)s * (double)r_delta[row];
                unsigned long long Z = 0;
                for (int b = 0; b < kNB; ++b) Z += hm[row][b];
                const double tgt_a = (double)p * (1.0 + sd + 0x1.0p-16) * (double)Z;
                int bc = kNB - 1;
                unsigned long long cum = 0;
                for (int b = 0; b < kNB; ++b) {
                    cum += hm[row][b];
                    if ((double)cum >= tgt_a) {
                        bc = b;
                        break;
                    }
                }
                const int ue = (sd < 1.0 / 16.0) ? min(bc + 1, kNB - 1) : kNB - 1;
                unsigned long long zl = 0;
                for (int b = ue + 1; b < kNB; ++b) zl += hm[row][b];
                r_uend[row] = ue;
                r_zlight[row] = zl;
                // first exact level: the whole key range of U in exact-score space
                // (keys of U have MFMA scores above m' - (ue + 1) / (2 s), exact
                // scores within delta of them)
                if (ue == kNB - 1) {
                    r_klo[row] = 0u;
                } else {
                    const double dlo = (double)r_mp[row] - (double)(ue + 1) / ((double)kBin1 * (double)s) * 1.001 -
                                       2.0 * (double)r_delta[row];
                    r_klo[row] = score_key(__double2float_rd(dlo));
                }
                r_khi[row] = score_key(r_mp[row]);
                const uint32_t span = r_khi[row] - r_klo[row];
                const int bits = span ? 32 - __clz(span) : 0;
                r_shift[row] = bits > 6 ? bits - 6 : 0;
                r_shi[row] = 0ull;
                r_cnthi[row] = 0u;
            }
        }
        __syncthreads();
    }
    const int u_end = r_uend[lr];

    // ---- exact levels: radix on the order-preserving key of the exact score
    // of U's keys, 64 buckets per level, highest scores first; then one gather
    // pass collects the cut bucket's keys for the final sort.
    for (int level = 0; level < 8; ++level) {
        // clear the level histograms
        for (int x = tid; x < kTR * kNB; x += 256) {
            (&hm[0][0])[x] = 0ull;
            (&hc[0][0])[x] = 0u;
        }
        if (tid == 0) s_any = 0;
        __syncthreads();
        if (tid < kTR && !r_done[tid]) s_any = 1;
        __syncthreads();
        if (!s_any) break;

        uint4 a = ntile > wid ? load_a(wid) : make_uint4(0, 0, 0, 0);
        int qbase = 0;                                    // wave-uniform queue fill
        // process the queued pairs of this wave: exact score, then either a
        // histogram update (level pass) or a gather into the candidates
        auto drain = [&](int n) {
            wave_lds_sync();
            if (lane < n) {
                const uint32_t e = qpair[wid][lane];
                const int row = (int)(e >> 26), key = (int)(e & 0x3FFFFFFu);
                const int page = bt[key >> 8];
                const uint4* kp = reinterpret_cast<const uint4*>(
                    k_low + (((size_t)page * g.n_ret + r) * kBlk + (key & 255)) * 16);
                const float d = exact_score(qs[row], kp[0], kp[1]);
                const uint32_t kd = score_key(d);
                if (r_gather[row]) {
                    if (kd >= r_klo[row] && kd <= r_khi[row]) {
                        const uint32_t slot = atomicAdd(&cand_n[row], 1u);
                        if (slot < (uint32_t)kCapC)
                            cand[row][slot] = ((unsigned long long)kd << 32) | (unsigned long long)(~(uint32_t)key);
                    }
                } else {
                    const unsigned long long w = weight_bin(d, r_mp[row], s).w;
                    if (level == 0) atomicAdd(&zu[row], w);
                    if (kd > r_khi[row]) {
                        // above the range: counted by earlier levels
                    } else if (kd >= r_klo[row]) {
                        const uint32_t bk = min((r_khi[row] - kd) >> r_shift[row], (uint32_t)(kNB - 1));
                        atomicAdd(&hm[row][bk], w);
                        atomicAdd(&hc[row][bk], 1u);
                    }
                    // below the range: ranks below the cut, mass already in zu
                }
            }
            wave_lds_sync();
        };
        for (int it = wid; it < ntile; it += 4) {
            const uint4 cur = a;
            if (it + 4 < ntile) a = load_a(it + 4);
            const f32x16_t sc = mfma_tile(cur);
            // which of this lane's pairs need an exact score
            uint32_t need = 0;
            if (row_ok && !r_done[lr]) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (key_of(it, i) > pos) continue;
                    const float x = s * (mp - sc[i]);
                    if (bin1_of(x) > u_end) continue;        // not in U
                    if (r_gather[lr] || level > 0) {
                        // only pairs whose exact score can fall inside [klo, khi]
                        const float lo = key_score(r_klo[lr]), hi = key_score(r_khi[lr]);
                        if (sc[i] + delta < lo || sc[i] - delta > hi) continue;
                    }
                    need |= 1u << i;
                }
            }
            // append to the wave queue in order, draining when full
            int cnt = __popc(need);
            int pre = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(pre, o);
                if (lane >= o) pre += y;
            }
            const int total = __shfl(pre, 63);
            pre -= cnt;
            int base = qbase;
            if (base + total > kQ) {
                drain(base);
                base = 0;
            }
            // total <= 64 * 16 may exceed the queue: spill in rounds of kQ
            int done = 0;
            while (done < total) {
                const int take = min(kQ - base, total - done);
                // lanes write their pairs with ordinal in [done, done + take)
                uint32_t m = need;
                int ord = pre;
                while (m) {
                    const int i = __ffs(m) - 1;
                    m &= m - 1;
                    if (ord >= done && ord < done + take)
                        qpair[wid][base + ord - done] = ((uint32_t)lr << 26) | (uint32_t)key_of(it, i);
                    ++ord;
                }
                done += take;
                base += take;
                if (base == kQ) {
                    drain(kQ);
                    base = 0;
                }
            }
            qbase = base;
        }
        drain(qbase);
        __syncthreads();

        // per-row step: resolve, narrow, or switch to gathering
        if (tid < kTR) {
            const int row = tid;
            if (!r_done[row]) {
                const float p = top_p[g.seq];
                if (r_gather[row]) {
                    // final sort of the cut bucket's keys
                    r_done[row] = 1;
                } else {
                    if (level == 0) {
                        const unsigned long long Z = zu[row] + r_zlight[row];
                        unsigned long long tgt = (unsigned long long)ceil((double)p * (double)Z);
                        if (tgt < 1ull) tgt = 1ull;
                        r_target[row] = tgt;
                    }
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
                        // U does not reach the target (its mass is within rounding
                        // of p): every key of U is selected
                        r_mode[row] = 1;
                        r_done[row] = 1;
                        r_ntie[row] = 0;
                    } else {
                        r_shi[row] = cum;
                        r_cnthi[row] = ch;
                        const uint32_t khi = r_khi[row] - ((uint32_t)bc << r_shift[row]);
                        const uint32_t wdt = r_shift[row] >= 32 ? 0xFFFFFFFFu : ((1u << r_shift[row]) - 1u);
                        const uint32_t klo = (khi - r_klo[row] > wdt) ? khi - wdt : r_klo[row];
                        r_khi[row] = khi;
                        r_klo[row] = klo;
                        const uint32_t n_c = hc[row][bc];
                        if (klo == khi && n_c > (uint32_t)kCapC) {
                            // one score value with many keys: a tie group cut by index
                            const unsigned long long wT = weight_bin(key_score(khi), r_mp[row], s).w;
                            const unsigned long long need = r_target[row] - cum;
                            r_T[row] = key_score(khi);
                            r_ntie[row] = (int)((need + wT - 1ull) / wT);
                            r_mode[row] = 2;
                            r_done[row] = 1;
                            r_gather[row] = 2;               // resolved without candidates
                        } else if (n_c <= (uint32_t)kCapC) {
                            r_gather[row] = 1;
                            cand_n[row] = 0u;
                        } else {
                            const uint32_t span = khi - klo;
                            const int bits = span ? 32 - __clz(span) : 0;
                            r_shift[row] = bits > 6 ? bits - 6 : 0;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- final sort of each row's candidates and the per-row result
    if (wid == 0) {
        for (int row = 0; row < n_valid; ++row) {
            CRow out;
            out.mp = r_mp[row];
            out.delta = r_delta[row];
            out.u_end = r_uend[row];
            out.mode = r_mode[row];
            out.T = 0.0f;
            out.n_tie = 0;
            out.count = 0;                                    // counted by the emit pass
            out.pad = 0;
            if (out.mode == 2 && r_gather[row] == 2) {
                out.T = r_T[row];
                out.n_tie = r_ntie[row];
            } else if (out.mode == 2) {
                const int n = min((int)cand_n[row], kCapC);
                if (n == 0 || r_gather[row] != 1 || !r_done[row]) {
                    out.mode = 1;                             // unresolved: all of U
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
                    // cumulative exact mass in rank order; the lane holds ranks
                    // 2 lane and 2 lane + 1
                    const int i0 = 2 * lane, i1 = 2 * lane + 1;
                    const float mpr = r_mp[row];
                    const unsigned long long w0 =
                        i0 < n ? weight_bin(key_score((uint32_t)(cr[i0] >> 32)), mpr, s).w : 0ull;
                    const unsigned long long w1 =
                        i1 < n ? weight_bin(key_score((uint32_t)(cr[i1] >> 32)), mpr, s).w : 0ull;
                    unsigned long long incl = w0 + w1;
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) {
                        const unsigned long long y = __shfl_up(incl, o);
                        if (lane >= o) incl += y;
                    }
                    const unsigned long long c0 = r_shi[row] + incl - w1;   // through rank i0
                    const unsigned long long c1 = c0 + w1;                  // through rank i1
                    const unsigned long long tgt = r_target[row];
                    int first = 1 << 30;
                    if (i0 < n && c0 >= tgt) first = i0;
                    else if (i1 < n && c1 >= tgt) first = i1;
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o));
                    const int ic = first < n ? first : n - 1;
                    const uint32_t kT = (uint32_t)(cr[ic] >> 32);
                    int tie = 0;
                    if (i0 <= ic && (uint32_t)(cr[i0] >> 32) == kT) ++tie;
                    if (i1 <= ic && (uint32_t)(cr[i1] >> 32) == kT) ++tie;
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) tie += __shfl_xor(tie, o);
                    out.T = key_score(kT);
                    out.n_tie = tie;
                }
            }
            if (lane == 0) rows_out[(size_t)(t0 + row) * g.n_ret + r] = out;
            wave_lds_sync();
        }
    }
}

// ---------------------------------------------------------------------------
// Emit.  grid (ceil(n_tok / 32), n_ret), one wavefront: keys in index order,
// selected keys written ascending at row_ptr[row].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_csel_emit(Geo g, const bf16_t* __restrict__ k_low,
                                                  const uint16_t* __restrict__ qlow, const CRow* __restrict__ rows,
                                                  const int64_t* __restrict__ row_ptr, int32_t* __restrict__ idx,
                                                  int64_t capacity, const int32_t* __restrict__ status,
                                                  int* __restrict__ counts, int pass) {
    const int lane = threadIdx.x;
    const int r = blockIdx.y, t0 = blockIdx.x * kTR;
    const int n_valid = min(kTR, g.n_tok - t0);
    const int lr = lane & 31, hh = lane >> 5;
    const bool row_ok = lr < n_valid;
    const int row = (t0 + min(lr, n_valid - 1)) * g.n_ret + r;
    const int pos = g.pos0 + t0 + lr;
    if (pass == 1 && *status != 0) return;
    const CRow cr = rows[row];
    const float s = g.idx_scale;
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
    int64_t wpos = (pass == 1 && row_ok) ? row_ptr[row] : 0;
    int run_sel = 0, run_tie = 0;
    auto load_a = [&](int it) {
        const int kk = min(it * 32 + lr, L_max - 1);
        const int page = bt[kk >> 8];
        return *reinterpret_cast<const uint4*>(
            k_low + (((size_t)page * g.n_ret + r) * kBlk + (kk & 255)) * 16 + 8 * hh);
    };
    constexpr int kPre = 4;                               // tiles in flight
    uint4 ring[kPre];
#pragma unroll
    for (int x = 0; x < kPre; ++x) ring[x] = load_a(min(x, ntile - 1));
    for (int it0 = 0; it0 < ntile; it0 += kPre) {
#pragma unroll
    for (int x = 0; x < kPre; ++x) {
        const int it = it0 + x;
        if (it >= ntile) break;
        const uint4 a = ring[x];
        if (it + kPre < ntile) ring[x] = load_a(it + kPre);
        f32x16_t sc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = 0.0f;
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qb), sc, 0, 0, 0);
        uint32_t sel = 0, tie = 0;
        if (row_ok) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int kj = it * 32 + (i >> 2) * 8 + 4 * hh + (i & 3);
                if (kj > pos) continue;
                if (cr.mode == 0) {
                    sel |= 1u << i;
                    continue;
                }
                const float x = s * (cr.mp - sc[i]);
                if (bin1_of(x) > cr.u_end) continue;          // outside U
                if (cr.mode == 1) {
                    sel |= 1u << i;
                    continue;
                }
                if (sc[i] - cr.delta > cr.T) {
                    sel |= 1u << i;
                } else if (sc[i] + cr.delta >= cr.T) {
                    const int pg = bt[kj >> 8];
                    const uint4* kp = reinterpret_cast<const uint4*>(
                        k_low + (((size_t)pg * g.n_ret + r) * kBlk + (kj & 255)) * 16);
                    const float d = exact_score(q16, kp[0], kp[1]);
                    if (d > cr.T) sel |= 1u << i;
                    else if (d == cr.T) tie |= 1u << i;
                }
            }
        }
        // ties in index order: groups of four keys alternate between the halves
        uint32_t tc[4], tp[4];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) tc[gq] = __popc((tie >> (4 * gq)) & 0xFu);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) tp[gq] = __shfl_xor(tc[gq], 32);
        // ordinal of this lane's first tie in each of its groups
        int acc = run_tie;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int mine = hh ? (int)tp[gq] : 0;        // the partner's group comes first for hh = 1
            const int start = acc + mine;
            int o = start;
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
        // ordered write of the selected keys
        uint32_t sc4[4], sp4[4];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) sc4[gq] = __popc((sel >> (4 * gq)) & 0xFu);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) sp4[gq] = __shfl_xor(sc4[gq], 32);
        int accs = run_sel;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            int o = accs + (hh ? (int)sp4[gq] : 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * gq + e;
                if ((sel >> i) & 1u) {
                    if (pass == 1 && row_ok && wpos + o < capacity)
                        idx[wpos + o] = it * 32 + (i >> 2) * 8 + 4 * hh + (i & 3);
                    ++o;
                }
            }
            accs += (int)sc4[gq] + (int)sp4[gq];
        }
        run_sel = accs;
    }
    }
    if (pass == 0 && row_ok && hh == 0) counts[row] = run_sel;
}

// CSR row pointers over all rows of the call and the capacity check.
__global__ __launch_bounds__(1024) void k_csel_rowptr(const int* __restrict__ counts, int rows,
                                                      int64_t* __restrict__ row_ptr, int64_t capacity,
                                                      int32_t* __restrict__ status) {
    const int tid = threadIdx.x;
    __shared__ unsigned long long scan_sh[1024 / 64 + 1];
    int64_t carry = 0;
    if (tid == 0) row_ptr[0] = 0;
    for (int i0 = 0; i0 < rows; i0 += 1024) {
        const int i = i0 + tid;
        const unsigned long long c = i < rows ? (unsigned long long)counts[i] : 0ull;
        unsigned long long tot;
        const unsigned long long ex = block_excl_scan_u64<1024>(c, &tot, scan_sh);
        if (i < rows) row_ptr[i + 1] = carry + (int64_t)(ex + c);
        carry += (int64_t)tot;
    }
    if (tid == 0) *status = carry > capacity ? 1 : 0;
}

}  // namespace

size_t chunk_select_ws_bytes(int rows) {
    return ((size_t)rows * sizeof(CRow) + 255) / 256 * 256 + ((size_t)rows * 16 * 2 + 255) / 256 * 256 +
           ((size_t)rows * 4 + 255) / 256 * 256;
}

hipError_t launch_chunk_select(const Geo& g, const void* q, const void* w_q, const uint16_t* k_low,
                               const float* top_p, void* ws, const SelOut& out, hipStream_t s) {
    const int rows = g.n_tok * g.n_ret;
    char* base = (char*)ws;
    CRow* crow = (CRow*)base;
    base += ((size_t)rows * sizeof(CRow) + 255) / 256 * 256;
    uint16_t* qlow = (uint16_t*)base;
    base += ((size_t)rows * 16 * 2 + 255) / 256 * 256;
    int* counts = (int*)base;
    const dim3 grid((g.n_tok + kTR - 1) / kTR, g.n_ret);
    hipLaunchKernelGGL(k_csel_main, grid, dim3(256), 0, s, g, (const bf16_t*)q, (const bf16_t*)w_q,
                       (const bf16_t*)k_low, top_p, crow, qlow);
    // counting pass (rows of mode "all of U" are counted here too), row pointers, writing pass
    hipLaunchKernelGGL(k_csel_emit, grid, dim3(64), 0, s, g, (const bf16_t*)k_low, qlow, crow, out.row_ptr,
                       out.idx, out.capacity, out.status, counts, 0);
    hipLaunchKernelGGL(k_csel_rowptr, dim3(1), dim3(1024), 0, s, counts, rows, out.row_ptr, out.capacity,
                       out.status);
    hipLaunchKernelGGL(k_csel_emit, grid, dim3(64), 0, s, g, (const bf16_t*)k_low, qlow, crow, out.row_ptr,
                       out.idx, out.capacity, out.status, counts, 1);
    return hipGetLastError();
}

}  // namespace rtp
