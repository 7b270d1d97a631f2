// attn_decode.hip -- decode attention on gfx950: exact attention of retrieval
// heads over their gathered selected rows, and of local heads over sinks plus a
// sliding window (dense = a window covering the whole context).
//
// Method: arXiv 2605.16928 abstract (retrieval heads keep the full KV cache
// and attend sparsely; the others use a restricted window); zhichai.net forum
// post "RTPurbo: Turning Dense LLMs into Sparse Attention Models ...", "Three
// Key Insights" item 1.
//
// Flash-decoding on one wavefront per work item.  A key row (D elements) is
// read by a group of LPK lanes, 16 bytes each, so one load instruction reads
// 64/LPK whole rows (1 KiB, coalesced).  Each group runs its own online
// softmax over the keys it reads (q.k partials are summed across the group's
// lanes with DPP row operations; no LDS, no barriers in the loop); the groups
// of the wave are merged at the end, and a combine kernel merges the work
// items of a row in a fixed order, so results are deterministic.
#include <algorithm>
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "win_mfma.hpp"

namespace rtp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
struct Pack;                        // 16-byte vector of T unpacked to floats
template <>
struct Pack<bf16_t> {
    static constexpr int N = 8;
    __device__ static __forceinline__ void unpack(const uint4& a, float* f) {
        f[0] = __uint_as_float(a.x << 16); f[1] = __uint_as_float(a.x & 0xFFFF0000u);
        f[2] = __uint_as_float(a.y << 16); f[3] = __uint_as_float(a.y & 0xFFFF0000u);
        f[4] = __uint_as_float(a.z << 16); f[5] = __uint_as_float(a.z & 0xFFFF0000u);
        f[6] = __uint_as_float(a.w << 16); f[7] = __uint_as_float(a.w & 0xFFFF0000u);
    }
};
template <>
struct Pack<float> {
    static constexpr int N = 4;
    __device__ static __forceinline__ void unpack(const uint4& a, float* f) {
        f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
        f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    }
};
template <>
struct Pack<fp8e4_t> {              // FP8 K/V codes (their scales are applied outside)
    static constexpr int N = 16;
    __device__ static __forceinline__ void unpack(const uint4& a, float* f) {
        fp8x4_to_f32(a.x, f);
        fp8x4_to_f32(a.y, f + 4);
        fp8x4_to_f32(a.z, f + 8);
        fp8x4_to_f32(a.w, f + 12);
    }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPK lanes; every lane of a group gets the same
// bits (each step adds a value and its mirror image, which commutes).
template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
    if (LPK >= 2) v += dpp<0xB1>(v);      // quad_perm [1,0,3,2]
    if (LPK >= 4) v += dpp<0x4E>(v);      // quad_perm [2,3,0,1]
    if (LPK >= 8) v += dpp<0x141>(v);     // row_half_mirror
    if (LPK >= 16) v += dpp<0x140>(v);    // row_mirror
    if (LPK >= 32) v += __shfl_xor(v, 16);
    return v;
}


template <typename T, int D, int NH, int UR = (NH > 4 ? 4 : 8)>
struct Stream {
    static constexpr int EPV = Pack<T>::N;      // elements per lane slice
    static constexpr int LPK = D / EPV;         // lanes per key row
    static constexpr int GPW = 64 / LPK;        // key rows per load instruction
    static constexpr int U = UR;                // rows per group per iteration

    float q[NH][EPV];
    float m[NH], l[NH], o[NH][EPV];
    bool act[NH];                               // slot h in use (indexed with constants only)

    __device__ void init() {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            m[h] = -INFINITY;
            l[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) o[h][e] = 0.0f;
        }
    }

    // Keys 0..n-1 of a work item; off(i) is the element offset of key i's row
    // (valid for 0 <= i < n).  Group g of the wave takes keys g, g + GPW, ...
    template <typename F>
    __device__ void run(int n, F off, const T* __restrict__ kc, const T* __restrict__ vc) {
        run(n, off, kc, vc, [](int) { return ~0u; });
    }
    // The same, with msk(i): bit h set when key i is one of head slot h's keys.
    template <typename F, typename MK>
    __device__ void run(int n, F off, const T* __restrict__ kc, const T* __restrict__ vc, MK msk) {
        const int lane = threadIdx.x & 63;
        const int g = lane / LPK, sl = (lane % LPK) * EPV;
        for (int base = 0; base < n; base += GPW * U) {
            size_t ro[U];
#pragma unroll
            for (int u = 0; u < U; ++u) ro[u] = off(min(base + u * GPW + g, n - 1));
            uint4 kb[U], vb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) kb[u] = *reinterpret_cast<const uint4*>(kc + ro[u] + sl);
#pragma unroll
            for (int u = 0; u < U; ++u) vb[u] = *reinterpret_cast<const uint4*>(vc + ro[u] + sl);
            float s[U][NH];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[EPV];
                Pack<T>::unpack(kb[u], f);
                const bool ok = base + u * GPW + g < n;
                const uint32_t km = msk(min(base + u * GPW + g, n - 1));
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    float acc = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc = __builtin_fmaf(q[h][e], f[e], acc);
                    acc = group_sum<LPK>(acc);
                    s[u][h] = ok && ((km >> h) & 1u) ? acc : -INFINITY;
                }
            }
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                if (!act[h]) continue;
                float cm = s[0][h];
#pragma unroll
                for (int u = 1; u < U; ++u) cm = fmaxf(cm, s[u][h]);
                const float mn = fmaxf(m[h], cm);
                if (mn == -INFINITY) continue;           // the group has no key yet
                // raw v_exp_f32: its results below 2^-126 weigh nothing
                // against the running maximum's weight of 1
                const float corr = __builtin_amdgcn_exp2f(m[h] - mn);
                m[h] = mn;
                l[h] *= corr;
#pragma unroll
                for (int e = 0; e < EPV; ++e) o[h][e] *= corr;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float p = __builtin_amdgcn_exp2f(s[u][h] - mn);
                    l[h] += p;
                    float f[EPV];
                    Pack<T>::unpack(vb[u], f);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) o[h][e] = __builtin_fmaf(p, f[e], o[h][e]);
                }
            }
        }
    }

    // Merge the groups of the wave; afterwards lanes 0..LPK-1 hold head h's
    // output slices and every lane holds the merged (m, l).
    __device__ void merge() {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            if (!act[h]) continue;
            float M = m[h];
            for (int off = LPK; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
            const float sc = M == -INFINITY ? 0.0f : exp2f(m[h] - M);
            float L = l[h] * sc;
            for (int off = LPK; off < 64; off <<= 1) L += __shfl_xor(L, off);
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                float x = o[h][e] * sc;
                for (int off = LPK; off < 64; off <<= 1) x += __shfl_xor(x, off);
                o[h][e] = x;
            }
            m[h] = M;
            l[h] = L;
        }
    }

    __device__ void write(int h, float* pp) const {
        const int lane = threadIdx.x & 63;
        if (lane < LPK) {
            const int sl = lane * EPV;
#pragma unroll
            for (int e = 0; e < EPV; ++e) pp[sl + e] = o[h][e];
            if (lane == 0) {
                pp[D] = m[h];
                pp[D + 1] = l[h];
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Sparse decode: one wavefront per (row, piece of kItem selected keys); the
// pieces of all rows form one flat list walked by a fixed grid.
// ---------------------------------------------------------------------------
constexpr int kItem = kSparseItem;
static_assert(kItem % 64 == 0, "whole wavefronts of selected keys per item");

// Rows per group and iteration of the sparse kernels: a whole item's K and V
// rows are requested in one round (at most 16 row pairs per lane group).
template <typename TKV, int D>
constexpr int sparse_u() {
    return kItem * D / (64 * Pack<TKV>::N) < 16 ? kItem * D / (64 * Pack<TKV>::N) : 16;
}

template <typename T, typename TKV, int D>
__global__ __launch_bounds__(64) void k_sparse_dec_part(Geo g, const T* __restrict__ q,
                                                        const TKV* __restrict__ kc,
                                                        const TKV* __restrict__ vc,
                                                        const int64_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ status,
                                                        AttnWs ws, int row0, int rows) {
    using S = Stream<TKV, D, 1, sparse_u<TKV, D>()>;
    if (*status != 0) return;
    const int lane = threadIdx.x;
    extern __shared__ int64_t dyn[];
    int64_t* rp = dyn;                                    // rows + 1
    int32_t* istart = reinterpret_cast<int32_t*>(dyn + rows + 1);   // rows + 1
    __shared__ uint32_t joff[kItem];                      // page-resolved row offsets / D
    {   // pieces per row and their prefix (every workgroup recomputes it; rows <= 4096)
        for (int r = lane; r <= rows; r += 64) rp[r] = row_ptr[row0 + r];
        __syncthreads();
        const int per = (rows + 63) / 64;
        const int r0 = lane * per;
        int run = 0;
        for (int i = 0; i < per; ++i) {
            const int r = r0 + i;
            if (r < rows) run += (int)((rp[r + 1] - rp[r] + kItem - 1) / kItem);
        }
        int ex = (int)wave_incl_scan_u32((uint32_t)run);
        const int total = (int)lane_u32((uint32_t)ex, 63);
        ex -= run;
        for (int i = 0; i < per; ++i) {
            const int r = r0 + i;
            if (r < rows) {
                istart[r] = ex;
                ex += (int)((rp[r + 1] - rp[r] + kItem - 1) / kItem);
            }
        }
        if (lane == 0) istart[rows] = total;
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int r = lane; r <= rows; r += 64) ws.item_start[r] = istart[r];
    const int total = istart[rows];
    const float sc = g.attn_scale * kLog2e * g.k_scale;    // the K scale of FP8 codes folded into q
    constexpr int EPV = S::EPV, LPK = S::LPK;

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int lo = 0, hi = rows - 1;       // last row with istart <= item
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (istart[mid] <= item) lo = mid; else hi = mid - 1;
        }
        const int row = lo;
        const int grow = row0 + row;
        const int t = grow / g.n_ret, r = grow - t * g.n_ret;
        const int h = g.ret_heads[r], kvh = h / g.group;
        const int64_t k0 = rp[row] + (int64_t)(item - istart[row]) * kItem;
        const int n = (int)min<int64_t>(kItem, rp[row + 1] - k0);
        const int32_t* bt = g.block_table + (size_t)row_seq(g, t) * g.max_blocks;
        // resolve the item's rows once: index -> page -> row offset (in units of D)
        int jl[kItem / 64];
#pragma unroll
        for (int i = 0; i < kItem / 64; ++i) jl[i] = idx[k0 + min(lane + 64 * i, n - 1)];
        int pg[kItem / 64];
#pragma unroll
        for (int i = 0; i < kItem / 64; ++i) pg[i] = bt[jl[i] >> 8];
#pragma unroll
        for (int i = 0; i < kItem / 64; ++i)
            joff[lane + 64 * i] = (uint32_t)kv_rowidx(g, pg[i], kvh, jl[i] & 255);
        S st;
        st.init();
        const int sl = (lane % LPK) * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) st.q[0][e] = ld(q + ((size_t)t * g.Hq + h) * D + sl + e) * sc;
        __syncthreads();
        auto off = [&](int i) { return (size_t)joff[i] * D; };
        st.act[0] = true;
        st.run(n, off, kc, vc);
        st.merge();
        st.write(0, ws.part + (size_t)item * (D + 2));
        __syncthreads();
    }
}

// Merge the n partial results of a row (stride D + 2: output[D], max, sum) in
// item order on one wavefront: o[d] = sum_i 2^(m_i - M) o_i[d] / L * post.
// Lane l owns dims l, l + 64, ...; the partials are read 16 items per round.
template <typename T, int D>
__device__ void combine_wave(const float* __restrict__ base, int n, T* __restrict__ o, float post,
                             int stride = D + 2) {
    constexpr int DPL = D / 64;
    constexpr int B = 16;
    const int lane = threadIdx.x & 63;
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) mx = fmaxf(mx, base[(size_t)i * stride + D]);
    const float M = wave_max(mx);
    float ls = 0.0f;
    for (int i = lane; i < n; i += 64) {
        const float mi = base[(size_t)i * stride + D];
        // a partial holding none of the row's keys (a shared gather's item) weighs nothing
        if (mi != -INFINITY) ls += exp2f(mi - M) * base[(size_t)i * stride + D + 1];
    }
    const float L = wave_sum(ls);
    float acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.0f;
    for (int i0 = 0; i0 < n; i0 += B) {
        float ov[B][DPL], mv[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int i = min(i0 + b, n - 1);
            mv[b] = base[(size_t)i * stride + D];
#pragma unroll
            for (int x = 0; x < DPL; ++x) ov[b][x] = base[(size_t)i * stride + lane + 64 * x];
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (i0 + b >= n) break;
            if (mv[b] == -INFINITY) continue;
            const float w = exp2f(mv[b] - M);
#pragma unroll
            for (int x = 0; x < DPL; ++x) acc[x] = __builtin_fmaf(ov[b][x], w, acc[x]);
        }
    }
#pragma unroll
    for (int x = 0; x < DPL; ++x) st<T>(o + lane + 64 * x, acc[x] / L * post);
}

// Merge the n partials of a retrieval row on kCombW wavefronts: wave w merges
// its own run of partials (relative to the run's maximum), and wave 0 merges
// the runs in order, so a row of hundreds of pieces is not one wavefront's
// serial loop.  Deterministic for a given n.  sh: kCombW * (D + 2) floats.
constexpr int kCombW = 8;
template <typename T, int D>
__device__ void combine_block(const float* __restrict__ base, int n, T* __restrict__ o, float post, int stride,
                              float* sh) {
    constexpr int DPL = D / 64;
    constexpr int B = 16;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int per = (n + kCombW - 1) / kCombW;
    const int i0 = min(wv * per, n), i1 = min(i0 + per, n);
    float mx = -INFINITY;
    for (int i = i0 + lane; i < i1; i += 64) mx = fmaxf(mx, base[(size_t)i * stride + D]);
    const float Mw = wave_max(mx);
    float ls = 0.0f;
    for (int i = i0 + lane; i < i1; i += 64) {
        const float mi = base[(size_t)i * stride + D];
        if (mi != -INFINITY) ls += exp2f(mi - Mw) * base[(size_t)i * stride + D + 1];
    }
    const float Lw = wave_sum(ls);
    float acc[DPL];
#pragma unroll
    for (int x = 0; x < DPL; ++x) acc[x] = 0.0f;
    for (int j0 = i0; j0 < i1; j0 += B) {
        float ov[B][DPL], mv[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int i = min(j0 + b, i1 - 1);
            mv[b] = base[(size_t)i * stride + D];
#pragma unroll
            for (int x = 0; x < DPL; ++x) ov[b][x] = base[(size_t)i * stride + lane + 64 * x];
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (j0 + b >= i1) break;
            if (mv[b] == -INFINITY) continue;
            const float w = exp2f(mv[b] - Mw);
#pragma unroll
            for (int x = 0; x < DPL; ++x) acc[x] = __builtin_fmaf(ov[b][x], w, acc[x]);
        }
    }
    float* me = sh + wv * (D + 2);
#pragma unroll
    for (int x = 0; x < DPL; ++x) me[lane + 64 * x] = acc[x];
    if (lane == 0) {
        me[D] = Mw;
        me[D + 1] = Lw;
    }
    __syncthreads();
    if (wv == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kCombW; ++w) M = fmaxf(M, sh[w * (D + 2) + D]);
        float L = 0.0f, a[DPL];
#pragma unroll
        for (int x = 0; x < DPL; ++x) a[x] = 0.0f;
#pragma unroll
        for (int w = 0; w < kCombW; ++w) {
            const float mw = sh[w * (D + 2) + D];
            if (mw == -INFINITY) continue;
            const float f = exp2f(mw - M);
            L = __builtin_fmaf(f, sh[w * (D + 2) + D + 1], L);
#pragma unroll
            for (int x = 0; x < DPL; ++x) a[x] = __builtin_fmaf(sh[w * (D + 2) + lane + 64 * x], f, a[x]);
        }
#pragma unroll
        for (int x = 0; x < DPL; ++x) st<T>(o + lane + 64 * x, a[x] / L * post);
    }
}

// Sparse decode straight from the selection's row records (the work items of
// k_sparse_dec_part): each row's selected keys are read from the selection
// workspace (its ordered list -- with the keys' K/V row numbers when the row
// pass wrote them --, its score array overwritten by the indices, or every
// key), and the items also write the CSR output: the first workgroup the row
// pointers and the capacity check, every item its own slice of idx.  The
// combine kernel merges each row's partials.  Rows of one call only (row0 = 0).
template <typename T, typename TKV, int D>
__global__ __launch_bounds__(64) void k_sparse_dec_sel(Geo g, const T* __restrict__ q,
                                                       const TKV* __restrict__ kc,
                                                       const TKV* __restrict__ vc, SelWs sw, SelOut so,
                                                       AttnWs ws, int rows) {
    using S = Stream<TKV, D, 1, sparse_u<TKV, D>()>;
    if (*so.status != 0) return;                          // an invalid top_p was reported: nothing emitted
    const int lane = threadIdx.x;
    extern __shared__ int64_t dyn[];
    int64_t* rp = dyn;                                    // rows + 1
    int32_t* istart = reinterpret_cast<int32_t*>(dyn + rows + 1);   // rows + 1
    int32_t* rinfo = istart + rows + 1;                   // rows: mode | has_jo << 8
    __shared__ uint32_t joff[kItem];
    {   // selected keys and pieces per row, and their prefixes (every workgroup)
        const int per = (rows + 63) / 64;
        const int r0 = lane * per;
        long long cs = 0;
        int run = 0;
        for (int i = 0; i < per; ++i) {
            const int r = r0 + i;
            if (r < rows) {
                const int c = sw.st[r].count;
                rinfo[r] = sw.st[r].mode | (sw.st[r].has_jo << 8);
                cs += c;
                run += (c + kItem - 1) / kItem;
            }
        }
        long long exs = (long long)wave_incl_scan_u64((unsigned long long)cs);
        int ex = (int)wave_incl_scan_u32((uint32_t)run);
        const long long total_s = (long long)lane_u64((unsigned long long)exs, 63);
        const int total = (int)lane_u32((uint32_t)ex, 63);
        exs -= cs;
        ex -= run;
        for (int i = 0; i < per; ++i) {
            const int r = r0 + i;
            if (r < rows) {
                const int c = sw.st[r].count;
                rp[r] = exs;
                istart[r] = ex;
                exs += c;
                ex += (c + kItem - 1) / kItem;
            }
        }
        if (lane == 0) {
            rp[rows] = total_s;
            istart[rows] = total;
        }
    }
    __syncthreads();
    const bool fits = rp[rows] <= so.capacity;
    if (blockIdx.x == 0) {
        for (int r = lane; r <= rows; r += 64) {
            so.row_ptr[r] = rp[r];
            ws.item_start[r] = fits ? istart[r] : 0;
        }
        if (!fits && lane == 0) *so.status = 1;           // capacity overflow: the size needed is row_ptr[rows]
    }
    if (!fits) return;
    const int total = istart[rows];
    const float sc = g.attn_scale * kLog2e * g.k_scale;    // the K scale of FP8 codes folded into q
    constexpr int EPV = S::EPV, LPK = S::LPK;
    static_assert(kItem == 64, "one selected key per lane of an item");

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int lo = 0, hi = rows - 1;       // last row with istart <= item
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (istart[mid] <= item) lo = mid; else hi = mid - 1;
        }
        const int row = lo;
        const int t = row / g.n_ret, r = row - t * g.n_ret;
        const int h = g.ret_heads[r], kvh = h / g.group;
        const int k0 = (item - istart[row]) * kItem;
        const int n = (int)min<int64_t>(kItem, rp[row + 1] - rp[row] - k0);
        const int mode = rinfo[row] & 255;
        const int32_t* bt = g.block_table + (size_t)row_seq(g, t) * g.max_blocks;
        const int i = k0 + min(lane, n - 1);
        const int j = mode == 0 ? i
                    : mode == 1 ? (int)sw.sel[(size_t)row * sw.ucap + i]
                                : reinterpret_cast<const int32_t*>(sw.scores + (size_t)row * sw.score_ld)[i];
        if (lane < n) so.idx[rp[row] + k0 + lane] = j;
        joff[lane] = (rinfo[row] >> 8) ? reinterpret_cast<const uint32_t*>(sw.ubuf + (size_t)row * sw.ucap)[i]
                                       : (uint32_t)kv_rowidx(g, bt[j >> 8], kvh, j & 255);
        S st;
        st.init();
        const int sl = (lane % LPK) * EPV;
#pragma unroll
        for (int e = 0; e < EPV; ++e) st.q[0][e] = ld(q + ((size_t)t * g.Hq + h) * D + sl + e) * sc;
        __syncthreads();
        auto off = [&](int x) { return (size_t)joff[x] * D; };
        st.act[0] = true;
        st.run(n, off, kc, vc);
        st.merge();
        st.write(0, ws.part + (size_t)item * (D + 2));
        __syncthreads();
    }
}

constexpr int kMaxParts = 4096;   // partial weights kept in LDS; more are recomputed

// Merge `n` partial results (stride D + 2: output[D], max, sum) in order.
template <typename T, int D>
__device__ void combine_parts(const float* __restrict__ base, int n, T* __restrict__ o, float* wsh, float post) {
    const int tid = threadIdx.x;
    __shared__ float red[4];
    float mx = -INFINITY;
    for (int i = tid; i < n; i += blockDim.x) mx = fmaxf(mx, base[(size_t)i * (D + 2) + D]);
    mx = wave_max(mx);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    float M = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) M = fmaxf(M, red[w]);
    __syncthreads();
    float ls = 0.0f;
    for (int i = tid; i < n; i += blockDim.x) {
        const float w = exp2f(base[(size_t)i * (D + 2) + D] - M);
        if (i < kMaxParts) wsh[i] = w;
        ls += w * base[(size_t)i * (D + 2) + D + 1];
    }
    ls = wave_sum(ls);
    if ((tid & 63) == 0) red[tid >> 6] = ls;
    __syncthreads();
    float L = 0.0f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) L += red[w];
    for (int d = tid; d < D; d += blockDim.x) {
        float acc = 0.0f;
#pragma unroll 8
        for (int i = 0; i < n; ++i) {
            const float w = i < kMaxParts ? wsh[i] : exp2f(base[(size_t)i * (D + 2) + D] - M);
            acc = __builtin_fmaf(base[(size_t)i * (D + 2) + d], w, acc);
        }
        st<T>(o + d, acc / L * post);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(64 * kCombW) void k_sparse_dec_combine(Geo g, const int32_t* __restrict__ status,
                                                           AttnWs ws, T* __restrict__ out, int row0) {
    if (*status != 0) return;
    const int row = blockIdx.x;
    const int grow = row0 + row;
    const int t = grow / g.n_ret, r = grow - t * g.n_ret;
    const int h = g.ret_heads[r];
    const int i0 = ws.item_start[row], i1 = ws.item_start[row + 1];
    T* o = out + ((size_t)t * g.Hq + h) * D;
    if (i1 <= i0) {
        for (int d = threadIdx.x; d < D; d += blockDim.x) st<T>(o + d, 0.0f);
        return;
    }
    __shared__ float sh[kCombW * (D + 2)];
    combine_block<T, D>(ws.part + (size_t)i0 * (D + 2), i1 - i0, o, g.v_scale, D + 2, sh);   // V scale of FP8 codes
}

// ---------------------------------------------------------------------------
// Shared gathers (GQA): the retrieval heads of one KV head form a group of
// consecutive retrieval rows of a token (retrieval heads are ascending, so
// heads of one KV head are adjacent); the group's first row holds the union
// of their selected keys and each key's membership bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int gqa_first(const Geo& g, int r) {
    const int kv = g.ret_heads[r] / g.group;
    while (r > 0 && g.ret_heads[r - 1] / g.group == kv) --r;
    return r;
}
__device__ __forceinline__ int gqa_size(const Geo& g, int r0) {
    const int kv = g.ret_heads[r0] / g.group;
    int n = 1;
    while (r0 + n < g.n_ret && g.ret_heads[r0 + n] / g.group == kv) ++n;
    return n;
}

// Key i of a row's selected set (ascending): every key (mode 0), the ordered
// list (mode 1) or the row's score array overwritten by the indices (mode 2).
__device__ __forceinline__ uint32_t sel_key(const SelWs& sw, int lrow, int mode, int i) {
    return mode == 0 ? (uint32_t)i
         : mode == 1 ? sw.sel[(size_t)lrow * sw.ucap + i]
                     : (uint32_t)reinterpret_cast<const int32_t*>(sw.scores + (size_t)lrow * sw.score_ld)[i];
}

constexpr int kUnionT = 512;      // union pass threads
constexpr int kUnionLds = 8192;   // keys of a group merged in LDS (a larger group concatenates its lists)

// Union pass, one workgroup per row: the row's CSR (row pointer, and its keys
// into idx), and for a group's first row the group's union.  Lists are merged
// in LDS with duplicates adjacent (a key of list a lands after the keys of the
// other lists below it, and after equal keys of lists before a), then each
// run of equal keys becomes one union entry carrying the run's membership
// bits, in ascending key order.
__global__ __launch_bounds__(kUnionT) void k_gqa_union(Geo g, SelWs sw, SelOut so, AttnWs ws, int rows) {
    const int tid = threadIdx.x;
    if (*so.status != 0) return;                          // an invalid top_p was reported: nothing emitted
    const int row = blockIdx.x;
    __shared__ unsigned long long red[2][kUnionT / 64];
    __shared__ uint32_t lst[kUnionLds], mrg[kUnionLds];
    __shared__ int32_t s_cnt[kGqaMax], s_mode[kGqaMax], s_off[kGqaMax + 1];
    __shared__ unsigned long long scan_sh[kUnionT / 64 + 1];
    unsigned long long before = 0ull, all = 0ull;
    for (int i = tid; i < rows; i += kUnionT) {
        const unsigned long long c = (unsigned long long)sw.st[i].count;
        all += c;
        if (i < row) before += c;
    }
    before = wave_sum_u64(before);
    all = wave_sum_u64(all);
    if ((tid & 63) == 0) {
        red[0][tid >> 6] = before;
        red[1][tid >> 6] = all;
    }
    __syncthreads();
    before = 0ull;
    all = 0ull;
#pragma unroll
    for (int w = 0; w < kUnionT / 64; ++w) {
        before += red[0][w];
        all += red[1][w];
    }
    const RowState st = sw.st[row];
    if (tid == 0) {
        so.row_ptr[row + 1] = (int64_t)(before + (unsigned long long)st.count);
        if (row == 0 && (int64_t)all > so.capacity) *so.status = 1;   // the size needed is row_ptr[rows]
    }
    if ((int64_t)all > so.capacity) return;
    for (int i = tid; i < st.count; i += kUnionT) so.idx[before + i] = (int32_t)sel_key(sw, row, st.mode, i);
    const int t = row / g.n_ret, r = row - t * g.n_ret;
    if (gqa_first(g, r) != r) return;
    const int n = gqa_size(g, r);
    if (tid < n) {
        const RowState sr = sw.st[row + tid];
        s_cnt[tid] = sr.count;
        s_mode[tid] = sr.mode;
    }
    __syncthreads();
    if (tid == 0) {
        s_off[0] = 0;
        for (int i = 0; i < n; ++i) s_off[i + 1] = s_off[i] + s_cnt[i];
    }
    __syncthreads();
    const int tot = s_off[n];
    uint32_t* uk = ws.ukey + (size_t)row * ws.ulen;      // the group's rows' regions, together >= tot entries
    uint8_t* um = ws.umask + (size_t)row * ws.ulen;
    if (n < 2 || tot > kUnionLds) {
        // one row, or too many keys to merge here: the lists one after another
        for (int i = 0; i < n; ++i)
            for (int k = tid; k < s_cnt[i]; k += kUnionT) {
                uk[s_off[i] + k] = sel_key(sw, row + i, s_mode[i], k);
                um[s_off[i] + k] = (uint8_t)(1u << i);
            }
        if (tid == 0) ws.ucnt[row] = tot;
        return;
    }
    for (int e = tid; e < tot; e += kUnionT) {
        int i = 0;
        while (e >= s_off[i + 1]) ++i;
        lst[e] = sel_key(sw, row + i, s_mode[i], e - s_off[i]);
    }
    __syncthreads();
    for (int e = tid; e < tot; e += kUnionT) {
        int i = 0;
        while (e >= s_off[i + 1]) ++i;
        const uint32_t x = lst[e];
        int pos = e - s_off[i];
        for (int b = 0; b < n; ++b) {
            if (b == i) continue;
            // keys of list b below x (and equal to x when b comes first)
            int lo = s_off[b], hi = s_off[b + 1];
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (lst[mid] < x || (b < i && lst[mid] == x)) lo = mid + 1; else hi = mid;
            }
            pos += lo - s_off[b];
        }
        mrg[pos] = (x << 2) | (uint32_t)i;
    }
    __syncthreads();
    // each thread a run of consecutive merged entries: one scan orders the kept ones
    const int per = (tot + kUnionT - 1) / kUnionT;
    const int e0 = min(tid * per, tot), e1 = min(e0 + per, tot);
    uint32_t nkeep = 0u;
    for (int e = e0; e < e1; ++e) nkeep += e == 0 || (mrg[e - 1] >> 2) != (mrg[e] >> 2);
    unsigned long long t2;
    uint32_t o = (uint32_t)block_excl_scan_u64<kUnionT>(nkeep, &t2, scan_sh);
    for (int e = e0; e < e1; ++e) {
        const uint32_t x = mrg[e] >> 2;
        if (e > 0 && (mrg[e - 1] >> 2) == x) continue;
        uint32_t msk = 0u;
        for (int q2 = e; q2 < tot && (mrg[q2] >> 2) == x; ++q2) msk |= 1u << (mrg[q2] & 3u);
        uk[o] = x;
        um[o] = (uint8_t)msk;
        ++o;
    }
    if (tid == 0) ws.ucnt[row] = (int32_t)t2;
}

// Sparse decode over the groups' unions: one wavefront per (group, piece of
// kItem union keys); each key row is read once and scored for every head of
// the group whose set holds it (the others see it masked out).  Partials:
// [item][kGqaMax][D + 2].
template <typename T, typename TKV, int D>
__global__ __launch_bounds__(64) void k_sparse_dec_gqa(Geo g, const T* __restrict__ q,
                                                       const TKV* __restrict__ kc,
                                                       const TKV* __restrict__ vc, SelOut so, AttnWs ws, int rows) {
    using S = Stream<TKV, D, kGqaMax, 8>;
    if (*so.status != 0) return;
    const int lane = threadIdx.x;
    extern __shared__ int32_t istart[];                   // rows + 1
    __shared__ uint32_t joff[kItem];
    __shared__ uint32_t jm[kItem];
    {
        const int per = (rows + 63) / 64;
        const int r0 = lane * per;
        int run = 0;
        for (int i = 0; i < per; ++i) {
            const int rr = r0 + i;
            if (rr < rows) {
                const int tt = rr / g.n_ret, r = rr - tt * g.n_ret;
                if (gqa_first(g, r) == r) run += (ws.ucnt[rr] + kItem - 1) / kItem;
            }
        }
        int ex = (int)wave_incl_scan_u32((uint32_t)run);
        const int total = (int)lane_u32((uint32_t)ex, 63);
        ex -= run;
        for (int i = 0; i < per; ++i) {
            const int rr = r0 + i;
            if (rr < rows) {
                istart[rr] = ex;
                const int tt = rr / g.n_ret, r = rr - tt * g.n_ret;
                if (gqa_first(g, r) == r) ex += (ws.ucnt[rr] + kItem - 1) / kItem;
            }
        }
        if (lane == 0) istart[rows] = total;
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int r = lane; r <= rows; r += 64) ws.item_start[r] = istart[r];
    const int total = istart[rows];
    const float sc = g.attn_scale * kLog2e * g.k_scale;
    constexpr int EPV = S::EPV, LPK = S::LPK;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        // the last row with istart <= item: istart[row + 1] > item, so the row
        // has items, i.e. it is the first row of its group
        int lo = 0, hi = rows - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (istart[mid] <= item) lo = mid; else hi = mid - 1;
        }
        const int row = lo;
        const int t = row / g.n_ret, r0 = row - t * g.n_ret;
        const int n = gqa_size(g, r0);
        const int kvh = g.ret_heads[r0] / g.group;
        const int k0 = (item - istart[row]) * kItem;
        const int nk = min(kItem, ws.ucnt[row] - k0);
        const int32_t* bt = g.block_table + (size_t)row_seq(g, t) * g.max_blocks;
        const int i = k0 + min(lane, nk - 1);
        const uint32_t j = ws.ukey[(size_t)row * ws.ulen + i];
        jm[lane] = ws.umask[(size_t)row * ws.ulen + i];
        joff[lane] = (uint32_t)kv_rowidx(g, bt[j >> 8], kvh, j & 255);
        S st;
        st.init();
        const int sl = (lane % LPK) * EPV;
#pragma unroll
        for (int hh = 0; hh < kGqaMax; ++hh) {
            st.act[hh] = hh < n;
            const int h = g.ret_heads[min(r0 + hh, g.n_ret - 1)];
#pragma unroll
            for (int e = 0; e < EPV; ++e) st.q[hh][e] = hh < n ? ld(q + ((size_t)t * g.Hq + h) * D + sl + e) * sc : 0.0f;
        }
        __syncthreads();
        auto off = [&](int x) { return (size_t)joff[x] * D; };
        auto msk = [&](int x) { return jm[x]; };
        st.run(nk, off, kc, vc, msk);
        st.merge();
#pragma unroll
        for (int hh = 0; hh < kGqaMax; ++hh)
            if (hh < n) st.write(hh, ws.part + ((size_t)item * kGqaMax + hh) * (D + 2));
        __syncthreads();
    }
}

// The decode step's combine: workgroups [0, rows) merge the retrieval rows'
// partials on kCombW wavefronts each (nothing when the selection reported an
// error), the others the window partials of (sequence, local head) pairs, one
// pair b Hq + h per wavefront, kCombW pairs per workgroup.
template <typename T, int D>
__global__ __launch_bounds__(64 * kCombW) void k_dec_combine_all(Geo g, const int32_t* __restrict__ status, AttnWs ws,
                                                        T* __restrict__ out, int rows, const float* __restrict__ wpart,
                                                        int nsplit, int split_keys, int gqa) {
    const int blk = blockIdx.x;
    if (blk < rows) {
        if (*status != 0) return;
        const int t = blk / g.n_ret, r = blk - t * g.n_ret;
        const int h = g.ret_heads[r];
        // shared gathers: the row's slot among the partials of its group's items
        const int r0 = gqa ? gqa_first(g, r) : r;
        const int lrow0 = t * g.n_ret + r0;
        const int i0 = ws.item_start[lrow0], i1 = ws.item_start[lrow0 + 1];
        T* o = out + ((size_t)t * g.Hq + h) * D;
        if (i1 <= i0) {
            for (int d = threadIdx.x; d < D; d += blockDim.x) st<T>(o + d, 0.0f);
            return;
        }
        __shared__ float sh[kCombW * (D + 2)];
        if (gqa)
            combine_block<T, D>(ws.part + ((size_t)i0 * kGqaMax + (r - r0)) * (D + 2), i1 - i0, o, g.v_scale,
                                kGqaMax * (D + 2), sh);
        else
            combine_block<T, D>(ws.part + (size_t)i0 * (D + 2), i1 - i0, o, g.v_scale, D + 2, sh);
        return;
    }
    // window pairs (sequence, head): one per wavefront, kCombW per workgroup
    const int bh = (blk - rows) * kCombW + (int)(threadIdx.x >> 6);
    if (bh >= g.batch * g.Hq) return;
    const int b = bh / g.Hq, h = bh - b * g.Hq;
    if (g.is_ret[h]) return;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, 0, &ns_end, &w_start);
    const int ns = min(nsplit, (n_all + split_keys - 1) / split_keys);
    combine_wave<T, D>(wpart + ((size_t)b * g.Hq + h) * nsplit * (D + 2), ns, out + ((size_t)b * g.Hq + h) * D,
                       g.v_scale);
}

// ---------------------------------------------------------------------------
// Window / dense decode: grid (nsplit, batch * Hkv), one wavefront each.  The
// wavefront serves every head of the KV group that needs it (the local heads,
// or all heads when dense), reading each key and value row once.
// ---------------------------------------------------------------------------

template <typename T, typename TKV, int D, int NH>
__global__ __launch_bounds__(64) void k_win_dec_part(Geo g, const T* __restrict__ q,
                                                     const TKV* __restrict__ kc_main,
                                                     const TKV* __restrict__ vc_main, float* __restrict__ part,
                                                     int nsplit, int split_keys, int dense) {
    using S = Stream<TKV, D, NH>;
    constexpr int EPV = S::EPV, LPK = S::LPK;
    const int lane = threadIdx.x;
    const int b = blockIdx.y / g.Hkv, kvh = blockIdx.y % g.Hkv;
    // K/V of this KV head: the paged cache, or the window-only ring
    const TKV* __restrict__ kc = g.kv_ring[kvh] ? (const TKV*)g.k_ring : kc_main;
    const TKV* __restrict__ vc = g.kv_ring[kvh] ? (const TKV*)g.v_ring : vc_main;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, dense, &ns_end, &w_start);
    const int v0 = blockIdx.x * split_keys;
    if (v0 >= n_all) return;
    const int n = min(split_keys, n_all - v0);

    // slot i serves query head kvh * group + i (group <= NH) if that head
    // needs this kernel; slots are indexed with constants only, so the
    // per-head state stays in registers
    const float sc = g.attn_scale * kLog2e * g.k_scale;    // the K scale of FP8 codes folded into q
    const int sl = (lane % LPK) * EPV;
    S st;
    st.init();
    bool any = false;
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        const int hh = kvh * g.group + i;
        st.act[i] = i < g.group && (dense || !g.is_ret[hh]);
        any = any || st.act[i];
        if (st.act[i]) {
            float f[EPV];
            const T* qp = q + ((size_t)b * g.Hq + hh) * D + sl;
            if (Pack<T>::N == EPV) {
                Pack<T>::unpack(*reinterpret_cast<const uint4*>(qp), f);
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e) f[e] = ld(qp + e);
            }
#pragma unroll
            for (int e = 0; e < EPV; ++e) st.q[i][e] = f[e] * sc;
        } else {
#pragma unroll
            for (int e = 0; e < EPV; ++e) st.q[i][e] = 0.0f;
        }
    }
    if (!any) return;
    // Page ids of the split, resolved once into LDS.  The split's virtual keys
    // [v0, v0 + n) are a run of sink positions followed by a run of window
    // positions; each run covers consecutive pages.
    __shared__ int pgs[64];
    const int vS1 = min(v0 + n, ns_end);
    const int pS0 = v0 >> 8;
    const int nPS = vS1 > v0 ? ((vS1 - 1) >> 8) - pS0 + 1 : 0;
    const int jW0 = w_start + max(v0, ns_end) - ns_end;
    const int jW1 = w_start + (v0 + n) - ns_end;
    const int pW0 = jW0 >> 8;
    const int nPW = jW1 > jW0 ? ((jW1 - 1) >> 8) - pW0 + 1 : 0;
    if (lane < nPS) pgs[lane] = kv_page(g, b, kvh, pS0 + lane);
    else if (lane < nPS + nPW) pgs[lane] = kv_page(g, b, kvh, pW0 + lane - nPS);
    __syncthreads();
    auto off = [&](int i) {
        const int vi = v0 + i;
        int j, pi;
        if (vi < ns_end) {
            j = vi;
            pi = (j >> 8) - pS0;
        } else {
            j = w_start + (vi - ns_end);
            pi = nPS + (j >> 8) - pW0;
        }
        return kv_off(g, pgs[pi], kvh, j & 255, D);
    };
    st.run(n, off, kc, vc);
    st.merge();
#pragma unroll
    for (int i = 0; i < NH; ++i)
        if (st.act[i]) st.write(i, part + (((size_t)b * g.Hq + kvh * g.group + i) * nsplit + blockIdx.x) * (D + 2));
}

// ---------------------------------------------------------------------------
// Local-head (or dense) decode on bf16 MFMA, D = 128: one wavefront per
// (sequence, KV head, split), the work item of win_mfma.hpp.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_win_dec_mfma(Geo g, const bf16_t* __restrict__ q,
                                                     const bf16_t* __restrict__ kc_main,
                                                     const bf16_t* __restrict__ vc_main, float* __restrict__ part,
                                                     int nsplit, int split_keys, int dense) {
    __shared__ int pgs[64];
    __shared__ __align__(16) bf16_t Vs[32 * kWVsLd];
    win_mfma_item<false>(g, q, kc_main, vc_main, part, nsplit, split_keys, dense, blockIdx.x, blockIdx.y, pgs, Vs);
}

template <typename T, int D>
__global__ __launch_bounds__(128) void k_win_dec_combine(Geo g, const float* __restrict__ part,
                                                         T* __restrict__ out, int nsplit, int split_keys,
                                                         int dense) {
    __shared__ float wsh[kMaxParts];
    const int b = blockIdx.y, h = blockIdx.x;
    if (!dense && g.is_ret[h]) return;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, dense, &ns_end, &w_start);
    const int ns = min(nsplit, (n_all + split_keys - 1) / split_keys);
    if (!dense) {
        // the window's few splits: the one-wavefront combine (the decode
        // step's combine merges the same partials the same way)
        if (threadIdx.x < 64)
            combine_wave<T, D>(part + ((size_t)b * g.Hq + h) * nsplit * (D + 2), ns, out + ((size_t)b * g.Hq + h) * D,
                               g.v_scale);
        return;
    }
    combine_parts<T, D>(part + ((size_t)b * g.Hq + h) * nsplit * (D + 2), ns,
                        out + ((size_t)b * g.Hq + h) * D, wsh, g.v_scale);
}

template <typename T, typename TKV, int D>
hipError_t sparse_dec(const Geo& g, const void* q, const void* k, const void* v, const int64_t* row_ptr,
                      const int32_t* idx, const int32_t* status, void* out, const AttnWs& ws, int row0,
                      int rows, hipStream_t s) {
    const int64_t grid = std::min<int64_t>(std::max<int64_t>(ws.max_items, 1), 4096);
    const size_t shmem = (sizeof(int64_t) + sizeof(int32_t)) * (rows + 1);
    hipLaunchKernelGGL((k_sparse_dec_part<T, TKV, D>), dim3((unsigned)grid), dim3(64), shmem, s, g,
                       (const T*)q, (const TKV*)k, (const TKV*)v, row_ptr, idx, status, ws, row0, rows);
    hipLaunchKernelGGL((k_sparse_dec_combine<T, D>), dim3(rows), dim3(64 * kCombW), 0, s, g, status, ws, (T*)out, row0);
    return hipGetLastError();
}

template <typename T, typename TKV, int D>
hipError_t sparse_dec_sel(const Geo& g, const void* q, const void* k, const void* v, const SelWs& sw,
                          const SelOut& so, void* out, const AttnWs& ws, int rows, const WinWork* win,
                          hipStream_t s) {
    // enough workgroups for every item of a small batch at once (a workgroup
    // past the last item only reads the row records)
    const int64_t grid = std::min<int64_t>(std::max<int64_t>(ws.max_items, 1), rows <= 128 ? 1024 : 4096);
    const size_t shmem = (sizeof(int64_t) + sizeof(int32_t)) * (rows + 1) + sizeof(int32_t) * rows;
    hipLaunchKernelGGL((k_sparse_dec_sel<T, TKV, D>), dim3((unsigned)grid), dim3(64), shmem, s, g, (const T*)q,
                       (const TKV*)k, (const TKV*)v, sw, so, ws, rows);
    if (win && win->items > 0)
        hipLaunchKernelGGL((k_dec_combine_all<T, D>), dim3(rows + (g.batch * g.Hq + kCombW - 1) / kCombW),
                           dim3(64 * kCombW), 0, s, g, so.status, ws,
                           (T*)out, rows, win->part, win->nsplit, win->split_keys, 0);
    else
        hipLaunchKernelGGL((k_sparse_dec_combine<T, D>), dim3(rows), dim3(64 * kCombW), 0, s, g, so.status, ws, (T*)out, 0);
    return hipGetLastError();
}

template <typename T, typename TKV, int D, int NH>
void win_dec_part(const Geo& g, const void* q, const void* k, const void* v, float* part, int nsplit,
                  int split_keys, int dense, hipStream_t s) {
    hipLaunchKernelGGL((k_win_dec_part<T, TKV, D, NH>), dim3(nsplit, g.batch * g.Hkv), dim3(64), 0, s, g,
                       (const T*)q, (const TKV*)k, (const TKV*)v, part, nsplit, split_keys, dense);
}

template <typename T, typename TKV, int D>
hipError_t win_dec(const Geo& g, const void* q, const void* k, const void* v, void* out, float* part,
                   int nsplit, int split_keys, int dense, hipStream_t s) {
    if (std::is_same<T, bf16_t>::value && std::is_same<TKV, bf16_t>::value && D == 128 && g.group <= 32)
        hipLaunchKernelGGL(k_win_dec_mfma, dim3(nsplit, g.batch * g.Hkv), dim3(64), 0, s, g, (const bf16_t*)q,
                           (const bf16_t*)k, (const bf16_t*)v, part, nsplit, split_keys, dense);
    else if (g.group <= 1)
        win_dec_part<T, TKV, D, 1>(g, q, k, v, part, nsplit, split_keys, dense, s);
    else if (g.group <= 2)
        win_dec_part<T, TKV, D, 2>(g, q, k, v, part, nsplit, split_keys, dense, s);
    else if (g.group <= 4)
        win_dec_part<T, TKV, D, 4>(g, q, k, v, part, nsplit, split_keys, dense, s);
    else
        win_dec_part<T, TKV, D, 8>(g, q, k, v, part, nsplit, split_keys, dense, s);
    hipLaunchKernelGGL((k_win_dec_combine<T, D>), dim3(g.Hq, g.batch), dim3(128), 0, s, g, part, (T*)out,
                       nsplit, split_keys, dense);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_decode(const Geo& g, const void* q, const void* k, const void* v,
                                const int64_t* row_ptr, const int32_t* idx, const int32_t* status,
                                void* out, const AttnWs& ws, int row0, int rows, int dtype, hipStream_t s) {
    if (g.kv_fp8 && g.D == 64)
        return sparse_dec<bf16_t, fp8e4_t, 64>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    if (g.kv_fp8) return sparse_dec<bf16_t, fp8e4_t, 128>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    if (dtype == 0 && g.D == 64) return sparse_dec<float, float, 64>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    if (dtype == 0 && g.D == 128) return sparse_dec<float, float, 128>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    if (dtype == 1 && g.D == 64) return sparse_dec<bf16_t, bf16_t, 64>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    return sparse_dec<bf16_t, bf16_t, 128>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
}

hipError_t launch_sparse_decode_sel(const Geo& g, const void* q, const void* k, const void* v, const SelWs& sw,
                                    const SelOut& so, void* out, const AttnWs& ws, int rows, int dtype,
                                    const WinWork* win, hipStream_t s) {
    if (g.kv_fp8 && g.D == 64) return sparse_dec_sel<bf16_t, fp8e4_t, 64>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    if (g.kv_fp8) return sparse_dec_sel<bf16_t, fp8e4_t, 128>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    if (dtype == 0 && g.D == 64) return sparse_dec_sel<float, float, 64>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    if (dtype == 0 && g.D == 128) return sparse_dec_sel<float, float, 128>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    if (dtype == 1 && g.D == 64) return sparse_dec_sel<bf16_t, bf16_t, 64>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    return sparse_dec_sel<bf16_t, bf16_t, 128>(g, q, k, v, sw, so, out, ws, rows, win, s);
}

template <typename T, typename TKV, int D>
hipError_t sparse_dec_gqa(const Geo& g, const void* q, const void* k, const void* v, const SelWs& sw,
                          const SelOut& so, void* out, const AttnWs& ws, int rows, const WinWork* win,
                          hipStream_t s) {
    hipLaunchKernelGGL(k_gqa_union, dim3(rows), dim3(kUnionT), 0, s, g, sw, so, ws, rows);
    const int64_t grid = std::min<int64_t>(std::max<int64_t>(ws.max_items, 1), rows <= 128 ? 1024 : 4096);
    const size_t shmem = sizeof(int32_t) * (rows + 1);
    hipLaunchKernelGGL((k_sparse_dec_gqa<T, TKV, D>), dim3((unsigned)grid), dim3(64), shmem, s, g, (const T*)q,
                       (const TKV*)k, (const TKV*)v, so, ws, rows);
    const bool wc = win && win->items > 0;
    hipLaunchKernelGGL((k_dec_combine_all<T, D>), dim3(rows + (wc ? (g.batch * g.Hq + kCombW - 1) / kCombW : 0)),
                       dim3(64 * kCombW), 0, s, g,
                       so.status, ws, (T*)out, rows, wc ? win->part : (const float*)nullptr, wc ? win->nsplit : 0,
                       wc ? win->split_keys : 0, 1);
    return hipGetLastError();
}

hipError_t launch_sparse_decode_gqa(const Geo& g, const void* q, const void* k, const void* v, const SelWs& sw,
                                    const SelOut& so, void* out, const AttnWs& ws, int rows, int dtype,
                                    const WinWork* win, hipStream_t s) {
    if (dtype == 0 && g.D == 64) return sparse_dec_gqa<float, float, 64>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    if (dtype == 0 && g.D == 128) return sparse_dec_gqa<float, float, 128>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    if (dtype == 1 && g.D == 64) return sparse_dec_gqa<bf16_t, bf16_t, 64>(g, q, k, v, sw, so, out, ws, rows, nullptr, s);
    return sparse_dec_gqa<bf16_t, bf16_t, 128>(g, q, k, v, sw, so, out, ws, rows, win, s);
}

hipError_t launch_window_decode(const Geo& g, const void* q, const void* k, const void* v, void* out,
                                float* part, int nsplit, int split_keys, int dense, int dtype,
                                hipStream_t s) {
    if (g.kv_fp8 && g.D == 64) return win_dec<bf16_t, fp8e4_t, 64>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    if (g.kv_fp8) return win_dec<bf16_t, fp8e4_t, 128>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    if (dtype == 0 && g.D == 64) return win_dec<float, float, 64>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    if (dtype == 0 && g.D == 128) return win_dec<float, float, 128>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    if (dtype == 1 && g.D == 64) return win_dec<bf16_t, bf16_t, 64>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    return win_dec<bf16_t, bf16_t, 128>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
}

}  // namespace rtp
