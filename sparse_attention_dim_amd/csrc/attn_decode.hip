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

__device__ __forceinline__ size_t kv_off(const Geo& g, int page, int kvh, int slot, int D) {
    return (((size_t)page * g.Hkv + kvh) * kBlk + slot) * (size_t)D;
}

template <typename T, int D, int NH>
struct Stream {
    static constexpr int EPV = Pack<T>::N;      // elements per lane slice
    static constexpr int LPK = D / EPV;         // lanes per key row
    static constexpr int GPW = 64 / LPK;        // key rows per load instruction
    static constexpr int U = NH > 4 ? 4 : 8;    // rows per group per iteration

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
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    float acc = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPV; ++e) acc = __builtin_fmaf(q[h][e], f[e], acc);
                    acc = group_sum<LPK>(acc);
                    s[u][h] = ok ? acc : -INFINITY;
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

template <typename T, int D>
__global__ __launch_bounds__(64) void k_sparse_dec_part(Geo g, const T* __restrict__ q,
                                                        const T* __restrict__ kc,
                                                        const T* __restrict__ vc,
                                                        const int64_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ status,
                                                        AttnWs ws, int row0, int rows) {
    using S = Stream<T, D, 1>;
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
        int ex = run;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(ex, o);
            if (lane >= o) ex += y;
        }
        const int total = __shfl(ex, 63);
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
    const float sc = g.attn_scale * kLog2e;
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
            joff[lane + 64 * i] = (uint32_t)(((size_t)pg[i] * g.Hkv + kvh) * kBlk + (jl[i] & 255));
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

constexpr int kMaxParts = 4096;   // partial weights kept in LDS; more are recomputed

// Merge `n` partial results (stride D + 2: output[D], max, sum) in order.
template <typename T, int D>
__device__ void combine_parts(const float* __restrict__ base, int n, T* __restrict__ o, float* wsh) {
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
        st<T>(o + d, acc / L);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void k_sparse_dec_combine(Geo g, const int32_t* __restrict__ status,
                                                            AttnWs ws, T* __restrict__ out, int row0) {
    if (*status != 0) return;
    __shared__ float wsh[kMaxParts];
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
    combine_parts<T, D>(ws.part + (size_t)i0 * (D + 2), i1 - i0, o, wsh);
}

// ---------------------------------------------------------------------------
// Window / dense decode: grid (nsplit, batch * Hkv), one wavefront each.  The
// wavefront serves every head of the KV group that needs it (the local heads,
// or all heads when dense), reading each key and value row once.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int win_count(const Geo& g, int pos, int dense, int* ns_end, int* w_start) {
    if (dense) {
        *ns_end = pos + 1;
        *w_start = pos + 1;
        return pos + 1;
    }
    const int ne = min(g.sinks, pos + 1);
    const int ws = max(pos - g.window + 1, ne);
    *ns_end = ne;
    *w_start = ws;
    return ne + (pos - ws + 1);
}

template <typename T, int D, int NH>
__global__ __launch_bounds__(64) void k_win_dec_part(Geo g, const T* __restrict__ q,
                                                     const T* __restrict__ kc,
                                                     const T* __restrict__ vc, float* __restrict__ part,
                                                     int nsplit, int split_keys, int dense) {
    using S = Stream<T, D, NH>;
    constexpr int EPV = S::EPV, LPK = S::LPK;
    const int lane = threadIdx.x;
    const int b = blockIdx.y / g.Hkv, kvh = blockIdx.y % g.Hkv;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, dense, &ns_end, &w_start);
    const int v0 = blockIdx.x * split_keys;
    if (v0 >= n_all) return;
    const int n = min(split_keys, n_all - v0);

    // slot i serves query head kvh * group + i (group <= NH) if that head
    // needs this kernel; slots are indexed with constants only, so the
    // per-head state stays in registers
    const float sc = g.attn_scale * kLog2e;
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
            Pack<T>::unpack(*reinterpret_cast<const uint4*>(q + ((size_t)b * g.Hq + hh) * D + sl), f);
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
    const int32_t* bt = g.block_table + (size_t)b * g.max_blocks;
    const int vS1 = min(v0 + n, ns_end);
    const int pS0 = v0 >> 8;
    const int nPS = vS1 > v0 ? ((vS1 - 1) >> 8) - pS0 + 1 : 0;
    const int jW0 = w_start + max(v0, ns_end) - ns_end;
    const int jW1 = w_start + (v0 + n) - ns_end;
    const int pW0 = jW0 >> 8;
    const int nPW = jW1 > jW0 ? ((jW1 - 1) >> 8) - pW0 + 1 : 0;
    if (lane < nPS) pgs[lane] = bt[pS0 + lane];
    else if (lane < nPS + nPW) pgs[lane] = bt[pW0 + lane - nPS];
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
// (sequence, KV head, split).  The query heads of the KV group are the 32
// columns of v_mfma_f32_32x32x16_bf16 (heads that do not need the kernel are
// zero columns), so every K/V row is read once for the group.  Per block of 32
// keys: S^T[key][head] = K . Q^T with the K rows straight from memory (each
// lane one key, 16 bytes per k-step); online softmax per head in-lane (a lane
// holds 16 of the block's keys of its head, the other half-wave the other 16);
// O^T[d][head] += V^T . P^T with V^T from a transposed LDS tile and P^T taken
// straight from the S^T registers (a fixed key permutation matches their
// layout).  Writes the same partials as k_win_dec_part.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kWVtLd = 32 + 4;     // V^T row stride in LDS (bf16): 8-byte aligned 4-key reads

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

__global__ __launch_bounds__(64) void k_win_dec_mfma(Geo g, const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
                                                     const bf16_t* __restrict__ vc, float* __restrict__ part,
                                                     int nsplit, int split_keys, int dense) {
    constexpr int D = 128;
    const int lane = threadIdx.x, hh = lane >> 5, col = lane & 31;
    const int b = blockIdx.y / g.Hkv, kvh = blockIdx.y % g.Hkv;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, dense, &ns_end, &w_start);
    const int v0 = blockIdx.x * split_keys;
    if (v0 >= n_all) return;
    const int n = min(split_keys, n_all - v0);
    const int hq = kvh * g.group + col;
    const bool act = col < g.group && (dense || !g.is_ret[col < g.group ? hq : 0]);
    if (__ballot(act) == 0ull) return;
    // B operand Q^T: lane holds q[hq][16 kk + 8 hh .. +8]
    uint4 qreg[8];
    {
        const bf16_t* qp = q + ((size_t)b * g.Hq + (act ? hq : 0)) * D + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            qreg[kk] = act ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
    }
    // page ids of the split: a run of sink positions, then a run of window positions
    __shared__ int pgs[64];
    __shared__ __align__(16) bf16_t Vt[D * kWVtLd];
    const int32_t* bt = g.block_table + (size_t)b * g.max_blocks;
    const int vS1 = min(v0 + n, ns_end);
    const int pS0 = v0 >> 8;
    const int nPS = vS1 > v0 ? ((vS1 - 1) >> 8) - pS0 + 1 : 0;
    const int jW0 = w_start + max(v0, ns_end) - ns_end;
    const int jW1 = w_start + (v0 + n) - ns_end;
    const int pW0 = jW0 >> 8;
    const int nPW = jW1 > jW0 ? ((jW1 - 1) >> 8) - pW0 + 1 : 0;
    if (lane < nPS) pgs[lane] = bt[pS0 + lane];
    else if (lane < nPS + nPW) pgs[lane] = bt[pW0 + lane - nPS];
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
    const float sc = g.attn_scale * kLog2e;
    f32x16_t oacc[4];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dd][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    for (int k0 = 0; k0 < n; k0 += 32) {
        // this lane's key row: K for the A operand, V for the transposed tile
        const bool live = k0 + col < n;
        const size_t ro = off(min(k0 + col, n - 1)) + 8 * hh;
        uint4 ka[8], va[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const uint4*>(kc + ro + 16 * kk);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) va[kk] = *reinterpret_cast<const uint4*>(vc + ro + 16 * kk);
        f32x16_t s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[kk]), as_bf16x8(qreg[kk]), s, 0, 0, 0);
        __syncthreads();                                  // the previous block's V^T reads are done
        // V^T[d][key col]: d = 16 kk + 8 hh + e; rows past the split stored as zeros
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const uint32_t w4[4] = {live ? va[kk].x : 0u, live ? va[kk].y : 0u, live ? va[kk].z : 0u,
                                    live ? va[kk].w : 0u};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int d = 16 * kk + 8 * hh + 2 * x;
                Vt[d * kWVtLd + col] = __builtin_bit_cast(bf16_t, (uint16_t)(w4[x] & 0xFFFFu));
                Vt[(d + 1) * kWVtLd + col] = __builtin_bit_cast(bf16_t, (uint16_t)(w4[x] >> 16));
            }
        }
        // scale, mask, block maximum of this lane's head
        float mt = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = k0 + (i >> 2) * 8 + 4 * hh + (i & 3);
            const float v = key < n ? s[i] * sc : -INFINITY;
            s[i] = v;
            mt = fmaxf(mt, v);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);             // finite: the block has a live key
        if (__ballot(m_new > m_run) != 0ull) {            // some head's maximum rose: rescale
            const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= corr;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dd][i] *= corr;
        }
        m_run = m_new;
        uint32_t pb[8];
        {
            float p[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
                l_run += p[i];
            }
#pragma unroll
            for (int x = 0; x < 8; ++x) pb[x] = pack_bf2(p[2 * x], p[2 * x + 1]);
        }
        __syncthreads();                                  // the V^T tile is written
        // O^T += V^T P^T; k-step kk covers keys 16 kk + 4 hh + {0..3, 8..11}
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const uint4 bp = make_uint4(pb[4 * kk], pb[4 * kk + 1], pb[4 * kk + 2], pb[4 * kk + 3]);
            const int kc0 = 16 * kk + 4 * hh;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const bf16_t* vr = &Vt[(32 * dd + col) * kWVtLd + kc0];
                const uint2 lo = *reinterpret_cast<const uint2*>(vr);
                const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
                const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
                oacc[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bp), oacc[dd], 0, 0, 0);
            }
        }
    }
    // partials: lane holds O^T[32 dd + 8 (i/4) + 4 hh + (i%4)][head col]
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (act) {
        float* pp = part + (((size_t)b * g.Hq + hq) * nsplit + blockIdx.x) * (D + 2);
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * dd + 8 * r4 + 4 * hh;    // partial records are 8-byte aligned
                *reinterpret_cast<float2*>(pp + d0) = make_float2(oacc[dd][4 * r4], oacc[dd][4 * r4 + 1]);
                *reinterpret_cast<float2*>(pp + d0 + 2) = make_float2(oacc[dd][4 * r4 + 2], oacc[dd][4 * r4 + 3]);
            }
        if (hh == 0) {
            pp[D] = m_run;
            pp[D + 1] = l_tot;
        }
    }
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
    combine_parts<T, D>(part + ((size_t)b * g.Hq + h) * nsplit * (D + 2), ns,
                        out + ((size_t)b * g.Hq + h) * D, wsh);
}

template <typename T, int D>
hipError_t sparse_dec(const Geo& g, const void* q, const void* k, const void* v, const int64_t* row_ptr,
                      const int32_t* idx, const int32_t* status, void* out, const AttnWs& ws, int row0,
                      int rows, hipStream_t s) {
    const int64_t grid = std::min<int64_t>(std::max<int64_t>(ws.max_items, 1), 4096);
    const size_t shmem = (sizeof(int64_t) + sizeof(int32_t)) * (rows + 1);
    hipLaunchKernelGGL((k_sparse_dec_part<T, D>), dim3((unsigned)grid), dim3(64), shmem, s, g,
                       (const T*)q, (const T*)k, (const T*)v, row_ptr, idx, status, ws, row0, rows);
    hipLaunchKernelGGL((k_sparse_dec_combine<T, D>), dim3(rows), dim3(128), 0, s, g, status, ws, (T*)out, row0);
    return hipGetLastError();
}

template <typename T, int D, int NH>
void win_dec_part(const Geo& g, const void* q, const void* k, const void* v, float* part, int nsplit,
                  int split_keys, int dense, hipStream_t s) {
    hipLaunchKernelGGL((k_win_dec_part<T, D, NH>), dim3(nsplit, g.batch * g.Hkv), dim3(64), 0, s, g,
                       (const T*)q, (const T*)k, (const T*)v, part, nsplit, split_keys, dense);
}

template <typename T, int D>
hipError_t win_dec(const Geo& g, const void* q, const void* k, const void* v, void* out, float* part,
                   int nsplit, int split_keys, int dense, hipStream_t s) {
    if (std::is_same<T, bf16_t>::value && D == 128 && g.group <= 32)
        hipLaunchKernelGGL(k_win_dec_mfma, dim3(nsplit, g.batch * g.Hkv), dim3(64), 0, s, g, (const bf16_t*)q,
                           (const bf16_t*)k, (const bf16_t*)v, part, nsplit, split_keys, dense);
    else if (g.group <= 1)
        win_dec_part<T, D, 1>(g, q, k, v, part, nsplit, split_keys, dense, s);
    else if (g.group <= 2)
        win_dec_part<T, D, 2>(g, q, k, v, part, nsplit, split_keys, dense, s);
    else if (g.group <= 4)
        win_dec_part<T, D, 4>(g, q, k, v, part, nsplit, split_keys, dense, s);
    else
        win_dec_part<T, D, 8>(g, q, k, v, part, nsplit, split_keys, dense, s);
    hipLaunchKernelGGL((k_win_dec_combine<T, D>), dim3(g.Hq, g.batch), dim3(128), 0, s, g, part, (T*)out,
                       nsplit, split_keys, dense);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_decode(const Geo& g, const void* q, const void* k, const void* v,
                                const int64_t* row_ptr, const int32_t* idx, const int32_t* status,
                                void* out, const AttnWs& ws, int row0, int rows, int dtype, hipStream_t s) {
    if (dtype == 0 && g.D == 64) return sparse_dec<float, 64>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    if (dtype == 0 && g.D == 128) return sparse_dec<float, 128>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    if (dtype == 1 && g.D == 64) return sparse_dec<bf16_t, 64>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
    return sparse_dec<bf16_t, 128>(g, q, k, v, row_ptr, idx, status, out, ws, row0, rows, s);
}

hipError_t launch_window_decode(const Geo& g, const void* q, const void* k, const void* v, void* out,
                                float* part, int nsplit, int split_keys, int dense, int dtype,
                                hipStream_t s) {
    if (dtype == 0 && g.D == 64) return win_dec<float, 64>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    if (dtype == 0 && g.D == 128) return win_dec<float, 128>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    if (dtype == 1 && g.D == 64) return win_dec<bf16_t, 64>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
    return win_dec<bf16_t, 128>(g, q, k, v, out, part, nsplit, split_keys, dense, s);
}

}  // namespace rtp
