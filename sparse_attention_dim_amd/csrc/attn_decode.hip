// attn_decode.hip -- decode attention on gfx950: exact attention of retrieval
// heads over their gathered selected rows, and of local heads over sinks plus a
// sliding window (dense = a window covering the whole context).
//
// Method: arXiv 2605.16928 abstract (retrieval heads keep the full KV cache
// and attend sparsely; the others use a restricted window); zhichai.net forum
// post "RTPurbo: Turning Dense LLMs into Sparse Attention Models ...", "Three
// Key Insights" item 1.
//
// Both are flash-decoding style: the key set of a row is split into chunks,
// each workgroup produces (max, sum, unnormalised output) for its chunk, and a
// combine kernel merges the chunks in a fixed order (deterministic).  A key row
// is read as 16-byte slices by a group of lanes (16 lanes for bf16/D=128), so
// every gathered 256-byte row is one contiguous burst.
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kItem = 128;          // selected keys per sparse work item

template <typename T, int D>
struct Lay {
    static constexpr int EPL = 16 / (int)sizeof(T);    // elements per lane (16 B)
    static constexpr int LPK = D / EPL;                 // lanes per key row
    static constexpr int KPW = 64 / LPK;                // key rows per wave step
};

template <typename T, int N>
__device__ __forceinline__ void load_slice(const T* p, float* f);
template <>
__device__ __forceinline__ void load_slice<bf16_t, 8>(const bf16_t* p, float* f) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    f[0] = __uint_as_float(a.x << 16); f[1] = __uint_as_float(a.x & 0xFFFF0000u);
    f[2] = __uint_as_float(a.y << 16); f[3] = __uint_as_float(a.y & 0xFFFF0000u);
    f[4] = __uint_as_float(a.z << 16); f[5] = __uint_as_float(a.z & 0xFFFF0000u);
    f[6] = __uint_as_float(a.w << 16); f[7] = __uint_as_float(a.w & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load_slice<float, 4>(const float* p, float* f) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
}

template <int LPK>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = 1; o < LPK; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ size_t kv_off(const Geo& g, int page, int kvh, int slot, int D) {
    return (((size_t)page * g.Hkv + kvh) * kBlk + slot) * (size_t)D;
}

// ---------------------------------------------------------------------------
// Sparse decode: persistent workgroups over (row, chunk of kItem selected keys).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void k_sparse_dec_part(Geo g, const T* __restrict__ q,
                                                         const T* __restrict__ kc,
                                                         const T* __restrict__ vc,
                                                         const int64_t* __restrict__ row_ptr,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ status,
                                                         AttnWs ws, int rows) {
    using LY = Lay<T, D>;
    constexpr int EPL = LY::EPL, LPK = LY::LPK, KPW = LY::KPW;
    if (*status != 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    extern __shared__ int32_t istart[];   // rows + 1
    __shared__ float lg[kItem];
    __shared__ int32_t jj[kItem];
    __shared__ float red[4];
    __shared__ float ored[4][D];

    // items per row and their prefix (every workgroup recomputes it)
    {
        constexpr int kPer = 16;                 // rows per thread (rows <= 4096)
        __shared__ unsigned long long scan_sh[5];
        int cnt[kPer];
        unsigned long long loc = 0;
        for (int i = 0; i < kPer; ++i) {
            const int r = tid * kPer + i;
            cnt[i] = 0;
            if (r < rows) {
                const int64_t n = row_ptr[r + 1] - row_ptr[r];
                cnt[i] = (int)((n + kItem - 1) / kItem);
            }
            loc += (unsigned long long)cnt[i];
        }
        unsigned long long tot;
        unsigned long long run = block_excl_scan_u64<256>(loc, &tot, scan_sh);
        for (int i = 0; i < kPer; ++i) {
            const int r = tid * kPer + i;
            if (r < rows) istart[r] = (int)run;
            run += (unsigned long long)cnt[i];
        }
        if (tid == 0) istart[rows] = (int)tot;
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int r = tid; r <= rows; r += 256) ws.item_start[r] = istart[r];
    const int total = istart[rows];
    const int sub = lane / LPK;          // key row within the wave step
    const int e0 = (lane % LPK) * EPL;   // first element of this lane's slice
    const float sc = g.attn_scale * kLog2e;

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        int lo = 0, hi = rows - 1;       // last row with istart <= item
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (istart[mid] <= item) lo = mid; else hi = mid - 1;
        }
        const int row = lo;
        const int t = row / g.n_ret, r = row - t * g.n_ret;
        const int h = g.ret_heads[r], kvh = h / g.group;
        const int b = t;
        const int64_t k0 = row_ptr[row] + (int64_t)(item - istart[row]) * kItem;
        const int n = (int)min<int64_t>(kItem, row_ptr[row + 1] - k0);
        const int32_t* bt = g.block_table + (size_t)b * g.max_blocks;

        float qv[EPL];
        load_slice<T, EPL>(q + ((size_t)t * g.Hq + h) * D + e0, qv);
        for (int i = tid; i < n; i += 256) jj[i] = idx[k0 + i];
        __syncthreads();
        // logits (log2 units)
        for (int s0 = wid * KPW; s0 < n; s0 += 4 * KPW) {
            const int kk = s0 + sub;
            float dot = 0.0f;
            if (kk < n) {
                const int j = jj[kk];
                float kv[EPL];
                load_slice<T, EPL>(kc + kv_off(g, bt[j >> 8], kvh, j & 255, D) + e0, kv);
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[e], kv[e], dot);
            }
            dot = group_sum<LPK>(dot);
            if (kk < n && (lane % LPK) == 0) lg[kk] = dot * sc;
        }
        __syncthreads();
        float mx = -INFINITY;
        for (int i = tid; i < n; i += 256) mx = fmaxf(mx, lg[i]);
        mx = wave_max(mx);
        if (lane == 0) red[wid] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float sm = 0.0f;
        for (int i = tid; i < n; i += 256) {
            const float p = exp2f(lg[i] - mx);
            lg[i] = p;
            sm += p;
        }
        sm = wave_sum(sm);
        if (lane == 0) red[wid] = sm;
        __syncthreads();
        sm = red[0] + red[1] + red[2] + red[3];
        // weighted values
        float o[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = 0.0f;
        for (int s0 = wid * KPW; s0 < n; s0 += 4 * KPW) {
            const int kk = s0 + sub;
            if (kk < n) {
                const int j = jj[kk];
                float vv[EPL];
                load_slice<T, EPL>(vc + kv_off(g, bt[j >> 8], kvh, j & 255, D) + e0, vv);
                const float p = lg[kk];
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[e] = __builtin_fmaf(p, vv[e], o[e]);
            }
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float x = o[e];
            for (int off = LPK; off < 64; off <<= 1) x += __shfl_xor(x, off);
            o[e] = x;
        }
        if (sub == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) ored[wid][e0 + e] = o[e];
        }
        __syncthreads();
        float* pp = ws.part + (size_t)item * (D + 2);
        for (int d = tid; d < D; d += 256) pp[d] = ored[0][d] + ored[1][d] + ored[2][d] + ored[3][d];
        if (tid == 0) {
            pp[D] = mx;
            pp[D + 1] = sm;
        }
        __syncthreads();
    }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void k_sparse_dec_combine(Geo g, const int32_t* __restrict__ status,
                                                            AttnWs ws, T* __restrict__ out) {
    if (*status != 0) return;
    const int row = blockIdx.x;
    const int t = row / g.n_ret, r = row - t * g.n_ret;
    const int h = g.ret_heads[r];
    const int i0 = ws.item_start[row], i1 = ws.item_start[row + 1];
    if (i1 <= i0) {
        for (int d = threadIdx.x; d < D; d += blockDim.x) st<T>(out + ((size_t)t * g.Hq + h) * D + d, 0.0f);
        return;
    }
    float M = -INFINITY;
    for (int i = i0; i < i1; ++i) M = fmaxf(M, ws.part[(size_t)i * (D + 2) + D]);
    float l = 0.0f;
    for (int i = i0; i < i1; ++i) {
        const float* pp = ws.part + (size_t)i * (D + 2);
        l += pp[D + 1] * exp2f(pp[D] - M);
    }
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float acc = 0.0f;
        for (int i = i0; i < i1; ++i) {
            const float* pp = ws.part + (size_t)i * (D + 2);
            acc += pp[d] * exp2f(pp[D] - M);
        }
        st<T>(out + ((size_t)t * g.Hq + h) * D + d, acc / l);
    }
}

// ---------------------------------------------------------------------------
// Window / dense decode: grid (nsplit, batch * Hkv).  One workgroup reads each
// key and value row of its split once and serves every head of the KV group
// that needs it (the local heads, or all heads when dense).
// ---------------------------------------------------------------------------
constexpr int kMaxGroup = 8;

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

template <typename T, int D>
__global__ __launch_bounds__(256) void k_win_dec_part(Geo g, const T* __restrict__ q,
                                                      const T* __restrict__ kc,
                                                      const T* __restrict__ vc, float* __restrict__ part,
                                                      int nsplit, int split_keys, int dense) {
    using LY = Lay<T, D>;
    constexpr int EPL = LY::EPL, LPK = LY::LPK, KPW = LY::KPW;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int b = blockIdx.y / g.Hkv, kvh = blockIdx.y % g.Hkv;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, dense, &ns_end, &w_start);
    const int v0 = blockIdx.x * split_keys;
    if (v0 >= n_all) return;
    const int n = min(split_keys, n_all - v0);

    // heads of this KV group that this call computes
    int heads[kMaxGroup];
    int nh = 0;
    for (int i = 0; i < g.group; ++i) {
        const int h = kvh * g.group + i;
        if (dense || !g.is_ret[h]) heads[nh++] = h;
    }
    if (nh == 0) return;

    extern __shared__ float lgs[];         // [kMaxGroup][split_keys]
    __shared__ float red[kMaxGroup][4];
    __shared__ float ored[4][D];
    const int sub = lane / LPK;
    const int e0 = (lane % LPK) * EPL;
    const float sc = g.attn_scale * kLog2e;
    const int32_t* bt = g.block_table + (size_t)b * g.max_blocks;

    float qv[kMaxGroup][EPL];
#pragma unroll
    for (int i = 0; i < kMaxGroup; ++i)
        if (i < nh) load_slice<T, EPL>(q + ((size_t)b * g.Hq + heads[i]) * D + e0, qv[i]);

    for (int s0 = wid * KPW; s0 < n; s0 += 4 * KPW) {
        const int kk = s0 + sub;
        float kv[EPL];
        if (kk < n) {
            const int vi = v0 + kk;
            const int j = vi < ns_end ? vi : w_start + (vi - ns_end);
            load_slice<T, EPL>(kc + kv_off(g, bt[j >> 8], kvh, j & 255, D) + e0, kv);
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) kv[e] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kMaxGroup; ++i) {
            if (i < nh) {
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[i][e], kv[e], dot);
                dot = group_sum<LPK>(dot);
                if (kk < n && (lane % LPK) == 0) lgs[i * split_keys + kk] = dot * sc;
            }
        }
    }
    __syncthreads();
    float mxh[kMaxGroup], smh[kMaxGroup];
    for (int i = 0; i < nh; ++i) {
        float mx = -INFINITY;
        for (int x = tid; x < n; x += 256) mx = fmaxf(mx, lgs[i * split_keys + x]);
        mx = wave_max(mx);
        if (lane == 0) red[i][wid] = mx;
    }
    __syncthreads();
    for (int i = 0; i < nh; ++i) mxh[i] = fmaxf(fmaxf(red[i][0], red[i][1]), fmaxf(red[i][2], red[i][3]));
    __syncthreads();
    for (int i = 0; i < nh; ++i) {
        float sm = 0.0f;
        for (int x = tid; x < n; x += 256) {
            const float p = exp2f(lgs[i * split_keys + x] - mxh[i]);
            lgs[i * split_keys + x] = p;
            sm += p;
        }
        sm = wave_sum(sm);
        if (lane == 0) red[i][wid] = sm;
    }
    __syncthreads();
    for (int i = 0; i < nh; ++i) smh[i] = red[i][0] + red[i][1] + red[i][2] + red[i][3];

    float o[kMaxGroup][EPL];
#pragma unroll
    for (int i = 0; i < kMaxGroup; ++i)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[i][e] = 0.0f;
    for (int s0 = wid * KPW; s0 < n; s0 += 4 * KPW) {
        const int kk = s0 + sub;
        if (kk < n) {
            const int vi = v0 + kk;
            const int j = vi < ns_end ? vi : w_start + (vi - ns_end);
            float vv[EPL];
            load_slice<T, EPL>(vc + kv_off(g, bt[j >> 8], kvh, j & 255, D) + e0, vv);
#pragma unroll
            for (int i = 0; i < kMaxGroup; ++i) {
                if (i < nh) {
                    const float p = lgs[i * split_keys + kk];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[i][e] = __builtin_fmaf(p, vv[e], o[i][e]);
                }
            }
        }
    }
    for (int i = 0; i < nh; ++i) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float x = o[i][e];
            for (int off = LPK; off < 64; off <<= 1) x += __shfl_xor(x, off);
            o[i][e] = x;
        }
        if (sub == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) ored[wid][e0 + e] = o[i][e];
        }
        __syncthreads();
        float* pp = part + (((size_t)b * g.Hq + heads[i]) * nsplit + blockIdx.x) * (D + 2);
        for (int d = tid; d < D; d += 256) pp[d] = ored[0][d] + ored[1][d] + ored[2][d] + ored[3][d];
        if (tid == 0) {
            pp[D] = mxh[i];
            pp[D + 1] = smh[i];
        }
        __syncthreads();
    }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void k_win_dec_combine(Geo g, const float* __restrict__ part,
                                                         T* __restrict__ out, int nsplit, int split_keys,
                                                         int dense) {
    const int b = blockIdx.y, h = blockIdx.x;
    if (!dense && g.is_ret[h]) return;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, dense, &ns_end, &w_start);
    const int ns = min(nsplit, (n_all + split_keys - 1) / split_keys);
    const float* base = part + ((size_t)b * g.Hq + h) * nsplit * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, base[(size_t)s * (D + 2) + D]);
    float l = 0.0f;
    for (int s = 0; s < ns; ++s) l += base[(size_t)s * (D + 2) + D + 1] * exp2f(base[(size_t)s * (D + 2) + D] - M);
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float acc = 0.0f;
        for (int s = 0; s < ns; ++s)
            acc += base[(size_t)s * (D + 2) + d] * exp2f(base[(size_t)s * (D + 2) + D] - M);
        st<T>(out + ((size_t)b * g.Hq + h) * D + d, acc / l);
    }
}

template <typename T, int D>
hipError_t sparse_dec(const Geo& g, const void* q, const void* k, const void* v, const int64_t* row_ptr,
                      const int32_t* idx, const int32_t* status, void* out, const AttnWs& ws, int rows,
                      hipStream_t s) {
    const int64_t grid = std::min<int64_t>(std::max<int64_t>(ws.max_items, 1), 2048);
    const size_t shmem = sizeof(int32_t) * (rows + 1);
    hipLaunchKernelGGL((k_sparse_dec_part<T, D>), dim3((unsigned)grid), dim3(256), shmem, s, g,
                       (const T*)q, (const T*)k, (const T*)v, row_ptr, idx, status, ws, rows);
    hipLaunchKernelGGL((k_sparse_dec_combine<T, D>), dim3(rows), dim3(128), 0, s, g, status, ws, (T*)out);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t win_dec(const Geo& g, const void* q, const void* k, const void* v, void* out, float* part,
                   int nsplit, int split_keys, int dense, hipStream_t s) {
    const size_t shmem = sizeof(float) * kMaxGroup * split_keys;
    hipLaunchKernelGGL((k_win_dec_part<T, D>), dim3(nsplit, g.batch * g.Hkv), dim3(256), shmem, s, g,
                       (const T*)q, (const T*)k, (const T*)v, part, nsplit, split_keys, dense);
    hipLaunchKernelGGL((k_win_dec_combine<T, D>), dim3(g.Hq, g.batch), dim3(128), 0, s, g, part, (T*)out,
                       nsplit, split_keys, dense);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_decode(const Geo& g, const void* q, const void* k, const void* v,
                                const int64_t* row_ptr, const int32_t* idx, const int32_t* status,
                                void* out, const AttnWs& ws, int rows, int dtype, hipStream_t s) {
    if (dtype == 0 && g.D == 64) return sparse_dec<float, 64>(g, q, k, v, row_ptr, idx, status, out, ws, rows, s);
    if (dtype == 0 && g.D == 128) return sparse_dec<float, 128>(g, q, k, v, row_ptr, idx, status, out, ws, rows, s);
    if (dtype == 1 && g.D == 64) return sparse_dec<bf16_t, 64>(g, q, k, v, row_ptr, idx, status, out, ws, rows, s);
    return sparse_dec<bf16_t, 128>(g, q, k, v, row_ptr, idx, status, out, ws, rows, s);
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
