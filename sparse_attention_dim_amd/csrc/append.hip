// append.hip -- indexer key append on gfx950: the 16-dim indexer key of every
// newly cached token and retrieval head (arXiv 2605.16928 abstract obs. (2),
// "16-dimensional indexer"; zhichai.net forum post "RTPurbo: Turning Dense LLMs
// into Sparse Attention Models ...", "Three Key Insights" item 2).
//
// One thread per output (token, retrieval head, c): an fp32 FMA chain over the
// head dimension, d ascending from +0, rounded once to bf16.  Bulk appends: a
// workgroup of 256 threads covers 16 tokens of one retrieval head, with the
// key rows and the head's projection staged in LDS.  A few tokens (a decode
// step): one wavefront per (token, four retrieval heads) with the chain's
// operands in registers, which shortens the dependent path.  k_kv_append
// stores new K/V rows and writes their indexer keys in one launch.
#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

template <typename T, typename TK, int D>
__global__ __launch_bounds__(256) void k_append(Geo g, const TK* __restrict__ kc, bf16_t* __restrict__ k_low,
                                                const T* __restrict__ w_k, const int32_t* __restrict__ seq_id,
                                                const int32_t* __restrict__ pos, int n) {
    // grid (ceil(n / 16), num_ret): 16 tokens of one retrieval head
    __shared__ float krow[16][D];
    __shared__ float wk[D * kIdx];
    const int tid = threadIdx.x;
    const int r = blockIdx.y;
    const int i0 = blockIdx.x * 16;
    const int kvh = g.ret_heads[r] / g.group;
    for (int x = tid; x < D * kIdx; x += 256) wk[x] = ld(w_k + (size_t)r * D * kIdx + x);
    for (int x = tid; x < 16 * D; x += 256) {
        const int tl = x / D, d = x % D;
        const int i = i0 + tl;
        float v = 0.0f;
        if (i < n) {
            const int b = seq_id[i], j = pos[i];
            if (b >= 0 && b < g.batch && j >= 0 && j < g.max_blocks * kBlk) {
                const int page = g.block_table[(size_t)b * g.max_blocks + (j >> 8)];
                v = ldk(kc + kv_rowidx(g, page, kvh, j & 255) * D + d, g.k_scale);
            }
        }
        krow[tl][d] = v;
    }
    __syncthreads();
    const int tl = tid >> 4, c = tid & 15;
    const int i = i0 + tl;
    if (i >= n) return;
    const int b = seq_id[i], j = pos[i];
    if (b < 0 || b >= g.batch || j < 0 || j >= g.max_blocks * kBlk) return;
    float acc = 0.0f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc = __builtin_fmaf(krow[tl][d], wk[d * kIdx + c], acc);
    const int page = g.block_table[(size_t)b * g.max_blocks + (j >> 8)];
    k_low[(((size_t)page * g.n_ret + r) * kBlk + (j & 255)) * kIdx + c] = f2bf(acc);
}

template <typename T, typename TK, int D>
__global__ __launch_bounds__(64) void k_append_few(Geo g, const TK* __restrict__ kc, bf16_t* __restrict__ k_low,
                                                   const T* __restrict__ w_k, const int32_t* __restrict__ seq_id,
                                                   const int32_t* __restrict__ pos) {
    // grid (n, ceil(num_ret / 4)): lane 16 h + c serves retrieval head 4 blockIdx.y + h;
    // seq_id == nullptr: token i is sequence i's last position (a decode step)
    const int lane = threadIdx.x;
    const int i = blockIdx.x;
    const int r = blockIdx.y * 4 + (lane >> 4), c = lane & 15;
    if (r >= g.n_ret) return;
    const int b = seq_id ? seq_id[i] : i, j = seq_id ? pos[i] : seq_len(g, i) - 1;
    if (b < 0 || b >= g.batch || j < 0 || j >= g.max_blocks * kBlk) return;
    const int page = g.block_table[(size_t)b * g.max_blocks + (j >> 8)];
    const int kvh = g.ret_heads[r] / g.group;
    const TK* kr = kc + kv_rowidx(g, page, kvh, j & 255) * D;
    const T* wc = w_k + (size_t)r * D * kIdx + c;
    float kv[D], wv[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        kv[d] = ldk(kr + d, g.k_scale);
        wv[d] = ld(wc + d * kIdx);
    }
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) acc = __builtin_fmaf(kv[d], wv[d], acc);
    k_low[(((size_t)page * g.n_ret + r) * kBlk + (j & 255)) * kIdx + c] = f2bf(acc);
}

template <typename T, typename TK, int D>
hipError_t append(const Geo& g, const void* k, void* k_low, const void* w_k, const int32_t* seq_id,
                  const int32_t* pos, int n, hipStream_t s) {
    if (n <= 256 || !seq_id)          // no seq_id: the last positions of a decode step
        hipLaunchKernelGGL((k_append_few<T, TK, D>), dim3((unsigned)n, (g.n_ret + 3) / 4), dim3(64), 0, s, g,
                           (const TK*)k, (bf16_t*)k_low, (const T*)w_k, seq_id, pos);
    else
        hipLaunchKernelGGL((k_append<T, TK, D>), dim3((unsigned)((n + 15) / 16), g.n_ret), dim3(256), 0, s, g,
                           (const TK*)k, (bf16_t*)k_low, (const T*)w_k, seq_id, pos, n);
    return hipGetLastError();
}

// K/V append with the indexer keys (the cache-side half of the method: the
// full K/V of the KV heads that serve a retrieval head, a window-only ring
// for the rest, and the 16-dim indexer key of every retrieval head written in
// the same launch).  grid (ceil(n / 16), num_ret + 1), 256 threads: workgroup
// y < num_ret computes retrieval head y's indexer keys of 16 tokens from the
// new K rows (the chain of k_append: d ascending from +0, one bf16 rounding);
// workgroup y = num_ret stores the 16 tokens' K and V rows of every KV head in
// 16-byte pieces.
template <typename T, typename TKV, int D>
__global__ __launch_bounds__(256) void k_kv_append(Geo g, const TKV* __restrict__ k_new,
                                                   const TKV* __restrict__ v_new, TKV* __restrict__ kc,
                                                   TKV* __restrict__ vc, bf16_t* __restrict__ k_low,
                                                   const T* __restrict__ w_k,
                                                   const int32_t* __restrict__ seq_id,
                                                   const int32_t* __restrict__ pos, int n) {
    const int tid = threadIdx.x;
    const int i0 = blockIdx.x * 16;
    const auto valid = [&](int b, int j) { return b >= 0 && b < g.batch && j >= 0 && j < g.max_blocks * kBlk; };
    if ((int)blockIdx.y == g.n_ret) {
        constexpr int V = 16 / sizeof(TKV);               // elements per 16-byte piece
        constexpr int PR = D / V;                         // pieces per row
        const int per_tok = g.Hkv * PR;
        for (int x = tid; x < 16 * per_tok; x += 256) {
            const int tl = x / per_tok, rem = x - tl * per_tok;
            const int kvh = rem / PR, pc = rem - kvh * PR;
            const int i = i0 + tl;
            if (i >= n) break;
            const int b = seq_id[i], j = pos[i];
            if (!valid(b, j)) continue;
            const size_t src = ((size_t)i * g.Hkv + kvh) * D + (size_t)pc * V;
            const size_t dst = kv_rowidx(g, kv_page(g, b, kvh, j >> 8), kvh, j & 255) * D + (size_t)pc * V;
            TKV* kd = g.kv_ring[kvh] ? (TKV*)g.k_ring : kc;
            TKV* vd = g.kv_ring[kvh] ? (TKV*)g.v_ring : vc;
            *reinterpret_cast<uint4*>(kd + dst) = *reinterpret_cast<const uint4*>(k_new + src);
            *reinterpret_cast<uint4*>(vd + dst) = *reinterpret_cast<const uint4*>(v_new + src);
        }
        return;
    }
    __shared__ float krow[16][D];
    __shared__ float wk[D * kIdx];
    const int r = blockIdx.y;
    const int kvh = g.ret_heads[r] / g.group;
    for (int x = tid; x < D * kIdx; x += 256) wk[x] = ld(w_k + (size_t)r * D * kIdx + x);
    for (int x = tid; x < 16 * D; x += 256) {
        const int tl = x / D, d = x % D;
        const int i = i0 + tl;
        krow[tl][d] = i < n ? ldk(k_new + ((size_t)i * g.Hkv + kvh) * D + d, g.k_scale) : 0.0f;
    }
    __syncthreads();
    const int tl = tid >> 4, c = tid & 15;
    const int i = i0 + tl;
    if (i >= n) return;
    const int b = seq_id[i], j = pos[i];
    if (!valid(b, j)) return;
    float acc = 0.0f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc = __builtin_fmaf(krow[tl][d], wk[d * kIdx + c], acc);
    const int page = g.block_table[(size_t)b * g.max_blocks + (j >> 8)];
    k_low[(((size_t)page * g.n_ret + r) * kBlk + (j & 255)) * kIdx + c] = f2bf(acc);
}

template <typename T, typename TKV, int D>
hipError_t kv_append(const Geo& g, const void* k_new, const void* v_new, void* k, void* v, void* k_low,
                     const void* w_k, const int32_t* seq_id, const int32_t* pos, int n, hipStream_t s) {
    hipLaunchKernelGGL((k_kv_append<T, TKV, D>), dim3((unsigned)((n + 15) / 16), g.n_ret + 1), dim3(256), 0, s, g,
                       (const TKV*)k_new, (const TKV*)v_new, (TKV*)k, (TKV*)v, (bf16_t*)k_low, (const T*)w_k, seq_id,
                       pos, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const Geo& g, const void* k_new, const void* v_new, void* k, void* v, void* k_low,
                            const void* w_k, const int32_t* seq_id, const int32_t* pos, int n, int dtype,
                            hipStream_t s) {
    if (g.kv_fp8 && g.D == 64)
        return kv_append<bf16_t, fp8e4_t, 64>(g, k_new, v_new, k, v, k_low, w_k, seq_id, pos, n, s);
    if (g.kv_fp8) return kv_append<bf16_t, fp8e4_t, 128>(g, k_new, v_new, k, v, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 0 && g.D == 64) return kv_append<float, float, 64>(g, k_new, v_new, k, v, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 0 && g.D == 128)
        return kv_append<float, float, 128>(g, k_new, v_new, k, v, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 1 && g.D == 64)
        return kv_append<bf16_t, bf16_t, 64>(g, k_new, v_new, k, v, k_low, w_k, seq_id, pos, n, s);
    return kv_append<bf16_t, bf16_t, 128>(g, k_new, v_new, k, v, k_low, w_k, seq_id, pos, n, s);
}

hipError_t launch_indexer_append_last(const Geo& g, const void* k, void* k_low, const void* w_k, int dtype,
                                      hipStream_t s) {
    return launch_indexer_append(g, k, k_low, w_k, nullptr, nullptr, g.batch, dtype, s);
}

hipError_t launch_indexer_append(const Geo& g, const void* k, void* k_low, const void* w_k,
                                 const int32_t* seq_id, const int32_t* pos, int n, int dtype,
                                 hipStream_t s) {
    if (g.kv_fp8 && g.D == 64) return append<bf16_t, fp8e4_t, 64>(g, k, k_low, w_k, seq_id, pos, n, s);
    if (g.kv_fp8) return append<bf16_t, fp8e4_t, 128>(g, k, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 0 && g.D == 64) return append<float, float, 64>(g, k, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 0 && g.D == 128) return append<float, float, 128>(g, k, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 1 && g.D == 64) return append<bf16_t, bf16_t, 64>(g, k, k_low, w_k, seq_id, pos, n, s);
    return append<bf16_t, bf16_t, 128>(g, k, k_low, w_k, seq_id, pos, n, s);
}

}  // namespace rtp
