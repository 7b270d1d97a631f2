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
// operands in registers, which shortens the dependent path.
#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_append(Geo g, const T* __restrict__ kc, bf16_t* __restrict__ k_low,
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
                v = ld(kc + (((size_t)page * g.Hkv + kvh) * kBlk + (j & 255)) * D + d);
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

template <typename T, int D>
__global__ __launch_bounds__(64) void k_append_few(Geo g, const T* __restrict__ kc, bf16_t* __restrict__ k_low,
                                                   const T* __restrict__ w_k, const int32_t* __restrict__ seq_id,
                                                   const int32_t* __restrict__ pos) {
    // grid (n, ceil(num_ret / 4)): lane 16 h + c serves retrieval head 4 blockIdx.y + h
    const int lane = threadIdx.x;
    const int i = blockIdx.x;
    const int r = blockIdx.y * 4 + (lane >> 4), c = lane & 15;
    if (r >= g.n_ret) return;
    const int b = seq_id[i], j = pos[i];
    if (b < 0 || b >= g.batch || j < 0 || j >= g.max_blocks * kBlk) return;
    const int page = g.block_table[(size_t)b * g.max_blocks + (j >> 8)];
    const int kvh = g.ret_heads[r] / g.group;
    const T* kr = kc + (((size_t)page * g.Hkv + kvh) * kBlk + (j & 255)) * D;
    const T* wc = w_k + (size_t)r * D * kIdx + c;
    float kv[D], wv[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        kv[d] = ld(kr + d);
        wv[d] = ld(wc + d * kIdx);
    }
    float acc = 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) acc = __builtin_fmaf(kv[d], wv[d], acc);
    k_low[(((size_t)page * g.n_ret + r) * kBlk + (j & 255)) * kIdx + c] = f2bf(acc);
}

template <typename T, int D>
hipError_t append(const Geo& g, const void* k, void* k_low, const void* w_k, const int32_t* seq_id,
                  const int32_t* pos, int n, hipStream_t s) {
    if (n <= 256)
        hipLaunchKernelGGL((k_append_few<T, D>), dim3((unsigned)n, (g.n_ret + 3) / 4), dim3(64), 0, s, g,
                           (const T*)k, (bf16_t*)k_low, (const T*)w_k, seq_id, pos);
    else
        hipLaunchKernelGGL((k_append<T, D>), dim3((unsigned)((n + 15) / 16), g.n_ret), dim3(256), 0, s, g,
                           (const T*)k, (bf16_t*)k_low, (const T*)w_k, seq_id, pos, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_append(const Geo& g, const void* k, void* k_low, const void* w_k,
                                 const int32_t* seq_id, const int32_t* pos, int n, int dtype,
                                 hipStream_t s) {
    if (dtype == 0 && g.D == 64) return append<float, 64>(g, k, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 0 && g.D == 128) return append<float, 128>(g, k, k_low, w_k, seq_id, pos, n, s);
    if (dtype == 1 && g.D == 64) return append<bf16_t, 64>(g, k, k_low, w_k, seq_id, pos, n, s);
    return append<bf16_t, 128>(g, k, k_low, w_k, seq_id, pos, n, s);
}

}  // namespace rtp
