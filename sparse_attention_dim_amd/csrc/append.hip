// append.hip -- indexer key append on gfx950: the 16-dim indexer key of every
// newly cached token and retrieval head (arXiv 2605.16928 abstract obs. (2),
// "16-dimensional indexer"; zhichai.net forum post "RTPurbo: Turning Dense LLMs
// into Sparse Attention Models ...", "Three Key Insights" item 2).
//
// One thread per output (token, retrieval head, c): an fp32 FMA chain over the
// head dimension, d ascending from +0, rounded once to bf16.  A workgroup of
// 256 threads covers 16 (token, head) pairs; the key rows it needs are staged
// in LDS so each is read from HBM once.
#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void k_append(Geo g, const T* __restrict__ kc, bf16_t* __restrict__ k_low,
                                                const T* __restrict__ w_k, const int32_t* __restrict__ seq_id,
                                                const int32_t* __restrict__ pos, int n) {
    __shared__ float krow[16][D];
    const int tid = threadIdx.x;
    const int pair0 = blockIdx.x * 16;                 // (token, head) pairs of this workgroup
    const int npairs = n * g.n_ret;
    // stage the 16 key rows
    for (int x = tid; x < 16 * D; x += 256) {
        const int pl = x / D, d = x % D;
        const int pr = pair0 + pl;
        float v = 0.0f;
        if (pr < npairs) {
            const int i = pr / g.n_ret, r = pr % g.n_ret;
            const int b = seq_id[i], j = pos[i];
            if (b < 0 || b >= g.batch || j < 0 || j >= g.max_blocks * kBlk) continue;
            const int page = g.block_table[(size_t)b * g.max_blocks + (j >> 8)];
            const int kvh = g.ret_heads[r] / g.group;
            v = ld(kc + (((size_t)page * g.Hkv + kvh) * kBlk + (j & 255)) * D + d);
        }
        krow[pl][d] = v;
    }
    __syncthreads();
    const int pl = tid >> 4, c = tid & 15;
    const int pr = pair0 + pl;
    if (pr >= npairs) return;
    const int i = pr / g.n_ret, r = pr % g.n_ret;
    const T* wp = w_k + (size_t)r * D * kIdx + c;
    float acc = 0.0f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) acc = __builtin_fmaf(krow[pl][d], ld(wp + d * kIdx), acc);
    const int b = seq_id[i], j = pos[i];
    if (b < 0 || b >= g.batch || j < 0 || j >= g.max_blocks * kBlk) return;
    const int page = g.block_table[(size_t)b * g.max_blocks + (j >> 8)];
    k_low[(((size_t)page * g.n_ret + r) * kBlk + (j & 255)) * kIdx + c] = f2bf(acc);
}

template <typename T, int D>
hipError_t append(const Geo& g, const void* k, void* k_low, const void* w_k, const int32_t* seq_id,
                  const int32_t* pos, int n, hipStream_t s) {
    const int64_t pairs = (int64_t)n * g.n_ret;
    const int64_t blocks = (pairs + 15) / 16;
    hipLaunchKernelGGL((k_append<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, g, (const T*)k,
                       (bf16_t*)k_low, (const T*)w_k, seq_id, pos, n);
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
