// attn_sparse_prefill.hip -- sparse attention of the retrieval heads over their
// selected rows for a prefill chunk, on gfx950 bf16 MFMA.
//
// Method: arXiv 2605.16928 abstract (retrieval heads keep the full KV cache
// and attend to the rows their indexer selects); zhichai.net forum post
// "RTPurbo: Turning Dense LLMs into Sparse Attention Models ...", "Three Key
// Insights" items 2-3.  Every chunk row attends to its own selected set with
// the softmax renormalised over the set.
//
// Consecutive chunk rows of one head select largely the same keys (the
// selected sets of 32 neighbouring rows fill ~85% of their union at the
// clustered workloads).  A workgroup takes 64 rows of one retrieval head and
// computes attention over the union of their sets, one 64-key union block at
// a time, with each row's keys masked to its own set:
//   union        the rows' sorted CSR lists are merged through an LDS bitmap
//                over a 2^16-key window; popcount prefixes give the rank of
//                any key in the window's union, and the k-th union key
//   membership   per window, each row's entries are read again and their
//                union ranks set bits of the row's 64-bit masks of up to 16
//                blocks at a time (lists are read 64 entries per load, the 32
//                rows of a wave with their loads in flight together)
//   attention    the gathered K rows (row-major) and V^T (transposed) are
//                staged in LDS; S^T = K . Q^T and O^T += V^T . P^T run on
//                v_mfma_f32_32x32x16_bf16 exactly as the prefill flash
//                attention does, with masked keys at -inf.
// A workgroup takes one window of one row tile (the windows of a tile run in
// parallel); a pre-pass finds where each row's sorted list enters every
// window, and a combine pass merges the windows' partial results of each row
// in window order (a single window writes the output directly).
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 2;
constexpr int kBM = 32 * kWaves;   // rows per workgroup
constexpr int kNT = 64 * kWaves;   // threads
constexpr int kBN = 64;            // union keys per block
constexpr int kD = 128;
constexpr int kKsLd = kD + 8;      // K row stride in LDS (bf16)
constexpr int kVtLd = kBN + 4;     // V^T row stride in LDS (bf16)
constexpr int kWinLog = 16;
constexpr int kWin = 1 << kWinLog; // keys per bitmap window
constexpr int kWords = kWin / 32;
constexpr int kMB = 16;            // union blocks whose masks are held at once
constexpr int kPS = kD + 4;        // floats per partial result: O[D], max, mass (16-byte rows)

// orders this wave's LDS writes before its following LDS reads
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Where each row's sorted list enters each window: woff[row][w] = position of
// the first entry >= w * kWin, w = 0..nwin.  grid (ceil(rows / 4)), 64 threads:
// lane 16 j + w searches boundary w of row 4 blockIdx + j (w <= 16 per pass).
__global__ __launch_bounds__(64) void k_sp_winoff(const int64_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ idx, const int32_t* __restrict__ status,
                                                  int rows, int nwin, int64_t* __restrict__ woff) {
    if (*status != 0) return;
    const int lane = threadIdx.x;
    const int row = blockIdx.x * 4 + (lane >> 4);
    if (row >= rows) return;
    const int64_t b = row_ptr[row], e = row_ptr[row + 1];
    for (int w = lane & 15; w <= nwin; w += 16) {
        const int64_t bound = (int64_t)w * kWin;
        int64_t lo = b, hi = e;                       // first position with idx >= bound
        while (lo < hi) {
            const int64_t mid = lo + ((hi - lo) >> 1);
            if (idx[mid] < bound) lo = mid + 1; else hi = mid;
        }
        woff[(size_t)row * (nwin + 1) + w] = lo;
    }
}

// grid (ceil(n_tok / kBM) * nwin, n_ret), kNT threads: tile blockIdx.x / nwin,
// window blockIdx.x % nwin.
__global__ __launch_bounds__(kNT) void k_sp_prefill(Geo g, const bf16_t* __restrict__ q,
                                                   const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
                                                   const int64_t* __restrict__ woff, int nwin,
                                                   const int32_t* __restrict__ idx, const int32_t* __restrict__ status,
                                                   bf16_t* __restrict__ out, float* __restrict__ part) {
    if (*status != 0) return;
    __shared__ __attribute__((aligned(16))) bf16_t Ks[kBN * kKsLd];
    __shared__ __attribute__((aligned(16))) bf16_t Vt[kD * kVtLd];
    __shared__ uint32_t bm[kWords];                  // union bitmap of the window
    __shared__ uint32_t wpre[kWords];                // exclusive prefix of its word popcounts
    __shared__ int ukey[kBN];                        // the block's union keys
    __shared__ uint32_t memb[kMB][kBM][2];           // per block and row: 64-bit key mask
    __shared__ int64_t cur_b[kBM], cur_m[kBM], r_end[kBM];
    __shared__ unsigned long long scan_sh[kNT / 64 + 1];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int r = blockIdx.y;
    const int hq = g.ret_heads[r], kvh = hq / g.group;
    const int tile = blockIdx.x / nwin, win = blockIdx.x - tile * nwin;
    const int t0 = tile * kBM;
    const int hh = lane >> 5, qi = lane & 31;
    const int t = t0 + wid * 32 + qi;                // query row of this lane
    const bool qok = t < g.n_tok;
    const float sc = g.attn_scale * kLog2e;
    const int32_t* bt = g.block_table + (size_t)g.seq * g.max_blocks;

    __shared__ int s_any;
    if (tid == 0) s_any = 0;
    __syncthreads();
    if (tid < kBM) {
        const int tr = t0 + tid;
        int64_t b = 0, e = 0;
        if (tr < g.n_tok) {
            const size_t o = ((size_t)tr * g.n_ret + r) * (nwin + 1) + win;
            b = woff[o];
            e = woff[o + 1];
        }
        cur_b[tid] = b;
        cur_m[tid] = b;
        r_end[tid] = e;
        if (e > b) s_any = 1;
    }
    __syncthreads();
    if (!s_any) return;                               // no row of the tile has a key in this window

    // Q^T operand: lane holds Q[t][16 kk + 8 hh + 0..7] for kk = 0..7
    uint4 qreg[8];
    {
        const bf16_t* qp = q + ((size_t)min(t, g.n_tok - 1) * g.Hq + hq) * kD + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            qreg[kk] = qok ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
    }
    f32x16_t oacc[4];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dd][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    {
        const int w0 = win * kWin, w1 = w0 + kWin;
        for (int x = tid; x < kWords; x += kNT) bm[x] = 0u;
        __syncthreads();
        // ---- union bitmap of the window: each wave walks its rows' lists, 64
        // entries per load, the 32 rows' loads in flight together, until every
        // row reaches an entry past the window
        for (;;) {
            int keys[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int row = wid * 32 + i;
                const int64_t p = cur_b[row] + lane;
                keys[i] = p < r_end[row] ? idx[p] : INT32_MAX;
            }
            bool more = false;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const bool in = keys[i] < w1;
                if (in) atomicOr(&bm[(keys[i] - w0) >> 5], 1u << ((keys[i] - w0) & 31));
                const int n = __popcll(__ballot(in));
                more = more || n == 64;
                if (lane == 0) cur_b[wid * 32 + i] += n;
            }
            wave_lds_fence();
            if (!more) break;
        }
        __syncthreads();
        // ---- word popcount prefix
        {
            constexpr int per = kWords / kNT;
            uint32_t cnt[per];
            uint32_t loc = 0;
#pragma unroll
            for (int k = 0; k < per; ++k) {
                cnt[k] = __popc(bm[tid * per + k]);
                loc += cnt[k];
            }
            unsigned long long tot;
            uint32_t ex = (uint32_t)block_excl_scan_u64<kNT>(loc, &tot, scan_sh);
#pragma unroll
            for (int k = 0; k < per; ++k) {
                wpre[tid * per + k] = ex;
                ex += cnt[k];
            }
            if (tid == 0) scan_sh[kNT / 64] = tot;
        }
        __syncthreads();
        const int nU = (int)scan_sh[kNT / 64];
        // ---- union blocks of the window, kMB at a time
        for (int g0 = 0; g0 < nU; g0 += kMB * kBN) {
            const int gend = min(nU, g0 + kMB * kBN);
            __syncthreads();
            for (int x = tid; x < kMB * kBM * 2; x += kNT) (&memb[0][0][0])[x] = 0u;
            __syncthreads();
            // membership masks of the group's blocks: entries with union rank < gend
            for (;;) {
                int keys[32];
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    const int row = wid * 32 + i;
                    const int64_t p = cur_m[row] + lane;
                    keys[i] = p < r_end[row] ? idx[p] : INT32_MAX;
                }
                bool more = false;
#pragma unroll
                for (int i = 0; i < 32; ++i) {
                    int rank = INT32_MAX;
                    if (keys[i] < w1) {
                        const int off = keys[i] - w0;
                        const int wd = off >> 5;
                        rank = (int)(wpre[wd] + __popc(bm[wd] & ((1u << (off & 31)) - 1u)));
                    }
                    const bool in = rank < gend;
                    if (in) {
                        const int lr = rank - g0;
                        atomicOr(&memb[lr >> 6][wid * 32 + i][(lr >> 5) & 1], 1u << (lr & 31));
                    }
                    const int n = __popcll(__ballot(in));
                    more = more || n == 64;
                    if (lane == 0) cur_m[wid * 32 + i] += n;
                }
                wave_lds_fence();
                if (!more) break;
            }
        for (int u0 = g0; u0 < gend; u0 += kBN) {
            __syncthreads();                          // the previous block's LDS reads are done
            const int nb = min(kBN, nU - u0);
            if (tid < kBN) {
                int key = -1;
                if (tid < nb) {
                    // the word holding union rank u0 + tid: the last word whose prefix is <= it
                    const uint32_t want = (uint32_t)(u0 + tid);
                    int lo = 0, hi = kWords - 1;
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (wpre[mid] <= want) lo = mid; else hi = mid - 1;
                    }
                    uint32_t bits = bm[lo];
                    for (uint32_t k = want - wpre[lo]; k > 0; --k) bits &= bits - 1u;
                    key = w0 + lo * 32 + (__ffs(bits) - 1);
                }
                ukey[tid] = key;
            }
            __syncthreads();
            // ---- K rows and V^T of the block's keys into LDS, in two halves of the
            // block (a thread per quarter row)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int kk = 32 * hb + (tid >> 2), qq = tid & 3;
                const int key = ukey[kk];
                uint4 kr[4], vr[4];
                if (key >= 0) {
                    const int page = bt[key >> 8];
                    const size_t base = (((size_t)page * g.Hkv + kvh) * kBlk + (key & 255)) * kD + 32 * qq;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kr[j] = reinterpret_cast<const uint4*>(kc + base)[j];
                        vr[j] = reinterpret_cast<const uint4*>(vc + base)[j];
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        kr[j] = make_uint4(0, 0, 0, 0);
                        vr[j] = make_uint4(0, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 32 * qq + 8 * j;
                    *reinterpret_cast<uint4*>(&Ks[kk * kKsLd + c]) = kr[j];
                    const uint32_t w[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        Vt[(c + 2 * x) * kVtLd + kk] = (bf16_t)(w[x] & 0xFFFFu);
                        Vt[(c + 2 * x + 1) * kVtLd + kk] = (bf16_t)(w[x] >> 16);
                    }
                }
            }
            __syncthreads();
            const int bl = (u0 - g0) >> 6;
            const unsigned long long mask = ((unsigned long long)memb[bl][wid * 32 + qi][1] << 32) |
                                            (unsigned long long)memb[bl][wid * 32 + qi][0];

            // ---- S^T for the two 32-key halves of the block
            f32x16_t s[2];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[sh][i] = 0.0f;
                const bf16_t* krow = &Ks[(32 * sh + qi) * kKsLd + 8 * hh];
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const uint4 a = *reinterpret_cast<const uint4*>(krow + 16 * kk);
                    s[sh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[kk]), s[sh], 0, 0, 0);
                }
            }
            // scale, mask, block maximum of this lane's query
            float mt = -INFINITY;
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kp = 32 * sh + (i >> 2) * 8 + 4 * hh + (i & 3);
                    const bool ok = qok && ((mask >> kp) & 1ull);
                    const float v = ok ? s[sh][i] * sc : -INFINITY;
                    s[sh][i] = v;
                    mt = fmaxf(mt, v);
                }
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt);
            uint32_t pb[2][8];                        // P^T as bf16 pairs, per half and kk
            if (m_new == -INFINITY) {
#pragma unroll
                for (int sh = 0; sh < 2; ++sh)
#pragma unroll
                    for (int x = 0; x < 8; ++x) pb[sh][x] = 0u;
            } else {
                const float corr = exp2f(m_run - m_new);
                m_run = m_new;
                l_run *= corr;
#pragma unroll
                for (int dd = 0; dd < 4; ++dd)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[dd][i] *= corr;
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
                    float p[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        p[i] = exp2f(s[sh][i] - m_new);
                        l_run += p[i];
                    }
#pragma unroll
                    for (int x = 0; x < 8; ++x) pb[sh][x] = pack2(p[2 * x], p[2 * x + 1]);
                }
            }
            // O^T += V^T P^T
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const uint4 bp = make_uint4(pb[sh][4 * kk], pb[sh][4 * kk + 1], pb[sh][4 * kk + 2], pb[sh][4 * kk + 3]);
                    const int kc0 = 32 * sh + 16 * kk + 4 * hh;
#pragma unroll
                    for (int dd = 0; dd < 4; ++dd) {
                        const bf16_t* vrp = &Vt[(32 * dd + qi) * kVtLd + kc0];
                        const uint2 lo = *reinterpret_cast<const uint2*>(vrp);
                        const uint2 hi = *reinterpret_cast<const uint2*>(vrp + 8);
                        const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
                        oacc[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bp), oacc[dd], 0, 0, 0);
                    }
                }
            }
        }
        }
    }
    // lane holds O[t][32 dd + 8 (i/4) + 4 hh + (i%4)]
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (nwin > 1) {
        // partial of this window: unnormalised O, the running maximum and mass
        if (qok) {
            float* pp = part + (((size_t)t * g.n_ret + r) * nwin + win) * kPS;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d0 = 32 * dd + 8 * r4 + 4 * hh;
                    *reinterpret_cast<float4*>(pp + d0) =
                        make_float4(oacc[dd][4 * r4], oacc[dd][4 * r4 + 1], oacc[dd][4 * r4 + 2], oacc[dd][4 * r4 + 3]);
                }
            if (hh == 0) {
                pp[kD] = m_run;
                pp[kD + 1] = l_tot;
            }
        }
        return;
    }
    if (qok && l_tot > 0.0f) {
        const float inv = 1.0f / l_tot;
        bf16_t* op = out + ((size_t)t * g.Hq + hq) * kD;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * dd + 8 * r4 + 4 * hh;
                uint2 v;
                v.x = pack2(oacc[dd][4 * r4 + 0] * inv, oacc[dd][4 * r4 + 1] * inv);
                v.y = pack2(oacc[dd][4 * r4 + 2] * inv, oacc[dd][4 * r4 + 3] * inv);
                *reinterpret_cast<uint2*>(op + d0) = v;
            }
        }
    }
}

// Merge of the windows' partials of each row, in window order.  grid (ceil(rows / 2)), 128 threads:
// a row per 64 lanes, two output elements per lane.
__global__ __launch_bounds__(128) void k_sp_combine(Geo g, const int64_t* __restrict__ woff, int nwin,
                                                   const float* __restrict__ part, const int32_t* __restrict__ status,
                                                   bf16_t* __restrict__ out) {
    if (*status != 0) return;
    const int row = blockIdx.x * 2 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int rows = g.n_tok * g.n_ret;
    if (row >= rows) return;
    const int t = row / g.n_ret, r = row - t * g.n_ret;
    const int64_t* wo = woff + (size_t)row * (nwin + 1);
    const float* pr = part + (size_t)row * nwin * kPS;
    float M = -INFINITY;
    for (int w = 0; w < nwin; ++w)
        if (wo[w + 1] > wo[w]) M = fmaxf(M, pr[(size_t)w * kPS + kD]);
    float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int w = 0; w < nwin; ++w) {
        if (wo[w + 1] <= wo[w]) continue;
        const float* pw = pr + (size_t)w * kPS;
        const float f = exp2f(pw[kD] - M);
        l += pw[kD + 1] * f;
        o0 += pw[2 * lane] * f;
        o1 += pw[2 * lane + 1] * f;
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    *reinterpret_cast<uint32_t*>(out + ((size_t)t * g.Hq + g.ret_heads[r]) * kD + 2 * lane) = pack2(o0 * inv, o1 * inv);
}

}  // namespace

int sparse_prefill_windows(int n_keys) { return (n_keys + kWin - 1) / kWin; }

size_t sparse_prefill_ws_bytes(int rows, int n_keys) {
    const int nwin = sparse_prefill_windows(n_keys);
    size_t b = ((size_t)rows * (nwin + 1) * 8 + 255) / 256 * 256;
    if (nwin > 1) b += (size_t)rows * nwin * kPS * 4;
    return b;
}

hipError_t launch_sparse_prefill(const Geo& g, const void* q, const void* k, const void* v, const int64_t* row_ptr,
                                 const int32_t* idx, const int32_t* status, void* out, void* ws, hipStream_t s) {
    const int rows = g.n_tok * g.n_ret;
    const int nwin = sparse_prefill_windows(g.pos0 + g.n_tok);
    int64_t* woff = (int64_t*)ws;
    float* part = (float*)((char*)ws + ((size_t)rows * (nwin + 1) * 8 + 255) / 256 * 256);
    hipLaunchKernelGGL(k_sp_winoff, dim3((rows + 3) / 4), dim3(64), 0, s, row_ptr, idx, status, rows, nwin, woff);
    const dim3 grid(((g.n_tok + kBM - 1) / kBM) * nwin, g.n_ret);
    hipLaunchKernelGGL(k_sp_prefill, grid, dim3(kNT), 0, s, g, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                       woff, nwin, idx, status, (bf16_t*)out, part);
    if (nwin > 1)
        hipLaunchKernelGGL(k_sp_combine, dim3((rows + 1) / 2), dim3(128), 0, s, g, woff, nwin, part, status,
                           (bf16_t*)out);
    return hipGetLastError();
}

}  // namespace rtp
