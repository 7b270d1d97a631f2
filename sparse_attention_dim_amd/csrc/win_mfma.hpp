// win_mfma.hpp -- local-head (window + sinks) and dense decode attention on
// gfx950 bf16 MFMA, D = 128: the work item of one wavefront, shared by the
// window decode kernel and the decode step's row pass, which runs these items
// on the CUs its selection leaves free.
//
// Method: arXiv 2605.16928 abstract obs. (1) (the heads that are not
// retrieval heads use a restricted window); zhichai.net forum post "RTPurbo:
// Turning Dense LLMs into Sparse Attention Models ...", "Three Key Insights"
// item 1 (local heads keep only a local window).
#pragma once
#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

__device__ __forceinline__ size_t kv_off(const Geo& g, int page, int kvh, int slot, int D) {
    return kv_rowidx(g, page, kvh, slot) * (size_t)D;
}

// Keys of a local head's row at position pos: sinks 0..ns_end-1, then the
// window w_start..pos (dense: every key).
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

// ---------------------------------------------------------------------------
// Local-head (or dense) decode on bf16 MFMA, D = 128: one wavefront per
// (sequence, KV head, split).  The query heads of the KV group are the 32
// columns of v_mfma_f32_32x32x16_bf16 (heads that do not need the kernel are
// zero columns), so every K/V row is read once for the group.  Per block of 32
// keys: S^T[key][head] = K . Q^T with the K rows straight from memory (each
// lane one key, 16 bytes per k-step); online softmax per head in-lane (a lane
// holds 16 of the block's keys of its head, the other half-wave the other 16);
// O^T[d][head] += V^T . P^T with V^T read by gfx950's transposing LDS loads
// from the block's row-major V tile (16-byte row stores) and P^T taken
// straight from the S^T registers (a fixed key permutation matches their
// layout).  Writes the same partials as k_win_dec_part.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kWVsLd = 128 + 32;   // V row stride in LDS (bf16), 320 B: the four rows of a transposing load hit disjoint banks

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Wave-local ordering of the item's LDS accesses: a barrier of the whole
// workgroup when the item is the workgroup (one wavefront), else of the
// wavefront only (items of other wavefronts run independently).
template <bool kInWave>
__device__ __forceinline__ void item_sync() {
    if (kInWave) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        __syncthreads();
    }
}

// One work item: split `split` of (sequence, KV head) bkv = b * Hkv + kvh, on
// one wavefront (lane = threadIdx.x % 64); pgs (64 ints) and Vs (32 x kWVsLd
// bf16) are the wavefront's own LDS.
template <bool kInWave>
__device__ __forceinline__ void win_mfma_item(const Geo& g, const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc_main,
                              const bf16_t* __restrict__ vc_main, float* __restrict__ part, int nsplit,
                              int split_keys, int dense, int split, int bkv, int* pgs, bf16_t* Vs) {
    constexpr int D = 128;
    const int lane = threadIdx.x & 63, hh = lane >> 5, col = lane & 31;
    const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
    // K/V of this KV head: the paged cache, or the window-only ring
    const bf16_t* __restrict__ kc = g.kv_ring[kvh] ? (const bf16_t*)g.k_ring : kc_main;
    const bf16_t* __restrict__ vc = g.kv_ring[kvh] ? (const bf16_t*)g.v_ring : vc_main;
    const int pos = seq_len(g, b) - 1;
    int ns_end, w_start;
    const int n_all = win_count(g, pos, dense, &ns_end, &w_start);
    const int v0 = split * split_keys;
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
    const int vS1 = min(v0 + n, ns_end);
    const int pS0 = v0 >> 8;
    const int nPS = vS1 > v0 ? ((vS1 - 1) >> 8) - pS0 + 1 : 0;
    const int jW0 = w_start + max(v0, ns_end) - ns_end;
    const int jW1 = w_start + (v0 + n) - ns_end;
    const int pW0 = jW0 >> 8;
    const int nPW = jW1 > jW0 ? ((jW1 - 1) >> 8) - pW0 + 1 : 0;
    if (lane < nPS) pgs[lane] = kv_page(g, b, kvh, pS0 + lane);
    else if (lane < nPS + nPW) pgs[lane] = kv_page(g, b, kvh, pW0 + lane - nPS);
    item_sync<kInWave>();
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
    const float sc = g.attn_scale * 1.4426950408889634f;   // log2(e): exp2 below
    f32x16_t oacc[4];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dd][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    // this lane's key row of a block: K for the A operand, V for the
    // transposed tile.  The next block's K rows are requested once this
    // block's S MFMAs have taken theirs, its V rows once this block's V^T
    // tile is written, so they arrive while this block finishes.
    uint4 ka[8], va[8];
    {
        const size_t ro = off(min(col, n - 1)) + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const uint4*>(kc + ro + 16 * kk);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) va[kk] = *reinterpret_cast<const uint4*>(vc + ro + 16 * kk);
    }
    for (int k0 = 0; k0 < n; k0 += 32) {
        const bool live = k0 + col < n;
        const bool more = k0 + 32 < n;
        const size_t ro_n = off(min(k0 + 32 + col, n - 1)) + 8 * hh;
        f32x16_t s;
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[kk]), as_bf16x8(qreg[kk]), s, 0, 0, 0);
        if (more) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const uint4*>(kc + ro_n + 16 * kk);
        }
        item_sync<kInWave>();                                  // the previous block's V^T reads are done
        // the block's V rows, row-major (key col, d = 16 kk + 8 hh ..); rows
        // past the split stored as zeros
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
            *reinterpret_cast<uint4*>(&Vs[col * kWVsLd + 16 * kk + 8 * hh]) = live ? va[kk] : make_uint4(0, 0, 0, 0);
        if (more) {
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) va[kk] = *reinterpret_cast<const uint4*>(vc + ro_n + 16 * kk);
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
        item_sync<kInWave>();                                  // the V tile is written
        // O^T += V^T P^T; k-step kk covers keys 16 kk + 4 hh + {0..3, 8..11}:
        // lane (d = 32 dd + col, half hh) reads V^T[d][those keys] from the
        // row-major tile by transposing loads (lane j of a 16-lane group
        // addresses key row kc0 + j / 4 (+ 8) at columns 32 dd + 16 (group &
        // 1) + 4 (j % 4))
        const int trr = (lane & 15) >> 2, trc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const uint4 bp = make_uint4(pb[4 * kk], pb[4 * kk + 1], pb[4 * kk + 2], pb[4 * kk + 3]);
            const int kc0 = 16 * kk + 4 * hh;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                const bf16_t* vr = &Vs[(kc0 + trr) * kWVsLd + 32 * dd + trc];
                const uint2 lo = lds_tr16(vr);
                const uint2 hi = lds_tr16(vr + 8 * kWVsLd);
                const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
                oacc[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bp), oacc[dd], 0, 0, 0);
            }
        }
    }
    // partials: lane holds O^T[32 dd + 8 (i/4) + 4 hh + (i%4)][head col]
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (act) {
        float* pp = part + (((size_t)b * g.Hq + hq) * nsplit + split) * (D + 2);
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

}  // namespace rtp
