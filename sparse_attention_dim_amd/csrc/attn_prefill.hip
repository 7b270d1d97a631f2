// attn_prefill.hip -- chunked-prefill attention of the local heads (sinks +
// causal sliding window) and dense causal attention, on gfx950 bf16 MFMA.
//
// Method: arXiv 2605.16928 abstract obs. (1) (most heads use a restricted
// window); zhichai.net forum post "RTPurbo: Turning Dense LLMs into Sparse
// Attention Models ...", "Three Key Insights" item 1.  Dense causal attention
// is the same-GPU baseline of the speedup.
//
// Flash attention, one workgroup per (128 query rows, query head), four
// wavefronts of 32 rows.  Per 64-key tile:
//   S^T[key][q] = K . Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                            B = Q^T held in registers (each lane one query)
//   online softmax           in-lane: a lane holds 16 keys of one query; the
//                            two half-waves hold the other 16 (one xor-32 swap)
//   O^T[d][q] += V^T . P^T   A = V^T read from the row-major V tile in LDS by
//                            transposing loads (ds_read_b64_tr_b16), B = P^T
//                            taken straight from the S^T registers
// The key order inside the second product is a fixed permutation that matches
// the register layout of S^T, so P never moves between lanes.  A 64-key tile
// of one KV head is one contiguous 16 KiB run of a page (pages hold 256 keys).
#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"

namespace rtp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBM = 128;           // query rows per workgroup
constexpr int kBN = 64;            // keys per tile
constexpr int kD = 128;            // head dim of this kernel
constexpr int kKsLd = kD + 8;      // K row stride in LDS (bf16), 272 B: conflict-free row reads
constexpr int kVsLd = kD + 32;     // V row stride in LDS (bf16), 320 B: the four rows of a transposing load hit disjoint banks

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

struct TileRange {
    int a0, a1;    // first run of tiles [a0, a1) (sinks), key positions
    int b0, b1;    // second run [b0, b1) (window / causal), key positions
};

__device__ __forceinline__ TileRange tile_range(const Geo& g, int p_min, int p_max, int dense) {
    TileRange r;
    if (dense) {
        r.a0 = 0;
        r.a1 = 0;
        r.b0 = 0;
        r.b1 = p_max + 1;
        return r;
    }
    r.a0 = 0;
    r.a1 = min(((g.sinks + kBN - 1) / kBN) * kBN, p_max + 1);
    int lo = max(p_min - g.window + 1, 0);
    lo = (lo / kBN) * kBN;
    r.b0 = max(lo, r.a1);
    r.b1 = p_max + 1;
    if (r.b0 >= r.b1) r.b0 = r.b1;
    return r;
}

// grid (ceil(n_tok / kBM), n_heads): heads[] lists the query heads to compute.
__global__ __launch_bounds__(256) void k_fa_prefill(Geo g, const bf16_t* __restrict__ q,
                                                    const bf16_t* __restrict__ kc_main,
                                                    const bf16_t* __restrict__ vc_main, bf16_t* __restrict__ out,
                                                    int dense) {
    __shared__ __attribute__((aligned(16))) bf16_t Ks[kBN * kKsLd];
    __shared__ __attribute__((aligned(16))) bf16_t Vs[kBN * kVsLd];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int hq = g.hlist[blockIdx.y];
    const int kvh = hq / g.group;
    // K/V of this KV head: the paged cache, or the window-only ring
    const bf16_t* __restrict__ kc = g.kv_ring[kvh] ? (const bf16_t*)g.k_ring : kc_main;
    const bf16_t* __restrict__ vc = g.kv_ring[kvh] ? (const bf16_t*)g.v_ring : vc_main;
    const int t0 = blockIdx.x * kBM;
    const int n_valid = min(kBM, g.n_tok - t0);
    const int p_min = g.pos0 + t0, p_max = g.pos0 + t0 + n_valid - 1;
    const int hh = lane >> 5;                        // half-wave
    const int qi = lane & 31;                        // query of this lane within the wave
    const int t = t0 + wid * 32 + qi;                // query row
    const bool qok = t < g.n_tok;
    const int pq = g.pos0 + t;                       // its position
    const float sc = g.attn_scale * kLog2e;
    // positions of the wave's 32 queries (all of them valid: wave_full)
    const int wt0 = t0 + wid * 32;
    const bool wave_full = wt0 + 31 < g.n_tok;
    const int wp_min = g.pos0 + wt0, wp_max = wp_min + 31;

    // Q^T operand: lane holds Q[t][16 kk + 8 hh + 0..7] for kk = 0..7
    uint4 qreg[8];
    {
        const bf16_t* qp = q + ((size_t)min(t, g.n_tok - 1) * g.Hq + hq) * kD + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qreg[kk] = qok ? *reinterpret_cast<const uint4*>(qp + 16 * kk)
                                                      : make_uint4(0, 0, 0, 0);
    }
    f32x16_t oacc[4];
#pragma unroll
    for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dd][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const TileRange tr = tile_range(g, p_min, p_max, dense);
    const int na = (tr.a1 - tr.a0 + kBN - 1) / kBN;
    const int nb = (tr.b1 - tr.b0 + kBN - 1) / kBN;
    const int ntiles = na + nb;

    // tile loads: 16 KiB of K and of V per tile, four 16-byte vectors per thread each
    auto tile_key0 = [&](int it) { return it < na ? tr.a0 + it * kBN : tr.b0 + (it - na) * kBN; };
    // the 16-byte pieces of a tile this thread loads: element offsets of the
    // K and V tile starts (the tile is one contiguous run of a page)
    auto tile_base = [&](int it) {
        const int k0 = tile_key0(it);
        return kv_rowidx(g, kv_page(g, g.seq, kvh, k0 >> 8), kvh, k0 & 255) * kD;
    };
    uint4 kk0, kk1, kk2, kk3, vv0, vv1, vv2, vv3;
#define RTP_LOAD_TILE(b)                                                            \
    {                                                                               \
        const uint4* kp = reinterpret_cast<const uint4*>(kc + (b)) + tid;           \
        const uint4* vp = reinterpret_cast<const uint4*>(vc + (b)) + tid;           \
        kk0 = kp[0]; kk1 = kp[256]; kk2 = kp[512]; kk3 = kp[768];                   \
        vv0 = vp[0]; vv1 = vp[256]; vv2 = vp[512]; vv3 = vp[768];                   \
    }
    if (ntiles > 0) RTP_LOAD_TILE(tile_base(0))

    for (int it = 0; it < ntiles; ++it) {
        const int k0 = tile_key0(it);
        __syncthreads();                              // previous tile's LDS reads are done
        {
            // thread piece j: element (tid + 256 j) * 8 of the 64 x 128 tile,
            // row tid / 16 + 16 j, column (tid % 16) * 8.  Keys past the last
            // query position may be unwritten cache slots: their V rows are
            // stored as zeros so that p = 0 never meets a non-finite value.
            const int r = tid >> 4, c = (tid & 15) * 8;
            // (an AND mask, not a select: a select of two vectors may be
            // lowered through scratch memory)
            const auto keep = [&](const uint4& x, int key) {
                const uint32_t m = key <= p_max ? ~0u : 0u;
                return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
            };
            *reinterpret_cast<uint4*>(&Ks[r * kKsLd + c]) = kk0;
            *reinterpret_cast<uint4*>(&Ks[(r + 16) * kKsLd + c]) = kk1;
            *reinterpret_cast<uint4*>(&Ks[(r + 32) * kKsLd + c]) = kk2;
            *reinterpret_cast<uint4*>(&Ks[(r + 48) * kKsLd + c]) = kk3;
            *reinterpret_cast<uint4*>(&Vs[r * kVsLd + c]) = keep(vv0, k0 + r);
            *reinterpret_cast<uint4*>(&Vs[(r + 16) * kVsLd + c]) = keep(vv1, k0 + r + 16);
            *reinterpret_cast<uint4*>(&Vs[(r + 32) * kVsLd + c]) = keep(vv2, k0 + r + 32);
            *reinterpret_cast<uint4*>(&Vs[(r + 48) * kVsLd + c]) = keep(vv3, k0 + r + 48);
        }
        __syncthreads();
        if (it + 1 < ntiles) RTP_LOAD_TILE(tile_base(it + 1))   // prefetch while computing

        // S^T for the two 32-key halves of the tile
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
        // scale, mask, tile maximum of this lane's query.  A tile that every
        // query of the wave sees whole (below the wave's first position, and
        // a sink tile or inside the window of its last position) skips the
        // per-key mask.
        float mt = -INFINITY;
        const bool whole = wave_full && k0 + kBN - 1 <= wp_min &&
                           (dense || k0 + kBN - 1 < g.sinks || k0 > wp_max - g.window);
        if (whole) {
#pragma unroll
            for (int sh = 0; sh < 2; ++sh)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[sh][i] *= sc;
                    mt = fmaxf(mt, s[sh][i]);
                }
        } else {
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = k0 + 32 * sh + (i >> 2) * 8 + 4 * hh + (i & 3);
                    bool ok = qok && key <= pq;
                    if (!dense) ok = ok && (key < g.sinks || key > pq - g.window);
                    const float v = ok ? s[sh][i] * sc : -INFINITY;
                    s[sh][i] = v;
                    mt = fmaxf(mt, v);
                }
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        uint32_t pb[2][8];                           // P^T as bf16 pairs, per half and kk
        if (m_new == -INFINITY) {
#pragma unroll
            for (int sh = 0; sh < 2; ++sh)
#pragma unroll
                for (int x = 0; x < 8; ++x) pb[sh][x] = 0u;
        } else {
            // v_exp_f32 directly: its results below 2^-126 (flushed) weigh
            // nothing against the running maximum's weight of 1.  The
            // accumulators are rescaled only when a query of the wave has a
            // new maximum (for the others the factor is exactly 1).
            if (__ballot(m_new > m_run) != 0ull) {
                const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= corr;
#pragma unroll
                for (int dd = 0; dd < 4; ++dd)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[dd][i] *= corr;
            }
            m_run = m_new;
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
                float p[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[i] = __builtin_amdgcn_exp2f(s[sh][i] - m_new);
                    l_run += p[i];
                }
#pragma unroll
                for (int x = 0; x < 8; ++x) pb[sh][x] = pack2(p[2 * x], p[2 * x + 1]);
            }
        }
        // O^T += V^T P^T: lane (d = 32 dd + qi, half hh) takes the keys
        // kc0 + 0..3 and kc0 + 8..11 (the rows of its S^T registers); in the
        // transposing loads, lane j of a 16-lane group addresses key row
        // kc0 + j / 4 (+ 8) at columns 32 dd + 16 (group & 1) + 4 (j % 4)
        const int trr = (lane & 15) >> 2, trc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint4 bp = make_uint4(pb[sh][4 * kk], pb[sh][4 * kk + 1], pb[sh][4 * kk + 2], pb[sh][4 * kk + 3]);
                const int kc0 = 32 * sh + 16 * kk + 4 * hh;
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    const bf16_t* vr = &Vs[(kc0 + trr) * kVsLd + 32 * dd + trc];
                    const uint2 lo = lds_tr16(vr);
                    const uint2 hi = lds_tr16(vr + 8 * kVsLd);
                    const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    oacc[dd] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(bp), oacc[dd], 0, 0, 0);
                }
            }
        }
    }
#undef RTP_LOAD_TILE
    // normalise and store: lane holds O[t][32 dd + 8 (i/4) + 4 hh + (i%4)]
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qok) {
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

}  // namespace

hipError_t launch_prefill_attn(const Geo& g, const void* q, const void* k, const void* v, void* out,
                               int dense, hipStream_t s) {
    if (g.n_hlist == 0) return hipSuccess;
    const dim3 grid((g.n_tok + kBM - 1) / kBM, g.n_hlist);
    hipLaunchKernelGGL(k_fa_prefill, grid, dim3(256), 0, s, g, (const bf16_t*)q, (const bf16_t*)k,
                       (const bf16_t*)v, (bf16_t*)out, dense);
    return hipGetLastError();
}

}  // namespace rtp
