// device.hpp -- gfx950 device helpers shared by the HIP kernels of librtp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtp {

constexpr int kIdx = 16;      // indexer width
constexpr int kBlk = 256;     // tokens per KV page
constexpr int kWave = 64;

typedef uint16_t bf16_t;
struct fp8e4_t {              // FP8 E4M3 (OCP: bias 7, no infinities) storage of K/V
    uint8_t b;
};

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// FP8 E4M3 codes to fp32 (exact, hardware conversion): 4 codes of a dword,
// byte 0 first.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}
__device__ __forceinline__ float fp82f(uint8_t c) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false)[0]; }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p) { return bf2f(*p); }
template <> __device__ __forceinline__ float ld<fp8e4_t>(const fp8e4_t* p) { return fp82f(p->b); }
// A stored K element as fp32: FP8 codes stand for fl32(code * scale)
template <typename T> __device__ __forceinline__ float ldk(const T* p, float) { return ld(p); }
template <> __device__ __forceinline__ float ldk<fp8e4_t>(const fp8e4_t* p, float scale) { return fp82f(p->b) * scale; }

// Stage n elements (n a multiple of 16 bytes' worth) into LDS as fp32, every
// thread of a 256-wide group moving 16-byte pieces; falls back to element
// loads when the source is not 16-byte aligned.  The caller synchronises.
template <typename T> __device__ __forceinline__ void stage_f32(const T* __restrict__ src, float* dst, int n,
                                                                int tid) {
    constexpr int V = 16 / sizeof(T);
    if (reinterpret_cast<uintptr_t>(src) & 15) {
        for (int x = tid; x < n; x += 256) dst[x] = ld(src + x);
        return;
    }
    for (int x = tid * V; x < n; x += 256 * V) {
        const uint4 u = *reinterpret_cast<const uint4*>(src + x);
        if (sizeof(T) == 4) {
            *reinterpret_cast<float4*>(dst + x) =
                make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
        } else {
            *reinterpret_cast<float4*>(dst + x) = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                                                              __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
            *reinterpret_cast<float4*>(dst + x + 4) = make_float4(__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xFFFF0000u),
                                                                  __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xFFFF0000u));
        }
    }
}

template <typename T> __device__ __forceinline__ void st(T* p, float v);
template <> __device__ __forceinline__ void st<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, float v) { *p = f2bf(v); }

// Transposing LDS load (gfx950): within each 16-lane group, lane 4 r + c
// supplies the address of 4 consecutive 16-bit elements (row r of a 4 x 16
// block, columns 4 c .. 4 c + 3); lane i receives column i of the block,
// rows 0..3.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr16(const bf16_t* p) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Order-preserving uint32 key of an fp32 score; -0 and +0 map to one key.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// ---- wave reductions and scans (wave64) ----
// Lane exchanges inside a row of 16 lanes are DPP operand modifiers of the
// VALU op itself (no LDS round trip, unlike a ds_bpermute shuffle); the four
// rows are joined through scalar lane reads.  Every lane gets the result.
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1] (lane xor 1, xor 2), the
// half-row mirror (lane i <-> 7 - i of each 8), the row mirror (i <-> 15 - i),
// and row_shr:n (lane i reads lane i - n of its row; 0 below the row's start).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long x) {
    return (unsigned long long)dpp32<CTRL>((uint32_t)x) | ((unsigned long long)dpp32<CTRL>((uint32_t)(x >> 32)) << 32);
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t x, int l) { return (uint32_t)__builtin_amdgcn_readlane((int)x, l); }
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long x, int l) {
    return (unsigned long long)lane_u32((uint32_t)x, l) | ((unsigned long long)lane_u32((uint32_t)(x >> 32), l) << 32);
}
// all-lane reduction of a 32-bit value under op (commutative, associative)
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce32(uint32_t x, Op op) {
    x = op(x, dpp32<kDppXor1>(x));
    x = op(x, dpp32<kDppXor2>(x));
    x = op(x, dpp32<kDppHalfMirror>(x));
    x = op(x, dpp32<kDppMirror>(x));
    return op(op(lane_u32(x, 0), lane_u32(x, 16)), op(lane_u32(x, 32), lane_u32(x, 48)));
}
template <typename Op>
__device__ __forceinline__ unsigned long long wave_reduce64(unsigned long long x, Op op) {
    x = op(x, dpp64<kDppXor1>(x));
    x = op(x, dpp64<kDppXor2>(x));
    x = op(x, dpp64<kDppHalfMirror>(x));
    x = op(x, dpp64<kDppMirror>(x));
    return op(op(lane_u64(x, 0), lane_u64(x, 16)), op(lane_u64(x, 32), lane_u64(x, 48)));
}
__device__ __forceinline__ float wave_max(float v) {
    return __uint_as_float(wave_reduce32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float wave_sum(float v) {
    return __uint_as_float(wave_reduce32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    return __longlong_as_double((long long)wave_reduce64((unsigned long long)__double_as_longlong(v),
        [](unsigned long long a, unsigned long long b) {
            return (unsigned long long)__double_as_longlong(__longlong_as_double((long long)a) +
                                                           __longlong_as_double((long long)b));
        }));
}
// sum over each row of 16 lanes (every lane of the row gets it)
__device__ __forceinline__ double row_sum_f64(double v) {
    const auto add = [](unsigned long long a, unsigned long long b) {
        return (unsigned long long)__double_as_longlong(__longlong_as_double((long long)a) +
                                                       __longlong_as_double((long long)b));
    };
    unsigned long long x = (unsigned long long)__double_as_longlong(v);
    x = add(x, dpp64<kDppXor1>(x));
    x = add(x, dpp64<kDppXor2>(x));
    x = add(x, dpp64<kDppHalfMirror>(x));
    x = add(x, dpp64<kDppMirror>(x));
    return __longlong_as_double((long long)x);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
    return wave_reduce32(v, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
    return wave_reduce64(v, [](unsigned long long a, unsigned long long b) { return a + b; });
}
// inclusive prefix sums over the wave's lanes (lane order)
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
    x += dpp32<0x111>(x);
    x += dpp32<0x112>(x);
    x += dpp32<0x114>(x);
    x += dpp32<0x118>(x);
    const uint32_t t0 = lane_u32(x, 15), t1 = lane_u32(x, 31), t2 = lane_u32(x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long x) {
    x += dpp64<0x111>(x);
    x += dpp64<0x112>(x);
    x += dpp64<0x114>(x);
    x += dpp64<0x118>(x);
    const unsigned long long t0 = lane_u64(x, 15), t1 = lane_u64(x, 31), t2 = lane_u64(x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? t0 : 0ull) + (row >= 2 ? t1 : 0ull) + (row >= 3 ? t2 : 0ull);
}

// Coherent (L2) loads of values written by other workgroups of the same grid.
__device__ __forceinline__ uint32_t ld_acquire(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_acquire(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_acquire(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int64_t ld_acquire(const int64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_acquire(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- indexer mass in fixed point -------------------------------------------
// Weight of a key relative to the row maximum m: w = exp(s (d - m)) in (0, 1],
// held as round(w * 2^43) in a uint64 so that sums are exact and independent of
// order (2^20 keys of weight <= 1 sum to <= 2^63).  The argument s (d - m) is
// carried exactly: d - m by TwoSum, s * t by an FMA residual, and the small
// remainder enters as exp(y + c) ~ exp(y) (1 + c).
//
// Level-1 bin of a key: floor(64 * x), x = -fl(s * fl(d - m)) >= 0, clamped to
// [0, kNB1 - 1].  fl() is monotone, so the bin never increases with d: all keys
// in bins below b rank above all keys in bin b.
constexpr int kNB1 = 2048;
constexpr float kBinsPerUnit = 64.0f;
constexpr double kFix = 8796093022208.0;   // 2^43

struct WeightBin {
    unsigned long long w;
    int bin;
};

__device__ __forceinline__ WeightBin weight_bin(float d, float m, float s) {
    float t = d - m;
    float bv = t - d;
    float e = (d - (t - bv)) + (-m - bv);    // d - m == t + e exactly
    float y = s * t;
    float ry = __builtin_fmaf(s, t, -y);     // s * t == y + ry exactly
    float c = ry + s * e;
    float w = expf(y);
    w = __builtin_fmaf(w, c, w);
    WeightBin r;
    r.w = (unsigned long long)__double2ll_rn((double)w * kFix);
    float x = -y * kBinsPerUnit;
    x = fminf(x, (float)(kNB1 - 1));
    r.bin = (int)x;
    return r;
}

// ---- block primitives (NT threads, NT a multiple of 64) ----

template <int NT>
__device__ __forceinline__ unsigned long long block_excl_scan_u64(unsigned long long v, unsigned long long* total,
                                                  unsigned long long* sh /* NT/64 */) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const unsigned long long x = wave_incl_scan_u64(v);
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    // every thread sums the wave totals itself (broadcast LDS reads)
    unsigned long long before = 0ull, all = 0ull;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const unsigned long long t = sh[w];
        before += w < wid ? t : 0ull;
        all += t;
    }
    *total = all;
    __syncthreads();
    return before + x - v;
}

template <int NT>
__device__ uint32_t block_sum_u32(uint32_t v, uint32_t* sh /* NT/64 */) {
    v = wave_sum_u32(v);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t t = 0;
    for (int w = 0; w < NT / 64; ++w) t += sh[w];
    __syncthreads();
    return t;
}

}  // namespace rtp
