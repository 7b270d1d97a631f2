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

// ---- wave reductions (wave64) ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) { uint32_t w = __shfl_xor(v, o); v = w > v ? w : v; }
    return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
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
    unsigned long long x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        unsigned long long y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
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
