/*
 * synth.c -- seeded synthetic inputs (post-RoPE Q/K/V, projection noise).
 *
 * Shared by the GPU tests, the benchmark and the oracle checks, so it holds
 * none of the method's arithmetic: it only draws numbers and rotates them.
 *
 *  - Counter-based generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 *    "Parallel random numbers: as easy as 1, 2, 3", SC'11), 10 rounds with the
 *    published multipliers and Weyl key increments.  Counter words are
 *    (pair index low, pair index high, stream, tensor id); the key is the
 *    64-bit seed.  Any element can be regenerated on its own.
 *  - Normals: Box-Muller on two 53-bit uniforms from one Philox block,
 *    giving the two members of a rotary pair.
 *  - RoPE (rotate-half layout): pair (i, i + D/2) is rotated by
 *    pos * base^(-2i/D), computed in double.
 *  - Output is rounded once to the tensor's storage type (fp32, or bf16 with
 *    round-to-nearest-even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(const uint32_t in[4], uint32_t k0, uint32_t k1,
                                 uint32_t out[4])
{
    uint32_t c0 = in[0], c1 = in[1], c2 = in[2], c3 = in[3];
    for (int r = 0; r < 10; r++) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* exported for the generator's own known-answer test */
void syn_philox(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    philox4x32_10(ctr, key[0], key[1], out);
}

/* two standard normals from one counter */
static inline void normal_pair(uint64_t seed, uint32_t tensor, uint32_t stream,
                               uint64_t idx, double *za, double *zb)
{
    uint32_t ctr[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), stream, tensor};
    uint32_t r[4];
    philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), r);
    uint64_t a = ((uint64_t)r[0] << 32) | r[1];
    uint64_t b = ((uint64_t)r[2] << 32) | r[3];
    double u1 = ((double)(a >> 11) + 0.5) * 0x1.0p-53;   /* (0,1) */
    double u2 = (double)(b >> 11) * 0x1.0p-53;           /* [0,1) */
    double rad = sqrt(-2.0 * log(u1));
    double phi = 6.283185307179586476925 * u2;
    *za = rad * cos(phi);
    *zb = rad * sin(phi);
}

static inline uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lower = u & 0xFFFFu, upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

static inline void store(void *out, int32_t dtype, int64_t i, double v)
{
    if (dtype == 0)
        ((float *)out)[i] = (float)v;
    else
        ((uint16_t *)out)[i] = to_bf16((float)v);
}

/*
 * out[t][h][e] for t < n_tok, h < H, e < D: N(0,1) * scale, then rotary
 * embedding at position pos0 + t (rope_base <= 0 disables the rotation).
 * Token t of the tensor uses generator indices of token (tok0 + t), so a
 * slice can be regenerated alone.  dtype 0 = fp32, 1 = bf16.
 */
void syn_normal_rope(uint64_t seed, uint32_t tensor, uint32_t stream,
                     int64_t tok0, int64_t n_tok, int32_t H, int32_t D,
                     double scale, double rope_base, int64_t pos0,
                     int32_t dtype, void *out, int32_t nthreads)
{
    const int half = D / 2;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t t = 0; t < n_tok; t++) {
        double cs[256], sn[256];
        int64_t pos = pos0 + t;
        for (int i = 0; i < half; i++) {
            if (rope_base > 0) {
                double theta = pow(rope_base, -2.0 * i / (double)D);
                double ang = (double)pos * theta;
                cs[i] = cos(ang);
                sn[i] = sin(ang);
            } else {
                cs[i] = 1.0;
                sn[i] = 0.0;
            }
        }
        for (int h = 0; h < H; h++) {
            int64_t base = ((tok0 + t) * H + h) * (int64_t)half;
            int64_t o = (t * H + h) * (int64_t)D;
            for (int i = 0; i < half; i++) {
                double za, zb;
                normal_pair(seed, tensor, stream, (uint64_t)(base + i), &za, &zb);
                za *= scale;
                zb *= scale;
                store(out, dtype, o + i, za * cs[i] - zb * sn[i]);
                store(out, dtype, o + i + half, za * sn[i] + zb * cs[i]);
            }
        }
    }
}

/* out[i] = N(0,1) * scale as double, i < n (plain draws, no rotation) */
void syn_normal(uint64_t seed, uint32_t tensor, uint32_t stream, int64_t n,
                double scale, double *out)
{
    for (int64_t i = 0; i < n; i += 2) {
        double za, zb;
        normal_pair(seed, tensor, stream, (uint64_t)(i / 2), &za, &zb);
        out[i] = za * scale;
        if (i + 1 < n) out[i + 1] = zb * scale;
    }
}

/* out[i] = uniform in [0,1) as double (53 bits), i < n */
void syn_uniform(uint64_t seed, uint32_t tensor, uint32_t stream, int64_t n,
                 double *out)
{
    for (int64_t i = 0; i < n; i += 2) {
        uint32_t ctr[4] = {(uint32_t)(i / 2), (uint32_t)((uint64_t)(i / 2) >> 32),
                           stream, tensor};
        uint32_t r[4];
        philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), r);
        uint64_t a = ((uint64_t)r[0] << 32) | r[1];
        uint64_t b = ((uint64_t)r[2] << 32) | r[3];
        out[i] = (double)(a >> 11) * 0x1.0p-53;
        if (i + 1 < n) out[i + 1] = (double)(b >> 11) * 0x1.0p-53;
    }
}
