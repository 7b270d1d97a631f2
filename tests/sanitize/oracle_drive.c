/*
 * Drives every oracle function on small seeded inputs and edge cases, for the
 * AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU oracle.
 * Exits 0 when every result is self-consistent.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

uint16_t orc_f32_to_bf16(float f);
float orc_bf16_to_f32(uint16_t h);
void orc_project(const float *x, int64_t rows, int64_t ld, int32_t D, const float *W, uint16_t *out);
int orc_scores(const uint16_t *q_low, const uint16_t *k_low, int64_t L, float *d);
int64_t orc_topp(const float *d, int64_t L, double s, float p, int32_t *sel, int64_t *order, double *cum);
int64_t orc_topk(const float *d, int64_t L, int64_t k, int32_t *sel);
void orc_attend(const float *q, const float *K, const float *V, int64_t ld, int32_t D, const int32_t *idx,
                int64_t n, double scale, double *out);
int64_t orc_window_set(int64_t pos, int64_t W, int64_t Ns, int32_t *out);
float orc_fp8e4m3_to_f32(uint8_t c);
void orc_fp8_dequant(const uint8_t *c, int64_t n, float scale, float *out);

static uint32_t rng = 12345u;
static float frand(void)
{
    rng = rng * 1664525u + 1013904223u;
    return (float)((rng >> 8) & 0xFFFF) / 32768.0f - 1.0f;
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main(void)
{
    enum { D = 64, L = 300 };
    static float K[L][D], V[L][D], W[D][16], q[D];
    static uint16_t klow[L][16], qlow[16];
    static float d[L];
    static int32_t sel[L], win[L];
    static int64_t order[L];
    static double cum[L], out[D];
    for (int j = 0; j < L; j++)
        for (int e = 0; e < D; e++) {
            K[j][e] = frand();
            V[j][e] = frand();
        }
    for (int e = 0; e < D; e++) {
        q[e] = frand();
        for (int c = 0; c < 16; c++) W[e][c] = frand();
    }
    orc_project(&K[0][0], L, D, D, &W[0][0], &klow[0][0]);
    orc_project(q, 1, D, D, &W[0][0], qlow);
    CHECK(orc_scores(qlow, &klow[0][0], L, d) == 0);
    for (int Lr = 1; Lr <= L; Lr += 37) {
        for (int pi = 0; pi < 5; pi++) {
            const float p = (float[]){1e-7f, 0.3f, 0.9f, 0.999f, 1.0f}[pi];
            int64_t k = orc_topp(d, Lr, 0.25, p, sel, order, cum);
            CHECK(k >= 1 && k <= Lr);
            for (int64_t i = 1; i < k; i++) CHECK(sel[i] > sel[i - 1]);
            CHECK(fabs(cum[Lr - 1] - 1.0) < 1e-12);
            orc_attend(q, &K[0][0], &V[0][0], D, D, sel, k, 0.125, out);
            for (int e = 0; e < D; e++) CHECK(isfinite(out[e]));
        }
        for (int64_t kk = 1; kk <= Lr + 3; kk += 5) {
            int64_t n = orc_topk(d, Lr, kk, sel);
            CHECK(n == (kk < Lr ? kk : Lr));
        }
    }
    CHECK(orc_topp(d, 0, 0.25, 0.5f, sel, NULL, NULL) == -1);
    CHECK(orc_topp(d, 10, 0.25, 0.0f, sel, NULL, NULL) == -1);
    CHECK(orc_topk(d, 10, 0, sel) == -1);
    orc_attend(q, &K[0][0], &V[0][0], D, D, sel, 0, 0.125, out);          /* empty set */
    for (int64_t pos = 0; pos < L; pos += 13) {
        int64_t n = orc_window_set(pos, 40, 4, win);
        CHECK(n >= 1 && n <= pos + 1 && win[n - 1] == pos);
    }
    static uint8_t codes[256];
    static float f8[256];
    for (int c = 0; c < 256; c++) codes[c] = (uint8_t)c;
    orc_fp8_dequant(codes, 256, 0.5f, f8);
    CHECK(f8[0x38] == 0.5f && isnan(f8[0x7F]) && orc_fp8e4m3_to_f32(0x7E) == 448.0f);
    CHECK(orc_bf16_to_f32(orc_f32_to_bf16(1.0f)) == 1.0f);
    printf("oracle drive ok\n");
    return 0;
}
