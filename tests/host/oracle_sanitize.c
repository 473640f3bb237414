/* Drives every function of oracle/oracle.c on exactly sized heap buffers, for a
 * build under the address and undefined-behaviour sanitizers (CPU only).  Each
 * product is also checked against a dense integer product, so the run fails on a
 * wrong result as well as on an out-of-bounds access. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_ternarize_absmean(const float *W, int64_t N, int64_t K, int8_t *T, float *S);
int oracle_pack_i2s(const int8_t *T, int64_t N, int64_t K, uint8_t *P);
int oracle_unpack_i2s(const uint8_t *P, int64_t N, int64_t K, int8_t *T);
int oracle_quant_act_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *s_a);
int oracle_quant_act_bf16(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s_a, float *scratch);
int oracle_w2a8(const uint8_t *P, const float *S, const int8_t *Q, const float *s_a, int64_t M, int64_t N,
                int64_t K, int32_t *acc, double *y64, float *y, double *mag);
int oracle_acc_dense(const int8_t *T, const int8_t *Q, int64_t M, int64_t N, int64_t K, int32_t *acc);
int oracle_f32_to_bf16(const float *x, int64_t n, uint16_t *out);
int oracle_fold_quant(const float *y, int64_t M, int64_t H, int8_t *q, float *s_a, float *scratch);
int oracle_glu_quant(const float *y, int64_t M, int64_t H, int8_t *q, float *s_a, float *scratch);
int oracle_ternarize_absmean_g(const float *W, int64_t N, int64_t K, int G, int8_t *T, float *S);
int oracle_pack_i2s_g(const int8_t *T, int64_t N, int64_t K, int G, uint8_t *P);
int oracle_unpack_i2s_g(const uint8_t *P, int64_t N, int64_t K, int G, int8_t *T);
int oracle_w2a8_g(const uint8_t *P, const float *S, const int8_t *Q, const float *s_a, int64_t M, int64_t N,
                  int64_t K, int G, int32_t *acc, double *y64, float *y, double *mag);

static uint64_t state = 88172645463325252ull;
static uint32_t next(void) { state ^= state << 13; state ^= state >> 7; state ^= state << 17; return (uint32_t)state; }
static float unit(void) { return (float)(next() >> 8) / 16777216.0f * 2.0f - 1.0f; }
static void *must(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }

static int failures = 0;
#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++failures; } } while (0)

static void run(int64_t M, int64_t N, int64_t K, int G)
{
    const int64_t nb = G == 0 ? 1 : N * (K / G);
    float *W = must(sizeof(float) * N * K);
    for (int64_t i = 0; i < N * K; ++i) W[i] = 0.02f * unit();
    int8_t *T = must(N * K), *T2 = must(N * K);
    float *S = must(sizeof(float) * nb);
    uint8_t *P = must(N * K / 4);
    CHECK(oracle_ternarize_absmean_g(W, N, K, G, T, S) == 0);
    CHECK(oracle_pack_i2s_g(T, N, K, G, P) == 0);
    CHECK(oracle_unpack_i2s_g(P, N, K, G, T2) == 0);
    CHECK(memcmp(T, T2, N * K) == 0);
    float *x = must(sizeof(float) * M * K);
    uint16_t *xb = must(sizeof(uint16_t) * M * K);
    for (int64_t i = 0; i < M * K; ++i) x[i] = 3.0f * unit();
    CHECK(oracle_f32_to_bf16(x, M * K, xb) == 0);
    int8_t *q = must(M * K);
    float *sa = must(sizeof(float) * M), *scratch = must(sizeof(float) * M * K);
    CHECK(oracle_quant_act_bf16(xb, M, K, q, sa, scratch) == 0);
    CHECK(oracle_quant_act_f32(x, M, K, q, sa) == 0);
    int32_t *acc = must(sizeof(int32_t) * M * N), *dense = must(sizeof(int32_t) * M * N);
    double *y64 = must(sizeof(double) * M * N), *mag = must(sizeof(double) * M * N);
    float *y = must(sizeof(float) * M * N);
    CHECK(oracle_w2a8_g(P, S, q, sa, M, N, K, G, acc, y64, y, mag) == 0);
    CHECK(oracle_acc_dense(T, q, M, N, K, dense) == 0);
    CHECK(memcmp(acc, dense, sizeof(int32_t) * M * N) == 0);
    if (G == 128) {
        CHECK(oracle_ternarize_absmean(W, N, K, T2, S) == 0);
        CHECK(memcmp(T, T2, N * K) == 0);
        CHECK(oracle_pack_i2s(T, N, K, P) == 0);
        CHECK(oracle_unpack_i2s(P, N, K, T2) == 0);
        CHECK(memcmp(T, T2, N * K) == 0);
        CHECK(oracle_w2a8(P, S, q, sa, M, N, K, acc, y64, y, mag) == 0);
        CHECK(memcmp(acc, dense, sizeof(int32_t) * M * N) == 0);
        CHECK(oracle_w2a8(P, S, q, sa, M, N, K, NULL, NULL, NULL, NULL) == 0);
    }
    /* junctions: the product output as a two-half [M][2H] input, H = N/2 */
    const int64_t H = N / 2;
    int8_t *qh = must(M * H);
    float *sh = must(sizeof(float) * M), *scr = must(sizeof(float) * M * H);
    CHECK(oracle_fold_quant(y, M, H, qh, sh, scr) == 0);
    CHECK(oracle_glu_quant(y, M, H, qh, sh, scr) == 0);
    /* rejected inputs write nothing and return an error */
    CHECK(oracle_w2a8(P, S, q, sa, M, N, K + 1, acc, y64, y, mag) < 0);
    CHECK(oracle_pack_i2s_g(T, N, K, 32, P) < 0);
    T[0] = 2;
    CHECK(oracle_pack_i2s_g(T, N, K, G, P) < 0);
    free(W); free(T); free(T2); free(S); free(P); free(x); free(xb); free(q); free(sa); free(scratch);
    free(acc); free(dense); free(y64); free(mag); free(y); free(qh); free(sh); free(scr);
}

int main(void)
{
    const int64_t shapes[][3] = {{1, 16, 128}, {3, 48, 384}, {8, 64, 640}, {2, 32, 1280}, {5, 80, 256}};
    const int Gs[] = {128, 64, 0};
    for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
        for (size_t g = 0; g < 3; ++g) run(shapes[s][0], shapes[s][1], shapes[s][2], Gs[g]);
    printf("ok (%d failures)\n", failures);
    return failures != 0;
}
