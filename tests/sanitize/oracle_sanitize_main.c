/*
 * Drives every exported function of oracle/oracle.c on small inputs that
 * reach its edge paths (lengths outside [0, N] and [0, pitch], empty rows,
 * k larger than the row, FP8 scoring with zero and non-finite query rows,
 * out-of-range key indices, every e4m3fn special value), so that a build
 * under AddressSanitizer and UndefinedBehaviorSanitizer can flag an
 * out-of-bounds access, a leak or undefined behaviour.  Test
 * infrastructure: built and run by tests/test_oracle_sanitize.py on the CPU.
 * Exits 0 when every result has the expected shape.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double ora_decode(int dtype, uint32_t bits);
uint8_t ora_encode_e4m3(float x);
void ora_encode_e4m3_array(const float *src, uint8_t *dst, int64_t n, int nthreads);
int ora_select_f64(const double *s, int64_t L, int k, int32_t *out_idx, double *out_val);
int ora_select_f32(const float *s, int64_t L, int k, int32_t *out_idx);
int ora_fused_topk(const void *Q, int q_t, const void *K, int k_t, const float *k_scale, const float *W,
                   const int32_t *kv_len, int64_t N, int H, int D, uint32_t flags, const int32_t *rows,
                   int nrows, int k, int32_t *out_idx, double *out_val, int32_t *out_n, int nthreads);
int ora_fused_scores_at(const void *Q, int q_t, const void *K, int k_t, const float *k_scale, const float *W,
                        int64_t N, int H, int D, uint32_t flags, const int32_t *t_idx, const int64_t *j_idx,
                        int64_t n, double *out);
int64_t ora_fused_score_row(const void *Q, int q_t, const void *K, int k_t, const float *k_scale,
                            const float *W, int64_t N, int H, int D, uint32_t flags, int t, int64_t L,
                            double *out);
int ora_topk_ragged(const float *scores, int64_t pitch, const int32_t *row_len, const int32_t *rows, int nrows,
                    int k, int32_t *out_idx, int32_t *out_n, int nthreads);
int ora_prior_from_topk(const int32_t *prev_idx, int64_t T_prev, int k, int64_t N, int k_prime, int32_t *out);

#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            return 1;                                                   \
        }                                                               \
    } while (0)

static uint32_t lcg(uint32_t *s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

int main(void)
{
    uint32_t seed = 12345u;
    /* fused: T = 5 queries, H = 3, D = 8, N = 20 fp32 keys; kv_len outside [0, N] */
    enum { T = 5, H = 3, D = 8, N = 20, K = 7 };
    float *Q = malloc(sizeof(float) * T * H * D), *Kf = malloc(sizeof(float) * N * D);
    uint8_t *K8 = malloc(N * D);
    float *S = malloc(sizeof(float) * N), *W = malloc(sizeof(float) * T * H);
    for (int i = 0; i < T * H * D; ++i) Q[i] = (float)((int)(lcg(&seed) % 9) - 4) * 0.25f;
    for (int i = 0; i < N * D; ++i) Kf[i] = (float)((int)(lcg(&seed) % 9) - 4) * 0.5f;
    for (int i = 0; i < N * D; ++i) K8[i] = ora_encode_e4m3(Kf[i]);
    for (int i = 0; i < N; ++i) S[i] = 0.5f;
    for (int i = 0; i < T * H; ++i) W[i] = 0.125f * (float)(1 + i % 3);
    for (int d = 0; d < D; ++d) Q[1 * H * D + 2 * D + d] = 0.0f;   /* a zero row: FP8 scale 1 */
    Q[2 * H * D + 0] = INFINITY;                                     /* a non-finite row */
    const int32_t kv[T] = {N, N + 1000, -5, 0, 3};
    const int32_t rows[T] = {0, 1, 2, 3, 4};
    int32_t idx[T * K], n[T];
    double val[T * K];
    for (uint32_t flags = 0; flags <= 2; flags += 2) {
        CHECK(ora_fused_topk(Q, 0, Kf, 0, NULL, W, kv, N, H, D, 0, rows, T, K, idx, val, n, 3) == 0);
        CHECK(n[0] == K && n[1] == K && n[2] == 0 && n[3] == 0 && n[4] == 3);
        CHECK(ora_fused_topk(Q, 0, K8, 3, S, W, kv, N, H, D, flags, rows, T, K, idx, val, n, 2) == 0);
        CHECK(n[1] == K && n[2] == 0 && idx[2 * K] == -1 && isinf(val[2 * K]));
    }
    double row[N];
    CHECK(ora_fused_score_row(Q, 0, Kf, 0, NULL, W, N, H, D, 0, 0, N + 50, row) == N);
    CHECK(ora_fused_score_row(Q, 0, Kf, 0, NULL, W, N, H, D, 0, 0, -3, row) == 0);
    const int32_t ti[2] = {0, 4};
    const int64_t ji_ok[2] = {0, N - 1}, ji_bad[2] = {0, N};
    double sv[2];
    CHECK(ora_fused_scores_at(Q, 0, K8, 3, S, W, N, H, D, 2, ti, ji_ok, 2, sv) == 0);
    CHECK(ora_fused_scores_at(Q, 0, Kf, 0, NULL, W, N, H, D, 0, ti, ji_bad, 2, sv) == -1);

    /* ragged: M = 4 rows at pitch 16; row_len outside [0, pitch] */
    enum { M = 4, PITCH = 16, KR = 5 };
    float *X = malloc(sizeof(float) * M * PITCH);
    for (int i = 0; i < M * PITCH; ++i) X[i] = (float)((int)(lcg(&seed) % 7) - 3);
    const int32_t rl[M] = {PITCH, PITCH + 9, -1, 2};
    const int32_t rrows[M] = {3, 2, 1, 0};
    int32_t ridx[M * KR], rn[M];
    CHECK(ora_topk_ragged(X, PITCH, rl, rrows, M, KR, ridx, rn, 2) == 0);
    CHECK(rn[0] == 2 && rn[1] == 0 && rn[2] == KR && rn[3] == KR && ridx[KR] == -1);

    /* selection edge cases */
    int32_t sidx[4];
    double svals[4];
    CHECK(ora_select_f64(row, 0, 4, sidx, svals) == 0 && sidx[0] == -1);
    CHECK(ora_select_f32(X, 3, 4, sidx) == 3 && sidx[3] == -1);
    CHECK(ora_select_f32(X, 3, 0, sidx) == -1);

    /* e4m3fn specials, and the array encoder over the decoded code table */
    float codes[256];
    uint8_t back[256];
    for (int c = 0; c < 256; ++c) codes[c] = (float)ora_decode(3, (uint32_t)c);
    ora_encode_e4m3_array(codes, back, 256, 4);
    for (int c = 0; c < 256; ++c) CHECK(back[c] == c || (isnan(codes[c]) && (back[c] & 0x7F) == 0x7F));
    CHECK(ora_encode_e4m3(NAN) == 0x7F && ora_encode_e4m3(-INFINITY) == 0xFF && ora_encode_e4m3(465.0f) == 0x7F);

    /* history list: -1 padding and keys outside [0, N), k' above N, no lists */
    const int32_t prev[12] = {3, 1, -1, 1, 4, 3, 5, 1, 9, 2147483647, -2147483647 - 1, 0};
    int32_t prior[10];
    CHECK(ora_prior_from_topk(prev, 4, 3, 6, 10, prior) == 6 && prior[0] == 1 && prior[9] == -1);
    CHECK(ora_prior_from_topk(prev, 0, 3, 6, 2, prior) == 2 && prior[0] == 0 && prior[1] == 1);
    CHECK(ora_prior_from_topk(prev, 4, 3, 0, 2, prior) == -1);

    free(Q); free(Kf); free(K8); free(S); free(W); free(X);
    printf("oracle sanitizer run ok\n");
    return 0;
}
