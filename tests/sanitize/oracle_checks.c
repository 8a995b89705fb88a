/*
 * oracle_checks.c -- drives every entry point of the CPU oracle (oracle/dspark_oracle.c)
 * built with AddressSanitizer and UndefinedBehaviorSanitizer, on small random inputs in both
 * dtypes, both samplers, greedy and sampled temperatures, ragged and empty drafts, subsets of
 * rows, the optional outputs and the recurrent head, plus the argument checks.  Output
 * arrays are allocated at exactly their documented sizes.  Prints "oracle checks: N
 * failures" and exits nonzero on any failure.  (Test infrastructure, like the oracle.)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
void oracle_philox_batch(int n, const uint32_t *ctrs, const uint32_t key[2], uint32_t *out);
double oracle_uniform(uint64_t seed, uint32_t req, uint32_t pos, uint32_t v, uint32_t stream);
double oracle_gumbel(uint64_t seed, uint32_t req, uint32_t pos, uint32_t v, uint32_t stream);
double oracle_block_uniform(uint64_t seed, uint32_t req, uint32_t pos, uint32_t beta,
                            uint32_t stream);
int oracle_two_level_sample(int n, const double *a, uint64_t seed, uint32_t req, uint32_t pos,
                            uint32_t race_stream, uint32_t within_stream, double *gap);
int oracle_token_sample(int n, const double *a, uint64_t seed, uint32_t req, uint32_t pos,
                        uint32_t stream, double *gap);
uint16_t oracle_float_to_bf16(float f);
int oracle_draft_block_head(int B, int K, int V, int r, int z_dtype, const void *Z,
                            int uw_dtype, const void *U, const void *W, const float *gru_wi,
                            const float *gru_wh, const float *gru_bi, const float *gru_bh,
                            const int32_t *prev_token, const int32_t *draft_len,
                            const float *temperature, const uint32_t *req_id, uint64_t seed,
                            const int32_t *rows, int n_rows, int32_t *draft_tokens,
                            double *q_tok, double *q_lse, float *corrected, double *gap,
                            uint16_t *state_out, int sampler);
int oracle_verify_head(int B, int K, int V, int r, int y_dtype, const void *Y,
                       const int32_t *draft_tokens, const float *q_tok, const float *q_lse,
                       int z_dtype, const void *Z, int uw_dtype, const void *U, const void *W,
                       const uint16_t *head_state, const int32_t *prev_token,
                       const int32_t *verify_len, const float *temperature,
                       const uint32_t *req_id, uint64_t seed, const int32_t *rows, int n_rows,
                       int32_t *accept_len, int32_t *next_token, double *p_tok, double *diag,
                       int sampler);
double oracle_profile(int n_knots, const double *knot_tokens, const double *knot_tps, double N);
void oracle_prefix_expected(int B, int n_items, const double *P, double *E_out);
int oracle_schedule(int B, int K, const float *conf_logits, const int32_t *draft_len,
                    int n_knots, const double *knot_tokens, const double *knot_tps, int enabled,
                    const double *inv_temp, int32_t *verify_len, double *expected_tokens,
                    double *diag);
int oracle_calibrate_step(int B, int K, const float *conf_logits, const int32_t *verify_len,
                          const int32_t *accept_len, double step, double ridge, double *inv_temp);
double oracle_ece(int n, const double *s, const double *y, int n_bins);

static int failures = 0;
#define CHECK(cond)                                                                 \
    do {                                                                            \
        if (!(cond)) {                                                              \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);         \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* splitmix64 -> [0, 1) */
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (double)((z ^ (z >> 31)) >> 11) * 0x1p-53;
}
static double nrand(void) { return sqrt(-2.0 * log(1.0 - urand())) * cos(6.283185307179586 * urand()); }

/* a factor / logit array of n elements in dtype d (0 = float32, 1 = bfloat16), scaled */
static void *fill(int d, size_t n, double scale) {
    void *p = malloc(n * (d ? 2 : 4) + 1);
    for (size_t i = 0; i < n; ++i) {
        float f = (float)(scale * nrand());
        if (d) ((uint16_t *)p)[i] = oracle_float_to_bf16(f);
        else ((float *)p)[i] = f;
    }
    return p;
}

static void rng_checks(void) {
    uint32_t key[2] = {0x12345678u, 0x9abcdef0u}, ctr[8] = {1, 2, 3, 4, 5, 6, 7, 8}, out[8];
    oracle_philox_batch(2, ctr, key, out);
    uint32_t one[4];
    oracle_philox4x32_10(ctr + 4, key, one);
    CHECK(memcmp(one, out + 4, sizeof one) == 0);
    for (uint32_t v = 0; v < 64; ++v) {
        const double u = oracle_uniform(42, 7, 3, v, v & 3);
        const double bu = oracle_block_uniform(42, 7, 3, v, 2);
        CHECK(u > 0.0 && u < 1.0 && bu > 0.0 && bu < 1.0);
        CHECK(isfinite(oracle_gumbel(42, 7, 3, v, 1)));
    }
}

static void sampler_checks(void) {
    for (int n = 1; n <= 40; n += 3) {
        double *a = malloc(sizeof(double) * n), gap = 0;
        for (int i = 0; i < n; ++i) a[i] = (i % 5 == 4) ? -INFINITY : nrand();
        a[0] = nrand(); /* at least one finite weight */
        const int x = oracle_token_sample(n, a, 9, 1, 2, 0, &gap);
        const int y = oracle_two_level_sample(n, a, 9, 1, 2, 0, 4, &gap);
        CHECK(x >= 0 && x < n && isfinite(a[x]));
        CHECK(y >= 0 && y < n && isfinite(a[y]));
        free(a);
    }
}

static void round_checks(int z_dtype, int uw_dtype, int sampler, int rnn) {
    const int B = 4, K = 4, V = 40, r = 8;
    void *Z = fill(z_dtype, (size_t)B * K * V, 2.0);
    void *U = fill(uw_dtype, (size_t)V * r, 0.4), *W = fill(uw_dtype, (size_t)V * r, 0.4);
    float *wi = NULL, *wh = NULL, *bi = NULL, *bh = NULL;
    if (rnn) {
        wi = fill(0, (size_t)3 * r * r, 0.3); wh = fill(0, (size_t)3 * r * r, 0.3);
        bi = fill(0, (size_t)3 * r, 0.1); bh = fill(0, (size_t)3 * r, 0.1);
    }
    int32_t prev[4] = {3, 0, 39, 17}, dlen[4] = {4, 0, 2, 3}, rows[4] = {0, 1, 2, 3};
    float temp[4] = {1.0f, 0.0f, 0.7f, 1.3f};
    uint32_t req[4] = {11, 12, 13, 14};
    int32_t *tok = malloc(sizeof(int32_t) * B * K);
    double *qt = malloc(sizeof(double) * B * K), *ql = malloc(sizeof(double) * B * K);
    double *gap = malloc(sizeof(double) * B * K);
    float *corr = malloc(sizeof(float) * (size_t)B * K * V);
    uint16_t *state = rnn ? calloc((size_t)B * K * r, sizeof(uint16_t)) : NULL;
    CHECK(oracle_draft_block_head(B, K, V, r, z_dtype, Z, uw_dtype, U, W, wi, wh, bi, bh, prev,
                                  dlen, temp, req, 5, rows, B, tok, qt, ql, corr, gap, state,
                                  sampler) == 0);
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < K; ++k) {
            const int t = tok[b * K + k];
            CHECK(k < dlen[b] ? (t >= 0 && t < V && qt[b * K + k] > 0.0) : t == -1);
        }
    /* a subset of rows without the optional outputs, and no rows at all */
    int32_t sub[2] = {3, 0};
    CHECK(oracle_draft_block_head(B, K, V, r, z_dtype, Z, uw_dtype, U, W, wi, wh, bi, bh, prev,
                                  NULL, temp, NULL, 5, sub, 2, tok, qt, ql, NULL, NULL, NULL,
                                  sampler) == 0);
    CHECK(oracle_draft_block_head(B, K, V, r, z_dtype, Z, uw_dtype, U, W, wi, wh, bi, bh, prev,
                                  dlen, temp, req, 5, rows, 0, tok, qt, ql, NULL, NULL, NULL,
                                  sampler) == 0);
    /* an out-of-range previous token is reported */
    int32_t bad_prev[4] = {3, -1, 40, 17};
    CHECK(oracle_draft_block_head(B, K, V, r, z_dtype, Z, uw_dtype, U, W, wi, wh, bi, bh,
                                  bad_prev, NULL, temp, req, 5, rows, B, tok, qt, ql, NULL, NULL,
                                  NULL, sampler) == -1);
    /* verification of the first draft against random targets */
    CHECK(oracle_draft_block_head(B, K, V, r, z_dtype, Z, uw_dtype, U, W, wi, wh, bi, bh, prev,
                                  dlen, temp, req, 5, rows, B, tok, qt, ql, NULL, NULL, state,
                                  sampler) == 0);
    void *Y = fill(0, (size_t)B * (K + 1) * V, 2.0);
    float *qtf = malloc(sizeof(float) * B * K), *qlf = malloc(sizeof(float) * B * K);
    for (int i = 0; i < B * K; ++i) {
        qtf[i] = (float)qt[i];
        qlf[i] = (float)ql[i];
    }
    int32_t vlen[4] = {4, 0, 1, 3}, acc[4], nxt[4];
    double *pt = malloc(sizeof(double) * B * K), *diag = malloc(sizeof(double) * B * 2);
    CHECK(oracle_verify_head(B, K, V, r, 0, Y, tok, qtf, qlf, z_dtype, Z, uw_dtype, U, W,
                             state, prev, vlen, temp, req, 5, rows, B, acc, nxt, pt, diag,
                             sampler) == 0);
    for (int b = 0; b < B; ++b) CHECK(acc[b] >= 0 && acc[b] <= vlen[b] && nxt[b] >= 0 && nxt[b] < V);
    CHECK(oracle_verify_head(B, K, V, r, 0, Y, tok, qtf, qlf, z_dtype, Z, uw_dtype, U, W,
                             state, prev, vlen, temp, NULL, 5, sub, 2, acc, nxt, NULL, NULL,
                             sampler) == 0);
    free(Z); free(U); free(W); free(wi); free(wh); free(bi); free(bh); free(tok); free(qt);
    free(ql); free(gap); free(corr); free(state); free(Y); free(qtf); free(qlf); free(pt);
    free(diag);
}

static void schedule_checks(void) {
    const int B = 6, K = 5;
    float conf[30];
    for (int i = 0; i < B * K; ++i) conf[i] = (float)(1.0 + nrand());
    int32_t dlen[6] = {5, 0, 3, 5, 1, 2}, vl[6];
    double kt[3] = {1.0, 20.0, 200.0}, kp[3] = {100.0, 1500.0, 2000.0}, th[5] = {1, 1.2, 0.8, 1, 1};
    double et[6], diag[2];
    for (int en = 0; en < 2; ++en) {
        CHECK(oracle_schedule(B, K, conf, dlen, 3, kt, kp, en, th, vl, et, diag) == 0);
        for (int b = 0; b < B; ++b) CHECK(vl[b] >= 0 && vl[b] <= dlen[b] && et[b] >= 1.0);
        CHECK(oracle_schedule(B, K, conf, NULL, 3, kt, kp, en, NULL, vl, NULL, NULL) == 0);
    }
    CHECK(oracle_schedule(-1, K, conf, dlen, 3, kt, kp, 1, th, vl, et, diag) == -1);
    CHECK(oracle_schedule(B, K, conf, dlen, 0, kt, kp, 1, th, vl, et, diag) == -1);
    CHECK(oracle_schedule(0, K, conf, dlen, 3, kt, kp, 1, th, vl, et, diag) == 0);
    CHECK(oracle_profile(3, kt, kp, 0.5) == 100.0 && oracle_profile(3, kt, kp, 1e9) == 2000.0);
    double P[4] = {0.9, 0.5, 0.25, 0.0}, E[5];
    oracle_prefix_expected(2, 4, P, E);
    CHECK(E[0] == 2.0 && fabs(E[4] - 3.65) < 1e-12);
    int32_t acc[6] = {5, 0, 1, 2, 0, 2};
    for (int b = 0; b < B; ++b) vl[b] = dlen[b];
    CHECK(oracle_calibrate_step(B, K, conf, vl, acc, 0.5, 1e-3, th) == 0);
    for (int k = 0; k < K; ++k) CHECK(th[k] >= 1.0 / 64 && th[k] <= 64.0);
    CHECK(oracle_calibrate_step(B, K, conf, vl, acc, 0.0, 1e-3, th) == -1);
    CHECK(oracle_calibrate_step(B, K, conf, vl, acc, 0.5, 1e-3, NULL) == -1);
    double s[8] = {0.1, 0.9, 0.5, 0.7, 0.2, 0.95, 0.4, 0.6}, y[8] = {0, 1, 1, 1, 0, 1, 0, 0};
    const double ece = oracle_ece(8, s, y, 4);
    CHECK(ece >= 0.0 && ece <= 1.0);
    CHECK(oracle_ece(0, s, y, 4) == 0.0);
}

int main(void) {
    rng_checks();
    sampler_checks();
    for (int zd = 0; zd < 2; ++zd)
        for (int ud = 0; ud < 2; ++ud)
            for (int samp = 0; samp < 2; ++samp) round_checks(zd, ud, samp, 0);
    round_checks(1, 1, 0, 1); /* recurrent head */
    round_checks(0, 1, 1, 1);
    schedule_checks();
    printf("oracle checks: %d failures\n", failures);
    return failures ? 1 : 0;
}
