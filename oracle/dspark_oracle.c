/*
 * dspark_oracle.c -- plain CPU oracle for the DSpark draft / schedule / verify round.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct definition that the
 * GPU library is checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or constant generator with
 * the HIP library, and it never takes a value produced by that library.
 *
 * Everything floating-point is done in double precision unless a step fixes the precision
 * itself (the corrected logits are rounded to float once, because that float is the value
 * both implementations take their argmax decisions on).  Loops are written in the order of
 * the definitions, with no blocking and no fusion.
 *
 * Sources (the pages are web articles about DeepSeek's DSpark; cited by title and section):
 *  - Markov sequential head: QbitAI, "DSpark in 10 concepts", section "Cheaper serial
 *    module: the Markov head" (the head looks only at the previous token and is a rank-256
 *    low-rank factorisation); 10100.com commentary, section "Parallel drafts are fast but may
 *    turn 'of course' into 'of problem'" (rank-256 low-rank transition correction, added to the
 *    block of base logits produced by the parallel backbone, left to right).
 *  - Confidence-scheduled verification length: QbitAI, section "Variable-length drafts and
 *    hardware-aware scheduling" (per-position survival score, throughput curve measured per
 *    batch size, per-request verify length); 10100.com, section "DSpark's hardest step: letting
 *    the GPU decide how much to verify" (survival given all earlier positions passed;
 *    longer at low load, low-return suffixes cut at high load); wangjunjian.com tag page,
 *    translated abstract (prefix survival probability and engine throughput profile).
 *  - Lossless verification: QbitAI, section "Speculative decoding" (accept the longest correct
 *    prefix, resample at the first divergence, output distribution equals the target's);
 *    10100.com, section "Speculative decoding is block checking" (rejection rule of
 *    Leviathan et al., arXiv 2211.17192); wangjunjian.com tag page, post "Speculative
 *    Decoding" steps 3-4 (accept by comparing the two probabilities with a random number;
 *    if all guesses pass, sample the next token from the target; else resample the rejected
 *    position from the adjusted distribution).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - U is [V][r] (row t = left factor of token t); W is stored [V][r] as well: row v holds
 *    column v of the r x V right factor, so bias_v = sum_i U[t][i] * W[v][i].
 *  - The corrected logit is purely additive: c_v = Z_v + bias_v.  The first draft position
 *    uses the last committed token t0.  Temperature T divides the corrected logit; T = 0
 *    means greedy (argmax).  Ties in every argmax go to the lowest vocabulary index.
 *  - Random numbers: Philox4x32 with 10 rounds (Salmon et al., SC'11), key = (seed low word,
 *    seed high word), counter = (v >> 2, position, request key, stream), output word v & 3,
 *    uniform = ((word >> 8) + 0.5) * 2^-24, which lies strictly inside (0, 1).
 *    Streams: 0 draft sampling, 1 accept test (v = 0), 2 residual resampling, 3 bonus
 *    (4 / 5 / 6: within-block draws of the optional two-level sampler).
 *  - Sampling a token from weights w_v = exp(a_v) (the pages fix the law: the draft token follows
 *    the drafter's softmax, the emitted token the target's): the plain Gumbel-max draw keyed per
 *    token, x = argmax_v (a_v + G_v), G_v = -log(-log u_v) with u_v the uniform of token v on the
 *    draw's stream at its position (streams: 0 draft, 2 residual, 3 bonus).  Tokens of weight 0
 *    (a_v = -inf) are never drawn; exact ties go to the lowest index.
 *    Optional second mode (the library's cheaper opt-in sampler, defined here so that it can be
 *    checked too; it keeps the law but not the per-token keying): a two-level Gumbel-max.  The
 *    vocabulary is cut into blocks of 16 consecutive ids (the last one may be shorter); block
 *    beta gets the log-weight A_beta = log sum_{v in beta} w_v and the race score
 *    A_beta + G_beta, where G_beta is the Gumbel draw of block beta on the race stream (block
 *    uniforms: see oracle_block_uniform); the best block wins, and inside it the token with the
 *    best a_v + G_v, G_v the Gumbel draw of token v on the within stream.  The block race picks
 *    beta with probability W_beta / sum W and the second step v with probability w_v / W_beta,
 *    so the token has probability w_v / sum w, the law of one Gumbel-max over all tokens.
 *    Streams of that mode: race 0 / 2 / 3 (draft / residual / bonus), within 4 / 5 / 6.
 *  - Accept test: u * q(x) < p(x)  (equivalent to u < p/q for q > 0; p >= q always accepts).
 *  - Residual: r_v = max(0, p_v - q_v); the correction is the draw from the weights r (residual
 *    stream); if every r_v is 0 it is the same draw from p.
 *  - Schedule: survival s = 1/(1+exp(-C)); P = running product over positions; rank all
 *    (request, position) items by (P desc, position asc, request asc); for n = 0..sum K_b
 *    E(n) = B + sum of the top-n P, N(n) = B + n, G(n) = E(n) * T(N(n)) / N(n) with T the
 *    piecewise-linear throughput profile clamped outside its knots; n* = smallest argmax;
 *    L_b = number of request b's items in the top n*.  E(n) is the float64 rounding of the
 *    exact sum (each P truncated to a multiple of 2^-80, which moves the sum by less than
 *    2^-67), so that its value does not depend on the order in which the terms are added.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of the arrays handed in (float32 or bfloat16 bit patterns) */
#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Philox stream identifiers */
#define ORACLE_STREAM_DRAFT 0u
#define ORACLE_STREAM_ACCEPT 1u
#define ORACLE_STREAM_RESIDUAL 2u
#define ORACLE_STREAM_BONUS 3u
#define ORACLE_STREAM_DRAFT_WITHIN 4u
#define ORACLE_STREAM_RESIDUAL_WITHIN 5u
#define ORACLE_STREAM_BONUS_WITHIN 6u

/* tokens per block of the two-level sampler */
#define ORACLE_SAMPLE_BLOCK 16

/* sampler modes: the per-token Gumbel-max (the definition) and the optional two-level race */
#define ORACLE_SAMPLER_TOKEN 0
#define ORACLE_SAMPLER_BLOCK16 1

/* ------------------------------------------------------------------------------------ */
/* element access                                                                         */
/* ------------------------------------------------------------------------------------ */

/* A bfloat16 value is the upper half of the float32 with the same sign/exponent/mantissa. */
static double bf16_bits_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(int dtype, const void *base, size_t idx)
{
    if (dtype == ORACLE_BF16)
        return bf16_bits_to_double(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/* ------------------------------------------------------------------------------------ */
/* Philox4x32-10 and the uniform / Gumbel draws built on it                               */
/* ------------------------------------------------------------------------------------ */

/* One Philox4x32 round: two 32x32->64 multiplies by the published multipliers, the high
 * halves mixed with the other counter words and the round key. */
static void philox_round(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    uint64_t prod_a = (uint64_t)0xD2511F53u * (uint64_t)c[0];
    uint64_t prod_b = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
    uint32_t n0 = (uint32_t)(prod_b >> 32) ^ c[1] ^ k0;
    uint32_t n1 = (uint32_t)prod_b;
    uint32_t n2 = (uint32_t)(prod_a >> 32) ^ c[3] ^ k1;
    uint32_t n3 = (uint32_t)prod_a;
    c[0] = n0;
    c[1] = n1;
    c[2] = n2;
    c[3] = n3;
}

/* Philox4x32-10: ten rounds; the key is advanced by the Weyl constants before every round
 * after the first. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        philox_round(c, k0, k1);
    }
    out[0] = c[0];
    out[1] = c[1];
    out[2] = c[2];
    out[3] = c[3];
}

/* Uniform in (0,1) for vocabulary index v at (request key, position, stream). */
double oracle_uniform(uint64_t seed, uint32_t req, uint32_t pos, uint32_t v, uint32_t stream)
{
    uint32_t ctr[4] = {v >> 2, pos, req, stream};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    uint32_t w = out[v & 3u];
    return ((double)(w >> 8) + 0.5) * (1.0 / 16777216.0);
}

/* Standard Gumbel draw from the uniform above. */
double oracle_gumbel(uint64_t seed, uint32_t req, uint32_t pos, uint32_t v, uint32_t stream)
{
    double u = oracle_uniform(seed, req, pos, v, stream);
    return -log(-log(u));
}

/* Uniform of block beta of the two-level sampler.  Writing beta = 16 a + 4 b + c
 * (b, c in 0..3), block beta takes word b of the Philox block at counter (4 a + c, position,
 * request key, stream): a one-to-one map from block ids to (counter, word) pairs, under which
 * four blocks that are 16 apart share one Philox block. */
double oracle_block_uniform(uint64_t seed, uint32_t req, uint32_t pos, uint32_t beta,
                            uint32_t stream)
{
    uint32_t a = beta >> 4, b = (beta >> 2) & 3u, c = beta & 3u;
    uint32_t ctr[4] = {4u * a + c, pos, req, stream};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return ((double)(out[b] >> 8) + 0.5) * (1.0 / 16777216.0);
}

static int argmax_double(const double *a, int n, double *gap);

/*
 * Two-level Gumbel-max draw from log-weights a[0..n) (-inf = weight 0; at least one finite).
 * Returns the token; *gap (optional) receives the smaller of the two decisions' margins over
 * their runners-up (block race, then within the block), so that tests can recognise near-ties.
 */
int oracle_two_level_sample(int n, const double *a, uint64_t seed, uint32_t req, uint32_t pos,
                            uint32_t race_stream, uint32_t within_stream, double *gap)
{
    int n_blocks = (n + ORACLE_SAMPLE_BLOCK - 1) / ORACLE_SAMPLE_BLOCK;
    double *race = (double *)malloc(sizeof(double) * (size_t)(n_blocks > 0 ? n_blocks : 1));
    for (int beta = 0; beta < n_blocks; ++beta) {
        int lo = beta * ORACLE_SAMPLE_BLOCK;
        int hi = lo + ORACLE_SAMPLE_BLOCK < n ? lo + ORACLE_SAMPLE_BLOCK : n;
        double m = -INFINITY;
        for (int v = lo; v < hi; ++v)
            if (a[v] > m)
                m = a[v];
        if (m == -INFINITY) {
            race[beta] = -INFINITY;
            continue;
        }
        double acc = 0.0;
        for (int v = lo; v < hi; ++v)
            acc += exp(a[v] - m);
        double u = oracle_block_uniform(seed, req, pos, (uint32_t)beta, race_stream);
        race[beta] = m + log(acc) - log(-log(u));
    }
    double g_race, g_within;
    int best = argmax_double(race, n_blocks, &g_race);
    free(race);
    int lo = best * ORACLE_SAMPLE_BLOCK;
    int len = (lo + ORACLE_SAMPLE_BLOCK < n ? ORACLE_SAMPLE_BLOCK : n - lo);
    double inner[ORACLE_SAMPLE_BLOCK];
    for (int i = 0; i < len; ++i)
        inner[i] = a[lo + i] + oracle_gumbel(seed, req, pos, (uint32_t)(lo + i), within_stream);
    int x = lo + argmax_double(inner, len, &g_within);
    if (gap)
        *gap = g_race < g_within ? g_race : g_within;
    return x;
}

/*
 * Per-token Gumbel-max draw from log-weights a[0..n) (-inf = weight 0; at least one finite):
 * x = argmax_v (a_v + G_v), G_v the Gumbel draw of token v on `stream` at position pos, lowest
 * index on exact ties.  P(x = v) = exp(a_v) / sum exp(a) (Gumbel, 1954; the "Gumbel-max trick").
 * *gap (optional) receives the winner's margin over the runner-up, so that tests can recognise
 * near-ties.
 */
int oracle_token_sample(int n, const double *a, uint64_t seed, uint32_t req, uint32_t pos,
                        uint32_t stream, double *gap)
{
    double *score = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int v = 0; v < n; ++v)
        score[v] = (a[v] == -INFINITY) ? -INFINITY
                                       : a[v] + oracle_gumbel(seed, req, pos, (uint32_t)v, stream);
    int x = argmax_double(score, n, gap);
    free(score);
    return x;
}

/* One draw of the round (kind 0 draft, 1 residual, 2 bonus) with the selected sampler. */
static int sample_draw(int sampler, int n, const double *a, uint64_t seed, uint32_t req,
                       uint32_t pos, int kind, double *gap)
{
    static const uint32_t token_stream[3] = {ORACLE_STREAM_DRAFT, ORACLE_STREAM_RESIDUAL,
                                             ORACLE_STREAM_BONUS};
    static const uint32_t within_stream[3] = {ORACLE_STREAM_DRAFT_WITHIN,
                                              ORACLE_STREAM_RESIDUAL_WITHIN,
                                              ORACLE_STREAM_BONUS_WITHIN};
    if (sampler == ORACLE_SAMPLER_BLOCK16)
        return oracle_two_level_sample(n, a, seed, req, pos, token_stream[kind],
                                       within_stream[kind], gap);
    return oracle_token_sample(n, a, seed, req, pos, token_stream[kind], gap);
}

/* ------------------------------------------------------------------------------------ */
/* Markov sequential head                                                                 */
/* ------------------------------------------------------------------------------------ */

/* ------------------------------------------------------------------------------------ */
/* Recurrent sequential head (optional)                                                   */
/* ------------------------------------------------------------------------------------ */
/*
 * Besides the default Markov head the pages mention an optional RNN head that follows the
 * whole prefix of the draft block; its gain was small and it is off by default (QbitAI, "DSpark
 * in 10 concepts", section "Cheaper serial module: the Markov head"; 10100.com commentary,
 * section "Parallel drafts are fast but may turn 'of course' into 'of problem'"; wangjunjian.com
 * tag page, DeepSpec overview: a light serial module at the output, the low-rank Markov head by
 * default or an RNN head).  The pages give no form for it.  The reading implemented:
 *   e_k    = U[prev_k]              the previous token's left factor (prev_0 = t0)
 *   h_{-1} = 0,  h_k = GRU(h_{k-1}, e_k), kept in float32 (rounded once per step)
 *   a_k    = h_k rounded to bfloat16 (nearest, ties to even): the contraction's left operand
 *   c_v    = Z_v + sum_i a_k[i] * W[v][i]
 * GRU: the gated recurrent unit of Cho et al. (EMNLP 2014) in the usual gate order (reset,
 * update, new) with separate input and hidden biases,
 *   g  = sigmoid(Wi_g e + bi_g + Wh_g h + bh_g)        reset gate
 *   z  = sigmoid(Wi_z e + bi_z + Wh_z h + bh_z)        update gate
 *   n  = tanh(Wi_n e + bi_n + g * (Wh_n h + bh_n))     candidate
 *   h' = (1 - z) * n + z * h
 * Wi, Wh: [3r][r] float32, rows 0..r-1 the reset units, r..2r-1 update, 2r..3r-1 new;
 * bi, bh: [3r].  The cell is evaluated in double from the float32 state.
 */
void oracle_gru_cell(int r, const float *wi, const float *wh, const float *bi, const float *bh,
                     const double *e, const double *h, double *h_out)
{
    for (int u = 0; u < r; ++u) {
        double a_g = (double)bi[u] + (double)bh[u];
        double a_z = (double)bi[r + u] + (double)bh[r + u];
        double a_ni = (double)bi[2 * r + u];
        double a_nh = (double)bh[2 * r + u];
        for (int i = 0; i < r; ++i) {
            a_g += (double)wi[(size_t)u * r + i] * e[i] + (double)wh[(size_t)u * r + i] * h[i];
            a_z += (double)wi[(size_t)(r + u) * r + i] * e[i] +
                   (double)wh[(size_t)(r + u) * r + i] * h[i];
            a_ni += (double)wi[(size_t)(2 * r + u) * r + i] * e[i];
            a_nh += (double)wh[(size_t)(2 * r + u) * r + i] * h[i];
        }
        double g = 1.0 / (1.0 + exp(-a_g));
        double z = 1.0 / (1.0 + exp(-a_z));
        double n = tanh(a_ni + g * a_nh);
        h_out[u] = (1.0 - z) * n + z * h[u];
    }
}

/* float -> bfloat16 bits, rounding to nearest with ties to even (NaN stays a NaN). */
uint16_t oracle_float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* Corrected logits from an explicit left operand (bfloat16 bits, length r):
 * c_v = Z_v + sum_i a[i] * W[v][i], accumulated in double and rounded once to float. */
void oracle_corrected_row_operand(int V, int r, int z_dtype, const void *z_row,
                                  const uint16_t *a, int uw_dtype, const void *W, float *c_out)
{
    for (int v = 0; v < V; ++v) {
        double bias = 0.0;
        for (int i = 0; i < r; ++i)
            bias += bf16_bits_to_double(a[i]) * load_elem(uw_dtype, W, (size_t)v * r + i);
        c_out[v] = (float)(load_elem(z_dtype, z_row, (size_t)v) + bias);
    }
}

/* Corrected logits of one draft row: c_v = Z_v + sum_i U[prev][i] * W[v][i].
 * The sum is accumulated in double; the result is rounded once to float, which is the
 * value the argmax and the softmax below start from. */
void oracle_corrected_row(int V, int r, int z_dtype, const void *z_row, int uw_dtype,
                          const void *U, const void *W, int prev, float *c_out)
{
    for (int v = 0; v < V; ++v) {
        double bias = 0.0;
        for (int i = 0; i < r; ++i)
            bias += load_elem(uw_dtype, U, (size_t)prev * r + i) *
                    load_elem(uw_dtype, W, (size_t)v * r + i);
        c_out[v] = (float)(load_elem(z_dtype, z_row, (size_t)v) + bias);
    }
}

/* argmax with ties to the lowest index; also reports the gap to the runner-up. */
static int argmax_double(const double *a, int n, double *gap)
{
    int best = 0;
    for (int v = 1; v < n; ++v)
        if (a[v] > a[best])
            best = v;
    double second = -INFINITY;
    for (int v = 0; v < n; ++v)
        if (v != best && a[v] > second)
            second = a[v];
    if (gap)
        *gap = a[best] - second;
    return best;
}

/* log of sum_v exp(s_v), with the maximum taken out first */
static double log_sum_exp(const double *s, int n)
{
    double m = -INFINITY;
    for (int v = 0; v < n; ++v)
        if (s[v] > m)
            m = s[v];
    double acc = 0.0;
    for (int v = 0; v < n; ++v)
        acc += exp(s[v] - m);
    return m + log(acc);
}

/* ------------------------------------------------------------------------------------ */
/* Draft block                                                                            */
/* ------------------------------------------------------------------------------------ */

/*
 * Draft tokens for the requests listed in rows[0..n_rows).  For request b and position
 * k = 0..K_b-1 (K_b = draft_len[b], or K when draft_len is NULL):
 *   prev = t0_b for k = 0, else x_{b,k-1};
 *   c = corrected row (above): the Markov head from U[prev], or, when the GRU weights are
 *       given (gru_wi non-NULL, all four then required), the recurrent head's operand a_k;
 *   T = 0: x = argmax c, q_tok = 1, q_lse = 0;
 *   T > 0: s = c / T, lse = log sum exp s, x = Gumbel-max draw from s on the draft stream
 *          (per token, or the two-level race when sampler = ORACLE_SAMPLER_BLOCK16),
 *          q_tok = exp(s_x - lse), q_lse = lse.
 * Positions k >= K_b get x = -1, q_tok = 0, q_lse = 0.
 * Arrays are full-size ([B][K] / [B][K][V]); only the listed requests are written.
 * corrected (optional, [B][K][V]) receives the float corrected logits.
 * gap (optional, [B][K]) receives the winning score's margin over the runner-up
 * (c for greedy; the perturbed score for a sampled token, the smaller margin of the two
 * decisions of the two-level race) so that near-ties can be recognised by the tests.
 * state_out (optional, recurrent head only, [B][K][r] bfloat16 bits) receives a_k for the
 * drafted positions (other positions are left as they are).
 * Returns 0, or -1 when a token index is out of range.
 */
int oracle_draft_block_head(int B, int K, int V, int r, int z_dtype, const void *Z,
                            int uw_dtype, const void *U, const void *W, const float *gru_wi,
                            const float *gru_wh, const float *gru_bi, const float *gru_bh,
                            const int32_t *prev_token, const int32_t *draft_len,
                            const float *temperature, const uint32_t *req_id, uint64_t seed,
                            const int32_t *rows, int n_rows, int32_t *draft_tokens,
                            double *q_tok, double *q_lse, float *corrected, double *gap,
                            uint16_t *state_out, int sampler)
{
    (void)B; /* arrays are [B][...]; only the listed rows are touched */
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ri = 0; ri < n_rows; ++ri) {
        int b = rows[ri];
        float *c = (float *)malloc(sizeof(float) * (size_t)V);
        double *s = (double *)malloc(sizeof(double) * (size_t)V);
        /* recurrent head: input, state (starts at zero), next state, operand */
        double *e = (double *)malloc(sizeof(double) * (size_t)r);
        double *h = (double *)calloc((size_t)r, sizeof(double));
        double *hn = (double *)malloc(sizeof(double) * (size_t)r);
        uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)r);
        int Kb = draft_len ? draft_len[b] : K;
        uint32_t req = req_id ? req_id[b] : (uint32_t)b;
        double T = (double)temperature[b];
        int prev = prev_token[b];
        for (int k = 0; k < K; ++k) {
            size_t bk = (size_t)b * K + k;
            if (k >= Kb || prev < 0 || prev >= V) {
                if (k < Kb) {
#pragma omp atomic write
                    status = -1;
                }
                draft_tokens[bk] = -1;
                q_tok[bk] = 0.0;
                q_lse[bk] = 0.0;
                if (gap)
                    gap[bk] = INFINITY;
                continue;
            }
            const void *z_row = (z_dtype == ORACLE_BF16)
                                    ? (const void *)((const uint16_t *)Z + bk * (size_t)V)
                                    : (const void *)((const float *)Z + bk * (size_t)V);
            if (gru_wi) {
                for (int i = 0; i < r; ++i)
                    e[i] = load_elem(uw_dtype, U, (size_t)prev * r + i);
                oracle_gru_cell(r, gru_wi, gru_wh, gru_bi, gru_bh, e, h, hn);
                for (int i = 0; i < r; ++i) {
                    h[i] = (double)(float)hn[i];
                    a[i] = oracle_float_to_bf16((float)h[i]);
                }
                if (state_out)
                    memcpy(state_out + bk * (size_t)r, a, sizeof(uint16_t) * (size_t)r);
                oracle_corrected_row_operand(V, r, z_dtype, z_row, a, uw_dtype, W, c);
            } else {
                oracle_corrected_row(V, r, z_dtype, z_row, uw_dtype, U, W, prev, c);
            }
            if (corrected)
                memcpy(corrected + bk * (size_t)V, c, sizeof(float) * (size_t)V);
            int x;
            double g;
            if (T == 0.0) {
                for (int v = 0; v < V; ++v)
                    s[v] = (double)c[v];
                x = argmax_double(s, V, &g);
                q_tok[bk] = 1.0;
                q_lse[bk] = 0.0;
            } else {
                for (int v = 0; v < V; ++v)
                    s[v] = (double)c[v] / T;
                double lse = log_sum_exp(s, V);
                x = sample_draw(sampler, V, s, seed, req, (uint32_t)k, 0, &g);
                q_tok[bk] = exp(s[x] - lse);
                q_lse[bk] = lse;
            }
            draft_tokens[bk] = x;
            if (gap)
                gap[bk] = g;
            prev = x;
        }
        free(c);
        free(s);
        free(e);
        free(h);
        free(hn);
        free(a);
    }
    return status;
}

/* The Markov head alone (no recurrent state). */
int oracle_draft_block(int B, int K, int V, int r, int z_dtype, const void *Z, int uw_dtype,
                       const void *U, const void *W, const int32_t *prev_token,
                       const int32_t *draft_len, const float *temperature, const uint32_t *req_id,
                       uint64_t seed, const int32_t *rows, int n_rows, int32_t *draft_tokens,
                       double *q_tok, double *q_lse, float *corrected, double *gap, int sampler)
{
    return oracle_draft_block_head(B, K, V, r, z_dtype, Z, uw_dtype, U, W, NULL, NULL, NULL,
                                   NULL, prev_token, draft_len, temperature, req_id, seed, rows,
                                   n_rows, draft_tokens, q_tok, q_lse, corrected, gap, NULL,
                                   sampler);
}

/* ------------------------------------------------------------------------------------ */
/* Confidence-scheduled verification length                                              */
/* ------------------------------------------------------------------------------------ */

/* Piecewise-linear throughput profile, clamped to the end knots outside their range. */
double oracle_profile(int n_knots, const double *knot_tokens, const double *knot_tps, double N)
{
    if (N <= knot_tokens[0])
        return knot_tps[0];
    if (N >= knot_tokens[n_knots - 1])
        return knot_tps[n_knots - 1];
    int i = 0;
    while (!(N >= knot_tokens[i] && N <= knot_tokens[i + 1]))
        ++i;
    double t = (N - knot_tokens[i]) / (knot_tokens[i + 1] - knot_tokens[i]);
    return knot_tps[i] + (knot_tps[i + 1] - knot_tps[i]) * t;
}

/*
 * E(n) = B + P_0 + ... + P_{n-1} for n = 0..n_items, each the float64 rounding (nearest, ties
 * to even) of the exact sum, with every P in [0, 1] first truncated to a multiple of 2^-80.
 * The sums are exact 128-bit integers in units of 2^-80 (B <= 2^14 and n_items <= 2^14 keep
 * them below 2^95); the conversion to float64 is the compiler's unsigned __int128 -> double,
 * and the scaling by 2^-80 is exact.
 */
static unsigned __int128 fixed80(double p)
{
    if (!(p > 0.0))
        return 0;
    int e;
    double f = frexp(p, &e);                      /* p = f 2^e, f in [0.5, 1) */
    uint64_t m = (uint64_t)ldexp(f, 53);          /* 53-bit integer, exact */
    int sh = e - 53 + 80;                         /* p 2^80 = m 2^sh */
    if (sh >= 0)
        return (unsigned __int128)m << sh;
    if (sh <= -64)
        return 0;
    return (unsigned __int128)(m >> (-sh));
}

void oracle_prefix_expected(int B, int n_items, const double *P, double *E_out)
{
    unsigned __int128 acc = (unsigned __int128)(unsigned)B << 80;
    for (int n = 0; n <= n_items; ++n) {
        if (n > 0)
            acc += fixed80(P[n - 1]);
        E_out[n] = ldexp((double)acc, -80);
    }
}

typedef struct {
    double P;
    int k;
    int b;
} sched_item;

/* (P desc, position asc, request asc) */
static int sched_item_cmp(const void *pa, const void *pb)
{
    const sched_item *a = (const sched_item *)pa, *b = (const sched_item *)pb;
    if (a->P > b->P)
        return -1;
    if (a->P < b->P)
        return 1;
    if (a->k != b->k)
        return a->k < b->k ? -1 : 1;
    if (a->b != b->b)
        return a->b < b->b ? -1 : 1;
    return 0;
}

/*
 * Per-request verification length.  enabled = 0 returns L_b = K_b.
 * inv_temp (optional, [K]): per-position inverse temperature theta_k of the confidence
 * logits, s = 1/(1+exp(-theta_k C)) (absent: theta = 1).
 * expected_tokens (optional, [B]) = 1 + sum_{k < L_b} P_{b,k}: the expected number of tokens
 * the round emits for request b (accepted prefix plus the one correction/bonus token).
 * diag (optional, [2]) = {n*, relative margin of G(n*) over the best other n}.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_schedule(int B, int K, const float *conf_logits, const int32_t *draft_len,
                    int n_knots, const double *knot_tokens, const double *knot_tps, int enabled,
                    const double *inv_temp, int32_t *verify_len, double *expected_tokens,
                    double *diag)
{
    if (B < 0 || K < 0 || n_knots < 1)
        return -1;
    double *P = (double *)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1) * (size_t)(K > 0 ? K : 1));
    for (int b = 0; b < B; ++b) {
        double run = 1.0;
        for (int k = 0; k < K; ++k) {
            double theta = inv_temp ? inv_temp[k] : 1.0;
            double C = theta * (double)conf_logits[(size_t)b * K + k];
            double surv = 1.0 / (1.0 + exp(-C));
            run = run * surv;
            P[(size_t)b * K + k] = run;
        }
    }
    if (!enabled) {
        for (int b = 0; b < B; ++b)
            verify_len[b] = draft_len ? draft_len[b] : K;
        if (diag) {
            diag[0] = -1.0;
            diag[1] = INFINITY;
        }
    } else {
        int total = 0;
        for (int b = 0; b < B; ++b)
            total += draft_len ? draft_len[b] : K;
        sched_item *items = (sched_item *)malloc(sizeof(sched_item) * (size_t)(total > 0 ? total : 1));
        int n_items = 0;
        for (int b = 0; b < B; ++b) {
            int Kb = draft_len ? draft_len[b] : K;
            for (int k = 0; k < Kb; ++k) {
                items[n_items].P = P[(size_t)b * K + k];
                items[n_items].k = k;
                items[n_items].b = b;
                ++n_items;
            }
        }
        qsort(items, (size_t)n_items, sizeof(sched_item), sched_item_cmp);
        double *Ps = (double *)malloc(sizeof(double) * (size_t)(n_items > 0 ? n_items : 1));
        double *Es = (double *)malloc(sizeof(double) * (size_t)(n_items + 1));
        for (int i = 0; i < n_items; ++i)
            Ps[i] = items[i].P;
        oracle_prefix_expected(B, n_items, Ps, Es);
        double best_G = -INFINITY, second_G = -INFINITY;
        int best_n = 0;
        for (int n = 0; n <= n_items; ++n) {
            double N = (double)B + (double)n;
            double G = Es[n] * oracle_profile(n_knots, knot_tokens, knot_tps, N) / N;
            if (G > best_G) {
                second_G = best_G;
                best_G = G;
                best_n = n;
            } else if (G > second_G) {
                second_G = G;
            }
        }
        for (int b = 0; b < B; ++b)
            verify_len[b] = 0;
        for (int i = 0; i < best_n; ++i)
            verify_len[items[i].b] += 1;
        if (diag) {
            diag[0] = (double)best_n;
            diag[1] = (best_G - second_G) / fabs(best_G);
        }
        free(Ps);
        free(Es);
        free(items);
    }
    if (expected_tokens) {
        for (int b = 0; b < B; ++b) {
            double e = 1.0;
            for (int k = 0; k < verify_len[b]; ++k)
                e += P[(size_t)b * K + k];
            expected_tokens[b] = e;
        }
    }
    free(P);
    return 0;
}

/* ------------------------------------------------------------------------------------ */
/* Online calibration of the confidence logits                                           */
/* ------------------------------------------------------------------------------------ */

/*
 * The pages report that raw survival scores are over-confident, that sequential temperature
 * scaling brings the expected calibration error from 3-8% to about 1%, and that the
 * thresholds are adjusted online from the acceptance the running drafter actually achieves
 * (QbitAI, "DSpark in 10 concepts", section "Online drafter calibration"; 10100.com
 * commentary, section "letting the GPU decide how much to verify").  They give no formula;
 * the plain reading taken here:
 *
 *  - position k (0-based) has its own inverse temperature theta_k > 0 and calibrated survival
 *    s = sigmoid(theta_k C) (theta = 1: the raw score);
 *  - a verified round labels the positions it tested: for request b with verify length L_b and
 *    accepted length a_b, position k is tested iff k < L_b and k <= a_b, and its label is
 *    y = 1 (accepted) for k < a_b, y = 0 for k = a_b.  Each position is thus fitted on the
 *    requests whose earlier positions all passed -- the "sequential" in the pages' name;
 *  - after each round, one damped Newton step on the round's log-loss
 *        l(theta) = sum over tested (b,k) of  log(1 + exp(theta C)) - y theta C
 *    per position:  theta_k <- clamp(theta_k - step * l'(theta_k) / (l''(theta_k) + ridge),
 *    1/64, 64), with l' = sum (sigmoid(theta C) - y) C and l'' = sum sigmoid(theta C)
 *    (1 - sigmoid(theta C)) C^2 (a position with no tested request keeps its theta).
 *
 * Lengths outside [0, K] and accepted lengths outside [0, L_b] are clamped.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_calibrate_step(int B, int K, const float *conf_logits, const int32_t *verify_len,
                          const int32_t *accept_len, double step, double ridge, double *inv_temp)
{
    if (B < 0 || K < 1 || !(step > 0.0) || !(ridge > 0.0) || !inv_temp)
        return -1;
    for (int k = 0; k < K; ++k) {
        double theta = inv_temp[k];
        double d1 = 0.0, d2 = 0.0;
        for (int b = 0; b < B; ++b) {
            int L = verify_len[b];
            L = L < 0 ? 0 : (L > K ? K : L);
            int a = accept_len[b];
            a = a < 0 ? 0 : (a > L ? L : a);
            if (!(k < L && k <= a))
                continue;
            double y = k < a ? 1.0 : 0.0;
            double C = (double)conf_logits[(size_t)b * K + k];
            double sg = 1.0 / (1.0 + exp(-theta * C));
            d1 += (sg - y) * C;
            d2 += sg * (1.0 - sg) * C * C;
        }
        theta = theta - step * d1 / (d2 + ridge);
        if (theta < 1.0 / 64.0)
            theta = 1.0 / 64.0;
        if (theta > 64.0)
            theta = 64.0;
        inv_temp[k] = theta;
    }
    return 0;
}

/*
 * Expected calibration error of n predictions s_i in [0, 1] against labels y_i in {0, 1}:
 * n_bins equal-width bins of [0, 1] (s = 1 falls in the last), ECE = sum over bins of
 * (bin count / n) * |mean label - mean prediction|.
 */
double oracle_ece(int n, const double *s, const double *y, int n_bins)
{
    if (n <= 0 || n_bins <= 0)
        return 0.0;
    double *cnt = (double *)calloc((size_t)n_bins, sizeof(double));
    double *sy = (double *)calloc((size_t)n_bins, sizeof(double));
    double *ss = (double *)calloc((size_t)n_bins, sizeof(double));
    for (int i = 0; i < n; ++i) {
        int m = (int)(s[i] * n_bins);
        if (m >= n_bins)
            m = n_bins - 1;
        if (m < 0)
            m = 0;
        cnt[m] += 1.0;
        sy[m] += y[i];
        ss[m] += s[i];
    }
    double e = 0.0;
    for (int m = 0; m < n_bins; ++m)
        if (cnt[m] > 0.0)
            e += (cnt[m] / n) * fabs(sy[m] / cnt[m] - ss[m] / cnt[m]);
    free(cnt);
    free(sy);
    free(ss);
    return e;
}

/* ------------------------------------------------------------------------------------ */
/* Lossless rejection-sampling verification                                              */
/* ------------------------------------------------------------------------------------ */

/*
 * For every listed request b with L = verify_len[b], temperature T, target rows Y[b][0..K]:
 *   for k = 0..L-1 (draft position k+1):
 *     T = 0: accept iff x_k == argmax Y[b][k];
 *     T > 0: p = softmax(Y[b][k] / T); u = uniform(accept stream, v = 0, position k);
 *            accept iff u * q_tok[b][k] < p(x_k).
 *     On the first rejection at k = j: accept_len = j and the correction is
 *       T = 0: argmax Y[b][j];
 *       T > 0: q_j(v) = exp(c_{j,v} / T - q_lse[b][j]) with c_j the corrected row of position j
 *              (previous token t0 for j = 0, else x_{j-1}; with head_state, [B][K][r]
 *              bfloat16 bits from a recurrent-head draft, its operand head_state[b][j]);
 *              r = max(0, p - q_j);
 *              Gumbel-max draw from log r (residual stream, position j);
 *              if r is identically zero, the same draw from log p.
 *   If all L pass: accept_len = L and the bonus token is argmax Y[b][L] (T = 0) or the
 *   Gumbel-max draw from Y[b][L]/T on the bonus stream at position L.
 * Every draw is the per-token Gumbel-max, or the two-level race when
 * sampler = ORACLE_SAMPLER_BLOCK16.
 * Outputs: accept_len[b], next_token[b]; p_tok (optional, [B][K]) = p(x_k) for the tested
 * positions (1 for a greedy match, 0 for a greedy mismatch); diag (optional, [B][2]) =
 * {|u - p/q| of the deciding test (inf for greedy / none), margin of the sampled correction
 * or bonus over its runner-up}.
 * Returns 0, or -1 when a token index is out of range.
 */
int oracle_verify_head(int B, int K, int V, int r, int y_dtype, const void *Y,
                       const int32_t *draft_tokens, const float *q_tok, const float *q_lse,
                       int z_dtype, const void *Z, int uw_dtype, const void *U, const void *W,
                       const uint16_t *head_state, const int32_t *prev_token,
                       const int32_t *verify_len, const float *temperature,
                       const uint32_t *req_id, uint64_t seed, const int32_t *rows, int n_rows,
                       int32_t *accept_len, int32_t *next_token, double *p_tok, double *diag,
                       int sampler)
{
    (void)B; /* arrays are [B][...]; only the listed rows are touched */
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int ri = 0; ri < n_rows; ++ri) {
        int b = rows[ri];
        int L = verify_len[b];
        double T = (double)temperature[b];
        uint32_t req = req_id ? req_id[b] : (uint32_t)b;
        double *y = (double *)malloc(sizeof(double) * (size_t)V);
        double *p = (double *)malloc(sizeof(double) * (size_t)V);
        double *score = (double *)malloc(sizeof(double) * (size_t)V);
        float *c = (float *)malloc(sizeof(float) * (size_t)V);
        double accept_margin = INFINITY, sample_margin = INFINITY;
        int a = L, token = -1, rejected = 0;

        for (int k = 0; k < L && !rejected; ++k) {
            size_t row = (size_t)b * (K + 1) + k;
            int x = draft_tokens[(size_t)b * K + k];
            if (x < 0 || x >= V) {
#pragma omp atomic write
                status = -1;
                x = 0;
            }
            for (int v = 0; v < V; ++v)
                y[v] = load_elem(y_dtype, Y, row * V + v);
            int accept;
            if (T == 0.0) {
                int am = argmax_double(y, V, NULL);
                accept = (x == am);
                if (p_tok)
                    p_tok[(size_t)b * K + k] = accept ? 1.0 : 0.0;
                if (!accept)
                    token = am;
            } else {
                for (int v = 0; v < V; ++v)
                    score[v] = y[v] / T;
                double lse_p = log_sum_exp(score, V);
                for (int v = 0; v < V; ++v)
                    p[v] = exp(score[v] - lse_p);
                double u = oracle_uniform(seed, req, (uint32_t)k, 0u, ORACLE_STREAM_ACCEPT);
                double q = (double)q_tok[(size_t)b * K + k];
                accept = (u * q < p[x]);
                if (p_tok)
                    p_tok[(size_t)b * K + k] = p[x];
                accept_margin = (q > 0.0) ? fabs(u - p[x] / q) : INFINITY;
                if (!accept) {
                    /* recompute the draft distribution of this position */
                    int prev = (k == 0) ? prev_token[b] : draft_tokens[(size_t)b * K + k - 1];
                    if (prev < 0 || prev >= V) {
#pragma omp atomic write
                        status = -1;
                        prev = 0;
                    }
                    size_t zrow = (size_t)b * K + k;
                    const void *z_row =
                        (z_dtype == ORACLE_BF16)
                            ? (const void *)((const uint16_t *)Z + zrow * (size_t)V)
                            : (const void *)((const float *)Z + zrow * (size_t)V);
                    if (head_state)
                        oracle_corrected_row_operand(V, r, z_dtype, z_row,
                                                     head_state + zrow * (size_t)r, uw_dtype, W,
                                                     c);
                    else
                        oracle_corrected_row(V, r, z_dtype, z_row, uw_dtype, U, W, prev, c);
                    double lq = (double)q_lse[(size_t)b * K + k];
                    int any = 0;
                    for (int v = 0; v < V; ++v) {
                        double qv = exp((double)c[v] / T - lq);
                        double rv = p[v] - qv;
                        if (rv > 0.0) {
                            any = 1;
                            score[v] = log(rv);
                        } else {
                            score[v] = -INFINITY;
                        }
                    }
                    if (!any)
                        for (int v = 0; v < V; ++v)
                            score[v] = log(p[v]);
                    token = sample_draw(sampler, V, score, seed, req, (uint32_t)k, 1,
                                        &sample_margin);
                }
            }
            if (!accept) {
                a = k;
                rejected = 1;
            }
        }
        if (!rejected) {
            size_t row = (size_t)b * (K + 1) + L;
            for (int v = 0; v < V; ++v)
                y[v] = load_elem(y_dtype, Y, row * V + v);
            if (T == 0.0) {
                token = argmax_double(y, V, NULL);
            } else {
                for (int v = 0; v < V; ++v)
                    score[v] = y[v] / T;
                token = sample_draw(sampler, V, score, seed, req, (uint32_t)L, 2, &sample_margin);
            }
        }
        accept_len[b] = a;
        next_token[b] = token;
        if (diag) {
            diag[(size_t)b * 2 + 0] = accept_margin;
            diag[(size_t)b * 2 + 1] = sample_margin;
        }
        free(y);
        free(p);
        free(score);
        free(c);
    }
    return status;
}

/* Verification of a Markov-head draft (the recompute takes U[prev]). */
int oracle_verify(int B, int K, int V, int r, int y_dtype, const void *Y,
                  const int32_t *draft_tokens, const float *q_tok, const float *q_lse,
                  int z_dtype, const void *Z, int uw_dtype, const void *U, const void *W,
                  const int32_t *prev_token, const int32_t *verify_len, const float *temperature,
                  const uint32_t *req_id, uint64_t seed, const int32_t *rows, int n_rows,
                  int32_t *accept_len, int32_t *next_token, double *p_tok, double *diag,
                  int sampler)
{
    return oracle_verify_head(B, K, V, r, y_dtype, Y, draft_tokens, q_tok, q_lse, z_dtype, Z,
                              uw_dtype, U, W, NULL, prev_token, verify_len, temperature, req_id,
                              seed, rows, n_rows, accept_len, next_token, p_tok, diag, sampler);
}

/* Number of threads the parallel loops above use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Batch helpers for the tests: n Philox blocks for explicit counters / n uniforms. */
void oracle_philox_batch(int n, const uint32_t *ctrs, const uint32_t key[2], uint32_t *out)
{
    for (int i = 0; i < n; ++i)
        oracle_philox4x32_10(ctrs + 4 * (size_t)i, key, out + 4 * (size_t)i);
}

void oracle_uniform_batch(int n, uint64_t seed, const uint32_t *req, const uint32_t *pos,
                          const uint32_t *v, uint32_t stream, double *out)
{
    for (int i = 0; i < n; ++i)
        out[i] = oracle_uniform(seed, req[i], pos[i], v[i], stream);
}
