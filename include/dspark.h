/*
 * dspark.h -- C ABI of the MI355X (gfx950) DSpark round library, libdspark.so.
 *
 * One speculative-decoding round of a DSpark-style drafter is three calls, in the order the
 * pages state the problem:
 *
 *   1. dspark_draft_block  -- the lightweight sequential head on top of the parallel backbone.
 *      The backbone has already produced base logits for every draft position of the block;
 *      the head walks the block left to right, adds a prefix-dependent bias taken from the
 *      previous token only (a rank-r low-rank Markov factorisation, r = 256 by default), and
 *      samples each position from the corrected distribution.
 *      (QbitAI "DSpark in 10 concepts", sections "DSpark = Eagle + DFlash" and "Cheaper serial
 *      module: the Markov head"; 10100.com commentary, section on parallel drafts turning
 *      "of course" into "of problem".)
 *   2. dspark_schedule     -- confidence-scheduled verification length: per-position survival
 *      scores, their running products (probability that the whole prefix survives), and a
 *      measured engine throughput curve decide how many draft tokens of each request are
 *      worth verifying this round; all on the GPU, no host round trip.
 *      (QbitAI, section "Variable-length drafts and hardware-aware scheduling"; 10100.com,
 *      section "letting the GPU decide how much to verify"; wangjunjian.com tag page,
 *      translated abstract.)
 *   3. dspark_verify       -- lossless rejection-sampling verification against the target
 *      model's logits: accept the longest prefix whose tokens pass the probability-ratio test,
 *      resample the first rejected position from the normalised positive part of (p - q), or
 *      draw a bonus token from p when every verified token passes.
 *      (QbitAI, section "Speculative decoding"; 10100.com, section "speculative decoding is
 *      block checking", rule of Leviathan et al. arXiv 2211.17192; wangjunjian.com tag page,
 *      post "Speculative Decoding", steps 3-4.)
 *
 * Conventions shared by every call
 *   - All array pointers are DEVICE pointers, caller-owned, row-major, densely packed.
 *     The library allocates no device memory and keeps no global state: scratch space comes
 *     from the caller's workspace (size from the *_workspace_size queries, 256-byte aligned).
 *     Calls on distinct workspaces may run concurrently.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is asynchronous on
 *     that stream and never synchronises the host, except dspark_query_device_status.  The
 *     three round calls only enqueue kernels (no allocation, memset or copy), so a whole round
 *     can be captured into a HIP graph and replayed.
 *   - Host-visible argument errors (null pointers, sizes, dtypes, workspace) are returned
 *     before anything is launched.  A failed launch returns DSPARK_EHIP.  Errors in device
 *     data (a token id outside [0, V), a negative or NaN temperature, a bad verify length,
 *     non-increasing profile knots) cannot be seen without a host sync: the kernels record
 *     them as bits of a status word in the workspace, replace the bad value by a safe one
 *     (token 0, greedy, clamped length) so that no access leaves its buffer, and
 *     dspark_query_device_status reports them.
 *   - Dtypes: DSPARK_F32 (IEEE float32) or DSPARK_BF16 (bfloat16 bit patterns).
 *   - Vocabulary size V must be a multiple of 8 (vectorised row loads).
 *
 * Randomness (all three calls): Philox4x32-10 (Salmon et al., SC'11) keyed by `seed`
 * (low word, high word); a draw takes one output word w and u = ((w >> 8) + 0.5) / 2^24 in
 * (0, 1), G = -log(-log u) a standard Gumbel draw.  Token v's draw on stream s at position k
 * uses word v & 3 of the block at counter (v >> 2, k, request key, s).
 *
 * Sampling a token from weights w_v = exp(a_v) (the pages fix the law: the draft token follows
 * the drafter's softmax and the emitted token the target's; QbitAI "DSpark in 10 concepts",
 * section "Speculative decoding"; wangjunjian.com tag page, post "Speculative Decoding", steps
 * 3-4).  Two samplers, chosen per call by the `sampler` field of the arguments:
 *   DSPARK_SAMPLER_TOKEN (0, the default): the per-token Gumbel-max, x = argmax_v (a_v + G_v)
 *     with G_v the draw of token v on the call's stream at its position -- stream 0 for a draft
 *     token, 2 for a residual correction, 3 for a bonus token.
 *   DSPARK_SAMPLER_BLOCK16 (1, opt-in, cheaper): a two-level Gumbel-max with the same law but
 *     one uniform per 16 tokens instead of one per token.  The vocabulary is cut into blocks of
 *     16 consecutive ids (the last one may be shorter); block beta has the log-weight
 *     A = log sum_{v in beta} w_v and the race score A + G_beta, where G_beta comes from word b
 *     of the Philox block at counter (4 a + c, k, request key, race stream) for
 *     beta = 16 a + 4 b + c (b, c in 0..3).  The best block wins; inside it the token with the
 *     best a_v + G_v (token draws on the within stream) is drawn.  Token v then has probability
 *     w_v / sum w.  Streams (race / within): 0 / 4 draft, 2 / 5 residual, 3 / 6 bonus.
 * Stream 1 is the accept test (v = 0).  Results therefore depend only on (inputs, seed, request
 * keys, sampler), not on launch geometry.  Every argmax, and the race, breaks exact ties
 * towards the lowest index.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSPARK_OK = 0,
    DSPARK_EINVAL = -1,     /* a size, pointer or flag is invalid                       */
    DSPARK_EDTYPE = -2,     /* unsupported dtype combination                            */
    DSPARK_EWORKSPACE = -3, /* workspace missing, misaligned or smaller than required   */
    DSPARK_EHIP = -4,       /* the HIP runtime reported an error (launch or sync)       */
    DSPARK_EDEVICE = -5,    /* device data was invalid (see dspark_query_device_status) */
    DSPARK_ESCRATCH = -6    /* sizes exceed the static scratch of dspark_draft_block_static */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* How sampled tokens are drawn (see "Sampling" above). */
typedef enum { DSPARK_SAMPLER_TOKEN = 0, DSPARK_SAMPLER_BLOCK16 = 1 } dspark_sampler;

/* Bits of the device status word. */
#define DSPARK_DEV_BAD_TOKEN 0x1u       /* a token id outside [0, V) was replaced by 0     */
#define DSPARK_DEV_BAD_TEMPERATURE 0x2u /* a negative / NaN temperature was taken as 0     */
#define DSPARK_DEV_BAD_LENGTH 0x4u      /* a draft / verify length was clamped to [0, K]   */
#define DSPARK_DEV_BAD_PROFILE 0x8u     /* profile knots not increasing / not positive     */

/* Optional per-kernel timing: when an args struct carries a trace handle, the library records
 * a pair of HIP events around every kernel it launches for that call. */
typedef struct dspark_trace dspark_trace;

/*
 * dspark_draft_block -- draft one block with the Markov sequential head (default) or the
 * optional recurrent head.
 *
 * For request b and position k = 0 .. K_b - 1 (K_b = draft_len[b], or K):
 *   prev   = prev_token[b] for k = 0, else x[b][k-1]          (previous token only)
 *   c[v]   = Z[b][k][v] + sum_i U[prev][i] * W[v][i]          (float32 accumulation)
 *   T_b = 0: x = argmax_v c[v],  q_tok = 1, q_lse = 0
 *   T_b > 0: s = c / T_b, q_lse = log sum_v exp(s_v), x = the sampler's draw from s on the
 *            draft stream(s) at position k, q_tok = exp(s_x - q_lse)
 * Positions k >= K_b get x = -1, q_tok = 0, q_lse = 0.
 *
 * Layouts: Z [B][K][V]; U [V][r] (row t is the left factor of token t); W [V][r] -- row v
 * holds column v of the r x V right factor (the same layout as an output-projection weight;
 * a factor held as r x V is converted once, when the weights are loaded, by dspark_pack_w).
 * U and W share a dtype.  Z may be float32 or bfloat16.  Supported: r in [1, 1024]; bfloat16
 * factors with r = 64, 128 or 256 run on the matrix cores, anything else on the
 * vector ALUs.  K in [1, 64].  B in [0, 2^24) (B = 0 launches nothing).
 * Outputs: draft_tokens [B][K] int32, q_tok [B][K] float32, q_lse [B][K] float32; corrected
 * [B][K][V] float32 is optional (NULL skips it) and receives c.
 * req_id [B] (NULL: the request index) keys the random streams of each request.
 *
 * Recurrent head (QbitAI "DSpark in 10 concepts", section "Cheaper serial module: the Markov
 * head", and 10100.com, section "Parallel drafts are fast but may turn 'of course' into 'of
 * problem'": an optional RNN head that follows the whole draft prefix, of limited gain and
 * off by default; the pages give no form).  When gru_wi is non-NULL (then gru_wh, gru_bi and
 * gru_bh are required too) the left operand U[prev] above is replaced by a_k, the state of a
 * GRU (Cho et al., EMNLP 2014) over the previous tokens' factors rounded to bfloat16:
 *   e_k = U[prev_k];  h_{-1} = 0;  h_k = GRU(h_{k-1}, e_k) in float32
 *   g = sigmoid(Wi_g e + bi_g + Wh_g h + bh_g), z = sigmoid(Wi_z e + bi_z + Wh_z h + bh_z),
 *   n = tanh(Wi_n e + bi_n + g * (Wh_n h + bh_n)), h' = (1 - z) * n + z * h
 *   a_k = bfloat16(h_k) (nearest, ties to even);  c[v] = Z[b][k][v] + sum_i a_k[i] W[v][i]
 * gru_wi, gru_wh [3r][r] float32 (rows: reset units, update units, new units), gru_bi,
 * gru_bh [3r].  Requires bfloat16 factors with r = 64, 128 or 256 (else DSPARK_EINVAL).
 * head_state (optional, [B][K][r] bfloat16) receives a_k for every drafted position (other
 * positions are not written); dspark_verify needs it to recompute a rejected position.
 */
typedef struct {
    int32_t B, K, V, r;
    int32_t z_dtype, uw_dtype; /* dspark_dtype */
    const void *Z;
    const void *U;
    const void *W;
    const int32_t *prev_token;  /* [B]                          */
    const int32_t *draft_len;   /* [B] in [0, K], or NULL (= K) */
    const float *temperature;   /* [B] >= 0; 0 = greedy         */
    const uint32_t *req_id;     /* [B] or NULL                  */
    uint64_t seed;
    int32_t *draft_tokens; /* out [B][K]                 */
    float *q_tok;          /* out [B][K]                 */
    float *q_lse;          /* out [B][K]                 */
    float *corrected;      /* optional out [B][K][V]     */
    dspark_trace *trace;   /* optional                   */
    const float *gru_wi;   /* recurrent head: [3r][r], or NULL (Markov head) */
    const float *gru_wh;   /* [3r][r]                    */
    const float *gru_bi;   /* [3r]                       */
    const float *gru_bh;   /* [3r]                       */
    uint16_t *head_state;  /* optional out [B][K][r] bfloat16 (recurrent head) */
    int32_t sampler;       /* dspark_sampler; 0 (a zero-initialised struct) = per token */
} dspark_draft_args;

/*
 * dspark_schedule -- per-request verification length.
 *
 * surv[b][k] = 1 / (1 + exp(-theta[k] * conf_logits[b][k])); P[b][k] = prod_{j <= k} surv[b][j]
 * (float64), theta = conf_inv_temp (per-position inverse temperatures, e.g. kept by
 * dspark_calibrate), or 1 when NULL.  Every item (b, k) with k < K_b is ranked by (P desc, k asc, b asc).  For
 * n = 0 .. sum_b K_b:  E(n) = B + (sum of the top-n P), N(n) = B + n,
 * G(n) = E(n) * T(N(n)) / N(n), where T is the throughput profile (tokens/s as a function of
 * the total tokens in the verify batch) interpolated linearly between knots and clamped
 * outside them.  n* = the smallest n maximising G; verify_len[b] = the number of request b's
 * items among the top n* (always a prefix of its draft).  E counts one correction / bonus
 * token per request, N one target position per verified token plus one per request.
 * enabled = 0: verify_len = draft_len (or K).
 * expected_tokens [B] (optional, float64) = 1 + sum_{k < verify_len[b]} P[b][k].
 * Limits: K in [1, 64]; when enabled, B * K <= 8192 and n_knots in [1, 64]; knot tokens
 * strictly increasing and positive, throughputs positive (checked on the device).
 * Workspace: dspark_schedule_workspace_size(B, K): the status word, then, for up to 8192
 * items, each item's float64 prefix product and int32 rank (filled when enabled).
 */
typedef struct {
    int32_t B, K;
    const float *conf_logits;  /* [B][K]            */
    const int32_t *draft_len;  /* [B] or NULL (= K) */
    int32_t n_knots;
    const double *knot_tokens; /* [n_knots]         */
    const double *knot_tps;    /* [n_knots]         */
    int32_t enabled;
    int32_t *verify_len;       /* out [B]           */
    double *expected_tokens;   /* optional out [B]  */
    const double *conf_inv_temp; /* [K] or NULL (= 1) */
    dspark_trace *trace;
} dspark_schedule_args;

/*
 * dspark_calibrate -- online calibration of the confidence logits, one step per verified
 * round (QbitAI "DSpark in 10 concepts", section "Online drafter calibration": raw survival
 * scores are over-confident, sequential temperature scaling brings the expected calibration
 * error from 3-8% to about 1%, and the thresholds follow the acceptance the running drafter
 * actually achieves; 10100.com commentary, section "letting the GPU decide how much to
 * verify").  The pages give no formula; the reading implemented:
 *
 *   position k has an inverse temperature theta[k] > 0, calibrated survival
 *   sigmoid(theta[k] * C[b][k]);  a round labels the positions it tested: position k of
 *   request b is tested iff k < verify_len[b] and k <= accept_len[b], with label 1 (accepted)
 *   for k < accept_len[b] and 0 for k = accept_len[b] -- each position is fitted on the
 *   requests whose earlier positions all passed;  then, per position, one damped Newton step
 *   on the round's log-loss  l(theta) = sum log(1 + exp(theta C)) - y theta C:
 *     theta[k] <- clamp(theta[k] - step * l'(theta[k]) / (l''(theta[k]) + ridge), 1/64, 64)
 *   with l' = sum (sigmoid(theta C) - y) C and l'' = sum sigmoid(theta C)(1 - sigmoid(theta C)) C^2
 *   (float64; a position with no tested request keeps its theta).
 *
 * conf_logits, verify_len, accept_len: the round's schedule input and verify outputs (device).
 * inv_temp [K] (device, float64): read and updated in place; start from 1.
 * Lengths outside [0, K] and accepted lengths outside [0, verify_len] are clamped and flagged
 * (DSPARK_DEV_BAD_LENGTH).  step in (0, 1], ridge > 0 (host-validated: DSPARK_EINVAL).
 * Limits: K in [1, 64].  Workspace: dspark_calibrate_workspace_size (the status word).
 */
typedef struct {
    int32_t B, K;
    const float *conf_logits;  /* [B][K]                         */
    const int32_t *verify_len; /* [B]                            */
    const int32_t *accept_len; /* [B]                            */
    double *inv_temp;          /* [K], updated in place          */
    double step, ridge;
    dspark_trace *trace;
} dspark_calibrate_args;

/*
 * dspark_verify -- lossless rejection-sampling verification.
 *
 * For request b with L = verify_len[b] (<= K) and temperature T = temperature[b]:
 *   for k = 0 .. L-1:
 *     T = 0: accept iff draft_tokens[b][k] == argmax_v Y[b][k][v];
 *     T > 0: p = softmax(Y[b][k] / T); u = uniform(stream 1, position k, v = 0);
 *            accept iff u * q_tok[b][k] < p(x_k)   (u < p/q; p >= q always passes).
 *   First rejection at k = j: accept_len = j and next_token is
 *     T = 0: argmax_v Y[b][j][v];
 *     T > 0: q_j(v) = exp(c_j[v] / T - q_lse[b][j]) with c_j recomputed by the Markov head
 *            (previous token prev_token[b] for j = 0, else draft_tokens[b][j-1]), or, when
 *            head_state is given (a recurrent-head draft), from its operand head_state[b][j];
 *            r = max(0, p - q_j); the sampler's draw from the weights r on the residual
 *            stream(s) at position j; if r is identically zero, the same draw from p.
 *   No rejection: accept_len = L and next_token is argmax_v Y[b][L][v] (T = 0) or the
 *   sampler's draw from Y[b][L] / T on the bonus stream(s) at position L (the bonus token).
 * Layouts: Y [B][K+1][V] (row K+1 exists for the bonus); draft_tokens, q_tok, q_lse [B][K]
 * as written by dspark_draft_block; Z, U, W, prev_token, req_id, seed, temperature, the
 * sampler and the dtypes must be the ones the draft used.  Temperature matters for the law,
 * not only for parity: the residual rebuilds q_j from this call's T and the draft's q_lse, so
 * a draft taken at another temperature (a greedy draft verified with T > 0 included) gives a
 * residual that is not max(0, p - q) of the distribution the draft was drawn from, and
 * next_token no longer has the target's law.  The call cannot detect such a mismatch (q_tok
 * and q_lse of a sampled draft may equal a greedy draft's 1 and 0).
 * Y may be float32 or bfloat16.
 * Outputs: accept_len [B], next_token [B]; p_tok [B][K] optional: p(x_k) for each tested
 * position (1 / 0 for a greedy match / mismatch), 0 for untested positions.
 * head_state [B][K][r] bfloat16 (as written by dspark_draft_block's recurrent head) requires
 * bfloat16 factors with r = 64, 128 or 256 (else DSPARK_EINVAL).
 */
typedef struct {
    int32_t B, K, V, r;
    int32_t y_dtype, z_dtype, uw_dtype;
    const void *Y;
    const int32_t *draft_tokens; /* [B][K] */
    const float *q_tok;          /* [B][K] */
    const float *q_lse;          /* [B][K] */
    const void *Z;
    const void *U;
    const void *W;
    const int32_t *prev_token;   /* [B]    */
    const int32_t *verify_len;   /* [B]    */
    const float *temperature;    /* [B]    */
    const uint32_t *req_id;      /* [B] or NULL */
    uint64_t seed;
    int32_t *accept_len;         /* out [B]               */
    int32_t *next_token;         /* out [B]               */
    float *p_tok;                /* optional out [B][K]   */
    dspark_trace *trace;
    const uint16_t *head_state;  /* [B][K][r] bfloat16 from a recurrent-head draft, or NULL */
    int32_t sampler;             /* dspark_sampler of the residual / bonus draws; 0 = per token */
} dspark_verify_args;

/* Workspace bytes each call needs for the given sizes (0 on invalid sizes). */
size_t dspark_draft_workspace_size(int32_t B, int32_t K, int32_t V, int32_t r);
size_t dspark_schedule_workspace_size(int32_t B, int32_t K);
size_t dspark_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t r);
size_t dspark_calibrate_workspace_size(int32_t B, int32_t K);

/* The three calls.  `ws` is a device buffer of at least the queried size, 256-byte aligned;
 * `stream` is a hipStream_t.  Return DSPARK_OK once everything is enqueued. */
dspark_status dspark_draft_block(const dspark_draft_args *args, void *ws, size_t ws_bytes,
                                 void *stream);
dspark_status dspark_schedule(const dspark_schedule_args *args, void *ws, size_t ws_bytes,
                              void *stream);
dspark_status dspark_verify(const dspark_verify_args *args, void *ws, size_t ws_bytes,
                            void *stream);
dspark_status dspark_calibrate(const dspark_calibrate_args *args, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * dspark_draft_block_static -- dspark_draft_block without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: its scratch (the same layout the
 * workspace would hold, dspark_draft_workspace_size(B, K, V, r) bytes) is a fixed array of
 * DSPARK_STATIC_SCRATCH_BYTES inside the library, one copy per GPU, kept until the process
 * ends; its address on the current device is looked up on the first call on that device.
 *   args           as for dspark_draft_block (same checks, same results)
 *   device_status  caller-owned DEVICE pointer to one uint32_t (required): receives the
 *                  device status bits of the call (cleared by its first kernel), readable with
 *                  dspark_query_device_status(device_status, stream, &bits)
 *   stream         a hipStream_t of the CURRENT device
 * Returns DSPARK_ESCRATCH when dspark_draft_workspace_size(B, K, V, r) exceeds the array
 * (e.g. B = 256, K = 16, V = 151936, r = 256 needs about 2.6 MB), and the errors of
 * dspark_draft_block otherwise.  Every call on one GPU shares that GPU's array and nothing is
 * carried from one call to the next: calls that may overlap on one GPU (two streams, two host
 * threads) race on it and must be serialised by the caller.
 */
#define DSPARK_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
dspark_status dspark_draft_block_static(const dspark_draft_args *args, uint32_t *device_status,
                                        void *stream);

/*
 * dspark_pack_w -- convert the Markov head's right factor from r x V (row i = rank component
 * i over the vocabulary, the factorisation's own shape) to the [V][r] layout every call above
 * reads (QbitAI "DSpark in 10 concepts", section "Cheaper serial module: the Markov head": the
 * bias is a rank-r factorisation U . W).  A one-off step when the weights are loaded, not part
 * of a round.  w_rv [r][V] and w_vr [V][r] are distinct device buffers of dtype DSPARK_F32 or
 * DSPARK_BF16, caller-owned; 1 <= r <= 1024.  Asynchronous on `stream`.  Returns DSPARK_EINVAL
 * (null, aliased or bad sizes), DSPARK_EDTYPE or DSPARK_EHIP.
 */
dspark_status dspark_pack_w(const void *w_rv, void *w_vr, int32_t r, int32_t V, int32_t dtype,
                           void *stream);

/* Synchronises `stream`, then reads the device status word of workspace `ws` (written by the
 * last call that used it).  Returns DSPARK_OK, DSPARK_EDEVICE (and the bits in *bits when
 * bits is not NULL) or DSPARK_EHIP. */
dspark_status dspark_query_device_status(const void *ws, void *stream, uint32_t *bits);

/* Human-readable name of a status code (static string). */
const char *dspark_status_string(dspark_status s);

/* Per-kernel timing.  create: room for `capacity` launches (NULL on failure); reset: forget
 * the recorded launches; count: launches recorded so far; get: synchronises on the i-th
 * launch's end event and returns its kernel name and duration in milliseconds (DSPARK_EINVAL
 * for an index out of range). */
dspark_trace *dspark_trace_create(int32_t capacity);
void dspark_trace_destroy(dspark_trace *t);
void dspark_trace_reset(dspark_trace *t);
int32_t dspark_trace_count(const dspark_trace *t);
dspark_status dspark_trace_get(dspark_trace *t, int32_t i, const char **kernel_name,
                               float *milliseconds);

/* Library version string. */
const char *dspark_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
