// verify.hip -- lossless rejection-sampling verification of a drafted block.
//
// The target model has scored every verified position in one pass; its logits Y[b][k] are
// the input.  Draft token x_k is accepted when a uniform draw u satisfies u * q(x_k) < p(x_k);
// the longest accepted prefix is kept; the first rejected position is resampled from the
// normalised positive part of p - q; if nothing is rejected one extra token is drawn from p
// (QbitAI "DSpark in 10 concepts", section "Speculative decoding"; 10100.com commentary,
// section "speculative decoding is block checking", rule of Leviathan et al.; wangjunjian.com
// tag page, post "Speculative Decoding", steps 3-4).
//
// Kernels, in launch order:
//   verify_rows      one launch per chunk of target rows ([0,2), [2,5), [5,9), [9,17), ...),
//                    over the requests still being verified there (the first launch also
//                    clears the status word, the residual flag, the per-chunk request counts
//                    and the per-request first rejection, and lists every request for the
//                    first decide launch): a fixed grid takes the
//                    (request, row of the chunk, vocabulary slab) items in turn and streams
//                    each slab of Y[b][k] once: softmax max / sum-exp of Y/T in log2 units,
//                    the argmax for greedy rows, and the bonus row's per-token candidates (or
//                    its block race with the two-level sampler).  Rows after
//                    the first rejection are never needed, so only the chunks up to it are
//                    read; the kernel boundaries order the data between chunks.
//   verify_decide    after every chunk but the last, one wave per listed request: merges the
//                    chunk's slab statistics, takes its accept decisions and lists the
//                    request for the next chunk if it is still being verified
//   verify_finish    one wave per request: decides the last chunk, then the accepted length,
//                    the greedy correction / the bonus token (the merged per-token winner, or
//                    the draw inside the winning block), or marks the first rejected row for a
//                    residual draw
//   (markov_head.hip) the residual rows: recompute q_j with the Markov head on the matrix
//                    cores and keep the per-token candidates of max(0, p - q_j) and p (or run
//                    their block races)
//   verify_residual_reduce  merge the candidates (two-level sampler: draw the token inside
//                    the winning block)
#include "dspark_common.hpp"

namespace dspark {

// A listed request: {b, L clamped to [0, K], T as bits, RNG request key}, one 16-byte load.
__device__ __forceinline__ int4 make_req_rec(int b, int K, const int32_t *verify_len,
                                             const float *temperature, const uint32_t *req_id) {
    const int L = verify_len[b];
    const float T = temperature[b];
    const uint32_t req = req_id ? req_id[b] : (uint32_t)b;
    // out-of-range lengths and NaN / negative temperatures are flagged by the finish kernel;
    // here they act as the nearest bound and as greedy
    return make_int4(b, L < 0 ? 0 : (L > K ? K : L), __float_as_int(T), (int)req);
}

// The first chunk lists every request: its row launch also sets up the verification state
// (status word, residual flag, per-chunk counts, first rejections, chunk 0's records) for the
// launches after it, and takes its own requests' records straight from the arguments.
struct FirstChunk {
    int B;  // > 0: this launch is the first chunk
    const int32_t *verify_len;
    const float *temperature;
    const uint32_t *req_id;
    uint32_t *status;
    int32_t *n_resid, *first_reject, *n_alive;
    int4 *list0;
};
__device__ __forceinline__ void first_chunk_setup(const FirstChunk &fc, int K) {
    const int i0 = blockIdx.x * blockDim.x + threadIdx.x, stride = gridDim.x * blockDim.x;
    if (i0 == 0) {
        *fc.status = 0u;
        *fc.n_resid = 0;
    }
    if (i0 < kMaxChunks) fc.n_alive[i0] = i0 == 0 ? fc.B : 0;
    for (int i = i0; i < fc.B; i += stride) {
        fc.first_reject[i] = K + 1;
        fc.list0[i] = make_req_rec(i, K, fc.verify_len, fc.temperature, fc.req_id);
    }
}

__device__ __forceinline__ int clamp_len(int L, int K, uint32_t *status, bool report) {
    if (L < 0 || L > K) {
        if (report) atomicOr(status, DSPARK_DEV_BAD_LENGTH);
        return L < 0 ? 0 : K;
    }
    return L;
}

template <typename YT>
__device__ __forceinline__ float load1(const void *Y, size_t idx);
template <>
__device__ __forceinline__ float load1<float>(const void *Y, size_t idx) {
    return reinterpret_cast<const float *>(Y)[idx];
}
template <>
__device__ __forceinline__ float load1<uint16_t>(const void *Y, size_t idx) {
    return bf16_to_f32(reinterpret_cast<const uint16_t *>(Y)[idx]);
}

// Per-request constants of the verifier.
struct ReqInfo {
    int L;
    float T, inv;
    bool greedy;
    uint32_t req;
};

__device__ __forceinline__ ReqInfo req_info(int4 rec) {
    ReqInfo r;
    r.L = rec.y;
    r.T = __int_as_float(rec.z);
    r.greedy = !(r.T > 0.f);
    r.inv = r.greedy ? 1.f : kLog2e / r.T;
    r.req = (uint32_t)rec.w;
    return r;
}

__device__ __forceinline__ ReqInfo req_info(int b, int K, const int32_t *verify_len,
                                            const float *temperature, const uint32_t *req_id) {
    return req_info(make_req_rec(b, K, verify_len, temperature, req_id));
}

// One wave: merge the slab statistics of rows [k0, k1) of request b (rows past L are not
// verified) and take their accept decisions in order.  Returns the first rejected row, or -1.
// The writer records row statistics, p(x_k) and the rejection; every caller computes the same.
// *last receives the statistics of the deciding row (the rejected row, or row L).
// Rows go eight at a time, one group of eight lanes per row: lane i of group j folds slots
// i, i + 8, i + 16, ... of its row in that order, then the group merges over xor masks 1, 2, 4
// -- a fixed order, so a row's statistics are the same in every caller.  Each group takes its
// row's accept decision; the first deciding row of the eight (a rejection, or row L) is found
// with one ballot.  Everything a pass reads goes out together (the slab partials, and each
// row's draft token, q and target logit), so eight rows cost one or two memory round trips.
template <typename YT>
__device__ int decide_rows(int b, int k0, int k1, const ReqInfo &ri, int K, int V, int S,
                           const void *Y, const int32_t *draft_tokens, const float *q_tok,
                           const Partial *row_partials, uint32_t key0, uint32_t key1,
                           bool writer, float4 *rowstats, float *p_tok, int32_t *first_reject,
                           uint32_t *status, float4 *last = nullptr) {
    const int lane = threadIdx.x & 63;
    const int n = min(k1, ri.L + 1) - k0;  // rows to merge (at most 64)
    if (n <= 0) return -1;
    constexpr int G = 8, LPR = 64 / G, PF = 8;  // rows per pass, lanes per row, slots in flight
    const int j = lane / LPR, i = lane % LPR;
    const size_t rbase = (size_t)b * (K + 1);
    for (int g0 = 0; g0 < n; g0 += G) {
        const bool valid = g0 + j < n;
        const int k = k0 + min(g0 + j, n - 1);  // rows past the pass's end repeat its last row
        const size_t row = rbase + k;
        const bool tested = k < ri.L;
        int x = 0;
        float yx = 0.f, q = 0.f;
        if (tested) {
            x = draft_tokens[(size_t)b * K + k];
            if (x < 0 || x >= V) {
                if (writer && i == 0) atomicOr(status, DSPARK_DEV_BAD_TOKEN);
                x = 0;
            }
            if (!ri.greedy) {
                q = q_tok[(size_t)b * K + k];
                yx = load1<YT>(Y, row * (size_t)V + x);
            }
        }
        Partial pr[PF];
#pragma unroll
        for (int t = 0; t < PF; ++t) pr[t] = row_partials[row * S + min(i + LPR * t, S - 1)];
        SampleState a = sample_state_init();
#pragma unroll
        for (int t = 0; t < PF; ++t)
            if (i + LPR * t < S) merge_into(a, from_partial(pr[t]), ri.greedy);
        for (int sl = i + LPR * PF; sl < S; sl += LPR)
            merge_into(a, from_partial(row_partials[row * S + sl]), ri.greedy);
#pragma unroll
        for (int mask = 1; mask < LPR; mask <<= 1) {
            const SampleState o = shfl_xor_state(a, mask);
            merge_into(a, o, ri.greedy);
        }
        bool accept = true;
        float p = 0.f;
        if (tested) {
            if (ri.greedy) {
                accept = x == a.idx;
                p = accept ? 1.f : 0.f;
            } else {
                // against the row's base m, with one rounding: exact to a few ulps at any T
                p = fast_exp2(fmaf(yx, ri.inv, -a.m) - fast_log2(a.l));
                const Philox4 ph = philox4x32_10(0u, (uint32_t)k, ri.req, kStreamAccept, key0, key1);
                accept = uniform_from_word(ph.w[0]) * q < p;
            }
        }
        // the first deciding row of the pass: a rejection, or row L (nothing to test there)
        const unsigned long long dec = __ballot(valid && i == 0 && (k == ri.L || !accept));
        const int jd = dec ? (int)(__builtin_ctzll(dec) / LPR) : G;  // uniform
        if (writer && valid && i == 0 && j <= jd) {
            rowstats[row] = make_float4(a.m, a.l, __int_as_float(a.idx), a.g);
            if (tested && p_tok) p_tok[(size_t)b * K + k] = p;
            if (j == jd && tested && !accept)
                __hip_atomic_store(first_reject + b, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (jd < G) {
            const int src = jd * LPR;
            if (last)
                *last = make_float4(__shfl(a.m, src), __shfl(a.l, src),
                                    __int_as_float(__shfl(a.idx, src)), __shfl(a.g, src));
            const int kd = k0 + g0 + jd;
            return kd == ri.L ? -1 : kd;
        }
    }
    return -1;
}

// Statistics of one vocabulary slab of one target row (whole workgroup).  Each thread takes
// kRowBlocks sampler blocks per sweep and issues all their loads before using any.  The bonus
// row of a sampled request also carries its draw: per-token candidates (weight against the
// running base, E2, token), or the two-level sampler's block race.
template <typename YT>
__device__ __forceinline__ void row_slab_stats(const void *Y, size_t row, int V, int blk_lo,
                                               int blk_hi, const ReqInfo &ri, bool bonus,
                                               int sampler, int k, uint32_t key0, uint32_t key1,
                                               SampleState &st) {
    const bool tok_bonus = bonus && sampler == DSPARK_SAMPLER_TOKEN;
    TokLane tl = tok_lane_init();
    for (int blk = blk_lo + (int)threadIdx.x; blk < blk_hi; blk += kRowBlocks * kRowThreads) {
        Raw16<YT> y[kRowBlocks];
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
            const int bb = blk + h * kRowThreads;
            y[h].load(Y, row, V, (bb < blk_hi ? bb : blk) * kSampleBlock);
        }
#pragma unroll
        for (int h = 0; h < kRowBlocks; ++h) {
            const int bb = blk + h * kRowThreads;
            if (bb >= blk_hi) break;
            const int v0 = bb * kSampleBlock;
            const int n_live = min(kSampleBlock, V - v0);
            if (ri.greedy) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    greedy_update(st, e < n_live ? y[h].get(e) : -INFINITY, v0 + e);
            } else {
                // weights exp2(y * inv - base), one fused multiply-add each: the base is the
                // largest y scaled once (rounding is monotonic), no scaled logit is rounded
                float s[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) s[e] = e < n_live ? y[h].get(e) : -INFINITY;
                float m16 = s[0];
#pragma unroll
                for (int e = 1; e < 16; ++e) m16 = fmaxf(m16, s[e]);
                m16 *= ri.inv;
                const float mn = fmaxf(st.m, m16);
                const float base = (mn == -INFINITY) ? 0.f : mn;
                const float f = fast_exp2(st.m - base);
                if (tok_bonus) {  // uniform per wave: one row per workgroup pass
                    float acc = 0.f;
                    tl.bw *= f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const Philox4 ph = philox4x32_10(((uint32_t)v0 >> 2) + (uint32_t)c,
                                                         (uint32_t)k, ri.req, kStreamBonus, key0,
                                                         key1);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float w = fast_exp2(fmaf(s[4 * c + i], ri.inv, -base));
                            acc += w;
                            tok_take(tl, w, exp2_from_word(ph.w[i]), v0 + 4 * c + i);
                        }
                    }
                    st.l = st.l * f + acc;
                    st.m = mn;
                } else {
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc += fast_exp2(fmaf(s[e], ri.inv, -base));
                    st.l = st.l * f + acc;
                    st.m = mn;
                    if (bonus) {
                        const uint32_t w = race_word((uint32_t)bb, (uint32_t)k, ri.req,
                                                     kStreamBonus, key0, key1);
                        race_update(st.g, st.idx, base, acc, w, v0);
                    }
                }
            }
        }
    }
    if (tok_bonus) {
        tl.m = st.m;
        const TokState ts = tok_finish(tl);
        st.g = ts.g;
        st.idx = ts.idx;
    }
}

// Chunk [k_lo, k_hi) of the target rows for the n_alive requests listed for it.  Row i of the
// chunk (list entry i / R, row k_lo + i % R) is cut into `runs` runs of blocks at fixed places
// (run s: blocks [s*len, (s+1)*len), len = ceil(blocks / runs)); the chunk's n_alive*R*runs
// runs are shared out as equal contiguous ranges, one per workgroup, and wave w of the
// workgroup that takes run s of a row leaves its partial in slot s * kRowWaves + w.  The list
// order (requests are appended as they survive) thus changes which workgroup computes a run
// but not the partials, so row statistics are reproducible; and the waves never wait for one
// another.
template <typename YT>
__global__ __launch_bounds__(kRowThreads) void verify_rows_kernel(
    int K, int V, const void *Y, uint32_t key0, uint32_t key1, int sampler, int S, int k_lo,
    int k_hi, const int32_t *n_alive, const int4 *alive, Partial *row_partials, FirstChunk fc) {
    const bool first = fc.B > 0;
    if (first) first_chunk_setup(fc, K);
    const int R = k_hi - k_lo;
    const int runs = S / kRowWaves;
    const int n_blk = (V + kSampleBlock - 1) / kSampleBlock;
    const int run_len = (n_blk + runs - 1) / runs;
    const long long T = (long long)(first ? fc.B : *n_alive) * R * runs;
    if (T == 0) return;
    const long long G = T < (long long)gridDim.x ? T : (long long)gridDim.x;
    const long long w = blockIdx.x;
    if (w >= G) return;  // uniform
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long g1 = (w + 1) * T / G;
    long long rec_i = -1;  // list entry of `rec` (consecutive runs mostly share a row)
    int4 rec = make_int4(0, 0, 0, 0);
    for (long long gr = w * T / G; gr < g1; ++gr) {  // uniform: one run per pass
        const long long ri = gr / runs;
        const int run = (int)(gr % runs);
        if (ri / R != rec_i) {
            rec_i = ri / R;
            rec = first ? make_req_rec((int)rec_i, K, fc.verify_len, fc.temperature, fc.req_id)
                        : alive[rec_i];
        }
        const int k = k_lo + (int)(ri % R);
        const ReqInfo info = req_info(rec);
        if (k <= info.L) {  // rows past L are not verified
            const size_t row = (size_t)rec.x * (K + 1) + k;
            const int blk_lo = min(n_blk, run * run_len), blk_hi = min(n_blk, blk_lo + run_len);
            SampleState st = sample_state_init();
            row_slab_stats<YT>(Y, row, V, blk_lo, blk_hi, info, !info.greedy && k == info.L,
                               sampler, k, key0, key1, st);
            for (int mask = 1; mask < 64; mask <<= 1) {
                const SampleState o = shfl_xor_state(st, mask);
                merge_into(st, o, info.greedy);
            }
            if (lane == 0) row_partials[row * S + run * kRowWaves + wave] = to_partial(st);
        }
    }
}

// One wave per request of chunk [k_lo, k_hi) (all B for the first chunk, else the listed
// ones): merge the chunk's slab statistics, take its accept decisions, and list the request
// for the next chunk when it is still being verified there.
template <typename YT>
__global__ __launch_bounds__(256) void verify_decide_kernel(
    int K, int V, const void *Y, const int32_t *draft_tokens, const float *q_tok, uint32_t key0,
    uint32_t key1, int S, int k_lo, int k_hi, const int32_t *n_alive, const int4 *alive,
    const Partial *row_partials, int32_t *first_reject, float4 *rowstats, float *p_tok,
    int32_t *n_next, int4 *next, uint32_t *status) {
    const int lane = threadIdx.x & 63;
    const int ai = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    const int n_req = *n_alive;
    if (ai >= n_req) return;  // uniform per wave
    const int4 rec = alive[ai];
    const int b = rec.x;
    const ReqInfo ri = req_info(rec);
    const int rej = decide_rows<YT>(b, k_lo, k_hi, ri, K, V, S, Y, draft_tokens, q_tok,
                                    row_partials, key0, key1, true, rowstats, p_tok, first_reject,
                                    status);
    if (lane == 0 && rej < 0 && ri.L >= k_hi) next[atomicAdd(n_next, 1)] = rec;
}

// One wave per request.  [c_lo, c_hi) is the last chunk of rows, which no later launch has
// decided.
template <typename YT>
__global__ __launch_bounds__(256) void verify_finish_kernel(
    int B, int K, int V, const void *Y, const int32_t *draft_tokens, const float *q_tok,
    const int32_t *verify_len, const float *temperature, const uint32_t *req_id, uint32_t key0,
    uint32_t key1, int sampler, int S, int c_lo, int c_hi, const Partial *row_partials,
    int32_t *first_reject, float4 *rowstats, int32_t *accept_len, int32_t *next_token,
    float *p_tok, int32_t *n_resid, int32_t *resid_rows, uint32_t *status) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (b >= B) return;  // uniform per wave
    if (lane == 0) {
        clamp_len(verify_len[b], K, status, true);
        checked_temperature(temperature[b], status);
    }
    const ReqInfo ri = req_info(b, K, verify_len, temperature, req_id);
    const size_t rbase = (size_t)b * (K + 1);
    if (lane == 0) resid_rows[b] = -1;  // replaced below when the request needs a residual draw
    int fr = first_reject[b];
    bool here = false;  // the deciding row is in the last chunk, merged by this wave
    float4 rs = make_float4(0.f, 0.f, 0.f, 0.f);
    if (fr >= c_lo && ri.L >= c_lo) {
        const int rej = decide_rows<YT>(b, c_lo, c_hi, ri, K, V, S, Y, draft_tokens, q_tok,
                                        row_partials, key0, key1, true, rowstats, p_tok,
                                        first_reject, status, &rs);
        if (rej >= 0) fr = rej;
        here = true;
    }
    // every position before the first rejection was decided
    const bool rejected = fr < ri.L;
    const int a = rejected ? fr : ri.L;
    if (p_tok)  // positions after the deciding one were not tested
        for (int k = a + (rejected ? 1 : 0) + lane; k < K; k += 64) p_tok[(size_t)b * K + k] = 0.f;
    if (lane == 0) accept_len[b] = a;
    if (rejected && !ri.greedy) {
        // row b of the residual pass (no compaction: a shared counter would serialise the
        // waves' atomics); the flag only tells the residual launches that there is work
        if (lane == 0) {
            resid_rows[b] = b * 128 + a;
            *n_resid = 1;
            next_token[b] = -1;  // written by the residual reduction
        }
        return;
    }
    // row a's statistics: merged just now, or written by an earlier launch
    if (!here) rs = rowstats[rbase + a];
    int t = __float_as_int(rs.z);
    if (!ri.greedy && sampler == DSPARK_SAMPLER_TOKEN) {
        // bonus: the merged per-token winner of row L (none when the row has no finite logit)
        if (!(rs.w > -INFINITY)) t = -1;
    } else if (!ri.greedy) {
        // bonus: the token inside the winning block of row L
        const int v0 = t;
        t = -1;
        if (v0 >= 0 && v0 < V && v0 % kSampleBlock == 0) {
            const int e = lane & 15;
            const int v = min(v0 + e, V - 1);
            const uint32_t w = token_word((uint32_t)(v0 + e), (uint32_t)ri.L, ri.req,
                                          kStreamBonusWithin, key0, key1);
            float sc = v0 + e < V ? load1<YT>(Y, (rbase + ri.L) * (size_t)V + v) * ri.inv +
                                        gumbel2_from_word(w)
                                  : -INFINITY;
            int tok = v0 + e;
            float aux = 0.f;
            wave_argmax16(sc, tok, aux);
            if (sc > -INFINITY) t = tok;
        }
    }
    if (lane == 0) {
        if (t < 0 || t >= V) {  // no finite logit in the row
            atomicOr(status, DSPARK_DEV_BAD_TOKEN);
            t = 0;
        }
        next_token[b] = t;
    }
}

// One wave per residual row: merge the block races, then draw inside the winning block from
// the recomputed weights r_v = max(p_v - q_v, 0) (or p_v when the residual is zero).
__global__ __launch_bounds__(256) void verify_residual_reduce_kernel(
    int K, int V, int r, int y_dtype, int z_dtype, int uw_dtype, const void *Y,
    const void *Z, const void *U, const void *W, const int32_t *prev_token,
    const int32_t *draft_tokens, const float *q_lse, const float *temperature,
    const uint32_t *req_id, uint32_t key0, uint32_t key1, const float4 *rowstats,
    const int32_t *n_resid, const int32_t *resid_rows, const Partial *partials, int n_slabs,
    const uint16_t *head_state, int sampler, int32_t *next_token, uint32_t *status, int B) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);  // = request b
    if (row >= B || *n_resid == 0) return;  // uniform per wave
    // the row's record, its slab partials (four per lane) and the request's values go out
    // together (absent optional arrays are read at a stand-in address and replaced)
    const int packed = resid_rows[row];
    constexpr int kPer = 4;
    const Partial *prow = partials + (size_t)row * n_slabs;
    Partial pp[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) pp[i] = prow[min(lane + 64 * i, n_slabs - 1)];
    const int b = row;
    const uint32_t *rq = req_id ? req_id : reinterpret_cast<const uint32_t *>(prev_token);
    const float T = temperature[b];  // > 0: greedy rows never need a residual
    const uint32_t req_ld = rq[b];
    const int pt = prev_token[b];
    if (packed < 0) return;  // no residual draw for this request
    // then the loads that need the record's position
    const int j = packed & 127;
    const size_t zrow = (size_t)b * K + j, yrow = (size_t)b * (K + 1) + j;
    const int dt = draft_tokens[(size_t)b * K + (j > 0 ? j - 1 : 0)];
    const float4 rs = rowstats[yrow];
    const float ql = q_lse[zrow];
    float gr = -INFINITY, gp = -INFINITY;
    int ir = 0x7FFFFFFF, ip = 0x7FFFFFFF;
    auto take = [&](const Partial &q) {
        const int qip = __float_as_int(q.l);
        if (q.g > gr || (q.g == gr && q.idx < ir)) {
            gr = q.g;
            ir = q.idx;
        }
        if (q.m > gp || (q.m == gp && qip < ip)) {
            gp = q.m;
            ip = qip;
        }
    };
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        if (lane + 64 * i < n_slabs) take(pp[i]);
    for (int s = lane + 64 * kPer; s < n_slabs; s += 64) take(prow[s]);
    for (int mask = 1; mask < 64; mask <<= 1) {
        const float ogr = __shfl_xor(gr, mask), ogp = __shfl_xor(gp, mask);
        const int oir = __shfl_xor(ir, mask), oip = __shfl_xor(ip, mask);
        if (ogr > gr || (ogr == gr && oir < ir)) {
            gr = ogr;
            ir = oir;
        }
        if (ogp > gp || (ogp == gp && oip < ip)) {
            gp = ogp;
            ip = oip;
        }
    }
    const bool use_r = gr > -INFINITY;
    const int v0 = use_r ? ir : ip;
    int t = -1;
    if (sampler == DSPARK_SAMPLER_TOKEN) {
        if (use_r) {
            // the merged per-token winner over r
            if (v0 >= 0 && v0 < V) t = v0;
        } else {
            // no positive residual anywhere in the row (unreachable in exact arithmetic after a
            // rejection): this wave draws from p over the whole row, per token, on the residual
            // stream -- weights p_v = exp2(y_v / T - lse2 of the row), candidates as weight / E2
            const float inv = kLog2e / T;
            const float lse2p = rs.x + fast_log2(rs.y);
            const uint32_t req = req_id ? req_ld : (uint32_t)b;
            float bw = 0.f, be = 1.f;
            int bi = 0x7FFFFFFF;
            for (int v4 = 4 * lane; v4 < V; v4 += 4 * 64) {  // V % 4 == 0: v4 + 3 < V
                const Philox4 ph = philox4x32_10((uint32_t)v4 >> 2, (uint32_t)j, req,
                                                 kStreamResidual, key0, key1);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = fast_exp2(
                        fmaf(load_value(Y, y_dtype, yrow * (size_t)V + v4 + i), inv, -lse2p));
                    const float E = exp2_from_word(ph.w[i]);
                    const bool take_v = pv * be > bw * E;
                    bw = take_v ? pv : bw;
                    be = take_v ? E : be;
                    bi = take_v ? v4 + i : bi;
                }
            }
            float sc = bw > 0.f ? fast_log2(bw) - fast_log2(be) : -INFINITY;
            int tok = bi;
            for (int mask = 1; mask < 64; mask <<= 1) {
                const float os = __shfl_xor(sc, mask);
                const int ot = __shfl_xor(tok, mask);
                if (os > sc || (os == sc && ot < tok)) {
                    sc = os;
                    tok = ot;
                }
            }
            if (sc > -INFINITY && tok >= 0 && tok < V) t = tok;
        }
    } else if (v0 >= 0 && v0 < V && v0 % kSampleBlock == 0) {
        const float inv = kLog2e / T;
        const uint32_t req = req_id ? req_ld : (uint32_t)b;
        int prev = (j == 0) ? pt : dt;
        if (prev < 0 || prev >= V) prev = 0;  // flagged by the rows / finish kernels
        const float lse2p = rs.x + fast_log2(rs.y);
        const float qlse2 = ql * kLog2e;
        // the left operand: U[prev] (Markov head) or the stored recurrent-head operand
        const void *op = head_state ? static_cast<const void *>(head_state + zrow * (size_t)r) : U;
        const float c = wave_corrected16(Z, z_dtype, zrow, op, W, uw_dtype, r, V,
                                         head_state ? 0 : prev, v0);
        const int e = lane & 15;
        const int v = min(v0 + e, V - 1);
        const bool in = v0 + e < V;
        const float pv = fast_exp2(fmaf(load_value(Y, y_dtype, yrow * (size_t)V + v), inv, -lse2p));
        const float rv = pv - fast_exp2(fmaf(c, inv, -qlse2));
        const float g = gumbel2_from_word(token_word((uint32_t)(v0 + e), (uint32_t)j, req,
                                                     kStreamResidualWithin, key0, key1));
        const float lw_r = (in && rv > 0.f) ? fast_log2(rv) : -INFINITY;
        const float lw_p = (in && pv > 0.f) ? fast_log2(pv) : -INFINITY;
        float sc = (use_r ? lw_r : lw_p) + g;
        int tok = v0 + e;
        float aux = 0.f;
        wave_argmax16(sc, tok, aux);
        if (!(sc > -INFINITY) && use_r) {
            // the recomputed residual of the chosen block rounded to zero: draw from p there
            sc = lw_p + g;
            tok = v0 + e;
            wave_argmax16(sc, tok, aux);
        }
        if (sc > -INFINITY) t = tok;
    }
    if (lane == 0) {
        if (t < 0 || t >= V) {
            atomicOr(status, DSPARK_DEV_BAD_TOKEN);
            t = 0;
        }
        next_token[b] = t;
    }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------

// Chunk plan of a call.  Rows 0 .. K go in chunks of 2, 3, 4, 8, 16, ... rows: short first
// chunks, since most requests stop within a few rows.  When the whole target stream is small
// (at most kOneChunkBytes, a few microseconds of reading) the launches dominate -- a row
// launch and a decide launch cost ~6 us each -- and all rows go in one chunk, read for every
// request.  A chunk holds at most 64 rows (one decide wave has a lane per row).
int verify_chunks(const dspark_verify_args &a, int bounds[kMaxChunks + 1]) {
    constexpr double kOneChunkBytes = 32.0 * (1 << 20);
    const int rows = a.K + 1;
    const double bytes = (double)a.B * a.V * (a.y_dtype == DSPARK_BF16 ? 2 : 4) * rows;
    bounds[0] = 0;
    if (rows <= 64 && bytes <= kOneChunkBytes) {
        bounds[1] = rows;
        return 1;
    }
    static const int edges[] = {0, 2, 5, 9, 17, 33, 65};
    int n = 0;
    for (int i = 1; i < (int)(sizeof(edges) / sizeof(edges[0])); ++i) {
        const int e = edges[i] < rows ? edges[i] : rows;
        if (e > bounds[n]) bounds[++n] = e;
        if (e == rows) break;
    }
    return n;
}

// records of the requests listed for chunk c (chunk 0: all of them)
static int4 *alive_list(const VerifyWs &ws, int c, int B) { return ws.alive + (size_t)c * B; }

hipError_t launch_verify_rows(const dspark_verify_args &a, const VerifyWs &ws, int chunk,
                              hipStream_t s) {
    int bounds[kMaxChunks + 1];
    const int n = verify_chunks(a, bounds);
    if (chunk < 0 || chunk >= n) return hipErrorInvalidValue;
    const int k_lo = bounds[chunk], k_hi = bounds[chunk + 1];
    const uint32_t k0 = (uint32_t)(a.seed & 0xFFFFFFFFu), k1 = (uint32_t)(a.seed >> 32);
    // enough workgroups for every run of every request of the chunk; the kernel uses fewer
    // when fewer are listed
    long long grid = (long long)a.B * (k_hi - k_lo) * (ws.n_row_slabs / kRowWaves);
    grid = grid < 1 ? 1 : (grid > kRowGrid ? kRowGrid : grid);
    const int4 *list = alive_list(ws, chunk, a.B);
    const int32_t *cnt = ws.n_alive + chunk;
    FirstChunk fc{};
    if (chunk == 0)
        fc = FirstChunk{a.B,       a.verify_len,     a.temperature, a.req_id,  ws.status,
                        ws.n_resid, ws.first_reject, ws.n_alive,    ws.alive};
    if (a.y_dtype == DSPARK_BF16)
        verify_rows_kernel<uint16_t><<<(unsigned)grid, kRowThreads, 0, s>>>(
            a.K, a.V, a.Y, k0, k1, a.sampler, ws.n_row_slabs, k_lo, k_hi, cnt, list,
            ws.row_partials, fc);
    else
        verify_rows_kernel<float><<<(unsigned)grid, kRowThreads, 0, s>>>(
            a.K, a.V, a.Y, k0, k1, a.sampler, ws.n_row_slabs, k_lo, k_hi, cnt, list,
            ws.row_partials, fc);
    return hipGetLastError();
}

hipError_t launch_verify_decide(const dspark_verify_args &a, const VerifyWs &ws, int chunk,
                                hipStream_t s) {
    int bounds[kMaxChunks + 1];
    const int n = verify_chunks(a, bounds);
    if (chunk < 0 || chunk + 1 >= n) return hipErrorInvalidValue;  // not the last chunk
    const int k_lo = bounds[chunk], k_hi = bounds[chunk + 1];
    const uint32_t k0 = (uint32_t)(a.seed & 0xFFFFFFFFu), k1 = (uint32_t)(a.seed >> 32);
    const int per_block = 1;  // one wave per request and workgroup: spread over the CUs
    const dim3 grid((a.B + per_block - 1) / per_block), block(64 * per_block);
    const int4 *list = alive_list(ws, chunk, a.B);
    const int32_t *cnt = ws.n_alive + chunk;
    int4 *next = alive_list(ws, chunk + 1, a.B);
    int32_t *n_next = ws.n_alive + chunk + 1;
    if (a.y_dtype == DSPARK_BF16)
        verify_decide_kernel<uint16_t><<<grid, block, 0, s>>>(
            a.K, a.V, a.Y, a.draft_tokens, a.q_tok, k0, k1, ws.n_row_slabs, k_lo, k_hi, cnt,
            list, ws.row_partials, ws.first_reject, ws.rowstats, a.p_tok, n_next, next,
            ws.status);
    else
        verify_decide_kernel<float><<<grid, block, 0, s>>>(
            a.K, a.V, a.Y, a.draft_tokens, a.q_tok, k0, k1, ws.n_row_slabs, k_lo, k_hi, cnt,
            list, ws.row_partials, ws.first_reject, ws.rowstats, a.p_tok, n_next, next,
            ws.status);
    return hipGetLastError();
}

hipError_t launch_verify_finish(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s) {
    int bounds[kMaxChunks + 1];
    const int n = verify_chunks(a, bounds);
    const uint32_t k0 = (uint32_t)(a.seed & 0xFFFFFFFFu), k1 = (uint32_t)(a.seed >> 32);
    const int per_block = 1;  // one wave per request and workgroup: spread over the CUs
    const dim3 grid((a.B + per_block - 1) / per_block), block(64 * per_block);
    const int c_lo = bounds[n - 1], c_hi = bounds[n];
    if (a.y_dtype == DSPARK_BF16)
        verify_finish_kernel<uint16_t><<<grid, block, 0, s>>>(
            a.B, a.K, a.V, a.Y, a.draft_tokens, a.q_tok, a.verify_len, a.temperature, a.req_id,
            k0, k1, a.sampler, ws.n_row_slabs, c_lo, c_hi, ws.row_partials, ws.first_reject, ws.rowstats,
            a.accept_len, a.next_token, a.p_tok, ws.n_resid, ws.resid_rows, ws.status);
    else
        verify_finish_kernel<float><<<grid, block, 0, s>>>(
            a.B, a.K, a.V, a.Y, a.draft_tokens, a.q_tok, a.verify_len, a.temperature, a.req_id,
            k0, k1, a.sampler, ws.n_row_slabs, c_lo, c_hi, ws.row_partials, ws.first_reject, ws.rowstats,
            a.accept_len, a.next_token, a.p_tok, ws.n_resid, ws.resid_rows, ws.status);
    return hipGetLastError();
}

hipError_t launch_verify_residual_reduce(const dspark_verify_args &a, const VerifyWs &ws,
                                         hipStream_t s) {
    const int per_block = 1;  // one wave per request and workgroup
    verify_residual_reduce_kernel<<<(a.B + per_block - 1) / per_block, 64 * per_block, 0, s>>>(
        a.K, a.V, a.r, a.y_dtype, a.z_dtype, a.uw_dtype, a.Y, a.Z, a.U, a.W, a.prev_token,
        a.draft_tokens, a.q_lse, a.temperature, a.req_id, (uint32_t)(a.seed & 0xFFFFFFFFu),
        (uint32_t)(a.seed >> 32), ws.rowstats, ws.n_resid, ws.resid_rows, ws.partials,
        ws.n_slabs, a.head_state, a.sampler, a.next_token, ws.status, a.B);
    return hipGetLastError();
}

}  // namespace dspark
