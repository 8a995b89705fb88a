// dspark_common.hpp -- device helpers and internal launch interfaces of libdspark.so.
//
// Everything here is written for gfx950 (CDNA4, wave64).  The random-number definition, the
// sampling rules (the per-token Gumbel-max, and the optional two-level block race) and the
// tie-break rule are those stated in include/dspark.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Philox stream ids: the per-token draws of the draft, residual and bonus tokens (which are
// also the race streams of the optional two-level sampler), the accept test, and the
// within-block draws of the two-level sampler.
constexpr uint32_t kStreamDraft = 0, kStreamAccept = 1, kStreamResidual = 2, kStreamBonus = 3,
                   kStreamDraftWithin = 4, kStreamResidualWithin = 5, kStreamBonusWithin = 6;
constexpr int kSampleBlock = 16;  // tokens per block of the two-level sampler

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// float -> bfloat16 bits, nearest with ties to even (a NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Each round multiplies counter words 0
// and 2 by the published multipliers (one v_mad_u64_u32 each, full rate on gfx950), xors the
// high halves into the other two words together with the round key (one three-input
// v_bitop3_b32 each: truth table 0x96 is a ^ b ^ c), and the key advances by the Weyl
// constants.
// ---------------------------------------------------------------------------------------

struct Philox4 {
    uint32_t w[4];
};

__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t pa = (uint64_t)0xD2511F53u * (uint64_t)c0;
        const uint64_t pb = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        const uint32_t n0 = xor3((uint32_t)(pb >> 32), c1, k0);
        const uint32_t n2 = xor3((uint32_t)(pa >> 32), c3, k1);
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Philox4 r;
    r.w[0] = c0;
    r.w[1] = c1;
    r.w[2] = c2;
    r.w[3] = c3;
    return r;
}

// Uniform u = ((word >> 8) + 0.5) / 2^24 as float.  Exact for u < 1/2; above that the float
// rounds to the 2^-24 grid (the accept test tolerates it; the samplers use exp_from_word).
__device__ __forceinline__ float uniform_from_word(uint32_t word) {
    return fmaf((float)(word >> 8), 0x1p-24f, 0x1p-25f);
}

// E = -ln(u) for the uniform of `word`, accurate in relative terms over the whole range:
// for u < 1/2 the float u is exact; for u >= 1/2 the complement d = 1 - u is exact in float
// and, when d < 2^-8, E = d + d^2/2 + d^3/3 (truncation < 2^-26 relative) -- this is the
// region where E is tiny and the Gumbel draw -ln E is large, i.e. where samples are decided.
__device__ __forceinline__ float exp_from_word(uint32_t word) {
    const uint32_t m = word >> 8;
    const float u = fmaf((float)m, 0x1p-24f, 0x1p-25f);
    const float d = fmaf((float)(0xFFFFFFu - m), 0x1p-24f, 0x1p-25f);
    const float series = d * fmaf(d, fmaf(d, 0.33333334f, 0.5f), 1.0f);
    const float direct = -fast_log2(u) * kLn2;
    return d < 0x1p-8f ? series : direct;
}

// Gumbel draw of a word in log2 units: -log2(E) = log2(e) * (-ln E).
__device__ __forceinline__ float gumbel2_from_word(uint32_t word) {
    return -fast_log2(exp_from_word(word));
}

// E2 = -log2(u) = log2(e) * E for the uniform of `word`, accurate in relative terms (the
// per-token draws rank tokens by w / E2, which orders them as w / E does).  u = (m + 1/2) 2^-24
// is exact in float for u < 1/2 and rounds to the 2^-24 grid above; the rounding
// e = u - fl(u) (0 or +-2^-25) is recovered exactly (m 2^-24 - fl(u) is exact, then + 2^-25),
// and -log2(u) = -log2(fl(u)) - log2(e) e / u to first order, with 1/u replaced by 1 (the
// difference is e (1 - u) / u, below 2^-25 relative to E2).  v_log_f32 keeps its relative
// accuracy near 1 (measured on gfx950 over every float in [1/2, 1): 1.0e-7), so E2 is within
// 1.5e-7 relative of -log2(u) for every word -- also where E2 is tiny and the draw is large,
// i.e. where samples are decided.
__device__ __forceinline__ float exp2_from_word(uint32_t word) {
    const float fm = (float)(word >> 8);
    const float u = fmaf(fm, 0x1p-24f, 0x1p-25f);
    const float e = fmaf(fm, 0x1p-24f, -u) + 0x1p-25f;  // u - fl(u), exact
    return fmaf(e, -kLog2e, -fast_log2(u));
}

// ---------------------------------------------------------------------------------------
// Per-token Gumbel-max, streamed.  Token v wins when it maximises a_v + G_v, i.e. w_v / E_v
// with w_v = exp(a_v - base) for any common base and E_v = -log u_v.  A lane keeps its best
// candidate as (weight against the lane's running base, E2, token); when the base rises the
// weight is rescaled with the same factor as the running sum.  At the end the candidate's
// score in log2 units is base + log2(w) - log2(E2) (the offset -log2(log2 e) from a_v + G_v in
// log2 units is the same for every token) and its scaled logit a_x in log2 units is
// base + log2(w).
// ---------------------------------------------------------------------------------------

struct TokLane {
    float m, l;   // running base (log2 units; -inf before any live entry) and sum of weights
    float bw, be; // best candidate: weight against the base, and its E2
    int bi;       // its token
};

__device__ __forceinline__ TokLane tok_lane_init() {
    TokLane t;
    t.m = -INFINITY;
    t.l = 0.f;
    t.bw = 0.f;
    t.be = 1.f;
    t.bi = 0x7FFFFFFF;
    return t;
}

// Candidate token v with weight w (against the lane's current base) and E2 = e: strict >, so
// within a lane (tokens visited in increasing order) exact ties keep the lower token.
__device__ __forceinline__ void tok_take(TokLane &t, float w, float e, int v) {
    const bool take = w * t.be > t.bw * e;
    t.bw = take ? w : t.bw;
    t.be = take ? e : t.be;
    t.bi = take ? v : t.bi;
}

// Per-token state of a row for merging: softmax statistics (m, l), the best score g (log2
// units), its token, and its scaled logit sx taken against the base m (log2 of its weight):
// q(x) = exp2(sx) / l needs no difference of two large numbers, so it stays exact to a few
// ulps at any temperature (the scaled logits themselves reach the hundreds at small T).
struct TokState {
    float m, l, g, sx;
    int idx;
};

__device__ __forceinline__ TokState tok_state_init() {
    TokState s;
    s.m = -INFINITY;
    s.l = 0.f;
    s.g = -INFINITY;
    s.sx = -INFINITY;
    s.idx = 0x7FFFFFFF;
    return s;
}

__device__ __forceinline__ TokState tok_finish(const TokLane &t) {
    TokState s;
    s.m = t.m;
    s.l = t.l;
    const bool any = t.bw > 0.f;
    const float base = (t.m == -INFINITY) ? 0.f : t.m;
    const float lw = any ? fast_log2(t.bw) : -INFINITY;
    s.sx = lw;
    s.g = any ? (base + lw) - fast_log2(t.be) : -INFINITY;
    s.idx = any ? t.bi : 0x7FFFFFFF;
    return s;
}

__device__ __forceinline__ TokState merge_token(TokState a, TokState b) {
    const float mn = fmaxf(a.m, b.m);
    const float l = (mn == -INFINITY) ? 0.f
                                      : a.l * fast_exp2(a.m - mn) + b.l * fast_exp2(b.m - mn);
    const bool take_b = (b.g > a.g) || (b.g == a.g && b.idx < a.idx);
    // the kept candidate's sx moves to the merged base (a state with no entry has none)
    const float sa = (a.m == -INFINITY) ? -INFINITY : a.sx + (a.m - mn);
    const float sb = (b.m == -INFINITY) ? -INFINITY : b.sx + (b.m - mn);
    a.sx = take_b ? sb : sa;
    if (take_b) {
        a.g = b.g;
        a.idx = b.idx;
    }
    a.m = mn;
    a.l = l;
    return a;
}

__device__ __forceinline__ TokState shfl_xor_tok(TokState s, int mask) {
    TokState r;
    r.m = __shfl_xor(s.m, mask);
    r.l = __shfl_xor(s.l, mask);
    r.g = __shfl_xor(s.g, mask);
    r.sx = __shfl_xor(s.sx, mask);
    r.idx = __shfl_xor(s.idx, mask);
    return r;
}

// Two-level sampler, block uniforms: block beta = 16 a + 4 b + c (b, c in 0..3) takes word b
// of the Philox block at counter (4 a + c, position, request key, stream).  Four blocks 16
// apart share one Philox block, so a lane that visits blocks beta, beta + 16, ... of one
// lane-group position needs one Philox call per four of them.
__device__ __forceinline__ uint32_t race_counter(uint32_t beta) {
    return ((beta >> 4) << 2) | (beta & 3u);
}

__device__ __forceinline__ uint32_t pick_word(const Philox4 &ph, uint32_t i) {
    return i == 0 ? ph.w[0] : (i == 1 ? ph.w[1] : (i == 2 ? ph.w[2] : ph.w[3]));
}

__device__ __forceinline__ uint32_t race_word(uint32_t beta, uint32_t pos, uint32_t req,
                                              uint32_t stream, uint32_t k0, uint32_t k1) {
    const Philox4 ph = philox4x32_10(race_counter(beta), pos, req, stream, k0, k1);
    return pick_word(ph, (beta >> 2) & 3u);
}

// Word of token v for the within-block draw (and every per-token draw): word v & 3 of the
// Philox block at counter (v >> 2, position, request key, stream).
__device__ __forceinline__ uint32_t token_word(uint32_t v, uint32_t pos, uint32_t req,
                                               uint32_t stream, uint32_t k0, uint32_t k1) {
    const Philox4 ph = philox4x32_10(v >> 2, pos, req, stream, k0, k1);
    return pick_word(ph, v & 3u);
}

// ---------------------------------------------------------------------------------------
// Online softmax statistics + block-race / argmax candidate, in log2 units.
//   sampled: s2 = c * log2(e) / T; m = max s2; l = sum exp2(s2 - m);
//            g = best race score A2 - log2(E) of a 16-token block (A2 = log2 of the block's
//            total weight), idx = first token of that block.
//   greedy:  m = max c, idx = its index (l, g unused).
// Elements are visited in increasing index inside a lane (strict > keeps the lowest index);
// merges across lanes / blocks break exact ties towards the lower index explicitly.
// ---------------------------------------------------------------------------------------

struct SampleState {
    float m, l, g;
    int idx;
};

__device__ __forceinline__ SampleState sample_state_init() {
    SampleState s;
    s.m = -INFINITY;
    s.l = 0.f;
    s.g = -INFINITY;
    s.idx = 0x7FFFFFFF;
    return s;
}

__device__ __forceinline__ void greedy_update(SampleState &st, float c, int v) {
    const bool take = c > st.m;
    st.m = take ? c : st.m;
    st.idx = take ? v : st.idx;
}

// Softmax statistics of four consecutive scores (already in log2 units; -inf = masked),
// branch-free: an all -inf history and group leave l = 0.
// Running max / sum of exp2(c * inv) over four logits c (-inf: no entry).  The base is the
// largest c scaled once (rounding is monotonic and inv > 0), and every weight is
// exp2(c * inv - base) with one fused multiply-add, so no scaled logit is rounded before the
// base is taken off.
__device__ __forceinline__ void lse_update4(SampleState &st, const float c[4], float inv) {
    const float m4 = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3])) * inv;
    const float mn = fmaxf(st.m, m4);
    const float base = (mn == -INFINITY) ? 0.f : mn;
    st.l = st.l * fast_exp2(st.m - base) + fast_exp2(fmaf(c[0], inv, -base)) +
           fast_exp2(fmaf(c[1], inv, -base)) + fast_exp2(fmaf(c[2], inv, -base)) +
           fast_exp2(fmaf(c[3], inv, -base));
    st.m = mn;
}

// One block of the race: `ref` + log2(sum) is the block's log2 weight (sum = 0: weight 0,
// never drawn), `word` its race uniform, v0 its first token.
__device__ __forceinline__ void race_update(float &g, int &idx, float ref, float sum,
                                            uint32_t word, int v0) {
    // log2(0) = -inf: a block of weight 0 scores -inf and is never taken (branch-free)
    const float sc = ref + fast_log2(sum) + gumbel2_from_word(word);
    const bool take = sc > g;
    g = take ? sc : g;
    idx = take ? v0 : idx;
}

__device__ __forceinline__ SampleState merge_stochastic(SampleState a, SampleState b) {
    const float mn = fmaxf(a.m, b.m);
    const float l = (mn == -INFINITY) ? 0.f
                                      : a.l * fast_exp2(a.m - mn) + b.l * fast_exp2(b.m - mn);
    const bool take_b = (b.g > a.g) || (b.g == a.g && b.idx < a.idx);
    if (take_b) {
        a.g = b.g;
        a.idx = b.idx;
    }
    a.m = mn;
    a.l = l;
    return a;
}

__device__ __forceinline__ SampleState merge_greedy(SampleState a, SampleState b) {
    const bool take_b = (b.m > a.m) || (b.m == a.m && b.idx < a.idx);
    if (take_b) {
        a.m = b.m;
        a.idx = b.idx;
    }
    return a;
}

// Merge with the rule of the row's mode (if/else, not ?:, so the states stay in registers).
__device__ __forceinline__ void merge_into(SampleState &st, SampleState o, bool greedy) {
    if (greedy)
        st = merge_greedy(st, o);
    else
        st = merge_stochastic(st, o);
}

__device__ __forceinline__ SampleState shfl_xor_state(SampleState s, int mask) {
    SampleState r;
    r.m = __shfl_xor(s.m, mask);
    r.l = __shfl_xor(s.l, mask);
    r.g = __shfl_xor(s.g, mask);
    r.idx = __shfl_xor(s.idx, mask);
    return r;
}

// Partial record written per (request row, V-slab): 16 bytes.  Draft rows: the sample state.
// Residual rows: m = best p-race score, l = its block (int bits), g = best r-race score,
// idx = its block.
struct __align__(16) Partial {
    float m, l, g;
    int idx;
};

__device__ __forceinline__ Partial to_partial(const SampleState &s) {
    Partial p;
    p.m = s.m;
    p.l = s.l;
    p.g = s.g;
    p.idx = s.idx;
    return p;
}

__device__ __forceinline__ SampleState from_partial(const Partial &p) {
    SampleState s;
    s.m = p.m;
    s.l = p.l;
    s.g = p.g;
    s.idx = p.idx;
    return s;
}

// Partial record of a drafting row per V-slab: 32 bytes.  Per-token sampler: the TokState
// (p = {m, l, g, idx}, sx the winner's scaled logit); two-level sampler and greedy rows: the
// SampleState in p (sx unused).
struct __align__(16) DraftPartial {
    Partial p;
    float sx, pad0, pad1, pad2;
};

__device__ __forceinline__ DraftPartial to_draft_partial(const TokState &t) {
    DraftPartial d;
    d.p.m = t.m;
    d.p.l = t.l;
    d.p.g = t.g;
    d.p.idx = t.idx;
    d.sx = t.sx;
    d.pad0 = d.pad1 = d.pad2 = 0.f;
    return d;
}

__device__ __forceinline__ DraftPartial to_draft_partial(const SampleState &s) {
    DraftPartial d;
    d.p = to_partial(s);
    d.sx = 0.f;
    d.pad0 = d.pad1 = d.pad2 = 0.f;
    return d;
}

__device__ __forceinline__ TokState tok_from_partial(const DraftPartial &d) {
    TokState t;
    t.m = d.p.m;
    t.l = d.p.l;
    t.g = d.p.g;
    t.idx = d.p.idx;
    t.sx = d.sx;
    return t;
}

// ---------------------------------------------------------------------------------------
// Logit loads
// ---------------------------------------------------------------------------------------

// 16 consecutive logits of one row (v0 % 16 == 0) held by one lane, in storage format.
template <typename T>
struct Raw16;
template <>
struct Raw16<uint16_t> {
    uint4 q[2];
    __device__ __forceinline__ void load(const void *base, size_t row, int V, int v0) {
        // every lane issues both loads (a fixed count per wave); chunks past V re-read the
        // row's last chunk and are masked by the caller
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + row * (size_t)V;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int v = min(v0 + 8 * h, V - 8);
            q[h] = *reinterpret_cast<const uint4 *>(p + v);
        }
    }
    // entries 8h .. 8h + 7 only (one 16-byte load)
    __device__ __forceinline__ void load_half(const void *base, size_t row, int V, int v0, int h) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + row * (size_t)V;
        q[h] = *reinterpret_cast<const uint4 *>(p + min(v0 + 8 * h, V - 8));
    }
    // the same when entries v0 + 8h .. + 7 are known to lie inside the row
    __device__ __forceinline__ void load_half_nc(const void *base, size_t row, int V, int v0, int h) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(base) + row * (size_t)V;
        q[h] = *reinterpret_cast<const uint4 *>(p + v0 + 8 * h);
    }
    __device__ __forceinline__ void zero() {
        q[0] = make_uint4(0u, 0u, 0u, 0u);
        q[1] = q[0];
    }
    __device__ __forceinline__ float get(int e) const {  // e is a compile-time constant
        const uint4 &u = q[e >> 3];
        const uint32_t w = ((e >> 1) & 3) == 0 ? u.x : ((e >> 1) & 3) == 1 ? u.y : ((e >> 1) & 3) == 2 ? u.z : u.w;
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};
template <>
struct Raw16<float> {
    float4 q[4];
    __device__ __forceinline__ void load(const void *base, size_t row, int V, int v0) {
        const float *p = reinterpret_cast<const float *>(base) + row * (size_t)V;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int v = min(v0 + 4 * h, V - 4);
            q[h] = *reinterpret_cast<const float4 *>(p + v);
        }
    }
    // entries 8h .. 8h + 7 only (two 16-byte loads)
    __device__ __forceinline__ void load_half(const void *base, size_t row, int V, int v0, int h) {
        const float *p = reinterpret_cast<const float *>(base) + row * (size_t)V;
#pragma unroll
        for (int k = 0; k < 2; ++k) q[2 * h + k] = *reinterpret_cast<const float4 *>(p + min(v0 + 8 * h + 4 * k, V - 4));
    }
    __device__ __forceinline__ void load_half_nc(const void *base, size_t row, int V, int v0, int h) {
        const float *p = reinterpret_cast<const float *>(base) + row * (size_t)V;
#pragma unroll
        for (int k = 0; k < 2; ++k) q[2 * h + k] = *reinterpret_cast<const float4 *>(p + v0 + 8 * h + 4 * k);
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int h = 0; h < 4; ++h) q[h] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ __forceinline__ float get(int e) const {
        const float4 &u = q[e >> 2];
        return (e & 3) == 0 ? u.x : (e & 3) == 1 ? u.y : (e & 3) == 2 ? u.z : u.w;
    }
};

// ---------------------------------------------------------------------------------------
// Within-block step of the two-level sampler (one wave, all 64 lanes must call)
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float load_value(const void *base, int dtype, size_t idx) {
    return dtype == DSPARK_BF16 ? bf16_to_f32(reinterpret_cast<const uint16_t *>(base)[idx])
                                : reinterpret_cast<const float *>(base)[idx];
}

// Corrected logit c_v = Z[zrow][v] + sum_i U[prev][i] W[v][i] of token v = v0 + (lane & 15),
// accumulated in float; quarter h = lane >> 4 of the wave takes one quarter of the rank.  When
// the quarter is a whole number of 16-byte chunks its loads are issued together as vectors.
// Lanes whose token is past V read token V - 1; the caller masks them.
template <typename FT, int N>
__device__ __forceinline__ float dot_chunks(const FT *u, const FT *w, int n_chunks) {
    // eight chunks per round: a rank-256 bfloat16 quarter is one round of loads
    constexpr int kRound = 8;
    float acc = 0.f;
    for (int c = 0; c < n_chunks; c += kRound) {
        uint4 ru[kRound], rw[kRound];
#pragma unroll
        for (int j = 0; j < kRound; ++j) {
            const int cc = c + j < n_chunks ? c + j : n_chunks - 1;
            ru[j] = *reinterpret_cast<const uint4 *>(u + cc * N);
            rw[j] = *reinterpret_cast<const uint4 *>(w + cc * N);
        }
#pragma unroll
        for (int j = 0; j < kRound; ++j) {
            if (c + j >= n_chunks) break;
            const uint32_t *a = reinterpret_cast<const uint32_t *>(&ru[j]);
            const uint32_t *b = reinterpret_cast<const uint32_t *>(&rw[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (N == 8) {  // bf16 pairs
                    acc = fmaf(bf16_lo(a[q]), bf16_lo(b[q]), acc);
                    acc = fmaf(bf16_hi(a[q]), bf16_hi(b[q]), acc);
                } else {
                    acc = fmaf(__uint_as_float(a[q]), __uint_as_float(b[q]), acc);
                }
            }
        }
    }
    return acc;
}

__device__ __forceinline__ float wave_corrected16(const void *Z, int z_dtype, size_t zrow,
                                                  const void *U, const void *W, int uw_dtype,
                                                  int r, int V, int prev, int v0) {
    const int lane = threadIdx.x & 63, h = lane >> 4;
    const int v = min(v0 + (lane & 15), V - 1);
    const float z = load_value(Z, z_dtype, zrow * (size_t)V + v);
    float acc = 0.f;
    const int per = uw_dtype == DSPARK_BF16 ? 8 : 4;  // elements per 16-byte chunk
    const bool aligned = ((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(W)) & 15u) == 0;
    if (aligned && r % (4 * per) == 0) {
        const int q = r / 4, n_chunks = q / per;
        if (uw_dtype == DSPARK_BF16)
            acc = dot_chunks<uint16_t, 8>(reinterpret_cast<const uint16_t *>(U) + (size_t)prev * r + h * q,
                                          reinterpret_cast<const uint16_t *>(W) + (size_t)v * r + h * q,
                                          n_chunks);
        else
            acc = dot_chunks<float, 4>(reinterpret_cast<const float *>(U) + (size_t)prev * r + h * q,
                                       reinterpret_cast<const float *>(W) + (size_t)v * r + h * q,
                                       n_chunks);
    } else {
        for (int i = h; i < r; i += 4)
            acc = fmaf(load_value(U, uw_dtype, (size_t)prev * r + i),
                       load_value(W, uw_dtype, (size_t)v * r + i), acc);
    }
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    return z + acc;
}

// Best (score, token) over the 16 lanes of each quarter of the wave, ties to the lower
// token; `aux` travels with the winner.
__device__ __forceinline__ void wave_argmax16(float &score, int &token, float &aux) {
#pragma unroll
    for (int mask = 1; mask < 16; mask <<= 1) {
        const float os = __shfl_xor(score, mask), oa = __shfl_xor(aux, mask);
        const int ot = __shfl_xor(token, mask);
        const bool take = os > score || (os == score && ot < token);
        if (take) {
            score = os;
            token = ot;
            aux = oa;
        }
    }
}

// Temperature handling shared by every kernel: negative / NaN -> greedy and flagged.
__device__ __forceinline__ float checked_temperature(float t, uint32_t *status) {
    if (!(t >= 0.f)) {  // NaN or negative
        atomicOr(status, DSPARK_DEV_BAD_TEMPERATURE);
        return 0.f;
    }
    return t;
}

__device__ __forceinline__ int checked_token(int t, int V, uint32_t *status) {
    if (t < 0 || t >= V) {
        atomicOr(status, DSPARK_DEV_BAD_TOKEN);
        return 0;
    }
    return t;
}

// ---------------------------------------------------------------------------------------
// Launch geometry shared by host and device code
// ---------------------------------------------------------------------------------------

constexpr int kMaxK = 64;            // draft positions per request
constexpr int kTileV = 64;           // vocabulary rows per W tile (4 MFMA row blocks)
constexpr int kMfmaWaves = 8;        // waves per matrix-core workgroup
constexpr int kRowsPerWave = 32;     // requests per wave (two 16-wide MFMA column blocks)
constexpr int kRowsPerGroup = kMfmaWaves * kRowsPerWave;  // 256 requests per workgroup
constexpr int kTargetSlabs = 256;    // aim for this many workgroups per launch (one per CU)

// Number of V-slabs (workgroups along the vocabulary) a launch over n_rows rows uses; a
// multiple of 8 so that the slab -> XCD mapping is a bijection.
inline int num_vslabs(int V, int n_rows) {
    const int n_tiles = (int)(((long long)V + kTileV - 1) / kTileV);
    const int groups = (int)(((long long)n_rows + kRowsPerGroup - 1) / kRowsPerGroup);
    int s = kTargetSlabs / (groups > 0 ? groups : 1);
    if (s > n_tiles) s = n_tiles;
    s = (s + 7) / 8 * 8;
    return s < 8 ? 8 : s;
}

// ---------------------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned)
// ---------------------------------------------------------------------------------------

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct DraftWs {
    uint32_t *status;    // [1] device status bits
    int32_t *prev_cur;   // [B] previous token of the current step
    uint16_t *a_rows;    // [B][r] bf16: left operand of the current position (matrix-core path)
    float *h_state;      // [2][B][r] recurrent head: state of the last two positions
    DraftPartial *partials;  // [B][n_slabs]
    int n_slabs;
};

// Verification spreads a chunk's target rows evenly over the workgroups of a launch: every
// row is cut into the same runs of at most kRowSweep blocks, and each workgroup takes a
// contiguous range of the chunk's runs, so a chunk keeps every CU streaming to its end
// whatever the number of requests still being verified.
constexpr int kRowThreads = 256;
constexpr int kRowBlocks = 4;    // sampler blocks per thread and sweep, loads issued together
constexpr int kRowSweep = kRowBlocks * kRowThreads;
constexpr int kRowGrid = 1024;   // workgroups of a row-statistics launch (4 per CU)
constexpr int kMaxChunks = 8;    // chunks of target rows (K + 1 <= 65 rows)
// A target row is cut into runs of 16-token blocks at fixed places (ceil(blocks / kRowSweep)
// runs of equal length but the last), and each wave of the workgroup that takes a run leaves
// one partial: slot run * (kRowThreads / 64) + wave.  A row's statistics then merge the same
// partials in the same order whichever workgroups computed them.
constexpr int kRowWaves = kRowThreads / 64;
inline int num_row_runs(int V) {
    const int n_blk = (V + kSampleBlock - 1) / kSampleBlock;
    return (n_blk + kRowSweep - 1) / kRowSweep;
}
inline int num_row_slabs(int V, int B) {
    (void)B;
    return num_row_runs(V) * kRowWaves;
}

struct VerifyWs {
    uint32_t *status;      // [1]
    int32_t *n_resid;      // [1] nonzero when some request needs a residual draw
    int32_t *n_alive;      // [kMaxChunks] requests listed for each chunk
    int4 *alive;           // [kMaxChunks][B] records {b, L, T bits, req} of the listed requests
    int32_t *first_reject; // [B] first rejected position (K + 1: none so far)
    int32_t *resid_rows;   // [B] packed (b * 128 + j) of request b's residual row, or -1
    float4 *rowstats;      // [B][K+1] {m2, l, idx-as-bits, g}
    Partial *row_partials; // [B][K+1][n_row_slabs]
    Partial *partials;     // [B][n_slabs] residual candidates
    int n_slabs, n_row_slabs;
};

// ---------------------------------------------------------------------------------------
// Host-side launchers (one per kernel family), implemented next to their kernels.
// Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------------------

struct DraftStepParams {
    int B, K, V, r, k;             // k: the draft position of this step
    const void *Z;                 // [B][K][V]
    const void *U, *W;             // [V][r]
    const int32_t *draft_len;      // [B] or null
    const float *temperature;      // [B]
    const uint32_t *req_id;        // [B] or null
    uint32_t key0, key1;
    const int32_t *prev_cur;       // [B]
    const uint16_t *a_rows;        // [B][r] gathered U rows (matrix-core path)
    DraftPartial *partials;        // [B][n_slabs]
    float *corrected;              // [B][K][V] or null
    uint32_t *status;
    int n_slabs;
    int sampler;                   // dspark_sampler
};

// Whether the drafting steps run on the matrix cores, which take each request's U row from a
// gathered copy that the prepare and reduce kernels keep up to date.
bool draft_gathers_rows(const dspark_draft_args &a);
// Recurrent head: the GRU update of position k for every live request (k = 0 starts from a
// zero state), writing the float32 state, the bfloat16 operand and, when asked, head_state.
hipError_t launch_rnn_step(const dspark_draft_args &a, const DraftWs &ws, int k, hipStream_t s);
hipError_t launch_draft_prepare(const dspark_draft_args &a, const DraftWs &ws, hipStream_t s);
hipError_t launch_draft_step(const DraftStepParams &p, int z_dtype, int uw_dtype, hipStream_t s);
hipError_t launch_draft_reduce(const dspark_draft_args &a, const DraftWs &ws, int k,
                               hipStream_t s);
bool draft_uses_rnn(const dspark_draft_args &a);
// bfloat16 factors of a rank the matrix-core kernels take (64, 128 or 256)
bool matrix_core_factors(int uw_dtype, int r);

// r x V right factor (row-major) -> [V][r]
hipError_t launch_pack_w(const void *w_rv, void *w_vr, int r, int V, int dtype, hipStream_t s);

hipError_t launch_schedule(const dspark_schedule_args &a, uint32_t *status, long long *key,
                           int *rank, hipStream_t s);
hipError_t launch_calibrate(const dspark_calibrate_args &a, uint32_t *status, hipStream_t s);

// Target rows are verified in chunks (one launch each, and a decide launch after every chunk
// but the last); verify_chunks fills the chunk edges of a call and returns their count.
int verify_chunks(const dspark_verify_args &a, int bounds[kMaxChunks + 1]);
hipError_t launch_verify_rows(const dspark_verify_args &a, const VerifyWs &ws, int chunk,
                              hipStream_t s);
hipError_t launch_verify_decide(const dspark_verify_args &a, const VerifyWs &ws, int chunk,
                                hipStream_t s);
hipError_t launch_verify_finish(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s);
hipError_t launch_verify_residual(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s);
hipError_t launch_verify_residual_reduce(const dspark_verify_args &a, const VerifyWs &ws,
                                         hipStream_t s);

}  // namespace dspark
