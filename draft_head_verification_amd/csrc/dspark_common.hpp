// dspark_common.hpp -- device helpers and internal launch interfaces of libdspark.so.
//
// Everything here is written for gfx950 (CDNA4, wave64).  The random-number definition, the
// sampling rule and the tie-break rule are those stated in include/dspark.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr uint32_t kStreamDraft = 0, kStreamAccept = 1, kStreamResidual = 2, kStreamBonus = 3;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------
// element conversion
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  Each round multiplies counter words 0
// and 2 by the published multipliers (one v_mad_u64_u32 each), xors the high halves into the
// other two words together with the round key, and the key advances by the Weyl constants.
// ---------------------------------------------------------------------------------------

struct Philox4 {
    uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t pa = (uint64_t)0xD2511F53u * (uint64_t)c0;
        const uint64_t pb = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        const uint32_t n0 = (uint32_t)(pb >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
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
// rounds to the 2^-24 grid (the accept test tolerates it; the sampler uses exp_from_word).
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

// ---------------------------------------------------------------------------------------
// Online softmax statistics + Gumbel-max / argmax candidate, in log2 units.
//   stochastic: s2 = c * log2(e) / T; m = max s2; l = sum exp2(s2 - m);
//               g = best s2 - log2(E) (the Gumbel-perturbed score scaled by log2 e, minus a
//               constant), sb = s2 at the best, idx = its index.
//   greedy:     m = max c, idx = its index (l, g, sb unused).
// Elements are visited in increasing index inside a lane (strict > keeps the lowest index);
// merges across lanes / blocks break exact ties towards the lower index explicitly.
// ---------------------------------------------------------------------------------------

struct SampleState {
    float m, l, g, sb;
    int idx;
};

__device__ __forceinline__ SampleState sample_state_init() {
    SampleState s;
    s.m = -INFINITY;
    s.l = 0.f;
    s.g = -INFINITY;
    s.sb = -INFINITY;
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
__device__ __forceinline__ void lse_update4(SampleState &st, const float s[4]) {
    const float m4 = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    const float mn = fmaxf(st.m, m4);
    const float base = (mn == -INFINITY) ? 0.f : mn;
    st.l = st.l * fast_exp2(st.m - base) + fast_exp2(s[0] - base) + fast_exp2(s[1] - base) +
           fast_exp2(s[2] - base) + fast_exp2(s[3] - base);
    st.m = mn;
}

// Order-preserving map of a float to an unsigned key (key 0 is reserved for "no bound"), so
// that the best score found by any workgroup can be shared with one unsigned atomic max.
__device__ __forceinline__ uint32_t ordered_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
    if (k == 0u) return -INFINITY;
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Current shared bound (read around the L1, which may hold a stale line; a stale value is
// still a valid, only weaker, bound).
__device__ __forceinline__ float load_bound(const uint32_t *b) {
    return key_to_float(__hip_atomic_load(b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Exact pruning of Gumbel-max work.  An element with noise-free score a (log2 units) beats
// the running best g only if a - log2(E) > g, i.e. E < 2^(a - g); since E = -ln u >= 1 - u,
// that needs 1 - u < 2^(a - g).  With k = 2^24 - 1 - (word >> 8), 1 - u = (k + 0.5) 2^-24, so
// only words w >= candidate_threshold(max a, g) can win.  The 0.1% margin covers the rounding
// of exp2, so every element skipped here would have lost by more than 1e-3 in log2 units: the
// selected index is identical to evaluating every element.
__device__ __forceinline__ uint32_t candidate_threshold(float amax, float g) {
    const float y = fast_exp2(amax - g) * (1.001f * 16777216.0f);
    if (!(y < 16777215.0f)) return 0u;  // also NaN / inf: everything is a candidate
    return (0xFFFFFFu - (uint32_t)y) << 8;
}

// Per-entry form of the same test.  With a = log2 of the entry's weight and g the best
// perturbed score, the entry can win only if E < exp2(a - g); E >= 1 - u = (d + 1/2) 2^-24
// with d = 2^24 - 1 - (word >> 8), so d <= x * scale is necessary, where x = exp2(a - ref)
// is already at hand and scale = exp2(ref - g + 24) (with the same 0.1% margin).  A weak
// bound (ref - g >= 100, or no bound at all) makes every entry a candidate.
struct PruneScale {
    float scale;
    bool all;
};

__device__ __forceinline__ PruneScale prune_scale(float ref_minus_g) {
    PruneScale ps;
    ps.all = !(ref_minus_g < 100.f);
    ps.scale = fast_exp2(fminf(ref_minus_g, 100.f) + 24.f) * 1.001f;
    return ps;
}

__device__ __forceinline__ bool may_win(const PruneScale &ps, float x, uint32_t word) {
    return ps.all || (float)(0xFFFFFFu - (word >> 8)) <= x * ps.scale;
}

__device__ __forceinline__ void gumbel_update(SampleState &st, float s2, uint32_t word, int v) {
    const float g = s2 - fast_log2(exp_from_word(word));
    const bool take = g > st.g;
    st.g = take ? g : st.g;
    st.sb = take ? s2 : st.sb;
    st.idx = take ? v : st.idx;
}

// Gumbel-max over four consecutive scores with their Philox words, pruned as above against
// the larger of the running best and `lb`, a perturbed score some element of the same row
// has reached (shared between workgroups): an element below it cannot be the row's winner.
__device__ __forceinline__ void gumbel_update4(SampleState &st, const float s[4], const uint32_t w[4],
                                               int v, float lb = -INFINITY) {
    const float amax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    const uint32_t t = candidate_threshold(amax, fmaxf(st.g, lb));
    if ((w[0] >= t) | (w[1] >= t) | (w[2] >= t) | (w[3] >= t)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (w[i] >= t) gumbel_update(st, s[i], w[i], v + i);
    }
}

__device__ __forceinline__ SampleState merge_stochastic(SampleState a, SampleState b) {
    const float mn = fmaxf(a.m, b.m);
    const float l = (mn == -INFINITY) ? 0.f
                                      : a.l * fast_exp2(a.m - mn) + b.l * fast_exp2(b.m - mn);
    const bool take_b = (b.g > a.g) || (b.g == a.g && b.idx < a.idx);
    if (take_b) {
        a.g = b.g;
        a.sb = b.sb;
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
    r.sb = __shfl_xor(s.sb, mask);
    r.idx = __shfl_xor(s.idx, mask);
    return r;
}

// Partial record written per (request row, V-slab): 6 words, 8-byte aligned.
struct __align__(8) Partial {
    float m, l, g, sb;
    int idx;
    int pad;
};

__device__ __forceinline__ Partial to_partial(const SampleState &s) {
    Partial p;
    p.m = s.m;
    p.l = s.l;
    p.g = s.g;
    p.sb = s.sb;
    p.idx = s.idx;
    p.pad = 0;
    return p;
}

__device__ __forceinline__ SampleState from_partial(const Partial &p) {
    SampleState s;
    s.m = p.m;
    s.l = p.l;
    s.g = p.g;
    s.sb = p.sb;
    s.idx = p.idx;
    return s;
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

constexpr int kTileV = 64;           // vocabulary rows per W tile (4 MFMA row blocks)
constexpr int kMfmaWaves = 8;        // waves per matrix-core workgroup
constexpr int kRowsPerWave = 32;     // requests per wave (two 16-wide MFMA column blocks)
constexpr int kRowsPerGroup = kMfmaWaves * kRowsPerWave;  // 256 requests per workgroup
constexpr int kTargetSlabs = 256;    // aim for this many workgroups per launch (one per CU)

// Number of V-slabs (workgroups along the vocabulary) a launch over n_rows rows uses; a
// multiple of 8 so that the slab -> XCD mapping is a bijection.
inline int num_vslabs(int V, int n_rows) {
    const int n_tiles = (V + kTileV - 1) / kTileV;
    const int groups = (n_rows + kRowsPerGroup - 1) / kRowsPerGroup;
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
    Partial *partials;   // [B][n_slabs]
    uint32_t *bound;     // [K][B] shared pruning bounds (ordered keys, 0 = none)
    int n_slabs;
};

struct VerifyWs {
    uint32_t *status;     // [1]
    int32_t *n_resid;     // [1] number of rows needing a residual draw
    int32_t *resid_rows;  // [B] packed (b * 128 + j)
    float4 *rowstats;     // [B][K+1] {m2, l, idx-as-bits, unused}
    Partial *partials;    // [B][n_slabs] residual candidates
    uint32_t *bound;      // [B][2] shared pruning bounds of the residual / fallback draws
    int n_slabs;
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
    Partial *partials;             // [B][n_slabs]
    float *corrected;              // [B][K][V] or null
    uint32_t *bound;               // [B] shared pruning bounds of this step
    uint32_t *status;
    int n_slabs;
};

hipError_t launch_draft_prepare(const dspark_draft_args &a, const DraftWs &ws, hipStream_t s);
hipError_t launch_draft_step(const DraftStepParams &p, int z_dtype, int uw_dtype, hipStream_t s);
hipError_t launch_draft_reduce(const dspark_draft_args &a, const DraftWs &ws, int k,
                               hipStream_t s);

hipError_t launch_schedule(const dspark_schedule_args &a, uint32_t *status, hipStream_t s);

hipError_t launch_verify_prepare(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s);
hipError_t launch_verify_rowstats(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s);
hipError_t launch_verify_finish(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s);
hipError_t launch_verify_residual(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s);
hipError_t launch_verify_residual_reduce(const dspark_verify_args &a, const VerifyWs &ws,
                                         hipStream_t s);

}  // namespace dspark
