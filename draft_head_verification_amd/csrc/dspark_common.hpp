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
    if (c > st.m) {
        st.m = c;
        st.idx = v;
    }
}

// Softmax statistics of four consecutive scores (already in log2 units; -inf = masked).
__device__ __forceinline__ void lse_update4(SampleState &st, const float s[4]) {
    const float m4 = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (m4 == -INFINITY) return;
    const float mn = fmaxf(st.m, m4);
    const float scale = fast_exp2(st.m - mn);  // st.m = -inf gives 0
    st.l = st.l * scale + fast_exp2(s[0] - mn) + fast_exp2(s[1] - mn) + fast_exp2(s[2] - mn) +
           fast_exp2(s[3] - mn);
    st.m = mn;
}

__device__ __forceinline__ void gumbel_update(SampleState &st, float s2, uint32_t word, int v) {
    const float g = s2 - fast_log2(exp_from_word(word));
    if (g > st.g) {
        st.g = g;
        st.sb = s2;
        st.idx = v;
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
constexpr int kTargetSlabs = 1024;   // aim for this many workgroups per launch

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
    int n_slabs;
};

struct VerifyWs {
    uint32_t *status;     // [1]
    int32_t *n_resid;     // [1] number of rows needing a residual draw
    int32_t *resid_rows;  // [B] packed (b * 128 + j)
    float4 *rowstats;     // [B][K+1] {m2, l, idx-as-bits, unused}
    Partial *partials;    // [B][n_slabs] residual candidates
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
