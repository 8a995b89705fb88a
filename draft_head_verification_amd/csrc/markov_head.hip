// markov_head.hip -- the Markov sequential head and its fused sampling epilogue.
//
// One draft step k computes, for every request b, the corrected row
//     c[b][v] = Z[b][k][v] + sum_i U[prev_b][i] * W[v][i]
// and folds it straight into softmax statistics and a Gumbel-max (or argmax) candidate,
// without ever writing c (unless the caller asks for it).  The head looks at the previous
// token only and is a low-rank (rank r) factorisation of a token-to-token bias (QbitAI "DSpark
// in 10 concepts", section "Cheaper serial module: the Markov head"; 10100.com commentary,
// section on parallel drafts and the rank-256 transition correction).  Steps run left to right
// because position k needs the token sampled at k-1 (QbitAI, section "DSpark = Eagle + DFlash").
//
// Sampled rows use the per-token Gumbel-max draw by default: every token of the row gets its
// own Philox uniform, and each lane keeps its best token (as weight / E, against the running
// softmax base) together with the softmax statistics; the reduction kernels merge the slabs'
// candidates and take the winner, whose scaled logit travels with it.  The optional two-level
// sampler races 16-token blocks weighted by their total softmax weight (one uniform per block)
// in the head kernels; its reduction kernels recompute the 16 corrected logits of the winning
// block and draw the token inside it.
//
// Matrix-core path (bf16 factors, r = 64, 128 or 256):
//   GEMM view: rows = vocabulary (M), columns = requests (N), reduction = r (K).
//   A workgroup owns up to 256 requests and a contiguous slab of the vocabulary: 16 waves of
//   16 requests at ranks 128 and 256 (8 waves of 32, two 16-wide column blocks, at rank 64
//   and in the two-level sampler's residual pass).  Each wave keeps its requests' gathered U
//   rows in registers as MFMA B fragments for the whole slab.  The slab streams through LDS
//   in tiles of 64 vocabulary rows of W (direct global->LDS loads, four stages, one barrier
//   per tile); every wave reads its A fragments from the shared tile, so W leaves HBM once
//   per 256 requests.  The fragment layout leaves each lane 16 consecutive vocabulary entries
//   of a request per tile: one Philox call per four of them, and for the two-level sampler
//   exactly one block, whose sums then need no data exchange.
//   Workgroups are laid out so that the request groups sharing a vocabulary slab are
//   dispatched to the same XCD and meet the slab's W tiles in that XCD's L2.
// Vector-ALU path (any other factor dtype / rank): one workgroup per (request, slab); four
// neighbouring lanes hold one sampler block.
#include <algorithm>
#include <type_traits>

#include "dspark_common.hpp"

namespace dspark {

enum class HeadMode { Draft, Residual };

// Everything a Markov-head kernel needs; the residual mode (the verifier's recompute of the
// draft distribution at the first rejected position) reuses the same GEMM.
struct HeadParams {
    int B, K, V, r;
    int n_rows_max;                 // grid is sized for this many GEMM rows
    const int32_t *n_rows_dev;      // residual mode: nonzero when any row needs the pass
    int k;                          // draft mode: the position of this step
    const void *Z;                  // [B][K][V]
    const uint16_t *U, *W;          // [V][r] bf16 (matrix-core path)
    const float *Uf, *Wf;           // [V][r] f32 (vector path)
    const int32_t *draft_len;       // [B] or null
    const float *temperature;       // [B]
    const uint32_t *req_id;         // [B] or null
    uint32_t key0, key1;
    const int32_t *prev_cur;        // draft: [B]
    const uint16_t *A;              // draft, matrix-core path: [B][r] left operands
    const uint16_t *S;              // residual: [B][K][r] recurrent-head operands, or null
    const int32_t *resid_rows;      // residual: packed rows
    const int32_t *prev_token;      // residual: [B]
    const int32_t *draft_tokens;    // residual: [B][K]
    const void *Y;                  // residual: [B][K+1][V]
    const float4 *rowstats;         // residual: [B][K+1]
    const float *q_lse;             // residual: [B][K]
    int sampler;                    // dspark_sampler
    Partial *partials;              // residual: [rows][n_slabs]
    DraftPartial *dpartials;        // draft: [rows][n_slabs]
    float *corrected;               // draft: optional [B][K][V]
    uint32_t *status;
    int n_slabs;
};

constexpr int kSampToken = DSPARK_SAMPLER_TOKEN, kSampBlock = DSPARK_SAMPLER_BLOCK16;

// Per-row description resolved on the device.
struct RowInfo {
    bool valid;
    int b, pos, prev;
    size_t zrow, yrow;
    float T;
    uint32_t req;
    float qlse2, lse2p;  // residual mode
};

// A drafting row's metadata in two steps, so that its loads can go out before other work and
// be consumed after it.  Absent optional arrays are read at a valid stand-in address and the
// value replaced afterwards, which keeps every load unconditional.
struct DraftRowRaw {
    int kb, prev;
    float T;
    uint32_t req;
};
__device__ __forceinline__ DraftRowRaw draft_row_load(const HeadParams &p, int row) {
    const int b = min(row, p.n_rows_max - 1);
    const int32_t *dl = p.draft_len ? p.draft_len : p.prev_cur;
    const uint32_t *rq = p.req_id ? p.req_id : reinterpret_cast<const uint32_t *>(p.prev_cur);
    DraftRowRaw raw;
    raw.kb = dl[b];
    raw.prev = p.prev_cur[b];  // validated by the prepare / reduce kernels
    raw.T = p.temperature[b];
    raw.req = rq[b];
    return raw;
}
__device__ __forceinline__ RowInfo draft_row_resolve(const HeadParams &p, int row, int n_rows,
                                                     const DraftRowRaw &raw) {
    RowInfo ri;
    const int b = min(row, p.n_rows_max - 1);
    const int kb_raw = p.draft_len ? raw.kb : p.K;
    const int kb = kb_raw < 0 ? 0 : (kb_raw > p.K ? p.K : kb_raw);
    ri.valid = row < n_rows && p.k < kb;
    ri.b = b;
    ri.pos = p.k;
    ri.prev = ri.valid ? raw.prev : 0;
    ri.zrow = ri.valid ? (size_t)b * p.K + p.k : 0;
    ri.yrow = 0;
    ri.T = (ri.valid && raw.T >= 0.f) ? raw.T : 0.f;
    ri.req = p.req_id ? raw.req : (uint32_t)b;
    ri.qlse2 = 0.f;
    ri.lse2p = 0.f;
    return ri;
}

// Branch-free: every load is issued at an in-bounds (clamped) index whether or not the row is
// live, and dead rows are masked with selects afterwards, so that independent loads go out
// together rather than each behind a branch that an earlier load decides.
template <HeadMode MODE>
__device__ __forceinline__ RowInfo row_info(const HeadParams &p, int row, int n_rows) {
    RowInfo ri;
    const bool in = row < n_rows;
    const int rc = min(row, p.n_rows_max - 1);
    ri.qlse2 = 0.f;
    ri.lse2p = 0.f;
    if constexpr (MODE == HeadMode::Draft) {
        return draft_row_resolve(p, row, n_rows, draft_row_load(p, row));
    } else {
        // row b of the batch: its packed (b, j), or -1 when request b needs no residual draw
        // (such rows read request 0's first rows, shared and cached, and are dropped)
        const int raw = p.resid_rows[rc];
        const bool live = in && raw >= 0;
        const int packed = live ? raw : 0;
        const int b = packed >> 7, j = packed & 127;
        ri.valid = live;
        ri.b = b;
        ri.pos = j;
        const int pt = p.prev_token[b];
        const int dt = p.draft_tokens[(size_t)b * p.K + (j > 0 ? j - 1 : 0)];
        ri.zrow = (size_t)b * p.K + j;
        ri.yrow = (size_t)b * (p.K + 1) + j;
        ri.T = p.temperature[b];  // > 0: greedy rows never need a residual
        const float4 rs = p.rowstats[ri.yrow];
        const float ql = p.q_lse[ri.zrow];
        ri.req = p.req_id ? p.req_id[b] : (uint32_t)b;
        int prev = j == 0 ? pt : dt;
        prev = (prev < 0 || prev >= p.V) ? 0 : prev;  // flagged by the verifier's finish kernel
        ri.prev = prev;
        ri.lse2p = rs.x + fast_log2(rs.y);
        ri.qlse2 = ql * kLog2e;
    }
    return ri;
}

// Residual race: best block over the weights r = max(p - q, 0) and, as the fallback when the
// residual is identically zero, best block over p.  Packed into a Partial as
// {g: best r-score, idx: its block, m: best p-score, l: its block (int bits)}.
struct ResidState {
    float gr, gp;
    int ir, ip;
};

__device__ __forceinline__ ResidState resid_init() {
    ResidState s;
    s.gr = -INFINITY;
    s.gp = -INFINITY;
    s.ir = 0x7FFFFFFF;
    s.ip = 0x7FFFFFFF;
    return s;
}

__device__ __forceinline__ ResidState resid_merge(ResidState a, ResidState b) {
    if ((b.gr > a.gr) || (b.gr == a.gr && b.ir < a.ir)) {
        a.gr = b.gr;
        a.ir = b.ir;
    }
    if ((b.gp > a.gp) || (b.gp == a.gp && b.ip < a.ip)) {
        a.gp = b.gp;
        a.ip = b.ip;
    }
    return a;
}

__device__ __forceinline__ ResidState resid_shfl_xor(ResidState s, int mask) {
    ResidState r;
    r.gr = __shfl_xor(s.gr, mask);
    r.gp = __shfl_xor(s.gp, mask);
    r.ir = __shfl_xor(s.ir, mask);
    r.ip = __shfl_xor(s.ip, mask);
    return r;
}

// Four consecutive logits of a row starting at v (v % 4 == 0, v + 3 < V when v < V), kept
// in their storage format until the epilogue needs them.
template <typename T>
struct Raw4;
template <>
struct Raw4<uint16_t> {
    uint2 q;
    __device__ __forceinline__ void load(const void *base, size_t row, int V, int v) {
        q = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(base) +
                                             row * (size_t)V + v);
    }
    __device__ __forceinline__ void zero() { q = make_uint2(0u, 0u); }
    __device__ __forceinline__ void get(float out[4]) const {
        out[0] = bf16_lo(q.x);
        out[1] = bf16_hi(q.x);
        out[2] = bf16_lo(q.y);
        out[3] = bf16_hi(q.y);
    }
};
template <>
struct Raw4<float> {
    float4 q;
    __device__ __forceinline__ void load(const void *base, size_t row, int V, int v) {
        q = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) +
                                              row * (size_t)V + v);
    }
    __device__ __forceinline__ void zero() { q = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void get(float out[4]) const {
        out[0] = q.x;
        out[1] = q.y;
        out[2] = q.z;
        out[3] = q.w;
    }
};

template <typename T>
__device__ __forceinline__ void load4(const void *base, size_t row, int V, int v, float out[4]) {
    Raw4<T> r;
    r.load(base, row, V, v);
    r.get(out);
}

// Epilogue for four consecutive corrected logits c[0..3] = entries v..v+3 of one row, v a
// multiple of 4.  Per-token sampler: the lane draws its four tokens' uniforms (one Philox
// block, counter v / 4) and keeps its best perturbed score with the token's scaled logit.
// Two-level sampler: lanes 4j..4j+3 of the workgroup hold one 16-token sampler block and every
// lane must call this (the block sums are exchanged between them).  `live` is false past the
// slab end (no output, weight 0).
template <HeadMode MODE, int SAMP, typename YT>
__device__ __forceinline__ void head_epilogue4(const HeadParams &p, const RowInfo &ri, int v,
                                               bool live, const float c[4], SampleState &st,
                                               TokState &ts, ResidState &rs) {
    const bool lead = (threadIdx.x & 3) == 0;  // holds the block's first token
    if constexpr (MODE == HeadMode::Draft) {
        if (p.corrected && live) {
            float4 o;
            o.x = c[0];
            o.y = c[1];
            o.z = c[2];
            o.w = c[3];
            *reinterpret_cast<float4 *>(p.corrected + ri.zrow * (size_t)p.V + v) = o;
        }
        if (ri.T == 0.f) {  // uniform: one row per workgroup
#pragma unroll
            for (int i = 0; i < 4; ++i) greedy_update(st, live ? c[i] : -INFINITY, v + i);
            return;
        }
        const float inv = kLog2e / ri.T;
        float cl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cl[i] = live ? c[i] : -INFINITY;
        if constexpr (SAMP == kSampToken) {
            SampleState ls;
            ls.m = ts.m;
            ls.l = ts.l;
            lse_update4(ls, cl, inv);
            ts.m = ls.m;
            ts.l = ls.l;
            const Philox4 ph = philox4x32_10((uint32_t)v >> 2, (uint32_t)ri.pos, ri.req,
                                             kStreamDraft, p.key0, p.key1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sc = fmaf(cl[i], inv, -fast_log2(exp2_from_word(ph.w[i])));
                if (sc > ts.g) {  // increasing tokens inside a lane: ties keep the lower one
                    ts.g = sc;
                    ts.sx = cl[i];  // the logit itself until the row's base is final
                    ts.idx = v + i;
                }
            }
            return;
        }
        lse_update4(st, cl, inv);
        float M = fmaxf(fmaxf(cl[0], cl[1]), fmaxf(cl[2], cl[3])) * inv;
        M = fmaxf(M, __shfl_xor(M, 1));
        M = fmaxf(M, __shfl_xor(M, 2));
        const float ref = (M == -INFINITY) ? 0.f : M;
        float a = fast_exp2(fmaf(cl[0], inv, -ref)) + fast_exp2(fmaf(cl[1], inv, -ref)) +
                  fast_exp2(fmaf(cl[2], inv, -ref)) + fast_exp2(fmaf(cl[3], inv, -ref));
        a += __shfl_xor(a, 1);
        a += __shfl_xor(a, 2);
        if (lead) {
            const uint32_t w = race_word((uint32_t)v >> 4, (uint32_t)ri.pos, ri.req,
                                         kStreamDraft, p.key0, p.key1);
            race_update(st.g, st.idx, ref, a, w, v);
        }
    } else {
        float y[4];
        if (live) {
            load4<YT>(p.Y, ri.yrow, p.V, v, y);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = -INFINITY;
        }
        const float inv = kLog2e / ri.T;
        if constexpr (SAMP == kSampToken) {
            const Philox4 ph = philox4x32_10((uint32_t)v >> 2, (uint32_t)ri.pos, ri.req,
                                             kStreamResidual, p.key0, p.key1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = live ? fast_exp2(fmaf(y[i], inv, -ri.lse2p)) : 0.f;
                const float rv = pv - fast_exp2(fmaf(c[i], inv, -ri.qlse2));
                // log2 of a zero weight is -inf: never taken (a row with no positive residual
                // is drawn from p by the reduction kernel)
                const float sr = (live && rv > 0.f)
                                     ? fast_log2(rv) - fast_log2(exp2_from_word(ph.w[i]))
                                     : -INFINITY;
                if (sr > rs.gr) {
                    rs.gr = sr;
                    rs.ir = v + i;
                }
            }
            return;
        }
        float R = 0.f, P = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float pv = fast_exp2(fmaf(y[i], inv, -ri.lse2p));
            const float rv = pv - fast_exp2(fmaf(c[i], inv, -ri.qlse2));
            R += live ? fmaxf(rv, 0.f) : 0.f;
            P += pv;
        }
        R += __shfl_xor(R, 1);
        R += __shfl_xor(R, 2);
        P += __shfl_xor(P, 1);
        P += __shfl_xor(P, 2);
        if (lead) {
            const uint32_t w = race_word((uint32_t)v >> 4, (uint32_t)ri.pos, ri.req,
                                         kStreamResidual, p.key0, p.key1);
            race_update(rs.gr, rs.ir, 0.f, R, w, v);
            race_update(rs.gp, rs.ip, 0.f, P, w, v);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Matrix-core kernel
//
// Work split: workgroup = 16 / NQ waves of 16 NQ requests = up to 256 GEMM rows; a slab of
// 64-row W tiles.
// MFMA mapping: block j (0..3) of a tile, MFMA row m (= lane & 15) is tile row
//   trow(j, m) = 16 (m >> 2) + 4 j + (m & 3),
// so lane l (g = l >> 4) ends up holding tile rows 16 g .. 16 g + 15 of request (l & 15) across
// the four blocks: 16 contiguous vocabulary entries (four Philox calls of the per-token draw,
// or one block of the two-level sampler with its race uniform: block 4 t + g of tile t) and
// 16-byte base-logit loads.
// W tiles reach LDS through direct global->LDS loads into a 4-stage ring (3 tiles ahead, no
// registers); each 16-byte chunk sits at column (col ^ swz(row)) of its row, which makes the
// A-fragment reads of the 16 lanes of a row group hit 16 different bank groups.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ int tile_row(int j, int m) { return 16 * (m >> 2) + 4 * j + (m & 3); }

template <int CPR>
__device__ __forceinline__ int w_swizzle(int row) {
    return ((((row >> 4) & 3) << 2) | (row & 3)) & (CPR - 1);
}

// The residual pass maps tile rows so that each half of a tile is one contiguous half of the
// vocabulary range: lane group g holds entries 32h + 8g .. +7 in half h (blocks j = 2h, 2h+1).
// The target-logit rows it streams are float32, 128 bytes per half: each half is then one
// cache line, requested once, instead of both halves touching both lines one phase apart.
// A 16-token block is split between lane groups 2b' and 2b'+1 (lanes l and l ^ 16).
__device__ __forceinline__ int tile_row_resid(int j, int m) {
    return 32 * (j >> 1) + 8 * (m >> 2) + 4 * (j & 1) + (m & 3);
}

template <int CPR>
__device__ __forceinline__ int w_swizzle_resid(int row) {
    return ((((row >> 3) & 3) << 2) | (row & 3)) & (CPR - 1);
}

// Epilogues of one lane for one request, one half at a time: half h holds entries
// v0 + 8h .. v0 + 8h + 7 of the lane's 16-entry sampler block (n_live = how many of its
// entries are < V).  All are branch-free, so that the compiler can interleave them with the
// matrix-core instructions of the other half.
//   kEpiGreedy   every request of the wave is greedy: running max / argmax of c
//   kEpiSampled  every request is sampled: online softmax statistics and the per-token
//                candidate (two-level sampler: the block race once both halves of a block are
//                in, the block's weight being its sum against the running maximum)
//   kEpiMixed    both, with the greedy max / argmax kept in (gm, gi)
//   kEpiResid    residual mode: the per-token candidate of max(p - q, 0) (two-level sampler:
//                block races over max(p - q, 0) and over p)
enum { kEpiGreedy = 0, kEpiSampled = 1, kEpiMixed = 2, kEpiResid = 3 };

// The low half's contribution to a block's race weight, carried to the high half.
struct BlockPart {
    float ref, sum;  // sampled: sum of exp2(s - ref); residual: ref = sum of p, sum = sum of r
};

// MASK: the half may run past V (only in a slab holding a partial last tile); entries
// e >= n_live then have no weight.  Without it every entry is live and no test is emitted.
template <bool MASK>
__device__ __forceinline__ void epi_greedy8(const float c[8], int v, int n_live, float &m,
                                            int &idx) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = (!MASK || e < n_live) ? c[e] : -INFINITY;
        const bool take = x > m;
        m = take ? x : m;
        idx = take ? v + e : idx;
    }
}

// The block maximum is taken on c and scaled once (exact: rounding is monotonic and inv > 0),
// and each weight is exp2(c * inv - base) with one fused multiply-add.
template <int H, bool MASK>
__device__ __forceinline__ void epi_sampled8(const float c[8], int v0, int n_live, float inv,
                                             uint32_t word, SampleState &st, BlockPart &bp) {
    float cm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cm[e] = (!MASK || e < n_live) ? c[e] : -INFINITY;
    float m8 = fmaxf(fmaxf(fmaxf(cm[0], cm[1]), fmaxf(cm[2], cm[3])),
                     fmaxf(fmaxf(cm[4], cm[5]), fmaxf(cm[6], cm[7])));
    const float mn = fmaxf(st.m, m8 * inv);
    const float base = (mn == -INFINITY) ? 0.f : mn;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += fast_exp2(fmaf(cm[e], inv, -base));
    st.l = st.l * fast_exp2(st.m - base) + acc;
    st.m = mn;
    if constexpr (H == 0) {
        bp.ref = base;
        bp.sum = acc;
    } else {
        // the low half's sum was taken against a maximum <= base (0 when it had no weight)
        const float sum = (bp.sum > 0.f ? bp.sum * fast_exp2(bp.ref - base) : 0.f) + acc;
        race_update(st.g, st.idx, base, sum, word, v0);
    }
}

// Residual epilogue with the residual tile-row map: the lane's 8 entries are half of the
// 16-token block that starts at vb; the block's sums are completed with the partner lane
// (lane ^ 16), and both lanes run the same race (a duplicate candidate merges away).
template <typename YT, bool MASK, int H>
__device__ __forceinline__ void epi_resid_pair(const float c[8], const Raw16<YT> &yr, int vb,
                                               int n_live, const RowInfo &ri, uint32_t word,
                                               ResidState &rs) {
    const float inv = kLog2e / ri.T;
    float R = 0.f, P = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool in = !MASK || e < n_live;
        const float pv = in ? fast_exp2(fmaf(yr.get(8 * H + e), inv, -ri.lse2p)) : 0.f;  // p_v
        const float rv = pv - fast_exp2(fmaf(c[e], inv, -ri.qlse2));                   // p - q
        R += in ? fmaxf(rv, 0.f) : 0.f;
        P += pv;
    }
    R += __shfl_xor(R, 16);
    P += __shfl_xor(P, 16);
    race_update(rs.gr, rs.ir, 0.f, R, word, vb);
    race_update(rs.gp, rs.ip, 0.f, P, word, vb);
}

// Per-token sampled epilogue (drafting map): half H of the lane's 16-entry block, entries
// v .. v + 7 (v = v0 + 8H) with their Philox words (w0: v .. v + 3, w1: v + 4 .. v + 7).  The
// base rises to the running maximum of c * inv (taken on c and scaled once: rounding is
// monotonic and inv > 0); each weight is exp2(c * inv - base) with one fused multiply-add and
// feeds both the running sum and the lane's candidate.
template <bool MASK>
__device__ __forceinline__ void epi_token8(const float c[8], int v, int n_live, float inv,
                                           const Philox4 &w0, const Philox4 &w1, TokLane &tl) {
    float cm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cm[e] = (!MASK || e < n_live) ? c[e] : -INFINITY;
    const float m8 = fmaxf(fmaxf(fmaxf(cm[0], cm[1]), fmaxf(cm[2], cm[3])),
                           fmaxf(fmaxf(cm[4], cm[5]), fmaxf(cm[6], cm[7])));
    const float mn = fmaxf(tl.m, m8 * inv);
    const float base = (mn == -INFINITY) ? 0.f : mn;
    const float f = fast_exp2(tl.m - base);  // 0 before the first live entry
    float l = tl.l * f;
    tl.bw *= f;
    // the winner's token is formed once per call: the last taken offset e (an immediate in
    // each select) is all the loop tracks
    int le = 0;
    bool any = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float w = fast_exp2(fmaf(cm[e], inv, -base));
        l += w;
        const float E = exp2_from_word(e < 4 ? w0.w[e] : w1.w[e - 4]);
        const bool take = w * tl.be > tl.bw * E;  // strict: ties keep the lower token
        tl.bw = take ? w : tl.bw;
        tl.be = take ? E : tl.be;
        le = take ? e : le;
        any = any || take;
    }
    tl.bi = any ? v + le : tl.bi;
    tl.l = l;
    tl.m = mn;
}

// Per-token residual candidate of one lane: the best token for the weights r = max(p - q, 0),
// which are absolute (p and q normalised by their known log-normalisers), so no running base is
// needed.  The fallback for a residual that is identically zero (unreachable in exact arithmetic
// after a rejection) is not carried here: the reduction kernel draws from p itself when no
// candidate has a positive weight.
struct ResTok {
    float br, er;
    int ir;
};

__device__ __forceinline__ ResTok restok_init() {
    ResTok t;
    t.br = 0.f;
    t.er = 1.f;
    t.ir = 0x7FFFFFFF;
    return t;
}

__device__ __forceinline__ ResidState restok_finish(const ResTok &t) {
    ResidState s;
    s.gr = t.br > 0.f ? fast_log2(t.br) - fast_log2(t.er) : -INFINITY;
    s.ir = t.br > 0.f ? t.ir : 0x7FFFFFFF;
    s.gp = -INFINITY;  // no p candidate (see above)
    s.ip = 0x7FFFFFFF;
    return s;
}

// Per-token residual epilogue (residual map): the lane's 8 entries v .. v + 7 of half H.
template <typename YT, bool MASK, int H>
__device__ __forceinline__ void epi_resid_token8(const float c[8], const Raw16<YT> &yr, int v,
                                                 int n_live, const RowInfo &ri, const Philox4 &w0,
                                                 const Philox4 &w1, ResTok &rt) {
    const float inv = kLog2e / ri.T;
    int le = 0;  // the last taken offset; the token is formed once per call
    bool any = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool in = !MASK || e < n_live;
        const float pv = fast_exp2(fmaf(yr.get(8 * H + e), inv, -ri.lse2p));             // p_v
        const float rv = in ? fmaxf(pv - fast_exp2(fmaf(c[e], inv, -ri.qlse2)), 0.f) : 0.f;
        const float E = exp2_from_word(e < 4 ? w0.w[e] : w1.w[e - 4]);
        const bool tr = rv * rt.er > rt.br * E;
        rt.br = tr ? rv : rt.br;
        rt.er = tr ? E : rt.er;
        le = tr ? e : le;
        any = any || tr;
    }
    rt.ir = any ? v + le : rt.ir;
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding)
#define DSPARK_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Workgroup barrier of the tile pipeline.  The only LDS writes are the global->LDS loads,
// each retired by its own wave's explicit vmcnt wait before that wave reaches the barrier, so
// the barrier needs no wait on global memory.  It does retire this wave's LDS reads: the
// compiler may sink the matrix-core instructions that consume them below the barrier, and a
// stage must not be refilled while a read of it is still in flight.  The "memory" clobber
// keeps every memory access on its side.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <HeadMode MODE, int SAMP, typename ZT, typename YT, int R, int NQ, bool SPLIT>
__global__ __launch_bounds__(16 / NQ * 64, 1) void markov_mfma_kernel(HeadParams p) {
    static_assert(R == 64 || R == 128 || R == 256, "matrix-core path: rank 64, 128 or 256");
    // SPLIT (drafting with the per-token sampler, at most 128 requests): the two waves of a
    // pair take one request block, one half of every tile each, so a small batch keeps twice
    // as many waves busy; the pair's candidates merge through LDS at the end.
    static_assert(!SPLIT || (NQ == 1 && MODE == HeadMode::Draft && SAMP == kSampToken),
                  "split pairs: drafting, per-token sampler, one request block per wave");
    static_assert(NQ == 1 || NQ == 2, "one or two 16-wide request blocks per wave");
    constexpr int WAVES = 16 / NQ;                 // waves per workgroup (256 requests)
    constexpr int RPW = 16 * NQ;                   // requests per wave
    constexpr int KS = R / 32;                     // MFMA k-steps of 32
    constexpr int CPR = R / 8;                     // 16-byte chunks per W row
    constexpr int TILE_CH = kTileV * CPR;          // chunks per W tile
    constexpr int LPW = TILE_CH / 64 / WAVES;      // direct loads per wave per tile
    static_assert(LPW * 64 * WAVES == TILE_CH, "the W tile splits evenly over the waves");
    constexpr int STAGES = 4;
    constexpr bool kResid = MODE == HeadMode::Residual;
    // Software pipeline over half tiles.  Phase A of tile t: W(t+3) goes out to LDS, then the
    // matrix-core work of the low half of tile t (blocks j = 0, 1) runs together with the
    // epilogue of the high half of tile t - 1.  Phase B: the high logit registers take the
    // high half of tile t, then the high half's matrix-core work runs with the low half's
    // epilogue, and the low logit registers take tile t + 1.  Every wave issues every load,
    // unconditionally (clamped addresses: a W tile past the slab re-reads the slab's last,
    // cache-resident tile into a stage that is never read), and loads retire in issue order,
    // so:
    //  * in phase A, once at most NL + LPW operations are pending after W(t+3) (the low
    //    logits of tile t, W(t+3)), the high logits of tile t - 1 have landed, and with them
    //    W(t+2);
    //  * in phase B, once at most LPW + NH are pending (W(t+3), the high logits of tile t),
    //    the low logits of tile t have landed.
    // W(t) was thus forced two phases before phase A of tile t in every wave; the barrier
    // there makes all of it visible and retires every read of stage (t-1) % 4 (last used in
    // phase B of tile t - 1), which W(t+3) overwrites.
    // vector loads per half tile and wave: per request block, one 16-byte load of bfloat16
    // base logits or two of float32 ones (and the same for the target logits in residual mode)
    constexpr int NH = NQ * ((int)sizeof(ZT) / 2 + (kResid ? (int)sizeof(YT) / 2 : 0));
    constexpr int NL = NH;
    constexpr int WAIT_A = NL + LPW, WAIT_B = LPW + NH;
    static_assert(WAIT_A <= 63 && WAIT_B <= 63 && NL + 2 * LPW <= 63, "vmcnt range");
    // Cache policy of the W tile loads.  The residual pass streams target logits as well, and
    // W read there as non-temporal leaves the level-2 cache to the logit rows, whose two halves
    // are read one phase apart (measured: fewer refetches, shorter launch).  A drafting step
    // keeps the default policy: there W is re-read every step and gains from staying cached.
    static constexpr int kWPolicy = kResid ? 2 /* nt */ : 0;
    __shared__ __align__(16) uint4 wt[STAGES * TILE_CH];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar addressing
    const int m = lane & 15, g = lane >> 4;
    constexpr int ROWS_PER_GROUP = SPLIT ? kRowsPerGroup / 2 : kRowsPerGroup;
    const int hw = SPLIT ? (wave & 1) : 0;       // split: the half of every tile this wave takes
    const int rblk = SPLIT ? (wave >> 1) : wave;  // its request block
    const int n_groups = (p.n_rows_max + ROWS_PER_GROUP - 1) / ROWS_PER_GROUP;
    const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
    const int group = slot % n_groups;
    const int slab = (slot / n_groups) * 8 + xcd;
    // residual mode: every request has its row (B rows) as soon as one needs a residual draw
    const int n_rows = kResid ? (*p.n_rows_dev ? p.n_rows_max : 0) : p.n_rows_max;
    if (group * ROWS_PER_GROUP >= n_rows || slab >= p.n_slabs) return;  // uniform exit

    const int n_tiles = (p.V + kTileV - 1) / kTileV;
    const int t_begin = (int)((long long)slab * n_tiles / p.n_slabs);
    const int t_end = (int)((long long)(slab + 1) * n_tiles / p.n_slabs);
    // an empty slab (more slabs than tiles) still writes its (empty) partials
    const bool have_tiles = t_begin < t_end;
    const int t0 = t_begin;

    // W tile t -> LDS stage s, 16 bytes per lane, swizzled; tiles past the slab re-read the
    // slab's last tile (cache-resident) so every wave issues the same number of loads.  The
    // lane's element offsets inside a tile are fixed; CLAMP (only for a partial last tile of
    // the vocabulary) keeps the rows past V on row V - 1.
    int w_row[LPW], w_off[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int P = (wave * LPW + i) * 64 + lane;
        const int row = P / CPR, pc = P % CPR;
        w_row[i] = row;
        const int key = kResid ? w_swizzle_resid<CPR>(row) : w_swizzle<CPR>(row);
        w_off[i] = row * R + (pc ^ key) * 8;
    }
    auto issue_w = [&](int t, int s, auto clamp_tag) {
        constexpr bool CL = decltype(clamp_tag)::value;
        const int tc = max(t < t_end ? t : t_end - 1, 0);
        const uint16_t *tile = p.W + (size_t)tc * kTileV * R;
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const uint16_t *src = tile + w_off[i];
            if constexpr (CL) {
                const int over = tc * kTileV + w_row[i] - (p.V - 1);  // rows past V - 1
                if (over > 0) src -= (size_t)over * R;
            }
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)src,
                (void __attribute__((address_space(3))) *)(wt + s * TILE_CH + (wave * LPW + i) * 64),
                16, 0, kWPolicy);
        }
    };
    using B0 = std::integral_constant<bool, false>;
    using B1 = std::integral_constant<bool, true>;

    // Prologue.  The first matrix-core step needs W(t0) and the U rows of the previous tokens.
    // A drafting step reads those rows from the copy the previous reduction gathered, and its
    // logit rows follow from the row index alone, so nothing it loads waits on another load:
    // row metadata, U rows, W(t0), the low logits of t0 and W(t0+1), W(t0+2) all go out
    // together, and one explicit count waits for all but the last three.  A residual row's
    // metadata is a two-load chain, then its U gather; its W(t0) goes out first.
    RowInfo ri[NQ];
    bf16x8 ufrag[NQ][KS];
    int rowid[NQ];
    size_t zr[NQ] = {}, yr[NQ] = {};  // logit rows of the tile loads
    // (an empty slab issues the same loads, of a valid tile, and never reads them)
#pragma unroll
    for (int q = 0; q < NQ; ++q) rowid[q] = group * ROWS_PER_GROUP + rblk * RPW + q * 16 + m;
    auto load_u = [&](int q, const uint16_t *urow) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
            ufrag[q][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(urow + 32 * kk));
    };
    DraftRowRaw raw[NQ];
    if constexpr (!kResid) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) raw[q] = draft_row_load(p, rowid[q]);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            // rows past the batch (or past their draft) read a valid row; results are dropped
            const int b = min(rowid[q], p.n_rows_max - 1);
            zr[q] = (size_t)b * p.K + p.k;
            load_u(q, p.A + (size_t)b * R + 8 * g);
        }
        issue_w(t0, 0, B1{});
    } else {
        issue_w(t0, 0, B1{});
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            ri[q] = row_info<MODE>(p, rowid[q], n_rows);
            zr[q] = ri[q].zrow;
            yr[q] = ri[q].yrow;
        }
        // U[prev] (Markov head) or the stored operand of a recurrent-head draft (rows past the
        // batch read request 0's first row; their results are dropped)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            load_u(q, p.S ? p.S + ((size_t)ri[q].b * p.K + ri[q].pos) * R + 8 * g
                          : p.U + (size_t)ri[q].prev * R + 8 * g);
    }
    SampleState st[NQ];
    ResidState rs[NQ];
    TokLane tl[NQ];   // per-token sampler, drafting
    ResTok rt[NQ];    // per-token sampler, residual
    float gm[NQ];     // greedy rows of a mixed wave
    int gi[NQ];
    BlockPart bp[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        st[q] = sample_state_init();
        rs[q] = resid_init();
        tl[q] = tok_lane_init();
        rt[q] = restok_init();
        gm[q] = -INFINITY;
        gi[q] = 0x7FFFFFFF;
        bp[q] = BlockPart{0.f, 0.f};
    }

    // per-lane A-fragment offsets (in chunks) of the four blocks, and the column key
    int a_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a_off[j] = (kResid ? tile_row_resid(j, m) : tile_row(j, m)) * CPR;
    // (the same for every j under either map)
    const int a_key = kResid ? w_swizzle_resid<CPR>(tile_row_resid(0, m))
                             : w_swizzle<CPR>(tile_row(0, m));

    // matrix-core work of half h (blocks j = 2h, 2h + 1) of the tile in stage s
    auto mfma_half = [&](int s, int h, floatx4 (&acc)[2][NQ]) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int q = 0; q < NQ; ++q) acc[jj][q] = floatx4{0.f, 0.f, 0.f, 0.f};
        const uint4 *base = wt + s * TILE_CH;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = 2 * h + jj;
                const bf16x8 a = __builtin_bit_cast(bf16x8, base[a_off[j] + ((4 * kk + g) ^ a_key)]);
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    acc[jj][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ufrag[q][kk], acc[jj][q],
                                                                          0, 0, 0);
            }
        }
    };
    // logits (base, and target in residual mode) of half h of tile t; invalid rows read row 0
    Raw16<ZT> z[NQ];
    Raw16<YT> y[NQ];
    // (CLAMP: the tile may be the vocabulary's partial last one)
    auto load_half = [&](int t, int h, auto clamp_tag) {
        constexpr bool CL = decltype(clamp_tag)::value;
        const int tc = max(t < t_end ? t : t_end - 1, 0);
        // half h's 8 entries start at lane_v + 8h (the loaders add 8h)
        const int lane_v = kResid ? tc * kTileV + 8 * g + 24 * h : tc * kTileV + 16 * g;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if constexpr (CL) {
                z[q].load_half(p.Z, zr[q], p.V, lane_v, h);
                if constexpr (kResid) y[q].load_half(p.Y, yr[q], p.V, lane_v, h);
            } else {
                z[q].load_half_nc(p.Z, zr[q], p.V, lane_v, h);
                if constexpr (kResid) y[q].load_half_nc(p.Y, yr[q], p.V, lane_v, h);
            }
        }
    };

    // Race uniforms for four tiles at a time (block beta = 16a + 4b + c takes word b of the
    // Philox call at counter 4a + c): the lane's block of tile t is 4t + g (drafting map: one
    // call per row), or 4t + 2h + (g >> 1) in half h (residual map: one call per row and half).
    constexpr int NH_WORDS = kResid ? 2 : 1;
    uint32_t rw[NQ][2][4] = {};
    const uint32_t stream = kResid ? kStreamResidual : kStreamDraft;
    auto race_words = [&](int t) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int hh = 0; hh < NH_WORDS; ++hh) {
                const uint32_t c = kResid ? (uint32_t)(2 * hh + (g >> 1)) : (uint32_t)g;
                const Philox4 ph = philox4x32_10(((uint32_t)(t >> 2) << 2) | c,
                                                 (uint32_t)ri[q].pos, ri[q].req, stream, p.key0,
                                                 p.key1);
#pragma unroll
                for (int i = 0; i < 4; ++i) rw[q][hh][i] = ph.w[i];
            }
    };
    // word t & 3 of half h's four (drafting: h ignored), selected with masks (no branches
    // inside the pipeline)
    auto word_of = [&](int q, int t, int h) {
        const int hh = kResid ? h : 0;
        const uint32_t i = (uint32_t)t & 3u;
        const uint32_t m0 = 0u - (uint32_t)(i == 0), m1 = 0u - (uint32_t)(i == 1);
        const uint32_t m2 = 0u - (uint32_t)(i == 2), m3 = 0u - (uint32_t)(i == 3);
        return (rw[q][hh][0] & m0) | (rw[q][hh][1] & m1) | (rw[q][hh][2] & m2) | (rw[q][hh][3] & m3);
    };

    floatx4 acc_lo[2][NQ], acc_hi[2][NQ];
    auto run = [&](auto epi_tag, auto store_tag, auto mask_tag) {
        constexpr int EPI = decltype(epi_tag)::value;
        constexpr bool STORE = decltype(store_tag)::value;
        constexpr bool MASK = decltype(mask_tag)::value;
        constexpr bool WORDS = EPI != kEpiGreedy && SAMP == kSampBlock;
        constexpr bool TOKEN = SAMP == kSampToken;
        // epilogue of half H of tile t from acc, with the race words w[q] of that tile (two-level
        // sampler); the per-token sampler draws the words of the half's 8 tokens here
        auto epilogue = [&](auto half_tag, int t, const floatx4 (&acc)[2][NQ], const uint32_t (&w)[NQ],
                            const Raw16<ZT> (&zz)[NQ]) {
            constexpr int H = decltype(half_tag)::value;
            const int v0 = t * kTileV + 16 * g;  // drafting map: the lane's block
            // residual map: the lane's 8 entries and the start of their block
            const int v8 = t * kTileV + 32 * H + 8 * g, vb = t * kTileV + 32 * H + 16 * (g >> 1);
            const int live = MASK ? min(8, p.V - (kResid ? v8 : v0 + 8 * H)) : 8;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                float c[8];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) c[4 * jj + i] = zz[q].get(8 * H + 4 * jj + i) + acc[jj][q][i];
                if constexpr (STORE) {
                    if (ri[q].valid) {
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            if (4 * hh < live)
                                *reinterpret_cast<float4 *>(p.corrected + ri[q].zrow * (size_t)p.V + v0 + 8 * H + 4 * hh) =
                                    make_float4(c[4 * hh], c[4 * hh + 1], c[4 * hh + 2], c[4 * hh + 3]);
                    }
                }
                // per-token words of the half's 8 tokens: Philox blocks (v >> 2) and (v >> 2) + 1
                const int vt = kResid ? v8 : v0 + 8 * H;
                auto tok_words = [&](uint32_t stream, Philox4 &a, Philox4 &b) {
                    a = philox4x32_10((uint32_t)vt >> 2, (uint32_t)ri[q].pos, ri[q].req, stream,
                                      p.key0, p.key1);
                    b = philox4x32_10(((uint32_t)vt >> 2) + 1u, (uint32_t)ri[q].pos, ri[q].req,
                                      stream, p.key0, p.key1);
                };
                if constexpr (EPI == kEpiGreedy) {
                    epi_greedy8<MASK>(c, v0 + 8 * H, live, st[q].m, st[q].idx);
                } else if constexpr (EPI == kEpiSampled || EPI == kEpiMixed) {
                    const bool samp = EPI == kEpiSampled || ri[q].T > 0.f;
                    const float inv = samp ? kLog2e / ri[q].T : 1.f;
                    if constexpr (TOKEN) {
                        Philox4 wa, wb;
                        tok_words(kStreamDraft, wa, wb);
                        epi_token8<MASK>(c, vt, live, inv, wa, wb, tl[q]);
                    } else {
                        epi_sampled8<H, MASK>(c, v0, live, inv, w[q], st[q], bp[q]);
                    }
                    if constexpr (EPI == kEpiMixed) epi_greedy8<MASK>(c, v0 + 8 * H, live, gm[q], gi[q]);
                } else {
                    if constexpr (TOKEN) {
                        Philox4 wa, wb;
                        tok_words(kStreamResidual, wa, wb);
                        epi_resid_token8<YT, MASK, H>(c, y[q], v8, live, ri[q], wa, wb, rt[q]);
                    } else {
                        epi_resid_pair<YT, MASK, H>(c, y[q], vb, live, ri[q], w[q], rs[q]);
                    }
                }
            }
        };
        using H0 = std::integral_constant<int, 0>;
        using H1 = std::integral_constant<int, 1>;

        if constexpr (SPLIT) {
            // Half H of every tile; its base logits go out one tile ahead, into two buffers
            // taken in turn (tile t0 + i in zs[i & 1]).  Tile t0: its logits, the barrier,
            // W(t0+3), the logits of t0+1, then a wait that forces W(t0+1), W(t0+2), and the
            // matrix-core work of tile t0.  Tile t: the barrier, W(t+3), then once at most
            // 2 LPW + NH operations are pending (W(t+2), the logits of t, W(t+3)) the logits
            // of t-1 have landed, and with them W(t+1): the epilogue of t-1, the logits of
            // t+1 into the buffer it freed, and the matrix-core work of tile t, whose results
            // the next tile's epilogue takes.
            Raw16<ZT> zs[2][NQ];
            auto load_z = [&](int t, int h, auto clamp_tag, Raw16<ZT> (&zd)[NQ]) {
                constexpr bool CL = decltype(clamp_tag)::value;
                const int tc = max(t < t_end ? t : t_end - 1, 0);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    if constexpr (CL)
                        zd[q].load_half(p.Z, zr[q], p.V, tc * kTileV + 16 * g, h);
                    else
                        zd[q].load_half_nc(p.Z, zr[q], p.V, tc * kTileV + 16 * g, h);
                }
            };
            auto split_run = [&](auto half_tag) {
                constexpr int H = decltype(half_tag)::value;
                const uint32_t w0[NQ] = {};
                load_z(t0, H, mask_tag, zs[0]);
                tile_barrier();
                issue_w(t0 + 3, 3, mask_tag);
                load_z(t0 + 1, H, mask_tag, zs[1]);
                DSPARK_WAIT_VMCNT(LPW + 2 * NH);
                mfma_half(0, H, acc_lo);
                auto step = [&](int t, Raw16<ZT> (&zp)[NQ]) {  // zp: the logits of t - 1
                    tile_barrier();
                    issue_w(t + 3, (t + 3 - t0) & 3, mask_tag);
                    DSPARK_WAIT_VMCNT(2 * LPW + NH);
                    epilogue(half_tag, t - 1, acc_lo, w0, zp);
                    load_z(t + 1, H, mask_tag, zp);
                    mfma_half((t - t0) & 3, H, acc_lo);
                };
                int t = t0 + 1;
                for (; t + 1 < t_end; t += 2) {
                    step(t, zs[0]);
                    step(t + 1, zs[1]);
                }
                if (t < t_end) {
                    step(t, zs[0]);
                    ++t;
                }
                DSPARK_WAIT_VMCNT(0);
                // the last tile, t_end - 1 = t - 1, sits in zs[(t - 1 - t0) & 1]
                if (((t - 1 - t0) & 1) == 0)
                    epilogue(half_tag, t - 1, acc_lo, w0, zs[0]);
                else
                    epilogue(half_tag, t - 1, acc_lo, w0, zs[1]);
            };
            if (hw == 0)
                split_run(H0{});
            else
                split_run(H1{});
            return;
        }

        if constexpr (WORDS) race_words(t0);
        // tile t0: phase A without an epilogue
        tile_barrier();
        issue_w(t0 + 3, 3, mask_tag);
        mfma_half(0, 0, acc_lo);
        // phase B of tile t0
        load_half(t0, 1, mask_tag);
        DSPARK_WAIT_VMCNT(WAIT_B);
        mfma_half(0, 1, acc_hi);
        {
            uint32_t w[NQ] = {};
            if constexpr (WORDS) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) w[q] = word_of(q, t0, 0);
            }
            epilogue(H0{}, t0, acc_lo, w, z);
        }
        load_half(t0 + 1, 0, mask_tag);
        for (int t = t0 + 1; t < t_end; ++t) {
            const int stg = (t - t0) & 3;
            uint32_t wp[NQ] = {}, wc[NQ] = {};  // race words of tiles t - 1 and t
            if constexpr (WORDS) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) wp[q] = word_of(q, t - 1, 1);
            }
            // phase A
            tile_barrier();
            issue_w(t + 3, (t + 3 - t0) & 3, mask_tag);
            if constexpr (WORDS) {
                if ((t & 3) == 0) race_words(t);
#pragma unroll
                for (int q = 0; q < NQ; ++q) wc[q] = word_of(q, t, 0);
            }
            DSPARK_WAIT_VMCNT(WAIT_A);
            mfma_half(stg, 0, acc_lo);
            epilogue(H1{}, t - 1, acc_hi, wp, z);
            // phase B (the high logit registers are free again)
            load_half(t, 1, mask_tag);
            DSPARK_WAIT_VMCNT(WAIT_B);
            mfma_half(stg, 1, acc_hi);
            epilogue(H0{}, t, acc_lo, wc, z);
            load_half(t + 1, 0, mask_tag);
        }
        // the high half of the last tile
        uint32_t w[NQ] = {};
        if constexpr (WORDS) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) w[q] = word_of(q, t_end - 1, 1);
        }
        DSPARK_WAIT_VMCNT(0);
        epilogue(H1{}, t_end - 1, acc_hi, w, z);
    };

    // A wave whose rows are all empty (past the batch, or past their drafts) keeps only its
    // share of the workgroup's W pipeline: the same W loads into the same stages and the same
    // barriers as `run` (one before tile t0's work, one per later tile), and no logit loads,
    // matrix-core work or sampling.  Its wait after each issue leaves W(t+2), W(t+3) pending,
    // so W(t+1) has landed before the barrier that opens tile t+1 (the live waves force it no
    // later), and the barrier before each issue retires every read of the stage it refills.
    auto run_loader = [&](auto mask_tag) {
        tile_barrier();
        issue_w(t0 + 3, 3, mask_tag);
        DSPARK_WAIT_VMCNT(2 * LPW);
        for (int t = t0 + 1; t < t_end; ++t) {
            tile_barrier();
            issue_w(t + 3, (t + 3 - t0) & 3, mask_tag);
            DSPARK_WAIT_VMCNT(2 * LPW);
        }
    };

    using I0 = std::integral_constant<int, kEpiGreedy>;
    using I1 = std::integral_constant<int, kEpiSampled>;
    using I2 = std::integral_constant<int, kEpiMixed>;
    using I3 = std::integral_constant<int, kEpiResid>;
    // the low logits of t0, then W(t0+1), W(t0+2); the metadata, the U fragments and W(t0)
    // have landed once only those are pending (phase B of t0 waits for the rest)
    if constexpr (SPLIT) {  // a split wave loads its half's logits in tile t0
        issue_w(t0 + 1, 1, B1{});
        issue_w(t0 + 2, 2, B1{});
        DSPARK_WAIT_VMCNT(2 * LPW);
    } else {
        load_half(t0, 0, B1{});
        issue_w(t0 + 1, 1, B1{});
        issue_w(t0 + 2, 2, B1{});
        DSPARK_WAIT_VMCNT(NL + 2 * LPW);
    }
    if constexpr (!kResid) {
        // Every use of the metadata is made to depend on a clock read that stays after the
        // wait (both have side effects), so none is moved above it, where the compiler would
        // wait for every outstanding load.  The clock never reads all ones.
        const bool never = __builtin_amdgcn_s_memtime() == ~0ull;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            raw[q].kb = never ? 0 : raw[q].kb;
            raw[q].T = never ? 0.f : raw[q].T;
            raw[q].req = never ? 0u : raw[q].req;
        }
    }
    bool any_valid = false, any_sampled = false, any_greedy = false;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if constexpr (!kResid) ri[q] = draft_row_resolve(p, rowid[q], n_rows, raw[q]);
        any_valid |= ri[q].valid;
        any_sampled |= ri[q].valid && ri[q].T > 0.f;
        any_greedy |= ri[q].valid && !(ri[q].T > 0.f);
    }
    const bool wave_active = __any(any_valid);
    const bool wave_sampled = __any(any_sampled);
    const bool wave_greedy = __any(any_greedy);
    if (have_tiles) {  // uniform
        // only the slab holding a partial last tile needs the masked (and clamped) variant;
        // writing the corrected logits out is rare and always takes it
        const bool partial = t_end == n_tiles && p.V % kTileV != 0;
        if (!wave_active) {
            if (partial) run_loader(B1{});
            else run_loader(B0{});
        } else if constexpr (kResid) {
            if (partial) run(I3{}, B0{}, B1{});
            else run(I3{}, B0{}, B0{});
        } else if (p.corrected) {
            run(I2{}, B1{}, B1{});
        } else if (!wave_sampled) {
            if (partial) run(I0{}, B0{}, B1{});
            else run(I0{}, B0{}, B0{});
        } else if (!wave_greedy) {
            if (partial) run(I1{}, B0{}, B1{});
            else run(I1{}, B0{}, B0{});
        } else {
            if (partial) run(I2{}, B0{}, B1{});
            else run(I2{}, B0{}, B0{});
        }
    }

    // every global->LDS load has landed before the workgroup can exit
    DSPARK_WAIT_VMCNT(0);
    TokState tsq[NQ];
    if constexpr (MODE == HeadMode::Draft) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (!(ri[q].T > 0.f) && (wave_sampled || p.corrected)) {  // the mixed epilogue kept it aside
                st[q].m = gm[q];
                st[q].idx = gi[q];
            }
            tsq[q] = tok_finish(tl[q]);
        }
    }
    if constexpr (SPLIT) {
        // The high-half wave of each pair hands its lanes' states to the low-half wave through
        // LDS (the W stages, free once every wave has passed the first barrier); the low-half
        // wave merges them and writes the partials.  Every wave meets both barriers.
        struct PairState {
            SampleState st;
            TokState ts;
        };
        static_assert(sizeof(PairState) * 64 * (16 / 2) <= sizeof(wt), "pair states fit the stages");
        PairState *ps = reinterpret_cast<PairState *>(wt);
        tile_barrier();
        if (wave_active && hw == 1) ps[rblk * 64 + lane] = PairState{st[0], tsq[0]};
        tile_barrier();
        if (!wave_active || hw == 1) return;
        const PairState o = ps[rblk * 64 + lane];
        merge_into(st[0], o.st, !(ri[0].T > 0.f));
        tsq[0] = merge_token(tsq[0], o.ts);
    }
    if (!wave_active) return;
    // merge the four lanes that share a request (lane, lane^16, lane^32, lane^48); every lane
    // runs every shuffle (partners hold the same request and so take the same branches)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if constexpr (MODE == HeadMode::Draft) {
            const bool greedy = !(ri[q].T > 0.f);
            TokState ts = tsq[q];
#pragma unroll
            for (int mask = 16; mask <= 32; mask <<= 1) {
                const SampleState o = shfl_xor_state(st[q], mask);
                merge_into(st[q], o, greedy);
                if constexpr (SAMP == kSampToken) ts = merge_token(ts, shfl_xor_tok(ts, mask));
            }
            if (lane < 16 && ri[q].valid)
                p.dpartials[(size_t)rowid[q] * p.n_slabs + slab] =
                    (SAMP == kSampToken && !greedy) ? to_draft_partial(ts) : to_draft_partial(st[q]);
        } else {
            if constexpr (SAMP == kSampToken) rs[q] = restok_finish(rt[q]);
#pragma unroll
            for (int mask = 16; mask <= 32; mask <<= 1)
                rs[q] = resid_merge(rs[q], resid_shfl_xor(rs[q], mask));
            if (lane < 16 && ri[q].valid) {
                Partial out;
                out.g = rs[q].gr;
                out.idx = rs[q].ir;
                out.m = rs[q].gp;
                out.l = __int_as_float(rs[q].ip);
                p.partials[(size_t)rowid[q] * p.n_slabs + slab] = out;
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Vector-ALU kernel: one workgroup per (row, slab); float32 or bfloat16 factors, any rank.
// ---------------------------------------------------------------------------------------

template <typename FT>
__device__ __forceinline__ float factor_at(const void *base, size_t idx);
template <>
__device__ __forceinline__ float factor_at<float>(const void *base, size_t idx) {
    return reinterpret_cast<const float *>(base)[idx];
}
template <>
__device__ __forceinline__ float factor_at<uint16_t>(const void *base, size_t idx) {
    return bf16_to_f32(reinterpret_cast<const uint16_t *>(base)[idx]);
}

constexpr int kValuThreads = 256;
constexpr int kMaxValuRank = 1024;

template <HeadMode MODE, int SAMP, typename ZT, typename YT, typename FT>
__global__ __launch_bounds__(kValuThreads) void markov_valu_kernel(HeadParams p) {
    __shared__ float urow[kMaxValuRank];
    __shared__ SampleState red_st[kValuThreads / 64];
    __shared__ TokState red_ts[kValuThreads / 64];
    __shared__ ResidState red_rs[kValuThreads / 64];
    const int slab = (int)(blockIdx.x % (unsigned)p.n_slabs);
    const int row = (int)(blockIdx.x / (unsigned)p.n_slabs);
    // residual mode: row b is request b's residual row, when it has one (the flag is set)
    const int n_rows = (MODE == HeadMode::Residual) ? (*p.n_rows_dev ? p.n_rows_max : 0)
                                                    : p.n_rows_max;
    const RowInfo ri = row_info<MODE>(p, row, n_rows);
    if (!ri.valid) return;  // uniform per block
    const void *Ub = p.Uf ? (const void *)p.Uf : (const void *)p.U;
    const void *Wb = p.Wf ? (const void *)p.Wf : (const void *)p.W;
    for (int i = threadIdx.x; i < p.r; i += kValuThreads)
        urow[i] = factor_at<FT>(Ub, (size_t)ri.prev * p.r + i);
    __syncthreads();

    const int n_tiles = (p.V + kTileV - 1) / kTileV;
    const int v_begin = (int)((long long)slab * n_tiles / p.n_slabs) * kTileV;
    int v_end = (int)((long long)(slab + 1) * n_tiles / p.n_slabs) * kTileV;
    if (v_end > p.V) v_end = p.V;

    SampleState st = sample_state_init();
    TokState ts = tok_state_init();
    ResidState rs = resid_init();
    // every lane runs every iteration: the epilogue exchanges block sums between lanes
    for (int vb = v_begin; vb < v_end; vb += 4 * kValuThreads) {
        const int v = vb + 4 * threadIdx.x;
        const bool live = v < v_end;
        float c[4] = {0.f, 0.f, 0.f, 0.f};
        if (live) {
            float z[4];
            load4<ZT>(p.Z, ri.zrow, p.V, v, z);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float acc = 0.f;
                const size_t wrow = (size_t)(v + i) * p.r;
                for (int j = 0; j < p.r; ++j) acc = fmaf(urow[j], factor_at<FT>(Wb, wrow + j), acc);
                c[i] = z[i] + acc;
            }
        }
        head_epilogue4<MODE, SAMP, YT>(p, ri, v, live, c, st, ts, rs);
    }
    // block reduction
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool greedy = ri.T == 0.f;
    const bool token = MODE == HeadMode::Draft && SAMP == kSampToken && !greedy;  // uniform
    // the candidate's logit against the lane's final base (see TokState)
    if (token) ts.sx = ts.g > -INFINITY ? fmaf(ts.sx, kLog2e / ri.T, -ts.m) : -INFINITY;
    for (int mask = 1; mask < 64; mask <<= 1) {
        if constexpr (MODE == HeadMode::Draft) {
            if (token) {
                ts = merge_token(ts, shfl_xor_tok(ts, mask));
            } else {
                const SampleState o = shfl_xor_state(st, mask);
                merge_into(st, o, greedy);
            }
        } else {
            rs = resid_merge(rs, resid_shfl_xor(rs, mask));
        }
    }
    if (lane == 0) {
        red_st[wave] = st;
        red_ts[wave] = ts;
        red_rs[wave] = rs;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if constexpr (MODE == HeadMode::Draft) {
            DraftPartial out;
            if (token) {
                TokState a = red_ts[0];
                for (int w = 1; w < kValuThreads / 64; ++w) a = merge_token(a, red_ts[w]);
                out = to_draft_partial(a);
            } else {
                SampleState a = red_st[0];
                for (int w = 1; w < kValuThreads / 64; ++w) merge_into(a, red_st[w], greedy);
                out = to_draft_partial(a);
            }
            p.dpartials[(size_t)row * p.n_slabs + slab] = out;
        } else {
            ResidState a = red_rs[0];
            for (int w = 1; w < kValuThreads / 64; ++w) a = resid_merge(a, red_rs[w]);
            Partial out;
            out.g = a.gr;
            out.idx = a.ir;
            out.m = a.gp;
            out.l = __int_as_float(a.ip);
            p.partials[(size_t)row * p.n_slabs + slab] = out;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Draft: prepare (status, validated first tokens) and per-step row reduction
// ---------------------------------------------------------------------------------------

// The first position's previous tokens (workgroup 0, which also clears the status word) and,
// on the matrix-core path (a_rows set), their U rows gathered into a_rows, one 16-byte chunk
// per thread over the whole grid.
__global__ __launch_bounds__(256) void draft_prepare_kernel(int B, int V, int r,
                                                            const int32_t *prev_token,
                                                            const uint16_t *U, int32_t *prev_cur,
                                                            uint16_t *a_rows, uint32_t *status) {
    if (blockIdx.x == 0) {
        if (threadIdx.x == 0) *status = 0u;
        __syncthreads();
        for (int b = threadIdx.x; b < B; b += blockDim.x)
            prev_cur[b] = checked_token(prev_token[b], V, status);
    }
    if (a_rows) {
        const int cpr = r / 8;  // 16-byte chunks per row
        const int i = blockIdx.x * blockDim.x + threadIdx.x;
        if (i < B * cpr) {
            const int b = i / cpr, c = i - b * cpr;
            const int t = prev_token[b];
            const int tc = (t < 0 || t >= V) ? 0 : t;  // as checked_token (flagged there)
            *reinterpret_cast<uint4 *>(a_rows + (size_t)b * r + 8 * c) =
                *reinterpret_cast<const uint4 *>(U + (size_t)tc * r + 8 * c);
        }
    }
}

// One wave per request: merge the slabs' partials of position k.  Per-token sampler: the
// winning token and its scaled logit come with the merged candidates.  Two-level sampler: draw
// the token inside the winning 16-token block from its recomputed corrected logits.  On the
// matrix-core path (a_rows set) it also copies the drawn token's U row for the next position.
__global__ __launch_bounds__(256) void draft_reduce_kernel(
    int B, int K, int V, int r, int k, int z_dtype, int uw_dtype, const void *Z, const void *U,
    const void *W, const int32_t *draft_len, const float *temperature, const uint32_t *req_id,
    uint32_t key0, uint32_t key1, const DraftPartial *partials, int n_slabs, int sampler,
    int32_t *prev_cur, uint16_t *a_rows, const uint16_t *op_rows, int32_t *tokens, float *q_tok,
    float *q_lse, uint32_t *status) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (b >= B) return;  // uniform per wave
    // Every load that depends on no other goes out first (absent optional arrays are read at a
    // valid stand-in address and replaced), the slab partials four per lane at a time.
    const int32_t *dl = draft_len ? draft_len : prev_cur;
    const uint32_t *rq = req_id ? req_id : reinterpret_cast<const uint32_t *>(prev_cur);
    const int kb_ld = dl[b];
    const float T_ld = temperature[b];
    const int prev = prev_cur[b];
    const uint32_t req_ld = rq[b];
    constexpr int kPer = 4;
    DraftPartial pp[kPer];
    const DraftPartial *prow = partials + (size_t)b * n_slabs;
#pragma unroll
    for (int i = 0; i < kPer; ++i) pp[i] = prow[min(lane + 64 * i, n_slabs - 1)];

    int kb = draft_len ? kb_ld : K;
    if (kb < 0 || kb > K) {
        if (lane == 0 && k == 0) atomicOr(status, DSPARK_DEV_BAD_LENGTH);
        kb = kb < 0 ? 0 : K;
    }
    const size_t o = (size_t)b * K + k;
    if (k >= kb) {
        if (lane == 0) {
            tokens[o] = -1;
            q_tok[o] = 0.f;
            q_lse[o] = 0.f;
        }
        return;
    }
    const float T = (lane == 0 && k == 0) ? checked_temperature(T_ld, status) : T_ld;
    const bool greedy = !(T > 0.f);
    // a row with no finite score (all -inf / NaN logits) has no winner: token 0, flagged,
    // so that the next step's gather stays inside U
    int x;
    float qt = 1.f, ql = 0.f;
    if (!greedy && sampler == kSampToken) {
        TokState ts = tok_state_init();
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (lane + 64 * i < n_slabs) ts = merge_token(ts, tok_from_partial(pp[i]));
        for (int s = lane + 64 * kPer; s < n_slabs; s += 64) ts = merge_token(ts, tok_from_partial(prow[s]));
        for (int mask = 1; mask < 64; mask <<= 1) ts = merge_token(ts, shfl_xor_tok(ts, mask));
        x = (ts.g > -INFINITY && ts.idx >= 0 && ts.idx < V) ? ts.idx : -1;
        const float l2 = fast_log2(ts.l);
        qt = fast_exp2(ts.sx - l2);  // sx is taken against the base m
        ql = (ts.m + l2) * kLn2;
    } else {
        SampleState st = sample_state_init();
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (lane + 64 * i < n_slabs) merge_into(st, from_partial(pp[i].p), greedy);
        for (int s = lane + 64 * kPer; s < n_slabs; s += 64) {
            const SampleState o2 = from_partial(prow[s].p);
            merge_into(st, o2, greedy);
        }
        for (int mask = 1; mask < 64; mask <<= 1) {
            const SampleState o2 = shfl_xor_state(st, mask);
            merge_into(st, o2, greedy);
        }
        if (greedy) {
            x = st.idx;
            if (x < 0 || x >= V) x = -1;
        } else {
            const int v0 = st.idx;
            if (v0 < 0 || v0 >= V || (v0 % kSampleBlock) != 0) {
                x = -1;
            } else {
                const int e = lane & 15;
                const bool in = v0 + e < V;
                // left operand: U[prev] (Markov head) or the recurrent head's current operand
                const void *op = op_rows ? static_cast<const void *>(op_rows + (size_t)b * r) : U;
                const float c = wave_corrected16(Z, z_dtype, o, op, W, uw_dtype, r, V,
                                                 op_rows ? 0 : prev, v0);
                const float inv = kLog2e / T;
                const uint32_t req = req_id ? req_ld : (uint32_t)b;
                const uint32_t w = token_word((uint32_t)(v0 + e), (uint32_t)k, req,
                                              kStreamDraftWithin, key0, key1);
                const float sc = in ? c * inv + gumbel2_from_word(w) : -INFINITY;
                int best = v0 + e;
                float bsc = sc, bc = c;
                wave_argmax16(bsc, best, bc);
                x = (bsc > -INFINITY) ? best : -1;
                // q from the winner's logit against the row's base (one rounding, any T)
                const float l2 = fast_log2(st.l);
                qt = fast_exp2(fmaf(bc, inv, -st.m) - l2);
                ql = (st.m + l2) * kLn2;
            }
        }
    }
    if (lane == 0) {
        if (x < 0) {
            atomicOr(status, DSPARK_DEV_BAD_TOKEN);
            x = 0;
            qt = 0.f;
        }
        tokens[o] = x;
        prev_cur[b] = x;
        q_tok[o] = qt;
        q_lse[o] = ql;
    }
    // the next position's U row (a flagged row takes token 0's)
    x = __shfl(x, 0);
    if (a_rows && k + 1 < kb) {
        const int xs = x < 0 ? 0 : x;
        const uint16_t *src = reinterpret_cast<const uint16_t *>(U) + (size_t)xs * r;
        for (int c = lane; c < r / 8; c += 64)
            *reinterpret_cast<uint4 *>(a_rows + (size_t)b * r + 8 * c) =
                *reinterpret_cast<const uint4 *>(src + 8 * c);
    }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------

static bool use_mfma(int uw_dtype, int r) {
    return uw_dtype == DSPARK_BF16 && (r == 64 || r == 128 || r == 256);
}

template <HeadMode MODE, int SAMP, typename ZT, typename YT>
static hipError_t launch_head_t(const HeadParams &p, int uw_dtype, hipStream_t s) {
    if (use_mfma(uw_dtype, p.r)) {
        // Drafting at most 128 requests with the per-token sampler (ranks 128, 256, bfloat16
        // base logits): split pairs, so that a small batch has two waves per request block
        // (one per half tile).
        if constexpr (MODE == HeadMode::Draft && SAMP == kSampToken &&
                      std::is_same<ZT, uint16_t>::value) {
            if (p.n_rows_max <= kRowsPerGroup / 2 && (p.r == 128 || p.r == 256)) {
                const dim3 grid(p.n_slabs);
                if (p.r == 128)
                    markov_mfma_kernel<MODE, SAMP, ZT, YT, 128, 1, true><<<grid, 16 * 64, 0, s>>>(p);
                else
                    markov_mfma_kernel<MODE, SAMP, ZT, YT, 256, 1, true><<<grid, 16 * 64, 0, s>>>(p);
                return hipGetLastError();
            }
        }
        const int groups = (p.n_rows_max + kRowsPerGroup - 1) / kRowsPerGroup;
        // Ranks 128 and 256: 16 waves of 16 requests (four waves per SIMD in 128 registers: the
        // per-token epilogues are bound by vector-ALU issue and hide their latency across
        // waves), except the two-level sampler's residual pass, whose epilogue needs more
        // registers than four waves leave.  Rank 64, whose W tile is too small to split 16
        // ways: 8 waves of 32.
        const dim3 grid(p.n_slabs * groups);
        constexpr int NQ = (MODE == HeadMode::Residual && SAMP == kSampBlock) ? 2 : 1;
        switch (p.r) {
            case 64: markov_mfma_kernel<MODE, SAMP, ZT, YT, 64, 2, false><<<grid, 8 * 64, 0, s>>>(p); break;
            case 128: markov_mfma_kernel<MODE, SAMP, ZT, YT, 128, NQ, false><<<grid, 16 / NQ * 64, 0, s>>>(p); break;
            case 256: markov_mfma_kernel<MODE, SAMP, ZT, YT, 256, NQ, false><<<grid, 16 / NQ * 64, 0, s>>>(p); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        const dim3 grid((unsigned)p.n_slabs * (unsigned)p.n_rows_max), block(kValuThreads);
        if (uw_dtype == DSPARK_F32)
            markov_valu_kernel<MODE, SAMP, ZT, YT, float><<<grid, block, 0, s>>>(p);
        else
            markov_valu_kernel<MODE, SAMP, ZT, YT, uint16_t><<<grid, block, 0, s>>>(p);
    }
    return hipGetLastError();
}

template <HeadMode MODE, typename ZT, typename YT>
static hipError_t launch_head_s(const HeadParams &p, int uw_dtype, hipStream_t s) {
    if (p.sampler == kSampBlock) return launch_head_t<MODE, kSampBlock, ZT, YT>(p, uw_dtype, s);
    return launch_head_t<MODE, kSampToken, ZT, YT>(p, uw_dtype, s);
}

// (drafting steps read no target logits: one instantiation per base-logit type)
template <HeadMode MODE>
static hipError_t launch_head(const HeadParams &p, int z_dtype, int uw_dtype, int y_dtype,
                              hipStream_t s) {
    if constexpr (MODE == HeadMode::Draft) {
        (void)y_dtype;
        if (z_dtype == DSPARK_BF16) return launch_head_s<MODE, uint16_t, float>(p, uw_dtype, s);
        return launch_head_s<MODE, float, float>(p, uw_dtype, s);
    } else {
        if (z_dtype == DSPARK_BF16) {
            if (y_dtype == DSPARK_BF16) return launch_head_s<MODE, uint16_t, uint16_t>(p, uw_dtype, s);
            return launch_head_s<MODE, uint16_t, float>(p, uw_dtype, s);
        }
        if (y_dtype == DSPARK_BF16) return launch_head_s<MODE, float, uint16_t>(p, uw_dtype, s);
        return launch_head_s<MODE, float, float>(p, uw_dtype, s);
    }
}

static void set_factors(HeadParams &hp, const void *U, const void *W, int uw_dtype) {
    if (uw_dtype == DSPARK_F32) {
        hp.Uf = reinterpret_cast<const float *>(U);
        hp.Wf = reinterpret_cast<const float *>(W);
        hp.U = nullptr;
        hp.W = nullptr;
    } else {
        hp.U = reinterpret_cast<const uint16_t *>(U);
        hp.W = reinterpret_cast<const uint16_t *>(W);
        hp.Uf = nullptr;
        hp.Wf = nullptr;
    }
}

bool draft_gathers_rows(const dspark_draft_args &a) { return use_mfma(a.uw_dtype, a.r); }
bool draft_uses_rnn(const dspark_draft_args &a) { return a.gru_wi != nullptr; }
bool matrix_core_factors(int uw_dtype, int r) { return use_mfma(uw_dtype, r); }

hipError_t launch_draft_prepare(const dspark_draft_args &a, const DraftWs &ws, hipStream_t s) {
    // (the recurrent head's first operand comes from its own kernel instead)
    uint16_t *gather = draft_uses_rnn(a) ? nullptr : ws.a_rows;
    const int chunks = gather ? a.B * (a.r / 8) : 0;
    const int grid = std::max(1, (chunks + 255) / 256);
    draft_prepare_kernel<<<grid, 256, 0, s>>>(a.B, a.V, a.r, a.prev_token,
                                            reinterpret_cast<const uint16_t *>(a.U), ws.prev_cur,
                                            gather, ws.status);
    return hipGetLastError();
}

hipError_t launch_draft_step(const DraftStepParams &d, int z_dtype, int uw_dtype, hipStream_t s) {
    HeadParams hp{};
    hp.B = d.B;
    hp.K = d.K;
    hp.V = d.V;
    hp.r = d.r;
    hp.n_rows_max = d.B;
    hp.n_rows_dev = nullptr;
    hp.k = d.k;
    hp.Z = d.Z;
    set_factors(hp, d.U, d.W, uw_dtype);
    hp.draft_len = d.draft_len;
    hp.temperature = d.temperature;
    hp.req_id = d.req_id;
    hp.key0 = d.key0;
    hp.key1 = d.key1;
    hp.prev_cur = d.prev_cur;
    hp.A = d.a_rows;
    hp.partials = nullptr;
    hp.dpartials = d.partials;
    hp.sampler = d.sampler;
    hp.corrected = d.corrected;
    hp.status = d.status;
    hp.n_slabs = d.n_slabs;
    return launch_head<HeadMode::Draft>(hp, z_dtype, uw_dtype, DSPARK_F32, s);
}

hipError_t launch_draft_reduce(const dspark_draft_args &a, const DraftWs &ws, int k,
                               hipStream_t s) {
    const int per_block = 1;  // one wave per request and workgroup: spread over the CUs
    draft_reduce_kernel<<<(a.B + per_block - 1) / per_block, 64 * per_block, 0, s>>>(
        a.B, a.K, a.V, a.r, k, a.z_dtype, a.uw_dtype, a.Z, a.U, a.W, a.draft_len, a.temperature,
        a.req_id, (uint32_t)(a.seed & 0xFFFFFFFFu), (uint32_t)(a.seed >> 32), ws.partials,
        ws.n_slabs, a.sampler, ws.prev_cur, draft_uses_rnn(a) ? nullptr : ws.a_rows,
        draft_uses_rnn(a) ? ws.a_rows : nullptr, a.draft_tokens, a.q_tok, a.q_lse, ws.status);
    return hipGetLastError();
}

hipError_t launch_verify_residual(const dspark_verify_args &a, const VerifyWs &ws,
                                  hipStream_t s) {
    HeadParams hp{};
    hp.B = a.B;
    hp.K = a.K;
    hp.V = a.V;
    hp.r = a.r;
    hp.n_rows_max = a.B;
    hp.n_rows_dev = ws.n_resid;
    hp.k = 0;
    hp.Z = a.Z;
    set_factors(hp, a.U, a.W, a.uw_dtype);
    hp.draft_len = nullptr;
    hp.temperature = a.temperature;
    hp.req_id = a.req_id;
    hp.key0 = (uint32_t)(a.seed & 0xFFFFFFFFu);
    hp.key1 = (uint32_t)(a.seed >> 32);
    hp.resid_rows = ws.resid_rows;
    hp.prev_token = a.prev_token;
    hp.draft_tokens = a.draft_tokens;
    hp.Y = a.Y;
    hp.rowstats = ws.rowstats;
    hp.q_lse = a.q_lse;
    hp.S = a.head_state;
    hp.partials = ws.partials;
    hp.dpartials = nullptr;
    hp.sampler = a.sampler;
    hp.corrected = nullptr;
    hp.status = ws.status;
    hp.n_slabs = ws.n_slabs;
    return launch_head<HeadMode::Residual>(hp, a.z_dtype, a.uw_dtype, a.y_dtype, s);
}

}  // namespace dspark
