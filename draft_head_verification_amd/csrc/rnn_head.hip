// Recurrent sequential head: the GRU update of the drafting state, one position per launch.
//
// Besides the default Markov head, the pages mention an optional RNN head that follows the
// whole prefix of the draft block, of limited gain and off by default (QbitAI, "DSpark in 10
// concepts", section "Cheaper serial module: the Markov head"; 10100.com commentary, section
// "Parallel drafts are fast but may turn 'of course' into 'of problem'").  They give no form;
// the reading implemented is a GRU (Cho et al., EMNLP 2014; gate order reset, update, new,
// separate input and hidden biases) over the previous tokens' left factors,
//   h_k = GRU(h_{k-1}, U[prev_k]),  h_{-1} = 0,
// whose state, rounded to bfloat16, replaces U[prev] as the left operand of the low-rank
// contraction.  The drafting step kernels are unchanged: they read the operand of each
// request from the same gathered-row array the Markov head uses.
//
// Work: per request 6 r x r products (input and hidden weights of three gates), B * 6 r^2
// multiply-adds per position (0.1 GFLOP at B = r = 256), float32 throughout: about 3 us of the
// vector ALUs over 256 CUs, about half that on the matrix cores.  A workgroup takes 16
// requests x 16 hidden units (256 workgroups at B = r = 256); every load it needs -- the 16
// input rows (bfloat16, widened), the 16 state rows and the 6 x 16 weight rows -- goes out at
// once into shared memory (133 KB at r = 256).  The four pre-activations (reset, update,
// new-input, new-hidden) are 16 x 16 float32 matrix-core products, each wave summing a
// quarter of the inputs; the quarters are added in shared memory and one thread per
// (request, unit) finishes the gates.
#include "dspark_common.hpp"

namespace dspark {

constexpr int kRnnRows = 16;    // requests per workgroup
constexpr int kRnnUnits = 16;   // hidden units per workgroup
constexpr int kRnnThreads = kRnnRows * kRnnUnits;
constexpr int kRnnPad = 4;      // floats of padding per shared row (spreads the banks)

template <int R>
__global__ __launch_bounds__(kRnnThreads) void rnn_step_kernel(
    int B, int K, int k, int V, const uint16_t *U, const int32_t *prev_cur,
    const int32_t *draft_len, const float *wi, const float *wh, const float *bi,
    const float *bh, const float *h_prev, float *h_next, uint16_t *a_rows,
    uint16_t *state_out) {
    static_assert(R % kRnnUnits == 0 && R % 8 == 0, "rank");
    constexpr int RS = R + kRnnPad;  // shared row stride (floats)
    __shared__ __align__(16) float smem[(2 * kRnnRows + 6 * kRnnUnits) * RS];
    float *es = smem;                          // [kRnnRows][RS] inputs
    float *hs = es + kRnnRows * RS;            // [kRnnRows][RS] states
    float *ws = hs + kRnnRows * RS;            // [6][kRnnUnits][RS]: Wi gates 0..2, Wh gates 0..2
    const int t = threadIdx.x;
    const int row0 = blockIdx.x * kRnnRows, unit0 = blockIdx.y * kRnnUnits;

    // ---- every load at once: inputs (8 bfloat16 per 16 bytes), states, weights (4 floats)
    constexpr int E_CH = kRnnRows * R / 8, H_CH = kRnnRows * R / 4, W_CH = 6 * kRnnUnits * R / 4;
    constexpr int E_PER = (E_CH + kRnnThreads - 1) / kRnnThreads;
    constexpr int H_PER = (H_CH + kRnnThreads - 1) / kRnnThreads;
    // A weight row of rank 256 is 1 KB, exactly one wave's 16-byte-per-lane global->shared
    // load, so those rows go straight to shared memory; smaller ranks pass through registers.
    constexpr bool W_DIRECT = R == 256;
    constexpr int W_PER = W_DIRECT ? 1 : (W_CH + kRnnThreads - 1) / kRnnThreads;
    uint4 ev[E_PER];
    float4 hv[H_PER], wv[W_PER];
    if constexpr (W_DIRECT) {
        const int lane = t & 63, wave = t >> 6;
        for (int pu = wave; pu < 6 * kRnnUnits; pu += kRnnThreads / 64) {
            const float *src = (pu < 3 * kRnnUnits ? wi : wh) +
                               (size_t)((pu / kRnnUnits) % 3 * R + unit0 + pu % kRnnUnits) * R;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(src + 4 * lane),
                (void __attribute__((address_space(3))) *)(ws + pu * RS), 16, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < E_PER; ++i) {
        const int c = min(t + i * kRnnThreads, E_CH - 1);
        const int rr = c / (R / 8), j = (c % (R / 8)) * 8;
        const int x = prev_cur[min(row0 + rr, B - 1)];
        const int tok = (x < 0 || x >= V) ? 0 : x;  // validated by the prepare / reduce kernels
        ev[i] = *reinterpret_cast<const uint4 *>(U + (size_t)tok * R + j);
    }
#pragma unroll
    for (int i = 0; i < H_PER; ++i) {
        const int c = min(t + i * kRnnThreads, H_CH - 1);
        const int rr = c / (R / 4), j = (c % (R / 4)) * 4;
        hv[i] = h_prev ? *reinterpret_cast<const float4 *>(h_prev + (size_t)min(row0 + rr, B - 1) * R + j)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < W_PER; ++i) {
        if constexpr (W_DIRECT) break;
        const int c = min(t + i * kRnnThreads, W_CH - 1);
        const int part = c / (kRnnUnits * R / 4), rem = c % (kRnnUnits * R / 4);
        const int uu = rem / (R / 4), j = (rem % (R / 4)) * 4;
        const float *src = part < 3 ? wi : wh;
        const int gate = part % 3;
        wv[i] = *reinterpret_cast<const float4 *>(src + (size_t)(gate * R + unit0 + uu) * R + j);
    }
#pragma unroll
    for (int i = 0; i < E_PER; ++i) {
        const int c = t + i * kRnnThreads;
        if (c < E_CH) {
            const int rr = c / (R / 8), j = (c % (R / 8)) * 8;
            const uint32_t w4[4] = {ev[i].x, ev[i].y, ev[i].z, ev[i].w};
            float *d = es + rr * RS + j;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                d[2 * q] = bf16_lo(w4[q]);
                d[2 * q + 1] = bf16_hi(w4[q]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < H_PER; ++i) {
        const int c = t + i * kRnnThreads;
        if (c < H_CH) {
            const int rr = c / (R / 4), j = (c % (R / 4)) * 4;
            *reinterpret_cast<float4 *>(hs + rr * RS + j) = hv[i];
        }
    }
#pragma unroll
    for (int i = 0; i < W_PER; ++i) {
        if constexpr (W_DIRECT) break;
        const int c = t + i * kRnnThreads;
        if (c < W_CH) {
            const int pu = c / (R / 4), j = (c % (R / 4)) * 4;  // pu = part * kRnnUnits + unit
            *reinterpret_cast<float4 *>(ws + pu * RS + j) = wv[i];
        }
    }
    // the global->shared loads are counted by vmcnt: every wave retires its own before the
    // barrier
    if constexpr (W_DIRECT) __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- pre-activations on the matrix cores (v_mfma_f32_16x16x4_f32): D[request][unit] +=
    // A[request][input] * B[input][unit], B[i][j] = weight row (unit j), column i.  Wave w
    // takes the inputs [w R/4, (w+1) R/4) in blocks of 16, where lane group g = lane / 16
    // supplies inputs 4g .. 4g+3 of the block over four steps (any order of the sum is the
    // sum).  Lane l holds D[4g + r][l % 16], r = 0..3.
    const int lane = t & 63, wave = t >> 6, m = lane & 15, g4 = 4 * (lane >> 4);
    const float *er = es + m * RS + g4, *hr = hs + m * RS + g4;
    const float *wrow = ws + m * RS + g4;  // + part * kRnnUnits * RS: weight row of unit m
    floatx4 acc_g = {0.f, 0.f, 0.f, 0.f}, acc_z = acc_g, acc_ni = acc_g, acc_nh = acc_g;
    for (int kb = wave * (R / 4); kb < (wave + 1) * (R / 4); kb += 16) {
        const float4 e = *reinterpret_cast<const float4 *>(er + kb);
        const float4 h = *reinterpret_cast<const float4 *>(hr + kb);
        float4 w[6];
#pragma unroll
        for (int part = 0; part < 6; ++part)
            w[part] = *reinterpret_cast<const float4 *>(wrow + part * kRnnUnits * RS + kb);
        const float ev4[4] = {e.x, e.y, e.z, e.w}, hv4[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const float wc[6] = {st == 0 ? w[0].x : st == 1 ? w[0].y : st == 2 ? w[0].z : w[0].w,
                                 st == 0 ? w[1].x : st == 1 ? w[1].y : st == 2 ? w[1].z : w[1].w,
                                 st == 0 ? w[2].x : st == 1 ? w[2].y : st == 2 ? w[2].z : w[2].w,
                                 st == 0 ? w[3].x : st == 1 ? w[3].y : st == 2 ? w[3].z : w[3].w,
                                 st == 0 ? w[4].x : st == 1 ? w[4].y : st == 2 ? w[4].z : w[4].w,
                                 st == 0 ? w[5].x : st == 1 ? w[5].y : st == 2 ? w[5].z : w[5].w};
            acc_g = __builtin_amdgcn_mfma_f32_16x16x4f32(ev4[st], wc[0], acc_g, 0, 0, 0);
            acc_g = __builtin_amdgcn_mfma_f32_16x16x4f32(hv4[st], wc[3], acc_g, 0, 0, 0);
            acc_z = __builtin_amdgcn_mfma_f32_16x16x4f32(ev4[st], wc[1], acc_z, 0, 0, 0);
            acc_z = __builtin_amdgcn_mfma_f32_16x16x4f32(hv4[st], wc[4], acc_z, 0, 0, 0);
            acc_ni = __builtin_amdgcn_mfma_f32_16x16x4f32(ev4[st], wc[2], acc_ni, 0, 0, 0);
            acc_nh = __builtin_amdgcn_mfma_f32_16x16x4f32(hv4[st], wc[5], acc_nh, 0, 0, 0);
        }
    }
    // the four waves' partial sums meet in shared memory, over the weights (no longer read;
    // 96 rows of at least 68 floats hold the 4 x 4 x 64 x 4 sums)
    __syncthreads();
    float *red = ws;  // [wave][4 sums][64 lanes][4]
    static_assert(6 * kRnnUnits * RS >= 4 * 4 * 64 * 4, "reduction space");
    const floatx4 accs[4] = {acc_g, acc_z, acc_ni, acc_nh};
#pragma unroll
    for (int a = 0; a < 4; ++a)
        *reinterpret_cast<floatx4 *>(red + ((wave * 4 + a) * 64 + lane) * 4) = accs[a];
    __syncthreads();
    // thread t finishes request rq = t / 16, unit u = t % 16 (held by lane 16 (rq / 4) + u,
    // element rq % 4)
    const int rq = t / kRnnUnits, u = t % kRnnUnits;
    const int src_lane = 16 * (rq / 4) + u, src_el = rq % 4;
    float pre[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        float sum = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) sum += red[((w2 * 4 + a) * 64 + src_lane) * 4 + src_el];
        pre[a] = sum;
    }
    const float a_g = pre[0], a_z = pre[1], a_ni = pre[2], a_nh = pre[3];

    const int b = row0 + rq, unit = unit0 + u;
    if (b >= B) return;
    int kb = draft_len ? draft_len[b] : K;
    kb = kb < 0 ? 0 : (kb > K ? K : kb);  // (a bad length is flagged by the reduce kernel)
    if (k >= kb) return;                   // past this request's draft
    const float g = 1.f / (1.f + expf(-(a_g + bi[unit] + bh[unit])));
    const float z = 1.f / (1.f + expf(-(a_z + bi[R + unit] + bh[R + unit])));
    const float n = tanhf(a_ni + bi[2 * R + unit] + g * (a_nh + bh[2 * R + unit]));
    const float hp = hs[rq * RS + unit];  // (zero at k = 0)
    const float hnew = (1.f - z) * n + z * hp;
    h_next[(size_t)b * R + unit] = hnew;
    const uint16_t a = f32_to_bf16(hnew);
    a_rows[(size_t)b * R + unit] = a;
    if (state_out) state_out[((size_t)b * K + k) * R + unit] = a;
}

hipError_t launch_rnn_step(const dspark_draft_args &a, const DraftWs &ws, int k, hipStream_t s) {
    if (k < 0 || k >= a.K) return hipErrorInvalidValue;
    // the state of position k lives in plane k & 1; position k - 1's in the other one
    const size_t plane = (size_t)a.B * a.r;
    const float *h_prev = k == 0 ? nullptr : ws.h_state + (size_t)((k + 1) & 1) * plane;
    float *h_next = ws.h_state + (size_t)(k & 1) * plane;
    const dim3 grid((a.B + kRnnRows - 1) / kRnnRows, a.r / kRnnUnits);
    const uint16_t *U = reinterpret_cast<const uint16_t *>(a.U);
#define DSPARK_RNN_LAUNCH(RR)                                                                  \
    rnn_step_kernel<RR><<<grid, kRnnThreads, 0, s>>>(a.B, a.K, k, a.V, U, ws.prev_cur,        \
                                                     a.draft_len, a.gru_wi, a.gru_wh,          \
                                                     a.gru_bi, a.gru_bh, h_prev, h_next,       \
                                                     ws.a_rows, a.head_state)
    switch (a.r) {
        case 64: DSPARK_RNN_LAUNCH(64); break;
        case 128: DSPARK_RNN_LAUNCH(128); break;
        case 256: DSPARK_RNN_LAUNCH(256); break;
        default: return hipErrorInvalidValue;
    }
#undef DSPARK_RNN_LAUNCH
    return hipGetLastError();
}

}  // namespace dspark
