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
//   verify_prepare   clear the status word and the residual-row counter (1 workgroup)
//   verify_rowstats  one workgroup per target row k <= L_b: streams Y once; softmax max /
//                    sum-exp of Y/T (log2 units), argmax for greedy rows, and for the bonus
//                    row of a sampled request the Gumbel-max bonus candidate
//   verify_finish    one thread per request: the accept scan, then the greedy correction /
//                    bonus, or enqueue the first rejected row for a residual draw
//   (markov_head.hip) the residual rows: recompute q_j with the Markov head on the matrix
//                    cores and take the Gumbel-max of max(0, p - q_j)
//   verify_residual_reduce  merge the residual candidates of each row -> next_token
#include "dspark_common.hpp"

namespace dspark {

constexpr int kRowThreads = 512;

__global__ __launch_bounds__(256) void verify_prepare_kernel(int B, uint32_t *status,
                                                             int32_t *n_resid, uint32_t *bound) {
    if (threadIdx.x == 0) {
        *status = 0u;
        *n_resid = 0;
    }
    for (int i = threadIdx.x; i < 2 * B; i += blockDim.x) bound[i] = 0u;
}

__device__ __forceinline__ int clamp_len(int L, int K, uint32_t *status, bool report) {
    if (L < 0 || L > K) {
        if (report) atomicOr(status, DSPARK_DEV_BAD_LENGTH);
        return L < 0 ? 0 : K;
    }
    return L;
}

// Eight consecutive logits starting at v (v % 8 == 0).
template <typename YT>
__device__ __forceinline__ void load8(const void *Y, size_t row, int V, int v, float y[8]);

template <>
__device__ __forceinline__ void load8<float>(const void *Y, size_t row, int V, int v, float y[8]) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(Y) +
                                                       row * (size_t)V + v);
    const float4 a = p[0], b = p[1];
    y[0] = a.x;
    y[1] = a.y;
    y[2] = a.z;
    y[3] = a.w;
    y[4] = b.x;
    y[5] = b.y;
    y[6] = b.z;
    y[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const void *Y, size_t row, int V, int v,
                                                float y[8]) {
    const uint4 q = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(Y) +
                                                     row * (size_t)V + v);
    y[0] = bf16_lo(q.x);
    y[1] = bf16_hi(q.x);
    y[2] = bf16_lo(q.y);
    y[3] = bf16_hi(q.y);
    y[4] = bf16_lo(q.z);
    y[5] = bf16_hi(q.z);
    y[6] = bf16_lo(q.w);
    y[7] = bf16_hi(q.w);
}

template <typename YT>
__global__ __launch_bounds__(kRowThreads) void verify_rowstats_kernel(
    int B, int K, int V, const void *Y, const int32_t *verify_len, const float *temperature,
    const uint32_t *req_id, uint32_t key0, uint32_t key1, float4 *rowstats, uint32_t *status) {
    __shared__ SampleState red[kRowThreads / 64];
    const int row = blockIdx.x;
    const int b = row / (K + 1), k = row % (K + 1);
    const int L = clamp_len(verify_len[b], K, status, threadIdx.x == 0 && k == 0);
    if (k > L) return;
    const float T = temperature[b];
    const bool greedy = !(T > 0.f);
    const bool bonus = !greedy && k == L;
    const float inv = greedy ? 1.f : kLog2e / T;
    const uint32_t req = req_id ? req_id[b] : (uint32_t)b;

    SampleState st = sample_state_init();
    for (int v = 8 * threadIdx.x; v < V; v += 8 * kRowThreads) {
        float y[8];
        load8<YT>(Y, (size_t)row, V, v, y);
        if (greedy) {
#pragma unroll
            for (int i = 0; i < 8; ++i) greedy_update(st, y[i], v + i);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float s[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = y[4 * h + i] * inv;
                lse_update4(st, s);
                if (bonus) {
                    const Philox4 ph = philox4x32_10((uint32_t)(v + 4 * h) >> 2, (uint32_t)k, req,
                                                     kStreamBonus, key0, key1);
                    gumbel_update4(st, s, ph.w, v + 4 * h);
                }
            }
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int mask = 1; mask < 64; mask <<= 1) {
        const SampleState o = shfl_xor_state(st, mask);
        merge_into(st, o, greedy);
    }
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (threadIdx.x == 0) {
        SampleState a = red[0];
        for (int w = 1; w < kRowThreads / 64; ++w)
            merge_into(a, red[w], greedy);
        float4 out;
        out.x = a.m;
        out.y = a.l;
        out.z = __int_as_float(a.idx);
        out.w = 0.f;
        rowstats[row] = out;
    }
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

template <typename YT>
__global__ __launch_bounds__(256) void verify_finish_kernel(
    int B, int K, int V, const void *Y, const int32_t *draft_tokens, const float *q_tok,
    const int32_t *verify_len, const float *temperature, const uint32_t *req_id, uint32_t key0,
    uint32_t key1, const float4 *rowstats, int32_t *accept_len, int32_t *next_token,
    float *p_tok, int32_t *n_resid, int32_t *resid_rows, uint32_t *status) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int L = clamp_len(verify_len[b], K, status, false);
    const float T = checked_temperature(temperature[b], status);
    const bool greedy = !(T > 0.f);
    const float inv = greedy ? 1.f : kLog2e / T;
    const uint32_t req = req_id ? req_id[b] : (uint32_t)b;
    const size_t rbase = (size_t)b * (K + 1);
    int a = L;
    bool rejected = false;
    for (int k = 0; k < L; ++k) {
        const int x = checked_token(draft_tokens[(size_t)b * K + k], V, status);
        const float4 rs = rowstats[rbase + k];
        bool accept;
        float p;
        if (greedy) {
            accept = (x == __float_as_int(rs.z));
            p = accept ? 1.f : 0.f;
        } else {
            const float lse2 = rs.x + fast_log2(rs.y);
            p = fast_exp2(load1<YT>(Y, (rbase + k) * (size_t)V + x) * inv - lse2);
            const Philox4 ph = philox4x32_10(0u, (uint32_t)k, req, kStreamAccept, key0, key1);
            const float u = uniform_from_word(ph.w[0]);
            accept = u * q_tok[(size_t)b * K + k] < p;
        }
        if (p_tok) p_tok[(size_t)b * K + k] = p;
        if (!accept) {
            a = k;
            rejected = true;
            break;
        }
    }
    if (p_tok)
        for (int k = a + (rejected ? 1 : 0); k < K; ++k) p_tok[(size_t)b * K + k] = 0.f;
    accept_len[b] = a;
    if (rejected && !greedy) {
        const int slot = atomicAdd(n_resid, 1);
        resid_rows[slot] = b * 128 + a;
        next_token[b] = -1;  // written by the residual reduction
    } else {
        int t = __float_as_int(rowstats[rbase + a].z);
        if (t < 0 || t >= V) {  // no finite logit in the row
            atomicOr(status, DSPARK_DEV_BAD_TOKEN);
            t = 0;
        }
        next_token[b] = t;
    }
}

__global__ __launch_bounds__(256) void verify_residual_reduce_kernel(
    int B, int V, const int32_t *n_resid, const int32_t *resid_rows, const Partial *partials,
    int n_slabs, int32_t *next_token) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (row >= *n_resid) return;
    float gr = -INFINITY, gp = -INFINITY;
    int ir = 0x7FFFFFFF, ip = 0x7FFFFFFF;
    for (int s = lane; s < n_slabs; s += 64) {
        const Partial q = partials[(size_t)row * n_slabs + s];
        if (q.g > gr || (q.g == gr && q.idx < ir)) {
            gr = q.g;
            ir = q.idx;
        }
        if (q.m > gp || (q.m == gp && q.pad < ip)) {
            gp = q.m;
            ip = q.pad;
        }
    }
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
    if (lane == 0) {
        const int b = resid_rows[row] >> 7;
        const int t = (gr > -INFINITY) ? ir : ip;
        next_token[b] = (t >= 0 && t < V) ? t : 0;
    }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------

hipError_t launch_verify_prepare(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s) {
    verify_prepare_kernel<<<1, 256, 0, s>>>(a.B, ws.status, ws.n_resid, ws.bound);
    return hipGetLastError();
}

hipError_t launch_verify_rowstats(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s) {
    const uint32_t k0 = (uint32_t)(a.seed & 0xFFFFFFFFu), k1 = (uint32_t)(a.seed >> 32);
    const dim3 grid((unsigned)a.B * (unsigned)(a.K + 1)), block(kRowThreads);
    if (a.y_dtype == DSPARK_BF16)
        verify_rowstats_kernel<uint16_t><<<grid, block, 0, s>>>(
            a.B, a.K, a.V, a.Y, a.verify_len, a.temperature, a.req_id, k0, k1, ws.rowstats,
            ws.status);
    else
        verify_rowstats_kernel<float><<<grid, block, 0, s>>>(a.B, a.K, a.V, a.Y, a.verify_len,
                                                             a.temperature, a.req_id, k0, k1,
                                                             ws.rowstats, ws.status);
    return hipGetLastError();
}

hipError_t launch_verify_finish(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t s) {
    const uint32_t k0 = (uint32_t)(a.seed & 0xFFFFFFFFu), k1 = (uint32_t)(a.seed >> 32);
    const dim3 grid((a.B + 255) / 256), block(256);
    if (a.y_dtype == DSPARK_BF16)
        verify_finish_kernel<uint16_t><<<grid, block, 0, s>>>(
            a.B, a.K, a.V, a.Y, a.draft_tokens, a.q_tok, a.verify_len, a.temperature, a.req_id,
            k0, k1, ws.rowstats, a.accept_len, a.next_token, a.p_tok, ws.n_resid, ws.resid_rows,
            ws.status);
    else
        verify_finish_kernel<float><<<grid, block, 0, s>>>(
            a.B, a.K, a.V, a.Y, a.draft_tokens, a.q_tok, a.verify_len, a.temperature, a.req_id,
            k0, k1, ws.rowstats, a.accept_len, a.next_token, a.p_tok, ws.n_resid, ws.resid_rows,
            ws.status);
    return hipGetLastError();
}

hipError_t launch_verify_residual_reduce(const dspark_verify_args &a, const VerifyWs &ws,
                                         hipStream_t s) {
    const int per_block = 4;
    verify_residual_reduce_kernel<<<(a.B + per_block - 1) / per_block, 64 * per_block, 0, s>>>(
        a.B, a.V, ws.n_resid, ws.resid_rows, ws.partials, ws.n_slabs, a.next_token);
    return hipGetLastError();
}

}  // namespace dspark
