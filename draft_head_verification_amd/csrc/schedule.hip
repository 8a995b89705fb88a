// schedule.hip -- confidence-scheduled verification length, entirely on the GPU.
//
// The drafter scores every draft position with the probability that it survives verification
// given that all earlier positions passed; their running product is the probability that the
// prefix up to that position is accepted.  Combined with a pre-measured engine throughput
// curve (tokens/s against the number of tokens in the verify batch), the scheduler picks, per
// request, how many draft tokens to send to the target: more when the engine is idle, fewer
// (low-return suffixes cut) when it is loaded, with no trip back to the host
// (QbitAI "DSpark in 10 concepts", section "Variable-length drafts and hardware-aware
// scheduling"; 10100.com commentary, section "letting the GPU decide how much to verify";
// wangjunjian.com tag page, translated abstract).
//
// Objective (the pages give its ingredients, not a formula; this is the plain reading):
// maximise expected emitted tokens per unit of verify time, E(n) * T(N(n)) / N(n), over the
// n most probable prefix items; see include/dspark.h for the exact statement.
//
// One workgroup of 1024 threads: survival products in float64, an LDS bitonic sort of up to
// 8192 (P, position, request) keys, a block prefix sum, a parallel argmax over n and an
// LDS count per request.
#include "dspark_common.hpp"

namespace dspark {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxItems = 8192;
constexpr int kSchedMaxKnots = 64;

// calibrated survival of confidence logit c at inverse temperature theta (float64)
__device__ __forceinline__ double survival(float c, double theta) {
    return 1.0 / (1.0 + exp(-theta * (double)c));
}

__device__ __forceinline__ double profile_at(const double *kt, const double *kp, int n, double N) {
    if (N <= kt[0]) return kp[0];
    if (N >= kt[n - 1]) return kp[n - 1];
    int lo = 0, hi = n - 1;  // kt[lo] <= N < kt[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (kt[mid] <= N)
            lo = mid;
        else
            hi = mid;
    }
    const double t = (N - kt[lo]) / (kt[lo + 1] - kt[lo]);
    return kp[lo] + (kp[lo + 1] - kp[lo]) * t;
}

// (key desc, id asc) is "a before b"
__device__ __forceinline__ bool sched_before(unsigned long long ka, int ia, unsigned long long kb,
                                             int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(
    int B, int K, const float *conf, const int32_t *draft_len, int n_knots,
    const double *knot_tokens, const double *knot_tps, int enabled, const double *inv_temp,
    int32_t *verify_len, double *expected_tokens, uint32_t *status) {
    __shared__ unsigned long long key[kSchedMaxItems];  // float64 bits of P (P >= 0)
    __shared__ int ids[kSchedMaxItems];                 // k * B + b; sentinel 0x7FFFFFFF
    __shared__ int len[kSchedMaxItems];                 // per-request length being built
    __shared__ double kt[kSchedMaxKnots], kp[kSchedMaxKnots];
    __shared__ double wsum[kSchedThreads / 64];
    __shared__ double best_g[kSchedThreads / 64];
    __shared__ int best_n[kSchedThreads / 64];
    __shared__ int s_ok, s_items, s_nstar;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    if (tid == 0) {
        *status = 0u;
        s_items = 0;
    }
    __syncthreads();
    for (int b = tid; b < B; b += kSchedThreads) {
        int kb = draft_len ? draft_len[b] : K;
        if (kb < 0 || kb > K) {
            atomicOr(status, DSPARK_DEV_BAD_LENGTH);
            kb = kb < 0 ? 0 : K;
        }
        len[b] = kb;  // the answer when scheduling is off
        atomicAdd(&s_items, kb);
    }
    if (enabled)
        for (int i = tid; i < n_knots; i += kSchedThreads) {
            kt[i] = knot_tokens[i];
            kp[i] = knot_tps[i];
        }
    __syncthreads();
    if (tid == 0) {
        bool ok = enabled != 0;
        if (ok) {
            for (int i = 0; i < n_knots; ++i) {
                if (!(kt[i] > 0.0) || !(kp[i] > 0.0)) ok = false;
                if (i > 0 && !(kt[i] > kt[i - 1])) ok = false;
            }
            if (!ok) atomicOr(status, DSPARK_DEV_BAD_PROFILE);
        }
        s_ok = ok ? 1 : 0;
    }
    __syncthreads();
    const int n_items = s_items;

    if (s_ok) {
        // slot b*K + k holds (P[b][k], k*B + b) for k < K_b and a sentinel otherwise;
        // "before" order = (P desc, k asc, b asc), sentinels last
        int n_slots = 1;
        while (n_slots < B * K) n_slots <<= 1;
        for (int b = tid; b < B; b += kSchedThreads) {
            const int kb = len[b];
            double run_p = 1.0;
            for (int k = 0; k < K; ++k) {
                run_p = run_p * survival(conf[(size_t)b * K + k], inv_temp ? inv_temp[k] : 1.0);
                const bool real = k < kb;
                key[b * K + k] = real ? (unsigned long long)__double_as_longlong(run_p) : 0ull;
                ids[b * K + k] = real ? k * B + b : 0x7FFFFFFF;
            }
        }
        for (int i = B * K + tid; i < n_slots; i += kSchedThreads) {
            key[i] = 0ull;
            ids[i] = 0x7FFFFFFF;
        }
        __syncthreads();
        for (int size = 2; size <= n_slots; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < n_slots; i += kSchedThreads) {
                    const int j = i ^ stride;
                    if (j > i) {
                        const unsigned long long ki = key[i], kj = key[j];
                        const int ii = ids[i], ij = ids[j];
                        const bool forward = (i & size) == 0;
                        const bool swap = forward ? sched_before(kj, ij, ki, ii)
                                                  : sched_before(ki, ii, kj, ij);
                        if (swap) {
                            key[i] = kj;
                            key[j] = ki;
                            ids[i] = ij;
                            ids[j] = ii;
                        }
                    }
                }
                __syncthreads();
            }
        }
        // thread t evaluates G(n) for n in [n0, n1), a tiling of 0..n_items; its item range
        // [n0, min(n1, n_items)) tiles the sorted items, so E(n0) = B + (sum over earlier
        // threads' item ranges)
        const int per = (n_items + 1 + kSchedThreads - 1) / kSchedThreads;
        const int n0 = min(tid * per, n_items + 1), n1 = min(n0 + per, n_items + 1);
        const int i1 = min(n1, n_items);
        double own = 0.0;
        for (int i = n0; i < i1; ++i) own += __longlong_as_double((long long)key[i]);
        double incl = own;
        for (int d = 1; d < 64; d <<= 1) {
            const double o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        double off = 0.0;
        for (int w = 0; w < wave; ++w) off += wsum[w];
        double e = (double)B + (off + (incl - own));
        double bg = -INFINITY;
        int bn = 0x7FFFFFFF;
        for (int n = n0; n < n1; ++n) {
            const double N = (double)B + (double)n;
            const double g = e * profile_at(kt, kp, n_knots, N) / N;
            if (g > bg) {
                bg = g;
                bn = n;
            }
            if (n < n_items) e += __longlong_as_double((long long)key[n]);
        }
        for (int mask = 1; mask < 64; mask <<= 1) {
            const double og = __shfl_xor(bg, mask);
            const int on = __shfl_xor(bn, mask);
            if (og > bg || (og == bg && on < bn)) {
                bg = og;
                bn = on;
            }
        }
        if (lane == 0) {
            best_g[wave] = bg;
            best_n[wave] = bn;
        }
        __syncthreads();
        if (tid == 0) {
            double g = best_g[0];
            int n = best_n[0];
            for (int w = 1; w < kSchedThreads / 64; ++w)
                if (best_g[w] > g || (best_g[w] == g && best_n[w] < n)) {
                    g = best_g[w];
                    n = best_n[w];
                }
            s_nstar = n;
        }
        for (int b = tid; b < B; b += kSchedThreads) len[b] = 0;
        __syncthreads();
        // the top n* items of each request form a prefix of its draft: count them
        const int nstar = s_nstar;
        for (int i = tid; i < nstar; i += kSchedThreads) atomicAdd(&len[ids[i] % B], 1);
        __syncthreads();
    }
    for (int b = tid; b < B; b += kSchedThreads) {
        const int L = len[b];
        verify_len[b] = L;
        if (expected_tokens) {
            double run_p = 1.0, e = 1.0;
            for (int k = 0; k < L; ++k) {
                run_p = run_p * survival(conf[(size_t)b * K + k], inv_temp ? inv_temp[k] : 1.0);
                e += run_p;
            }
            expected_tokens[b] = e;
        }
    }
}

hipError_t launch_schedule(const dspark_schedule_args &a, uint32_t *status, hipStream_t s) {
    schedule_kernel<<<1, kSchedThreads, 0, s>>>(a.B, a.K, a.conf_logits, a.draft_len, a.n_knots,
                                                 a.knot_tokens, a.knot_tps, a.enabled,
                                                 a.conf_inv_temp, a.verify_len,
                                                 a.expected_tokens, status);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Online calibration of the confidence logits (see dspark_calibrate in include/dspark.h):
// one workgroup per draft position; each thread sums the log-loss derivatives of its share of
// the requests that tested the position (float64), a fixed-order LDS tree adds them up, and
// thread 0 takes the damped Newton step.
// ---------------------------------------------------------------------------------------

constexpr int kCalThreads = 256;

__global__ __launch_bounds__(kCalThreads) void calibrate_kernel(
    int B, int K, const float *conf, const int32_t *verify_len, const int32_t *accept_len,
    double *inv_temp, double step, double ridge, uint32_t *status) {
    __shared__ double s1[kCalThreads], s2[kCalThreads];
    const int k = blockIdx.x, tid = threadIdx.x;
    if (k == 0 && tid == 0) *status = 0u;  // only workgroup 0 reports, after this clear
    __syncthreads();
    const double theta = inv_temp[k];
    double d1 = 0.0, d2 = 0.0;
    for (int b = tid; b < B; b += kCalThreads) {
        int L = verify_len[b], a = accept_len[b];
        const bool bad = L < 0 || L > K || a < 0 || a > (L < 0 ? 0 : (L > K ? K : L));
        if (bad && k == 0) atomicOr(status, DSPARK_DEV_BAD_LENGTH);
        L = L < 0 ? 0 : (L > K ? K : L);
        a = a < 0 ? 0 : (a > L ? L : a);
        if (k < L && k <= a) {  // position k was tested for request b
            const double y = k < a ? 1.0 : 0.0;
            const double c = (double)conf[(size_t)b * K + k];
            const double sg = 1.0 / (1.0 + exp(-theta * c));
            d1 += (sg - y) * c;
            d2 += sg * (1.0 - sg) * c * c;
        }
    }
    s1[tid] = d1;
    s2[tid] = d2;
    __syncthreads();
    for (int w = kCalThreads / 2; w > 0; w >>= 1) {
        if (tid < w) {
            s1[tid] += s1[tid + w];
            s2[tid] += s2[tid + w];
        }
        __syncthreads();
    }
    if (tid == 0) {
        double t = theta - step * s1[0] / (s2[0] + ridge);
        t = t < 1.0 / 64.0 ? 1.0 / 64.0 : (t > 64.0 ? 64.0 : t);
        inv_temp[k] = t;
    }
}

hipError_t launch_calibrate(const dspark_calibrate_args &a, uint32_t *status, hipStream_t s) {
    calibrate_kernel<<<a.K, kCalThreads, 0, s>>>(a.B, a.K, a.conf_logits, a.verify_len,
                                                a.accept_len, a.inv_temp, a.step, a.ridge,
                                                status);
    return hipGetLastError();
}

}  // namespace dspark
