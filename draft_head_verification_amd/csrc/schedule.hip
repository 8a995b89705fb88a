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
// Survival products in float64; every item ranked against every request's run across the
// whole GPU (a request's prefix products never increase along its draft, each factor being
// at most 1, so its items form one sorted run and an item's place in it is a binary search);
// then one workgroup takes the items in rank order, forms E(n) by a block prefix sum, takes
// the argmax over n, and counts each request's items ranked below n*.  E(n) is the float64
// rounding of the exact sum (products truncated to multiples of 2^-80, summed as 128-bit
// integers), so the parallel prefix sum gives the value a sequential one would, bit for bit;
// the profile interpolation and G(n) are evaluated with separately rounded float64 operations
// (no fused multiply-add), as written.  With scheduling off a small kernel copies the draft
// lengths and forms the expected tokens.
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
#pragma clang fp contract(off)
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

// Unsigned 128-bit integers for the exact prefix sums of E(n), in units of 2^-80.
struct U128 {
    unsigned long long lo, hi;
};

__device__ __forceinline__ U128 u128_add(U128 a, U128 b) {
    U128 r;
    r.lo = a.lo + b.lo;
    r.hi = a.hi + b.hi + (r.lo < a.lo ? 1ull : 0ull);
    return r;
}

__device__ __forceinline__ U128 u128_sub(U128 a, U128 b) {
    U128 r;
    r.lo = a.lo - b.lo;
    r.hi = a.hi - b.hi - (a.lo < b.lo ? 1ull : 0ull);
    return r;
}

// floor(p * 2^80) for p in [0, 1], from the float64 fields: p = m 2^(e - 1075) (normal) or
// m 2^-1074 (subnormal), so p 2^80 = m 2^sh with sh = e - 995 (or -994) <= 28.
__device__ __forceinline__ U128 fixed80(double p) {
    U128 r = {0ull, 0ull};
    if (!(p > 0.0)) return r;
    const unsigned long long bits = (unsigned long long)__double_as_longlong(p);
    const int ex = (int)((bits >> 52) & 0x7FF);
    unsigned long long m = bits & ((1ull << 52) - 1);
    int sh;
    if (ex == 0) {
        sh = -1074 + 80;
    } else {
        m |= 1ull << 52;
        sh = ex - 1075 + 80;
    }
    if (sh >= 0) {
        r.lo = m << sh;
        r.hi = sh == 0 ? 0ull : m >> (64 - sh);
    } else if (sh > -64) {
        r.lo = m >> (-sh);
    }
    return r;
}

// v 2^-80 rounded to the nearest float64 (ties to even).
__device__ __forceinline__ double u128_to_double_scaled(U128 v) {
    if (v.hi == 0) return ldexp(__ull2double_rn(v.lo), -80);
    const int lz = __clzll((long long)v.hi);  // 0..63
    // the value is (top + rest / 2^64) 2^(64 - lz) with top its leading 64 bits
    const unsigned long long top = lz == 0 ? v.hi : (v.hi << lz) | (v.lo >> (64 - lz));
    const unsigned long long rest = lz == 0 ? v.lo : v.lo << lz;
    unsigned long long m = top >> 11;  // 53 bits
    const unsigned long long r = top & 0x7FFull;
    const bool up = r > 0x400ull || (r == 0x400ull && (rest != 0ull || (m & 1ull)));
    m += up ? 1ull : 0ull;  // 2^53 at most: exact in float64
    return ldexp((double)m, 11 + 64 - lz - 80);
}

// "a before b": (P desc, k asc, b asc), with P as its float64 bits (P >= 0; -1 marks a slot
// past the request's draft, after every item) and t = k * B + b (unique per item)
__device__ __forceinline__ bool sched_before(long long ka, int ta, long long kb, int tb) {
    return ka > kb || (ka == kb && ta < tb);
}

// the request's draft length, clamped to [0, K] (out-of-range values are flagged by the select
// kernel)
__device__ __forceinline__ int sched_len(const int32_t *draft_len, int b, int K) {
    const int kb = draft_len ? draft_len[b] : K;
    return kb < 0 ? 0 : (kb > K ? K : kb);
}

// Ranking runs in three launches: prepare (one thread per request: its prefix products into
// key[b*K + k], rank counters cleared), rank (every item against every request's run), and
// select (one workgroup: items in rank order, the objective over n, lengths).
constexpr int kPrepThreads = 256;
constexpr int kRankThreads = 256;
constexpr int kRankRuns = 32;  // request runs staged per rank workgroup

// Workgroup g takes requests [g*R, g*R + R), R = 256 / K (K <= 64): every thread forms one
// item's survival factor, then one thread per request multiplies its factors in order.
static_assert(kMaxK <= kPrepThreads, "a request's factors fit one workgroup");
__global__ __launch_bounds__(kPrepThreads) void schedule_prepare_kernel(
    int B, int K, const float *conf, const int32_t *draft_len, const double *inv_temp,
    long long *key, int *rank) {
    __shared__ double sv[kPrepThreads];
    const int R = kPrepThreads / K;
    const int t = threadIdx.x;
    const int b0 = blockIdx.x * R;
    if (t < R * K && b0 + t / K < B)
        sv[t] = survival(conf[(size_t)(b0 + t / K) * K + t % K], inv_temp ? inv_temp[t % K] : 1.0);
    __syncthreads();
    const int b = b0 + t;
    if (t >= R || b >= B) return;
    const int kb = sched_len(draft_len, b, K);
    double run_p = 1.0;
    for (int k = 0; k < K; ++k) {
        if (k < kb) run_p = run_p * sv[t * K + k];
        key[(size_t)b * K + k] = k < kb ? __double_as_longlong(run_p) : -1ll;
        rank[(size_t)b * K + k] = 0;
    }
}

// Item i's rank is the number of items before it.  A request's items are sorted along its
// draft (P never increases, k rises; empty slots last), so those before item i form a prefix
// of each run, found by binary lifting.  Workgroup (x, y) ranks items [256x, 256x + 256)
// against the runs of requests [32y, 32y + 32), staged in LDS; the counts of all y add up.
__global__ __launch_bounds__(kRankThreads) void schedule_rank_kernel(int B, int K,
                                                                     const long long *key,
                                                                     int *rank) {
    __shared__ long long rk[kRankRuns * kMaxK];
    const int tid = threadIdx.x;
    const int r0 = blockIdx.y * kRankRuns;
    const int nr = min(kRankRuns, B - r0);
    for (int i = tid; i < nr * K; i += kRankThreads) rk[i] = key[(size_t)r0 * K + i];
    __syncthreads();
    const int n_total = B * K;
    const int i = blockIdx.x * kRankThreads + tid;
    if (i >= n_total) return;
    const long long mk = key[i];
    if (mk < 0) return;  // a slot past the draft has no rank
    const int mt = (i % K) * B + i / K;
    int top = 1;
    while (top * 2 <= K) top <<= 1;
    int lo[kRankRuns];
#pragma unroll
    for (int rr = 0; rr < kRankRuns; ++rr) lo[rr] = 0;
    for (int step = top; step > 0; step >>= 1) {
        long long km[kRankRuns];
        // (all reads of a step first, clamped inside the staged runs; bitwise logic after)
#pragma unroll
        for (int rr = 0; rr < kRankRuns; ++rr)
            km[rr] = rk[min(rr, nr - 1) * K + min(lo[rr] + step, K) - 1];
#pragma unroll
        for (int rr = 0; rr < kRankRuns; ++rr) {
            const int cand = lo[rr] + step;
            const int tm = (cand - 1) * B + r0 + rr;
            const int ok = (int)(cand <= K) & (int)(rr < nr) &
                           ((int)(km[rr] > mk) | ((int)(km[rr] == mk) & (int)(tm < mt)));
            lo[rr] += ok * step;
        }
    }
    int cnt = 0;
#pragma unroll
    for (int rr = 0; rr < kRankRuns; ++rr) cnt += lo[rr];
    if (cnt) atomicAdd(rank + i, cnt);
}

// One workgroup: validation, then (scheduling on) the items in rank order, E(n) by a block
// prefix sum, the argmax of G(n), and each request's length = its items ranked below n*.
// With scheduling off every request verifies its draft and nothing else was launched: the
// products are formed here.
__global__ __launch_bounds__(kSchedThreads) void schedule_select_kernel(
    int B, int K, const float *conf, const int32_t *draft_len, int n_knots,
    const double *knot_tokens, const double *knot_tps, int enabled, const double *inv_temp,
    const long long *key, const int *rank, int32_t *verify_len, double *expected_tokens,
    uint32_t *status) {
    __shared__ long long sorted[kSchedMaxItems];  // products in rank order
    __shared__ int ranks[kSchedMaxItems];         // rank of item b*K + k
    __shared__ double kt[kSchedMaxKnots], kp[kSchedMaxKnots];
    __shared__ unsigned long long wsum_lo[kSchedThreads / 64], wsum_hi[kSchedThreads / 64];
    __shared__ double best_g[kSchedThreads / 64];
    __shared__ int best_n[kSchedThreads / 64];
    __shared__ int s_ok, s_items, s_nstar;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // Everything that depends on no other load goes out first and is held in registers
    // across the barrier that orders the status word's reset before its flags: the draft
    // lengths, the knots and (scheduling on) the items' products and ranks.
    constexpr int kPer = kSchedMaxItems / kSchedThreads;  // B <= 8192; B*K <= 8192 when on
    int raw_len[kPer];
    long long ik[kPer];
    int ir[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int b = tid + j * kSchedThreads;
        raw_len[j] = b < B ? (draft_len ? draft_len[b] : K) : 0;
        const int i = tid + j * kSchedThreads;
        const bool has = enabled && i < B * K;
        ik[j] = has ? key[i] : -1ll;
        ir[j] = has ? rank[i] : -1;
    }
    const bool knot = enabled && tid < n_knots;
    const double ktv = knot ? knot_tokens[tid] : 0.0, kpv = knot ? knot_tps[tid] : 0.0;
    if (tid == 0) {
        *status = 0u;
        s_items = 0;
    }
    __syncthreads();
    int my_items = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int raw = raw_len[j];
        if (tid + j * kSchedThreads < B) {
            if (raw < 0 || raw > K) atomicOr(status, DSPARK_DEV_BAD_LENGTH);
            my_items += raw < 0 ? 0 : (raw > K ? K : raw);
        }
    }
    if (my_items) atomicAdd(&s_items, my_items);
    if (knot) {
        kt[tid] = ktv;
        kp[tid] = kpv;
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
        s_nstar = -1;  // no schedule: every request verifies its whole draft
    }
    __syncthreads();
    const int n_items = s_items;

    if (s_ok) {
        // ranks of the items are a permutation of 0 .. n_items - 1
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = tid + j * kSchedThreads;
            const bool item = ik[j] >= 0 && ir[j] >= 0 && ir[j] < n_items;
            if (item) sorted[ir[j]] = ik[j];
            if (i < B * K) ranks[i] = item ? ir[j] : -1;
        }
        __syncthreads();
        // thread t evaluates G(n) for n in [n0, n1), a tiling of 0..n_items; its item range
        // [n0, min(n1, n_items)) tiles the sorted items, so E(n0) = B + (sum over earlier
        // threads' item ranges)
        const int per = (n_items + 1 + kSchedThreads - 1) / kSchedThreads;
        const int n0 = min(tid * per, n_items + 1), n1 = min(n0 + per, n_items + 1);
        const int i1 = min(n1, n_items);
        U128 own = {0ull, 0ull};
        for (int i = n0; i < i1; ++i) own = u128_add(own, fixed80(__longlong_as_double(sorted[i])));
        U128 incl = own;
        for (int d = 1; d < 64; d <<= 1) {
            U128 o;
            o.lo = __shfl_up(incl.lo, d);
            o.hi = __shfl_up(incl.hi, d);
            if (lane >= d) incl = u128_add(incl, o);
        }
        if (lane == 63) {
            wsum_lo[wave] = incl.lo;
            wsum_hi[wave] = incl.hi;
        }
        __syncthreads();
        U128 e = {0ull, (unsigned long long)B << 16};  // B 2^80
        for (int w = 0; w < wave; ++w) e = u128_add(e, U128{wsum_lo[w], wsum_hi[w]});
        e = u128_add(e, u128_sub(incl, own));
        double bg = -INFINITY;
        int bn = 0x7FFFFFFF;
        for (int n = n0; n < n1; ++n) {
#pragma clang fp contract(off)
            const double N = (double)B + (double)n;
            const double g = u128_to_double_scaled(e) * profile_at(kt, kp, n_knots, N) / N;
            if (g > bg) {
                bg = g;
                bn = n;
            }
            if (n < n_items) e = u128_add(e, fixed80(__longlong_as_double(sorted[n])));
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
        __syncthreads();
    }
    // request b verifies its items ranked below n* (a prefix of its draft: ranks rise along
    // it); expected tokens add up the same float64 products that were ranked
    const int nstar = s_nstar;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int b = tid + j * kSchedThreads;
        if (b >= B) break;
        const int kb = raw_len[j] < 0 ? 0 : (raw_len[j] > K ? K : raw_len[j]);
        double run_p = 1.0, e = 1.0;
        int L = 0;
        for (int k = 0; k < kb; ++k) {
            if (s_ok) {
                const int r = ranks[b * K + k];
                if (r < 0 || r >= nstar) break;
                run_p = __longlong_as_double(sorted[r]);
            } else {  // a bad profile: the products were still formed
                run_p = __longlong_as_double(key[(size_t)b * K + k]);
            }
            L = k + 1;
            e += run_p;
        }
        verify_len[b] = L;
        if (expected_tokens) expected_tokens[b] = e;
    }
}

// Scheduling off: every request verifies its whole draft.  One thread per request, spread
// over small workgroups: its survival factors (independent, so their exponentials overlap),
// then 1 + sum_{k < L} P in draft order, as the scheduled path forms it.  Workgroup 0 alone
// writes the status word -- the OR of every request's length check, as a plain store -- so no
// workgroup clears a flag another has raised.
constexpr int kOffThreads = 64;
__global__ __launch_bounds__(kOffThreads) void schedule_off_kernel(
    int B, int K, const float *conf, const int32_t *draft_len, const double *inv_temp,
    int32_t *verify_len, double *expected_tokens, uint32_t *status) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0) {
        bool bad = false;
        if (draft_len)
            for (int b = tid; b < B; b += kOffThreads) bad |= draft_len[b] < 0 || draft_len[b] > K;
        bad = __any(bad);
        if (tid == 0) *status = bad ? DSPARK_DEV_BAD_LENGTH : 0u;
    }
    const int b = blockIdx.x * kOffThreads + tid;
    if (b >= B) return;
    const int raw = draft_len ? draft_len[b] : K;
    const int kb = raw < 0 ? 0 : (raw > K ? K : raw);
    verify_len[b] = kb;
    if (expected_tokens) {
        double run_p = 1.0, e = 1.0;
        for (int k = 0; k < kb; ++k) {
            run_p = run_p * survival(conf[(size_t)b * K + k], inv_temp ? inv_temp[k] : 1.0);
            e += run_p;
        }
        expected_tokens[b] = e;
    }
}

hipError_t launch_schedule(const dspark_schedule_args &a, uint32_t *status, long long *key,
                           int *rank, hipStream_t s) {
    if (!a.enabled) {
        schedule_off_kernel<<<(a.B + kOffThreads - 1) / kOffThreads, kOffThreads, 0, s>>>(
            a.B, a.K, a.conf_logits, a.draft_len, a.conf_inv_temp, a.verify_len,
            a.expected_tokens, status);
        return hipGetLastError();
    }
    const int per = kPrepThreads / a.K;
    schedule_prepare_kernel<<<(a.B + per - 1) / per, kPrepThreads, 0, s>>>(
        a.B, a.K, a.conf_logits, a.draft_len, a.conf_inv_temp, key, rank);
    const dim3 grid((unsigned)((a.B * a.K + kRankThreads - 1) / kRankThreads),
                    (unsigned)((a.B + kRankRuns - 1) / kRankRuns));
    schedule_rank_kernel<<<grid, kRankThreads, 0, s>>>(a.B, a.K, key, rank);
    schedule_select_kernel<<<1, kSchedThreads, 0, s>>>(
        a.B, a.K, a.conf_logits, a.draft_len, a.n_knots, a.knot_tokens, a.knot_tps, a.enabled,
        a.conf_inv_temp, key, rank, a.verify_len, a.expected_tokens, status);
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
