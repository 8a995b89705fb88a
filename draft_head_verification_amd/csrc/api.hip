// api.hip -- the C ABI of libdspark.so: argument checks, workspace carving and the launch
// sequence of each call.  See include/dspark.h for the contract of every entry point.
#include <atomic>
#include <cstring>
#include <mutex>
#include <new>

#include "dspark_common.hpp"

using namespace dspark;

struct dspark_trace {
    int cap = 0, n = 0;
    hipEvent_t *start = nullptr, *stop = nullptr;
    const char **names = nullptr;
};

namespace {

constexpr int kMaxRank = 1024;
constexpr int kMaxBatch = 1 << 24;  // requests per call
constexpr int kMaxV = 1 << 30;

bool valid_dtype(int d) { return d == DSPARK_F32 || d == DSPARK_BF16; }
bool valid_sampler(int s) { return s == DSPARK_SAMPLER_TOKEN || s == DSPARK_SAMPLER_BLOCK16; }

// Records HIP events around one kernel launch when a trace is attached.
template <typename F>
hipError_t traced(dspark_trace *t, const char *name, hipStream_t s, F &&launch) {
    const bool rec = t && t->n < t->cap;
    if (rec) {
        hipError_t e = hipEventRecord(t->start[t->n], s);
        if (e != hipSuccess) return e;
    }
    hipError_t e = launch();
    if (e != hipSuccess) return e;
    if (rec) {
        e = hipEventRecord(t->stop[t->n], s);
        if (e != hipSuccess) return e;
        t->names[t->n] = name;
        ++t->n;
    }
    return hipSuccess;
}

bool check_ws(const void *ws, size_t ws_bytes, size_t need) {
    return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0 && ws_bytes >= need;
}

bool head_sizes_ok(int32_t B, int32_t K, int32_t V, int32_t r) {
    return B >= 0 && B < kMaxBatch && K >= 1 && K <= kMaxK && V >= 8 && V <= kMaxV && V % 8 == 0 && r >= 1 &&
           r <= kMaxRank;
}

// draft workspace: status | prev_cur[B] | a_rows[B][r] (bf16) | h_state[2][B][r] (f32) |
// partials[B][n_slabs]
size_t draft_layout(int32_t B, int32_t K, int32_t V, int32_t r, DraftWs *ws, char *base) {
    (void)K;
    const int ns = num_vslabs(V, B);
    size_t off = 0;
    if (ws) ws->status = reinterpret_cast<uint32_t *>(base + off);
    off += 256;
    if (ws) ws->prev_cur = reinterpret_cast<int32_t *>(base + off);
    off += align256((size_t)B * sizeof(int32_t));
    if (ws) ws->a_rows = reinterpret_cast<uint16_t *>(base + off);
    off += align256((size_t)B * r * sizeof(uint16_t));
    if (ws) ws->h_state = reinterpret_cast<float *>(base + off);
    off += align256((size_t)2 * B * r * sizeof(float));
    if (ws) ws->partials = reinterpret_cast<DraftPartial *>(base + off);
    off += align256((size_t)B * ns * sizeof(DraftPartial));
    if (ws) ws->n_slabs = ns;
    return off;
}

// verify workspace: status | n_resid | n_alive[kMaxChunks] | alive[kMaxChunks][B] |
// first_reject[B] | resid_rows[B] | rowstats[B][K+1] | row_partials[B][K+1][n_row_slabs] |
// partials[B][n_slabs]
size_t verify_layout(int32_t B, int32_t K, int32_t V, VerifyWs *ws, char *base) {
    const int ns = num_vslabs(V, B);
    const int nrs = num_row_slabs(V, B);
    const size_t rows = (size_t)B * (K + 1);
    size_t off = 0;
    if (ws) ws->status = reinterpret_cast<uint32_t *>(base + off);
    off += 256;
    if (ws) ws->n_resid = reinterpret_cast<int32_t *>(base + off);
    off += 256;
    if (ws) ws->n_alive = reinterpret_cast<int32_t *>(base + off);
    off += 256;
    if (ws) ws->alive = reinterpret_cast<int4 *>(base + off);
    off += align256((size_t)kMaxChunks * B * sizeof(int4));
    if (ws) ws->first_reject = reinterpret_cast<int32_t *>(base + off);
    off += align256((size_t)B * sizeof(int32_t));
    if (ws) ws->resid_rows = reinterpret_cast<int32_t *>(base + off);
    off += align256((size_t)B * sizeof(int32_t));
    if (ws) ws->rowstats = reinterpret_cast<float4 *>(base + off);
    off += align256(rows * sizeof(float4));
    if (ws) ws->row_partials = reinterpret_cast<Partial *>(base + off);
    off += align256(rows * nrs * sizeof(Partial));
    if (ws) ws->partials = reinterpret_cast<Partial *>(base + off);
    off += align256((size_t)B * ns * sizeof(Partial));
    if (ws) {
        ws->n_slabs = ns;
        ws->n_row_slabs = nrs;
    }
    return off;
}

}  // namespace

extern "C" {

const char *dspark_version(void) { return "dspark-mi355x 0.1 (gfx950)"; }

const char *dspark_status_string(dspark_status s) {
    // a C caller may pass any int: read the raw value, not the enumeration (whose range in
    // C++ is only that of its enumerators)
    int v = 0;
    std::memcpy(&v, &s, sizeof v < sizeof s ? sizeof v : sizeof s);
    switch (v) {
        case DSPARK_OK: return "ok";
        case DSPARK_EINVAL: return "invalid argument";
        case DSPARK_EDTYPE: return "unsupported dtype";
        case DSPARK_EWORKSPACE: return "workspace missing, misaligned or too small";
        case DSPARK_EHIP: return "HIP runtime error";
        case DSPARK_EDEVICE: return "invalid device data (see device status bits)";
        case DSPARK_ESCRATCH: return "sizes exceed the static scratch of the allocation-free call";
    }
    return "unknown status";
}

size_t dspark_draft_workspace_size(int32_t B, int32_t K, int32_t V, int32_t r) {
    if (!head_sizes_ok(B, K, V, r)) return 0;
    return draft_layout(B, K, V, r, nullptr, nullptr);
}

size_t dspark_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t r) {
    if (!head_sizes_ok(B, K, V, r)) return 0;
    return verify_layout(B, K, V, nullptr, nullptr);
}

// status word, then (scheduling on) the items' prefix products and ranks
static size_t schedule_items(int32_t B, int32_t K) {
    const long long n = (long long)B * K;
    return (size_t)(n < 8192 ? n : 8192);
}

size_t dspark_schedule_workspace_size(int32_t B, int32_t K) {
    if (B < 0 || B > 8192 || K < 1 || K > kMaxK) return 0;
    const size_t n = schedule_items(B, K);
    return 256 + align256(n * sizeof(long long)) + align256(n * sizeof(int));
}

// Host-side checks of a draft call that do not involve the workspace; DSPARK_OK to go on.
static dspark_status check_draft_args(const dspark_draft_args *a) {
    if (!a) return DSPARK_EINVAL;
    if (!head_sizes_ok(a->B, a->K, a->V, a->r)) return DSPARK_EINVAL;
    if (!valid_dtype(a->z_dtype) || !valid_dtype(a->uw_dtype)) return DSPARK_EDTYPE;
    if (!valid_sampler(a->sampler)) return DSPARK_EINVAL;
    if (a->B == 0) return DSPARK_OK;
    if (!a->Z || !a->U || !a->W || !a->prev_token || !a->temperature || !a->draft_tokens ||
        !a->q_tok || !a->q_lse)
        return DSPARK_EINVAL;
    // recurrent head: all four GRU arrays, matrix-core factors; head_state is its output
    const bool rnn = a->gru_wi || a->gru_wh || a->gru_bi || a->gru_bh;
    if (rnn && (!a->gru_wi || !a->gru_wh || !a->gru_bi || !a->gru_bh ||
                !matrix_core_factors(a->uw_dtype, a->r)))
        return DSPARK_EINVAL;
    if (a->head_state && !rnn) return DSPARK_EINVAL;
    return DSPARK_OK;
}

// The launch sequence of a draft call on a carved workspace (arguments already checked).
static dspark_status run_draft(const dspark_draft_args *a, DraftWs &w, hipStream_t s) {
    const bool rnn = a->gru_wi != nullptr;
    if (!draft_gathers_rows(*a)) w.a_rows = nullptr;
    hipError_t e = traced(a->trace, "draft_prepare", s,
                          [&] { return launch_draft_prepare(*a, w, s); });
    if (e != hipSuccess) return DSPARK_EHIP;
    // recurrent head: the state of each position is computed from the previous token (which
    // the preceding reduce step wrote) before the position's head step reads its operand
    auto rnn_step = [&](int k) {
        return traced(a->trace, "rnn_step", s, [&] { return launch_rnn_step(*a, w, k, s); });
    };
    if (rnn && rnn_step(0) != hipSuccess) return DSPARK_EHIP;
    DraftStepParams p{};
    p.B = a->B;
    p.K = a->K;
    p.V = a->V;
    p.r = a->r;
    p.Z = a->Z;
    p.U = a->U;
    p.W = a->W;
    p.draft_len = a->draft_len;
    p.temperature = a->temperature;
    p.req_id = a->req_id;
    p.key0 = (uint32_t)(a->seed & 0xFFFFFFFFu);
    p.key1 = (uint32_t)(a->seed >> 32);
    p.prev_cur = w.prev_cur;
    p.a_rows = w.a_rows;
    p.partials = w.partials;
    p.corrected = a->corrected;
    p.status = w.status;
    p.n_slabs = w.n_slabs;
    p.sampler = a->sampler;
    for (int k = 0; k < a->K; ++k) {
        p.k = k;
        e = traced(a->trace, "markov_head_step", s,
                   [&] { return launch_draft_step(p, a->z_dtype, a->uw_dtype, s); });
        if (e != hipSuccess) return DSPARK_EHIP;
        e = traced(a->trace, "draft_reduce", s, [&] { return launch_draft_reduce(*a, w, k, s); });
        if (e != hipSuccess) return DSPARK_EHIP;
        if (rnn && k + 1 < a->K && rnn_step(k + 1) != hipSuccess) return DSPARK_EHIP;
    }
    return DSPARK_OK;
}

dspark_status dspark_draft_block(const dspark_draft_args *a, void *ws, size_t ws_bytes,
                                 void *stream) {
    const dspark_status st = check_draft_args(a);
    if (st != DSPARK_OK || a->B == 0) return st;
    if (!check_ws(ws, ws_bytes, dspark_draft_workspace_size(a->B, a->K, a->V, a->r)))
        return DSPARK_EWORKSPACE;
    DraftWs w;
    draft_layout(a->B, a->K, a->V, a->r, &w, reinterpret_cast<char *>(ws));
    return run_draft(a, w, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// Allocation-free draft: the workspace is a fixed device array of this library, one copy per
// GPU, whose device address is looked up once per device (hipGetSymbolAddress) with that
// device current.  Host code only ever uses the looked-up address: the array's own name is a
// host-side stand-in, not a device address.
// ---------------------------------------------------------------------------------------

namespace {

constexpr size_t kStaticScratchBytes = DSPARK_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (nullptr on a HIP error).
void *current_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void *q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    return q;
}

}  // namespace

extern "C" {

dspark_status dspark_draft_block_static(const dspark_draft_args *a, uint32_t *device_status,
                                        void *stream) {
    const dspark_status st = check_draft_args(a);
    if (st != DSPARK_OK || a->B == 0) return st;
    if (!device_status) return DSPARK_EINVAL;
    if (dspark_draft_workspace_size(a->B, a->K, a->V, a->r) > kStaticScratchBytes)
        return DSPARK_ESCRATCH;
    char *base = reinterpret_cast<char *>(current_scratch());
    if (!base) return DSPARK_EHIP;
    DraftWs w;
    draft_layout(a->B, a->K, a->V, a->r, &w, base);
    w.status = device_status;  // the caller's word: cleared by the first kernel, read by the caller
    return run_draft(a, w, reinterpret_cast<hipStream_t>(stream));
}

dspark_status dspark_schedule(const dspark_schedule_args *a, void *ws, size_t ws_bytes,
                              void *stream) {
    if (!a) return DSPARK_EINVAL;
    if (a->B < 0 || a->B > 8192 || a->K < 1 || a->K > kMaxK) return DSPARK_EINVAL;
    if (a->B == 0) return DSPARK_OK;
    if (!a->conf_logits || !a->verify_len) return DSPARK_EINVAL;
    if (a->enabled) {
        if (!a->knot_tokens || !a->knot_tps || a->n_knots < 1 || a->n_knots > 64)
            return DSPARK_EINVAL;
        if ((long long)a->B * a->K > 8192) return DSPARK_EINVAL;
    }
    if (!check_ws(ws, ws_bytes, dspark_schedule_workspace_size(a->B, a->K)))
        return DSPARK_EWORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *base = reinterpret_cast<char *>(ws);
    uint32_t *status = reinterpret_cast<uint32_t *>(base);
    long long *key = reinterpret_cast<long long *>(base + 256);
    int *rank = reinterpret_cast<int *>(
        base + 256 + align256(schedule_items(a->B, a->K) * sizeof(long long)));
    hipError_t e = traced(a->trace, "schedule", s,
                          [&] { return launch_schedule(*a, status, key, rank, s); });
    return e == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

size_t dspark_calibrate_workspace_size(int32_t B, int32_t K) {
    if (B < 0 || K < 1 || K > kMaxK) return 0;
    return 256;
}

dspark_status dspark_calibrate(const dspark_calibrate_args *a, void *ws, size_t ws_bytes,
                               void *stream) {
    if (!a) return DSPARK_EINVAL;
    if (a->B < 0 || a->K < 1 || a->K > kMaxK) return DSPARK_EINVAL;
    if (!(a->step > 0.0 && a->step <= 1.0) || !(a->ridge > 0.0)) return DSPARK_EINVAL;
    if (a->B == 0) return DSPARK_OK;
    if (!a->conf_logits || !a->verify_len || !a->accept_len || !a->inv_temp) return DSPARK_EINVAL;
    if (!check_ws(ws, ws_bytes, dspark_calibrate_workspace_size(a->B, a->K)))
        return DSPARK_EWORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t *status = reinterpret_cast<uint32_t *>(ws);
    hipError_t e = traced(a->trace, "calibrate", s, [&] { return launch_calibrate(*a, status, s); });
    return e == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

dspark_status dspark_verify(const dspark_verify_args *a, void *ws, size_t ws_bytes, void *stream) {
    if (!a) return DSPARK_EINVAL;
    if (!head_sizes_ok(a->B, a->K, a->V, a->r)) return DSPARK_EINVAL;
    if (!valid_dtype(a->y_dtype) || !valid_dtype(a->z_dtype) || !valid_dtype(a->uw_dtype))
        return DSPARK_EDTYPE;
    if (!valid_sampler(a->sampler)) return DSPARK_EINVAL;
    if (a->B == 0) return DSPARK_OK;
    if (!a->Y || !a->draft_tokens || !a->q_tok || !a->q_lse || !a->Z || !a->U || !a->W ||
        !a->prev_token || !a->verify_len || !a->temperature || !a->accept_len || !a->next_token)
        return DSPARK_EINVAL;
    // a recurrent-head draft's operands are recomputed on the matrix-core path only
    if (a->head_state && !matrix_core_factors(a->uw_dtype, a->r)) return DSPARK_EINVAL;
    if (!check_ws(ws, ws_bytes, dspark_verify_workspace_size(a->B, a->K, a->V, a->r)))
        return DSPARK_EWORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    VerifyWs w;
    verify_layout(a->B, a->K, a->V, &w, reinterpret_cast<char *>(ws));
    hipError_t e;
    int bounds[kMaxChunks + 1];
    const int n_chunks = verify_chunks(*a, bounds);
    for (int c = 0; c < n_chunks; ++c) {
        e = traced(a->trace, "verify_rows", s, [&] { return launch_verify_rows(*a, w, c, s); });
        if (e != hipSuccess) return DSPARK_EHIP;
        if (c + 1 < n_chunks) {
            e = traced(a->trace, "verify_decide", s,
                       [&] { return launch_verify_decide(*a, w, c, s); });
            if (e != hipSuccess) return DSPARK_EHIP;
        }
    }
    e = traced(a->trace, "verify_finish", s, [&] { return launch_verify_finish(*a, w, s); });
    if (e != hipSuccess) return DSPARK_EHIP;
    e = traced(a->trace, "verify_residual", s, [&] { return launch_verify_residual(*a, w, s); });
    if (e != hipSuccess) return DSPARK_EHIP;
    e = traced(a->trace, "verify_residual_reduce", s,
               [&] { return launch_verify_residual_reduce(*a, w, s); });
    return e == hipSuccess ? DSPARK_OK : DSPARK_EHIP;
}

dspark_status dspark_pack_w(const void *w_rv, void *w_vr, int32_t r, int32_t V, int32_t dtype,
                           void *stream) {
    if (!w_rv || !w_vr || w_rv == w_vr || r < 1 || r > kMaxRank || V < 1 || V > kMaxV)
        return DSPARK_EINVAL;
    if (!valid_dtype(dtype)) return DSPARK_EDTYPE;
    return launch_pack_w(w_rv, w_vr, r, V, dtype, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
               ? DSPARK_OK
               : DSPARK_EHIP;
}

dspark_status dspark_query_device_status(const void *ws, void *stream, uint32_t *bits) {
    if (!ws) return DSPARK_EINVAL;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return DSPARK_EHIP;
    uint32_t v = 0;
    if (hipMemcpy(&v, ws, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return DSPARK_EHIP;
    if (bits) *bits = v;
    return v ? DSPARK_EDEVICE : DSPARK_OK;
}

dspark_trace *dspark_trace_create(int32_t capacity) {
    if (capacity <= 0) return nullptr;
    dspark_trace *t = new (std::nothrow) dspark_trace;
    if (!t) return nullptr;
    t->cap = capacity;
    t->start = new (std::nothrow) hipEvent_t[capacity];
    t->stop = new (std::nothrow) hipEvent_t[capacity];
    t->names = new (std::nothrow) const char *[capacity];
    if (!t->start || !t->stop || !t->names) {
        dspark_trace_destroy(t);
        return nullptr;
    }
    for (int i = 0; i < capacity; ++i) {
        t->start[i] = nullptr;
        t->stop[i] = nullptr;
    }
    for (int i = 0; i < capacity; ++i) {
        if (hipEventCreate(&t->start[i]) != hipSuccess || hipEventCreate(&t->stop[i]) != hipSuccess) {
            dspark_trace_destroy(t);
            return nullptr;
        }
    }
    return t;
}

void dspark_trace_destroy(dspark_trace *t) {
    if (!t) return;
    if (t->start)
        for (int i = 0; i < t->cap; ++i)
            if (t->start[i]) (void)hipEventDestroy(t->start[i]);
    if (t->stop)
        for (int i = 0; i < t->cap; ++i)
            if (t->stop[i]) (void)hipEventDestroy(t->stop[i]);
    delete[] t->start;
    delete[] t->stop;
    delete[] t->names;
    delete t;
}

void dspark_trace_reset(dspark_trace *t) {
    if (t) t->n = 0;
}

int32_t dspark_trace_count(const dspark_trace *t) { return t ? t->n : 0; }

dspark_status dspark_trace_get(dspark_trace *t, int32_t i, const char **kernel_name,
                               float *milliseconds) {
    if (!t || i < 0 || i >= t->n) return DSPARK_EINVAL;
    if (hipEventSynchronize(t->stop[i]) != hipSuccess) return DSPARK_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t->start[i], t->stop[i]) != hipSuccess) return DSPARK_EHIP;
    if (kernel_name) *kernel_name = t->names[i];
    if (milliseconds) *milliseconds = ms;
    return DSPARK_OK;
}

}  // extern "C"
