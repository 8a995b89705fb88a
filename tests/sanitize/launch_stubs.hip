// launch_stubs.hip -- CPU stand-ins for the library's kernel launchers, linked with api.hip in
// the host sanitizer build (tests/test_sanitize.py).  Each stand-in records its name and writes
// every byte of the workspace regions and outputs it is handed -- host memory in that build --
// so a region carved past the queried workspace size, or an output shorter than its documented
// shape, is reported by AddressSanitizer.  No HIP call is made.
#include <cstring>
#include <string>

#include "dspark_common.hpp"

namespace {
std::string g_log;
void note(const char *name) {
    g_log += name;
    g_log += ';';
}
template <typename T>
void touch(T *p, size_t n) {
    if (p && n) std::memset(static_cast<void *>(p), 0x5A, n * sizeof(T));
}
// a region the kernel only reads: every byte is read
volatile unsigned char g_sink;
template <typename T>
void read_all(const T *p, size_t n) {
    const unsigned char *c = reinterpret_cast<const unsigned char *>(p);
    unsigned char acc = 0;
    if (p)
        for (size_t i = 0; i < n * sizeof(T); ++i) acc ^= c[i];
    g_sink = acc;
}
void touch_draft(const dspark_draft_args &a, const dspark::DraftWs &ws) {
    const size_t B = (size_t)a.B, r = (size_t)a.r;
    touch(ws.status, 1);
    touch(ws.prev_cur, B);
    touch(ws.a_rows, B * r);
    touch(ws.h_state, 2 * B * r);
    touch(ws.partials, B * (size_t)ws.n_slabs);
}
void touch_verify(const dspark_verify_args &a, const dspark::VerifyWs &ws) {
    const size_t B = (size_t)a.B, rows = B * (size_t)(a.K + 1);
    touch(ws.status, 1);
    touch(ws.n_resid, 1);
    touch(ws.n_alive, (size_t)dspark::kMaxChunks);
    touch(ws.alive, (size_t)dspark::kMaxChunks * B);
    touch(ws.first_reject, B);
    touch(ws.resid_rows, B);
    touch(ws.rowstats, rows);
    touch(ws.row_partials, rows * (size_t)ws.n_row_slabs);
    touch(ws.partials, B * (size_t)ws.n_slabs);
    touch(a.accept_len, B);
    touch(a.next_token, B);
    touch(a.p_tok, B * (size_t)a.K);
}
}  // namespace

extern "C" const char *stub_log() { return g_log.c_str(); }
extern "C" void stub_reset() { g_log.clear(); }

namespace dspark {

// the library's own rules, restated for the stand-ins
bool matrix_core_factors(int uw_dtype, int r) {
    return uw_dtype == DSPARK_BF16 && (r == 64 || r == 128 || r == 256);
}
bool draft_gathers_rows(const dspark_draft_args &a) { return matrix_core_factors(a.uw_dtype, a.r); }
bool draft_uses_rnn(const dspark_draft_args &a) { return a.gru_wi != nullptr; }
int verify_chunks(const dspark_verify_args &a, int bounds[kMaxChunks + 1]) {
    // one of the library's plans (any valid plan exercises the same workspace regions)
    const int K = a.K;
    static const int edges[] = {0, 2, 5, 9, 17, 33, 65};
    int n = 0;
    bounds[0] = 0;
    for (int i = 1; i < (int)(sizeof(edges) / sizeof(edges[0])); ++i) {
        const int e = edges[i] < K + 1 ? edges[i] : K + 1;
        if (e > bounds[n]) bounds[++n] = e;
        if (e == K + 1) break;
    }
    return n;
}

hipError_t launch_draft_prepare(const dspark_draft_args &a, const DraftWs &ws, hipStream_t) {
    note("draft_prepare");
    touch_draft(a, ws);
    return hipSuccess;
}
hipError_t launch_rnn_step(const dspark_draft_args &a, const DraftWs &ws, int k, hipStream_t) {
    note("rnn_step");
    touch_draft(a, ws);
    touch(a.head_state, (size_t)a.B * a.K * a.r);
    (void)k;
    return hipSuccess;
}
hipError_t launch_draft_step(const DraftStepParams &p, int, int, hipStream_t) {
    note("markov_head_step");
    touch(p.status, 1);
    read_all(p.prev_cur, (size_t)p.B);
    read_all(p.a_rows, (size_t)p.B * p.r);
    touch(p.partials, (size_t)p.B * p.n_slabs);
    touch(p.corrected, (size_t)p.B * p.K * p.V);
    return hipSuccess;
}
hipError_t launch_draft_reduce(const dspark_draft_args &a, const DraftWs &ws, int, hipStream_t) {
    note("draft_reduce");
    touch_draft(a, ws);
    touch(a.draft_tokens, (size_t)a.B * a.K);
    touch(a.q_tok, (size_t)a.B * a.K);
    touch(a.q_lse, (size_t)a.B * a.K);
    return hipSuccess;
}
hipError_t launch_pack_w(const void *, void *w_vr, int r, int V, int dtype, hipStream_t) {
    note("pack_w");
    std::memset(w_vr, 0x5A, (size_t)r * V * (dtype == DSPARK_BF16 ? 2 : 4));
    return hipSuccess;
}
hipError_t launch_schedule(const dspark_schedule_args &a, uint32_t *status, long long *key,
                           int *rank, hipStream_t) {
    note("schedule");
    touch(status, 1);
    const size_t n = (size_t)a.B * a.K;
    if (a.enabled) {  // the ranked items: only when scheduling is on (B * K <= 8192)
        touch(key, n);
        touch(rank, n);
    }
    touch(a.verify_len, (size_t)a.B);
    touch(a.expected_tokens, (size_t)a.B);
    return hipSuccess;
}
hipError_t launch_calibrate(const dspark_calibrate_args &a, uint32_t *status, hipStream_t) {
    note("calibrate");
    touch(status, 1);
    touch(a.inv_temp, (size_t)a.K);
    return hipSuccess;
}
hipError_t launch_verify_rows(const dspark_verify_args &a, const VerifyWs &ws, int, hipStream_t) {
    note("verify_rows");
    touch_verify(a, ws);
    return hipSuccess;
}
hipError_t launch_verify_decide(const dspark_verify_args &a, const VerifyWs &ws, int,
                                hipStream_t) {
    note("verify_decide");
    touch_verify(a, ws);
    return hipSuccess;
}
hipError_t launch_verify_finish(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t) {
    note("verify_finish");
    touch_verify(a, ws);
    return hipSuccess;
}
hipError_t launch_verify_residual(const dspark_verify_args &a, const VerifyWs &ws, hipStream_t) {
    note("verify_residual");
    touch_verify(a, ws);
    return hipSuccess;
}
hipError_t launch_verify_residual_reduce(const dspark_verify_args &a, const VerifyWs &ws,
                                         hipStream_t) {
    note("verify_residual_reduce");
    touch_verify(a, ws);
    return hipSuccess;
}

}  // namespace dspark
