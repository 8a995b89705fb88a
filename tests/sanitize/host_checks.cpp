// host_checks.cpp -- drives every entry point of the C ABI (include/dspark.h) through api.hip
// built with host AddressSanitizer and UndefinedBehaviorSanitizer and linked against CPU
// stand-ins for the kernel launchers (launch_stubs.hip): argument rejection, workspace size
// queries at the limits, the carving of every workspace region (the stand-ins write each
// region in full, into buffers of exactly the queried size), and the launch sequence of each
// call.  Prints "host checks: N failures" and exits nonzero on any failure.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "dspark.h"

extern "C" const char *stub_log();
extern "C" void stub_reset();
namespace dspark {
int verify_chunks(const dspark_verify_args &a, int *bounds);  // the stand-ins' chunk plan
}

static int failures = 0;
#define CHECK(cond)                                                                 \
    do {                                                                            \
        if (!(cond)) {                                                              \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);    \
            ++failures;                                                             \
        }                                                                           \
    } while (0)

// A 256-byte aligned buffer of exactly n bytes (so AddressSanitizer bounds it at n).
struct Buf {
    void *p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes) : n(bytes) {
        if (posix_memalign(&p, 256, bytes ? bytes : 1) != 0) p = nullptr;
        if (p) std::memset(p, 0, bytes);
    }
    ~Buf() { std::free(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
    template <typename T>
    T *as() const { return static_cast<T *>(p); }
};

static std::string repeat(const std::string &s, int n) {
    std::string r;
    for (int i = 0; i < n; ++i) r += s;
    return r;
}

struct DraftCase {
    int B, K, V, r, z_dtype, uw_dtype;
    bool rnn, corrected;
};

static void draft_cases() {
    const DraftCase cases[] = {
        {5, 3, 64, 64, DSPARK_BF16, DSPARK_BF16, false, true},
        {3, 4, 152, 256, DSPARK_F32, DSPARK_BF16, false, false},
        {2, 2, 151936, 256, DSPARK_BF16, DSPARK_BF16, false, false},
        {4, 5, 96, 24, DSPARK_F32, DSPARK_F32, false, true},   // vector-ALU factors
        {3, 4, 128, 64, DSPARK_BF16, DSPARK_BF16, true, false},  // recurrent head
        {300, 2, 64, 128, DSPARK_BF16, DSPARK_BF16, false, false},  // two request groups
    };
    for (const DraftCase &c : cases) {
        const size_t B = c.B, K = c.K, V = c.V, r = c.r;
        const size_t ze = c.z_dtype == DSPARK_BF16 ? 2 : 4, ue = c.uw_dtype == DSPARK_BF16 ? 2 : 4;
        Buf Z(B * K * V * ze), U(V * r * ue), W(V * r * ue), prev(B * 4), dlen(B * 4), temp(B * 4),
            toks(B * K * 4), qt(B * K * 4), ql(B * K * 4), corr(c.corrected ? B * K * V * 4 : 0),
            wi(3 * r * r * 4), wh(3 * r * r * 4), bi(3 * r * 4), bh(3 * r * 4), hs(B * K * r * 2);
        dspark_draft_args a{};
        a.B = c.B; a.K = c.K; a.V = c.V; a.r = c.r;
        a.z_dtype = c.z_dtype; a.uw_dtype = c.uw_dtype;
        a.Z = Z.p; a.U = U.p; a.W = W.p;
        a.prev_token = prev.as<int32_t>(); a.draft_len = dlen.as<int32_t>();
        a.temperature = temp.as<float>();
        a.draft_tokens = toks.as<int32_t>(); a.q_tok = qt.as<float>(); a.q_lse = ql.as<float>();
        a.corrected = c.corrected ? corr.as<float>() : nullptr;
        if (c.rnn) {
            a.gru_wi = wi.as<float>(); a.gru_wh = wh.as<float>();
            a.gru_bi = bi.as<float>(); a.gru_bh = bh.as<float>();
            a.head_state = hs.as<uint16_t>();
        }
        const size_t need = dspark_draft_workspace_size(c.B, c.K, c.V, c.r);
        CHECK(need > 0 && need % 256 == 0);
        Buf ws(need);
        // workspace: missing, misaligned, one byte short
        CHECK(dspark_draft_block(&a, nullptr, need, nullptr) == DSPARK_EWORKSPACE);
        CHECK(dspark_draft_block(&a, ws.as<char>() + 8, need - 8, nullptr) == DSPARK_EWORKSPACE);
        CHECK(dspark_draft_block(&a, ws.p, need - 1, nullptr) == DSPARK_EWORKSPACE);
        for (int samp = 0; samp < 2; ++samp) {
            a.sampler = samp;
            stub_reset();
            CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_OK);
            const std::string step = std::string(c.rnn ? "rnn_step;" : "") +
                                     "markov_head_step;draft_reduce;";
            std::string want = "draft_prepare;" + repeat(step, c.K);
            if (c.rnn) want = "draft_prepare;rnn_step;" +
                              repeat("markov_head_step;draft_reduce;rnn_step;", c.K - 1) +
                              "markov_head_step;draft_reduce;";
            CHECK(want == stub_log());
        }
        a.sampler = 0;
        // each required pointer missing
        const void **req[] = {&a.Z, &a.U, &a.W, (const void **)&a.prev_token,
                              (const void **)&a.temperature};
        for (const void **f : req) {
            const void *keep = *f;
            *f = nullptr;
            CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
            *f = keep;
        }
        int32_t *keep_t = a.draft_tokens;
        a.draft_tokens = nullptr;
        CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.draft_tokens = keep_t;
        // dtype and sampler outside their sets
        a.z_dtype = 7;
        CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EDTYPE);
        a.z_dtype = c.z_dtype;
        a.sampler = 2;
        CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.sampler = -1;
        CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.sampler = 0;
        // an incomplete recurrent head, or its output without it
        if (c.rnn) {
            a.gru_bh = nullptr;
            CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
            a.gru_bh = bh.as<float>();
        } else {
            a.head_state = hs.as<uint16_t>();
            CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
            a.head_state = nullptr;
            a.gru_wi = wi.as<float>();
            CHECK(dspark_draft_block(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
            a.gru_wi = nullptr;
        }
    }
    // the recurrent head needs matrix-core factors
    {
        dspark_draft_args a{};
        a.B = 1; a.K = 1; a.V = 64; a.r = 32; a.z_dtype = DSPARK_F32; a.uw_dtype = DSPARK_BF16;
        float dummy[8] = {};
        a.Z = a.U = a.W = dummy; a.prev_token = reinterpret_cast<int32_t *>(dummy);
        a.temperature = dummy; a.draft_tokens = reinterpret_cast<int32_t *>(dummy);
        a.q_tok = a.q_lse = dummy;
        a.gru_wi = a.gru_wh = a.gru_bi = a.gru_bh = dummy;
        Buf ws(dspark_draft_workspace_size(1, 1, 64, 32));
        CHECK(dspark_draft_block(&a, ws.p, ws.n, nullptr) == DSPARK_EINVAL);
        // B = 0 launches nothing and needs nothing else
        dspark_draft_args z{};
        z.B = 0; z.K = 1; z.V = 8; z.r = 1;
        stub_reset();
        CHECK(dspark_draft_block(&z, nullptr, 0, nullptr) == DSPARK_OK);
        CHECK(std::string(stub_log()).empty());
        CHECK(dspark_draft_block(nullptr, nullptr, 0, nullptr) == DSPARK_EINVAL);
    }
}

static void size_queries() {
    // invalid sizes give 0
    CHECK(dspark_draft_workspace_size(-1, 4, 64, 64) == 0);
    CHECK(dspark_draft_workspace_size(1, 0, 64, 64) == 0);
    CHECK(dspark_draft_workspace_size(1, 65, 64, 64) == 0);
    CHECK(dspark_draft_workspace_size(1, 4, 12, 64) == 0);
    CHECK(dspark_draft_workspace_size(1, 4, 0, 64) == 0);
    CHECK(dspark_draft_workspace_size(1, 4, 64, 0) == 0);
    CHECK(dspark_draft_workspace_size(1, 4, 64, 1025) == 0);
    CHECK(dspark_verify_workspace_size(1 << 24, 4, 64, 64) == 0);
    CHECK(dspark_schedule_workspace_size(8193, 4) == 0);
    CHECK(dspark_schedule_workspace_size(1, 65) == 0);
    CHECK(dspark_calibrate_workspace_size(-1, 4) == 0);
    // extreme valid sizes: no overflow (the workspace is not monotone in B: the vocabulary
    // slabs per request shrink as request groups are added)
    const int32_t bigB[] = {1, 255, 256, 257, 8192, (1 << 24) - 1};
    for (int32_t B : bigB) {
        const size_t d = dspark_draft_workspace_size(B, 64, 1 << 30, 1024);
        const size_t v = dspark_verify_workspace_size(B, 64, 1 << 30, 1024);
        CHECK(d > 0 && d % 256 == 0 && d >= (size_t)B * 1024 * 2);  // holds the gathered rows
        CHECK(v > 0 && v % 256 == 0 && v >= (size_t)B * 65 * 16);   // holds the row statistics
    }
    // batches from 2^24 on are refused, up to the largest int32
    CHECK(dspark_draft_workspace_size(1 << 24, 4, 64, 64) == 0);
    CHECK(dspark_draft_workspace_size(0x7FFFFFFF, 64, 1 << 30, 1024) == 0);
    CHECK(dspark_verify_workspace_size(0x7FFFFFFF, 64, 1 << 30, 1024) == 0);
}

static void schedule_cases() {
    for (int enabled = 0; enabled < 2; ++enabled) {
        const int B = 100, K = 7;
        Buf conf(B * K * 4), dlen(B * 4), kt(3 * 8), kp(3 * 8), vl(B * 4), et(B * 8), th(K * 8);
        dspark_schedule_args a{};
        a.B = B; a.K = K; a.conf_logits = conf.as<float>(); a.draft_len = dlen.as<int32_t>();
        a.n_knots = 3; a.knot_tokens = kt.as<double>(); a.knot_tps = kp.as<double>();
        a.enabled = enabled; a.verify_len = vl.as<int32_t>(); a.expected_tokens = et.as<double>();
        a.conf_inv_temp = th.as<double>();
        const size_t need = dspark_schedule_workspace_size(B, K);
        Buf ws(need);
        stub_reset();
        CHECK(dspark_schedule(&a, ws.p, need, nullptr) == DSPARK_OK);
        CHECK(std::string("schedule;") == stub_log());
        CHECK(dspark_schedule(&a, ws.p, need - 1, nullptr) == DSPARK_EWORKSPACE);
        a.verify_len = nullptr;
        CHECK(dspark_schedule(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.verify_len = vl.as<int32_t>();
        if (enabled) {
            a.n_knots = 0;
            CHECK(dspark_schedule(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
            a.n_knots = 65;
            CHECK(dspark_schedule(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
            a.n_knots = 3;
            a.knot_tps = nullptr;
            CHECK(dspark_schedule(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        }
    }
    // scheduling on is limited to 8192 items; off is not
    {
        const int B = 2000, K = 64;
        Buf conf((size_t)B * K * 4), vl(B * 4), kt(8), kp(8);
        dspark_schedule_args a{};
        a.B = B; a.K = K; a.conf_logits = conf.as<float>(); a.verify_len = vl.as<int32_t>();
        a.n_knots = 1; a.knot_tokens = kt.as<double>(); a.knot_tps = kp.as<double>();
        const size_t need = dspark_schedule_workspace_size(B, K);
        Buf ws(need);
        a.enabled = 1;
        CHECK(dspark_schedule(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.enabled = 0;
        CHECK(dspark_schedule(&a, ws.p, need, nullptr) == DSPARK_OK);
    }
    dspark_schedule_args z{};
    z.B = 0; z.K = 1;
    CHECK(dspark_schedule(&z, nullptr, 0, nullptr) == DSPARK_OK);
    z.B = 8193;
    CHECK(dspark_schedule(&z, nullptr, 0, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_schedule(nullptr, nullptr, 0, nullptr) == DSPARK_EINVAL);
}

static void calibrate_cases() {
    const int B = 9, K = 5;
    Buf conf(B * K * 4), vl(B * 4), al(B * 4), th(K * 8);
    dspark_calibrate_args a{};
    a.B = B; a.K = K; a.conf_logits = conf.as<float>(); a.verify_len = vl.as<int32_t>();
    a.accept_len = al.as<int32_t>(); a.inv_temp = th.as<double>(); a.step = 0.5; a.ridge = 1e-3;
    const size_t need = dspark_calibrate_workspace_size(B, K);
    Buf ws(need);
    stub_reset();
    CHECK(dspark_calibrate(&a, ws.p, need, nullptr) == DSPARK_OK);
    CHECK(std::string("calibrate;") == stub_log());
    a.step = 0.0;
    CHECK(dspark_calibrate(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
    a.step = 1.5;
    CHECK(dspark_calibrate(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
    a.step = 0.5;
    a.ridge = -1.0;
    CHECK(dspark_calibrate(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
    a.ridge = 1e-3;
    a.inv_temp = nullptr;
    CHECK(dspark_calibrate(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_calibrate(nullptr, ws.p, need, nullptr) == DSPARK_EINVAL);
}

static void verify_cases() {
    struct VCase { int B, K, V, r, y_dtype, uw_dtype; bool state, ptok; };
    const VCase cases[] = {
        {4, 16, 64, 64, DSPARK_F32, DSPARK_BF16, false, true},
        {3, 64, 152, 256, DSPARK_BF16, DSPARK_BF16, true, false},
        {2, 1, 151936, 256, DSPARK_F32, DSPARK_BF16, false, true},
        {5, 7, 96, 24, DSPARK_F32, DSPARK_F32, false, true},
    };
    for (const VCase &c : cases) {
        const size_t B = c.B, K = c.K, V = c.V, r = c.r;
        const size_t ye = c.y_dtype == DSPARK_BF16 ? 2 : 4, ue = c.uw_dtype == DSPARK_BF16 ? 2 : 4;
        Buf Y(B * (K + 1) * V * ye), toks(B * K * 4), qt(B * K * 4), ql(B * K * 4),
            Z(B * K * V * 2), U(V * r * ue), W(V * r * ue), prev(B * 4), vl(B * 4), temp(B * 4),
            acc(B * 4), nxt(B * 4), pt(B * K * 4), hs(B * K * r * 2);
        dspark_verify_args a{};
        a.B = c.B; a.K = c.K; a.V = c.V; a.r = c.r;
        a.y_dtype = c.y_dtype; a.z_dtype = DSPARK_BF16; a.uw_dtype = c.uw_dtype;
        a.Y = Y.p; a.draft_tokens = toks.as<int32_t>(); a.q_tok = qt.as<float>();
        a.q_lse = ql.as<float>(); a.Z = Z.p; a.U = U.p; a.W = W.p;
        a.prev_token = prev.as<int32_t>(); a.verify_len = vl.as<int32_t>();
        a.temperature = temp.as<float>(); a.accept_len = acc.as<int32_t>();
        a.next_token = nxt.as<int32_t>(); a.p_tok = c.ptok ? pt.as<float>() : nullptr;
        a.head_state = c.state ? hs.as<uint16_t>() : nullptr;
        const size_t need = dspark_verify_workspace_size(c.B, c.K, c.V, c.r);
        CHECK(need > 0 && need % 256 == 0);
        Buf ws(need);
        for (int samp = 0; samp < 2; ++samp) {
            a.sampler = samp;
            stub_reset();
            CHECK(dspark_verify(&a, ws.p, need, nullptr) == DSPARK_OK);
            // one row launch per chunk of rows, a decide launch between chunks, then the tail
            int bounds[16];
            const int n = dspark::verify_chunks(a, bounds);
            std::string want;
            for (int ch = 0; ch < n; ++ch)
                want += ch + 1 < n ? "verify_rows;verify_decide;" : "verify_rows;";
            want += "verify_finish;verify_residual;verify_residual_reduce;";
            CHECK(want == stub_log());
        }
        a.sampler = 0;
        CHECK(dspark_verify(&a, ws.p, need - 1, nullptr) == DSPARK_EWORKSPACE);
        CHECK(dspark_verify(&a, ws.as<char>() + 16, need - 16, nullptr) == DSPARK_EWORKSPACE);
        const void *keep = a.Y;
        a.Y = nullptr;
        CHECK(dspark_verify(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.Y = keep;
        int32_t *keep_n = a.next_token;
        a.next_token = nullptr;
        CHECK(dspark_verify(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.next_token = keep_n;
        a.y_dtype = 3;
        CHECK(dspark_verify(&a, ws.p, need, nullptr) == DSPARK_EDTYPE);
        a.y_dtype = c.y_dtype;
        a.sampler = 5;
        CHECK(dspark_verify(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
        a.sampler = 0;
        if (c.uw_dtype == DSPARK_F32) {  // a recurrent draft needs matrix-core factors
            a.head_state = hs.as<uint16_t>();
            CHECK(dspark_verify(&a, ws.p, need, nullptr) == DSPARK_EINVAL);
            a.head_state = nullptr;
        }
    }
    dspark_verify_args z{};
    z.B = 0; z.K = 1; z.V = 8; z.r = 1;
    CHECK(dspark_verify(&z, nullptr, 0, nullptr) == DSPARK_OK);
    CHECK(dspark_verify(nullptr, nullptr, 0, nullptr) == DSPARK_EINVAL);
}

static void pack_cases() {
    const int r = 64, V = 40;
    Buf src((size_t)r * V * 2), dst((size_t)r * V * 2);
    stub_reset();
    CHECK(dspark_pack_w(src.p, dst.p, r, V, DSPARK_BF16, nullptr) == DSPARK_OK);
    CHECK(std::string("pack_w;") == stub_log());
    CHECK(dspark_pack_w(src.p, src.p, r, V, DSPARK_BF16, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_pack_w(nullptr, dst.p, r, V, DSPARK_BF16, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_pack_w(src.p, dst.p, 0, V, DSPARK_BF16, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_pack_w(src.p, dst.p, 1025, V, DSPARK_BF16, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_pack_w(src.p, dst.p, r, 0, DSPARK_BF16, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_pack_w(src.p, dst.p, r, V, 9, nullptr) == DSPARK_EDTYPE);
}

static void misc_cases(bool have_gpu) {
    const dspark_status all[] = {DSPARK_OK,        DSPARK_EINVAL, DSPARK_EDTYPE, DSPARK_EWORKSPACE,
                                 DSPARK_EHIP,      DSPARK_EDEVICE, DSPARK_ESCRATCH};
    for (dspark_status s : all) CHECK(dspark_status_string(s) && *dspark_status_string(s));
    CHECK(std::strcmp(dspark_status_string((dspark_status)-99), "unknown status") == 0);
    CHECK(dspark_version() && std::strlen(dspark_version()) > 0);
    CHECK(dspark_query_device_status(nullptr, nullptr, nullptr) == DSPARK_EINVAL);
    CHECK(dspark_trace_create(0) == nullptr);
    CHECK(dspark_trace_count(nullptr) == 0);
    dspark_trace_reset(nullptr);
    dspark_trace_destroy(nullptr);
    CHECK(dspark_trace_get(nullptr, 0, nullptr, nullptr) == DSPARK_EINVAL);
    if (!have_gpu) {
        // no device: event creation fails and the handle is released, not leaked or kept
        CHECK(dspark_trace_create(4) == nullptr);
    }
    // the allocation-free call: sizes past its static array are refused before any HIP call
    {
        dspark_draft_args a{};
        a.B = 4096; a.K = 64; a.V = 151936; a.r = 256;
        a.z_dtype = a.uw_dtype = DSPARK_BF16;
        float dummy[8] = {};
        a.Z = a.U = a.W = dummy; a.prev_token = reinterpret_cast<int32_t *>(dummy);
        a.temperature = dummy; a.draft_tokens = reinterpret_cast<int32_t *>(dummy);
        a.q_tok = a.q_lse = dummy;
        uint32_t st = 0;
        CHECK(dspark_draft_block_static(&a, &st, nullptr) == DSPARK_ESCRATCH);
        CHECK(dspark_draft_block_static(&a, nullptr, nullptr) == DSPARK_EINVAL);
        if (!have_gpu) {
            a.B = 2; a.K = 2;
            stub_reset();
            CHECK(dspark_draft_block_static(&a, &st, nullptr) == DSPARK_EHIP);
            CHECK(std::string(stub_log()).empty());
        }
    }
}

int main() {
    int n_dev = 0;
    const bool have_gpu = hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0;
    size_queries();
    draft_cases();
    schedule_cases();
    calibrate_cases();
    verify_cases();
    pack_cases();
    misc_cases(have_gpu);
    std::printf("host checks: %d failures\n", failures);
    return failures ? 1 : 0;
}
