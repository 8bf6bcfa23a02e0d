// C ABI of the sparse LoRA linear library: argument validation and dispatch.
// Every entry point validates before enqueueing anything, so an error return
// means no device work was launched and no output was touched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <new>

#include "sl_internal.h"

namespace {

sl_status fail(sl_handle* h, sl_status s, const char* fmt, ...) {
    if (h) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        h->err = buf;
    }
    return s;
}

sl_status hip_check(sl_handle* h, hipError_t e, const char* what) {
    if (e == hipSuccess) return SL_OK;
    return fail(h, SL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define SL_REQUIRE(h, cond, ...)                                    \
    do {                                                            \
        if (!(cond)) return fail((h), SL_ERR_INVALID, __VA_ARGS__); \
    } while (0)

#define SL_HIP(h, expr, what)                          \
    do {                                               \
        sl_status _s = hip_check((h), (expr), (what)); \
        if (_s != SL_OK) return _s;                    \
    } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(sl_dtype dt) { return dt == SL_BF16 ? 2 : 4; }

// Leading-dimension rule: 16-byte rows.
bool ld_ok(int64_t ld, sl_dtype dt) { return ld > 0 && (ld * (int64_t)esize(dt)) % 16 == 0; }

sl_status check_matrix(sl_handle* h, const void* p, int64_t ld, int64_t cols, sl_dtype dt,
                       const char* name) {
    SL_REQUIRE(h, p != nullptr, "%s is NULL", name);
    SL_REQUIRE(h, aligned16(p), "%s is not 16-byte aligned", name);
    SL_REQUIRE(h, ld >= cols, "%s: leading dimension %lld < columns %lld", name, (long long)ld,
               (long long)cols);
    SL_REQUIRE(h, ld_ok(ld, dt), "%s: leading dimension %lld must give 16-byte rows", name,
               (long long)ld);
    return SL_OK;
}

#define SL_CHECK(expr)                 \
    do {                               \
        sl_status _s = (expr);         \
        if (_s != SL_OK) return _s;    \
    } while (0)

sl_status ensure_ws(sl_handle* h, size_t bytes) {
    if (bytes <= h->ws_bytes) return SL_OK;
    size_t want = bytes + (bytes >> 3) + 4096;
    if (h->ws) {
        SL_HIP(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
        SL_HIP(h, hipFree(h->ws), "hipFree");
        h->ws = nullptr;
        h->ws_bytes = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) {
        (void)hipGetLastError();
        return fail(h, SL_ERR_WORKSPACE, "workspace allocation of %zu bytes failed", want);
    }
    h->ws = p;
    h->ws_bytes = want;
    return SL_OK;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------- measurement
// Kernel classes whose launches are bracketed by HIP events on the handle's
// stream while timing is enabled.
const char* const kClassNames[] = {"gemm_bf16_nt", "gemm_bf16_nn", "gemm_f32",   "estimate",
                                   "score",        "topk",         "lora",       "swiglu",
                                   "gather",       "fill",         "token_split", "index"};
constexpr int kNumClasses = sizeof(kClassNames) / sizeof(kClassNames[0]);
enum { K_GEMM_NT, K_GEMM_NN, K_GEMM_F32, K_EST, K_SCORE, K_TOPK, K_LORA, K_SWIGLU, K_GATHER,
       K_FILL, K_SPLIT, K_INDEX };

hipEvent_t take_event(sl_handle* h) {
    if (!h->event_pool.empty()) {
        hipEvent_t e = h->event_pool.back();
        h->event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return e;
}

struct Timed {
    sl_handle* h;
    int cls;
    double flops, bytes;
    hipEvent_t a = nullptr, b = nullptr;
    Timed(sl_handle* h_, int cls_, double flops_, double bytes_)
        : h(h_), cls(cls_), flops(flops_), bytes(bytes_) {
        if (!h->timing) return;
        a = take_event(h);
        b = take_event(h);
        if (a && b) (void)hipEventRecord(a, h->stream);
    }
    ~Timed() {
        if (!h->timing || !a || !b) return;
        (void)hipEventRecord(b, h->stream);
        h->timed.push_back({cls, a, b, flops, bytes});
    }
};

double gemm_flops(const GemmProblem* p, int np) {
    double f = 0;
    for (int i = 0; i < np; ++i) f += 2.0 * (double)p[i].M * (double)p[i].N * (double)p[i].K;
    return f;
}
// Algorithmic HBM bytes of a GEMM launch: each operand element read once,
// each output element written once (read too when accumulating).
double gemm_bytes(const GemmProblem* p, int np, size_t es) {
    double b = 0;
    for (int i = 0; i < np; ++i)
        b += (double)es * ((double)p[i].M * p[i].K + (double)p[i].N * p[i].K +
                           (double)p[i].M * p[i].N * (p[i].beta ? 2 : 1));
    return b;
}

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) prev = -1;
        if (prev != dev) (void)hipSetDevice(dev);
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

sl_status check_rows(sl_handle* h, const int32_t* ctx, int64_t Tc, const int32_t* out,
                     int64_t To, int64_t T) {
    SL_REQUIRE(h, Tc >= 0 && To >= 0 && Tc + To == T, "T_c (%lld) + T_o (%lld) != T (%lld)",
               (long long)Tc, (long long)To, (long long)T);
    SL_REQUIRE(h, Tc == 0 || ctx != nullptr, "ctx_rows is NULL");
    SL_REQUIRE(h, To == 0 || out != nullptr, "out_rows is NULL");
    return SL_OK;
}

}  // namespace

extern "C" {

const char* sl_version(void) { return "sparselora-gfx950 0.1"; }

const char* sl_status_str(sl_status s) {
    switch (s) {
        case SL_OK: return "SL_OK";
        case SL_ERR_INVALID: return "SL_ERR_INVALID";
        case SL_ERR_UNSUPPORTED: return "SL_ERR_UNSUPPORTED";
        case SL_ERR_HIP: return "SL_ERR_HIP";
        case SL_ERR_WORKSPACE: return "SL_ERR_WORKSPACE";
    }
    return "SL_ERR_UNKNOWN";
}

sl_status sl_create(sl_handle** out, int device) {
    if (!out) return SL_ERR_INVALID;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) {
        (void)hipGetLastError();
        return SL_ERR_INVALID;
    }
    sl_handle* h = new (std::nothrow) sl_handle();
    if (!h) return SL_ERR_WORKSPACE;
    h->device = device;
    DeviceGuard g(device);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess) h->num_cu = prop.multiProcessorCount;
    if (hipMalloc(&h->dev_flags, 64) != hipSuccess ||
        hipMemset(h->dev_flags, 0, 64) != hipSuccess) {
        delete h;
        return SL_ERR_HIP;
    }
    *out = h;
    return SL_OK;
}

sl_status sl_destroy(sl_handle* h) {
    if (!h) return SL_ERR_INVALID;
    DeviceGuard g(h->device);
    (void)hipStreamSynchronize(h->stream);
    if (h->ws) (void)hipFree(h->ws);
    if (h->dev_flags) (void)hipFree(h->dev_flags);
    for (auto& t : h->timed) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    for (auto e : h->event_pool) (void)hipEventDestroy(e);
    delete h;
    return SL_OK;
}

sl_status sl_set_stream(sl_handle* h, void* stream) {
    if (!h) return SL_ERR_INVALID;
    h->stream = (hipStream_t)stream;
    return SL_OK;
}

sl_status sl_reserve_workspace(sl_handle* h, size_t bytes) {
    if (!h) return SL_ERR_INVALID;
    DeviceGuard g(h->device);
    return ensure_ws(h, bytes);
}

sl_status sl_sync(sl_handle* h) {
    if (!h) return SL_ERR_INVALID;
    DeviceGuard g(h->device);
    SL_HIP(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
    int flags = 0;
    SL_HIP(h, hipMemcpy(&flags, h->dev_flags, sizeof(int), hipMemcpyDeviceToHost), "hipMemcpy");
    if (flags) {
        SL_HIP(h, hipMemset(h->dev_flags, 0, sizeof(int)), "hipMemset");
        return fail(h, SL_ERR_INVALID, "token roles disagree with the given T_c / T_o");
    }
    return SL_OK;
}

const char* sl_last_error(const sl_handle* h) { return h ? h->err.c_str() : "null handle"; }

sl_status sl_timing_enable(sl_handle* h, int enable) {
    if (!h) return SL_ERR_INVALID;
    h->timing = enable != 0;
    return SL_OK;
}

sl_status sl_timing_reset(sl_handle* h) {
    if (!h) return SL_ERR_INVALID;
    DeviceGuard g(h->device);
    SL_HIP(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
    for (auto& t : h->timed) {
        h->event_pool.push_back(t.start);
        h->event_pool.push_back(t.stop);
    }
    h->timed.clear();
    return SL_OK;
}

sl_status sl_timing_query(sl_handle* h, const char* kernel_class, int64_t* launches,
                          double* total_ms, double* flops, double* bytes) {
    if (!h || !kernel_class) return SL_ERR_INVALID;
    int cls = -1;
    for (int i = 0; i < kNumClasses; ++i)
        if (std::string(kClassNames[i]) == kernel_class) cls = i;
    SL_REQUIRE(h, cls >= 0, "unknown kernel class '%s'", kernel_class);
    DeviceGuard g(h->device);
    SL_HIP(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
    int64_t n = 0;
    double ms = 0, fl = 0, by = 0;
    for (auto& t : h->timed) {
        if (t.kclass != cls) continue;
        float e = 0.f;
        SL_HIP(h, hipEventElapsedTime(&e, t.start, t.stop), "hipEventElapsedTime");
        ++n;
        ms += e;
        fl += t.flops;
        by += t.bytes;
    }
    if (launches) *launches = n;
    if (total_ms) *total_ms = ms;
    if (flops) *flops = fl;
    if (bytes) *bytes = by;
    return SL_OK;
}

const char* sl_timing_class_name(int i) {
    return (i >= 0 && i < kNumClasses) ? kClassNames[i] : nullptr;
}

// ---------------------------------------------------------------- a1
sl_status sl_token_split(sl_handle* h, const uint8_t* roles, int64_t T, int32_t* ctx_rows,
                         int64_t T_c, int32_t* out_rows, int64_t T_o) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, T >= 0 && T <= INT32_MAX, "T out of range");
    SL_REQUIRE(h, T == 0 || roles != nullptr, "roles is NULL");
    SL_CHECK(check_rows(h, ctx_rows, T_c, out_rows, T_o, T));
    if (T == 0) return SL_OK;
    DeviceGuard g(h->device);
    Timed tm(h, K_SPLIT, 0, (double)T + 4.0 * T);
    return hip_check(h, launch_token_split(roles, T, ctx_rows, T_c, out_rows, T_o, h->dev_flags,
                                           h->stream), "token_split");
}

// ---------------------------------------------------------------- a2
sl_status sl_svd_estimate(sl_handle* h, const void* x, sl_dtype xdt, int64_t ldx,
                          const int32_t* ctx_rows, int64_t T_c, int64_t D_in, const float* WA,
                          int64_t k_tot, float* xa) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, xdt == SL_BF16 || xdt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T_c >= 0 && D_in >= 1, "bad sizes");
    SL_REQUIRE(h, k_tot >= 1 && k_tot <= 128, "k_tot must be in [1, 128]");
    if (T_c == 0) return SL_OK;
    SL_REQUIRE(h, x && ctx_rows && WA && xa, "NULL pointer");
    SL_REQUIRE(h, ldx >= D_in, "ldx < D_in");
    SL_REQUIRE(h, aligned16(WA), "W_A must be 16-byte aligned");
    DeviceGuard g(h->device);
    Timed tm(h, K_EST, 2.0 * T_c * D_in * k_tot,
             (double)T_c * D_in * (xdt == SL_BF16 ? 2 : 4) + 4.0 * D_in * k_tot + 4.0 * T_c * k_tot);
    return hip_check(h, launch_stage1(x, xdt == SL_BF16, ldx, ctx_rows, T_c, D_in, WA, k_tot, xa,
                                      h->stream), "svd_estimate");
}

// ---------------------------------------------------------------- a3 + a4
sl_status sl_score_select(sl_handle* h, sl_criterion crit, const float* xa, int64_t ld_xa,
                          int64_t T_c, int64_t off0, const float* WB0, int64_t off1,
                          const float* WB1, int64_t k, int64_t C, int64_t n_rep, int64_t head_dim,
                          int64_t n_keep, float* scores, int32_t* idx) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, crit == SL_CRIT_L2 || crit == SL_CRIT_SWIGLU_L2 || crit == SL_CRIT_QK,
               "bad criterion");
    SL_REQUIRE(h, k >= 1 && k <= 64, "k must be in [1, 64]");
    SL_REQUIRE(h, C >= 1 && C <= INT32_MAX, "C out of range");
    SL_REQUIRE(h, n_keep >= 0 && n_keep <= C, "n_keep must be in [0, C]");
    SL_REQUIRE(h, T_c >= 0, "T_c < 0");
    SL_REQUIRE(h, n_keep == 0 || idx != nullptr, "idx is NULL");
    SL_REQUIRE(h, WB0 != nullptr, "WB0 is NULL");
    SL_REQUIRE(h, crit == SL_CRIT_L2 || WB1 != nullptr, "WB1 is NULL");
    SL_REQUIRE(h, T_c == 0 || xa != nullptr, "xa is NULL");
    SL_REQUIRE(h, off0 >= 0 && off0 + k <= ld_xa, "off0 + k exceeds ld_xa");
    if (crit == SL_CRIT_SWIGLU_L2) SL_REQUIRE(h, off1 >= 0 && off1 + k <= ld_xa, "off1 + k exceeds ld_xa");
    if (crit == SL_CRIT_QK) {
        SL_REQUIRE(h, n_rep >= 1 && head_dim >= 1 && C % head_dim == 0, "bad QK grouping");
        SL_REQUIRE(h, off1 >= 0 && off1 + k <= ld_xa, "off1 + k exceeds ld_xa");
    }
    DeviceGuard g(h->device);
    size_t need = 0;
    const int64_t Cq = crit == SL_CRIT_QK ? C * n_rep : 0;
    if (!scores) need += round_up((size_t)C * 4, 256);
    if (crit == SL_CRIT_QK) need += round_up((size_t)Cq * 4, 256) + round_up((size_t)C * 4, 256);
    SL_CHECK(ensure_ws(h, need));
    char* ws = (char*)h->ws;
    float* sc = scores;
    if (!sc) {
        sc = (float*)ws;
        ws += round_up((size_t)C * 4, 256);
    }
    hipError_t e;
    {
    const int nwb = crit == SL_CRIT_L2 ? 1 : 2;
    const double Cs = crit == SL_CRIT_QK ? (double)(C * n_rep + C) : (double)C * nwb;
    Timed tm(h, K_SCORE, 2.0 * T_c * k * Cs, 4.0 * T_c * (double)(nwb * k) + 4.0 * k * Cs + 4.0 * C);
    if (crit == SL_CRIT_QK) {
        float* sq = (float*)ws;
        float* sk = (float*)(ws + round_up((size_t)Cq * 4, 256));
        e = launch_ssq(0, xa, ld_xa, T_c, off0, WB0, 0, nullptr, k, Cq, sq, h->stream);
        if (e == hipSuccess) e = launch_ssq(0, xa, ld_xa, T_c, off1, WB1, 0, nullptr, k, C, sk, h->stream);
        if (e == hipSuccess) e = launch_qk_combine(sq, sk, C / head_dim, n_rep, head_dim, sc, h->stream);
    } else {
        e = launch_ssq(crit == SL_CRIT_SWIGLU_L2 ? 1 : 0, xa, ld_xa, T_c, off0, WB0, off1, WB1, k,
                       C, sc, h->stream);
    }
    }
    if (e == hipSuccess) {
        Timed tm(h, K_TOPK, 0, 4.0 * C + 4.0 * n_keep);
        e = launch_topk(sc, C, n_keep, idx, h->stream);
    }
    return hip_check(h, e, "score_select");
}

// ---------------------------------------------------------------- a5
sl_status sl_expand_gqa(sl_handle* h, const int32_t* idx_kv, int64_t n, int64_t n_rep,
                        int64_t head_dim, int32_t* idx_q) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n >= 0 && n_rep >= 1 && head_dim >= 1, "bad sizes");
    if (n == 0) return SL_OK;
    SL_REQUIRE(h, idx_kv && idx_q, "NULL pointer");
    DeviceGuard g(h->device);
    return hip_check(h, launch_expand_gqa(idx_kv, n, n_rep, head_dim, idx_q, h->stream),
                     "expand_gqa");
}

sl_status sl_stack_index(sl_handle* h, const int32_t* idx, int64_t n, int64_t C, int64_t copies,
                         int32_t* idx_out) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n >= 0 && C >= 1 && copies >= 1 && C * copies <= INT32_MAX, "bad sizes");
    if (n == 0) return SL_OK;
    SL_REQUIRE(h, idx && idx_out, "NULL pointer");
    DeviceGuard g(h->device);
    return hip_check(h, launch_stack_index(idx, n, C, copies, idx_out, h->stream), "stack_index");
}

// ---------------------------------------------------------------- a6/a7
static sl_status run_gemm(sl_handle* h, sl_dtype dt, bool nn, const GemmProblem* p, int np) {
    Timed tm(h, dt == SL_BF16 ? (nn ? K_GEMM_NN : K_GEMM_NT) : K_GEMM_F32, gemm_flops(p, np),
             gemm_bytes(p, np, esize(dt)));
    hipError_t e = dt == SL_BF16 ? launch_gemm_bf16(nn, p, np, h->stream)
                                 : launch_gemm_f32(nn, p, np, h->stream);
    return hip_check(h, e, "gemm");
}

sl_status sl_sparse_linear_fwd(sl_handle* h, sl_side side, sl_dtype dt, const void* x,
                               int64_t ldx, int64_t T, int64_t D_in, const void* W, int64_t ldw,
                               int64_t D_out, const int32_t* ctx_rows, int64_t T_c,
                               const int32_t* out_rows, int64_t T_o, const int32_t* idx,
                               int64_t n, void* y, int64_t ldy, int beta) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, side == SL_SIDE_OUT || side == SL_SIDE_IN, "bad side");
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 65535 && D_in >= 1 && D_out >= 1, "bad sizes");
    SL_CHECK(check_rows(h, ctx_rows, T_c, out_rows, T_o, T));
    const int64_t C = side == SL_SIDE_OUT ? D_out : D_in;
    SL_REQUIRE(h, n >= 0 && n <= C, "n must be in [0, C]");
    SL_REQUIRE(h, n == 0 || idx != nullptr, "idx is NULL");
    if (T == 0) return SL_OK;
    SL_CHECK(check_matrix(h, x, ldx, D_in, dt, "x"));
    SL_CHECK(check_matrix(h, y, ldy, D_out, dt, "y"));
    if (side == SL_SIDE_OUT) SL_CHECK(check_matrix(h, W, ldw, D_in, dt, "W"));
    else SL_CHECK(check_matrix(h, W, ldw, D_out, dt, "W"));
    DeviceGuard g(h->device);
    const bool nn = side == SL_SIDE_IN;
    if (n == C || T_c == 0) {
        // every channel kept (or no context rows): the dense product over all rows
        GemmProblem p = {x, ldx, nullptr, W, ldw, nullptr, y, ldy, nullptr, nullptr, T, D_out, D_in, beta};
        return run_gemm(h, dt, nn, &p, 1);
    }
    if (side == SL_SIDE_OUT) {
        // output rows dense; context rows gather the selected weight rows (N-gather)
        if (!beta && n < C) {
            Timed tm(h, K_FILL, 0, (double)T_c * (C - n) * esize(dt));
            SL_HIP(h, launch_zero_unselected(dt == SL_BF16, y, ldy, ctx_rows, T_c, idx, n, C,
                                             nullptr, h->stream), "zero_unselected");
        }
        GemmProblem p[2] = {};
        p[0] = {x, ldx, out_rows, W, ldw, nullptr, y, ldy, out_rows, nullptr, T_o, D_out, D_in, beta};
        p[1] = {x, ldx, ctx_rows, W, ldw, idx, y, ldy, ctx_rows, idx, T_c, n, D_in, beta};
        return run_gemm(h, dt, false, p, 2);
    }
    // side IN: output rows dense over all input channels; context rows use the
    // selected input channels: compact x[ctx][:, idx] then a K-gathered GEMM.
    const int64_t ldc = n > 0 ? (n + 7) / 8 * 8 : 8;
    SL_CHECK(ensure_ws(h, round_up((size_t)(T_c * ldc) * esize(dt), 256)));
    void* xc = h->ws;
    if (n > 0) {
        Timed tm(h, K_GATHER, 0, 2.0 * T_c * n * esize(dt));
        SL_HIP(h, launch_gather_cols(dt == SL_BF16, x, ldx, ctx_rows, T_c, idx, n, xc, ldc,
                                     h->stream), "gather_cols");
    }
    GemmProblem p[2] = {};
    p[0] = {x, ldx, out_rows, W, ldw, nullptr, y, ldy, out_rows, nullptr, T_o, D_out, D_in, beta};
    p[1] = {xc, ldc, nullptr, W, ldw, idx, y, ldy, ctx_rows, nullptr, T_c, D_out, n, beta};
    return run_gemm(h, dt, true, p, 2);
}

// ---------------------------------------------------------------- a10/a11
sl_status sl_sparse_linear_bwd(sl_handle* h, sl_side side, sl_dtype dt, const void* dy,
                               int64_t lddy, int64_t T, int64_t D_out, const void* W, int64_t ldw,
                               int64_t D_in, const int32_t* ctx_rows, int64_t T_c,
                               const int32_t* out_rows, int64_t T_o, const int32_t* idx,
                               int64_t n, void* dx, int64_t lddx, int beta) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, side == SL_SIDE_OUT || side == SL_SIDE_IN, "bad side");
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 65535 && D_in >= 1 && D_out >= 1, "bad sizes");
    SL_CHECK(check_rows(h, ctx_rows, T_c, out_rows, T_o, T));
    const int64_t C = side == SL_SIDE_OUT ? D_out : D_in;
    SL_REQUIRE(h, n >= 0 && n <= C, "n must be in [0, C]");
    SL_REQUIRE(h, n == 0 || idx != nullptr, "idx is NULL");
    if (T == 0) return SL_OK;
    SL_CHECK(check_matrix(h, dy, lddy, D_out, dt, "dy"));
    SL_CHECK(check_matrix(h, dx, lddx, D_in, dt, "dx"));
    if (side == SL_SIDE_OUT) SL_CHECK(check_matrix(h, W, ldw, D_in, dt, "W"));
    else SL_CHECK(check_matrix(h, W, ldw, D_out, dt, "W"));
    DeviceGuard g(h->device);
    const bool nn = side == SL_SIDE_OUT;   // dx = dy W contracts over W's rows
    if (n == C || T_c == 0) {
        GemmProblem p = {dy, lddy, nullptr, W, ldw, nullptr, dx, lddx, nullptr, nullptr, T, D_in, D_out, beta};
        return run_gemm(h, dt, nn, &p, 1);
    }
    if (side == SL_SIDE_IN) {
        // dx = dy Wt^T; context rows produce only the selected input channels
        if (!beta && n < C) {
            Timed tm(h, K_FILL, 0, (double)T_c * (C - n) * esize(dt));
            SL_HIP(h, launch_zero_unselected(dt == SL_BF16, dx, lddx, ctx_rows, T_c, idx, n, C,
                                             nullptr, h->stream), "zero_unselected");
        }
        GemmProblem p[2] = {};
        p[0] = {dy, lddy, out_rows, W, ldw, nullptr, dx, lddx, out_rows, nullptr, T_o, D_in, D_out, beta};
        p[1] = {dy, lddy, ctx_rows, W, ldw, idx, dx, lddx, ctx_rows, idx, T_c, n, D_out, beta};
        return run_gemm(h, dt, false, p, 2);
    }
    // side OUT: dx = dy W; context rows contract over the selected channels only
    const int64_t ldc = n > 0 ? (n + 7) / 8 * 8 : 8;
    SL_CHECK(ensure_ws(h, round_up((size_t)(T_c * ldc) * esize(dt), 256)));
    void* dyc = h->ws;
    if (n > 0) {
        Timed tm(h, K_GATHER, 0, 2.0 * T_c * n * esize(dt));
        SL_HIP(h, launch_gather_cols(dt == SL_BF16, dy, lddy, ctx_rows, T_c, idx, n, dyc, ldc,
                                     h->stream), "gather_cols");
    }
    GemmProblem p[2] = {};
    p[0] = {dy, lddy, out_rows, W, ldw, nullptr, dx, lddx, out_rows, nullptr, T_o, D_in, D_out, beta};
    p[1] = {dyc, ldc, nullptr, W, ldw, idx, dx, lddx, ctx_rows, nullptr, T_c, D_in, n, beta};
    return run_gemm(h, dt, true, p, 2);
}

// ---------------------------------------------------------------- a8/a12
sl_status sl_lora_fwd_bwd(sl_handle* h, int mode, sl_dtype dt, const void* x, int64_t ldx,
                          int64_t T, int64_t D_in, int64_t D_out, const void* A, const void* B,
                          int64_t r, float scale, float* xl, int64_t ldxl, void* y, int64_t ldy,
                          const void* dy, int64_t lddy, void* dx, int64_t lddx, float* dA,
                          float* dB) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, (mode & ~7) == 0 && mode != 0, "bad mode");
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, r >= 1 && r <= 64, "r must be in [1, 64]");
    SL_REQUIRE(h, T >= 0 && T <= 65535 * 32 && D_in >= 1 && D_out >= 1, "bad sizes");
    SL_REQUIRE(h, xl != nullptr && ldxl >= r, "xl is NULL or ldxl < r");
    const bool bf = dt == SL_BF16;
    if (mode & (SL_LORA_XL | SL_LORA_BWD)) {
        SL_CHECK(check_matrix(h, x, ldx, D_in, dt, "x"));
        SL_CHECK(check_matrix(h, A, D_in, D_in, dt, "A"));
    }
    if (mode & (SL_LORA_ADD | SL_LORA_BWD)) SL_REQUIRE(h, B != nullptr, "B is NULL");
    if (mode & SL_LORA_ADD) SL_CHECK(check_matrix(h, y, ldy, D_out, dt, "y"));
    if (mode & SL_LORA_BWD) {
        SL_CHECK(check_matrix(h, dy, lddy, D_out, dt, "dy"));
        SL_REQUIRE(h, dA && dB, "dA / dB is NULL");
        if (dx) SL_CHECK(check_matrix(h, dx, lddx, D_in, dt, "dx"));
    }
    DeviceGuard g(h->device);
    const double es = (double)esize(dt);
    Timed tm(h, K_LORA,
             ((mode & SL_LORA_XL) ? 2.0 * T * D_in * r : 0) + ((mode & SL_LORA_ADD) ? 2.0 * T * D_out * r : 0) +
                 ((mode & SL_LORA_BWD) ? 2.0 * T * r * (2.0 * D_out + D_in + (dx ? D_in : 0)) : 0),
             ((mode & SL_LORA_XL) ? es * T * D_in + 4.0 * T * r : 0) +
                 ((mode & SL_LORA_ADD) ? 2 * es * T * D_out + 4.0 * T * r : 0) +
                 ((mode & SL_LORA_BWD) ? es * T * (D_in + D_out) + (dx ? 2 * es * T * D_in : 0) : 0));
    if (mode & SL_LORA_XL)
        SL_HIP(h, launch_lora_xl(bf, x, ldx, T, D_in, A, D_in, r, xl, ldxl, nullptr, h->stream),
               "lora_xl");
    if (mode & SL_LORA_ADD)
        SL_HIP(h, launch_lora_add(bf, xl, ldxl, T, r, B, r, 1, D_out, scale, y, ldy, h->stream),
               "lora_add");
    if (mode & SL_LORA_BWD) {
        // workspace: B^T [r, D_out] (dt), gB [T, r] fp32, chunk partials
        const int64_t nch = T > 0 ? ceil_div(T, 256) : 1;
        const int64_t ldbt = ceil_div(D_out, 8) * 8;
        const size_t bt_bytes = round_up((size_t)(r * ldbt) * esize(dt), 256);
        const size_t gb_bytes = round_up((size_t)(T > 0 ? T : 1) * r * 4, 256);
        const int64_t ncol = D_in > D_out ? D_in : D_out;
        const size_t part_floats = (size_t)(nch * r * ncol);
        SL_CHECK(ensure_ws(h, bt_bytes + gb_bytes + part_floats * 4));
        char* ws = (char*)h->ws;
        void* Bt = ws;
        float* gB = (float*)(ws + bt_bytes);
        float* part = (float*)(ws + bt_bytes + gb_bytes);
        SL_HIP(h, launch_transpose(bf, B, r, D_out, r, Bt, ldbt, h->stream), "transpose");
        SL_HIP(h, launch_lora_xl(bf, dy, lddy, T, D_out, Bt, ldbt, r, gB, r, nullptr, h->stream),
               "lora_gB");
        SL_HIP(h, launch_outer_accum(bf, gB, r, T, r, x, ldx, D_in, scale, dA, D_in, 1, part,
                                     part_floats, h->stream), "lora_dA");
        SL_HIP(h, launch_outer_accum(bf, xl, ldxl, T, r, dy, lddy, D_out, scale, dB, 1, r, part,
                                     part_floats, h->stream), "lora_dB");
        if (dx)
            SL_HIP(h, launch_lora_add(bf, gB, r, T, r, A, 1, D_in, D_in, scale, dx, lddx, h->stream),
                   "lora_dx");
    }
    return SL_OK;
}

// ---------------------------------------------------------------- support
sl_status sl_swiglu_fwd(sl_handle* h, sl_dtype dt, const void* g, int64_t ldg, const void* u,
                        int64_t ldu, int64_t T, int64_t F, void* hout, int64_t ldh) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 65535 && F >= 1, "bad sizes");
    if (T == 0) return SL_OK;
    SL_CHECK(check_matrix(h, g, ldg, F, dt, "g"));
    SL_CHECK(check_matrix(h, u, ldu, F, dt, "u"));
    SL_CHECK(check_matrix(h, hout, ldh, F, dt, "h"));
    DeviceGuard gd(h->device);
    Timed tm(h, K_SWIGLU, 0, 3.0 * T * F * esize(dt));
    return hip_check(h, launch_swiglu_fwd(dt == SL_BF16, g, ldg, u, ldu, T, F, hout, ldh, h->stream),
                     "swiglu_fwd");
}

sl_status sl_swiglu_bwd(sl_handle* h, sl_dtype dt, const void* dh, int64_t lddh, const void* g,
                        int64_t ldg, const void* u, int64_t ldu, int64_t T, int64_t F, void* dg,
                        int64_t lddg, void* du, int64_t lddu) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 65535 && F >= 1, "bad sizes");
    if (T == 0) return SL_OK;
    SL_CHECK(check_matrix(h, dh, lddh, F, dt, "dh"));
    SL_CHECK(check_matrix(h, g, ldg, F, dt, "g"));
    SL_CHECK(check_matrix(h, u, ldu, F, dt, "u"));
    SL_CHECK(check_matrix(h, dg, lddg, F, dt, "dg"));
    SL_CHECK(check_matrix(h, du, lddu, F, dt, "du"));
    DeviceGuard gd(h->device);
    Timed tm(h, K_SWIGLU, 0, 5.0 * T * F * esize(dt));
    return hip_check(h, launch_swiglu_bwd(dt == SL_BF16, dh, lddh, g, ldg, u, ldu, T, F, dg, lddg,
                                          du, lddu, h->stream), "swiglu_bwd");
}

sl_status sl_transpose(sl_handle* h, sl_dtype dt, const void* in, int64_t ldi, int64_t rows,
                       int64_t cols, void* out, int64_t ldo) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, rows >= 0 && cols >= 0 && rows <= 65535 * 32, "bad sizes");
    if (rows == 0 || cols == 0) return SL_OK;
    SL_REQUIRE(h, in && out && ldi >= cols && ldo >= rows, "bad pointers or leading dimensions");
    DeviceGuard gd(h->device);
    return hip_check(h, launch_transpose(dt == SL_BF16, in, ldi, rows, cols, out, ldo, h->stream),
                     "transpose");
}

}  // extern "C"
