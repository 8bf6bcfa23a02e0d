// C ABI of the sparse LoRA linear library: argument validation and dispatch.
// Every entry point validates before enqueueing anything, so an error return
// means no device work was launched and no output was touched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <mutex>
#include <vector>
#include <new>

#include <cmath>

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
    if (h->ws_fixed)
        return fail(h, SL_ERR_WORKSPACE, "the call needs %zu bytes of workspace, above the fixed %zu", bytes,
                    h->ws_bytes);
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

// Debug mode (SL_DEBUG=1, or sl_set_option "debug"): before launching, copy a
// caller's index list to the host (after synchronising the stream) and check
// that it is strictly ascending with every entry in [0, bound).  Off by
// default: the hot path never synchronises.
sl_status debug_check_list(sl_handle* h, const int32_t* list, int64_t n, int64_t bound, const char* name) {
    if (!h->debug || n <= 0 || !list) return SL_OK;
    std::vector<int32_t> v((size_t)n);
    SL_HIP(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
    SL_HIP(h, hipMemcpy(v.data(), list, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost), "hipMemcpy");
    for (int64_t i = 0; i < n; ++i) {
        if (v[(size_t)i] < 0 || v[(size_t)i] >= bound)
            return fail(h, SL_ERR_INVALID, "%s[%lld] = %d is outside [0, %lld)", name, (long long)i, v[(size_t)i],
                        (long long)bound);
        if (i > 0 && v[(size_t)i] <= v[(size_t)i - 1])
            return fail(h, SL_ERR_INVALID, "%s is not strictly ascending at %lld (%d after %d)", name, (long long)i,
                        v[(size_t)i], v[(size_t)i - 1]);
    }
    return SL_OK;
}

int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return (e && *e) ? atoi(e) : dflt;
}

// ---------------------------------------------------------------- measurement
// Kernel classes whose launches are bracketed by HIP events on the handle's
// stream while timing is enabled.
const char* const kClassNames[] = {"gemm_bf16_nt", "gemm_bf16_nn", "gemm_f32",   "estimate",
                                   "score",        "topk",         "lora",       "swiglu",
                                   "gather",       "fill",         "token_split", "index",
                                   "splitk_reduce", "norm",        "attention"};
constexpr int kNumClasses = sizeof(kClassNames) / sizeof(kClassNames[0]);
enum { K_GEMM_NT, K_GEMM_NN, K_GEMM_F32, K_EST, K_SCORE, K_TOPK, K_LORA, K_SWIGLU, K_GATHER,
       K_FILL, K_SPLIT, K_INDEX, K_REDUCE, K_NORM, K_ATTN };

hipEvent_t take_event(sl_handle* h) {
    if (!h->event_pool.empty()) {
        hipEvent_t e = h->event_pool.back();
        h->event_pool.pop_back();
        return e;
    }
    // timing only: no system-scope fence when the event is recorded (the
    // stream is synchronised before any elapsed time is read), so the markers
    // do not add cache write-back and invalidation between the timed launches
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
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
        if (!h || !h->timing || (h->timing_cls >= 0 && h->timing_cls != cls)) return;
        a = take_event(h);
        b = take_event(h);
        if (a && b) (void)hipEventRecord(a, h->stream);
    }
    ~Timed() {
        if (!h || !h->timing || !a || !b) return;
        (void)hipEventRecord(b, h->stream);
        h->timed.push_back({cls, a, b, flops, bytes});
    }
};

double gemm_flops(const GemmProblem* p, int np) {
    double f = 0;
    for (int i = 0; i < np; ++i)
        f += 2.0 * (double)p[i].M * (double)p[i].N * (double)(p[i].k_alg ? p[i].k_alg : p[i].K);
    return f;
}
// Algorithmic HBM bytes of a GEMM launch: each operand element read once,
// each output element written once (read too when accumulating).
double gemm_bytes(const GemmProblem* p, int np, size_t es) {
    double b = 0;
    for (int i = 0; i < np; ++i) {
        const double k = (double)(p[i].k_alg ? p[i].k_alg : p[i].K);
        b += (double)es * ((double)p[i].M * k + (double)p[i].N * k +
                           (double)p[i].M * p[i].N * (p[i].beta ? 2 : 1));
    }
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

// device address of the allocation-free scratch (defined with the score selection)
sl_status scratch_init(int device);

sl_status check_rows(sl_handle* h, const int32_t* ctx, int64_t Tc, const int32_t* out,
                     int64_t To, int64_t T) {
    SL_REQUIRE(h, Tc >= 0 && To >= 0 && Tc + To == T, "T_c (%lld) + T_o (%lld) != T (%lld)",
               (long long)Tc, (long long)To, (long long)T);
    SL_REQUIRE(h, Tc == 0 || ctx != nullptr, "ctx_rows is NULL");
    SL_REQUIRE(h, To == 0 || out != nullptr, "out_rows is NULL");
    return SL_OK;
}

}  // namespace

// (k_attn.hip) bytes of the bf16 dS tiles the matrix-core attention backward keeps
size_t attn_bwd_ds_bytes(int64_t B, int64_t S, int64_t H);

// (k_select.hip)
hipError_t launch_qkv_index(const int32_t* idx_qk, int64_t n_qk, const int32_t* idx_vo, int64_t n_vo,
                            int64_t n_rep, int64_t d, int64_t Cq, int64_t Ckv, int32_t* idx_q, int32_t* idx_o,
                            int32_t* idx_qkv, hipStream_t st);

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
    // tuning knobs and debug mode: read once per handle
    h->tune.gemm_cfg = env_int("SL_GEMM_CFG", h->tune.gemm_cfg);
    h->tune.gemm_grp = env_int("SL_GEMM_GRP", h->tune.gemm_grp);
    h->tune.gemm_split = env_int("SL_GEMM_SPLIT", h->tune.gemm_split);
    h->tune.splitk_max = env_int("SL_SPLITK_MAX", h->tune.splitk_max);
    h->tune.splitk_min = env_int("SL_SPLITK_MIN", h->tune.splitk_min);
    h->tune.merge_rows = env_int("SL_MERGE_ROWS", h->tune.merge_rows);
    h->tune.lora_xl_split = env_int("SL_LORA_XL_SPLIT", h->tune.lora_xl_split);
    h->tune.swiglu_rows = env_int("SL_SWIGLU_ROWS", h->tune.swiglu_rows);
    if (h->tune.swiglu_rows < 4 || h->tune.swiglu_rows % 4 != 0) h->tune.swiglu_rows = 256;
    if (h->tune.gemm_grp < 1 || h->tune.gemm_grp > 64) h->tune.gemm_grp = 8;
    if (h->tune.splitk_max < 1 || h->tune.splitk_max > 16) h->tune.splitk_max = 4;
    if (h->tune.splitk_min < 2 || h->tune.splitk_min > 16) h->tune.splitk_min = 2;
    if (h->tune.merge_rows != 16 && h->tune.merge_rows != 32) h->tune.merge_rows = 64;
    h->debug = env_int("SL_DEBUG", 0) != 0;
    DeviceGuard g(device);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess) h->num_cu = prop.multiProcessorCount;
    if (hipMalloc(&h->dev_flags, 64) != hipSuccess ||
        hipMemset(h->dev_flags, 0, 64) != hipSuccess) {
        delete h;
        return SL_ERR_HIP;
    }
    // the device address of this device's allocation-free scratch (once per device)
    if (scratch_init(device) != SL_OK) {
        (void)hipFree(h->dev_flags);
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
    if (h->gws) (void)hipFree(h->gws);
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

sl_status sl_set_option(sl_handle* h, const char* name, int64_t value) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, name != nullptr, "option name is NULL");
    const std::string n(name);
    if (n == "gemm_cfg") h->tune.gemm_cfg = (int)value;
    else if (n == "gemm_grp") {
        SL_REQUIRE(h, value >= 1 && value <= 64, "gemm_grp must be in [1, 64]");
        h->tune.gemm_grp = (int)value;
    } else if (n == "gemm_split") h->tune.gemm_split = (int)value;
    else if (n == "splitk_max") {
        SL_REQUIRE(h, value >= 1 && value <= 16, "splitk_max must be in [1, 16]");
        h->tune.splitk_max = (int)value;
    } else if (n == "splitk_min") {
        SL_REQUIRE(h, value >= 2 && value <= 16, "splitk_min must be in [2, 16]");
        h->tune.splitk_min = (int)value;
    } else if (n == "merge_rows") {
        SL_REQUIRE(h, value == 16 || value == 32 || value == 64, "merge_rows must be 16, 32 or 64");
        h->tune.merge_rows = (int)value;
    }
    else if (n == "lora_xl_split") h->tune.lora_xl_split = (int)value;
    else if (n == "swiglu_rows") {
        SL_REQUIRE(h, value >= 4 && value <= 65536 && value % 4 == 0, "swiglu_rows must be a multiple of 4 in [4, 65536]");
        h->tune.swiglu_rows = (int)value;
    }
    else if (n == "workspace_fixed") h->ws_fixed = value != 0;
    else if (n == "debug") h->debug = value != 0;
    else return fail(h, SL_ERR_INVALID, "unknown option '%s'", name);
    return SL_OK;
}

sl_status sl_workspace_bytes(sl_handle* h, size_t* bytes) {
    if (!h || !bytes) return SL_ERR_INVALID;
    *bytes = h->ws_bytes + h->gws_bytes;
    return SL_OK;
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

sl_status sl_timing_only(sl_handle* h, const char* kernel_class) {
    if (!h) return SL_ERR_INVALID;
    int cls = -1;
    if (kernel_class && *kernel_class) {
        for (int i = 0; i < kNumClasses; ++i)
            if (std::string(kClassNames[i]) == kernel_class) cls = i;
        SL_REQUIRE(h, cls >= 0, "unknown kernel class '%s'", kernel_class);
    }
    h->timing_cls = cls;
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
    SL_REQUIRE(h, k_tot >= 1 && k_tot <= 65535 * 16, "k_tot must be in [1, 65535 * 16]");
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
}  // extern "C"

namespace {

// Bytes of scratch score selection needs for these sizes (scores kept in the
// workspace when the caller passes none, the QK criterion's two ssq vectors,
// the chain partials of the split scoring form).
size_t score_select_ws_bytes(sl_criterion crit, int64_t k, int64_t C, int64_t n_rep, bool scores_given) {
    size_t need = 0;
    const int64_t Cq = crit == SL_CRIT_QK ? C * n_rep : 0;
    if (!scores_given) need += round_up((size_t)C * 4, 256);
    if (crit == SL_CRIT_QK) need += round_up((size_t)Cq * 4, 256) + round_up((size_t)C * 4, 256);
    const int64_t Cmax = crit == SL_CRIT_QK ? Cq : C;
    const bool split = k == 16 && (C < SSQ_SPLIT_C || Cq < SSQ_SPLIT_C);
    if (split) need += round_up((size_t)64 * (Cmax < SSQ_SPLIT_C ? Cmax : C) * 4, 256);
    return need;
}

sl_status score_select_check(sl_handle* h, sl_criterion crit, const float* xa, int64_t ld_xa, int64_t T_c,
                             int64_t off0, const float* WB0, int64_t off1, const float* WB1, int64_t k,
                             int64_t C, int64_t n_rep, int64_t head_dim, int64_t n_keep, int32_t* idx) {
    SL_REQUIRE(h, crit == SL_CRIT_L2 || crit == SL_CRIT_SWIGLU_L2 || crit == SL_CRIT_QK,
               "bad criterion");
    SL_REQUIRE(h, k >= 1 && k <= 65536, "k must be in [1, 65536]");
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
        SL_REQUIRE(h, C * n_rep <= INT32_MAX, "C * n_rep out of range");
    }
    return SL_OK;
}

// Score and select with the scratch at ws (score_select_ws_bytes of it).
// timed: bracket the launches with the handle's timing events.
sl_status score_select_run(sl_handle* h, sl_criterion crit, const float* xa, int64_t ld_xa, int64_t T_c,
                           int64_t off0, const float* WB0, int64_t off1, const float* WB1, int64_t k,
                           int64_t C, int64_t n_rep, int64_t head_dim, int64_t n_keep, float* scores,
                           int32_t* idx, char* ws, bool timed) {
    const int64_t Cq = crit == SL_CRIT_QK ? C * n_rep : 0;
    const int64_t Cmax = crit == SL_CRIT_QK ? Cq : C;
    const bool split = k == 16 && (C < SSQ_SPLIT_C || Cq < SSQ_SPLIT_C);
    const size_t part_bytes = split ? round_up((size_t)64 * (Cmax < SSQ_SPLIT_C ? Cmax : C) * 4, 256) : 0;
    float* part = split ? (float*)ws : nullptr;
    ws += part_bytes;
    float* sc = scores;
    if (!sc) {
        sc = (float*)ws;
        ws += round_up((size_t)C * 4, 256);
    }
    hipError_t e;
    {
    const int nwb = crit == SL_CRIT_L2 ? 1 : 2;
    const double Cs = crit == SL_CRIT_QK ? (double)(C * n_rep + C) : (double)C * nwb;
    sl_handle* th = timed ? h : nullptr;
    Timed tm(th, K_SCORE, 2.0 * T_c * k * Cs, 4.0 * T_c * (double)(nwb * k) + 4.0 * k * Cs + 4.0 * C);
    if (crit == SL_CRIT_QK) {
        float* sq = (float*)ws;
        float* sk = (float*)(ws + round_up((size_t)Cq * 4, 256));
        e = launch_ssq(0, xa, ld_xa, T_c, off0, WB0, 0, nullptr, k, Cq, sq, h->stream,
                       Cq < SSQ_SPLIT_C ? part : nullptr);
        if (e == hipSuccess)
            e = launch_ssq(0, xa, ld_xa, T_c, off1, WB1, 0, nullptr, k, C, sk, h->stream,
                           C < SSQ_SPLIT_C ? part : nullptr);
        if (e == hipSuccess) e = launch_qk_combine(sq, sk, C / head_dim, n_rep, head_dim, sc, h->stream);
    } else {
        e = launch_ssq(crit == SL_CRIT_SWIGLU_L2 ? 1 : 0, xa, ld_xa, T_c, off0, WB0, off1, WB1, k,
                       C, sc, h->stream, C < SSQ_SPLIT_C ? part : nullptr);
    }
    }
    if (e == hipSuccess) {
        Timed tm(timed ? h : nullptr, K_TOPK, 0, 4.0 * C + 4.0 * n_keep);
        e = launch_topk(sc, C, n_keep, idx, h->stream);
    }
    return hip_check(h, e, "score_select");
}

// ---------------------------------------------------------------- allocation-free scratch
// Device memory of the allocation-free entry points: one array per device
// (each device that loads the library holds its own copy until the process
// ends).  Host code never uses the array's name as an address: its device
// address comes from hipGetSymbolAddress, once per device, at sl_create.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// with `device` current
sl_status scratch_init(int device) {
    if (device < 0 || device >= kMaxDevices) return SL_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[device]) return SL_OK;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return SL_ERR_HIP;
    }
    g_scratch_ptr[device] = p;
    return SL_OK;
}

void* scratch_ptr(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    return g_scratch_ptr[device];
}

}  // namespace

extern "C" {

sl_status sl_score_select(sl_handle* h, sl_criterion crit, const float* xa, int64_t ld_xa,
                          int64_t T_c, int64_t off0, const float* WB0, int64_t off1,
                          const float* WB1, int64_t k, int64_t C, int64_t n_rep, int64_t head_dim,
                          int64_t n_keep, float* scores, int32_t* idx) {
    if (!h) return SL_ERR_INVALID;
    SL_CHECK(score_select_check(h, crit, xa, ld_xa, T_c, off0, WB0, off1, WB1, k, C, n_rep, head_dim,
                                n_keep, idx));
    DeviceGuard g(h->device);
    SL_CHECK(ensure_ws(h, score_select_ws_bytes(crit, k, C, n_rep, scores != nullptr)));
    return score_select_run(h, crit, xa, ld_xa, T_c, off0, WB0, off1, WB1, k, C, n_rep, head_dim, n_keep,
                            scores, idx, (char*)h->ws, true);
}

sl_status sl_score_select_noalloc(sl_handle* h, sl_criterion crit, const float* xa, int64_t ld_xa,
                                  int64_t T_c, int64_t off0, const float* WB0, int64_t off1,
                                  const float* WB1, int64_t k, int64_t C, int64_t n_rep,
                                  int64_t head_dim, int64_t n_keep, float* scores, int32_t* idx) {
    if (!h) return SL_ERR_INVALID;
    SL_CHECK(score_select_check(h, crit, xa, ld_xa, T_c, off0, WB0, off1, WB1, k, C, n_rep, head_dim,
                                n_keep, idx));
    const size_t need = score_select_ws_bytes(crit, k, C, n_rep, scores != nullptr);
    if (need > kNoAllocScratchBytes)
        return fail(h, SL_ERR_WORKSPACE, "sl_score_select_noalloc needs %zu bytes of scratch, above its fixed %zu",
                    need, kNoAllocScratchBytes);
    char* ws = (char*)scratch_ptr(h->device);
    if (!ws) return fail(h, SL_ERR_HIP, "the allocation-free scratch of device %d is not set up", h->device);
    DeviceGuard g(h->device);
    return score_select_run(h, crit, xa, ld_xa, T_c, off0, WB0, off1, WB1, k, C, n_rep, head_dim, n_keep,
                            scores, idx, ws, false);
}

// ---------------------------------------------------------------- criterion variants
sl_status sl_select_top(sl_handle* h, const float* scores, int64_t C, int64_t n_keep, int32_t* idx) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, C >= 1 && C <= INT32_MAX, "C out of range");
    SL_REQUIRE(h, n_keep >= 0 && n_keep <= C, "n_keep must be in [0, C]");
    if (n_keep == 0) return SL_OK;
    SL_REQUIRE(h, scores && idx, "NULL pointer");
    DeviceGuard g(h->device);
    Timed tm(h, K_TOPK, 0, 4.0 * C + 4.0 * n_keep);
    return hip_check(h, launch_topk(scores, C, n_keep, idx, h->stream), "select_top");
}

sl_status sl_random_scores(sl_handle* h, uint64_t seed, int64_t C, float* scores) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, C >= 0 && C <= INT32_MAX, "C out of range");
    if (C == 0) return SL_OK;
    SL_REQUIRE(h, scores != nullptr, "NULL pointer");
    DeviceGuard g(h->device);
    Timed tm(h, K_SCORE, 0, 4.0 * C);
    return hip_check(h, launch_random_scores(seed, C, scores, h->stream), "random_scores");
}

sl_status sl_dense_scores(sl_handle* h, sl_criterion crit, sl_dtype dt, const void* Y0, int64_t ld0,
                          const void* Y1, int64_t ld1, const int32_t* rows, int64_t T_c, int64_t C,
                          int64_t n_rep, int64_t head_dim, float* scores) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, crit == SL_CRIT_L2 || crit == SL_CRIT_SWIGLU_L2 || crit == SL_CRIT_QK,
               "bad criterion");
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, C >= 1 && C <= INT32_MAX && T_c >= 0, "bad sizes");
    SL_REQUIRE(h, scores != nullptr && (T_c == 0 || rows != nullptr), "NULL pointer");
    const int64_t Cq = crit == SL_CRIT_QK ? C * n_rep : 0;
    if (crit == SL_CRIT_QK)
        SL_REQUIRE(h, n_rep >= 1 && head_dim >= 1 && C % head_dim == 0, "bad QK grouping");
    if (T_c > 0) {
        SL_REQUIRE(h, Y0 != nullptr && (crit == SL_CRIT_L2 || Y1 != nullptr), "NULL pointer");
        SL_REQUIRE(h, ld0 >= (crit == SL_CRIT_QK ? Cq : C), "ld0 too small");
        if (crit != SL_CRIT_L2) SL_REQUIRE(h, ld1 >= C, "ld1 too small");
    }
    DeviceGuard g(h->device);
    const int64_t Cmax = crit == SL_CRIT_QK ? Cq : C;
    const size_t part_bytes = round_up((size_t)64 * Cmax * 4, 256);
    const size_t qk_bytes = crit == SL_CRIT_QK ? round_up((size_t)Cq * 4, 256) + round_up((size_t)C * 4, 256) : 0;
    SL_CHECK(ensure_ws(h, part_bytes + qk_bytes));
    float* part = (float*)h->ws;
    const bool bf = dt == SL_BF16;
    const double es = (double)esize(dt);
    Timed tm(h, K_SCORE, (crit == SL_CRIT_QK ? 2.0 * (Cq + C) : 2.0 * C) * T_c,
             es * T_c * (crit == SL_CRIT_L2 ? C : (crit == SL_CRIT_QK ? Cq + C : 2.0 * C)) + 4.0 * C);
    hipError_t e;
    if (crit == SL_CRIT_QK) {
        float* sq = (float*)((char*)h->ws + part_bytes);
        float* sk = (float*)((char*)h->ws + part_bytes + round_up((size_t)Cq * 4, 256));
        e = launch_dense_ssq(0, bf, Y0, ld0, nullptr, 0, rows, T_c, Cq, part, sq, h->stream);
        if (e == hipSuccess) e = launch_dense_ssq(0, bf, Y1, ld1, nullptr, 0, rows, T_c, C, part, sk, h->stream);
        if (e == hipSuccess) e = launch_qk_combine(sq, sk, C / head_dim, n_rep, head_dim, scores, h->stream);
    } else {
        e = launch_dense_ssq(crit == SL_CRIT_SWIGLU_L2 ? 1 : 0, bf, Y0, ld0, Y1, ld1, rows, T_c, C, part,
                             scores, h->stream);
    }
    return hip_check(h, e, "dense_scores");
}

sl_status sl_select_heads(sl_handle* h, const float* scores, int64_t n_heads, int64_t head_dim,
                          int64_t heads_keep, int32_t* idx) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n_heads >= 1 && head_dim >= 1 && n_heads * head_dim <= INT32_MAX, "bad sizes");
    SL_REQUIRE(h, heads_keep >= 0 && heads_keep <= n_heads, "heads_keep must be in [0, n_heads]");
    if (heads_keep == 0) return SL_OK;
    SL_REQUIRE(h, scores && idx, "NULL pointer");
    DeviceGuard g(h->device);
    SL_CHECK(ensure_ws(h, round_up((size_t)n_heads * 4, 256) * 2));
    float* hs = (float*)h->ws;
    int32_t* heads = (int32_t*)((char*)h->ws + round_up((size_t)n_heads * 4, 256));
    Timed tm(h, K_TOPK, (double)n_heads * head_dim, 4.0 * n_heads * head_dim + 4.0 * heads_keep * head_dim);
    return hip_check(h, launch_head_select(scores, n_heads, head_dim, heads_keep, hs, heads, idx, h->stream),
                     "select_heads");
}

// ---------------------------------------------------------------- a5
sl_status sl_expand_gqa(sl_handle* h, const int32_t* idx_kv, int64_t n, int64_t n_rep,
                        int64_t head_dim, int32_t* idx_q) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n >= 0 && n_rep >= 1 && head_dim >= 1, "bad sizes");
    if (n == 0) return SL_OK;
    SL_REQUIRE(h, idx_kv && idx_q, "NULL pointer");
    DeviceGuard g(h->device);
    SL_CHECK(debug_check_list(h, idx_kv, n, INT32_MAX, "idx_kv"));
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
    SL_CHECK(debug_check_list(h, idx, n, C, "idx"));
    return hip_check(h, launch_stack_index(idx, n, C, copies, idx_out, h->stream), "stack_index");
}

sl_status sl_offset_index(sl_handle* h, const int32_t* idx, int64_t n, int64_t offset,
                          int64_t C_max, int32_t* idx_out) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n >= 0 && offset >= 0 && C_max >= 0 && offset + C_max <= INT32_MAX, "bad sizes");
    if (n == 0) return SL_OK;
    SL_REQUIRE(h, idx && idx_out, "NULL pointer");
    DeviceGuard g(h->device);
    return hip_check(h, launch_offset_index(idx, n, offset, idx_out, h->stream), "offset_index");
}

sl_status sl_qkv_index(sl_handle* h, const int32_t* idx_qk, int64_t n_qk, const int32_t* idx_vo, int64_t n_vo,
                       int64_t n_kv_heads, int64_t n_rep, int64_t head_dim, int32_t* idx_q, int32_t* idx_o,
                       int32_t* idx_qkv) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n_kv_heads >= 1 && n_rep >= 1 && head_dim >= 1, "bad sizes");
    const int64_t Ckv = n_kv_heads * head_dim, Cq = Ckv * n_rep;
    SL_REQUIRE(h, n_qk >= 0 && n_vo >= 0 && n_qk <= Ckv && n_vo <= Ckv && Cq + 2 * Ckv <= INT32_MAX,
               "bad sizes");
    if (n_qk + n_vo == 0) return SL_OK;
    SL_REQUIRE(h, idx_qkv && (n_qk == 0 || (idx_qk && idx_q)) && (n_vo == 0 || (idx_vo && idx_o)),
               "NULL pointer");
    DeviceGuard g(h->device);
    SL_CHECK(debug_check_list(h, idx_qk, n_qk, Ckv, "idx_qk"));
    SL_CHECK(debug_check_list(h, idx_vo, n_vo, Ckv, "idx_vo"));
    return hip_check(h, launch_qkv_index(idx_qk, n_qk, idx_vo, n_vo, n_rep, head_dim, Cq, Ckv, idx_q, idx_o,
                                         idx_qkv, h->stream), "qkv_index");
}

// ---------------------------------------------------------------- a6/a7
static sl_status run_gemm(sl_handle* h, sl_dtype dt, bool nn, const GemmProblem* p, int np,
                          const SplitkRed* red = nullptr, bool* red_done = nullptr) {
    if (red_done) *red_done = false;
    float* skws = nullptr;
    size_t skf = 0;
    // tune.gemm_split = 0 turns the split tail off (tuning comparisons)
    const bool split_on = h->tune.gemm_split != 0;
    if ((dt == SL_BF16 && !nn && split_on) || (dt == SL_F32 && split_on)) {
        // scratch for the split tail (bf16: partial tiles of the last, partial
        // round) or the K split (fp32: launches with few tiles); with a fixed
        // workspace a launch it does not fit runs every tile whole
        skf = dt == SL_BF16 ? gemm_split_tail_floats(p, np, h->num_cu, h->tune)
                            : gemm_f32_split_floats(p, np, h->num_cu);
        if (skf && skf * 4 > h->gws_bytes && !h->ws_fixed) {
            const size_t want = skf * 4 + (skf >> 1) + 4096;
            if (h->gws) {
                SL_HIP(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
                SL_HIP(h, hipFree(h->gws), "hipFree");
                h->gws = nullptr;
                h->gws_bytes = 0;
            }
            if (hipMalloc(&h->gws, want) != hipSuccess) {
                (void)hipGetLastError();
                h->gws = nullptr;          // no scratch: the launch runs every tile whole
            } else {
                h->gws_bytes = want;
            }
        }
        if (h->gws) skws = (float*)h->gws;
        skf = h->gws_bytes / 4;
    }
    Timed tm(h, dt == SL_BF16 ? (nn ? K_GEMM_NN : K_GEMM_NT) : K_GEMM_F32, gemm_flops(p, np),
             gemm_bytes(p, np, esize(dt)));
    hipError_t e = dt == SL_BF16
                       ? launch_gemm_bf16(nn, p, np, h->stream, skws, skf, h->num_cu, h->tune, red, red_done)
                       : launch_gemm_f32(nn, p, np, h->stream, skws, skf, h->num_cu);
    return hip_check(h, e, "gemm");
}

}  // extern "C"

namespace {

struct LoraEpi {
    const float* P;
    int64_t ldP;
    const void* B;
    int64_t ldB;
    int64_t r;
    float scale;
};

sl_status check_lora(sl_handle* h, const LoraEpi& l, int64_t T, int64_t Nout, sl_dtype dt) {
    if (!l.P) return SL_OK;
    SL_REQUIRE(h, l.r >= 1 && l.r <= 128, "lora_r must be in [1, 128]");
    SL_REQUIRE(h, l.ldP >= l.r && l.ldB >= l.r, "LoRA leading dimension < lora_r");
    SL_REQUIRE(h, l.B != nullptr, "lora_B is NULL");
    (void)T; (void)Nout; (void)dt;
    return SL_OK;
}

void set_lora(GemmProblem& p, const LoraEpi& l) {
    p.lP = l.P;
    p.ldlP = l.ldP;
    p.lB = l.B;
    p.ldlB = l.ldB;
    p.lr = l.P ? (int)l.r : 0;
    p.lscale = l.scale;
}

GemmProblem problem(const void* A, int64_t lda, const int32_t* a_rows, const void* B, int64_t ldb,
                    const int32_t* b_rows, void* C, int64_t ldc, const int32_t* c_rows,
                    const int32_t* c_cols, int64_t M, int64_t N, int64_t K, int beta,
                    const LoraEpi& l, int64_t a_nrows, int64_t b_nrows) {
    GemmProblem p = {A, lda, a_rows, B, ldb, b_rows, C, ldc, c_rows, c_cols, M, N, K, beta,
                     nullptr, 0, nullptr, 0, 0, 0.f, 0, nullptr, a_nrows, b_nrows, 0};
    set_lora(p, l);
    return p;
}

// Flag bits of the sparse products.  row_side: the call's side is the one
// whose products are side-OUT-shaped (fwd OUT, bwd IN), where the row-subset
// and compact-output flags apply.
sl_status check_flags(sl_handle* h, int flags, bool row_side) {
    const int rows2 = SL_ONLY_OUT_ROWS | SL_ONLY_CTX_ROWS;
    SL_REQUIRE(h, (flags & ~(SL_NO_FILL | rows2 | SL_CTX_COMPACT)) == 0 && (flags & rows2) != rows2, "bad flags");
    SL_REQUIRE(h, row_side || !(flags & (rows2 | SL_CTX_COMPACT)),
               "row-subset and compact flags apply to side-OUT-shaped products (fwd OUT, bwd IN)");
    SL_REQUIRE(h, !(flags & SL_CTX_COMPACT) || (flags & SL_ONLY_CTX_ROWS),
               "SL_CTX_COMPACT needs SL_ONLY_CTX_ROWS");
    return SL_OK;
}

// Output-channel-sparse product (context rows keep only the selected output
// channels): fwd side OUT and bwd side IN share this shape.
//   Z[t, :] = X[t, :] Wc^T  over all channels for output rows,
//   Z[t, c] = X[t, :] . Wc[c, :] for selected c on context rows,
//   unselected context channels: the rank-r term if given, else 0.
sl_status out_sparse(sl_handle* h, sl_dtype dt, const void* X, int64_t ldx, int64_t T,
                     int64_t Kdim, const void* Wc, int64_t ldw, int64_t C,
                     const int32_t* ctx_rows, int64_t T_c, const int32_t* out_rows, int64_t T_o,
                     const int32_t* idx, int64_t n, void* Z, int64_t ldz, int beta,
                     const LoraEpi& l, int flags = 0) {
    const bool only_out = flags & SL_ONLY_OUT_ROWS, only_ctx = flags & SL_ONLY_CTX_ROWS;
    if (only_out && T_o == 0) return SL_OK;
    if (only_ctx && T_c == 0) return SL_OK;
    if (T_c == 0 || (n == C && !only_out && !only_ctx)) {
        GemmProblem p = problem(X, ldx, nullptr, Wc, ldw, nullptr, Z, ldz, nullptr, nullptr, T, C,
                                Kdim, beta, l, T, C);
        return run_gemm(h, dt, false, &p, 1);
    }
    GemmProblem p[2];
    int np = 0;
    // output rows: every channel (they do not depend on the selection)
    if (!only_ctx)
        p[np++] = problem(X, ldx, out_rows, Wc, ldw, nullptr, Z, ldz, out_rows, nullptr, T_o, C, Kdim,
                          beta, l, T, C);
    if (only_out) return run_gemm(h, dt, false, p, np);
    if (flags & SL_CTX_COMPACT) {
        // the context rows' product of the selected channels, stored compactly
        // in Z (row m, column j), the rank-r term of those channels included
        if (n == 0) return SL_OK;
        GemmProblem pc = problem(X, ldx, ctx_rows, Wc, ldw, idx, Z, ldz, nullptr, nullptr, T_c, n, Kdim, 0, l, T, C);
        pc.l_rows = ctx_rows;
        pc.l_cols = idx;
        return run_gemm(h, dt, false, &pc, 1);
    }
    if (dt == SL_BF16 && !beta && !(flags & SL_NO_FILL)) {
        // context rows: the product of the selected channels is stored compactly
        // ([T_c, n], whole 16-byte rows), then one pass writes every channel of
        // those rows: the compact values at the selected channels, the rank-r
        // term (or 0) at the others
        const int64_t ldn = n > 0 ? (n + 7) / 8 * 8 : 8;
        SL_CHECK(ensure_ws(h, round_up((size_t)(T_c * ldn) * 2, 256)));
        void* yc = h->ws;
        if (n > 0) {
            GemmProblem pc = problem(X, ldx, ctx_rows, Wc, ldw, idx, yc, ldn, nullptr, nullptr, T_c, n, Kdim, 0,
                                     l, T, C);
            pc.l_rows = ctx_rows;
            pc.l_cols = idx;
            p[np++] = pc;
            SL_CHECK(run_gemm(h, dt, false, p, np));
        } else if (np) {
            SL_CHECK(run_gemm(h, dt, false, p, np));
        }
        Timed tm(h, K_FILL, 2.0 * T_c * (C - n) * l.r, (double)T_c * (C + n) * 2);
        return hip_check(h, launch_lora_merge_rows(Z, ldz, ctx_rows, T_c, C, l.P, l.ldP, l.B, l.ldB, l.r, l.scale,
                                                   yc, ldn, idx, n, h->stream, h->tune.merge_rows),
                         "lora_merge");
    }
    p[np++] = problem(X, ldx, ctx_rows, Wc, ldw, idx, Z, ldz, ctx_rows, idx, T_c, n, Kdim, beta, l, T,
                      C);
    if (flags & SL_NO_FILL) {
        // the caller writes the unselected channels of context rows itself
        // (sl_lora_fill_unselected), possibly while this product runs
    } else if (l.P && dt == SL_BF16) {
        // rank-r term of the unselected channels of context rows: written for
        // every channel (beta = 0: the product below then overwrites the
        // selected ones) or, when accumulating, for the unselected ones only
        SL_CHECK(ensure_ws(h, round_up((size_t)ceil_div(C, 32) * 4, 256)));
        Timed tm(h, K_FILL, 2.0 * T_c * (C - n) * l.r, (double)T_c * (beta ? 2 * (C - n) : C) * esize(dt));
        SL_HIP(h, launch_lora_fill_rows(Z, ldz, ctx_rows, T_c, C, l.P, l.ldP, l.B, l.ldB, l.r,
                                        l.scale, idx, n, (uint32_t*)h->ws, beta, h->stream),
               "lora_fill");
    } else if (l.P) {
        SL_CHECK(ensure_ws(h, round_up((size_t)(C - n) * 4, 256)));
        int32_t* comp = (int32_t*)h->ws;
        {
            Timed tm(h, K_INDEX, 0, 4.0 * (C + n));
            SL_HIP(h, launch_complement(idx, n, C, comp, h->stream), "complement");
        }
        // fp32: the unselected channels of context rows get the rank-r term alone
        GemmProblem pc = problem(nullptr, 0, ctx_rows, nullptr, 0, nullptr, Z, ldz, ctx_rows, comp,
                                 T_c, C - n, 0, beta, l, 0, 0);
        {
            Timed tm(h, K_FILL, 2.0 * T_c * (C - n) * l.r, (double)T_c * (C - n) * esize(dt));
            SL_HIP(h, launch_gemm_f32(false, &pc, 1, h->stream), "lora_fill");
        }
    } else if (!beta) {
        Timed tm(h, K_FILL, 0, (double)T_c * (C - n) * esize(dt));
        SL_HIP(h, launch_zero_unselected(dt == SL_BF16, Z, ldz, ctx_rows, T_c, idx, n, C, nullptr,
                                         h->stream), "zero_unselected");
    }
    return run_gemm(h, dt, false, p, np);
}

// Input-channel-sparse product (context rows contract over the selected
// channels only): fwd side IN and bwd side OUT share this shape.
//   Wd [Nout, C]: the product's weight with K = C contiguous (dense rows);
//   Wc [C, Nout]: the same weight with one channel per row.
// Output rows: Z = X[out] Wd^T over all C channels.  Context rows: the
// selected columns of X are compacted (Xc [T_c, n]) and the selected rows of
// Wc are gathered and transposed into a slice Ws [Nout, n] (contiguous K), so
// both products run on the NT kernel.
sl_status in_sparse(sl_handle* h, sl_dtype dt, const void* X, int64_t ldx, int64_t T, int64_t C,
                    const void* Wd, int64_t ldwd, const void* Wc, int64_t ldwc, int64_t Nout,
                    const int32_t* ctx_rows, int64_t T_c, const int32_t* out_rows, int64_t T_o,
                    const int32_t* idx, int64_t n, void* Z, int64_t ldz, int beta,
                    const LoraEpi& l, const void* w_slice = nullptr, int64_t ld_w_slice = 0,
                    const void* x_slice = nullptr, int64_t ld_x_slice = 0) {
    if (n == C || T_c == 0) {
        GemmProblem p = problem(X, ldx, nullptr, Wd, ldwd, nullptr, Z, ldz, nullptr, nullptr, T, Nout,
                                C, beta, l, T, Nout);
        return run_gemm(h, dt, false, &p, 1);
    }
    const int64_t ldn = n > 0 ? (n + 7) / 8 * 8 : 8;
    // The dense output-row product contracts over all C channels, the
    // context-row product over n of them.  When C is several times n the dense
    // part may be split along K (fp32 partials + one ordered reduction) so the
    // tiles of the launch carry similar work.  SL_SPLITK_MAX caps the split
    // (tuning sweeps; default 4), SL_SPLITK_MIN is the smallest split taken
    // (default 2).  At C about 3.3n (the FFN down product at 70 %) splitting
    // saves about a third of the product's time; at C about 2n (the attention
    // projections at half sparsity) the two-way split was measured 2 % faster
    // in a step whose LoRA reductions run on a second stream and 2 % slower
    // in a step on one stream.
    const int64_t smax = h->tune.splitk_max;
    int64_t S = 1, Ks = C;
    if (dt == SL_BF16 && T_o > 0 && n > 0 && smax > 1) {
        S = (C + n / 2) / n;
        S = S < h->tune.splitk_min ? 1 : (S > smax ? smax : S);
        if (S > 1) {
            Ks = ceil_div(ceil_div(C, S), 64) * 64;
            S = ceil_div(C, Ks);
        }
    }
    const size_t xc_bytes = x_slice ? 0 : round_up((size_t)(T_c * ldn) * esize(dt), 256);
    const size_t ws_bytes = w_slice ? 0 : round_up((size_t)(Nout * ldn) * esize(dt), 256);
    const size_t part_bytes = S > 1 ? round_up((size_t)(S * T_o * Nout) * 4, 256) : 0;
    SL_CHECK(ensure_ws(h, xc_bytes + ws_bytes + part_bytes));
    const void* xc = x_slice ? x_slice : h->ws;
    const int64_t ldxc = x_slice ? ld_x_slice : ldn;
    const void* wsl = (char*)h->ws + xc_bytes;
    int64_t ldwsl = ldn;
    float* part = (float*)((char*)h->ws + xc_bytes + ws_bytes);
    if (w_slice) {
        wsl = w_slice;
        ldwsl = ld_w_slice;
    }
    if (n > 0 && !(x_slice && w_slice)) {
        Timed tm(h, K_GATHER, 0, 2.0 * ((x_slice ? 0 : T_c) + (w_slice ? 0 : Nout)) * n * esize(dt));
        // both compacted operands are zero-padded to ldn columns, so the
        // context product may contract over K = ldn (a multiple of 8); a weight
        // slice built beforehand (sl_weight_slice) and compact activations
        // written by their producer are used as given
        if (!x_slice)
            SL_HIP(h, launch_gather_cols(dt == SL_BF16, X, ldx, ctx_rows, T_c, idx, n, ldn, (void*)xc, ldn,
                                         h->stream), "gather_cols");
        if (!w_slice)
            SL_HIP(h, launch_gather_rows_t(dt == SL_BF16, Wc, ldwc, idx, n, ldn, Nout, (void*)wsl, ldn,
                                           h->stream), "gather_rows_t");
    }
    GemmProblem p[5];
    int np = 0;
    if (S == 1) {
        p[np++] = problem(X, ldx, out_rows, Wd, ldwd, nullptr, Z, ldz, out_rows, nullptr, T_o, Nout, C,
                          beta, l, T, Nout);
    } else {
        for (int64_t q = 0; q < S; ++q) {
            const int64_t k0 = q * Ks, kn = (C - k0) < Ks ? (C - k0) : Ks;
            LoraEpi lq = l;
            if (q > 0) lq.P = nullptr;      // the rank-r term goes into the first partial
            GemmProblem pp = problem((const char*)X + k0 * esize(dt), ldx, out_rows,
                                     (const char*)Wd + k0 * esize(dt), ldwd, nullptr,
                                     part + q * T_o * Nout, Nout, nullptr, nullptr, T_o, Nout, kn, 0,
                                     lq, T, Nout);
            pp.f32out = 1;
            pp.l_rows = out_rows;
            p[np++] = pp;
        }
    }
    // n > 0: contract over the zero-padded width ldn; n == 0: an empty sum
    p[np++] = problem(xc, ldxc, nullptr, wsl, ldwsl, nullptr, Z, ldz, ctx_rows, nullptr, T_c, Nout,
                      n > 0 ? ldn : 0, beta, l, T_c, Nout);
    p[np - 1].k_alg = n;
    // the ordered sum of the output rows' K-split partials goes with the
    // product's tail-sum launch when it has one, else it follows as its own
    const SplitkRed red = {part, S, T_o, Nout, Z, ldz, out_rows, beta};
    bool red_done = false;
    SL_CHECK(run_gemm(h, dt, false, p, np, (S > 1 && dt == SL_BF16) ? &red : nullptr, &red_done));
    if (S > 1 && !red_done) {
        Timed tm(h, K_REDUCE, (double)S * T_o * Nout, (double)(S * 4 + 2 * esize(dt)) * T_o * Nout);
        SL_HIP(h, launch_splitk_reduce(dt == SL_BF16, part, S, T_o, Nout, Z, ldz, out_rows, nullptr,
                                       beta, h->stream), "splitk_reduce");
    }
    return SL_OK;
}

}  // namespace

extern "C" {

sl_status sl_sparse_linear_fwd(sl_handle* h, sl_side side, sl_dtype dt, const void* x,
                               int64_t ldx, int64_t T, int64_t D_in, const void* W, int64_t ldw,
                               const void* Wt, int64_t ldwt, int64_t D_out, const int32_t* ctx_rows, int64_t T_c,
                               const int32_t* out_rows, int64_t T_o, const int32_t* idx,
                               int64_t n, void* y, int64_t ldy, int beta, const float* lora_P,
                               int64_t ld_lora_P, const void* lora_B, int64_t ld_lora_B,
                               int64_t lora_r, float lora_scale, const void* w_slice,
                               int64_t ld_w_slice, const void* x_slice, int64_t ld_x_slice, int flags) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, side == SL_SIDE_OUT || side == SL_SIDE_IN, "bad side");
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 65535 && D_in >= 1 && D_out >= 1, "bad sizes");
    SL_CHECK(check_flags(h, flags, side == SL_SIDE_OUT));
    SL_CHECK(check_rows(h, ctx_rows, T_c, out_rows, T_o, T));
    const int64_t C = side == SL_SIDE_OUT ? D_out : D_in;
    if (w_slice) {
        SL_REQUIRE(h, side == SL_SIDE_IN, "w_slice applies to side IN");
        SL_CHECK(check_matrix(h, w_slice, ld_w_slice, (n + 7) / 8 * 8, dt, "w_slice"));
    }
    if (x_slice) {
        SL_REQUIRE(h, side == SL_SIDE_IN, "x_slice applies to side IN");
        SL_CHECK(check_matrix(h, x_slice, ld_x_slice, (n + 7) / 8 * 8, dt, "x_slice"));
    }
    SL_REQUIRE(h, n >= 0 && n <= C, "n must be in [0, C]");
    SL_REQUIRE(h, n == 0 || idx != nullptr, "idx is NULL");
    const LoraEpi l = {lora_P, ld_lora_P, lora_B, ld_lora_B, lora_r, lora_scale};
    SL_CHECK(check_lora(h, l, T, D_out, dt));
    if (T == 0) return SL_OK;
    SL_CHECK(debug_check_list(h, idx, n, C, "idx"));
    SL_CHECK(debug_check_list(h, ctx_rows, T_c, T, "ctx_rows"));
    SL_CHECK(debug_check_list(h, out_rows, T_o, T, "out_rows"));
    SL_CHECK(check_matrix(h, x, ldx, D_in, dt, "x"));
    SL_CHECK(check_matrix(h, y, ldy, (flags & SL_CTX_COMPACT) ? (n > 0 ? n : 1) : D_out, dt, "y"));
    SL_CHECK(check_matrix(h, W, ldw, D_in, dt, "W"));
    const bool need_t = side == SL_SIDE_IN && n < C && T_c > 0 && !w_slice;
    if (need_t) SL_CHECK(check_matrix(h, Wt, ldwt, D_out, dt, "Wt"));
    DeviceGuard g(h->device);
    if (side == SL_SIDE_OUT)
        return out_sparse(h, dt, x, ldx, T, D_in, W, ldw, D_out, ctx_rows, T_c, out_rows, T_o, idx,
                          n, y, ldy, beta, l, flags);
    return in_sparse(h, dt, x, ldx, T, D_in, W, ldw, Wt, ldwt, D_out, ctx_rows, T_c, out_rows, T_o,
                     idx, n, y, ldy, beta, l, w_slice, ld_w_slice, x_slice, ld_x_slice);
}

// ---------------------------------------------------------------- a10/a11
sl_status sl_sparse_linear_bwd(sl_handle* h, sl_side side, sl_dtype dt, const void* dy,
                               int64_t lddy, int64_t T, int64_t D_out, const void* W, int64_t ldw,
                               const void* Wt, int64_t ldwt, int64_t D_in, const int32_t* ctx_rows, int64_t T_c,
                               const int32_t* out_rows, int64_t T_o, const int32_t* idx,
                               int64_t n, void* dx, int64_t lddx, int beta, const float* lora_P,
                               int64_t ld_lora_P, const void* lora_B, int64_t ld_lora_B,
                               int64_t lora_r, float lora_scale, const void* w_slice,
                               int64_t ld_w_slice, const void* x_slice, int64_t ld_x_slice, int flags) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, side == SL_SIDE_OUT || side == SL_SIDE_IN, "bad side");
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 65535 && D_in >= 1 && D_out >= 1, "bad sizes");
    SL_CHECK(check_flags(h, flags, side == SL_SIDE_IN));
    SL_CHECK(check_rows(h, ctx_rows, T_c, out_rows, T_o, T));
    const int64_t C = side == SL_SIDE_OUT ? D_out : D_in;
    if (w_slice) {
        SL_REQUIRE(h, side == SL_SIDE_OUT, "w_slice applies to side OUT");
        SL_CHECK(check_matrix(h, w_slice, ld_w_slice, (n + 7) / 8 * 8, dt, "w_slice"));
    }
    if (x_slice) {
        SL_REQUIRE(h, side == SL_SIDE_OUT, "x_slice applies to side OUT");
        SL_CHECK(check_matrix(h, x_slice, ld_x_slice, (n + 7) / 8 * 8, dt, "x_slice"));
    }
    SL_REQUIRE(h, n >= 0 && n <= C, "n must be in [0, C]");
    SL_REQUIRE(h, n == 0 || idx != nullptr, "idx is NULL");
    const LoraEpi l = {lora_P, ld_lora_P, lora_B, ld_lora_B, lora_r, lora_scale};
    SL_CHECK(check_lora(h, l, T, D_in, dt));
    if (T == 0) return SL_OK;
    SL_CHECK(debug_check_list(h, idx, n, C, "idx"));
    SL_CHECK(debug_check_list(h, ctx_rows, T_c, T, "ctx_rows"));
    SL_CHECK(debug_check_list(h, out_rows, T_o, T, "out_rows"));
    SL_CHECK(check_matrix(h, dy, lddy, D_out, dt, "dy"));
    SL_CHECK(check_matrix(h, dx, lddx, (flags & SL_CTX_COMPACT) ? (n > 0 ? n : 1) : D_in, dt, "dx"));
    SL_CHECK(check_matrix(h, Wt, ldwt, D_out, dt, "Wt"));
    const bool need_w = side == SL_SIDE_OUT && n < C && T_c > 0 && !w_slice;
    if (need_w) SL_CHECK(check_matrix(h, W, ldw, D_in, dt, "W"));
    DeviceGuard g(h->device);
    if (side == SL_SIDE_IN)   // dx = dy W: context rows produce the selected channels only
        return out_sparse(h, dt, dy, lddy, T, D_out, Wt, ldwt, D_in, ctx_rows, T_c, out_rows, T_o,
                          idx, n, dx, lddx, beta, l, flags);
    // side OUT: context rows contract over the selected output channels only
    return in_sparse(h, dt, dy, lddy, T, D_out, Wt, ldwt, W, ldw, D_in, ctx_rows, T_c, out_rows,
                     T_o, idx, n, dx, lddx, beta, l, w_slice, ld_w_slice, x_slice, ld_x_slice);
}

sl_status sl_weight_slice(sl_handle* h, sl_dtype dt, const void* Wc, int64_t ldwc, int64_t C,
                          const int32_t* idx, int64_t n, int64_t Nout, void* out, int64_t ld_out) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, C >= 1 && Nout >= 1 && n >= 1 && n <= C, "bad sizes");
    SL_REQUIRE(h, idx != nullptr, "idx is NULL");
    SL_CHECK(check_matrix(h, Wc, ldwc, Nout, dt, "Wc"));
    const int64_t ldn = (n + 7) / 8 * 8;
    SL_CHECK(check_matrix(h, out, ld_out, ldn, dt, "out"));
    DeviceGuard g(h->device);
    SL_CHECK(debug_check_list(h, idx, n, C, "idx"));
    Timed tm(h, K_GATHER, 0, 2.0 * Nout * n * esize(dt));
    return hip_check(h, launch_gather_rows_t(dt == SL_BF16, Wc, ldwc, idx, n, ldn, Nout, out, ld_out,
                                             h->stream), "weight_slice");
}

sl_status sl_lora_fill_unselected(sl_handle* h, sl_dtype dt, void* y, int64_t ldy, const int32_t* ctx_rows,
                                  int64_t T_c, int64_t C, const float* lora_P, int64_t ld_lora_P,
                                  const void* lora_B, int64_t ld_lora_B, int64_t lora_r, float lora_scale,
                                  const int32_t* idx, int64_t n) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16, "bf16 only");
    SL_REQUIRE(h, T_c >= 0 && C >= 1 && n >= 0 && n <= C, "bad sizes");
    SL_REQUIRE(h, lora_r >= 1 && lora_r <= 128 && ld_lora_P >= lora_r && ld_lora_B >= lora_r, "bad rank");
    if (T_c == 0 || n == C) return SL_OK;
    SL_REQUIRE(h, ctx_rows && lora_P && lora_B && (n == 0 || idx), "NULL pointer");
    SL_CHECK(check_matrix(h, y, ldy, C, dt, "y"));
    DeviceGuard g(h->device);
    SL_CHECK(debug_check_list(h, idx, n, C, "idx"));
    SL_CHECK(ensure_ws(h, round_up((size_t)ceil_div(C, 32) * 4, 256)));
    Timed tm(h, K_FILL, 2.0 * T_c * (C - n) * lora_r, (double)T_c * (C - n) * esize(dt));
    return hip_check(h, launch_lora_fill_rows(y, ldy, ctx_rows, T_c, C, lora_P, ld_lora_P, lora_B, ld_lora_B,
                                              lora_r, lora_scale, idx, n, (uint32_t*)h->ws, 2, h->stream),
                     "lora_fill_unselected");
}

// ---------------------------------------------------------------- a8/a12
sl_status sl_lora_fwd_bwd(sl_handle* h, int mode, sl_dtype dt, const void* x, int64_t ldx,
                          int64_t T, int64_t D_in, int64_t D_out, const void* A, const void* B,
                          int64_t r, float scale, float* xl, int64_t ldxl, void* y, int64_t ldy,
                          const void* dy, int64_t lddy, void* dx, int64_t lddx, float* dA,
                          float* dB, float* gB_io, int64_t ldgB) {
    if (!h) return SL_ERR_INVALID;
    const int all = SL_LORA_XL | SL_LORA_ADD | SL_LORA_GB | SL_LORA_DA | SL_LORA_DB | SL_LORA_DX |
                    SL_LORA_BT;
    SL_REQUIRE(h, (mode & ~all) == 0 && mode != 0, "bad mode");
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, r >= 1 && r <= 128, "r must be in [1, 128]");
    SL_REQUIRE(h, r <= 64 || !(mode & (SL_LORA_ADD | SL_LORA_DX)), "r > 64 with ADD or DX");
    SL_REQUIRE(h, T >= 0 && T <= 65535 * 32 && D_in >= 1 && D_out >= 1, "bad sizes");
    const bool bf = dt == SL_BF16;
    const bool gb = mode & SL_LORA_GB, da = mode & SL_LORA_DA, db = mode & SL_LORA_DB,
               dxm = mode & SL_LORA_DX;
    if (mode & (SL_LORA_XL | SL_LORA_ADD | SL_LORA_DB))
        SL_REQUIRE(h, xl != nullptr && ldxl >= r, "xl is NULL or ldxl < r");
    if (mode & (SL_LORA_XL | SL_LORA_DA)) SL_CHECK(check_matrix(h, x, ldx, D_in, dt, "x"));
    if (mode & (SL_LORA_XL | SL_LORA_DX)) SL_CHECK(check_matrix(h, A, D_in, D_in, dt, "A"));
    if (mode & (SL_LORA_ADD | SL_LORA_GB)) SL_REQUIRE(h, B != nullptr, "B is NULL");
    const bool bt_given = mode & SL_LORA_BT;   // B passed as B^T [r, ceil8(D_out)]
    SL_REQUIRE(h, !bt_given || !(mode & SL_LORA_ADD), "SL_LORA_BT with SL_LORA_ADD");
    if (bt_given && (mode & SL_LORA_GB)) SL_REQUIRE(h, aligned16(B), "B^T is not 16-byte aligned");
    if (mode & SL_LORA_ADD) SL_CHECK(check_matrix(h, y, ldy, D_out, dt, "y"));
    if (gb || db) SL_CHECK(check_matrix(h, dy, lddy, D_out, dt, "dy"));
    if (da) SL_REQUIRE(h, dA != nullptr, "dA is NULL");
    if (db) SL_REQUIRE(h, dB != nullptr, "dB is NULL");
    if (dxm) SL_CHECK(check_matrix(h, dx, lddx, D_in, dt, "dx"));
    if ((da || dxm) && !gb) SL_REQUIRE(h, gB_io != nullptr, "gB input is NULL");
    if (gB_io) SL_REQUIRE(h, ldgB >= r, "ldgB < r");
    DeviceGuard g(h->device);
    const double es = (double)esize(dt);
    const double fl = ((mode & SL_LORA_XL) ? 2.0 * T * D_in * r : 0) +
                      ((mode & SL_LORA_ADD) ? 2.0 * T * D_out * r : 0) + (gb ? 2.0 * T * D_out * r : 0) +
                      (da ? 2.0 * T * D_in * r : 0) + (db ? 2.0 * T * D_out * r : 0) +
                      (dxm ? 2.0 * T * D_in * r : 0);
    const double by = ((mode & SL_LORA_XL) ? es * T * D_in + 4.0 * T * r : 0) +
                      ((mode & SL_LORA_ADD) ? 2 * es * T * D_out + 4.0 * T * r : 0) +
                      (gb ? es * T * D_out + 4.0 * T * r : 0) + (da ? es * T * D_in : 0) +
                      (db ? es * T * D_out : 0) + (dxm ? 2 * es * T * D_in : 0);
    Timed tm(h, K_LORA, fl, by);
    // ranks above 64 run as column chunks of at most 64 (the columns of xl,
    // gB, the rows of dA and the columns of dB are independent of each other)
    const int64_t RC = 64;
    const int64_t rc_max = r < RC ? r : RC;
    // x A^T-type products: the split-K form (more blocks, a reduction launch)
    // pays off only for long rows; tune.lora_xl_split = 0/1 forces a form
    auto xl_split_for = [&](int64_t Dk) {
        if (h->tune.lora_xl_split >= 0) return h->tune.lora_xl_split != 0;
        return Dk > 16384;
    };
    const bool xl_split = xl_split_for(D_in);
    const bool gb_split = xl_split_for(D_out);
    if (mode & SL_LORA_XL) {
        float* xw = nullptr;   // split-K partials (bf16)
        if (bf && xl_split) {
            SL_CHECK(ensure_ws(h, round_up(lora_xl_ws_floats(T, D_in, rc_max) * 4, 256)));
            xw = (float*)h->ws;
        }
        for (int64_t c0 = 0; c0 < r; c0 += RC) {
            const int64_t rc = (r - c0) < RC ? (r - c0) : RC;
            SL_HIP(h, launch_lora_xl(bf, x, ldx, T, D_in, (const char*)A + c0 * D_in * esize(dt), D_in,
                                     rc, xl + c0, ldxl, xw, h->stream), "lora_xl");
        }
    }
    if (mode & SL_LORA_ADD)
        SL_HIP(h, launch_lora_add(bf, xl, ldxl, T, r, B, r, 1, D_out, scale, y, ldy, h->stream),
               "lora_add");
    if (gb || da || db || dxm) {
        // workspace: B^T [r, D_out] (dt), gB [T, r] fp32, chunk partials
        const int64_t nch = T > 0 ? ceil_div(T, 256) : 1;
        const int64_t ldbt = ceil_div(D_out, 8) * 8;
        const size_t bt_bytes = round_up((size_t)(r * ldbt) * esize(dt), 256);
        const size_t gb_bytes = round_up((size_t)(T > 0 ? T : 1) * r * 4, 256);
        const int64_t ncol = D_in > D_out ? D_in : D_out;
        size_t part_floats = (size_t)(nch * r * ncol);
        const size_t xl_floats = bf ? lora_xl_ws_floats(T, D_out, rc_max) : 0;
        if (part_floats < xl_floats) part_floats = xl_floats;
        SL_CHECK(ensure_ws(h, bt_bytes + gb_bytes + part_floats * 4));
        char* ws = (char*)h->ws;
        void* Bt = ws;
        float* gB = gB_io ? gB_io : (float*)(ws + bt_bytes);
        const int64_t ldg = gB_io ? ldgB : r;
        float* part = (float*)(ws + bt_bytes + gb_bytes);
        const void* Bt_use = Bt;
        if (gb && bt_given) Bt_use = B;
        else if (gb) SL_HIP(h, launch_transpose(bf, B, r, D_out, r, Bt, ldbt, h->stream), "transpose");
        for (int64_t c0 = 0; c0 < r; c0 += RC) {
            const int64_t rc = (r - c0) < RC ? (r - c0) : RC;
            if (gb)
                SL_HIP(h, launch_lora_xl(bf, dy, lddy, T, D_out, (const char*)Bt_use + c0 * ldbt * esize(dt),
                                         ldbt, rc, gB + c0, ldg, (bf && gb_split) ? part : nullptr, h->stream),
                       "lora_gB");
            if (da)
                SL_HIP(h, launch_outer_accum(bf, gB + c0, ldg, T, rc, x, ldx, D_in, scale, dA + c0 * D_in,
                                             D_in, 1, part, part_floats, h->stream), "lora_dA");
            if (db)
                SL_HIP(h, launch_outer_accum(bf, xl + c0, ldxl, T, rc, dy, lddy, D_out, scale, dB + c0, 1,
                                             r, part, part_floats, h->stream), "lora_dB");
        }
        if (dxm)
            SL_HIP(h, launch_lora_add(bf, gB, ldg, T, r, A, 1, D_in, D_in, scale, dx, lddx, h->stream),
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

sl_status sl_swiglu_fwd_lora(sl_handle* h, sl_dtype dt, const void* g, int64_t ldg, const void* u, int64_t ldu,
                             int64_t T, int64_t F, const int32_t* rows, int64_t n_rows, void* hout, int64_t ldh,
                             const void* A, int64_t lda, int64_t r, float* xl, int64_t ldxl) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    if (dt != SL_BF16) return fail(h, SL_ERR_UNSUPPORTED, "the fused SwiGLU + LoRA pass is bf16 only");
    SL_REQUIRE(h, T >= 0 && T <= 65535 * 16 && F >= 1 && F % 8 == 0, "bad sizes (F must be a multiple of 8)");
    SL_REQUIRE(h, r >= 1 && r <= 32, "r must be in [1, 32]");
    SL_REQUIRE(h, !rows || (n_rows >= 0 && n_rows <= T), "n_rows must be in [0, T]");
    const int64_t nr = rows ? n_rows : T;
    if (nr == 0) return SL_OK;
    SL_CHECK(check_matrix(h, g, ldg, F, dt, "g"));
    SL_CHECK(check_matrix(h, u, ldu, F, dt, "u"));
    SL_CHECK(check_matrix(h, hout, ldh, F, dt, "h"));
    SL_CHECK(check_matrix(h, A, lda, F, dt, "A"));
    SL_REQUIRE(h, xl != nullptr && ldxl >= r, "xl is NULL or ldxl < r");
    if (rows) SL_CHECK(debug_check_list(h, rows, nr, T, "rows"));
    SL_CHECK(ensure_ws(h, round_up(swiglu_fwd_lora_ws_floats(nr, F, r) * 4, 256)));
    DeviceGuard gd(h->device);
    Timed tm(h, K_SWIGLU, 2.0 * nr * F * r, 3.0 * nr * F * 2 + 2.0 * r * F + 4.0 * nr * r);
    return hip_check(h, launch_swiglu_fwd_lora(g, ldg, u, ldu, rows, nr, F, hout, ldh, A, lda, r, xl, ldxl,
                                               (float*)h->ws, h->stream), "swiglu_fwd_lora");
}

sl_status sl_swiglu_fwd_ctx(sl_handle* h, sl_dtype dt, const void* Yc, int64_t ldyc, const int32_t* ctx_rows,
                            int64_t T_c, int64_t T, int64_t F, const int32_t* idx, int64_t n, const float* lora_P,
                            int64_t ld_lora_P, const void* lora_B, int64_t ld_lora_B, int64_t lora_r,
                            float lora_scale, void* gu, int64_t ldgu, void* hc, int64_t ldhc, const void* A,
                            int64_t lda, int64_t r, float* xl, int64_t ldxl, void* h_rows, int64_t ld_h_rows) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    if (dt != SL_BF16) return fail(h, SL_ERR_UNSUPPORTED, "the fused context-row SwiGLU pass is bf16 only");
    SL_REQUIRE(h, T >= 0 && T <= 65535 * 64 && T_c >= 0 && T_c <= T, "bad sizes");
    SL_REQUIRE(h, F >= 1 && F % 8 == 0, "F must be a positive multiple of 8");
    SL_REQUIRE(h, n >= 0 && n <= F, "n must be in [0, F]");
    SL_REQUIRE(h, lora_r >= 1 && lora_r <= 64 && r >= 1 && r <= 32, "lora_r must be in [1, 64] and r in [1, 32]");
    if (T_c == 0) return SL_OK;
    SL_REQUIRE(h, ctx_rows != nullptr && (n == 0 || idx != nullptr), "ctx_rows or idx is NULL");
    SL_REQUIRE(h, lora_P != nullptr && ld_lora_P >= lora_r, "lora_P is NULL or ld_lora_P < lora_r");
    SL_REQUIRE(h, xl != nullptr && ldxl >= r, "xl is NULL or ldxl < r");
    if (n > 0) SL_CHECK(check_matrix(h, Yc, ldyc, 2 * n, dt, "Yc"));
    SL_CHECK(check_matrix(h, lora_B, ld_lora_B, lora_r, dt, "lora_B"));
    SL_CHECK(check_matrix(h, gu, ldgu, 2 * F, dt, "gu"));
    SL_CHECK(check_matrix(h, hc, ldhc, (n + 7) / 8 * 8 > 0 ? (n + 7) / 8 * 8 : 8, dt, "hc"));
    SL_CHECK(check_matrix(h, A, lda, F, dt, "A"));
    if (h_rows) SL_CHECK(check_matrix(h, h_rows, ld_h_rows, F, dt, "h_rows"));
    SL_CHECK(debug_check_list(h, idx, n, F, "idx"));
    SL_CHECK(debug_check_list(h, ctx_rows, T_c, T, "ctx_rows"));
    SL_CHECK(ensure_ws(h, round_up(swiglu_fwd_ctx_ws_floats(T_c, F, r) * 4, 256)));
    DeviceGuard gd(h->device);
    Timed tm(h, K_SWIGLU, 2.0 * T_c * F * (r + 2 * lora_r),
             2.0 * T_c * (2.0 * n + 2.0 * F + n) + 4.0 * T_c * (lora_r + r) + 2.0 * F * (2 * lora_r + r));
    return hip_check(h, launch_swiglu_fwd_ctx(gu, ldgu, ctx_rows, T_c, F, lora_P, ld_lora_P, lora_B, ld_lora_B,
                                              lora_r, lora_scale, Yc, ldyc, idx, n, hc, ldhc, (n + 7) / 8 * 8, A,
                                              lda, r, xl, ldxl, h_rows, ld_h_rows, (float*)h->ws, h->stream),
                     "swiglu_fwd_ctx");
}

sl_status sl_swiglu_bwd_lora(sl_handle* h, sl_dtype dt, const void* dh, int64_t lddh, const void* g, int64_t ldg,
                             const void* u, int64_t ldu, int64_t T, int64_t F, void* dg, int64_t lddg, void* du,
                             int64_t lddu, const float* gB, int64_t ldgB, const float* xl_g, int64_t ldxlg,
                             const float* xl_u, int64_t ldxlu, int64_t r, float scale, float* dA, float* dB_g,
                             float* dB_u) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    if (dt != SL_BF16) return fail(h, SL_ERR_UNSUPPORTED, "the fused SwiGLU + LoRA pass is bf16 only");
    SL_REQUIRE(h, T >= 0 && T <= 65535 * 4 && F >= 1 && F % 8 == 0, "bad sizes (F must be a multiple of 8)");
    SL_REQUIRE(h, r >= 1 && r <= 32, "r must be in [1, 32]");
    SL_REQUIRE(h, dA && dB_g && dB_u, "dA, dB_g or dB_u is NULL");
    if (T > 0) {
        SL_CHECK(check_matrix(h, dh, lddh, F, dt, "dh"));
        SL_CHECK(check_matrix(h, g, ldg, F, dt, "g"));
        SL_CHECK(check_matrix(h, u, ldu, F, dt, "u"));
        SL_CHECK(check_matrix(h, dg, lddg, F, dt, "dg"));
        SL_CHECK(check_matrix(h, du, lddu, F, dt, "du"));
        SL_REQUIRE(h, gB && xl_g && xl_u && ldgB >= r && ldxlg >= r && ldxlu >= r,
                   "gB / xl_g / xl_u NULL or leading dimension < r");
    }
    const int64_t rpc = h->tune.swiglu_rows;
    DeviceGuard gd(h->device);
    // T = 0: no rows to read; the sums write zero gradients
    if (T > 0) SL_CHECK(ensure_ws(h, round_up(swiglu_bwd_lora_ws_floats(T, F, r, rpc) * 4, 256)));
    Timed tm(h, K_SWIGLU, 3.0 * 2.0 * T * F * r, 5.0 * T * F * 2 + 3.0 * 4 * T * r + 3.0 * 4 * r * F);
    return hip_check(h, launch_swiglu_bwd_lora(dh, lddh, g, ldg, u, ldu, T, F, dg, lddg, du, lddu, gB, ldgB, xl_g,
                                               ldxlg, xl_u, ldxlu, r, scale, dA, dB_g, dB_u, rpc,
                                               T > 0 ? (float*)h->ws : nullptr, h->stream), "swiglu_bwd_lora");
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

sl_status sl_svd_factors(sl_handle* h, sl_dtype dt, const void* W, int64_t ldw, const void* Wt, int64_t ldwt,
                         int64_t D_out, int64_t D_in, int64_t k, int64_t oversample, int64_t iters,
                         uint64_t seed, float* WA_t, float* WB) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, D_out >= 1 && D_in >= 1 && k >= 1 && oversample >= 0 && iters >= 0 && iters <= 16,
               "bad sizes");
    const int64_t p = k + oversample;
    SL_REQUIRE(h, p <= 64 && p <= D_in && p <= D_out, "k + oversample must be <= 64 and <= min(D_in, D_out)");
    SL_REQUIRE(h, W && Wt && WA_t && WB, "NULL pointer");
    SL_REQUIRE(h, ldw >= D_in && ldwt >= D_out, "bad leading dimension");
    DeviceGuard g(h->device);
    SL_CHECK(ensure_ws(h, svd_factors_ws_bytes(D_out, D_in, (int)p)));
    return hip_check(h, launch_svd_factors(dt == SL_BF16, W, ldw, Wt, ldwt, D_out, D_in, (int)k, (int)p, (int)iters,
                                           seed, WA_t, WB, h->ws, h->stream), "svd_factors");
}

sl_status sl_dot_stats(sl_handle* h, const float* a, const float* b, int64_t n, double* out) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n >= 0, "bad size");
    SL_REQUIRE(h, out != nullptr && (n == 0 || (a && b)), "NULL pointer");
    SL_REQUIRE(h, ((uintptr_t)a & 3) == 0 && ((uintptr_t)b & 3) == 0 && ((uintptr_t)out & 7) == 0,
               "misaligned pointer");
    DeviceGuard gd(h->device);
    SL_CHECK(ensure_ws(h, 256 * 3 * sizeof(double)));
    return hip_check(h, launch_dot_stats(a, b, n, (double*)h->ws, out, h->stream), "dot_stats");
}

// ---------------------------------------------------------------- training step
sl_status sl_token_ce(sl_handle* h, sl_dtype dt, const void* logits, int64_t ld, const int32_t* rows,
                      int64_t n_rows, const int32_t* labels, int64_t V, float scale, void* dlogits,
                      int64_t ld_d, double* loss) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, n_rows >= 0 && n_rows <= INT32_MAX && V >= 1, "bad sizes");
    SL_REQUIRE(h, loss != nullptr && ((uintptr_t)loss & 7) == 0, "loss is NULL or misaligned");
    DeviceGuard g(h->device);
    if (n_rows > 0) {
        SL_REQUIRE(h, logits && rows && labels && dlogits, "NULL pointer");
        SL_REQUIRE(h, ld >= V && ld_d >= V, "leading dimension below V");
    }
    SL_CHECK(ensure_ws(h, round_up((size_t)(n_rows > 0 ? n_rows : 1) * 4, 256)));
    Timed tm(h, K_REDUCE, 4.0 * n_rows * V, (double)esize(dt) * 2.0 * n_rows * V);
    return hip_check(h, launch_ce_rows(dt == SL_BF16, logits, ld, rows, n_rows, labels, V, scale, dlogits,
                                       ld_d, (float*)h->ws, loss, h->stream), "token_ce");
}

sl_status sl_adamw_step(sl_handle* h, const sl_adamw_tensor* tensors, int n, float lr, float beta1,
                        float beta2, float eps, float weight_decay, int64_t step) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, n >= 0 && n <= SL_ADAMW_MAXT, "at most %d tensors per call", SL_ADAMW_MAXT);
    SL_REQUIRE(h, step >= 1, "step counts from 1");
    SL_REQUIRE(h, beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f && eps > 0.f, "bad hyperparameters");
    if (n == 0) return SL_OK;
    SL_REQUIRE(h, tensors != nullptr, "tensors is NULL");
    AdamwArgs a{};
    int64_t blocks = 0;
    for (int i = 0; i < n; ++i) {
        const sl_adamw_tensor& t = tensors[i];
        SL_REQUIRE(h, t.rows >= 0 && t.cols >= 0, "tensor %d: bad shape", i);
        SL_REQUIRE(h, t.param && t.grad && t.m && t.v, "tensor %d: NULL pointer", i);
        SL_REQUIRE(h, !t.out || t.ld_out >= t.cols, "tensor %d: ld_out < cols", i);
        SL_REQUIRE(h, t.out_dtype == SL_BF16 || t.out_dtype == SL_F32, "tensor %d: bad out_dtype", i);
        a.t[i] = AdamwTensor{t.param, t.grad, t.m, t.v, t.out, t.ld_out, t.out_dtype == SL_F32 ? 1 : 0,
                             t.rows, t.cols, blocks};
        blocks += ceil_div(t.rows * t.cols, 256);
    }
    a.n = n;
    a.lr = lr;
    a.b1 = beta1;
    a.b2 = beta2;
    a.eps = eps;
    a.wd = weight_decay;
    a.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
    a.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
    DeviceGuard g(h->device);
    Timed tm(h, K_LORA, 0, 20.0 * 256 * blocks);
    return hip_check(h, launch_adamw(a, blocks, h->stream), "adamw");
}

// ---------------------------------------------------------------- a14: layer glue
sl_status sl_rmsnorm_fwd(sl_handle* h, sl_dtype dt, const void* x, int64_t ldx, const void* res,
                         int64_t ldres, int64_t T, int64_t D, float eps, void* hsum, int64_t ldh,
                         void* y, int64_t ldy, float* rstd) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 2147483647LL && D >= 1 && eps >= 0.0f, "bad sizes");
    if (T == 0) return SL_OK;
    SL_CHECK(check_matrix(h, x, ldx, D, dt, "x"));
    SL_CHECK(check_matrix(h, y, ldy, D, dt, "y"));
    if (res) SL_CHECK(check_matrix(h, res, ldres, D, dt, "res"));
    if (hsum) {
        SL_REQUIRE(h, res != nullptr, "hsum needs res");
        SL_CHECK(check_matrix(h, hsum, ldh, D, dt, "hsum"));
    }
    SL_REQUIRE(h, rstd != nullptr, "rstd is NULL");
    DeviceGuard gd(h->device);
    Timed tm(h, K_NORM, 0, (res ? 3.0 : 2.0) * T * D * esize(dt));
    return hip_check(h, launch_rmsnorm_fwd(dt == SL_BF16, x, ldx, res, ldres, T, D, eps, hsum, ldh, y,
                                           ldy, rstd, h->stream), "rmsnorm_fwd");
}

sl_status sl_rmsnorm_bwd(sl_handle* h, sl_dtype dt, const void* x, int64_t ldx, const float* rstd,
                         const void* dy, int64_t lddy, const void* dres, int64_t lddres, int64_t T,
                         int64_t D, void* dx, int64_t lddx) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 2147483647LL && D >= 1, "bad sizes");
    if (T == 0) return SL_OK;
    SL_CHECK(check_matrix(h, x, ldx, D, dt, "x"));
    SL_CHECK(check_matrix(h, dy, lddy, D, dt, "dy"));
    SL_CHECK(check_matrix(h, dx, lddx, D, dt, "dx"));
    if (dres) SL_CHECK(check_matrix(h, dres, lddres, D, dt, "dres"));
    SL_REQUIRE(h, rstd != nullptr, "rstd is NULL");
    DeviceGuard gd(h->device);
    Timed tm(h, K_NORM, 0, (dres ? 4.0 : 3.0) * T * D * esize(dt));
    return hip_check(h, launch_rmsnorm_bwd(dt == SL_BF16, x, ldx, rstd, dy, lddy, dres, lddres, T, D,
                                           dx, lddx, h->stream), "rmsnorm_bwd");
}

sl_status sl_add(sl_handle* h, sl_dtype dt, const void* a, int64_t lda, const void* b, int64_t ldb,
                 int64_t T, int64_t D, void* out, int64_t ldo) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_REQUIRE(h, T >= 0 && T <= 65535 && D >= 1, "bad sizes");
    if (T == 0) return SL_OK;
    SL_CHECK(check_matrix(h, a, lda, D, dt, "a"));
    SL_CHECK(check_matrix(h, b, ldb, D, dt, "b"));
    SL_CHECK(check_matrix(h, out, ldo, D, dt, "out"));
    DeviceGuard gd(h->device);
    Timed tm(h, K_NORM, 0, 3.0 * T * D * esize(dt));
    return hip_check(h, launch_add(dt == SL_BF16, a, lda, b, ldb, T, D, out, ldo, h->stream), "add");
}

static sl_status check_attn(sl_handle* h, int64_t B, int64_t S, int64_t H, int64_t Hkv, int64_t hd) {
    SL_REQUIRE(h, B >= 0 && S >= 0 && B <= 65535 && S <= 2147483647LL / 32, "bad sizes");
    SL_REQUIRE(h, H >= 1 && Hkv >= 1 && H % Hkv == 0 && H <= 65535, "n_heads must be a multiple of n_kv_heads");
    SL_REQUIRE(h, hd == 32 || hd == 64 || hd == 128, "head_dim must be 32, 64 or 128");
    return SL_OK;
}

sl_status sl_attention_fwd(sl_handle* h, sl_dtype dt, const void* q, int64_t ldq, const void* k,
                           int64_t ldk, const void* v, int64_t ldv, int64_t batch, int64_t seq,
                           int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, void* o,
                           int64_t ldo, float* lse) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_CHECK(check_attn(h, batch, seq, n_heads, n_kv_heads, head_dim));
    if (batch == 0 || seq == 0) return SL_OK;
    SL_CHECK(check_matrix(h, q, ldq, n_heads * head_dim, dt, "q"));
    SL_CHECK(check_matrix(h, k, ldk, n_kv_heads * head_dim, dt, "k"));
    SL_CHECK(check_matrix(h, v, ldv, n_kv_heads * head_dim, dt, "v"));
    SL_CHECK(check_matrix(h, o, ldo, n_heads * head_dim, dt, "o"));
    SL_REQUIRE(h, lse != nullptr, "lse is NULL");
    DeviceGuard gd(h->device);
    const double pairs = (double)batch * n_heads * seq * (seq + 1) / 2.0;
    Timed tm(h, K_ATTN, 4.0 * pairs * head_dim, 0);
    return hip_check(h, launch_attn_fwd(dt == SL_BF16, q, ldq, k, ldk, v, ldv, batch, seq, n_heads,
                                        n_kv_heads, head_dim, o, ldo, lse, h->stream), "attention_fwd");
}

sl_status sl_attention_bwd(sl_handle* h, sl_dtype dt, const void* q, int64_t ldq, const void* k,
                           int64_t ldk, const void* v, int64_t ldv, const void* o, int64_t ldo,
                           const void* dout, int64_t lddout, const float* lse, int64_t batch,
                           int64_t seq, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                           void* dq, int64_t lddq, void* dk, int64_t lddk, void* dv, int64_t lddv) {
    if (!h) return SL_ERR_INVALID;
    SL_REQUIRE(h, dt == SL_BF16 || dt == SL_F32, "bad dtype");
    SL_CHECK(check_attn(h, batch, seq, n_heads, n_kv_heads, head_dim));
    if (batch == 0 || seq == 0) return SL_OK;
    const int64_t Cq = n_heads * head_dim, Ckv = n_kv_heads * head_dim;
    SL_CHECK(check_matrix(h, q, ldq, Cq, dt, "q"));
    SL_CHECK(check_matrix(h, k, ldk, Ckv, dt, "k"));
    SL_CHECK(check_matrix(h, v, ldv, Ckv, dt, "v"));
    SL_CHECK(check_matrix(h, o, ldo, Cq, dt, "o"));
    SL_CHECK(check_matrix(h, dout, lddout, Cq, dt, "dout"));
    SL_CHECK(check_matrix(h, dq, lddq, Cq, dt, "dq"));
    SL_CHECK(check_matrix(h, dk, lddk, Ckv, dt, "dk"));
    SL_CHECK(check_matrix(h, dv, lddv, Ckv, dt, "dv"));
    SL_REQUIRE(h, lse != nullptr, "lse is NULL");
    DeviceGuard gd(h->device);
    // delta (fp32 per query row), then for bf16 the dS tiles of the backward
    SL_CHECK(ensure_ws(h, round_up((size_t)(batch * n_heads * seq) * 4, 256) +
                              (dt == SL_BF16 ? attn_bwd_ds_bytes(batch, seq, n_heads) : 0)));
    const double pairs = (double)batch * n_heads * seq * (seq + 1) / 2.0;
    Timed tm(h, K_ATTN, 10.0 * pairs * head_dim, 0);
    return hip_check(h, launch_attn_bwd(dt == SL_BF16, q, ldq, k, ldk, v, ldv, o, ldo, dout, lddout,
                                        lse, (float*)h->ws, batch, seq, n_heads, n_kv_heads, head_dim,
                                        dq, lddq, dk, lddk, dv, lddv, h->stream), "attention_bwd");
}

}  // extern "C"
