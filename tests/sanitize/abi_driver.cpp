// Host-side argument validation of the C ABI, run under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU.  A handle is built on the host
// (no device calls), and every call below is malformed in one way: each must
// return SL_ERR_INVALID (or SL_ERR_WORKSPACE for an oversized allocation-free
// call) with an error text, before any device work.  Exit status 0 when every
// expectation holds.
#include <cstdio>
#include <cstring>
#include <string>

#include "../../contextual_sparsity_lora_amd/csrc/sl_internal.h"

static int g_fail = 0, g_checks = 0;

static void expect(sl_handle* h, sl_status got, sl_status want, const char* what) {
    ++g_checks;
    const char* e = sl_last_error(h);
    const bool text_ok = want == SL_OK || (e && std::strlen(e) > 0);
    if (got != want || !text_ok) {
        std::printf("FAIL %s: status %d (want %d), error text '%s'\n", what, (int)got, (int)want, e ? e : "(null)");
        ++g_fail;
    }
    if (h) h->err.clear();
}

int main() {
    sl_handle hh;           // host-built: no stream, no workspace, no device flags
    sl_handle* h = &hh;
    alignas(64) static unsigned char buf[1 << 16];
    void* p = buf;          // aligned host memory standing in for device buffers
    void* mis = buf + 4;    // misaligned
    int32_t* ip = (int32_t*)buf;
    float* fp = (float*)buf;
    const sl_status INV = SL_ERR_INVALID;

    // library info and handle options
    for (int s = 0; s >= -4; --s) ++g_checks, g_fail += sl_status_str((sl_status)s) == nullptr;
    ++g_checks, g_fail += sl_version() == nullptr;
    ++g_checks, g_fail += sl_last_error(nullptr) == nullptr;
    expect(h, sl_set_option(h, nullptr, 1), INV, "option name NULL");
    expect(h, sl_set_option(h, "no_such_option", 1), INV, "unknown option");
    std::string longname(3000, 'x');
    expect(h, sl_set_option(h, longname.c_str(), 1), INV, "very long option name");
    expect(h, sl_set_option(h, "gemm_grp", 0), INV, "gemm_grp 0");
    expect(h, sl_set_option(h, "splitk_max", 17), INV, "splitk_max 17");
    expect(h, sl_set_option(h, "gemm_grp", 4), SL_OK, "gemm_grp 4");
    expect(h, sl_set_option(h, "workspace_fixed", 1), SL_OK, "workspace_fixed");
    expect(h, sl_timing_only(h, "no_such_class"), INV, "timing class");
    size_t b = 1;
    expect(h, sl_workspace_bytes(h, &b), SL_OK, "workspace bytes");
    ++g_checks, g_fail += b != 0;
    expect(nullptr, sl_workspace_bytes(nullptr, &b), INV, "workspace bytes, NULL handle");

    // token split
    expect(h, sl_token_split(h, nullptr, 10, ip, 5, ip, 5), INV, "token_split roles NULL");
    expect(h, sl_token_split(h, (const uint8_t*)p, -1, ip, 0, ip, 0), INV, "token_split T < 0");
    expect(h, sl_token_split(h, (const uint8_t*)p, 10, ip, 4, ip, 5), INV, "token_split T_c + T_o != T");

    // estimator and selection
    expect(h, sl_svd_estimate(h, p, SL_F32, 64, ip, 4, 64, (const float*)mis, 16, fp), INV,
           "svd_estimate W_A misaligned");
    expect(h, sl_svd_estimate(h, p, SL_F32, 64, ip, 4, 64, fp, 0, fp), INV, "svd_estimate k_tot 0");
    expect(h, sl_svd_estimate(h, p, SL_F32, 60, ip, 4, 64, fp, 16, fp), INV, "svd_estimate ldx < D_in");
    expect(h, sl_score_select(h, (sl_criterion)99, fp, 16, 4, 0, fp, 0, nullptr, 16, 64, 1, 1, 8, nullptr, ip),
           INV, "score_select criterion");
    expect(h, sl_score_select(h, SL_CRIT_L2, fp, 16, 4, 0, fp, 0, nullptr, 16, 64, 1, 1, 65, nullptr, ip), INV,
           "score_select n_keep > C");
    expect(h, sl_score_select(h, SL_CRIT_L2, nullptr, 16, 4, 0, fp, 0, nullptr, 16, 64, 1, 1, 8, nullptr, ip), INV,
           "score_select xa NULL");
    expect(h, sl_score_select(h, SL_CRIT_L2, fp, 8, 4, 0, fp, 0, nullptr, 16, 64, 1, 1, 8, nullptr, ip), INV,
           "score_select ld_xa < k");
    expect(h, sl_score_select_noalloc(h, SL_CRIT_L2, fp, 16, 4, 0, fp, 0, nullptr, 16, 64, 1, 1, -1, nullptr, ip),
           INV, "noalloc n_keep < 0");
    expect(h, sl_score_select_noalloc(h, SL_CRIT_L2, fp, 16, 4, 0, fp, 0, nullptr, 16, int64_t(1) << 30, 1, 1, 8,
                                      nullptr, ip),
           SL_ERR_WORKSPACE, "noalloc scratch too small");
    expect(h, sl_select_top(h, fp, 64, -1, ip), INV, "select_top n_keep < 0");
    expect(h, sl_select_top(h, nullptr, 64, 8, ip), INV, "select_top scores NULL");

    // sparse products
    auto fwd = [&](sl_side side, sl_dtype dt, const void* x, int64_t ldx, int64_t T, const int32_t* idx,
                   int64_t n, int flags) {
        return sl_sparse_linear_fwd(h, side, dt, x, ldx, T, 64, p, 64, p, 64, 64, ip, T / 2, ip, T - T / 2, idx, n,
                                    p, 64, 0, nullptr, 0, nullptr, 0, 0, 1.0f, nullptr, 0, nullptr, 0, flags);
    };
    expect(h, fwd((sl_side)7, SL_BF16, p, 64, 8, ip, 4, 0), INV, "fwd side");
    expect(h, fwd(SL_SIDE_OUT, (sl_dtype)5, p, 64, 8, ip, 4, 0), INV, "fwd dtype");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, p, 64, 70000, ip, 4, 0), INV, "fwd T too large");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, p, 64, 8, ip, 4, SL_ONLY_OUT_ROWS | SL_ONLY_CTX_ROWS), INV, "fwd both row flags");
    expect(h, fwd(SL_SIDE_IN, SL_BF16, p, 64, 8, ip, 4, SL_ONLY_OUT_ROWS), INV, "fwd row flag on side in");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, p, 64, 8, ip, 65, 0), INV, "fwd n > C");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, p, 64, 8, nullptr, 4, 0), INV, "fwd idx NULL");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, mis, 64, 8, ip, 4, 0), INV, "fwd x misaligned");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, p, 68, 8, ip, 4, 0), INV, "fwd ldx not 16-byte rows");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, p, 64, 8, ip, 4, 1 << 9), INV, "fwd unknown flag");
    expect(h, fwd(SL_SIDE_OUT, SL_BF16, p, 64, 8, ip, 4, SL_CTX_COMPACT), INV, "fwd compact without ctx-only");
    expect(h, fwd(SL_SIDE_IN, SL_BF16, p, 64, 8, ip, 4, SL_CTX_COMPACT | SL_ONLY_CTX_ROWS), INV,
           "fwd compact on side in");
    expect(h, sl_swiglu_fwd_lora(h, SL_BF16, p, 64, p, 64, 8, 64, ip, 9, p, 64, p, 64, 16, fp, 16), INV,
           "swiglu_fwd_lora n_rows > T");
    expect(h, sl_swiglu_fwd_ctx(h, SL_BF16, p, 64, ip, 4, 8, 60, ip, 4, fp, 32, p, 32, 32, 1.0f, p, 128, p, 8, p,
                                64, 16, fp, 16, nullptr, 0),
           INV, "swiglu_fwd_ctx F not a multiple of 8");
    expect(h, sl_swiglu_fwd_ctx(h, SL_BF16, p, 64, ip, 4, 8, 64, ip, 4, fp, 32, p, 32, 80, 1.0f, p, 128, p, 8, p,
                                64, 16, fp, 16, nullptr, 0),
           INV, "swiglu_fwd_ctx lora_r above 64");
    expect(h, sl_swiglu_bwd_lora(h, SL_BF16, p, 64, p, 64, p, 64, 8, 64, p, 64, p, 64, fp, 16, fp, 32, fp, 32, 40,
                                 1.0f, fp, fp, fp),
           INV, "swiglu_bwd_lora r above 32");
    expect(h, sl_sparse_linear_bwd(h, SL_SIDE_IN, SL_BF16, p, 64, 8, 64, p, 64, nullptr, 64, 64, ip, 4, ip, 4, ip,
                                   4, p, 64, 0, fp, 16, p, 16, 200, 1.0f, nullptr, 0, nullptr, 0, 0),
           INV, "bwd LoRA rank above the limit");
    expect(h, sl_sparse_linear_bwd(h, SL_SIDE_OUT, SL_BF16, p, 64, 8, 64, p, 64, nullptr, 64, 64, ip, 4, ip, 4, ip,
                                   4, nullptr, 64, 0, nullptr, 0, nullptr, 0, 0, 1.0f, nullptr, 0, nullptr, 0, 0),
           INV, "bwd dx NULL");
    expect(h, sl_weight_slice(h, SL_BF16, p, 64, 64, ip, 65, 64, p, 72), INV, "weight_slice n > C");
    expect(h, sl_lora_fill_unselected(h, SL_BF16, p, 64, ip, 4, 64, nullptr, 16, p, 16, 16, 1.0f, ip, 4), INV,
           "lora_fill P NULL");

    // LoRA branch
    auto lora = [&](int mode, int64_t r) {
        return sl_lora_fwd_bwd(h, mode, SL_BF16, p, 64, 8, 64, 64, p, p, r, 1.0f, fp, 64, p, 64, p, 64, p, 64, fp, fp,
                               fp, 64);
    };
    expect(h, lora(0, 16), INV, "lora mode 0");
    expect(h, lora(1 << 10, 16), INV, "lora unknown mode bit");
    expect(h, lora(SL_LORA_XL, 0), INV, "lora r 0");
    expect(h, lora(SL_LORA_ADD, 100), INV, "lora r > 64 with ADD");
    expect(h, lora(SL_LORA_ADD | SL_LORA_BT, 16), INV, "lora B^T with ADD");

    // training step, elementwise, attention
    expect(h, sl_token_ce(h, SL_BF16, p, 64, nullptr, 4, ip, 64, 1.0f, p, 64, (double*)p), INV, "token_ce rows NULL");
    expect(h, sl_token_ce(h, SL_BF16, p, 64, ip, 4, ip, 0, 1.0f, p, 64, (double*)p), INV, "token_ce V 0");
    expect(h, sl_adamw_step(h, nullptr, 1, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 1), INV, "adamw tensors NULL");
    expect(h, sl_swiglu_fwd(h, SL_BF16, p, 60, p, 64, 8, 64, p, 64), INV, "swiglu ldg < F");
    expect(h, sl_transpose(h, SL_F32, p, 60, 8, 64, p, 8), INV, "transpose ldi < cols");
    expect(h, sl_attention_fwd(h, SL_BF16, p, 64, p, 64, p, 64, 1, 8, 6, 4, 16, p, 64, fp), INV,
           "attention heads not a multiple of kv heads");
    expect(h, sl_attention_fwd(h, SL_BF16, p, 64, p, 64, p, 64, 1, 8, 4, 4, 0, p, 64, fp), INV, "attention head_dim 0");

    // a NULL handle is refused everywhere
    expect(nullptr, sl_sync(nullptr), INV, "sync NULL handle");
    expect(nullptr, sl_set_option(nullptr, "debug", 1), INV, "set_option NULL handle");
    expect(nullptr, sl_select_top(nullptr, fp, 64, 8, ip), INV, "select_top NULL handle");
    expect(nullptr, sl_sparse_linear_fwd(nullptr, SL_SIDE_OUT, SL_BF16, p, 64, 8, 64, p, 64, p, 64, 64, ip, 4, ip, 4,
                                         ip, 4, p, 64, 0, nullptr, 0, nullptr, 0, 0, 1.0f, nullptr, 0, nullptr, 0,
                                         0),
           INV, "fwd NULL handle");

    std::printf("%d checks, %d failed\n", g_checks, g_fail);
    return g_fail == 0 ? 0 : 1;
}
