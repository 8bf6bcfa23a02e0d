/* Runs the oracle's C functions (oracle/csa.c) on inputs read from a file and
 * writes their outputs to another, so that a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer can be compared with the ordinary build.
 *
 * Input (little-endian): int64 T, D, T_c, k, C, n_keep, then x [T, D] fp32,
 * ctx_rows [T_c] int32, WA_t [2k, D] fp32, WB0 [k, C] fp32, WB1 [k, C] fp32.
 * Output: xa [T_c, 2k], ssq_l2 [C], ssq_swiglu [C], qk [C], exp_sl of every
 * xa entry, the selection count, then idx [count] int32 of each score vector
 * in that order, and orc_r64 of x's first row with itself. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef int64_t i64;
float orc_exp_sl(float z);
float orc_r64(const float* a, i64 sa, const float* b, i64 sb, i64 L);
void orc_stage1(const float* x, i64 ldx, const int32_t* ctx_rows, i64 T_c, i64 D_in, const float* WA_t, i64 k_tot,
                float* xa);
void orc_ssq(int crit, const float* xa, i64 ld_xa, i64 T_c, i64 off0, const float* WB0, i64 off1, const float* WB1,
             i64 k, i64 C, float* ssq);
void orc_qk_combine(const float* ssqQ, const float* ssqK, i64 H_kv, i64 n_rep, i64 d, float* score);
i64 orc_select(const float* score, i64 C, i64 n, int32_t* idx);

static void* take(FILE* f, size_t bytes) {
    void* p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "short input\n");
        exit(2);
    }
    return p;
}

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    FILE* f = fopen(argv[1], "rb");
    if (!f) return 2;
    i64 h[6];
    if (fread(h, sizeof h, 1, f) != 1) return 2;
    const i64 T = h[0], D = h[1], T_c = h[2], k = h[3], C = h[4], n = h[5];
    float* x = take(f, sizeof(float) * (size_t)(T * D));
    int32_t* rows = take(f, sizeof(int32_t) * (size_t)T_c);
    float* WA_t = take(f, sizeof(float) * (size_t)(2 * k * D));
    float* WB0 = take(f, sizeof(float) * (size_t)(k * C));
    float* WB1 = take(f, sizeof(float) * (size_t)(k * C));
    fclose(f);
    float* xa = malloc(sizeof(float) * (size_t)(T_c * 2 * k + 1));
    float* s[3];
    for (int i = 0; i < 3; ++i) s[i] = malloc(sizeof(float) * (size_t)(C + 1));
    orc_stage1(x, D, rows, T_c, D, WA_t, 2 * k, xa);
    orc_ssq(0, xa, 2 * k, T_c, 0, WB0, 0, NULL, k, C, s[0]);
    orc_ssq(1, xa, 2 * k, T_c, 0, WB0, k, WB1, k, C, s[1]);
    orc_qk_combine(s[0], s[1], 1, 1, C, s[2]);
    FILE* o = fopen(argv[2], "wb");
    if (!o) return 2;
    fwrite(xa, sizeof(float), (size_t)(T_c * 2 * k), o);
    for (int i = 0; i < 3; ++i) fwrite(s[i], sizeof(float), (size_t)C, o);
    for (i64 i = 0; i < T_c * 2 * k; ++i) {
        const float e = orc_exp_sl(xa[i]);
        fwrite(&e, sizeof e, 1, o);
    }
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)(C + 1));
    for (int i = 0; i < 3; ++i) {
        const i64 cnt = orc_select(s[i], C, n, idx);
        fwrite(&cnt, sizeof cnt, 1, o);
        fwrite(idx, sizeof(int32_t), (size_t)cnt, o);
    }
    const float r = orc_r64(x, 1, x, 1, D);
    fwrite(&r, sizeof r, 1, o);
    fclose(o);
    free(idx);
    for (int i = 0; i < 3; ++i) free(s[i]);
    free(xa);
    free(WB1);
    free(WB0);
    free(WA_t);
    free(rows);
    free(x);
    return 0;
}
