/*
 * CPU oracle, fp32 part: the canonical score arithmetic of the channel
 * selection (estimator stage 1, estimator stage 2 fused with the criterion,
 * the per-channel token reduction, keys and top-n selection).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links or calls this; only
 * the tests, the smoke check and the benchmark's CPU-baseline leg do.
 *
 * Pages followed (all titled "SparseLoRA: Accelerating LLM Fine-Tuning with
 * Contextual Sparsity"):
 *   - paper-graph summary, §3.4 "SVD Sparsity Estimator", runtime usage
 *     (Algorithm 1): y_hat = (x W_A) W_B; scores from y_hat; keep the top
 *     ceil(r * D_out) channels;
 *   - paper-graph summary, §3.4 "Oracle Sparse Neuron Selection Criteria":
 *     FFN score = L2 norm over batch and sequence of h = SiLU(x W_gate) *
 *     (x W_up); VO score = L2 norm of the value-side activations; QK score =
 *     ||Q||_2 (elementwise) ||K||_2 per channel;
 *   - paper-graph summary, §3.4 "Token Sensitivity": only context tokens are
 *     estimated and scored;
 *   - Paper-Notes page, "SVD 稀疏估计器" and "QK Norm 准则" (same formulas).
 *
 * The pages fix no floating-point detail, so the selection is *defined* by
 * the fp32 operations below; the GPU kernels perform the same IEEE
 * operations in the same order, which makes the selected channel set
 * bit-exact.  Every function states its order.  Build with
 * -O2 -ffp-contract=off and without fast-math: each `+`, `*`, `/` is one
 * correctly rounded binary32 operation and fmaf() is a fused multiply-add.
 *
 * R64(a, b, L): the 64-way strided reduction.  p[0..63] = +0; for m = 0..L-1
 * in ascending order p[m mod 64] = fma(a[m], b[m], p[m mod 64]); then for
 * w = 32, 16, 8, 4, 2, 1: p[l] = p[l] + p[l + w] for l < w; the result is
 * p[0].
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif

typedef int64_t i64;

/* ------------------------------------------------------------------ */
/* exp and SiLU                                                        */
/* ------------------------------------------------------------------ */

/* Cody-Waite additive range reduction (Cody & Waite, "Software Manual for
 * the Elementary Functions", 1980) followed by the degree-7 Taylor
 * polynomial of exp on the reduced argument.  Constants are formed here
 * from their mathematical definitions:
 *   LOG2E = 1/ln 2 rounded to binary32;
 *   LN2_HI = ln 2 rounded to 12 significant bits (2839/4096), so n*LN2_HI is
 *            exact for |n| < 2^12;
 *   LN2_LO = (ln 2 - LN2_HI) rounded to binary32;
 *   C_i    = 1/i! rounded to binary32, i = 0..7. */
static float K_LOG2E, K_LN2_HI, K_LN2_LO, K_C[8];
static int k_ready = 0;

static void init_constants(void) {
    if (k_ready) return;
    const double ln2 = 0.693147180559945309417232121458176568;
    K_LOG2E = (float)(1.0 / ln2);
    K_LN2_HI = (float)(nearbyint(ln2 * 4096.0) / 4096.0);
    K_LN2_LO = (float)(ln2 - (double)K_LN2_HI);
    double f = 1.0;
    for (int i = 0; i < 8; ++i) {
        if (i > 0) f *= (double)i;
        K_C[i] = (float)(1.0 / f);
    }
    k_ready = 1;
}

static float pow2i(int e) { /* 2^e for e in [-126, 127] */
    uint32_t u = (uint32_t)(e + 127) << 23;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* exp_sl(z):
 *   NaN -> NaN; z >= 89 -> +inf; z <= -104 -> +0;
 *   n = nearbyint(z * LOG2E)            (ties to even)
 *   r = fma(-n, LN2_HI, z); r = fma(-n, LN2_LO, r)
 *   p = C7; p = fma(p, r, C_i) for i = 6..0
 *   a = floor(n / 2); b = n - a; result = (p * 2^a) * 2^b           */
float orc_exp_sl(float z) {
    init_constants();
    if (isnan(z)) return z;
    if (z >= 89.0f) return INFINITY;
    if (z <= -104.0f) return 0.0f;
    float t = z * K_LOG2E;
    float n = nearbyintf(t);
    float r = fmaf(-n, K_LN2_HI, z);
    r = fmaf(-n, K_LN2_LO, r);
    float p = K_C[7];
    for (int i = 6; i >= 0; --i) p = fmaf(p, r, K_C[i]);
    int ni = (int)n;
    int a = (ni >= 0) ? ni / 2 : -((-ni + 1) / 2); /* floor(ni / 2) */
    int b = ni - a;
    float s = p * pow2i(a);
    return s * pow2i(b);
}

/* silu_sl(z) = z / (1 + exp_sl(-z)) */
float orc_silu_sl(float z) {
    float e = orc_exp_sl(-z);
    float den = 1.0f + e;
    return z / den;
}

/* The derived constants, in the order LOG2E, LN2_HI, LN2_LO, C0..C7. */
void orc_get_exp_constants11(float* out11) {
    init_constants();
    out11[0] = K_LOG2E;
    out11[1] = K_LN2_HI;
    out11[2] = K_LN2_LO;
    for (int i = 0; i < 8; ++i) out11[3 + i] = K_C[i];
}

void orc_exp_sl_vec(const float* z, float* out, i64 n) {
    for (i64 i = 0; i < n; ++i) out[i] = orc_exp_sl(z[i]);
}

void orc_silu_sl_vec(const float* z, float* out, i64 n) {
    for (i64 i = 0; i < n; ++i) out[i] = orc_silu_sl(z[i]);
}

/* Strided sweep of every binary32 bit pattern whose value lies in
 * [lo, hi], comparing exp_sl with the double-precision exp.  Reports the
 * largest error in units of the binary32 spacing at the true value
 * (for subnormal results: the subnormal spacing 2^-149). */
double orc_exp_sweep(uint32_t stride, float lo, float hi, i64* count) {
    double worst = 0.0;
    i64 cnt = 0;
    for (uint64_t u = 0; u < 0x100000000ull; u += stride) {
        uint32_t b = (uint32_t)u;
        float z;
        memcpy(&z, &b, 4);
        if (!(z >= lo && z <= hi)) continue;
        double ref = exp((double)z);
        float got = orc_exp_sl(z);
        double ulp;
        if (ref >= 1.1754943508222875e-38) {
            int e;
            frexp(ref, &e);              /* ref = m * 2^e, m in [0.5, 1) */
            ulp = ldexp(1.0, e - 24);
        } else {
            ulp = ldexp(1.0, -149);
        }
        if (ref > 3.4028234663852886e38) continue; /* overflows to inf by design */
        double err = fabs((double)got - ref) / ulp;
        if (err > worst) worst = err;
        ++cnt;
    }
    if (count) *count = cnt;
    return worst;
}

/* ------------------------------------------------------------------ */
/* R64 reduction                                                       */
/* ------------------------------------------------------------------ */

float orc_r64(const float* a, i64 sa, const float* b, i64 sb, i64 L) {
    float p[64];
    for (int l = 0; l < 64; ++l) p[l] = 0.0f;
    for (i64 m = 0; m < L; ++m) p[m & 63] = fmaf(a[m * sa], b[m * sb], p[m & 63]);
    for (int w = 32; w >= 1; w >>= 1)
        for (int l = 0; l < w; ++l) p[l] = p[l] + p[l + w];
    return p[0];
}

/* ------------------------------------------------------------------ */
/* Estimator stage 1                                                   */
/* ------------------------------------------------------------------ */

/* xa[m, j] = R64 over i = 0..D_in-1 of (x[ctx_rows[m], i], W_A[i, j]),
 * m = 0..T_c-1 (the context rows, in the order given), j = 0..k_tot-1.
 * x: fp32 values [*, ldx]; WA_t: W_A transposed, [k_tot, D_in];
 * xa: [T_c, k_tot]. */
void orc_stage1(const float* x, i64 ldx, const int32_t* ctx_rows, i64 T_c, i64 D_in,
                const float* WA_t, i64 k_tot, float* xa) {
    for (i64 m = 0; m < T_c; ++m) {
        const float* xr = x + (i64)ctx_rows[m] * ldx;
        for (i64 j = 0; j < k_tot; ++j)
            xa[m * k_tot + j] = orc_r64(xr, 1, WA_t + j * D_in, 1, D_in);
    }
}

/* ------------------------------------------------------------------ */
/* Estimator stage 2 and the criteria                                  */
/* ------------------------------------------------------------------ */

/* y_hat[m, c] = fma chain over j = 0..k-1 starting from +0:
 *   acc = fma(xa[m, j], WB[j, c], acc). */
static float stage2(const float* xa_row, const float* WB, i64 C, i64 c, i64 k) {
    float acc = 0.0f;
    for (i64 j = 0; j < k; ++j) acc = fmaf(xa_row[j], WB[j * C + c], acc);
    return acc;
}

/* crit 0 (L2):        v = y_hat from (xa[:, off0 : off0+k], WB0)
 * crit 1 (SWIGLU_L2): v = silu_sl(g_hat) * u_hat, g_hat from (xa[:, off0:], WB0),
 *                     u_hat from (xa[:, off1:], WB1)
 * ssq[c] = R64 over context tokens m of (v[m, c], v[m, c]). */
void orc_ssq(int crit, const float* xa, i64 ld_xa, i64 T_c, i64 off0, const float* WB0,
             i64 off1, const float* WB1, i64 k, i64 C, float* ssq) {
    float* v = (float*)malloc(sizeof(float) * (size_t)(T_c > 0 ? T_c : 1));
    for (i64 c = 0; c < C; ++c) {
        for (i64 m = 0; m < T_c; ++m) {
            const float* row = xa + m * ld_xa;
            if (crit == 0) {
                v[m] = stage2(row + off0, WB0, C, c, k);
            } else {
                float g = stage2(row + off0, WB0, C, c, k);
                float u = stage2(row + off1, WB1, C, c, k);
                v[m] = orc_silu_sl(g) * u;
            }
        }
        ssq[c] = orc_r64(v, 1, v, 1, T_c);
    }
    free(v);
}

/* QK criterion in the key/value channel space (size H_kv * d):
 *   q2[g*d + j] = sum over r = 0..n_rep-1, ascending, starting from +0, of
 *                 ssqQ[(g*n_rep + r)*d + j]
 *   score[g*d + j] = q2[g*d + j] * ssqK[g*d + j]
 * For n_rep = 1 this is ssqQ * ssqK exactly. */
void orc_qk_combine(const float* ssqQ, const float* ssqK, i64 H_kv, i64 n_rep, i64 d,
                    float* score) {
    for (i64 g = 0; g < H_kv; ++g)
        for (i64 j = 0; j < d; ++j) {
            float q2 = 0.0f;
            for (i64 r = 0; r < n_rep; ++r) q2 = q2 + ssqQ[(g * n_rep + r) * d + j];
            score[g * d + j] = q2 * ssqK[g * d + j];
        }
}

/* ------------------------------------------------------------------ */
/* Keys and selection                                                  */
/* ------------------------------------------------------------------ */

/* key = the binary32 bit pattern of the score; every NaN maps to
 * 0x7FC00000 (above +inf).  Scores are sums of squares, hence >= +0. */
uint32_t orc_key(float s) {
    if (isnan(s)) return 0x7FC00000u;
    uint32_t u;
    memcpy(&u, &s, 4);
    return u;
}

/* Channel c is selected iff fewer than n channels c' precede it, where c'
 * precedes c when key[c'] > key[c], or key[c'] == key[c] and c' < c.
 * The selected channels are written in ascending order; returns the count
 * (always min(n, C)). */
i64 orc_select(const float* score, i64 C, i64 n, int32_t* idx) {
    uint32_t* key = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(C > 0 ? C : 1));
    for (i64 c = 0; c < C; ++c) key[c] = orc_key(score[c]);
    i64 cnt = 0;
    for (i64 c = 0; c < C; ++c) {
        i64 before = 0;
        for (i64 c2 = 0; c2 < C && before < n; ++c2)
            if (key[c2] > key[c] || (key[c2] == key[c] && c2 < c)) ++before;
        if (before < n) idx[cnt++] = (int32_t)c;
    }
    free(key);
    return cnt;
}
