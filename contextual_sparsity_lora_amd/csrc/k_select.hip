// Channel-selection kernels: token-role split, estimator stage 1, estimator
// stage 2 fused with the channel criteria, the QK group product, radix top-n,
// and index propagation.
//
// Pages (all titled "SparseLoRA: Accelerating LLM Fine-Tuning with Contextual
// Sparsity"): paper-graph summary ("PG") §3.4 "SVD Sparsity Estimator" and its
// Algorithm 1 (runtime usage), §3.4 "Oracle Sparse Neuron Selection
// Criteria", §3.4 "Token Sensitivity"; Paper-Notes ("PN") "SVD 稀疏估计器",
// "L2 Norm 准则", "QK Norm 准则".
//
// The pages fix no floating-point detail, so the score arithmetic is fixed
// here as a sequence of binary32 operations (this file is built with
// -ffp-contract=off and IEEE denormals; every fused multiply-add is written
// out).  With that, the selected channel set is reproducible bit for bit:
//   R64(a, b, L): p[0..63] = +0; p[m mod 64] = fma(a[m], b[m], p[m mod 64])
//   for m ascending; then p[l] += p[l + w] for w = 32, 16, ..., 1 (l < w);
//   result p[0].
//   stage 1:  xa[m, j] = R64 over i of (x[ctx[m], i], W_A[i, j])
//   stage 2:  y_hat[m, c] = fma chain over j ascending from +0
//   SiLU:     z / (1 + exp_sl(-z)), exp_sl below
//   ssq[c]:   R64 over context tokens m of (v[m, c], v[m, c])
#include "sl_internal.h"

#pragma clang fp contract(off)

namespace {

constexpr int WAVE = 64;

// ---------------------------------------------------------------- exp / SiLU
// exp by Cody-Waite additive range reduction (Cody & Waite, "Software Manual
// for the Elementary Functions", 1980) and the degree-7 Taylor polynomial.
// Constants, each the binary32 rounding of its mathematical value:
//   1/ln 2                          0x3FB8AA3B
//   ln 2 to 12 significant bits     2839/4096 = 0x3F317000 (exact multiples)
//   ln 2 - 2839/4096                0x3805FDF4
//   1/i!, i = 0..7                  1, 1, 1/2, 0x3E2AAAAB, 0x3D2AAAAB,
//                                   0x3C088889, 0x3AB60B61, 0x39500D01
__device__ __forceinline__ float pow2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

__device__ __forceinline__ float exp_sl(float z) {
    if (__builtin_isnan(z)) return z;
    if (z >= 89.0f) return __builtin_huge_valf();
    if (z <= -104.0f) return 0.0f;
    const float LOG2E = __uint_as_float(0x3FB8AA3Bu);
    const float LN2_HI = __uint_as_float(0x3F317000u);
    const float LN2_LO = __uint_as_float(0x3805FDF4u);
    float t = z * LOG2E;
    float n = __builtin_rintf(t);
    float r = __builtin_fmaf(-n, LN2_HI, z);
    r = __builtin_fmaf(-n, LN2_LO, r);
    float p = __uint_as_float(0x39500D01u);
    p = __builtin_fmaf(p, r, __uint_as_float(0x3AB60B61u));
    p = __builtin_fmaf(p, r, __uint_as_float(0x3C088889u));
    p = __builtin_fmaf(p, r, __uint_as_float(0x3D2AAAABu));
    p = __builtin_fmaf(p, r, __uint_as_float(0x3E2AAAABu));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    int ni = (int)n;
    int a = ni >> 1;  // floor(ni / 2)
    int b = ni - a;
    float s = p * pow2i(a);
    return s * pow2i(b);
}

__device__ __forceinline__ float silu_sl(float z) {
    float e = exp_sl(-z);
    float den = 1.0f + e;
    return z / den;
}

// The same exp_sl without branches: the reduction and polynomial run on the
// input clamped to [-104, 89] (the identity wherever their value is used) and
// the special cases are selected afterwards, so a wave never splits.
__device__ __forceinline__ float exp_sl_nb(float z) {
    const float zc = __builtin_fminf(__builtin_fmaxf(z, -104.0f), 89.0f);
    const float LOG2E = __uint_as_float(0x3FB8AA3Bu);
    const float LN2_HI = __uint_as_float(0x3F317000u);
    const float LN2_LO = __uint_as_float(0x3805FDF4u);
    float t = zc * LOG2E;
    float n = __builtin_rintf(t);
    float r = __builtin_fmaf(-n, LN2_HI, zc);
    r = __builtin_fmaf(-n, LN2_LO, r);
    float p = __uint_as_float(0x39500D01u);
    p = __builtin_fmaf(p, r, __uint_as_float(0x3AB60B61u));
    p = __builtin_fmaf(p, r, __uint_as_float(0x3C088889u));
    p = __builtin_fmaf(p, r, __uint_as_float(0x3D2AAAABu));
    p = __builtin_fmaf(p, r, __uint_as_float(0x3E2AAAABu));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    int ni = (int)n;
    int a = ni >> 1;
    int b = ni - a;
    float v = (p * pow2i(a)) * pow2i(b);
    v = z >= 89.0f ? __builtin_huge_valf() : v;
    v = z <= -104.0f ? 0.0f : v;
    return __builtin_isnan(z) ? z : v;
}

__device__ __forceinline__ float silu_sl_nb(float z) {
    const float den = 1.0f + exp_sl_nb(-z);
    return z / den;
}

__device__ __forceinline__ uint32_t score_key(float s) {
    return __builtin_isnan(s) ? 0x7FC00000u : __float_as_uint(s);
}

// ---------------------------------------------------------------- block scan
// Exclusive prefix sum over a 1024-thread block; returns the exclusive value
// and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int* sh /*[32]*/, int* total) {
    const int lane = threadIdx.x & (WAVE - 1), wid = threadIdx.x / WAVE;
    int x = v;
    for (int o = 1; o < WAVE; o <<= 1) {
        int y = __shfl_up(x, o, WAVE);
        if (lane >= o) x += y;
    }
    if (lane == WAVE - 1) sh[wid] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < (int)(blockDim.x / WAVE); ++w) {
            int t = sh[w];
            sh[w] = run;
            run += t;
        }
        sh[16] = run;
    }
    __syncthreads();
    int excl = sh[wid] + x - v;
    *total = sh[16];
    __syncthreads();
    return excl;
}

// ---------------------------------------------------------------- token split
__global__ __launch_bounds__(1024) void token_split_kernel(const uint8_t* __restrict__ roles,
                                                           int64_t T, int32_t* ctx, int64_t Tc,
                                                           int32_t* out, int64_t To, int* flag) {
    __shared__ int sh[32];
    const int64_t chunk = (T + blockDim.x - 1) / blockDim.x;
    const int64_t beg = (int64_t)threadIdx.x * chunk;
    const int64_t end = beg + chunk < T ? beg + chunk : T;
    int nc = 0;
    for (int64_t t = beg; t < end; ++t) nc += roles[t] == 0;
    int total;
    int pc = block_exclusive_scan(nc, sh, &total);
    int64_t po = beg < T ? beg - pc : 0;  // output rows before this chunk
    for (int64_t t = beg; t < end; ++t) {
        if (roles[t] == 0) {
            if (pc < Tc) ctx[pc] = (int32_t)t;
            ++pc;
        } else {
            if (po < To) out[po] = (int32_t)t;
            ++po;
        }
    }
    if (threadIdx.x == 0 && (int64_t)total != Tc) atomicOr(flag, 1);
}

// ---------------------------------------------------------------- stage 1
// Stage 1, second form: a block of 4 waves takes S1T context tokens and
// 4 S1J columns of W_A (S1J per wave); lane l owns chain l of every (token,
// column) pair it holds (S1T x S1J = 64 pairs).  The 64 chains of each pair
// then go through LDS (pair-major rows, pitch 68 floats) and lane p folds pair
// p with the pairwise tree.  16 tokens per block keep the W_A rows a block
// streams (D x 16 floats) shared by 16 tokens.
constexpr int S1T = 16, S1J = 4;

template <bool BF16>
__global__ __launch_bounds__(256) void stage1b_kernel(const void* __restrict__ xv, int64_t ldx,
                                                      const int32_t* __restrict__ rows, int64_t Tc,
                                                      int64_t D, const float* __restrict__ WA,
                                                      int64_t kt, float* __restrict__ xa) {
    __shared__ __attribute__((aligned(16))) float red[4][S1T * S1J][68];
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
    const int64_t m0 = (int64_t)blockIdx.x * S1T;
    const int64_t j0 = (int64_t)blockIdx.y * (4 * S1J) + w * S1J;
    // rows past Tc read a valid row (the last one); their sums are never
    // stored, so every load is unconditional and the loads of an iteration overlap
    int64_t rowoff[S1T];
#pragma unroll
    for (int t = 0; t < S1T; ++t) rowoff[t] = (int64_t)rows[m0 + t < Tc ? m0 + t : Tc - 1] * ldx;
    const bool wvec = (kt % 4 == 0) && (j0 + S1J <= kt) && (((uintptr_t)WA & 15) == 0);
    float acc[S1T][S1J];
#pragma unroll
    for (int t = 0; t < S1T; ++t)
#pragma unroll
        for (int j = 0; j < S1J; ++j) acc[t][j] = 0.0f;
#pragma unroll 2
    for (int64_t i = lane; i < D; i += WAVE) {
        float xs[S1T];
#pragma unroll
        for (int t = 0; t < S1T; ++t) {
            xs[t] = BF16 ? bf16_to_f32(((const bf16_t*)xv)[rowoff[t] + i]) : ((const float*)xv)[rowoff[t] + i];
        }
        float wv[S1J];
        const float* wr = WA + i * kt + j0;
        if (wvec) {
#pragma unroll
            for (int q = 0; q < S1J; q += 4) {
                const float4 a = *(const float4*)(wr + q);
                wv[q] = a.x; wv[q + 1] = a.y; wv[q + 2] = a.z; wv[q + 3] = a.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < S1J; ++j) {
                const float v = wr[j0 + j < kt ? j : 0];
                wv[j] = j0 + j < kt ? v : 0.0f;
            }
        }
#pragma unroll
        for (int t = 0; t < S1T; ++t)
#pragma unroll
            for (int j = 0; j < S1J; ++j) acc[t][j] = __builtin_fmaf(xs[t], wv[j], acc[t][j]);
    }
#pragma unroll
    for (int t = 0; t < S1T; ++t)
#pragma unroll
        for (int j = 0; j < S1J; ++j) red[w][t * S1J + j][lane] = acc[t][j];
    __syncthreads();
    {
        const int pr = lane;                      // pair: token pr / S1J, column pr % S1J
        float v[64];
#pragma unroll
        for (int l = 0; l < 64; l += 4) {
            const float4 q = *(const float4*)&red[w][pr][l];
            v[l] = q.x; v[l + 1] = q.y; v[l + 2] = q.z; v[l + 3] = q.w;
        }
#pragma unroll
        for (int s2 = 32; s2 >= 1; s2 >>= 1)
#pragma unroll
            for (int l = 0; l < s2; ++l) v[l] = v[l] + v[l + s2];
        const int64_t m = m0 + pr / S1J, j = j0 + pr % S1J;
        if (m < Tc && j < kt) xa[m * kt + j] = v[0];
    }
}

// Stage 2 + criterion, second form (SwiGLU or L2 with K = 16 estimator
// columns): 16 waves over 64 channels; wave w owns the token chains
// 4w .. 4w+3.  The columns of xa the criterion reads are staged in LDS 64
// tokens at a time (double-buffered, one barrier per chunk) and read back as
// broadcasts; SiLU runs without branches.
template <int CRIT>
__global__ __launch_bounds__(1024) void ssq16_kernel(const float* __restrict__ xa, int64_t ld,
                                                     int64_t Tc, int64_t off0,
                                                     const float* __restrict__ WB0, int64_t off1,
                                                     const float* __restrict__ WB1, int64_t C,
                                                     float* __restrict__ ssq) {
    constexpr int K = 16;
    constexpr int NCOL = CRIT == 1 ? 2 * K : K;
    __shared__ __attribute__((aligned(16))) float xs[2][64][NCOL];
    __shared__ float chains[64 * 64];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t c = (int64_t)blockIdx.x * WAVE + lane;
    const int64_t cc = c < C ? c : C - 1;
    float wg[K], wu[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        wg[j] = WB0[(int64_t)j * C + cc];
        wu[j] = CRIT == 1 ? WB1[(int64_t)j * C + cc] : 0.0f;
    }
    // staging of a 64-token chunk of xa: each thread's elements are loaded
    // into registers (fetch) and written to LDS later (put), so the loads of
    // chunk ch + 1 are in flight while chunk ch is scored
    constexpr int NSL = (64 * NCOL + 1023) / 1024;
    float sv[NSL];
    auto fetch = [&](int64_t mb) {
#pragma unroll
        for (int s = 0; s < NSL; ++s) {
            const int q = tid + 1024 * s;
            const int r = q / NCOL, k = q % NCOL;
            const int64_t m = mb + r;
            const int64_t col = k < K ? off0 + k : off1 + (k - K);
            sv[s] = (q < 64 * NCOL && m < Tc) ? xa[m * ld + col] : 0.0f;
        }
    };
    auto put = [&](int buf) {
#pragma unroll
        for (int s = 0; s < NSL; ++s) {
            const int q = tid + 1024 * s;
            if (q < 64 * NCOL) xs[buf][q / NCOL][q % NCOL] = sv[s];
        }
    };
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int64_t nchunk = (Tc + 63) / 64;
    if (nchunk > 0) {
        fetch(0);
        put(0);
    }
    // the channel factors (loaded once above) are in registers before the
    // loop, so no wait inside it is held for them
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __syncthreads();
    for (int64_t ch = 0; ch < nchunk; ++ch) {
        const int buf = (int)(ch & 1);
        if (ch + 1 < nchunk) fetch((ch + 1) * 64);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 4 * w + q;
            const int64_t m = ch * 64 + r;
            if (m >= Tc) continue;
            const float* row = &xs[buf][r][0];
            float g = 0.0f;
#pragma unroll
            for (int j = 0; j < K; ++j) g = __builtin_fmaf(row[j], wg[j], g);
            float v = g;
            if (CRIT == 1) {
                float u = 0.0f;
#pragma unroll
                for (int j = 0; j < K; ++j) u = __builtin_fmaf(row[K + j], wu[j], u);
                v = silu_sl_nb(g) * u;
            }
            p[q] = __builtin_fmaf(v, v, p[q]);
        }
        if (ch + 1 < nchunk) put(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) chains[(4 * w + q) * 64 + lane] = p[q];
    __syncthreads();
    if (w == 0) {
        float v[64];
#pragma unroll
        for (int l = 0; l < 64; ++l) v[l] = chains[l * 64 + lane];
#pragma unroll
        for (int s2 = 32; s2 >= 1; s2 >>= 1)
#pragma unroll
            for (int l = 0; l < s2; ++l) v[l] = v[l] + v[l + s2];
        if (c < C) ssq[c] = v[0];
    }
}

// Stage 2 + criterion for few channels (k = 16): the 64 token chains of a
// channel are spread over 16 blocks (4 waves, one chain per wave), so a
// launch over C channels has 16 ceil(C / 64) blocks instead of ceil(C / 64).
// Chain l = 4 blockIdx.y + w takes tokens m = l, l + 64, ... in order with the
// same fused chain and criterion as ssq16_kernel; its sum goes to part[l, c]
// and r64_tree_kernel applies the pairwise tree (the same result bit for bit).
template <int CRIT>
__global__ __launch_bounds__(256) void ssq16_chain_kernel(const float* __restrict__ xa, int64_t ld,
                                                          int64_t Tc, int64_t off0,
                                                          const float* __restrict__ WB0, int64_t off1,
                                                          const float* __restrict__ WB1, int64_t C,
                                                          float* __restrict__ part) {
    constexpr int K = 16;
    const int lane = threadIdx.x & (WAVE - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = (int)blockIdx.y * 4 + w;
    const int64_t c = (int64_t)blockIdx.x * WAVE + lane;
    const int64_t cc = c < C ? c : C - 1;
    float wg[K], wu[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        wg[j] = WB0[(int64_t)j * C + cc];
        wu[j] = CRIT == 1 ? WB1[(int64_t)j * C + cc] : 0.0f;
    }
    // the criterion values of four tokens of the chain are independent: they
    // are formed together, then folded into the chain in token order
    auto value = [&](int64_t m) -> float {
        const float* row = xa + m * ld;
        float g = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) g = __builtin_fmaf(row[off0 + j], wg[j], g);
        if (CRIT == 0) return g;
        float u = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) u = __builtin_fmaf(row[off1 + j], wu[j], u);
        return silu_sl_nb(g) * u;
    };
    float p = 0.0f;
    int64_t m = l;
    for (; m + 192 < Tc; m += 256) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = value(m + 64 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q) p = __builtin_fmaf(v[q], v[q], p);
    }
    for (; m < Tc; m += 64) {
        const float v = value(m);
        p = __builtin_fmaf(v, v, p);
    }
    if (c < C) part[(int64_t)l * C + c] = p;
}

// ---------------------------------------------------------------- stage 2 + criterion
// Block = 8 waves over 64 channels (one channel per lane).  Wave w owns the
// token chains l = 8w .. 8w+7 (tokens m with m mod 64 = l), so the 64 chains
// of a channel are spread over the block; xa rows are wave-uniform and come
// in through scalar loads.  The chains meet in LDS for the pairwise tree.
template <int CRIT, int K>
__device__ __forceinline__ float crit_value(const float* __restrict__ row, int64_t off0,
                                            int64_t off1, const float* wg, const float* wu,
                                            int krt) {
    if (K > 0) {
        float g = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) g = __builtin_fmaf(row[off0 + j], wg[j], g);
        if (CRIT == 0) return g;
        float u = 0.0f;
#pragma unroll
        for (int j = 0; j < K; ++j) u = __builtin_fmaf(row[off1 + j], wu[j], u);
        return silu_sl(g) * u;
    } else {
        float g = 0.0f;
        for (int j = 0; j < krt; ++j) g = __builtin_fmaf(row[off0 + j], wg[j], g);
        if (CRIT == 0) return g;
        float u = 0.0f;
        for (int j = 0; j < krt; ++j) u = __builtin_fmaf(row[off1 + j], wu[j], u);
        return silu_sl(g) * u;
    }
}

// Any rank k (the estimator up to full rank): the factor columns are read
// from memory inside the chain instead of living in registers; the same
// fma chain over j ascending from +0.
template <int CRIT>
__device__ __forceinline__ float crit_value_mem(const float* __restrict__ row, int64_t off0, int64_t off1,
                                                const float* __restrict__ WB0, const float* __restrict__ WB1,
                                                int64_t C, int64_t c, int krt) {
    float g = 0.0f;
    for (int j = 0; j < krt; ++j) g = __builtin_fmaf(row[off0 + j], WB0[(int64_t)j * C + c], g);
    if (CRIT == 0) return g;
    float u = 0.0f;
    for (int j = 0; j < krt; ++j) u = __builtin_fmaf(row[off1 + j], WB1[(int64_t)j * C + c], u);
    return silu_sl(g) * u;
}

// K > 0: that rank, factor columns in registers; K = 0: rank krt <= 64 in
// registers; K = -1: rank krt of any size, factor columns read in the chain.
template <int CRIT, int K>
__global__ __launch_bounds__(512) void ssq_kernel(const float* __restrict__ xa, int64_t ld,
                                                  int64_t Tc, int64_t off0,
                                                  const float* __restrict__ WB0, int64_t off1,
                                                  const float* __restrict__ WB1, int krt,
                                                  int64_t C, float* __restrict__ ssq) {
    constexpr int KR = K > 0 ? K : (K == 0 ? 64 : 1);
    __shared__ float chains[64 * 64];
    const int lane = threadIdx.x & (WAVE - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c = (int64_t)blockIdx.x * WAVE + lane;
    const int64_t cc = c < C ? c : C - 1;
    const int kk = K > 0 ? K : krt;
    float wg[KR], wu[KR];
    if constexpr (K >= 0) {
#pragma unroll
        for (int j = 0; j < KR; ++j) {
            wg[j] = (j < kk) ? WB0[(int64_t)j * C + cc] : 0.0f;
            wu[j] = (CRIT == 1 && j < kk) ? WB1[(int64_t)j * C + cc] : 0.0f;
        }
    }
    float p[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) p[q] = 0.0f;
    for (int64_t mb = 0; mb < Tc; mb += 64) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int64_t m = mb + 8 * w + q;
            if (m < Tc) {
                const float* row = xa + m * ld;
                float v;
                if constexpr (K >= 0) v = crit_value<CRIT, K>(row, off0, off1, wg, wu, kk);
                else v = crit_value_mem<CRIT>(row, off0, off1, WB0, WB1, C, cc, kk);
                p[q] = __builtin_fmaf(v, v, p[q]);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) chains[(8 * w + q) * 64 + lane] = p[q];
    __syncthreads();
    if (w == 0) {
        float v[64];
#pragma unroll
        for (int l = 0; l < 64; ++l) v[l] = chains[l * 64 + lane];
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1)
#pragma unroll
            for (int l = 0; l < s; ++l) v[l] = v[l] + v[l + s];
        if (c < C) ssq[c] = v[0];
    }
}

__global__ void qk_combine_kernel(const float* __restrict__ Q, const float* __restrict__ Kk,
                                  int64_t H_kv, int64_t n_rep, int64_t d, float* __restrict__ s) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= H_kv * d) return;
    const int64_t g = i / d, j = i % d;
    float q2 = 0.0f;
    for (int64_t r = 0; r < n_rep; ++r) q2 = q2 + Q[(g * n_rep + r) * d + j];
    s[i] = q2 * Kk[i];
}

// ---------------------------------------------------------------- top-n (radix select)
// One 1024-thread block; thread t owns the contiguous channel range
// [t chunk, (t+1) chunk) and keeps up to TKR of its keys in registers.  Four
// 8-bit passes from the most significant byte find the n-th largest key K*:
// each wave counts into its own 256-bin histogram, the 16 histograms are summed
// per bin, and a scan over the bins (from the top) locates the bin that holds
// the n-th key.  Channels with key > K* are kept, and of those with key == K*
// the lowest-indexed fill the remainder; a block scan writes the kept channels
// in ascending order.
constexpr int TKR = 16;

__global__ __launch_bounds__(1024) void topk_kernel(const float* __restrict__ sc, int64_t C,
                                                    int64_t n, int32_t* __restrict__ idx) {
    __shared__ unsigned hist[16][256];
    __shared__ unsigned tot[256];
    __shared__ int sh[32];
    __shared__ uint32_t s_prefix;
    __shared__ int64_t s_rem;
    if (n <= 0) return;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wid = tid / WAVE;
    const int64_t chunk = (C + blockDim.x - 1) / blockDim.x;
    const int64_t beg = (int64_t)tid * chunk;
    const int64_t end = beg + chunk < C ? beg + chunk : C;
    const bool inreg = chunk <= TKR;
    uint32_t kr[TKR];
#pragma unroll
    for (int i = 0; i < TKR; ++i) kr[i] = (inreg && beg + i < end) ? score_key(sc[beg + i]) : 0u;
    auto key = [&](int64_t c) -> uint32_t { return score_key(sc[c]); };

    uint32_t prefix = 0, pmask = 0;
    int64_t rem = n;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 16 * 256; i += blockDim.x) (&hist[0][0])[i] = 0;
        __syncthreads();
        if (inreg) {
#pragma unroll
            for (int i = 0; i < TKR; ++i)
                if (beg + i < end && (kr[i] & pmask) == prefix) atomicAdd(&hist[wid][(kr[i] >> shift) & 255u], 1u);
        } else {
            for (int64_t c = beg; c < end; ++c) {
                const uint32_t k = key(c);
                if ((k & pmask) == prefix) atomicAdd(&hist[wid][(k >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        if (tid < 256) {
            unsigned t = 0;
            for (int w = 0; w < 16; ++w) t += hist[w][tid];
            tot[tid] = t;
        }
        __syncthreads();
        // bins from the top: thread d < 256 handles bin 255 - d; inclusive scan over d
        if (tid < 256) {
            const int d = 255 - tid;
            unsigned v = tot[d];
            unsigned x = v;
            for (int o = 1; o < WAVE; o <<= 1) {
                const unsigned y = __shfl_up(x, o, WAVE);
                if (lane >= o) x += y;
            }
            if (lane == WAVE - 1) sh[wid] = (int)x;
            // wave sums of the 4 waves are combined below
            hist[0][tid] = x;   // inclusive within the wave (hist row 0 is free now)
        }
        __syncthreads();
        if (tid < 256) {
            unsigned base = 0;
            for (int w = 0; w < wid; ++w) base += (unsigned)sh[w];
            const unsigned incl = base + hist[0][tid];
            const unsigned excl = incl - tot[255 - tid];
            if ((int64_t)excl < rem && rem <= (int64_t)incl) {
                s_prefix = prefix | ((uint32_t)(255 - tid) << shift);
                s_rem = rem - (int64_t)excl;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        rem = s_rem;
        pmask |= 255u << shift;
        __syncthreads();
    }
    const uint32_t thr = prefix;
    const int64_t need_eq = rem;
    int neq = 0;
    if (inreg) {
#pragma unroll
        for (int i = 0; i < TKR; ++i) neq += (beg + i < end && kr[i] == thr);
    } else {
        for (int64_t c = beg; c < end; ++c) neq += key(c) == thr;
    }
    int total;
    const int eq_before = block_exclusive_scan(neq, sh, &total);
    int nsel = 0;
    {
        int e = eq_before;
        for (int64_t c = beg; c < end; ++c) {
            const uint32_t k = inreg ? kr[c - beg] : key(c);
            if (k > thr) ++nsel;
            else if (k == thr) { if (e < need_eq) ++nsel; ++e; }
        }
    }
    int pos = block_exclusive_scan(nsel, sh, &total);
    {
        int e = eq_before;
        for (int64_t c = beg; c < end; ++c) {
            const uint32_t k = inreg ? kr[c - beg] : key(c);
            bool take = false;
            if (k > thr) take = true;
            else if (k == thr) { take = e < need_eq; ++e; }
            if (take) {
                if (pos < n) idx[pos] = (int32_t)c;
                ++pos;
            }
        }
    }
}

// ---------------------------------------------------------------- index propagation
__device__ __forceinline__ int64_t lower_bound_i32(const int32_t* a, int64_t n, int64_t v) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = (lo + hi) >> 1;
        if (a[mid] < v) lo = mid + 1; else hi = mid;
    }
    return lo;
}

__global__ void expand_gqa_kernel(const int32_t* __restrict__ idx, int64_t n, int64_t n_rep,
                                  int64_t d, int32_t* __restrict__ out) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n) return;
    const int64_t e = idx[p], g = e / d, j = e % d;
    const int64_t sg = lower_bound_i32(idx, n, g * d);
    const int64_t cg = lower_bound_i32(idx, n, (g + 1) * d) - sg;
    for (int64_t r = 0; r < n_rep; ++r)
        out[sg * n_rep + r * cg + (p - sg)] = (int32_t)((g * n_rep + r) * d + j);
}

__global__ void stack_index_kernel(const int32_t* __restrict__ idx, int64_t n, int64_t C,
                                   int64_t copies, int32_t* __restrict__ out) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n * copies) return;
    const int64_t b = p / n, q = p % n;
    out[p] = (int32_t)(idx[q] + b * C);
}

__global__ void offset_index_kernel(const int32_t* __restrict__ idx, int64_t n, int64_t offset,
                                    int32_t* __restrict__ out) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p < n) out[p] = (int32_t)(idx[p] + offset);
}

// q|k|v index lists of one attention block in one launch: thread p < n_qk
// expands QK key/value channel idx_qk[p] to its n_rep query channels (idx_q)
// and writes its key row idx_qk[p] + Cq; thread n_qk + p' does the same for
// VO channel idx_vo[p'] (idx_o, value row idx_vo[p'] + Cq + Ckv).  The stacked
// list is [idx_q | idx_qk + Cq | idx_vo + Cq + Ckv].
__global__ void qkv_index_kernel(const int32_t* __restrict__ idx_qk, int64_t n_qk,
                                 const int32_t* __restrict__ idx_vo, int64_t n_vo, int64_t n_rep, int64_t d,
                                 int64_t Cq, int64_t Ckv, int32_t* __restrict__ idx_q,
                                 int32_t* __restrict__ idx_o, int32_t* __restrict__ idx_qkv) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= n_qk + n_vo) return;
    const bool qk = p < n_qk;
    const int32_t* idx = qk ? idx_qk : idx_vo;
    const int64_t n = qk ? n_qk : n_vo, i = qk ? p : p - n_qk;
    int32_t* ex = qk ? idx_q : idx_o;
    const int64_t e = idx[i], g = e / d, j = e % d;
    const int64_t sg = lower_bound_i32(idx, n, g * d);
    const int64_t cg = lower_bound_i32(idx, n, (g + 1) * d) - sg;
    for (int64_t r = 0; r < n_rep; ++r) {
        const int64_t pos = sg * n_rep + r * cg + (i - sg);
        const int32_t v = (int32_t)((g * n_rep + r) * d + j);
        ex[pos] = v;
        if (qk) idx_qkv[pos] = v;
    }
    const int64_t nq = n_qk * n_rep;
    if (qk) idx_qkv[nq + i] = (int32_t)(e + Cq);
    else idx_qkv[nq + n_qk + i] = (int32_t)(e + Cq + Ckv);
}

// ---------------------------------------------------------------- criterion variants
template <typename T> __device__ __forceinline__ float ldv(const T* p, int64_t i);
template <> __device__ __forceinline__ float ldv<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldv<bf16_t>(const bf16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// Dense ("oracle") criterion: the same metric on exact outputs instead of the
// estimate, ssq[c] = R64 over listed rows m of (v[m, c], v[m, c]) with
// v = Y0 (L2) or silu(Y0) * Y1 (FFN).  Block = 4 waves; chain l = 4 by + w
// (64 chains, by = blockIdx.y < 16) takes rows m = l, l + 64, ...; a lane owns
// 8 consecutive channels.  The 64 chain sums go to part[l][c]; the second
// kernel runs the R64 pairwise tree per channel.
template <typename T, int CRIT>
__global__ __launch_bounds__(256) void dense_chain_kernel(const T* __restrict__ Y0, int64_t ld0,
                                                          const T* __restrict__ Y1, int64_t ld1,
                                                          const int32_t* __restrict__ rows,
                                                          int64_t Tc, int64_t C,
                                                          float* __restrict__ part) {
    const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x >> 6;
    const int l = (int)blockIdx.y * 4 + w;
    const int64_t c0 = ((int64_t)blockIdx.x * WAVE + lane) * 8;
    if (c0 >= C) return;
    const int nc = (C - c0) < 8 ? (int)(C - c0) : 8;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = 0.0f;
    for (int64_t m = l; m < Tc; m += 64) {
        const int64_t t = rows[m];
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = 0.0f;
            if (e < nc) {
                y = ldv<T>(Y0, t * ld0 + c0 + e);
                if (CRIT == 1) y = silu_sl_nb(y) * ldv<T>(Y1, t * ld1 + c0 + e);
            }
            v[e] = y;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_fmaf(v[e], v[e], p[e]);
    }
    for (int e = 0; e < nc; ++e) part[(int64_t)l * C + c0 + e] = p[e];
}

__global__ void r64_tree_kernel(const float* __restrict__ part, int64_t C, float* __restrict__ ssq) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= C) return;
    float v[64];
#pragma unroll
    for (int l = 0; l < 64; ++l) v[l] = part[(int64_t)l * C + c];
#pragma unroll
    for (int s2 = 32; s2 >= 1; s2 >>= 1)
#pragma unroll
        for (int l = 0; l < s2; ++l) v[l] = v[l] + v[l + s2];
    ssq[c] = v[0];
}

// Random selection scores from a counter-based generator: score[c] is the top
// 24 bits of the (c + 1)-th output of SplitMix64 (Steele, Lea and Flood, 2014)
// started at state `seed`, scaled by 2^-24 (a uniform value in [0, 1), exact in
// fp32).  Output c needs only the counter c, so every channel is independent.
__global__ void random_scores_kernel(uint64_t seed, int64_t C, float* __restrict__ sc) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= C) return;
    uint64_t z = seed + (uint64_t)(c + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    sc[c] = (float)(uint32_t)(z >> 40) * 0x1p-24f;
}

// Head-level selection: hs[g] = sum over j < d of score[g d + j] (fp32, j
// ascending from +0); the kept heads (top-n over hs) expand to their channels.
__global__ void head_score_kernel(const float* __restrict__ sc, int64_t H, int64_t d,
                                  float* __restrict__ hs) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= H) return;
    float s = 0.0f;
    for (int64_t j = 0; j < d; ++j) s = s + sc[g * d + j];
    hs[g] = s;
}

__global__ void head_expand_kernel(const int32_t* __restrict__ heads, int64_t nh, int64_t d,
                                   int32_t* __restrict__ idx) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= nh * d) return;
    idx[p] = (int32_t)(heads[p / d] * d + p % d);
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_offset_index(const int32_t* idx, int64_t n, int64_t offset, int32_t* out,
                               hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(offset_index_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, idx, n,
                       offset, out);
    return hipGetLastError();
}

hipError_t launch_token_split(const uint8_t* roles, int64_t T, int32_t* ctx, int64_t Tc,
                              int32_t* out, int64_t To, int* flag, hipStream_t st) {
    hipLaunchKernelGGL(token_split_kernel, dim3(1), dim3(1024), 0, st, roles, T, ctx, Tc, out, To,
                       flag);
    return hipGetLastError();
}

hipError_t launch_stage1(const void* x, bool bf16, int64_t ldx, const int32_t* rows, int64_t Tc,
                         int64_t D, const float* WA, int64_t kt, float* xa, hipStream_t st) {
    if (Tc <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(Tc, S1T), (unsigned)ceil_div(kt, 4 * S1J));
    if (bf16)
        hipLaunchKernelGGL(stage1b_kernel<true>, grid, dim3(256), 0, st, x, ldx, rows, Tc, D, WA, kt, xa);
    else
        hipLaunchKernelGGL(stage1b_kernel<false>, grid, dim3(256), 0, st, x, ldx, rows, Tc, D, WA, kt, xa);
    return hipGetLastError();
}

hipError_t launch_ssq(int crit, const float* xa, int64_t ld, int64_t Tc, int64_t off0,
                      const float* WB0, int64_t off1, const float* WB1, int64_t k, int64_t C,
                      float* ssq, hipStream_t st, float* part) {
    const dim3 grid((unsigned)ceil_div(C, 64)), block(512);
    if (k == 16 && part && C < SSQ_SPLIT_C) {
        const dim3 g2((unsigned)ceil_div(C, 64), 16);
        if (crit == 0)
            hipLaunchKernelGGL(ssq16_chain_kernel<0>, g2, dim3(256), 0, st, xa, ld, Tc, off0, WB0, off1, WB1, C, part);
        else
            hipLaunchKernelGGL(ssq16_chain_kernel<1>, g2, dim3(256), 0, st, xa, ld, Tc, off0, WB0, off1, WB1, C, part);
        hipLaunchKernelGGL(r64_tree_kernel, dim3((unsigned)ceil_div(C, 256)), dim3(256), 0, st, part, C, ssq);
        return hipGetLastError();
    }
    const int kr = (int)k;
#define SSQ_LAUNCH(CR, KK)                                                                       \
    hipLaunchKernelGGL((ssq_kernel<CR, KK>), grid, block, 0, st, xa, ld, Tc, off0, WB0, off1, WB1, \
                       kr, C, ssq)
    if (k == 16) {
        if (crit == 0)
            hipLaunchKernelGGL(ssq16_kernel<0>, grid, dim3(1024), 0, st, xa, ld, Tc, off0, WB0, off1, WB1, C, ssq);
        else
            hipLaunchKernelGGL(ssq16_kernel<1>, grid, dim3(1024), 0, st, xa, ld, Tc, off0, WB0, off1, WB1, C, ssq);
    } else if (crit == 0) {
        if (k == 8) SSQ_LAUNCH(0, 8);
        else if (k <= 64) SSQ_LAUNCH(0, 0);
        else SSQ_LAUNCH(0, -1);
    } else {
        if (k == 8) SSQ_LAUNCH(1, 8);
        else if (k <= 64) SSQ_LAUNCH(1, 0);
        else SSQ_LAUNCH(1, -1);
    }
#undef SSQ_LAUNCH
    return hipGetLastError();
}

hipError_t launch_qk_combine(const float* ssqQ, const float* ssqK, int64_t H_kv, int64_t n_rep,
                             int64_t d, float* score, hipStream_t st) {
    const int64_t n = H_kv * d;
    hipLaunchKernelGGL(qk_combine_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, ssqQ,
                       ssqK, H_kv, n_rep, d, score);
    return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int64_t C, int64_t n, int32_t* idx, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(1024), 0, st, scores, C, n, idx);
    return hipGetLastError();
}

hipError_t launch_expand_gqa(const int32_t* idx, int64_t n, int64_t n_rep, int64_t d,
                             int32_t* out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(expand_gqa_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, idx,
                       n, n_rep, d, out);
    return hipGetLastError();
}

hipError_t launch_qkv_index(const int32_t* idx_qk, int64_t n_qk, const int32_t* idx_vo, int64_t n_vo,
                            int64_t n_rep, int64_t d, int64_t Cq, int64_t Ckv, int32_t* idx_q, int32_t* idx_o,
                            int32_t* idx_qkv, hipStream_t st) {
    if (n_qk + n_vo <= 0) return hipSuccess;
    hipLaunchKernelGGL(qkv_index_kernel, dim3((unsigned)ceil_div(n_qk + n_vo, 256)), dim3(256), 0, st, idx_qk,
                       n_qk, idx_vo, n_vo, n_rep, d, Cq, Ckv, idx_q, idx_o, idx_qkv);
    return hipGetLastError();
}

hipError_t launch_stack_index(const int32_t* idx, int64_t n, int64_t C, int64_t copies,
                              int32_t* out, hipStream_t st) {
    if (n <= 0 || copies <= 0) return hipSuccess;
    hipLaunchKernelGGL(stack_index_kernel, dim3((unsigned)ceil_div(n * copies, 256)), dim3(256), 0,
                       st, idx, n, C, copies, out);
    return hipGetLastError();
}

hipError_t launch_dense_ssq(int crit, bool bf16, const void* Y0, int64_t ld0, const void* Y1, int64_t ld1,
                            const int32_t* rows, int64_t Tc, int64_t C, float* part, float* ssq,
                            hipStream_t st) {
    if (C <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(C, WAVE * 8), 16);
#define DCH(TT, CR)                                                                                   \
    hipLaunchKernelGGL((dense_chain_kernel<TT, CR>), grid, dim3(256), 0, st, (const TT*)Y0, ld0,     \
                       (const TT*)Y1, ld1, rows, Tc, C, part)
    if (bf16) {
        if (crit == 1) DCH(bf16_t, 1); else DCH(bf16_t, 0);
    } else {
        if (crit == 1) DCH(float, 1); else DCH(float, 0);
    }
#undef DCH
    // rows past Tc leave chains at +0: every chain slot of every channel is written
    hipLaunchKernelGGL(r64_tree_kernel, dim3((unsigned)ceil_div(C, 256)), dim3(256), 0, st, part, C, ssq);
    return hipGetLastError();
}

hipError_t launch_head_select(const float* scores, int64_t H, int64_t d, int64_t nh, float* hs,
                              int32_t* heads, int32_t* idx, hipStream_t st) {
    if (nh <= 0) return hipSuccess;
    hipLaunchKernelGGL(head_score_kernel, dim3((unsigned)ceil_div(H, 256)), dim3(256), 0, st, scores, H,
                       d, hs);
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(1024), 0, st, hs, H, nh, heads);
    hipLaunchKernelGGL(head_expand_kernel, dim3((unsigned)ceil_div(nh * d, 256)), dim3(256), 0, st, heads,
                       nh, d, idx);
    return hipGetLastError();
}

hipError_t launch_random_scores(uint64_t seed, int64_t C, float* scores, hipStream_t st) {
    if (C <= 0) return hipSuccess;
    hipLaunchKernelGGL(random_scores_kernel, dim3((unsigned)ceil_div(C, 256)), dim3(256), 0, st, seed, C,
                       scores);
    return hipGetLastError();
}
