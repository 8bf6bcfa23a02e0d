// Internal declarations of the sparse LoRA linear library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>
#include <vector>

#include "../../include/sparselora.h"

typedef uint16_t bf16_t;  // raw bf16 storage

struct sl_timed_launch {
    int kclass;              // index into the kernel-class name table
    hipEvent_t start, stop;
    double flops, bytes;     // algorithmic work of this launch
};

// Tuning knobs of the launchers, read from the environment once per handle
// (sl_create) and settable with sl_set_option.
struct sl_tuning {
    int gemm_cfg = 10;        // SL_GEMM_CFG: tile configuration of the bf16 NT GEMM
    int gemm_grp = 8;         // SL_GEMM_GRP: tile rows per group of the GEMM tile order
    int gemm_split = 1;       // SL_GEMM_SPLIT: split the last partial round into K-chunks
    int splitk_max = 4;       // SL_SPLITK_MAX: largest split-K of dense output rows
    int splitk_min = 2;       // SL_SPLITK_MIN: smallest split-K taken (smaller: none)
    int merge_rows = 64;      // SL_MERGE_ROWS: rows per wave of the compact-product merge (16, 32, 64)
    int lora_xl_split = -1;   // SL_LORA_XL_SPLIT: x A^T split-K form (-1: by row length)
    int swiglu_rows = 256;    // SL_SWIGLU_ROWS: rows per partial of the fused SwiGLU backward
};

struct sl_handle {
    int device = 0;
    sl_tuning tune;
    bool ws_fixed = false;    // workspace growth is an error (sl_set_option "workspace_fixed")
    bool debug = false;       // SL_DEBUG: host checks of index lists (synchronises)
    bool timing = false;                  // record events around the main launches
    int timing_cls = -1;                  // only launches of this class (-1: all)
    std::vector<sl_timed_launch> timed;   // launches recorded since timing was enabled
    std::vector<hipEvent_t> event_pool;
    hipStream_t stream = nullptr;
    void* ws = nullptr;          // workspace (device)
    size_t ws_bytes = 0;
    void* gws = nullptr;         // GEMM split-tail partial tiles (device)
    size_t gws_bytes = 0;
    int* dev_flags = nullptr;    // device error flags (token split count mismatch, ...)
    int num_cu = 256;
    std::string err;
};

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}
// round to nearest even (the gfx950 conversion instruction, v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, (__bf16)f);
}
// two values rounded to bf16 in one instruction: lo in bits 0-15, hi in 16-31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t h = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------- SwiGLU activation
// Logistic sigmoid on the hardware exponential and reciprocal (v_exp_f32,
// v_rcp_f32, about one ulp each): 1 / (1 + 2^(-z log2 e)).  The activation of
// the SwiGLU passes; the selection criterion evaluates SiLU with its own fixed
// exp instead, so that its scores are reproducible bit for bit.
__device__ __forceinline__ float sigmoid_hw(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504088896341f));
}

// ---------------------------------------------------------------- ascending-list search
// One round of a wave's search for #{j : a[j] < v} in [lo, hi] (the answer is
// known to lie there): the 64 lanes probe 64 evenly spaced entries of the range
// and a ballot keeps the one step that holds the answer.  lo, hi, v uniform.
__device__ __forceinline__ void wave_lb_round(const int32_t* __restrict__ a, int64_t v, int lane, int64_t& lo,
                                              int64_t& hi) {
    const int64_t st = (hi - lo + 63) / 64;
    const int64_t p = lo + lane * st;
    const uint64_t m = __ballot(p < hi && a[p] >= v);
    if (m == 0) {                        // every probe below v: past the last one
        lo = lo + ((hi - 1 - lo) / st) * st + 1;
    } else {
        const int f = __builtin_ctzll(m);
        if (f == 0) {
            hi = lo;                     // a[lo] >= v: the answer is lo
        } else {
            hi = lo + (int64_t)f * st;   // a[lo + f st] >= v > a[lo + (f - 1) st]
            lo = lo + (int64_t)(f - 1) * st + 1;
        }
    }
}
__device__ __forceinline__ int64_t wave_lb_final(const int32_t* __restrict__ a, int64_t v, int lane, int64_t lo,
                                                 int64_t hi) {
    const uint64_t m = __ballot(lo + lane < hi && a[lo + lane] >= v);
    return m ? lo + __builtin_ctzll(m) : hi;
}
// j0 = #{j : a[j] < v0} and j1 = #{j : a[j] < v1} over the ascending list
// a[0..n), by the whole wave: each round narrows a range 64-fold with one
// dependent load (two rounds for n up to 262144), instead of the ~log2(n)
// dependent loads of a one-lane binary search.
__device__ __forceinline__ void wave_lower_bounds(const int32_t* __restrict__ a, int64_t n, int64_t v0, int64_t v1,
                                                  int lane, int64_t& j0, int64_t& j1) {
    int64_t lo0 = 0, hi0 = n, lo1 = 0, hi1 = n;
    while (hi0 - lo0 > 64 || hi1 - lo1 > 64) {
        if (hi0 - lo0 > 64) wave_lb_round(a, v0, lane, lo0, hi0);
        if (hi1 - lo1 > 64) wave_lb_round(a, v1, lane, lo1, hi1);
    }
    j0 = wave_lb_final(a, v0, lane, lo0, hi0);
    j1 = wave_lb_final(a, v1, lane, lo1, hi1);
}

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `st` and returns hipGetLastError().
struct GemmProblem {
    const void* A;  int64_t lda;  const int32_t* a_rows;   // A row m -> a_rows[m] (or m)
    const void* B;  int64_t ldb;  const int32_t* b_rows;   // NT: B row n; NN: B row k
    void* C;        int64_t ldc;  const int32_t* c_rows;   // C row m -> c_rows[m] (or m)
    const int32_t* c_cols;                                 // C col n -> c_cols[n] (or n)
    int64_t M, N, K;
    int beta;                                              // 1: C += result
    // optional rank-lr term added before the single rounding of C:
    //   C[cm, cn] += lscale * sum_j lP[cm, j] * lB[cn, j]   (cm, cn: mapped row/col)
    const float* lP;  int64_t ldlP;
    const void* lB;   int64_t ldlB;
    int lr;           float lscale;
    int f32out;       // 1: store the raw fp32 accumulators (split-K partials)
    const int32_t* l_rows;  // rank-r row map (token rows) when C rows are unmapped partials
    int64_t a_nrows, b_nrows;  // heights of the A / B matrices (0: unknown)
    int64_t k_alg;             // contraction length counted as work (0: K; K may include zero padding)
    const int32_t* l_cols;     // rank-r column map (rows of lB) when C columns are stored unmapped
};
// Ordered sum of split-K partials of bf16 output rows:
//   Z[rows[m], n] = round(sum over s ascending of part[s][m][n] (+ Z if beta))
// (the arithmetic of launch_splitk_reduce).  A launch with a split tail runs it
// in its tail-sum launch, next to the tail tiles' sums, on the compute units
// those leave idle; it needs N % 8 == 0, ldz % 8 == 0 and a 16-byte aligned Z.
struct SplitkRed {
    const float* part;
    int64_t S, M, N;
    void* Z;
    int64_t ldz;
    const int32_t* rows;
    int beta;
};
// bf16 inputs, fp32 accumulate, bf16 output.  nn = false: B is [N, K] ("NT");
// nn = true: B is [K, N] ("NN").  Up to three problems in one launch.
// skws: fp32 scratch for the split tail of the default NT configuration (the
// partial round's tiles run as K-chunks); nullptr or too small: no split.
// red (optional): a split-K sum the launch may take over (see SplitkRed);
// *red_done says whether it did (else the caller launches it afterwards).
hipError_t launch_gemm_bf16(bool nn, const GemmProblem* probs, int nprob, hipStream_t st,
                            float* skws, size_t skws_floats, int ncu, const sl_tuning& tune,
                            const SplitkRed* red = nullptr, bool* red_done = nullptr);
// floats of scratch the split tail of these problems wants (0: none)
size_t gemm_split_tail_floats(const GemmProblem* probs, int nprob, int ncu, const sl_tuning& tune);
// rank-r term only (K = 0 problem), bf16 output
// y[rows[m], c] (+)= scale * P[rows[m], :] . B[c, :] over all C channels (bf16 y,
// fp32 P, bf16 B [C, r]); beta = 0 writes every channel, beta = 1 only the
// channels not in the ascending list idx (mask: ceil(C / 32) words of scratch)
hipError_t launch_lora_fill_rows(void* y, int64_t ldy, const int32_t* rows, int64_t nrows,
                                 int64_t C, const float* P, int64_t ldp, const void* B,
                                 int64_t ldb, int64_t r, float scale, const int32_t* idx,
                                 int64_t n, uint32_t* mask, int beta, hipStream_t st);
// y[rows[m], c] = Yc[m, j] for the selected channels c = idx[j] (a product
// stored compactly, [nrows, >= n] bf16), and scale * P[rows[m], :] . B[c, :]
// (0 when P is null) for every other channel of the row; bf16 y and B
hipError_t launch_lora_merge_rows(void* y, int64_t ldy, const int32_t* rows, int64_t nrows,
                                  int64_t C, const float* P, int64_t ldp, const void* B,
                                  int64_t ldb, int64_t r, float scale, const void* Yc,
                                  int64_t ldyc, const int32_t* idx, int64_t n, hipStream_t st,
                                  int merge_rows = 64);
// fp32 version (VALU), same semantics.
// fp32 products (vector unit).  skws: fp32 scratch for the K split of launches
// with few tiles (nullptr or too small: no split); ncu: compute units.
hipError_t launch_gemm_f32(bool nn, const GemmProblem* probs, int nprob, hipStream_t st,
                           float* skws = nullptr, size_t skws_floats = 0, int ncu = 0);
// floats of scratch the K split of these fp32 problems wants (0: none)
size_t gemm_f32_split_floats(const GemmProblem* probs, int nprob, int ncu);

hipError_t launch_token_split(const uint8_t* roles, int64_t T, int32_t* ctx, int64_t Tc,
                              int32_t* out, int64_t To, int* flag, hipStream_t st);
hipError_t launch_stage1(const void* x, bool bf16, int64_t ldx, const int32_t* rows, int64_t Tc,
                         int64_t D, const float* WA_t, int64_t kt, float* xa, hipStream_t st);
// part: 64 * C floats of scratch for the chain-split form (C < SSQ_SPLIT_C, k = 16), or null
constexpr int64_t SSQ_SPLIT_C = 16384;
hipError_t launch_ssq(int crit, const float* xa, int64_t ld, int64_t Tc, int64_t off0,
                      const float* WB0, int64_t off1, const float* WB1, int64_t k, int64_t C,
                      float* ssq, hipStream_t st, float* part = nullptr);
hipError_t launch_qk_combine(const float* ssqQ, const float* ssqK, int64_t H_kv, int64_t n_rep,
                             int64_t d, float* score, hipStream_t st);
hipError_t launch_topk(const float* scores, int64_t C, int64_t n, int32_t* idx, hipStream_t st);
// dense criterion: ssq[c] = R64 over rows of v^2, v = Y0 (crit 0) or silu(Y0) * Y1
// (crit 1); part holds 64 * C floats
hipError_t launch_dense_ssq(int crit, bool bf16, const void* Y0, int64_t ld0, const void* Y1, int64_t ld1,
                            const int32_t* rows, int64_t Tc, int64_t C, float* part, float* ssq,
                            hipStream_t st);
// random selection scores: SplitMix64 output c + 1 from state seed, top 24 bits / 2^24
hipError_t launch_random_scores(uint64_t seed, int64_t C, float* scores, hipStream_t st);
// head-level selection: hs [H], heads [nh] scratch; idx [nh * d] out
hipError_t launch_head_select(const float* scores, int64_t H, int64_t d, int64_t nh, float* hs,
                              int32_t* heads, int32_t* idx, hipStream_t st);
hipError_t launch_expand_gqa(const int32_t* idx, int64_t n, int64_t n_rep, int64_t d,
                             int32_t* out, hipStream_t st);
hipError_t launch_offset_index(const int32_t* idx, int64_t n, int64_t offset, int32_t* out,
                              hipStream_t st);
hipError_t launch_stack_index(const int32_t* idx, int64_t n, int64_t C, int64_t copies,
                              int32_t* out, hipStream_t st);
// out[m, q] = in[rows[m], cols[q]] for q < ncols, 0 for ncols <= q < npad
hipError_t launch_gather_cols(bool bf16, const void* in, int64_t ldi, const int32_t* rows,
                              int64_t nrows, const int32_t* cols, int64_t ncols, int64_t npad,
                              void* out, int64_t ldo, hipStream_t st);
// Z[c_rows[m], c_cols[n]] = round(sum_s part[s][m][n] (+ Z if beta)), s ascending
hipError_t launch_splitk_reduce(bool bf16, const float* part, int64_t S, int64_t M, int64_t N,
                                void* Z, int64_t ldz, const int32_t* c_rows, const int32_t* c_cols,
                                int beta, hipStream_t st);
// out[j, q] = src[idx[q], j] for j < Dd, q < n (row gather + transpose)
// out[j, q] = src[idx[q], j] for q < n, 0 for n <= q < npad
hipError_t launch_gather_rows_t(bool bf16, const void* src, int64_t lds, const int32_t* idx,
                                int64_t n, int64_t npad, int64_t Dd, void* out, int64_t ldo,
                                hipStream_t st);
// comp[q] = the q-th channel in [0, C) not in the ascending list idx[0..n)
hipError_t launch_complement(const int32_t* idx, int64_t n, int64_t C, int32_t* comp,
                             hipStream_t st);
hipError_t launch_zero_unselected(bool bf16, void* y, int64_t ldy, const int32_t* rows,
                                  int64_t nrows, const int32_t* idx, int64_t n, int64_t C,
                                  uint8_t* mask_ws, hipStream_t st);
// bf16 xl uses a split-K form when a workspace of lora_xl_ws_floats() floats is given
size_t lora_xl_ws_floats(int64_t T, int64_t D, int64_t r);
hipError_t launch_lora_xl(bool bf16, const void* x, int64_t ldx, int64_t T, int64_t D,
                          const void* A, int64_t lda, int64_t r, float* xl, int64_t ldxl,
                          float* ws, hipStream_t st);
hipError_t launch_lora_add(bool bf16, const float* P, int64_t ldp, int64_t T, int64_t r,
                           const void* Bm, int64_t sb_c, int64_t sb_j, int64_t Ncols,
                           float scale, void* y, int64_t ldy, hipStream_t st);
hipError_t launch_outer_accum(bool bf16, const float* P, int64_t ldp, int64_t T, int64_t r,
                              const void* Q, int64_t ldq, int64_t Ncols, float scale,
                              float* out, int64_t so_j, int64_t so_c, float* ws, size_t ws_floats,
                              hipStream_t st);
hipError_t launch_rmsnorm_fwd(bool bf16, const void* x, int64_t ldx, const void* res, int64_t ldr,
                              int64_t T, int64_t D, float eps, void* hout, int64_t ldh, void* y,
                              int64_t ldy, float* rstd, hipStream_t st);
hipError_t launch_rmsnorm_bwd(bool bf16, const void* x, int64_t ldx, const float* rstd, const void* dy,
                              int64_t lddy, const void* dres, int64_t lddr, int64_t T, int64_t D,
                              void* dx, int64_t lddx, hipStream_t st);
hipError_t launch_add(bool bf16, const void* a, int64_t lda, const void* b, int64_t ldb, int64_t T,
                      int64_t D, void* out, int64_t ldo, hipStream_t st);
hipError_t launch_attn_fwd(bool bf16, const void* q, int64_t ldq, const void* k, int64_t ldk,
                           const void* v, int64_t ldv, int64_t B, int64_t S, int64_t H, int64_t Hkv,
                           int64_t hd, void* o, int64_t ldo, float* lse, hipStream_t st);
hipError_t launch_attn_bwd(bool bf16, const void* q, int64_t ldq, const void* k, int64_t ldk,
                           const void* v, int64_t ldv, const void* o, int64_t ldo, const void* dO,
                           int64_t lddo, const float* lse, float* delta, int64_t B, int64_t S,
                           int64_t H, int64_t Hkv, int64_t hd, void* dq, int64_t lddq, void* dk,
                           int64_t lddk, void* dv, int64_t lddv, hipStream_t st);
// (a.b, a.a, b.b) in fp64 over n fp32 values, fixed order; part holds 256 x 3 doubles
// ---------------------------------------------------------------- training step
constexpr int SL_ADAMW_MAXT = 16;
struct AdamwTensor {
    float* p;            // fp32 master [rows * cols]
    const float* g;      // gradient [rows * cols]
    float* m;
    float* v;
    void* out;           // compute copy written after the update (may be null), [rows, ld_out]
    int64_t ld_out;
    int out_f32;         // the copy is fp32 (else bf16)
    int64_t rows, cols;
    int64_t first_block; // first 256-element block of this tensor in the launch
};
struct AdamwArgs {
    AdamwTensor t[SL_ADAMW_MAXT];
    int n;
    float lr, b1, b2, eps, wd, bc1, bc2;
};
hipError_t launch_adamw(const AdamwArgs& a, int64_t blocks, hipStream_t st);
hipError_t launch_ce_rows(bool bf16, const void* L, int64_t ldl, const int32_t* rows, int64_t nrows,
                          const int32_t* labels, int64_t V, float scale, void* dL, int64_t lddl,
                          float* loss_rows, double* loss_sum, hipStream_t st);
// rank-k factors by randomized subspace iteration (p = k + oversample <= 64)
size_t svd_factors_ws_bytes(int64_t D_out, int64_t D_in, int p);
hipError_t launch_svd_factors(bool bf16, const void* W, int64_t ldw, const void* Wt, int64_t ldwt, int64_t D_out,
                              int64_t D_in, int k, int p, int iters, uint64_t seed, float* WA_t, float* WB,
                              void* ws, hipStream_t st);
hipError_t launch_dot_stats(const float* a, const float* b, int64_t n, double* part, double* out,
                            hipStream_t st);
hipError_t launch_transpose(bool bf16, const void* in, int64_t ldi, int64_t rows, int64_t cols,
                            void* out, int64_t ldo, hipStream_t st);
hipError_t launch_swiglu_fwd(bool bf16, const void* g, int64_t ldg, const void* u, int64_t ldu,
                             int64_t T, int64_t F, void* h, int64_t ldh, hipStream_t st);
// SwiGLU with the LoRA reductions reading the same tensors (bf16, r <= 32).
size_t swiglu_fwd_lora_ws_floats(int64_t T, int64_t F, int64_t r);
hipError_t launch_swiglu_fwd_lora(const void* g, int64_t ldg, const void* u, int64_t ldu, const int32_t* rows,
                                  int64_t nr, int64_t F, void* h, int64_t ldh, const void* A, int64_t lda, int64_t r,
                                  float* xl, int64_t ldxl, float* part, hipStream_t st);
// Context rows from their compact gate|up product: merged gu rows, compact h,
// and the rows of h A^T (bf16, 2r <= 64, r <= 32).
size_t swiglu_fwd_ctx_ws_floats(int64_t nrows, int64_t F, int64_t r);
hipError_t launch_swiglu_fwd_ctx(void* gu, int64_t ldgu, const int32_t* rows, int64_t nrows, int64_t F,
                                 const float* P, int64_t ldp, const void* B, int64_t ldb, int64_t r2, float scale,
                                 const void* Yc, int64_t ldyc, const int32_t* idx, int64_t n, void* hc, int64_t ldhc,
                                 int64_t npad, const void* A, int64_t lda, int64_t r, float* xl, int64_t ldxl,
                                 void* hf, int64_t ldhf, float* part, hipStream_t st);
size_t swiglu_bwd_lora_ws_floats(int64_t T, int64_t F, int64_t r, int64_t rows_per_chunk);
hipError_t launch_swiglu_bwd_lora(const void* dh, int64_t lddh, const void* g, int64_t ldg, const void* u,
                                  int64_t ldu, int64_t T, int64_t F, void* dg, int64_t lddg, void* du,
                                  int64_t lddu, const float* Y0, int64_t ldy0, const float* Y1, int64_t ldy1,
                                  const float* Y2, int64_t ldy2, int64_t r, float scale, float* dA, float* dB1,
                                  float* dB2, int64_t rows_per_chunk, float* part, hipStream_t st);
hipError_t launch_swiglu_bwd(bool bf16, const void* dh, int64_t lddh, const void* g, int64_t ldg,
                             const void* u, int64_t ldu, int64_t T, int64_t F, void* dg,
                             int64_t lddg, void* du, int64_t lddu, hipStream_t st);
static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
