/*
 * sparselora.h -- C ABI of the MI355X (gfx950) library for the contextually
 * sparse frozen main-branch linear layer of LoRA fine-tuning (SparseLoRA).
 *
 * Pages cited (all titled "SparseLoRA: Accelerating LLM Fine-Tuning with
 * Contextual Sparsity"): the paper-graph summary ("PG"), sections given as
 * §n "heading"; the Paper-Notes page ("PN"), sections given by heading.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked "device" point to device memory on the handle's device;
 *    the caller allocates and owns all of them.  The library owns only its
 *    handle and an internal workspace (grown on demand, or sized up front
 *    with sl_reserve_workspace so that no allocation happens in the hot path).
 *  - Matrices are row-major with an explicit leading dimension (in elements).
 *    bf16 matrices must start on a 16-byte boundary and have a leading
 *    dimension that is a multiple of 8; fp32 matrices: 16-byte boundary and a
 *    multiple of 4.
 *  - Frozen weights are passed in both layouts: W in the nn.Linear layout
 *    [D_out, D_in] (y = x W^T) and its transposed copy Wt [D_in, D_out]
 *    (made once with sl_transpose).  Every main-branch product then reads
 *    contiguous weight rows: forward products read W, backward products Wt,
 *    and a selection over input channels (forward) or output channels
 *    (backward) gathers rows of the other copy into a per-call slice.
 *  - Sizes (T, T_c, T_o, n, ...) are host integers: nothing on the hot path
 *    copies data back to the host or synchronises.
 *  - Work is enqueued on the handle's stream (sl_set_stream) and runs
 *    asynchronously.  Every call validates its arguments before launching
 *    anything: a non-SL_OK return means nothing was enqueued and no output
 *    was written.  The message of the last error is sl_last_error(h).
 *    Device-side faults surface at a later call or at sl_sync.
 *  - One handle per host thread; calls that overlap on one handle race.
 *  - bf16 results are rounded to nearest even from fp32 accumulators.
 */
#ifndef SPARSELORA_H
#define SPARSELORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sl_handle sl_handle;

typedef enum {
    SL_OK = 0,
    SL_ERR_INVALID = -1,      /* bad argument: null pointer, size, alignment, range */
    SL_ERR_UNSUPPORTED = -2,  /* valid but not implemented (dtype / shape class)   */
    SL_ERR_HIP = -3,          /* a HIP runtime call failed                          */
    SL_ERR_WORKSPACE = -4     /* the internal workspace could not be allocated      */
} sl_status;

typedef enum { SL_F32 = 0, SL_BF16 = 1 } sl_dtype;

/* Channel criteria (PG §3.4 "Oracle Sparse Neuron Selection Criteria"). */
typedef enum {
    SL_CRIT_L2 = 0,        /* score[c] = sum over context tokens of y_hat[., c]^2      */
    SL_CRIT_SWIGLU_L2 = 1, /* score[c] = sum of (SiLU(g_hat) * u_hat)[., c]^2          */
    SL_CRIT_QK = 2         /* score[c] = (sum over the group's query heads of
                              sum q_hat^2) * (sum k_hat^2), in key/value space     */
} sl_criterion;

/* Which side of the weight the selection applies to. */
typedef enum {
    SL_SIDE_OUT = 0,  /* output channels (gate, up, q, k, v); W is [D_out, D_in]  */
    SL_SIDE_IN = 1    /* input channels (down, o); W is the copy [D_in, D_out]    */
} sl_side;

/* sl_sparse_linear_fwd / _bwd flag bits. */
enum {
    SL_NO_FILL = 1,       /* side-OUT-shaped products: leave the unselected channels
                             of context rows unwritten (the caller writes them
                             itself, e.g. with sl_lora_fill_unselected) */
    SL_ONLY_OUT_ROWS = 2, /* side-OUT-shaped products: compute the output rows only
                             (dense over every channel; idx is not read, so the
                             selection may still be in the making on another
                             stream); context rows untouched */
    SL_ONLY_CTX_ROWS = 4, /* the complement: context rows only (selected channels,
                             and the unselected ones unless SL_NO_FILL) */
    SL_CTX_COMPACT = 8    /* side-OUT-shaped products, with SL_ONLY_CTX_ROWS: the
                             context rows' product over the selected channels
                             is stored compactly, y[m, j] for context row m and
                             selected channel idx[j] (y then has T_c rows and
                             ldy >= n), the rank-r term included; the
                             unselected channels are not formed */
};

/* sl_lora_fwd_bwd mode bits. */
enum {
    SL_LORA_XL = 1,   /* forward: xl = x A^T                                      */
    SL_LORA_ADD = 2,  /* forward: y += scale * xl B^T (uses xl as given)          */
    SL_LORA_GB = 4,   /* backward: gB = dy B                                      */
    SL_LORA_DA = 8,   /* backward: dA = scale gB^T x                              */
    SL_LORA_DB = 16,  /* backward: dB = scale dy^T xl                             */
    SL_LORA_DX = 32,  /* backward: dx += scale gB A                               */
    SL_LORA_BT = 64,  /* with GB: B is passed transposed, B^T [r, ceil8(D_out)]   */
    SL_LORA_BWD = 60  /* all four backward steps                                  */
};

/* ---------------------------------------------------------------- handle */

/* Create a handle bound to HIP device `device` (makes it current while the
 * handle's calls run).  The stream defaults to the null stream. */
sl_status sl_create(sl_handle** h, int device);
/* Destroy a handle and free its workspace (synchronises its stream first). */
sl_status sl_destroy(sl_handle* h);
/* Set the hipStream_t (passed as void*) that all later calls enqueue on. */
sl_status sl_set_stream(sl_handle* h, void* hip_stream);
/* Ensure the internal workspace holds at least `bytes` (allocates now). */
sl_status sl_reserve_workspace(sl_handle* h, size_t bytes);
/* Bytes of device memory the handle's workspaces hold now (the internal
 * workspace plus the GEMM's split-tail scratch). */
sl_status sl_workspace_bytes(sl_handle* h, size_t* bytes);
/* Handle options (integers):
 *   "workspace_fixed"  1: no call grows the workspace any more -- a call that
 *                      would need more returns SL_ERR_WORKSPACE before
 *                      launching, and a GEMM whose split tail (bf16) or K
 *                      split (fp32) does not fit the scratch runs every tile
 *                      whole.  For steady-state steps
 *                      after a first step has sized the workspace: no
 *                      allocation, free or synchronisation happens in them.
 *   "debug"            1: before launching, calls that take index lists
 *                      (selections, row lists) copy them to the host after a
 *                      stream synchronisation and return SL_ERR_INVALID unless
 *                      they are strictly ascending and in range (also set by
 *                      the environment variable SL_DEBUG=1 at sl_create).
 *   "gemm_cfg", "gemm_grp", "gemm_split", "splitk_max", "splitk_min",
 *   "lora_xl_split", "swiglu_rows", "merge_rows"
 *                      launch tuning of the GEMM and LoRA kernels (tile
 *                      configuration, tile-order group, split tail of bf16
 *                      launches and K split of fp32 launches with few tiles
 *                      on/off,
 *                      largest and smallest split-K of the dense output rows
 *                      of an input-sparse product, x A^T split form, rows per
 *                      partial of the fused SwiGLU backward, rows per wave of
 *                      the merge of a compact product); read from the
 *                      environment variables of the same names in upper case
 *                      with an SL_ prefix at sl_create.
 * Unknown names return SL_ERR_INVALID. */
sl_status sl_set_option(sl_handle* h, const char* name, int64_t value);
/* Wait for the handle's stream; reports asynchronous HIP errors. */
sl_status sl_sync(sl_handle* h);
/* Human-readable text of the last error on this handle ("" if none). */
const char* sl_last_error(const sl_handle* h);
/* Name of a status code. */
const char* sl_status_str(sl_status s);
/* Library version string. */
const char* sl_version(void);

/* ---------------------------------------------------------------- measurement */

/* While enabled, each main launch of the library (kernel classes
 * "gemm_bf16_nt", "gemm_bf16_nn", "gemm_f32", "estimate", "score", "topk",
 * "lora", "swiglu", "gather", "fill", "token_split") is bracketed by HIP
 * events recorded on the handle's stream, together with its algorithmic
 * work (flops, and HBM bytes as if every operand element were read once and
 * every result written once).  Enabling does not clear earlier records. */
sl_status sl_timing_enable(sl_handle* h, int enable);
/* Record only the launches of one kernel class from now on (NULL or "": every
 * class, the default).  Each record adds two event markers to the stream,
 * which cost time between launches; timing one class keeps that cost off the
 * other launches.  Unknown class: SL_ERR_INVALID. */
sl_status sl_timing_only(sl_handle* h, const char* kernel_class);
/* Drop all records (waits for the stream first). */
sl_status sl_timing_reset(sl_handle* h);
/* Totals over the records of one kernel class: number of launches, summed
 * event time in ms, summed algorithmic flops and bytes.  Waits for the stream.
 * Unknown class: SL_ERR_INVALID. */
sl_status sl_timing_query(sl_handle* h, const char* kernel_class, int64_t* launches,
                          double* total_ms, double* flops, double* bytes);
/* Name of kernel class i (NULL past the last). */
const char* sl_timing_class_name(int i);

/* ---------------------------------------------------------------- a1: token roles */

/* Split tokens by role (PG §3.4 "Token Sensitivity", implementation and
 * Figure 8: output tokens take the dense path, context tokens the sparse path;
 * PN "Token 敏感性").
 *   roles    device uint8[T]; 0 = context token, any other value = output token
 *   ctx_rows device int32[T_c] out: context rows, ascending
 *   out_rows device int32[T_o] out: output rows, ascending
 * T_c and T_o are the caller's counts (known from the sequence structure),
 * T_c + T_o = T.  If the roles hold a different count, the lists are written
 * only up to the given sizes and sl_sync reports SL_ERR_INVALID. */
sl_status sl_token_split(sl_handle* h, const uint8_t* roles, int64_t T,
                         int32_t* ctx_rows, int64_t T_c, int32_t* out_rows, int64_t T_o);

/* ---------------------------------------------------------------- a2: estimator stage 1 */

/* Low-rank estimator, first product (PG §3.4 "SVD Sparsity Estimator",
 * Algorithm 1 step 1: y_hat = (x W_A) W_B; PN "SVD 稀疏估计器"), context
 * tokens only:
 *   xa[m, j] = sum_i x[ctx_rows[m], i] * W_A[i, j],   m < T_c, j < k_tot,
 * summed in fp32 as R64 (64 strided fused multiply-add chains over i, then a
 * pairwise tree 32, 16, ..., 1), which fixes the result bit for bit.
 *   x        device [*, ldx] of dtype xdt (rows indexed by ctx_rows)
 *   WA       device fp32 [D_in, k_tot]: W_A in its math layout (row i holds
 *            W_A[i, :]); factors of projections that share the input are
 *            placed side by side (gate|up: 2k columns; q|k|v: 3k)
 *   xa       device fp32 [T_c, k_tot] out
 * Constraints: 1 <= k_tot <= 65535 * 16 (any rank up to the full one), D_in >= 1.
 * T_c = 0 is a no-op. */
sl_status sl_svd_estimate(sl_handle* h, const void* x, sl_dtype xdt, int64_t ldx,
                          const int32_t* ctx_rows, int64_t T_c, int64_t D_in,
                          const float* WA, int64_t k_tot, float* xa);

/* ---------------------------------------------------------------- a3+a4: score, select */

/* Estimator second product fused with the criterion, then top-n selection
 * (PG §3.4 Algorithm 1 steps 2-3; "Oracle Sparse Neuron Selection Criteria";
 * PN "L2 Norm 准则", "QK Norm 准则").
 *   y_hat[m, c] = sum_j xa[m, off + j] * WB[j, c]  (fp32 fused chain, j ascending)
 *   SL_CRIT_L2:        v = y_hat from (off0, WB0)
 *   SL_CRIT_SWIGLU_L2: v = silu(g_hat) * u_hat, g_hat from (off0, WB0),
 *                      u_hat from (off1, WB1); silu(z) = z / (1 + exp(-z)) with
 *                      the library's fixed fp32 exp (Cody-Waite reduction and a
 *                      degree-7 Taylor polynomial, within 1 ulp)
 *   ssq[c] = sum over context tokens of v^2, in R64 order over m
 *   SL_CRIT_QK: C = H_kv * head_dim (key/value channel space);
 *     WB0 = W_B of q [k, C * n_rep], WB1 = W_B of k [k, C];
 *     score[g*d + j] = (sum_r ssq_q[(g*n_rep + r)*d + j]) * ssq_k[g*d + j]
 *   otherwise score = ssq (squared norms rank like norms).
 * Selection: the n_keep channels with the largest score bit patterns (NaN
 * above +inf), equal scores ordered by lower channel index; idx is written
 * ascending.  n_keep = ceil(keep_ratio * C) is the caller's integer.
 *   xa      device fp32 [T_c, ld_xa]
 *   WB0/WB1 device fp32 [k, *] row-major (WB1 unused, may be NULL, for L2)
 *   scores  device fp32 [C] out, or NULL (then kept in the workspace)
 *   idx     device int32[n_keep] out
 * Constraints: 1 <= k <= 65536 (ranks above 64 read the factor columns
 * inside the chain: the same arithmetic, more memory traffic);
 * 0 <= n_keep <= C; n_rep >= 1 and head_dim >= 1 for QK (ignored
 * otherwise).  T_c = 0 gives all-zero scores. */
sl_status sl_score_select(sl_handle* h, sl_criterion crit, const float* xa, int64_t ld_xa,
                          int64_t T_c, int64_t off0, const float* WB0, int64_t off1,
                          const float* WB1, int64_t k, int64_t C, int64_t n_rep,
                          int64_t head_dim, int64_t n_keep, float* scores, int32_t* idx);

/* The same score selection for callers that cannot allocate device memory:
 * code being captured into a HIP graph, tight serving loops, and harnesses
 * that forbid hipMalloc.  Arguments, results and error behaviour are those of
 * sl_score_select; the scratch it needs (the scores when scores is NULL, the
 * QK criterion's two ssq vectors, chain partials of the split scoring form)
 * lives in a fixed 4 MiB device array of the library, one per device, whose
 * address is taken once per device in sl_create.  A call that would need more
 * than 4 MiB returns SL_ERR_WORKSPACE before launching anything.  The call
 * allocates nothing, records no timing events, and leaves no state that a
 * later call relies on; calls that overlap on one device (other handles or
 * streams included) share that array and race. */
sl_status sl_score_select_noalloc(sl_handle* h, sl_criterion crit, const float* xa, int64_t ld_xa,
                                  int64_t T_c, int64_t off0, const float* WB0, int64_t off1,
                                  const float* WB1, int64_t k, int64_t C, int64_t n_rep,
                                  int64_t head_dim, int64_t n_keep, float* scores, int32_t* idx);

/* ---------------------------------------------------------------- criterion variants */

/* Top-n of given scores, the selection rule of sl_score_select (largest score
 * bit patterns, NaN above +inf, ties to the lower index, idx ascending).  With
 * scores drawn at random by the caller this is the pages' random-selection
 * ablation (paper-graph summary, "Ablation Studies and Robustness Checks",
 * pruning criteria, Table 10); with sl_dense_scores it selects by the exact
 * ("oracle") criterion.  scores device fp32 [C]; idx device int32 [n_keep]
 * out; 0 <= n_keep <= C. */
sl_status sl_select_top(sl_handle* h, const float* scores, int64_t C, int64_t n_keep, int32_t* idx);

/* Scores for the random-selection ablation, from a counter-based generator:
 * scores[c] = (z_{c+1} >> 40) * 2^-24, where z_i is the i-th output of
 * SplitMix64 (Steele, Lea and Flood, 2014: state += 0x9E3779B97F4A7C15;
 * z = state; z = (z ^ z >> 30) * 0xBF58476D1CE4E5B9; z = (z ^ z >> 27) *
 * 0x94D049BB133111EB; z ^= z >> 31) started at state `seed`.  Uniform in
 * [0, 1), exact in fp32; with sl_select_top it keeps a uniformly random
 * channel subset (the caller varies the seed per step and layer).
 * scores device fp32 [C] out. */
sl_status sl_random_scores(sl_handle* h, uint64_t seed, int64_t C, float* scores);

/* The channel criteria of sl_score_select evaluated on exact outputs instead
 * of the rank-k estimate (paper-graph summary §3.4, "Oracle Sparse Neuron
 * Selection Criteria": the oracle row of Table 7; these need the dense
 * outputs, which is what the estimator avoids):
 *   SL_CRIT_L2:        v = Y0[t, c]
 *   SL_CRIT_SWIGLU_L2: v = silu(Y0[t, c]) * Y1[t, c]  (Y0 = gate, Y1 = up;
 *                      silu with the library's fixed fp32 exp)
 *   ssq[c] = R64 over m < T_c of (v, v) at t = rows[m] (the order of
 *            sl_score_select: 64 chains m mod 64, then the pairwise tree)
 *   SL_CRIT_QK: Y0 = Q [*, C n_rep], Y1 = K [*, C]; scores[g d + j] =
 *            (sum over the group's query heads of ssq_Q) * ssq_K[g d + j]
 *   otherwise scores = ssq.
 * Y0/Y1 device (dt) with leading dimensions ld0/ld1 (the main-branch outputs
 * x W^T of the frozen weight); rows device int32 [T_c] (context rows);
 * scores device fp32 [C] out.  T_c = 0 gives zeros. */
sl_status sl_dense_scores(sl_handle* h, sl_criterion crit, sl_dtype dt, const void* Y0, int64_t ld0,
                          const void* Y1, int64_t ld1, const int32_t* rows, int64_t T_c, int64_t C,
                          int64_t n_rep, int64_t head_dim, float* scores);

/* Head-level selection, the coarser alternative the pages weigh against
 * channel-level QK sparsity (paper-graph summary §3.4, "Why not head-level
 * pruning for QK?"; Table 10): head score hs[g] = sum over j < head_dim of
 * scores[g head_dim + j] (fp32, j ascending from +0); the heads_keep heads
 * with the largest hs (rule of sl_select_top) keep all their channels:
 * idx[i head_dim + j] = head_i head_dim + j, heads ascending.
 * scores device fp32 [n_heads head_dim]; idx device int32 [heads_keep
 * head_dim] out. */
sl_status sl_select_heads(sl_handle* h, const float* scores, int64_t n_heads, int64_t head_dim,
                          int64_t heads_keep, int32_t* idx);

/* ---------------------------------------------------------------- a5: index propagation */

/* Key/value-space selection -> query-space (or o-input) selection under
 * grouped-query attention: query channel (g*n_rep + r)*head_dim + j is kept
 * iff key/value channel g*head_dim + j is (PG §3.4 "VO projection sparsity":
 * indices propagate between projections sharing a channel space).
 *   idx_kv device int32[n] ascending; idx_q device int32[n * n_rep] out, ascending. */
sl_status sl_expand_gqa(sl_handle* h, const int32_t* idx_kv, int64_t n, int64_t n_rep,
                        int64_t head_dim, int32_t* idx_q);

/* Channel selection shared by stacked projections (PG §3.4 "FFN structure":
 * one index serves gate and up): idx_out[b*n + q] = idx[q] + b*C for
 * b < copies.  idx_out device int32[n * copies], ascending. */
sl_status sl_stack_index(sl_handle* h, const int32_t* idx, int64_t n, int64_t C,
                         int64_t copies, int32_t* idx_out);

/* Channel numbers of one projection inside a stack of projections with their
 * own selections (q | k | v in one stacked product, PG §3.4 "QK projection
 * sparsity" and "VO projection sparsity"): idx_out[q] = idx[q] + offset, the
 * offset being the number of rows stacked above this projection.  idx_out
 * device int32[n] (may be a slice of a larger index list); n = 0 is a no-op;
 * SL_ERR_INVALID if offset < 0 or a shifted value could exceed INT32_MAX
 * (checked as offset + C_max with C_max = max_channel + 1 supplied by the
 * caller). */
sl_status sl_offset_index(sl_handle* h, const int32_t* idx, int64_t n, int64_t offset,
                          int64_t C_max, int32_t* idx_out);

/* The three index lists of one attention block's q|k|v and o products in one
 * call (PG §3.4 "QK projection sparsity" and "VO projection sparsity": a
 * selection in key/value channel space serves every query head of its group):
 *   idx_q   = sl_expand_gqa(idx_qk)                    int32[n_qk * n_rep]
 *   idx_o   = sl_expand_gqa(idx_vo)                    int32[n_vo * n_rep]
 *   idx_qkv = [idx_q | idx_qk + Cq | idx_vo + Cq + Ckv] int32[n_qk * n_rep + n_qk + n_vo]
 * with Ckv = n_kv_heads * head_dim, Cq = n_rep * Ckv.  idx_qk, idx_vo: device
 * int32, ascending, values < Ckv; every output list is ascending and device
 * memory the caller owns.  n_qk = n_vo = 0 is a no-op; SL_ERR_INVALID for bad
 * sizes (n > Ckv, Cq + 2 Ckv > INT32_MAX) or NULL pointers of a non-empty
 * part. */
sl_status sl_qkv_index(sl_handle* h, const int32_t* idx_qk, int64_t n_qk, const int32_t* idx_vo, int64_t n_vo,
                       int64_t n_kv_heads, int64_t n_rep, int64_t head_dim, int32_t* idx_q, int32_t* idx_o,
                       int32_t* idx_qkv);

/* ---------------------------------------------------------------- a6/a7: main forward */

/* Sparse main-branch forward (PG §3.4 Algorithm 1 steps 4-5 and "Token
 * Sensitivity" implementation; §3.4 "Preliminary": dropped channels are zero):
 *   output rows:  y[t, :] = x[t, :] W^T                       (dense)
 *   context rows, side OUT: y[t, c] = x[t, :] . W[c, :] for c in idx, 0 else
 *   context rows, side IN:  y[t, :] = sum_{c in idx} x[t, c] Wt[c, :]
 * computed as gathered-channel GEMMs (only the selected weight rows are read
 * for context rows).  beta = 1 adds into y instead of overwriting.
 * Optional fused dense LoRA term (Algorithm 1 step 6), lora_P != NULL:
 *   y[t, o] += lora_scale * sum_{j < lora_r} lora_P[t, j] * lora_B[o, j]
 * on every row and every output channel, accumulated in fp32 before the one
 * rounding of y; the unselected channels of context rows (side OUT) then hold
 * this term instead of 0.  lora_P: device fp32 [T, ld_lora_P] (xl = x A^T);
 * lora_B: device (dt) [D_out, ld_lora_B] (the LoRA B).  1 <= lora_r <= 128.
 *   x   device [T, ldx] (dt), channels of side IN are its columns
 *   W   device (dt) [D_out, ldw >= D_in], nn.Linear layout
 *   Wt  device (dt) [D_in, ldwt >= D_out], W transposed; read only for side IN
 *       (its selected rows form the context-row slice), may be NULL otherwise
 *   ctx_rows/out_rows  device int32 row lists (sl_token_split)
 *   idx device int32[n], ascending, in [0, C), C = D_out (OUT) or D_in (IN)
 *   y   device [T, ldy] (dt) out
 *   w_slice  optional (side IN only): the context-row weight slice built
 *       beforehand by sl_weight_slice from Wt and the same idx, dt
 *       [D_out, ld_w_slice >= ceil8(n)]; NULL builds it inside the call
 *   x_slice  optional (side IN only): the context rows' selected input
 *       channels given compactly, x_slice[m, j] = x[ctx_rows[m], idx[j]],
 *       dt [T_c, ld_x_slice >= ceil8(n)] with columns n .. ceil8(n) zero (as
 *       sl_swiglu_fwd_ctx writes it); NULL gathers them from x inside the call
 *   flags  SL_NO_FILL (side OUT: the unselected channels of context rows
 *       are left unwritten; with lora_P they must be written by
 *       sl_lora_fill_unselected, without it the caller zeroes them), and at
 *       most one of SL_ONLY_OUT_ROWS / SL_ONLY_CTX_ROWS (side OUT: one of the
 *       two row sets per call; the two calls together compute what one call
 *       without them computes, up to the order of fp32 accumulation), and
 *       SL_CTX_COMPACT with SL_ONLY_CTX_ROWS (side OUT, bf16: the compact
 *       context-row product, see the flag)
 * dt = SL_BF16 (MFMA path) or SL_F32. */
sl_status sl_sparse_linear_fwd(sl_handle* h, sl_side side, sl_dtype dt,
                               const void* x, int64_t ldx, int64_t T, int64_t D_in,
                               const void* W, int64_t ldw, const void* Wt, int64_t ldwt,
                               int64_t D_out,
                               const int32_t* ctx_rows, int64_t T_c,
                               const int32_t* out_rows, int64_t T_o,
                               const int32_t* idx, int64_t n,
                               void* y, int64_t ldy, int beta,
                               const float* lora_P, int64_t ld_lora_P,
                               const void* lora_B, int64_t ld_lora_B,
                               int64_t lora_r, float lora_scale,
                               const void* w_slice, int64_t ld_w_slice,
                               const void* x_slice, int64_t ld_x_slice, int flags);

/* ---------------------------------------------------------------- a10/a11: main backward */

/* Input gradient of sl_sparse_linear_fwd with the selection held fixed (PG
 * §3.2 "Information flow during a backward pass": gradients flow only
 * through the active channels; the frozen weight receives none):
 *   output rows:  dx[t, :] = dy[t, :] W                        (dense)
 *   context rows, side OUT: dx[t, :] = sum_{c in idx} dy[t, c] W[c, :]
 *   context rows, side IN:  dx[t, c] = dy[t, :] . Wt[c, :] for c in idx, 0 else
 *   dy  device [T, lddy] (dt); Wt device (dt) [D_in, ldwt >= D_out] (read by
 *       every backward product); W device (dt) [D_out, ldw >= D_in], read only
 *       for side OUT (its selected rows form the context-row slice)
 *   dx  device [T, lddx] (dt) out; beta = 1 accumulates.
 * Optional fused LoRA input-gradient term, lora_P != NULL:
 *   dx[t, i] += lora_scale * sum_j lora_P[t, j] * lora_B[i, j]
 * with lora_P = gB = dy B (fp32 [T, ld], from sl_lora_fwd_bwd) and
 * lora_B = A^T (dt [D_in, ld]); unselected context channels (side IN) then
 * hold this term instead of 0.
 *   w_slice  optional (side OUT only): sl_weight_slice of W with the same idx,
 *       dt [D_in, ld_w_slice >= ceil8(n)]; NULL builds it inside the call
 *   x_slice  optional (side OUT only): dy's context rows at the selected
 *       channels, compact and zero-padded as for the forward; NULL gathers
 *   flags  as for the forward, with side IN in place of side OUT
 *       (SL_NO_FILL, SL_ONLY_OUT_ROWS, SL_ONLY_CTX_ROWS, SL_CTX_COMPACT) */
sl_status sl_sparse_linear_bwd(sl_handle* h, sl_side side, sl_dtype dt,
                               const void* dy, int64_t lddy, int64_t T, int64_t D_out,
                               const void* W, int64_t ldw, const void* Wt, int64_t ldwt,
                               int64_t D_in,
                               const int32_t* ctx_rows, int64_t T_c,
                               const int32_t* out_rows, int64_t T_o,
                               const int32_t* idx, int64_t n,
                               void* dx, int64_t lddx, int beta,
                               const float* lora_P, int64_t ld_lora_P,
                               const void* lora_B, int64_t ld_lora_B,
                               int64_t lora_r, float lora_scale,
                               const void* w_slice, int64_t ld_w_slice,
                               const void* x_slice, int64_t ld_x_slice, int flags);

/* Context-row weight slice of a sparse product, built ahead of the product
 * (e.g. on another stream right after the selection) so the product itself
 * only gathers the activations (PG §3.4 Algorithm 1 step 5, the sliced
 * matmul; the slice is its weight operand):
 *   out[o, j] = Wc[idx[j], o] for j < n,  out[o, j] = 0 for n <= j < ceil8(n)
 * for o < Nout.  Wc device (dt) [C, ldwc >= Nout] (channel-major: Wt for a
 * forward side IN product, W for a backward side OUT product); idx device
 * int32[n] ascending in [0, C), 1 <= n; out device (dt) [Nout, ld_out >=
 * ceil8(n)].  dt = SL_BF16 or SL_F32. */
sl_status sl_weight_slice(sl_handle* h, sl_dtype dt, const void* Wc, int64_t ldwc, int64_t C,
                          const int32_t* idx, int64_t n, int64_t Nout, void* out,
                          int64_t ld_out);

/* The unselected channels of context rows of a side-OUT-shaped sparse product
 * run with SL_NO_FILL: for t in ctx_rows and c not in idx,
 *   y[t, c] = bf16(lora_scale * sum_{j < lora_r} lora_P[t, j] * lora_B[c, j])
 * (the dense LoRA term alone, as the fused product would write them); the
 * selected channels are not touched, so this may run on another stream
 * concurrently with the product.  y bf16 [T, ldy >= C]; lora_P fp32 [T,
 * ld_lora_P]; lora_B bf16 [C, ld_lora_B]; 1 <= lora_r <= 128.  bf16 only. */
sl_status sl_lora_fill_unselected(sl_handle* h, sl_dtype dt, void* y, int64_t ldy,
                                  const int32_t* ctx_rows, int64_t T_c, int64_t C,
                                  const float* lora_P, int64_t ld_lora_P, const void* lora_B,
                                  int64_t ld_lora_B, int64_t lora_r, float lora_scale,
                                  const int32_t* idx, int64_t n);

/* ---------------------------------------------------------------- estimator factors */

/* Rank-k estimator factors of a frozen weight, computed on the GPU (the
 * offline step of paper-graph summary §3.4 "SVD Sparsity Estimator": W_A =
 * U_k sqrt(S_k), W_B = sqrt(S_k) V_k^T from the truncated SVD of W = W_lin^T
 * [D_in, D_out]).  Randomized subspace iteration (Halko, Martinsson and
 * Tropp, 2011): Omega [D_out, p] standard normal from a counter-based
 * generator (SplitMix64 uniforms, Box-Muller) seeded by `seed`, p = k +
 * oversample; Q = orth(W Omega); `iters` power steps Z = orth(W^T Q), Q =
 * orth(W Z) (orth = CholeskyQR2); then the SVD of Q^T W through the
 * eigen-decomposition of its Gram matrix (Jacobi, fp64).  Each singular pair
 * is signed so that the largest-magnitude entry of its left vector is
 * positive.  The result approaches the truncated SVD as iters grows (exactly
 * on a planted spectrum with a gap at k).
 *   W  device (dt) [D_out, ldw >= D_in] (nn.Linear layout); Wt its transposed
 *      copy [D_in, ldwt >= D_out]
 *   WA_t device fp32 [k, D_in] out (W_A transposed: the layout sl_svd_estimate
 *      reads after a transpose to [D_in, k]); WB device fp32 [k, D_out] out
 * 1 <= k, k + oversample <= 64 and <= min(D_in, D_out); iters <= 16. */
sl_status sl_svd_factors(sl_handle* h, sl_dtype dt, const void* W, int64_t ldw, const void* Wt, int64_t ldwt,
                         int64_t D_out, int64_t D_in, int64_t k, int64_t oversample, int64_t iters,
                         uint64_t seed, float* WA_t, float* WB);

/* ---------------------------------------------------------------- training step */

/* Token loss on the listed rows (paper-graph summary, "Putting It All
 * Together": only the target positions enter the objective, as in ordinary
 * next-token fine-tuning): for m < n_rows, t = rows[m], z = logits[t, 0:V],
 * y = labels[t],
 *   row loss   = logsumexp(z) - z[y]                       (fp32, max-shifted)
 *   dlogits[t, c] = scale * (softmax(z)[c] - [c == y])     (dt)
 *   *loss      = scale * sum of the row losses             (fp64, fixed order)
 * A label outside [0, V) (an ignore index such as -100) marks its row as
 * ignored: row loss 0 and dlogits[t, :] = 0.  scale = 1 / (number of rows
 * with a label in range) gives the mean loss and its gradient.  Rows not
 * listed are not touched.  logits, dlogits device (dt) [*, ld >= V]; rows device
 * int32 [n_rows]; labels device int32 [*] (indexed by row); loss device fp64
 * [1] out.  dt = SL_BF16 or SL_F32. */
sl_status sl_token_ce(sl_handle* h, sl_dtype dt, const void* logits, int64_t ld, const int32_t* rows,
                      int64_t n_rows, const int32_t* labels, int64_t V, float scale, void* dlogits,
                      int64_t ld_d, double* loss);

/* One AdamW step (decoupled weight decay) on up to 16 tensors (paper-graph
 * summary, "Putting It All Together": only the LoRA parameters are updated),
 * elementwise in fp32:
 *   p = p * (1 - lr wd);  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2
 *   p = p - lr * (m / bc1) / (sqrt(v / bc2) + eps),  bc_i = 1 - b_i^step
 * then, if out is set, out[r, c] = p[r cols + c] rounded to out_dtype (the
 * copy the sparse products read).  param/grad/m/v: device fp32 [rows * cols],
 * contiguous; out: device (out_dtype) [rows, ld_out >= cols] or NULL.  step >= 1
 * (the number of this update); lr is the caller's scheduled rate. */
typedef struct {
    float* param;
    const float* grad;
    float* m;
    float* v;
    void* out;
    int64_t ld_out;
    int64_t rows;
    int64_t cols;
    sl_dtype out_dtype;
} sl_adamw_tensor;
sl_status sl_adamw_step(sl_handle* h, const sl_adamw_tensor* tensors, int n, float lr, float beta1,
                        float beta2, float eps, float weight_decay, int64_t step);

/* ---------------------------------------------------------------- gradient fidelity */

/* Dot statistics of two fp32 vectors, for the cosine between a sparse and a
 * dense gradient of the same LoRA adapter (paper-graph summary, "Follow-Up
 * Research This Work Enables": gradient cosine similarity as a fidelity
 * measure of training sparsity):
 *   out[0] = sum a[i] b[i],  out[1] = sum a[i]^2,  out[2] = sum b[i]^2
 * over i < n, in fp64 with every product exact and a fixed summation order
 * (the result does not depend on timing).  a, b device fp32 [n] (4-byte
 * aligned, contiguous); out device fp64 [3] (8-byte aligned).  n = 0 gives
 * zeros. */
sl_status sl_dot_stats(sl_handle* h, const float* a, const float* b, int64_t n, double* out);

/* ---------------------------------------------------------------- a8/a12: dense LoRA */

/* Dense LoRA branch on every token and channel (PG §3.4 Algorithm 1 step 6:
 * y_final = y_sparse + B A x; §3.2: LoRA gradients are always computed fully).
 * A [r, D_in], B [D_out, r] (dt, contiguous), scale = alpha / r.
 *   SL_LORA_XL:  xl = x A^T                       (xl fp32 [T, ldxl], out)
 *   SL_LORA_ADD: y += scale * xl B^T               (y dt [T, ldy], in/out)
 *   SL_LORA_GB:  gB = dy B                         (gB fp32 [T, ldgB] out; if gB
 *                                                   is NULL it stays internal)
 *   SL_LORA_DA:  dA = scale gB^T x                 (fp32 [r, D_in] out; gB from
 *                                                   this call or given)
 *   SL_LORA_DB:  dB = scale dy^T xl                (fp32 [D_out, r] out)
 *   SL_LORA_DX:  dx += scale gB A                  (dt [T, lddx]); leave it out
 *                and pass gB to sl_sparse_linear_bwd to fuse that term there
 * Modes combine; the steps run in the order listed.  Pointers not used by the
 * mode may be NULL.  SL_LORA_BT: B holds B^T, row-major [r, ld] with ld = D_out
 * rounded up to a multiple of 8 (a caller that keeps the transposed copy
 * saves the per-call transpose; not with ADD).
 * 1 <= r <= 128 (r <= 64 with ADD or DX; ranks above 64
 * run as column chunks of 64).  dA / dB are deterministic (fixed-order token
 * reduction). */
sl_status sl_lora_fwd_bwd(sl_handle* h, int mode, sl_dtype dt,
                          const void* x, int64_t ldx, int64_t T, int64_t D_in, int64_t D_out,
                          const void* A, const void* B, int64_t r, float scale,
                          float* xl, int64_t ldxl, void* y, int64_t ldy,
                          const void* dy, int64_t lddy, void* dx, int64_t lddx,
                          float* dA, float* dB, float* gB, int64_t ldgB);

/* ---------------------------------------------------------------- support (glue) */

/* SwiGLU (PG §3.4 "FFN structure"): h = silu(g) * u (fp32 math, dt storage).
 * g, u, h: device [T, ld*] with F columns. */
sl_status sl_swiglu_fwd(sl_handle* h, sl_dtype dt, const void* g, int64_t ldg,
                        const void* u, int64_t ldu, int64_t T, int64_t F,
                        void* hout, int64_t ldh);
/* dg = dh * u * silu'(g), du = dh * silu(g). */
sl_status sl_swiglu_bwd(sl_handle* h, sl_dtype dt, const void* dh, int64_t lddh,
                        const void* g, int64_t ldg, const void* u, int64_t ldu,
                        int64_t T, int64_t F, void* dg, int64_t lddg, void* du, int64_t lddu);
/* SwiGLU forward fused with the LoRA down-projection of the down projection
 * (PG §3.4 "FFN structure"; Algorithm 1 step 6: the LoRA branch is dense, so
 * its input is the whole hidden state h):
 *   h = silu(g) * u                  (exactly as sl_swiglu_fwd, stored in dt)
 *   xl[t, j] = sum_c h[t, c] A[j, c] (fp32, from the stored h; as SL_LORA_XL)
 * so h is read once.  rows: NULL for all T rows, else the n_rows listed rows
 * (e.g. the output rows of a sparse FFN; each row index < T).  A [r, lda >=
 * F] (dt) is the down projection's LoRA A; xl fp32 [T, ldxl >= r] out (the
 * processed rows).  bf16 only (SL_ERR_UNSUPPORTED otherwise),
 * F % 8 == 0, 1 <= r <= 32.  xl's sum is a fixed-order reduction over column
 * blocks (deterministic). */
sl_status sl_swiglu_fwd_lora(sl_handle* h, sl_dtype dt, const void* g, int64_t ldg,
                             const void* u, int64_t ldu, int64_t T, int64_t F,
                             const int32_t* rows, int64_t n_rows,
                             void* hout, int64_t ldh, const void* A, int64_t lda, int64_t r,
                             float* xl, int64_t ldxl);
/* The same pass for the context rows of a sparse SwiGLU FFN, from the compact
 * gate|up product (PG §3.4 Algorithm 1 steps 5-6 and "FFN structure": the
 * context rows' gate and up outputs are the selected channels' products, the
 * dense LoRA term alone at the others; "Token Sensitivity": output rows are
 * dense and take sl_swiglu_fwd_lora):  for m < T_c, t = ctx_rows[m], c < F,
 *   g[t, c] = Yc[m, j] if c = idx[j], else lora_scale * P[t, :] . B[c, :]
 *   u[t, c] = Yc[m, n + j] if c = idx[j], else lora_scale * P[t, :] . B[F + c, :]
 *     (the rank-r values formed exactly as the SL_LORA fill/merge of a sparse
 *     product forms them: s P rounded to dt, fp32 accumulation, one rounding),
 *     stored to gu[t, c] and gu[t, F + c] (the backward reads them);
 *   h = silu(g) u (exactly as sl_swiglu_fwd), of which only the selected
 *     channels are stored: hc[m, j] = h[t, idx[j]], columns n .. ceil8(n) of
 *     hc zero (the x_slice of the down product);
 *   xl[t, :] = sum over every channel c of h[t, c] A[:, c] (fp32, as
 *     sl_swiglu_fwd_lora);
 *   h_rows[t, :] = h[t, :] when h_rows is not NULL (whole rows; a check of
 *     the pass, not needed by the FFN: the down product reads hc).
 * Yc: dt [T_c, ldyc >= 2n], the SL_CTX_COMPACT product of the gate|up weight
 * [2F, D] with the stacked selection (idx, idx + F); P fp32 [T, ld_P] (x A^T
 * of gate|up), B dt [2F, ld_B] (the block-diagonal gate|up LoRA B, 2r ranks);
 * gu dt [T, ldgu >= 2F]; hc dt [T_c, ldhc >= ceil8(n)]; A dt [r, lda >= F]
 * (the down projection's LoRA A); xl fp32 [T, ldxl >= r] (rows t = ctx_rows[m]
 * written).  bf16 only, F % 8 == 0, lora_r = 2r <= 64, r <= 32. */
sl_status sl_swiglu_fwd_ctx(sl_handle* h, sl_dtype dt, const void* Yc, int64_t ldyc,
                            const int32_t* ctx_rows, int64_t T_c, int64_t T, int64_t F,
                            const int32_t* idx, int64_t n,
                            const float* lora_P, int64_t ld_lora_P, const void* lora_B,
                            int64_t ld_lora_B, int64_t lora_r, float lora_scale,
                            void* gu, int64_t ldgu, void* hc, int64_t ldhc,
                            const void* A, int64_t lda, int64_t r, float* xl, int64_t ldxl,
                            void* h_rows, int64_t ld_h_rows);
/* SwiGLU backward fused with the three LoRA gradient reductions that read the
 * same tensors (PG §3.2 "Information flow during a backward pass": the LoRA
 * gradients are computed in full; §3.4 "FFN structure"):
 *   dg, du                     exactly as sl_swiglu_bwd (stored in dt)
 *   dA[j, c]   = scale * sum_t gB[t, j] h[t, c]     (h = silu(g) u recomputed
 *                                                     exactly as the forward
 *                                                     stored it; the down
 *                                                     projection's dA)
 *   dB_g[c, j] = scale * sum_t dg[t, c] xl_g[t, j]  (gate's dB, from stored dg)
 *   dB_u[c, j] = scale * sum_t du[t, c] xl_u[t, j]  (up's dB, from stored du)
 * so dh, g and u are read once and dg, du are not read back.  gB fp32 [T,
 * ldgB] (the down projection's dy B_down), xl_g / xl_u fp32 [T, ld >= r] (the
 * gate and up x A^T); dA fp32 [r, F], dB_g / dB_u fp32 [F, r] (contiguous,
 * out, the layouts of SL_LORA_DA / SL_LORA_DB).  bf16 only, F % 8 == 0,
 * 1 <= r <= 32; the token sums are fixed-order reductions over row chunks
 * (deterministic). */
sl_status sl_swiglu_bwd_lora(sl_handle* h, sl_dtype dt, const void* dh, int64_t lddh,
                             const void* g, int64_t ldg, const void* u, int64_t ldu,
                             int64_t T, int64_t F, void* dg, int64_t lddg, void* du, int64_t lddu,
                             const float* gB, int64_t ldgB, const float* xl_g, int64_t ldxlg,
                             const float* xl_u, int64_t ldxlu, int64_t r, float scale,
                             float* dA, float* dB_g, float* dB_u);
/* out[j, i] = in[i, j]; in [rows, ldi], out [cols, ldo] (dt). */
sl_status sl_transpose(sl_handle* h, sl_dtype dt, const void* in, int64_t ldi,
                       int64_t rows, int64_t cols, void* out, int64_t ldo);

/* ---------------------------------------------------------------- a14: decoder-layer glue
 * Support steps between the sparse linears of a decoder layer (the pages'
 * LLaMA layers; topology here: pre-norm, residual adds, plain causal softmax
 * attention with scale 1/sqrt(d), no position encoding, grouped-query heads).
 * fp32 arithmetic; dt storage. */

/* RMSNorm with unit weight: hsum = x + res (res optional; when hsum != NULL
 * the sum is stored there, rounded to dt, and the norm reads the stored
 * value), rstd[t] = 1 / sqrt(mean_j hsum[t, j]^2 + eps) (fp32 [T], caller
 * owned), y = hsum * rstd.  All matrices [T, D] with leading dimensions. */
sl_status sl_rmsnorm_fwd(sl_handle* h, sl_dtype dt, const void* x, int64_t ldx, const void* res,
                         int64_t ldres, int64_t T, int64_t D, float eps, void* hsum, int64_t ldh,
                         void* y, int64_t ldy, float* rstd);
/* Gradient of sl_rmsnorm_fwd with respect to its normalised input x (the
 * stored hsum when a residual was fused): dx = rstd dy - rstd^3 x (dy . x) / D,
 * plus dres when dres != NULL (the residual branch's gradient). */
sl_status sl_rmsnorm_bwd(sl_handle* h, sl_dtype dt, const void* x, int64_t ldx, const float* rstd,
                         const void* dy, int64_t lddy, const void* dres, int64_t lddres, int64_t T,
                         int64_t D, void* dx, int64_t lddx);
/* out = a + b, [T, D] (residual adds); out may alias a or b. */
sl_status sl_add(sl_handle* h, sl_dtype dt, const void* a, int64_t lda, const void* b, int64_t ldb,
                 int64_t T, int64_t D, void* out, int64_t ldo);
/* Causal softmax attention per sequence and query head.  q [batch*seq,
 * n_heads*head_dim], k, v [batch*seq, n_kv_heads*head_dim], rows sequence-
 * major; query head h reads key/value head h / (n_heads / n_kv_heads).
 * o [batch*seq, n_heads*head_dim]; lse fp32 [batch, n_heads, seq] receives
 * the log of each softmax denominator (with its max) for the backward pass.
 * head_dim 32, 64 or 128; n_heads a multiple of n_kv_heads. */
sl_status sl_attention_fwd(sl_handle* h, sl_dtype dt, const void* q, int64_t ldq, const void* k,
                           int64_t ldk, const void* v, int64_t ldv, int64_t batch, int64_t seq,
                           int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, void* o,
                           int64_t ldo, float* lse);
/* Gradients of sl_attention_fwd for upstream dout (softmax probabilities
 * recomputed from lse): dq, and dk, dv summed over the query heads that read
 * each key/value head.  Uses the handle's workspace: batch*n_heads*seq*4
 * bytes (per-row softmax terms) rounded up to 256, plus for bf16
 * batch*n_heads*seq*ceil64(seq)*2 bytes (the dS tiles handed from the dK/dV
 * pass to the dQ pass; 1 GiB at batch 4, 32 heads, seq 2048) -- reserve that
 * much with sl_reserve_workspace to keep the call allocation-free. */
sl_status sl_attention_bwd(sl_handle* h, sl_dtype dt, const void* q, int64_t ldq, const void* k,
                           int64_t ldk, const void* v, int64_t ldv, const void* o, int64_t ldo,
                           const void* dout, int64_t lddout, const float* lse, int64_t batch,
                           int64_t seq, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                           void* dq, int64_t lddq, void* dk, int64_t lddk, void* dv, int64_t lddv);

#ifdef __cplusplus
}
#endif
#endif /* SPARSELORA_H */
