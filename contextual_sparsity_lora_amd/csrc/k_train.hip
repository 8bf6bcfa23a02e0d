// Training-step kernels around the sparse path: the token loss on output
// rows (softmax cross-entropy over a vocabulary) with its gradient, and the
// AdamW update of the LoRA parameters.
//
// Pages (all titled "SparseLoRA: Accelerating LLM Fine-Tuning with Contextual
// Sparsity"): paper-graph summary, "Putting It All Together": the training
// objective counts the target (output) positions alone, as in ordinary
// next-token fine-tuning, and the adapters' A and B are the only trained
// parameters; "Interaction with the
// learning rate schedule": cosine schedule with a 4 % warm-up (the rate is the
// caller's scalar per step).
#include "sl_internal.h"

namespace {

constexpr int CE_T = 256;   // threads per row block

__device__ __forceinline__ float ldl(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float ldl(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void stl(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void stl(float* p, int64_t i, float v) { p[i] = v; }

// Block-wide max / sum over CE_T threads (pairwise tree in LDS, fixed order).
template <typename Op>
__device__ __forceinline__ float block_tree(float v, float* sh, Op op) {
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int w = CE_T / 2; w >= 1; w >>= 1) {
        if (tid < w) sh[tid] = op(sh[tid], sh[tid + w]);
        __syncthreads();
    }
    const float r = sh[0];
    __syncthreads();
    return r;
}

// Row m of the listed rows: t = rows[m], logits z = L[t, 0:V], label y = labels[t].
//   loss[m] = logsumexp(z) - z[y]   (fp32, max-shifted)
//   dL[t, c] = scale * (softmax(z)[c] - [c == y])
// A label outside [0, V) (an ignore index such as -100) marks the row as
// ignored: loss[m] = 0 and dL[t, :] = 0; z is then not read at all.
// Thread i takes columns i, i + CE_T, ... (fixed order), then the block tree.
template <typename T>
__global__ __launch_bounds__(CE_T) void ce_rows_kernel(const T* __restrict__ L, int64_t ldl_,
                                                       const int32_t* __restrict__ rows,
                                                       const int32_t* __restrict__ labels, int64_t V,
                                                       float scale, T* __restrict__ dL, int64_t lddl,
                                                       float* __restrict__ loss) {
    __shared__ float sh[CE_T];
    const int64_t t = rows[blockIdx.x];
    const T* z = L + t * ldl_;
    const int tid = threadIdx.x;
    const int64_t y = labels[t];
    T* d = dL + t * lddl;
    if (y < 0 || y >= V) {   // ignored row (uniform across the block)
        if (tid == 0) loss[blockIdx.x] = 0.0f;
        for (int64_t c = tid; c < V; c += CE_T) stl(d, c, 0.0f);
        return;
    }
    float mx = -__builtin_huge_valf();
    for (int64_t c = tid; c < V; c += CE_T) mx = fmaxf(mx, ldl(z, c));
    mx = block_tree(mx, sh, [](float a, float b) { return fmaxf(a, b); });
    float s = 0.0f;
    for (int64_t c = tid; c < V; c += CE_T) s += expf(ldl(z, c) - mx);
    s = block_tree(s, sh, [](float a, float b) { return a + b; });
    const float lse = mx + logf(s);
    if (tid == 0) loss[blockIdx.x] = lse - ldl(z, y);
    for (int64_t c = tid; c < V; c += CE_T) {
        const float p = expf(ldl(z, c) - lse);
        stl(d, c, scale * (p - (c == y ? 1.0f : 0.0f)));
    }
}

// loss_out[0] = scale * sum of the row losses (fp64, one block, fixed order).
__global__ __launch_bounds__(256) void ce_sum_kernel(const float* __restrict__ loss, int64_t n,
                                                     double scale, double* __restrict__ out) {
    __shared__ double sh[256];
    const int tid = threadIdx.x;
    double s = 0.0;
    for (int64_t i = tid; i < n; i += 256) s += (double)loss[i];
    sh[tid] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (tid < w) sh[tid] += sh[tid + w];
        __syncthreads();
    }
    if (tid == 0) out[0] = scale * sh[0];
}

// AdamW (decoupled weight decay) over up to SL_ADAMW_MAXT tensors in one
// launch; block b works on the tensor whose block range holds b.
__global__ __launch_bounds__(256) void adamw_kernel(AdamwArgs a) {
    int i = 0;
#pragma unroll
    for (int q = 1; q < SL_ADAMW_MAXT; ++q)
        if (q < a.n && (int64_t)blockIdx.x >= a.t[q].first_block) i = q;
    AdamwTensor ten;
#pragma unroll
    for (int q = 0; q < SL_ADAMW_MAXT; ++q)
        if (q == i) ten = a.t[q];
    const int64_t e = ((int64_t)blockIdx.x - ten.first_block) * 256 + threadIdx.x;
    const int64_t count = ten.rows * ten.cols;
    if (e >= count) return;
    const int64_t r = e / ten.cols, c = e % ten.cols;
    const float g = ten.g[e];
    float p = ten.p[e];
    p = p * (1.0f - a.lr * a.wd);
    const float m = a.b1 * ten.m[e] + (1.0f - a.b1) * g;
    const float v = a.b2 * ten.v[e] + (1.0f - a.b2) * g * g;
    ten.m[e] = m;
    ten.v[e] = v;
    const float mh = m / a.bc1, vh = v / a.bc2;
    p = p - a.lr * mh / (sqrtf(vh) + a.eps);
    ten.p[e] = p;
    if (ten.out) {
        if (ten.out_f32) ((float*)ten.out)[r * ten.ld_out + c] = p;
        else ((bf16_t*)ten.out)[r * ten.ld_out + c] = f32_to_bf16(p);
    }
}

}  // namespace

hipError_t launch_ce_rows(bool bf16, const void* L, int64_t ldl, const int32_t* rows, int64_t nrows,
                          const int32_t* labels, int64_t V, float scale, void* dL, int64_t lddl,
                          float* loss_rows, double* loss_sum, hipStream_t st) {
    // no rows: the sum kernel alone writes a zero loss
    if (nrows > 0 && bf16)
        hipLaunchKernelGGL(ce_rows_kernel<bf16_t>, dim3((unsigned)nrows), dim3(CE_T), 0, st, (const bf16_t*)L, ldl,
                           rows, labels, V, scale, (bf16_t*)dL, lddl, loss_rows);
    else if (nrows > 0)
        hipLaunchKernelGGL(ce_rows_kernel<float>, dim3((unsigned)nrows), dim3(CE_T), 0, st, (const float*)L, ldl,
                           rows, labels, V, scale, (float*)dL, lddl, loss_rows);
    hipLaunchKernelGGL(ce_sum_kernel, dim3(1), dim3(256), 0, st, loss_rows, nrows, (double)scale, loss_sum);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamwArgs& a, int64_t blocks, hipStream_t st) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}
