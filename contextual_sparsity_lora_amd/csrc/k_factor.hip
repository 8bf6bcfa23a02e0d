// Rank-k estimator factors on the GPU: randomized subspace iteration on the
// frozen weight, then the SVD of the small projected matrix (Halko,
// Martinsson and Tropp, 2011: the range finder with power iterations and
// re-orthonormalisation, and the direct SVD of the projection).
//
// Pages (all titled "SparseLoRA: Accelerating LLM Fine-Tuning with Contextual
// Sparsity"): paper-graph summary §3.4 "SVD Sparsity Estimator": offline,
// the weight's truncated SVD gives W_A = U_k sqrt(S_k) and W_B = sqrt(S_k)
// V_k^T, and y_hat = (x W_A) W_B approximates x W.
//
// W = W_lin^T [D_in, D_out] (math layout).  With p = k + oversample columns:
//   Y = W Omega, Q = orth(Y); per power step: Z = orth(W^T Q), Q = orth(W Z);
//   Z = W^T Q; G = Z^T Z = Ub diag(lambda) Ub^T (Jacobi, fp64);
//   s = sqrt(lambda), U = Q Ub, V = Z Ub / s  (top k, descending);
//   sign: the largest-magnitude entry of each U column positive (first on ties);
//   W_A^T[j, :] = sqrt(s_j) U[:, j]^T, W_B[j, :] = sqrt(s_j) V[:, j]^T.
// orth() is CholeskyQR2: R = chol(Y^T Y), Y <- Y R^-1, twice.
#include <cmath>

#include "sl_internal.h"

namespace {

constexpr int FK_ROWS = 16;   // rows of A per block in the skinny product
constexpr int FK_KC = 64;     // K chunk staged in LDS
constexpr int FK_PMAX = 64;   // max columns p

__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Omega[e] ~ N(0, 1): Box-Muller on two SplitMix64 uniforms in (0, 1).
__global__ void omega_kernel(uint64_t seed, int64_t n, float* __restrict__ om) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    const uint64_t g = 0x9E3779B97F4A7C15ull;
    const double u1 = ((double)(mix64(seed + (uint64_t)(2 * e + 1) * g) >> 11) + 0.5) * 0x1p-53;
    const double u2 = ((double)(mix64(seed + (uint64_t)(2 * e + 2) * g) >> 11) + 0.5) * 0x1p-53;
    om[e] = (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

// C[M, p] = A[M, K] B[K, p]: A row-major (dt), B, C fp32 row-major (ld = p).
// Block = 256 threads over FK_ROWS rows; thread t owns row t / 16 and columns
// (t % 16) + 16 c; K in FK_KC chunks through LDS, sums in K order.
template <typename T>
__global__ __launch_bounds__(256) void skinny_kernel(const T* __restrict__ A, int64_t lda, int64_t M,
                                                     int64_t K, const float* __restrict__ B, int p,
                                                     float* __restrict__ C) {
    __shared__ float as[FK_ROWS][FK_KC + 1];
    __shared__ float bs[FK_KC][FK_PMAX];
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.x * FK_ROWS;
    const int r = tid / 16, cl = tid % 16;
    float acc[FK_PMAX / 16];
#pragma unroll
    for (int c = 0; c < FK_PMAX / 16; ++c) acc[c] = 0.0f;
    for (int64_t k0 = 0; k0 < K; k0 += FK_KC) {
        for (int q = tid; q < FK_ROWS * FK_KC; q += 256) {
            const int rr = q / FK_KC, kk = q % FK_KC;
            const int64_t m = m0 + rr, k = k0 + kk;
            as[rr][kk] = (m < M && k < K) ? ldf(A, m * lda + k) : 0.0f;
        }
        for (int q = tid; q < FK_KC * FK_PMAX; q += 256) {
            const int kk = q / FK_PMAX, c = q % FK_PMAX;
            const int64_t k = k0 + kk;
            bs[kk][c] = (k < K && c < p) ? B[k * p + c] : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < FK_KC; ++kk) {
            const float a = as[r][kk];
#pragma unroll
            for (int c = 0; c < FK_PMAX / 16; ++c) acc[c] = fmaf(a, bs[kk][cl + 16 * c], acc[c]);
        }
        __syncthreads();
    }
    const int64_t m = m0 + r;
    if (m < M)
#pragma unroll
        for (int c = 0; c < FK_PMAX / 16; ++c)
            if (cl + 16 * c < p) C[m * p + cl + 16 * c] = acc[c];
}

// Partial Gram matrices: block b sums rows [b R, (b+1) R) of Y [M, p] (fp64).
__global__ __launch_bounds__(256) void gram_partial_kernel(const float* __restrict__ Y, int64_t M, int p,
                                                           int64_t rows_per_block, double* __restrict__ part) {
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < M ? r0 + rows_per_block : M;
    for (int e = threadIdx.x; e < p * p; e += 256) {
        const int i = e / p, j = e % p;
        double s = 0.0;
        if (j >= i)
            for (int64_t m = r0; m < r1; ++m) s = fma((double)Y[m * p + i], (double)Y[m * p + j], s);
        part[(int64_t)blockIdx.x * p * p + e] = s;
    }
}

// G = sum of the partials in block order (upper triangle mirrored).
__global__ void gram_final_kernel(const double* __restrict__ part, int nb, int p, double* __restrict__ G) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= p * p) return;
    const int i = e / p, j = e % p;
    const int src = j >= i ? e : j * p + i;
    double s = 0.0;
    for (int b = 0; b < nb; ++b) s += part[(int64_t)b * p * p + src];
    G[e] = s;
}

// Cholesky G = R^T R (R upper, fp64), one thread; a non-positive pivot is
// floored at 1e-300 so the triangular solve stays finite.
__global__ void chol_kernel(const double* __restrict__ G, int p, double* __restrict__ R) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    for (int i = 0; i < p * p; ++i) R[i] = 0.0;
    for (int j = 0; j < p; ++j) {
        double d = G[j * p + j];
        for (int l = 0; l < j; ++l) d -= R[l * p + j] * R[l * p + j];
        d = d > 1e-300 ? sqrt(d) : 1e-150;
        R[j * p + j] = d;
        for (int i = j + 1; i < p; ++i) {
            double s = G[j * p + i];
            for (int l = 0; l < j; ++l) s -= R[l * p + j] * R[l * p + i];
            R[j * p + i] = s / d;
        }
    }
}

// Y[m, :] <- Y[m, :] R^-1 (row-wise forward substitution, fp64).
__global__ void trsm_rows_kernel(float* __restrict__ Y, int64_t M, int p, const double* __restrict__ R) {
    const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    double x[FK_PMAX];
    for (int j = 0; j < p; ++j) {
        double s = Y[m * p + j];
        for (int l = 0; l < j; ++l) s -= x[l] * R[l * p + j];
        x[j] = s / R[j * p + j];
    }
    for (int j = 0; j < p; ++j) Y[m * p + j] = (float)x[j];
}

// Eigen-decomposition of the symmetric G (fp64) by cyclic Jacobi rotations,
// one thread: Ub columns sorted by descending eigenvalue into lam.
__global__ void jacobi_kernel(const double* __restrict__ G, int p, double* __restrict__ A,
                              double* __restrict__ Vm, double* __restrict__ Ub, double* __restrict__ lam) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    for (int i = 0; i < p * p; ++i) {
        A[i] = G[i];
        Vm[i] = (i / p == i % p) ? 1.0 : 0.0;
    }
    for (int sweep = 0; sweep < 60; ++sweep) {
        double off = 0.0, tot = 0.0;
        for (int i = 0; i < p; ++i)
            for (int j = 0; j < p; ++j) {
                const double a = A[i * p + j] * A[i * p + j];
                tot += a;
                if (i != j) off += a;
            }
        if (off <= 1e-30 * tot) break;
        for (int i = 0; i < p - 1; ++i)
            for (int j = i + 1; j < p; ++j) {
                const double aij = A[i * p + j];
                if (aij == 0.0) continue;
                const double th = (A[j * p + j] - A[i * p + i]) / (2.0 * aij);
                const double t = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(th * th + 1.0));
                const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
                for (int l = 0; l < p; ++l) {          // A <- J^T A J
                    const double ali = A[l * p + i], alj = A[l * p + j];
                    A[l * p + i] = c * ali - s * alj;
                    A[l * p + j] = s * ali + c * alj;
                }
                for (int l = 0; l < p; ++l) {
                    const double ail = A[i * p + l], ajl = A[j * p + l];
                    A[i * p + l] = c * ail - s * ajl;
                    A[j * p + l] = s * ail + c * ajl;
                }
                for (int l = 0; l < p; ++l) {          // V <- V J
                    const double vli = Vm[l * p + i], vlj = Vm[l * p + j];
                    Vm[l * p + i] = c * vli - s * vlj;
                    Vm[l * p + j] = s * vli + c * vlj;
                }
            }
    }
    // selection sort by descending eigenvalue (ties: lower index first)
    int order[FK_PMAX];
    for (int i = 0; i < p; ++i) order[i] = i;
    for (int i = 0; i < p; ++i) {
        int b = i;
        for (int j = i + 1; j < p; ++j)
            if (A[order[j] * p + order[j]] > A[order[b] * p + order[b]]) b = j;
        const int t = order[i];
        order[i] = order[b];
        order[b] = t;
    }
    for (int j = 0; j < p; ++j) {
        lam[j] = A[order[j] * p + order[j]];
        for (int l = 0; l < p; ++l) Ub[l * p + j] = Vm[l * p + order[j]];
    }
}

// Out[m, j] = scale_j * sum_l X[m, l] Ub[l, j] for j < k (fp64 sums), with
// scale_j = 1 / sqrt(lam_j) (inv = 1) or 1.
__global__ void rotate_kernel(const float* __restrict__ X, int64_t M, int p, int k, const double* __restrict__ Ub,
                              const double* __restrict__ lam, int inv, float* __restrict__ out) {
    const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (m >= M) return;
    for (int j = 0; j < k; ++j) {
        double s = 0.0;
        for (int l = 0; l < p; ++l) s = fma((double)X[m * p + l], Ub[l * p + j], s);
        if (inv) s = lam[j] > 0.0 ? s / sqrt(lam[j]) : 0.0;
        out[m * k + j] = (float)s;
    }
}

// Sign of column j of U [M, k]: +1 unless its largest-magnitude entry (the
// first one on ties) is negative.  One block per column.
__global__ __launch_bounds__(256) void sign_kernel(const float* __restrict__ U, int64_t M, int k,
                                                   float* __restrict__ sgn) {
    __shared__ float bv[256];
    __shared__ int64_t bi[256];
    const int j = blockIdx.x, tid = threadIdx.x;
    float best = -1.0f;
    int64_t at = M;
    for (int64_t m = tid; m < M; m += 256) {
        const float a = fabsf(U[m * k + j]);
        if (a > best) { best = a; at = m; }
    }
    bv[tid] = best;
    bi[tid] = at;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if (tid < w) {
            const float o = bv[tid + w];
            const int64_t oi = bi[tid + w];
            if (o > bv[tid] || (o == bv[tid] && oi < bi[tid])) { bv[tid] = o; bi[tid] = oi; }
        }
        __syncthreads();
    }
    if (tid == 0) sgn[j] = (bi[0] < M && U[bi[0] * k + j] < 0.0f) ? -1.0f : 1.0f;
}

// F_t[j, m] = sgn_j * sqrt(sqrt(lam_j)) * X[m, j]  (the transposed factor rows).
__global__ void factor_rows_kernel(const float* __restrict__ X, int64_t M, int k, const double* __restrict__ lam,
                                   const float* __restrict__ sgn, float* __restrict__ Ft) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)k * M) return;
    const int j = (int)(e / M);
    const int64_t m = e % M;
    const double sj = lam[j] > 0.0 ? sqrt(sqrt(lam[j])) : 0.0;
    Ft[e] = (float)(sgn[j] * sj * (double)X[m * k + j]);
}

}  // namespace

// Workspace layout (each piece 256-byte aligned), walked the same way by
// the size query and the launcher.
struct FactorWs {
    char* base;
    size_t off = 0;
    void* take(size_t bytes) {
        void* r = base ? base + off : nullptr;
        off += (bytes + 255) / 256 * 256;
        return r;
    }
};

constexpr int FK_NB = 256;   // Gram partial blocks

size_t svd_factors_ws_bytes(int64_t D_out, int64_t D_in, int p) {
    FactorWs w{nullptr};
    w.take(sizeof(float) * D_out * p);
    w.take(sizeof(float) * D_in * p);
    w.take(sizeof(float) * D_out * p);
    w.take(sizeof(float) * D_in * FK_PMAX);
    w.take(sizeof(float) * D_out * FK_PMAX);
    w.take(sizeof(float) * FK_PMAX);
    w.take(sizeof(double) * FK_NB * p * p);
    for (int i = 0; i < 5; ++i) w.take(sizeof(double) * p * p);
    w.take(sizeof(double) * p);
    return w.off;
}

hipError_t launch_svd_factors(bool bf16, const void* W, int64_t ldw, const void* Wt, int64_t ldwt, int64_t D_out,
                              int64_t D_in, int k, int p, int iters, uint64_t seed, float* WA_t, float* WB,
                              void* ws, hipStream_t st) {
    FactorWs w{(char*)ws};
    float* om = (float*)w.take(sizeof(float) * D_out * p);
    float* Q = (float*)w.take(sizeof(float) * D_in * p);
    float* Z = (float*)w.take(sizeof(float) * D_out * p);
    float* U = (float*)w.take(sizeof(float) * D_in * FK_PMAX);
    float* V = (float*)w.take(sizeof(float) * D_out * FK_PMAX);
    float* sgn = (float*)w.take(sizeof(float) * FK_PMAX);
    const int nb = FK_NB;
    double* part = (double*)w.take(sizeof(double) * nb * p * p);
    double* G = (double*)w.take(sizeof(double) * p * p);
    double* R = (double*)w.take(sizeof(double) * p * p);
    double* A = (double*)w.take(sizeof(double) * p * p);
    double* Vm = (double*)w.take(sizeof(double) * p * p);
    double* Ub = (double*)w.take(sizeof(double) * p * p);
    double* lam = (double*)w.take(sizeof(double) * p);
    hipError_t e = hipSuccess;
    // C[M, p] = A[M, K] B[K, p]
    auto skinny = [&](const void* Am, int64_t lda, int64_t M, int64_t K, const float* B, float* C) {
        const dim3 grid((unsigned)((M + FK_ROWS - 1) / FK_ROWS));
        if (bf16)
            hipLaunchKernelGGL(skinny_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)Am, lda, M, K, B, p, C);
        else
            hipLaunchKernelGGL(skinny_kernel<float>, grid, dim3(256), 0, st, (const float*)Am, lda, M, K, B, p, C);
    };
    auto gram = [&](const float* X, int64_t M) {
        const int64_t rpb = (M + nb - 1) / nb;
        hipLaunchKernelGGL(gram_partial_kernel, dim3(nb), dim3(256), 0, st, X, M, p, rpb, part);
        hipLaunchKernelGGL(gram_final_kernel, dim3((unsigned)((p * p + 255) / 256)), dim3(256), 0, st, part, nb, p, G);
    };
    auto orth = [&](float* X, int64_t M) {      // CholeskyQR2 in place
        for (int pass = 0; pass < 2; ++pass) {
            gram(X, M);
            hipLaunchKernelGGL(chol_kernel, dim3(1), dim3(64), 0, st, G, p, R);
            hipLaunchKernelGGL(trsm_rows_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, st, X, M, p, R);
        }
    };
    hipLaunchKernelGGL(omega_kernel, dim3((unsigned)((D_out * p + 255) / 256)), dim3(256), 0, st, seed, D_out * p, om);
    skinny(Wt, ldwt, D_in, D_out, om, Q);            // Y = W Omega   (W = Wt rows, K = D_out)
    orth(Q, D_in);
    for (int it = 0; it < iters; ++it) {
        skinny(W, ldw, D_out, D_in, Q, Z);           // Z = W^T Q     (W_lin rows, K = D_in)
        orth(Z, D_out);
        skinny(Wt, ldwt, D_in, D_out, Z, Q);         // Q = W Z
        orth(Q, D_in);
    }
    skinny(W, ldw, D_out, D_in, Q, Z);               // Z = W^T Q = (Q^T W)^T
    gram(Z, D_out);                                  // G = Z^T Z
    hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(64), 0, st, G, p, A, Vm, Ub, lam);
    hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)((D_in + 255) / 256)), dim3(256), 0, st, Q, D_in, p, k, Ub, lam, 0, U);
    hipLaunchKernelGGL(rotate_kernel, dim3((unsigned)((D_out + 255) / 256)), dim3(256), 0, st, Z, D_out, p, k, Ub, lam, 1, V);
    hipLaunchKernelGGL(sign_kernel, dim3((unsigned)k), dim3(256), 0, st, U, D_in, k, sgn);
    hipLaunchKernelGGL(factor_rows_kernel, dim3((unsigned)((k * D_in + 255) / 256)), dim3(256), 0, st, U, D_in, k, lam,
                       sgn, WA_t);
    hipLaunchKernelGGL(factor_rows_kernel, dim3((unsigned)((k * D_out + 255) / 256)), dim3(256), 0, st, V, D_out, k, lam,
                       sgn, WB);
    e = hipGetLastError();
    return e;
}
