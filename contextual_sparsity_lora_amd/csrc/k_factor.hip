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

constexpr int FK_KC = 32;       // K chunk staged in LDS by the skinny product
constexpr int FK_PMAX = 64;     // max columns p
constexpr int FK_BLOCKS = 1024; // blocks a skinny product aims for (row blocks x K splits)

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

// C[M, p] = A[M, K] B[K, p] over one K span: A row-major (dt), B fp32 row-major
// (ld = p), out fp32 row-major (ld = p) at out + blockIdx.y * ostride.
// p is padded to P (16, 32 or 64).  Block = 256 threads = RG row groups x CL
// column lanes (CL = P / 4); thread (ty, tx) owns the 4 x 4 tile of rows
// 4 ty .. 4 ty + 3 and columns 4 tx .. 4 tx + 3, so one block covers
// RB = 4096 / P rows.  Block y sums K in [y kspan, (y + 1) kspan) through LDS in
// FK_KC chunks: A transposed (a thread's 4 rows are one 16-byte read), B as is
// (its 4 columns are one 16-byte read), 16 FMAs per pair of reads.
template <typename T, int P>
__global__ __launch_bounds__(256) void skinny_kernel(const T* __restrict__ A, int64_t lda, int64_t M,
                                                     int64_t K, const float* __restrict__ B, int p,
                                                     int64_t kspan, float* __restrict__ out, int64_t ostride) {
    constexpr int CL = P / 4, RB = 4096 / P, AS = RB + 4;
    __shared__ __align__(16) float at[FK_KC * AS];
    __shared__ __align__(16) float bs[FK_KC * P];
    const int tid = threadIdx.x;
    const int tx = tid % CL, ty = tid / CL;
    const int64_t m0 = (int64_t)blockIdx.x * RB;
    const int64_t kb = (int64_t)blockIdx.y * kspan;
    const int64_t ke = kb + kspan < K ? kb + kspan : K;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    for (int64_t k0 = kb; k0 < ke; k0 += FK_KC) {
        for (int q = tid; q < RB * FK_KC; q += 256) {
            const int rr = q / FK_KC, kk = q % FK_KC;
            const int64_t m = m0 + rr, k = k0 + kk;
            at[kk * AS + rr] = (m < M && k < ke) ? ldf(A, m * lda + k) : 0.0f;
        }
        for (int q = tid; q < FK_KC * P; q += 256) {
            const int kk = q / P, c = q % P;
            const int64_t k = k0 + kk;
            bs[q] = (k < ke && c < p) ? B[k * p + c] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < FK_KC; ++kk) {
            const float4 av = *(const float4*)&at[kk * AS + 4 * ty];
            const float4 bv = *(const float4*)&bs[kk * P + 4 * tx];
            const float a4[4] = {av.x, av.y, av.z, av.w}, b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a4[i], b4[j], acc[i][j]);
        }
        __syncthreads();
    }
    float* o = out + (int64_t)blockIdx.y * ostride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + 4 * ty + i;
        if (m < M)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * tx + j < p) o[m * p + 4 * tx + j] = acc[i][j];
    }
}

// C[e] = sum over s of part[s n + e], s in order (the K splits of one product).
__global__ void skinny_sum_kernel(const float* __restrict__ part, int64_t n, int S, float* __restrict__ C) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n) return;
    float v = part[e];
    for (int s = 1; s < S; ++s) v += part[(int64_t)s * n + e];
    C[e] = v;
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

// Cholesky G = R^T R (R upper, fp64); a non-positive pivot is floored at
// 1e-300 so the triangular solve stays finite.  One wave, R in LDS: column j's
// entries below the diagonal are independent, so thread i forms R[j][i] with
// the same sequential sum over l as a one-thread loop would (same values).
__global__ __launch_bounds__(64) void chol_kernel(const double* __restrict__ G, int p, double* __restrict__ R) {
    __shared__ double Rs[FK_PMAX * FK_PMAX];
    const int tid = threadIdx.x;
    for (int e = tid; e < p * p; e += blockDim.x) Rs[e] = 0.0;
    __syncthreads();
    for (int j = 0; j < p; ++j) {
        double d = G[j * p + j];
        for (int l = 0; l < j; ++l) d -= Rs[l * p + j] * Rs[l * p + j];
        d = d > 1e-300 ? sqrt(d) : 1e-150;
        const int i = tid;
        if (i == j) Rs[j * p + j] = d;
        if (i > j && i < p) {
            double s = G[j * p + i];
            for (int l = 0; l < j; ++l) s -= Rs[l * p + j] * Rs[l * p + i];
            Rs[j * p + i] = s / d;
        }
        __syncthreads();
    }
    for (int e = tid; e < p * p; e += blockDim.x) R[e] = Rs[e];
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

// Eigen-decomposition of the symmetric G (fp64) by cyclic Jacobi rotations:
// Ub columns sorted by descending eigenvalue into lam.  One wave with A and V
// in LDS: the rotations run in the cyclic order, and within a rotation the
// column update (rows l of columns i, j), then the row update (rows i, j) and
// V's columns are each independent over l, so thread l applies them to its
// entries with the same arithmetic as a one-thread loop (same values); the
// convergence sums stay sequential on thread 0.
__global__ __launch_bounds__(64) void jacobi_kernel(const double* __restrict__ G, int p, double* __restrict__ Ub,
                                                    double* __restrict__ lam) {
    __shared__ double As[FK_PMAX * FK_PMAX];
    __shared__ double Vs[FK_PMAX * FK_PMAX];
    __shared__ int s_done;
    const int tid = threadIdx.x;
    for (int e = tid; e < p * p; e += blockDim.x) {
        As[e] = G[e];
        Vs[e] = (e / p == e % p) ? 1.0 : 0.0;
    }
    __syncthreads();
    for (int sweep = 0; sweep < 60; ++sweep) {
        if (tid == 0) {
            double off = 0.0, tot = 0.0;
            for (int i = 0; i < p; ++i)
                for (int j = 0; j < p; ++j) {
                    const double a = As[i * p + j] * As[i * p + j];
                    tot += a;
                    if (i != j) off += a;
                }
            s_done = off <= 1e-30 * tot;
        }
        __syncthreads();
        if (s_done) break;
        for (int i = 0; i < p - 1; ++i)
            for (int j = i + 1; j < p; ++j) {
                const double aij = As[i * p + j];
                if (aij == 0.0) continue;             // (the same value in every thread)
                const double th = (As[j * p + j] - As[i * p + i]) / (2.0 * aij);
                const double t = (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + sqrt(th * th + 1.0));
                const double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
                __syncthreads();                       // every thread has read the pivot entries
                const int l = tid;
                if (l < p) {                           // A <- J^T A J: columns i, j
                    const double ali = As[l * p + i], alj = As[l * p + j];
                    As[l * p + i] = c * ali - s * alj;
                    As[l * p + j] = s * ali + c * alj;
                }
                __syncthreads();
                if (l < p) {                           // rows i, j; V <- V J
                    const double ail = As[i * p + l], ajl = As[j * p + l];
                    As[i * p + l] = c * ail - s * ajl;
                    As[j * p + l] = s * ail + c * ajl;
                    const double vli = Vs[l * p + i], vlj = Vs[l * p + j];
                    Vs[l * p + i] = c * vli - s * vlj;
                    Vs[l * p + j] = s * vli + c * vlj;
                }
                __syncthreads();
            }
    }
    if (tid != 0) return;
    // selection sort by descending eigenvalue (ties: lower index first)
    int order[FK_PMAX];
    for (int i = 0; i < p; ++i) order[i] = i;
    for (int i = 0; i < p; ++i) {
        int b = i;
        for (int j = i + 1; j < p; ++j)
            if (As[order[j] * p + order[j]] > As[order[b] * p + order[b]]) b = j;
        const int t = order[i];
        order[i] = order[b];
        order[b] = t;
    }
    for (int j = 0; j < p; ++j) {
        lam[j] = As[order[j] * p + order[j]];
        for (int l = 0; l < p; ++l) Ub[l * p + j] = Vs[l * p + order[j]];
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

// Launch shape of one skinny product C[M, p] = A[M, K] B[K, p]: P = p padded to
// 16, 32 or 64, RB = 4096 / P rows per block, and K cut into S spans of cps
// chunks so that row blocks x S reaches about FK_BLOCKS; S > 1 sums the spans'
// partial products (S M p floats of workspace) afterwards.
struct SkinnyPlan {
    int P;
    int64_t rb, rowblocks, cps, S;
};
SkinnyPlan skinny_plan(int64_t M, int64_t K, int p) {
    SkinnyPlan s;
    s.P = p <= 16 ? 16 : (p <= 32 ? 32 : 64);
    s.rb = 4096 / s.P;
    s.rowblocks = (M + s.rb - 1) / s.rb;
    const int64_t chunks = (K + FK_KC - 1) / FK_KC;
    int64_t want = (FK_BLOCKS + s.rowblocks - 1) / s.rowblocks;
    if (want > chunks) want = chunks;
    if (want < 1) want = 1;
    s.cps = (chunks + want - 1) / want;
    if (s.cps < 1) s.cps = 1;
    s.S = (chunks + s.cps - 1) / s.cps;
    if (s.S < 1) s.S = 1;
    return s;
}
int64_t skinny_part_floats(int64_t D_out, int64_t D_in, int p) {
    const SkinnyPlan a = skinny_plan(D_in, D_out, p), b = skinny_plan(D_out, D_in, p);
    const int64_t fa = a.S > 1 ? a.S * D_in * p : 0, fb = b.S > 1 ? b.S * D_out * p : 0;
    return fa > fb ? fa : fb;
}

size_t svd_factors_ws_bytes(int64_t D_out, int64_t D_in, int p) {
    FactorWs w{nullptr};
    w.take(sizeof(float) * D_out * p);
    w.take(sizeof(float) * D_in * p);
    w.take(sizeof(float) * D_out * p);
    w.take(sizeof(float) * D_in * FK_PMAX);
    w.take(sizeof(float) * D_out * FK_PMAX);
    w.take(sizeof(float) * FK_PMAX);
    w.take(sizeof(double) * FK_NB * p * p);
    for (int i = 0; i < 3; ++i) w.take(sizeof(double) * p * p);
    w.take(sizeof(double) * p);
    w.take(sizeof(float) * skinny_part_floats(D_out, D_in, p));
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
    double* Ub = (double*)w.take(sizeof(double) * p * p);
    double* lam = (double*)w.take(sizeof(double) * p);
    float* spart = (float*)w.take(sizeof(float) * skinny_part_floats(D_out, D_in, p));
    hipError_t e = hipSuccess;
    // C[M, p] = A[M, K] B[K, p]
    auto skinny = [&](const void* Am, int64_t lda, int64_t M, int64_t K, const float* B, float* C) {
        const SkinnyPlan pl = skinny_plan(M, K, p);
        const dim3 grid((unsigned)pl.rowblocks, (unsigned)pl.S);
        const int64_t kspan = pl.cps * FK_KC;
        float* o = pl.S > 1 ? spart : C;
        const int64_t os = M * p;
#define SL_SKINNY(P_)                                                                                         \
    if (bf16)                                                                                                 \
        hipLaunchKernelGGL((skinny_kernel<bf16_t, P_>), grid, dim3(256), 0, st, (const bf16_t*)Am, lda, M, K, B, \
                           p, kspan, o, os);                                                                  \
    else                                                                                                      \
        hipLaunchKernelGGL((skinny_kernel<float, P_>), grid, dim3(256), 0, st, (const float*)Am, lda, M, K, B,  \
                           p, kspan, o, os);
        if (pl.P == 16) {
            SL_SKINNY(16)
        } else if (pl.P == 32) {
            SL_SKINNY(32)
        } else {
            SL_SKINNY(64)
        }
#undef SL_SKINNY
        if (pl.S > 1)
            hipLaunchKernelGGL(skinny_sum_kernel, dim3((unsigned)((os + 255) / 256)), dim3(256), 0, st, spart, os,
                               (int)pl.S, C);
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
    hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(64), 0, st, G, p, Ub, lam);
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
