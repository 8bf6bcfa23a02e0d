// Dense LoRA branch (every token, every channel) and the elementwise glue.
//
// Pages ("SparseLoRA: Accelerating LLM Fine-Tuning with Contextual
// Sparsity"): paper-graph summary §3.4 Algorithm 1 step 6 (y_final =
// y_sparse + B A x, dense), §3.2 "Information flow during a backward pass"
// (LoRA gradients always dense), §3.4 "FFN structure" (h = SiLU(g) * u).
//
//   lora_xl:      xl[t, j] = sum_i x[t, i] A[j, i]        (bf16: MFMA 16x16x32)
//   lora_add:     y[t, c] += s * sum_j P[t, j] Bm(c, j)   (fp32 math, one rounding)
//   outer_accum:  out(j, c) = s * sum_t P[t, j] Q[t, c]   (deterministic split over t)
#include "sl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<bf16_t>(const bf16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}
template <typename T> __device__ __forceinline__ void st(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void st<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st<bf16_t>(bf16_t* p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
}

// ---------------------------------------------------------------- xl = x A^T
// Block of 4 waves covers 16 rows; each wave takes a quarter of K and all
// r columns (16 per MFMA block); partial sums meet in LDS in wave order.
__global__ __launch_bounds__(256) void lora_xl_bf16_kernel(const bf16_t* __restrict__ x,
                                                           int64_t ldx, int64_t T, int64_t D,
                                                           const bf16_t* __restrict__ A,
                                                           int64_t lda, int64_t r,
                                                           float* __restrict__ xl, int64_t ldxl) {
    __shared__ float part[4][4][16 * 16];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    const int64_t kq = ((D + 127) / 128) * 32;  // per-wave K range, multiple of 32
    const int64_t kbeg = wid * kq, kend = (kbeg + kq < D) ? kbeg + kq : D;
    const int nb = (int)((r + 15) / 16);
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int64_t row = t0 + (lane & 15);
    const bool rv = row < T;
    const int ko = (lane >> 4) * 8;
    for (int64_t k0 = kbeg; k0 < kend; k0 += 32) {
        const int64_t k = k0 + ko;
        uint4 av = {0u, 0u, 0u, 0u};
        if (rv) {
            if (k + 8 <= kend) av = *(const uint4*)(x + row * ldx + k);
            else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 8; ++e)
                    if (k + e < kend) w[e >> 1] |= (uint32_t)x[row * ldx + k + e] << ((e & 1) * 16);
                av = {w[0], w[1], w[2], w[3]};
            }
        }
        bf16x8 a = *(bf16x8*)&av;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b < nb) {
                const int64_t j = b * 16 + (lane & 15);
                uint4 bv = {0u, 0u, 0u, 0u};
                if (j < r) {
                    if (k + 8 <= kend) bv = *(const uint4*)(A + j * lda + k);
                    else {
                        uint32_t w[4] = {0u, 0u, 0u, 0u};
                        for (int e = 0; e < 8; ++e)
                            if (k + e < kend) w[e >> 1] |= (uint32_t)A[j * lda + k + e] << ((e & 1) * 16);
                        bv = {w[0], w[1], w[2], w[3]};
                    }
                }
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, *(bf16x8*)&bv, acc[b], 0, 0, 0);
            }
        }
    }
    // lane holds C[4*(lane/16) + e][lane % 16]
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wid][b][(4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[b][e];
    __syncthreads();
    for (int q = threadIdx.x; q < 16 * 64; q += 256) {
        const int rr = q / 64, j = q % 64;
        if (j >= r) continue;
        const int64_t t = t0 + rr;
        if (t >= T) continue;
        const int b = j / 16, jj = j % 16;
        float s = part[0][b][rr * 16 + jj];
        s += part[1][b][rr * 16 + jj];
        s += part[2][b][rr * 16 + jj];
        s += part[3][b][rr * 16 + jj];
        xl[t * ldxl + j] = s;
    }
}

__global__ void lora_xl_f32_kernel(const float* __restrict__ x, int64_t ldx, int64_t T, int64_t D,
                                   const float* __restrict__ A, int64_t lda, int64_t r,
                                   float* __restrict__ xl, int64_t ldxl) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= T * r) return;
    const int64_t t = q / r, j = q % r;
    float s = 0.0f;
    for (int64_t i = 0; i < D; ++i) s += x[t * ldx + i] * A[j * lda + i];
    xl[t * ldxl + j] = s;
}

// ---------------------------------------------------------------- y += s P Bm^T
// Tile 32 rows x 256 columns; thread = 8 consecutive columns x 4 rows.
template <typename T>
__global__ __launch_bounds__(256) void lora_add_kernel(const float* __restrict__ P, int64_t ldp,
                                                       int64_t Tn, int64_t r,
                                                       const T* __restrict__ Bm, int64_t sbc,
                                                       int64_t sbj, int64_t Nc, float scale,
                                                       T* __restrict__ y, int64_t ldy) {
    __shared__ float Ps[32][65];
    __shared__ float Bs[256][65];
    const int64_t t0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 256;
    for (int q = threadIdx.x; q < 32 * r; q += 256) {
        const int rr = q / (int)r, j = q % (int)r;
        const int64_t t = t0 + rr;
        Ps[rr][j] = t < Tn ? P[t * ldp + j] : 0.0f;
    }
    if (sbc == 1) {  // B(c, j) contiguous along c: walk c fastest (coalesced)
        for (int q = threadIdx.x; q < 256 * r; q += 256) {
            const int cc = q & 255, j = q >> 8;
            const int64_t c = c0 + cc;
            Bs[cc][j] = c < Nc ? ld<T>(Bm, c + j * sbj) : 0.0f;
        }
    } else {         // contiguous along j: walk j fastest
        for (int q = threadIdx.x; q < 256 * r; q += 256) {
            const int cc = q / (int)r, j = q % (int)r;
            const int64_t c = c0 + cc;
            Bs[cc][j] = c < Nc ? ld<T>(Bm, c * sbc + j * sbj) : 0.0f;
        }
    }
    __syncthreads();
    const int cg = threadIdx.x & 31, rs = threadIdx.x >> 5;
    for (int i = 0; i < 4; ++i) {
        const int rr = rs * 4 + i;
        const int64_t t = t0 + rr;
        if (t >= Tn) continue;
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = 0.0f;
        for (int j = 0; j < r; ++j) {
            const float pv = Ps[rr][j];
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] += pv * Bs[cg * 8 + e][j];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t c = c0 + cg * 8 + e;
            if (c < Nc) {
                const int64_t o = t * ldy + c;
                st<T>(y, o, ld<T>(y, o) + scale * a[e]);
            }
        }
    }
}

// ---------------------------------------------------------------- out = s P^T Q
// Partial sums over 256-token chunks into ws[chunk][j][c], then an ordered
// reduction over chunks (deterministic).
template <typename T, int RB>
__global__ __launch_bounds__(256) void outer_partial_kernel(const float* __restrict__ P,
                                                            int64_t ldp, int64_t Tn, int64_t r,
                                                            const T* __restrict__ Q, int64_t ldq,
                                                            int64_t Nc, float* __restrict__ ws) {
    constexpr int TCH = 256;
    __shared__ float Ps[TCH][65];
    const int64_t ch = blockIdx.y, t0 = ch * TCH;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int q = threadIdx.x; q < TCH * r; q += 256) {
        const int tt = q / (int)r, j = q % (int)r;
        const int64_t t = t0 + tt;
        Ps[tt][j] = t < Tn ? P[t * ldp + j] : 0.0f;
    }
    __syncthreads();
    if (c >= Nc) return;
    float acc[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[j] = 0.0f;
    const int64_t tn = (Tn - t0) < TCH ? (Tn - t0) : TCH;
    for (int tt = 0; tt < tn; ++tt) {
        const float qv = ld<T>(Q, (t0 + tt) * ldq + c);
#pragma unroll
        for (int j = 0; j < RB; ++j) acc[j] += Ps[tt][j] * qv;
    }
#pragma unroll
    for (int j = 0; j < RB; ++j)
        if (j < r) ws[(ch * r + j) * Nc + c] = acc[j];
}

__global__ void outer_reduce_kernel(const float* __restrict__ ws, int64_t nch, int64_t r,
                                    int64_t Nc, float scale, float* __restrict__ out, int64_t soj,
                                    int64_t soc) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= r * Nc) return;
    const int64_t j = q / Nc, c = q % Nc;
    float s = 0.0f;
    for (int64_t ch = 0; ch < nch; ++ch) s += ws[(ch * r + j) * Nc + c];
    out[j * soj + c * soc] = scale * s;
}

// ---------------------------------------------------------------- glue
template <typename T>
__global__ void transpose_kernel(const T* __restrict__ in, int64_t ldi, int64_t rows,
                                 int64_t cols, T* __restrict__ out, int64_t ldo) {
    __shared__ T tile[32][33];
    const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
    for (int i = threadIdx.y; i < 32; i += blockDim.y) {
        const int64_t r = r0 + i, c = c0 + threadIdx.x;
        if (r < rows && c < cols) tile[i][threadIdx.x] = in[r * ldi + c];
    }
    __syncthreads();
    for (int i = threadIdx.y; i < 32; i += blockDim.y) {
        const int64_t c = c0 + i, r = r0 + threadIdx.x;
        if (r < rows && c < cols) out[c * ldo + r] = tile[threadIdx.x][i];
    }
}

template <typename T>
__global__ void swiglu_fwd_kernel(const T* __restrict__ g, int64_t ldg, const T* __restrict__ u,
                                  int64_t ldu, int64_t Tn, int64_t F, T* __restrict__ h,
                                  int64_t ldh) {
    const int64_t t = blockIdx.y;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < F;
         c += (int64_t)gridDim.x * blockDim.x) {
        const float gv = ld<T>(g, t * ldg + c), uv = ld<T>(u, t * ldu + c);
        const float s = gv / (1.0f + expf(-gv));
        st<T>(h, t * ldh + c, s * uv);
    }
}

template <typename T>
__global__ void swiglu_bwd_kernel(const T* __restrict__ dh, int64_t lddh, const T* __restrict__ g,
                                  int64_t ldg, const T* __restrict__ u, int64_t ldu, int64_t Tn,
                                  int64_t F, T* __restrict__ dg, int64_t lddg, T* __restrict__ du,
                                  int64_t lddu) {
    const int64_t t = blockIdx.y;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < F;
         c += (int64_t)gridDim.x * blockDim.x) {
        const float d = ld<T>(dh, t * lddh + c), gv = ld<T>(g, t * ldg + c),
                    uv = ld<T>(u, t * ldu + c);
        const float sg = 1.0f / (1.0f + expf(-gv));
        const float silu = gv * sg;
        const float dsilu = sg * (1.0f + gv * (1.0f - sg));
        st<T>(dg, t * lddg + c, d * uv * dsilu);
        st<T>(du, t * lddu + c, d * silu);
    }
}

template <typename T>
__global__ void gather_cols_kernel(const T* __restrict__ in, int64_t ldi,
                                   const int32_t* __restrict__ rows, int64_t nrows,
                                   const int32_t* __restrict__ cols, int64_t ncols,
                                   T* __restrict__ out, int64_t ldo) {
    const int64_t m = blockIdx.y;
    const int64_t src = (int64_t)rows[m] * ldi;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < ncols;
         q += (int64_t)gridDim.x * blockDim.x)
        out[m * ldo + q] = in[src + cols[q]];
}

// Zero the unselected channels of the given rows.  Thread = 8 consecutive
// channels; membership by a binary search in the ascending index list.
template <typename T>
__global__ void zero_unselected_kernel(T* __restrict__ y, int64_t ldy,
                                       const int32_t* __restrict__ rows, int64_t C,
                                       const int32_t* __restrict__ idx, int64_t n) {
    const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (c0 >= C) return;
    T* yr = y + (int64_t)rows[blockIdx.y] * ldy;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (idx[mid] < c0) lo = mid + 1; else hi = mid;
    }
    int64_t p = lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t c = c0 + e;
        if (c >= C) break;
        while (p < n && idx[p] < c) ++p;
        if (!(p < n && idx[p] == c)) yr[c] = (T)0;
    }
}

unsigned grid_x(int64_t n, int per) {
    int64_t g = ceil_div(n, per);
    return (unsigned)(g < 1 ? 1 : (g > 65535 ? 65535 : g));
}

}  // namespace

hipError_t launch_lora_xl(bool bf16, const void* x, int64_t ldx, int64_t T, int64_t D,
                          const void* A, int64_t lda, int64_t r, float* xl, int64_t ldxl,
                          float* ws, hipStream_t st) {
    (void)ws;
    if (T <= 0) return hipSuccess;
    if (bf16)
        hipLaunchKernelGGL(lora_xl_bf16_kernel, dim3((unsigned)ceil_div(T, 16)), dim3(256), 0, st,
                           (const bf16_t*)x, ldx, T, D, (const bf16_t*)A, lda, r, xl, ldxl);
    else
        hipLaunchKernelGGL(lora_xl_f32_kernel, dim3((unsigned)ceil_div(T * r, 256)), dim3(256), 0,
                           st, (const float*)x, ldx, T, D, (const float*)A, lda, r, xl, ldxl);
    return hipGetLastError();
}

hipError_t launch_lora_add(bool bf16, const float* P, int64_t ldp, int64_t T, int64_t r,
                           const void* Bm, int64_t sb_c, int64_t sb_j, int64_t Ncols,
                           float scale, void* y, int64_t ldy, hipStream_t st) {
    if (T <= 0 || Ncols <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(Ncols, 256), (unsigned)ceil_div(T, 32));
    if (bf16)
        hipLaunchKernelGGL(lora_add_kernel<bf16_t>, grid, dim3(256), 0, st, P, ldp, T, r,
                           (const bf16_t*)Bm, sb_c, sb_j, Ncols, scale, (bf16_t*)y, ldy);
    else
        hipLaunchKernelGGL(lora_add_kernel<float>, grid, dim3(256), 0, st, P, ldp, T, r,
                           (const float*)Bm, sb_c, sb_j, Ncols, scale, (float*)y, ldy);
    return hipGetLastError();
}

hipError_t launch_outer_accum(bool bf16, const float* P, int64_t ldp, int64_t T, int64_t r,
                              const void* Q, int64_t ldq, int64_t Ncols, float scale, float* out,
                              int64_t so_j, int64_t so_c, float* ws, size_t ws_floats,
                              hipStream_t st) {
    if (Ncols <= 0 || r <= 0) return hipSuccess;
    const int64_t nch = T > 0 ? ceil_div(T, 256) : 1;
    if ((size_t)(nch * r * Ncols) > ws_floats) return hipErrorInvalidValue;
    const dim3 grid((unsigned)ceil_div(Ncols, 256), (unsigned)nch);
    if (T > 0) {
#define OUTER(TT, RB)                                                                         \
    hipLaunchKernelGGL((outer_partial_kernel<TT, RB>), grid, dim3(256), 0, st, P, ldp, T, r, \
                       (const TT*)Q, ldq, Ncols, ws)
        if (bf16) {
            if (r <= 8) OUTER(bf16_t, 8);
            else if (r <= 16) OUTER(bf16_t, 16);
            else if (r <= 32) OUTER(bf16_t, 32);
            else OUTER(bf16_t, 64);
        } else {
            if (r <= 8) OUTER(float, 8);
            else if (r <= 16) OUTER(float, 16);
            else if (r <= 32) OUTER(float, 32);
            else OUTER(float, 64);
        }
#undef OUTER
    }
    hipLaunchKernelGGL(outer_reduce_kernel, dim3((unsigned)ceil_div(r * Ncols, 256)), dim3(256), 0,
                       st, ws, T > 0 ? nch : 0, r, Ncols, scale, out, so_j, so_c);
    return hipGetLastError();
}

hipError_t launch_transpose(bool bf16, const void* in, int64_t ldi, int64_t rows, int64_t cols,
                            void* out, int64_t ldo, hipStream_t st) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(cols, 32), (unsigned)ceil_div(rows, 32)), block(32, 8);
    if (bf16)
        hipLaunchKernelGGL(transpose_kernel<bf16_t>, grid, block, 0, st, (const bf16_t*)in, ldi,
                           rows, cols, (bf16_t*)out, ldo);
    else
        hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, st, (const float*)in, ldi, rows,
                           cols, (float*)out, ldo);
    return hipGetLastError();
}

hipError_t launch_swiglu_fwd(bool bf16, const void* g, int64_t ldg, const void* u, int64_t ldu,
                             int64_t T, int64_t F, void* h, int64_t ldh, hipStream_t st) {
    if (T <= 0 || F <= 0) return hipSuccess;
    const dim3 grid(grid_x(F, 256), (unsigned)T);
    if (bf16)
        hipLaunchKernelGGL(swiglu_fwd_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)g, ldg,
                           (const bf16_t*)u, ldu, T, F, (bf16_t*)h, ldh);
    else
        hipLaunchKernelGGL(swiglu_fwd_kernel<float>, grid, dim3(256), 0, st, (const float*)g, ldg,
                           (const float*)u, ldu, T, F, (float*)h, ldh);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(bool bf16, const void* dh, int64_t lddh, const void* g, int64_t ldg,
                             const void* u, int64_t ldu, int64_t T, int64_t F, void* dg,
                             int64_t lddg, void* du, int64_t lddu, hipStream_t st) {
    if (T <= 0 || F <= 0) return hipSuccess;
    const dim3 grid(grid_x(F, 256), (unsigned)T);
    if (bf16)
        hipLaunchKernelGGL(swiglu_bwd_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)dh,
                           lddh, (const bf16_t*)g, ldg, (const bf16_t*)u, ldu, T, F, (bf16_t*)dg,
                           lddg, (bf16_t*)du, lddu);
    else
        hipLaunchKernelGGL(swiglu_bwd_kernel<float>, grid, dim3(256), 0, st, (const float*)dh, lddh,
                           (const float*)g, ldg, (const float*)u, ldu, T, F, (float*)dg, lddg,
                           (float*)du, lddu);
    return hipGetLastError();
}

hipError_t launch_gather_cols(bool bf16, const void* in, int64_t ldi, const int32_t* rows,
                              int64_t nrows, const int32_t* cols, int64_t ncols, void* out,
                              int64_t ldo, hipStream_t st) {
    if (nrows <= 0 || ncols <= 0) return hipSuccess;
    const dim3 grid(grid_x(ncols, 256), (unsigned)nrows);
    if (bf16)
        hipLaunchKernelGGL(gather_cols_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)in,
                           ldi, rows, nrows, cols, ncols, (bf16_t*)out, ldo);
    else
        hipLaunchKernelGGL(gather_cols_kernel<float>, grid, dim3(256), 0, st, (const float*)in, ldi,
                           rows, nrows, cols, ncols, (float*)out, ldo);
    return hipGetLastError();
}

hipError_t launch_zero_unselected(bool bf16, void* y, int64_t ldy, const int32_t* rows,
                                  int64_t nrows, const int32_t* idx, int64_t n, int64_t C,
                                  uint8_t* unused, hipStream_t st) {
    (void)unused;
    if (nrows <= 0 || C <= 0 || n >= C) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(C, 256 * 8), (unsigned)nrows);
    if (bf16)
        hipLaunchKernelGGL(zero_unselected_kernel<bf16_t>, grid, dim3(256), 0, st, (bf16_t*)y, ldy,
                           rows, C, idx, n);
    else
        hipLaunchKernelGGL(zero_unselected_kernel<float>, grid, dim3(256), 0, st, (float*)y, ldy,
                           rows, C, idx, n);
    return hipGetLastError();
}
