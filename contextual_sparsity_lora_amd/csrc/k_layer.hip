// Decoder-layer glue between the sparse linears: RMSNorm (unit weight) with an
// optional fused residual add, an elementwise add, and plain causal softmax
// attention (forward and backward).
//
// These are support steps around the method (the pages train LLaMA layers
// whose linears are the sparse ones; the topology used here is pre-norm,
// residual adds, causal softmax with scale 1/sqrt(d), no position encoding,
// grouped-query heads).  They are written for correctness and plain
// bandwidth/VALU efficiency: fp32 arithmetic, bf16 or fp32 storage.
#include "sl_internal.h"

namespace {

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }
template <typename T> __device__ __forceinline__ void stf(T* p, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void stf<bf16_t>(bf16_t* p, float v) { *p = f32_to_bf16(v); }
// value as stored (bf16 rounding for bf16 storage)
template <typename T> __device__ __forceinline__ float rnd(float v);
template <> __device__ __forceinline__ float rnd<float>(float v) { return v; }
template <> __device__ __forceinline__ float rnd<bf16_t>(float v) { return bf16_to_f32(f32_to_bf16(v)); }

__device__ __forceinline__ float block_sum(float v, float* sh) {
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) sh[w] = v;
    __syncthreads();
    float t = 0.0f;
    const int nw = (int)(blockDim.x >> 6);
    for (int i = 0; i < nw; ++i) t += sh[i];
    __syncthreads();
    return t;
}

// ---------------------------------------------------------------- RMSNorm
// Row t: hsum = x + res (stored to hout when given; the norm reads the stored
// value), rstd = 1 / sqrt(mean(hsum^2) + eps), y = hsum * rstd.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const T* __restrict__ x, int64_t ldx,
                                                          const T* __restrict__ res, int64_t ldr,
                                                          int64_t D, float eps, T* __restrict__ hout,
                                                          int64_t ldh, T* __restrict__ y, int64_t ldy,
                                                          float* __restrict__ rstd) {
    __shared__ float sh[4];
    const int64_t t = blockIdx.x;
    const T* xr = x + t * ldx;
    const T* rr = res ? res + t * ldr : nullptr;
    float ss = 0.0f;
    for (int64_t i = threadIdx.x; i < D; i += blockDim.x) {
        float v = ldf<T>(xr + i);
        if (rr) {
            v = rnd<T>(v + ldf<T>(rr + i));
            if (hout) stf<T>(hout + t * ldh + i, v);
        }
        ss += v * v;
    }
    const float tot = block_sum(ss, sh);
    const float r = 1.0f / sqrtf(tot / (float)D + eps);
    if (threadIdx.x == 0) rstd[t] = r;
    for (int64_t i = threadIdx.x; i < D; i += blockDim.x) {
        float v = ldf<T>(xr + i);
        if (rr) v = rnd<T>(v + ldf<T>(rr + i));
        stf<T>(y + t * ldy + i, v * r);
    }
}

// dx = r dy - r^3 x (sum_j dy_j x_j) / D  (+ dres when given)
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const T* __restrict__ x, int64_t ldx,
                                                          const float* __restrict__ rstd,
                                                          const T* __restrict__ dy, int64_t lddy,
                                                          const T* __restrict__ dres, int64_t lddr,
                                                          int64_t D, T* __restrict__ dx, int64_t lddx) {
    __shared__ float sh[4];
    const int64_t t = blockIdx.x;
    const T* xr = x + t * ldx;
    const T* gr = dy + t * lddy;
    float s = 0.0f;
    for (int64_t i = threadIdx.x; i < D; i += blockDim.x) s += ldf<T>(gr + i) * ldf<T>(xr + i);
    const float dot = block_sum(s, sh);
    const float r = rstd[t];
    const float c = r * r * r * dot / (float)D;
    for (int64_t i = threadIdx.x; i < D; i += blockDim.x) {
        float v = r * ldf<T>(gr + i) - c * ldf<T>(xr + i);
        if (dres) v += ldf<T>(dres + t * lddr + i);
        stf<T>(dx + t * lddx + i, v);
    }
}

template <typename T>
__global__ void add_kernel(const T* __restrict__ a, int64_t lda, const T* __restrict__ b, int64_t ldb,
                           int64_t D, T* __restrict__ out, int64_t ldo) {
    const int64_t t = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < D) stf<T>(out + t * ldo + i, ldf<T>(a + t * lda + i) + ldf<T>(b + t * ldb + i));
}

// ---------------------------------------------------------------- attention
// Thread layout shared by the attention kernels: 8 threads per row (query or
// key); thread s of a row holds head dimensions s, s + 8, s + 16, ... (so the
// 8 threads read 8 different LDS banks); dot products over the head dimension
// are reduced across the 8 threads with xor shuffles.
constexpr int AQ = 32;   // rows per block (32 rows x 8 threads = 256)
constexpr int AK = 64;   // staged rows per LDS step

__device__ __forceinline__ float reduce8(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    return v;
}

template <typename T, int HD>
__device__ __forceinline__ void load_slice(const T* p, float (&v)[HD / 8]) {
#pragma unroll
    for (int i = 0; i < HD / 8; ++i) v[i] = ldf<T>(p + 8 * i);
}

// Forward: block = (32 queries, head h, sequence b); online softmax over key
// blocks of 64 staged in LDS as fp32; lse[b, h, q] = m + log(l) is kept for
// the backward pass.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ q, int64_t ldq,
                                                       const T* __restrict__ k, int64_t ldk,
                                                       const T* __restrict__ v, int64_t ldv,
                                                       int64_t S, int64_t H, int64_t n_rep,
                                                       T* __restrict__ o, int64_t ldo,
                                                       float* __restrict__ lse) {
    constexpr int SL = HD / 8;
    __shared__ float Ks[AK][HD + 4];
    __shared__ float Vs[AK][HD + 4];
    const int tid = threadIdx.x, row = tid >> 3, sl = tid & 7;
    const int64_t b = blockIdx.z, h = blockIdx.y, g = h / n_rep;
    const int64_t q0 = (int64_t)blockIdx.x * AQ, qi = q0 + row;
    const bool qv = qi < S;
    const int64_t t0 = b * S;
    const float scale = 1.0f / sqrtf((float)HD);
    float qr[SL], acc[SL];
    if (qv) load_slice<T, HD>(q + (t0 + qi) * ldq + h * HD + sl, qr);
    else
#pragma unroll
        for (int i = 0; i < SL; ++i) qr[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < SL; ++i) acc[i] = 0.0f;
    float m = -INFINITY, l = 0.0f;
    const int64_t kend = (q0 + AQ < S) ? q0 + AQ : S;     // causal: keys <= last query of the block
    for (int64_t k0 = 0; k0 < kend; k0 += AK) {
        __syncthreads();
        for (int e = tid; e < AK * HD; e += 256) {
            const int j = e / HD, c = e % HD;
            const int64_t kj = k0 + j;
            Ks[j][c] = kj < S ? ldf<T>(k + (t0 + kj) * ldk + g * HD + c) : 0.0f;
            Vs[j][c] = kj < S ? ldf<T>(v + (t0 + kj) * ldv + g * HD + c) : 0.0f;
        }
        __syncthreads();
        float s[AK];
        float mb = -INFINITY;
#pragma unroll
        for (int j = 0; j < AK; ++j) {
            float p = 0.0f;
#pragma unroll
            for (int i = 0; i < SL; ++i) p += qr[i] * Ks[j][sl + 8 * i];
            p = reduce8(p) * scale;
            const int64_t kj = k0 + j;
            s[j] = (kj <= qi && kj < S) ? p : -INFINITY;
            mb = fmaxf(mb, s[j]);
        }
        const float mn = fmaxf(m, mb);
        if (mn == -INFINITY) continue;                    // no visible key yet (padding rows)
        const float corr = expf(m - mn);
        l *= corr;
#pragma unroll
        for (int i = 0; i < SL; ++i) acc[i] *= corr;
#pragma unroll
        for (int j = 0; j < AK; ++j) {
            const float p = expf(s[j] - mn);
            l += p;
#pragma unroll
            for (int i = 0; i < SL; ++i) acc[i] += p * Vs[j][sl + 8 * i];
        }
        m = mn;
    }
    if (!qv) return;
    const float inv = 1.0f / l;
    T* op = o + (t0 + qi) * ldo + h * HD + sl;
#pragma unroll
    for (int i = 0; i < SL; ++i) stf<T>(op + 8 * i, acc[i] * inv);
    if (sl == 0) lse[(b * H + h) * S + qi] = m + logf(l);
}

// delta[b, h, q] = sum_c dO[q, c] O[q, c] (row term of the softmax backward)
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T* __restrict__ o, int64_t ldo,
                                                         const T* __restrict__ dO, int64_t lddo,
                                                         int64_t S, int64_t H,
                                                         float* __restrict__ delta) {
    constexpr int SL = HD / 8;
    const int tid = threadIdx.x, row = tid >> 3, sl = tid & 7;
    const int64_t b = blockIdx.z, h = blockIdx.y;
    const int64_t qi = (int64_t)blockIdx.x * AQ + row;
    if (qi >= S) return;
    const int64_t t = b * S + qi;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < SL; ++i)
        s += ldf<T>(o + t * ldo + h * HD + sl + 8 * i) * ldf<T>(dO + t * lddo + h * HD + sl + 8 * i);
    s = reduce8(s);
    if (sl == 0) delta[(b * H + h) * S + qi] = s;
}

// dK, dV: block = (32 keys, key/value head g, sequence b); loops over the
// group's query heads and the query blocks at or after the keys, with Q and dO
// staged in LDS; P is recomputed from lse.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(
    const T* __restrict__ q, int64_t ldq, const T* __restrict__ k, int64_t ldk,
    const T* __restrict__ v, int64_t ldv, const T* __restrict__ dO, int64_t lddo,
    const float* __restrict__ lse, const float* __restrict__ delta, int64_t S, int64_t H,
    int64_t n_rep, T* __restrict__ dk, int64_t lddk, T* __restrict__ dv, int64_t lddv) {
    constexpr int SL = HD / 8;
    __shared__ float Qs[AK][HD + 4];
    __shared__ float Gs[AK][HD + 4];
    __shared__ float Ls[AK], Ds[AK];
    const int tid = threadIdx.x, row = tid >> 3, sl = tid & 7;
    const int64_t b = blockIdx.z, g = blockIdx.y;
    const int64_t k0 = (int64_t)blockIdx.x * AQ, kj = k0 + row;
    const bool kv = kj < S;
    const int64_t t0 = b * S;
    const float scale = 1.0f / sqrtf((float)HD);
    float kr[SL], vr[SL], dkr[SL], dvr[SL];
    if (kv) {
        load_slice<T, HD>(k + (t0 + kj) * ldk + g * HD + sl, kr);
        load_slice<T, HD>(v + (t0 + kj) * ldv + g * HD + sl, vr);
    } else {
#pragma unroll
        for (int i = 0; i < SL; ++i) kr[i] = vr[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < SL; ++i) dkr[i] = dvr[i] = 0.0f;
    for (int64_t hr = 0; hr < n_rep; ++hr) {
        const int64_t h = g * n_rep + hr;
        for (int64_t i0 = k0; i0 < S; i0 += AK) {
            __syncthreads();
            for (int e = tid; e < AK * HD; e += 256) {
                const int j = e / HD, c = e % HD;
                const int64_t qi = i0 + j;
                Qs[j][c] = qi < S ? ldf<T>(q + (t0 + qi) * ldq + h * HD + c) : 0.0f;
                Gs[j][c] = qi < S ? ldf<T>(dO + (t0 + qi) * lddo + h * HD + c) : 0.0f;
            }
            for (int j = tid; j < AK; j += 256) {
                const int64_t qi = i0 + j;
                Ls[j] = qi < S ? lse[(b * H + h) * S + qi] : 0.0f;
                Ds[j] = qi < S ? delta[(b * H + h) * S + qi] : 0.0f;
            }
            __syncthreads();
            for (int j = 0; j < AK; ++j) {
                const int64_t qi = i0 + j;
                float sdot = 0.0f, pdot = 0.0f;
#pragma unroll
                for (int i = 0; i < SL; ++i) {
                    sdot += Qs[j][sl + 8 * i] * kr[i];
                    pdot += Gs[j][sl + 8 * i] * vr[i];
                }
                sdot = reduce8(sdot);
                pdot = reduce8(pdot);
                const bool vis = kv && qi < S && kj <= qi;
                const float p = vis ? expf(sdot * scale - Ls[j]) : 0.0f;
                const float ds = p * (pdot - Ds[j]) * scale;
#pragma unroll
                for (int i = 0; i < SL; ++i) {
                    dvr[i] += p * Gs[j][sl + 8 * i];
                    dkr[i] += ds * Qs[j][sl + 8 * i];
                }
            }
        }
    }
    if (!kv) return;
#pragma unroll
    for (int i = 0; i < SL; ++i) {
        stf<T>(dk + (t0 + kj) * lddk + g * HD + sl + 8 * i, dkr[i]);
        stf<T>(dv + (t0 + kj) * lddv + g * HD + sl + 8 * i, dvr[i]);
    }
}

// dQ: block = (32 queries, head h, sequence b); loops over key blocks up to
// the queries with K and V staged in LDS.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(
    const T* __restrict__ q, int64_t ldq, const T* __restrict__ k, int64_t ldk,
    const T* __restrict__ v, int64_t ldv, const T* __restrict__ dO, int64_t lddo,
    const float* __restrict__ lse, const float* __restrict__ delta, int64_t S, int64_t H,
    int64_t n_rep, T* __restrict__ dq, int64_t lddq) {
    constexpr int SL = HD / 8;
    __shared__ float Ks[AK][HD + 4];
    __shared__ float Vs[AK][HD + 4];
    const int tid = threadIdx.x, row = tid >> 3, sl = tid & 7;
    const int64_t b = blockIdx.z, h = blockIdx.y, g = h / n_rep;
    const int64_t q0 = (int64_t)blockIdx.x * AQ, qi = q0 + row;
    const bool qv = qi < S;
    const int64_t t0 = b * S;
    const float scale = 1.0f / sqrtf((float)HD);
    float qr[SL], gr[SL], dqr[SL];
    if (qv) {
        load_slice<T, HD>(q + (t0 + qi) * ldq + h * HD + sl, qr);
        load_slice<T, HD>(dO + (t0 + qi) * lddo + h * HD + sl, gr);
    } else {
#pragma unroll
        for (int i = 0; i < SL; ++i) qr[i] = gr[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < SL; ++i) dqr[i] = 0.0f;
    const float L = qv ? lse[(b * H + h) * S + qi] : 0.0f;
    const float Dl = qv ? delta[(b * H + h) * S + qi] : 0.0f;
    const int64_t kend = (q0 + AQ < S) ? q0 + AQ : S;
    for (int64_t k0 = 0; k0 < kend; k0 += AK) {
        __syncthreads();
        for (int e = tid; e < AK * HD; e += 256) {
            const int j = e / HD, c = e % HD;
            const int64_t kj = k0 + j;
            Ks[j][c] = kj < S ? ldf<T>(k + (t0 + kj) * ldk + g * HD + c) : 0.0f;
            Vs[j][c] = kj < S ? ldf<T>(v + (t0 + kj) * ldv + g * HD + c) : 0.0f;
        }
        __syncthreads();
        for (int j = 0; j < AK; ++j) {
            const int64_t kj = k0 + j;
            float sdot = 0.0f, pdot = 0.0f;
#pragma unroll
            for (int i = 0; i < SL; ++i) {
                sdot += qr[i] * Ks[j][sl + 8 * i];
                pdot += gr[i] * Vs[j][sl + 8 * i];
            }
            sdot = reduce8(sdot);
            pdot = reduce8(pdot);
            const bool vis = qv && kj < S && kj <= qi;
            const float p = vis ? expf(sdot * scale - L) : 0.0f;
            const float ds = p * (pdot - Dl) * scale;
#pragma unroll
            for (int i = 0; i < SL; ++i) dqr[i] += ds * Ks[j][sl + 8 * i];
        }
    }
    if (!qv) return;
#pragma unroll
    for (int i = 0; i < SL; ++i) stf<T>(dq + (t0 + qi) * lddq + h * HD + sl + 8 * i, dqr[i]);
}

}  // namespace

// ---------------------------------------------------------------- launchers
#define SL_DISPATCH_T(bf16, ...) \
    if (bf16) { typedef bf16_t TT; __VA_ARGS__ } else { typedef float TT; __VA_ARGS__ }

hipError_t launch_rmsnorm_fwd(bool bf16, const void* x, int64_t ldx, const void* res, int64_t ldr,
                              int64_t T, int64_t D, float eps, void* hout, int64_t ldh, void* y,
                              int64_t ldy, float* rstd, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    SL_DISPATCH_T(bf16, hipLaunchKernelGGL(rmsnorm_fwd_kernel<TT>, dim3((unsigned)T), dim3(256), 0, st,
                                           (const TT*)x, ldx, (const TT*)res, ldr, D, eps, (TT*)hout,
                                           ldh, (TT*)y, ldy, rstd);)
    return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(bool bf16, const void* x, int64_t ldx, const float* rstd, const void* dy,
                              int64_t lddy, const void* dres, int64_t lddr, int64_t T, int64_t D,
                              void* dx, int64_t lddx, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    SL_DISPATCH_T(bf16, hipLaunchKernelGGL(rmsnorm_bwd_kernel<TT>, dim3((unsigned)T), dim3(256), 0, st,
                                           (const TT*)x, ldx, rstd, (const TT*)dy, lddy,
                                           (const TT*)dres, lddr, D, (TT*)dx, lddx);)
    return hipGetLastError();
}

hipError_t launch_add(bool bf16, const void* a, int64_t lda, const void* b, int64_t ldb, int64_t T,
                      int64_t D, void* out, int64_t ldo, hipStream_t st) {
    if (T <= 0 || D <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(D, 256), (unsigned)T);
    SL_DISPATCH_T(bf16, hipLaunchKernelGGL(add_kernel<TT>, grid, dim3(256), 0, st, (const TT*)a, lda,
                                           (const TT*)b, ldb, D, (TT*)out, ldo);)
    return hipGetLastError();
}

#define SL_DISPATCH_HD(hd, ...)                                  \
    switch (hd) {                                                \
        case 32: { constexpr int HDV = 32; __VA_ARGS__ } break;  \
        case 64: { constexpr int HDV = 64; __VA_ARGS__ } break;  \
        case 128: { constexpr int HDV = 128; __VA_ARGS__ } break; \
        default: return hipErrorInvalidValue;                    \
    }

// matrix-core attention (k_attn.hip): bf16, head dimension 32 / 64 / 128, 16-byte rows
bool attn_mfma_ok(int64_t hd, const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                  int64_t ldv, const void* o, int64_t ldo);
hipError_t launch_attn_fwd_mfma(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                                int64_t ldv, int64_t B, int64_t S, int64_t H, int64_t Hkv, int64_t hd, void* o,
                                int64_t ldo, float* lse, hipStream_t st);
bool attn_mfma_bwd_ok(int64_t hd, const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                      int64_t ldv, const void* dO, int64_t lddo, const void* dq, int64_t lddq, const void* dk,
                      int64_t lddk, const void* dv, int64_t lddv);
hipError_t launch_attn_bwd_mfma(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                                int64_t ldv, const void* dO, int64_t lddo, const float* lse, const float* delta,
                                int64_t B, int64_t S, int64_t H, int64_t Hkv, int64_t hd, void* dq, int64_t lddq,
                                void* dk, int64_t lddk, void* dv, int64_t lddv, void* ds, hipStream_t st);

hipError_t launch_attn_fwd(bool bf16, const void* q, int64_t ldq, const void* k, int64_t ldk,
                           const void* v, int64_t ldv, int64_t B, int64_t S, int64_t H, int64_t Hkv,
                           int64_t hd, void* o, int64_t ldo, float* lse, hipStream_t st) {
    if (B <= 0 || S <= 0) return hipSuccess;
    if (bf16 && attn_mfma_ok(hd, q, ldq, k, ldk, v, ldv, o, ldo))
        return launch_attn_fwd_mfma(q, ldq, k, ldk, v, ldv, B, S, H, Hkv, hd, o, ldo, lse, st);
    const dim3 grid((unsigned)ceil_div(S, AQ), (unsigned)H, (unsigned)B);
    const int64_t n_rep = H / Hkv;
    SL_DISPATCH_HD(hd, SL_DISPATCH_T(bf16, hipLaunchKernelGGL((attn_fwd_kernel<TT, HDV>), grid, dim3(256), 0,
                                                          st, (const TT*)q, ldq, (const TT*)k, ldk,
                                                          (const TT*)v, ldv, S, H, n_rep, (TT*)o, ldo,
                                                          lse);))
    return hipGetLastError();
}

hipError_t launch_attn_bwd(bool bf16, const void* q, int64_t ldq, const void* k, int64_t ldk,
                           const void* v, int64_t ldv, const void* o, int64_t ldo, const void* dO,
                           int64_t lddo, const float* lse, float* delta, int64_t B, int64_t S,
                           int64_t H, int64_t Hkv, int64_t hd, void* dq, int64_t lddq, void* dk,
                           int64_t lddk, void* dv, int64_t lddv, hipStream_t st) {
    if (B <= 0 || S <= 0) return hipSuccess;
    const int64_t n_rep = H / Hkv;
    const dim3 gq((unsigned)ceil_div(S, AQ), (unsigned)H, (unsigned)B);
    const dim3 gk((unsigned)ceil_div(S, AQ), (unsigned)Hkv, (unsigned)B);
    if (bf16 && attn_mfma_bwd_ok(hd, q, ldq, k, ldk, v, ldv, dO, lddo, dq, lddq, dk, lddk, dv, lddv)) {
        SL_DISPATCH_HD(hd, hipLaunchKernelGGL((attn_delta_kernel<bf16_t, HDV>), gq, dim3(256), 0, st,
                                              (const bf16_t*)o, ldo, (const bf16_t*)dO, lddo, S, H, delta);)
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        // the caller's workspace holds delta, then (at the next 256-byte
        // boundary) the bf16 dS tiles of the matrix-core backward
        void* ds = (char*)delta + (((size_t)(B * H * S) * sizeof(float) + 255) / 256) * 256;
        return launch_attn_bwd_mfma(q, ldq, k, ldk, v, ldv, dO, lddo, lse, delta, B, S, H, Hkv, hd, dq, lddq, dk,
                                    lddk, dv, lddv, ds, st);
    }
    SL_DISPATCH_HD(hd, SL_DISPATCH_T(bf16,
        hipLaunchKernelGGL((attn_delta_kernel<TT, HDV>), gq, dim3(256), 0, st, (const TT*)o, ldo,
                           (const TT*)dO, lddo, S, H, delta);
        hipLaunchKernelGGL((attn_bwd_kv_kernel<TT, HDV>), gk, dim3(256), 0, st, (const TT*)q, ldq,
                           (const TT*)k, ldk, (const TT*)v, ldv, (const TT*)dO, lddo, lse, delta, S, H,
                           n_rep, (TT*)dk, lddk, (TT*)dv, lddv);
        hipLaunchKernelGGL((attn_bwd_q_kernel<TT, HDV>), gq, dim3(256), 0, st, (const TT*)q, ldq,
                           (const TT*)k, ldk, (const TT*)v, ldv, (const TT*)dO, lddo, lse, delta, S, H,
                           n_rep, (TT*)dq, lddq);))
    return hipGetLastError();
}
