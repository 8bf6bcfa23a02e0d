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

// Orders this wave's LDS accesses across its lanes (a tile written by some
// lanes and read by others).  LDS only: the wave's outstanding global loads
// and stores are not waited for.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

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

// 8 consecutive elements, 16-byte aligned (bf16) / 32-byte aligned (fp32)
template <typename T> __device__ __forceinline__ void load8(const T* p, float* v);
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* v) {
    const uint4 u = *(const uint4*)p;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float* v) {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename T> __device__ __forceinline__ void store8(T* p, const float* v);
template <> __device__ __forceinline__ void store8<bf16_t>(bf16_t* p, const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *(uint4*)p = make_uint4(w[0], w[1], w[2], w[3]);
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float* v) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// ---------------------------------------------------------------- xl = x A^T
// Block of XW waves covers 16 rows; each wave takes one XW-th of K (a multiple
// of 32) and all r columns (16 per MFMA block), with XU 32-wide K steps in
// flight; partial sums meet in LDS and are added in wave order.
constexpr int XW = 8, XU = 8;

__global__ __launch_bounds__(XW * 64) void lora_xl_bf16_kernel(const bf16_t* __restrict__ x,
                                                               int64_t ldx, int64_t T, int64_t D,
                                                               const bf16_t* __restrict__ A,
                                                               int64_t lda, int64_t r,
                                                               float* __restrict__ xl, int64_t ldxl) {
    __shared__ float part[XW][4][16 * 16];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * 16;
    const int64_t kq = ((D + 32 * XW - 1) / (32 * XW)) * 32;  // per-wave K range, multiple of 32
    const int64_t kbeg = wid * kq, kend = (kbeg + kq < D) ? kbeg + kq : D;
    const int nb = (int)((r + 15) / 16);
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int64_t row = t0 + (lane & 15);
    const bool rv = row < T;
    const int ko = (lane >> 4) * 8;
    const bool vec = (ldx % 8 == 0) && (lda % 8 == 0) && ((uintptr_t)x & 15) == 0 &&
                     ((uintptr_t)A & 15) == 0;
    auto loadv = [&](const bf16_t* base, int64_t k) -> uint4 {
        if (vec && k + 8 <= kend) return *(const uint4*)(base + k);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 8; ++e)
            if (k + e < kend) w[e >> 1] |= (uint32_t)base[k + e] << ((e & 1) * 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    };
    const bf16_t* xrow = x + (rv ? row : 0) * ldx;
    const bf16_t* arow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t j = b * 16 + (lane & 15);
        arow[b] = (b < nb && j < r) ? A + j * lda : nullptr;
    }
    for (int64_t k0 = kbeg; k0 < kend; k0 += 32 * XU) {
        uint4 av[XU], bv[XU][4];
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int64_t k = k0 + 32 * u + ko;
            const bool kin = k < kend;
            av[u] = (rv && kin) ? loadv(xrow, k) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                bv[u][b] = (b < nb && arow[b] && kin) ? loadv(arow[b], k) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < XU; ++u)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (b < nb)
                    acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(bf16x8*)&av[u], *(bf16x8*)&bv[u][b],
                                                                     acc[b], 0, 0, 0);
    }
    // lane holds C[4*(lane/16) + e][lane % 16]
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wid][b][(4 * (lane >> 4) + e) * 16 + (lane & 15)] = acc[b][e];
    __syncthreads();
    for (int q = threadIdx.x; q < 16 * 64; q += XW * 64) {
        const int rr = q / 64, j = q % 64;
        if (j >= r) continue;
        const int64_t t = t0 + rr;
        if (t >= T) continue;
        const int b = j / 16, jj = j % 16;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < XW; ++w) s += part[w][b][rr * 16 + jj];
        xl[t * ldxl + j] = s;
    }
}

// Split-K form for bf16: a block of 4 waves takes 64 rows (16 per wave) and
// one K chunk; the chunk is walked in steps of 256 whose slice of A
// (r x 256) is staged in LDS once for the four waves, while each wave keeps 8
// 16-byte loads of its rows in flight.  Partial sums go to part[ks][t][R] and
// an ordered reduction over the chunks follows (deterministic).
constexpr int XR = 64, XKC = 256;

template <int R>
__global__ __launch_bounds__(256) void lora_xl_split_kernel(const bf16_t* __restrict__ x, int64_t ldx,
                                                            int64_t T, int64_t D,
                                                            const bf16_t* __restrict__ A, int64_t lda,
                                                            int64_t r, int64_t kchunk,
                                                            float* __restrict__ part) {
    constexpr int NB = R / 16;
    __shared__ __attribute__((aligned(16))) bf16_t As[R][XKC + 8];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * XR;
    const int64_t ks = blockIdx.y;
    const int64_t kb = ks * kchunk, ke = (kb + kchunk < D) ? kb + kchunk : D;
    const int64_t row = t0 + wid * 16 + (lane & 15);
    const bool rv = row < T;
    const int ko = (lane >> 4) * 8;
    const bool xvec = (ldx % 8 == 0) && (((uintptr_t)x & 15) == 0);
    const bool avec = (lda % 8 == 0) && (((uintptr_t)A & 15) == 0);
    const bf16_t* xrow = x + (rv ? row : 0) * ldx;
    auto load8 = [&](const bf16_t* base, int64_t k, bool vec) -> uint4 {
        if (vec && k + 8 <= ke) return *(const uint4*)(base + k);
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < 8; ++e)
            if (k + e < ke) w[e >> 1] |= (uint32_t)base[k + e] << ((e & 1) * 16);
        return make_uint4(w[0], w[1], w[2], w[3]);
    };
    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int64_t k0 = kb; k0 < ke; k0 += XKC) {
        uint4 xv[XKC / 32];
#pragma unroll
        for (int u = 0; u < XKC / 32; ++u) {
            const int64_t k = k0 + 32 * u + ko;
            xv[u] = (rv && k < ke) ? load8(xrow, k, xvec) : make_uint4(0u, 0u, 0u, 0u);
        }
        __syncthreads();                          // the previous slice has been read
#pragma unroll
        for (int c = 0; c < R / 8; ++c) {
            const int q = tid + 256 * c;
            const int j = q / 32, kk = (q % 32) * 8;
            const int64_t k = k0 + kk;
            *(uint4*)&As[j][kk] = (j < r && k < ke) ? load8(A + j * lda, k, avec) : make_uint4(0u, 0u, 0u, 0u);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < XKC / 32; ++u)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    *(bf16x8*)&xv[u], *(const bf16x8*)&As[16 * b + (lane & 15)][32 * u + ko], acc[b], 0, 0, 0);
    }
    // lane holds C[4 (lane / 16) + e][lane % 16] of rank block b
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t t = t0 + wid * 16 + 4 * (lane >> 4) + e;
            const int j = 16 * b + (lane & 15);
            if (t < T && j < r) part[(ks * T + t) * R + j] = acc[b][e];
        }
}

__global__ void lora_xl_reduce_kernel(const float* __restrict__ part, int64_t KS, int64_t T, int64_t r,
                                      int64_t R, float* __restrict__ xl, int64_t ldxl) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= T * r) return;
    const int64_t t = q / r, j = q % r;
    float s = 0.0f;
    for (int64_t k = 0; k < KS; ++k) s += part[(k * T + t) * R + j];
    xl[t * ldxl + j] = s;
}

// fp32: one wave per row t; lane l sums the columns i = l, l + 64, .. of 16
// ranks at a time (four columns' loads issued together), then the 64 lane
// sums of each rank are combined by a fixed butterfly (deterministic).
__global__ __launch_bounds__(256) void lora_xl_f32_kernel(const float* __restrict__ x, int64_t ldx, int64_t T,
                                                          int64_t D, const float* __restrict__ A, int64_t lda,
                                                          int64_t r, float* __restrict__ xl, int64_t ldxl) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // (wave-uniform)
    const float* xr = x + t * ldx;
    for (int64_t j0 = 0; j0 < r; j0 += 16) {
        float s[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) s[q] = 0.0f;
        for (int64_t i0 = lane; i0 < D; i0 += 256) {
            float xv[4], av[4][16];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t i = i0 + 64 * u;
                const bool iv = i < D;
                xv[u] = iv ? xr[i] : 0.0f;
#pragma unroll
                for (int q = 0; q < 16; ++q) av[u][q] = (iv && j0 + q < r) ? A[(j0 + q) * lda + i] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int q = 0; q < 16; ++q) s[q] += xv[u] * av[u][q];
        }
        float out = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) s[q] += __shfl_xor(s[q], o, 64);
            if (lane == q) out = s[q];
        }
        if (lane < 16 && j0 + lane < r) xl[t * ldxl + j0 + lane] = out;
    }
}

// ---------------------------------------------------------------- y += s P Bm^T
// A wave covers 64*CPL consecutive columns (CPL per lane, their Bm rows held
// in registers) and walks a run of rows; the row of P is wave-uniform and is
// read with scalar loads.  fp32 math, one rounding of y per element.
template <typename T, int R, int CPL>
__global__ __launch_bounds__(256) void lora_add_kernel(const float* __restrict__ P, int64_t ldp,
                                                       int64_t Tn, int64_t r,
                                                       const T* __restrict__ Bm, int64_t sbc,
                                                       int64_t sbj, int64_t Nc, float scale,
                                                       T* __restrict__ y, int64_t ldy, int64_t rpw) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c0 = (int64_t)blockIdx.x * (64 * CPL) + lane * CPL;
    float b[CPL][R];
#pragma unroll
    for (int q = 0; q < CPL; ++q)
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t c = c0 + q;
            b[q][j] = (c < Nc && j < r) ? ld<T>(Bm, c * sbc + j * sbj) : 0.0f;
        }
    const int64_t t0 = ((int64_t)blockIdx.y * 4 + w) * rpw;
    const int64_t t1 = (t0 + rpw < Tn) ? t0 + rpw : Tn;
    const bool full = c0 + CPL <= Nc;
    for (int64_t t = t0; t < t1; ++t) {
        const float* __restrict__ prow = P + t * ldp;
        float pj[R];
#pragma unroll
        for (int j = 0; j < R; ++j) pj[j] = (j < r) ? prow[j] : 0.0f;
        float acc[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            float a = 0.0f;
#pragma unroll
            for (int j = 0; j < R; ++j) a += pj[j] * b[q][j];
            acc[q] = a;
        }
        T* yr = y + t * ldy + c0;
        if (full) {
#pragma unroll
            for (int q = 0; q < CPL; ++q) st<T>(yr, q, ld<T>(yr, q) + scale * acc[q]);
        } else {
#pragma unroll
            for (int q = 0; q < CPL; ++q)
                if (c0 + q < Nc) st<T>(yr, q, ld<T>(yr, q) + scale * acc[q]);
        }
    }
}

// ---------------------------------------------------------------- rank-r fill of rows
// y[rows[m], c] (+)= s * sum_j P[rows[m], j] B[c, j] for every channel c of the
// given rows; with beta = 0 every channel is written (the main product of the
// selected channels is launched afterwards and overwrites them), with beta = 1
// only channels whose bit in `mask` is clear are updated (accumulated), with
// beta = 2 only those are written (so the product of the selected channels may
// run at the same time: the two write disjoint elements).
// bf16 matrix cores (v_mfma_f32_16x16x32_bf16), channel as M, row as N, rank as
// K: s P is rounded to bf16 as a bf16 LoRA product rounds its down-projection,
// accumulation is fp32.  Row slot m of MFMA (g, e) is channel
// c0 + 32 g + 8 (m / 4) + 4 e + m % 4, so lane l ends up holding the 8
// consecutive channels c0 + 32 g + 8 (l / 16) + 0..7 of row l % 16 (one
// 16-byte store per g).  A wave keeps the B rows of its 128 channels in
// registers and walks FTW rows; a block of 4 waves covers 128 x 4 FTW.
constexpr int FTW = 64;

template <int R>
__global__ __launch_bounds__(256) void lora_fill_rows_kernel(
    bf16_t* __restrict__ y, int64_t ldy, const int32_t* __restrict__ rows, int64_t nrows, int64_t C,
    const float* __restrict__ P, int64_t ldp, const bf16_t* __restrict__ B, int64_t ldb, int64_t r,
    float scale, const uint32_t* __restrict__ mask, int beta) {
    constexpr int KS = (R + 31) / 32;     // 32-wide rank steps
    __shared__ __attribute__((aligned(16))) bf16_t tile[4][16][128 + 8];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * 128;
    const int64_t t0 = ((int64_t)blockIdx.y * 4 + wid) * FTW;
    const int kl = 8 * (lane >> 4);       // this lane's first rank within a step
    const bool bvec = (ldb % 8 == 0) && (((uintptr_t)B & 15) == 0);
    const bool pvec = (ldp % 4 == 0) && (((uintptr_t)P & 15) == 0);
    bf16x8 wa[KS][4][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int m = lane & 15;
                const int64_t c = c0 + 32 * g + 8 * (m >> 2) + 4 * e + (m & 3);
                const int k = 32 * ks + kl;
                uint4 u = make_uint4(0u, 0u, 0u, 0u);
                if (c < C) {
                    const bf16_t* br = B + c * ldb;
                    if (bvec && k + 8 <= r) {
                        u = *(const uint4*)(br + k);
                    } else {
                        uint32_t w[4] = {0u, 0u, 0u, 0u};
                        for (int q = 0; q < 8; ++q)
                            if (k + q < r) w[q >> 1] |= (uint32_t)br[k + q] << ((q & 1) * 16);
                        u = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                }
                wa[ks][g][e] = __builtin_bit_cast(bf16x8, u);
            }
    const int64_t cl = c0 + 8 * (lane >> 4);   // + 32 g: this lane's 8 output channels
    const bool aligned = (ldy % 8 == 0) && (((uintptr_t)y & 15) == 0);
    for (int64_t tg = t0; tg < t0 + FTW && tg < nrows; tg += 16) {
        const int64_t m = tg + (lane & 15);
        const bool mv = m < nrows;
        const int64_t row = mv ? (int64_t)rows[m] : 0;
        const float* prow = P + row * ldp;
        bf16x8 pb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k = 32 * ks + kl;
            float v[8];
            if (mv && pvec && k + 8 <= r) {
                const float4 v0 = *(const float4*)(prow + k), v1 = *(const float4*)(prow + k + 4);
                v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
                v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) v[q] = (mv && k + q < r) ? prow[k + q] : 0.0f;
            }
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = pack_bf16x2(scale * v[2 * q], scale * v[2 * q + 1]);
            pb[ks] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
        // whole 128-channel block written without a mask: the 16 x 128 tile
        // goes through this wave's LDS rows so each output row leaves as 256
        // contiguous bytes (16 lanes x 16 B) instead of four 64-byte pieces
        const bool whole = beta == 0 && aligned && c0 + 128 <= C;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 acc[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks][g][e], pb[ks], acc[e], 0, 0, 0);
            const int64_t c = cl + 32 * g;
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = acc[0][i];
                v[4 + i] = acc[1][i];
            }
            if (whole) {
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
                *(uint4*)&tile[wid][lane & 15][8 * (lane >> 4) + 32 * g] = make_uint4(w[0], w[1], w[2], w[3]);
                continue;
            }
            if (!mv || c >= C) continue;
            bf16_t* dst = y + row * ldy + c;
            const uint32_t bits = beta ? ((mask[c >> 5] >> (c & 31)) & 0xffu) : 0u;   // c % 8 == 0: one word
            if (beta != 1 && bits == 0u && aligned && c + 8 <= C) {
                store8<bf16_t>(dst, v);           // every channel of the run is written
            } else {
                for (int q = 0; q < 8; ++q) {
                    if (c + q >= C || ((bits >> q) & 1u)) continue;
                    dst[q] = f32_to_bf16(v[q] + (beta == 1 ? bf16_to_f32(dst[q]) : 0.0f));
                }
            }
        }
        if (whole) {
            // (this wave's own LDS rows: in-order LDS access within the wave)
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 4 * j + (lane >> 4);               // tile row: lane rr holds its row number
                const int64_t orow = __shfl(row, rr, 64);
                const int ov = __shfl((int)mv, rr, 64);
                const uint4 d = *(const uint4*)&tile[wid][rr][8 * (lane & 15)];
                if (ov) *(uint4*)(y + orow * ldy + c0 + 8 * (lane & 15)) = d;
            }
            wave_lds_sync();
        }
    }
}

// ---------------------------------------------------------------- merge of a compact product
// y[rows[m], c] = Yc[m, j] for the selected channels c = idx[j] (the context
// rows' product stored compactly, one row per listed row, one column per
// selected channel), and s * P[rows[m], :] . B[c, :] (0 without a rank-r term)
// for every other channel.  Same tiling and matrix-core rank-r product as the
// fill above; the wave's 16 x 128 tile goes to its LDS rows, the selected
// channels of the 128-channel block (idx[j0 .. j1): one contiguous run of each
// compact row, since idx is ascending) overwrite their slots, and each row
// leaves as 256 contiguous bytes.  Every element of the listed rows is written
// exactly once, with 16-byte stores.
template <int R, int MTW>
__global__ __launch_bounds__(256) void lora_merge_rows_kernel(
    bf16_t* __restrict__ y, int64_t ldy, const int32_t* __restrict__ rows, int64_t nrows, int64_t C,
    const float* __restrict__ P, int64_t ldp, const bf16_t* __restrict__ B, int64_t ldb, int64_t r,
    float scale, const bf16_t* __restrict__ Yc, int64_t ldyc, const int32_t* __restrict__ idx, int64_t n) {
    constexpr int KS = (R + 31) / 32;     // 32-wide rank steps
    __shared__ __attribute__((aligned(16))) bf16_t tile[4][16][128 + 8];
    __shared__ __attribute__((aligned(16))) bf16_t cb[4][16][136];   // compact runs of the wave's 16 rows
    static_assert(MTW == 16 || MTW == 32 || MTW == 64, "rows per wave");
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c0 = (int64_t)blockIdx.x * 128;
    const int64_t t0 = ((int64_t)blockIdx.y * 4 + wid) * MTW;
    const int kl = 8 * (lane >> 4);
    const bool lora = P != nullptr;
    const bool bvec = (ldb % 8 == 0) && (((uintptr_t)B & 15) == 0);
    const bool pvec = (ldp % 4 == 0) && (((uintptr_t)P & 15) == 0);
    bf16x8 wa[KS][4][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int m = lane & 15;
                const int64_t c = c0 + 32 * g + 8 * (m >> 2) + 4 * e + (m & 3);
                const int k = 32 * ks + kl;
                uint4 u = make_uint4(0u, 0u, 0u, 0u);
                if (lora && c < C) {
                    const bf16_t* br = B + c * ldb;
                    if (bvec && k + 8 <= r) {
                        u = *(const uint4*)(br + k);
                    } else {
                        uint32_t w[4] = {0u, 0u, 0u, 0u};
                        for (int q = 0; q < 8; ++q)
                            if (k + q < r) w[q >> 1] |= (uint32_t)br[k + q] << ((q & 1) * 16);
                        u = make_uint4(w[0], w[1], w[2], w[3]);
                    }
                }
                wa[ks][g][e] = __builtin_bit_cast(bf16x8, u);
            }
    // the block's selected channels: idx[j0 .. j1), at most 128 of them; lane
    // holds entries j0 + lane and j0 + 64 + lane (slot in the block, or -1)
    int64_t j0, j1;
    wave_lower_bounds(idx, n, c0, c0 + 128, lane, j0, j1);
    const bool has0 = j0 + lane < j1, has1 = j0 + 64 + lane < j1;
    const int sl0 = has0 ? (int)(idx[j0 + lane] - c0) : -1;
    const int sl1 = has1 ? (int)(idx[j0 + 64 + lane] - c0) : -1;
    // Branch-free inner loop: every load reads an in-bounds address (rows past
    // the list read the last listed row, lanes without a selected channel read
    // the run's first compact value) and the values that must not count are
    // never stored: tile rows past the list are not written out, and a lane
    // without a selected channel puts its value in the tile's padding columns.
    const bool any = j1 > j0, run64 = j1 - j0 > 64;      // wave-uniform
    const int ds0 = has0 ? sl0 : 128 + (lane & 7), ds1 = has1 ? sl1 : 128 + (lane & 7);
    // the compact values of a row's run (positions j0 .. j1) come in as
    // 16-byte chunks from jb = j0 rounded down to 8 (lane l: chunk l % 16 of
    // row 4 s + l / 16; lanes 0-15 also chunk 16 of row l when the run needs
    // it); the chunks go to the wave's LDS rows cb, from which lane l takes
    // its entry j0 + l (and j0 + 64 + l) at og + l (og + 64 + l)
    const int64_t jb = j0 & ~(int64_t)7;
    const int og = (int)(j0 - jb);
    const bool two = j1 - jb > 128;                       // a 17th chunk (wave-uniform)
    const int cq = lane & 15, rq = lane >> 4;
    const bool ldc = jb + 8 * cq < j1, ldc17 = two && jb + 128 < j1 && lane < 16;
    const bool pfast = lora && pvec && r % 8 == 0;        // whole 8-rank runs of P
    const bool aligned = (ldy % 8 == 0) && (((uintptr_t)y & 15) == 0);
    const bool whole = aligned && c0 + 128 <= C;
    // the wave's rows (list entries t0 .. t0 + MTW), read once: lane l holds
    // entry t0 + l (clamped to the list); a 16-row step takes its rows by lane shuffle
    const int32_t rowv = rows[t0 + (lane % MTW) < nrows ? t0 + (lane % MTW) : nrows - 1];
    for (int64_t tg = t0; tg < t0 + MTW && tg < nrows; tg += 16) {
        const int64_t m = tg + (lane & 15);
        const bool mv = m < nrows;
        const int64_t row = (int64_t)__shfl(rowv, (int)(tg - t0) + (lane & 15), 64);
        // the rank-r operand's loads go out first, then the compact values of
        // the 16 rows; both are in flight before the first is used
        float pv[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k = 32 * ks + kl;
            if (pfast) {
                const bool kin = k < r;
                const float* prow = P + row * ldp + (kin ? k : 0);
                const float4 v0 = *(const float4*)prow, v1 = *(const float4*)(prow + 4);
                pv[ks][0] = v0.x; pv[ks][1] = v0.y; pv[ks][2] = v0.z; pv[ks][3] = v0.w;
                pv[ks][4] = v1.x; pv[ks][5] = v1.y; pv[ks][6] = v1.z; pv[ks][7] = v1.w;
#pragma unroll
                for (int q = 0; q < 8; ++q) pv[ks][q] = kin ? pv[ks][q] : 0.0f;
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) pv[ks][q] = (lora && mv && k + q < r) ? P[row * ldp + k + q] : 0.0f;
            }
        }
        uint4 cc[4], cx = make_uint4(0u, 0u, 0u, 0u);
        if (any) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int64_t mr = tg + 4 * s4 + rq;
                const bf16_t* yc = Yc + (mr < nrows ? mr : nrows - 1) * ldyc;
                cc[s4] = ldc ? *(const uint4*)(yc + jb + 8 * cq) : make_uint4(0u, 0u, 0u, 0u);
            }
            if (ldc17) {
                const int64_t mr = tg + lane;
                cx = *(const uint4*)(Yc + (mr < nrows ? mr : nrows - 1) * ldyc + jb + 128);
            }
        }
        bf16x8 pb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float* v = pv[ks];
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = pack_bf16x2(scale * v[2 * q], scale * v[2 * q + 1]);
            pb[ks] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 acc[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
            if (lora) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks][g][e], pb[ks], acc[e], 0, 0, 0);
            }
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                w[q] = pack_bf16x2(acc[0][2 * q], acc[0][2 * q + 1]);
                w[2 + q] = pack_bf16x2(acc[1][2 * q], acc[1][2 * q + 1]);
            }
            *(uint4*)&tile[wid][lane & 15][8 * (lane >> 4) + 32 * g] = make_uint4(w[0], w[1], w[2], w[3]);
        }
        // (this wave's own LDS rows: in-order LDS access within the wave)
        wave_lds_sync();
        // the selected channels from the compact rows, through cb
        if (any) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) *(uint4*)&cb[wid][4 * s4 + rq][8 * cq] = cc[s4];
            if (two && lane < 16) *(uint4*)&cb[wid][lane][128] = cx;
            wave_lds_sync();
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) tile[wid][rr][ds0] = cb[wid][rr][og + lane];
            if (run64) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) tile[wid][rr][ds1] = cb[wid][rr][og + 64 + lane];
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 4 * j + (lane >> 4);               // tile row: lane rr holds its row number
            const int64_t orow = __shfl(row, rr, 64);
            const int ov = __shfl((int)mv, rr, 64);
            if (!ov) continue;
            const int64_t c = c0 + 8 * (lane & 15);
            if (whole) {
                *(uint4*)(y + orow * ldy + c) = *(const uint4*)&tile[wid][rr][8 * (lane & 15)];
            } else {
                for (int q = 0; q < 8; ++q)
                    if (c + q < C) y[orow * ldy + c + q] = tile[wid][rr][8 * (lane & 15) + q];
            }
        }
        wave_lds_sync();
    }
}

// mask[w] bit b set <=> channel 32 w + b is in the ascending list idx
__global__ void select_mask_kernel(const int32_t* __restrict__ idx, int64_t n, int64_t C,
                                   uint32_t* __restrict__ mask) {
    const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (w * 32 >= C) return;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (idx[mid] < w * 32) lo = mid + 1; else hi = mid;
    }
    uint32_t bits = 0u;
    for (; lo < n && idx[lo] < w * 32 + 32; ++lo) bits |= 1u << (idx[lo] - w * 32);
    mask[w] = bits;
}

// ---------------------------------------------------------------- out = s P^T Q
// Block = 256 columns (one per thread) x one chunk of TCH tokens.  The chunk of
// P is staged in LDS once and read back as wave-wide broadcasts; Q is read
// once, 8 tokens in flight per thread.  Partial sums per chunk go to
// ws[chunk][j][c]; an ordered reduction over chunks follows (deterministic).
constexpr int TCH = 256;

template <typename T, int R>
__global__ __launch_bounds__(256) void outer_partial_kernel(const float* __restrict__ P,
                                                            int64_t ldp, int64_t Tn, int64_t r,
                                                            const T* __restrict__ Q, int64_t ldq,
                                                            int64_t Nc, float* __restrict__ ws) {
    __shared__ __attribute__((aligned(16))) float Ps[TCH][R];
    const int64_t chunk = blockIdx.y;
    const int64_t t0 = chunk * TCH;
    const int64_t tn = (Tn - t0) < TCH ? (Tn - t0) : TCH;
    for (int q = threadIdx.x; q < TCH * R; q += 256) {
        const int tt = q / R, j = q % R;
        Ps[tt][j] = (tt < tn && j < r) ? P[(t0 + tt) * ldp + j] : 0.0f;
    }
    __syncthreads();
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= Nc) return;
    float acc[R];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = 0.0f;
    const T* qc = Q + t0 * ldq + c;
    int tt = 0;
    for (; tt + 8 <= tn; tt += 8) {
        float qv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) qv[u] = ld<T>(qc, (int64_t)(tt + u) * ldq);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float4* pr = (const float4*)&Ps[tt + u][0];
#pragma unroll
            for (int j4 = 0; j4 < R / 4; ++j4) {
                const float4 p4 = pr[j4];
                acc[4 * j4 + 0] += p4.x * qv[u];
                acc[4 * j4 + 1] += p4.y * qv[u];
                acc[4 * j4 + 2] += p4.z * qv[u];
                acc[4 * j4 + 3] += p4.w * qv[u];
            }
        }
    }
    for (; tt < tn; ++tt) {
        const float qv = ld<T>(qc, (int64_t)tt * ldq);
#pragma unroll
        for (int j = 0; j < R; ++j) acc[j] += Ps[tt][j] * qv;
    }
#pragma unroll
    for (int j = 0; j < R; ++j)
        if (j < r) ws[(chunk * r + j) * Nc + c] = acc[j];
}

// bf16 Q on the matrix cores: v_mfma_f32_16x16x4_f32 with the rank as M, the
// token as K and a channel slot as N.  Lane l of a step owns token l/16 and the
// 8 consecutive channels c0 + 8 (l % 16) + e (one 16-byte load); MFMA number e
// takes element e, so output column n of MFMA e is channel c0 + 8 n + e and a
// lane ends up holding 8 consecutive channels of 4 ranks.  A block of OW waves
// shares 128 channels; wave w takes OTW tokens of the block's chunk; the waves'
// partial sums meet in LDS in wave order, and the block writes its chunk's
// partial to ws[chunk][j][c] for the ordered reduction over chunks.
constexpr int OW = 8, OTW = 64, OTC = OW * OTW;   // 512 tokens per chunk

template <int R>
__global__ __launch_bounds__(OW * 64) void outer_mfma_kernel(const float* __restrict__ P, int64_t ldp,
                                                             int64_t Tn, int64_t r,
                                                             const bf16_t* __restrict__ Q,
                                                             int64_t ldq, int64_t Nc,
                                                             float* __restrict__ ws) {
    constexpr int JB = R / 16;
    constexpr int U = 8;                      // 4-token steps in flight
    __shared__ float red[R * 128];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.x * 128;
    const int64_t chunk = blockIdx.y;
    const int64_t tb = chunk * OTC + (int64_t)wid * OTW;
    const int64_t cl = c0 + 8 * (lane & 15);
    const int kt = lane >> 4;
    const bool cfull = cl + 8 <= Nc;
    f32x4 acc[JB][8];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[jb][e] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < OTW / 4; s0 += U) {
        uint4 qv[U];
        float pv[U][JB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = tb + 4 * (s0 + u) + kt;
            qv[u] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) pv[u][jb] = 0.0f;
            if (t < Tn) {
                const bf16_t* qr = Q + t * ldq + cl;
                if (cfull) {
                    qv[u] = *(const uint4*)qr;
                } else {
                    uint32_t w[4] = {0u, 0u, 0u, 0u};
                    for (int e = 0; e < 8; ++e)
                        if (cl + e < Nc) w[e >> 1] |= (uint32_t)qr[e] << ((e & 1) * 16);
                    qv[u] = make_uint4(w[0], w[1], w[2], w[3]);
                }
#pragma unroll
                for (int jb = 0; jb < JB; ++jb) {
                    const int j = 16 * jb + (lane & 15);
                    pv[u][jb] = j < r ? P[t * ldp + j] : 0.0f;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t w[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float b = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
#pragma unroll
                for (int jb = 0; jb < JB; ++jb)
                    acc[jb][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[u][jb], b, acc[jb][e], 0, 0, 0);
            }
        }
    }
    // lane holds rank 16 jb + 4 (lane / 16) + i of channel slot 8 (lane % 16) + e
    for (int w = 0; w < OW; ++w) {
        if (wid == w) {
#pragma unroll
            for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float& d = red[(16 * jb + 4 * kt + i) * 128 + 8 * (lane & 15) + e];
                        d = (w == 0 ? 0.0f : d) + acc[jb][e][i];
                    }
        }
        __syncthreads();
    }
    for (int q = threadIdx.x; q < R * 128; q += OW * 64) {
        const int j = q >> 7, cc = q & 127;
        if (j < r && c0 + cc < Nc) ws[(chunk * r + j) * Nc + c0 + cc] = red[q];
    }
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
    const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (c0 >= F) return;
    float gv[8], uv[8], hv[8];
    if (c0 + 8 <= F) {
        load8<T>(g + t * ldg + c0, gv);
        load8<T>(u + t * ldu + c0, uv);
#pragma unroll
        for (int e = 0; e < 8; ++e) hv[e] = gv[e] * sigmoid_hw(gv[e]) * uv[e];
        store8<T>(h + t * ldh + c0, hv);
    } else {
        for (int64_t c = c0; c < F; ++c) {
            const float a = ld<T>(g, t * ldg + c), b = ld<T>(u, t * ldu + c);
            st<T>(h, t * ldh + c, a * sigmoid_hw(a) * b);
        }
    }
}

template <typename T>
__global__ void swiglu_bwd_kernel(const T* __restrict__ dh, int64_t lddh, const T* __restrict__ g,
                                  int64_t ldg, const T* __restrict__ u, int64_t ldu, int64_t Tn,
                                  int64_t F, T* __restrict__ dg, int64_t lddg, T* __restrict__ du,
                                  int64_t lddu) {
    const int64_t t = blockIdx.y;
    const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (c0 >= F) return;
    if (c0 + 8 <= F) {
        float d[8], gv[8], uv[8], a[8], b[8];
        load8<T>(dh + t * lddh + c0, d);
        load8<T>(g + t * ldg + c0, gv);
        load8<T>(u + t * ldu + c0, uv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float sg = sigmoid_hw(gv[e]);
            a[e] = d[e] * uv[e] * (sg * (1.0f + gv[e] * (1.0f - sg)));
            b[e] = d[e] * (gv[e] * sg);
        }
        store8<T>(dg + t * lddg + c0, a);
        store8<T>(du + t * lddu + c0, b);
    } else {
        for (int64_t c = c0; c < F; ++c) {
            const float d = ld<T>(dh, t * lddh + c), gv = ld<T>(g, t * ldg + c),
                        uv = ld<T>(u, t * ldu + c);
            const float sg = sigmoid_hw(gv);
            st<T>(dg, t * lddg + c, d * uv * (sg * (1.0f + gv * (1.0f - sg))));
            st<T>(du, t * lddu + c, d * (gv * sg));
        }
    }
}

// ---------------------------------------------------------------- SwiGLU with the LoRA reductions
// The SwiGLU passes also form the LoRA reductions that read the same tensors,
// so each tensor is read once (bf16, 16-byte rows, F % 8 == 0).  The
// reductions run on the matrix cores in fp32 (v_mfma_f32_16x16x4_f32): the
// bf16 values and the fp32 factors enter exactly and accumulate in fp32; a
// fixed-order sum over the blocks' partials follows (deterministic).

__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(w[q] << 16);
        f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
}

// Forward: h = silu(g) u (as swiglu_fwd) and the row partials of
// xl[t, j] = sum_c h[t, c] A[j, c] from the stored (bf16) h, over rows t =
// rows[m] (or m) for m < Tn; partials are indexed by m.  A block of 4
// waves shares 16 rows; wave w takes SFW columns from its block's start, 128
// at a time.  Loads and stores go 4 rows at a time with 16 lanes on each
// row's 256 bytes (lane l: row 4 s + l / 16, columns 8 (l % 16) + e); h then
// passes through the wave's LDS tile to the matrix-core layout (lane l: row
// l % 16, columns 32 s + 8 (l / 16) + e).  MFMA (s, e): A[m][k] = h[t0 + m][32 s
// + 8 k + e], B[k][n] = A_lora[n][same column]; D[m][n] gathers the row's sum
// over the wave's columns.  The waves' sums meet in LDS in wave order; the
// block writes part[blockIdx.x][t][j].
constexpr int SFW = 512;

template <int NR>
__global__ __launch_bounds__(256) void swiglu_fwd_lora_kernel(
    const bf16_t* __restrict__ g, int64_t ldg, const bf16_t* __restrict__ u, int64_t ldu,
    const int32_t* __restrict__ rows, int64_t Tn, int64_t F, bf16_t* __restrict__ h, int64_t ldh,
    const bf16_t* __restrict__ A, int64_t lda, int64_t r, float* __restrict__ part) {
    constexpr int RW = 16 * NR;
    __shared__ float red[4][16][RW + 1];
    __shared__ __attribute__((aligned(16))) bf16_t tile[4][16][128 + 8];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int rr = lane & 15, kq = lane >> 4;       // matrix-core layout
    const int cg = lane & 15, rs = lane >> 4;       // load layout
    const int64_t t0 = (int64_t)blockIdx.y * 16;
    const int64_t cw = (int64_t)blockIdx.x * (4 * SFW) + (int64_t)wid * SFW;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    f32x4 acc[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) acc[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // the loads of a 128-channel step; step cs + 128's go out before step cs
    // is processed
    uint4 gv[4], uv[4], av[4][NR], gn[4], un[4], an[4][NR];
    const int64_t cend = (cw + SFW < F) ? cw + SFW : F;
    auto fetch = [&](int64_t cs, uint4 (&g4)[4], uint4 (&u4)[4], uint4 (&a4)[4][NR]) {
        const int64_t cl = cs + 8 * cg;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t m = t0 + 4 * s + rs;
            const bool ok = m < Tn && cl < F;
            const int64_t t = (rows && m < Tn) ? (int64_t)rows[m] : m;
            g4[s] = ok ? *(const uint4*)(g + t * ldg + cl) : zero;
            u4[s] = ok ? *(const uint4*)(u + t * ldu + cl) : zero;
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                const int64_t j = 16 * k + rr, c = cs + 32 * s + 8 * kq;
                a4[s][k] = (c < F && j < r) ? *(const uint4*)(A + j * lda + c) : zero;
            }
        }
    };
    if (cw < cend) fetch(cw, gv, uv, av);
    for (int64_t cs = cw; cs < cend; cs += 128) {
        const int64_t cl = cs + 8 * cg;
        if (cs + 128 < cend) fetch(cs + 128, gn, un, an);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float gf[8], uf[8];
            unpack_bf16x8(gv[s], gf);
            unpack_bf16x8(uv[s], uf);
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float h0 = gf[2 * q] * sigmoid_hw(gf[2 * q]) * uf[2 * q];
                const float h1 = gf[2 * q + 1] * sigmoid_hw(gf[2 * q + 1]) * uf[2 * q + 1];
                w[q] = pack_bf16x2(h0, h1);
            }
            const uint4 hv = make_uint4(w[0], w[1], w[2], w[3]);
            const int64_t m = t0 + 4 * s + rs;
            if (m < Tn && cl < F) *(uint4*)(h + ((rows ? (int64_t)rows[m] : m) * ldh) + cl) = hv;
            *(uint4*)&tile[wid][4 * s + rs][8 * cg] = hv;   // rows past T / columns past F: zeros
        }
        // (this wave's own LDS rows: in-order LDS access within the wave)
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float hb[8];
            unpack_bf16x8(*(const uint4*)&tile[wid][rr][32 * s + 8 * kq], hb);
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                float af[8];
                unpack_bf16x8(av[s][k], af);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(hb[e], af[e], acc[k], 0, 0, 0);
            }
        }
        wave_lds_sync();
        if (cs + 128 < cend) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                gv[s] = gn[s];
                uv[s] = un[s];
#pragma unroll
                for (int k = 0; k < NR; ++k) av[s][k] = an[s][k];
            }
        }
    }
    // lane holds D[4 (l / 16) + i][l % 16]: row t0 + 4 kq + i, rank 16 k + rr
#pragma unroll
    for (int k = 0; k < NR; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wid][4 * kq + i][16 * k + rr] = acc[k][i];
    __syncthreads();
    for (int q = threadIdx.x; q < 16 * RW; q += 256) {
        const int row = q / RW, j = q % RW;
        const float v = ((red[0][row][j] + red[1][row][j]) + red[2][row][j]) + red[3][row][j];
        if (t0 + row < Tn) part[((int64_t)blockIdx.x * Tn + t0 + row) * RW + j] = v;
    }
}

// Backward: dg, du as swiglu_bwd, plus the token reductions over the same
// tiles: P0[c][j] = sum_t h[t, c] Y0[t, j] (h = silu(g) u recomputed exactly
// as the forward stored it), P1[c][j] = sum_t dg[t, c] Y1[t, j], P2[c][j] =
// sum_t du[t, c] Y2[t, j] (dg, du as stored).  A block of 4 waves covers 512
// columns (wave: 128; lane l: the 8 columns 8 (l % 16) + e of row t0 + l / 16,
// so a row's 256 bytes leave as one run) and the rows of one chunk, 4 at a
// time.  MFMA (e): A[m][k] = X[t0 + k][cw + 8 m + e], B[k][n] = Y[t0 + k][n];
// D accumulates over the chunk; each chunk writes part[p][chunk][c][j].
template <int NR>
__global__ __launch_bounds__(256) void swiglu_bwd_lora_kernel(
    const bf16_t* __restrict__ dh, int64_t lddh, const bf16_t* __restrict__ g, int64_t ldg,
    const bf16_t* __restrict__ u, int64_t ldu, int64_t Tn, int64_t F, bf16_t* __restrict__ dg, int64_t lddg,
    bf16_t* __restrict__ du, int64_t lddu, const float* __restrict__ Y0, int64_t ldy0,
    const float* __restrict__ Y1, int64_t ldy1, const float* __restrict__ Y2, int64_t ldy2, int64_t r,
    int64_t rows_per_chunk, float* __restrict__ part) {
    constexpr int RW = 16 * NR;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int cg = lane & 15, rs = lane >> 4;
    const int64_t cw = (int64_t)blockIdx.x * 512 + (int64_t)wid * 128;
    const int64_t c = cw + 8 * cg;
    const bool cv = c < F;
    const int64_t tb = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t te = (Tn - tb) < rows_per_chunk ? Tn : tb + rows_per_chunk;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    f32x4 acc[3][NR][8];
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[p][k][e] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // one 4-row slab at a time, the next slab's loads in flight while this
    // one is processed (its matrix-core work would otherwise sit between a
    // wave's loads; two waves per SIMD do not cover that)
    uint4 vd, vg, vu;
    float y0[NR], y1[NR], y2[NR];
    auto fetch = [&](int64_t tu) {
        const int64_t t = tu + rs;
        const bool tv = t < te;
        const bool ok = cv && tv;
        vd = ok ? *(const uint4*)(dh + t * lddh + c) : zero;
        vg = ok ? *(const uint4*)(g + t * ldg + c) : zero;
        vu = ok ? *(const uint4*)(u + t * ldu + c) : zero;
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int64_t j = 16 * k + cg;
            const bool yv = tv && j < r;
            y0[k] = yv ? Y0[t * ldy0 + j] : 0.0f;
            y1[k] = yv ? Y1[t * ldy1 + j] : 0.0f;
            y2[k] = yv ? Y2[t * ldy2 + j] : 0.0f;
        }
    };
    if (tb < te) fetch(tb);
    for (int64_t tu = tb; tu < te; tu += 4) {
        const uint4 cd = vd, cgv = vg, cu = vu;
        float z0[NR], z1[NR], z2[NR];
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            z0[k] = y0[k];
            z1[k] = y1[k];
            z2[k] = y2[k];
        }
        if (tu + 4 < te) fetch(tu + 4);
        {
            const int64_t t = tu + rs;
            const bool ok = cv && t < te;
            float d[8], gf[8], uf[8];
            unpack_bf16x8(cd, d);
            unpack_bf16x8(cgv, gf);
            unpack_bf16x8(cu, uf);
            uint32_t wa[4], wb[4], wh[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float a2[2], b2[2], h2[2];
#pragma unroll
                for (int o = 0; o < 2; ++o) {
                    const int e = 2 * q + o;
                    const float sg = sigmoid_hw(gf[e]);
                    a2[o] = d[e] * uf[e] * (sg * (1.0f + gf[e] * (1.0f - sg)));
                    b2[o] = d[e] * (gf[e] * sg);
                    h2[o] = gf[e] * sg * uf[e];
                }
                wa[q] = pack_bf16x2(a2[0], a2[1]);
                wb[q] = pack_bf16x2(b2[0], b2[1]);
                wh[q] = pack_bf16x2(h2[0], h2[1]);
            }
            const uint4 va = make_uint4(wa[0], wa[1], wa[2], wa[3]);
            const uint4 vb = make_uint4(wb[0], wb[1], wb[2], wb[3]);
            if (ok) {
                *(uint4*)(dg + t * lddg + c) = va;
                *(uint4*)(du + t * lddu + c) = vb;
            }
            float hb[8], ab[8], bb[8];
            unpack_bf16x8(make_uint4(wh[0], wh[1], wh[2], wh[3]), hb);
            unpack_bf16x8(va, ab);
            unpack_bf16x8(vb, bb);
#pragma unroll
            for (int k = 0; k < NR; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    acc[0][k][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(hb[e], z0[k], acc[0][k][e], 0, 0, 0);
                    acc[1][k][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(ab[e], z1[k], acc[1][k][e], 0, 0, 0);
                    acc[2][k][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(bb[e], z2[k], acc[2][k][e], 0, 0, 0);
                }
        }
    }
    // lane holds D[4 (l / 16) + i][l % 16] of MFMA e: column cw + 8 (4 rs + i) + e, rank 16 k + cg
    const int64_t nch = gridDim.y;
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t col = cw + 8 * (4 * rs + i) + e;
                    const int64_t j = 16 * k + cg;
                    if (col < F && j < r)
                        part[(((int64_t)p * nch + blockIdx.y) * F + col) * RW + j] = acc[p][k][e][i];
                }
}

// out[a' soa + j soj] = scale * sum over ch = 0.. of part[(ch A + a) RW + j]
// (ascending ch), j < r, a' = amap[a] (or a): the ordered sum of the fused
// kernels' partials.
__global__ __launch_bounds__(256) void chunk_sum_kernel(const float* __restrict__ part, int64_t nch, int64_t Adim,
                                                       int RW, int64_t r, float scale, float* __restrict__ out,
                                                       int64_t soa, int64_t soj, const int32_t* __restrict__ amap) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= Adim * r) return;
    const int64_t a = q / r, j = q % r;
    // (eight chunks' loads go out together; the sum keeps chunk order)
    float s = 0.0f;
    int64_t ch = 0;
    for (; ch + 8 <= nch; ch += 8) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = part[((ch + e) * Adim + a) * RW + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) s += v[e];
    }
    for (; ch < nch; ++ch) s += part[(ch * Adim + a) * RW + j];
    const int64_t ao = amap ? (int64_t)amap[a] : a;   // output row of partial row a
    out[ao * soa + j * soj] = scale * s;
}

// The three ordered sums of the fused SwiGLU backward in one launch:
// blockIdx.y = p sums partial set p (at part + p pstride) into out[p] with
// strides soa[p], soj[p], exactly as chunk_sum_kernel does.
struct ChunkSum3 {
    float* out[3];
    int64_t soa[3], soj[3];
};
__global__ __launch_bounds__(256) void chunk_sum3_kernel(const float* __restrict__ part, int64_t pstride, int64_t nch,
                                                        int64_t Adim, int RW, int64_t r, float scale, ChunkSum3 o) {
    const int p = (int)blockIdx.y;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= Adim * r) return;
    const int64_t a = q / r, j = q % r;
    const float* __restrict__ pp = part + p * pstride;
    float s = 0.0f;
    int64_t ch = 0;
    for (; ch + 8 <= nch; ch += 8) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = pp[((ch + e) * Adim + a) * RW + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) s += v[e];
    }
    for (; ch < nch; ++ch) s += pp[(ch * Adim + a) * RW + j];
    o.out[p][a * o.soa[p] + j * o.soj[p]] = scale * s;
}

// ---------------------------------------------------------------- forward SwiGLU of context rows from their compact product
// For the listed (context) rows t = rows[m] and every channel c < F:
//   g = Yc[m, j]     if c = idx[j] (selected), else s P[t, :] . B[c, :]
//   u = Yc[m, n + j] if c = idx[j],            else s P[t, :] . B[F + c, :]
// exactly as the merge of the gate|up compact product forms them (the
// rank-r values on the matrix cores from s P rounded to bf16, one bf16
// rounding), stored to gu[t, c] and gu[t, F + c]; then h = silu(g) u (bf16,
// as swiglu_fwd) goes to the compact hc[m, j] = h[t, idx[j]] (columns n ..
// npad zero), optionally to hf[t, :] (the whole row), and into the row sums
// xl[t, :] = sum over every c of h[t, c] A[:, c] (fp32 matrix cores, row
// partials per 512 channels, a fixed-order sum follows).  Block = 4 waves on 64 rows (four 16-row tiles) and 512
// channels, wave w on 128 of them; the tiles pass through the wave's LDS
// rows between the matrix-core layout (lane l: row l % 16, 8 channels at
// 32 g + 8 (l / 16)) and the row-store layout (lane l: row 4 q + l / 16, 8
// channels at 8 (l % 16)).
constexpr int SCR = 64;   // rows per block

template <int R, int NR>
__global__ __launch_bounds__(256) void swiglu_fwd_ctx_kernel(
    bf16_t* __restrict__ gu, int64_t ldgu, const int32_t* __restrict__ rows, int64_t nrows, int64_t F,
    const float* __restrict__ P, int64_t ldp, const bf16_t* __restrict__ B, int64_t ldb, int64_t r2, float scale,
    const bf16_t* __restrict__ Yc, int64_t ldyc, const int32_t* __restrict__ idx, int64_t n,
    bf16_t* __restrict__ hc, int64_t ldhc, int64_t npad, const bf16_t* __restrict__ A, int64_t lda, int64_t r,
    bf16_t* __restrict__ hf, int64_t ldhf, float* __restrict__ part) {
    constexpr int KS = (R + 31) / 32;
    constexpr int RW = 16 * NR;
    __shared__ __attribute__((aligned(16))) bf16_t tg[4][16][128 + 8];
    __shared__ __attribute__((aligned(16))) bf16_t tu[4][16][128 + 8];
    __shared__ __attribute__((aligned(16))) bf16_t cb[4][16][136];   // compact values of the wave's run
    __shared__ float red[4][SCR][RW + 1];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int rr = lane & 15, kq = lane >> 4;
    const int64_t c0 = (int64_t)blockIdx.x * 512 + (int64_t)wid * 128;
    const int64_t mb = (int64_t)blockIdx.y * SCR;
    const int kl = 8 * kq;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    // the rank-r factor rows of this wave's gate and up channels (slot order
    // of the matrix-core layout), and A's columns for the row sums
    bf16x8 wg[KS][4][2], wu[KS][4][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int64_t c = c0 + 32 * g + 8 * (rr >> 2) + 4 * e + (rr & 3);
                const int k = 32 * ks + kl;
                uint4 a = zero, b = zero;
                if (c < F && k < r2) {
                    if (k + 8 <= r2) {
                        a = *(const uint4*)(B + c * ldb + k);
                        b = *(const uint4*)(B + (F + c) * ldb + k);
                    } else {
                        uint32_t wa[4] = {0u, 0u, 0u, 0u}, wb[4] = {0u, 0u, 0u, 0u};
                        for (int q = 0; q < 8; ++q)
                            if (k + q < r2) {
                                wa[q >> 1] |= (uint32_t)B[c * ldb + k + q] << ((q & 1) * 16);
                                wb[q >> 1] |= (uint32_t)B[(F + c) * ldb + k + q] << ((q & 1) * 16);
                            }
                        a = make_uint4(wa[0], wa[1], wa[2], wa[3]);
                        b = make_uint4(wb[0], wb[1], wb[2], wb[3]);
                    }
                }
                wg[ks][g][e] = __builtin_bit_cast(bf16x8, a);
                wu[ks][g][e] = __builtin_bit_cast(bf16x8, b);
            }
    uint4 av[4][NR];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int64_t j = 16 * k + rr, c = c0 + 32 * s + kl;
            av[s][k] = (c < F && j < r) ? *(const uint4*)(A + j * lda + c) : zero;
        }
    // this wave's selected channels: idx[j0 .. j1) (at most 128); lane holds
    // entries j0 + lane and j0 + 64 + lane (slot in the wave's block, or -1)
    int64_t j0, j1;
    wave_lower_bounds(idx, n, c0, c0 + 128, lane, j0, j1);
    const int sl0 = j0 + lane < j1 ? (int)(idx[j0 + lane] - c0) : -1;
    const int sl1 = j0 + 64 + lane < j1 ? (int)(idx[j0 + 64 + lane] - c0) : -1;
    // the compact values of a row arrive as 16-byte chunks (lane l: chunk
    // l % 16 of row 4 s + l / 16, and chunk 16 + l % 16 when the run needs a
    // 17th), aligned from jbg (gate, compact positions j) or jbu (up, n + j);
    // they pass through the wave's LDS rows, from which lane l moves compact
    // value j0 + l (and j0 + 64 + l) to its slot sl0 (sl1) of the tile
    const int cq = lane & 15;
    const int64_t jbg = j0 & ~(int64_t)7, jbu = (n + j0) & ~(int64_t)7;
    const bool two = (j1 - jbg > 128) || (n + j1 - jbu > 128);   // a 17th chunk (wave-uniform)
    const bool run64 = j1 - j0 > 64;                                 // wave-uniform
    const bool ldg0 = jbg + 8 * cq < j1, ldu0 = jbu + 8 * cq < n + j1;
    const bool ldg1 = two && jbg + 8 * (cq + 16) < j1, ldu1 = two && jbu + 8 * (cq + 16) < n + j1;
    const int og = (int)(j0 - jbg), ou = (int)(n + j0 - jbu);      // run start within the LDS rows
    f32x4 acc[SCR / 16][NR];
#pragma unroll
    for (int q = 0; q < SCR / 16; ++q)
#pragma unroll
        for (int k = 0; k < NR; ++k) acc[q][k] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < SCR / 16; ++q) {
        const int64_t m0 = mb + 16 * q;
        if (m0 >= nrows) break;   // uniform across the block
        const int64_t m = m0 + rr;
        const bool mv = m < nrows;
        const int64_t row = mv ? (int64_t)rows[m] : 0;
        // the compact values of the 16 rows, loaded ahead (16-byte chunks)
        uint4 cg[4], cu[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int64_t mr = m0 + 4 * s4 + kq;
            const bool ok = mr < nrows;
            const bf16_t* yr = Yc + mr * ldyc;
            cg[s4] = (ok && ldg0) ? *(const uint4*)(yr + jbg + 8 * cq) : zero;
            cu[s4] = (ok && ldu0) ? *(const uint4*)(yr + jbu + 8 * cq) : zero;
        }
        bf16x8 pb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int k = 32 * ks + kl;
            float v[8];
            if (mv && k + 8 <= r2 && (ldp & 3) == 0) {
                const float4 v0 = *(const float4*)(P + row * ldp + k), v1 = *(const float4*)(P + row * ldp + k + 4);
                v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
                v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (mv && k + e < r2) ? P[row * ldp + k + e] : 0.0f;
            }
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(scale * v[2 * e], scale * v[2 * e + 1]);
            pb[ks] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            f32x4 ag[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
            f32x4 au[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    ag[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg[ks][g][e], pb[ks], ag[e], 0, 0, 0);
                    au[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wu[ks][g][e], pb[ks], au[e], 0, 0, 0);
                }
            uint32_t w0[4], w1[4];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                w0[e] = pack_bf16x2(ag[0][2 * e], ag[0][2 * e + 1]);
                w0[2 + e] = pack_bf16x2(ag[1][2 * e], ag[1][2 * e + 1]);
                w1[e] = pack_bf16x2(au[0][2 * e], au[0][2 * e + 1]);
                w1[2 + e] = pack_bf16x2(au[1][2 * e], au[1][2 * e + 1]);
            }
            *(uint4*)&tg[wid][rr][kl + 32 * g] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
            *(uint4*)&tu[wid][rr][kl + 32 * g] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
        }
        // (this wave's own LDS rows: in-order LDS access within the wave)
        wave_lds_sync();
        // gate: the compact chunks to the LDS rows, then each run value to its slot
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) *(uint4*)&cb[wid][4 * s4 + kq][8 * cq] = cg[s4];
        if (two && cq == 0) {   // chunk 16 (lanes 0, 16, 32, 48: one per row)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int64_t mr = m0 + 4 * s4 + kq;
                *(uint4*)&cb[wid][4 * s4 + kq][128] =
                    (mr < nrows && ldg1) ? *(const uint4*)(Yc + mr * ldyc + jbg + 128) : zero;
            }
        }
        wave_lds_sync();
        if (sl0 >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) tg[wid][i][sl0] = cb[wid][i][og + lane];
        }
        if (run64 && sl1 >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) tg[wid][i][sl1] = cb[wid][i][og + 64 + lane];
        }
        wave_lds_sync();
        // up: the same through the same LDS rows
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) *(uint4*)&cb[wid][4 * s4 + kq][8 * cq] = cu[s4];
        if (two && cq == 0) {   // chunk 16 (lanes 0, 16, 32, 48: one per row)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int64_t mr = m0 + 4 * s4 + kq;
                *(uint4*)&cb[wid][4 * s4 + kq][128] =
                    (mr < nrows && ldu1) ? *(const uint4*)(Yc + mr * ldyc + jbu + 128) : zero;
            }
        }
        wave_lds_sync();
        if (sl0 >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) tu[wid][i][sl0] = cb[wid][i][ou + lane];
        }
        if (run64 && sl1 >= 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) tu[wid][i][sl1] = cb[wid][i][ou + 64 + lane];
        }
        wave_lds_sync();
        // whole rows of g and u to gu; h into the g tile (each element is
        // read and rewritten by the same lane)
        const int64_t cs = c0 + 8 * rr;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int tr = 4 * jj + kq;
            const int64_t orow = __shfl(row, tr, 64);
            const int ov = __shfl((int)mv, tr, 64);
            const uint4 gv = *(const uint4*)&tg[wid][tr][8 * rr];
            const uint4 uv = *(const uint4*)&tu[wid][tr][8 * rr];
            if (ov && cs < F) {
                *(uint4*)(gu + orow * ldgu + cs) = gv;
                *(uint4*)(gu + orow * ldgu + F + cs) = uv;
            }
            float gf[8], uf[8];
            unpack_bf16x8(gv, gf);
            unpack_bf16x8(uv, uf);
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float h0 = gf[2 * e] * sigmoid_hw(gf[2 * e]) * uf[2 * e];
                const float h1 = gf[2 * e + 1] * sigmoid_hw(gf[2 * e + 1]) * uf[2 * e + 1];
                w[e] = pack_bf16x2(h0, h1);
            }
            const uint4 hv = make_uint4(w[0], w[1], w[2], w[3]);
            *(uint4*)&tg[wid][tr][8 * rr] = hv;
            if (hf && ov && cs < F) *(uint4*)(hf + orow * ldhf + cs) = hv;   // optional full rows of h
        }
        wave_lds_sync();
        // the selected channels of h to the compact rows
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (m0 + i >= nrows) break;
            bf16_t* hr = hc + (m0 + i) * ldhc + j0;
            if (sl0 >= 0) hr[lane] = tg[wid][i][sl0];
            if (sl1 >= 0) hr[64 + lane] = tg[wid][i][sl1];
        }
        // row sums of h A^T: MFMA (s, e) with A[m][k] = h[m][32 s + 8 k + e]
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float hb[8];
            unpack_bf16x8(*(const uint4*)&tg[wid][rr][32 * s + kl], hb);
#pragma unroll
            for (int k = 0; k < NR; ++k) {
                float af[8];
                unpack_bf16x8(av[s][k], af);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[q][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(hb[e], af[e], acc[q][k], 0, 0, 0);
            }
        }
        wave_lds_sync();
    }
    // zero padding of the compact rows (columns n .. npad)
    if (blockIdx.x == 0 && wid == 0 && npad > n) {
        const int64_t w = npad - n;
        for (int64_t q = lane; q < SCR * w; q += 64) {
            const int64_t m = mb + q / w;
            if (m < nrows) hc[m * ldhc + n + q % w] = (bf16_t)0;
        }
    }
    // lane holds D[4 (l / 16) + i][l % 16] of tile q: row m0 + 4 kq + i, rank 16 k + rr
#pragma unroll
    for (int q = 0; q < SCR / 16; ++q)
#pragma unroll
        for (int k = 0; k < NR; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wid][16 * q + 4 * kq + i][16 * k + rr] = acc[q][k][i];
    __syncthreads();
    for (int q = threadIdx.x; q < SCR * RW; q += 256) {
        const int row = q / RW, j = q % RW;
        const float v = ((red[0][row][j] + red[1][row][j]) + red[2][row][j]) + red[3][row][j];
        if (mb + row < nrows) part[((int64_t)blockIdx.x * nrows + mb + row) * RW + j] = v;
    }
}

// out[m, q..q+7] = in[rows[m], cols[q..q+7]]: gathered loads, one vector store.
template <typename T>
__global__ void gather_cols_kernel(const T* __restrict__ in, int64_t ldi,
                                   const int32_t* __restrict__ rows, int64_t nrows,
                                   const int32_t* __restrict__ cols, int64_t ncols,
                                   int64_t npad, T* __restrict__ out, int64_t ldo) {
    const int64_t m = blockIdx.y;
    const int64_t q0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (q0 >= npad) return;
    const T* src = in + (int64_t)rows[m] * ldi;
    T* dst = out + m * ldo + q0;
    if (q0 + 8 <= ncols) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = ld<T>(src, cols[q0 + e]);
        store8<T>(dst, v);
    } else {
        // ragged end: the last selected columns, then zeros up to npad
        for (int64_t q = q0; q < npad && q < q0 + 8; ++q) dst[q - q0] = q < ncols ? src[cols[q]] : (T)0;
    }
}

// Zero the unselected channels of the given rows.  Thread = 8 consecutive
// channels (membership found once by a binary search in the ascending index
// list) x 16 rows; all-unselected groups are cleared with one vector store.
template <typename T>
__global__ void zero_unselected_kernel(T* __restrict__ y, int64_t ldy,
                                       const int32_t* __restrict__ rows, int64_t nrows, int64_t C,
                                       const int32_t* __restrict__ idx, int64_t n) {
    const int64_t c0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (c0 >= C) return;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (idx[mid] < c0) lo = mid + 1; else hi = mid;
    }
    unsigned keep = 0;
    for (int e = 0; e < 8; ++e) {
        const int64_t c = c0 + e;
        while (lo < n && idx[lo] < c) ++lo;
        if (lo < n && idx[lo] == c) keep |= 1u << e;
    }
    const int64_t r0 = (int64_t)blockIdx.y * 16;
    const int64_t r1 = (r0 + 16 < nrows) ? r0 + 16 : nrows;
    const float zeros[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t rr = r0; rr < r1; ++rr) {
        T* yr = y + (int64_t)rows[rr] * ldy + c0;
        if (keep == 0 && c0 + 8 <= C) {
            store8<T>(yr, zeros);
        } else {
            for (int e = 0; e < 8; ++e)
                if (c0 + e < C && !((keep >> e) & 1u)) yr[e] = (T)0;
        }
    }
}


// out[j, q] = src[idx[q], j]: gather rows of a channel-major matrix and
// transpose them (a 64 x 64 tile through LDS; coalesced on both sides).
template <typename T>
__global__ __launch_bounds__(256) void gather_rows_t_kernel(const T* __restrict__ src, int64_t lds,
                                                            const int32_t* __restrict__ idx,
                                                            int64_t n, int64_t npad, int64_t Dd,
                                                            T* __restrict__ out, int64_t ldo) {
    __shared__ T tile[64][65];
    const int64_t q0 = (int64_t)blockIdx.x * 64, j0 = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int64_t q = q0 + i, j = j0 + tx;
        T v = (T)0;
        if (q < n && j < Dd) v = src[(int64_t)idx[q] * lds + j];
        tile[i][tx] = v;
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int64_t j = j0 + i, q = q0 + tx;
        if (j < Dd && q < npad) out[j * ldo + q] = tile[tx][i];   // zeros past n
    }
}
// bf16 form: tile of 64 selected channels x 128 output rows; 16-byte loads
// along the source rows, 16-byte stores along the output rows, the transpose
// in LDS (row pitch 136 elements: the 8 strided 2-byte reads of a store hit
// different banks).
__global__ __launch_bounds__(256) void gather_rows_t_bf16_kernel(const bf16_t* __restrict__ src,
                                                                 int64_t lds,
                                                                 const int32_t* __restrict__ idx,
                                                                 int64_t n, int64_t npad, int64_t Dd,
                                                                 bf16_t* __restrict__ out, int64_t ldo) {
    __shared__ __attribute__((aligned(16))) bf16_t tile[64][136];
    const int64_t q0 = (int64_t)blockIdx.x * 64, j0 = (int64_t)blockIdx.y * 128;
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int qq = tid + 256 * c;
        const int i = qq >> 4, jj = (qq & 15) * 8;        // source row i of the tile, columns jj..jj+7
        const int64_t q = q0 + i, j = j0 + jj;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (q < n && j < Dd) {
            const bf16_t* sp = src + (int64_t)idx[q] * lds + j;
            if (j + 8 <= Dd) {
                v = *(const uint4*)sp;
            } else {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int e = 0; e < 8; ++e)
                    if (j + e < Dd) w[e >> 1] |= (uint32_t)sp[e] << ((e & 1) * 16);
                v = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        *(uint4*)&tile[i][jj] = v;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int qq = tid + 256 * c;
        const int jj = qq >> 3, i8 = (qq & 7) * 8;        // output row jj of the tile, channels i8..i8+7
        const int64_t j = j0 + jj, q = q0 + i8;
        if (j >= Dd || q >= npad) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)tile[i8 + 2 * e][jj] | ((uint32_t)tile[i8 + 2 * e + 1][jj] << 16);
        bf16_t* op = out + j * ldo + q;
        if (q + 8 <= npad) {
            *(uint4*)op = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            for (int e = 0; e < 8 && q + e < npad; ++e) op[e] = (bf16_t)(w[e >> 1] >> ((e & 1) * 16));
        }
    }
}


// comp[c - #selected below c] = c for every unselected channel c
__global__ void complement_kernel(const int32_t* __restrict__ idx, int64_t n, int64_t C,
                                  int32_t* __restrict__ comp) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= C) return;
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (idx[mid] < c) lo = mid + 1; else hi = mid;
    }
    if (!(lo < n && idx[lo] == c)) comp[c - lo] = (int32_t)c;
}

}  // namespace

// workspace floats the bf16 split-K form needs (0: none)
size_t lora_xl_ws_floats(int64_t T, int64_t D, int64_t r) {
    if (T <= 0 || r <= 0) return 0;
    const int64_t rb = ceil_div(T, XR);
    int64_t ks = ceil_div(D, 1024);
    if (rb * ks < 512) ks = ceil_div(512, rb);
    if (ks > 16) ks = 16;
    const int64_t kmax = ceil_div(D, XKC);
    if (ks > kmax) ks = kmax;
    const int64_t R = r <= 16 ? 16 : (r <= 32 ? 32 : 64);
    return (size_t)(ks * T * R);
}

hipError_t launch_lora_xl(bool bf16, const void* x, int64_t ldx, int64_t T, int64_t D,
                          const void* A, int64_t lda, int64_t r, float* xl, int64_t ldxl,
                          float* ws, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (bf16 && ws) {
        const int64_t rb = ceil_div(T, XR);
        const int64_t R = r <= 16 ? 16 : (r <= 32 ? 32 : 64);
        const int64_t ks = (int64_t)(lora_xl_ws_floats(T, D, r) / (size_t)(T * R));
        const int64_t kchunk = ceil_div(ceil_div(D, ks), XKC) * XKC;
        const int64_t ksn = ceil_div(D, kchunk);     // chunks actually used
        const dim3 grid((unsigned)rb, (unsigned)ksn);
#define XL(RR)                                                                                  \
    hipLaunchKernelGGL((lora_xl_split_kernel<RR>), grid, dim3(256), 0, st, (const bf16_t*)x, ldx, T, \
                       D, (const bf16_t*)A, lda, r, kchunk, ws)
        if (R == 16) XL(16);
        else if (R == 32) XL(32);
        else XL(64);
#undef XL
        hipLaunchKernelGGL(lora_xl_reduce_kernel, dim3((unsigned)ceil_div(T * r, 256)), dim3(256), 0, st,
                           ws, ksn, T, r, R, xl, ldxl);
    } else if (bf16) {
        hipLaunchKernelGGL(lora_xl_bf16_kernel, dim3((unsigned)ceil_div(T, 16)), dim3(XW * 64), 0, st,
                           (const bf16_t*)x, ldx, T, D, (const bf16_t*)A, lda, r, xl, ldxl);
    } else {
        hipLaunchKernelGGL(lora_xl_f32_kernel, dim3((unsigned)ceil_div(T, 4)), dim3(256), 0,
                           st, (const float*)x, ldx, T, D, (const float*)A, lda, r, xl, ldxl);
    }
    return hipGetLastError();
}

hipError_t launch_lora_add(bool bf16, const float* P, int64_t ldp, int64_t T, int64_t r,
                           const void* Bm, int64_t sb_c, int64_t sb_j, int64_t Ncols,
                           float scale, void* y, int64_t ldy, hipStream_t st) {
    if (T <= 0 || Ncols <= 0) return hipSuccess;
    constexpr int64_t RPW = 32;  // rows per wave
    const dim3 block(256);
#define ADD(TT, RR, CP)                                                                        \
    hipLaunchKernelGGL((lora_add_kernel<TT, RR, CP>),                                          \
                       dim3((unsigned)ceil_div(Ncols, 64 * CP), (unsigned)ceil_div(T, 4 * RPW)), \
                       block, 0, st, P, ldp, T, r, (const TT*)Bm, sb_c, sb_j, Ncols, scale,     \
                       (TT*)y, ldy, RPW)
    if (bf16) {
        if (r <= 8) ADD(bf16_t, 8, 4);
        else if (r <= 16) ADD(bf16_t, 16, 4);
        else if (r <= 32) ADD(bf16_t, 32, 4);
        else ADD(bf16_t, 64, 2);
    } else {
        if (r <= 8) ADD(float, 8, 4);
        else if (r <= 16) ADD(float, 16, 4);
        else if (r <= 32) ADD(float, 32, 4);
        else ADD(float, 64, 2);
    }
#undef ADD
    return hipGetLastError();
}

hipError_t launch_outer_accum(bool bf16, const float* P, int64_t ldp, int64_t T, int64_t r,
                              const void* Q, int64_t ldq, int64_t Ncols, float scale, float* out,
                              int64_t so_j, int64_t so_c, float* ws, size_t ws_floats,
                              hipStream_t st) {
    if (Ncols <= 0 || r <= 0) return hipSuccess;
    // bf16 Q with 16-byte aligned rows: matrix-core kernel, 512-token chunks
    const bool mfma = bf16 && ldq % 8 == 0 && ((uintptr_t)Q & 15) == 0;
    const int64_t tch = mfma ? OTC : TCH;
    const int64_t nch = T > 0 ? ceil_div(T, tch) : 0;
    if ((size_t)(nch * r * Ncols) > ws_floats) return hipErrorInvalidValue;
    if (T > 0 && mfma) {
        const dim3 grid((unsigned)ceil_div(Ncols, 128), (unsigned)nch);
#define OUTERM(RR)                                                                             \
    hipLaunchKernelGGL((outer_mfma_kernel<RR>), grid, dim3(OW * 64), 0, st, P, ldp, T, r,      \
                       (const bf16_t*)Q, ldq, Ncols, ws)
        if (r <= 16) OUTERM(16);
        else if (r <= 32) OUTERM(32);
        else OUTERM(64);
#undef OUTERM
    } else if (T > 0) {
        const dim3 grid((unsigned)ceil_div(Ncols, 256), (unsigned)nch);
#define OUTER(TT, RR)                                                                          \
    hipLaunchKernelGGL((outer_partial_kernel<TT, RR>), grid, dim3(256), 0, st, P, ldp, T, r,   \
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
                       st, ws, nch, r, Ncols, scale, out, so_j, so_c);
    return hipGetLastError();
}

hipError_t launch_lora_fill_rows(void* y, int64_t ldy, const int32_t* rows, int64_t nrows,
                                 int64_t C, const float* P, int64_t ldp, const void* B,
                                 int64_t ldb, int64_t r, float scale, const int32_t* idx,
                                 int64_t n, uint32_t* mask, int beta, hipStream_t st) {
    if (nrows <= 0 || C <= 0) return hipSuccess;
    if (r < 1 || r > 128) return hipErrorInvalidValue;
    if (beta) {
        hipLaunchKernelGGL(select_mask_kernel, dim3((unsigned)ceil_div(ceil_div(C, 32), 256)),
                           dim3(256), 0, st, idx, n, C, mask);
    }
    const dim3 grid((unsigned)ceil_div(C, 128), (unsigned)ceil_div(nrows, 4 * FTW));
#define FILL(RR)                                                                                  \
    hipLaunchKernelGGL((lora_fill_rows_kernel<RR>), grid, dim3(256), 0, st, (bf16_t*)y, ldy, rows, \
                       nrows, C, P, ldp, (const bf16_t*)B, ldb, r, scale, (const uint32_t*)mask, beta)
    if (r <= 32) FILL(32);
    else if (r <= 64) FILL(64);
    else FILL(128);
#undef FILL
    return hipGetLastError();
}

hipError_t launch_lora_merge_rows(void* y, int64_t ldy, const int32_t* rows, int64_t nrows,
                                  int64_t C, const float* P, int64_t ldp, const void* B,
                                  int64_t ldb, int64_t r, float scale, const void* Yc,
                                  int64_t ldyc, const int32_t* idx, int64_t n, hipStream_t st,
                                  int merge_rows) {
    if (nrows <= 0 || C <= 0) return hipSuccess;
    if (P && (r < 1 || r > 128)) return hipErrorInvalidValue;
    const int mtw = merge_rows == 16 || merge_rows == 32 ? merge_rows : 64;
    const dim3 grid((unsigned)ceil_div(C, 128), (unsigned)ceil_div(nrows, 4 * mtw));
#define MERGE(RR, TW)                                                                                  \
    hipLaunchKernelGGL((lora_merge_rows_kernel<RR, TW>), grid, dim3(256), 0, st, (bf16_t*)y, ldy, rows, \
                       nrows, C, P, ldp, (const bf16_t*)B, ldb, P ? r : 0, scale, (const bf16_t*)Yc, ldyc, idx, n)
#define MERGE_R(TW)                    \
    if (!P || r <= 32) MERGE(32, TW);  \
    else if (r <= 64) MERGE(64, TW);   \
    else MERGE(128, TW);
    if (mtw == 16) { MERGE_R(16) }
    else if (mtw == 32) { MERGE_R(32) }
    else { MERGE_R(64) }
#undef MERGE_R
#undef MERGE
    return hipGetLastError();
}

// ---------------------------------------------------------------- dot statistics
// (a.b, a.a, b.b) over n fp32 values in fp64 (each product exact), in a fixed
// order: thread i of block g sums elements g*256 + i + k*DOT_G*256, k = 0, 1,
// ...; a block combines its 256 thread sums by a pairwise tree in LDS, and a
// second launch combines the DOT_G block sums by the same tree.
constexpr int DOT_G = 256;

__device__ __forceinline__ void tree3(double (*s)[256], int tid) {
    for (int w = 128; w >= 1; w >>= 1) {
        if (tid < w) {
#pragma unroll
            for (int j = 0; j < 3; ++j) s[j][tid] += s[j][tid + w];
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void dot_stats_partial_kernel(const float* __restrict__ a,
                                                                const float* __restrict__ b,
                                                                int64_t n, double* __restrict__ part) {
    __shared__ double s[3][256];
    const int tid = threadIdx.x;
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n; i += (int64_t)DOT_G * 256) {
        const double x = a[i], y = b[i];
        ab = __builtin_fma(x, y, ab);
        aa = __builtin_fma(x, x, aa);
        bb = __builtin_fma(y, y, bb);
    }
    s[0][tid] = ab;
    s[1][tid] = aa;
    s[2][tid] = bb;
    __syncthreads();
    tree3(s, tid);
    if (tid < 3) part[(int64_t)blockIdx.x * 3 + tid] = s[tid][0];
}

__global__ __launch_bounds__(256) void dot_stats_final_kernel(const double* __restrict__ part,
                                                              double* __restrict__ out) {
    __shared__ double s[3][256];
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 3; ++j) s[j][tid] = part[tid * 3 + j];
    __syncthreads();
    tree3(s, tid);
    if (tid < 3) out[tid] = s[tid][0];
}

hipError_t launch_dot_stats(const float* a, const float* b, int64_t n, double* part, double* out,
                            hipStream_t st) {
    hipLaunchKernelGGL(dot_stats_partial_kernel, dim3(DOT_G), dim3(256), 0, st, a, b, n, part);
    hipLaunchKernelGGL(dot_stats_final_kernel, dim3(1), dim3(256), 0, st, part, out);
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
    const dim3 grid((unsigned)ceil_div(F, 256 * 8), (unsigned)T);
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
    const dim3 grid((unsigned)ceil_div(F, 256 * 8), (unsigned)T);
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
                              int64_t nrows, const int32_t* cols, int64_t ncols, int64_t npad,
                              void* out, int64_t ldo, hipStream_t st) {
    if (nrows <= 0 || npad <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(npad, 256 * 8), (unsigned)nrows);
    if (bf16)
        hipLaunchKernelGGL(gather_cols_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)in,
                           ldi, rows, nrows, cols, ncols, npad, (bf16_t*)out, ldo);
    else
        hipLaunchKernelGGL(gather_cols_kernel<float>, grid, dim3(256), 0, st, (const float*)in, ldi,
                           rows, nrows, cols, ncols, npad, (float*)out, ldo);
    return hipGetLastError();
}

hipError_t launch_zero_unselected(bool bf16, void* y, int64_t ldy, const int32_t* rows,
                                  int64_t nrows, const int32_t* idx, int64_t n, int64_t C,
                                  uint8_t* unused, hipStream_t st) {
    (void)unused;
    if (nrows <= 0 || C <= 0 || n >= C) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(C, 256 * 8), (unsigned)ceil_div(nrows, 16));
    if (bf16)
        hipLaunchKernelGGL(zero_unselected_kernel<bf16_t>, grid, dim3(256), 0, st, (bf16_t*)y, ldy,
                           rows, nrows, C, idx, n);
    else
        hipLaunchKernelGGL(zero_unselected_kernel<float>, grid, dim3(256), 0, st, (float*)y, ldy,
                           rows, nrows, C, idx, n);
    return hipGetLastError();
}

hipError_t launch_complement(const int32_t* idx, int64_t n, int64_t C, int32_t* comp,
                             hipStream_t st) {
    if (C <= 0 || n >= C) return hipSuccess;
    hipLaunchKernelGGL(complement_kernel, dim3((unsigned)ceil_div(C, 256)), dim3(256), 0, st, idx, n,
                       C, comp);
    return hipGetLastError();
}

hipError_t launch_gather_rows_t(bool bf16, const void* src, int64_t lds, const int32_t* idx,
                                int64_t n, int64_t npad, int64_t Dd, void* out, int64_t ldo,
                                hipStream_t st) {
    if (npad <= 0 || Dd <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(npad, 64), (unsigned)ceil_div(Dd, 64));
    const bool vec = lds % 8 == 0 && ldo % 8 == 0 && ((uintptr_t)src & 15) == 0 && ((uintptr_t)out & 15) == 0;
    if (bf16 && vec)
        hipLaunchKernelGGL(gather_rows_t_bf16_kernel, dim3((unsigned)ceil_div(npad, 64), (unsigned)ceil_div(Dd, 128)),
                           dim3(256), 0, st, (const bf16_t*)src, lds, idx, n, npad, Dd, (bf16_t*)out, ldo);
    else if (bf16)
        hipLaunchKernelGGL(gather_rows_t_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)src,
                           lds, idx, n, npad, Dd, (bf16_t*)out, ldo);
    else
        hipLaunchKernelGGL(gather_rows_t_kernel<float>, grid, dim3(256), 0, st, (const float*)src,
                           lds, idx, n, npad, Dd, (float*)out, ldo);
    return hipGetLastError();
}

size_t swiglu_fwd_lora_ws_floats(int64_t T, int64_t F, int64_t r) {
    const int64_t RW = r <= 16 ? 16 : 32;
    return (size_t)(ceil_div(F, 4 * SFW) * T * RW);
}

hipError_t launch_swiglu_fwd_lora(const void* g, int64_t ldg, const void* u, int64_t ldu, const int32_t* rows,
                                  int64_t nr, int64_t F, void* h, int64_t ldh, const void* A, int64_t lda, int64_t r,
                                  float* xl, int64_t ldxl, float* part, hipStream_t st) {
    if (nr <= 0 || F <= 0) return hipSuccess;
    const int64_t ncb = ceil_div(F, 4 * SFW);
    const dim3 grid((unsigned)ncb, (unsigned)ceil_div(nr, 16));
    const int RW = r <= 16 ? 16 : 32;
    if (r <= 16)
        hipLaunchKernelGGL(swiglu_fwd_lora_kernel<1>, grid, dim3(256), 0, st, (const bf16_t*)g, ldg,
                           (const bf16_t*)u, ldu, rows, nr, F, (bf16_t*)h, ldh, (const bf16_t*)A, lda, r, part);
    else
        hipLaunchKernelGGL(swiglu_fwd_lora_kernel<2>, grid, dim3(256), 0, st, (const bf16_t*)g, ldg,
                           (const bf16_t*)u, ldu, rows, nr, F, (bf16_t*)h, ldh, (const bf16_t*)A, lda, r, part);
    hipLaunchKernelGGL(chunk_sum_kernel, dim3((unsigned)ceil_div(nr * r, 256)), dim3(256), 0, st, part, ncb, nr, RW,
                       r, 1.0f, xl, ldxl, (int64_t)1, rows);
    return hipGetLastError();
}

size_t swiglu_bwd_lora_ws_floats(int64_t T, int64_t F, int64_t r, int64_t rows_per_chunk) {
    const int64_t RW = r <= 16 ? 16 : 32;
    return (size_t)(3 * ceil_div(T, rows_per_chunk) * F * RW);
}

hipError_t launch_swiglu_bwd_lora(const void* dh, int64_t lddh, const void* g, int64_t ldg, const void* u,
                                  int64_t ldu, int64_t T, int64_t F, void* dg, int64_t lddg, void* du,
                                  int64_t lddu, const float* Y0, int64_t ldy0, const float* Y1, int64_t ldy1,
                                  const float* Y2, int64_t ldy2, int64_t r, float scale, float* dA, float* dB1,
                                  float* dB2, int64_t rows_per_chunk, float* part, hipStream_t st) {
    if (F <= 0) return hipSuccess;
    // T = 0: no partials; the sums below write zero gradients
    const int64_t nch = T > 0 ? ceil_div(T, rows_per_chunk) : 0;
    const dim3 grid((unsigned)ceil_div(F, 512), (unsigned)nch);
    const int RW = r <= 16 ? 16 : 32;
#define SBL(NRR)                                                                                               \
    hipLaunchKernelGGL((swiglu_bwd_lora_kernel<NRR>), grid, dim3(256), 0, st, (const bf16_t*)dh, lddh,          \
                       (const bf16_t*)g, ldg, (const bf16_t*)u, ldu, T, F, (bf16_t*)dg, lddg, (bf16_t*)du, lddu, \
                       Y0, ldy0, Y1, ldy1, Y2, ldy2, r, rows_per_chunk, part)
    if (T <= 0) {
    } else if (r <= 16) {
        SBL(1);
    } else {
        SBL(2);
    }
#undef SBL
    // dA [r, F] (row j, column c); dB [F, r]: the three ordered sums in one launch
    const size_t pstride = (size_t)nch * F * RW;
    ChunkSum3 o;
    o.out[0] = dA;  o.soa[0] = 1; o.soj[0] = F;
    o.out[1] = dB1; o.soa[1] = r; o.soj[1] = 1;
    o.out[2] = dB2; o.soa[2] = r; o.soj[2] = 1;
    hipLaunchKernelGGL(chunk_sum3_kernel, dim3((unsigned)ceil_div(F * r, 256), 3), dim3(256), 0, st, part,
                       (int64_t)pstride, nch, F, RW, r, scale, o);
    return hipGetLastError();
}

size_t swiglu_fwd_ctx_ws_floats(int64_t nrows, int64_t F, int64_t r) {
    const int64_t RW = r <= 16 ? 16 : 32;
    return (size_t)(ceil_div(F, 512) * nrows * RW);
}

hipError_t launch_swiglu_fwd_ctx(void* gu, int64_t ldgu, const int32_t* rows, int64_t nrows, int64_t F,
                                 const float* P, int64_t ldp, const void* B, int64_t ldb, int64_t r2, float scale,
                                 const void* Yc, int64_t ldyc, const int32_t* idx, int64_t n, void* hc, int64_t ldhc,
                                 int64_t npad, const void* A, int64_t lda, int64_t r, float* xl, int64_t ldxl,
                                 void* hf, int64_t ldhf, float* part, hipStream_t st) {
    if (nrows <= 0 || F <= 0) return hipSuccess;
    if (r2 > 64 || r > 32) return hipErrorInvalidValue;
    const int64_t ncb = ceil_div(F, 512);
    const dim3 grid((unsigned)ncb, (unsigned)ceil_div(nrows, SCR));
    const int RW = r <= 16 ? 16 : 32;
#define SFC(RR, NRR)                                                                                          \
    hipLaunchKernelGGL((swiglu_fwd_ctx_kernel<RR, NRR>), grid, dim3(256), 0, st, (bf16_t*)gu, ldgu, rows, nrows, \
                       F, P, ldp, (const bf16_t*)B, ldb, r2, scale, (const bf16_t*)Yc, ldyc, idx, n, (bf16_t*)hc,  \
                       ldhc, npad, (const bf16_t*)A, lda, r, (bf16_t*)hf, ldhf, part)
    if (r2 <= 32) {
        if (r <= 16) SFC(32, 1);
        else SFC(32, 2);
    } else {
        if (r <= 16) SFC(64, 1);
        else SFC(64, 2);
    }
#undef SFC
    hipLaunchKernelGGL(chunk_sum_kernel, dim3((unsigned)ceil_div(nrows * r, 256)), dim3(256), 0, st, part, ncb,
                       nrows, RW, r, 1.0f, xl, ldxl, (int64_t)1, rows);
    return hipGetLastError();
}
