// Gathered-channel GEMMs of the sparse main branch.
//
// C[c_rows[m], c_cols[n]] (+)= sum_k A[a_rows[m], k] * B(n, k)
//   NT: B(n, k) = B[b_rows[n], k]      (weight rows are the selected channels)
//   NN: B(n, k) = B[b_rows[k], n]      (weight rows are the selected K channels)
// Any map may be absent (identity).  This covers every main-branch product:
// dense output-token rows (a_rows = c_rows = output rows), N-gathered context
// rows (b_rows = c_cols = selected channels) and K-gathered context rows
// (b_rows = selected channels over a compacted activation).  Only the selected
// weight rows are read; each is a contiguous row of the channel-major weight.
//
// bf16 path: v_mfma_f32_32x32x16_bf16, 128x128x64 block tile, 4 waves of
// 64x64, register-staged double-buffered LDS (row stride 72 bf16 so the
// 16-byte MFMA operand reads are conflict-free).  NN tiles are transposed on
// their way into LDS (pairs of rows repacked with byte permutes) so both
// layouts feed the same K-contiguous LDS format.  Block ids are remapped so
// that each XCD works on a contiguous run of tiles (shared weight tiles stay
// in that XCD's L2).
#include "sl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64, LDK = 72;
constexpr int NXCD = 8;

struct GemmArgs {
    GemmProblem p0, p1;
    int tiles0, tiles_m0, tiles_m1, total;
};

__device__ __forceinline__ int xcd_remap(int b, int nb) {
    const int xcd = b % NXCD, slot = b / NXCD;
    const int per = nb / NXCD, extra = nb % NXCD;
    return xcd * per + (xcd < extra ? xcd : extra) + slot;
}

__device__ __forceinline__ uint4 load16_guard(const bf16_t* rowp, int64_t k, int64_t K, bool rv) {
    uint4 v = {0u, 0u, 0u, 0u};
    if (!rv) return v;
    if (k + 8 <= K) return *(const uint4*)(rowp + k);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int e = 0; e < 8; ++e)
        if (k + e < K) w[e >> 1] |= (uint32_t)rowp[k + e] << ((e & 1) * 16);
    v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
    return v;
}

template <bool NN>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDK];

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const bool second = L >= args.tiles0;
    const GemmProblem P = second ? args.p1 : args.p0;
    const int t = second ? L - args.tiles0 : L;
    const int tiles_m = second ? args.tiles_m1 : args.tiles_m0;
    const int64_t m0 = (int64_t)(t % tiles_m) * BM;
    const int64_t n0 = (int64_t)(t / tiles_m) * BN;
    const int64_t M = P.M, N = P.N, K = P.K;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid & 1, wn = wid >> 1;
    const bf16_t* __restrict__ Ag = (const bf16_t*)P.A;
    const bf16_t* __restrict__ Bg = (const bf16_t*)P.B;

    // A-tile (and NT B-tile) load slots: 4 chunks of 16 B per thread.
    const bf16_t* arow[4];
    bool av[4];
    int aslot[4], akc[4];
    const bf16_t* brow[4];
    bool bv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int q = tid + 256 * c, r = q >> 3;
        aslot[c] = r;
        akc[c] = (q & 7) * 8;
        const int64_t m = m0 + r;
        av[c] = m < M;
        const int64_t ar = av[c] ? (P.a_rows ? (int64_t)P.a_rows[m] : m) : 0;
        arow[c] = Ag + ar * P.lda;
        if (!NN) {
            const int64_t n = n0 + r;
            bv[c] = n < N;
            const int64_t br = bv[c] ? (P.b_rows ? (int64_t)P.b_rows[n] : n) : 0;
            brow[c] = Bg + br * P.ldb;
        }
    }

    uint4 ra[4], rb[4];
    uint32_t rnn[2][8];

    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) ra[c] = load16_guard(arow[c], k0 + akc[c], K, av[c]);
        if (!NN) {
#pragma unroll
            for (int c = 0; c < 4; ++c) rb[c] = load16_guard(brow[c], k0 + akc[c], K, bv[c]);
        } else {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int q = tid + 256 * g, kq = q >> 6, np = q & 63;
                const int64_t n = n0 + 2 * np;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int64_t k = k0 + 8 * kq + e;
                    uint32_t v = 0u;
                    if (k < K && n < N) {
                        const int64_t br = P.b_rows ? (int64_t)P.b_rows[k] : k;
                        const bf16_t* p = Bg + br * P.ldb + n;
                        if (n + 1 < N) v = *(const uint32_t*)p;
                        else v = (uint32_t)p[0];
                    }
                    rnn[g][e] = v;
                }
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int c = 0; c < 4; ++c) *(uint4*)&As[buf][aslot[c] * LDK + akc[c]] = ra[c];
        if (!NN) {
#pragma unroll
            for (int c = 0; c < 4; ++c) *(uint4*)&Bs[buf][aslot[c] * LDK + akc[c]] = rb[c];
        } else {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int q = tid + 256 * g, kq = q >> 6, np = q & 63;
                uint4 lo, hi;  // column 2np (low halves) and 2np+1 (high halves)
                lo.x = (rnn[g][0] & 0xffffu) | (rnn[g][1] << 16);
                lo.y = (rnn[g][2] & 0xffffu) | (rnn[g][3] << 16);
                lo.z = (rnn[g][4] & 0xffffu) | (rnn[g][5] << 16);
                lo.w = (rnn[g][6] & 0xffffu) | (rnn[g][7] << 16);
                hi.x = (rnn[g][0] >> 16) | (rnn[g][1] & 0xffff0000u);
                hi.y = (rnn[g][2] >> 16) | (rnn[g][3] & 0xffff0000u);
                hi.z = (rnn[g][4] >> 16) | (rnn[g][5] & 0xffff0000u);
                hi.w = (rnn[g][6] >> 16) | (rnn[g][7] & 0xffff0000u);
                *(uint4*)&Bs[buf][(2 * np) * LDK + 8 * kq] = lo;
                *(uint4*)&Bs[buf][(2 * np + 1) * LDK + 8 * kq] = hi;
            }
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t nk = (K + BK - 1) / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) load_tile((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm * 64 + i * 32 + (lane & 31);
                a[i] = *(const bf16x8*)&As[cur][r * LDK + ks * 16 + (lane >> 5) * 8];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn * 64 + j * 32 + (lane & 31);
                b[j] = *(const bf16x8*)&Bs[cur][r * LDK + ks * 16 + (lane >> 5) * 8];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(e/4) + 4*(lane/32) + e%4
    bf16_t* __restrict__ Cg = (bf16_t*)P.C;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (n >= N) continue;
        const int64_t cn = P.c_cols ? (int64_t)P.c_cols[n] : n;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m >= M) continue;
                const int64_t cm = P.c_rows ? (int64_t)P.c_rows[m] : m;
                bf16_t* dst = Cg + cm * P.ldc + cn;
                float v = acc[i][j][e];
                if (P.beta) v += bf16_to_f32(*dst);
                *dst = f32_to_bf16(v);
            }
    }
}

// ---------------------------------------------------------------- fp32 (VALU)
constexpr int FB = 64, FK = 16;

template <bool NN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs args) {
    __shared__ float As[FK][FB + 1];
    __shared__ float Bs[FK][FB + 1];
    const int L = blockIdx.x;
    const bool second = L >= args.tiles0;
    const GemmProblem P = second ? args.p1 : args.p0;
    const int t = second ? L - args.tiles0 : L;
    const int tiles_m = second ? args.tiles_m1 : args.tiles_m0;
    const int64_t m0 = (int64_t)(t % tiles_m) * FB, n0 = (int64_t)(t / tiles_m) * FB;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const float* Ag = (const float*)P.A;
    const float* Bg = (const float*)P.B;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < P.K; k0 += FK) {
        for (int q = threadIdx.x; q < FK * FB; q += 256) {
            const int kk = q % FK, r = q / FK;
            const int64_t m = m0 + r, k = k0 + kk;
            float a = 0.0f;
            if (m < P.M && k < P.K) a = Ag[(P.a_rows ? (int64_t)P.a_rows[m] : m) * P.lda + k];
            As[kk][r] = a;
            const int64_t n = n0 + r;
            float b = 0.0f;
            if (n < P.N && k < P.K) {
                if (!NN) b = Bg[(P.b_rows ? (int64_t)P.b_rows[n] : n) * P.ldb + k];
                else b = Bg[(P.b_rows ? (int64_t)P.b_rows[k] : k) * P.ldb + n];
            }
            Bs[kk][r] = b;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < FK; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += As[kk][ty * 4 + i] * Bs[kk][tx * 4 + j];
        __syncthreads();
    }
    float* Cg = (float*)P.C;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= P.M) continue;
        const int64_t cm = P.c_rows ? (int64_t)P.c_rows[m] : m;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n >= P.N) continue;
            const int64_t cn = P.c_cols ? (int64_t)P.c_cols[n] : n;
            float* dst = Cg + cm * P.ldc + cn;
            *dst = acc[i][j] + (P.beta ? *dst : 0.0f);
        }
    }
}

GemmArgs make_args(const GemmProblem* probs, int nprob, int bm, int bn) {
    GemmArgs a;
    a.p0 = probs[0];
    a.p1 = nprob > 1 ? probs[1] : probs[0];
    const int tm0 = (int)ceil_div(a.p0.M, bm), tn0 = (int)ceil_div(a.p0.N, bn);
    a.tiles_m0 = tm0 > 0 ? tm0 : 1;
    a.tiles0 = (a.p0.M > 0 && a.p0.N > 0) ? tm0 * tn0 : 0;
    int tiles1 = 0;
    a.tiles_m1 = 1;
    if (nprob > 1 && a.p1.M > 0 && a.p1.N > 0) {
        const int tm1 = (int)ceil_div(a.p1.M, bm), tn1 = (int)ceil_div(a.p1.N, bn);
        a.tiles_m1 = tm1;
        tiles1 = tm1 * tn1;
    }
    a.total = a.tiles0 + tiles1;
    return a;
}

}  // namespace

hipError_t launch_gemm_bf16(bool nn, const GemmProblem* probs, int nprob, hipStream_t st) {
    GemmArgs a = make_args(probs, nprob, BM, BN);
    if (a.total == 0) return hipSuccess;
    if (nn) hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3(a.total), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3(a.total), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(bool nn, const GemmProblem* probs, int nprob, hipStream_t st) {
    GemmArgs a = make_args(probs, nprob, FB, FB);
    if (a.total == 0) return hipSuccess;
    if (nn) hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(a.total), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(a.total), dim3(256), 0, st, a);
    return hipGetLastError();
}
