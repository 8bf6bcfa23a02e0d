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
// bf16 path: v_mfma_f32_32x32x16_bf16.  Block tile BM x BN x 64 split over
// WGM x WGN waves; register-staged, double-buffered LDS with a 72-element row
// stride so the 16-byte MFMA operand reads are conflict-free.  NN tiles are
// transposed on their way into LDS (pairs of rows repacked) so both layouts
// feed the same K-contiguous LDS format.  Block ids are remapped so that each
// XCD works on a contiguous run of tiles (tiles sharing a weight tile stay in
// one XCD's L2), with the M tile index fastest.
//
// Optional rank-r term (the dense LoRA branch): before the single rounding of
// C, lscale * lP[cm, :] . lB[cn, :] is accumulated into the same fp32
// accumulators on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, with
// lscale * lP rounded to bf16 as a bf16 LoRA product rounds its
// down-projection), cm / cn being the mapped output row / channel.  A problem
// with K = 0 carries only this term (the unselected channels of context rows).
#include "sl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64, LDK = 72;
constexpr int MAXP = 5;
constexpr int NXCD = 8;

struct GemmArgs {
    GemmProblem p[MAXP];
    int first[MAXP + 1];   // first tile of each problem (prefix sums)
    int tiles_m[MAXP];
    int nprob;
    int grp;               // tile rows per group of the tile order
    // split tail: tiles [dp, total) each run as sks K-chunks whose fp32
    // partial tiles go to skws (in the accumulator layout); a second launch
    // sums them and runs the epilogue.  sks = 0: every tile whole.
    int dp;
    int sks;
    float* skws;
    // split-K sum run by blocks past the tail sums of the tail-sum launch
    // (nred of them; 0: none)
    SplitkRed red;
    int nred;
};

// Tile order inside a problem: groups of `grp` tile rows, M fastest inside a
// group, so the tiles that one XCD runs together (a contiguous run of ids)
// form a grp-row block of C whose A and B slices that XCD's L2 shares.
__device__ __forceinline__ void tile_origin(int t, int tiles_m, int64_t N, int BM, int BN, int grp,
                                            int64_t& m0, int64_t& n0) {
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int g = t / (grp * tiles_n), first_m = g * grp;
    const int gm = (tiles_m - first_m) < grp ? (tiles_m - first_m) : grp;
    const int tg = t - g * grp * tiles_n;
    m0 = (int64_t)(first_m + tg % gm) * BM;
    n0 = (int64_t)(tg / gm) * BN;
}

__device__ __forceinline__ void pick_problem(const GemmArgs& args, int L, GemmProblem& P, int& t,
                                             int& tiles_m) {
    // uniform selects (no dynamic indexing of the argument block)
    int i = 0;
#pragma unroll
    for (int q = 1; q < MAXP; ++q)
        if (q < args.nprob && L >= args.first[q]) i = q;
#pragma unroll
    for (int q = 0; q < MAXP; ++q)
        if (q == i) {
            P = args.p[q];
            t = L - args.first[q];
            tiles_m = args.tiles_m[q];
        }
}

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

// LDS-typed float pointer: keeps accesses on ds_read / ds_write (a generic
// pointer chosen at run time would become flat accesses)
typedef __attribute__((address_space(3))) float lds_f32;

// Block barrier for LDS hand-offs: waits for this wave's LDS operations only
// (lgkmcnt(0)), not for its outstanding global loads or stores.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
}

// Epilogue shared by the bf16 kernels: optional rank-r term into the fp32
// accumulators, then one rounding and the store through the row / column maps
// (or raw fp32 partials).  Lane holds column (lane & 31) and rows
// 8*(e/4) + 4*(lane/32) + e%4 of each 32 x 32 block.
template <int FM, int FN, int WTM, int WTN>
__device__ __forceinline__ void gemm_lora_term(const GemmProblem& P, f32x16 (&acc)[FM][FN],
                                              int64_t m0, int64_t n0, int wm, int wn, int lane) {
    const int64_t M = P.M, N = P.N;
    // rank-r term on the bf16 matrix cores: A operand lP[cm, k..k+7] (fp32,
    // rounded to bf16 as a bf16 LoRA product rounds its down-projection), B
    // operand lB[cn, k..k+7], k = kk + 8 (lane / 32); fp32 accumulation into the
    // same accumulators as the main product
    if (P.lr > 0) {
        const float* __restrict__ lP = P.lP;
        const bf16_t* __restrict__ lB = (const bf16_t*)P.lB;
        const int lr = P.lr;
        const bool pvec = (P.ldlP % 4 == 0) && (((uintptr_t)lP & 15) == 0);
        const bool bvec = (P.ldlB % 8 == 0) && (((uintptr_t)lB & 15) == 0);
        const float* prow[FM];
        const bf16_t* bcol[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t m = m0 + wm * WTM + i * 32 + (lane & 31);
            const int32_t* lmap = P.l_rows ? P.l_rows : P.c_rows;
            const int64_t cm = m < M ? (lmap ? (int64_t)lmap[m] : m) : -1;
            prow[i] = cm >= 0 ? lP + cm * P.ldlP : nullptr;
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + wn * WTN + j * 32 + (lane & 31);
            const int32_t* lmap = P.l_cols ? P.l_cols : P.c_cols;
            const int64_t cn = n < N ? (lmap ? (int64_t)lmap[n] : n) : -1;
            bcol[j] = cn >= 0 ? lB + cn * P.ldlB : nullptr;
        }
        for (int kk = 0; kk < lr; kk += 16) {
            const int k = kk + 8 * (lane >> 5);
            bf16x8 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                float v[8];
                if (prow[i] && pvec && k + 8 <= lr) {
                    const float4 v0 = *(const float4*)(prow[i] + k), v1 = *(const float4*)(prow[i] + k + 4);
                    v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
                    v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (prow[i] && k + e < lr) ? prow[i][k + e] : 0.0f;
                }
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = pack_bf16x2(P.lscale * v[2 * e], P.lscale * v[2 * e + 1]);
                a[i] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                uint4 u = make_uint4(0u, 0u, 0u, 0u);
                if (bcol[j] && bvec && k + 8 <= lr) {
                    u = *(const uint4*)(bcol[j] + k);
                } else if (bcol[j]) {
                    uint32_t w[4] = {0u, 0u, 0u, 0u};
                    for (int e = 0; e < 8; ++e)
                        if (k + e < lr) w[e >> 1] |= (uint32_t)bcol[j][k + e] << ((e & 1) * 16);
                    u = make_uint4(w[0], w[1], w[2], w[3]);
                }
                b[j] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
}

// Direct store of the accumulators (one element per lane and instruction),
// through the row / column maps, or raw fp32 partials.
template <int FM, int FN, int WTM, int WTN>
__device__ __forceinline__ void gemm_store_direct(const GemmProblem& P, f32x16 (&acc)[FM][FN],
                                                  int64_t m0, int64_t n0, int wm, int wn, int lane) {
    const int64_t M = P.M, N = P.N;
    // epilogue: lane holds column (lane & 31) and rows 8*(e/4) + 4*(lane/32) + e%4
    if (P.f32out) {   // split-K partial: raw fp32, unmapped
        float* __restrict__ Cf = (float*)P.C;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + wn * WTN + j * 32 + (lane & 31);
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t m = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    if (m < M) Cf[m * P.ldc + n] = acc[i][j][e];
                }
        }
        return;
    }
    bf16_t* __restrict__ Cg = (bf16_t*)P.C;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t n = n0 + wn * WTN + j * 32 + (lane & 31);
        if (n >= N) continue;
        const int64_t cn = P.c_cols ? (int64_t)P.c_cols[n] : n;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m >= M) continue;
                const int64_t cm = P.c_rows ? (int64_t)P.c_rows[m] : m;
                bf16_t* dst = Cg + cm * P.ldc + cn;
                float v = acc[i][j][e];
                if (P.beta) v += bf16_to_f32(*dst);
                *dst = f32_to_bf16(v);
            }
    }
}

template <int FM, int FN, int WTM, int WTN>
__device__ __forceinline__ void gemm_epilogue(const GemmProblem& P, f32x16 (&acc)[FM][FN],
                                              int64_t m0, int64_t n0, int wm, int wn, int lane) {
    gemm_lora_term<FM, FN, WTM, WTN>(P, acc, m0, n0, wm, wn, lane);
    gemm_store_direct<FM, FN, WTM, WTN>(P, acc, m0, n0, wm, wn, lane);
}

// Store through LDS (the staging buffers are free once the K loop is done): the
// tile goes out in FM passes of 32 WGM rows; each pass writes its rows to LDS
// as fp32 (lanes 0-31 of a wave: 32 consecutive columns, conflict free), then
// every thread takes runs of 8 consecutive columns of one row: one 16-byte
// bf16 store (or two for fp32 partials) per run, read-modify-write when
// accumulating.  With a column map each lane stores single elements, the lanes
// of a wave on consecutive columns of one row.
template <int FM, int FN, int WTM, int WTN, int WGM, int WGN>
__device__ __forceinline__ void gemm_store_lds(const GemmProblem& P, f32x16 (&acc)[FM][FN],
                                               int64_t m0, int64_t n0, int wm, int wn, int lane,
                                               int tid, lds_f32* const (&csr)[WGM]) {
    constexpr int NTH = 64 * WGM * WGN;
    constexpr int BN = WGN * WTN;
    constexpr int PR = 32 * WGM;                 // rows per pass
    constexpr int LDC = BN + 4;                  // fp32 row pitch in LDS
    constexpr int RUNS = PR * (BN / 8);          // 8-column runs per pass
    const int64_t M = P.M, N = P.N;
    const bool vec = P.c_cols == nullptr && (P.ldc % 8 == 0) && (((uintptr_t)P.C & 15) == 0);
    // mapped column of this thread's column (column-map path), -1 past N
    int64_t cn_tile = -1;
    if (P.c_cols && !P.f32out && n0 + tid % BN < N) cn_tile = P.c_cols[n0 + tid % BN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        lds_barrier();                          // LDS free (K loop done / previous pass read)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                csr[wm][(r - wm * 32) * LDC + wn * WTN + j * 32 + (lane & 31)] = acc[i][j][e];
            }
        lds_barrier();
        if (P.c_cols && !P.f32out) {
            // mapped columns: each thread keeps one column (its mapped channel is
            // read once per tile) and walks the pass's rows; the row of a wave is
            // uniform, so its map entry is one scalar load and each store
            // instruction covers 64 consecutive columns of one row
            constexpr int RSTEP = NTH / BN;
            static_assert(RSTEP >= 1 && NTH % BN == 0, "one column per thread");
            const int c = tid % BN;
            if (cn_tile < 0) continue;
            bf16_t* __restrict__ Ccol = (bf16_t*)P.C + cn_tile;
            for (int r = __builtin_amdgcn_readfirstlane(tid / BN); r < PR; r += RSTEP) {
                const int64_t m = m0 + (r / 32) * WTM + 32 * i + (r % 32);
                if (m >= M) continue;
                const int64_t cm = P.c_rows ? (int64_t)P.c_rows[m] : m;
                bf16_t* dst = Ccol + cm * P.ldc;
                float x = csr[r / 32][(r % 32) * LDC + c];
                if (P.beta) x += bf16_to_f32(*dst);
                *dst = f32_to_bf16(x);
            }
            continue;
        }
        for (int q = tid; q < RUNS; q += NTH) {
            const int r = q / (BN / 8), c8 = (q % (BN / 8)) * 8;
            const int64_t m = m0 + (r / 32) * WTM + 32 * i + (r % 32);
            const int64_t n = n0 + c8;
            if (m >= M || n >= N) continue;
            const lds_f32* src = csr[r / 32] + (r % 32) * LDC + c8;
            typedef float f32x4n __attribute__((ext_vector_type(4)));
            const f32x4n v0 = *(const __attribute__((address_space(3))) f32x4n*)src;
            const f32x4n v1 = *(const __attribute__((address_space(3))) f32x4n*)(src + 4);
            float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            const bool full = n + 8 <= N;
            if (P.f32out) {                       // split-K partial: raw fp32, unmapped
                float* dst = (float*)P.C + m * P.ldc + n;
                if (full && (P.ldc % 4 == 0) && (((uintptr_t)P.C & 15) == 0)) {
                    *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
                    *(float4*)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
                } else {
                    for (int q2 = 0; q2 < 8; ++q2)
                        if (n + q2 < N) dst[q2] = v[q2];
                }
                continue;
            }
            const int64_t cm = P.c_rows ? (int64_t)P.c_rows[m] : m;
            bf16_t* Cg = (bf16_t*)P.C + cm * P.ldc;
            if (vec && full) {
                bf16_t* dst = Cg + n;
                if (P.beta) {
                    const uint4 o = *(const uint4*)dst;
                    const uint32_t w[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
                    for (int q2 = 0; q2 < 4; ++q2) {
                        v[2 * q2] += bf16_to_f32((bf16_t)(w[q2] & 0xffffu));
                        v[2 * q2 + 1] += bf16_to_f32((bf16_t)(w[q2] >> 16));
                    }
                }
                uint32_t w[4];
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2)
                    w[q2] = pack_bf16x2(v[2 * q2], v[2 * q2 + 1]);
                *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
            } else {
                for (int q2 = 0; q2 < 8; ++q2) {
                    if (n + q2 >= N) break;
                    bf16_t* dst = Cg + n + q2;
                    float x = v[q2];
                    if (P.beta) x += bf16_to_f32(*dst);
                    *dst = f32_to_bf16(x);
                }
            }
        }
    }
}

template <int FM, int FN, int WTM, int WTN, int WGM, int WGN>
__device__ __forceinline__ void gemm_store_lds(const GemmProblem& P, f32x16 (&acc)[FM][FN],
                                               int64_t m0, int64_t n0, int wm, int wn, int lane,
                                               int tid, float* cs) {
    lds_f32* csr[WGM];
#pragma unroll
    for (int g = 0; g < WGM; ++g) csr[g] = (lds_f32*)cs + g * 32 * (WGN * WTN + 4);
    gemm_store_lds<FM, FN, WTM, WTN, WGM, WGN>(P, acc, m0, n0, wm, wn, lane, tid, csr);
}

template <int BM, int BN, int WGM, int WGN, bool NN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_kernel(GemmArgs args) {
    constexpr int NTH = 64 * WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;     // 32x32 MFMA blocks per wave
    constexpr int ACH = BM * 8 / NTH;               // 16-byte A chunks per thread
    constexpr int BCH = BN * 8 / NTH;               // 16-byte B chunks per thread (NT)
    constexpr int NNG = BN * 4 / NTH;               // (8 rows x 2 cols) groups per thread (NN)
    static_assert(ACH >= 1 && BCH >= 1 && NNG >= 1, "tile too small for the block");
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    bf16_t* As = smem;                       // [2][BM * LDK]
    bf16_t* Bs = smem + 2 * BM * LDK;        // [2][BN * LDK]

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    GemmProblem P;
    int t, tiles_m;
    pick_problem(args, L, P, t, tiles_m);
    const int64_t m0 = (int64_t)(t % tiles_m) * BM;
    const int64_t n0 = (int64_t)(t / tiles_m) * BN;
    const int64_t M = P.M, N = P.N, K = P.K;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WGM, wn = wid / WGM;
    const bf16_t* __restrict__ Ag = (const bf16_t*)P.A;
    const bf16_t* __restrict__ Bg = (const bf16_t*)P.B;

    const bf16_t* arow[ACH];
    bool av[ACH];
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int q = tid + NTH * c, r = q >> 3;
        const int64_t m = m0 + r;
        av[c] = m < M;
        const int64_t ar = av[c] ? (P.a_rows ? (int64_t)P.a_rows[m] : m) : 0;
        arow[c] = Ag + ar * P.lda;
    }
    const bf16_t* brow[NN ? 1 : BCH];
    bool bv[NN ? 1 : BCH];
    if (!NN) {
#pragma unroll
        for (int c = 0; c < (NN ? 1 : BCH); ++c) {
            const int q = tid + NTH * c, r = q >> 3;
            const int64_t n = n0 + r;
            bv[c] = n < N;
            const int64_t br = bv[c] ? (P.b_rows ? (int64_t)P.b_rows[n] : n) : 0;
            brow[c] = Bg + br * P.ldb;
        }
    }

    uint4 ra[ACH];
    uint4 rb[NN ? 1 : BCH];
    uint32_t rnn[NN ? NNG : 1][8];

    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int c = 0; c < ACH; ++c) ra[c] = load16_guard(arow[c], k0 + ((tid + NTH * c) & 7) * 8, K, av[c]);
        if (!NN) {
#pragma unroll
            for (int c = 0; c < (NN ? 1 : BCH); ++c)
                rb[c] = load16_guard(brow[c], k0 + ((tid + NTH * c) & 7) * 8, K, bv[c]);
        } else {
#pragma unroll
            for (int g = 0; g < (NN ? NNG : 1); ++g) {
                const int q = tid + NTH * g, np = q % (BN / 2), kq = q / (BN / 2);
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
        bf16_t* as = As + buf * BM * LDK;
        bf16_t* bs = Bs + buf * BN * LDK;
#pragma unroll
        for (int c = 0; c < ACH; ++c) {
            const int q = tid + NTH * c;
            *(uint4*)&as[(q >> 3) * LDK + (q & 7) * 8] = ra[c];
        }
        if (!NN) {
#pragma unroll
            for (int c = 0; c < (NN ? 1 : BCH); ++c) {
                const int q = tid + NTH * c;
                *(uint4*)&bs[(q >> 3) * LDK + (q & 7) * 8] = rb[c];
            }
        } else {
#pragma unroll
            for (int g = 0; g < (NN ? NNG : 1); ++g) {
                const int q = tid + NTH * g, np = q % (BN / 2), kq = q / (BN / 2);
                uint4 lo, hi;  // column 2np (low halves) and 2np+1 (high halves)
                lo.x = (rnn[g][0] & 0xffffu) | (rnn[g][1] << 16);
                lo.y = (rnn[g][2] & 0xffffu) | (rnn[g][3] << 16);
                lo.z = (rnn[g][4] & 0xffffu) | (rnn[g][5] << 16);
                lo.w = (rnn[g][6] & 0xffffu) | (rnn[g][7] << 16);
                hi.x = (rnn[g][0] >> 16) | (rnn[g][1] & 0xffff0000u);
                hi.y = (rnn[g][2] >> 16) | (rnn[g][3] & 0xffff0000u);
                hi.z = (rnn[g][4] >> 16) | (rnn[g][5] & 0xffff0000u);
                hi.w = (rnn[g][6] >> 16) | (rnn[g][7] & 0xffff0000u);
                *(uint4*)&bs[(2 * np) * LDK + 8 * kq] = lo;
                *(uint4*)&bs[(2 * np + 1) * LDK + 8 * kq] = hi;
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t nk = (K + BK - 1) / BK;
    if (nk > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
    }
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) load_tile((kt + 1) * BK);
        const bf16_t* as = As + cur * BM * LDK;
        const bf16_t* bs = Bs + cur * BN * LDK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WTM + i * 32 + (lane & 31);
                a[i] = *(const bf16x8*)&as[r * LDK + ks * 16 + (lane >> 5) * 8];
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * WTN + j * 32 + (lane & 31);
                b[j] = *(const bf16x8*)&bs[r * LDK + ks * 16 + (lane >> 5) * 8];
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    gemm_epilogue<FM, FN, WTM, WTN>(P, acc, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------- NT main loop v3
// NT only, K a multiple of 8 (operands zero-padded to it).  Loads are raw
// buffer loads: a 32-bit per-lane byte offset (row base + k sub-offset, fixed
// for the whole tile) plus the K-tile offset in a scalar register, so the loop
// spends no vector instructions on addresses; rows past M / N and chunks past
// K use an out-of-range offset and read zeros.  Two register sets keep the
// loads of tiles kt+1 and kt+2 in flight while tile kt is multiplied out of
// LDS; the block barrier is a bare s_barrier (this wave's LDS writes are
// waited for, its outstanding global loads are not).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB_OFF = 0x80000000u;   // >= num_records: the load returns zeros

__device__ __forceinline__ rsrc_t make_rsrc(const void* p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}


template <int BM, int BN, int WGM, int WGN, int NSET, bool PART = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_nt_kernel(GemmArgs args) {
    constexpr int NTH = 64 * WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int ACH = BM * 8 / NTH, BCH = BN * 8 / NTH;
    static_assert(ACH >= 1 && BCH >= 1 && (NTH % 8) == 0, "tile too small for the block");
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    bf16_t* As = smem;
    bf16_t* Bs = smem + 2 * BM * LDK;

    // PART: block u is K-chunk u % sks of tail tile dp + u / sks (the quotients
    // are formed on the vector unit; they are block-uniform); else whole tiles
    constexpr bool part = PART;
    const int u = part ? (int)blockIdx.x : 0;
    const int sk1 = args.sks > 1 ? args.sks : 1;
    const int L = part ? __builtin_amdgcn_readfirstlane(args.dp + u / sk1) : xcd_remap(blockIdx.x, gridDim.x);
    const int q = part ? __builtin_amdgcn_readfirstlane(u % sk1) : 0;
    GemmProblem P;
    int t, tiles_m;
    pick_problem(args, L, P, t, tiles_m);
    int64_t m0, n0;
    tile_origin(t, tiles_m, P.N, BM, BN, args.grp, m0, n0);
    const int64_t M = P.M, N = P.N, K = P.K;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WGM, wn = wid / WGM;
    const int kc8 = (tid & 7) * 8;          // every chunk of this thread has the same k sub-offset

    uint32_t aoff[ACH], boff[BCH];
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int64_t m = m0 + ((tid + NTH * c) >> 3);
        aoff[c] = m < M ? (uint32_t)(((P.a_rows ? (int64_t)P.a_rows[m] : m) * P.lda + kc8) * 2) : OOB_OFF;
    }
#pragma unroll
    for (int c = 0; c < BCH; ++c) {
        const int64_t n = n0 + ((tid + NTH * c) >> 3);
        boff[c] = n < N ? (uint32_t)(((P.b_rows ? (int64_t)P.b_rows[n] : n) * P.ldb + kc8) * 2) : OOB_OFF;
    }
    const rsrc_t ra = make_rsrc(P.A), rb = make_rsrc(P.B);
    // K steps [kb, kb + nk): the whole K, or chunk q of sks
    const int64_t nk_all = (K + BK - 1) / BK;
    int64_t kb = 0, nk = nk_all;
    if (part) {
        // (vector-unit quotient, block-uniform: keep it in scalars so the
        // buffer loads' offsets stay scalar)
        const int kc = __builtin_amdgcn_readfirstlane((int)((nk_all + args.sks - 1) / args.sks));
        kb = (int64_t)q * kc;
        nk = nk_all - kb < kc ? nk_all - kb : kc;
        if (nk < 0) nk = 0;
    }

    auto load = [&](uint4 (&sa)[ACH], uint4 (&sb)[BCH], int64_t kt0) {
        // the step index is block-uniform: keep the K offset a scalar operand
        const int kt = __builtin_amdgcn_readfirstlane((int)(kb + kt0));
        const uint32_t soff = (uint32_t)kt * (BK * 2);
        const bool kin = kt * BK + kc8 < K;   // whole 8-element chunk inside K (K % 8 == 0)
#pragma unroll
        for (int c = 0; c < ACH; ++c) sa[c] = bload16(ra, kin ? aoff[c] : OOB_OFF, soff);
#pragma unroll
        for (int c = 0; c < BCH; ++c) sb[c] = bload16(rb, kin ? boff[c] : OOB_OFF, soff);
    };
    auto store = [&](int buf, const uint4 (&sa)[ACH], const uint4 (&sb)[BCH]) {
        bf16_t* as = As + buf * BM * LDK;
        bf16_t* bs = Bs + buf * BN * LDK;
#pragma unroll
        for (int c = 0; c < ACH; ++c) *(uint4*)&as[((tid + NTH * c) >> 3) * LDK + kc8] = sa[c];
#pragma unroll
        for (int c = 0; c < BCH; ++c) *(uint4*)&bs[((tid + NTH * c) >> 3) * LDK + kc8] = sb[c];
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto compute = [&](int buf) {
        const bf16_t* as = As + buf * BM * LDK;
        const bf16_t* bs = Bs + buf * BN * LDK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *(const bf16x8*)&as[(wm * WTM + i * 32 + (lane & 31)) * LDK + ks * 16 + (lane >> 5) * 8];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                b[j] = *(const bf16x8*)&bs[(wn * WTN + j * 32 + (lane & 31)) * LDK + ks * 16 + (lane >> 5) * 8];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    if (NSET == 1 && nk > 0) {
        // one register set: tile kt+1 is in flight while tile kt is multiplied
        uint4 sa[ACH], sb[BCH];
        const int64_t last = nk - 1;
        load(sa, sb, 0);
        store(0, sa, sb);
        lds_barrier();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int buf = (int)(kt & 1);
            load(sa, sb, kt + 1 <= last ? kt + 1 : last);
            compute(buf);
            if (kt + 1 <= last) store(buf ^ 1, sa, sb);
            lds_barrier();
        }
    } else if (NSET == 2 && nk > 0) {
        uint4 sa0[ACH], sb0[BCH], sa1[ACH], sb1[BCH];
        const int64_t last = nk - 1;
        load(sa0, sb0, 0);
        load(sa1, sb1, nk > 1 ? 1 : last);
        store(0, sa0, sb0);
        lds_barrier();
        for (int64_t kt = 0; kt < nk; kt += 2) {
            // even step: tile kt in LDS 0; tile kt+1 in set 1; fetch tile kt+2 into set 0
            load(sa0, sb0, kt + 2 <= last ? kt + 2 : last);
            compute(0);
            if (kt + 1 <= last) store(1, sa1, sb1);
            lds_barrier();
            if (kt + 1 > last) break;
            // odd step: tile kt+1 in LDS 1; tile kt+2 in set 0; fetch tile kt+3 into set 1
            load(sa1, sb1, kt + 3 <= last ? kt + 3 : last);
            compute(1);
            if (kt + 2 <= last) store(0, sa0, sb0);
            lds_barrier();
        }
    }
    if (part) {
        // raw fp32 partial in the accumulator layout: 16-byte runs
        // acc[i][j][4g .. 4g+3] of each lane, a 1 KB row of lanes per store
        // (buffer stores: one lane offset, the run offset in a scalar)
        const int wid_s = __builtin_amdgcn_readfirstlane(wid);   // (a scalar resource base)
        const rsrc_t rw = make_rsrc(args.skws + (size_t)u * BM * BN + (size_t)wid_s * FM * FN * 16 * 64);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint4 d = make_uint4(__float_as_uint(acc[i][j][4 * g]), __float_as_uint(acc[i][j][4 * g + 1]),
                                               __float_as_uint(acc[i][j][4 * g + 2]), __float_as_uint(acc[i][j][4 * g + 3]));
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, d),
                                                           rw, lane * 16, ((i * FN + j) * 4 + g) * 1024, 0);
                }
        return;
    }
    gemm_lora_term<FM, FN, WTM, WTN>(P, acc, m0, n0, wm, wn, lane);
    gemm_store_lds<FM, FN, WTM, WTN, WGM, WGN>(P, acc, m0, n0, wm, wn, lane, tid, (float*)smem);
}

// Split tail, second launch: tile dp + blockIdx.x sums its sks partials in
// chunk order (deterministic), then runs the same epilogue as a whole tile.
// Blocks past the tail sums: Z[rows[m], n..n+7] = round(sum over s ascending
// of part[s][m][n..n+7] (+ Z if beta)), each element formed exactly as
// splitk_reduce_kernel forms it; 8 columns per thread, grid-strided.
__device__ __forceinline__ void splitk_red_block(const SplitkRed& R, int b, int nb, int tid, int nth) {
    const int64_t n8 = R.N / 8, items = R.M * n8;
    for (int64_t i = (int64_t)b * nth + tid; i < items; i += (int64_t)nb * nth) {
        const int64_t m = i / n8, q = (i - m * n8) * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        for (int64_t s = 0; s < R.S; ++s) {
            const float* p = R.part + (s * R.M + m) * R.N + q;
            const float4 a = *(const float4*)p, c = *(const float4*)(p + 4);
            v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
            v[4] += c.x; v[5] += c.y; v[6] += c.z; v[7] += c.w;
        }
        bf16_t* d = (bf16_t*)R.Z + (R.rows ? (int64_t)R.rows[m] : m) * R.ldz + q;
        if (R.beta) {
            const uint4 o = *(const uint4*)d;
            const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += bf16_to_f32((bf16_t)((ow[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
        }
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)f32_to_bf16(v[2 * e]) | ((uint32_t)f32_to_bf16(v[2 * e + 1]) << 16);
        *(uint4*)d = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_nt_fixup_kernel(GemmArgs args) {
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
    const int ntail = args.first[MAXP] - args.dp;
    if ((int)blockIdx.x >= ntail) {   // (block-uniform)
        splitk_red_block(args.red, (int)blockIdx.x - ntail, args.nred, (int)threadIdx.x, 64 * WGM * WGN);
        return;
    }
    const int L = args.dp + (int)blockIdx.x;
    GemmProblem P;
    int t, tiles_m;
    pick_problem(args, L, P, t, tiles_m);
    int64_t m0, n0;
    tile_origin(t, tiles_m, P.N, BM, BN, args.grp, m0, n0);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WGM, wn = wid / WGM;
    f32x16 acc[FM][FN];
    const float* __restrict__ w0 = args.skws + (size_t)blockIdx.x * args.sks * BM * BN +
                                   (size_t)wid * FM * FN * 16 * 64 + lane * 4;
    // one partial at a time, all of its loads in flight together; each element
    // is still summed in chunk order
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 v = *(const float4*)(w0 + ((i * FN + j) * 4 + g) * 256);
                acc[i][j][4 * g] = v.x;
                acc[i][j][4 * g + 1] = v.y;
                acc[i][j][4 * g + 2] = v.z;
                acc[i][j][4 * g + 3] = v.w;
            }
    for (int c = 1; c < args.sks; ++c) {
        const float* __restrict__ wc = w0 + (size_t)c * BM * BN;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 x = *(const float4*)(wc + ((i * FN + j) * 4 + g) * 256);
                    acc[i][j][4 * g] += x.x;
                    acc[i][j][4 * g + 1] += x.y;
                    acc[i][j][4 * g + 2] += x.z;
                    acc[i][j][4 * g + 3] += x.w;
                }
    }
    gemm_lora_term<FM, FN, WTM, WTN>(P, acc, m0, n0, wm, wn, lane);
    gemm_store_lds<FM, FN, WTM, WTN, WGM, WGN>(P, acc, m0, n0, wm, wn, lane, tid, (float*)smem);
}

// ---------------------------------------------------------------- NT main loop v5 (LDS DMA)
// 256 x 256 tile; K in stages of BKS (32 or 64) held in NST LDS stages (4 or 2)
// that buffer loads fill directly (buffer_load_dwordx4 ... lds): no register
// staging and no LDS store instructions.  A stage is 512 rows (A rows 0-255,
// B rows 256-511) of BKS bf16, i.e. CPR 16-byte chunks per row.  One load
// instruction of a wave fills a 1 KB slab with lane i at byte 16 i, so lane i
// fetches row i / CPR of the slab and the k-chunk that the row swizzle puts at
// position i % CPR: chunk c of row R sits at position c ^ ((R / (16 / CPR)) % CPR),
// so that 16 consecutive rows (the lanes one LDS cycle of a 16-byte fragment
// read serves) hit 16 different 16-byte bank groups of the 256-byte bank row.  The stages are separate LDS arrays and the K loop is
// unrolled by NST so that every read names its stage.  Step t issues the loads
// of tile t + NST - 1 into the stage of tile t - 1, multiplies tile t, waits
// for this wave's loads of tile t + 1 and ends with the one barrier of the step
// (it publishes tile t + 1 and retires the reads of tile t).
__host__ __device__ constexpr uint16_t vmcnt_imm(int n) {
    // s_waitcnt immediate: vmcnt(n) only (expcnt, lgkmcnt at their maxima)
    return (uint16_t)((n & 15) | 0x70 | 0xF00 | ((n >> 4) << 14));
}

template <int BKS, int NW, int DPT>
__device__ __forceinline__ void nt5_dma(rsrc_t ra, rsrc_t rb, bf16_t* st, int64_t kt, int64_t K, int ck,
                                        int wid, const uint32_t* goff) {
    const uint32_t soff = (uint32_t)(kt * BKS * 2);
    const bool kin = kt * BKS + ck * 8 < K;
#pragma unroll
    for (int d = 0; d < DPT / 2; ++d)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(st + (wid + NW * d) * 512),
                                                 16, kin ? goff[d] : OOB_OFF, soff, 0, 0);
#pragma unroll
    for (int d = DPT / 2; d < DPT; ++d)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(st + (wid + NW * d) * 512),
                                                 16, kin ? goff[d] : OOB_OFF, soff, 0, 0);
}

// Scheduling hints for one step (mask 0x008 MFMA, 0x100 LDS read, 0x020 global
// read): before the step barrier, the fragment reads of the next K sub-step
// and the stage loads are spread between the MFMAs of the current one; after
// it, the reads of the next tile's first sub-step between the last MFMAs.
template <int NRD, int NMF, int NSUB, int NLD>
__device__ __forceinline__ void nt5_sched_pre() {
#pragma unroll
    for (int q = 0; q < NSUB; ++q) {
#pragma unroll
        for (int i = 0; i < NRD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < NMF - NRD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < (NLD + NSUB - 1) / NSUB) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    }
}
template <int NRD, int NMF>
__device__ __forceinline__ void nt5_sched_post() {
    constexpr int PER = NMF / NRD;
#pragma unroll
    for (int i = 0; i < NRD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
    }
}

template <int WGM, int WGN, int BKS, int NST, bool PART = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_nt5_kernel(GemmArgs args) {
    constexpr int BM = 256, BN = 256;
    constexpr int NW = WGM * WGN;
    constexpr int WTM = BM / WGM, WTN = BN / WGN, FM = WTM / 32, FN = WTN / 32;
    constexpr int CPR = BKS / 8;                 // 16-byte chunks per row
    constexpr int SLABS = 512 * BKS * 2 / 1024;  // 1 KB slabs per stage
    constexpr int DPT = SLABS / NW;              // load instructions per wave per stage
    static_assert(DPT * NW == SLABS && DPT % 2 == 0, "A slabs first half, B slabs second half");
    static_assert(NST == 2 || NST == 4, "two or four stages");
    static_assert(WGM == 2, "store epilogue: one stage array per row group");
    // a stage array also holds 32 rows x (BN + 4) fp32 of the store epilogue
    constexpr int SZ = (512 * BKS > 32 * (BN + 4) * 2) ? 512 * BKS : 32 * (BN + 4) * 2;
    __shared__ __attribute__((aligned(16))) bf16_t s0[SZ];
    __shared__ __attribute__((aligned(16))) bf16_t s1[SZ];
    __shared__ __attribute__((aligned(16))) bf16_t s2[NST == 4 ? SZ : 8];
    __shared__ __attribute__((aligned(16))) bf16_t s3[NST == 4 ? SZ : 8];

    // PART: block u is K-chunk u % sks of tail tile dp + u / sks (split tail,
    // as in the v3 kernel); else whole tiles
    const int u = PART ? (int)blockIdx.x : 0;
    const int sk1 = args.sks > 1 ? args.sks : 1;
    const int L = PART ? __builtin_amdgcn_readfirstlane(args.dp + u / sk1) : xcd_remap(blockIdx.x, gridDim.x);
    const int qch = PART ? __builtin_amdgcn_readfirstlane(u % sk1) : 0;
    GemmProblem P;
    int t, tiles_m;
    pick_problem(args, L, P, t, tiles_m);
    int64_t m0, n0;
    tile_origin(t, tiles_m, P.N, BM, BN, args.grp, m0, n0);
    const int64_t M = P.M, N = P.N, K = P.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % WGM, wn = wid / WGM;

    // loads: slab q = wid + NW d holds rows (1024 / (2 BKS)) q ..; lane i: row i / CPR of it
    constexpr int SR = 1024 / (2 * BKS);         // rows per slab
    // k-chunk this lane fetches: (stage row / (16 / CPR)) mod CPR does not depend
    // on the slab's d (the slabs of one wave are NW apart, 16 NW / (16 / CPR) rows)
    const int ck = (lane % CPR) ^ (((SR * wid + lane / CPR) / (16 / CPR)) % CPR);
    uint32_t goff[DPT];
#pragma unroll
    for (int d = 0; d < DPT; ++d) {
        const int q = wid + NW * d;
        const int64_t rr = SR * q + lane / CPR;            // stage row
        if (d < DPT / 2) {
            const int64_t m = m0 + rr;
            goff[d] = m < M ? (uint32_t)(((P.a_rows ? (int64_t)P.a_rows[m] : m) * P.lda + ck * 8) * 2) : OOB_OFF;
        } else {
            const int64_t n = n0 + rr - 256;
            goff[d] = n < N ? (uint32_t)(((P.b_rows ? (int64_t)P.b_rows[n] : n) * P.ldb + ck * 8) * 2) : OOB_OFF;
        }
    }
    const rsrc_t ra = make_rsrc(P.A), rb = make_rsrc(P.B);
    // K steps of this block: [kb, kb + nk), nk a whole number of stage rotations
    // (steps past K load zeros); a PART chunk covers kc steps of the tile
    const int nk_all = (int)((K + BKS - 1) / BKS);
    int kb = 0, nk = (nk_all + NST - 1) / NST * NST;
    if (PART) {
        const int kc = ((nk_all + sk1 - 1) / sk1 + NST - 1) / NST * NST;
        kb = qch * kc;
        const int rest = nk_all - kb;
        nk = rest <= 0 ? 0 : (rest < kc ? (rest + NST - 1) / NST * NST : kc);
    }
    const int64_t kb64 = kb;
    auto dma = [&](bf16_t* st, int kt) { nt5_dma<BKS, NW, DPT>(ra, rb, st, kb64 + kt, K, ck, wid, goff); };

    // fragment reads: row R = base + lane % 32 (base a multiple of 32), chunk 2 ks + lane / 32
    const int swz = ((lane & 31) / (16 / CPR)) % CPR;
    const int arow = (wm * WTM + (lane & 31)) * BKS;
    const int brow = (256 + wn * WTN + (lane & 31)) * BKS;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // two fragment sets: the reads of sub-step ks + 1 overlap the MFMAs of ks,
    // and the reads of the next tile's sub-step 0 (after the step barrier) the
    // MFMAs of the last sub-step
    constexpr int KS = BKS / 16;
    bf16x8 fa[2][FM], fb[2][FN];
    auto rd = [&](const bf16_t* st, int ks, int set) {
        const int ko = ((2 * ks + (lane >> 5)) ^ swz) * 8;
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[set][i] = *(const bf16x8*)&st[arow + i * 32 * BKS + ko];
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[set][j] = *(const bf16x8*)&st[brow + j * 32 * BKS + ko];
    };
    auto mm = [&](int set) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
    };

    constexpr int INFL = (NST - 2) * DPT;         // this wave's loads allowed in flight at a step's end
    dma(s0, 0);
    if (NST == 4) {
        dma(s1, 1);
        dma(s2, 2);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFL));
    __builtin_amdgcn_s_barrier();
    rd(s0, 0, 0);
#define NT5_STEP(CUR, NXTL, NXTC, T)                                          \
    dma(NXTL, (T) + NST - 1);                                                 \
    for (int ks = 0; ks < KS - 1; ++ks) {                                     \
        rd(CUR, ks + 1, (ks + 1) & 1);                                        \
        mm(ks & 1);                                                           \
    }                                                                         \
    nt5_sched_pre<FM + FN, FM * FN, KS - 1, DPT>();                           \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(INFL));                              \
    __builtin_amdgcn_s_barrier();                                             \
    rd(NXTC, 0, KS & 1);                                                      \
    mm((KS - 1) & 1);                                                         \
    nt5_sched_post<FM + FN, FM * FN>();
    if (NST == 4) {
        for (int kt = 0; kt < nk; kt += 4) {
            NT5_STEP(s0, s3, s1, kt)
            NT5_STEP(s1, s0, s2, kt + 1)
            NT5_STEP(s2, s1, s3, kt + 2)
            NT5_STEP(s3, s2, s0, kt + 3)
        }
    } else {
        for (int kt = 0; kt < nk; kt += 2) {
            NT5_STEP(s0, s1, s1, kt)
            NT5_STEP(s1, s0, s0, kt + 1)
        }
    }
#undef NT5_STEP
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));     // the stages are reused below
    if (PART) {
        // raw fp32 partial in the accumulator layout (as the v3 kernel's tail chunks)
        const rsrc_t rw = make_rsrc(args.skws + (size_t)u * BM * BN + (size_t)wid * FM * FN * 16 * 64);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint4 d = make_uint4(__float_as_uint(acc[i][j][4 * g]), __float_as_uint(acc[i][j][4 * g + 1]),
                                               __float_as_uint(acc[i][j][4 * g + 2]), __float_as_uint(acc[i][j][4 * g + 3]));
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, d),
                                                           rw, lane * 16, ((i * FN + j) * 4 + g) * 1024, 0);
                }
        return;
    }
    gemm_lora_term<FM, FN, WTM, WTN>(P, acc, m0, n0, wm, wn, lane);
    lds_f32* csr[2];
    csr[0] = (lds_f32*)s0;
    csr[1] = (lds_f32*)s1;
    gemm_store_lds<FM, FN, WTM, WTN, WGM, WGN>(P, acc, m0, n0, wm, wn, lane, tid, csr);
}

// ---------------------------------------------------------------- fp32 (VALU)
constexpr int FB = 64, FK = 16;

// Epilogue of the fp32 kernels for element (m, n) of problem P with product
// value v: the rank-r term, then the store through the row / column maps (or
// the raw value of a split-K partial problem).
__device__ __forceinline__ void f32_store(const GemmProblem& P, int64_t m, int64_t n, float v) {
    float* Cg = (float*)P.C;
    const int64_t cm = P.c_rows ? (int64_t)P.c_rows[m] : m;
    const int64_t cn = P.c_cols ? (int64_t)P.c_cols[n] : n;
    if (P.lr > 0) {
        const int64_t lm = P.l_rows ? (int64_t)P.l_rows[m] : cm;
        const float* lP = P.lP + lm * P.ldlP;
        const float* lB = (const float*)P.lB + cn * P.ldlB;
        float l = 0.0f;
        for (int k = 0; k < P.lr; ++k) l += lP[k] * lB[k];
        v += P.lscale * l;
    }
    if (P.f32out) {
        Cg[m * P.ldc + n] = v;
        return;
    }
    float* dst = Cg + cm * P.ldc + cn;
    *dst = v + (P.beta ? *dst : 0.0f);
}

// fp32 products on the vector unit: a 64 x 64 output tile per block of 256
// threads (4 x 4 per thread), K in steps of 16 staged through LDS; the next
// step's operands are loaded into registers while the current one is
// multiplied, and the operand rows of the tile are looked up once.  A launch
// with few tiles against the compute units splits K: with args.sks = S > 1,
// block b runs K-chunk b mod S of tile b / S and stores its fp32 partial tile
// to args.skws; gemm_f32_sum_kernel then adds the S chunks of each element in
// chunk order and runs the epilogue (deterministic).
template <bool NN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs args) {
    __shared__ float As[FK][FB + 1];
    __shared__ float Bs[FK][FB + 1];
    const int S = args.sks > 1 ? args.sks : 1;
    const int L = (int)blockIdx.x / S, q = (int)blockIdx.x % S;
    GemmProblem P;
    int t, tiles_m;
    pick_problem(args, L, P, t, tiles_m);
    const int64_t m0 = (int64_t)(t % tiles_m) * FB, n0 = (int64_t)(t / tiles_m) * FB;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const float* Ag = (const float*)P.A;
    const float* Bg = (const float*)P.B;
    // load slots: element (kk, r) with kk = tid % 16 (the same for all four
    // slots of a thread) and r = tid / 16 + 16 c
    const int kk = tid & 15;
    int64_t aoff[4], boff[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t m = m0 + ty + 16 * c, n = n0 + ty + 16 * c;
        aoff[c] = m < P.M ? (P.a_rows ? (int64_t)P.a_rows[m] : m) * P.lda : -1;
        if (!NN) boff[c] = n < P.N ? (P.b_rows ? (int64_t)P.b_rows[n] : n) * P.ldb : -1;
        else boff[c] = n < P.N ? n : -1;
    }
    // K steps of this block
    const int64_t nk_all = (P.K + FK - 1) / FK;
    const int64_t kc = (nk_all + S - 1) / S;
    const int64_t kb = (int64_t)q * kc;
    const int64_t ke = nk_all < kb + kc ? nk_all : kb + kc;
    float ra[4], rb[4];
    auto load = [&](int64_t ks) {
        const int64_t k = ks * FK + kk;
        const bool kin = k < P.K;
        int64_t bk = 0;
        if (NN && kin) bk = (P.b_rows ? (int64_t)P.b_rows[k] : k) * P.ldb;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ra[c] = (kin && aoff[c] >= 0) ? Ag[aoff[c] + k] : 0.0f;
            if (!NN) rb[c] = (kin && boff[c] >= 0) ? Bg[boff[c] + k] : 0.0f;
            else rb[c] = (kin && boff[c] >= 0) ? Bg[bk + boff[c]] : 0.0f;
        }
    };
    float acc[4][4] = {};
    if (kb < ke) load(kb);
    for (int64_t ks = kb; ks < ke; ++ks) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            As[kk][ty + 16 * c] = ra[c];
            Bs[kk][ty + 16 * c] = rb[c];
        }
        __syncthreads();
        if (ks + 1 < ke) load(ks + 1);
#pragma unroll
        for (int k2 = 0; k2 < FK; ++k2)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += As[k2][ty * 4 + i] * Bs[k2][tx * 4 + j];
        __syncthreads();
    }
    if (S > 1) {
        float* w = args.skws + (size_t)blockIdx.x * FB * FB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(float4*)&w[(ty * 4 + i) * FB + tx * 4] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= P.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n < P.N) f32_store(P, m, n, acc[i][j]);
        }
    }
}

// Split-K sum of the fp32 kernel: 16 blocks per tile (block 16 L + g takes
// elements 256 g .. 256 g + 255 of tile L, one per thread); a thread loads its
// S (<= 16) partials together, adds them in chunk order, then the epilogue.
__global__ __launch_bounds__(256) void gemm_f32_sum_kernel(GemmArgs args) {
    const int S = args.sks;
    const int L = (int)blockIdx.x / 16;
    const int e = ((int)blockIdx.x % 16) * 256 + (int)threadIdx.x;
    GemmProblem P;
    int t, tiles_m;
    pick_problem(args, L, P, t, tiles_m);
    const int64_t m0 = (int64_t)(t % tiles_m) * FB, n0 = (int64_t)(t / tiles_m) * FB;
    const int64_t m = m0 + e / FB, n = n0 + e % FB;
    if (m >= P.M || n >= P.N) return;
    const float* w = args.skws + (size_t)L * S * FB * FB + e;
    float p[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) p[c] = c < S ? w[(size_t)c * FB * FB] : 0.0f;
    float v = p[0];
#pragma unroll
    for (int c = 1; c < 16; ++c)
        if (c < S) v += p[c];
    f32_store(P, m, n, v);
}

GemmArgs make_args(const GemmProblem* probs, int nprob, int bm, int bn, int grp = 8) {
    GemmArgs a = {};
    a.nprob = nprob;
    a.grp = grp > 0 ? grp : 8;     // tile rows per group of the tile order
    a.first[0] = 0;
    for (int i = 0; i < MAXP; ++i) {
        if (i < nprob) {
            a.p[i] = probs[i];
            const int tm = (int)ceil_div(probs[i].M, bm), tn = (int)ceil_div(probs[i].N, bn);
            a.tiles_m[i] = tm > 0 ? tm : 1;
            a.first[i + 1] = a.first[i] + ((probs[i].M > 0 && probs[i].N > 0) ? tm * tn : 0);
        } else {
            a.p[i] = probs[0];
            a.tiles_m[i] = 1;
            a.first[i + 1] = a.first[i];
        }
    }
    a.dp = a.first[MAXP];   // every tile whole unless a launcher plans a split tail
    a.sks = 0;
    a.skws = nullptr;
    return a;
}

template <int BM, int BN, int WGM, int WGN, bool NN>
hipError_t launch_cfg(const GemmProblem* probs, int nprob, hipStream_t st) {
    GemmArgs a = make_args(probs, nprob, BM, BN);
    const int total = a.first[MAXP];
    if (total == 0) return hipSuccess;
    bool any_k = false;
    for (int i = 0; i < nprob; ++i) any_k |= probs[i].K > 0;
    // rank-r-only launches (K = 0 everywhere) never touch the staging LDS
    const size_t lds = any_k ? (size_t)2 * (BM + BN) * LDK * sizeof(bf16_t) : 0;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)gemm_bf16_kernel<BM, BN, WGM, WGN, NN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, NN>), dim3(total), dim3(64 * WGM * WGN),
                       lds, st, a);
    return hipGetLastError();
}

template <typename T>
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int64_t S, int64_t M,
                                     int64_t N, T* __restrict__ Z, int64_t ldz,
                                     const int32_t* __restrict__ c_rows,
                                     const int32_t* __restrict__ c_cols, int beta) {
    const int64_t m = blockIdx.y;
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float v = 0.0f;
    for (int64_t s = 0; s < S; ++s) v += part[(s * M + m) * N + n];
    const int64_t cm = c_rows ? (int64_t)c_rows[m] : m;
    const int64_t cn = c_cols ? (int64_t)c_cols[n] : n;
    T* dst = Z + cm * ldz + cn;
    if (sizeof(T) == 2) {
        bf16_t* d = (bf16_t*)dst;
        if (beta) v += bf16_to_f32(*d);
        *d = f32_to_bf16(v);
    } else {
        float* d = (float*)dst;
        if (beta) v += *d;
        *d = v;
    }
}

}  // namespace

namespace {

// Split-tail plan for a launch of `total` 256 x 256 tiles on ncu compute
// units: the last (total mod ncu) tiles would run as a partial round; split
// each into s K-chunks (s = ncu / rem, at most 8, each chunk at least 4 K
// steps) so that the chunks fill one round.  Returns s (0: no split) and the
// number of whole tiles.
int split_tail_plan(const GemmArgs& a, int ncu, int& dp) {
    const int total = a.first[MAXP];
    dp = total;
    if (ncu <= 0 || total <= 0) return 0;
    const int rem = total % ncu;
    if (rem == 0) return 0;
    int sks = ncu / rem;
    if (sks > 8) sks = 8;
    // every tail tile must have K steps for sks chunks of >= 4 steps
    for (int i = 0; i < a.nprob; ++i) {
        if (a.first[i + 1] <= total - rem) continue;      // no tail tile in problem i
        const int64_t nk = (a.p[i].K + BK - 1) / BK;
        while (sks >= 2 && nk < 4 * sks) --sks;
    }
    if (sks < 2) return 0;
    dp = total - rem;
    return sks;
}

template <int BM, int BN, int WGM, int WGN, int NSET>
hipError_t launch_nt_cfg(const GemmProblem* probs, int nprob, hipStream_t st, float* skws,
                         size_t skws_floats, int ncu, int grp, const SplitkRed* red = nullptr,
                         bool* red_done = nullptr) {
    GemmArgs a = make_args(probs, nprob, BM, BN, grp);
    const int total = a.first[MAXP];
    if (total == 0) return hipSuccess;
    // staging buffers; the store epilogue reuses them (always needed)
    const size_t lds = (size_t)2 * (BM + BN) * LDK * sizeof(bf16_t);
    static bool attr_set = false;
    if (!attr_set) {
        const void* fns[3] = {(const void*)gemm_nt_kernel<BM, BN, WGM, WGN, NSET, false>,
                              (const void*)gemm_nt_kernel<BM, BN, WGM, WGN, NSET, true>,
                              (const void*)gemm_nt_fixup_kernel<BM, BN, WGM, WGN>};
        for (const void* f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        attr_set = true;
    }
    int dp = total;
    int sks = (BM == 256 && BN == 256 && skws) ? split_tail_plan(a, ncu, dp) : 0;
    if (sks && (size_t)(total - dp) * sks * BM * BN > skws_floats) sks = 0, dp = total;
    a.dp = dp;
    a.sks = sks;
    a.skws = skws;
    // a split-K sum given by the caller rides in the tail-sum launch (its
    // tail tiles leave compute units idle), when its layout allows
    int nred = 0;
    // (not when a tail tile belongs to a partial-output problem: its sum
    // would write the partials the split-K sum reads)
    bool tail_f32 = false;
    for (int i = 0; i < a.nprob; ++i)
        if (a.first[i + 1] > dp && a.p[i].f32out) tail_f32 = true;
    if (sks && red && !tail_f32 && red->S > 0 && red->M > 0 && red->N > 0 && red->N % 8 == 0 &&
        red->ldz % 8 == 0 && ((uintptr_t)red->Z & 15) == 0 && ((uintptr_t)red->part & 15) == 0) {
        const int64_t items = red->M * (red->N / 8);
        const int64_t want = ceil_div(items, (int64_t)(64 * WGM * WGN));
        int64_t nb = ncu - (total - dp);
        if (nb < 32) nb = 32;
        nred = (int)(nb < want ? nb : want);
        a.red = *red;
    }
    a.nred = nred;
    if (red_done) *red_done = nred > 0;
    // whole tiles (complete rounds), then the tail's K-chunks, then their sums
    if (dp > 0)
        hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WGM, WGN, NSET, false>), dim3(dp), dim3(64 * WGM * WGN), lds,
                           st, a);
    if (sks) {
        hipLaunchKernelGGL((gemm_nt_kernel<BM, BN, WGM, WGN, NSET, true>), dim3((total - dp) * sks),
                           dim3(64 * WGM * WGN), lds, st, a);
        hipLaunchKernelGGL((gemm_nt_fixup_kernel<BM, BN, WGM, WGN>), dim3(total - dp + nred), dim3(64 * WGM * WGN),
                           lds, st, a);
    }
    return hipGetLastError();
}

template <int WGM, int WGN, int BKS, int NST>
hipError_t launch_nt5(const GemmProblem* probs, int nprob, hipStream_t st, int grp, float* skws = nullptr,
                      size_t skws_floats = 0, int ncu = 256) {
    GemmArgs a = make_args(probs, nprob, 256, 256, grp);
    const int total = a.first[MAXP];
    if (total == 0) return hipSuccess;
    // fixup launch: its store epilogue uses WGM row groups of 32 x (BN + 4) fp32
    const size_t fix_lds = (size_t)WGM * 32 * (256 + 4) * sizeof(float);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)gemm_nt_fixup_kernel<256, 256, WGM, WGN>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)fix_lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    int dp = total;
    int sks = skws ? split_tail_plan(a, ncu, dp) : 0;
    if (sks && (size_t)(total - dp) * sks * 256 * 256 > skws_floats) sks = 0, dp = total;
    a.dp = dp;
    a.sks = sks;
    a.skws = skws;
    if (dp > 0)
        hipLaunchKernelGGL((gemm_nt5_kernel<WGM, WGN, BKS, NST, false>), dim3(dp), dim3(64 * WGM * WGN), 0, st, a);
    if (sks) {
        hipLaunchKernelGGL((gemm_nt5_kernel<WGM, WGN, BKS, NST, true>), dim3((total - dp) * sks),
                           dim3(64 * WGM * WGN), 0, st, a);
        hipLaunchKernelGGL((gemm_nt_fixup_kernel<256, 256, WGM, WGN>), dim3(total - dp), dim3(64 * WGM * WGN),
                           fix_lds, st, a);
    }
    return hipGetLastError();
}


// The v3 loop needs K % 8 == 0 (zero-padded operands) and byte offsets that
// stay below 2^31 (row index * ld + K, in bytes).
bool nt_v3_ok(const GemmProblem* probs, int nprob) {
    for (int i = 0; i < nprob; ++i) {
        const GemmProblem& p = probs[i];
        if (p.M <= 0 || p.N <= 0 || p.K <= 0) continue;
        if (p.K % 8 != 0 || p.lda % 8 != 0 || p.ldb % 8 != 0) return false;
        if (p.a_nrows <= 0 || p.b_nrows <= 0) return false;
        if ((p.a_nrows * p.lda + p.K) * 2 >= (int64_t)0x7fffffff) return false;
        if ((p.b_nrows * p.ldb + p.K) * 2 >= (int64_t)0x7fffffff) return false;
    }
    return true;
}

}  // namespace

size_t gemm_split_tail_floats(const GemmProblem* probs, int nprob, int ncu, const sl_tuning& tune) {
    GemmArgs a = make_args(probs, nprob, 256, 256, tune.gemm_grp);
    int dp;
    const int sks = split_tail_plan(a, ncu, dp);
    return sks ? (size_t)(a.first[MAXP] - dp) * sks * 256 * 256 : 0;
}

hipError_t launch_gemm_bf16(bool nn, const GemmProblem* probs, int nprob, hipStream_t st, float* skws,
                            size_t skws_floats, int ncu, const sl_tuning& tune, const SplitkRed* red,
                            bool* red_done) {
    if (red_done) *red_done = false;
    // tune.gemm_cfg selects a tile configuration by number (tuning sweeps).
    // The default (10, the eight-wave 256 x 256 kernel) was the fastest inside
    // whole FFN and attention steps at T = 4096 on launches of every size; the
    // smaller-tile and four-wave kernels win only on a product repeated with
    // its weights still in the caches.
    int cfg = tune.gemm_cfg;
    const int grp = tune.gemm_grp;
    if (!nn && cfg >= 10 && nt_v3_ok(probs, nprob)) {
        switch (cfg) {
            case 11: return launch_nt_cfg<256, 256, 2, 4, 2>(probs, nprob, st, skws, skws_floats, ncu, grp);
            case 12: return launch_nt_cfg<256, 256, 2, 4, 1>(probs, nprob, st, nullptr, 0, ncu, grp);
            case 13: return launch_nt_cfg<256, 128, 2, 2, 2>(probs, nprob, st, nullptr, 0, ncu, grp);
            case 14: return launch_nt_cfg<128, 128, 2, 2, 2>(probs, nprob, st, nullptr, 0, ncu, grp);
            case 15: return launch_nt_cfg<256, 256, 2, 2, 1>(probs, nprob, st, nullptr, 0, ncu, grp);
            case 20: return launch_nt5<2, 4, 32, 4>(probs, nprob, st, grp);
            case 21: return launch_nt5<2, 2, 32, 4>(probs, nprob, st, grp);
            case 31: return launch_nt5<2, 2, 32, 4>(probs, nprob, st, grp, skws, skws_floats, ncu);
            case 33: return launch_nt5<2, 2, 64, 2>(probs, nprob, st, grp, skws, skws_floats, ncu);
            case 22: return launch_nt5<2, 4, 64, 2>(probs, nprob, st, grp);
            case 23: return launch_nt5<2, 2, 64, 2>(probs, nprob, st, grp);
            default: return launch_nt_cfg<256, 256, 2, 4, 2>(probs, nprob, st, skws, skws_floats, ncu, grp, red,
                                                             red_done);
        }
    }
    if (cfg >= 10) cfg = 2;
    switch (cfg) {
        case 0: return nn ? launch_cfg<128, 128, 2, 2, true>(probs, nprob, st)
                          : launch_cfg<128, 128, 2, 2, false>(probs, nprob, st);
        case 1: return nn ? launch_cfg<256, 256, 2, 2, true>(probs, nprob, st)
                          : launch_cfg<256, 256, 2, 2, false>(probs, nprob, st);
        case 2: return nn ? launch_cfg<256, 256, 2, 4, true>(probs, nprob, st)
                          : launch_cfg<256, 256, 2, 4, false>(probs, nprob, st);
        case 3: return nn ? launch_cfg<256, 128, 2, 2, true>(probs, nprob, st)
                          : launch_cfg<256, 128, 2, 2, false>(probs, nprob, st);
        default: return nn ? launch_cfg<128, 256, 2, 2, true>(probs, nprob, st)
                           : launch_cfg<128, 256, 2, 2, false>(probs, nprob, st);
    }
}

namespace {
// K-chunks per tile of an fp32 launch: a launch of at most half a round of
// tiles splits K so that its blocks fill about one round (at most 16 chunks,
// each of at least 4 K steps of the longest problem); 1: no split.
int f32_split_plan(const GemmArgs& a, int ncu) {
    const int total = a.first[MAXP];
    if (ncu <= 0 || total <= 0 || 2 * total > ncu) return 1;
    int64_t nk = 0;
    for (int i = 0; i < a.nprob; ++i)
        if (a.first[i + 1] > a.first[i]) {
            const int64_t k = (a.p[i].K + FK - 1) / FK;
            nk = k > nk ? k : nk;
        }
    int S = ncu / total;
    if (S > 16) S = 16;
    while (S >= 2 && nk < 4 * S) --S;
    return S >= 2 ? S : 1;
}
}  // namespace

size_t gemm_f32_split_floats(const GemmProblem* probs, int nprob, int ncu) {
    GemmArgs a = make_args(probs, nprob, FB, FB);
    const int S = f32_split_plan(a, ncu);
    return S > 1 ? (size_t)a.first[MAXP] * S * FB * FB : 0;
}

hipError_t launch_gemm_f32(bool nn, const GemmProblem* probs, int nprob, hipStream_t st, float* skws,
                           size_t skws_floats, int ncu) {
    GemmArgs a = make_args(probs, nprob, FB, FB);
    const int total = a.first[MAXP];
    if (total == 0) return hipSuccess;
    int S = skws ? f32_split_plan(a, ncu) : 1;
    if (S > 1 && (size_t)total * S * FB * FB > skws_floats) S = 1;
    a.sks = S;
    a.skws = skws;
    if (nn) hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(total * S), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(total * S), dim3(256), 0, st, a);
    if (S > 1) hipLaunchKernelGGL(gemm_f32_sum_kernel, dim3(total * 16), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(bool bf16, const float* part, int64_t S, int64_t M, int64_t N,
                                void* Z, int64_t ldz, const int32_t* c_rows, const int32_t* c_cols,
                                int beta, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(N, 256), (unsigned)M);
    if (bf16)
        hipLaunchKernelGGL(splitk_reduce_kernel<bf16_t>, grid, dim3(256), 0, st, part, S, M, N,
                           (bf16_t*)Z, ldz, c_rows, c_cols, beta);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<float>, grid, dim3(256), 0, st, part, S, M, N,
                           (float*)Z, ldz, c_rows, c_cols, beta);
    return hipGetLastError();
}

