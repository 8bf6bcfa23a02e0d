// Causal softmax attention on the matrix cores (bf16 in, fp32 accumulation and
// softmax), forward and backward, for head dimensions 32, 64 and 128.
//
// Pages (all titled "SparseLoRA: Accelerating LLM Fine-Tuning with Contextual
// Sparsity"): the layers whose linears the method sparsifies are LLaMA decoder
// layers; between the q/k/v and o projections sits causal softmax attention
// with scale 1/sqrt(d) (paper-graph summary §3.4, "QK projection sparsity").
//
// All products use v_mfma_f32_16x16x32_bf16 (A 16x32, B 32x16, C 16x16 per
// wave; lane l holds A[l % 16][8 (l / 16) .. + 8], B[8 (l / 16) .. + 8][l % 16]
// and C[4 (l / 16) + i][l % 16], i < 4).  The score tiles are computed
// transposed, S^T = K Q^T, so a lane's four C entries belong to one query (its
// column): the online softmax of that query needs only its four lane groups
// (xor 16, 32).  The probability tile then feeds the next product directly as
// its B operand, with the product's K index read as "lane group g, entry j ->
// key 4 g + j (j < 4) or 16 + 4 g + (j - 4)" -- the same relabelling applied to
// the A operand, so the sum over keys is unchanged.
#include <cmath>

#include "sl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int FQ = 64;   // backward: queries (or keys) per block, 4 waves x 16

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// Transposed tiles keep each 32-row half in the products' relabelled K order:
// row quad q (rows 4 q .. 4 q + 3) of a half sits at column 8 (q % 4) +
// 4 (q / 4), so lane group g's eight K entries (rows 4 g .. + 3 and
// 16 + 4 g .. + 3) are one contiguous 16-byte run at column 8 g.
__device__ __forceinline__ int kpos(int rq) { return 32 * (rq >> 3) + 8 * (rq & 3) + 4 * ((rq >> 2) & 1); }

// the relabelled 8 K entries of lane group g in half hk of a transposed row
__device__ __forceinline__ bf16x8 lds_k8(const bf16_t* row, int hk, int g) {
    return *(const bf16x8*)(row + 32 * hk + 8 * g);
}

__device__ __forceinline__ uint4 gload16(const bf16_t* p, bool ok) {
    return ok ? *(const uint4*)p : make_uint4(0u, 0u, 0u, 0u);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Plain tiles keep row r's 16-byte chunk c at chunk c ^ ((r >> 4) & 3): the 16
// lanes of a quarter-wave store rows 4 apart (16 banks apart at a 68-word
// pitch), which the swizzle spreads over all 64 banks; a product reads one
// 16-row tile t at a time, where the swizzle is the fixed xor by t.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 4) & 3); }

// A tile of FR sequence rows (r0 .. r0 + FR - 1; rows at or past S read as 0)
// by HD columns of a [*, ld] slice at column c0, fetched into registers so the
// loads of the next step are in flight while the current one is multiplied.
// Unit e < FR / 4 * HD / 8 holds rows 4 (e % (FR / 4)) .. + 3 of the 8-column
// chunk e / (FR / 4): its transposed store is eight 8-byte runs of 4 rows.
template <int HD, int FR>
struct Tile {
    static constexpr int NQ = FR / 4, NE = NQ * HD / 8, PER = (NE + 255) / 256;
    uint4 r[PER][4];
    __device__ __forceinline__ void load(const bf16_t* __restrict__ src, int64_t ld, int64_t t0, int64_t r0,
                                         int64_t S, int64_t c0) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = threadIdx.x + 256 * p;
            if (NE % 256 != 0 && e >= NE) continue;
            const int rq = e % NQ, ci = e / NQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = r0 + 4 * rq + i;
                r[p][i] = gload16(src + (t0 + (row < S ? row : 0)) * ld + c0 + 8 * ci, row < S);
            }
        }
    }
    __device__ __forceinline__ void store_plain(bf16_t (*pl)[HD + 8]) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = threadIdx.x + 256 * p;
            if (NE % 256 != 0 && e >= NE) continue;
            const int rq = e % NQ, ci = e / NQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) *(uint4*)&pl[4 * rq + i][8 * swz(4 * rq + i, ci)] = r[p][i];
        }
    }
    template <int TP>
    __device__ __forceinline__ void store_trans(bf16_t (*tr)[TP]) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = threadIdx.x + 256 * p;
            if (NE % 256 != 0 && e >= NE) continue;
            const int rq = e % NQ, ci = e / NQ;
            const u32x4 x0 = __builtin_bit_cast(u32x4, r[p][0]), x1 = __builtin_bit_cast(u32x4, r[p][1]);
            const u32x4 x2 = __builtin_bit_cast(u32x4, r[p][2]), x3 = __builtin_bit_cast(u32x4, r[p][3]);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // column 8 ci + 2 w: low halves; column 8 ci + 2 w + 1: high halves
                const uint2 lo = make_uint2((x0[w] & 0xffffu) | (x1[w] << 16), (x2[w] & 0xffffu) | (x3[w] << 16));
                const uint2 hi = make_uint2((x0[w] >> 16) | (x1[w] & 0xffff0000u), (x2[w] >> 16) | (x3[w] & 0xffff0000u));
                *(uint2*)&tr[8 * ci + 2 * w][kpos(rq)] = lo;
                *(uint2*)&tr[8 * ci + 2 * w + 1][kpos(rq)] = hi;
            }
        }
    }
};

constexpr int F2Q = 128;       // forward: queries per block, 4 waves x 32
constexpr int F2K = 64;        // keys (forward, dQ) or queries (dK, dV) per step
// transposed-tile pitch (elements): 8-byte aligned rows, banks balanced for the
// 4-row stores above
constexpr int TP64 = F2K + 8;

// ---------------------------------------------------------------- forward
// Block = (128 queries, head h, sequence b), heaviest (latest) query blocks
// first; wave w owns queries q0 + 32 w .. + 31 as two 16-query column tiles,
// lane l queries q0 + 32 w + 16 qt + (l % 16).  Per step of 64 keys (K plain,
// V transposed, double-buffered in LDS, the next step's loads in flight):
// S^T (4 key tiles x 2 query tiles x HD/32 chunks), online softmax,
// O^T += V^T P^T (2 key halves x HD/16 tiles per query tile).  A wave skips
// the steps whose keys all lie after its queries.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_mfma_kernel(const bf16_t* __restrict__ q, int64_t ldq,
                                                            const bf16_t* __restrict__ k, int64_t ldk,
                                                            const bf16_t* __restrict__ v, int64_t ldv,
                                                            int64_t S, int64_t H, int64_t n_rep,
                                                            bf16_t* __restrict__ o, int64_t ldo,
                                                            float* __restrict__ lse) {
    constexpr int NC = HD / 32, NU = HD / 16;
    __shared__ __attribute__((aligned(16))) bf16_t Ks[2][F2K][HD + 8];
    __shared__ __attribute__((aligned(16))) bf16_t Vt[2][HD][TP64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, grp = lane >> 4, cn = lane & 15;
    const int64_t b = blockIdx.z, h = blockIdx.y, g = h / n_rep, t0 = b * S;
    const int64_t q0 = (int64_t)(gridDim.x - 1 - blockIdx.x) * F2Q, qw = q0 + 32 * w;
    // scores in base-2 units (log2 e folded into the scale): the softmax's
    // exponentials are single v_exp_f32 instructions
    const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
    bf16x8 qf[2][NC];
    int64_t qn[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        qn[qt] = qw + 16 * qt + cn;
        const bool ok = qn[qt] < S;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            qf[qt][c] = __builtin_bit_cast(
                bf16x8, gload16(q + (t0 + (ok ? qn[qt] : 0)) * ldq + h * HD + 32 * c + 8 * grp, ok));
    }
    f32x4 acc[2][NU];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[qt][u] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.0f, 0.0f};
    const int64_t kend = q0 + F2Q < S ? q0 + F2Q : S;
    const int nsteps = (int)((kend + F2K - 1) / F2K);
    Tile<HD, F2K> tk, tv;
    tk.load(k, ldk, t0, 0, S, g * HD);
    tv.load(v, ldv, t0, 0, S, g * HD);
    tk.store_plain(Ks[0]);
    tv.store_trans(Vt[0]);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1;
        const int64_t k0 = (int64_t)s * F2K;
        if (s + 1 < nsteps) {
            tk.load(k, ldk, t0, k0 + F2K, S, g * HD);
            tv.load(v, ldv, t0, k0 + F2K, S, g * HD);
        }
        // wave-uniform: which of the two query tiles see a key of this step
        bool vis[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) vis[qt] = !(k0 > qw + 16 * qt + 15 || qw + 16 * qt >= S);
        if (vis[0] || vis[1]) {
            // S^T for both query tiles, each K fragment read from LDS once
            f32x4 st[2][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                st[0][t] = st[1][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const bf16x8 kf = *(const bf16x8*)&Ks[buf][16 * t + cn][8 * ((4 * c + grp) ^ t)];
                    st[0][t] = mfma16(kf, qf[0][c], st[0][t]);
                    st[1][t] = mfma16(kf, qf[1][c], st[1][t]);
                }
            }
            bf16x8 pb[2][2];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float p[16], mloc = -INFINITY;
                // wave-uniform: every key of the step precedes the tile's first
                // query and lies inside the sequence, so nothing is masked
                const bool whole = k0 + F2K - 1 <= qw + 16 * qt && k0 + F2K <= S;
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t key = k0 + 16 * t + 4 * grp + i;
                        const float sv = (whole || (key <= qn[qt] && key < S)) ? st[qt][t][i] * sl2 : -INFINITY;
                        p[4 * t + i] = sv;
                        mloc = fmaxf(mloc, sv);
                    }
                mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
                mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
                const float mnew = fmaxf(m[qt], mloc);
                const float mu = mnew == -INFINITY ? 0.0f : mnew;   // no visible key yet: everything stays 0
                const float corr = __builtin_amdgcn_exp2f(m[qt] - mu);
                float ps = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    p[e] = __builtin_amdgcn_exp2f(p[e] - mu);
                    ps += p[e];
                }
                lsum[qt] = lsum[qt] * corr + ps;
                m[qt] = mnew;
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[qt][u][i] *= corr;
#pragma unroll
                for (int hk = 0; hk < 2; ++hk) {
                    float ph[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) ph[e] = p[8 * hk + e];
                    pb[qt][hk] = pack8(ph);
                }
            }
            // O^T += V^T P^T for both query tiles, each V^T fragment read once
            // (a tile with no visible key has P = 0 and corr = 1: unchanged)
#pragma unroll
            for (int hk = 0; hk < 2; ++hk)
#pragma unroll
                for (int u = 0; u < NU; ++u) {
                    const bf16x8 vf = lds_k8(Vt[buf][16 * u + cn], hk, grp);
                    acc[0][u] = mfma16(vf, pb[0][hk], acc[0][u]);
                    acc[1][u] = mfma16(vf, pb[1][hk], acc[1][u]);
                }
        }
        if (s + 1 < nsteps) {
            tk.store_plain(Ks[buf ^ 1]);
            tv.store_trans(Vt[buf ^ 1]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        float l = lsum[qt] + __shfl_xor(lsum[qt], 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (qn[qt] >= S) continue;
        const float inv = 1.0f / l;
        bf16_t* op = o + (t0 + qn[qt]) * ldo + h * HD + 4 * grp;
#pragma unroll
        for (int u = 0; u < NU; ++u)
            *(uint2*)(op + 16 * u) = make_uint2(pack_bf16x2(acc[qt][u][0] * inv, acc[qt][u][1] * inv),
                                                pack_bf16x2(acc[qt][u][2] * inv, acc[qt][u][3] * inv));
        // natural-log units for the backward: (m + log2 l) ln 2
        if (grp == 0) lse[(b * H + h) * S + qn[qt]] = (m[qt] + log2f(l)) * 0.6931471805599453f;
    }
}

// ---------------------------------------------------------------- backward
// With P = exp(s / sqrt(d) - lse) recomputed per tile and
// dS = P (dP - delta) / sqrt(d), delta[q] = sum_c dO[q, c] O[q, c]:
//   dQ = dS K, dK = dS^T Q, dV = P^T dO, dP = dO V^T.
// The dK/dV kernel (launched first) recomputes S and dP once per tile, and
// stores the bf16 dS it multiplies; the dQ kernel then needs one product per
// tile.  (This file's forward and backward kernels are reached for bf16; the
// fp32 path has kernels of its own.)

// dQ = dS K from the dS tiles the dK/dV kernel stored (bf16, the values its
// own products used): block = (64 queries, head h, sequence b), heaviest query
// blocks first; wave w owns queries q0 + 16 w .. + 15.  Per step of 64 keys,
// K and the dS tile [keys][queries] are staged transposed (the next step's
// loads in flight) and dQ^T += K^T dS^T.  dS rows are padded to a multiple of
// 64 queries; entries above the diagonal of a diagonal tile hold 0.
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_q_mfma_kernel(const bf16_t* __restrict__ k, int64_t ldk,
                                                              const bf16_t* __restrict__ dS, int64_t S,
                                                              int64_t Sp, int64_t H, int64_t n_rep,
                                                              bf16_t* __restrict__ dq, int64_t lddq) {
    constexpr int NU = HD / 16;
    __shared__ __attribute__((aligned(16))) bf16_t Kt[HD][TP64];
    __shared__ __attribute__((aligned(16))) bf16_t Dt[FQ][TP64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, grp = lane >> 4, cn = lane & 15;
    const int64_t b = blockIdx.z, h = blockIdx.y, g = h / n_rep, t0 = b * S;
    const int64_t q0 = (int64_t)(gridDim.x - 1 - blockIdx.x) * FQ, qw = q0 + 16 * w, qn = qw + cn;
    const bf16_t* dsh = dS + (b * H + h) * S * Sp;
    f32x4 acc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int64_t kend = q0 + FQ < S ? q0 + FQ : S;
    Tile<HD, F2K> tk;
    Tile<FQ, F2K> td;   // rows: keys; columns: this block's queries
    tk.load(k, ldk, t0, 0, S, g * HD);
    td.load(dsh, Sp, 0, 0, S, q0);
    for (int64_t k0 = 0; k0 < kend; k0 += F2K) {
        __syncthreads();
        tk.store_trans(Kt);
        td.store_trans(Dt);
        __syncthreads();
        if (k0 + F2K < kend) {
            tk.load(k, ldk, t0, k0 + F2K, S, g * HD);
            td.load(dsh, Sp, 0, k0 + F2K, S, q0);
        }
        if (k0 > qw + 15 || qw >= S) continue;   // wave-uniform: no visible key
#pragma unroll
        for (int hk = 0; hk < F2K / 32; ++hk) {
            const bf16x8 db = lds_k8(Dt[16 * w + cn], hk, grp);
#pragma unroll
            for (int u = 0; u < NU; ++u)
                acc[u] = mfma16(lds_k8(Kt[16 * u + cn], hk, grp), db, acc[u]);
        }
    }
    if (qn >= S) return;
    bf16_t* op = dq + (t0 + qn) * lddq + h * HD + 4 * grp;
#pragma unroll
    for (int u = 0; u < NU; ++u)
        *(uint2*)(op + 16 * u) = make_uint2(pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3]));
}

// dK, dV: block = (64 keys, key/value head g, sequence b); wave w owns keys
// k0 + 16 w .. + 15.  Steps run over the group's query heads and, per head,
// the 64-query runs at or after the keys (Q and dO plain and transposed; the
// next step's loads in flight).  S and dP are computed untransposed
// (S = Q K^T, dP = dO V^T with K^T, V^T fragments in registers), so a lane's
// four C entries belong to one key; then dV^T += dO^T P and dK^T += Q^T dS.
template <int HD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_kv_mfma_kernel(
    const bf16_t* __restrict__ q, int64_t ldq, const bf16_t* __restrict__ k, int64_t ldk,
    const bf16_t* __restrict__ v, int64_t ldv, const bf16_t* __restrict__ dO, int64_t lddo,
    const float* __restrict__ lse, const float* __restrict__ delta, int64_t S, int64_t H, int64_t n_rep,
    bf16_t* __restrict__ dk, int64_t lddk, bf16_t* __restrict__ dv, int64_t lddv, bf16_t* __restrict__ dS,
    int64_t Sp) {
    constexpr int NC = HD / 32, NU = HD / 16, NT = F2K / 16;
    __shared__ __attribute__((aligned(16))) bf16_t Qs[F2K][HD + 8];
    __shared__ __attribute__((aligned(16))) bf16_t Qt[HD][TP64];
    __shared__ __attribute__((aligned(16))) bf16_t Gs[F2K][HD + 8];
    __shared__ __attribute__((aligned(16))) bf16_t Gt[HD][TP64];
    __shared__ float Ls[F2K], Ds[F2K];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, grp = lane >> 4, cn = lane & 15;
    const int64_t b = blockIdx.z, g = blockIdx.y, t0 = b * S;
    const int64_t k0 = (int64_t)blockIdx.x * FQ, kw = k0 + 16 * w, kn = kw + cn;
    const bool kv = kn < S;
    const float scale = 1.0f / sqrtf((float)HD), sl2 = 1.4426950408889634f * scale;
    bf16x8 kf[NC], vf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int64_t off = t0 + (kv ? kn : 0);
        kf[c] = __builtin_bit_cast(bf16x8, gload16(k + off * ldk + g * HD + 32 * c + 8 * grp, kv));
        vf[c] = __builtin_bit_cast(bf16x8, gload16(v + off * ldv + g * HD + 32 * c + 8 * grp, kv));
    }
    f32x4 dka[NU], dva[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) dka[u] = dva[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // steps (query head hr, queries i0 .. i0 + 63), i0 from k0 to S, flattened
    const int64_t nsi = (S - k0 + F2K - 1) / F2K, nst = nsi * n_rep;
    Tile<HD, F2K> tq, tg;
    float lr = 0.0f, dr = 0.0f;
    auto fetch = [&](int64_t sidx) {
        const int64_t h = g * n_rep + sidx / nsi, i0 = k0 + (sidx % nsi) * F2K;
        tq.load(q, ldq, t0, i0, S, h * HD);
        tg.load(dO, lddo, t0, i0, S, h * HD);
        if (threadIdx.x < F2K) {
            const int64_t qi = i0 + threadIdx.x;
            lr = qi < S ? lse[(b * H + h) * S + qi] * 1.4426950408889634f : 0.0f;   // base 2
            dr = qi < S ? delta[(b * H + h) * S + qi] : 0.0f;
        }
    };
    fetch(0);
    for (int64_t sidx = 0; sidx < nst; ++sidx) {
        const int64_t i0 = k0 + (sidx % nsi) * F2K;
        __syncthreads();
        tq.store_plain(Qs);
        tq.store_trans(Qt);
        tg.store_plain(Gs);
        tg.store_trans(Gt);
        if (threadIdx.x < F2K) Ls[threadIdx.x] = lr, Ds[threadIdx.x] = dr;
        __syncthreads();
        if (sidx + 1 < nst) fetch(sidx + 1);
        if (i0 + F2K - 1 < kw || kw >= S) continue;   // wave-uniform: every query precedes the wave's keys
        f32x4 st[NT], dp[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            st[t] = dp[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                st[t] = mfma16(*(const bf16x8*)&Qs[16 * t + cn][8 * ((4 * c + grp) ^ t)], kf[c], st[t]);
                dp[t] = mfma16(*(const bf16x8*)&Gs[16 * t + cn][8 * ((4 * c + grp) ^ t)], vf[c], dp[t]);
            }
        }
        // wave-uniform: every query of the step follows the wave's keys and
        // both lie inside the sequence, so nothing is masked
        const bool whole = i0 >= kw + 15 && i0 + F2K <= S && kw + 16 <= S;
#pragma unroll
        for (int hk = 0; hk < NT / 2; ++hk) {
            float p[8], ds[8];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 2 * hk + tt, j = 16 * t + 4 * grp + i;
                    const int64_t qi = i0 + j;
                    const float pv = (whole || (kv && qi < S && kn <= qi))
                                         ? __builtin_amdgcn_exp2f(st[t][i] * sl2 - Ls[j]) : 0.0f;
                    p[4 * tt + i] = pv;
                    ds[4 * tt + i] = pv * (dp[t][i] - Ds[j]) * scale;
                }
            const bf16x8 pb = pack8(p), db = pack8(ds);
            if (kv) {
                // dS[b, h][key][query]: the 4 consecutive queries of each 16-query tile
                const uint4 dw = __builtin_bit_cast(uint4, db);
                bf16_t* dr = dS + ((b * H + g * n_rep + sidx / nsi) * S + kn) * Sp + i0 + 32 * hk + 4 * grp;
                *(uint2*)dr = make_uint2(dw.x, dw.y);
                *(uint2*)(dr + 16) = make_uint2(dw.z, dw.w);
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                dva[u] = mfma16(lds_k8(Gt[16 * u + cn], hk, grp), pb, dva[u]);
                dka[u] = mfma16(lds_k8(Qt[16 * u + cn], hk, grp), db, dka[u]);
            }
        }
    }
    if (!kv) return;
    bf16_t* kp = dk + (t0 + kn) * lddk + g * HD + 4 * grp;
    bf16_t* vp = dv + (t0 + kn) * lddv + g * HD + 4 * grp;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        *(uint2*)(kp + 16 * u) = make_uint2(pack_bf16x2(dka[u][0], dka[u][1]), pack_bf16x2(dka[u][2], dka[u][3]));
        *(uint2*)(vp + 16 * u) = make_uint2(pack_bf16x2(dva[u][0], dva[u][1]), pack_bf16x2(dva[u][2], dva[u][3]));
    }
}

}  // namespace

bool attn_mfma_ok(int64_t hd, const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                  int64_t ldv, const void* o, int64_t ldo) {
    const auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    return (hd == 32 || hd == 64 || hd == 128) && a16(q) && a16(k) && a16(v) && ((uintptr_t)o & 7) == 0 &&
           ldq % 8 == 0 && ldk % 8 == 0 && ldv % 8 == 0 && ldo % 4 == 0;
}

hipError_t launch_attn_fwd_mfma(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                                int64_t ldv, int64_t B, int64_t S, int64_t H, int64_t Hkv, int64_t hd, void* o,
                                int64_t ldo, float* lse, hipStream_t st) {
    if (B <= 0 || S <= 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(S, F2Q), (unsigned)H, (unsigned)B);
    const int64_t n_rep = H / Hkv;
#define AF(HDV)                                                                                      \
    hipLaunchKernelGGL((attn_fwd_mfma_kernel<HDV>), grid, dim3(256), 0, st, (const bf16_t*)q, ldq,      \
                       (const bf16_t*)k, ldk, (const bf16_t*)v, ldv, S, H, n_rep, (bf16_t*)o, ldo, lse)
    if (hd == 32) AF(32);
    else if (hd == 64) AF(64);
    else if (hd == 128) AF(128);
    else return hipErrorInvalidValue;
#undef AF
    return hipGetLastError();
}


bool attn_mfma_bwd_ok(int64_t hd, const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                      int64_t ldv, const void* dO, int64_t lddo, const void* dq, int64_t lddq, const void* dk,
                      int64_t lddk, const void* dv, int64_t lddv) {
    const auto a8 = [](const void* p, int64_t ld) { return ((uintptr_t)p & 7) == 0 && ld % 4 == 0; };
    return attn_mfma_ok(hd, q, ldq, k, ldk, v, ldv, dq, lddq) && ((uintptr_t)dO & 15) == 0 && lddo % 8 == 0 &&
           a8(dk, lddk) && a8(dv, lddv);
}

size_t attn_bwd_ds_bytes(int64_t B, int64_t S, int64_t H) {
    return (size_t)B * H * S * (size_t)(ceil_div(S, FQ) * FQ) * sizeof(bf16_t);
}

hipError_t launch_attn_bwd_mfma(const void* q, int64_t ldq, const void* k, int64_t ldk, const void* v,
                                int64_t ldv, const void* dO, int64_t lddo, const float* lse, const float* delta,
                                int64_t B, int64_t S, int64_t H, int64_t Hkv, int64_t hd, void* dq, int64_t lddq,
                                void* dk, int64_t lddk, void* dv, int64_t lddv, void* ds, hipStream_t st) {
    if (B <= 0 || S <= 0) return hipSuccess;
    const dim3 gq((unsigned)ceil_div(S, FQ), (unsigned)H, (unsigned)B);
    const dim3 gk((unsigned)ceil_div(S, FQ), (unsigned)Hkv, (unsigned)B);
    const int64_t n_rep = H / Hkv, Sp = ceil_div(S, FQ) * FQ;
#define AB(HDV)                                                                                               \
    hipLaunchKernelGGL((attn_bwd_kv_mfma_kernel<HDV>), gk, dim3(256), 0, st, (const bf16_t*)q, ldq,             \
                       (const bf16_t*)k, ldk, (const bf16_t*)v, ldv, (const bf16_t*)dO, lddo, lse, delta, S, H, \
                       n_rep, (bf16_t*)dk, lddk, (bf16_t*)dv, lddv, (bf16_t*)ds, Sp);                          \
    hipLaunchKernelGGL((attn_bwd_q_mfma_kernel<HDV>), gq, dim3(256), 0, st, (const bf16_t*)k, ldk,              \
                       (const bf16_t*)ds, S, Sp, H, n_rep, (bf16_t*)dq, lddq)
    if (hd == 32) { AB(32); }
    else if (hd == 64) { AB(64); }
    else if (hd == 128) { AB(128); }
    else return hipErrorInvalidValue;
#undef AB
    return hipGetLastError();
}
