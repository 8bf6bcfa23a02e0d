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

constexpr int FQ = 64;   // queries (or keys) per block: 4 waves x 16
constexpr int FK = 32;   // keys (or queries) per inner step

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// 8 bf16 of one LDS row: two 4-element runs (the relabelled K index)
__device__ __forceinline__ bf16x8 lds_pair4(const bf16_t* row, int a0, int a1) {
    const uint2 x = *(const uint2*)(row + a0), y = *(const uint2*)(row + a1);
    return __builtin_bit_cast(bf16x8, make_uint4(x.x, x.y, y.x, y.y));
}

__device__ __forceinline__ uint4 gload16(const bf16_t* p, bool ok) {
    return ok ? *(const uint4*)p : make_uint4(0u, 0u, 0u, 0u);
}

// Stage FK rows (row r = r0 + j of the sequence) of a [*, ld] matrix slice at
// column c0: plain (rows x HD, pitch HD + 8) and/or transposed (HD x FK, pitch
// FK + 8).
template <int HD, bool PLAIN, bool TRANS>
__device__ __forceinline__ void stage(const bf16_t* __restrict__ src, int64_t ld, int64_t t0, int64_t r0,
                                      int64_t S, int64_t c0, bf16_t (*pl)[HD + 8], bf16_t (*tr)[FK + 8]) {
    for (int e = threadIdx.x; e < FK * HD / 8; e += 256) {
        const int j = e / (HD / 8), c8 = (e % (HD / 8)) * 8;
        const int64_t r = r0 + j;
        const uint4 v = gload16(src + (t0 + r) * ld + c0 + c8, r < S);
        if (PLAIN) *(uint4*)&pl[j][c8] = v;
        if (TRANS) {
            const bf16_t* vb = (const bf16_t*)&v;
#pragma unroll
            for (int q = 0; q < 8; ++q) tr[c8 + q][j] = vb[q];
        }
    }
}

// ---------------------------------------------------------------- forward
// Block = (64 queries, head h, sequence b); wave w owns queries q0 + 16 w ..
// + 15, lane l query q0 + 16 w + (l % 16).  Per step of 32 keys: S^T (2 tiles
// x HD/32 chunks), online softmax, O^T += V^T P^T (HD/16 tiles).
template <int HD>
__global__ __launch_bounds__(256) void attn_fwd_mfma_kernel(const bf16_t* __restrict__ q, int64_t ldq,
                                                            const bf16_t* __restrict__ k, int64_t ldk,
                                                            const bf16_t* __restrict__ v, int64_t ldv,
                                                            int64_t S, int64_t H, int64_t n_rep,
                                                            bf16_t* __restrict__ o, int64_t ldo,
                                                            float* __restrict__ lse) {
    constexpr int NC = HD / 32, NU = HD / 16;
    __shared__ __attribute__((aligned(16))) bf16_t Ks[FK][HD + 8];
    __shared__ __attribute__((aligned(16))) bf16_t Vt[HD][FK + 8];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, grp = lane >> 4, cn = lane & 15;
    const int64_t b = blockIdx.z, h = blockIdx.y, g = h / n_rep, t0 = b * S;
    const int64_t q0 = (int64_t)blockIdx.x * FQ, qn = q0 + 16 * w + cn;
    const float scale = 1.0f / sqrtf((float)HD);
    bf16x8 qf[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
        qf[c] = __builtin_bit_cast(bf16x8, gload16(q + (t0 + (qn < S ? qn : 0)) * ldq + h * HD + 32 * c + 8 * grp,
                                                   qn < S));
    f32x4 acc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lsum = 0.0f;
    const int64_t kend = q0 + FQ < S ? q0 + FQ : S;
    for (int64_t k0 = 0; k0 < kend; k0 += FK) {
        __syncthreads();
        stage<HD, true, false>(k, ldk, t0, k0, S, g * HD, Ks, nullptr);
        stage<HD, false, true>(v, ldv, t0, k0, S, g * HD, nullptr, Vt);
        __syncthreads();
        f32x4 st[2] = {(f32x4){0.f, 0.f, 0.f, 0.f}, (f32x4){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int c = 0; c < NC; ++c)
                st[t] = mfma16(*(const bf16x8*)&Ks[16 * t + cn][32 * c + 8 * grp], qf[c], st[t]);
        float p[8], mloc = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t key = k0 + 16 * t + 4 * grp + i;
                const float s = (key <= qn && key < S) ? st[t][i] * scale : -INFINITY;
                p[4 * t + i] = s;
                mloc = fmaxf(mloc, s);
            }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        const float mnew = fmaxf(m, mloc);
        const float mu = mnew == -INFINITY ? 0.0f : mnew;     // no visible key yet: everything stays 0
        const float corr = expf(m - mu);
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = expf(p[e] - mu);
            ps += p[e];
        }
        lsum = lsum * corr + ps;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[u][i] *= corr;
        const bf16x8 pb = pack8(p);
#pragma unroll
        for (int u = 0; u < NU; ++u)
            acc[u] = mfma16(lds_pair4(Vt[16 * u + cn], 4 * grp, 16 + 4 * grp), pb, acc[u]);
        m = mnew;
    }
    float l = lsum + __shfl_xor(lsum, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (qn >= S) return;
    const float inv = 1.0f / l;
    bf16_t* op = o + (t0 + qn) * ldo + h * HD + 4 * grp;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const uint2 pk = make_uint2(pack_bf16x2(acc[u][0] * inv, acc[u][1] * inv),
                                    pack_bf16x2(acc[u][2] * inv, acc[u][3] * inv));
        *(uint2*)(op + 16 * u) = pk;
    }
    if (grp == 0) lse[(b * H + h) * S + qn] = m + logf(l);
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
    const dim3 grid((unsigned)ceil_div(S, FQ), (unsigned)H, (unsigned)B);
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
