// gdn_verify.hip -- gated delta rule over a K-token verify window with
// intermediate-state capture, chunkwise in WY form (gfx950).
//
// The step the pages describe as a fused WY-chunkwise GDN verify that writes
// the final state and every intermediate state in one pass (atlas PR #297,
// commit message on gated_delta_rule_wy16.cu), with the raw gates applied in
// the kernel, q/k broadcast from key heads and one L2 normalisation of the
// q|k slab (lucebox PR #637, commit messages on raw-gate gated_delta_net and
// the DeltaNet block; review excerpt of gated_delta_net.cu).
//
// Math, per sequence b and value head h, with G_t = sum_{s<=t} g_s:
//   A[t][s] = beta_t e^{G_t-G_s} k^_t.k^_s      (s < t)
//   u       = (I + A)^{-1} beta (v - e^{G} S_in k^)     (one column per state row)
//   o_t     = e^{G_t} S_in q^_t + sum_{s<=t} e^{G_t-G_s} (q^_t.k^_s) u_s
//   H_t     = e^{g_t} H_{t-1} + u_t k^_t^T,  H_{-1} = S_in
// Only exponentials of G_t - G_s with s <= t are formed (no ratio of decays).
//
// Mapping.  Each state row (a value index i) evolves on its own once the
// per-head prologue (norms, gates, A, M) is known, so a workgroup is one wave
// that owns 8 rows of one head: 8 lanes per row, each lane holding DK/8
// columns as DK/32 float4 chunks at columns 32m + 4*sub.  A store instruction
// then writes 8 rows x 128 contiguous bytes.  The wave:
//   1. issues the loads of its 8 state rows and their v values;
//   2. stages the raw q, k of the key head in LDS and computes the gates;
//   3. forms the Gram matrices K K^T, Q K^T (and the diagonal of Q Q^T) with
//      MFMA from the raw inputs -- 16x16x32 bf16 for bf16 inputs (products of
//      bf16 are exact, accumulation fp32), 16x16x4 f32 for f32 inputs -- and
//      scales them by the inverse norms to get A and M in LDS;
//   4. per row: K dot products S_in k_t and S_in q_t (VALU, 8-lane DPP sums),
//      forward substitution for u, the outputs o_t;
//   5. streams H_t = gamma_t H_{t-1} + u_t k^_t^T, storing every H_t and the
//      final state -- the bulk of the bytes of the whole step.
#include "gdn_device.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {
namespace {

constexpr int kLanes = 64;

template <int DK, int KMAX, bool IN_BF16>
struct VerifySmem {
    using in_t = typename std::conditional<IN_BF16, uint16_t, float>::type;
    in_t q[KMAX][DK];        // raw q of the key head, rows >= K zero
    in_t k[KMAX][DK];        // raw k
    float A[KMAX][KMAX];     // beta_t e^{G_t-G_s} k^_t.k^_s, s < t
    float M[KMAX][KMAX];     // e^{G_t-G_s} q^_t.k^_s, s <= t
    float nq2[KMAX], nk2[KMAX];
    float rq[KMAX], rk[KMAX];
    float beta[KMAX], g[KMAX], G[KMAX], eG[KMAX], gam[KMAX];
};

// gates of token t for value head h
__device__ __forceinline__ void gate(float braw, float al, const float* dt_bias, const float* A_log, int h,
                                     float& beta, float& g)
{
    if (dt_bias != nullptr) {
        beta = 1.0f / (1.0f + __expf(-braw));
        const float a = al + dt_bias[h];
        const float sp = a > 20.0f ? a : log1pf(__expf(a));
        g = -sp * __expf(A_log[h]);
    } else {
        beta = braw;
        g = al;
    }
}

// Gram tile D[m][n] = sum_k X[tm*16+m][k] Y[tn*16+n][k] over the DK columns,
// X, Y raw in LDS.  Lane l feeds row l%16 of both operands with the same
// k-slice, so the product is the Gram block whatever order the instruction
// assigns to the k elements within a lane.
template <int DK, bool IN_BF16, typename in_t>
__device__ __forceinline__ f32x4_t gram_tile(const in_t (*X)[DK], const in_t (*Y)[DK], int tm, int tn, int lane)
{
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int r = lane & 15, ks = lane >> 4;
    if constexpr (IN_BF16) {
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&X[tm * 16 + r][32 * kk + 8 * ks]);
            const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&Y[tn * 16 + r][32 * kk + 8 * ks]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < DK / 4; ++kk) {
            const float a = X[tm * 16 + r][4 * kk + ks];
            const float b = Y[tn * 16 + r][4 * kk + ks];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
    }
    return acc;
}

template <int DK, int KMAX, bool IN_BF16, bool O_BF16, bool NT>
__global__ __launch_bounds__(kLanes) void verify_kernel(VerifyArgs a)
{
    constexpr int NCH = DK / 32;                 // float4 chunks per lane
    constexpr int TB = (KMAX + 15) / 16;         // 16-token blocks for the MFMA tiles
    constexpr int KP = TB * 16;                  // padded token count of the LDS tiles
    using Smem = VerifySmem<DK, KP, IN_BF16>;
    using in_t = typename Smem::in_t;
    __shared__ Smem sm;

    const int lane = threadIdx.x;
    const int rloc = lane >> 3, sub = lane & 7;
    const int h = blockIdx.y, b = blockIdx.z;
    const int i = blockIdx.x * 8 + rloc;
    const int K = a.K, Hk = a.Hk, Hv = a.Hv, dv = a.dv;
    const int C = 2 * Hk * DK + Hv * dv;
    const int hk = h / (Hv / Hk);
    const size_t SD = (size_t)dv * DK;

    // ---- 1. state rows and v values (independent of the prologue)
    const size_t srow = ((size_t)b * Hv + h) * SD + (size_t)i * DK;
    f32x4_t S[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) S[m] = load_f4(a.S_in + srow + 32 * m + 4 * sub);
    float v[KMAX];
#pragma unroll
    for (int t = 0; t < KMAX; ++t)
        v[t] = t < K ? load1<IN_BF16>(a.qkv, ((size_t)b * K + t) * C + 2 * (size_t)Hk * DK + (size_t)h * dv + i)
                     : 0.0f;

    // ---- 2. stage raw q, k (16 bytes per lane per step), gates
    {
        constexpr int EPV = IN_BF16 ? 8 : 4;     // elements per 16-byte vector
        constexpr int VPR = DK / EPV;            // vectors per row
        for (int idx = lane; idx < KP * VPR; idx += kLanes) {
            const int t = idx / VPR, c = (idx % VPR) * EPV;
            uint4 qv = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
            if (t < K) {
                const size_t rowoff = ((size_t)b * K + t) * C;
                const in_t* base = reinterpret_cast<const in_t*>(a.qkv) + rowoff;
                qv = *reinterpret_cast<const uint4*>(base + (size_t)hk * DK + c);
                kv = *reinterpret_cast<const uint4*>(base + (size_t)Hk * DK + (size_t)hk * DK + c);
            }
            *reinterpret_cast<uint4*>(&sm.q[t][c]) = qv;
            *reinterpret_cast<uint4*>(&sm.k[t][c]) = kv;
        }
        if (lane < KP) {
            float be = 0.f, g = 0.f;
            if (lane < K) {
                const size_t gi = ((size_t)b * K + lane) * Hv + h;
                gate(load1<IN_BF16>(a.beta_raw, gi), load1<IN_BF16>(a.alpha, gi), a.dt_bias, a.A_log, h, be, g);
            }
            sm.beta[lane] = be;
            sm.g[lane] = g;
        }
    }
    __syncthreads();

    // ---- 3. Gram tiles with MFMA; norms from their diagonals; A and M
    {
        // running sums of g; G_t for t >= K is never used
        if (lane < KP) {
            float G = 0.f;
            for (int s = 0; s <= lane; ++s) G += sm.g[s];
            sm.G[lane] = G;
            sm.eG[lane] = __expf(G);
            sm.gam[lane] = __expf(sm.g[lane]);
        }
        const int n = lane & 15, mq = (lane >> 4) * 4;
        f32x4_t kk[TB][TB], qk[TB][TB];
#pragma unroll
        for (int tm = 0; tm < TB; ++tm) {
#pragma unroll
            for (int tn = 0; tn <= tm; ++tn) {
                kk[tm][tn] = gram_tile<DK, IN_BF16, in_t>(sm.k, sm.k, tm, tn, lane);
                qk[tm][tn] = gram_tile<DK, IN_BF16, in_t>(sm.q, sm.k, tm, tn, lane);
            }
            const f32x4_t qq = gram_tile<DK, IN_BF16, in_t>(sm.q, sm.q, tm, tm, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (mq + e == n) {
                    sm.nk2[tm * 16 + n] = kk[tm][tm][e];
                    sm.nq2[tm * 16 + n] = qq[e];
                }
            }
        }
        __syncthreads();
        if (lane < KP) {
            sm.rk[lane] = 1.0f / sqrtf(sm.nk2[lane] + a.eps);
            sm.rq[lane] = 1.0f / sqrtf(sm.nq2[lane] + a.eps);
        }
        __syncthreads();
        // D layout of a 16x16 MFMA tile: lane l, element e holds row 4*(l/16)+e, column l%16
#pragma unroll
        for (int tm = 0; tm < TB; ++tm) {
#pragma unroll
            for (int tn = 0; tn < TB; ++tn) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = tm * 16 + mq + e, s = tn * 16 + n;
                    float av = 0.f, mv = 0.f;
                    if (tn <= tm && t < K && s <= t) {
                        const float dec = __expf(sm.G[t] - sm.G[s]);
                        const float rks = sm.rk[s];
                        mv = dec * qk[tm][tn][e] * sm.rq[t] * rks;
                        if (s < t) av = sm.beta[t] * dec * kk[tm][tn][e] * sm.rk[t] * rks;
                    }
                    sm.A[t][s] = av;
                    sm.M[t][s] = mv;
                }
            }
        }
    }
    __syncthreads();

    // ---- 4. per row: S_in k_t, S_in q_t, substitution, outputs
    float p[KMAX], r[KMAX];
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
        float pk = 0.f, pq = 0.f;
        if (t < K) {
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const int c = 32 * m + 4 * sub;
                float kx[4], qx[4];
                if constexpr (IN_BF16) {
                    const uint2 ku = *reinterpret_cast<const uint2*>(&sm.k[t][c]);
                    const uint2 qu = *reinterpret_cast<const uint2*>(&sm.q[t][c]);
                    kx[0] = bf16_lo(ku.x); kx[1] = bf16_hi(ku.x); kx[2] = bf16_lo(ku.y); kx[3] = bf16_hi(ku.y);
                    qx[0] = bf16_lo(qu.x); qx[1] = bf16_hi(qu.x); qx[2] = bf16_lo(qu.y); qx[3] = bf16_hi(qu.y);
                } else {
                    const float4 kf = *reinterpret_cast<const float4*>(&sm.k[t][c]);
                    const float4 qf = *reinterpret_cast<const float4*>(&sm.q[t][c]);
                    kx[0] = kf.x; kx[1] = kf.y; kx[2] = kf.z; kx[3] = kf.w;
                    qx[0] = qf.x; qx[1] = qf.y; qx[2] = qf.z; qx[3] = qf.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pk = __builtin_fmaf(S[m][e], kx[e], pk);
                    pq = __builtin_fmaf(S[m][e], qx[e], pq);
                }
            }
        }
        p[t] = pk;
        r[t] = pq;
    }
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
        if (t < K) {
            p[t] = sum8(p[t]) * sm.rk[t];
            r[t] = sum8(r[t]) * sm.rq[t];
        }
    }
    float u[KMAX];
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
        float acc = 0.f;
        if (t < K) {
            acc = sm.beta[t] * (v[t] - sm.eG[t] * p[t]);
#pragma unroll
            for (int s = 0; s < t; ++s) acc = __builtin_fmaf(-sm.A[t][s], u[s], acc);
        }
        u[t] = acc;
    }
    {
        float mine[(KMAX + 7) / 8];
#pragma unroll
        for (int j = 0; j < (KMAX + 7) / 8; ++j) mine[j] = 0.f;
#pragma unroll
        for (int t = 0; t < KMAX; ++t) {
            if (t < K) {
                float ot = sm.eG[t] * r[t];
#pragma unroll
                for (int s = 0; s <= t; ++s) ot = __builtin_fmaf(sm.M[t][s], u[s], ot);
                if ((t & 7) == sub) mine[t >> 3] = ot;
            }
        }
#pragma unroll
        for (int j = 0; j < (KMAX + 7) / 8; ++j) {
            const int t = 8 * j + sub;
            if (t < K) store1<O_BF16>(a.o, (((size_t)b * K + t) * Hv + h) * dv + i, mine[j]);
        }
    }

    // ---- 5. stream the states: H_t = gamma_t H_{t-1} + (u_t rk_t) k_t
#pragma unroll
    for (int t = 0; t < KMAX; ++t) {
        if (t < K) {
            const float gm = sm.gam[t];
            const float cu = u[t] * sm.rk[t];
            float* dst;
            if (t < K - 1) {
                if (a.H == nullptr) dst = nullptr;
                else dst = a.H + (((size_t)b * (K - 1) + t) * Hv + h) * SD + (size_t)i * DK;
            } else {
                dst = a.S_out + srow;
            }
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const int c = 32 * m + 4 * sub;
                float kx[4];
                if constexpr (IN_BF16) {
                    const uint2 ku = *reinterpret_cast<const uint2*>(&sm.k[t][c]);
                    kx[0] = bf16_lo(ku.x); kx[1] = bf16_hi(ku.x); kx[2] = bf16_lo(ku.y); kx[3] = bf16_hi(ku.y);
                } else {
                    const float4 kf = *reinterpret_cast<const float4*>(&sm.k[t][c]);
                    kx[0] = kf.x; kx[1] = kf.y; kx[2] = kf.z; kx[3] = kf.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) S[m][e] = __builtin_fmaf(cu, kx[e], gm * S[m][e]);
                if (dst != nullptr) {
                    if (t < K - 1) store_f4<NT>(dst + c, S[m]);
                    else store_f4<false>(dst + c, S[m]);
                }
            }
        }
    }
}

template <int DK, int KMAX, bool IN_BF16, bool O_BF16>
hipError_t launch_k(const VerifyArgs& a, hipStream_t s)
{
    dim3 grid(a.dv / 8, a.Hv, a.B);
    verify_kernel<DK, KMAX, IN_BF16, O_BF16, false><<<grid, dim3(kLanes), 0, s>>>(a);
    return hipGetLastError();
}

template <int DK, bool IN_BF16, bool O_BF16>
hipError_t launch_d(const VerifyArgs& a, hipStream_t s)
{
    if (a.K <= 1) return launch_k<DK, 1, IN_BF16, O_BF16>(a, s);
    if (a.K <= 2) return launch_k<DK, 2, IN_BF16, O_BF16>(a, s);
    if (a.K <= 4) return launch_k<DK, 4, IN_BF16, O_BF16>(a, s);
    if (a.K <= 8) return launch_k<DK, 8, IN_BF16, O_BF16>(a, s);
    if (a.K <= 16) return launch_k<DK, 16, IN_BF16, O_BF16>(a, s);
    return launch_k<DK, 32, IN_BF16, O_BF16>(a, s);
}

template <bool IN_BF16, bool O_BF16>
hipError_t launch_io(const VerifyArgs& a, hipStream_t s)
{
    switch (a.dk) {
    case 32: return launch_d<32, IN_BF16, O_BF16>(a, s);
    case 64: return launch_d<64, IN_BF16, O_BF16>(a, s);
    case 128: return launch_d<128, IN_BF16, O_BF16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, bool in_bf16, bool o_bf16, hipStream_t s)
{
    if (in_bf16) return o_bf16 ? launch_io<true, true>(a, s) : launch_io<true, false>(a, s);
    return o_bf16 ? launch_io<false, true>(a, s) : launch_io<false, false>(a, s);
}

}  // namespace gdn
