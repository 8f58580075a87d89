// gdn_prefill.hip -- the gated delta rule over a long prompt, final state only
// (fp32 q|k|v slabs; bf16 slabs go to the MFMA kernel of gdn_prefill_wy.hip).
//
// The same recurrence as the verify step (gates, L2-normalised q/k broadcast
// from key heads, S_t = e^{g_t} S_{t-1}(I - beta k k^T) + beta v k^T,
// o_t = S_t q_t), run over T prompt tokens.  Only the state after the last
// token is written, plus every output o_t.
//
// The prompt is consumed in chunks: for every chunk the workgroup stages the
// raw q, k of its key head, the v of its rows and the gates of its value head
// in LDS, computes the chunk's q/k norms once, and then advances its state
// rows token by token.  Each state row evolves on its own given the staged
// vectors, so a workgroup of 4 waves owns 32 rows of one head (8 lanes per
// row, DK/8 columns per lane, the state in registers for the whole prompt).
#include "gdn_device.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 32;   // state rows per workgroup

template <int DK, int CH, bool IN_BF16>
struct PrefillSmem {
    using in_t = typename std::conditional<IN_BF16, uint16_t, float>::type;
    in_t q[CH][DK];
    in_t k[CH][DK];
    float v[CH][kRows];
    float rq[CH], rk[CH], beta[CH], gam[CH];
};

__device__ __forceinline__ void gate_p(float braw, float al, const float* dt_bias, const float* A_log, int h,
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

template <int DK, int CH, bool IN_BF16, bool O_BF16>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a)
{
    constexpr int NCH = DK / 32;
    using Smem = PrefillSmem<DK, CH, IN_BF16>;
    using in_t = typename Smem::in_t;
    __shared__ Smem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int rloc = wave * 8 + (lane >> 3), sub = lane & 7;
    const int h = blockIdx.y, b = blockIdx.z;
    const int i = blockIdx.x * kRows + rloc;
    const int T = a.T, Hk = a.Hk, Hv = a.Hv, dv = a.dv;
    const int C = 2 * Hk * DK + Hv * dv;
    const int hk = h / (Hv / Hk);
    const size_t SD = (size_t)dv * DK;
    const bool live = i < dv;

    const size_t srow = ((size_t)b * Hv + h) * SD + (size_t)i * DK;
    f32x4_t S[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m)
        S[m] = live ? load_f4(a.S_in + srow + 32 * m + 4 * sub) : f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < T; c0 += CH) {
        const int L = min(CH, T - c0);
        __syncthreads();  // the previous chunk is done with the LDS
        {
            constexpr int EPV = IN_BF16 ? 8 : 4;
            constexpr int VPR = DK / EPV;
            for (int idx = tid; idx < L * VPR; idx += kThreads) {
                const int t = idx / VPR, c = (idx % VPR) * EPV;
                const in_t* base = reinterpret_cast<const in_t*>(a.qkv) + ((size_t)b * T + c0 + t) * C;
                *reinterpret_cast<uint4*>(&sm.q[t][c]) = *reinterpret_cast<const uint4*>(base + (size_t)hk * DK + c);
                *reinterpret_cast<uint4*>(&sm.k[t][c]) =
                    *reinterpret_cast<const uint4*>(base + (size_t)Hk * DK + (size_t)hk * DK + c);
            }
            for (int idx = tid; idx < L * kRows; idx += kThreads) {
                const int t = idx / kRows, rr = idx % kRows;
                const int row = blockIdx.x * kRows + rr;
                sm.v[t][rr] = row < dv ? load1<IN_BF16>(a.qkv, ((size_t)b * T + c0 + t) * C + 2 * (size_t)Hk * DK +
                                                                   (size_t)h * dv + row)
                                       : 0.0f;
            }
            if (tid < L) {
                const size_t gi = ((size_t)b * T + c0 + tid) * Hv + h;
                float be, g;
                gate_p(load1<IN_BF16>(a.beta_raw, gi), load1<IN_BF16>(a.alpha, gi), a.dt_bias, a.A_log, h, be, g);
                sm.beta[tid] = be;
                sm.gam[tid] = __expf(g);
            }
        }
        __syncthreads();
        // norms: 4 threads per (token, q|k), each a quarter of the row
        for (int idx = tid; idx < 2 * CH * 4; idx += kThreads) {
            const int part = idx & 3, which = (idx >> 2) & 1, t = idx >> 3;
            float s2 = 0.f;
            if (t < L) {
                const in_t* row = which ? sm.k[t] : sm.q[t];
#pragma unroll 8
                for (int c = part * (DK / 4); c < (part + 1) * (DK / 4); ++c) {
                    float x;
                    if constexpr (IN_BF16) x = bf16_to_f32(row[c]);
                    else x = row[c];
                    s2 = __builtin_fmaf(x, x, s2);
                }
            }
            s2 += dpp_mov<kDppQuadXor1>(s2);
            s2 += dpp_mov<kDppQuadXor2>(s2);
            if (part == 0 && t < L) {
                const float rn = 1.0f / sqrtf(s2 + a.eps);
                if (which) sm.rk[t] = rn;
                else sm.rq[t] = rn;
            }
        }
        __syncthreads();

        for (int t = 0; t < L; ++t) {
            float kx[NCH][4], qx[NCH][4];
#pragma unroll
            for (int m = 0; m < NCH; ++m) {
                const int c = 32 * m + 4 * sub;
                if constexpr (IN_BF16) {
                    const uint2 ku = *reinterpret_cast<const uint2*>(&sm.k[t][c]);
                    const uint2 qu = *reinterpret_cast<const uint2*>(&sm.q[t][c]);
                    kx[m][0] = bf16_lo(ku.x); kx[m][1] = bf16_hi(ku.x); kx[m][2] = bf16_lo(ku.y); kx[m][3] = bf16_hi(ku.y);
                    qx[m][0] = bf16_lo(qu.x); qx[m][1] = bf16_hi(qu.x); qx[m][2] = bf16_lo(qu.y); qx[m][3] = bf16_hi(qu.y);
                } else {
                    const float4 kf = *reinterpret_cast<const float4*>(&sm.k[t][c]);
                    const float4 qf = *reinterpret_cast<const float4*>(&sm.q[t][c]);
                    kx[m][0] = kf.x; kx[m][1] = kf.y; kx[m][2] = kf.z; kx[m][3] = kf.w;
                    qx[m][0] = qf.x; qx[m][1] = qf.y; qx[m][2] = qf.z; qx[m][3] = qf.w;
                }
            }
            const float gm = sm.gam[t], be = sm.beta[t], rkt = sm.rk[t];
            float pk = 0.f;
#pragma unroll
            for (int m = 0; m < NCH; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) pk = __builtin_fmaf(S[m][e], kx[m][e], pk);
            pk = sum8(pk) * rkt;
            const float u = be * (sm.v[t][rloc] - gm * pk);
            const float cu = u * rkt;
            float pq = 0.f;
#pragma unroll
            for (int m = 0; m < NCH; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    S[m][e] = __builtin_fmaf(cu, kx[m][e], gm * S[m][e]);
                    pq = __builtin_fmaf(S[m][e], qx[m][e], pq);
                }
            pq = sum8(pq) * sm.rq[t];
            if (live && (t & 7) == sub)
                store1<O_BF16>(a.o, (((size_t)b * T + c0 + t) * Hv + h) * dv + i, pq);
        }
    }
    if (live) {
#pragma unroll
        for (int m = 0; m < NCH; ++m) store_f4<false>(a.S_out + srow + 32 * m + 4 * sub, S[m]);
    }
}

template <int DK, int CH, bool IN_BF16, bool O_BF16>
hipError_t launch_c(const PrefillArgs& a, hipStream_t s)
{
    dim3 grid((a.dv + kRows - 1) / kRows, a.Hv, a.B);
    prefill_kernel<DK, CH, IN_BF16, O_BF16><<<grid, dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

template <int DK, bool IN_BF16, bool O_BF16>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s)
{
    // f32 inputs at 64-token chunks would exceed 64 KB of LDS: stage 32 at a
    // time (the token recurrence gives the same result for any staging length)
    switch (a.chunk) {
    case 16: return launch_c<DK, 16, IN_BF16, O_BF16>(a, s);
    case 32: return launch_c<DK, 32, IN_BF16, O_BF16>(a, s);
    default:
        if constexpr (IN_BF16 || DK < 128) return launch_c<DK, 64, IN_BF16, O_BF16>(a, s);
        else return launch_c<DK, 32, IN_BF16, O_BF16>(a, s);
    }
}

template <bool IN_BF16, bool O_BF16>
hipError_t launch_io(const PrefillArgs& a, hipStream_t s)
{
    switch (a.dk) {
    case 32: return launch_d<32, IN_BF16, O_BF16>(a, s);
    case 64: return launch_d<64, IN_BF16, O_BF16>(a, s);
    case 128: return launch_d<128, IN_BF16, O_BF16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, bool o_bf16, hipStream_t s)
{
    // bf16 slabs take the chunkwise WY form on MFMA (raw bf16 q, k, v are exact
    // MFMA operands); fp32 slabs keep the fp32 token recurrence
    if (in_bf16) return launch_prefill_wy(a, o_bf16, s);
    return o_bf16 ? launch_io<false, true>(a, s) : launch_io<false, false>(a, s);
}

}  // namespace gdn
