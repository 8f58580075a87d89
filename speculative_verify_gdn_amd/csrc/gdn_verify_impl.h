// gdn_verify_impl.h -- gated delta rule over a K-token verify window with
// intermediate-state capture (gfx950): the chain as a token recurrence with
// the state in registers, the draft tree chunkwise in WY form on MFMA.
//
// The step the pages describe as a fused GDN verify that writes the final
// state and every intermediate state in one pass (atlas PR #297, commit message
// on gated_delta_rule_wy16.cu), with the raw gates applied in the kernel, q/k
// broadcast from key heads and one L2 normalisation of the q|k slab (lucebox
// PR #637, commit messages on raw-gate gated_delta_net and the DeltaNet block;
// review excerpt of gated_delta_net.cu).
//
// Chain (a window of consecutive tokens), per sequence b and value head h:
//   p = H_{t-1} k^_t,  u_t = beta_t (v_t - gamma_t p),
//   H_t = gamma_t H_{t-1} + u_t k^_t^T,  o_t = H_t q^_t,  H_{-1} = S_in.
// Every H_t is written out, so the chunkwise WY form would save no bytes here;
// the token order lets H_0 leave as soon as the window is staged, and each later
// state one row sum after its predecessor.  (Measured on the K=16 window: the
// WY form's MFMA prologue and triangular solve put the first store 1 us later,
// and the launch took 0.7 us longer.)
//
// Tree verify (the drafted tokens form a tree; lucebox PR #637, DDTree drafting
// in the commit messages), with G_t = sum of g along the root path of node t:
//   A[t][s] = beta_t e^{G_t-G_s} k^_t.k^_s        (s a strict ancestor of t)
//   M[t][s] = e^{G_t-G_s} q^_t.k^_s                (s an ancestor of t or t)
//   (I + A) u = beta (v - e^{G} S_in k^)            (one column per state row)
//   o_t = e^{G_t} S_in q^_t + sum_s M[t][s] u_s
//   H_t = e^{G_t} S_in + sum over the path of e^{G_t-G_s} u_s k^_s^T
// (I + A)^{-1} is the WY / UT transform of the tree: it turns the delta
// corrections into one triangular solve that needs S_in only through the
// contractions S_in K^T and S_in Q^T, so nodes of different branches, which
// interleave in the numbering, need no state chain.  Only exponentials of
// G_t - G_s with s an ancestor are formed (no ratio of decays).
//
// Mapping.  A workgroup is 4 waves holding RPG = 1024/DK consecutive state
// rows of one head.  A lane owns one float4 of one row (a row is DK/4 lanes),
// so one store instruction of a wave writes whole rows -- 1 KB contiguous at
// DK=128.
//   1. the raw q, k of the key head and the v values of the workgroup's rows
//      go to LDS with a few 16-byte loads per thread (branch-free, so they are
//      in flight together); the q/k norms come from the staging threads (dot
//      products and DPP row sums), the gates and their running sums from one
//      wave; each lane keeps its own state float4 in registers;
//   chain: 2. per token, the two row sums (p, o_t) are DPP sums over the row's
//      lanes; every lane streams H_t with one 16-byte store -- the bulk of the
//      bytes of the whole step -- and lane j of a row keeps o_j;
//   tree: 2. the contractions run on MFMA, one job per wave: K K^T and A (wave
//      0); Q K^T and M (wave 3); K S^T (wave 1) and Q S^T (wave 2).  Operands:
//      raw q, k in bf16 (products of bf16 are exact, accumulation is fp32)
//      against the state split into two bf16 halves (hi + lo keeps about 16
//      bits, split once while staging), 16x16x32 bf16 instructions; for f32
//      inputs 16x16x4 f32 instructions on the unsplit values;
//   tree: 3. per row: the forward substitution for u_t is shared by the row's
//      lanes (lane j owns node j, each finished u_t is broadcast with
//      v_readlane), which also gives o_t; node states stream as their u_t
//      become known.
#pragma once

#include "gdn_conv_math.h"
#include "gdn_debug.h"
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_verify_common.h"

#include <type_traits>

namespace gdn {
namespace {

template <int DK, int KP, int RPG, bool IN_BF16, bool TREE>
struct VerifySmem {
    using in_t = typename std::conditional<IN_BF16, uint16_t, float>::type;
    static constexpr int NP = RPG < 16 ? 16 : RPG;   // row tiles padded to 16
    static constexpr int QW = DK + (IN_BF16 ? 8 : 4);   // padded row: rows start 4 banks apart
    in_t q[KP][QW];                 // raw q of the key head, rows >= K zero
    in_t k[KP][QW];                 // raw k
    // S_in rows of the workgroup (rows >= RPG zero): fp32 rows for f32 inputs; for bf16
    // inputs the MFMA operands, each value split into bf16 halves hi + lo (hi = top 16
    // bits, lo = top 16 bits of the remainder), rows padded like q and k
    // (the MFMA phase's arrays exist for the tree only: the chain keeps its state in registers)
    using s_t = typename std::conditional<IN_BF16, uint16_t, float>::type;
    static constexpr int SW = IN_BF16 ? DK + 8 : DK + 4;
    static constexpr int TNP = TREE ? NP : 1, TRPG = TREE ? RPG : 1, TKP = TREE ? KP : 1;
    s_t S[TNP][SW];                 // the rows, or their hi halves
    s_t Slo[IN_BF16 ? TNP : 1][SW]; // lo halves (bf16 inputs only)
    float P[TRPG][KP + 4];          // raw k_t . S_in[row]
    float R[TRPG][KP + 4];          // raw q_t . S_in[row]
    float A[TKP][KP + 4];           // beta_t e^{G_t-G_s} k^_t.k^_s, s < t
    float M[TKP][KP + 4];           // e^{G_t-G_s} q^_t.k^_s, s <= t
    float V[KP][RPG];               // v of the workgroup's rows, per token
    float4 tok[KP];                 // per token: beta, e^{G}, 1/|k|, 1/|q|
    float gam[KP];                  // e^{g}
    float Gv[KP];                   // running sums of g (along the root path for a tree)
    // tree only (one element otherwise)
    static constexpr int TK = TREE ? KP : 1, TR = TREE ? RPG : 1;
    uint32_t anc[TK];               // strict ancestors of node t, one bit per node
    int par[TK];                    // parent of node t (-1: a root)
    float Cm[TK][KP + 4];           // e^{G_t-G_s}/|k_s| for s an ancestor of t or t itself, else 0
    float U[TR][KP + 4];            // u_s of each row, for the direct state sums
};

// D[m][n] = sum_c X[tm*16+m][c] Y[tn*16+n][c] over the DK columns.
// X, Y raw q/k rows in LDS.  Lane l feeds row l%16 of both operands with the
// same k-slice, so the product is the contraction whatever order the
// instruction assigns to the k elements inside a lane.
template <int DK, int QW, bool IN_BF16, typename in_t>
__device__ __forceinline__ f32x4_t gram_tile(const in_t (*X)[QW], const in_t (*Y)[QW], int tm, int tn, int lane)
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

// D[m][n] = sum_c X[tm*16+m][c] S[tn*16+n][c]: raw q/k rows against the state rows
// (bf16: S holds the hi halves and Sl the lo halves of the fp32 state)
template <int DK, int QW, int SW, bool IN_BF16, typename in_t, typename s_t>
__device__ __forceinline__ f32x4_t state_tile(const in_t (*X)[QW], const s_t (*S)[SW], const s_t (*Sl)[SW], int tm,
                                              int tn, int lane)
{
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const int r = lane & 15, ks = lane >> 4;
    if constexpr (IN_BF16) {
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&X[tm * 16 + r][32 * kk + 8 * ks]);
            const bf16x8_t hi = *reinterpret_cast<const bf16x8_t*>(&S[tn * 16 + r][32 * kk + 8 * ks]);
            const bf16x8_t lo = *reinterpret_cast<const bf16x8_t*>(&Sl[tn * 16 + r][32 * kk + 8 * ks]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo, acc, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < DK / 4; ++kk) {
            const float a = X[tm * 16 + r][4 * kk + ks];
            const float b = S[tn * 16 + r][4 * kk + ks];
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
    }
    return acc;
}

template <int DK, int KMAX, bool IN_BF16, bool O_BF16, bool NT, bool TREE, bool STEP, int NG = 1, bool SEL = false>
__global__ __launch_bounds__(kThreads * NG) void verify_kernel(VerifyArgs a)
{
    constexpr int LPR = DK / 4;                  // lanes per state row (one float4 each)
    constexpr int RPW = 64 / LPR;                // rows per wave
    constexpr int RPG = kWaves * RPW;            // rows per workgroup
    constexpr int TB = (KMAX + 15) / 16;         // 16-token MFMA blocks
    constexpr int KP = TB * 16;
    constexpr int NTL = (RPG + 15) / 16;         // 16-row MFMA blocks
    using Smem = VerifySmem<DK, KP, RPG, IN_BF16, TREE>;
    using in_t = typename Smem::in_t;
    // NG value heads of one key head per workgroup (fused step): group `sub` of four
    // waves owns head h and its own copy of the head's LDS; the q|k conv of the key
    // head is shared by the whole workgroup
    __shared__ Smem smg[NG];
    const int gtid = threadIdx.x, sub = gtid / kThreads;
    Smem& sm = smg[sub];
    // the raw q, k of the key head: one copy, the first group's
    in_t(&qs)[KP][Smem::QW] = smg[0].q;
    in_t(&ks)[KP][Smem::QW] = smg[0].k;

    const int tid = gtid % kThreads, lane = tid & 63, wave = tid >> 6;
    const int j = lane % LPR;                    // float4 index inside the row
    const int c = 4 * j;
    const int rloc = wave * RPW + lane / LPR;    // row inside the workgroup
    const int h = blockIdx.y * NG + sub, b = blockIdx.z;
    const int i = blockIdx.x * RPG + rloc;
    // Kb: the window of the buffers (strides); K: this sequence's tokens (masks)
    const int Kb = a.K, Hk = a.Hk, Hv = a.Hv, dv = a.dv;
    // SEL: the previous tree's accepted node is the first load (a vector load whose index is zero but
    // lane-dependent -- eps >= 0 is checked on the host -- so the loads issued after it need not wait for it;
    // the start state's address waits for it)
    int nd_raw = -1;
    if constexpr (SEL) {
        const int z0 = (int)(a.eps < 0.f) & (int)(threadIdx.x & 63);
        if (a.acc_prev) nd_raw = a.acc_prev[b + z0];
    }
    int K = a.lens ? min(max(a.lens[b], 1), Kb) : Kb;
    const int gs = a.gstride > 0 ? a.gstride : Hv;
    if (a.replay) {
        // replay of the accepted prefix from the checkpoint S_in: nothing to do when the
        // whole window was kept (S_out holds its final state), a copy when none was
        const int acc_raw = a.replay[b];
        GDN_COUNT_CLAMP(threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && (acc_raw < 0 || acc_raw > Kb));
        const int acc = min(max(acc_raw, 0), Kb);
        if (acc >= Kb) return;
        if (acc == 0) {
            const int rl = blockIdx.x * RPG + wave * RPW + lane / LPR;
            if (rl < a.dv) {
                const size_t off = (((size_t)b * Hv + h) * a.dv + rl) * DK + 4 * (lane % LPR);
                store_f4<false>(a.S_out + off, load_f4(a.S_in + off));
            }
            return;
        }
        K = acc;
    }
    const bool live = i < dv;
    const int ic = live ? i : dv - 1;            // clamped row for loads
    const int C = 2 * Hk * DK + Hv * dv;
    const int hk = h / (Hv / Hk);
    const size_t SD = (size_t)dv * DK;
    const float* Sh = a.S_in + ((size_t)b * Hv + h) * SD;
    // this sequence's rows: q|k|v, or for the fused step the raw tokens before the conv
    const in_t* X = reinterpret_cast<const in_t*>(STEP ? a.x : a.qkv) + (size_t)b * Kb * C;
    const size_t qoff = (size_t)hk * DK, koff = (size_t)(Hk + hk) * DK;
    constexpr int EPV = IN_BF16 ? 8 : 4;         // elements per 16-byte vector
    constexpr int VPR = DK / EPV;                // consecutive threads per token row
    constexpr int CW = 4;                        // conv width of the fused step
    // fused step: the start state and the W-1 history rows come from the previous
    // window, picked by its accept length a -- S_ckpt (a = 0), H[a-1], or its final
    // state (a = K_prev), and window rows a .. a+W-2 -- or from S_in and hist
    // The accept length is loaded only once every load that does not depend on it has
    // been issued (pick_start), so its round trip overlaps theirs.
    const in_t* HS = nullptr;
    // (SEL, the fused tree step: the start state is the previous tree's state at its accepted node, or its
    // start state when no node was kept, and is written out as this tree's checkpoint)
    auto pick_start = [&]() {
        if constexpr (SEL) {
            if (a.acc_prev) {
                const int nd = __builtin_amdgcn_readfirstlane(nd_raw);
                Sh = (nd >= 0 && nd < a.Kp) ? a.Sp_H + (((size_t)b * a.Kp + nd) * Hv + h) * SD
                                            : a.Sp_ckpt + ((size_t)b * Hv + h) * SD;
            } else {
                Sh = a.Sp_ckpt + ((size_t)b * Hv + h) * SD;
            }
        } else if constexpr (STEP) {
            int ap = 0;
            if (a.acc_prev) {
                const int ap_raw = a.acc_prev[b];
                GDN_COUNT_CLAMP(threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && (ap_raw < 0 || ap_raw > a.Kp));
                ap = min(max(ap_raw, 0), a.Kp);
                const size_t hb = ((size_t)b * Hv + h) * SD;
                Sh = ap == 0 ? a.Sp_ckpt + hb
                             : (ap == a.Kp ? a.Sp_out + hb : a.Sp_H + (((size_t)b * (a.Kp - 1) + ap - 1) * Hv + h) * SD);
            }
            HS = reinterpret_cast<const in_t*>(a.hsrc) + ((size_t)b * a.hrows + ap) * C;
        }
    };
    // row r of this window [W-1 history rows ; K tokens]; only rows r < W-1 depend on the
    // accept length, so rows known to be tokens take xrow_at and their loads need not wait for it
    auto wrow = [&](int r) -> const in_t* { return r < CW - 1 ? HS + (size_t)r * C : X + (size_t)(r - (CW - 1)) * C; };
    auto xrow_at = [&](int r) -> const in_t* { return X + (size_t)(r - (CW - 1)) * C; };

    f32x4_t S;
    // ---- 1. stage q, k and their norms, the state rows, v; gates and their running sums.
    // Every global load of the phase is issued first (addresses clamped into
    // range instead of branching), so they are in flight together.
    {
        static_assert(64 % VPR == 0 && (KP * VPR) % 64 == 0, "a token row is a lane group of one wave");
        constexpr int NQ = (KP * VPR + kThreads - 1) / kThreads;     // q/k pieces per thread
        constexpr int NV = (KMAX * RPG + kThreads - 1) / kThreads;   // v elements per thread
        uint4 qv[NQ], kv[NQ];
        // fused step: thread tid convolves one q|k channel of the key head over a run of
        // TPG tokens (its W-1+TPG window rows and its taps: coalesced loads, one read per
        // row); threads (t, row) convolve the v channels; the window rows this step keeps
        // for the next one are loaded here too
        constexpr int QKC = 2 * DK;                                   // q|k channels
        constexpr int TPC = kThreads * NG / QKC;                       // threads per channel
        static_assert((kThreads * NG) % QKC == 0, "whole channels per workgroup");
        constexpr int TPG = STEP ? (KP + TPC - 1) / TPC : 1;          // tokens per thread
        constexpr int NXR = STEP ? TPG + CW - 1 : 1;
        constexpr int NWV = STEP ? ((CW - 1 + KMAX) * RPG + kThreads - 1) / kThreads : 1;
        // QKC is a multiple of 64, so a wave shares its run of tokens t0 .. t0+TPG-1
        const int chi = gtid % QKC, t0 = __builtin_amdgcn_readfirstlane((gtid / QKC) * TPG);
        const size_t choff = chi < DK ? qoff + chi : koff + (chi - DK);
        uint32_t xrow[NXR];                                           // raw window rows
        float4 tp = make_float4(0.f, 0.f, 0.f, 0.f);
        uint32_t vrow[STEP ? NV : 1][CW];
        float4 vtp[STEP ? NV : 1];
        uint32_t wv[NWV];
        int par = -1;
        // the gates of group sub are formed by wave kWaves-1-sub, so that in a workgroup of
        // several groups they fall on different SIMDs.  Every lane loads the raw bits of
        // one token's gates (index clamped, no branch), and they are converted where they
        // are used, so no wave waits for them here.
        const int gwave = kWaves - 1 - sub % kWaves;
        uint32_t braw_bits, bal_bits;
        const bool raw_gates = a.dt_bias != nullptr;
        float dtb, alog;                             // the head's dt_bias and A_log (raw gates)
        {
            // (with pre-activated gates these read a word of the token rows, and are ignored)
            const float* fb = reinterpret_cast<const float*>(X);
            dtb = *(raw_gates ? a.dt_bias + h : fb);
            alog = *(raw_gates ? a.A_log + h : fb);
            const size_t gi = ((size_t)b * Kb + (lane < K ? lane : K - 1)) * gs + h;
            if constexpr (IN_BF16) {
                braw_bits = reinterpret_cast<const uint16_t*>(a.beta_raw)[gi];
                bal_bits = reinterpret_cast<const uint16_t*>(a.alpha)[gi];
            } else {
                braw_bits = reinterpret_cast<const uint32_t*>(a.beta_raw)[gi];
                bal_bits = reinterpret_cast<const uint32_t*>(a.alpha)[gi];
            }
            if constexpr (TREE) {
                if (wave == gwave && lane < K) par = a.parent[(size_t)b * Kb + lane];
            }
        }
        // the gates of every token and their running sums (the last wave): they need only
        // the gate loads, so the fused step forms them before its conv, in the wait for the rows
        auto do_gates = [&]() {
            if (wave == gwave) {
                // lane t: gates of token t, then G_t = g_0 + ... + g_t by a scan over the lanes
                float be = 0.f, g = 0.f;
                const float braw = __uint_as_float(IN_BF16 ? braw_bits << 16 : braw_bits);
                const float bal = __uint_as_float(IN_BF16 ? bal_bits << 16 : bal_bits);
                if (lane < K) gate(braw, bal, raw_gates, dtb, alog, be, g);
                float G;
                if constexpr (TREE) {
                    // G_t = sum of g over the root path of node t, and its strict ancestors, by
                    // pointer jumping: after round r, G covers the 2^r nearest nodes of the path
                    // (t included) and nxt is the next node above them (-1 past the root)
                    int nxt = (lane < K && par >= 0 && par < lane) ? par : -1;
                    uint32_t anc = nxt >= 0 ? 1u << nxt : 0u;
                    if (lane < KP) sm.par[lane] = nxt;
                    G = g;
    #pragma unroll
                    for (int r = 1; r < KP; r *= 2) {
                        const int src = nxt >= 0 ? nxt : lane;
                        const float Gn = __shfl(G, src, 64);
                        const uint32_t an = (uint32_t)__shfl((int)anc, src, 64);
                        const int nn = __shfl(nxt, src, 64);
                        if (nxt >= 0) {
                            G += Gn;
                            anc |= an;
                            nxt = nn;
                        }
                    }
                    if (lane < KP) sm.anc[lane] = anc;
                } else {
                    G = lane_scan<KP>(g);
                }
                if (lane < KP) {
                    sm.Gv[lane] = G;
                    sm.tok[lane].x = be;
                    sm.tok[lane].y = __expf(G);
                    sm.gam[lane] = __expf(g);
                }
            }
        };
        if constexpr (STEP) {
            // in issue order: first every load that does not depend on the accept length
            // (taps, token rows), then the history rows it selects
            tp = *reinterpret_cast<const float4*>(a.w + choff * CW);
#pragma unroll
            for (int m = CW - 1; m < NXR; ++m) {
                const int r = t0 + m < CW - 2 + K ? t0 + m : CW - 2 + K;
                xrow[m] = ldraw<IN_BF16>(xrow_at(r), choff);
            }
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                const int idx = tid + n * kThreads;
                const int t = idx / RPG, rr = idx % RPG;
                const int gr = blockIdx.x * RPG + rr;
                const size_t vch = 2 * (size_t)Hk * DK + (size_t)h * dv + (gr < dv ? gr : dv - 1);
                const int tc = t < K ? t : K - 1;
                vtp[n] = *reinterpret_cast<const float4*>(a.w + vch * CW);
                vrow[n][CW - 1] = ldraw<IN_BF16>(xrow_at(tc + CW - 1), vch);
            }
            // then the accept length, the start state it picks and the window rows that
            // depend on it (the history rows; for runs past them, token rows again)
            pick_start();
#pragma unroll
            for (int m = 0; m < CW - 1; ++m) {
                const int r = t0 + m < CW - 2 + K ? t0 + m : CW - 2 + K;
                xrow[m] = ldraw<IN_BF16>(wrow(r), choff);
            }
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                const int idx = tid + n * kThreads;
                const int t = idx / RPG, rr = idx % RPG;
                const int gr = blockIdx.x * RPG + rr;
                const size_t vch = 2 * (size_t)Hk * DK + (size_t)h * dv + (gr < dv ? gr : dv - 1);
                const int tc = t < K ? t : K - 1;
#pragma unroll
                for (int jj = 0; jj < CW - 1; ++jj) vrow[n][jj] = ldraw<IN_BF16>(wrow(tc + jj), vch);
            }
#pragma unroll
            for (int n = 0; n < NWV; ++n) {
                const int idx = tid + n * kThreads;
                const int r = idx / RPG, gr = blockIdx.x * RPG + idx % RPG;
                const size_t vch = 2 * (size_t)Hk * DK + (size_t)h * dv + (gr < dv ? gr : dv - 1);
                wv[n] = ldraw<IN_BF16>(wrow(r < CW - 2 + K ? r : CW - 2 + K), vch);
            }
        } else {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const int idx = tid + n * kThreads;
                if (idx < KP * VPR) {
                    const int t = idx / VPR, cc = (idx % VPR) * EPV;
                    const in_t* row = X + (size_t)(t < K ? t : K - 1) * C;
                    qv[n] = *reinterpret_cast<const uint4*>(row + qoff + cc);
                    kv[n] = *reinterpret_cast<const uint4*>(row + koff + cc);
                }
            }
        }
        float vv[NV];
        auto load_v = [&]() {
            if constexpr (!STEP) {
#pragma unroll
                for (int n = 0; n < NV; ++n) {
                    const int idx = tid + n * kThreads;
                    const int t = idx / RPG, rr = idx % RPG;
                    const int gr = blockIdx.x * RPG + rr;
                    const size_t vch = 2 * (size_t)Hk * DK + (size_t)h * dv + (gr < dv ? gr : dv - 1);
                    vv[n] = idx < KMAX * RPG ? load1<IN_BF16>(X + (size_t)(t < K ? t : K - 1) * C, vch) : 0.f;
                }
            }
        };
        // SEL: the v loads go before the accepted node, whose value the start state's address waits for
        if constexpr (SEL) {
            load_v();
            pick_start();
        }
        f32x4_t S0 = load_f4(Sh + (size_t)ic * DK + c);
        if constexpr (!SEL) load_v();
        if constexpr (STEP) {
            do_gates();
            // the conv, as the conv kernels compute it; the conv outputs and the window
            // rows are written by one workgroup per key head (q, k) and by each
            // workgroup for its own rows (v).  The tokens whose rows are all token rows
            // come first, so the history rows picked by the accept length arrive meanwhile.
            const bool qk_writer = ((blockIdx.y * NG) % (Hv / Hk)) == 0 && blockIdx.x == 0;
            const int cl = chi < DK ? chi : chi - DK;
            const float tap[CW] = {tp.x, tp.y, tp.z, tp.w};
#pragma unroll
            for (int mm = 0; mm < TPG; ++mm) {
                const int m = (mm + CW - 1) % TPG;   // a rotation of 0 .. TPG-1
                const int t = t0 + m;
                if (t < KP) {
                    const float col[CW] = {rawf<IN_BF16>(xrow[m]), rawf<IN_BF16>(xrow[m + 1]), rawf<IN_BF16>(xrow[m + 2]),
                                           rawf<IN_BF16>(xrow[m + 3])};
                    if constexpr (IN_BF16) {
                        const uint16_t hb = t < K ? conv_silu_bf16(conv_pre<CW>(tap, col)) : (uint16_t)0;
                        (chi < DK ? qs : ks)[t][cl] = hb;
                        if (a.y && qk_writer && t < K)
                            reinterpret_cast<uint16_t*>(a.y)[((size_t)b * Kb + t) * C + choff] = hb;
                    } else {
                        const float v = t < K ? conv_silu(conv_pre<CW>(tap, col)) : 0.f;
                        (chi < DK ? qs : ks)[t][cl] = v;
                        if (a.y && qk_writer && t < K) reinterpret_cast<float*>(a.y)[((size_t)b * Kb + t) * C + choff] = v;
                    }
                }
            }
            // the checkpoint: this window's start state
            if (a.S_ckpt && live) store_f4<true>(a.S_ckpt + ((size_t)b * Hv + h) * SD + (size_t)i * DK + c, S0);
            in_t* Wb = a.win ? reinterpret_cast<in_t*>(a.win) + (size_t)b * (CW - 1 + Kb) * C : nullptr;
            if (Wb && qk_writer) {
                // rows t0+W-1 .. t0+TPG+W-2 (the newest of each token), and the history rows for t0 = 0
#pragma unroll
                for (int m = 0; m < NXR; ++m) {
                    const int r = t0 + m;
                    if ((m >= CW - 1 || t0 == 0) && r < CW - 1 + K) straw<IN_BF16>(Wb, (size_t)r * C + choff, xrow[m]);
                }
            }
            if (Wb) {
#pragma unroll
                for (int n = 0; n < NWV; ++n) {
                    const int idx = tid + n * kThreads;
                    const int r = idx / RPG, gr = blockIdx.x * RPG + idx % RPG;
                    if (idx < (CW - 1 + KMAX) * RPG && r < CW - 1 + K && gr < dv)
                        straw<IN_BF16>(Wb, (size_t)r * C + 2 * (size_t)Hk * DK + (size_t)h * dv + gr, wv[n]);
                }
            }
#pragma unroll
            for (int n = 0; n < NV; ++n) {
                const int idx = tid + n * kThreads;
                const int t = idx / RPG, rr = idx % RPG;
                const int gr = blockIdx.x * RPG + rr;
                const float tv[CW] = {vtp[n].x, vtp[n].y, vtp[n].z, vtp[n].w};
                float vc[CW];
#pragma unroll
                for (int jj = 0; jj < CW; ++jj) vc[jj] = rawf<IN_BF16>(vrow[n][jj]);
                float v;
                if constexpr (IN_BF16) v = bf16_to_f32(conv_silu_bf16(conv_pre<CW>(tv, vc)));
                else v = conv_silu(conv_pre<CW>(tv, vc));
                vv[n] = idx < KMAX * RPG ? v : 0.f;
                if (a.y && idx < KMAX * RPG && t < K && gr < dv)
                    store1<IN_BF16>(a.y, ((size_t)b * Kb + t) * C + 2 * (size_t)Hk * DK + (size_t)h * dv + gr, v);
            }
            __syncthreads();  // q, k of every token in LDS
            // their norms, as the staging threads of the plain verify form them
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const int idx = tid + n * kThreads;
                if (idx < KP * VPR) {
                    const int t = idx / VPR, cc = (idx % VPR) * EPV;
                    const float sq = group_sum<VPR>(sumsq16<IN_BF16>(*reinterpret_cast<const uint4*>(&qs[t][cc])));
                    const float sk = group_sum<VPR>(sumsq16<IN_BF16>(*reinterpret_cast<const uint4*>(&ks[t][cc])));
                    if (cc == 0) {
                        sm.tok[t].z = t < K ? __builtin_amdgcn_rsqf(sk + a.eps) : 0.0f;
                        sm.tok[t].w = t < K ? __builtin_amdgcn_rsqf(sq + a.eps) : 0.0f;
                    }
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const int idx = tid + n * kThreads;
                if (idx < KP * VPR) {
                    const int t = idx / VPR, cc = (idx % VPR) * EPV;
                    if (t >= K) qv[n] = kv[n] = make_uint4(0, 0, 0, 0);
                    *reinterpret_cast<uint4*>(&qs[t][cc]) = qv[n];
                    *reinterpret_cast<uint4*>(&ks[t][cc]) = kv[n];
                    // 1/|q_t|, 1/|k_t| (padded tokens keep q^ = k^ = 0, never 0 * 1/sqrt(0))
                    const float sq = group_sum<VPR>(sumsq16<IN_BF16>(qv[n]));
                    const float sk = group_sum<VPR>(sumsq16<IN_BF16>(kv[n]));
                    if (cc == 0) {
                        sm.tok[t].z = t < K ? __builtin_amdgcn_rsqf(sk + a.eps) : 0.0f;
                        sm.tok[t].w = t < K ? __builtin_amdgcn_rsqf(sq + a.eps) : 0.0f;
                    }
                }
            }
        }
        if constexpr (SEL) {
            // the checkpoint: this tree's start state
            if (a.S_ckpt && live) store_f4<true>(a.S_ckpt + ((size_t)b * Hv + h) * SD + (size_t)i * DK + c, S0);
        }
        if (!live) S0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        S = S0;
        if constexpr (!TREE) {
            // the chain path keeps the state in registers only
        } else if constexpr (IN_BF16) {
            // the MFMA operands of this lane's four values: bf16 halves
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t u0 = __float_as_uint(S0[2 * e]), u1 = __float_as_uint(S0[2 * e + 1]);
                const uint32_t h0 = u0 & 0xffff0000u, h1 = u1 & 0xffff0000u;
                const uint32_t l0 = __float_as_uint(S0[2 * e] - __uint_as_float(h0)) >> 16;
                const uint32_t l1 = __float_as_uint(S0[2 * e + 1] - __uint_as_float(h1)) & 0xffff0000u;
                hw[e] = (h0 >> 16) | h1;
                lw[e] = l0 | l1;
            }
            *reinterpret_cast<uint2*>(&sm.S[rloc][c]) = make_uint2(hw[0], hw[1]);
            *reinterpret_cast<uint2*>(&sm.Slo[rloc][c]) = make_uint2(lw[0], lw[1]);
        } else {
            *reinterpret_cast<f32x4_t*>(&sm.S[rloc][c]) = S0;
        }
        if constexpr (TREE && RPG < 16) {
            for (int idx = tid; idx < (16 - RPG) * LPR; idx += kThreads) {
                const int rr = RPG + idx / LPR, cc = 4 * (idx % LPR);
                if constexpr (IN_BF16) {
                    *reinterpret_cast<uint2*>(&sm.S[rr][cc]) = make_uint2(0, 0);
                    *reinterpret_cast<uint2*>(&sm.Slo[rr][cc]) = make_uint2(0, 0);
                } else {
                    *reinterpret_cast<f32x4_t*>(&sm.S[rr][cc]) = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int idx = tid + n * kThreads;
            if (idx < KMAX * RPG) sm.V[idx / RPG][idx % RPG] = vv[n];
        }
        if constexpr (!STEP) do_gates();
    }
    __syncthreads();

    if constexpr (!TREE) {
        // ---- 2. the chain: the token recurrence, state in registers.  Every state is
        // written out, so the WY form would save no bytes here, and the token order lets
        // H_0 leave as soon as phase 1 is done.  Per token, with the row sums over the
        // row's lanes (DPP):
        //   p = S k^_t,  u = beta_t (v_t - gamma_t p),  S = gamma_t S + u k^_t,  o_t = S q^_t
        float* Hrow = a.H ? a.H + ((size_t)b * (Kb - 1) * Hv + h) * SD + (size_t)i * DK + c : nullptr;
        const size_t Hstep = (size_t)Hv * SD;
        constexpr int NO = (KMAX + LPR - 1) / LPR;   // outputs held per lane: lane j keeps o_{j + m LPR}
        float ot[NO];
#pragma unroll
        for (int m = 0; m < NO; ++m) ot[m] = 0.f;
#pragma unroll
        for (int t = 0; t < KMAX; ++t) {
            if (t < K) {
                const float4 tt = sm.tok[t];          // beta, e^{G}, 1/|k|, 1/|q|
                const float gm = sm.gam[t];
                const float4 kx = lds4<IN_BF16>(&ks[t][c]);
                const float v = sm.V[t][rloc];
                const float sk = group_sum<LPR>(S[0] * kx.x + S[1] * kx.y + S[2] * kx.z + S[3] * kx.w) * tt.z;
                const float cu = tt.x * (v - gm * sk) * tt.z;   // u / |k_t|
                S[0] = __builtin_fmaf(cu, kx.x, gm * S[0]);
                S[1] = __builtin_fmaf(cu, kx.y, gm * S[1]);
                S[2] = __builtin_fmaf(cu, kx.z, gm * S[2]);
                S[3] = __builtin_fmaf(cu, kx.w, gm * S[3]);
                if (live) {
                    if (t < K - 1) {
                        if (Hrow) store_f4<NT>(Hrow + (size_t)t * Hstep, S);
                    } else {
                        store_f4<NT>(a.S_out + ((size_t)b * Hv + h) * SD + (size_t)i * DK + c, S);
                    }
                }
                if (a.o) {
                    const float4 qx = lds4<IN_BF16>(&qs[t][c]);
                    const float o = group_sum<LPR>(S[0] * qx.x + S[1] * qx.y + S[2] * qx.z + S[3] * qx.w) * tt.w;
                    if (j == t % LPR) ot[t / LPR] = o;
                }
            }
        }
        if (a.o && live) {
#pragma unroll
            for (int m = 0; m < NO; ++m) {
                const int t = m * LPR + j;
                if (t < K) store1<O_BF16>(a.o, (((size_t)b * Kb + t) * Hv + h) * dv + i, ot[m]);
            }
        }
        return;
    } else {

    // ---- 2. contractions on MFMA (tree)
    // wave 0: K K^T -> A
    // wave 3: Q K^T -> M
    // waves 1, 2: K S^T, Q S^T
    const int n16 = lane & 15, m0 = (lane >> 4) * 4;   // 16x16 result layout: row m0+e, column n16
    if (wave == 0 || wave == 3) {
        const bool wa = wave == 0;
#pragma unroll
        for (int tm = 0; tm < TB; ++tm)
#pragma unroll
            for (int tn = 0; tn < TB; ++tn) {
                const int s2 = tn * 16 + n16;
                if (tn > tm) {
                    // tiles above the diagonal are zero
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (wa) sm.A[tm * 16 + m0 + e][s2] = 0.f;
                        else sm.M[tm * 16 + m0 + e][s2] = 0.f;
                    }
                    continue;
                }
                const f32x4_t d = wa ? gram_tile<DK, Smem::QW, IN_BF16, in_t>(ks, ks, tm, tn, lane)
                                     : gram_tile<DK, Smem::QW, IN_BF16, in_t>(qs, ks, tm, tn, lane);
                const float Gs = sm.Gv[s2], rks = sm.tok[s2].z;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = tm * 16 + m0 + e;
                    const float4 tt = sm.tok[t];
                    const float dec = __expf(fminf(sm.Gv[t] - Gs, 0.f));
                    // s2 is an earlier token of the chain, or an ancestor of node t in a tree
                    const bool before = TREE ? ((sm.anc[t] >> s2) & 1u) != 0 : s2 < t;
                    if (wa) {
                        sm.A[t][s2] = before ? tt.x * tt.z * rks * dec * d[e] : 0.f;
                    } else {
                        sm.M[t][s2] = (before || s2 == t) ? tt.w * rks * dec * d[e] : 0.f;
                        if constexpr (TREE) sm.Cm[t][s2] = (before || s2 == t) ? rks * dec : 0.f;
                    }
                }
            }
    } else {
        // raw K S^T (wave 1) or Q S^T (wave 2), stored per state row
        const in_t(*Xs)[Smem::QW] = wave == 1 ? ks : qs;
        float(*D)[KP + 4] = wave == 1 ? sm.P : sm.R;
#pragma unroll
        for (int tm = 0; tm < TB; ++tm)
#pragma unroll
            for (int tn = 0; tn < NTL; ++tn) {
                const f32x4_t d = state_tile<DK, Smem::QW, Smem::SW, IN_BF16, in_t, typename Smem::s_t>(
                    Xs, sm.S, sm.Slo, tm, tn, lane);
                const int row = tn * 16 + n16;
                if (row < RPG) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) D[row][tm * 16 + m0 + e] = d[e];
                }
            }
    }
    __syncthreads();

    // ---- 3. u = (I + A)^{-1} b with b_t = beta_t (v_t - e^{G_t} S_in k^_t), o_t, and the
    // stream of the states H_t = gamma_t H_{t-1} + (u_t / |k_t|) k_t.  A state leaves as
    // soon as its u_t is known, so the stores of the first tokens overlap the rest of
    // the substitution.
    // H holds K-1 states per sequence for a chain (the last one goes to S_out), K for a tree
    float* Hrow = a.H ? a.H + ((size_t)b * (TREE ? Kb : Kb - 1) * Hv + h) * SD + (size_t)i * DK + c : nullptr;
    const size_t Hstep = (size_t)Hv * SD;
    // a tree node's state.  When its parent is one of the four nodes before it (or a root),
    // from the parent's state kept in registers: H_t = gamma_t H_parent + u_t k^_t (slot
    // t mod 4 of hc holds H_t; t is a constant of the unrolled token loop, so the slots are
    // registers); otherwise directly from S_in (kept in S) and the u_s of its path:
    //   H_t = e^{G_t} S_in + sum_{s on the path, s <= t} e^{G_t-G_s} u_s k^_s
    // The parent and the ancestor mask are the same over the workgroup, so every branch
    // here is uniform.
    f32x4_t hc[4];
    auto stream_node = [&](int t, float ut) {
        const int p = __builtin_amdgcn_readfirstlane(sm.par[t]);
        f32x4_t Ht;
        const int back = t - 1 - p;               // 0..3: the parent is in slot (t-1-back) mod 4
        if (p < 0 || back < 4) {
            f32x4_t base = S;
            if (p >= 0) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (back == q && t - 1 - q >= 0) base = hc[(t - 1 - q) & 3];
            }
            const float gm = sm.gam[t];
            const float cu = ut * sm.tok[t].z;
            const float4 kx = lds4<IN_BF16>(&ks[t][c]);
            Ht[0] = __builtin_fmaf(cu, kx.x, gm * base[0]);
            Ht[1] = __builtin_fmaf(cu, kx.y, gm * base[1]);
            Ht[2] = __builtin_fmaf(cu, kx.z, gm * base[2]);
            Ht[3] = __builtin_fmaf(cu, kx.w, gm * base[3]);
        } else {
            uint32_t m = __builtin_amdgcn_readfirstlane(sm.anc[t]) | (1u << t);
            const float eG = sm.tok[t].y;
            Ht = f32x4_t{eG * S[0], eG * S[1], eG * S[2], eG * S[3]};
            while (m) {
                const int s = __builtin_ctz(m);
                m &= m - 1;
                const float cf = sm.Cm[t][s] * sm.U[rloc][s];
                const float4 kx = lds4<IN_BF16>(&ks[s][c]);
                Ht[0] = __builtin_fmaf(cf, kx.x, Ht[0]);
                Ht[1] = __builtin_fmaf(cf, kx.y, Ht[1]);
                Ht[2] = __builtin_fmaf(cf, kx.z, Ht[2]);
                Ht[3] = __builtin_fmaf(cf, kx.w, Ht[3]);
            }
        }
        hc[t & 3] = Ht;
        if (live && t < K) store_f4<NT>(Hrow + (size_t)t * Hstep, Ht);
    };
    if constexpr (KMAX <= LPR) {
        // Lane j of a row owns token j: it forms b_j, keeps row j of A and of M in
        // registers, and at step t the owner of token t has its u_t final; every
        // lane reads it with v_readlane (per row of the wave), updates its own
        // partial sum and streams H_t.
        const int tj = j < KMAX ? j : KMAX - 1;  // this lane's token (clamped; lanes past K carry zeros)
        const bool own = j < K;
        const float4 tt = sm.tok[tj];            // beta, e^{G}, 1/|k|, 1/|q|
        float part = own ? tt.x * (sm.V[tj][rloc] - tt.y * (sm.P[rloc][tj] * tt.z)) : 0.f;
        float arow[KMAX], mrow[KMAX];
#pragma unroll
        for (int s4 = 0; s4 < KMAX; s4 += 4) {
            if (s4 + 4 <= KMAX) {
                const float4 a4 = *reinterpret_cast<const float4*>(&sm.A[tj][s4]);
                const float4 m4 = *reinterpret_cast<const float4*>(&sm.M[tj][s4]);
                arow[s4] = a4.x; arow[s4 + 1] = a4.y; arow[s4 + 2] = a4.z; arow[s4 + 3] = a4.w;
                mrow[s4] = m4.x; mrow[s4 + 1] = m4.y; mrow[s4 + 2] = m4.z; mrow[s4 + 3] = m4.w;
            } else {
#pragma unroll
                for (int e = 0; e < KMAX - s4; ++e) { arow[s4 + e] = sm.A[tj][s4 + e]; mrow[s4 + e] = sm.M[tj][s4 + e]; }
            }
        }
        const int wr = lane / LPR;               // row of this lane inside the wave
        float ot = own ? tt.y * (sm.R[rloc][tj] * tt.w) : 0.f;
#pragma unroll
        for (int t = 0; t < KMAX; ++t) {
            float mine = 0.f;
#pragma unroll
            for (int r2 = 0; r2 < RPW; ++r2) {
                const float ur = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(part), r2 * LPR + t));
                if (r2 == wr) mine = ur;
            }
            // A[j][t] = 0 for t >= j, so finished lanes keep their value
            part = __builtin_fmaf(-arow[t], mine, part);
            ot = __builtin_fmaf(mrow[t], mine, ot);  // M[j][t] = 0 for t > j
            // one lane per row publishes u_t; the row's lanes read it back in program
            // order (same wave), so no barrier is needed
            if (j == 0) sm.U[rloc][t] = mine;
            stream_node(t, mine);
        }
        if (own && live && a.o) store1<O_BF16>(a.o, (((size_t)b * Kb + j) * Hv + h) * dv + i, ot);
    } else {
        // more tokens than lanes per row: every lane solves its row's system
        float u[KMAX];
#pragma unroll
        for (int t = 0; t < KMAX; ++t) {
            const float4 tt = sm.tok[t];
            float acc = tt.x * (sm.V[t][rloc] - tt.y * (sm.P[rloc][t] * tt.z));
#pragma unroll
            for (int s2 = 0; s2 < t; ++s2) acc = __builtin_fmaf(-sm.A[t][s2], u[s2], acc);
            u[t] = acc;
        }
#pragma unroll
        for (int t0 = 0; t0 < KMAX; t0 += LPR) {
            const int t = t0 + j;
            if (t < K && live && a.o) {
                const float4 tt = sm.tok[t];
                float ot = tt.y * (sm.R[rloc][t] * tt.w);
#pragma unroll
                for (int s2 = 0; s2 < KMAX; ++s2) ot = __builtin_fmaf(sm.M[t][s2], u[s2], ot);
                store1<O_BF16>(a.o, (((size_t)b * Kb + t) * Hv + h) * dv + i, ot);
            }
        }
        if (j == 0) {
#pragma unroll
            for (int t = 0; t < KMAX; ++t) sm.U[rloc][t] = u[t];
        }
#pragma unroll
        for (int t = 0; t < KMAX; ++t) stream_node(t, u[t]);
    }
    }  // tree
}

// One token (K = 1: a decode step) needs no solve, no LDS and no barrier.  A lane
// owns one float4 of one state row (a row is DK/4 lanes of one wave); the q/k norms
// and the contractions are sums over the row's lanes (DPP):
//   u = beta (v - gamma S k^),   S' = gamma S + u k^^T,   o = S' q^
// The same recurrence as the window kernel's first token, with the norms summed in
// another order.
template <int DK, bool IN_BF16, bool O_BF16>
__global__ __launch_bounds__(kThreads) void decode_kernel(VerifyArgs a)
{
    constexpr int LPR = DK / 4, RPW = 64 / LPR, RPG = kWaves * RPW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = 4 * (lane % LPR);
    const int h = blockIdx.y, b = blockIdx.z;
    const int i = blockIdx.x * RPG + wave * RPW + lane / LPR;
    const int Hk = a.Hk, Hv = a.Hv, dv = a.dv;
    const bool live = i < dv;
    const int ic = live ? i : dv - 1;
    const size_t C = 2 * (size_t)Hk * DK + (size_t)Hv * dv;
    const int hk = h / (Hv / Hk);
    const size_t SD = (size_t)dv * DK;
    const size_t xb = (size_t)b * C;                 // the token's row (K = 1)
    const size_t gi = (size_t)b * (a.gstride > 0 ? a.gstride : Hv) + h;
    const size_t so = ((size_t)b * Hv + h) * SD + (size_t)ic * DK + c;
    // the head's dt_bias and A_log with the other loads (no branch: with pre-activated gates a
    // word of the token row is read instead and ignored), so the gates wait for one round trip.
    // The index is zero (the host rejects a negative eps) but depends on the lane, so these are
    // vector loads issued here rather than scalar loads placed next to their first use.
    const bool raw_gates = a.dt_bias != nullptr;
    const float* fb = reinterpret_cast<const float*>(a.qkv);
    const int z0 = (int)(a.eps < 0.f) & (int)(threadIdx.x & 63);
    const float dtb = (raw_gates ? a.dt_bias + h : fb)[z0];
    const float alog = (raw_gates ? a.A_log + h : fb)[z0];
    const float4 qx = load4<IN_BF16>(a.qkv, xb + (size_t)hk * DK + c);
    const float4 kx = load4<IN_BF16>(a.qkv, xb + (size_t)(Hk + hk) * DK + c);
    const float v = load1<IN_BF16>(a.qkv, xb + 2 * (size_t)Hk * DK + (size_t)h * dv + ic);
    const f32x4_t S = load_f4(a.S_in + so);
    const float braw = load1<IN_BF16>(a.beta_raw, gi), bal = load1<IN_BF16>(a.alpha, gi);
    float beta, g;
    gate(braw, bal, raw_gates, dtb, alog, beta, g);
    const float gm = __expf(g);
    const float rk = __builtin_amdgcn_rsqf(
        group_sum<LPR>(kx.x * kx.x + kx.y * kx.y + kx.z * kx.z + kx.w * kx.w) + a.eps);
    const float rq = __builtin_amdgcn_rsqf(
        group_sum<LPR>(qx.x * qx.x + qx.y * qx.y + qx.z * qx.z + qx.w * qx.w) + a.eps);
    const float sk = group_sum<LPR>(S[0] * kx.x + S[1] * kx.y + S[2] * kx.z + S[3] * kx.w) * rk;
    const float cu = beta * (v - gm * sk) * rk;      // u / |k|
    f32x4_t Sn;
    Sn[0] = __builtin_fmaf(cu, kx.x, gm * S[0]);
    Sn[1] = __builtin_fmaf(cu, kx.y, gm * S[1]);
    Sn[2] = __builtin_fmaf(cu, kx.z, gm * S[2]);
    Sn[3] = __builtin_fmaf(cu, kx.w, gm * S[3]);
    const float o = group_sum<LPR>(Sn[0] * qx.x + Sn[1] * qx.y + Sn[2] * qx.z + Sn[3] * qx.w) * rq;
    if (live) {
        store_f4<false>(a.S_out + so, Sn);
        if (a.o && c == 0) store1<O_BF16>(a.o, ((size_t)b * Hv + h) * dv + i, o);
    }
}

template <int DK, int KMAX, bool IN_BF16, bool O_BF16>
hipError_t launch_k(const VerifyArgs& a, hipStream_t s)
{
    constexpr int RPG = 1024 / DK;
    dim3 grid((a.dv + RPG - 1) / RPG, a.Hv, a.B);
    if (a.parent) {
        // (the tree calls take at most kTreeMax nodes: their ancestor masks are 32-bit words)
        if constexpr (KMAX <= kTreeMax) {
            if (a.pick)   // the fused tree step: start state picked by the previous tree's accepted node
                verify_kernel<DK, KMAX, IN_BF16, O_BF16, true, true, false, 1, true><<<grid, dim3(kThreads), 0, s>>>(a);
            else
                verify_kernel<DK, KMAX, IN_BF16, O_BF16, true, true, false><<<grid, dim3(kThreads), 0, s>>>(a);
        } else {
            return hipErrorInvalidValue;
        }
    } else if (a.x) {
        // the fused step: three value heads per workgroup when the heads come in groups of
        // three and three copies of the head's LDS fit in a CU
        using Sm = VerifySmem<DK, (KMAX + 15) / 16 * 16, RPG, IN_BF16, false>;
        constexpr bool kFit3 = 3 * sizeof(Sm) <= 160 * 1024;
        bool three = false;
        if constexpr (kFit3) three = (a.Hv / a.Hk) % 3 == 0;
        if (three) {
            grid.y = a.Hv / 3;
            if constexpr (kFit3)
                verify_kernel<DK, KMAX, IN_BF16, O_BF16, true, false, true, 3><<<grid, dim3(3 * kThreads), 0, s>>>(a);
        } else {
            verify_kernel<DK, KMAX, IN_BF16, O_BF16, true, false, true, 1><<<grid, dim3(kThreads), 0, s>>>(a);
        }
    } else if (KMAX == 1 && a.K == 1 && !a.replay) {
        decode_kernel<DK, IN_BF16, O_BF16><<<grid, dim3(kThreads), 0, s>>>(a);
    } else {
        verify_kernel<DK, KMAX, IN_BF16, O_BF16, true, false, false><<<grid, dim3(kThreads), 0, s>>>(a);
    }
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
    if (a.K <= 32) return launch_k<DK, 32, IN_BF16, O_BF16>(a, s);
    static_assert(kVerifyMax == 64, "one instance per power of two up to the longest window");
    return launch_k<DK, 64, IN_BF16, O_BF16>(a, s);
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

}  // namespace gdn
