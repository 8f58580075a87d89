// gdn_prefill_wy.hip -- chunked prefill in the chunkwise WY form on MFMA
// (bf16 q|k|v slab).
//
// Per chunk of L tokens and value head (G_t = running sum of the gates g from
// the chunk start, k^ = rk k and q^ = rq q the L2-normalised raw vectors,
// S the state at the chunk start):
//   A[t][s] = beta_t e^{G_t-G_s} k^_t.k^_s          (s < t)
//   (I + A) U = beta (V - e^{G} (S K^^T)^T)          U, V: L x dv
//   O[t]    = e^{G_t} S q^_t + sum_{s<=t} e^{G_t-G_s} (q^_t.k^_s) u_s
//   S'      = e^{G_L} S + sum_s e^{G_L-G_s} u_s k^_s^T
// This is the UT/WY evaluation of the gated delta rule: the same values as
// the token recurrence up to rounding (Gated Delta Networks, Yang, Kautz and
// Hatamizadeh, ICLR 2025: section 3.3, hardware-efficient chunkwise
// training; atlas PR #297 "dflash scheduler/server verify-step glue": commit
// message on the fused WY-chunkwise gated_delta_rule kernel).
//
// Workgroup: 12 waves for up to 128 state rows of one (sequence, value head)
// -- the whole head at d = 128, one workgroup per CU.  The work of a chunk
// splits into a part that needs the state and a part that does not, and two
// groups of waves run them on consecutive chunks at once:
//   state waves (8): each owns 16 state rows for the whole prompt, kept in
//     registers as the MFMA accumulator tiles of S^T (lane <-> state row, 4 key
//     columns per tile).  For chunk c: P = K S^T and R = Q S^T with the state
//     split into bf16 hi + lo, the right-hand sides beta (v - e^G rk P) and the
//     state part of O; then block forward substitution for U (its 16 columns),
//     O += M U, and S^T <- e^{G_L} S^T + K^T diag(e^{G_L-G} rk) U per 32 tokens.
//   prep waves (4): for chunk c+1, meanwhile: stage q, k (raw bf16) in MFMA
//     operand order and K^T for the state update; norms by DPP row sums; gates,
//     their running sum and decay factors; the K K^T and K Q^T tiles scaled to
//     -A and M (bf16 hi/lo pairs); the diagonal blocks of A inverted by forward
//     substitution, one lane per column.
// The chunk operands live in two LDS buffers (chunk c read by the state waves,
// chunk c+1 written by the prep waves); two barriers per chunk separate the
// phases: [state: P, R, X | prep: stage c+1] [state: solve, O, S | prep: grams
// and inverses of c+1].  The v values go straight from memory into the state
// waves' registers, a chunk ahead.
// fp32 operands enter the MFMA as a bf16 hi + lo pair (about 16 bits); a
// product of two such operands keeps the three largest partial products.
//
// Heads are mapped to workgroups so that the value heads of one key head run
// on one XCD (workgroup i goes to XCD i mod 8): they read the same q and k,
// which then come from that XCD's L2 instead of three times from HBM.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_timeline.h"
#include "gdn_wy_mfma.h"

namespace gdn {
namespace {

using namespace wy;

constexpr int kStateWaves = 8;                           // waves holding state rows (16 each)
constexpr int kPrepWaves = 4;                            // waves preparing the next chunk
constexpr int kThreads = 64 * (kStateWaves + kPrepWaves);
constexpr int kPrepThreads = 64 * kPrepWaves;
constexpr int kRows = 16 * kStateWaves;                  // state rows per workgroup

template <int DK, int L>
struct WyShape {
    static constexpr int NT = L / 16;             // 16-token tiles of a chunk
    static constexpr int NS = (NT + 1) / 2;       // 32-token slices
    static constexpr int NJ = DK / 32;            // 32-wide slices of the key dimension
    static constexpr int JT = DK / 16;            // 16-wide tiles of the key dimension
    static constexpr int NA = NT * (NT - 1) / 2;  // strictly lower 16x16 tiles
    static constexpr int NM = NT * (NT + 1) / 2;  // lower 16x16 tiles with the diagonal
    static constexpr int NO = NA + NM;            // gram tiles besides the diagonal of A
    static constexpr int CPR = DK / 8;            // 16-byte pieces per q/k row
    static constexpr int TPP = kPrepThreads / CPR;  // tokens per staging pass
    static constexpr int NP = (L + TPP - 1) / TPP;
};

// One chunk's operands, written by the prep waves, read by the state waves.
// Operand order: element [tile][slice][lane] holds what lane `lane` feeds to the
// MFMA for that tile, so every operand read is one contiguous 16- or 8-byte
// access per lane.  Records are permuted inside a tile (the swizzles below) so
// the staging writes spread over the banks.
template <int DK, int L>
struct WyChunk {
    using S = WyShape<DK, L>;
    bf16x8_t qop[S::NT][S::NJ][64];  // raw q: lane (token r, group g), key dims pi(g, 0..7)
    bf16x8_t kop[S::NT][S::NJ][64];  // raw k, same order
    bf16x8_t ktop[S::JT * (S::NS * 64 + 1)];  // raw k^T: per key tile jt, NS slices of 64 records
                                              // (lane (key dim r, group g), tokens pi(g, 0..7)) + 1 pad
    uint2 Ah[S::NA > 0 ? S::NA : 1][64];  // -A tiles (row block > column block), bf16 hi
    uint2 Al[S::NA > 0 ? S::NA : 1][64];  //   and lo
    uint2 Th[S::NT][64];             // (I + A_ii)^-1, hi
    uint2 Tl[S::NT][64];             //   and lo
    uint2 Mh[S::NM][64];             // M tiles, hi
    uint2 Ml[S::NM][64];             //   and lo
    // per token t of the chunk; padding tokens carry beta = 0, rk = rq = 0
    float beta[L], eG[L], eGL[L];    // beta, e^{G_t}, e^{G_L - G_t}
    float rk[L], rq[L];              // 1/|k|, 1/|q|
};

template <int DK, int L>
struct WySmem {
    using S = WyShape<DK, L>;
    WyChunk<DK, L> ch[2];            // chunk c (state waves) and chunk c+1 (prep waves)
    // the prep waves' own scratch for the chunk they prepare
    float Ad[S::NT][16][16];         // fp32 diagonal blocks of A
    float Gv[L];                     // G_t
    float F[L];                      // e^{G_end(block of t) - G_t}
    float E[S::NT][L];               // e^{G_t - G_end(k)} for blocks k before t's block
};

template <int NS>
__device__ __forceinline__ int kt_rec(int jt, int ms, int lane) { return jt * (NS * 64 + 1) + ms * 64 + lane; }

// linear index of a gram tile other than the diagonal blocks of A ->
// (M tile?, row block ib, column block kb): first the strictly lower A tiles
// in row order, then the lower M tiles with the diagonal in row order
template <int NT>
__device__ __forceinline__ void other_tile(int i, bool& is_m, int& ib, int& kb)
{
    constexpr int NA = NT * (NT - 1) / 2;
    is_m = i >= NA;
    int r = is_m ? i - NA : i;
    ib = is_m ? 0 : 1;
#pragma unroll
    for (int k = 0; k < NT; ++k) {
        const int n = is_m ? ib + 1 : ib;  // tiles in row ib
        if (r >= n) {
            r -= n;
            ++ib;
        }
    }
    kb = r;
}

template <int DK, int L, bool O_BF16>
__global__ __launch_bounds__(kThreads) void prefill_wy_kernel(PrefillArgs a)
{
    using Sh = WyShape<DK, L>;
    constexpr int NT = Sh::NT, NJ = Sh::NJ, JT = Sh::JT, NO = Sh::NO;
    constexpr int CPR = Sh::CPR, TPP = Sh::TPP, NP = Sh::NP;
    constexpr int OE = O_BF16 ? 2 : 4;
    __shared__ WySmem<DK, L> sm;
    GDN_TL_BEGIN();

    const int tid = threadIdx.x;
    const int lane0 = tid & 63, wave = tid >> 6;
    const bool prep = wave >= kStateWaves;
    const int b = blockIdx.z;
    const int T = a.T, Hk = a.Hk, Hv = a.Hv, dv = a.dv;
    const int h = head_of_row(blockIdx.y, Hv, Hk, gridDim.x);
    const int C = 2 * Hk * DK + Hv * dv;
    const int hk = h / (Hv / Hk);
    const uint16_t* qkv = reinterpret_cast<const uint16_t*>(a.qkv);
    auto chunk_rsrc = [&](int c0) __attribute__((always_inline)) {
        // the chunk's tokens of the slab: loads past the prompt read as zero
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qkv + ((size_t)b * T + c0) * C), 0,
                                                 min(L, T - c0) * C * 2, kBufferFlags);
    };

    // ---------------------------------------------------------------- prep waves
    const int ptid = tid - kStateWaves * 64, pwave = wave - kStateWaves;
    uint4 qreg[NP], kreg[NP];  // the q|k pieces of the chunk to stage next
    // prep wave 0, lane t: raw beta and raw alpha, each in its own register (combining them at load
    // time would wait for the prefetch right away)
    uint32_t gbr = 0, gal = 0;
    float dtb, eal;                               // the head's dt_bias and e^{A_log}
    head_gate_consts(a.dt_bias, a.A_log, h, dtb, eal);
    const bool raw_gates = a.dt_bias != nullptr;
    // staging role: piece sr of token row stp (+ TPP per pass)
    const int qoff = ((ptid / CPR) * C + hk * DK + 8 * (ptid % CPR)) * 2;
    const int goff = (lane0 * Hv + h) * 2;
    auto prefetch_qk = [&](int c0) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(c0);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            // the lane's offset in a VGPR, the pass's and k's (uniform) in the SGPR offset
            const int so = __builtin_amdgcn_readfirstlane(p * TPP * C * 2);
            qreg[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, so, 0));
            kreg[p] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, __builtin_amdgcn_readfirstlane(so + Hk * DK * 2), 0));
        }
        if (pwave == 0) {
            const int Lv = min(L, T - c0);
            const size_t g0 = ((size_t)b * T + c0) * Hv;
            const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.beta_raw) + g0), 0, Lv * Hv * 2,
                kBufferFlags);
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.alpha) + g0), 0, Lv * Hv * 2,
                kBufferFlags);
            gbr = __builtin_amdgcn_raw_buffer_load_b16(rb, goff, 0, 0);
            gal = __builtin_amdgcn_raw_buffer_load_b16(ra, goff, 0, 0);
        }
    };

    // stage the prefetched chunk (starting at token c0) into buffer x: q, k in operand order, k^T,
    // norms; gates, their running sums and decay factors (prep wave 0)
    auto stage = [&](int c0, WyChunk<DK, L>& x) __attribute__((always_inline)) {
        const int Lv = min(L, T - c0);
        int sr = ptid % CPR, stp = ptid / CPR, lane = lane0;
        asm volatile("" : "+v"(sr), "+v"(stp), "+v"(lane));
        const int lg = lane >> 4;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int t = p * TPP + stp;
            const bool in_chunk = TPP * NP == L || t < L;
            const uint4 q = qreg[p], k = kreg[p];  // zero past the prompt
            if (in_chunk) {
                // q, k in operand order: key dims 8 sr .. 8 sr + 7 of token t
                const int tt = t >> 4, tr = t & 15;
                const int m = sr >> 2, hf = (sr & 3) >> 1, g0 = (sr & 1) << 1;
                char* qd = reinterpret_cast<char*>(&x.qop[tt][m][0]) + 8 * hf;
                char* kd = reinterpret_cast<char*>(&x.kop[tt][m][0]) + 8 * hf;
                const int r0 = qk_rec(tr + 16 * g0, m) * 16, r1 = qk_rec(tr + 16 * (g0 + 1), m) * 16;
                *reinterpret_cast<uint2*>(qd + r0) = make_uint2(q.x, q.y);
                *reinterpret_cast<uint2*>(qd + r1) = make_uint2(q.z, q.w);
                *reinterpret_cast<uint2*>(kd + r0) = make_uint2(k.x, k.y);
                *reinterpret_cast<uint2*>(kd + r1) = make_uint2(k.z, k.w);
                // k^T in operand order: token t is group pi_group, slot pi_slot of its 32-token slice
                const int ms = t >> 5, tg = pi_group(t & 31), ts = pi_slot(t & 31);
                const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
                uint16_t* dst =
                    reinterpret_cast<uint16_t*>(&x.ktop[kt_rec<Sh::NS>(sr >> 1, ms, 8 * (sr & 1) + 16 * tg)]) + ts;
#pragma unroll
                for (int e = 0; e < 8; ++e)  // key dim 8 sr + e: record + e
                    dst[8 * e] = (uint16_t)((e & 1) ? (kw[e >> 1] >> 16) : (kw[e >> 1] & 0xffffu));
            }
            // norms: every token row is CPR consecutive lanes
            const float sq = group_sum<CPR>(sq8(q, 0.f));
            const float sk = group_sum<CPR>(sq8(k, 0.f));
            if (sr == 0 && in_chunk) {
                const bool valid = t < Lv;
                x.rk[t] = valid ? __builtin_amdgcn_rsqf(sk + a.eps) : 0.f;
                x.rq[t] = valid ? __builtin_amdgcn_rsqf(sq + a.eps) : 0.f;
            }
        }
        if (pwave == 0) {
            // gates, their running sum and the decay factors; lane = token
            float beta = 0.f, g = 0.f;
            if (lane < Lv) gate(bf16_lo(gbr), bf16_lo(gal), raw_gates, dtb, eal, beta, g);
            float G = g;
#pragma unroll
            for (int d = 1; d < L; d <<= 1) {
                const float o = __shfl_up(G, d, 64);
                if (lane >= d) G += o;
            }
            const float GL = __shfl(G, L - 1, 64);
            float Gend[NT];
#pragma unroll
            for (int k = 0; k < NT; ++k) Gend[k] = __shfl(G, 16 * k + 15, 64);
            if (lane < L) {
                const int blk = lane >> 4;
                x.beta[lane] = beta;
                x.eG[lane] = __expf(G);
                x.eGL[lane] = __expf(GL - G);
                sm.Gv[lane] = G;
                float ge = Gend[0];
#pragma unroll
                for (int k = 1; k < NT; ++k)
                    if (blk == k) ge = Gend[k];
                sm.F[lane] = __expf(fminf(ge - G, 0.f));
#pragma unroll
                for (int k = 0; k < NT; ++k) sm.E[k][lane] = k < blk ? __expf(fminf(G - Gend[k], 0.f)) : 0.f;
            }
        }
        (void)lg;
    };

    // the gram tiles of the staged chunk in buffer x: prep wave 0 the diagonal blocks of A and their
    // inverses, prep waves 1..3 the other tiles (-A below the diagonal, M)
    auto grams = [&](WyChunk<DK, L>& x) __attribute__((always_inline)) {
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        const int lr = lane & 15, lg = lane >> 4;
        if (pwave == 0) {
            f32x4_t D[NT];
#pragma unroll
            for (int ib = 0; ib < NT; ++ib) {
                D[ib] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < NJ; ++m) {
                    const bf16x8_t kk = x.kop[ib][m][qk_rec(lane, m)];
                    D[ib] = mfma32(kk, kk, D[ib]);
                }
                asm volatile("" ::: "memory");  // one block's operands at a time
            }
#pragma unroll
            for (int ib = 0; ib < NT; ++ib) {
                // lane: row t = 16 ib + lr, columns s = 16 ib + 4 lg + e
                const int t = 16 * ib + lr;
                const float bt = x.beta[t] * x.rk[t], Gt = sm.Gv[t];
                const float4 rks = lds_f4(&x.rk[16 * ib + 4 * lg]);
                const float4 Gs = lds_f4(&sm.Gv[16 * ib + 4 * lg]);
                const float rk4[4] = {rks.x, rks.y, rks.z, rks.w}, G4[4] = {Gs.x, Gs.y, Gs.z, Gs.w};
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = 4 * lg + e;
                    y[e] = s < lr ? bt * rk4[e] * __expf(fminf(Gt - G4[e], 0.f)) * D[ib][e] : 0.f;
                }
                *reinterpret_cast<float4*>(&sm.Ad[ib][lr][4 * lg]) = make_float4(y[0], y[1], y[2], y[3]);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            const int blk = lg, jc = lr;
            if (blk < NT) {
                // column jc of (I + A_blk)^-1: x_t = [t == jc] - sum_{s<t} A[t][s] x_s
                float xs[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float acc0 = t == jc ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
                    for (int s4 = 0; s4 < (t + 3) / 4; ++s4) {
                        const float4 ar = lds_f4(&sm.Ad[blk][t][4 * s4]);
                        const float av[4] = {ar.x, ar.y, ar.z, ar.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * s4 + e < t) {
                                if (e & 1) acc1 = __builtin_fmaf(-av[e], xs[4 * s4 + e], acc1);
                                else acc0 = __builtin_fmaf(-av[e], xs[4 * s4 + e], acc0);
                            }
                    }
                    xs[t] = acc0 + acc1;
                    // one step at a time: hoisting every step's row loads would not fit the registers
                    asm volatile("" ::: "memory");
                }
                // T[t][jc] -> operand lane t + 16 (jc / 4), slot jc % 4
                uint16_t* th = reinterpret_cast<uint16_t*>(&x.Th[blk][0]);
                uint16_t* tl = reinterpret_cast<uint16_t*>(&x.Tl[blk][0]);
#pragma unroll
                for (int t = 0; t < 16; t += 2) {
                    uint32_t hi, lo;
                    split2(xs[t], xs[t + 1], hi, lo);
                    const int at = (t + 16 * (jc >> 2)) * 4 + (jc & 3);
                    th[at] = (uint16_t)hi;
                    tl[at] = (uint16_t)lo;
                    th[at + 4] = (uint16_t)(hi >> 16);
                    tl[at + 4] = (uint16_t)(lo >> 16);
                }
            }
        } else {
            // one tile per round (not unrolled: the operand loads of all tiles at once would not fit
            // in the registers left beside the prefetched q and k)
#pragma unroll 1
            for (int i = pwave - 1; i < NO; i += kPrepWaves - 1) {
                bool ism;
                int ib, kb;
                other_tile<NT>(i, ism, ib, kb);
                f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < NJ; ++m) {
                    const int rec = qk_rec(lane, m);
                    const bf16x8_t ka = x.kop[kb][m][rec];
                    const bf16x8_t xb = ism ? x.qop[ib][m][rec] : x.kop[ib][m][rec];
                    D = mfma32(ka, xb, D);
                }
                // lane: row t of the tile (ib, kb), columns s = 16 kb + 4 lg + e
                const int t = 16 * ib + lr, s0 = 16 * kb + 4 * lg;
                const float4 rks = lds_f4(&x.rk[s0]);
                const float rk4[4] = {rks.x, rks.y, rks.z, rks.w};
                float y[4];
                if (kb < ib) {
                    // e^{G_t - G_s} = E[kb][t] F[s]
                    const float4 Fs = lds_f4(&sm.F[s0]);
                    const float F4[4] = {Fs.x, Fs.y, Fs.z, Fs.w};
                    const float ct = (ism ? x.rq[t] : x.beta[t] * x.rk[t]) * sm.E[kb][t];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = ct * F4[e] * rk4[e] * D[e];
                } else {
                    // diagonal tile of M: direct decay, s <= t
                    const float Gt = sm.Gv[t], rqt = x.rq[t];
                    const float4 Gs = lds_f4(&sm.Gv[s0]);
                    const float G4[4] = {Gs.x, Gs.y, Gs.z, Gs.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        y[e] = 4 * lg + e <= lr ? rqt * rk4[e] * __expf(fminf(Gt - G4[e], 0.f)) * D[e] : 0.f;
                }
                uint2 hi, lo;
                if (ism) {
                    split4(f32x4_t{y[0], y[1], y[2], y[3]}, hi, lo);
                    const int im = ib * (ib + 1) / 2 + kb;
                    x.Mh[im][lane] = hi;
                    x.Ml[im][lane] = lo;
                } else {
                    // stored negated: the solve accumulates -A U onto the right-hand side
                    split4(f32x4_t{-y[0], -y[1], -y[2], -y[3]}, hi, lo);
                    const int ia = ib * (ib - 1) / 2 + kb;
                    x.Ah[ia][lane] = hi;
                    x.Al[ia][lane] = lo;
                }
            }
        }
    };

    // ---------------------------------------------------------------- state waves
    // this lane's state row; rows past dv carry zeros and store nothing
    const int row = blockIdx.x * kRows + wave * 16 + (lane0 & 15);
    const bool live = !prep && row < dv;
    const int rowc = live ? row : 0;
    f32x4_t S[JT];                   // S^T tiles: tile jt holds S[row][16 jt + 4 lg + e]
    uint32_t vreg[NT * 4];           // v[token 16 tt + 4 lg + e][row] of the chunk to process next (raw bf16)
    const int voff = ((4 * (lane0 >> 4)) * C + 2 * Hk * DK + h * dv + row) * 2;
    auto prefetch_v = [&](int c0) __attribute__((always_inline)) {
        // rows past dv read another channel or past the chunk (zero): unused
        const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(c0);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e)  // the token's (uniform) offset in the SGPR offset
                vreg[4 * tt + e] = __builtin_amdgcn_raw_buffer_load_b16(
                    rv, voff, __builtin_amdgcn_readfirstlane((16 * tt + e) * C * 2), 0);
    };

    // Each role runs its own loop (their registers then need not coexist); both pass the same
    // barriers: two before the first chunk, two per chunk.
    if (prep) {
        // the preparation shares each SIMD with state waves and sets the pace: its instructions go
        // first when both are ready (dk 64 / chunk 64: 396 -> 337 us; dk 128 / chunk 32: 565 -> 490 us)
        __builtin_amdgcn_s_setprio(1);
        prefetch_qk(0);
        stage(0, sm.ch[0]);
        if (L < T) prefetch_qk(L);
        __syncthreads();
        grams(sm.ch[0]);
        __syncthreads();
        for (int c0 = 0, it = 0; c0 < T; c0 += L, ++it) {
            const bool more = c0 + L < T;
            WyChunk<DK, L>& nxt = sm.ch[(it & 1) ^ 1];
            if (it == 10) GDN_TL(0);
            // phase 1: stage the next chunk
            if (more) {
                stage(c0 + L, nxt);
                // the next loads only once this chunk's registers are written to LDS
                asm volatile("" ::: "memory");
                if (c0 + 2 * L < T) prefetch_qk(c0 + 2 * L);
            }
            if (it == 10) GDN_TL(1);
            __syncthreads();
            if (it == 10) GDN_TL(2);
            // phase 2: its gram tiles and inverses
            if (more) grams(nxt);
            if (it == 10) GDN_TL(3);
            __syncthreads();
            if (it == 10) GDN_TL(4);
        }
        GDN_TL_END();
        return;
    }

    {
        const float* sp = a.S_in + (((size_t)b * Hv + h) * dv + rowc) * DK + 4 * (lane0 >> 4);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            const f32x4_t v = load_f4(sp + 16 * jt);
            S[jt] = live ? v : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        prefetch_v(0);
    }
    __syncthreads();
    __syncthreads();
    for (int c0 = 0, it = 0; c0 < T; c0 += L, ++it) {
        const int Lv = min(L, T - c0);
        const bool more = c0 + L < T;
        WyChunk<DK, L>& cur = sm.ch[it & 1];
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        const int lg = lane >> 4;
        if (it == 10) GDN_TL(0);
        // ================= phase 1: P = K S^T, R = Q S^T -> right-hand sides X and the state part of O
        f32x4_t X[NT], O[NT];
        {
            f32x4_t P[NT], R[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                P[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                R[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int m = 0; m < NJ; ++m) {
                // the state's columns of key slice m as bf16 hi + lo, once for all token tiles
                uint2 h0, l0, h1, l1;
                split4(S[2 * m], h0, l0);
                split4(S[2 * m + 1], h1, l1);
                const bf16x8_t shi = as8(h0, h1), slo = as8(l0, l1);
                const int rec = qk_rec(lane, m);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const bf16x8_t ka = cur.kop[tt][m][rec];
                    const bf16x8_t qa = cur.qop[tt][m][rec];
                    P[tt] = mfma32(ka, shi, P[tt]);
                    P[tt] = mfma32(ka, slo, P[tt]);
                    R[tt] = mfma32(qa, shi, R[tt]);
                    R[tt] = mfma32(qa, slo, R[tt]);
                }
                asm volatile("" ::: "memory");  // one slice's operands at a time (registers)
            }
            // X = beta (v - e^{G} rk P), O = e^{G} rq R (token t = 16 tt + 4 lg + e)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int t0 = 16 * tt + 4 * lg;
                const float4 be = lds_f4(&cur.beta[t0]), eg = lds_f4(&cur.eG[t0]);
                const float4 rk4 = lds_f4(&cur.rk[t0]), rq4 = lds_f4(&cur.rq[t0]);
                const float bv[4] = {be.x, be.y, be.z, be.w}, gv[4] = {eg.x, eg.y, eg.z, eg.w};
                const float kv[4] = {rk4.x, rk4.y, rk4.z, rk4.w}, qv[4] = {rq4.x, rq4.y, rq4.z, rq4.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = live ? bf16_lo(vreg[4 * tt + e]) : 0.f;
                    X[tt][e] = bv[e] * __builtin_fmaf(-gv[e] * kv[e], P[tt][e], v);
                    O[tt][e] = gv[e] * qv[e] * R[tt][e];
                }
            }
        }
        if (it == 10) GDN_TL(1);
        __syncthreads();
        if (it == 10) GDN_TL(2);

        // ================= phase 2: U by block forward substitution, the outputs, the state update
        {
            const float eGL = cur.eG[L - 1];
#pragma unroll
            for (int jt = 0; jt < JT; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[jt][e] *= eGL;
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<char*>(a.o) + ((size_t)b * T + c0) * Hv * dv * OE, 0, Lv * Hv * dv * OE,
                kBufferFlags);
            // rows past dv and tokens past the prompt fall outside the resource: dropped
            const int ostride = __builtin_amdgcn_readfirstlane(Hv * dv * OE);
            const int ooff = live ? ((4 * lg * Hv + h) * dv + row) * OE : 0x7ffffff0;
            uint2 Uh[NT], Ul[NT];
            uint2 ch0 = make_uint2(0, 0), cl0 = make_uint2(0, 0);
#pragma unroll
            for (int ib = 0; ib < NT; ++ib) {
                f32x4_t x = X[ib];
#pragma unroll
                for (int kb = 0; kb < ib; ++kb) {
                    const int ia = ib * (ib - 1) / 2 + kb;
                    const uint2 ah = cur.Ah[ia][lane], al = cur.Al[ia][lane];
                    x = mfma16(ah, Uh[kb], x);
                    x = mfma16(ah, Ul[kb], x);
                    x = mfma16(al, Uh[kb], x);
                }
                uint2 xh, xl;
                split4(x, xh, xl);
                const uint2 th = cur.Th[ib][lane], tl = cur.Tl[ib][lane];
                f32x4_t u = {0.f, 0.f, 0.f, 0.f};
                u = mfma16(th, xh, u);
                u = mfma16(th, xl, u);
                u = mfma16(tl, xh, u);
                split4(u, Uh[ib], Ul[ib]);

                f32x4_t o = O[ib];
#pragma unroll
                for (int kb = 0; kb <= ib; ++kb) {
                    const int im = ib * (ib + 1) / 2 + kb;
                    const uint2 mh = cur.Mh[im][lane], ml = cur.Ml[im][lane];
                    o = mfma16(mh, Uh[kb], o);
                    o = mfma16(mh, Ul[kb], o);
                    o = mfma16(ml, Uh[kb], o);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int so = __builtin_amdgcn_readfirstlane((16 * ib + e) * ostride);   // the token's
                    if constexpr (O_BF16)
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)o[e]), ro, ooff, so, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[e]), ro, ooff, so, 0);
                }

                // c_t u_t with c_t = e^{G_L - G_t} rk_t: operand of the state update
                const float4 el = lds_f4(&cur.eGL[16 * ib + 4 * lg]), rk4 = lds_f4(&cur.rk[16 * ib + 4 * lg]);
                const f32x4_t cu = {el.x * rk4.x * u[0], el.y * rk4.y * u[1], el.z * rk4.z * u[2], el.w * rk4.w * u[3]};
                uint2 ch, cl;
                split4(cu, ch, cl);
                if (ib & 1) {
                    // tiles ib-1, ib form the 32-token slice ib/2
                    const bf16x8_t chi = as8(ch0, ch), clo = as8(cl0, cl);
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const bf16x8_t ka = cur.ktop[kt_rec<Sh::NS>(jt, ib >> 1, lane)];
                        S[jt] = mfma32(ka, chi, S[jt]);
                        S[jt] = mfma32(ka, clo, S[jt]);
                        if (jt % 4 == 3) asm volatile("" ::: "memory");  // four key tiles' operands at a time
                    }
                } else if (ib == NT - 1) {
                    // a lone 16-token tile: slots 0..3 of its slice
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const uint4 kk = __builtin_bit_cast(uint4, cur.ktop[kt_rec<Sh::NS>(jt, ib >> 1, lane)]);
                        const uint2 ka = make_uint2(kk.x, kk.y);
                        S[jt] = mfma16(ka, ch, S[jt]);
                        S[jt] = mfma16(ka, cl, S[jt]);
                    }
                } else {
                    ch0 = ch;
                    cl0 = cl;
                }
                asm volatile("" ::: "memory");  // one block's operands at a time (registers)
            }
        }
        // the next chunk's v: loaded here rather than after X, so that the registers are free
        // during the solve
        if (more) prefetch_v(c0 + L);
        if (it == 10) GDN_TL(3);
        __syncthreads();
        if (it == 10) GDN_TL(4);
    }

    if (live) {
        float* sp = a.S_out + (((size_t)b * Hv + h) * dv + row) * DK + 4 * (lane0 >> 4);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) store_f4<false>(sp + 16 * jt, S[jt]);
    }
    GDN_TL_END();
}

template <int DK, int L, bool O_BF16>
hipError_t launch_l(const PrefillArgs& a, hipStream_t s)
{
    dim3 grid((a.dv + kRows - 1) / kRows, a.Hv, a.B);
    prefill_wy_kernel<DK, L, O_BF16><<<grid, dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

template <int DK, bool O_BF16>
hipError_t launch_d(const PrefillArgs& a, hipStream_t s)
{
    switch (a.chunk) {
    case 16: return launch_l<DK, 16, O_BF16>(a, s);
    case 32: return launch_l<DK, 32, O_BF16>(a, s);
    case 64: return launch_l<DK, 64, O_BF16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <bool O_BF16>
hipError_t launch_o(const PrefillArgs& a, hipStream_t s)
{
    switch (a.dk) {
    case 32: return launch_d<32, O_BF16>(a, s);
    case 64: return launch_d<64, O_BF16>(a, s);
    case 128: return launch_d<128, O_BF16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_wy(const PrefillArgs& a, bool o_bf16, hipStream_t s)
{
    // dk = 128 with chunks of 64 tokens: the kernel with 32-row state waves
    if (a.dk == 128 && a.chunk == 64) return launch_prefill_c64(a, o_bf16, s);
    return o_bf16 ? launch_o<true>(a, s) : launch_o<false>(a, s);
}

}  // namespace gdn

#ifdef GDN_TIMELINE
GDN_TIMELINE_READER(gdn_timeline_prefill)
#endif
