// gdn_step.hip -- one verify step of a GDN layer in one launch (gfx950):
// the rollback of the previous window by selection, the conv step of this
// window and the chain verify with capture, for bf16 slabs.
//
// The pages describe the pieces as separate fused ops: the conv step that
// replaces the transpose/concat/conv/silu/copy chain (lucebox PR #637, commit
// message on ggml_ssm_conv_step; review note on its four sources), the verify
// that writes the final state and every intermediate state in one pass (atlas
// PR #297, commit message on gated_delta_rule_wy16.cu) and the rollback to an
// accepted prefix (strix-llama.cpp PR #14, commit messages on recurrent
// snapshot rollback).  Here they are one launch, bit for bit what
// gdn_rollback + gdn_conv_step + gdn_verify give.
//
// Start state.  Sequence b starts from the previous window's checkpoint
// (accept length a = 0), its capture H[a-1] (0 < a < K_prev) or its final state
// (a = K_prev), and its conv history is window rows a .. a+2 of the previous
// window; the start state is written out as this window's checkpoint.  The
// accept length is the kernel's first load; every load that does not depend on
// it is issued next, the start state and the history rows after it.
//
// Mapping.  A workgroup holds the three value heads of one key head (12 waves,
// four per head, each wave two state rows of 128 columns: a lane owns one float4
// of a row, as in gdn_verify).  The key head's q|k conv is done once per
// workgroup and pipelined with the state stream, in chunks of tokens (the
// first of two tokens, then TC each):
//   - a conv item is one token's q (or k) row of DK channels; IL = DK/2 lanes
//     hold one bf16 pair each (one 4-byte load per window row), so a wave does
//     64/IL items and the 12 waves a chunk of 2*TC items at once;
//   - the item's norm is a sum over its lanes, in the summation tree of
//     gdn_verify's staging threads (a chain of bf16 dot2 over each 16-byte
//     piece, then pairs of pieces, pairs of pairs, ...), so the fused step
//     gives its bits;
//   - chunk 0 (tokens 0 and 1, on four waves) is convolved before the first
//     barrier, while other waves form the gates and the v conv; then for every chunk c
//     the waves run the token recurrence over chunk c (each state streams out
//     as soon as it is formed) and convolve chunk c+1 while those stores drain,
//     then meet at a barrier.  A barrier waits for LDS only, not for the
//     stores in flight, so HBM stays busy across it.
// The v conv of a head's rows (one wave per head, a lane per channel pair and
// token) and the gates (another wave per head) are formed before the first
// barrier, on waves that have no chunk-0 item.  Only the loads on the way to the first state are issued at the
// start (the accept length, the taps, then the start state and chunk 0's rows):
// at kernel start every wave of the chip loads at once, and the number of load
// instructions sets how long the round trips take.
#include "gdn_conv_math.h"
#include "gdn_debug.h"
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_timeline.h"
#include "gdn_verify_common.h"

namespace gdn {
namespace {

constexpr int kGroups = 3;                       // value heads per workgroup
constexpr int kStepWaves = kGroups * kWaves;     // 12
constexpr int kStepThreads = kStepWaves * 64;    // 768
constexpr int kCW = 4;                           // conv width

template <int DK, int KP, int RPG>
struct StepSmem {
    static constexpr int QW = DK + 8;            // padded bf16 row: rows start 4 banks apart
    uint16_t q[KP][QW];                          // conv outputs of the key head's q channels (bf16 bits)
    uint16_t k[KP][QW];                          // ... and of its k channels
    uint16_t win[KP + 3][2 * DK];                // the window rows of the key head's q|k channels (raw bits)
    float4 tok[kGroups][KP];                     // per head and token: beta, gamma = e^g, 1/|k|, 1/|q|
    float V[2][kGroups][KP][RPG];                // v of the head's rows, per token (two row blocks)
};

// bf16 dot2 of a packed pair with itself, accumulated onto acc
__device__ __forceinline__ float sq2(uint32_t w, float acc)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_shift(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum of squares of a row of DK bf16 values held as pairs by IL = DK/2 consecutive
// lanes (lane il: values 2il, 2il+1), in gdn_verify's order: per 16-byte piece
// (four lanes) a chain of dot2 over its four pairs, then the VPR = DK/8 piece sums
// added in pairs (p, p^1), then pairs of those, and so on.  Every lane of the item
// gets the total.
template <int DK>
__device__ __forceinline__ float item_sumsq(uint32_t w, int lane)
{
    constexpr int IL = DK / 2;
    // the chain: lane 4p+e continues the partial sum of lane 4p+e-1
    float s = sq2(w, 0.0f);
    s = sq2(w, dpp_shift<0x111>(s));             // row_shr:1
    s = sq2(w, dpp_shift<0x111>(s));
    s = sq2(w, dpp_shift<0x111>(s));             // lane 4p+3: piece p
    // pieces p and p^1 (lanes 4 apart), then p and p^2 (lanes 8 apart): every lane exchanges with
    // its partner (no select between two shifts, which the compiler turns into a branch that
    // masks off the very lanes the shift reads)
    s = s + __shfl_xor(s, 4, 64);
    s = s + __shfl_xor(s, 8, 64);                // lane 16r+3: the four pieces of row r
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 3));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 19));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 35));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), 51));
    if constexpr (IL == 64) {
        return (r0 + r1) + (r2 + r3);
    } else if constexpr (IL == 32) {
        return lane < 32 ? r0 + r1 : r2 + r3;
    } else {
        static_assert(IL == 16, "dk 32, 64 or 128");
        const int rr = lane >> 4;
        return rr == 0 ? r0 : (rr == 1 ? r1 : (rr == 2 ? r2 : r3));
    }
}

// CAPTURE: H is written (every state of the window); LIVE: every row of every workgroup is a
// state row (dv a multiple of the rows per head and workgroup).  With both, each token's state
// store is one unconditional instruction, so the compiler's wait for a chunk's window rows
// (loaded before the previous chunk's stores) counts those stores exactly instead of draining
// them.
// RB: row blocks per workgroup (at large batches a workgroup takes RB consecutive row blocks of
// one key head: the q|k conv, the gates and the staging are done once, and the next block's start
// state and v rows load while the current block streams; RB > 1 needs CAPTURE and LIVE)
template <int DK, int KMAX, bool O_BF16, bool CAPTURE, bool LIVE, int RB>
__global__ __launch_bounds__(kStepThreads) void step_kernel(VerifyArgs a)
{
    constexpr int LPR = DK / 4;                  // lanes per state row (one float4 each)
    constexpr int RPW = 64 / LPR;                // rows per wave
    constexpr int RPG = kWaves * RPW;            // rows per head
    constexpr int KP = (KMAX + 15) / 16 * 16;
    constexpr int IL = DK / 2;                   // lanes per q|k conv item
    constexpr int IPW = 64 / IL;                 // items per wave
    constexpr int NS = kStepWaves * IPW;         // items per chunk
    constexpr int T0 = 2;                        // tokens of chunk 0 (on the way to the first store)
    constexpr int TC = NS / 2;                   // tokens of every later chunk
    static_assert(2 * T0 <= NS && 2 * T0 <= 4 * IPW, "chunk 0 fits the first four waves");
    constexpr int NC = KMAX <= T0 ? 1 : 1 + (KMAX - T0 + TC - 1) / TC;   // chunks
    auto chunk_start = [](int cc) { return cc == 0 ? 0 : T0 + (cc - 1) * TC; };
    using Smem = StepSmem<DK, KP, RPG>;
    __shared__ Smem sm;

    GDN_TL_BEGIN();
    GDN_TL(8);
    const int b = blockIdx.z;
    // the row blocks of one group of value heads on one XCD (workgroup i runs on XCD i mod 8): they
    // share the key head's q|k rows and taps through that XCD's L2
    int bx = blockIdx.x, by = blockIdx.y;
    if ((gridDim.y & 7) == 0) {
        const int wi = blockIdx.x + gridDim.x * blockIdx.y, slot = wi >> 3;
        by = (wi & 7) + 8 * (slot / gridDim.x);
        bx = slot % gridDim.x;
    }
    // the wave's value head (uniform: the checkpoint's buffer resource, built from it, is then a scalar
    // one; otherwise the compiler wraps each checkpoint store in a loop over the lanes' resources)
    const int gtid = threadIdx.x, g = __builtin_amdgcn_readfirstlane(gtid / kThreads);
    const int tid = gtid % kThreads, lane = tid & 63, wave = tid >> 6;
    // the previous window's accept length first: the start state and the history rows wait for
    // it.  It is read as a vector load (index zero, but lane-dependent: eps >= 0 is checked on the
    // host), so that the loads issued after it do not wait for it, and used only after them.
    const int z0 = (int)(a.eps < 0.f) & lane;
    const int32_t* accp = a.acc_prev ? a.acc_prev : reinterpret_cast<const int32_t*>(a.w);
    const int ap_raw = accp[(a.acc_prev ? b : 0) + z0];
    GDN_TL(0);

    const int gw = gtid >> 6;                    // wave of the workgroup, 0..11
    const int j = lane % LPR, c = 4 * j;
    const int rloc = wave * RPW + lane / LPR;
    const int h = by * kGroups + g;
    static_assert(RB == 1 || (CAPTURE && LIVE), "several row blocks per workgroup need capture and live rows");
    const int blk0 = bx * RB;                    // the workgroup's first row block
    const int i = blk0 * RPG + rloc;             // this lane's row in the first block
    const int K = a.K, Hk = a.Hk, Hv = a.Hv, dv = a.dv;
    const bool live = LIVE || i < dv;
    const int ic = live ? i : dv - 1;
    const size_t C = 2 * (size_t)Hk * DK + (size_t)Hv * dv;
    const int hk = h / (Hv / Hk);
    const size_t SD = (size_t)dv * DK;
    const size_t hb = ((size_t)b * Hv + h) * SD;
    const int gs = a.gstride > 0 ? a.gstride : Hv;
    const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x) + (size_t)b * K * C;
    const uint16_t* HS0 = reinterpret_cast<const uint16_t*>(a.hsrc) + (size_t)b * a.hrows * C;
    // one workgroup per key head writes the q|k window rows and conv outputs
    const bool qk_writer = bx == 0 && (by * kGroups) % (Hv / Hk) == 0;

    // roles: waves 0..3 convolve chunk 0's q|k items (tokens 0 and 1); waves 4..6 form the gates of
    // head rg = gw - 4 and waves 7..9 the v conv of head rg = gw - 7's rows (waves of the
    // workgroup take the SIMDs in turn, so each role is spread over the SIMDs); every wave
    // convolves q|k items of the later chunks
    const bool gate_wave = gw >= 4 && gw < 4 + kGroups;
    const bool v_wave = gw >= 7 && gw < 7 + kGroups;
    const int rg = gate_wave ? gw - 4 : (v_wave ? gw - 7 : g);   // the head of the role
    const int hr = by * kGroups + rg;

    // ---- loads that do not depend on the accept length
    // conv item of this lane: slot q of every chunk (token chunk_start(cc) + q/2; q even: q, odd: k;
    // chunk 0 takes slots 0 .. 2 T0 - 1), channel pair ch, ch+1 of the key head
    const int slot = gw * IPW + lane / IL, il = lane % IL;
    const int which = slot & 1;
    const size_t ch = (which ? (size_t)(Hk + hk) * DK : (size_t)hk * DK) + 2 * il;
    const float4 tq0 = *reinterpret_cast<const float4*>(a.w + ch * kCW);
    const float4 tq1 = *reinterpret_cast<const float4*>(a.w + (ch + 1) * kCW);
    // window rows t .. t+3 of the item's pair, raw bits: chunk 0's in registers (loaded after the
    // accept length); the later chunks' come from the window staged in LDS
    uint32_t rows0[kCW];
    // the window of the key head's q|k channels staged in LDS as 16-byte pieces (PPR per row):
    // token rows now, history rows (after the accept length) by the first 3 PPR threads
    constexpr int PPR = 2 * DK / 8;
    constexpr int NTP = (KMAX * PPR + kStepThreads - 1) / kStepThreads;   // token-row pieces per thread
    auto piece_chan = [&](int pc) -> size_t {
        return pc < PPR / 2 ? (size_t)hk * DK + 8 * pc : (size_t)(Hk + hk) * DK + 8 * (pc - PPR / 2);
    };
    uint4 tpc[NTP];
#pragma unroll
    for (int n = 0; n < NTP; ++n) {
        const int e = gtid + n * kStepThreads;
        const int t = e / PPR < K ? e / PPR : K - 1;
        tpc[n] = *reinterpret_cast<const uint4*>(X + (size_t)t * C + piece_chan(e % PPR));
    }
    // the v conv (v wave): lane l convolves channel pair p = l mod NPR of the head's rows for tokens
    // (l + 64 n) / NPR, from 4-byte loads of its window rows
    constexpr int NPR = RPG / 2;                 // channel pairs per head and workgroup
    constexpr int NVP = (KMAX * NPR + 63) / 64;  // (token, pair) items per lane
    const int vp = lane % NPR;
    const int vi0 = blk0 * RPG + 2 * vp;         // the pair's first row (first block)
    const bool vlive = vi0 < dv;                 // dv is even: both rows or neither
    const size_t vch = 2 * (size_t)Hk * DK + (size_t)hr * dv + (vlive ? vi0 : 0);
    float4 vt0 = make_float4(0.f, 0.f, 0.f, 0.f), vt1 = vt0;
    uint32_t vrow[NVP][kCW];
    if (v_wave) {
        vt0 = *reinterpret_cast<const float4*>(a.w + vch * kCW);
        vt1 = *reinterpret_cast<const float4*>(a.w + (vch + 1) * kCW);
    }
    // gates (gate wave): lane t the raw bits of token t (clamped), dt_bias and A_log (with
    // pre-activated gates a word of the token rows instead, ignored)
    const bool raw_gates = a.dt_bias != nullptr;
    uint32_t braw_bits = 0, bal_bits = 0;
    float dtb = 0.f, alog = 0.f;
    if (gate_wave) {
        const float* fb = reinterpret_cast<const float*>(X);
        dtb = *(raw_gates ? a.dt_bias + hr : fb);
        alog = *(raw_gates ? a.A_log + hr : fb);
        const size_t gi = ((size_t)b * K + (lane < K ? lane : K - 1)) * gs + hr;
        braw_bits = reinterpret_cast<const uint16_t*>(a.beta_raw)[gi];
        bal_bits = reinterpret_cast<const uint16_t*>(a.alpha)[gi];
    }

    // ---- the start state and the rows that the accept length picks
    const int ap_u = __builtin_amdgcn_readfirstlane(ap_raw);
    GDN_COUNT_CLAMP(a.acc_prev && gtid == 0 && blockIdx.x == 0 && blockIdx.y == 0 && (ap_u < 0 || ap_u > a.Kp));
    const int ap = a.acc_prev ? min(max(ap_u, 0), a.Kp) : 0;
    GDN_TLV(5, ap);
    const float* Sh;
    if (a.acc_prev)
        Sh = ap == 0 ? a.Sp_ckpt + hb
                     : (ap == a.Kp ? a.Sp_out + hb : a.Sp_H + (((size_t)b * (a.Kp - 1) + ap - 1) * Hv + h) * SD);
    else
        Sh = a.S_in + hb;
    const uint16_t* HS = HS0 + (size_t)ap * C;
    // window row r: a history row (r < 3) or token r-3
    auto wrow = [&](int r) -> const uint16_t* { return r < kCW - 1 ? HS + (size_t)r * C : X + (size_t)(r - (kCW - 1)) * C; };
    const f32x4_t S0 = load_f4(Sh + (size_t)ic * DK + c);
    if (gw * IPW < 2 * T0) {                     // the waves of chunk 0's items
        const int t = slot / 2 < K ? slot / 2 : K - 1;
#pragma unroll
        for (int m = 0; m < kCW; ++m) rows0[m] = *reinterpret_cast<const uint32_t*>(wrow(t + m) + ch);
    }
    uint4 hpc = make_uint4(0, 0, 0, 0);
    if (gtid < (kCW - 1) * PPR) hpc = *reinterpret_cast<const uint4*>(HS + (size_t)(gtid / PPR) * C + piece_chan(gtid % PPR));
    if (v_wave) {
#pragma unroll
        for (int n = 0; n < NVP; ++n) {
            const int t = (lane + 64 * n) / NPR;
            const int tl = t < K ? t : K - 1;
#pragma unroll
            for (int m = 0; m < kCW; ++m) vrow[n][m] = *reinterpret_cast<const uint32_t*>(wrow(tl + m) + vch);
        }
    }
    GDN_TLV(6, S0[0]);

    // ---- gates: lane t the token's beta and gamma = e^g
    if (gate_wave) {
        float be = 0.f, gg = 0.f;
        if (lane < K)
            gate(__uint_as_float(braw_bits << 16), __uint_as_float(bal_bits << 16), raw_gates, dtb, alog, be, gg);
        if (lane < KP) {
            sm.tok[rg][lane].x = be;
            sm.tok[rg][lane].y = __expf(gg);
        }
    }

    uint16_t* Wb = a.win ? reinterpret_cast<uint16_t*>(a.win) + (size_t)b * (kCW - 1 + K) * C : nullptr;
    uint16_t* Yb = a.y ? reinterpret_cast<uint16_t*>(a.y) + (size_t)b * K * C : nullptr;

    // ---- v conv of the head's rows (row block r: channel pair vch + r RPG), every token; their
    // window rows and conv outputs
    auto vconv = [&](int r) __attribute__((always_inline)) {
        if (!v_wave) return;
        const float ta[kCW] = {vt0.x, vt0.y, vt0.z, vt0.w};
        const float tb[kCW] = {vt1.x, vt1.y, vt1.z, vt1.w};
        const bool vl = vlive && vi0 + r * RPG < dv;
        const size_t vc = vch + (size_t)r * RPG;
#pragma unroll
        for (int n = 0; n < NVP; ++n) {
            const int t = (lane + 64 * n) / NPR;
            if (t < K) {
                float c0[kCW], c1[kCW];
#pragma unroll
                for (int m = 0; m < kCW; ++m) {
                    c0[m] = bf16_lo(vrow[n][m]);
                    c1[m] = bf16_hi(vrow[n][m]);
                }
                const uint32_t y0 = conv_silu_bf16(conv_pre<kCW>(ta, c0));
                const uint32_t y1 = conv_silu_bf16(conv_pre<kCW>(tb, c1));
                *reinterpret_cast<float2*>(&sm.V[r & 1][rg][t][2 * vp]) = make_float2(bf16_to_f32(y0), bf16_to_f32(y1));
                if (vl) {
                    if (Yb) *reinterpret_cast<uint32_t*>(Yb + (size_t)t * C + vc) = y0 | (y1 << 16);
                    if (Wb) {
                        *reinterpret_cast<uint32_t*>(Wb + (size_t)(t + kCW - 1) * C + vc) = vrow[n][kCW - 1];
                        if (t == 0) {
#pragma unroll
                            for (int m = 0; m < kCW - 1; ++m)
                                *reinterpret_cast<uint32_t*>(Wb + (size_t)m * C + vc) = vrow[n][m];
                        }
                    }
                }
            }
        }
    };
    vconv(0);

    GDN_TL(7);
    // ---- the q|k conv of one chunk: this lane's item, its norm, LDS, window rows and outputs
    const float tap0[kCW] = {tq0.x, tq0.y, tq0.z, tq0.w};
    const float tap1[kCW] = {tq1.x, tq1.y, tq1.z, tq1.w};
    uint16_t(*qk)[Smem::QW] = which ? sm.k : sm.q;
    auto conv_chunk = [&](int cc) {
        const int t = chunk_start(cc) + slot / 2;
        if (t < K && (cc > 0 || slot < 2 * T0)) {
            uint32_t rw[kCW];
#pragma unroll
            for (int m = 0; m < kCW; ++m)
                rw[m] = cc == 0 ? rows0[m] : *reinterpret_cast<const uint32_t*>(&sm.win[t + m][which * DK + 2 * il]);
            float c0[kCW], c1[kCW];
#pragma unroll
            for (int m = 0; m < kCW; ++m) {
                c0[m] = bf16_lo(rw[m]);
                c1[m] = bf16_hi(rw[m]);
            }
            const uint32_t y0 = conv_silu_bf16(conv_pre<kCW>(tap0, c0));
            const uint32_t y1 = conv_silu_bf16(conv_pre<kCW>(tap1, c1));
            const uint32_t yw = y0 | (y1 << 16);
            *reinterpret_cast<uint32_t*>(&qk[t][2 * il]) = yw;
            const float r = __builtin_amdgcn_rsqf(item_sumsq<DK>(yw, lane) + a.eps);
            if (il == 0) {
#pragma unroll
                for (int gg = 0; gg < kGroups; ++gg) {
                    if (which) sm.tok[gg][t].z = r;
                    else sm.tok[gg][t].w = r;
                }
            }
            if (qk_writer && Yb) *reinterpret_cast<uint32_t*>(Yb + (size_t)t * C + ch) = yw;
        }
    };
    // the q|k window in LDS (read by the later chunks after the first barrier) and, by one workgroup
    // per key head, in the window output
#pragma unroll
    for (int n = 0; n < NTP; ++n) {
        const int e = gtid + n * kStepThreads;
        if (e < K * PPR) {
            const int r = kCW - 1 + e / PPR, pc = e % PPR;
            *reinterpret_cast<uint4*>(&sm.win[r][8 * pc]) = tpc[n];
            if (qk_writer && Wb) *reinterpret_cast<uint4*>(Wb + (size_t)r * C + piece_chan(pc)) = tpc[n];
        }
    }
    if (gtid < (kCW - 1) * PPR) {
        const int r = gtid / PPR, pc = gtid % PPR;
        *reinterpret_cast<uint4*>(&sm.win[r][8 * pc]) = hpc;
        if (qk_writer && Wb) *reinterpret_cast<uint4*>(Wb + (size_t)r * C + piece_chan(pc)) = hpc;
    }
    conv_chunk(0);
    // stores through buffer resources whose range is empty when the output is not wanted (or, for
    // o, past the window): one unconditional instruction each, so the compiler counts them
    // exactly when it waits for the next row block's loads
    constexpr int kNt = 2;                       // cache policy: non-temporal
    const __amdgpu_buffer_rsrc_t rck = __builtin_amdgcn_make_buffer_rsrc(
        a.S_ckpt ? a.S_ckpt + hb : nullptr, 0, a.S_ckpt ? (int)(SD * 4) : 0, 0x00020000);
    constexpr int OE = O_BF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        a.o ? reinterpret_cast<char*>(a.o) + (size_t)b * K * Hv * dv * OE : nullptr, 0,
        a.o ? K * Hv * dv * OE : 0, 0x00020000);
    // the checkpoint: this window's start state
    auto store_ckpt = [&](int ir, f32x4_t v) __attribute__((always_inline)) {
        typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rck,
                                               live ? ((ir * DK + c) * 4) : 0x7ffffff0, 0, kNt);
    };
    store_ckpt(i, S0);
    GDN_TL(1);
    __syncthreads();
    GDN_TL(2);

    // ---- per row block: the token recurrence, chunk by chunk, state in registers; per token, with
    // the row sums over the row's lanes (DPP):
    //   p = S k^_t,  u = beta_t (v_t - gamma_t p),  S = gamma_t S + u k^_t,  o_t = S q^_t
    f32x4_t S = live ? S0 : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const size_t Hstep = (size_t)Hv * SD;
    constexpr int NO = (KMAX + LPR - 1) / LPR;   // outputs held per lane: lane j keeps o_{j + m LPR}
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int ir = i + r * RPG;              // this lane's row in block r
        float* Hrow = CAPTURE ? a.H + ((size_t)b * (K - 1) * Hv + h) * SD + (size_t)ir * DK + c : nullptr;
        float* Srow = a.S_out + hb + (size_t)ir * DK + c;
        // the next block's start state, taps and v rows, before this block's stores
        f32x4_t Sn = S;
        if (r + 1 < RB) {
            Sn = load_f4(Sh + (size_t)(ir + RPG) * DK + c);
            if (v_wave) {
                const size_t vc = vch + (size_t)(r + 1) * RPG;
                vt0 = *reinterpret_cast<const float4*>(a.w + vc * kCW);
                vt1 = *reinterpret_cast<const float4*>(a.w + (vc + 1) * kCW);
#pragma unroll
                for (int n = 0; n < NVP; ++n) {
                    const int t = (lane + 64 * n) / NPR;
                    const int tl = t < K ? t : K - 1;
#pragma unroll
                    for (int m = 0; m < kCW; ++m)
                        vrow[n][m] = *reinterpret_cast<const uint32_t*>(wrow(tl + m) + vc);
                }
            }
        }
        float ot[NO];
#pragma unroll
        for (int m = 0; m < NO; ++m) ot[m] = 0.f;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
            for (int tt0 = 0; tt0 < (cc == 0 ? T0 : TC); ++tt0) {
                const int t = chunk_start(cc) + tt0;
                if (t < KMAX && t < K) {
                    const float4 tk = sm.tok[g][t];          // beta, gamma, 1/|k|, 1/|q|
                    const float4 kx = lds4<true>(&sm.k[t][c]);
                    const float v = sm.V[r & 1][g][t][rloc];
                    const float sk = group_sum<LPR>(S[0] * kx.x + S[1] * kx.y + S[2] * kx.z + S[3] * kx.w) * tk.z;
                    const float cu = tk.x * (v - tk.y * sk) * tk.z;   // u / |k_t|
                    S[0] = __builtin_fmaf(cu, kx.x, tk.y * S[0]);
                    S[1] = __builtin_fmaf(cu, kx.y, tk.y * S[1]);
                    S[2] = __builtin_fmaf(cu, kx.z, tk.y * S[2]);
                    S[3] = __builtin_fmaf(cu, kx.w, tk.y * S[3]);
                    if constexpr (CAPTURE) {
                        float* dst = t < K - 1 ? Hrow + (size_t)t * Hstep : Srow;
                        if (live) store_f4<true>(dst, S);
                    } else {
                        if (live && t == K - 1) store_f4<true>(Srow, S);
                    }
                    if (r == 0 && t == 0) GDN_TL(3);
                    if (a.o) {
                        const float4 qx = lds4<true>(&sm.q[t][c]);
                        const float o = group_sum<LPR>(S[0] * qx.x + S[1] * qx.y + S[2] * qx.z + S[3] * qx.w) * tk.w;
                        if (j == t % LPR) ot[t / LPR] = o;
                    }
                }
            }
            if (r == 0 && cc + 1 < NC) {
                conv_chunk(cc + 1);
                __syncthreads();
            }
        }
#pragma unroll
        for (int m = 0; m < NO; ++m) {
            const int t = m * LPR + j;
            const int off = live && t < K ? ((t * Hv + h) * dv + ir) * OE : 0x7ffffff0;
            if constexpr (O_BF16)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(ot[m]), ro, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ot[m]), ro, off, 0, 0);
        }
        if (r + 1 < RB) {
            // the next block: its checkpoint, then its v conv (v waves), then one barrier (V of the
            // next block is written into the other buffer)
            S = Sn;
            store_ckpt(ir + RPG, S);
            vconv(r + 1);
            __syncthreads();
        }
    }
    GDN_TL(4);
    GDN_TL_END();
}

template <int DK, int KMAX, bool O_BF16, bool CAPTURE, bool LIVE>
hipError_t launch_rb(const VerifyArgs& a, int rb, hipStream_t s)
{
    constexpr int RPG = kWaves * (64 / (DK / 4));
    const dim3 block(kStepThreads);
    if constexpr (CAPTURE && LIVE && KMAX <= 16) {
        if (rb == 2) {
            const dim3 grid((a.dv + 2 * RPG - 1) / (2 * RPG), a.Hv / kGroups, a.B);
            step_kernel<DK, KMAX, O_BF16, CAPTURE, LIVE, 2><<<grid, block, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    const dim3 grid((a.dv + RPG - 1) / RPG, a.Hv / kGroups, a.B);
    step_kernel<DK, KMAX, O_BF16, CAPTURE, LIVE, 1><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

template <int DK, bool O_BF16, bool CAPTURE, bool LIVE>
hipError_t launch_k(const VerifyArgs& a, hipStream_t s)
{
    // two row blocks per workgroup once the launch has at least sixteen workgroups per CU that way
    // (B = 32 at K = 8: 189 us against 191 with four blocks and 252 with one)
    constexpr int RPG = kWaves * (64 / (DK / 4));
    const long long wg2 = (long long)a.B * (a.Hv / kGroups) * (a.dv / (2 * RPG));
    const int rb = (CAPTURE && LIVE && a.K <= 16 && a.dv % (2 * RPG) == 0 && wg2 >= 16 * 256) ? 2 : 1;
    if (a.K <= 1) return launch_rb<DK, 1, O_BF16, CAPTURE, LIVE>(a, rb, s);
    if (a.K <= 2) return launch_rb<DK, 2, O_BF16, CAPTURE, LIVE>(a, rb, s);
    if (a.K <= 4) return launch_rb<DK, 4, O_BF16, CAPTURE, LIVE>(a, rb, s);
    if (a.K <= 8) return launch_rb<DK, 8, O_BF16, CAPTURE, LIVE>(a, rb, s);
    if (a.K <= 16) return launch_rb<DK, 16, O_BF16, CAPTURE, LIVE>(a, rb, s);
    if (a.K <= 32) return launch_rb<DK, 32, O_BF16, CAPTURE, LIVE>(a, rb, s);
    return launch_rb<DK, 64, O_BF16, CAPTURE, LIVE>(a, rb, s);
}

template <int DK, bool O_BF16>
hipError_t launch_dk(const VerifyArgs& a, hipStream_t s)
{
    // dk 128 takes 8 rows per head and workgroup, so every row is live (dv is a multiple of 8);
    // dk 64 and 32 take 16 and 32 and keep the per-row check
    constexpr bool LIVE = DK == 128;
    return a.H ? launch_k<DK, O_BF16, true, LIVE>(a, s) : launch_k<DK, O_BF16, false, LIVE>(a, s);
}

template <bool O_BF16>
hipError_t launch_o(const VerifyArgs& a, hipStream_t s)
{
    switch (a.dk) {
    case 32: return launch_dk<32, O_BF16>(a, s);
    case 64: return launch_dk<64, O_BF16>(a, s);
    case 128: return launch_dk<128, O_BF16>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_step(const VerifyArgs& a, bool in_bf16, bool o_bf16, hipStream_t s)
{
    // bf16 slabs whose value heads come in groups of three per key head take the pipelined
    // kernel; other shapes the verify kernel's fused-step mode (same results)
    // (its buffer-resource offsets are 32-bit: an o plane of one sequence below 2 GiB)
    if (in_bf16 && (a.Hv / a.Hk) % kGroups == 0 && (long long)a.K * a.Hv * a.dv * 4 < (1LL << 31))
        return o_bf16 ? launch_o<true>(a, s) : launch_o<false>(a, s);
    return launch_verify(a, in_bf16, o_bf16, s);
}

}  // namespace gdn

GDN_CLAMP_READER(clamped_accepts_step)

#ifdef GDN_TIMELINE
// the marks of the last launches: [workgroup][wave][mark] 100 MHz counter values (0: not reached)
GDN_TIMELINE_READER(gdn_timeline)
#endif
