// gdn_prefill_c64.hip -- chunked prefill for dk = 128 and chunks of 64 tokens
// (bf16 q|k|v slab), the chunkwise WY form on MFMA.
//
// Per chunk of L = 64 tokens and value head (G_t the running sum of the gates
// g from the chunk start, k^ = rk k and q^ = rq q the L2-normalised raw
// vectors, S the state at the chunk start), as in the Gated Delta Networks
// paper (Yang, Kautz and Hatamizadeh, ICLR 2025, section 3.3,
// hardware-efficient chunkwise training):
//   A[t][s] = beta_t e^{G_t-G_s} k^_t.k^_s                 (s < t)
//   (I + A) U = beta V - diag(beta e^G) K^ S^T              U, V: L x dv
//   O[t]    = e^{G_t} S q^_t + sum_{s<=t} e^{G_t-G_s} (q^_t.k^_s) u_s
//   S'      = e^{G_L} S + sum_s e^{G_L-G_s} u_s k^_s^T
// the same values as the token recurrence up to rounding.
//
// Workgroup: 8 waves for 128 state rows of one (sequence, value head), one
// workgroup per CU, two waves per SIMD:
//   state waves (4): each owns 32 state rows for the whole prompt, kept in
//     registers as MFMA accumulator tiles of S^T (lane r <-> state rows 2r and
//     2r + 1, one per 16-row tile, 8 key tiles each).  Per chunk: P = K S^T and R = Q S^T
//     with the state split into bf16 hi + lo (one read of each K and Q
//     operand serves both row tiles), the right-hand sides and the state part
//     of O; then block forward substitution for U, O += M U and
//     S^T <- e^{G_L} S^T + K^T diag(e^{G_L-G} rk) U.  Products over two
//     16-token blocks use the 16x16x32 MFMA (on gfx950 the 16x16x16 form takes
//     as long for half the work).
//   prep waves (4): for the next chunk meanwhile.  Phase 1: prep wave p stages
//     token tile p (raw q, k in operand order; the state update reads its K^T
//     operands from the same k tiles with transposing LDS reads) and the
//     tile's norms (a token's pieces are one row of 16 lanes: DPP sums), the
//     gates of all 64 tokens (every prep wave forms them; a wave-wide DPP scan
//     gives the running sums) and the diagonal block p of A, which needs this
//     tile only.  Phase 2: the inverse of that block, (I + N)^-1 =
//     (I - N)(I + N^2)(I + N^4)(I + N^8) for the strictly lower 16x16 block N,
//     on MFMA, and four more gram tiles (K K^T and K Q^T scaled to -A and M,
//     stored as bf16 hi/lo pairs).
// Two LDS buffers hold the chunk operands (chunk c read by the state waves,
// chunk c+1 written by the prep waves); two barriers per chunk separate the
// phases: [state: P, R, X | prep: stage c+1, its gates] [state: solve, O, S |
// prep: grams and inverses of c+1].  The v values go straight from memory into
// the state waves' registers, a chunk ahead.  The prep waves run at a higher
// wave priority: each SIMD holds one wave of each role, the preparation was the
// longer of the two in both phases, and its instructions now go first whenever
// both waves are ready.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_timeline.h"
#include "gdn_wy_mfma.h"

namespace gdn {
namespace {

using namespace wy;

constexpr int kDK = 128;                         // key dimension
constexpr int kL = 64;                           // chunk length
constexpr int kSW = 4;                           // state waves (32 rows each)
constexpr int kPW = 4;                           // prep waves
constexpr int kC64Threads = 64 * (kSW + kPW);
constexpr int kC64Rows = 32 * kSW;

struct C64Chunk {
    bf16x8_t qop[4][4][64];      // raw q: [token tile][32-key slice][record]; record of lane (r, g):
                                 // token 16 tile + r, keys 32 slice + pi(g, 0..7)
    bf16x8_t kop[4][4][64];      // raw k, same order (any 4 consecutive keys of a token, aligned to 4,
                                 // are 8 contiguous bytes: the K^T operands are read from here with
                                 // transposing reads)
    uint2 Ah[6][64], Al[6][64];  // -A tiles (ib > kb, row order), 16x16x16 A-operand order, bf16 hi / lo
    uint2 Th[4][64], Tl[4][64];  // (I + A_ii)^-1
    uint2 Mh[10][64], Ml[10][64];  // M tiles (kb <= ib, row order)
    float fb[64];                // beta_t
    float fa[64];                // beta_t e^{G_t} rk_t
    float fe[64];                // e^{G_t} rq_t
    float fc[64];                // e^{G_L - G_t} rk_t
    float eGL;                   // e^{G_L}
    float pad[3];
};

struct C64Smem {
    C64Chunk ch[2];
    float rk[64], rq[64];        // 1/|k|, 1/|q| of the chunk being prepared (0 past the prompt)
    // per prep wave: the factors of its gram tiles
    float Gv[kPW][64];           // G_t
    float bk[kPW][64];           // beta_t rk_t
    float fs[kPW][64];           // rk_s e^{G_end(block of s) - G_s}
    float E[kPW][3][64];         // e^{G_t - G_end(kb)} for blocks kb before t's block, else 0
};

// gram tiles besides the diagonal blocks of A, five per prep wave with its own diagonal block:
// entry = M tile | ib << 1 | kb << 3
constexpr uint8_t kTile(int m, int ib, int kb) { return (uint8_t)(m | (ib << 1) | (kb << 3)); }
__constant__ const uint8_t kC64Tiles[16] = {
    kTile(1, 0, 0), kTile(1, 3, 0), kTile(1, 3, 1), kTile(0, 3, 0),
    kTile(1, 1, 0), kTile(1, 1, 1), kTile(1, 3, 2), kTile(0, 3, 1),
    kTile(1, 2, 0), kTile(1, 2, 1), kTile(0, 1, 0), kTile(0, 3, 2),
    kTile(1, 2, 2), kTile(1, 3, 3), kTile(0, 2, 0), kTile(0, 2, 1),
};

// a DPP move with row mask; lanes whose source lies outside their row, or whose row is masked
// off, read 0
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp0(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

// inclusive prefix sum over the 64 lanes: shifts inside each row of 16, then the
// row ends broadcast to the rows after them
__device__ __forceinline__ float wave_scan(float x)
{
    x += dpp0<0x111, 0xF>(x);   // row_shr:1
    x += dpp0<0x112, 0xF>(x);   // row_shr:2
    x += dpp0<0x114, 0xF>(x);   // row_shr:4
    x += dpp0<0x118, 0xF>(x);   // row_shr:8
    x += dpp0<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp0<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// transposing LDS read of 4 bf16 (see the K^T operand in the state update for the lane mapping)
typedef short v4i16_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 tr16(const char* p)
{
    typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
    const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
    return __builtin_bit_cast(uint2, v);
}

// hi/lo pair of a 16x16 tile in one operand order
struct HL {
    uint2 h, l;
};

__device__ __forceinline__ HL split(const f32x4_t x)
{
    HL r;
    split4(x, r.h, r.l);
    return r;
}

// X Y for X, Y given as hi/lo operands (X in A order, Y in B order), result in accumulator order
__device__ __forceinline__ f32x4_t mm16(const HL& x, const HL& y, f32x4_t c)
{
    c = mfma16(x.h, y.h, c);
    c = mfma16(x.h, y.l, c);
    c = mfma16(x.l, y.h, c);
    return c;
}

// the same over 32 contraction indices: two tiles side by side on each side
__device__ __forceinline__ f32x4_t mm32(const HL& x0, const HL& x1, const HL& y0, const HL& y1, f32x4_t c)
{
    c = mfma32(as8(x0.h, x1.h), as8(y0.h, y1.h), c);
    c = mfma32(as8(x0.h, x1.h), as8(y0.l, y1.l), c);
    c = mfma32(as8(x0.l, x1.l), as8(y0.h, y1.h), c);
    return c;
}

template <bool O_BF16>
__global__ __launch_bounds__(kC64Threads) void prefill_c64_kernel(PrefillArgs a)
{
    constexpr int OE = O_BF16 ? 2 : 4;
    __shared__ C64Smem sm;
    GDN_TL_BEGIN();

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int b = blockIdx.z;
    const int T = a.T, Hk = a.Hk, Hv = a.Hv, dv = a.dv;
    const int h = head_of_row(blockIdx.y, Hv, Hk, gridDim.x);
    const int C = 2 * Hk * kDK + Hv * dv;
    const int hk = h / (Hv / Hk);
    const uint16_t* qkv = reinterpret_cast<const uint16_t*>(a.qkv);
    auto chunk_rsrc = [&](int c0) __attribute__((always_inline)) {
        // the chunk's tokens of the slab: loads past the prompt read as zero
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qkv + ((size_t)b * T + c0) * C), 0,
                                                 min(kL, T - c0) * C * 2, kBufferFlags);
    };

    if (wave >= kSW) {
        // ============================================================ prep waves
        const int p = __builtin_amdgcn_readfirstlane(wave - kSW);
        // the preparation is the longer role of both phases and shares each SIMD with a state wave:
        // its instructions go first when both are ready (383-389 us against 419 at the default)
        __builtin_amdgcn_s_setprio(1);
        // staging: lane (u, jp) = (lane / 16, lane mod 16) takes piece jp (keys 8 jp .. 8 jp + 7) of token
        // 16 p + 4 i + u in pass i, so a token's 16 pieces sit in one row of 16 lanes (DPP sums)
        const int jp = lane & 15, u = lane >> 4;
        uint4 qreg[4], kreg[4];
        // lane t: raw beta and raw alpha of token t, each in its own register (combining them at load
        // time would wait for the prefetch right away)
        uint32_t gbr = 0, gal = 0;
        float dtb, eal;                           // the head's dt_bias and e^{A_log}
        head_gate_consts(a.dt_bias, a.A_log, h, dtb, eal);
        const bool raw_gates = a.dt_bias != nullptr;
        float gbeta = 0.f, gG = 0.f;              // lane t: beta_t and G_t of the chunk staged last
        f32x4_t gNa, gNb;                         // diagonal block p of A of the chunk staged last, A and B order
        const int qoff = ((16 * p + u) * C + hk * kDK + 8 * jp) * 2;
        auto prefetch = [&](int c0) __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t rq = chunk_rsrc(c0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int so = __builtin_amdgcn_readfirstlane(8 * i * C);   // 4 i tokens further
                qreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff, so, 0));
                kreg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rq, qoff, __builtin_amdgcn_readfirstlane(so + Hk * kDK * 2), 0));
            }
            const int Lv = min(kL, T - c0);
            const size_t g0 = ((size_t)b * T + c0) * Hv;
            const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.beta_raw) + g0), 0, Lv * Hv * 2, kBufferFlags);
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a.alpha) + g0), 0, Lv * Hv * 2, kBufferFlags);
            const int goff = (lane * Hv + h) * 2;
            gbr = __builtin_amdgcn_raw_buffer_load_b16(rb, goff, 0, 0);
            gal = __builtin_amdgcn_raw_buffer_load_b16(ra, goff, 0, 0);
        };

        // raw gram tile of buffer x: lane (r, g) element e holds k_{16 kb + 4 g + e} . (q or k)_{16 ib + r}
        auto gram = [&](const C64Chunk& x, int ib, int kb, bool ism) __attribute__((always_inline)) {
            f32x4_t D = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int rec = qk_rec(lane, m);
                const bf16x8_t* xs = ism ? &x.qop[ib][m][0] : &x.kop[ib][m][0];
                D = mfma32(x.kop[kb][m][rec], xs[rec], D);
            }
            return D;
        };

        // phase 1: token tile p of the chunk at c0 into buffer x, its norms, the gates of all tokens, and
        // the diagonal block p of A (it needs this tile only)
        auto stage = [&](int c0, C64Chunk& x, bool mk) __attribute__((always_inline)) {
            const int Lv = min(kL, T - c0);
            if (mk) GDN_TLV(5, qreg[3].w);
            const int m = jp >> 2, hf = (jp & 3) >> 1, g0 = (jp & 1) << 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 q = qreg[i], k = kreg[i];
                const int row = 4 * i + u, t = 16 * p + row;
                // keys 8 jp + 0..3 -> group g0 (slots 4 hf ..), keys + 4..7 -> group g0 + 1
                char* qd = reinterpret_cast<char*>(&x.qop[p][m][0]) + 8 * hf;
                char* kd = reinterpret_cast<char*>(&x.kop[p][m][0]) + 8 * hf;
                const int r0 = qk_rec(row + 16 * g0, m) * 16, r1 = qk_rec(row + 16 * (g0 + 1), m) * 16;
                *reinterpret_cast<uint2*>(qd + r0) = make_uint2(q.x, q.y);
                *reinterpret_cast<uint2*>(qd + r1) = make_uint2(q.z, q.w);
                *reinterpret_cast<uint2*>(kd + r0) = make_uint2(k.x, k.y);
                *reinterpret_cast<uint2*>(kd + r1) = make_uint2(k.z, k.w);
                // norms: the token's 16 pieces are one row of lanes
                const float sq = group_sum<16>(sq8(q, 0.f)), sk = group_sum<16>(sq8(k, 0.f));
                if (jp == 0) {
                    const bool valid = t < Lv;
                    sm.rk[t] = valid ? __builtin_amdgcn_rsqf(sk + a.eps) : 0.f;
                    sm.rq[t] = valid ? __builtin_amdgcn_rsqf(sq + a.eps) : 0.f;
                }
            }
            if (mk) GDN_TL(6);
            if (mk) GDN_TL(7);
            // the gates (lane = token) and their running sum, from the raw bits loaded with the chunk
            // (the next prefetch overwrites them)
            float beta = 0.f, gg = 0.f;
            if (lane < Lv) gate(bf16_lo(gbr), bf16_lo(gal), raw_gates, dtb, eal, beta, gg);
            gbeta = beta;
            gG = wave_scan(gg);
            if (mk) GDN_TLV(8, gG);
            // the diagonal block p of A in both operand orders (its tokens, norms and gates are this
            // wave's own)
            if ((lane >> 4) == p) {
                sm.Gv[p][lane] = gG;
                sm.bk[p][lane] = gbeta * sm.rk[lane];
            }
            const f32x4_t D = gram(x, p, p, false);   // symmetric: k_{4g+e} . k_r of block p
            const int t = 16 * p + r, s0 = 16 * p + 4 * g;
            const float bkt = sm.bk[p][t], Gt = sm.Gv[p][t], rkr = sm.rk[t];
            const float4 bks = lds_f4(&sm.bk[p][s0]), Gs = lds_f4(&sm.Gv[p][s0]), rks = lds_f4(&sm.rk[s0]);
            const float bk4[4] = {bks.x, bks.y, bks.z, bks.w}, G4[4] = {Gs.x, Gs.y, Gs.z, Gs.w};
            const float rk4[4] = {rks.x, rks.y, rks.z, rks.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sc = 4 * g + e;
                // A order: N[r][sc]; B order: N[sc][r]
                gNa[e] = sc < r ? bkt * rk4[e] * __expf(fminf(Gt - G4[e], 0.f)) * D[e] : 0.f;
                gNb[e] = r < sc ? bk4[e] * rkr * __expf(fminf(G4[e] - Gt, 0.f)) * D[e] : 0.f;
            }
            if (mk) GDN_TLV(10, gNb[0]);
        };

        // phase 2: the gate factors, this wave's gram tiles and its diagonal block's inverse, for
        // the chunk staged last (buffer x)
        auto build = [&](C64Chunk& x, bool mk) __attribute__((always_inline)) {
            const float beta = gbeta, G = gG;
            const float GL = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
            float Ge[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                Ge[kb] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 16 * kb + 15));
            const int blk = lane >> 4;
            const float ge = blk == 0 ? Ge[0] : (blk == 1 ? Ge[1] : (blk == 2 ? Ge[2] : Ge[3]));
            const float rkt = sm.rk[lane], rqt = sm.rq[lane];
            sm.Gv[p][lane] = G;
            sm.bk[p][lane] = beta * rkt;
            sm.fs[p][lane] = rkt * __expf(fminf(ge - G, 0.f));
#pragma unroll
            for (int kb = 0; kb < 3; ++kb) sm.E[p][kb][lane] = kb < blk ? __expf(fminf(G - Ge[kb], 0.f)) : 0.f;
            if (p == 0) {
                const float eg = __expf(G);
                x.fb[lane] = beta;
                x.fa[lane] = beta * eg * rkt;
                x.fe[lane] = eg * rqt;
                x.fc[lane] = __expf(GL - G) * rkt;
                if (lane == 0) x.eGL = __expf(GL);
            }

            if (mk) GDN_TL(9);
            // the inverse of the diagonal block p (formed at staging)
            {
                const f32x4_t Na = gNa, Nb = gNb;
                // (I + N)^-1 in A order is (I + M)^-1 of M = N^T in accumulator order:
                // (I - M)(I + M^2)(I + M^4)(I + M^8), M^16 = 0.  The A order of M is N's B order and
                // the B order of M is N's A order; a product's accumulator order is the B order of
                // the product and the A order of its transpose, so M^k and N^k are formed together.
                const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
                const HL na = split(Na), nb = split(Nb);
                const HL q2 = split(mm16(nb, na, z));        // M^2   (accumulator order)
                const HL n2 = split(mm16(na, nb, z));        // N^2   (= A order of M^2)
                const f32x4_t Q4 = mm16(n2, q2, z);           // M^4
                const HL q4 = split(Q4);
                const HL n4 = split(mm16(q2, n2, z));        // N^4   (= A order of M^4)
                const f32x4_t Q8 = mm16(n4, q4, z);           // M^8
                const HL q8 = split(Q8);
                const f32x4_t Q12 = mm16(n4, q8, z);          // M^12
                f32x4_t Y;
#pragma unroll
                for (int e = 0; e < 4; ++e) Y[e] = (4 * g + e == r ? 1.f : 0.f) + Q4[e] + Q8[e] + Q12[e];
                const HL y = split(Y);                        // (I + M^4)(I + M^8)
                const f32x4_t Z = mm16(n2, y, Y);             // (I + M^2) Y
                const HL zz = split(Z);
                const f32x4_t MZ = mm16(nb, zz, z);
                f32x4_t Ti;
#pragma unroll
                for (int e = 0; e < 4; ++e) Ti[e] = Z[e] - MZ[e];   // (I - M) Z = T^T, i.e. T in A order
                split4(Ti, x.Th[p][lane], x.Tl[p][lane]);
                if (mk) GDN_TL(11);
            }

            // four more tiles: -A below the diagonal, M on and below it
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ent = kC64Tiles[4 * p + i];
                const bool ism = ent & 1;
                const int ib = (ent >> 1) & 3, kb = (ent >> 3) & 3;
                const f32x4_t D = gram(x, ib, kb, ism);
                // lane: row t of tile (ib, kb), columns s = 16 kb + 4 g + e
                const int t = 16 * ib + r, s0 = 16 * kb + 4 * g;
                float y[4];
                if (kb < ib) {
                    // e^{G_t - G_s} = E[kb][t] (rk_s fs factor)
                    const float4 fs4 = lds_f4(&sm.fs[p][s0]);
                    const float f4[4] = {fs4.x, fs4.y, fs4.z, fs4.w};
                    const float ct = (ism ? sm.rq[t] : sm.bk[p][t]) * sm.E[p][kb][t];
#pragma unroll
                    for (int e = 0; e < 4; ++e) y[e] = ct * f4[e] * D[e];
                } else {
                    const float ct = ism ? sm.rq[t] : sm.bk[p][t];
                    const float Gt = sm.Gv[p][t];
                    const float4 Gs = lds_f4(&sm.Gv[p][s0]), rks = lds_f4(&sm.rk[s0]);
                    const float G4[4] = {Gs.x, Gs.y, Gs.z, Gs.w}, rk4[4] = {rks.x, rks.y, rks.z, rks.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool in = ism ? 4 * g + e <= r : 4 * g + e < r;
                        y[e] = in ? ct * rk4[e] * __expf(fminf(Gt - G4[e], 0.f)) * D[e] : 0.f;
                    }
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
            if (mk) GDN_TL(12);
        };

        prefetch(0);
        stage(0, sm.ch[0], false);
        if (kL < T) prefetch(kL);
        __syncthreads();
        build(sm.ch[0], false);
        __syncthreads();
        for (int c0 = 0, it = 0; c0 < T; c0 += kL, ++it) {
            const bool more = c0 + kL < T;
            C64Chunk& nxt = sm.ch[(it & 1) ^ 1];
            if (it == 10) GDN_TL(0);
            if (more) {
                stage(c0 + kL, nxt, it == 10);
                // the next loads only once this chunk's registers are written to LDS
                asm volatile("" ::: "memory");
                if (c0 + 2 * kL < T) prefetch(c0 + 2 * kL);
            }
            if (it == 10) GDN_TL(1);
            __syncthreads();
            if (it == 10) GDN_TL(2);
            if (more) build(nxt, it == 10);
            if (it == 10) GDN_TL(3);
            __syncthreads();
            if (it == 10) GDN_TL(4);
        }
        GDN_TL_END();
        return;
    }

    // ================================================================ state waves
    // rows of this lane: 32 wave + 2 r + rt of the workgroup's block (two adjacent rows, so each v
    // load and o store covers both); rows past dv carry zeros and store nothing (dv is even: both
    // rows or neither)
    const int row0 = blockIdx.x * kC64Rows + 32 * wave + 2 * r;
    const bool live0 = row0 < dv, live1 = row0 + 1 < dv;
    f32x4_t S[8][2];                 // S^T tiles: S[jt][rt] lane (r, g) e = S[row][16 jt + 4 g + e]
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const bool lv = rt ? live1 : live0;
        const float* sp = a.S_in + (((size_t)b * Hv + h) * dv + (lv ? row0 + rt : 0)) * kDK + 4 * g;
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            const f32x4_t v = load_f4(sp + 16 * jt);
            S[jt][rt] = lv ? v : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    // v[token 16 tt + 4 g + e][row of rt] of the chunk to process next (raw bf16)
    uint32_t vreg[4][4];             // v of rows row0, row0 + 1 (bf16 pair) for token 16 tt + 4 g + e
    // rows past dv address past the resource and read zeros (no select per value)
    const int voff = live0 ? ((4 * g) * C + 2 * Hk * kDK + h * dv + row0) * 2 : 0x7ffffff0;
    auto prefetch_v = [&](int c0) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rv = chunk_rsrc(c0);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int so = __builtin_amdgcn_readfirstlane((16 * tt + e) * C * 2);
                vreg[tt][e] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff, so, 0);
            }
    };
    prefetch_v(0);
    __syncthreads();
    __syncthreads();

    for (int c0 = 0, it = 0; c0 < T; c0 += kL, ++it) {
        const int Lv = min(kL, T - c0);
        const bool more = c0 + kL < T;
        const C64Chunk& cur = sm.ch[it & 1];
        if (it == 10) GDN_TL(0);
        // ================= phase 1: P = K S^T, R = Q S^T -> right-hand sides X and the state part of O
        f32x4_t X[4][2], O[4][2];
        {
            f32x4_t P[4][2], R[4][2];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    P[tt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    R[tt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // the state's columns of key slice m as bf16 hi + lo, once for all token tiles
                bf16x8_t shi[2], slo[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    uint2 h0, l0, h1, l1;
                    split4(S[2 * m][rt], h0, l0);
                    split4(S[2 * m + 1][rt], h1, l1);
                    shi[rt] = as8(h0, h1);
                    slo[rt] = as8(l0, l1);
                }
                const int rec = qk_rec(lane, m);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const bf16x8_t ka = cur.kop[tt][m][rec];
                    const bf16x8_t qa = cur.qop[tt][m][rec];
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) {
                        P[tt][rt] = mfma32(ka, shi[rt], P[tt][rt]);
                        P[tt][rt] = mfma32(ka, slo[rt], P[tt][rt]);
                        R[tt][rt] = mfma32(qa, shi[rt], R[tt][rt]);
                        R[tt][rt] = mfma32(qa, slo[rt], R[tt][rt]);
                    }
                }
            }
            if (it == 10) GDN_TLV(15, P[3][1][0]);
            // X = beta v - beta e^{G} rk P, O = e^{G} rq R (token t = 16 tt + 4 g + e)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int t0 = 16 * tt + 4 * g;
                const float4 fb4 = lds_f4(&cur.fb[t0]), fa4 = lds_f4(&cur.fa[t0]), fe4 = lds_f4(&cur.fe[t0]);
                const float bv[4] = {fb4.x, fb4.y, fb4.z, fb4.w}, av[4] = {fa4.x, fa4.y, fa4.z, fa4.w};
                const float ev[4] = {fe4.x, fe4.y, fe4.z, fe4.w};
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = rt ? bf16_hi(vreg[tt][e]) : bf16_lo(vreg[tt][e]);
                        X[tt][rt][e] = __builtin_fmaf(-av[e], P[tt][rt][e], bv[e] * v);
                        O[tt][rt][e] = ev[e] * R[tt][rt][e];
                    }
                }
            }
        }
        if (it == 10) GDN_TL(1);
        __syncthreads();
        if (it == 10) GDN_TL(2);

        // ================= phase 2: U by block forward substitution, the outputs, the state update
        {
            const float eGL = cur.eGL;
#pragma unroll
            for (int jt = 0; jt < 8; ++jt)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[jt][rt][e] *= eGL;
            const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
                reinterpret_cast<char*>(a.o) + ((size_t)b * T + c0) * Hv * dv * OE, 0, Lv * Hv * dv * OE,
                kBufferFlags);
            // rows past dv and tokens past the prompt fall outside the resource: dropped
            const int ostride = Hv * dv * OE;
            const int obase = ((4 * g * Hv + h) * dv + row0) * OE;
            const int ooff = live0 ? obase : 0x7ffffff0;
            HL U[4][2], CU[4][2];
            auto tileA = [&](int ib, int kb) __attribute__((always_inline)) {
                const int ia = ib * (ib - 1) / 2 + kb;
                return HL{cur.Ah[ia][lane], cur.Al[ia][lane]};
            };
            auto tileM = [&](int ib, int kb) __attribute__((always_inline)) {
                const int im = ib * (ib + 1) / 2 + kb;
                return HL{cur.Mh[im][lane], cur.Ml[im][lane]};
            };
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                // U_ib = T_ib (X_ib - sum_{kb < ib} A_ib,kb U_kb)
                const HL Ti{cur.Th[ib][lane], cur.Tl[ib][lane]};
                HL A01[2], A2;
                if (ib >= 2) {
                    A01[0] = tileA(ib, 0);
                    A01[1] = tileA(ib, 1);
                }
                if (ib == 1) A2 = tileA(1, 0);
                if (ib == 3) A2 = tileA(3, 2);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    f32x4_t x = X[ib][rt];
                    if (ib == 1) x = mm16(A2, U[0][rt], x);
                    if (ib >= 2) x = mm32(A01[0], A01[1], U[0][rt], U[1][rt], x);
                    if (ib == 3) x = mm16(A2, U[2][rt], x);
                    const HL xs = split(x);
                    const f32x4_t u = mm16(Ti, xs, f32x4_t{0.f, 0.f, 0.f, 0.f});
                    U[ib][rt] = split(u);
                    // c_t u_t, c_t = e^{G_L - G_t} rk_t: operand of the state update
                    const float4 fc4 = lds_f4(&cur.fc[16 * ib + 4 * g]);
                    CU[ib][rt] = split(f32x4_t{fc4.x * u[0], fc4.y * u[1], fc4.z * u[2], fc4.w * u[3]});
                }
                // O_ib += sum_{kb <= ib} M_ib,kb U_kb
                HL M0, M1, M2, M3;
                if (ib == 0) M0 = tileM(0, 0);
                if (ib >= 1) {
                    M0 = tileM(ib, 0);
                    M1 = tileM(ib, 1);
                }
                if (ib >= 2) M2 = tileM(ib, 2);
                if (ib == 3) M3 = tileM(3, 3);
                f32x4_t o2[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    f32x4_t o = O[ib][rt];
                    if (ib == 0) o = mm16(M0, U[0][rt], o);
                    if (ib >= 1) o = mm32(M0, M1, U[0][rt], U[1][rt], o);
                    if (ib == 2) o = mm16(M2, U[2][rt], o);
                    if (ib == 3) o = mm32(M2, M3, U[2][rt], U[3][rt], o);
                    o2[rt] = o;
                }
                // both rows of the lane in one store per token
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int so = __builtin_amdgcn_readfirstlane((16 * ib + e) * ostride);   // the token's
                    if constexpr (O_BF16) {
                        const bf16x2_t pr = {(__bf16)o2[0][e], (__bf16)o2[1][e]};
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pr), ro, ooff, so, 0);
                    } else {
                        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
                        const u32x2_t pr = {__float_as_uint(o2[0][e]), __float_as_uint(o2[1][e])};
                        __builtin_amdgcn_raw_buffer_store_b64(pr, ro, ooff, so, 0);
                    }
                }
                if (ib & 1) {
                    // tiles ib-1, ib form the 32-token slice ib/2.  The K^T operand of key tile jt: lane
                    // (r, g) needs k[32 s + pi(g, 0..7)][16 jt + r]; a transposing read hands lane r of
                    // each 16-lane group element r mod 4 of the 4-vector addressed by lane
                    // 4 s' + r / 4 of that group, so lane (j, g) addresses keys 16 jt + 4 (j mod 4) ..
                    // + 3 of token 32 s + 4 g + j / 4 (and + 16 for the second half)
#pragma unroll
                    for (int jt = 0; jt < 8; ++jt) {
                        const int m = jt >> 1, hb = 8 * (jt & 1);
                        const int rec = qk_rec(4 * g + (r >> 2) + 16 * (r & 3), m);
                        const char* k0 = reinterpret_cast<const char*>(&cur.kop[ib - 1][m][rec]) + hb;
                        const char* k1 = reinterpret_cast<const char*>(&cur.kop[ib][m][rec]) + hb;
                        const bf16x8_t ka = as8(tr16(k0), tr16(k1));
#pragma unroll
                        for (int rt = 0; rt < 2; ++rt) {
                            S[jt][rt] = mfma32(ka, as8(CU[ib - 1][rt].h, CU[ib][rt].h), S[jt][rt]);
                            S[jt][rt] = mfma32(ka, as8(CU[ib - 1][rt].l, CU[ib][rt].l), S[jt][rt]);
                        }
                        if (jt % 4 == 3) asm volatile("" ::: "memory");  // four key tiles' operands at a time
                    }
                }
                asm volatile("" ::: "memory");  // one block's operands at a time (registers)
                if (it == 10 && ib == 1) GDN_TLV(13, S[7][1][0]);
            }
        }
        if (it == 10) GDN_TLV(14, S[7][1][0]);
        // the next chunk's v
        if (more) prefetch_v(c0 + kL);
        if (it == 10) GDN_TL(3);
        __syncthreads();
        if (it == 10) GDN_TL(4);
    }

#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        if (rt ? live1 : live0) {
            float* sp = a.S_out + (((size_t)b * Hv + h) * dv + row0 + rt) * kDK + 4 * g;
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) store_f4<false>(sp + 16 * jt, S[jt][rt]);
        }
    }
    GDN_TL_END();
}

}  // namespace

// dk = 128, chunk = 64: one workgroup per (row block of 128, value head, sequence)
hipError_t launch_prefill_c64(const PrefillArgs& a, bool o_bf16, hipStream_t s)
{
    if (a.dk != kDK || a.chunk != kL) return hipErrorInvalidValue;
    const dim3 grid((a.dv + kC64Rows - 1) / kC64Rows, a.Hv, a.B);
    if (o_bf16)
        prefill_c64_kernel<true><<<grid, dim3(kC64Threads), 0, s>>>(a);
    else
        prefill_c64_kernel<false><<<grid, dim3(kC64Threads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace gdn

#ifdef GDN_TIMELINE
GDN_TIMELINE_READER(gdn_timeline_c64)
#endif
