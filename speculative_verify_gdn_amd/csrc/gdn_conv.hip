// gdn_conv.hip -- fused causal depthwise conv1d decode / verify step (gfx950).
//
// One kernel does what the pages describe as replacing transpose / concat /
// ssm_conv / silu / cpy: build the window [history ; new tokens], apply the
// W-tap depthwise conv and SiLU, write the history back in place and keep the
// whole window so that a partial accept can restore the conv state
// (lucebox PR #637, commit message on ggml_ssm_conv_step and the review note
// on its sources; atlas PR #297, commit message on
// causal_conv1d_update_prefill_inter).
//
// The result is bit-exact by construction: every rounding is fixed.
//   pre  = fmaf chain over the taps, oldest first, starting from 0
//   silu = pre / (1 + e^-pre) with the exp below and IEEE division
//   out  = round-to-nearest-even bfloat16 (or the float itself)
// This file is compiled with -ffp-contract=off, IEEE fp32 division and fp32
// denormals kept.
//
// Thread mapping: a thread computes one token of 4 consecutive channels; a
// workgroup is 16 tokens x 16 channel groups (64 channels), so a row access
// is 16 threads x 8 bytes (bf16) contiguous.  Only tokens
// t < W-1 read the old history, and they all sit in the first token tile; the
// threads of that tile that rewrite the history load their new rows first,
// wait at a workgroup barrier for every read of the old history, then store.
#include "gdn_conv_math.h"
#include "gdn_debug.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kCh = 4;          // channels per thread
constexpr int kTok = 16;        // tokens per workgroup; >= W-1
constexpr int kGroups = 16;     // 4-channel groups per workgroup
constexpr int kThreads = kTok * kGroups;

template <bool BF16>
__device__ __forceinline__ void load_row8(const void* base, size_t off, int nch, bool vec, float v[kCh])
{
    if (vec) {
        if constexpr (BF16) {
            const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
            v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        } else {
            const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        }
    } else {
        // ragged channel tail: elements past the row end re-read its last element (unused)
#pragma unroll
        for (int e = 0; e < kCh; ++e) v[e] = load1<BF16>(base, off + (e < nch ? e : nch - 1));
    }
}

template <bool BF16>
__device__ __forceinline__ void store_row8(void* base, size_t off, int nch, bool vec, const float v[kCh])
{
    if (vec) {
        if constexpr (BF16) {
            uint2 u;
            u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
            u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = u;
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < kCh; ++e)
            if (e < nch) store1<BF16>(base, off + e, v[e]);
    }
}

template <bool BF16, int W>
__global__ __launch_bounds__(kThreads) void conv_step_kernel(ConvArgs a)
{
    const int g = threadIdx.x % kGroups, tl = threadIdx.x / kGroups;
    const int c0 = (blockIdx.x * kGroups + g) * kCh;
    const int t = blockIdx.y * kTok + tl;
    const int b = blockIdx.z;
    const int T = a.T, C = a.C;
    const bool active = c0 < C && t < T;
    const int nch = c0 < C ? min(kCh, C - c0) : 0;
    const bool vec = (nch == kCh) && ((C & 3) == 0);
    const size_t xb = (size_t)b * T * C;
    const size_t hb = (size_t)b * (W - 1) * C;

    // window row r (absolute) is history row r for r < W-1, else token r-(W-1);
    // token t reads window rows t .. t+W-1
    float col[W][kCh];
    float wt[kCh][W];
    if (active) {
#pragma unroll
        for (int jj = 0; jj < W; ++jj) {
            const int row = t + jj;
            if (row < W - 1) load_row8<BF16>(a.hist, hb + (size_t)row * C + c0, nch, vec, col[jj]);
            else load_row8<BF16>(a.x, xb + (size_t)(row - (W - 1)) * C + c0, nch, vec, col[jj]);
        }
        // taps of the 4 channels: 4*W consecutive floats (16-byte aligned);
        // channels past C read channel C-1 (unused)
        if (vec) {
            const float4* wp = reinterpret_cast<const float4*>(a.w + (size_t)c0 * W);
            float wl[kCh * W];
#pragma unroll
            for (int q4 = 0; q4 < kCh * W / 4; ++q4) {
                const float4 f = wp[q4];
                wl[4 * q4 + 0] = f.x; wl[4 * q4 + 1] = f.y; wl[4 * q4 + 2] = f.z; wl[4 * q4 + 3] = f.w;
            }
#pragma unroll
            for (int e = 0; e < kCh; ++e)
#pragma unroll
                for (int jj = 0; jj < W; ++jj) wt[e][jj] = wl[e * W + jj];
        } else {
#pragma unroll
            for (int e = 0; e < kCh; ++e) {
                const int ce = c0 + e < C ? c0 + e : C - 1;
#pragma unroll
                for (int jj = 0; jj < W; ++jj) wt[e][jj] = a.w[(size_t)ce * W + jj];
            }
        }
    }
    // first token tile, threads tl < W-1: history row tl of the window (old)
    // and of the new history (window row Tb + tl, Tb = this sequence's tokens)
    float nh[kCh], oh[kCh];
    const bool hist_writer = blockIdx.y == 0 && tl < W - 1 && c0 < C;
    if (hist_writer) {
        load_row8<BF16>(a.hist, hb + (size_t)tl * C + c0, nch, vec, oh);
        const int row = (a.lens ? min(max(a.lens[b], 1), T) : T) + tl;
        if (row < W - 1) load_row8<BF16>(a.hist, hb + (size_t)row * C + c0, nch, vec, nh);
        else load_row8<BF16>(a.x, xb + (size_t)(row - (W - 1)) * C + c0, nch, vec, nh);
        if (a.win) store_row8<BF16>(a.win, (size_t)b * (W - 1 + T) * C + (size_t)tl * C + c0, nch, vec, oh);
    }

    if (active) {
        float out[kCh];
#pragma unroll
        for (int e = 0; e < kCh; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int jj = 0; jj < W; ++jj) acc = __builtin_fmaf(wt[e][jj], col[jj][e], acc);
            out[e] = BF16 ? bf16_to_f32(conv_silu_bf16(acc)) : conv_silu(acc);
        }
        store_row8<BF16>(a.y, xb + (size_t)t * C + c0, nch, vec, out);
        if (a.win) {
            const size_t wb = (size_t)b * (W - 1 + T) * C;
            store_row8<BF16>(a.win, wb + (size_t)(t + W - 1) * C + c0, nch, vec, col[W - 1]);
        }
    }
    __syncthreads();  // every read of the old history in this channel tile is done
    if (hist_writer) store_row8<BF16>(a.hist, hb + (size_t)tl * C + c0, nch, vec, nh);
}

// The rollback of the previous window fused with the conv step of the next
// tokens: exactly gdn_rollback followed by gdn_conv_step, in one launch.
// x of the grid: first the state slabs of the rollback (one float4 per
// thread), then the conv tiles (channel group tile, token tile); y: sequence.
// The conv history is read from the previous window (rows a .. a+W-2, which is
// what the rollback restores into hist) and hist is only written, so no
// workgroup waits for another.
template <bool BF16, int W>
__global__ __launch_bounds__(kThreads) void rollback_conv_kernel(RollConvArgs a, int state_blocks, int cgx)
{
    const int b = blockIdx.y;
    int acc = a.accept[b];
    GDN_COUNT_CLAMP(blockIdx.x == 0 && threadIdx.x == 0 && (acc < 0 || acc > a.Kp));
    acc = acc < 0 ? 0 : (acc > a.Kp ? a.Kp : acc);

    if ((int)blockIdx.x < state_blocks) {
        if (acc == a.Kp) return;
        const float* src = acc == 0 ? a.S_in + (size_t)b * a.state_elems
                                    : a.H + ((size_t)b * (a.Kp - 1) + (acc - 1)) * a.state_elems;
        float* dst = a.S_out + (size_t)b * a.state_elems;
        const long long e = ((long long)blockIdx.x * kThreads + threadIdx.x) * 4;
        if (e < a.state_elems)
            __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + e)),
                                        reinterpret_cast<f32x4_t*>(dst + e));
        return;
    }

    const int bx = blockIdx.x - state_blocks;
    const int g = threadIdx.x % kGroups, tl = threadIdx.x / kGroups;
    const int c0 = ((bx % cgx) * kGroups + g) * kCh;
    const int t = (bx / cgx) * kTok + tl;
    const int T = a.T, C = a.C;
    const bool active = c0 < C && t < T;
    const int nch = c0 < C ? min(kCh, C - c0) : 0;
    const bool vec = (nch == kCh) && ((C & 3) == 0);
    const size_t xb = (size_t)b * T * C;
    const size_t pb = ((size_t)b * (W - 1 + a.Kp) + acc) * C;   // previous window row acc

    // new window row r is previous window row acc + r for r < W-1, else token r-(W-1)
    float col[W][kCh];
    float wt[kCh][W];
    if (active) {
#pragma unroll
        for (int jj = 0; jj < W; ++jj) {
            const int row = t + jj;
            if (row < W - 1) load_row8<BF16>(a.win_prev, pb + (size_t)row * C + c0, nch, vec, col[jj]);
            else load_row8<BF16>(a.x, xb + (size_t)(row - (W - 1)) * C + c0, nch, vec, col[jj]);
        }
        if (vec) {
            const float4* wp = reinterpret_cast<const float4*>(a.w + (size_t)c0 * W);
            float wl[kCh * W];
#pragma unroll
            for (int q4 = 0; q4 < kCh * W / 4; ++q4) {
                const float4 f = wp[q4];
                wl[4 * q4 + 0] = f.x; wl[4 * q4 + 1] = f.y; wl[4 * q4 + 2] = f.z; wl[4 * q4 + 3] = f.w;
            }
#pragma unroll
            for (int e = 0; e < kCh; ++e)
#pragma unroll
                for (int jj = 0; jj < W; ++jj) wt[e][jj] = wl[e * W + jj];
        } else {
#pragma unroll
            for (int e = 0; e < kCh; ++e) {
                const int ce = c0 + e < C ? c0 + e : C - 1;
#pragma unroll
                for (int jj = 0; jj < W; ++jj) wt[e][jj] = a.w[(size_t)ce * W + jj];
            }
        }
    }
    // first token tile, threads tl < W-1: window row tl (the restored history)
    // and the new history (window row T + tl)
    if (bx / cgx == 0 && tl < W - 1 && c0 < C) {
        float oh[kCh], nh[kCh];
        load_row8<BF16>(a.win_prev, pb + (size_t)tl * C + c0, nch, vec, oh);
        const int row = T + tl;
        if (row < W - 1) load_row8<BF16>(a.win_prev, pb + (size_t)row * C + c0, nch, vec, nh);
        else load_row8<BF16>(a.x, xb + (size_t)(row - (W - 1)) * C + c0, nch, vec, nh);
        store_row8<BF16>(a.win, (size_t)b * (W - 1 + T) * C + (size_t)tl * C + c0, nch, vec, oh);
        store_row8<BF16>(a.hist, (size_t)b * (W - 1) * C + (size_t)tl * C + c0, nch, vec, nh);
    }
    if (active) {
        float out[kCh];
#pragma unroll
        for (int e = 0; e < kCh; ++e) {
            float acc2 = 0.0f;
#pragma unroll
            for (int jj = 0; jj < W; ++jj) acc2 = __builtin_fmaf(wt[e][jj], col[jj][e], acc2);
            out[e] = BF16 ? bf16_to_f32(conv_silu_bf16(acc2)) : conv_silu(acc2);
        }
        store_row8<BF16>(a.y, xb + (size_t)t * C + c0, nch, vec, out);
        store_row8<BF16>(a.win, (size_t)b * (W - 1 + T) * C + (size_t)(t + W - 1) * C + c0, nch, vec, col[W - 1]);
    }
}

// Conv of every node of a draft tree (the tree variant of the conv step,
// ggml_ssm_conv_tree in lucebox PR #637): node i's window is the W newest rows
// of [hist ; x along its root path], i.e. x_i, x of its parent, ... and then
// the history from its newest row.  Same thread mapping and rounding as the
// chain step (a chain-shaped tree gives its y bit for bit); the history is
// only read -- the tree rollback writes it once a node is accepted.
template <bool BF16, int W>
__global__ __launch_bounds__(kThreads) void conv_tree_kernel(ConvTreeArgs a)
{
    __shared__ int spar[kTreeMax];
    __shared__ int sprev[kTreeMax];               // parents of the previous tree (fused step)
    const int b = blockIdx.z, N = a.N, C = a.C;
    if ((int)threadIdx.x < N) {
        const int i = threadIdx.x;
        const int p = a.parent[(size_t)b * N + i];
        spar[i] = (p >= 0 && p < i) ? p : -1;
    }
    // the previous tree's accepted node (-1: none kept, or no previous tree)
    int acc = -1;
    if (a.node_prev) {
        const int nd = a.node_prev[b];
        acc = (nd >= 0 && nd < a.N_prev) ? nd : -1;
        if ((int)threadIdx.x < a.N_prev) {
            const int i = threadIdx.x;
            const int p = a.parent_prev[(size_t)b * a.N_prev + i];
            sprev[i] = (p >= 0 && p < i) ? p : -1;
        }
    }
    __syncthreads();
    const int g = threadIdx.x % kGroups, tl = threadIdx.x / kGroups;
    const int c0 = (blockIdx.x * kGroups + g) * kCh;
    const int t = blockIdx.y * kTok + tl;
    const int nch = c0 < C ? min(kCh, C - c0) : 0;
    const bool vec = (nch == kCh) && ((C & 3) == 0);
    const size_t xb = (size_t)b * N * C;
    const size_t hb = (size_t)b * (W - 1) * C;
    const size_t pb = (size_t)b * a.N_prev * C;

    // the history this tree's conv takes (fused step): row tl of hist_out, by the first token tile
    if (a.hist_out && blockIdx.y == 0 && tl < W - 1 && c0 < C) {
        int m = acc, hr = W - 2;
        for (int r = W - 2; r > tl; --r) {
            if (m >= 0) m = sprev[m];
            else --hr;
        }
        float row[kCh];
        if (m >= 0) load_row8<BF16>(a.x_prev, pb + (size_t)m * C + c0, nch, vec, row);
        else load_row8<BF16>(a.hist, hb + (size_t)hr * C + c0, nch, vec, row);
        store_row8<BF16>(a.hist_out, hb + (size_t)tl * C + c0, nch, vec, row);
    }
    if (c0 >= C || t >= N) return;

    // col[W-1] = x_t, then up the path; past a root the history rows, newest first (in the fused step
    // the previous tree's path from its accepted node comes first, then the history)
    float col[W][kCh];
    int n = t, m = acc, hr = W - 2;
#pragma unroll
    for (int jj = W - 1; jj >= 0; --jj) {
        if (n >= 0) {
            load_row8<BF16>(a.x, xb + (size_t)n * C + c0, nch, vec, col[jj]);
            n = spar[n];
        } else if (m >= 0) {
            load_row8<BF16>(a.x_prev, pb + (size_t)m * C + c0, nch, vec, col[jj]);
            m = sprev[m];
        } else {
            load_row8<BF16>(a.hist, hb + (size_t)hr * C + c0, nch, vec, col[jj]);
            --hr;
        }
    }
    float wt[kCh][W];
#pragma unroll
    for (int e = 0; e < kCh; ++e) {
        const int ce = c0 + e < C ? c0 + e : C - 1;
#pragma unroll
        for (int jj = 0; jj < W; ++jj) wt[e][jj] = a.w[(size_t)ce * W + jj];
    }
    float out[kCh];
#pragma unroll
    for (int e = 0; e < kCh; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int jj = 0; jj < W; ++jj) acc = __builtin_fmaf(wt[e][jj], col[jj][e], acc);
        out[e] = BF16 ? bf16_to_f32(conv_silu_bf16(acc)) : conv_silu(acc);
    }
    store_row8<BF16>(a.y, xb + (size_t)t * C + c0, nch, vec, out);
}

template <bool BF16>
hipError_t launch_ct(const ConvTreeArgs& a, hipStream_t s)
{
    const int groups = (a.C + kCh - 1) / kCh;
    dim3 grid((groups + kGroups - 1) / kGroups, (a.N + kTok - 1) / kTok, a.B);
    dim3 block(kThreads);
    switch (a.W) {
    case 2: conv_tree_kernel<BF16, 2><<<grid, block, 0, s>>>(a); break;
    case 3: conv_tree_kernel<BF16, 3><<<grid, block, 0, s>>>(a); break;
    case 4: conv_tree_kernel<BF16, 4><<<grid, block, 0, s>>>(a); break;
    case 5: conv_tree_kernel<BF16, 5><<<grid, block, 0, s>>>(a); break;
    case 6: conv_tree_kernel<BF16, 6><<<grid, block, 0, s>>>(a); break;
    case 7: conv_tree_kernel<BF16, 7><<<grid, block, 0, s>>>(a); break;
    case 8: conv_tree_kernel<BF16, 8><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_rc(const RollConvArgs& a, hipStream_t s)
{
    const int state_blocks = (int)((a.state_elems + (long long)kThreads * 4 - 1) / ((long long)kThreads * 4));
    const int groups = (a.C + kCh - 1) / kCh;
    const int cgx = (groups + kGroups - 1) / kGroups;
    const int tiles = cgx * ((a.T + kTok - 1) / kTok);
    dim3 grid(state_blocks + tiles, a.B);
    dim3 block(kThreads);
    switch (a.W) {
    case 2: rollback_conv_kernel<BF16, 2><<<grid, block, 0, s>>>(a, state_blocks, cgx); break;
    case 3: rollback_conv_kernel<BF16, 3><<<grid, block, 0, s>>>(a, state_blocks, cgx); break;
    case 4: rollback_conv_kernel<BF16, 4><<<grid, block, 0, s>>>(a, state_blocks, cgx); break;
    case 5: rollback_conv_kernel<BF16, 5><<<grid, block, 0, s>>>(a, state_blocks, cgx); break;
    case 6: rollback_conv_kernel<BF16, 6><<<grid, block, 0, s>>>(a, state_blocks, cgx); break;
    case 7: rollback_conv_kernel<BF16, 7><<<grid, block, 0, s>>>(a, state_blocks, cgx); break;
    case 8: rollback_conv_kernel<BF16, 8><<<grid, block, 0, s>>>(a, state_blocks, cgx); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_w(const ConvArgs& a, hipStream_t s)
{
    const int groups = (a.C + kCh - 1) / kCh;
    dim3 grid((groups + kGroups - 1) / kGroups, (a.T + kTok - 1) / kTok, a.B);
    dim3 block(kThreads);
    switch (a.W) {
    case 2: conv_step_kernel<BF16, 2><<<grid, block, 0, s>>>(a); break;
    case 3: conv_step_kernel<BF16, 3><<<grid, block, 0, s>>>(a); break;
    case 4: conv_step_kernel<BF16, 4><<<grid, block, 0, s>>>(a); break;
    case 5: conv_step_kernel<BF16, 5><<<grid, block, 0, s>>>(a); break;
    case 6: conv_step_kernel<BF16, 6><<<grid, block, 0, s>>>(a); break;
    case 7: conv_step_kernel<BF16, 7><<<grid, block, 0, s>>>(a); break;
    case 8: conv_step_kernel<BF16, 8><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_step(const ConvArgs& a, bool bf16, hipStream_t s)
{
    return bf16 ? launch_w<true>(a, s) : launch_w<false>(a, s);
}

hipError_t launch_rollback_conv(const RollConvArgs& a, bool bf16, hipStream_t s)
{
    return bf16 ? launch_rc<true>(a, s) : launch_rc<false>(a, s);
}

hipError_t launch_conv_tree(const ConvTreeArgs& a, bool bf16, hipStream_t s)
{
    return bf16 ? launch_ct<true>(a, s) : launch_ct<false>(a, s);
}

}  // namespace gdn

GDN_CLAMP_READER(clamped_accepts_conv)
