// gdn_rollback.hip -- restore the conv and GDN state to the accepted length.
//
// After a verify window of K tokens the host (or a later device step) decides
// how many tokens a in 0..K each sequence keeps.  The states after every
// prefix were captured by gdn_verify (H) and gdn_conv_step (the window), so
// rollback is a pure copy (the pages' recurrent snapshot rollback planes and
// per-token conv_state intermediates: strix-llama.cpp PR #14 commit messages;
// atlas PR #297 commit message on causal_conv1d_update_prefill_inter):
//   S_out[b] <- S_in[b] (a = 0) | H[b][a-1] (0 < a < K) | unchanged (a = K)
//   hist[b][j] <- win[b][a+j],  j < W-1
// The accept lengths are read on the device, so the copy needs no host sync.
//
// Grid: x covers one sequence's state in 4 KB slabs (256 threads x 1 float4,
// loaded and stored past the caches) followed by its conv rows; y is the
// sequence.  State workgroups of sequences with a == K return at once; the conv
// rows are copied for every a (for a == K they already hold win[K..] after an
// in-place conv step, so the copy is a no-op there).
#include "gdn_debug.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr long long kSlab = (long long)kThreads * 4;  // floats per workgroup

__global__ __launch_bounds__(kThreads) void rollback_kernel(RollbackArgs a, int state_blocks)
{
    const int b = blockIdx.y;
    const int Kb = a.K;                                        // window of the buffers
    const int K = a.lens ? min(max(a.lens[b], 1), Kb) : Kb;   // this sequence's window
    int acc = a.accept[b];
    // (the replay's launch has no state blocks: its verify launch counts)
    GDN_COUNT_CLAMP(state_blocks > 0 && blockIdx.x == 0 && threadIdx.x == 0 && (acc < 0 || acc > K));
    acc = acc < 0 ? 0 : (acc > K ? K : acc);

    if ((int)blockIdx.x < state_blocks) {
        if (acc == K) return;
        const float* src = acc == 0 ? a.S_in + (size_t)b * a.state_elems
                                    : a.H + ((size_t)b * (Kb - 1) + (acc - 1)) * a.state_elems;
        float* dst = a.S_out + (size_t)b * a.state_elems;
        const long long e = (long long)blockIdx.x * kSlab + (long long)threadIdx.x * 4;
        if (e < a.state_elems)
            __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + e)),
                                        reinterpret_cast<f32x4_t*>(dst + e));
        return;
    }

    // conv rows: (W-1)*C consecutive elements, 8 per thread
    if (a.hist == nullptr) return;
    const long long n = (long long)(a.W - 1) * a.C;
    const long long e = ((long long)(blockIdx.x - state_blocks) * kThreads + threadIdx.x) * 8;
    const size_t src0 = ((size_t)b * (a.W - 1 + Kb) + acc) * a.C;
    const size_t dst0 = (size_t)b * (a.W - 1) * a.C;
    if ((a.C & 7) == 0) {
        // every row starts 16-byte aligned (win and hist are): 16-byte copies, one per 8 bf16 or two
        // per 8 floats; n is a multiple of 8, so e < n leaves all 8 elements in range
        if (e < n) {
            const uint4* s = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.win) +
                                                            (src0 + e) * a.elem_bytes);
            uint4* d = reinterpret_cast<uint4*>(reinterpret_cast<char*>(a.hist) + (dst0 + e) * a.elem_bytes);
            d[0] = s[0];
            if (a.elem_bytes == 4) d[1] = s[1];
        }
        return;
    }
    // other channel counts: 16-bit units (bf16) or 32-bit units (f32)
    if (a.elem_bytes == 2) {
        const uint16_t* s = reinterpret_cast<const uint16_t*>(a.win) + src0;
        uint16_t* d = reinterpret_cast<uint16_t*>(a.hist) + dst0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (e + j < n) d[e + j] = s[e + j];
    } else {
        const uint32_t* s = reinterpret_cast<const uint32_t*>(a.win) + src0;
        uint32_t* d = reinterpret_cast<uint32_t*>(a.hist) + dst0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (e + j < n) d[e + j] = s[e + j];
    }
}

// Rollback after a tree verify: sequence b keeps the path from its root to node
// n = node[b] (none when n is outside [0, N)).
//   S_out[b] <- H[b][n]  (S_in[b] when nothing is kept)
//   hist[b]  <- the W-1 newest rows of [hist ; x along the path]  (unchanged when nothing is kept)
// Grid as above: the state slabs, then the conv columns.  A conv thread owns 8
// columns of one sequence for all W-1 rows: it reads every source row (the old
// history included) before it writes, so the in-place update needs no barrier.
template <typename E, int R>
__device__ __forceinline__ void tree_rows(const E* xs, E* hs, const size_t (&src)[R], const bool (&from_x)[R],
                                          size_t hb, int C, long long e, int cnt)
{
    E v[R][8];
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < cnt) v[m][j] = (from_x[m] ? xs : hs)[src[m] + e + j];
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < cnt) hs[hb + (size_t)(R - 1 - m) * C + e + j] = v[m][j];
}

template <int W>
__global__ __launch_bounds__(kThreads) void tree_rollback_kernel(TreeRollbackArgs a, int state_blocks)
{
    const int b = blockIdx.y, N = a.N;
    int n = a.node[b];
    n = (n >= 0 && n < N) ? n : -1;

    if ((int)blockIdx.x < state_blocks) {
        const float* src = n < 0 ? a.S_in + (size_t)b * a.state_elems
                                 : a.H + ((size_t)b * N + n) * a.state_elems;
        float* dst = a.S_out + (size_t)b * a.state_elems;
        const long long e = (long long)blockIdx.x * kSlab + (long long)threadIdx.x * 4;
        if (e < a.state_elems)
            __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + e)),
                                        reinterpret_cast<f32x4_t*>(dst + e));
        return;
    }
    if (a.hist == nullptr || n < 0) return;
    constexpr int R = W - 1;
    const long long e = ((long long)(blockIdx.x - state_blocks) * kThreads + threadIdx.x) * 8;
    if (e >= a.C) return;
    const int cnt = (int)min((long long)8, a.C - e);
    // source of new history row R-1-m (the m-th newest): x of the m-th node up the
    // path, then the old history from its newest row
    size_t src[R];
    bool from_x[R];
    int hr = R - 1;
#pragma unroll
    for (int m = 0; m < R; ++m) {
        from_x[m] = n >= 0;
        if (n >= 0) {
            src[m] = ((size_t)b * N + n) * a.C;
            const int p = a.parent[(size_t)b * N + n];
            n = (p >= 0 && p < n) ? p : -1;
        } else {
            src[m] = ((size_t)b * R + hr) * a.C;
            --hr;
        }
    }
    const size_t hb = (size_t)b * R * a.C;
    if (a.elem_bytes == 2)
        tree_rows<uint16_t, R>(reinterpret_cast<const uint16_t*>(a.x), reinterpret_cast<uint16_t*>(a.hist), src,
                               from_x, hb, a.C, e, cnt);
    else
        tree_rows<uint32_t, R>(reinterpret_cast<const uint32_t*>(a.x), reinterpret_cast<uint32_t*>(a.hist), src,
                               from_x, hb, a.C, e, cnt);
}

}  // namespace

hipError_t launch_tree_rollback(const TreeRollbackArgs& a, hipStream_t s)
{
    const int state_blocks = (int)((a.state_elems + kSlab - 1) / kSlab);
    const int conv_blocks = a.hist != nullptr ? (a.C + kThreads * 8 - 1) / (kThreads * 8) : 0;
    dim3 grid(state_blocks + conv_blocks, a.B);
    dim3 block(kThreads);
    switch (a.hist != nullptr ? a.W : 2) {
    case 2: tree_rollback_kernel<2><<<grid, block, 0, s>>>(a, state_blocks); break;
    case 3: tree_rollback_kernel<3><<<grid, block, 0, s>>>(a, state_blocks); break;
    case 4: tree_rollback_kernel<4><<<grid, block, 0, s>>>(a, state_blocks); break;
    case 5: tree_rollback_kernel<5><<<grid, block, 0, s>>>(a, state_blocks); break;
    case 6: tree_rollback_kernel<6><<<grid, block, 0, s>>>(a, state_blocks); break;
    case 7: tree_rollback_kernel<7><<<grid, block, 0, s>>>(a, state_blocks); break;
    case 8: tree_rollback_kernel<8><<<grid, block, 0, s>>>(a, state_blocks); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_rollback(const RollbackArgs& a, hipStream_t s)
{
    const int state_blocks = (int)((a.state_elems + kSlab - 1) / kSlab);
    int conv_blocks = 0;
    if (a.hist != nullptr) {
        const long long n = (long long)(a.W - 1) * a.C;
        conv_blocks = (int)((n + kThreads * 8 - 1) / (kThreads * 8));
    }
    dim3 grid(state_blocks + conv_blocks, a.B);
    rollback_kernel<<<grid, dim3(kThreads), 0, s>>>(a, state_blocks);
    return hipGetLastError();
}

}  // namespace gdn

GDN_CLAMP_READER(clamped_accepts_rollback)
