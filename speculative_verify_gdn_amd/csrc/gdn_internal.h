// gdn_internal.h -- launchers behind the C ABI of libgdn (include/gdn.h).
// The ABI layer validates every argument on the host; the launchers assume
// valid arguments and only pick a kernel instance and a grid.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct ConvArgs {
    const void* x;      // [B][T][C]
    const float* w;     // [C][W]
    void* hist;         // [B][W-1][C], read then written
    void* y;            // [B][T][C]
    void* win;          // [B][W-1+T][C] or nullptr
    int B, T, C, W;
    const int32_t* lens = nullptr;  // [B] tokens per sequence (<= T), or nullptr: all T
};

struct VerifyArgs {
    const void* qkv;       // [B][K][C]
    const void* beta_raw;  // [B][K][Hv]
    const void* alpha;     // [B][K][Hv]
    const float* dt_bias;  // [Hv] or nullptr (activated gates)
    const float* A_log;    // [Hv] or nullptr
    const float* S_in;     // [B][Hv][dv][dk]
    float* S_out;          // [B][Hv][dv][dk]
    float* H;              // [B][K-1][Hv][dv][dk] or nullptr
    void* o;               // [B][K][Hv][dv]
    int B, K, Hk, Hv, dk, dv;
    float eps;
    const int32_t* lens = nullptr;  // [B] tokens per sequence (<= K), or nullptr: all K
    int gstride = 0;                // elements between the gate rows of consecutive tokens (0: Hv)
    const int32_t* replay = nullptr;  // [B] accept lengths: rebuild S_out from S_in over that many tokens
    const int32_t* parent = nullptr;  // [B][K] tree verify: parent node per node (H then holds K states)
    // fused step (conv width 4): the conv of the window and the start state picked from the previous window
    const void* x = nullptr;           // [B][K][C] raw tokens (qkv unused)
    const float* w = nullptr;          // [C][4] taps
    const void* hsrc = nullptr;        // history rows: previous window [B][hrows][C] (rows a..a+2) or hist
    int hrows = 0;                     // rows per sequence of hsrc
    const int32_t* acc_prev = nullptr; // [B] accept lengths of the previous window, or nullptr: S_in and hist
    int Kp = 0;                        // previous window length
    const float* Sp_ckpt = nullptr;    // previous window's start state, capture and final state
    const float* Sp_H = nullptr;
    const float* Sp_out = nullptr;
    float* S_ckpt = nullptr;           // [B][Hv][dv][dk] this window's start state, or nullptr
    void* y = nullptr;                 // [B][K][C] conv outputs, or nullptr
    void* win = nullptr;               // [B][3+K][C] this window's conv window, or nullptr
    // tree verify whose start state is picked by the previous tree's accepted node: acc_prev (node,
    // outside [0, Kp): none kept), Kp (its node count), Sp_H (its node states), Sp_ckpt (its start
    // state, also the start when acc_prev is nullptr); the start state is written to S_ckpt
    bool pick = false;
};

// longest verify window (tokens per sequence) of the chain calls
constexpr int kVerifyMax = 64;

// largest draft tree (nodes per sequence) of the tree calls
constexpr int kTreeMax = 32;

struct ConvTreeArgs {
    const void* x;           // [B][N][C]
    const float* w;          // [C][W]
    const void* hist;        // [B][W-1][C], read only
    const int32_t* parent;   // [B][N]
    void* y;                 // [B][N][C]
    int B, N, C, W;
    // the fused tree step: the history is the W-1 newest rows of [hist ; x_prev along the path from the
    // previous tree's accepted node to its root]; hist_out receives them
    const int32_t* node_prev = nullptr;    // [B] accepted node of the previous tree (outside [0, N_prev): none)
    const int32_t* parent_prev = nullptr;  // [B][N_prev]
    const void* x_prev = nullptr;          // [B][N_prev][C]
    int N_prev = 0;
    void* hist_out = nullptr;              // [B][W-1][C] or nullptr
};

struct TreeRollbackArgs {
    const int32_t* node;     // [B] accepted node (outside [0, N): none)
    const int32_t* parent;   // [B][N]
    const float* S_in;       // [B][Hv][dv][dk]
    const float* H;          // [B][N][Hv][dv][dk]
    float* S_out;            // [B][Hv][dv][dk]
    long long state_elems;   // Hv*dv*dk
    const void* x;           // [B][N][C] conv inputs of the tree, or nullptr
    void* hist;              // [B][W-1][C], updated in place, or nullptr
    int B, N, C, W, elem_bytes;
};

struct RollbackArgs {
    const int32_t* accept;  // [B]
    const float* S_in;      // [B][Hv][dv][dk]
    const float* H;         // [B][K-1][Hv][dv][dk]
    float* S_out;           // [B][Hv][dv][dk]
    void* hist;             // [B][W-1][C] or nullptr
    const void* win;        // [B][W-1+K][C] or nullptr
    int B, K;
    long long state_elems;  // Hv*dv*dk
    int C, W, elem_bytes;
    const int32_t* lens = nullptr;  // [B] window length per sequence (<= K), or nullptr: all K
};

// rollback of the previous window fused with the conv step of the next tokens
struct RollConvArgs {
    const int32_t* accept;   // [B], accept lengths of the previous window
    int Kp;                  // previous window length
    const float* S_in;       // [B][Hv][dv][dk], state before the previous window
    const float* H;          // [B][Kp-1][Hv][dv][dk]
    float* S_out;            // [B][Hv][dv][dk]
    long long state_elems;   // Hv*dv*dk
    const void* win_prev;    // [B][W-1+Kp][C], previous conv window
    const void* x;           // [B][T][C]
    const float* w;          // [C][W]
    void* hist;              // [B][W-1][C], written only
    void* y;                 // [B][T][C]
    void* win;               // [B][W-1+T][C]
    int B, T, C, W;
};

struct PrefillArgs {
    const void* qkv;       // [B][T][C]
    const void* beta_raw;  // [B][T][Hv]
    const void* alpha;     // [B][T][Hv]
    const float* dt_bias;
    const float* A_log;
    const float* S_in;
    float* S_out;
    void* o;               // [B][T][Hv][dv]
    int B, T, chunk, Hk, Hv, dk, dv;
    float eps;
};

hipError_t launch_conv_step(const ConvArgs& a, bool bf16, hipStream_t s);
hipError_t launch_verify(const VerifyArgs& a, bool in_bf16, bool o_bf16, hipStream_t s);
// the fused verify step (VerifyArgs with x set): the pipelined step kernel, or the verify kernel's step mode
hipError_t launch_step(const VerifyArgs& a, bool in_bf16, bool o_bf16, hipStream_t s);
hipError_t launch_rollback(const RollbackArgs& a, hipStream_t s);
hipError_t launch_rollback_conv(const RollConvArgs& a, bool bf16, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, bool o_bf16, hipStream_t s);
hipError_t launch_prefill_wy(const PrefillArgs& a, bool o_bf16, hipStream_t s);
// the chunkwise kernel for dk = 128 and chunks of 64 tokens (hipErrorInvalidValue for other shapes)
hipError_t launch_prefill_c64(const PrefillArgs& a, bool o_bf16, hipStream_t s);
hipError_t launch_conv_tree(const ConvTreeArgs& a, bool bf16, hipStream_t s);
hipError_t launch_tree_rollback(const TreeRollbackArgs& a, hipStream_t s);

#ifdef GDN_DEBUG
// the debug build's counts of clamped accept lengths, one per translation unit (gdn_debug.h)
hipError_t clamped_accepts_rollback(unsigned long long* n, bool reset);
hipError_t clamped_accepts_conv(unsigned long long* n, bool reset);
hipError_t clamped_accepts_step(unsigned long long* n, bool reset);
hipError_t clamped_accepts_verify_bf16_bf16(unsigned long long* n, bool reset);
hipError_t clamped_accepts_verify_bf16_f32(unsigned long long* n, bool reset);
hipError_t clamped_accepts_verify_f32_bf16(unsigned long long* n, bool reset);
hipError_t clamped_accepts_verify_f32_f32(unsigned long long* n, bool reset);
#endif

}  // namespace gdn
