/*
 * gdn.h -- C ABI of libgdn.so: the speculative-decoding verify step of one
 * Gated-DeltaNet (GDN) layer on AMD Instinct MI355X (gfx950).
 *
 * The step, as the pages on the subject describe it:
 *   1. a fused depthwise causal conv1d over the verify window: history window,
 *      silu(conv), history written back in place, and the window kept so that
 *      a partial accept can restore the conv state (lucebox PR #637
 *      "NVLink fix for PR625": commit message on ggml_ssm_conv_step, review
 *      note on its sources x, weights, conv_state, conv_input_out; atlas
 *      PR #297 "dflash scheduler/server verify-step glue": commit message on
 *      causal_conv1d_update_prefill_inter and its per-token conv-state
 *      intermediates);
 *   2. the gated delta rule over the K window tokens with raw gates applied
 *      inside the kernel, q and k L2-normalised and broadcast from key heads
 *      to value heads, writing the final state plus every intermediate state
 *      H_0..H_{K-2} (token by token for a chain of drafts, chunkwise in WY
 *      form for a draft tree and for prefill) (lucebox PR #637: commit
 *      messages on raw-gate gated_delta_net and the single l2_norm over the
 *      q|k slab, review excerpt of gated_delta_net.cu; atlas PR #297: commit
 *      message on gated_delta_rule_wy16.cu and its opt-in fp32 output);
 *   3. rollback of the conv and GDN state to the accepted length (the same
 *      pages; strix-llama.cpp PR #14 "DSv4 + Qwen3.8 Flash runtime fixes":
 *      commit messages on recurrent snapshot rollback and device-resident
 *      checkpoints);
 *   4. chunked prefill of the same layer, final state only.
 *
 * Recurrence, per sequence b and value head h (key head hk = h / (Hv/Hk)):
 *   beta_t = sigmoid(beta_raw_t)
 *   g_t    = -softplus(alpha_t + dt_bias[h]) * exp(A_log[h])
 *   q^, k^ = q / sqrt(|q|^2 + l2_eps), k / sqrt(|k|^2 + l2_eps)
 *   S_t    = exp(g_t) S_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T
 *   o_t    = S_t q^_t
 * S is dv x dk (row i is value index i, columns are key dims), fp32.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or keeps device memory, never
 *     synchronises, and launches only on `stream` (a hipStream_t; NULL is the
 *     default stream).  Calls are stream-ordered; two calls that write the
 *     same buffer must not run concurrently on different streams.
 *   - Arrays are dense and row-major in the index order written next to them.
 *   - dtype codes: GDN_F32 (float) or GDN_BF16 (bfloat16 bits, uint16).
 *   - Pointers must be 16-byte aligned.
 *   - Arguments are checked on the host before anything is launched; a bad
 *     argument returns a negative code, launches nothing and leaves every
 *     buffer untouched.  gdn_last_error() gives a message (thread-local).
 *   - B == 0 is a valid empty call: GDN_OK, nothing launched.
 *   - Thread-safe: the only global state is the thread-local error message
 *     (and, in the debug build only, the device-side count read by
 *     gdn_debug_clamped_accepts).
 *   - Accept lengths outside the range of the window they refer to are
 *     clamped into it by the kernels (the rollback to an accepted prefix:
 *     strix-llama.cpp PR #14, commit messages on recurrent snapshot rollback);
 *     the debug build also counts them.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_VERSION 3

enum gdn_status {
    GDN_OK = 0,
    GDN_EINVAL = -1,       /* null / misaligned / overlapping pointer, bad size */
    GDN_EUNSUPPORTED = -2, /* valid request outside what the kernels implement */
    GDN_EHIP = -3          /* the HIP runtime reported an error at launch */
};

enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 };

/* GDN_VERSION of the built library. */
int gdn_version(void);

/* Message for the last non-zero return on this thread ("" if none). */
const char *gdn_last_error(void);

/*
 * gdn_debug_clamped_accepts -- debug build only (libgdn_debug.so, compiled
 * with GDN_DEBUG): the number of accept lengths that kernels of this library
 * found outside 0..K of their window and clamped, on the current device,
 * since the library was loaded or last reset -- one count per sequence and
 * call of gdn_rollback(_ex), gdn_rollback_conv_step, gdn_replay and
 * gdn_verify_step (accept_prev).  Reads device memory, so it waits for the
 * device's work to finish: for tests and debugging, not a serving loop.
 *   count  host pointer, receives the count
 *   reset  non-zero: the count is set to zero after it is read
 * The release build (libgdn.so) counts nothing and returns GDN_EUNSUPPORTED.
 */
int gdn_debug_clamped_accepts(long long *count, int reset);

/*
 * gdn_conv_step -- fused causal depthwise conv1d decode / verify step.
 *
 * For each sequence b and channel c the window is
 *     win[j] = hist[b][j][c]          for j < W-1
 *     win[j] = x[b][j-(W-1)][c]       for W-1 <= j < W-1+T
 * and for every new token t < T
 *     pre_t = sum_{j<W} w[c][j] * win[t+j]     (w[c][W-1] meets token t)
 *     y[b][t][c] = silu(pre_t) = pre_t / (1 + exp(-pre_t))
 * The history is then written back in place: hist[b][j][c] = win[T+j].
 * If win_out is not NULL it receives the whole window,
 *     win_out[b][j][c] = win[j],  j < W-1+T,
 * so that the conv state after a accepted tokens is rows a..a+W-2
 * (see gdn_rollback).
 *
 * Numerics: pre is an fmaf chain over j = 0..W-1 starting from 0; exp is
 * the library's own float exp (Cody-Waite reduction by ln 2, degree-7
 * Taylor polynomial in Horner form with fmaf, exact scaling by 2^n); the
 * division is correctly rounded; bf16 outputs are rounded to nearest even.
 * The result is therefore a fixed function of the inputs, reproducible bit
 * for bit by any implementation of the same steps.
 *
 *   x        [B][T][C]        io_dtype, the T new tokens
 *   w        [C][W]           float, depthwise taps
 *   hist     [B][W-1][C]      io_dtype, read then overwritten
 *   y        [B][T][C]        io_dtype, output (q|k|v slab for gdn_verify)
 *   win_out  [B][W-1+T][C]    io_dtype, output, may be NULL
 *   B >= 0, T >= 1, C >= 1, 2 <= W <= 8
 * y and win_out must not overlap x, w, hist or each other.
 */
int gdn_conv_step(const void *x, const float *w, void *hist, void *y, void *win_out,
                  int B, int T, int C, int W, int io_dtype, void *stream);

/*
 * gdn_verify -- gated delta rule over a K-token verify window, with capture.
 *
 * Gate mode: if dt_bias and A_log are both non-NULL, beta_raw and alpha are
 * raw projections and the gates above are applied in the kernel (softplus
 * switches to the identity above 20).  If both are NULL, beta_raw holds beta
 * and alpha holds g already activated.  One NULL and one not is GDN_EINVAL.
 *
 * Evaluation: the token recurrence over the window (every state is written, so
 * the chunkwise WY form, which the pages name, would save no bytes here; it is
 * the same recurrence, and gdn_verify_tree and gdn_prefill_chunked use it):
 *   u_t = beta_t (v_t - exp(g_t) H_{t-1} k^_t),
 *   H_t = exp(g_t) H_{t-1} + u_t k^_t^T,       H_{-1} = S_in,
 *   o_t = H_t q^_t.
 *
 *   qkv      [B][K][C]    in_dtype; C = 2*Hk*dk + Hv*dv; per token the q of
 *                         all key heads, then their k, then the v of all
 *                         value heads (the gdn_conv_step output)
 *   beta_raw [B][K][Hv]   in_dtype
 *   alpha    [B][K][Hv]   in_dtype
 *   dt_bias  [Hv]         float or NULL
 *   A_log    [Hv]         float or NULL
 *   S_in     [B][Hv][dv][dk] float, the state before the window
 *   S_out    [B][Hv][dv][dk] float, the state after all K tokens; may be
 *                         exactly S_in (in place; then rollback to 0 tokens
 *                         is impossible); any other overlap is GDN_EINVAL
 *   H        [B][K-1][Hv][dv][dk] float, H[b][t] = state after tokens
 *                         0..t; may be NULL (no capture); must not overlap
 *                         S_in / S_out
 *   o        [B][K][Hv][dv] o_dtype, o_t = S_t q^_t
 *   B >= 0; 1 <= K <= 64 (GDN_EUNSUPPORTED above); Hk >= 1; Hv % Hk == 0;
 *   dk in {32, 64, 128}; dv a multiple of 8
 *   l2_eps >= 0
 */
int gdn_verify(const void *qkv, const void *beta_raw, const void *alpha,
               const float *dt_bias, const float *A_log,
               const float *S_in, float *S_out, float *H, void *o,
               int B, int K, int Hk, int Hv, int dk, int dv,
               int in_dtype, int o_dtype, float l2_eps, void *stream);

/*
 * gdn_rollback -- restore conv and GDN state to the accepted length.
 *
 * For each sequence b, a = accept[b] (device int32; values outside 0..K are
 * clamped) is the number of window tokens kept:
 *   state: S_out[b] <- S_in[b]      if a == 0
 *          S_out[b] <- H[b][a-1]    if 0 < a < K
 *          unchanged                if a == K (gdn_verify already wrote it)
 *   conv:  hist[b][j] <- win[b][a+j], j < W-1
 * Bit-exact copies.  Needs the pre-window state, so S_out must not be S_in.
 *
 *   accept   [B] int32, device
 *   S_in     [B][Hv][dv][dk] float
 *   H        [B][K-1][Hv][dv][dk] float (may be NULL only when K == 1)
 *   S_out    [B][Hv][dv][dk] float
 *   hist     [B][W-1][C] io_dtype, or NULL together with win to skip conv
 *   win      [B][W-1+K][C] io_dtype (gdn_conv_step's win_out)
 *   B >= 0, K >= 1, 2 <= W <= 8 when hist is given
 */
int gdn_rollback(const int32_t *accept, int K,
                 const float *S_in, const float *H, float *S_out,
                 void *hist, const void *win,
                 int B, int Hv, int dv, int dk, int C, int W, int io_dtype, void *stream);

/*
 * Extended forms: per-sequence window lengths (a ragged batch in one launch)
 * and gates read from a stacked projection output.
 *
 * A verify loop that truncates drafts by confidence gives every sequence its
 * own verify length v_len <= K_max (lucebox PR #637: commit message on
 * v_len <= q_len and the review note on the verify-length buffer), and the
 * beta|alpha gates come from one stacked projection (commit message on the
 * stacked ssm_ba projection).  The _ex forms take
 *   lens         [B] int32 (device, nullable): tokens of sequence b; values
 *                are clamped into 1..K (or 1..T).  NULL means every
 *                sequence uses the whole window.  Sequence b then behaves
 *                exactly as a call with K = lens[b] on its own: S_out[b] is
 *                the state after lens[b] tokens, H[b][0..lens[b]-2] and
 *                o[b][0..lens[b]-1] are written and the rest of its slots are
 *                left untouched; the conv step keeps window rows
 *                lens[b]..lens[b]+W-2 as the new history; the rollback keeps
 *                the state for a == lens[b] and restores it for a < lens[b].
 *                The buffers keep their K-sized (T-sized) layout.  4-byte
 *                aligned.
 *   gate_stride  elements between the gate rows of consecutive tokens
 *                (>= Hv): Hv for separate [B][K][Hv] buffers, 2*Hv when
 *                beta_raw points at a stacked [B][K][2*Hv] beta|alpha row
 *                and alpha = beta_raw + Hv.  The gate pointers need only the
 *                alignment of their element type.
 * gdn_conv_step, gdn_verify and gdn_rollback are these with lens = NULL and
 * gate_stride = Hv.
 */
int gdn_conv_step_ex(const void *x, const float *w, void *hist, void *y, void *win_out,
                     const int32_t *lens, int B, int T, int C, int W, int io_dtype,
                     void *stream);

int gdn_verify_ex(const void *qkv, const void *beta_raw, const void *alpha, int gate_stride,
                  const float *dt_bias, const float *A_log,
                  const float *S_in, float *S_out, float *H, void *o, const int32_t *lens,
                  int B, int K, int Hk, int Hv, int dk, int dv,
                  int in_dtype, int o_dtype, float l2_eps, void *stream);

int gdn_rollback_ex(const int32_t *accept, const int32_t *lens, int K,
                    const float *S_in, const float *H, float *S_out,
                    void *hist, const void *win,
                    int B, int Hv, int dv, int dk, int C, int W, int io_dtype, void *stream);

/*
 * gdn_replay -- rollback by checkpoint and replay instead of capture.
 *
 * A verify without capture (gdn_verify with H = NULL) reads and writes one
 * state per head instead of K+1; the state before the window is kept as the
 * checkpoint.  On a partial accept the accepted prefix is replayed from the
 * checkpoint without verifying again (strix-llama.cpp PR #14: commit messages
 * on device-resident rolling checkpoints and replay of the accepted tokens).
 * For each sequence b, a = accept[b] (clamped into 0..K):
 *   a == K:      S_out[b] untouched (the verify wrote the final state)
 *   a == 0:      S_out[b] <- S_ckpt[b]
 *   0 < a < K:   S_out[b] <- the state after the first a window tokens from
 *                S_ckpt[b] (the same recurrence and arithmetic as gdn_verify
 *                over a tokens; no outputs, no intermediate states)
 *   conv (if hist/win given): hist[b][j] <- win[b][a+j], j < W-1
 *
 *   accept [B] int32 (device); qkv, beta_raw, alpha, gate_stride, dt_bias,
 *   A_log: the verify window's inputs as gdn_verify_ex; S_ckpt, S_out
 *   [B][Hv][dv][dk] float, distinct; hist [B][W-1][C], win [B][W-1+K][C]
 *   in_dtype, or both NULL.
 */
int gdn_replay(const int32_t *accept, const void *qkv, const void *beta_raw, const void *alpha,
               int gate_stride, const float *dt_bias, const float *A_log,
               const float *S_ckpt, float *S_out, void *hist, const void *win,
               int B, int K, int Hk, int Hv, int dk, int dv, int W, int in_dtype,
               float l2_eps, void *stream);

/*
 * gdn_rollback_conv_step -- gdn_rollback of the previous verify window
 * followed by gdn_conv_step of the next tokens, in one launch: in a verify
 * loop the rollback of step i and the conv step of step i+1 touch the same
 * layer state back to back (the conv-state intermediates and snapshot
 * rollback of the pages cited above), and one launch saves the fixed cost of
 * the second.  The results are exactly those of the two calls
 *   gdn_rollback(accept, K_prev, S_in, H, S_out, hist, win_prev, ...);
 *   gdn_conv_step(x, w, hist, y, win, B, T, C, W, ...);
 * (bit for bit): the conv history is taken from win_prev rows a..a+W-2,
 * which is what the rollback writes into hist, and hist ends as the last W-1
 * rows of the new window.
 *
 *   accept [B] int32 (device), K_prev, S_in, H, S_out: as gdn_rollback
 *           (K_prev is the previous window length, H [B][K_prev-1][Hv][dv][dk])
 *   win_prev [B][W-1+K_prev][C] io_dtype: the previous window (input)
 *   x [B][T][C], w [C][W] float, y [B][T][C], win [B][W-1+T][C]: as
 *           gdn_conv_step (win is required here)
 *   hist [B][W-1][C]: output only
 *   Every output (S_out, hist, y, win) must be disjoint from every input
 *   and from the other outputs: keep two window buffers and alternate them.
 */
int gdn_rollback_conv_step(const int32_t *accept, int K_prev, const float *S_in,
                           const float *H, float *S_out, const void *win_prev,
                           const void *x, const float *w, void *hist, void *y, void *win,
                           int B, int Hv, int dv, int dk, int T, int C, int W,
                           int io_dtype, void *stream);

/*
 * gdn_prefill_chunked -- the same recurrence over a long prompt, processed
 * in chunks of `chunk` tokens, writing only the final state and the outputs.
 *
 *   qkv      [B][T][C], beta_raw/alpha [B][T][Hv]: as gdn_verify with K -> T
 *   S_in, S_out [B][Hv][dv][dk] float (S_out may be exactly S_in)
 *   o        [B][T][Hv][dv] o_dtype
 *   B >= 0, T >= 1 (the last chunk may be shorter), chunk in {16, 32, 64},
 *   the other sizes as gdn_verify
 */
int gdn_prefill_chunked(const void *qkv, const void *beta_raw, const void *alpha,
                        const float *dt_bias, const float *A_log,
                        const float *S_in, float *S_out, void *o,
                        int B, int T, int chunk, int Hk, int Hv, int dk, int dv,
                        int in_dtype, int o_dtype, float l2_eps, void *stream);

/*
 * gdn_verify_step -- one whole verify step of the layer in one launch: the
 * rollback of the previous window, the conv step of this window and the GDN
 * verify with capture (gdn_rollback + gdn_conv_step + gdn_verify, the same
 * arithmetic and the same bits -- at K = 1, where gdn_verify takes a decode
 * kernel, the same recurrence in another rounding order -- with no state copy
 * and no intermediate launch; the pages' step in atlas PR #297 and lucebox
 * PR #637 as above).
 *
 * Previous window (accept_prev != NULL): sequence b starts from the state its
 * accept length a = accept_prev[b] (clamped into 0..K_prev) selects --
 * S_prev_ckpt[b] (a = 0), H_prev[b][a-1] (0 < a < K_prev) or S_prev_out[b]
 * (a = K_prev) -- and from the conv history rows a .. a+W-2 of win_prev.
 * First window (accept_prev == NULL): from S_in and hist.
 *   x [B][K][C] raw tokens, w [C][W] float taps, gates, dt_bias, A_log,
 *   gate_stride: as gdn_conv_step and gdn_verify_ex;
 *   S_prev_ckpt, S_prev_out [B][Hv][dv][dk], H_prev [B][K_prev-1][...],
 *   win_prev [B][W-1+K_prev][C]: the previous step's S_ckpt, S_out, H, win;
 *   S_in [B][Hv][dv][dk], hist [B][W-1][C]: the first window's start.
 * Outputs:
 *   S_ckpt [B][Hv][dv][dk]  this window's start state (nullable; the next
 *                           step's S_prev_ckpt)
 *   S_out, H, o             as gdn_verify (H nullable: no capture)
 *   y [B][K][C]             the conv outputs (nullable)
 *   win [B][W-1+K][C]       this window's conv window (nullable; the next
 *                           step's win_prev)
 * W must be 4.  Every output is disjoint from every input and from the other
 * outputs: a loop keeps two sets of (S_ckpt, S_out, H, win) and alternates
 * them.  To leave the loop, gdn_rollback(accept, K, S_ckpt, H, S_out, hist,
 * win) materialises the state and the history.
 */
int gdn_verify_step(const int32_t *accept_prev, int K_prev, const float *S_prev_ckpt,
                    const float *H_prev, const float *S_prev_out, const void *win_prev,
                    const float *S_in, const void *hist,
                    const void *x, const float *w, const void *beta_raw, const void *alpha,
                    int gate_stride, const float *dt_bias, const float *A_log,
                    float *S_ckpt, float *S_out, float *H, void *o, void *y, void *win,
                    int B, int K, int Hk, int Hv, int dk, int dv, int W,
                    int in_dtype, int o_dtype, float l2_eps, void *stream);

/*
 * Tree verify -- the drafter proposes a tree of candidate tokens instead of a
 * chain (lucebox PR #637: DDTree drafting in the commit messages, and the tree
 * variant of the conv, ggml_ssm_conv_tree, in the review excerpt of ggml.c).
 * Node i of sequence b continues node parent[b][i]: its conv window and its
 * GDN state are those its parent left, exactly as token t continues token
 * t-1 in a chain.  An entry outside [0, i) marks a root, which continues the
 * committed state (hist, S_in); nodes are therefore numbered parents first,
 * and parent[i] = i-1 is the plain chain.  N = nodes per sequence, 1..32.
 *   parent [B][N] int32 (device), 4-byte aligned, read only.
 *
 * gdn_conv_tree -- the conv step of every node: y[b][i] = silu(conv over the
 * W newest rows of [hist ; x along the path from the root to i]); the same
 * rounding as gdn_conv_step (a chain-shaped tree gives its y bit for bit).
 * hist is only read: the history changes once a node is accepted
 * (gdn_rollback_tree).
 *   x [B][N][C], hist [B][W-1][C], y [B][N][C] io_dtype; w [C][W] float;
 *   16-byte aligned; y disjoint from the inputs.
 */
int gdn_conv_tree(const void *x, const float *w, const void *hist, const int32_t *parent, void *y,
                  int B, int N, int C, int W, int io_dtype, void *stream);

/*
 * gdn_verify_tree -- the GDN recurrence over every node of the tree, each
 * node one step from its parent's state (S_in for a root):
 *   H [B][N][Hv][dv][dk] float   the state after every node (N planes: a tree
 *                                has no single final state)
 *   o [B][N][Hv][dv]     o_dtype o_i = S_i q^_i
 * The other arguments, their layouts, alignment and the gate forms are those
 * of gdn_verify_ex (with K -> N and no lens).  Computed in WY form with the
 * pairs (node, ancestor) only; every node's state is formed directly from
 * S_in and the corrections along its path.
 */
int gdn_verify_tree(const void *qkv, const void *beta_raw, const void *alpha, int gate_stride,
                    const float *dt_bias, const float *A_log, const int32_t *parent,
                    const float *S_in, float *H, void *o,
                    int B, int N, int Hk, int Hv, int dk, int dv,
                    int in_dtype, int o_dtype, float l2_eps, void *stream);

/*
 * gdn_rollback_tree -- sequence b keeps the path from its root to node
 * n = node[b] (device int32 [B]; outside [0, N): nothing kept):
 *   S_out[b] <- H[b][n]      (S_in[b] when nothing is kept)
 *   hist[b]  <- the W-1 newest rows of [hist ; x along the path]
 *               (unchanged when nothing is kept), a byte copy
 *   S_in, S_out [B][Hv][dv][dk] float, distinct; H as gdn_verify_tree;
 *   x [B][N][C] (the conv inputs of the tree) and hist [B][W-1][C] io_dtype,
 *   both given or both NULL (state only).
 */
int gdn_rollback_tree(const int32_t *node, const int32_t *parent, int N,
                      const float *S_in, const float *H, float *S_out,
                      const void *x, void *hist,
                      int B, int Hv, int dv, int dk, int C, int W, int io_dtype, void *stream);

/*
 * gdn_verify_tree_step -- one whole tree verify step: the rollback of the
 * previous tree to its accepted node, the conv of this tree's nodes and the
 * tree verify with every node's state -- gdn_rollback_tree + gdn_conv_tree +
 * gdn_verify_tree, bit for bit, without the state copy (the same tree
 * drafting as above; the step a serving loop runs, with the DDTree branch of
 * the spec loop in the lucebox PR #637 commit messages).  Two launches: the conv, then the verify.
 *
 * Previous tree (node_prev != NULL): sequence b keeps the path to node
 * a = node_prev[b] of the previous tree (N_prev nodes, parent_prev, raw
 * tokens x_prev, history hist_prev, states H_prev, start state S_prev_ckpt);
 * a outside [0, N_prev) keeps nothing.  This tree starts from H_prev[b][a]
 * (S_prev_ckpt[b] when nothing is kept), and its conv history is the W-1
 * newest rows of [hist_prev ; x_prev along the path from the root to a].
 * First tree (node_prev == NULL): from S_prev_ckpt and hist_prev (the
 * committed state and history); N_prev, parent_prev, H_prev, x_prev unused.
 *   node_prev [B] int32, parent_prev [B][N_prev] int32 (4-byte aligned);
 *   S_prev_ckpt [B][Hv][dv][dk], H_prev [B][N_prev][Hv][dv][dk] float;
 *   x_prev [B][N_prev][C], hist_prev [B][W-1][C] in_dtype;
 *   x [B][N][C] raw tokens, w [C][W] float taps, parent [B][N] int32, gates,
 *   gate_stride, dt_bias, A_log: as gdn_conv_tree and gdn_verify_tree.
 * Outputs:
 *   S_ckpt [B][Hv][dv][dk]  this tree's start state (nullable; the next
 *                           step's S_prev_ckpt)
 *   H, o                    as gdn_verify_tree
 *   y [B][N][C]             the conv outputs (required: the verify reads them)
 *   hist_out [B][W-1][C]    this tree's conv history (nullable; the next
 *                           step's hist_prev)
 * Every output is disjoint from every input and from the other outputs: a
 * loop keeps two sets of (S_ckpt, H, hist_out) and alternates them; to leave
 * it, gdn_rollback_tree(node, parent, S_ckpt, H, S_out, x, hist_out)
 * materialises the state and the history.
 */
int gdn_verify_tree_step(const int32_t *node_prev, int N_prev, const int32_t *parent_prev,
                         const float *S_prev_ckpt, const float *H_prev, const void *x_prev,
                         const void *hist_prev, const void *x, const float *w, const int32_t *parent,
                         const void *beta_raw, const void *alpha, int gate_stride,
                         const float *dt_bias, const float *A_log,
                         float *S_ckpt, float *H, void *o, void *y, void *hist_out,
                         int B, int N, int Hk, int Hv, int dk, int dv, int W,
                         int in_dtype, int o_dtype, float l2_eps, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
