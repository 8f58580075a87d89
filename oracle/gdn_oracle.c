/*
 * gdn_oracle.c -- CPU oracle for the speculative-verify step of one
 * Gated-DeltaNet (GDN) layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * reference that the HIP path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark load it.  The product
 * path never calls, links or includes it, and it shares no code, header,
 * table or constant generator with the HIP kernels.
 *
 * What it computes (sources: the three pages on the subject):
 *   - the fused causal conv1d decode/verify step: history window + silu(conv)
 *     + history write-back + rollback window copy
 *     (lucebox PR #637 "NVLink fix for PR625", commit message on
 *      ggml_ssm_conv_step; review note on the op's four sources
 *      (x, weights, conv_state, conv_input_out));
 *   - the raw-gate GDN: beta = sigmoid(raw beta), decay from
 *     softplus(alpha + dt_bias) scaled by A (same page, commit message on
 *     ggml_gated_delta_net_set_raw_gates and the review excerpt of
 *     gated_delta_net.cu);
 *   - the gated delta rule over a K-token verify window, writing the final
 *     state and the intermediate states H_0..H_{K-2} (atlas PR #297
 *     "dflash scheduler/server verify-step glue", commit message on
 *     gated_delta_rule_wy16.cu) and the per-token conv-state intermediates
 *     for partial-accept rollback (same commit, on
 *     causal_conv1d_update_prefill_inter);
 *   - rollback to an accept length (same pages; strix-llama.cpp PR #14,
 *     commit messages on recurrent snapshot rollback and device-resident
 *     checkpoints).
 *
 * The recurrence itself is S_t = exp(g_t) S_{t-1} (I - b_t k_t k_t^T)
 * + b_t v_t k_t^T, o_t = S_t q_t, with q and k L2-normalised; the pages name
 * it but do not print it, so it is written here in its plainest reading.
 *
 * Everything in the GDN part is double precision.  The conv step has two
 * versions: a double-precision definition, and a float version that fixes the
 * order of every rounding (fmaf chain, the exp below, correctly rounded
 * division, round-to-nearest-even bfloat16) so that a GPU implementation of
 * the same steps can be compared bit for bit.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* float bit helpers                                                          */
/* ------------------------------------------------------------------------- */
static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ------------------------------------------------------------------------- */
/* float exp with a fixed evaluation order                                    */
/*                                                                           */
/* Cody-Waite argument reduction x = n ln2 + r, |r| <= ln2/2, then the        */
/* degree-7 Taylor polynomial of e^r in Horner form with fused multiply-adds, */
/* then an exact scaling by 2^n split into two powers of two so that results  */
/* in the subnormal range are rounded once.                                   */
/*                                                                           */
/*   LOG2E  = nearest float to 1/ln 2                                         */
/*   LN2_HI = ln 2 rounded to a multiple of 2^-16 (16 significant bits, so    */
/*            n * LN2_HI is exact for |n| < 2^8)                              */
/*   LN2_LO = nearest float to (ln 2 - LN2_HI)                                */
/*   C[k]   = nearest float to 1/k!                                           */
/* ------------------------------------------------------------------------- */
static const float ORC_LOG2E = 0x1.715476p+0f;   /* 1.44269502162933349609375 */
static const float ORC_LN2_HI = 0x1.62e4p-1f;    /* 0.693145751953125 */
static const float ORC_LN2_LO = 0x1.7f7d1cp-20f; /* 1.428606765330187e-06 */

static float orc_taylor_coeff(int k)
{
    switch (k) {
    case 0: return 1.0f;
    case 1: return 1.0f;
    case 2: return 1.0f / 2.0f;
    case 3: return 1.0f / 6.0f;
    case 4: return 1.0f / 24.0f;
    case 5: return 1.0f / 120.0f;
    case 6: return 1.0f / 720.0f;
    default: return 1.0f / 5040.0f;
    }
}

float oracle_exp32(float x)
{
    if (x != x) return x;                 /* NaN propagates */
    if (x >= 89.0f) return INFINITY;      /* e^89 > FLT_MAX */
    if (x <= -104.0f) return 0.0f;        /* e^-104 < half the smallest subnormal */
    float n = rintf(x * ORC_LOG2E);       /* round half to even */
    float r = fmaf(-n, ORC_LN2_HI, x);
    r = fmaf(-n, ORC_LN2_LO, r);
    float p = orc_taylor_coeff(7);
    for (int k = 6; k >= 0; --k) p = fmaf(p, r, orc_taylor_coeff(k));
    int ni = (int)n;                      /* -150 <= n <= 129 */
    int n1 = ni / 2;                      /* truncates toward zero */
    int n2 = ni - n1;
    float s1 = bits_to_f32((uint32_t)(n1 + 127) << 23);
    float s2 = bits_to_f32((uint32_t)(n2 + 127) << 23);
    return (p * s1) * s2;
}

/* the constants above, for the tests that pin them */
void oracle_exp32_constants(float *out /* [11] */)
{
    out[0] = ORC_LOG2E;
    out[1] = ORC_LN2_HI;
    out[2] = ORC_LN2_LO;
    for (int k = 0; k < 8; ++k) out[3 + k] = orc_taylor_coeff(k);
}

/* float -> bfloat16, round to nearest even; NaN stays NaN (quiet bit set) */
uint16_t oracle_bf16_rne(float f)
{
    uint32_t u = f32_to_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float oracle_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* silu(p) = p * sigmoid(p) = p / (1 + e^-p), every step rounded to float */
float oracle_silu32(float p)
{
    float e = oracle_exp32(-p);
    float den = 1.0f + e;
    return p / den;
}

void oracle_bf16_rne_array(const float *in, uint16_t *out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = oracle_bf16_rne(in[i]);
}

void oracle_exp32_array(const float *in, float *out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = oracle_exp32(in[i]);
}

void oracle_silu32_array(const float *in, float *out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = oracle_silu32(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Conv step                                                                  */
/*                                                                           */
/* Layouts (row-major):                                                       */
/*   x    [B][T][C]        the T new tokens (verify window or prompt)         */
/*   w    [C][W]           depthwise taps; w[c][W-1] meets the newest token   */
/*   hist [B][W-1][C]      the W-1 tokens before x                            */
/*   y    [B][T][C]        silu(conv) per token                               */
/*   hist_out [B][W-1][C]  the last W-1 rows of the window                    */
/*   win  [B][W-1+T][C]    the whole window [hist ; x]; the conv state after  */
/*                         a accepted tokens is rows a .. a+W-2               */
/* For each (b, c) the window is col[j], j < W-1+T, and                       */
/*   pre_t = sum_{j<W} w[c][j] * col[t+j],   y_t = silu(pre_t).               */
/* ------------------------------------------------------------------------- */
void oracle_conv_step_f32(const float *x, const float *w, const float *hist,
                          float *y, float *hist_out, float *win,
                          int B, int T, int C, int W, int round_bf16)
{
    const int WT = W - 1 + T;
    float *col = (float *)malloc(sizeof(float) * (size_t)WT);
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < C; ++c) {
            for (int j = 0; j < W - 1; ++j) col[j] = hist[((size_t)b * (W - 1) + j) * C + c];
            for (int t = 0; t < T; ++t) col[W - 1 + t] = x[((size_t)b * T + t) * C + c];
            for (int t = 0; t < T; ++t) {
                float acc = 0.0f;
                for (int j = 0; j < W; ++j) acc = fmaf(w[(size_t)c * W + j], col[t + j], acc);
                float out = oracle_silu32(acc);
                if (round_bf16) out = oracle_bf16_to_f32(oracle_bf16_rne(out));
                y[((size_t)b * T + t) * C + c] = out;
            }
            for (int j = 0; j < W - 1; ++j) hist_out[((size_t)b * (W - 1) + j) * C + c] = col[T + j];
            if (win)
                for (int j = 0; j < WT; ++j) win[((size_t)b * WT + j) * C + c] = col[j];
        }
    }
    free(col);
}

/* double-precision definition; pre (nullable) receives the pre-activation */
void oracle_conv_step_f64(const double *x, const double *w, const double *hist,
                          double *y, double *pre, double *hist_out, double *win,
                          int B, int T, int C, int W)
{
    const int WT = W - 1 + T;
    double *col = (double *)malloc(sizeof(double) * (size_t)WT);
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < C; ++c) {
            for (int j = 0; j < W - 1; ++j) col[j] = hist[((size_t)b * (W - 1) + j) * C + c];
            for (int t = 0; t < T; ++t) col[W - 1 + t] = x[((size_t)b * T + t) * C + c];
            for (int t = 0; t < T; ++t) {
                double acc = 0.0;
                for (int j = 0; j < W; ++j) acc += w[(size_t)c * W + j] * col[t + j];
                size_t o = ((size_t)b * T + t) * C + c;
                if (pre) pre[o] = acc;
                y[o] = acc / (1.0 + exp(-acc));
            }
            for (int j = 0; j < W - 1; ++j) hist_out[((size_t)b * (W - 1) + j) * C + c] = col[T + j];
            if (win)
                for (int j = 0; j < WT; ++j) win[((size_t)b * WT + j) * C + c] = col[j];
        }
    }
    free(col);
}

/* ------------------------------------------------------------------------- */
/* Gates (raw-gate mode)                                                      */
/*   beta = 1 / (1 + e^-raw)                                                  */
/*   g    = -softplus(alpha + dt_bias) * e^{A_log}   (A = -e^{A_log} < 0)     */
/* softplus(a) = log(1 + e^a) is evaluated as max(a,0) + log1p(e^-|a|), which */
/* is exact in real arithmetic and never overflows.                           */
/* With dt_bias == A_log == NULL the inputs are already activated:            */
/*   beta = raw, g = alpha.                                                   */
/* ------------------------------------------------------------------------- */
static double orc_softplus(double a) { return fmax(a, 0.0) + log1p(exp(-fabs(a))); }

static void orc_gate(double braw, double alpha, const double *dt_bias, const double *A_log,
                     int h, double *beta, double *g)
{
    if (dt_bias && A_log) {
        *beta = 1.0 / (1.0 + exp(-braw));
        *g = -orc_softplus(alpha + dt_bias[h]) * exp(A_log[h]);
    } else {
        *beta = braw;
        *g = alpha;
    }
}

/* beta_raw, alpha [N][Hv] -> beta, g [N][Hv] */
void oracle_gates_f64(const double *beta_raw, const double *alpha,
                      const double *dt_bias, const double *A_log,
                      double *beta, double *g, int N, int Hv)
{
    for (int n = 0; n < N; ++n)
        for (int h = 0; h < Hv; ++h)
            orc_gate(beta_raw[(size_t)n * Hv + h], alpha[(size_t)n * Hv + h], dt_bias, A_log, h,
                     &beta[(size_t)n * Hv + h], &g[(size_t)n * Hv + h]);
}

/* q / sqrt(sum q^2 + eps) */
static void orc_l2norm(const double *in, double *out, int n, double eps)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += in[i] * in[i];
    double r = 1.0 / sqrt(s + eps);
    for (int i = 0; i < n; ++i) out[i] = in[i] * r;
}

/* ------------------------------------------------------------------------- */
/* GDN over a window of K tokens, sequential (the definition)                 */
/*                                                                           */
/* qkv      [B][K][C], C = 2*Hk*dk + Hv*dv: per token the q of all key heads, */
/*          then the k of all key heads, then the v of all value heads        */
/* beta_raw, alpha [B][K][Hv]                                                 */
/* dt_bias, A_log [Hv] (both NULL: gates given already activated)             */
/* S_in, S_out [B][Hv][dv][dk]   state S (dv x dk, row i = value index)       */
/* H   [B][K-1][Hv][dv][dk]      state after tokens 0..K-2 (nullable)         */
/* o   [B][K][Hv][dv]            o_t = S_t q_t                                */
/* Value head h reads key head h / (Hv/Hk).                                   */
/*                                                                           */
/* Per token:  S <- gamma S;  u = beta (v - S k);  S <- S + u k^T;  o = S q.  */
/* This is S_t = gamma S_{t-1} (I - beta k k^T) + beta v k^T written out.     */
/* ------------------------------------------------------------------------- */
void oracle_gdn_recurrent_f64(const double *qkv, const double *beta_raw, const double *alpha,
                              const double *dt_bias, const double *A_log,
                              const double *S_in, double *S_out, double *H, double *o,
                              int B, int K, int Hk, int Hv, int dk, int dv, double eps)
{
    const int C = 2 * Hk * dk + Hv * dv;
    const int grp = Hv / Hk;
    double *S = (double *)malloc(sizeof(double) * (size_t)dv * dk);
    double *qn = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kn = (double *)malloc(sizeof(double) * (size_t)dk);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hv; ++h) {
            const int hk = h / grp;
            memcpy(S, S_in + ((size_t)b * Hv + h) * dv * dk, sizeof(double) * (size_t)dv * dk);
            for (int t = 0; t < K; ++t) {
                const double *row = qkv + ((size_t)b * K + t) * C;
                orc_l2norm(row + (size_t)hk * dk, qn, dk, eps);
                orc_l2norm(row + (size_t)Hk * dk + (size_t)hk * dk, kn, dk, eps);
                const double *v = row + 2 * (size_t)Hk * dk + (size_t)h * dv;
                double beta, g;
                size_t gi = ((size_t)b * K + t) * Hv + h;
                orc_gate(beta_raw[gi], alpha[gi], dt_bias, A_log, h, &beta, &g);
                const double gam = exp(g);
                for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] *= gam;
                for (int i = 0; i < dv; ++i) {
                    double *Si = S + (size_t)i * dk;
                    double sk = 0.0;
                    for (int j = 0; j < dk; ++j) sk += Si[j] * kn[j];
                    double u = beta * (v[i] - sk);
                    for (int j = 0; j < dk; ++j) Si[j] += u * kn[j];
                    double sq = 0.0;
                    for (int j = 0; j < dk; ++j) sq += Si[j] * qn[j];
                    o[(((size_t)b * K + t) * Hv + h) * dv + i] = sq;
                }
                if (H && t < K - 1)
                    memcpy(H + (((size_t)b * (K - 1) + t) * Hv + h) * dv * dk, S,
                           sizeof(double) * (size_t)dv * dk);
            }
            memcpy(S_out + ((size_t)b * Hv + h) * dv * dk, S, sizeof(double) * (size_t)dv * dk);
        }
    }
    free(S);
    free(qn);
    free(kn);
}

/* ------------------------------------------------------------------------- */
/* GDN, chunkwise in WY (UT-transform) form -- the second implementation      */
/*                                                                           */
/* Within a chunk of L tokens (local index t = 0..L-1), with G_t the running  */
/* sum of g over the chunk up to and including t and S0 the state entering   */
/* the chunk:                                                                 */
/*   A[t][s] = beta_t e^{G_t - G_s} (k_t . k_s)        for s < t, else 0      */
/*   T       = (I + A)^{-1}                 (unit lower triangular)           */
/*   W       = T diag(beta e^{G}) K        (L x dk)                           */
/*   Ut      = T diag(beta) V              (L x dv)                           */
/*   U       = Ut - W S0^T                 (row t = u_t, the corrected value) */
/*   M[t][s] = e^{G_t - G_s} (q_t . k_s)   for s <= t, else 0                 */
/*   O       = diag(e^{G}) Q S0^T + M U                                       */
/* and the state after token t of the chunk is                                */
/*   S_t = gamma_t S_{t-1} + u_t k_t^T.                                       */
/* Only differences G_t - G_s with s <= t are exponentiated, so no ratio of   */
/* two tiny decays ever forms.                                                */
/* With H == NULL only the state after the whole chunk is formed:             */
/*   S <- e^{G_{L-1}} S0 + sum_s e^{G_{L-1} - G_s} u_s k_s^T.                 */
/* The window of K tokens is cut into chunks of `chunk` tokens; the last one  */
/* may be shorter.                                                            */
/* ------------------------------------------------------------------------- */
void oracle_gdn_chunked_f64(const double *qkv, const double *beta_raw, const double *alpha,
                            const double *dt_bias, const double *A_log,
                            const double *S_in, double *S_out, double *H, double *o,
                            int B, int K, int Hk, int Hv, int dk, int dv, double eps, int chunk)
{
    const int C = 2 * Hk * dk + Hv * dv;
    const int grp = Hv / Hk;
    const size_t SD = (size_t)dv * dk;
    const int Lm = chunk < K ? chunk : K;
    double *S = (double *)malloc(sizeof(double) * SD);
    double *Qn = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
    double *Kn = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
    double *V = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
    double *bet = (double *)malloc(sizeof(double) * (size_t)Lm);
    double *gg = (double *)malloc(sizeof(double) * (size_t)Lm);
    double *G = (double *)malloc(sizeof(double) * (size_t)Lm);
    double *A = (double *)malloc(sizeof(double) * (size_t)Lm * Lm);
    double *Tm = (double *)malloc(sizeof(double) * (size_t)Lm * Lm);
    double *Wm = (double *)malloc(sizeof(double) * (size_t)Lm * dk);
    double *Ut = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
    double *U = (double *)malloc(sizeof(double) * (size_t)Lm * dv);
    double *M = (double *)malloc(sizeof(double) * (size_t)Lm * Lm);
    double *Onew = (double *)malloc(sizeof(double) * (size_t)Lm * dv);

    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hv; ++h) {
            const int hk = h / grp;
            memcpy(S, S_in + ((size_t)b * Hv + h) * SD, sizeof(double) * SD);
            for (int c0 = 0; c0 < K; c0 += chunk) {
                const int L = (K - c0) < chunk ? (K - c0) : chunk;
                /* load, normalise, gates */
                for (int t = 0; t < L; ++t) {
                    const double *row = qkv + ((size_t)b * K + c0 + t) * C;
                    orc_l2norm(row + (size_t)hk * dk, Qn + (size_t)t * dk, dk, eps);
                    orc_l2norm(row + (size_t)Hk * dk + (size_t)hk * dk, Kn + (size_t)t * dk, dk, eps);
                    memcpy(V + (size_t)t * dv, row + 2 * (size_t)Hk * dk + (size_t)h * dv,
                           sizeof(double) * (size_t)dv);
                    size_t gi = ((size_t)b * K + c0 + t) * Hv + h;
                    orc_gate(beta_raw[gi], alpha[gi], dt_bias, A_log, h, &bet[t], &gg[t]);
                    G[t] = gg[t] + (t > 0 ? G[t - 1] : 0.0);
                }
                /* A (strictly lower) and M (lower, diagonal included) */
                for (int t = 0; t < L; ++t) {
                    for (int s = 0; s < L; ++s) {
                        double kk = 0.0, qk = 0.0;
                        for (int j = 0; j < dk; ++j) {
                            kk += Kn[(size_t)t * dk + j] * Kn[(size_t)s * dk + j];
                            qk += Qn[(size_t)t * dk + j] * Kn[(size_t)s * dk + j];
                        }
                        A[(size_t)t * L + s] = s < t ? bet[t] * exp(G[t] - G[s]) * kk : 0.0;
                        M[(size_t)t * L + s] = s <= t ? exp(G[t] - G[s]) * qk : 0.0;
                    }
                }
                /* T = (I + A)^{-1}: solve (I + A) T = I by forward substitution */
                for (int col = 0; col < L; ++col) {
                    for (int t = 0; t < L; ++t) {
                        double acc = (t == col) ? 1.0 : 0.0;
                        for (int s = 0; s < t; ++s) acc -= A[(size_t)t * L + s] * Tm[(size_t)s * L + col];
                        Tm[(size_t)t * L + col] = acc;
                    }
                }
                /* W = T diag(beta e^G) K,  Ut = T diag(beta) V */
                for (int t = 0; t < L; ++t) {
                    for (int j = 0; j < dk; ++j) {
                        double acc = 0.0;
                        for (int s = 0; s < L; ++s)
                            acc += Tm[(size_t)t * L + s] * bet[s] * exp(G[s]) * Kn[(size_t)s * dk + j];
                        Wm[(size_t)t * dk + j] = acc;
                    }
                    for (int i = 0; i < dv; ++i) {
                        double acc = 0.0;
                        for (int s = 0; s < L; ++s) acc += Tm[(size_t)t * L + s] * bet[s] * V[(size_t)s * dv + i];
                        Ut[(size_t)t * dv + i] = acc;
                    }
                }
                /* U = Ut - W S0^T;  O = diag(e^G) Q S0^T + M U */
                for (int t = 0; t < L; ++t) {
                    for (int i = 0; i < dv; ++i) {
                        double p = 0.0;
                        for (int j = 0; j < dk; ++j) p += S[(size_t)i * dk + j] * Wm[(size_t)t * dk + j];
                        U[(size_t)t * dv + i] = Ut[(size_t)t * dv + i] - p;
                    }
                }
                for (int t = 0; t < L; ++t) {
                    for (int i = 0; i < dv; ++i) {
                        double r = 0.0;
                        for (int j = 0; j < dk; ++j) r += S[(size_t)i * dk + j] * Qn[(size_t)t * dk + j];
                        double acc = exp(G[t]) * r;
                        for (int s = 0; s <= t; ++s) acc += M[(size_t)t * L + s] * U[(size_t)s * dv + i];
                        Onew[(size_t)t * dv + i] = acc;
                    }
                }
                for (int t = 0; t < L; ++t)
                    for (int i = 0; i < dv; ++i)
                        o[(((size_t)b * K + c0 + t) * Hv + h) * dv + i] = Onew[(size_t)t * dv + i];
                /* state: every intermediate, or only the chunk's last */
                if (H) {
                    for (int t = 0; t < L; ++t) {
                        const double gam = exp(gg[t]);
                        for (int i = 0; i < dv; ++i)
                            for (int j = 0; j < dk; ++j)
                                S[(size_t)i * dk + j] = gam * S[(size_t)i * dk + j]
                                                      + U[(size_t)t * dv + i] * Kn[(size_t)t * dk + j];
                        const int tg = c0 + t;
                        if (tg < K - 1)
                            memcpy(H + (((size_t)b * (K - 1) + tg) * Hv + h) * SD, S, sizeof(double) * SD);
                    }
                } else {
                    const double eL = exp(G[L - 1]);
                    for (int i = 0; i < dv; ++i) {
                        for (int j = 0; j < dk; ++j) {
                            double acc = eL * S[(size_t)i * dk + j];
                            for (int s = 0; s < L; ++s)
                                acc += exp(G[L - 1] - G[s]) * U[(size_t)s * dv + i] * Kn[(size_t)s * dk + j];
                            S[(size_t)i * dk + j] = acc;
                        }
                    }
                }
            }
            memcpy(S_out + ((size_t)b * Hv + h) * SD, S, sizeof(double) * SD);
        }
    }
    free(S); free(Qn); free(Kn); free(V); free(bet); free(gg); free(G);
    free(A); free(Tm); free(Wm); free(Ut); free(U); free(M); free(Onew);
}

/* ------------------------------------------------------------------------- */
/* Rollback to an accept length                                              */
/*                                                                           */
/* a = accept[b] clamped to 0..K is the number of window tokens kept.         */
/*   state: S_out[b] <- S_in[b] (a = 0), H[b][a-1] (0 < a < K), unchanged     */
/*          (a = K: S_out already holds the state after all K tokens)         */
/*   conv:  hist[b] <- win[b] rows a .. a+W-2                                 */
/* A plain byte copy: `state_bytes` is the size of one sequence's state       */
/* (Hv*dv*dk elements), `row_bytes` the size of one conv row (C elements).    */
/* Pass hist = win = NULL to skip the conv part, H = NULL only when K == 1.   */
/* ------------------------------------------------------------------------- */
void oracle_rollback(const int32_t *accept, int K, int B,
                     const void *S_in, const void *H, void *S_out, long state_bytes,
                     const void *win, void *hist, long row_bytes, int W)
{
    for (int b = 0; b < B; ++b) {
        int a = accept[b];
        if (a < 0) a = 0;
        if (a > K) a = K;
        unsigned char *dst = (unsigned char *)S_out + (size_t)b * state_bytes;
        if (a == 0)
            memcpy(dst, (const unsigned char *)S_in + (size_t)b * state_bytes, (size_t)state_bytes);
        else if (a < K)
            memcpy(dst, (const unsigned char *)H + ((size_t)b * (K - 1) + (a - 1)) * state_bytes,
                   (size_t)state_bytes);
        if (hist && win) {
            const int WT = W - 1 + K;
            memcpy((unsigned char *)hist + (size_t)b * (W - 1) * row_bytes,
                   (const unsigned char *)win + ((size_t)b * WT + a) * row_bytes,
                   (size_t)(W - 1) * row_bytes);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Tree verify: the drafted tokens form a tree instead of a chain             */
/* (lucebox PR #637: DDTree drafting and the tree variant of the conv,        */
/* ggml_ssm_conv_tree, in the commit messages and the review excerpt of       */
/* ggml.c).  The pages give the op's name and that the drafter proposes a     */
/* tree; what it computes is read here as the chain step applied along every  */
/* root path: a node continues the state its parent left, exactly as token t  */
/* continues token t-1 in a chain.                                            */
/*                                                                           */
/* parent [B][N]: node i continues node parent[b][i].  An entry outside      */
/* [0, i) marks a root, which continues the committed state (S_in, hist).     */
/* So the nodes are numbered parents-first and parent[i] = i-1 is the chain.  */
/* ------------------------------------------------------------------------- */
static int orc_parent(const int32_t *parent, int b, int N, int i)
{
    const int p = parent[(size_t)b * N + i];
    return (p >= 0 && p < i) ? p : -1;
}

/* The conv window of node i, oldest first: the W newest rows of             */
/* [hist ; x along the path root .. i].  col[W-1] = x_i, col[W-2] = x of its */
/* parent, ..., and once the path ends the history rows from the newest.     */
static void orc_tree_window(const float *x, const float *hist, const int32_t *parent,
                            int b, int N, int C, int W, int c, int i, float *col)
{
    int m = 0, n = i;
    while (m < W && n >= 0) {
        col[W - 1 - m] = x[((size_t)b * N + n) * C + c];
        n = orc_parent(parent, b, N, n);
        ++m;
    }
    for (int h = W - 2; m < W; --h, ++m) col[W - 1 - m] = hist[((size_t)b * (W - 1) + h) * C + c];
}

/* Conv of every tree node, same precision and rounding order as             */
/* oracle_conv_step_f32 (fmaf chain over the taps, oldest first).            */
/*   x [B][N][C], hist [B][W-1][C] (read only), y [B][N][C].                  */
void oracle_conv_tree_f32(const float *x, const float *w, const float *hist, const int32_t *parent,
                          float *y, int B, int N, int C, int W, int round_bf16)
{
    float *col = (float *)malloc(sizeof(float) * (size_t)W);
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < N; ++i)
            for (int c = 0; c < C; ++c) {
                orc_tree_window(x, hist, parent, b, N, C, W, c, i, col);
                float acc = 0.0f;
                for (int j = 0; j < W; ++j) acc = fmaf(w[(size_t)c * W + j], col[j], acc);
                float out = oracle_silu32(acc);
                if (round_bf16) out = oracle_bf16_to_f32(oracle_bf16_rne(out));
                y[((size_t)b * N + i) * C + c] = out;
            }
    free(col);
}

/* GDN over a tree of N nodes, one token step per node from its parent's     */
/* state (S_in for a root), the same step as oracle_gdn_recurrent_f64.        */
/*   qkv [B][N][C], beta_raw, alpha [B][N][Hv]                                */
/*   H [B][N][Hv][dv][dk]   the state after every node                        */
/*   o [B][N][Hv][dv]       o_i = S_i q_i                                     */
void oracle_gdn_tree_f64(const double *qkv, const double *beta_raw, const double *alpha,
                         const double *dt_bias, const double *A_log, const int32_t *parent,
                         const double *S_in, double *H, double *o,
                         int B, int N, int Hk, int Hv, int dk, int dv, double eps)
{
    const int C = 2 * Hk * dk + Hv * dv;
    const int grp = Hv / Hk;
    const size_t SD = (size_t)dv * dk;
    double *qn = (double *)malloc(sizeof(double) * (size_t)dk);
    double *kn = (double *)malloc(sizeof(double) * (size_t)dk);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hv; ++h) {
            const int hk = h / grp;
            for (int t = 0; t < N; ++t) {
                const int p = orc_parent(parent, b, N, t);
                double *S = H + (((size_t)b * N + t) * Hv + h) * SD;
                const double *from = p < 0 ? S_in + ((size_t)b * Hv + h) * SD
                                           : H + (((size_t)b * N + p) * Hv + h) * SD;
                memcpy(S, from, sizeof(double) * SD);
                const double *row = qkv + ((size_t)b * N + t) * C;
                orc_l2norm(row + (size_t)hk * dk, qn, dk, eps);
                orc_l2norm(row + (size_t)Hk * dk + (size_t)hk * dk, kn, dk, eps);
                const double *v = row + 2 * (size_t)Hk * dk + (size_t)h * dv;
                double beta, g;
                const size_t gi = ((size_t)b * N + t) * Hv + h;
                orc_gate(beta_raw[gi], alpha[gi], dt_bias, A_log, h, &beta, &g);
                const double gam = exp(g);
                for (size_t e = 0; e < SD; ++e) S[e] *= gam;
                for (int i = 0; i < dv; ++i) {
                    double *Si = S + (size_t)i * dk;
                    double sk = 0.0;
                    for (int j = 0; j < dk; ++j) sk += Si[j] * kn[j];
                    const double u = beta * (v[i] - sk);
                    for (int j = 0; j < dk; ++j) Si[j] += u * kn[j];
                    double sq = 0.0;
                    for (int j = 0; j < dk; ++j) sq += Si[j] * qn[j];
                    o[(((size_t)b * N + t) * Hv + h) * dv + i] = sq;
                }
            }
        }
    }
    free(qn);
    free(kn);
}

/* Rollback after a tree verify: sequence b keeps the path root .. node[b]    */
/* (node[b] outside [0, N): nothing accepted).                                */
/*   state: S_out[b] <- H[b][node] (S_in[b] when nothing is accepted)         */
/*   conv:  hist[b] <- the W-1 newest rows of [hist ; x along the path]       */
/* x, hist hold elements of elem_bytes bytes (a byte copy).                   */
void oracle_tree_rollback(const int32_t *node, const int32_t *parent, int N, int B,
                          const void *S_in, const void *H, void *S_out, long state_bytes,
                          const void *x, void *hist, int C, int W, int elem_bytes)
{
    const size_t rb = (size_t)C * elem_bytes;
    unsigned char *rows = (unsigned char *)malloc(rb * (size_t)(W > 1 ? W - 1 : 1));
    for (int b = 0; b < B; ++b) {
        int n = node[b];
        if (n < 0 || n >= N) n = -1;
        unsigned char *dst = (unsigned char *)S_out + (size_t)b * state_bytes;
        if (n < 0)
            memcpy(dst, (const unsigned char *)S_in + (size_t)b * state_bytes, (size_t)state_bytes);
        else
            memcpy(dst, (const unsigned char *)H + ((size_t)b * N + n) * state_bytes, (size_t)state_bytes);
        if (!hist || !x || W < 2 || n < 0) continue;
        unsigned char *hb = (unsigned char *)hist + (size_t)b * (W - 1) * rb;
        /* newest first: x of the path from node n upward, then the old history */
        int m = 0;
        while (m < W - 1 && n >= 0) {
            memcpy(rows + (size_t)(W - 2 - m) * rb, (const unsigned char *)x + ((size_t)b * N + n) * rb, rb);
            n = orc_parent(parent, b, N, n);
            ++m;
        }
        for (int h = W - 2; m < W - 1; --h, ++m)
            memcpy(rows + (size_t)(W - 2 - m) * rb, hb + (size_t)h * rb, rb);
        memcpy(hb, rows, rb * (size_t)(W - 1));
    }
    free(rows);
}

int oracle_version(void) { return 2; }
