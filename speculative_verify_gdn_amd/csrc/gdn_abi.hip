// gdn_abi.hip -- the extern "C" entry points of libgdn (declared in
// include/gdn.h): argument validation on the host, then one launch on the
// caller's stream.  Nothing is allocated, nothing is synchronised.
//
// Every check happens before any launch, because a device fault takes the
// whole context down with it (the pages report exactly that failure mode:
// atlas PR #297, commit message on the illegal-address crash that poisoned
// the CUDA context).
#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok()
{
    g_err[0] = '\0';
    return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const void* p;
    size_t bytes;
};

bool overlap(Span a, Span b)
{
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

int launch_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(GDN_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

size_t elem_size(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

bool valid_dtype(int d) { return d == GDN_F32 || d == GDN_BF16; }

#define REQUIRE(cond, code, ...)          \
    do {                                  \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

// shared checks of the GDN shapes (verify and prefill)
int check_gdn_shape(const char* fn, int B, int K, int Hk, int Hv, int dk, int dv, int in_dtype, int o_dtype,
                    float eps)
{
    REQUIRE(B >= 0, GDN_EINVAL, "%s: B = %d < 0", fn, B);
    REQUIRE(K >= 1, GDN_EINVAL, "%s: token count %d < 1", fn, K);
    REQUIRE(Hk >= 1 && Hv >= 1, GDN_EINVAL, "%s: Hk = %d, Hv = %d must be >= 1", fn, Hk, Hv);
    REQUIRE(Hv % Hk == 0, GDN_EINVAL, "%s: Hv = %d is not a multiple of Hk = %d", fn, Hv, Hk);
    REQUIRE(dk >= 1 && dv >= 1, GDN_EINVAL, "%s: dk = %d, dv = %d must be >= 1", fn, dk, dv);
    REQUIRE(dk == 32 || dk == 64 || dk == 128, GDN_EUNSUPPORTED, "%s: dk = %d not in {32, 64, 128}", fn, dk);
    REQUIRE(dv % 8 == 0, GDN_EUNSUPPORTED, "%s: dv = %d is not a multiple of 8", fn, dv);
    REQUIRE(valid_dtype(in_dtype) && valid_dtype(o_dtype), GDN_EINVAL, "%s: bad dtype code (%d, %d)", fn,
            in_dtype, o_dtype);
    REQUIRE(eps >= 0.0f, GDN_EINVAL, "%s: l2_eps < 0", fn);
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_version(void) { return GDN_VERSION; }

const char* gdn_last_error(void) { return g_err; }

int gdn_debug_clamped_accepts(long long* count, int reset)
{
    const char* fn = "gdn_debug_clamped_accepts";
#ifdef GDN_DEBUG
    REQUIRE(count, GDN_EINVAL, "%s: null count", fn);
    // one counter per translation unit that clamps accept lengths
    hipError_t (*const readers[])(unsigned long long*, bool) = {
        gdn::clamped_accepts_rollback,          gdn::clamped_accepts_conv,
        gdn::clamped_accepts_step,              gdn::clamped_accepts_verify_bf16_bf16,
        gdn::clamped_accepts_verify_bf16_f32,   gdn::clamped_accepts_verify_f32_bf16,
        gdn::clamped_accepts_verify_f32_f32};
    unsigned long long total = 0;
    for (auto rd : readers) {
        unsigned long long n = 0;
        const hipError_t e = rd(&n, reset != 0);
        if (e != hipSuccess) return fail(GDN_EHIP, "%s: %s", fn, hipGetErrorString(e));
        total += n;
    }
    *count = (long long)total;
    return ok();
#else
    (void)count;
    (void)reset;
    return fail(GDN_EUNSUPPORTED, "%s: counted only in the debug build (libgdn_debug.so)", fn);
#endif
}

int gdn_conv_step(const void* x, const float* w, void* hist, void* y, void* win_out, int B, int T, int C, int W,
                  int io_dtype, void* stream)
{
    return gdn_conv_step_ex(x, w, hist, y, win_out, nullptr, B, T, C, W, io_dtype, stream);
}

int gdn_conv_step_ex(const void* x, const float* w, void* hist, void* y, void* win_out, const int32_t* lens, int B,
                     int T, int C, int W, int io_dtype, void* stream)
{
    const char* fn = "gdn_conv_step";
    REQUIRE(B >= 0, GDN_EINVAL, "%s: B = %d < 0", fn, B);
    REQUIRE(T >= 1, GDN_EINVAL, "%s: T = %d < 1", fn, T);
    REQUIRE(C >= 1, GDN_EINVAL, "%s: C = %d < 1", fn, C);
    REQUIRE(W >= 2 && W <= 8, GDN_EUNSUPPORTED, "%s: W = %d not in 2..8", fn, W);
    REQUIRE(valid_dtype(io_dtype), GDN_EINVAL, "%s: bad dtype code %d", fn, io_dtype);
    REQUIRE((long long)B * T * C < (1LL << 40), GDN_EUNSUPPORTED, "%s: problem too large", fn);
    if (B == 0) return ok();
    REQUIRE(x && w && hist && y, GDN_EINVAL, "%s: null pointer (x, w, hist and y are required)", fn);
    REQUIRE(aligned16(x) && aligned16(w) && aligned16(hist) && aligned16(y) && (!win_out || aligned16(win_out)),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(!lens || ((uintptr_t)lens & 3) == 0, GDN_EINVAL, "%s: lens must be 4-byte aligned", fn);
    const size_t es = elem_size(io_dtype);
    const Span sx{x, (size_t)B * T * C * es}, sw{w, (size_t)C * W * 4}, sh{hist, (size_t)B * (W - 1) * C * es},
        sy{y, (size_t)B * T * C * es}, swin{win_out, win_out ? (size_t)B * (W - 1 + T) * C * es : 0};
    REQUIRE(!overlap(sy, sx) && !overlap(sy, sw) && !overlap(sy, sh), GDN_EINVAL, "%s: y overlaps an input", fn);
    REQUIRE(!overlap(swin, sx) && !overlap(swin, sw) && !overlap(swin, sh) && !overlap(swin, sy), GDN_EINVAL,
            "%s: win_out overlaps another buffer", fn);
    REQUIRE(!overlap(sh, sx) && !overlap(sh, sw), GDN_EINVAL, "%s: hist overlaps x or w", fn);
    REQUIRE(T <= 65535 * 16, GDN_EUNSUPPORTED, "%s: T = %d too large", fn, T);
    REQUIRE(B <= 65535, GDN_EUNSUPPORTED, "%s: B = %d too large", fn, B);
    REQUIRE(!overlap(sh, Span{lens, lens ? (size_t)B * 4 : 0}) && !overlap(sy, Span{lens, lens ? (size_t)B * 4 : 0}) &&
                !overlap(swin, Span{lens, lens ? (size_t)B * 4 : 0}),
            GDN_EINVAL, "%s: an output overlaps lens", fn);
    gdn::ConvArgs a{x, w, hist, y, win_out, B, T, C, W, lens};
    return launch_status(gdn::launch_conv_step(a, io_dtype == GDN_BF16, (hipStream_t)stream), fn);
}

int gdn_verify(const void* qkv, const void* beta_raw, const void* alpha, const float* dt_bias, const float* A_log,
               const float* S_in, float* S_out, float* H, void* o, int B, int K, int Hk, int Hv, int dk, int dv,
               int in_dtype, int o_dtype, float l2_eps, void* stream)
{
    return gdn_verify_ex(qkv, beta_raw, alpha, Hv, dt_bias, A_log, S_in, S_out, H, o, nullptr, B, K, Hk, Hv, dk, dv,
                         in_dtype, o_dtype, l2_eps, stream);
}

int gdn_verify_ex(const void* qkv, const void* beta_raw, const void* alpha, int gate_stride, const float* dt_bias,
                  const float* A_log, const float* S_in, float* S_out, float* H, void* o, const int32_t* lens, int B,
                  int K, int Hk, int Hv, int dk, int dv, int in_dtype, int o_dtype, float l2_eps, void* stream)
{
    const char* fn = "gdn_verify";
    int rc = check_gdn_shape(fn, B, K, Hk, Hv, dk, dv, in_dtype, o_dtype, l2_eps);
    if (rc) return rc;
    REQUIRE(K <= gdn::kVerifyMax, GDN_EUNSUPPORTED, "%s: K = %d > %d", fn, K, gdn::kVerifyMax);
    REQUIRE(B <= 65535 && Hv <= 65535, GDN_EUNSUPPORTED, "%s: B or Hv too large", fn);
    REQUIRE((dt_bias == nullptr) == (A_log == nullptr), GDN_EINVAL,
            "%s: dt_bias and A_log must be both given (raw gates) or both NULL (activated gates)", fn);
    if (B == 0) return ok();
    REQUIRE(qkv && beta_raw && alpha && S_in && S_out && o, GDN_EINVAL, "%s: null pointer", fn);
    REQUIRE(gate_stride >= Hv, GDN_EINVAL, "%s: gate_stride = %d < Hv = %d", fn, gate_stride, Hv);
    const size_t ie = elem_size(in_dtype), oe = elem_size(o_dtype);
    REQUIRE(aligned16(qkv) && aligned16(S_in) && aligned16(S_out) && aligned16(o) && (!H || aligned16(H)) &&
                (!dt_bias || (aligned16(dt_bias) && aligned16(A_log))),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(((uintptr_t)beta_raw % ie) == 0 && ((uintptr_t)alpha % ie) == 0 && (!lens || ((uintptr_t)lens & 3) == 0),
            GDN_EINVAL, "%s: gate or lens pointers not aligned to their element size", fn);
    const size_t C = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    const size_t SD = (size_t)B * Hv * dv * dk * 4;
    const size_t gspan = ((size_t)B * K - 1) * gate_stride + Hv;   // elements from the first to the last gate
    const Span sq{qkv, (size_t)B * K * C * ie}, sb{beta_raw, gspan * ie}, sa{alpha, gspan * ie},
        ssi{S_in, SD}, sso{S_out, SD},
        sH{H, H ? (size_t)B * (K - 1) * Hv * dv * dk * 4 : 0}, so{o, (size_t)B * K * Hv * dv * oe},
        sdt{dt_bias, dt_bias ? (size_t)Hv * 4 : 0}, sal{A_log, A_log ? (size_t)Hv * 4 : 0};
    REQUIRE(!(overlap(sso, ssi) && S_out != S_in), GDN_EINVAL, "%s: S_out partially overlaps S_in", fn);
    const Span sl{lens, lens ? (size_t)B * 4 : 0};
    const Span ins[] = {sq, sb, sa, sdt, sal, sl};
    for (const Span& s : ins) {
        REQUIRE(!overlap(sso, s), GDN_EINVAL, "%s: S_out overlaps an input", fn);
        REQUIRE(!overlap(sH, s) && !overlap(so, s), GDN_EINVAL, "%s: H or o overlaps an input", fn);
    }
    REQUIRE(!overlap(sH, ssi) && !overlap(sH, sso) && !overlap(so, ssi) && !overlap(so, sso) && !overlap(so, sH),
            GDN_EINVAL, "%s: H, o and the state buffers must not overlap", fn);
    gdn::VerifyArgs a{qkv, beta_raw, alpha, dt_bias, A_log, S_in, S_out, H, o, B, K, Hk, Hv, dk, dv, l2_eps, lens,
                      gate_stride};
    return launch_status(gdn::launch_verify(a, in_dtype == GDN_BF16, o_dtype == GDN_BF16, (hipStream_t)stream), fn);
}

int gdn_rollback(const int32_t* accept, int K, const float* S_in, const float* H, float* S_out, void* hist,
                 const void* win, int B, int Hv, int dv, int dk, int C, int W, int io_dtype, void* stream)
{
    return gdn_rollback_ex(accept, nullptr, K, S_in, H, S_out, hist, win, B, Hv, dv, dk, C, W, io_dtype, stream);
}

int gdn_rollback_ex(const int32_t* accept, const int32_t* lens, int K, const float* S_in, const float* H,
                    float* S_out, void* hist, const void* win, int B, int Hv, int dv, int dk, int C, int W,
                    int io_dtype, void* stream)
{
    const char* fn = "gdn_rollback";
    REQUIRE(B >= 0, GDN_EINVAL, "%s: B = %d < 0", fn, B);
    REQUIRE(K >= 1, GDN_EINVAL, "%s: K = %d < 1", fn, K);
    REQUIRE(Hv >= 1 && dv >= 1 && dk >= 1, GDN_EINVAL, "%s: bad state shape", fn);
    REQUIRE(((long long)Hv * dv * dk) % 4 == 0, GDN_EUNSUPPORTED, "%s: Hv*dv*dk must be a multiple of 4", fn);
    REQUIRE((hist == nullptr) == (win == nullptr), GDN_EINVAL, "%s: hist and win must be both given or both NULL",
            fn);
    if (hist) {
        REQUIRE(C >= 1, GDN_EINVAL, "%s: C = %d < 1", fn, C);
        REQUIRE(W >= 2 && W <= 8, GDN_EUNSUPPORTED, "%s: W = %d not in 2..8", fn, W);
        REQUIRE(valid_dtype(io_dtype), GDN_EINVAL, "%s: bad dtype code %d", fn, io_dtype);
    }
    REQUIRE(B <= 65535, GDN_EUNSUPPORTED, "%s: B = %d too large", fn, B);
    if (B == 0) return ok();
    REQUIRE(accept && S_in && S_out, GDN_EINVAL, "%s: null pointer", fn);
    REQUIRE(H || K == 1, GDN_EINVAL, "%s: H is required when K > 1", fn);
    REQUIRE(S_in != S_out, GDN_EINVAL, "%s: S_out must not be S_in (the pre-window state is needed)", fn);
    REQUIRE(aligned16(S_in) && aligned16(S_out) && (!H || aligned16(H)) && aligned16(accept) &&
                (!hist || (aligned16(hist) && aligned16(win))),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    const size_t st = (size_t)Hv * dv * dk * 4;
    const Span ssi{S_in, B * st}, sso{S_out, B * st}, sH{H, H ? (size_t)B * (K - 1) * st : 0};
    REQUIRE(!overlap(sso, ssi) && !overlap(sso, sH), GDN_EINVAL, "%s: S_out overlaps S_in or H", fn);
    REQUIRE(!lens || ((uintptr_t)lens & 3) == 0, GDN_EINVAL, "%s: lens must be 4-byte aligned", fn);
    REQUIRE(!overlap(sso, Span{lens, lens ? (size_t)B * 4 : 0}), GDN_EINVAL, "%s: S_out overlaps lens", fn);
    if (hist) {
        const size_t es = elem_size(io_dtype);
        const Span sh{hist, (size_t)B * (W - 1) * C * es}, sw{win, (size_t)B * (W - 1 + K) * C * es};
        REQUIRE(!overlap(sh, sw) && !overlap(sh, sso) && !overlap(sh, ssi) && !overlap(sh, sH), GDN_EINVAL,
                "%s: hist overlaps another buffer", fn);
    }
    gdn::RollbackArgs a{accept, S_in, H, S_out, hist, win, B, K, (long long)Hv * dv * dk, C, W,
                        (int)elem_size(io_dtype), lens};
    return launch_status(gdn::launch_rollback(a, (hipStream_t)stream), fn);
}

int gdn_replay(const int32_t* accept, const void* qkv, const void* beta_raw, const void* alpha, int gate_stride,
               const float* dt_bias, const float* A_log, const float* S_ckpt, float* S_out, void* hist,
               const void* win, int B, int K, int Hk, int Hv, int dk, int dv, int W, int in_dtype, float l2_eps,
               void* stream)
{
    const char* fn = "gdn_replay";
    int rc = check_gdn_shape(fn, B, K, Hk, Hv, dk, dv, in_dtype, GDN_F32, l2_eps);
    if (rc) return rc;
    REQUIRE(K <= gdn::kVerifyMax, GDN_EUNSUPPORTED, "%s: K = %d > %d", fn, K, gdn::kVerifyMax);
    REQUIRE(B <= 65535 && Hv <= 65535, GDN_EUNSUPPORTED, "%s: B or Hv too large", fn);
    REQUIRE((dt_bias == nullptr) == (A_log == nullptr), GDN_EINVAL,
            "%s: dt_bias and A_log must be both given (raw gates) or both NULL (activated gates)", fn);
    REQUIRE((hist == nullptr) == (win == nullptr), GDN_EINVAL, "%s: hist and win must be both given or both NULL",
            fn);
    if (hist) REQUIRE(W >= 2 && W <= 8, GDN_EUNSUPPORTED, "%s: W = %d not in 2..8", fn, W);
    if (B == 0) return ok();
    REQUIRE(accept && qkv && beta_raw && alpha && S_ckpt && S_out, GDN_EINVAL, "%s: null pointer", fn);
    REQUIRE(S_ckpt != S_out, GDN_EINVAL, "%s: S_out must not be the checkpoint", fn);
    REQUIRE(gate_stride >= Hv, GDN_EINVAL, "%s: gate_stride = %d < Hv = %d", fn, gate_stride, Hv);
    const size_t ie = elem_size(in_dtype);
    REQUIRE(aligned16(accept) && aligned16(qkv) && aligned16(S_ckpt) && aligned16(S_out) &&
                (!dt_bias || (aligned16(dt_bias) && aligned16(A_log))) && (!hist || (aligned16(hist) && aligned16(win))),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(((uintptr_t)beta_raw % ie) == 0 && ((uintptr_t)alpha % ie) == 0, GDN_EINVAL,
            "%s: gate pointers not aligned to their element size", fn);
    const size_t C = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    const size_t SD = (size_t)B * Hv * dv * dk * 4;
    const size_t gspan = ((size_t)B * K - 1) * gate_stride + Hv;
    const Span sq{qkv, (size_t)B * K * C * ie}, sb{beta_raw, gspan * ie}, sa{alpha, gspan * ie}, sc{S_ckpt, SD},
        sso{S_out, SD}, sacc{accept, (size_t)B * 4}, sdt{dt_bias, dt_bias ? (size_t)Hv * 4 : 0},
        sal{A_log, A_log ? (size_t)Hv * 4 : 0}, sh{hist, hist ? (size_t)B * (W - 1) * C * ie : 0},
        sw{win, win ? (size_t)B * (W - 1 + K) * C * ie : 0};
    const Span ins[] = {sq, sb, sa, sc, sacc, sdt, sal, sw};
    for (const Span& s : ins)
        REQUIRE(!overlap(sso, s) && !overlap(sh, s), GDN_EINVAL, "%s: an output overlaps an input", fn);
    REQUIRE(!overlap(sso, sh), GDN_EINVAL, "%s: S_out overlaps hist", fn);
    gdn::VerifyArgs a{qkv, beta_raw, alpha, dt_bias, A_log, S_ckpt, S_out, nullptr, nullptr, B, K, Hk, Hv, dk, dv,
                      l2_eps, nullptr, gate_stride, accept};
    rc = launch_status(gdn::launch_verify(a, in_dtype == GDN_BF16, false, (hipStream_t)stream), fn);
    if (rc || !hist) return rc;
    // the conv history of the accepted prefix: the rollback's conv rows only
    gdn::RollbackArgs r{accept, S_ckpt, nullptr, S_out, hist, win, B, K, 0, (int)C, W, (int)ie};
    return launch_status(gdn::launch_rollback(r, (hipStream_t)stream), fn);
}

int gdn_rollback_conv_step(const int32_t* accept, int K_prev, const float* S_in, const float* H, float* S_out,
                           const void* win_prev, const void* x, const float* w, void* hist, void* y, void* win,
                           int B, int Hv, int dv, int dk, int T, int C, int W, int io_dtype, void* stream)
{
    const char* fn = "gdn_rollback_conv_step";
    REQUIRE(B >= 0, GDN_EINVAL, "%s: B = %d < 0", fn, B);
    REQUIRE(K_prev >= 1, GDN_EINVAL, "%s: K_prev = %d < 1", fn, K_prev);
    REQUIRE(T >= 1, GDN_EINVAL, "%s: T = %d < 1", fn, T);
    REQUIRE(C >= 1, GDN_EINVAL, "%s: C = %d < 1", fn, C);
    REQUIRE(Hv >= 1 && dv >= 1 && dk >= 1, GDN_EINVAL, "%s: bad state shape", fn);
    REQUIRE(((long long)Hv * dv * dk) % 4 == 0, GDN_EUNSUPPORTED, "%s: Hv*dv*dk must be a multiple of 4", fn);
    REQUIRE(W >= 2 && W <= 8, GDN_EUNSUPPORTED, "%s: W = %d not in 2..8", fn, W);
    REQUIRE(valid_dtype(io_dtype), GDN_EINVAL, "%s: bad dtype code %d", fn, io_dtype);
    REQUIRE((long long)B * (T + K_prev) * C < (1LL << 40), GDN_EUNSUPPORTED, "%s: problem too large", fn);
    REQUIRE(T <= 65535 * 16, GDN_EUNSUPPORTED, "%s: T = %d too large", fn, T);
    REQUIRE(B <= 65535, GDN_EUNSUPPORTED, "%s: B = %d too large", fn, B);
    if (B == 0) return ok();
    REQUIRE(accept && S_in && S_out && win_prev && x && w && hist && y && win, GDN_EINVAL,
            "%s: null pointer (only H may be NULL, and only when K_prev == 1)", fn);
    REQUIRE(H || K_prev == 1, GDN_EINVAL, "%s: H is required when K_prev > 1", fn);
    REQUIRE(S_in != S_out, GDN_EINVAL, "%s: S_out must not be S_in (the pre-window state is needed)", fn);
    REQUIRE(aligned16(accept) && aligned16(S_in) && aligned16(S_out) && (!H || aligned16(H)) && aligned16(win_prev) &&
                aligned16(x) && aligned16(w) && aligned16(hist) && aligned16(y) && aligned16(win),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    const size_t st = (size_t)Hv * dv * dk * 4, es = elem_size(io_dtype);
    const Span ssi{S_in, B * st}, sso{S_out, B * st}, sH{H, H ? (size_t)B * (K_prev - 1) * st : 0},
        swp{win_prev, (size_t)B * (W - 1 + K_prev) * C * es}, sx{x, (size_t)B * T * C * es},
        sw{w, (size_t)C * W * 4}, sh{hist, (size_t)B * (W - 1) * C * es}, sy{y, (size_t)B * T * C * es},
        swin{win, (size_t)B * (W - 1 + T) * C * es}, sacc{accept, (size_t)B * 4};
    const Span ins[] = {ssi, sH, swp, sx, sw, sacc};
    const Span outs[] = {sso, sh, sy, swin};
    for (const Span& o : outs)
        for (const Span& i : ins) REQUIRE(!overlap(o, i), GDN_EINVAL, "%s: an output overlaps an input", fn);
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            REQUIRE(!overlap(outs[i], outs[j]), GDN_EINVAL, "%s: two outputs overlap", fn);
    gdn::RollConvArgs a{accept, K_prev, S_in, H, S_out, (long long)Hv * dv * dk, win_prev, x, w, hist, y, win,
                        B, T, C, W};
    return launch_status(gdn::launch_rollback_conv(a, io_dtype == GDN_BF16, (hipStream_t)stream), fn);
}

int gdn_prefill_chunked(const void* qkv, const void* beta_raw, const void* alpha, const float* dt_bias,
                        const float* A_log, const float* S_in, float* S_out, void* o, int B, int T, int chunk,
                        int Hk, int Hv, int dk, int dv, int in_dtype, int o_dtype, float l2_eps, void* stream)
{
    const char* fn = "gdn_prefill_chunked";
    int rc = check_gdn_shape(fn, B, T, Hk, Hv, dk, dv, in_dtype, o_dtype, l2_eps);
    if (rc) return rc;
    REQUIRE(chunk == 16 || chunk == 32 || chunk == 64, GDN_EUNSUPPORTED, "%s: chunk = %d not in {16, 32, 64}", fn,
            chunk);
    REQUIRE(B <= 65535 && Hv <= 65535, GDN_EUNSUPPORTED, "%s: B or Hv too large", fn);
    REQUIRE((dt_bias == nullptr) == (A_log == nullptr), GDN_EINVAL,
            "%s: dt_bias and A_log must be both given or both NULL", fn);
    if (B == 0) return ok();
    REQUIRE(qkv && beta_raw && alpha && S_in && S_out && o, GDN_EINVAL, "%s: null pointer", fn);
    REQUIRE(aligned16(qkv) && aligned16(beta_raw) && aligned16(alpha) && aligned16(S_in) && aligned16(S_out) &&
                aligned16(o) && (!dt_bias || (aligned16(dt_bias) && aligned16(A_log))),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    const size_t ie = elem_size(in_dtype), oe = elem_size(o_dtype);
    const size_t C = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    const size_t SD = (size_t)B * Hv * dv * dk * 4;
    const Span sq{qkv, (size_t)B * T * C * ie}, sb{beta_raw, (size_t)B * T * Hv * ie},
        sa{alpha, (size_t)B * T * Hv * ie}, ssi{S_in, SD}, sso{S_out, SD}, so{o, (size_t)B * T * Hv * dv * oe};
    REQUIRE(!(overlap(sso, ssi) && S_out != S_in), GDN_EINVAL, "%s: S_out partially overlaps S_in", fn);
    const Span ins[] = {sq, sb, sa};
    for (const Span& s : ins)
        REQUIRE(!overlap(sso, s) && !overlap(so, s), GDN_EINVAL, "%s: an output overlaps an input", fn);
    REQUIRE(!overlap(so, ssi) && !overlap(so, sso), GDN_EINVAL, "%s: o overlaps the state", fn);
    gdn::PrefillArgs a{qkv, beta_raw, alpha, dt_bias, A_log, S_in, S_out, o, B, T, chunk, Hk, Hv, dk, dv, l2_eps};
    return launch_status(gdn::launch_prefill(a, in_dtype == GDN_BF16, o_dtype == GDN_BF16, (hipStream_t)stream),
                         fn);
}

int gdn_verify_step(const int32_t* accept_prev, int K_prev, const float* S_prev_ckpt, const float* H_prev,
                    const float* S_prev_out, const void* win_prev, const float* S_in, const void* hist, const void* x,
                    const float* w, const void* beta_raw, const void* alpha, int gate_stride, const float* dt_bias,
                    const float* A_log, float* S_ckpt, float* S_out, float* H, void* o, void* y, void* win, int B,
                    int K, int Hk, int Hv, int dk, int dv, int W, int in_dtype, int o_dtype, float l2_eps,
                    void* stream)
{
    const char* fn = "gdn_verify_step";
    int rc = check_gdn_shape(fn, B, K, Hk, Hv, dk, dv, in_dtype, o_dtype, l2_eps);
    if (rc) return rc;
    REQUIRE(K <= gdn::kVerifyMax, GDN_EUNSUPPORTED, "%s: K = %d > %d", fn, K, gdn::kVerifyMax);
    REQUIRE(W == 4, GDN_EUNSUPPORTED, "%s: W = %d (the fused step takes conv width 4)", fn, W);
    REQUIRE(B <= 65535 && Hv <= 65535, GDN_EUNSUPPORTED, "%s: B or Hv too large", fn);
    REQUIRE((dt_bias == nullptr) == (A_log == nullptr), GDN_EINVAL,
            "%s: dt_bias and A_log must be both given (raw gates) or both NULL (activated gates)", fn);
    if (accept_prev)
        REQUIRE(K_prev >= 1 && K_prev <= gdn::kVerifyMax, GDN_EINVAL, "%s: K_prev = %d not in 1..%d", fn, K_prev,
                gdn::kVerifyMax);
    if (B == 0) return ok();
    REQUIRE(x && w && beta_raw && alpha && S_out && o, GDN_EINVAL, "%s: null pointer", fn);
    if (accept_prev) {
        REQUIRE(S_prev_ckpt && S_prev_out && win_prev && (H_prev || K_prev == 1), GDN_EINVAL,
                "%s: the previous window needs S_prev_ckpt, S_prev_out, win_prev and (K_prev > 1) H_prev", fn);
    } else {
        REQUIRE(S_in && hist, GDN_EINVAL, "%s: the first window needs S_in and hist", fn);
    }
    REQUIRE(gate_stride >= Hv, GDN_EINVAL, "%s: gate_stride = %d < Hv = %d", fn, gate_stride, Hv);
    const size_t ie = elem_size(in_dtype), oe = elem_size(o_dtype);
    auto a16 = [](const void* q) { return q == nullptr || aligned16(q); };
    REQUIRE(a16(x) && a16(w) && a16(S_prev_ckpt) && a16(H_prev) && a16(S_prev_out) && a16(win_prev) && a16(S_in) &&
                a16(hist) && a16(dt_bias) && a16(A_log) && a16(S_ckpt) && a16(S_out) && a16(H) && a16(o) && a16(y) &&
                a16(win),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(((uintptr_t)beta_raw % ie) == 0 && ((uintptr_t)alpha % ie) == 0 && ((uintptr_t)accept_prev & 3) == 0,
            GDN_EINVAL, "%s: gate or accept pointers not aligned to their element size", fn);
    const size_t C = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    const size_t st = (size_t)Hv * dv * dk * 4;
    const size_t gspan = ((size_t)B * K - 1) * gate_stride + Hv;
    const Span ins[] = {Span{x, (size_t)B * K * C * ie},
                        Span{w, C * 4 * 4},
                        Span{beta_raw, gspan * ie},
                        Span{alpha, gspan * ie},
                        Span{dt_bias, dt_bias ? (size_t)Hv * 4 : 0},
                        Span{A_log, A_log ? (size_t)Hv * 4 : 0},
                        Span{accept_prev, accept_prev ? (size_t)B * 4 : 0},
                        Span{accept_prev ? S_prev_ckpt : nullptr, B * st},
                        Span{accept_prev ? H_prev : nullptr, H_prev ? (size_t)B * (K_prev - 1) * st : 0},
                        Span{accept_prev ? S_prev_out : nullptr, B * st},
                        Span{accept_prev ? win_prev : nullptr, (size_t)B * (W - 1 + K_prev) * C * ie},
                        Span{accept_prev ? nullptr : S_in, B * st},
                        Span{accept_prev ? nullptr : hist, (size_t)B * (W - 1) * C * ie}};
    const Span outs[] = {Span{S_ckpt, B * st}, Span{S_out, B * st}, Span{H, H ? (size_t)B * (K - 1) * st : 0},
                         Span{o, (size_t)B * K * Hv * dv * oe}, Span{y, (size_t)B * K * C * ie},
                         Span{win, (size_t)B * (W - 1 + K) * C * ie}};
    for (const Span& q : outs)
        for (const Span& i : ins) REQUIRE(!overlap(q, i), GDN_EINVAL, "%s: an output overlaps an input", fn);
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j) REQUIRE(!overlap(outs[i], outs[j]), GDN_EINVAL, "%s: two outputs overlap", fn);
    gdn::VerifyArgs a{x, beta_raw, alpha, dt_bias, A_log, accept_prev ? nullptr : S_in, S_out, H, o, B, K, Hk, Hv,
                      dk, dv, l2_eps, nullptr, gate_stride};
    a.x = x;
    a.w = w;
    a.hsrc = accept_prev ? win_prev : hist;
    a.hrows = accept_prev ? W - 1 + K_prev : W - 1;
    a.acc_prev = accept_prev;
    a.Kp = accept_prev ? K_prev : 0;
    a.Sp_ckpt = S_prev_ckpt;
    a.Sp_H = H_prev;
    a.Sp_out = S_prev_out;
    a.S_ckpt = S_ckpt;
    a.y = y;
    a.win = win;
    return launch_status(gdn::launch_step(a, in_dtype == GDN_BF16, o_dtype == GDN_BF16, (hipStream_t)stream), fn);
}

int gdn_conv_tree(const void* x, const float* w, const void* hist, const int32_t* parent, void* y, int B, int N,
                  int C, int W, int io_dtype, void* stream)
{
    const char* fn = "gdn_conv_tree";
    REQUIRE(B >= 0, GDN_EINVAL, "%s: B = %d < 0", fn, B);
    REQUIRE(N >= 1, GDN_EINVAL, "%s: N = %d < 1", fn, N);
    REQUIRE(N <= gdn::kTreeMax, GDN_EUNSUPPORTED, "%s: N = %d > %d", fn, N, gdn::kTreeMax);
    REQUIRE(C >= 1, GDN_EINVAL, "%s: C = %d < 1", fn, C);
    REQUIRE(W >= 2 && W <= 8, GDN_EUNSUPPORTED, "%s: W = %d not in 2..8", fn, W);
    REQUIRE(valid_dtype(io_dtype), GDN_EINVAL, "%s: bad dtype code %d", fn, io_dtype);
    REQUIRE((long long)B * N * C < (1LL << 40), GDN_EUNSUPPORTED, "%s: problem too large", fn);
    REQUIRE(B <= 65535, GDN_EUNSUPPORTED, "%s: B = %d too large", fn, B);
    if (B == 0) return ok();
    REQUIRE(x && w && hist && parent && y, GDN_EINVAL, "%s: null pointer", fn);
    REQUIRE(aligned16(x) && aligned16(w) && aligned16(hist) && aligned16(y), GDN_EINVAL,
            "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(((uintptr_t)parent & 3) == 0, GDN_EINVAL, "%s: parent must be 4-byte aligned", fn);
    const size_t es = elem_size(io_dtype);
    const Span sy{y, (size_t)B * N * C * es};
    const Span ins[] = {Span{x, (size_t)B * N * C * es}, Span{w, (size_t)C * W * 4},
                        Span{hist, (size_t)B * (W - 1) * C * es}, Span{parent, (size_t)B * N * 4}};
    for (const Span& s : ins) REQUIRE(!overlap(sy, s), GDN_EINVAL, "%s: y overlaps an input", fn);
    gdn::ConvTreeArgs a{x, w, hist, parent, y, B, N, C, W};
    return launch_status(gdn::launch_conv_tree(a, io_dtype == GDN_BF16, (hipStream_t)stream), fn);
}

int gdn_verify_tree(const void* qkv, const void* beta_raw, const void* alpha, int gate_stride, const float* dt_bias,
                    const float* A_log, const int32_t* parent, const float* S_in, float* H, void* o, int B, int N,
                    int Hk, int Hv, int dk, int dv, int in_dtype, int o_dtype, float l2_eps, void* stream)
{
    const char* fn = "gdn_verify_tree";
    int rc = check_gdn_shape(fn, B, N, Hk, Hv, dk, dv, in_dtype, o_dtype, l2_eps);
    if (rc) return rc;
    REQUIRE(N <= gdn::kTreeMax, GDN_EUNSUPPORTED, "%s: N = %d > %d", fn, N, gdn::kTreeMax);
    REQUIRE(B <= 65535 && Hv <= 65535, GDN_EUNSUPPORTED, "%s: B or Hv too large", fn);
    REQUIRE((dt_bias == nullptr) == (A_log == nullptr), GDN_EINVAL,
            "%s: dt_bias and A_log must be both given (raw gates) or both NULL (activated gates)", fn);
    if (B == 0) return ok();
    REQUIRE(qkv && beta_raw && alpha && parent && S_in && H && o, GDN_EINVAL, "%s: null pointer", fn);
    REQUIRE(gate_stride >= Hv, GDN_EINVAL, "%s: gate_stride = %d < Hv = %d", fn, gate_stride, Hv);
    const size_t ie = elem_size(in_dtype), oe = elem_size(o_dtype);
    REQUIRE(aligned16(qkv) && aligned16(S_in) && aligned16(H) && aligned16(o) &&
                (!dt_bias || (aligned16(dt_bias) && aligned16(A_log))),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(((uintptr_t)beta_raw % ie) == 0 && ((uintptr_t)alpha % ie) == 0 && ((uintptr_t)parent & 3) == 0,
            GDN_EINVAL, "%s: gate or parent pointers not aligned to their element size", fn);
    const size_t C = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    const size_t st = (size_t)Hv * dv * dk * 4;
    const size_t gspan = ((size_t)B * N - 1) * gate_stride + Hv;
    const Span sH{H, (size_t)B * N * st}, so{o, (size_t)B * N * Hv * dv * oe};
    const Span ins[] = {Span{qkv, (size_t)B * N * C * ie}, Span{beta_raw, gspan * ie}, Span{alpha, gspan * ie},
                        Span{dt_bias, dt_bias ? (size_t)Hv * 4 : 0}, Span{A_log, A_log ? (size_t)Hv * 4 : 0},
                        Span{parent, (size_t)B * N * 4}, Span{S_in, B * st}};
    for (const Span& s : ins)
        REQUIRE(!overlap(sH, s) && !overlap(so, s), GDN_EINVAL, "%s: H or o overlaps an input", fn);
    REQUIRE(!overlap(sH, so), GDN_EINVAL, "%s: H and o overlap", fn);
    gdn::VerifyArgs a{qkv, beta_raw, alpha, dt_bias, A_log, S_in, nullptr, H, o, B, N, Hk, Hv, dk, dv, l2_eps,
                      nullptr, gate_stride, nullptr, parent};
    return launch_status(gdn::launch_verify(a, in_dtype == GDN_BF16, o_dtype == GDN_BF16, (hipStream_t)stream), fn);
}

int gdn_rollback_tree(const int32_t* node, const int32_t* parent, int N, const float* S_in, const float* H,
                      float* S_out, const void* x, void* hist, int B, int Hv, int dv, int dk, int C, int W,
                      int io_dtype, void* stream)
{
    const char* fn = "gdn_rollback_tree";
    REQUIRE(B >= 0, GDN_EINVAL, "%s: B = %d < 0", fn, B);
    REQUIRE(N >= 1, GDN_EINVAL, "%s: N = %d < 1", fn, N);
    REQUIRE(N <= gdn::kTreeMax, GDN_EUNSUPPORTED, "%s: N = %d > %d", fn, N, gdn::kTreeMax);
    REQUIRE(Hv >= 1 && dv >= 1 && dk >= 1, GDN_EINVAL, "%s: bad state shape", fn);
    REQUIRE(((long long)Hv * dv * dk) % 4 == 0, GDN_EUNSUPPORTED, "%s: Hv*dv*dk must be a multiple of 4", fn);
    REQUIRE((hist == nullptr) == (x == nullptr), GDN_EINVAL, "%s: x and hist must be both given or both NULL", fn);
    if (hist) {
        REQUIRE(C >= 1, GDN_EINVAL, "%s: C = %d < 1", fn, C);
        REQUIRE(W >= 2 && W <= 8, GDN_EUNSUPPORTED, "%s: W = %d not in 2..8", fn, W);
        REQUIRE(valid_dtype(io_dtype), GDN_EINVAL, "%s: bad dtype code %d", fn, io_dtype);
    }
    REQUIRE(B <= 65535, GDN_EUNSUPPORTED, "%s: B = %d too large", fn, B);
    if (B == 0) return ok();
    REQUIRE(node && parent && S_in && H && S_out, GDN_EINVAL, "%s: null pointer", fn);
    REQUIRE(S_in != S_out, GDN_EINVAL, "%s: S_out must not be S_in", fn);
    REQUIRE(aligned16(S_in) && aligned16(S_out) && aligned16(H) && (!hist || (aligned16(hist) && aligned16(x))),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(((uintptr_t)node & 3) == 0 && ((uintptr_t)parent & 3) == 0, GDN_EINVAL,
            "%s: node and parent must be 4-byte aligned", fn);
    const size_t st = (size_t)Hv * dv * dk * 4;
    const Span sso{S_out, B * st}, sh{hist, hist ? (size_t)B * (W - 1) * C * elem_size(io_dtype) : 0};
    const Span ins[] = {Span{S_in, B * st}, Span{H, (size_t)B * N * st}, Span{node, (size_t)B * 4},
                        Span{parent, (size_t)B * N * 4},
                        Span{x, x ? (size_t)B * N * C * elem_size(io_dtype) : 0}};
    for (const Span& s : ins)
        REQUIRE(!overlap(sso, s) && !overlap(sh, s), GDN_EINVAL, "%s: an output overlaps an input", fn);
    REQUIRE(!overlap(sso, sh), GDN_EINVAL, "%s: S_out overlaps hist", fn);
    gdn::TreeRollbackArgs a{node, parent, S_in, H, S_out, (long long)Hv * dv * dk, x, hist, B, N, C, W,
                            (int)elem_size(io_dtype)};
    return launch_status(gdn::launch_tree_rollback(a, (hipStream_t)stream), fn);
}

int gdn_verify_tree_step(const int32_t* node_prev, int N_prev, const int32_t* parent_prev, const float* S_prev_ckpt,
                         const float* H_prev, const void* x_prev, const void* hist_prev, const void* x, const float* w,
                         const int32_t* parent, const void* beta_raw, const void* alpha, int gate_stride,
                         const float* dt_bias, const float* A_log, float* S_ckpt, float* H, void* o, void* y,
                         void* hist_out, int B, int N, int Hk, int Hv, int dk, int dv, int W, int in_dtype,
                         int o_dtype, float l2_eps, void* stream)
{
    const char* fn = "gdn_verify_tree_step";
    int rc = check_gdn_shape(fn, B, N, Hk, Hv, dk, dv, in_dtype, o_dtype, l2_eps);
    if (rc) return rc;
    REQUIRE(N <= gdn::kTreeMax, GDN_EUNSUPPORTED, "%s: N = %d > %d", fn, N, gdn::kTreeMax);
    REQUIRE(W >= 2 && W <= 8, GDN_EUNSUPPORTED, "%s: W = %d not in 2..8", fn, W);
    REQUIRE(B <= 65535 && Hv <= 65535, GDN_EUNSUPPORTED, "%s: B or Hv too large", fn);
    REQUIRE((dt_bias == nullptr) == (A_log == nullptr), GDN_EINVAL,
            "%s: dt_bias and A_log must be both given (raw gates) or both NULL (activated gates)", fn);
    if (node_prev)
        REQUIRE(N_prev >= 1 && N_prev <= gdn::kTreeMax, GDN_EINVAL, "%s: N_prev = %d not in 1..%d", fn, N_prev,
                gdn::kTreeMax);
    if (B == 0) return ok();
    REQUIRE(S_prev_ckpt && hist_prev && x && w && parent && beta_raw && alpha && H && o && y, GDN_EINVAL,
            "%s: null pointer", fn);
    if (node_prev)
        REQUIRE(parent_prev && H_prev && x_prev, GDN_EINVAL,
                "%s: a previous tree needs parent_prev, H_prev and x_prev", fn);
    REQUIRE(gate_stride >= Hv, GDN_EINVAL, "%s: gate_stride = %d < Hv = %d", fn, gate_stride, Hv);
    const size_t ie = elem_size(in_dtype), oe = elem_size(o_dtype);
    auto a16 = [](const void* q) { return q == nullptr || aligned16(q); };
    REQUIRE(a16(S_prev_ckpt) && a16(H_prev) && a16(x_prev) && a16(hist_prev) && a16(x) && a16(w) && a16(dt_bias) &&
                a16(A_log) && a16(S_ckpt) && a16(H) && a16(o) && a16(y) && a16(hist_out),
            GDN_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    REQUIRE(((uintptr_t)beta_raw % ie) == 0 && ((uintptr_t)alpha % ie) == 0 && ((uintptr_t)parent & 3) == 0 &&
                ((uintptr_t)node_prev & 3) == 0 && ((uintptr_t)parent_prev & 3) == 0,
            GDN_EINVAL, "%s: gate, node or parent pointers not aligned to their element size", fn);
    const size_t C = (size_t)2 * Hk * dk + (size_t)Hv * dv;
    const size_t st = (size_t)Hv * dv * dk * 4;
    const size_t gspan = ((size_t)B * N - 1) * gate_stride + Hv;
    const size_t hrows = (size_t)B * (W - 1) * C * ie;
    const Span ins[] = {Span{node_prev, node_prev ? (size_t)B * 4 : 0},
                        Span{node_prev ? parent_prev : nullptr, node_prev ? (size_t)B * N_prev * 4 : 0},
                        Span{S_prev_ckpt, B * st},
                        Span{node_prev ? H_prev : nullptr, node_prev ? (size_t)B * N_prev * st : 0},
                        Span{node_prev ? x_prev : nullptr, node_prev ? (size_t)B * N_prev * C * ie : 0},
                        Span{hist_prev, hrows},
                        Span{x, (size_t)B * N * C * ie},
                        Span{w, C * W * 4},
                        Span{parent, (size_t)B * N * 4},
                        Span{beta_raw, gspan * ie},
                        Span{alpha, gspan * ie},
                        Span{dt_bias, dt_bias ? (size_t)Hv * 4 : 0},
                        Span{A_log, A_log ? (size_t)Hv * 4 : 0}};
    const Span outs[] = {Span{S_ckpt, B * st}, Span{H, (size_t)B * N * st}, Span{o, (size_t)B * N * Hv * dv * oe},
                         Span{y, (size_t)B * N * C * ie}, Span{hist_out, hist_out ? hrows : 0}};
    for (const Span& q : outs)
        for (const Span& i : ins) REQUIRE(!overlap(q, i), GDN_EINVAL, "%s: an output overlaps an input", fn);
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j) REQUIRE(!overlap(outs[i], outs[j]), GDN_EINVAL, "%s: two outputs overlap", fn);
    // 1. the conv of every node, its history the previous tree's accepted path (then hist_prev)
    gdn::ConvTreeArgs c{x, w, hist_prev, parent, y, B, N, (int)C, W};
    c.node_prev = node_prev;
    c.parent_prev = parent_prev;
    c.x_prev = x_prev;
    c.N_prev = node_prev ? N_prev : 0;
    c.hist_out = hist_out;
    rc = launch_status(gdn::launch_conv_tree(c, in_dtype == GDN_BF16, (hipStream_t)stream), fn);
    if (rc) return rc;
    // 2. the tree verify from the start state the accepted node picks, written out as the checkpoint
    gdn::VerifyArgs a{y, beta_raw, alpha, dt_bias, A_log, S_prev_ckpt, nullptr, H, o, B, N, Hk, Hv, dk, dv, l2_eps,
                      nullptr, gate_stride, nullptr, parent};
    a.acc_prev = node_prev;
    a.Kp = node_prev ? N_prev : 0;
    a.Sp_ckpt = S_prev_ckpt;
    a.Sp_H = H_prev;
    a.S_ckpt = S_ckpt;
    a.pick = true;
    return launch_status(gdn::launch_verify(a, in_dtype == GDN_BF16, o_dtype == GDN_BF16, (hipStream_t)stream), fn);
}

}  // extern "C"
