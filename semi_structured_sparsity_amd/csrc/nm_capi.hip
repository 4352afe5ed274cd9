// C ABI of libnmsparse: argument validation, error reporting and dispatch to
// the kernels.  Nothing is enqueued unless every check passes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "nm_internal.h"

namespace nm {

static thread_local char g_err[512] = "";

nm_status set_error(nm_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

nm_status check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(NM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return NM_OK;
}

static int64_t esize(nm_dtype d) { return d == NM_BF16 ? 2 : (d == NM_I8 || d == NM_FP8) ? 1 : 4; }
static bool dtype_ok(nm_dtype d) { return d == NM_F32 || d == NM_BF16 || d == NM_I8 || d == NM_I32 || d == NM_FP8; }
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Range {
    uintptr_t lo, hi;
};
// Byte range touched by a row-major [rows, cols] view with leading dimension ld.
static Range span(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t es) {
    if (!p || rows <= 0 || cols <= 0) return {0, 0};
    const uintptr_t b = (uintptr_t)p;
    return {b, b + (uintptr_t)(((rows - 1) * ld + cols) * es)};
}
static bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

#define NM_REQ(cond, st, ...)                                                \
    do {                                                                     \
        if (!(cond)) return set_error(st, __VA_ARGS__);                      \
    } while (0)

static nm_status check_pattern(int N, int M, const char* fn) {
    NM_REQ(M == 4 || M == 8, NM_ERR_PATTERN, "%s: M must be 4 or 8 (got %d)", fn, M);
    NM_REQ(N >= 1 && N < M, NM_ERR_PATTERN, "%s: need 1 <= N < M (got N=%d, M=%d)", fn, N, M);
    return NM_OK;
}

static int64_t idx_words_needed(int64_t K, int N, int M) { return (K / M * N * index_bits(M) + 31) / 32; }

static nm_status check_score_src(const void* W, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh,
                                 nm_score_mode mode, int64_t R, int64_t K, const char* fn) {
    NM_REQ(W || R * K == 0, NM_ERR_NULL, "%s: score source is NULL", fn);
    NM_REQ(sdt == NM_F32 || sdt == NM_BF16, NM_ERR_DTYPE, "%s: score source must be f32 or bf16", fn);
    NM_REQ(ldsc >= K, NM_ERR_SHAPE, "%s: score leading dimension %lld < K %lld", fn, (long long)ldsc, (long long)K);
    NM_REQ(mode == NM_SCORE_HESSIAN || mode == NM_SCORE_MAGNITUDE, NM_ERR_SHAPE, "%s: unknown score mode", fn);
    if (mode == NM_SCORE_HESSIAN) {
        NM_REQ(H || R * K == 0, NM_ERR_NULL, "%s: H is NULL in HESSIAN mode", fn);
        NM_REQ(ldh == 0 || ldh >= K, NM_ERR_SHAPE, "%s: ldh must be 0 or >= K", fn);
    }
    return NM_OK;
}

}  // namespace nm

using namespace nm;

extern "C" {

int nm_abi_version(void) { return NM_ABI_VERSION; }

const char* nm_last_error(void) { return g_err; }

size_t nm_colsumsq_workspace(int64_t n, int64_t K) { return (n <= 0 || K <= 0) ? 0 : colsumsq_ws(n, K); }

nm_status nm_hdiag_colsumsq(const void* X, nm_dtype xdt, int64_t n, int64_t K, int64_t ldx, float* H, void* ws,
                            size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_hdiag_colsumsq";
    NM_REQ(n >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    if (K == 0) return NM_OK;
    NM_REQ(H, NM_ERR_NULL, "%s: H is NULL", fn);
    NM_REQ(X || n == 0, NM_ERR_NULL, "%s: X is NULL", fn);
    NM_REQ(xdt == NM_BF16 || xdt == NM_F32, NM_ERR_DTYPE, "%s: X must be bf16 or f32", fn);
    NM_REQ(ldx >= K, NM_ERR_SHAPE, "%s: ldx < K", fn);
    const int64_t vec = 16 / esize(xdt);
    NM_REQ(K % vec == 0 && ldx % vec == 0 && aligned16(X), NM_ERR_ALIGN,
           "%s: X must be 16-byte aligned with K and ldx multiples of %lld", fn, (long long)vec);
    const size_t need = nm_colsumsq_workspace(n, K);
    NM_REQ(need == 0 || (ws && ws_bytes >= need), NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    NM_REQ(!overlap(span(H, 1, K, K, 4), span(X, n, K, ldx, esize(xdt))), NM_ERR_ALIAS, "%s: H overlaps X", fn);
    launch_colsumsq(X, xdt, n, K, ldx, H, ws, (hipStream_t)stream);
    return check_launch(fn);
}

size_t nm_hutchinson_workspace(int64_t n, int64_t K, int64_t R, int probes) {
    if (n <= 0 || K <= 0 || R <= 0 || probes <= 0) return 0;
    return hutch_ws(n, K, R, probes);
}

nm_status nm_hdiag_hutchinson(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes, uint64_t seed,
                              float* D, int64_t ldd, void* ws, size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_hdiag_hutchinson";
    NM_REQ(n >= 0 && K >= 0 && R >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(probes >= 1, NM_ERR_SHAPE, "%s: probes must be >= 1", fn);
    if (R == 0 || K == 0) return NM_OK;
    NM_REQ(X && D, NM_ERR_NULL, "%s: NULL pointer", fn);
    NM_REQ(n >= 1, NM_ERR_SHAPE, "%s: need at least one calibration row", fn);
    NM_REQ(ldx >= K && ldd >= K, NM_ERR_SHAPE, "%s: leading dimension < K", fn);
    NM_REQ(K % 64 == 0 && n % 64 == 0 && ldx % 8 == 0 && aligned16(X), NM_ERR_ALIGN,
           "%s: need K %% 64 == 0, n %% 64 == 0, 16-byte aligned X with ldx %% 8 == 0", fn);
    NM_REQ((int64_t)probes * R < (1LL << 31) && (uint64_t)R * (uint64_t)(K / 64) < (1ull << 40), NM_ERR_SHAPE,
           "%s: too many probe rows", fn);
    const size_t need = hutch_ws(n, K, R, probes);
    NM_REQ(ws && ws_bytes >= need, NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    NM_REQ(!overlap(span(D, R, K, ldd, 4), span(X, n, K, ldx, 2)), NM_ERR_ALIAS, "%s: D overlaps X", fn);
    launch_hutchinson(X, n, K, ldx, R, probes, seed, D, ldd, ws, (hipStream_t)stream);
    return check_launch(fn);
}

size_t nm_hutchinson_score_workspace(int64_t n, int64_t K, int64_t R, int probes) {
    if (n <= 0 || K <= 0 || R <= 0 || probes <= 0) return 0;
    return hutch_score_ws(n, K, R, probes);
}

nm_status nm_hutchinson_score(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes, uint64_t seed,
                              const void* W, nm_dtype wdt, int64_t ldw, float eps, float* S, int64_t lds,
                              double* stats, void* ws, size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_hutchinson_score";
    NM_REQ(n >= 0 && K >= 0 && R >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(probes >= 1, NM_ERR_SHAPE, "%s: probes must be >= 1", fn);
    NM_REQ(wdt == NM_BF16, NM_ERR_DTYPE, "%s: W must be bf16", fn);
    if (R == 0 || K == 0) return NM_OK;
    NM_REQ(X && W && S, NM_ERR_NULL, "%s: NULL pointer", fn);
    NM_REQ(n >= 1, NM_ERR_SHAPE, "%s: need at least one calibration row", fn);
    NM_REQ(ldx >= K && ldw >= K && lds >= K, NM_ERR_SHAPE, "%s: leading dimension < K", fn);
    NM_REQ(K % 64 == 0 && n % 64 == 0 && ldx % 8 == 0 && aligned16(X), NM_ERR_ALIGN,
           "%s: need K %% 64 == 0, n %% 64 == 0, 16-byte aligned X with ldx %% 8 == 0", fn);
    NM_REQ(((uintptr_t)W & 7u) == 0 && ldw % 4 == 0 && aligned16(S) && lds % 4 == 0 && aligned16(ws), NM_ERR_ALIGN,
           "%s: need 8-byte aligned W (ldw %% 4), 16-byte aligned S (lds %% 4) and workspace", fn);
    // the fused epilogue lives in the dense split ring: its 32-bit offsets must hold
    NM_REQ((int64_t)probes * R < (1LL << 31) && (uint64_t)R * (uint64_t)(K / 64) < (1ull << 40) &&
               (int64_t)probes * R * n * 2 < (1LL << 32) && K * n * 2 < (1LL << 32),
           NM_ERR_SHAPE, "%s: problem too large for the fused kernel (use nm_hdiag_hutchinson + nm_score)", fn);
    const size_t need = hutch_score_ws(n, K, R, probes);
    NM_REQ(ws && ws_bytes >= need, NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    const Range rs = span(S, R, K, lds, 4), rw = Range{(uintptr_t)ws, (uintptr_t)ws + need};
    const Range rst = span(stats, 1, 2, 2, 8);
    NM_REQ(!overlap(rs, span(X, n, K, ldx, 2)) && !overlap(rs, span(W, R, K, ldw, 2)) && !overlap(rs, rw) &&
               !overlap(rst, rs) && !overlap(rst, rw) && !overlap(rst, span(X, n, K, ldx, 2)) &&
               !overlap(rst, span(W, R, K, ldw, 2)) && !overlap(rw, span(X, n, K, ldx, 2)) &&
               !overlap(rw, span(W, R, K, ldw, 2)),
           NM_ERR_ALIAS, "%s: an output or the workspace overlaps an input", fn);
    return launch_hutchinson_score(X, n, K, ldx, R, probes, seed, (const uint16_t*)W, ldw, eps, S, lds, stats, ws,
                                   (hipStream_t)stream);
}

nm_status nm_score(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const float* H, int64_t ldh,
                   float eps, nm_score_mode mode, float* S, int64_t lds, nm_stream_t stream) {
    const char* fn = "nm_score";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    if (R * K == 0) return NM_OK;
    nm_status st = check_score_src(W, wdt, ldw, H, ldh, mode, R, K, fn);
    if (st != NM_OK) return st;
    NM_REQ(S, NM_ERR_NULL, "%s: S is NULL", fn);
    NM_REQ(lds >= K, NM_ERR_SHAPE, "%s: lds < K", fn);
    const Range rs = span(S, R, K, lds, 4);
    NM_REQ(!overlap(rs, span(W, R, K, ldw, esize(wdt))), NM_ERR_ALIAS, "%s: S overlaps W", fn);
    if (mode == NM_SCORE_HESSIAN)
        NM_REQ(!overlap(rs, span(H, ldh ? R : 1, K, ldh ? ldh : K, 4)), NM_ERR_ALIAS, "%s: S overlaps H", fn);
    launch_score(W, wdt, R, K, ldw, H, ldh, eps, mode, S, lds, (hipStream_t)stream);
    return check_launch(fn);
}

size_t nm_stats_workspace(int64_t R, int64_t K) { return reduce_ws(R, K); }

nm_status nm_score_stats(const float* S, int64_t R, int64_t K, int64_t lds, double* stats, void* ws, size_t ws_bytes,
                         nm_stream_t stream) {
    const char* fn = "nm_score_stats";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(stats, NM_ERR_NULL, "%s: stats is NULL", fn);
    NM_REQ(S || R * K == 0, NM_ERR_NULL, "%s: S is NULL", fn);
    NM_REQ(lds >= K, NM_ERR_SHAPE, "%s: lds < K", fn);
    const size_t need = reduce_ws(R, K);
    NM_REQ(ws && ws_bytes >= need, NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    NM_REQ(!overlap(span(stats, 1, 2, 2, 8), span(S, R, K, lds, 4)), NM_ERR_ALIAS, "%s: stats overlaps S", fn);
    launch_stats(S, R, K, lds, stats, ws, (hipStream_t)stream);
    return check_launch(fn);
}

size_t nm_gate_workspace(int64_t R, int64_t K, int steps) { return gate_ws(R, K, steps); }

nm_status nm_gate(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats, int N, int M, float T0,
                  float rho, int steps, int m_step, float* m, int64_t ldf, uint8_t* hard_mask, int64_t ldm,
                  double* lmid, void* ws, size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_gate";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    nm_status st = check_pattern(N, M, fn);
    if (st != NM_OK) return st;
    NM_REQ(K % M == 0, NM_ERR_SHAPE, "%s: K %% M != 0", fn);
    NM_REQ(steps >= 1 && steps <= 64, NM_ERR_SHAPE, "%s: steps must be in [1, 64]", fn);
    NM_REQ(!m || (m_step >= 0 && m_step < steps), NM_ERR_SHAPE, "%s: m_step must be in [0, steps)", fn);
    NM_REQ(T0 > 0.f && rho > 0.f, NM_ERR_SHAPE, "%s: T0 and rho must be positive", fn);
    NM_REQ(stats && lmid, NM_ERR_NULL, "%s: stats / lmid is NULL", fn);
    NM_REQ((S && hard_mask) || R * K == 0, NM_ERR_NULL, "%s: NULL pointer", fn);
    NM_REQ(lds >= K && ldm >= (K + 7) / 8 && (!m || ldf >= K), NM_ERR_SHAPE, "%s: leading dimension too small", fn);
    const size_t need = gate_ws(R, K, steps);
    NM_REQ(ws && ws_bytes >= need, NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    const Range rs = span(S, R, K, lds, 4), rh = span(hard_mask, R, (K + 7) / 8, ldm, 1), rm = span(m, R, K, ldf, 4);
    const Range rl = span(lmid, 1, steps, steps, 8), rw = Range{(uintptr_t)ws, (uintptr_t)ws + need};
    const Range ins[2] = {rs, span(stats, 1, 2, 2, 8)};
    for (const Range& x : ins)
        NM_REQ(!overlap(x, rh) && !overlap(x, rm) && !overlap(x, rl) && !overlap(x, rw), NM_ERR_ALIAS,
               "%s: an output or the workspace overlaps S or stats", fn);
    NM_REQ(!overlap(rh, rm) && !overlap(rh, rl) && !overlap(rm, rl), NM_ERR_ALIAS, "%s: outputs overlap", fn);
    launch_gate(S, R, K, lds, stats, N, M, T0, rho, steps, m ? m_step : -1, m, ldf, hard_mask, ldm, lmid, ws,
                (hipStream_t)stream);
    return check_launch(fn);
}

nm_status nm_mask(const float* S, int64_t R, int64_t K, int64_t lds, int N, int M, uint8_t* mask, int64_t ldm,
                  nm_stream_t stream) {
    const char* fn = "nm_mask";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    nm_status st = check_pattern(N, M, fn);
    if (st != NM_OK) return st;
    NM_REQ(K % M == 0, NM_ERR_SHAPE, "%s: K %% M != 0", fn);
    if (R * K == 0) return NM_OK;
    NM_REQ(S && mask, NM_ERR_NULL, "%s: NULL pointer", fn);
    NM_REQ(lds >= K && ldm >= (K + 7) / 8, NM_ERR_SHAPE, "%s: leading dimension too small", fn);
    NM_REQ(!overlap(span(mask, R, (K + 7) / 8, ldm, 1), span(S, R, K, lds, 4)), NM_ERR_ALIAS, "%s: mask overlaps S",
           fn);
    launch_mask(S, R, K, lds, N, M, mask, ldm, (hipStream_t)stream);
    return check_launch(fn);
}

static nm_status check_pack_out(const char* fn, nm_dtype wdt, nm_dtype vdt, int64_t R, int64_t K, int64_t slots,
                                int64_t words, const void* vals, int64_t ldv, const uint32_t* idx, int64_t ldi) {
    NM_REQ(dtype_ok(wdt) && dtype_ok(vdt), NM_ERR_DTYPE, "%s: unknown dtype", fn);
    NM_REQ(vdt == wdt || (wdt == NM_F32 && vdt == NM_BF16), NM_ERR_DTYPE,
           "%s: value dtype must equal the weight dtype (or f32 -> bf16)", fn);
    NM_REQ(vals && idx, NM_ERR_NULL, "%s: vals / idx is NULL", fn);
    NM_REQ(ldv >= slots && ldi >= words, NM_ERR_SHAPE, "%s: ldv/ldi too small (need %lld / %lld)", fn,
           (long long)slots, (long long)words);
    NM_REQ(!overlap(span(vals, R, slots, ldv, esize(vdt)), span(idx, R, words, ldi, 4)), NM_ERR_ALIAS,
           "%s: vals overlaps idx", fn);
    (void)K;
    return NM_OK;
}

// NM_FLAG_VALIDATE: count the mask's groups with more than cap bits (a stream
// synchronisation) and refuse to pack when there are any.
static nm_status validate_mask(const char* fn, unsigned flags, const uint8_t* mask, int64_t ldm, int64_t R, int64_t K,
                               int G, int cap, nm_stream_t stream) {
    if (!(flags & NM_FLAG_VALIDATE)) return NM_OK;
    int64_t bad = 0;
    const nm_status st = count_overfull(mask, ldm, R, K, G, cap, (hipStream_t)stream, &bad);
    if (st != NM_OK) return st;
    NM_REQ(bad == 0, NM_ERR_PATTERN, "%s: %lld groups of %d have more than %d mask bits", fn, (long long)bad, G, cap);
    return NM_OK;
}

nm_status nm_pack(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask, int64_t ldm,
                  int N, int M, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx, int64_t ldi, unsigned flags,
                  nm_stream_t stream) {
    const char* fn = "nm_pack";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ((flags & ~NM_FLAG_VALIDATE) == 0, NM_ERR_SHAPE, "%s: unknown flags 0x%x", fn, flags);
    nm_status st = check_pattern(N, M, fn);
    if (st != NM_OK) return st;
    NM_REQ(K % M == 0, NM_ERR_SHAPE, "%s: K %% M != 0", fn);
    if (R * K == 0) return NM_OK;
    NM_REQ(W && mask, NM_ERR_NULL, "%s: W / mask is NULL", fn);
    NM_REQ(ldw >= K && ldm >= (K + 7) / 8, NM_ERR_SHAPE, "%s: leading dimension too small", fn);
    const int64_t slots = K / M * N, words = idx_words_needed(K, N, M);
    st = check_pack_out(fn, wdt, vdt, R, K, slots, words, vals, ldv, idx, ldi);
    if (st != NM_OK) return st;
    const Range rv = span(vals, R, slots, ldv, esize(vdt)), ri = span(idx, R, words, ldi, 4);
    const Range rw = span(W, R, K, ldw, esize(wdt)), rm = span(mask, R, (K + 7) / 8, ldm, 1);
    NM_REQ(!overlap(rv, rw) && !overlap(rv, rm) && !overlap(ri, rw) && !overlap(ri, rm), NM_ERR_ALIAS,
           "%s: an output overlaps an input", fn);
    st = validate_mask(fn, flags, mask, ldm, R, K, M, N, stream);
    if (st != NM_OK) return st;
    launch_pack(W, wdt, R, K, ldw, mask, ldm, N, M, vdt, vals, ldv, idx, ldi, (hipStream_t)stream);
    return check_launch(fn);
}

nm_status nm_gate_pack(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats, int N, int M,
                       float T0, float rho, int steps, int m_step, float* m, int64_t ldf, uint8_t* hard_mask,
                       int64_t ldm, double* lmid, const void* W, nm_dtype wdt, int64_t ldw, nm_dtype vdt, void* vals,
                       int64_t ldv, uint32_t* idx, int64_t ldi, void* ws, size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_gate_pack";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    nm_status st = check_pattern(N, M, fn);
    if (st != NM_OK) return st;
    NM_REQ(K % M == 0, NM_ERR_SHAPE, "%s: K %% M != 0", fn);
    NM_REQ(steps >= 1 && steps <= 64, NM_ERR_SHAPE, "%s: steps must be in [1, 64]", fn);
    NM_REQ(!m || (m_step >= 0 && m_step < steps), NM_ERR_SHAPE, "%s: m_step must be in [0, steps)", fn);
    NM_REQ(T0 > 0.f && rho > 0.f, NM_ERR_SHAPE, "%s: T0 and rho must be positive", fn);
    NM_REQ(stats && lmid, NM_ERR_NULL, "%s: stats / lmid is NULL", fn);
    NM_REQ((S && hard_mask && W) || R * K == 0, NM_ERR_NULL, "%s: NULL pointer", fn);
    NM_REQ(lds >= K && ldm >= (K + 7) / 8 && ldw >= K && (!m || ldf >= K), NM_ERR_SHAPE,
           "%s: leading dimension too small", fn);
    const size_t need = gate_ws(R, K, steps);
    NM_REQ(ws && ws_bytes >= need, NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    const int64_t slots = K / M * N, words = idx_words_needed(K, N, M);
    if (R * K > 0) {
        st = check_pack_out(fn, wdt, vdt, R, K, slots, words, vals, ldv, idx, ldi);
        if (st != NM_OK) return st;
    }
    const Range outs[6] = {span(hard_mask, R, (K + 7) / 8, ldm, 1), span(m, R, K, ldf, 4),
                           span(lmid, 1, steps, steps, 8), span(vals, R, slots, ldv, esize(vdt)),
                           span(idx, R, words, ldi, 4), Range{(uintptr_t)ws, (uintptr_t)ws + need}};
    const Range ins[3] = {span(S, R, K, lds, 4), span(stats, 1, 2, 2, 8), span(W, R, K, ldw, esize(wdt))};
    for (const Range& x : ins)
        for (const Range& y : outs)
            NM_REQ(!overlap(x, y), NM_ERR_ALIAS, "%s: an output or the workspace overlaps an input", fn);
    for (int a = 0; a < 6; ++a)
        for (int b = a + 1; b < 6; ++b) NM_REQ(!overlap(outs[a], outs[b]), NM_ERR_ALIAS, "%s: outputs overlap", fn);
    const int ms = m ? m_step : -1;
    const bool fused = R * K > 0 && wdt == NM_BF16 && vdt == NM_BF16 &&
                       launch_gate_pack(S, R, K, lds, stats, N, M, T0, rho, steps, ms, m, ldf, hard_mask, ldm, lmid,
                                        (const uint16_t*)W, ldw, (uint16_t*)vals, ldv, idx, ldi, ws, (hipStream_t)stream);
    if (!fused) {
        // any other shape: the gate, then the pack of its hard mask on the same stream
        launch_gate(S, R, K, lds, stats, N, M, T0, rho, steps, ms, m, ldf, hard_mask, ldm, lmid, ws, (hipStream_t)stream);
        if (R * K > 0)
            launch_pack(W, wdt, R, K, ldw, hard_mask, ldm, N, M, vdt, vals, ldv, idx, ldi, (hipStream_t)stream);
    }
    return check_launch(fn);
}

nm_status nm_prune_pack(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh, float eps,
                        nm_score_mode mode, const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K, int N,
                        int M, uint8_t* mask, int64_t ldm, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx,
                        int64_t ldi, nm_stream_t stream) {
    const char* fn = "nm_prune_pack";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    nm_status st = check_pattern(N, M, fn);
    if (st != NM_OK) return st;
    NM_REQ(K % M == 0, NM_ERR_SHAPE, "%s: K %% M != 0", fn);
    if (R * K == 0) return NM_OK;
    st = check_score_src(Wsc, sdt, ldsc, H, ldh, mode, R, K, fn);
    if (st != NM_OK) return st;
    NM_REQ(Wv, NM_ERR_NULL, "%s: Wv is NULL", fn);
    NM_REQ(ldwv >= K, NM_ERR_SHAPE, "%s: ldwv < K", fn);
    NM_REQ(!mask || ldm >= (K + 7) / 8, NM_ERR_SHAPE, "%s: ldm too small", fn);
    const int64_t slots = K / M * N, words = idx_words_needed(K, N, M);
    st = check_pack_out(fn, wdt, vdt, R, K, slots, words, vals, ldv, idx, ldi);
    if (st != NM_OK) return st;
    // the fused 2:4 path reads 16-byte vectors and writes 8-byte value pairs
    if (N == 2 && M == 4 && Wsc == Wv && vdt == NM_BF16) {
        const int64_t vec = 16 / esize(wdt);
        NM_REQ(aligned16(Wv) && ldwv % vec == 0 && ((uintptr_t)vals & 7u) == 0 && ldv % 4 == 0 &&
                   (mode == NM_SCORE_MAGNITUDE || (aligned16(H) && ldh % 4 == 0)),
               NM_ERR_ALIGN, "%s: fused 2:4 path needs 16-byte aligned W (ld %% %lld), H (ldh %% 4) and vals (ldv %% 4)",
               fn, (long long)vec);
    }
    const Range rv = span(vals, R, slots, ldv, esize(vdt)), ri = span(idx, R, words, ldi, 4);
    const Range rm = span(mask, R, (K + 7) / 8, ldm, 1);
    const Range in[3] = {span(Wsc, R, K, ldsc, esize(sdt)), span(Wv, R, K, ldwv, esize(wdt)),
                         mode == NM_SCORE_HESSIAN ? span(H, ldh ? R : 1, K, ldh ? ldh : K, 4) : Range{0, 0}};
    for (const Range& x : in)
        NM_REQ(!overlap(rv, x) && !overlap(ri, x) && !overlap(rm, x), NM_ERR_ALIAS, "%s: an output overlaps an input",
               fn);
    NM_REQ(!overlap(rm, rv) && !overlap(rm, ri), NM_ERR_ALIAS, "%s: mask overlaps vals/idx", fn);
    launch_prune_pack(Wsc, sdt, ldsc, H, ldh, eps, mode, Wv, wdt, ldwv, R, K, N, M, mask, ldm, vdt, vals, ldv, idx, ldi,
                      (hipStream_t)stream);
    return check_launch(fn);
}

static nm_status slide_common(const char* fn, bool select, const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H,
                              int64_t ldh, float eps, nm_score_mode mode, const void* Wv, nm_dtype wdt, int64_t ldwv,
                              int64_t R, int64_t K, int Ns, const uint8_t* mask_in, uint8_t* mask_out, int64_t ldm,
                              nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx, int64_t ldi, unsigned flags,
                              nm_stream_t stream) {
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ((flags & ~NM_FLAG_VALIDATE) == 0, NM_ERR_SHAPE, "%s: unknown flags 0x%x", fn, flags);
    NM_REQ(Ns >= 2 && Ns <= 8, NM_ERR_PATTERN, "%s: slide N must be in [2, 8] (got %d)", fn, Ns);
    NM_REQ(K % (2 * Ns) == 0, NM_ERR_SHAPE, "%s: K %% 2N != 0", fn);
    if (R * K == 0) return NM_OK;
    if (select) {
        nm_status st = check_score_src(Wsc, sdt, ldsc, H, ldh, mode, R, K, fn);
        if (st != NM_OK) return st;
        NM_REQ(!mask_out || ldm >= (K + 7) / 8, NM_ERR_SHAPE, "%s: ldm too small", fn);
    } else {
        NM_REQ(mask_in, NM_ERR_NULL, "%s: mask is NULL", fn);
        NM_REQ(ldm >= (K + 7) / 8, NM_ERR_SHAPE, "%s: ldm too small", fn);
    }
    NM_REQ(Wv, NM_ERR_NULL, "%s: W is NULL", fn);
    NM_REQ(ldwv >= K, NM_ERR_SHAPE, "%s: ldw < K", fn);
    const int64_t Kl = K / (2 * Ns) * 4 * (Ns - 1);
    const int64_t slots = Kl / 2, words = (Kl + 31) / 32;
    nm_status st = check_pack_out(fn, wdt, vdt, R, K, slots, words, vals, ldv, idx, ldi);
    if (st != NM_OK) return st;
    const Range rv = span(vals, R, slots, ldv, esize(vdt)), ri = span(idx, R, words, ldi, 4);
    const Range rm = select ? span(mask_out, R, (K + 7) / 8, ldm, 1) : Range{0, 0};
    const Range in[4] = {select ? span(Wsc, R, K, ldsc, esize(sdt)) : Range{0, 0}, span(Wv, R, K, ldwv, esize(wdt)),
                         (select && mode == NM_SCORE_HESSIAN) ? span(H, ldh ? R : 1, K, ldh ? ldh : K, 4) : Range{0, 0},
                         select ? Range{0, 0} : span(mask_in, R, (K + 7) / 8, ldm, 1)};
    for (const Range& x : in)
        NM_REQ(!overlap(rv, x) && !overlap(ri, x) && !overlap(rm, x), NM_ERR_ALIAS, "%s: an output overlaps an input",
               fn);
    NM_REQ(!overlap(rm, rv) && !overlap(rm, ri), NM_ERR_ALIAS, "%s: mask overlaps vals/idx", fn);
    if (!select) {
        st = validate_mask(fn, flags, mask_in, ldm, R, K, 2 * Ns, 2 * Ns - 2, stream);
        if (st != NM_OK) return st;
    }
    launch_slide(Wsc, sdt, ldsc, H, ldh, eps, mode, select, Wv, wdt, ldwv, R, K, Ns, mask_in, mask_out, ldm, vdt, vals,
                 ldv, idx, ldi, (hipStream_t)stream);
    return check_launch(fn);
}

nm_status nm_slide_decompose(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask,
                             int64_t ldm, int Ns, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx, int64_t ldi,
                             unsigned flags, nm_stream_t stream) {
    return slide_common("nm_slide_decompose", false, nullptr, NM_F32, 0, nullptr, 0, 0.f, NM_SCORE_MAGNITUDE, W, wdt,
                        ldw, R, K, Ns, mask, nullptr, ldm, vdt, vals, ldv, idx, ldi, flags, stream);
}

nm_status nm_prune_slide(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh, float eps,
                         nm_score_mode mode, const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K, int Ns,
                         uint8_t* mask, int64_t ldm, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx,
                         int64_t ldi, nm_stream_t stream) {
    return slide_common("nm_prune_slide", true, Wsc, sdt, ldsc, H, ldh, eps, mode, Wv, wdt, ldwv, R, K, Ns, nullptr,
                        mask, ldm, vdt, vals, ldv, idx, ldi, 0u, stream);
}

nm_status nm_absmean(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, float* alpha, void* ws,
                     size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_absmean";
    NM_REQ(R >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(alpha, NM_ERR_NULL, "%s: alpha is NULL", fn);
    NM_REQ(W || R * K == 0, NM_ERR_NULL, "%s: W is NULL", fn);
    NM_REQ(dtype_ok(wdt) && wdt != NM_FP8, NM_ERR_DTYPE, "%s: W must be f32, bf16, int8 or int32", fn);
    NM_REQ(ldw >= K, NM_ERR_SHAPE, "%s: ldw < K", fn);
    const size_t need = reduce_ws(R, K);
    NM_REQ(ws && ws_bytes >= need, NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    NM_REQ(!overlap(span(alpha, 1, 1, 1, 4), span(W, R, K, ldw, esize(wdt))), NM_ERR_ALIAS, "%s: alpha overlaps W",
           fn);
    launch_absmean(W, wdt, R, K, ldw, alpha, ws, (hipStream_t)stream);
    return check_launch(fn);
}

nm_status nm_quant_lift(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx, int Ns, nm_dtype qdt,
                        void* Xq, int64_t ldq, float* x_scale, nm_stream_t stream) {
    const char* fn = "nm_quant_lift";
    NM_REQ(Mtok >= 0 && K >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(Ns == 0 || (Ns >= 3 && Ns <= 8), NM_ERR_PATTERN,
           "%s: supported: no lift (Ns=0) and the (2N-2):2N lift (3 <= Ns <= 8), got Ns=%d", fn, Ns);
    NM_REQ(xdt == NM_BF16 && (qdt == NM_I8 || qdt == NM_FP8), NM_ERR_DTYPE, "%s: X must be bf16, codes I8 or FP8",
           fn);
    NM_REQ(K % 8 == 0 && (Ns == 0 || K % (2 * Ns) == 0), NM_ERR_SHAPE, "%s: K must be a multiple of 8 and of 2N", fn);
    if (Mtok == 0 || K == 0) return NM_OK;
    NM_REQ(X && Xq && x_scale, NM_ERR_NULL, "%s: NULL argument", fn);
    const int64_t Kl = Ns ? K / (2 * Ns) * 4 * (Ns - 1) : K;
    NM_REQ(ldx >= K && ldq >= Kl, NM_ERR_SHAPE, "%s: leading dimension too small", fn);
    NM_REQ(aligned16(X) && (ldx * 2) % 16 == 0 && ((uintptr_t)Xq & (Ns ? 3u : 7u)) == 0 && ldq % (Ns ? 4 : 8) == 0,
           NM_ERR_ALIGN, "%s: X needs 16-byte aligned rows, Xq 4-byte (lifted) or 8-byte aligned rows", fn);
    const Range rx = span(X, Mtok, K, ldx, 2), rq = span(Xq, Mtok, Kl, ldq, 1), rs = span(x_scale, 1, Mtok, Mtok, 4);
    NM_REQ(!overlap(rq, rx) && !overlap(rs, rx) && !overlap(rq, rs), NM_ERR_ALIAS, "%s: outputs overlap", fn);
    launch_quant_lift(X, Mtok, K, ldx, Ns, qdt, Xq, ldq, x_scale, (hipStream_t)stream);
    return check_launch(fn);
}

size_t nm_spmm_workspace(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt) {
    if (Mtok <= 0 || K <= 0 || R <= 0) return 0;
    return spmm_ws(Mtok, K, R, Ns, xdt);
}

}  // extern "C"

// Argument checks of nm_spmm and nm_spmm_noalloc (everything but the workspace).  *run is
// false when there is nothing to compute.
static nm_status spmm_check(const char* fn, const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx,
                            const void* vals, nm_dtype vdt, const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi,
                            int Ns, const float* x_scale, void* Y, nm_dtype ydt, int64_t ldy, bool* run) {
    *run = false;
    NM_REQ(Mtok >= 0 && K >= 0 && R >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(Ns == 0 || (Ns >= 3 && Ns <= 8), NM_ERR_PATTERN,
           "%s: supported patterns are plain 2:4 (Ns=0) and (2N-2):2N via slide (3 <= Ns <= 8), got Ns=%d", fn, Ns);
    NM_REQ((xdt == NM_BF16 && vdt == NM_BF16 && (ydt == NM_BF16 || ydt == NM_F32)) ||
               (xdt == NM_I8 && vdt == NM_I8 && (ydt == NM_I32 || ydt == NM_F32 || ydt == NM_BF16)) ||
               (xdt == NM_FP8 && vdt == NM_FP8 && (ydt == NM_F32 || ydt == NM_BF16)),
           NM_ERR_DTYPE, "%s: supported: bf16 x bf16 -> bf16/f32, int8 x int8 -> int32/f32/bf16, fp8 x fp8 -> f32/bf16",
           fn);
    // the 2:4 product runs over the lifted width K' = (2 - 2/N) K: K' a multiple of one sparse
    // instruction's half depth (16 bf16, 32 one-byte columns)
    const int64_t kmult = xdt == NM_BF16 ? 16 : 32;
    NM_REQ(Ns == 0 || K % (2 * Ns) == 0, NM_ERR_SHAPE, "%s: K must be a multiple of 2N = %d", fn, 2 * Ns);
    const int64_t Kl = Ns ? K / (2 * Ns) * 4 * (Ns - 1) : K;
    NM_REQ(Kl % kmult == 0, NM_ERR_SHAPE, "%s: the (lifted) width %lld must be a multiple of %lld for this dtype", fn,
           (long long)Kl, (long long)kmult);
    if (xdt == NM_I8) NM_REQ(Kl * 127 * 127 < (1LL << 31), NM_ERR_SHAPE, "%s: int8 sum may overflow int32", fn);
    if (Mtok == 0 || R == 0) return NM_OK;
    NM_REQ(Y, NM_ERR_NULL, "%s: Y is NULL", fn);
    NM_REQ(ldy >= R, NM_ERR_SHAPE, "%s: ldy < R", fn);
    if (K == 0) return set_error(NM_ERR_SHAPE, "%s: K == 0", fn);
    NM_REQ(X && vals && idx, NM_ERR_NULL, "%s: NULL input", fn);
    const int64_t es = esize(xdt);
    const int64_t iw = (Kl + 31) / 32;   // index words per row
    NM_REQ(ldx >= K && ldv >= Kl / 2 && ldi >= iw, NM_ERR_SHAPE, "%s: leading dimension too small", fn);
    NM_REQ(aligned16(X) && aligned16(vals) && (ldx * es) % 16 == 0 && (ldv * es) % 16 == 0, NM_ERR_ALIGN,
           "%s: X and vals must be 16-byte aligned with 16-byte row strides", fn);
    NM_REQ(((uintptr_t)idx & 3u) == 0, NM_ERR_ALIGN, "%s: idx must be 4-byte aligned", fn);
    const Range ry = span(Y, Mtok, R, ldy, esize(ydt));
    NM_REQ(!overlap(ry, span(X, Mtok, K, ldx, es)) && !overlap(ry, span(vals, R, Kl / 2, ldv, es)) &&
               !overlap(ry, span(idx, R, iw, ldi, 4)) && !overlap(ry, span(x_scale, 1, Mtok, Mtok, 4)),
           NM_ERR_ALIAS, "%s: Y overlaps an input", fn);
    *run = true;
    return NM_OK;
}

// ------------------------------------------------------------------ the product's own scratch
// The workspace of nm_spmm_noalloc: a static device array of NM_SPMM_SCRATCH_BYTES, one copy per
// GPU, held until the process ends.  In host code `g_spmm_scratch` names a host-side stand-in;
// its device address on a GPU comes from hipGetSymbolAddress with that GPU current, looked up
// once per device and kept in g_scratch_dev[] -- only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t g_spmm_scratch[NM_SPMM_SCRATCH_BYTES];

static nm_status scratch_for(nm_stream_t stream, void** out) {
    constexpr int kMaxDev = 64;
    static void* dev_ptr[kMaxDev] = {};
    static std::mutex mu;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_error(NM_ERR_DEVICE, "nm_spmm_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    NM_REQ(dev >= 0 && dev < kMaxDev, NM_ERR_DEVICE, "nm_spmm_noalloc: device %d out of range", dev);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice((hipStream_t)stream, &sdev);
        if (e != hipSuccess)
            return set_error(NM_ERR_DEVICE, "nm_spmm_noalloc: hipStreamGetDevice: %s", hipGetErrorString(e));
        NM_REQ(sdev == dev, NM_ERR_DEVICE, "nm_spmm_noalloc: the stream belongs to device %d, the current device is %d",
               (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_spmm_scratch));
        if (e != hipSuccess || !p)
            return set_error(NM_ERR_DEVICE, "nm_spmm_noalloc: hipGetSymbolAddress of the scratch buffer: %s",
                             hipGetErrorString(e));
        dev_ptr[dev] = p;
    }
    *out = dev_ptr[dev];
    return NM_OK;
}

extern "C" {

nm_status nm_spmm(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx, const void* vals, nm_dtype vdt,
                  const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi, int Ns, const float* x_scale,
                  float w_scale, void* Y, nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_spmm";
    bool run = false;
    nm_status st = spmm_check(fn, X, xdt, Mtok, K, ldx, vals, vdt, idx, R, ldv, ldi, Ns, x_scale, Y, ydt, ldy, &run);
    if (st != NM_OK || !run) return st;
    const Range ry = span(Y, Mtok, R, ldy, esize(ydt));
    const size_t need = spmm_ws(Mtok, K, R, Ns, xdt);
    NM_REQ(need == 0 || (ws && ws_bytes >= need), NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    NM_REQ(need == 0 || aligned16(ws), NM_ERR_ALIGN, "%s: ws must be 16-byte aligned", fn);
    if (need) NM_REQ(!overlap(ry, Range{(uintptr_t)ws, (uintptr_t)ws + need}), NM_ERR_ALIAS, "%s: Y overlaps ws", fn);
    return launch_spmm(X, xdt, Mtok, K, ldx, vals, idx, R, ldv, ldi, Ns, x_scale, w_scale, Y, ydt, ldy, ws, ws_bytes,
                       (hipStream_t)stream);
}

nm_status nm_spmm_noalloc(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx, const void* vals,
                          nm_dtype vdt, const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi, int Ns,
                          const float* x_scale, float w_scale, void* Y, nm_dtype ydt, int64_t ldy,
                          nm_stream_t stream) {
    const char* fn = "nm_spmm_noalloc";
    bool run = false;
    nm_status st = spmm_check(fn, X, xdt, Mtok, K, ldx, vals, vdt, idx, R, ldv, ldi, Ns, x_scale, Y, ydt, ldy, &run);
    if (st != NM_OK || !run) return st;
    const size_t need = spmm_ws(Mtok, K, R, Ns, xdt);
    NM_REQ(need <= NM_SPMM_SCRATCH_BYTES, NM_ERR_WORKSPACE,
           "%s: this product needs %zu bytes of workspace, more than the %zu-byte scratch buffer; use nm_spmm", fn,
           need, (size_t)NM_SPMM_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need) {
        st = scratch_for(stream, &ws);
        if (st != NM_OK) return st;
    }
    return launch_spmm(X, xdt, Mtok, K, ldx, vals, idx, R, ldv, ldi, Ns, x_scale, w_scale, Y, ydt, ldy, ws, need,
                       (hipStream_t)stream);
}

nm_status nm_bitmap_encode(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask,
                           int64_t ldm, void* vals, int64_t ldv, int32_t* offs, int64_t ldo, nm_stream_t stream) {
    const char* fn = "nm_bitmap_encode";
    NM_REQ(R >= 0 && K >= 0 && ldv >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(wdt == NM_BF16, NM_ERR_DTYPE, "%s: W must be bf16", fn);
    NM_REQ(K % 64 == 0, NM_ERR_SHAPE, "%s: K must be a multiple of 64", fn);
    if (R == 0) return NM_OK;
    NM_REQ(W && mask && offs && (vals || ldv == 0), NM_ERR_NULL, "%s: NULL argument", fn);
    NM_REQ(ldw >= K && ldm >= K / 8 && ldo >= K / 64 + 1, NM_ERR_SHAPE, "%s: leading dimension too small", fn);
    NM_REQ(aligned16(W) && ldw % 8 == 0 && ((uintptr_t)mask & 7u) == 0 && ldm % 8 == 0 && ((uintptr_t)offs & 3u) == 0 &&
               ((uintptr_t)vals & 1u) == 0,
           NM_ERR_ALIGN, "%s: W needs 16-byte aligned rows, mask 8-byte aligned rows", fn);
    const Range rv = span(vals, R, ldv, ldv, 2), ro = span(offs, R, K / 64 + 1, ldo, 4);
    NM_REQ(!overlap(rv, ro) && !overlap(rv, span(W, R, K, ldw, 2)) && !overlap(ro, span(W, R, K, ldw, 2)) &&
               !overlap(rv, span(mask, R, K / 8, ldm, 1)) && !overlap(ro, span(mask, R, K / 8, ldm, 1)),
           NM_ERR_ALIAS, "%s: an output overlaps an input or the other output", fn);
    launch_bitmap_encode(W, R, K, ldw, mask, ldm, vals, ldv, offs, ldo, (hipStream_t)stream);
    return check_launch(fn);
}

size_t nm_spmm_bitmap_workspace(int64_t Mtok, int64_t K, int64_t R) { return bitmap_spmm_ws(Mtok, K, R); }

nm_status nm_spmm_bitmap(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals, int64_t ldv,
                         const uint8_t* mask, int64_t ldm, const int32_t* offs, int64_t ldo, int64_t R, void* Y,
                         nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, nm_stream_t stream) {
    const char* fn = "nm_spmm_bitmap";
    NM_REQ(Mtok >= 0 && K >= 0 && R >= 0 && ldv >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(ydt == NM_BF16 || ydt == NM_F32, NM_ERR_DTYPE, "%s: Y must be bf16 or f32", fn);
    NM_REQ(K % 64 == 0, NM_ERR_SHAPE, "%s: K must be a multiple of 64", fn);
    if (Mtok == 0 || R == 0) return NM_OK;
    NM_REQ(K > 0, NM_ERR_SHAPE, "%s: K == 0", fn);
    NM_REQ(X && mask && offs && Y && vals, NM_ERR_NULL, "%s: NULL argument", fn);
    NM_REQ(ldx >= K && ldm >= K / 8 && ldo >= K / 64 + 1 && ldy >= R && ldv >= 8, NM_ERR_SHAPE,
           "%s: leading dimension too small (ldv >= 8)", fn);
    NM_REQ(aligned16(X) && ldx % 8 == 0 && ((uintptr_t)mask & 7u) == 0 && ldm % 8 == 0 && ((uintptr_t)offs & 3u) == 0 &&
               aligned16(vals) && ldv % 8 == 0,
           NM_ERR_ALIGN, "%s: X and vals need 16-byte aligned rows, mask 8-byte aligned rows", fn);
    const Range ry = span(Y, Mtok, R, ldy, esize(ydt));
    NM_REQ(!overlap(ry, span(X, Mtok, K, ldx, 2)) && !overlap(ry, span(vals, R, ldv, ldv, 2)) &&
               !overlap(ry, span(mask, R, K / 8, ldm, 1)) && !overlap(ry, span(offs, R, K / 64 + 1, ldo, 4)),
           NM_ERR_ALIAS, "%s: Y overlaps an input", fn);
    const size_t need = bitmap_spmm_ws(Mtok, K, R);
    NM_REQ(need == 0 || (ws && ws_bytes >= need), NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    if (need) NM_REQ(!overlap(ry, Range{(uintptr_t)ws, (uintptr_t)ws + need}), NM_ERR_ALIAS, "%s: Y overlaps ws", fn);
    return launch_bitmap_spmm(X, Mtok, K, ldx, vals, ldv, mask, ldm, offs, ldo, R, Y, ydt, ldy, ws, ws_bytes,
                              (hipStream_t)stream);
}

size_t nm_spmm_lowrank_workspace(int64_t Mtok, int64_t K, int64_t R, int Ns, int rank) {
    if (Mtok <= 0 || K <= 0 || R <= 0 || rank <= 0) return 0;
    return spmm_lowrank_ws(Mtok, K, R, Ns, rank);
}

nm_status nm_spmm_lowrank(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals, const uint32_t* idx,
                          int64_t R, int64_t ldv, int64_t ldi, int Ns, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int rank, void* Y, nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes,
                          nm_stream_t stream) {
    const char* fn = "nm_spmm_lowrank";
    NM_REQ(Mtok >= 0 && K >= 0 && R >= 0, NM_ERR_SHAPE, "%s: negative size", fn);
    NM_REQ(Ns == 0 || (Ns >= 3 && Ns <= 8), NM_ERR_PATTERN,
           "%s: supported patterns are plain 2:4 (Ns=0) and (2N-2):2N via slide (3 <= Ns <= 8), got Ns=%d", fn, Ns);
    NM_REQ(ydt == NM_BF16 || ydt == NM_F32, NM_ERR_DTYPE, "%s: Y must be bf16 or f32", fn);
    NM_REQ(rank >= 8 && rank <= 256 && rank % 8 == 0, NM_ERR_SHAPE, "%s: rank must be a multiple of 8 in [8, 256]", fn);
    NM_REQ(K % 16 == 0 && (Ns == 0 || K % (2 * Ns) == 0), NM_ERR_SHAPE, "%s: K must be a multiple of 16 and of 2N", fn);
    NM_REQ((Ns ? K / (2 * Ns) * 4 * (Ns - 1) : K) % 16 == 0, NM_ERR_SHAPE,
           "%s: the lifted width must be a multiple of 16", fn);
    if (Mtok == 0 || R == 0) return NM_OK;
    NM_REQ(K > 0, NM_ERR_SHAPE, "%s: K == 0", fn);
    NM_REQ(X && vals && idx && A && B && Y, NM_ERR_NULL, "%s: NULL argument", fn);
    const int64_t Kl = Ns ? K / (2 * Ns) * 4 * (Ns - 1) : K;
    const int64_t iw = (Kl + 31) / 32;
    NM_REQ(ldx >= K && ldv >= Kl / 2 && ldi >= iw && lda >= K && ldb >= rank && ldy >= R, NM_ERR_SHAPE,
           "%s: leading dimension too small", fn);
    NM_REQ(aligned16(X) && aligned16(vals) && aligned16(A) && aligned16(B) && aligned16(idx) && ldx % 8 == 0 &&
               ldv % 8 == 0 && lda % 8 == 0 && ldb % 8 == 0 && ldi % 4 == 0,
           NM_ERR_ALIGN, "%s: X, vals, idx, A and B need 16-byte aligned bases and row strides", fn);
    const Range ry = span(Y, Mtok, R, ldy, esize(ydt));
    NM_REQ(!overlap(ry, span(X, Mtok, K, ldx, 2)) && !overlap(ry, span(vals, R, Kl / 2, ldv, 2)) &&
               !overlap(ry, span(idx, R, iw, ldi, 4)) && !overlap(ry, span(A, rank, K, lda, 2)) &&
               !overlap(ry, span(B, R, rank, ldb, 2)),
           NM_ERR_ALIAS, "%s: Y overlaps an input", fn);
    const size_t need = spmm_lowrank_ws(Mtok, K, R, Ns, rank);
    NM_REQ(ws && ws_bytes >= need, NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
    NM_REQ(aligned16(ws), NM_ERR_ALIGN, "%s: ws must be 16-byte aligned", fn);
    NM_REQ(!overlap(ry, Range{(uintptr_t)ws, (uintptr_t)ws + need}), NM_ERR_ALIAS, "%s: Y overlaps ws", fn);
    const LowRankIn lr{(const uint16_t*)A, lda, (const uint16_t*)B, ldb, rank};
    return launch_spmm_lowrank(X, Mtok, K, ldx, vals, idx, R, ldv, ldi, Ns, lr, Y, ydt, ldy, ws, ws_bytes,
                               (hipStream_t)stream);
}

}  // extern "C"
