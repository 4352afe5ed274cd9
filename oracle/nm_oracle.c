/*
 * nm_oracle.c - plain, slow, obviously-correct CPU oracle for the N:M
 * sparsification hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the GPU library is
 * checked against; it is used by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg, and by nothing else.  It shares no code,
 * header or table with the HIP library and includes none of its files.
 *
 * Style: scalar loops written straight from the definitions on the pages,
 * floating point in double unless a comment says the precision is fixed to
 * float because a float value decides an integer outcome downstream (the
 * score that the top-N selection compares).  OpenMP parallelism is used only
 * across independent weight rows (or token rows) so results never depend on
 * the thread count.  Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp.
 *
 * Sources (page title, section):
 *   [SF]  "SparseForge" technical summary: Methodology 2 (Hessian-aware
 *         importance: score (H+eps)*W^2, Hutchinson/Rademacher diagonal,
 *         standardised scores through a temperature sigmoid) and Methodology 3
 *         (progressive annealing: binary-preference term m(1-m), blend with the
 *         top-N hard target by a factor beta, geometric temperature, final
 *         projection to a hard 2:4 mask).
 *   [SI]  "Sparsity Induction" summary, section 2C (fast Hessian update with a
 *         diagonal Gauss-Newton proxy).
 *   [SB]  "Sparse-BitNet" technical summary: section 1 (N:M: at most N nonzero
 *         in every M consecutive weights; ternary {-1,0,+1}) and section 2
 *         (magnitude mask from the high-precision master weights, top-N per
 *         group; quantise then mask).
 *   [SS]  "SlideSparse" summary: section 2A (N-1 overlapping width-4 windows
 *         with stride 2 cover any (2N-2):2N block; expansion 2-2/N), 2B
 *         (activation lifting is a pure index remap, fused into the per-token
 *         quantisation) and 2C (offline packer; per request: quantise + lift,
 *         then the sparse GEMM).
 *   [SA]  "SALR" summary, Methodology 1 (magnitude pruning of the frozen base),
 *         2 (truncated-SVD adapter of the pruning residual), 3 (all low-rank
 *         adapters stacked along the rank into one product) and 4 (bitmap of the
 *         kept positions, compact values, lookup table for the decode).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_I8 2
#define OR_I32 3

#define OR_SCORE_HESSIAN 0
#define OR_SCORE_MAGNITUDE 1

/* ------------------------------------------------------------------ numerics
 * bfloat16 is the upper half of an IEEE binary32.  Widening is exact.
 * Narrowing rounds to nearest, ties to even; NaN stays NaN (quiet bit set). */
static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

static double load_as_double(const void* p, int dt, int64_t i) {
    switch (dt) {
        case OR_F32: return (double)((const float*)p)[i];
        case OR_BF16: return (double)bf16_to_f32(((const uint16_t*)p)[i]);
        case OR_I8: return (double)((const int8_t*)p)[i];
        default: return (double)((const int32_t*)p)[i];
    }
}

static float load_as_float(const void* p, int dt, int64_t i) {
    switch (dt) {
        case OR_F32: return ((const float*)p)[i];
        case OR_BF16: return bf16_to_f32(((const uint16_t*)p)[i]);
        case OR_I8: return (float)((const int8_t*)p)[i];
        default: return (float)((const int32_t*)p)[i];
    }
}

/* Copy element src[i] (dtype sdt) into dst[j] (dtype ddt).  Float -> bf16 rounds
 * to nearest even; same-dtype copies are bitwise; int8 only copies to int8. */
static void convert_store(void* dst, int ddt, int64_t j, const void* src, int sdt, int64_t i) {
    if (ddt == sdt) {
        size_t es = (ddt == OR_BF16) ? 2 : (ddt == OR_I8) ? 1 : 4;
        memcpy((char*)dst + j * es, (const char*)src + i * es, es);
        return;
    }
    float v = load_as_float(src, sdt, i);
    if (ddt == OR_BF16) ((uint16_t*)dst)[j] = f32_to_bf16(v);
    else if (ddt == OR_F32) ((float*)dst)[j] = v;
    else if (ddt == OR_I8) ((int8_t*)dst)[j] = (int8_t)v;
    else ((int32_t*)dst)[j] = (int32_t)v;
}

static void store_zero(void* dst, int ddt, int64_t j) {
    size_t es = (ddt == OR_BF16) ? 2 : (ddt == OR_I8) ? 1 : 4;
    memset((char*)dst + j * es, 0, es);
}

void or_f32_to_bf16(const float* x, int64_t n, uint16_t* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = f32_to_bf16(x[i]);
}

void or_bf16_to_f32(const uint16_t* x, int64_t n, float* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = bf16_to_f32(x[i]);
}

/* ------------------------------------------------------------------ mask bits
 * Mask layout: one bit per weight, LSB-first, row stride ldm bytes. */
static int mask_get(const uint8_t* mask, int64_t ldm, int64_t r, int64_t k) {
    return (mask[r * ldm + (k >> 3)] >> (k & 7)) & 1;
}

static void mask_set(uint8_t* mask, int64_t ldm, int64_t r, int64_t k) {
    mask[r * ldm + (k >> 3)] |= (uint8_t)(1u << (k & 7));
}

/* In-group index bitstream: field j of a row is b bits wide, LSB-first,
 * starting at bit j*b of that row's words (row stride ldi 32-bit words). */
static void idx_put(uint32_t* idx, int64_t ldi, int64_t r, int64_t j, int b, uint32_t v) {
    for (int t = 0; t < b; ++t) {
        int64_t bit = j * b + t;
        if ((v >> t) & 1u) idx[r * ldi + (bit >> 5)] |= 1u << (bit & 31);
    }
}

static uint32_t idx_get(const uint32_t* idx, int64_t ldi, int64_t r, int64_t j, int b) {
    uint32_t v = 0;
    for (int t = 0; t < b; ++t) {
        int64_t bit = j * b + t;
        v |= ((idx[r * ldi + (bit >> 5)] >> (bit & 31)) & 1u) << t;
    }
    return v;
}

int or_index_bits(int M) {
    int b = 0;
    while ((1 << b) < M) ++b;
    return b;
}

/* ------------------------------------------------------------------ A1
 * [SI] 2C: the diagonal Gauss-Newton proxy of a linear layer's Hessian is the
 * per-input-column sum of squared calibration activations, H_k = sum_i x_ik^2.
 * Plain definition, double accumulation. */
void or_colsumsq(const void* X, int xdt, int64_t n, int64_t K, double* H) {
    for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            double x = load_as_double(X, xdt, i * K + k);
            acc += x * x;
        }
        H[k] = acc;
    }
}

/* ------------------------------------------------------------------ A3
 * [SF] Methodology 2: s = (H + eps) * W^2 elementwise.  [SB] section 2 and [SA]
 * Methodology 1: magnitude score |W|.
 * Precision: float.  The score decides the integer top-N selection, so it is
 * computed in the precision the kernel uses, with one rounding per operation
 * in this order: t = w*w, u = h + eps, s = u*t.
 * H has row stride ldh: ldh == 0 means one [K] vector shared by every row
 * (per-input-column curvature), ldh >= K means a full [R,K] diagonal. */
void or_score(const void* W, int wdt, int64_t R, int64_t K, const float* H, int64_t ldh,
              float eps, int mode, float* S) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t k = 0; k < K; ++k) {
            float w = load_as_float(W, wdt, r * K + k);
            float s;
            if (mode == OR_SCORE_MAGNITUDE) {
                s = fabsf(w);
            } else {
                float h = H[r * ldh + k];
                volatile float t = w * w;
                volatile float u = h + eps;
                s = u * t;
            }
            S[r * K + k] = s;
        }
    }
}

/* ------------------------------------------------------------------ A7
 * [SB] sections 1-2, [SF] Methodology 3: keep the N largest scores of every M
 * consecutive weights along a row.  Ties go to the lower index; NaN ranks below
 * everything; -0 equals +0.  Element i beats j iff key_i > key_j, or the keys
 * are equal and i < j.  A position is kept iff fewer than N group members beat
 * it.  Output: mask bits (row stride ldm bytes), exactly N set per group. */
static float rank_key(float x) {
    if (isnan(x)) return -INFINITY;
    return x + 0.0f;
}

void or_topn_mask(const float* S, int64_t R, int64_t K, int64_t lds, int N, int M,
                  uint8_t* mask, int64_t ldm) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        memset(mask + r * ldm, 0, (size_t)((K + 7) / 8));
        for (int64_t g = 0; g < K / M; ++g) {
            for (int i = 0; i < M; ++i) {
                float ki = rank_key(S[r * lds + g * M + i]);
                int beaten_by = 0;
                for (int j = 0; j < M; ++j) {
                    if (j == i) continue;
                    float kj = rank_key(S[r * lds + g * M + j]);
                    if (kj > ki || (kj == ki && j < i)) ++beaten_by;
                }
                if (beaten_by < N) mask_set(mask, ldm, r, g * M + i);
            }
        }
    }
}

/* ------------------------------------------------------------------ A8
 * Pack kept values with their in-group positions.  For group g the kept
 * positions i_0 < ... < i_{N-1} (the first N set mask bits, ascending) give
 * vals[g*N + j] = W[g*M + i_j] converted to the value dtype, and index field
 * g*N + j = i_j (b = ceil(log2 M) bits).  If a group has fewer than N set bits
 * it is padded with value 0 at the smallest unused positions, so every group
 * always carries N distinct ascending positions.
 * vals row stride ldv elements, idx row stride ldi words; idx must be zeroed
 * by this function's caller contract: it is zeroed here row by row. */
void or_pack(const void* W, int wdt, int64_t R, int64_t K, int64_t ldw,
             const uint8_t* mask, int64_t ldm, int N, int M, int vdt,
             void* vals, int64_t ldv, uint32_t* idx, int64_t ldi) {
    int b = or_index_bits(M);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        memset(idx + r * ldi, 0, (size_t)ldi * 4);
        for (int64_t g = 0; g < K / M; ++g) {
            int pos[8];
            int isval[8];
            int cnt = 0;
            for (int i = 0; i < M && cnt < N; ++i)
                if (mask_get(mask, ldm, r, g * M + i)) { pos[cnt] = i; isval[cnt] = 1; ++cnt; }
            /* pad: smallest positions not already taken */
            for (int i = 0; i < M && cnt < N; ++i) {
                int taken = 0;
                for (int q = 0; q < cnt; ++q) if (pos[q] == i) taken = 1;
                if (!taken) { pos[cnt] = i; isval[cnt] = 0; ++cnt; }
            }
            /* sort ascending by position (insertion sort on <= 8 items) */
            for (int a = 1; a < N; ++a)
                for (int c = a; c > 0 && pos[c - 1] > pos[c]; --c) {
                    int tp = pos[c]; pos[c] = pos[c - 1]; pos[c - 1] = tp;
                    int tv = isval[c]; isval[c] = isval[c - 1]; isval[c - 1] = tv;
                }
            for (int j = 0; j < N; ++j) {
                int64_t slot = g * N + j;
                if (isval[j]) convert_store(vals, vdt, r * ldv + slot, W, wdt, r * ldw + g * M + pos[j]);
                else store_zero(vals, vdt, r * ldv + slot);
                idx_put(idx, ldi, r, slot, b, (uint32_t)pos[j]);
            }
        }
    }
}

/* Pattern check of a caller's mask before packing: the number of groups of G
 * consecutive mask bits of a row (G = M for N:M, 2N for the (2N-2):2N slide) that
 * hold more than cap set bits (cap = N, or 2N-2).  [SB] section 1: an N:M group
 * holds at most N nonzeros; [SS] 2A: the N-1 windows hold at most 2N-2.  The
 * packers keep only the first cap set bits of such a group. */
int64_t or_mask_overfull(const uint8_t* mask, int64_t R, int64_t K, int64_t ldm, int G, int cap) {
    int64_t bad = 0;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t g = 0; g < K / G; ++g) {
            int cnt = 0;
            for (int i = 0; i < G; ++i) cnt += mask_get(mask, ldm, r, g * G + i) ? 1 : 0;
            if (cnt > cap) ++bad;
        }
    return bad;
}

/* Inverse of or_pack: dense [R,K] in the value dtype, zeros off the kept set. */
void or_unpack(const void* vals, int vdt, int64_t ldv, const uint32_t* idx, int64_t ldi,
               int64_t R, int64_t K, int N, int M, void* Wd) {
    int b = or_index_bits(M);
    size_t es = (vdt == OR_BF16) ? 2 : (vdt == OR_I8) ? 1 : 4;
    memset(Wd, 0, (size_t)(R * K) * es);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t g = 0; g < K / M; ++g)
            for (int j = 0; j < N; ++j) {
                int64_t slot = g * N + j;
                uint32_t p = idx_get(idx, ldi, r, slot, b);
                memcpy((char*)Wd + (size_t)(r * K + g * M + p) * es,
                       (const char*)vals + (size_t)(r * ldv + slot) * es, es);
            }
}

/* ------------------------------------------------------------------ A9
 * [SS] 2A: a 2N-wide group with up to 2N-2 kept positions is covered by N-1
 * windows of width 4 and stride 2 (window w covers local positions 2w..2w+3);
 * each window is a 2:4 group in the lifted weight of width K' = (2-2/N)K.
 * Assignment (the page fixes coverage, not the assignment): kept positions are
 * visited in ascending order and each goes to the earliest covering window that
 * still has a free slot; windows left with fewer than 2 entries are padded with
 * value 0 at their smallest unused local positions; entries in a window are
 * stored in ascending local order.  Output uses the 2:4 packed layout over K':
 * vals [R, K'/2] (stride ldv) and 2-bit indices (stride ldi words).
 * Returns the number of groups whose kept positions did not fit (0 for any mask
 * with at most 2N-2 set bits per group); extra positions are dropped. */
int64_t or_slide_decompose(const void* W, int wdt, int64_t R, int64_t K, int64_t ldw,
                           const uint8_t* mask, int64_t ldm, int Ns, int vdt,
                           void* vals, int64_t ldv, uint32_t* idx, int64_t ldi) {
    int64_t G = K / (2 * Ns);
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t r = 0; r < R; ++r) {
        memset(idx + r * ldi, 0, (size_t)ldi * 4);
        for (int64_t g = 0; g < G; ++g) {
            int wpos[8][2];
            int wcnt[8];
            for (int w = 0; w < Ns - 1; ++w) wcnt[w] = 0;
            for (int p = 0; p < 2 * Ns; ++p) {
                if (!mask_get(mask, ldm, r, g * 2 * Ns + p)) continue;
                int placed = 0;
                for (int w = p / 2 - 1; w <= p / 2 && !placed; ++w) {
                    if (w < 0 || w > Ns - 2) continue;
                    if (wcnt[w] < 2) { wpos[w][wcnt[w]++] = p; placed = 1; }
                }
                if (!placed) ++bad;
            }
            for (int w = 0; w < Ns - 1; ++w) {
                int loc[2], isval[2], c = 0;
                for (int q = 0; q < wcnt[w]; ++q) { loc[c] = wpos[w][q] - 2 * w; isval[c] = 1; ++c; }
                for (int l = 0; l < 4 && c < 2; ++l) {
                    int taken = 0;
                    for (int q = 0; q < c; ++q) if (loc[q] == l) taken = 1;
                    if (!taken) { loc[c] = l; isval[c] = 0; ++c; }
                }
                if (loc[0] > loc[1]) {
                    int t = loc[0]; loc[0] = loc[1]; loc[1] = t;
                    t = isval[0]; isval[0] = isval[1]; isval[1] = t;
                }
                int64_t wg = g * (Ns - 1) + w; /* 2:4 group index in K' */
                for (int j = 0; j < 2; ++j) {
                    int64_t slot = wg * 2 + j;
                    if (isval[j]) convert_store(vals, vdt, r * ldv + slot, W, wdt, r * ldw + g * 2 * Ns + 2 * w + loc[j]);
                    else store_zero(vals, vdt, r * ldv + slot);
                    idx_put(idx, ldi, r, slot, 2, (uint32_t)loc[j]);
                }
            }
        }
    }
    return bad;
}

/* Fold a lifted 2:4 weight back onto the original K columns: original column
 * g*2N + 2w + l receives window w's entry at local position l.  Windows overlap
 * on two columns, so values are accumulated in double; with the greedy
 * assignment each original column is held by at most one window. */
void or_slide_fold(const void* vals, int vdt, int64_t ldv, const uint32_t* idx, int64_t ldi,
                   int64_t R, int64_t K, int Ns, double* Wd) {
    int64_t G = K / (2 * Ns);
    memset(Wd, 0, (size_t)(R * K) * sizeof(double));
    for (int64_t r = 0; r < R; ++r)
        for (int64_t g = 0; g < G; ++g)
            for (int w = 0; w < Ns - 1; ++w)
                for (int j = 0; j < 2; ++j) {
                    int64_t slot = (g * (Ns - 1) + w) * 2 + j;
                    uint32_t l = idx_get(idx, ldi, r, slot, 2);
                    Wd[r * K + g * 2 * Ns + 2 * w + l] += load_as_double(vals, vdt, r * ldv + slot);
                }
}

/* [SS] 2B: the lifted activation repeats the columns each window reads:
 * X_lift[m, g*4(N-1) + 4w + l] = X[m, g*2N + 2w + l], w < N-1, l < 4.
 * Pure copy (no arithmetic). */
void or_lift(const void* X, int xdt, int64_t Mt, int64_t K, int Ns, void* Xl) {
    int64_t G = K / (2 * Ns);
    int64_t Kl = G * 4 * (Ns - 1);
    size_t es = (xdt == OR_BF16) ? 2 : (xdt == OR_I8) ? 1 : 4;
    for (int64_t m = 0; m < Mt; ++m)
        for (int64_t g = 0; g < G; ++g)
            for (int w = 0; w < Ns - 1; ++w)
                for (int l = 0; l < 4; ++l)
                    memcpy((char*)Xl + (size_t)(m * Kl + g * 4 * (Ns - 1) + 4 * w + l) * es,
                           (const char*)X + (size_t)(m * K + g * 2 * Ns + 2 * w + l) * es, es);
}

/* ------------------------------------------------------------------ per-token int8 quantisation [SS 2B, 2C]
 * The online step before the int8 sparse product: each token row of X is
 * scaled by its own absolute maximum, s = max|x| / 127, and rounded to the
 * nearest integer, q = rint(x / s) (ties to even), so that x ~= s * q with
 * q in [-127, 127].  The pages name per-token INT8 quantisation and fuse the
 * lift into it without fixing the formula; this is the plain absmax reading.
 * The quotients decide integers, so they are computed in float (one rounding
 * per operation); a zero row gives s = 0 and q = 0.  Inputs are finite. */
void or_quant_i8(const uint16_t* X, int64_t Mt, int64_t K, int64_t ldx, int8_t* Xq, float* sx) {
    for (int64_t m = 0; m < Mt; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float a = fabsf(bf16_to_f32(X[m * ldx + k]));
            if (a > amax) amax = a;
        }
        const float s = amax / 127.0f;
        sx[m] = s;
        for (int64_t k = 0; k < K; ++k) {
            float q = 0.0f;
            if (s > 0.0f) {
                q = rintf(bf16_to_f32(X[m * ldx + k]) / s);
                if (q > 127.0f) q = 127.0f;
                if (q < -127.0f) q = -127.0f;
            }
            Xq[m * K + k] = (int8_t)q;
        }
    }
}

/* ------------------------------------------------------------------ FP8 e4m3 [SS 3, precisions]
 * OCP FP8 e4m3 ("fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent 0 holds the subnormals m/8 * 2^-6; code 0x7f / 0xff is NaN; no
 * infinities; the largest finite magnitude is 448.  Decoding is exact in float.
 * Encoding rounds to the nearest code, ties to the code with the even low bit
 * (round-half-even), found by brute force over the 127 finite magnitudes;
 * magnitudes past 448 saturate to 448 (a reading: the pages fix no overflow
 * rule; every value the quantisation below produces is within 448 anyway). */
static float e4m3_decode(uint8_t c) {
    const int e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexpf((float)m, -9);
    else v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return (c & 0x80) ? -v : v;
}
static uint8_t e4m3_encode(float x) {
    if (x != x) return 0x7f;
    const uint8_t sign = signbit(x) ? 0x80 : 0x00;   /* -0 keeps its sign, as in IEEE conversions */
    const float a = fabsf(x);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 127; ++c) {           /* finite non-negative codes, ascending value */
        const double d = fabs((double)a - (double)e4m3_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}
void or_e4m3_decode(const uint8_t* c, int64_t n, float* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = e4m3_decode(c[i]);
}
void or_e4m3_encode(const float* x, int64_t n, uint8_t* c) {
    for (int64_t i = 0; i < n; ++i) c[i] = e4m3_encode(x[i]);
}
/* Per-token FP8 quantisation: s = max|x| / 448, code = e4m3(x / s) in float. */
void or_quant_fp8(const uint16_t* X, int64_t Mt, int64_t K, int64_t ldx, uint8_t* Xq, float* sx) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < Mt; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float a = fabsf(bf16_to_f32(X[m * ldx + k]));
            if (a > amax) amax = a;
        }
        const float s = amax / 448.0f;
        sx[m] = s;
        for (int64_t k = 0; k < K; ++k)
            Xq[m * K + k] = s > 0.0f ? e4m3_encode(bf16_to_f32(X[m * ldx + k]) / s) : 0;
    }
}
/* Y[m,o] = sum_k x[m,k] w[o,k] over FP8 codes (mask: as or_masked_matmul), in double:
 * each product of two e4m3 values is exact. */
void or_masked_matmul_fp8(const uint8_t* X, int64_t Mt, int64_t K, const uint8_t* W, int64_t R,
                          const uint8_t* mask, int64_t ldm, double* Y) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < Mt; ++m)
        for (int64_t o = 0; o < R; ++o) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                if (mask && !mask_get(mask, ldm, o, k)) continue;
                acc += (double)e4m3_decode(X[m * K + k]) * (double)e4m3_decode(W[o * K + k]);
            }
            Y[m * R + o] = acc;
        }
}

/* ------------------------------------------------------------------ A12 / A13
 * The structured-sparse linear layer is, by definition, the dense product with
 * the masked weight: Y[m,o] = sum_k X[m,k] * (mask * W)[o,k].  Double
 * accumulation over ascending k.  The weight may be dense with a mask
 * (mask != NULL) or already masked (mask == NULL).  Rows of Y are independent. */
void or_masked_matmul(const void* X, int xdt, int64_t Mt, int64_t K, int64_t ldx,
                      const void* W, int wdt, int64_t R, int64_t ldw,
                      const uint8_t* mask, int64_t ldm, double* Y) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < Mt; ++m)
        for (int64_t o = 0; o < R; ++o) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                if (mask && !mask_get(mask, ldm, o, k)) continue;
                acc += load_as_double(X, xdt, m * ldx + k) * load_as_double(W, wdt, o * ldw + k);
            }
            Y[m * R + o] = acc;
        }
}

/* Same product for a sample of (token, output) pairs. */
void or_masked_matmul_at(const void* X, int xdt, int64_t K, int64_t ldx,
                         const void* W, int wdt, int64_t ldw, const uint8_t* mask, int64_t ldm,
                         const int64_t* rows_m, const int64_t* rows_o, int64_t npairs, double* Y) {
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < npairs; ++q) {
        int64_t m = rows_m[q], o = rows_o[q];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            if (mask && !mask_get(mask, ldm, o, k)) continue;
            acc += load_as_double(X, xdt, m * ldx + k) * load_as_double(W, wdt, o * ldw + k);
        }
        Y[q] = acc;
    }
}

/* ------------------------------------------------------------------ sparse + low-rank linear
 * [SA] section 3 (adapter concatenation): every low-rank adapter of a layer (the
 * fine-tuning adapter and the truncated-SVD adapter of the pruning residual, section 2)
 * is stacked along the rank, so the layer is one structured-sparse product plus one
 * rank-r product on the same input:
 *   Y[m,o] = sum_k X[m,k] (mask*W)[o,k]  +  sum_j u[m,j] B[o,j],
 *   u[m,j] = bf16( sum_k X[m,k] A[j,k] ),
 * with A [r, K] (the stacked down-projections) and B [R, r] (the stacked
 * up-projections).  Reading: the pages fix no precision for the adapter's
 * intermediate; it is an activation of the layer, so it is held in bf16, rounded
 * once (to nearest, ties to even) from its exact value.  Everything else is in double. */

/* Correct bf16 rounding of a double: round to float with round-to-odd (truncate toward
 * zero, then set the last bit when inexact), then to bf16 to nearest even; with 16 more
 * bits than bf16 the intermediate cannot create a false tie. */
static uint16_t bf16_of_double(double d) {
    float f = (float)d;
    if (isfinite(f) && (double)f != d) {
        if (fabs((double)f) > fabs(d)) f = nextafterf(f, 0.0f);
        uint32_t u;
        memcpy(&u, &f, 4);
        u |= 1u;
        memcpy(&f, &u, 4);
    }
    return f32_to_bf16(f);
}

/* u[m, j] = sum_k X[m,k] A[j,k] in double (exact value; the layer rounds it to bf16). */
void or_lowrank_u(const void* X, int xdt, int64_t Mt, int64_t K, const void* A, int adt, int64_t r, double* U) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < Mt; ++m)
        for (int64_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += load_as_double(X, xdt, m * K + k) * load_as_double(A, adt, j * K + k);
            U[m * r + j] = acc;
        }
}

void or_sparse_lowrank(const void* X, int xdt, int64_t Mt, int64_t K, const void* W, int wdt, int64_t R,
                       const uint8_t* mask, int64_t ldm, const void* A, int adt, const void* B, int bdt, int64_t r,
                       double* Y) {
    double* U = (double*)malloc((size_t)(Mt * r > 0 ? Mt * r : 1) * sizeof(double));
    or_lowrank_u(X, xdt, Mt, K, A, adt, r, U);
    or_masked_matmul(X, xdt, Mt, K, K, W, wdt, R, K, mask, ldm, Y);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < Mt; ++m)
        for (int64_t o = 0; o < R; ++o) {
            double acc = 0.0;
            for (int64_t j = 0; j < r; ++j)
                acc += (double)bf16_to_f32(bf16_of_double(U[m * r + j])) * load_as_double(B, bdt, o * r + j);
            Y[m * R + o] += acc;
        }
    free(U);
}

/* ------------------------------------------------------------------ bitmap format
 * [SA] section 4: the pruned weight is stored as a bitmap of its nonzero positions plus
 * a compact array of the kept values (no per-element column indices, unlike CSR), and a
 * lookup table locates the values of each sub-block for the decode.  Reading: the bitmap
 * is the 1-bit-per-weight mask (LSB-first, [R, ceil(K/8)] bytes); the values of row r
 * are stored in ascending column order at vals[r, 0 .. nnz_r) (row stride ldv); the
 * table holds, for each row r and each block b of 64 columns, offs[r, b] = the number of
 * kept values of row r before column 64 b, with offs[r, K/64] = nnz_r.  A kept value
 * whose position in its row is ldv or beyond is not stored (the caller sizes ldv to the
 * largest row count).  The product is the masked product of A12. */
void or_bitmap_encode(const void* W, int wdt, int64_t R, int64_t K, const uint8_t* mask, int64_t ldm,
                      void* vals, int vdt, int64_t ldv, int32_t* offs, int64_t ldo) {
    const int64_t nb = (K + 63) / 64;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        int64_t count = 0;
        for (int64_t b = 0; b < nb; ++b) {
            offs[r * ldo + b] = (int32_t)count;
            for (int64_t k = 64 * b; k < K && k < 64 * b + 64; ++k) {
                if (!mask_get(mask, ldm, r, k)) continue;
                if (count < ldv) convert_store(vals, vdt, r * ldv + count, W, wdt, r * K + k);
                ++count;
            }
        }
        offs[r * ldo + nb] = (int32_t)count;
    }
}

/* Dense [R, K] from the bitmap format: W[r,k] = the value of k's rank among the row's
 * kept positions where the bit is set (0 if it was not stored), else 0. */
void or_bitmap_decode(const void* vals, int vdt, int64_t ldv, const uint8_t* mask, int64_t ldm, int64_t R, int64_t K,
                      void* Wd, int wdt) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        int64_t count = 0;
        for (int64_t k = 0; k < K; ++k) {
            if (mask_get(mask, ldm, r, k) && count < ldv) convert_store(Wd, wdt, r * K + k, vals, vdt, r * ldv + count);
            else store_zero(Wd, wdt, r * K + k);
            if (mask_get(mask, ldm, r, k)) ++count;
        }
    }
}

/* Integer form for int8 activations and ternary int8 weights: the exact sum in
 * 64-bit integers, then checked to fit int32 (returns the number of outputs
 * that would overflow int32).  y = (alpha * s_x[m]) * acc in float, one
 * rounding per operation in that order (the epilogue precision is the
 * kernel's; the integer sum is exact on both sides). */
int64_t or_masked_matmul_i8(const int8_t* Xq, int64_t Mt, int64_t K, int64_t ldx,
                            const int8_t* W, int64_t R, int64_t ldw, const uint8_t* mask, int64_t ldm,
                            const float* sx, float alpha, int32_t* acc_out, float* y_out) {
    int64_t overflow = 0;
#pragma omp parallel for schedule(static) reduction(+ : overflow)
    for (int64_t m = 0; m < Mt; ++m)
        for (int64_t o = 0; o < R; ++o) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                if (mask && !mask_get(mask, ldm, o, k)) continue;
                acc += (int64_t)Xq[m * ldx + k] * (int64_t)W[o * ldw + k];
            }
            if (acc > INT32_MAX || acc < INT32_MIN) ++overflow;
            if (acc_out) acc_out[m * R + o] = (int32_t)acc;
            if (y_out) {
                volatile float sc = alpha * sx[m];
                y_out[m * R + o] = sc * (float)acc;
            }
        }
    return overflow;
}

/* ------------------------------------------------------------------ A10
 * [SB] section 2: the ternary layer's scale is the mean absolute value of the
 * high-precision master weights; its mask is the top-N by |W_fp| per group;
 * the effective weight is the ternary code with the mask applied afterwards. */
double or_absmean(const void* W, int wdt, int64_t n) {
    double acc = 0.0;
    for (int64_t i = 0; i < n; ++i) acc += fabs(load_as_double(W, wdt, i));
    return n > 0 ? acc / (double)n : 0.0;
}

void or_apply_mask_i8(const int8_t* Wt, int64_t R, int64_t K, const uint8_t* mask, int64_t ldm, int8_t* Weff) {
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k)
            Weff[r * K + k] = mask_get(mask, ldm, r, k) ? Wt[r * K + k] : (int8_t)0;
}

/* ------------------------------------------------------------------ A2
 * SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014): the state advances by the odd constant
 * 0x9E3779B97F4A7C15 and each output is the state passed through the
 * variant-13 64-bit finaliser.  The i-th output (0-based) of a generator seeded
 * with s is therefore mix(s + (i+1)*gamma), which makes it counter-based. */
uint64_t or_splitmix64_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Rademacher probe entry V_p[o,k] in {-1,+1}: bit (k mod 64) of SplitMix64
 * output number p*2^40 + o*ceil(K/64) + floor(k/64); bit 1 -> -1. */
int or_rademacher(uint64_t seed, int p, int64_t o, int64_t k, int64_t K) {
    uint64_t ctr = ((uint64_t)p << 40) + (uint64_t)o * (uint64_t)((K + 63) / 64) + (uint64_t)(k / 64);
    uint64_t word = or_splitmix64_at(seed, ctr);
    return ((word >> (k % 64)) & 1u) ? -1 : 1;
}

/* [SF] Methodology 2: Hutchinson's estimator of the Hessian diagonal with
 * Rademacher probes, diag(H) ~ (1/P) sum_p v_p * (H v_p).
 * The loss is the layer's quadratic output energy L(W) = ||X W^T||_F^2, whose
 * Hessian-vector product for a probe V (same shape as W, [R,K]) is
 * (H V)[o,:] = 2 * ((V X^T) X)[o,:].  Rows o of the estimate are independent,
 * so the oracle evaluates any requested subset of rows.
 * X is [n, K] (dtype xdt); D gets one [K] row per requested row, in double. */
void or_hutchinson_rows(const void* X, int xdt, int64_t n, int64_t K, int probes, uint64_t seed,
                        const int64_t* rows, int64_t nrows, double* D) {
#pragma omp parallel for schedule(dynamic)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t o = rows[q];
        double* v = (double*)malloc((size_t)K * sizeof(double));
        double* u = (double*)malloc((size_t)n * sizeof(double));
        double* d = D + q * K;
        for (int64_t k = 0; k < K; ++k) d[k] = 0.0;
        for (int p = 0; p < probes; ++p) {
            for (int64_t k = 0; k < K; ++k) v[k] = (double)or_rademacher(seed, p, o, k, K);
            for (int64_t i = 0; i < n; ++i) {          /* u = v X^T */
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) acc += v[k] * load_as_double(X, xdt, i * K + k);
                u[i] = acc;
            }
            for (int64_t k = 0; k < K; ++k) {          /* (H v)_k = 2 (u X)_k */
                double acc = 0.0;
                for (int64_t i = 0; i < n; ++i) acc += u[i] * load_as_double(X, xdt, i * K + k);
                d[k] += v[k] * 2.0 * acc;
            }
        }
        for (int64_t k = 0; k < K; ++k) d[k] /= (double)probes;
        free(v);
        free(u);
    }
}

/* Hutchinson's probe products U_p[o,:] = V_p[o,:] X^T for the same rows (used
 * for the error bound of a reduced-precision evaluation). */
void or_hutchinson_u_rows(const void* X, int xdt, int64_t n, int64_t K, int probes, uint64_t seed,
                          const int64_t* rows, int64_t nrows, double* U /* [nrows, probes, n] */) {
#pragma omp parallel for schedule(dynamic)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t o = rows[q];
        for (int p = 0; p < probes; ++p)
            for (int64_t i = 0; i < n; ++i) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += (double)or_rademacher(seed, p, o, k, K) * load_as_double(X, xdt, i * K + k);
                U[(q * probes + p) * n + i] = acc;
            }
    }
}

/* ------------------------------------------------------------------ A4
 * [SF] Methodology 2: scores are standardised before the sigmoid.  Per-tensor
 * mean and population standard deviation, two passes in double. */
void or_stats(const float* S, int64_t count, double* mu, double* sigma) {
    double acc = 0.0;
    for (int64_t i = 0; i < count; ++i) acc += (double)S[i];
    double m = count > 0 ? acc / (double)count : 0.0;
    double v = 0.0;
    for (int64_t i = 0; i < count; ++i) {
        double d = (double)S[i] - m;
        v += d * d;
    }
    *mu = m;
    *sigma = count > 0 ? sqrt(v / (double)count) : 0.0;
}

/* ------------------------------------------------------------------ A5 / A6
 * [SF] Methodology 2 and 3.  For annealing step t = 0..S-1:
 *   T_t    = T0 * rho^t                       (geometric temperature)
 *   beta_t = t / (S-1)                         (blend factor, 0 -> 1)
 *   g_t    = 1 / (1 + exp(-z / T_t)),  z = (s - mu) / sigma   (sigma = 0 -> z = 0)
 *   h      = top-N of s per group (the hard target)
 *   m_t    = (1 - beta_t) g_t + beta_t h
 *   Lmid_t = sum m_t (1 - m_t)                 (binary-preference term)
 * The final projection keeps the top-N of m_{S-1} per group.
 * Outputs: m_t of step t = m_step as float [R,K] (m_out may be NULL), the hard
 * mask bits, and Lmid [S] in double.  All arithmetic in double. */
void or_gate_anneal(const float* S, int64_t R, int64_t K, double mu, double sigma,
                    int N, int M, double T0, double rho, int steps, int m_step,
                    float* m_out, uint8_t* hard_mask, int64_t ldm, double* lmid) {
    uint8_t* h = (uint8_t*)calloc((size_t)(R * ((K + 7) / 8)), 1);
    int64_t ldh = (K + 7) / 8;
    or_topn_mask(S, R, K, K, N, M, h, ldh);
    float* mlast = (float*)malloc((size_t)(R * K) * sizeof(float));
    double* rowsum = (double*)malloc((size_t)(R > 0 ? R : 1) * sizeof(double));
    for (int t = 0; t < steps; ++t) {
        double T = T0 * pow(rho, (double)t);
        double beta = steps > 1 ? (double)t / (double)(steps - 1) : 1.0;
        /* rows in parallel, each row's sum in column order, the row sums in row order */
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < R; ++r) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double z = sigma > 0.0 ? ((double)S[r * K + k] - mu) / sigma : 0.0;
                double g = 1.0 / (1.0 + exp(-z / T));
                double hv = mask_get(h, ldh, r, k) ? 1.0 : 0.0;
                double m = (1.0 - beta) * g + beta * hv;
                acc += m * (1.0 - m);
                if (t == steps - 1) mlast[r * K + k] = (float)m;
                if (m_out && t == m_step) m_out[r * K + k] = (float)m;
            }
            rowsum[r] = acc;
        }
        double acc = 0.0;
        for (int64_t r = 0; r < R; ++r) acc += rowsum[r];
        lmid[t] = acc;
    }
    free(rowsum);
    or_topn_mask(mlast, R, K, K, N, M, hard_mask, ldm);
    free(mlast);
    free(h);
}

/* Number of threads the parallel loops above use. */
int or_num_threads(void) { return omp_get_max_threads(); }

/* Sets the thread count of the parallel loops (results do not depend on it). */
void or_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

/* Gate value for a single element at step t (for sampled checks). */
double or_gate_value(float s, double mu, double sigma, double T0, double rho, int t) {
    double T = T0 * pow(rho, (double)t);
    double z = sigma > 0.0 ? ((double)s - mu) / sigma : 0.0;
    return 1.0 / (1.0 + exp(-z / T));
}
