/*
 * sanitize_check.c - drives every routine of the oracle (nm_oracle.c, compiled into this
 * program) once over small ragged shapes, with each buffer allocated at exactly the size
 * its caller contract gives, so that an AddressSanitizer / UndefinedBehaviorSanitizer
 * build reports any read or write past a buffer, any use of freed memory and any
 * undefined arithmetic.  It also checks the round trips that need no second
 * implementation: pack then unpack, slide decomposition then fold, bitmap encode then
 * decode, each against the masked weight.
 *
 * TEST INFRASTRUCTURE ONLY (part of the oracle).  Build and run (the test suite does):
 *   gcc -std=c11 -O1 -g -fopenmp -fsanitize=address,undefined -fno-sanitize-recover=all \
 *       -fno-omit-frame-pointer oracle/sanitize_check.c -o sanitize_check -lm && ./sanitize_check
 * Exit status 0 and the line "oracle sanitize check ok" mean every routine ran clean.
 */
#include "nm_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t rnd(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}
static float rndf(void) { return (float)((double)(rnd() >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0); }

/* exactly n bytes (at least one), filled with random bytes */
static void* xalloc(size_t n) {
    uint8_t* p = (uint8_t*)malloc(n ? n : 1);
    if (!p) abort();
    for (size_t i = 0; i < n; ++i) p[i] = (uint8_t)rnd();
    return p;
}

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static uint16_t* rand_bf16(int64_t n) {
    float* f = (float*)xalloc((size_t)n * 4);
    for (int64_t i = 0; i < n; ++i) f[i] = rndf();
    uint16_t* b = (uint16_t*)xalloc((size_t)n * 2);
    or_f32_to_bf16(f, n, b);
    free(f);
    return b;
}

static int64_t mask_ld(int64_t K) { return (K + 7) / 8; }

/* masked bf16 weight as doubles (0 where the mask bit is clear) */
static double masked_value(const uint16_t* W, const uint8_t* mask, int64_t ldm, int64_t K, int64_t r, int64_t k) {
    return mask_get(mask, ldm, r, k) ? (double)bf16_to_f32(W[r * K + k]) : 0.0;
}

static void check_numerics(void) {
    const int64_t n = 37;
    float* f = (float*)xalloc(n * 4);
    for (int64_t i = 0; i < n; ++i) f[i] = rndf() * 300.0f;
    uint16_t* b = (uint16_t*)xalloc(n * 2);
    float* g = (float*)xalloc(n * 4);
    or_f32_to_bf16(f, n, b);
    or_bf16_to_f32(b, n, g);
    uint8_t* c = (uint8_t*)xalloc(n);
    or_e4m3_encode(f, n, c);
    or_e4m3_decode(c, n, g);
    CHECK(or_index_bits(4) == 2 && or_index_bits(8) == 3);
    CHECK(or_splitmix64_at(0, 0) != or_splitmix64_at(0, 1));
    int r = or_rademacher(7, 1, 3, 5, 64);
    CHECK(r == 1 || r == -1);
    free(f), free(b), free(g), free(c);
}

static void check_prune_pack(int64_t R, int64_t K, int N, int M) {
    uint16_t* W = rand_bf16(R * K);
    const int64_t n = 5;
    uint16_t* X = rand_bf16(n * K);
    double* Hd = (double*)xalloc((size_t)K * 8);
    or_colsumsq(X, OR_BF16, n, K, Hd);
    float* H = (float*)xalloc((size_t)K * 4);
    for (int64_t k = 0; k < K; ++k) H[k] = (float)Hd[k];
    float* Hw = (float*)xalloc((size_t)(R * K) * 4);
    for (int64_t i = 0; i < R * K; ++i) Hw[i] = rndf() + 1.5f;
    float* S = (float*)xalloc((size_t)(R * K) * 4);
    or_score(W, OR_BF16, R, K, Hw, K, 1e-6f, OR_SCORE_HESSIAN, S);
    or_score(W, OR_BF16, R, K, H, 0, 0.0f, OR_SCORE_MAGNITUDE, S);
    or_score(W, OR_BF16, R, K, H, 0, 1e-6f, OR_SCORE_HESSIAN, S);
    const int64_t ldm = mask_ld(K);
    uint8_t* mask = (uint8_t*)xalloc((size_t)(R * ldm));
    memset(mask, 0, (size_t)(R * ldm));
    or_topn_mask(S, R, K, K, N, M, mask, ldm);
    CHECK(or_mask_overfull(mask, R, K, ldm, M, N) == 0);
    const int64_t slots = K / M * N, words = (slots * or_index_bits(M) + 31) / 32;
    uint16_t* vals = (uint16_t*)xalloc((size_t)(R * slots) * 2);
    uint32_t* idx = (uint32_t*)xalloc((size_t)(R * words) * 4);
    memset(idx, 0, (size_t)(R * words) * 4);
    or_pack(W, OR_BF16, R, K, K, mask, ldm, N, M, OR_BF16, vals, slots, idx, words);
    uint16_t* Wd = (uint16_t*)xalloc((size_t)(R * K) * 2);
    or_unpack(vals, OR_BF16, slots, idx, words, R, K, N, M, Wd);
    /* groups of M: the unpacked weight is the masked one (whole groups only) */
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K / M * M; ++k)
            CHECK((double)bf16_to_f32(Wd[r * K + k]) == masked_value(W, mask, ldm, K, r, k));
    free(W), free(X), free(Hd), free(H), free(Hw), free(S), free(mask), free(vals), free(idx), free(Wd);
}

static void check_slide(int64_t R, int Ns) {
    const int64_t K = 2 * Ns * 5, Kl = K / (2 * Ns) * 4 * (Ns - 1), ldm = mask_ld(K);
    uint16_t* W = rand_bf16(R * K);
    float* S = (float*)xalloc((size_t)(R * K) * 4);
    or_score(W, OR_BF16, R, K, NULL, 0, 0.0f, OR_SCORE_MAGNITUDE, S);
    uint8_t* mask = (uint8_t*)xalloc((size_t)(R * ldm));
    memset(mask, 0, (size_t)(R * ldm));
    or_topn_mask(S, R, K, K, 2 * Ns - 2, 2 * Ns, mask, ldm);
    const int64_t slots = Kl / 2, words = (slots * 2 + 31) / 32;
    uint16_t* vals = (uint16_t*)xalloc((size_t)(R * slots) * 2);
    uint32_t* idx = (uint32_t*)xalloc((size_t)(R * words) * 4);
    memset(idx, 0, (size_t)(R * words) * 4);
    CHECK(or_slide_decompose(W, OR_BF16, R, K, K, mask, ldm, Ns, OR_BF16, vals, slots, idx, words) == 0);
    double* Wd = (double*)xalloc((size_t)(R * K) * 8);
    or_slide_fold(vals, OR_BF16, slots, idx, words, R, K, Ns, Wd);
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < K; ++k) CHECK(Wd[r * K + k] == masked_value(W, mask, ldm, K, r, k));
    const int64_t Mt = 3;
    uint16_t* X = rand_bf16(Mt * K);
    uint16_t* Xl = (uint16_t*)xalloc((size_t)(Mt * Kl) * 2);
    or_lift(X, OR_BF16, Mt, K, Ns, Xl);
    /* the 2:4 product over the lifted activation equals the masked product over X */
    double* Y = (double*)xalloc((size_t)(Mt * R) * 8);
    double* Yl = (double*)xalloc((size_t)(Mt * R) * 8);
    or_masked_matmul(X, OR_BF16, Mt, K, K, W, OR_BF16, R, K, mask, ldm, Y);
    uint16_t* Wl = (uint16_t*)xalloc((size_t)(R * Kl) * 2);
    or_unpack(vals, OR_BF16, slots, idx, words, R, Kl, 2, 4, Wl);
    or_masked_matmul(Xl, OR_BF16, Mt, Kl, Kl, Wl, OR_BF16, R, Kl, NULL, 0, Yl);
    for (int64_t i = 0; i < Mt * R; ++i) CHECK(fabs(Y[i] - Yl[i]) <= 1e-9 * (1.0 + fabs(Y[i])));
    free(W), free(S), free(mask), free(vals), free(idx), free(Wd), free(X), free(Xl), free(Y), free(Yl), free(Wl);
}

static void check_products(void) {
    const int64_t Mt = 4, R = 7, K = 40, ldm = mask_ld(K), r = 8;
    uint16_t* X = rand_bf16(Mt * K);
    uint16_t* W = rand_bf16(R * K);
    float* S = (float*)xalloc((size_t)(R * K) * 4);
    or_score(W, OR_BF16, R, K, NULL, 0, 0.0f, OR_SCORE_MAGNITUDE, S);
    uint8_t* mask = (uint8_t*)xalloc((size_t)(R * ldm));
    memset(mask, 0, (size_t)(R * ldm));
    or_topn_mask(S, R, K, K, 2, 4, mask, ldm);
    double* Y = (double*)xalloc((size_t)(Mt * R) * 8);
    or_masked_matmul(X, OR_BF16, Mt, K, K, W, OR_BF16, R, K, mask, ldm, Y);
    or_masked_matmul(X, OR_BF16, Mt, K, K, W, OR_BF16, R, K, NULL, 0, Y);
    const int64_t np = 5;
    int64_t* rm = (int64_t*)xalloc(np * 8);
    int64_t* ro = (int64_t*)xalloc(np * 8);
    for (int64_t i = 0; i < np; ++i) rm[i] = (int64_t)(rnd() % Mt), ro[i] = (int64_t)(rnd() % R);
    double* Yat = (double*)xalloc(np * 8);
    or_masked_matmul_at(X, OR_BF16, K, K, W, OR_BF16, K, mask, ldm, rm, ro, np, Yat);
    uint16_t* A = rand_bf16(r * K);
    uint16_t* B = rand_bf16(R * r);
    double* U = (double*)xalloc((size_t)(Mt * r) * 8);
    or_lowrank_u(X, OR_BF16, Mt, K, A, OR_BF16, r, U);
    or_sparse_lowrank(X, OR_BF16, Mt, K, W, OR_BF16, R, mask, ldm, A, OR_BF16, B, OR_BF16, r, Y);
    /* int8 and FP8 */
    int8_t* Xq = (int8_t*)xalloc((size_t)(Mt * K));
    float* sx = (float*)xalloc((size_t)Mt * 4);
    or_quant_i8(X, Mt, K, K, Xq, sx);
    int8_t* Wt = (int8_t*)xalloc((size_t)(R * K));
    for (int64_t i = 0; i < R * K; ++i) Wt[i] = (int8_t)((int)(rnd() % 3) - 1);
    int8_t* Weff = (int8_t*)xalloc((size_t)(R * K));
    or_apply_mask_i8(Wt, R, K, mask, ldm, Weff);
    int32_t* acc = (int32_t*)xalloc((size_t)(Mt * R) * 4);
    float* y = (float*)xalloc((size_t)(Mt * R) * 4);
    CHECK(or_masked_matmul_i8(Xq, Mt, K, K, Wt, R, K, mask, ldm, sx, 0.5f, acc, y) == 0);
    uint8_t* Xf = (uint8_t*)xalloc((size_t)(Mt * K));
    or_quant_fp8(X, Mt, K, K, Xf, sx);
    uint8_t* Wf = (uint8_t*)xalloc((size_t)(R * K));
    float* wf = (float*)xalloc((size_t)(R * K) * 4);
    for (int64_t i = 0; i < R * K; ++i) wf[i] = rndf() * 4.0f;
    or_e4m3_encode(wf, R * K, Wf);
    or_masked_matmul_fp8(Xf, Mt, K, Wf, R, mask, ldm, Y);
    or_masked_matmul_fp8(Xf, Mt, K, Wf, R, NULL, 0, Y);
    CHECK(or_absmean(W, OR_BF16, R * K) >= 0.0);
    /* bitmap: full capacity and a capacity below the kept count (the overflow path) */
    const int64_t nb = (K + 63) / 64;
    for (int cap = 0; cap < 2; ++cap) {
        const int64_t ldv = cap ? K / 4 : K;
        uint16_t* bv = (uint16_t*)xalloc((size_t)(R * ldv) * 2);
        int32_t* offs = (int32_t*)xalloc((size_t)(R * (nb + 1)) * 4);
        or_bitmap_encode(W, OR_BF16, R, K, mask, ldm, bv, OR_BF16, ldv, offs, nb + 1);
        uint16_t* Wd = (uint16_t*)xalloc((size_t)(R * K) * 2);
        or_bitmap_decode(bv, OR_BF16, ldv, mask, ldm, R, K, Wd, OR_BF16);
        if (!cap)
            for (int64_t rr = 0; rr < R; ++rr)
                for (int64_t k = 0; k < K; ++k)
                    CHECK((double)bf16_to_f32(Wd[rr * K + k]) == masked_value(W, mask, ldm, K, rr, k));
        free(bv), free(offs), free(Wd);
    }
    free(X), free(W), free(S), free(mask), free(Y), free(rm), free(ro), free(Yat), free(A), free(B), free(U);
    free(Xq), free(sx), free(Wt), free(Weff), free(acc), free(y), free(Xf), free(Wf), free(wf);
}

static void check_hessian_gate(void) {
    const int64_t n = 6, K = 24, nr = 3, R = 5, ldm = mask_ld(K);
    const int P = 3, steps = 4;
    uint16_t* X = rand_bf16(n * K);
    int64_t rows[3] = {0, 4, 2};
    double* D = (double*)xalloc((size_t)(nr * K) * 8);
    or_hutchinson_rows(X, OR_BF16, n, K, P, 11, rows, nr, D);
    double* U = (double*)xalloc((size_t)(nr * P * n) * 8);
    or_hutchinson_u_rows(X, OR_BF16, n, K, P, 11, rows, nr, U);
    float* S = (float*)xalloc((size_t)(R * K) * 4);
    for (int64_t i = 0; i < R * K; ++i) S[i] = rndf() * rndf();
    double mu = 0.0, sigma = 0.0;
    or_stats(S, R * K, &mu, &sigma);
    CHECK(sigma >= 0.0);
    float* m = (float*)xalloc((size_t)(R * K) * 4);
    uint8_t* hm = (uint8_t*)xalloc((size_t)(R * ldm));
    memset(hm, 0, (size_t)(R * ldm));
    double* lm = (double*)xalloc((size_t)steps * 8);
    for (int t = 0; t < steps; ++t) or_gate_anneal(S, R, K, mu, sigma, 2, 4, 0.5, 0.8, steps, t, m, hm, ldm, lm);
    or_gate_anneal(S, R, K, mu, sigma, 6, 8, 0.5, 0.5, steps, 1, m, hm, ldm, lm);
    const double g = or_gate_value(S[0], mu, sigma, 0.5, 0.8, 2);
    CHECK(g >= 0.0 && g <= 1.0);
    free(X), free(D), free(U), free(S), free(m), free(hm), free(lm);
}

int main(void) {
    or_set_threads(2);
    check_numerics();
    const int nm[][2] = {{2, 4}, {1, 4}, {3, 4}, {6, 8}, {3, 8}, {1, 2}};
    for (size_t i = 0; i < sizeof nm / sizeof nm[0]; ++i) {
        check_prune_pack(5, 40, nm[i][0], nm[i][1]);
        check_prune_pack(3, 44, nm[i][0], nm[i][1]);   /* a short last group for M = 8 */
    }
    for (int Ns = 2; Ns <= 8; ++Ns) check_slide(4, Ns);
    check_products();
    check_hessian_gate();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitize check ok (threads: %d)\n", or_num_threads());
    return 0;
}
