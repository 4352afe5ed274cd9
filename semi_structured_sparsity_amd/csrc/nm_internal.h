// Internal declarations shared by the HIP translation units of libnmsparse.
// Device helpers, the thread-local error slot, and the host-side launchers
// that the C ABI (nm_capi.hip) calls after validating arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nmsparse.h"

namespace nm {

// ------------------------------------------------------------------ errors
nm_status set_error(nm_status st, const char* fmt, ...);
nm_status check_launch(const char* what);

// ------------------------------------------------------------------ numerics
// bf16 is the upper half of an IEEE binary32: widening is exact; narrowing
// rounds to nearest even and keeps NaN quiet.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Rank key of a score for top-N selection: NaN ranks below everything and
// -0 compares equal to +0 (x + 0 maps -0 to +0).
// sum over z < n of p[z * stride], added in z order starting from 0 (the order of a plain
// loop), with the loads of up to 8 terms issued together: the terms are split-K partials
// written by an earlier kernel on other XCDs, and one dependent load at a time costs a
// memory round trip per term
template <typename Acc>
__device__ __forceinline__ Acc split_sum(const Acc* __restrict__ p, int n, int64_t stride) {
    Acc v = 0;
    for (int z = 0; z < n; z += 8) {
        Acc t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = z + i < n ? p[(int64_t)(z + i) * stride] : Acc(0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (z + i < n) v += t[i];
    }
    return v;
}

// Ranking key of a score: NaN ranks below everything (max(NaN, -inf) is -inf); -0 and +0
// compare equal, as the keys only ever meet in comparisons.
__device__ __forceinline__ float rank_key(float x) { return __builtin_fmaxf(x, -__builtin_inff()); }

// Keep-bits of the top-N of M keys (ties to the lower index): bit i set iff
// fewer than N members beat member i; j beats i iff key_j > key_i, or the keys
// are equal and j < i.
// Keys come from rank_key (never NaN), so for i < j exactly one of "i beats j"
// (k_i >= k_j) and "j beats i" (k_j > k_i) holds: one comparison per pair.
template <int M>
__device__ __forceinline__ uint32_t topn_bits(const float (&k)[M], int N) {
    int beaten[M];
#pragma unroll
    for (int i = 0; i < M; ++i) beaten[i] = 0;
#pragma unroll
    for (int i = 0; i < M; ++i)
#pragma unroll
        for (int j = i + 1; j < M; ++j) {
            const int ib = k[i] >= k[j] ? 1 : 0;
            beaten[j] += ib;
            beaten[i] += 1 - ib;
        }
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < M; ++i) bits |= (beaten[i] < N ? 1u : 0u) << i;
    return bits;
}

// topn_bits<4>(k, 2) as lane-mask logic: member i is kept when it beats at least two of
// the other three (i beats j > i iff k_i >= k_j).  The six comparisons are the only
// per-lane work besides forming the bits; the majorities are boolean operations on
// wave masks.
__device__ __forceinline__ uint32_t top2of4_bits(const float (&k)[4]) {
    const bool c01 = k[0] >= k[1], c02 = k[0] >= k[2], c03 = k[0] >= k[3];
    const bool c12 = k[1] >= k[2], c13 = k[1] >= k[3], c23 = k[2] >= k[3];
    const bool b0 = (c01 && (c02 || c03)) || (c02 && c03);
    const bool b1 = (!c01 && (c12 || c13)) || (c12 && c13);
    const bool b2 = (!c02 && (!c12 || c23)) || (!c12 && c23);
    const bool b3 = (!c03 && (!c13 || !c23)) || (!c13 && !c23);
    return (b0 ? 1u : 0u) | (b1 ? 2u : 0u) | (b2 ? 4u : 0u) | (b3 ? 8u : 0u);
}

// topn_bits<8>(k, 6): every member but the two weakest, where x is weaker than y when
// k_x < k_y, or the keys are equal and x has the higher index.  A knockout over the
// index ranges [0,2), [2,4), ... carries each range's weakest (a) and second weakest (b);
// a member of a right range is weaker than one of the left range iff its key is <=.
// Merging ranges L and R: the weakest is the weaker of the two a's, the second weakest
// the weaker of the winner's b and the loser's a.
__device__ __forceinline__ uint32_t top6of8_bits(const float (&k)[8]) {
    float ka[4], kb[4];
    int ia[4], ib[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bool r = k[2 * q + 1] <= k[2 * q];
        ka[q] = r ? k[2 * q + 1] : k[2 * q];
        kb[q] = r ? k[2 * q] : k[2 * q + 1];
        ia[q] = r ? 2 * q + 1 : 2 * q;
        ib[q] = r ? 2 * q : 2 * q + 1;
    }
    auto merge = [](float la, float lb, int lia, int lib, float ra, float rb, int ria, int rib, float& ma, float& mb,
                    int& mia, int& mib) __attribute__((always_inline)) {
        const bool r = ra <= la;   // the right range holds the weakest
        ma = r ? ra : la;
        mia = r ? ria : lia;
        const float kr = r ? rb : ra, kl = r ? la : lb;   // the right and the left candidate
        const int ir = r ? rib : ria, il = r ? lia : lib;
        const bool rr = kr <= kl;
        mb = rr ? kr : kl;
        mib = rr ? ir : il;
    };
    float a01, b01, a23, b23, a, b;
    int i01, j01, i23, j23, ia8, ib8;
    merge(ka[0], kb[0], ia[0], ib[0], ka[1], kb[1], ia[1], ib[1], a01, b01, i01, j01);
    merge(ka[2], kb[2], ia[2], ib[2], ka[3], kb[3], ia[3], ib[3], a23, b23, i23, j23);
    merge(a01, b01, i01, j01, a23, b23, i23, j23, a, b, ia8, ib8);
    return 0xffu & ~((1u << ia8) | (1u << ib8));
}

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) as a counter-based
// generator: output number i of a generator seeded with s is the variant-13
// finaliser applied to s + (i+1) * 0x9E3779B97F4A7C15.
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Rademacher word of the Hutchinson probes: 64 signs (bit set = -1) for row o, columns
// [64*kb, 64*kb + 64) of probe p.
__device__ __forceinline__ uint64_t rad_word(uint64_t seed, int p, int64_t o, int64_t kb, int64_t kblocks) {
    return splitmix64_at(seed, ((uint64_t)p << 40) + (uint64_t)o * (uint64_t)kblocks + (uint64_t)kb);
}

// 8 sign bits -> 8 bf16 values of +-1 (bit set -> -1).
__device__ __forceinline__ uint4 signs_to_bf16x8(uint32_t byte) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = 0x3F80u | (((byte >> (2 * e)) & 1u) << 15);
        const uint32_t hi = 0x3F80u | (((byte >> (2 * e + 1)) & 1u) << 15);
        w[e] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Moments of a thread's, a block's or the tensor's elements: count, mean, sum of
// squared deviations.  Combined pairwise (Chan, Golub and LeVeque's update), always in
// the same order, so the statistics are run-to-run identical.
struct Moments {
    double n, mean, m2;
};
__device__ __forceinline__ Moments moments_combine(Moments a, Moments b) {
    if (a.n == 0.0) return b;
    if (b.n == 0.0) return a;
    const double n = a.n + b.n, d = b.mean - a.mean;
    return Moments{n, a.mean + d * (b.n / n), a.m2 + b.m2 + d * d * (a.n * b.n / n)};
}

inline int index_bits(int M) {
    int b = 0;
    while ((1 << b) < M) ++b;
    return b;
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int grid_cap(int64_t blocks, int64_t cap = 1 << 20) { return (int)(blocks < 1 ? 1 : (blocks > cap ? cap : blocks)); }

// ------------------------------------------------------------------ launchers
// colsumsq
size_t colsumsq_ws(int64_t n, int64_t K);
void launch_colsumsq(const void* X, nm_dtype xdt, int64_t n, int64_t K, int64_t ldx, float* H, void* ws,
                     hipStream_t s);
// score / mask / pack
void launch_score(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const float* H, int64_t ldh,
                  float eps, nm_score_mode mode, float* S, int64_t lds, hipStream_t s);
void launch_mask(const float* S, int64_t R, int64_t K, int64_t lds, int N, int M, uint8_t* mask, int64_t ldm,
                 hipStream_t s);
void launch_pack(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask, int64_t ldm,
                 int N, int M, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx, int64_t ldi, hipStream_t s);
// Groups of G consecutive bits of a caller's mask with more than cap set bits, counted on
// the device; synchronises the stream (NM_FLAG_VALIDATE).
nm_status count_overfull(const uint8_t* mask, int64_t ldm, int64_t R, int64_t K, int G, int cap, hipStream_t s,
                         int64_t* bad);
void launch_prune_pack(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh, float eps,
                       nm_score_mode mode, const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K, int N,
                       int M, uint8_t* mask, int64_t ldm, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx,
                       int64_t ldi, hipStream_t s);
void launch_slide(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh, float eps,
                  nm_score_mode mode, bool select, const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K,
                  int Ns, const uint8_t* mask_in, uint8_t* mask_out, int64_t ldm, nm_dtype vdt, void* vals,
                  int64_t ldv, uint32_t* idx, int64_t ldi, hipStream_t s);
// reductions / gate
size_t reduce_ws(int64_t R, int64_t K);
size_t gate_ws(int64_t R, int64_t K, int steps);
void launch_stats(const float* S, int64_t R, int64_t K, int64_t lds, double* stats, void* ws, hipStream_t s);
// stats = (mean, population std) from nparts block moments laid out [count | mean | m2][nparts]
void launch_moments_final(const double* part, int nparts, double* stats, hipStream_t s);
void launch_absmean(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, float* alpha, void* ws,
                    hipStream_t s);
void launch_gate(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats, int N, int M, float T0,
                 float rho, int steps, int m_step, float* m_out, int64_t ldf, uint8_t* hard_mask, int64_t ldm,
                 double* lmid, void* ws, hipStream_t s);
// the gate with the 2:4 pack of bf16 W under its hard mask in the same pass; false (nothing
// launched) where the fused kernel does not apply
bool launch_gate_pack(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats, int N, int M, float T0,
                      float rho, int steps, int m_step, float* m_out, int64_t ldf, uint8_t* hard_mask, int64_t ldm,
                      double* lmid, const uint16_t* W, int64_t ldw, uint16_t* vals, int64_t ldv, uint32_t* idx,
                      int64_t ldi, void* ws, hipStream_t s);
// sparse GEMM
void launch_quant_lift(const void* X, int64_t Mtok, int64_t K, int64_t ldx, int Ns, nm_dtype qdt, void* Xq,
                       int64_t ldq, float* x_scale, hipStream_t s);
size_t spmm_ws(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt);
// stacked low-rank adapters of a sparse layer: A [rank, K] (lda), B [R, rank] (ldb), bf16
struct LowRankIn {
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B;
    int64_t ldb;
    int rank;
};
size_t spmm_lowrank_ws(int64_t Mtok, int64_t K, int64_t R, int Ns, int rank);
nm_status launch_spmm_lowrank(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals,
                              const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi, int Ns, const LowRankIn& lr,
                              void* Y, nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s);
nm_status launch_spmm(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx, const void* vals,
                      const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi, int Ns, const float* x_scale,
                      float w_scale, void* Y, nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s);
// bitmap format (mask + compact values + per-64-column-block value offsets)
void launch_bitmap_encode(const void* W, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask, int64_t ldm,
                          void* vals, int64_t ldv, int32_t* offs, int64_t ldo, hipStream_t s);
size_t bitmap_spmm_ws(int64_t Mtok, int64_t K, int64_t R);
// Y = X W^T with a dense bf16 W [R, K] (ldw) on the dense split ring; NM_ERR_SHAPE without a
// launch when it does not apply (K % 64, unaligned rows, 32-bit offsets, fewer 256 x 256
// tiles than CUs).
// Hutchinson second product D = (2/P) sum_p V_p .* (U_p X) on the dense split ring (U [P*R, n]
// probes stacked along rows, XT [K, n] the transposed calibration rows); NM_ERR_SHAPE without
// a launch when it does not apply (unaligned workspace, 32-bit offsets).
// Score epilogue of the second product: W [R, K] bf16 (ldw), eps, block moments out.
struct HutchScore {
    const uint16_t* W;
    int64_t ldw;
    float eps;
    double* mpart;
};
nm_status launch_hutch_ring(const uint16_t* U, const uint16_t* XT, int64_t n, int64_t K, int64_t R, int probes,
                            uint64_t seed, float* D, int64_t ldd, hipStream_t s, const HutchScore* sc = nullptr);
int64_t hutch_ring_blocks(int64_t K, int64_t R);   // blocks (and moment partials) of the score epilogue
// Hutchinson first product U [P*R, n] (bf16, row stride n) = V X^T with the probe rows V
// generated into the dense split ring's LDS stages; NM_ERR_SHAPE without a launch when it
// does not apply (32-bit offsets).
nm_status launch_hutch_u_ring(const uint16_t* X, int64_t ldx, int64_t n, int64_t K, int64_t R, int probes,
                              uint64_t seed, uint16_t* U, hipStream_t s);
nm_status launch_dense_ring(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx, int64_t Mtok, int64_t K,
                            int64_t R, void* Y, nm_dtype ydt, int64_t ldy, hipStream_t s);
nm_status launch_bitmap_spmm(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals, int64_t ldv,
                             const uint8_t* mask, int64_t ldm, const int32_t* offs, int64_t ldo, int64_t R, void* Y,
                             nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s);
// Hutchinson
size_t hutch_ws(int64_t n, int64_t K, int64_t R, int probes);
size_t hutch_score_ws(int64_t n, int64_t K, int64_t R, int probes);
nm_status launch_hutchinson_score(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes,
                                  uint64_t seed, const uint16_t* W, int64_t ldw, float eps, float* S, int64_t lds,
                                  double* stats, void* ws, hipStream_t s);
void launch_hutchinson(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes, uint64_t seed,
                       float* D, int64_t ldd, void* ws, hipStream_t s);

}  // namespace nm
