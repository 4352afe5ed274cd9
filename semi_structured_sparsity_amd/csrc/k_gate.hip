// Per-tensor reductions and the soft-gate annealing pass.
//
// "SparseForge", Methodology 2: scores are standardised and passed through a
// temperature sigmoid to form a continuous gate.  Methodology 3: the gate is
// blended with the hard top-N target by a factor beta, the temperature is
// annealed geometrically, a binary-preference term sum m(1-m) measures how far
// the mask is from binary, and a final projection yields the hard N:M mask.
// "Sparse-BitNet", sections 1-2: a ternary layer carries one scale, the mean
// absolute value of its master weights.
//
// All reductions are deterministic: a fixed grid whose threads accumulate
// fixed subsets in f64, a fixed-order LDS tree per block, and a single-block
// pass over the block partials in block order.
#include "nm_internal.h"

namespace nm {

constexpr int kRedBlocks = 1024;
constexpr int kRedThreads = 256;
constexpr int kMaxSteps = 64;
constexpr int kGateBlocks = 2048;  // gate grid (its per-step partials are summed in block order)

__device__ __forceinline__ double block_sum(double v, double* sh) {
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    const double r = sh[0];
    __syncthreads();
    return r;
}

__device__ __forceinline__ float load_elem(const void* p, nm_dtype dt, int64_t i) {
    if (dt == NM_F32) return ((const float*)p)[i];
    if (dt == NM_BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
    if (dt == NM_I8) return (float)((const int8_t*)p)[i];
    return (float)((const int32_t*)p)[i];
}

// Fixed-order tree of the block's per-thread moments; the result is left in sh[*][0].
__device__ __forceinline__ void block_moments(Moments m, double (*sh)[kRedThreads]) {
    sh[0][threadIdx.x] = m.n;
    sh[1][threadIdx.x] = m.mean;
    sh[2][threadIdx.x] = m.m2;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            const Moments o = moments_combine(Moments{sh[0][threadIdx.x], sh[1][threadIdx.x], sh[2][threadIdx.x]},
                                              Moments{sh[0][threadIdx.x + w], sh[1][threadIdx.x + w],
                                                      sh[2][threadIdx.x + w]});
            sh[0][threadIdx.x] = o.n;
            sh[1][threadIdx.x] = o.mean;
            sh[2][threadIdx.x] = o.m2;
        }
        __syncthreads();
    }
}

// Elements of [R, K] (leading dim ld) are visited in units of VEC consecutive
// elements of a row; thread u of the fixed grid takes units u, u + stride, ...,
// UN units per round with all UN loads issued before any is used (the grid then
// reads UN regions a grid's width apart at a time).  When VEC > 1
// the caller guarantees K % VEC == 0, ld % VEC == 0 and 16-byte alignment.
template <typename T, int VEC, typename F>
__device__ __forceinline__ void for_units(const T* __restrict__ X, int64_t R, int64_t K, int64_t ld, F&& f) {
    constexpr int UN = 4;   // 8 or 16 in flight measured slower (the S statistics pass 177 -> 199 / 209 us)
    const int64_t upr = K / VEC, total = R * upr;
    const int64_t stride = (int64_t)kRedBlocks * kRedThreads;
    const int64_t u0 = (int64_t)blockIdx.x * kRedThreads + threadIdx.x;
    if (u0 >= total) return;
    int64_t r = u0 / upr, c = u0 - r * upr;
    const int64_t dr = stride / upr, dc = stride - dr * upr;
    auto step = [&]() __attribute__((always_inline)) {
        r += dr;
        c += dc;
        if (c >= upr) {
            c -= upr;
            r += 1;
        }
    };
    for (int64_t u = u0; u < total; u += UN * stride) {
        float x[UN][VEC];
#pragma unroll
        for (int j = 0; j < UN; ++j) {
            const bool ok = u + j * stride < total;
            const int64_t rr = ok ? r : 0, cc = ok ? c : 0;
            if constexpr (VEC == 1) {
                x[j][0] = load_elem(X, sizeof(T) == 2 ? NM_BF16 : NM_F32, rr * ld + cc);
            } else {
                const uint4 q = *(const uint4*)(X + rr * ld + cc * VEC);
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    if constexpr (sizeof(T) == 2) x[j][v] = bf16_bits_to_f32((w[v >> 1] >> (16 * (v & 1))) & 0xffffu);
                    else x[j][v] = __uint_as_float(w[v]);
                }
            }
            step();
        }
#pragma unroll
        for (int j = 0; j < UN; ++j)
            if (u + j * stride < total) f(x[j]);
    }
}

// Per-tensor mean and population standard deviation in one pass: each thread keeps
// sums of (x - c) and (x - c)^2 about its first element c, turns them into moments,
// and the moments are combined in a fixed tree per block.
template <int VEC>
__global__ __launch_bounds__(kRedThreads) void moments_partial_kernel(const float* __restrict__ S, int64_t R, int64_t K,
                                                                      int64_t ld, double* __restrict__ part) {
    __shared__ double sh[3][kRedThreads];
    double n = 0.0, s1 = 0.0, s2 = 0.0, c = 0.0;
    bool first = true;
    for_units<float, VEC>(S, R, K, ld, [&](const float* x) {
        if (first) {
            c = (double)x[0];
            first = false;
        }
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const double d = (double)x[v] - c;
            s1 += d;
            s2 += d * d;
        }
        n += VEC;
    });
    Moments m{n, n > 0.0 ? c + s1 / n : 0.0, n > 0.0 ? s2 - s1 * (s1 / n) : 0.0};
    if (m.m2 < 0.0) m.m2 = 0.0;
    block_moments(m, sh);
    if (threadIdx.x < 3) part[threadIdx.x * kRedBlocks + blockIdx.x] = sh[threadIdx.x][0];
}

// The block moments are combined in a fixed tree: thread t folds blocks t, t + 256,
// ... in order, then the threads' moments meet in the block tree.  (A combine
// divides in f64; a single thread folding all blocks one after another would
// spend its time waiting on those divisions.)
__global__ __launch_bounds__(kRedThreads) void moments_final_kernel(const double* __restrict__ part, int nparts,
                                                                    double* __restrict__ stats) {
    __shared__ double sh[3][kRedThreads];
    Moments m{0.0, 0.0, 0.0};
    // the partials of 16 passes are loaded before they are combined (in the same order):
    // they were written by blocks on every XCD, so each load waits on memory (12 -> 8 us at
    // 3584 partials)
    constexpr int PF = 16;
    for (int i0 = threadIdx.x; i0 < nparts; i0 += PF * kRedThreads) {
        Moments q[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int i = i0 + u * kRedThreads;
            q[u] = i < nparts ? Moments{part[i], part[nparts + i], part[2 * nparts + i]} : Moments{0.0, 0.0, 0.0};
        }
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (i0 + u * kRedThreads < nparts) m = moments_combine(m, q[u]);
    }
    block_moments(m, sh);
    if (threadIdx.x == 0) {
        const double nn = sh[0][0], mean = sh[1][0], m2 = sh[2][0];
        stats[0] = nn > 0.0 ? mean : 0.0;
        stats[1] = nn > 0.0 ? sqrt(m2 / nn) : 0.0;
    }
}

// sum |x| (for the ternary scale), f64 per thread, fixed-order LDS tree per block
template <typename T, int VEC>
__global__ __launch_bounds__(kRedThreads) void abssum_partial_kernel(const T* __restrict__ X, int64_t R, int64_t K,
                                                                     int64_t ld, double* __restrict__ part) {
    __shared__ double sh[kRedThreads];
    double acc = 0.0;
    for_units<T, VEC>(X, R, K, ld, [&](const float* x) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc += fabs((double)x[v]);
    });
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// kind 2: sum |x| for any dtype, element by element (the general path)
__global__ __launch_bounds__(kRedThreads) void reduce_partial_kernel(const void* __restrict__ X, nm_dtype dt,
                                                                     int64_t R, int64_t K, int64_t ld,
                                                                     double* __restrict__ part) {
    __shared__ double sh[kRedThreads];
    const int64_t total = R * K;
    double acc = 0.0;
    for (int64_t t = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; t < total; t += (int64_t)kRedBlocks * kRedThreads) {
        const int64_t r = t / K, k = t - r * K;
        acc += fabs((double)load_elem(X, dt, r * ld + k));
    }
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// out_f[0] = (float)(sum of the block partials, in block order, / n)
__global__ __launch_bounds__(kRedThreads) void reduce_final_kernel(const double* __restrict__ part, int nparts,
                                                                   int64_t n, float* out_f) {
    __shared__ double sh[kRedThreads];
    double acc = 0.0;
    for (int i = threadIdx.x; i < nparts; i += kRedThreads) acc += part[i];
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) out_f[0] = (float)(n > 0 ? s / (double)n : 0.0);
}

size_t reduce_ws(int64_t, int64_t) { return (size_t)3 * kRedBlocks * sizeof(double); }

static bool vec_ok(const void* p, int64_t K, int64_t ld, int vec) {
    return (K % vec) == 0 && (ld % vec) == 0 && (((uintptr_t)p) & 15) == 0;
}

void launch_stats(const float* S, int64_t R, int64_t K, int64_t lds, double* stats, void* ws, hipStream_t s) {
    double* part = (double*)ws;
    if (vec_ok(S, K, lds, 4))
        hipLaunchKernelGGL(moments_partial_kernel<4>, dim3(kRedBlocks), dim3(kRedThreads), 0, s, S, R, K, lds, part);
    else
        hipLaunchKernelGGL(moments_partial_kernel<1>, dim3(kRedBlocks), dim3(kRedThreads), 0, s, S, R, K, lds, part);
    hipLaunchKernelGGL(moments_final_kernel, dim3(1), dim3(kRedThreads), 0, s, (const double*)part, kRedBlocks, stats);
}

void launch_moments_final(const double* part, int nparts, double* stats, hipStream_t s) {
    hipLaunchKernelGGL(moments_final_kernel, dim3(1), dim3(kRedThreads), 0, s, part, nparts, stats);
}

void launch_absmean(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, float* alpha, void* ws,
                    hipStream_t s) {
    double* part = (double*)ws;
    const dim3 g(kRedBlocks), b(kRedThreads);
    if (wdt == NM_BF16 && vec_ok(W, K, ldw, 8))
        hipLaunchKernelGGL((abssum_partial_kernel<uint16_t, 8>), g, b, 0, s, (const uint16_t*)W, R, K, ldw, part);
    else if (wdt == NM_F32 && vec_ok(W, K, ldw, 4))
        hipLaunchKernelGGL((abssum_partial_kernel<float, 4>), g, b, 0, s, (const float*)W, R, K, ldw, part);
    else
        hipLaunchKernelGGL(reduce_partial_kernel, g, b, 0, s, W, wdt, R, K, ldw, part);
    hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(kRedThreads), 0, s, (const double*)part, kRedBlocks, R * K,
                       alpha);
}

// ------------------------------------------------------------------ gate / anneal
// A thread owns one mask byte: 8 consecutive scores of a row (two 4-groups or
// one 8-group).  For every step it forms the gate, the blend with the hard
// target and the binary-preference term; the block sums that term per step.
// The blend of one chosen step (m_step) is kept and written out when asked for.
// SMAX bounds the step count at compile time so that the per-step sums live in
// registers.  The gate uses the hardware 2^x and reciprocal (about 1 ulp each):
// sigmoid(z/T) = 1 / (1 + 2^(-z * log2(e) / T)); the blend (1 - beta) g + beta h and the
// sum of m (1 - m) are fused multiply-adds.  A step with beta = 1 blends nothing of the
// sigmoid: its m is the hard target and contributes 0 to L_mid.
__device__ __forceinline__ uint32_t group_topn_bits(const float* key, int g0, int M, int N) {
    uint32_t gb = 0;
    for (int i = 0; i < M; ++i) {
        int beaten = 0;
        for (int j = 0; j < M; ++j) {
            if (j == i) continue;
            beaten += ((j < i) ? (key[g0 + j] >= key[g0 + i]) : (key[g0 + j] > key[g0 + i])) ? 1 : 0;
        }
        if (beaten < N) gb |= 1u << i;
    }
    return gb;
}

template <int SMAX, bool HALVING>
__global__ __launch_bounds__(kRedThreads) void gate_kernel(const float* __restrict__ S, int64_t R, int64_t K,
                                                           int64_t lds, const double* __restrict__ stats, int N, int M,
                                                           float T0, float rho, int steps, int m_step,
                                                           float* __restrict__ m_out, int64_t ldf,
                                                           uint8_t* __restrict__ hard_mask, int64_t ldm,
                                                           double* __restrict__ part) {
    __shared__ double sh[kRedThreads];
    const double mu = stats[0], sigma = stats[1];
    const double inv_sigma = sigma > 0.0 ? 1.0 / sigma : 0.0;   // z = 0 when the scores are constant
    const int64_t bpr = (K + 7) / 8;
    const int64_t total = R * bpr;
    float cs[SMAX], beta[SMAX];  // log2(e) / T_t and the blend factor of step t
    double lm[SMAX];
    // HALVING (rho = 1/2): T_t halves every step, so in f32 the exponent -z log2(e) / T_t is
    // exactly twice the previous step's (scaling by a power of two commutes with rounding)
    // and the exponential is the previous one squared: one multiply instead of a 2^x.  Each
    // squaring doubles the relative error carried from the last 2^x, so the chain restarts
    // with a 2^x every fourth step (at most three squarings: about 8 ulps, 5e-7)
#pragma unroll
    for (int t = 0; t < SMAX; ++t) {
        const float T = T0 * powf(rho, (float)t);
        cs[t] = 1.4426950408889634f / T;
        beta[t] = steps > 1 ? (float)t / (float)(steps - 1) : 1.0f;
        lm[t] = 0.0;
    }
    const bool vec = (lds % 4) == 0 && (((uintptr_t)S) & 15) == 0 && (m_out == nullptr || ((ldf % 4) == 0 &&
                                                                        (((uintptr_t)m_out) & 15) == 0));
    const int64_t stride = (int64_t)kGateBlocks * kRedThreads;
    const int64_t u0 = (int64_t)blockIdx.x * kRedThreads + threadIdx.x;
    int64_t r = u0 / bpr, b = u0 - r * bpr;                   // (row, byte) of unit u, advanced without division
    const int64_t dr = stride / bpr, db = stride - dr * bpr;
    for (int64_t u = u0; u < total; u += stride) {
        const int64_t k0 = b * 8;
        const int ne = (K - k0) < 8 ? (int)(K - k0) : 8;
        float s[8], z[8], key[8];
        if (vec && ne == 8) {
            const float4 v0 = *(const float4*)(S + r * lds + k0);
            const float4 v1 = *(const float4*)(S + r * lds + k0 + 4);
            s[0] = v0.x; s[1] = v0.y; s[2] = v0.z; s[3] = v0.w; s[4] = v1.x; s[5] = v1.y; s[6] = v1.z; s[7] = v1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) s[i] = i < ne ? S[r * lds + k0 + i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            z[i] = sigma > 0.0 ? (float)(((double)s[i] - mu) * inv_sigma) : 0.f;
            key[i] = rank_key(s[i]);
        }
        // hard target h: top-N of the score per group
        uint32_t hbits = 0;
        if (M == 4 && ne == 8) {
            const float k0v[4] = {key[0], key[1], key[2], key[3]}, k1v[4] = {key[4], key[5], key[6], key[7]};
            hbits = topn_bits<4>(k0v, N) | (topn_bits<4>(k1v, N) << 4);
        } else if (M == 8 && ne == 8) {
            hbits = topn_bits<8>(key, N);
        } else {
            for (int g = 0; g * M < ne; ++g) hbits |= group_topn_bits(key, g * M, M, N) << (g * M);
        }
        float hv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = ((hbits >> i) & 1u) ? 1.0f : 0.0f;
        float m[8], mo[8], e[8];   // m_t of the current step and of step m_step; 2^(-z log2(e) / T_t)
#pragma unroll
        for (int i = 0; i < 8; ++i) m[i] = mo[i] = e[i] = 0.f;
#pragma unroll
        for (int t = 0; t < SMAX; ++t) {
            if (t < steps) {
                if (beta[t] == 1.0f) {
                    // the blend is the hard target itself (the sigmoid's weight is 0): m (1 - m) = 0
#pragma unroll
                    for (int i = 0; i < 8; ++i) m[i] = hv[i];
                } else {
                    float acc = 0.f;   // <= 8 terms in [0, 1/4]: f32 here, f64 across units
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if (HALVING && (t & 3) != 0) e[i] = e[i] * e[i];
                        else e[i] = __builtin_amdgcn_exp2f(-z[i] * cs[t]);
                        const float g = __builtin_amdgcn_rcpf(1.0f + e[i]);
                        m[i] = __builtin_fmaf(1.0f - beta[t], g, beta[t] * hv[i]);
                        const float mm = i < ne ? m[i] : 0.f;   // past the row end: adds 0
                        acc = __builtin_fmaf(mm, 1.0f - mm, acc);
                    }
                    lm[t] += (double)acc;
                }
                if (t == m_step) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) mo[i] = m[i];
                }
            }
        }
        // final projection: top-N of m_{steps-1}
        float km[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) km[i] = rank_key(m[i]);
        uint32_t fbits = 0;
        if (M == 4 && ne == 8) {
            const float k0v[4] = {km[0], km[1], km[2], km[3]}, k1v[4] = {km[4], km[5], km[6], km[7]};
            fbits = topn_bits<4>(k0v, N) | (topn_bits<4>(k1v, N) << 4);
        } else if (M == 8 && ne == 8) {
            fbits = topn_bits<8>(km, N);
        } else {
            for (int g = 0; g * M < ne; ++g) fbits |= group_topn_bits(km, g * M, M, N) << (g * M);
        }
        hard_mask[r * ldm + b] = (uint8_t)fbits;
        if (m_out) {
            if (vec && ne == 8) {
                *(float4*)(m_out + r * ldf + k0) = make_float4(mo[0], mo[1], mo[2], mo[3]);
                *(float4*)(m_out + r * ldf + k0 + 4) = make_float4(mo[4], mo[5], mo[6], mo[7]);
            } else {
                for (int i = 0; i < ne; ++i) m_out[r * ldf + k0 + i] = mo[i];
            }
        }
        r += dr;
        b += db;
        if (b >= bpr) {
            b -= bpr;
            r += 1;
        }
    }
#pragma unroll
    for (int t = 0; t < SMAX; ++t) {
        if (t < steps) {
            const double v = block_sum(lm[t], sh);
            if (threadIdx.x == 0) part[(int64_t)t * kGateBlocks + blockIdx.x] = v;
        }
    }
}

// The same pass for whole 8-score units (K a multiple of 8, 16-byte aligned rows) and a
// step count S fixed at compile time, M = GM: every step's beta is a constant, so the
// steps unroll with no per-step branch and the per-step sums stay in registers.  The
// arithmetic of each step is that of gate_kernel, operation for operation (beta * h is
// the select h ? beta : 0, which is exact), so both give the same bits.  The last step
// has beta = 1: its blend is the hard target, whose top-N (exactly N ones per group) is
// the hard target itself, so the final projection is h.  WANT_M: keep and write the
// blend of step m_step.
// PACK (2:4, K a multiple of 32): the unit's 8 bf16 weights are also packed under the hard
// mask, as the 2:4 packer does from a given mask: per 4-group the two kept values
// (positions p0 < p1, bytes 2p, 2p+1 of the group's 8) by one byte permute, and p0 | p1 << 2
// as the group's index nibble; the 4 lanes of a quad hold 32 consecutive columns of one row
// (the units of a row are consecutive and 4 | K/8), so their nibbles make one index word.
// The gate is bound by its vector instructions, so the weight's stream rides along.
struct GatePackOut {
    const uint16_t* W;   // [R, ldw] bf16
    int64_t ldw;
    uint16_t* vals;      // [R, ldv] bf16 kept values
    int64_t ldv;
    uint32_t* idx;       // [R, ldi] 2-bit in-group positions
    int64_t ldi;
};

template <int S, int GM, bool HALVING, bool WANT_M, bool PACK = false>
__global__ __launch_bounds__(kRedThreads) void gate_fast_kernel(const float* __restrict__ Sc, int64_t R, int64_t K,
                                                                int64_t lds, const double* __restrict__ stats, int N,
                                                                float T0, float rho, int m_step, float* __restrict__ m_out,
                                                                int64_t ldf, uint8_t* __restrict__ hard_mask, int64_t ldm,
                                                                double* __restrict__ part, GatePackOut po) {
    static_assert(!PACK || GM == 4, "the fused pack is for 2:4");
    static_assert(S >= 2 && (GM == 4 || GM == 8), "fixed schedules of at least two steps, 2:4-like or 6:8-like groups");
    __shared__ double sh[kRedThreads];
    const double mu = stats[0], sigma = stats[1];
    const double inv_sigma = sigma > 0.0 ? 1.0 / sigma : 0.0;
    const int64_t bpr = K / 8;
    const int64_t total = R * bpr;
    float cs[S - 1];
    double lm[S - 1];
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        const float T = T0 * powf(rho, (float)t);
        cs[t] = 1.4426950408889634f / T;
        lm[t] = 0.0;
    }
    const int64_t stride = (int64_t)kGateBlocks * kRedThreads;
    const int64_t u0 = (int64_t)blockIdx.x * kRedThreads + threadIdx.x;
    int64_t r = u0 / bpr, b = u0 - r * bpr;
    const int64_t dr = stride / bpr, db = stride - dr * bpr;
    for (int64_t u = u0; u < total; u += stride) {
        const int64_t k0 = b * 8;
        const float4 v0 = *(const float4*)(Sc + r * lds + k0);
        const float4 v1 = *(const float4*)(Sc + r * lds + k0 + 4);
        const float s[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        float z[8], key[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            z[i] = sigma > 0.0 ? (float)(((double)s[i] - mu) * inv_sigma) : 0.f;
            key[i] = rank_key(s[i]);
        }
        uint32_t hbits;
        if constexpr (GM == 4) {
            const float ka[4] = {key[0], key[1], key[2], key[3]}, kb[4] = {key[4], key[5], key[6], key[7]};
            if (N == 2) hbits = top2of4_bits(ka) | (top2of4_bits(kb) << 4);
            else hbits = topn_bits<4>(ka, N) | (topn_bits<4>(kb, N) << 4);
        } else {
            if (N == 6) hbits = top6of8_bits(key);
            else hbits = topn_bits<8>(key, N);
        }
        if constexpr (PACK) {
            const uint4 wv = *(const uint4*)(po.W + r * po.ldw + k0);
            const uint32_t wu[4] = {wv.x, wv.y, wv.z, wv.w};
            uint32_t packed[2], nib = 0;
#pragma unroll
            for (int gi = 0; gi < 2; ++gi) {
                const uint32_t bits = (hbits >> (4 * gi)) & 0xFu;
                const uint32_t p0 = __builtin_ctz(bits), p1 = 31u - __builtin_clz(bits);
                const uint32_t s0 = 0x0100u + p0 * 0x0202u, s1 = 0x0100u + p1 * 0x0202u;
                packed[gi] = __builtin_amdgcn_perm(wu[2 * gi + 1], wu[2 * gi], s0 | (s1 << 16));
                nib |= (p0 | (p1 << 2)) << (4 * gi);
            }
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u32x2_t{packed[0], packed[1]}, (u32x2_t*)(po.vals + r * po.ldv + (k0 >> 1)));
            const int q = threadIdx.x & 3;
            uint32_t v = nib << (8 * q);
            v |= (uint32_t)__shfl_xor((int)v, 1);
            v |= (uint32_t)__shfl_xor((int)v, 2);
            if (q == 0) __builtin_nontemporal_store(v, po.idx + r * po.ldi + (k0 >> 5));
        }
        bool h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (hbits >> i) & 1u;
        float e[8], mo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = mo[i] = 0.f;
#pragma unroll
        for (int t = 0; t < S - 1; ++t) {
            constexpr float kOne = 1.0f;
            const float beta = (float)t / (float)(S - 1);
            const float wg = kOne - beta;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (HALVING && (t & 3) != 0) e[i] = e[i] * e[i];
                else e[i] = __builtin_amdgcn_exp2f(-z[i] * cs[t]);
                const float g = __builtin_amdgcn_rcpf(1.0f + e[i]);
                const float m = __builtin_fmaf(wg, g, h[i] ? beta : 0.f);
                acc = __builtin_fmaf(m, 1.0f - m, acc);
                if constexpr (WANT_M) mo[i] = t == m_step ? m : mo[i];
            }
            lm[t] += (double)acc;
        }
        hard_mask[r * ldm + b] = (uint8_t)hbits;
        if constexpr (WANT_M) {
            if (m_step == S - 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) mo[i] = h[i] ? 1.0f : 0.0f;
            }
            *(float4*)(m_out + r * ldf + k0) = make_float4(mo[0], mo[1], mo[2], mo[3]);
            *(float4*)(m_out + r * ldf + k0 + 4) = make_float4(mo[4], mo[5], mo[6], mo[7]);
        }
        r += dr;
        b += db;
        if (b >= bpr) {
            b -= bpr;
            r += 1;
        }
    }
    // the per-step sums in the same order as gate_kernel (the beta = 1 step adds nothing)
#pragma unroll
    for (int t = 0; t < S; ++t) {
        const double v = block_sum(t < S - 1 ? lm[t < S - 1 ? t : 0] : 0.0, sh);
        if (threadIdx.x == 0) part[(int64_t)t * kGateBlocks + blockIdx.x] = v;
    }
}

// Block t sums step t's per-block partials (one block per step: the steps no longer wait
// for each other's loads and barrier trees; 28 -> 4 us for 8 steps, same sums).
__global__ __launch_bounds__(kRedThreads) void gate_final_kernel(const double* __restrict__ part,
                                                                 double* __restrict__ lmid) {
    __shared__ double sh[kRedThreads];
    const int t = blockIdx.x;
    double acc = 0.0;
    for (int i = threadIdx.x; i < kGateBlocks; i += kRedThreads) acc += part[(int64_t)t * kGateBlocks + i];
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) lmid[t] = s;
}

size_t gate_ws(int64_t, int64_t, int steps) { return (size_t)kGateBlocks * (size_t)(steps > 0 ? steps : 1) * sizeof(double); }

void launch_gate(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats, int N, int M, float T0,
                 float rho, int steps, int m_step, float* m_out, int64_t ldf, uint8_t* hard_mask, int64_t ldm,
                 double* lmid, void* ws, hipStream_t s) {
    double* part = (double*)ws;
    // the default schedule (8 steps) on whole 8-score units: the unrolled kernel
    const bool fast = steps == 8 && (M == 4 || M == 8) && K % 8 == 0 && lds % 4 == 0 && ((uintptr_t)S & 15) == 0 &&
                      (m_out == nullptr || (ldf % 4 == 0 && ((uintptr_t)m_out & 15) == 0));
    if (fast) {
#define NM_GATE_FAST(GM, HV, WM)                                                                                        \
    hipLaunchKernelGGL((gate_fast_kernel<8, GM, HV, WM>), dim3(kGateBlocks), dim3(kRedThreads), 0, s, S, R, K, lds, stats, \
                       N, T0, rho, m_step, m_out, ldf, hard_mask, ldm, part, GatePackOut{})
        const bool halving = rho == 0.5f, wm = m_out != nullptr;
        if (M == 4) {
            if (halving) {
                if (wm) NM_GATE_FAST(4, true, true);
                else NM_GATE_FAST(4, true, false);
            } else {
                if (wm) NM_GATE_FAST(4, false, true);
                else NM_GATE_FAST(4, false, false);
            }
        } else {
            if (halving) {
                if (wm) NM_GATE_FAST(8, true, true);
                else NM_GATE_FAST(8, true, false);
            } else {
                if (wm) NM_GATE_FAST(8, false, true);
                else NM_GATE_FAST(8, false, false);
            }
        }
#undef NM_GATE_FAST
        hipLaunchKernelGGL(gate_final_kernel, dim3((unsigned)steps), dim3(kRedThreads), 0, s, (const double*)part, lmid);
        return;
    }
#define NM_GATE(SM, HV)                                                                                             \
    hipLaunchKernelGGL((gate_kernel<SM, HV>), dim3(kGateBlocks), dim3(kRedThreads), 0, s, S, R, K, lds, stats, N, M, \
                       T0, rho, steps, m_step, m_out, ldf, hard_mask, ldm, part)
    const bool halving = rho == 0.5f;
    if (steps <= 8) {
        if (halving) NM_GATE(8, true);
        else NM_GATE(8, false);
    } else if (steps <= 16) {
        if (halving) NM_GATE(16, true);
        else NM_GATE(16, false);
    } else {
        if (halving) NM_GATE(kMaxSteps, true);
        else NM_GATE(kMaxSteps, false);
    }
#undef NM_GATE
    hipLaunchKernelGGL(gate_final_kernel, dim3((unsigned)steps), dim3(kRedThreads), 0, s, (const double*)part, lmid);
}

bool launch_gate_pack(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats, int N, int M, float T0,
                      float rho, int steps, int m_step, float* m_out, int64_t ldf, uint8_t* hard_mask, int64_t ldm,
                      double* lmid, const uint16_t* W, int64_t ldw, uint16_t* vals, int64_t ldv, uint32_t* idx,
                      int64_t ldi, void* ws, hipStream_t s) {
    // the unrolled 8-step kernel on 2:4 with whole index words per row, 16-byte weight rows
    // and 8-byte value rows
    const bool fused = steps == 8 && M == 4 && N == 2 && K % 32 == 0 && lds % 4 == 0 && ((uintptr_t)S & 15) == 0 &&
                       (m_out == nullptr || (ldf % 4 == 0 && ((uintptr_t)m_out & 15) == 0)) && ldw % 8 == 0 &&
                       ((uintptr_t)W & 15) == 0 && ldv % 4 == 0 && ((uintptr_t)vals & 7) == 0;
    if (!fused) return false;
    double* part = (double*)ws;
    const GatePackOut po{W, ldw, vals, ldv, idx, ldi};
#define NM_GATE_PACK(HV, WM)                                                                                            \
    hipLaunchKernelGGL((gate_fast_kernel<8, 4, HV, WM, true>), dim3(kGateBlocks), dim3(kRedThreads), 0, s, S, R, K, lds, \
                       stats, N, T0, rho, m_step, m_out, ldf, hard_mask, ldm, part, po)
    const bool halving = rho == 0.5f, wm = m_out != nullptr;
    if (halving) {
        if (wm) NM_GATE_PACK(true, true);
        else NM_GATE_PACK(true, false);
    } else {
        if (wm) NM_GATE_PACK(false, true);
        else NM_GATE_PACK(false, false);
    }
#undef NM_GATE_PACK
    hipLaunchKernelGGL(gate_final_kernel, dim3((unsigned)steps), dim3(kRedThreads), 0, s, (const double*)part, lmid);
    return true;
}

}  // namespace nm
