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

// kind 0: sum x; 1: sum (x - center[0])^2; 2: sum |x|
__global__ __launch_bounds__(kRedThreads) void reduce_partial_kernel(const void* __restrict__ X, nm_dtype dt,
                                                                     int64_t R, int64_t K, int64_t ld, int kind,
                                                                     const double* __restrict__ center,
                                                                     double* __restrict__ part) {
    __shared__ double sh[kRedThreads];
    const int64_t total = R * K;
    const double c = (kind == 1) ? center[0] : 0.0;
    double acc = 0.0;
    for (int64_t t = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; t < total; t += (int64_t)kRedBlocks * kRedThreads) {
        const int64_t r = t / K, k = t - r * K;
        const double x = (double)load_elem(X, dt, r * ld + k);
        if (kind == 0) acc += x;
        else if (kind == 1) acc += (x - c) * (x - c);
        else acc += fabs(x);
    }
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// out_kind 0: out_d[slot] = sum/n ; 1: out_d[slot] = sqrt(sum/n) ; 2: out_f[0] = (float)(sum/n)
__global__ __launch_bounds__(kRedThreads) void reduce_final_kernel(const double* __restrict__ part, int nparts,
                                                                   int64_t n, int out_kind, double* out_d, int slot,
                                                                   float* out_f) {
    __shared__ double sh[kRedThreads];
    double acc = 0.0;
    for (int i = threadIdx.x; i < nparts; i += kRedThreads) acc += part[i];
    const double s = block_sum(acc, sh);
    if (threadIdx.x == 0) {
        const double m = n > 0 ? s / (double)n : 0.0;
        if (out_kind == 0) out_d[slot] = m;
        else if (out_kind == 1) out_d[slot] = sqrt(m);
        else out_f[0] = (float)m;
    }
}

size_t reduce_ws(int64_t, int64_t) { return (size_t)kRedBlocks * sizeof(double); }

void launch_stats(const float* S, int64_t R, int64_t K, int64_t lds, double* stats, void* ws, hipStream_t s) {
    double* part = (double*)ws;
    const int64_t n = R * K;
    hipLaunchKernelGGL(reduce_partial_kernel, dim3(kRedBlocks), dim3(kRedThreads), 0, s, (const void*)S, NM_F32, R, K,
                       lds, 0, (const double*)nullptr, part);
    hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(kRedThreads), 0, s, (const double*)part, kRedBlocks, n, 0,
                       stats, 0, (float*)nullptr);
    hipLaunchKernelGGL(reduce_partial_kernel, dim3(kRedBlocks), dim3(kRedThreads), 0, s, (const void*)S, NM_F32, R, K,
                       lds, 1, (const double*)stats, part);
    hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(kRedThreads), 0, s, (const double*)part, kRedBlocks, n, 1,
                       stats, 1, (float*)nullptr);
}

void launch_absmean(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, float* alpha, void* ws,
                    hipStream_t s) {
    double* part = (double*)ws;
    hipLaunchKernelGGL(reduce_partial_kernel, dim3(kRedBlocks), dim3(kRedThreads), 0, s, W, wdt, R, K, ldw, 2,
                       (const double*)nullptr, part);
    hipLaunchKernelGGL(reduce_final_kernel, dim3(1), dim3(kRedThreads), 0, s, (const double*)part, kRedBlocks, R * K,
                       2, (double*)nullptr, 0, alpha);
}

// ------------------------------------------------------------------ gate / anneal
// A thread owns one mask byte: 8 consecutive scores of a row (two 4-groups or
// one 8-group).  For every step it forms the gate, the blend with the hard
// target and the binary-preference term; the block sums that term per step.
__global__ __launch_bounds__(kRedThreads) void gate_kernel(const float* __restrict__ S, int64_t R, int64_t K,
                                                           int64_t lds, const double* __restrict__ stats, int N, int M,
                                                           float T0, float rho, int steps, float* __restrict__ m_final,
                                                           int64_t ldf, uint8_t* __restrict__ hard_mask, int64_t ldm,
                                                           double* __restrict__ part) {
    __shared__ double sh[kRedThreads];
    const double mu = stats[0], sigma = stats[1];
    const int64_t bpr = (K + 7) / 8;
    const int64_t total = R * bpr;
    double lm[kMaxSteps];
    for (int t = 0; t < steps; ++t) lm[t] = 0.0;
    for (int64_t u = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; u < total; u += (int64_t)kRedBlocks * kRedThreads) {
        const int64_t r = u / bpr, b = u - r * bpr;
        const int64_t k0 = b * 8;
        const int ne = (K - k0) < 8 ? (int)(K - k0) : 8;
        float s[8], z[8], key[8];
        for (int i = 0; i < 8; ++i) {
            s[i] = i < ne ? S[r * lds + k0 + i] : 0.f;
            z[i] = sigma > 0.0 ? (float)(((double)s[i] - mu) / sigma) : 0.f;
            key[i] = rank_key(s[i]);
        }
        // hard target h: top-N of the score per group
        uint32_t hbits = 0;
        for (int g = 0; g * M < ne; ++g) {
            float kk[8];
            for (int i = 0; i < M; ++i) kk[i] = key[g * M + i];
            uint32_t gb = 0;
            for (int i = 0; i < M; ++i) {
                int beaten = 0;
                for (int j = 0; j < M; ++j) {
                    if (j == i) continue;
                    beaten += ((j < i) ? (kk[j] >= kk[i]) : (kk[j] > kk[i])) ? 1 : 0;
                }
                if (beaten < N) gb |= 1u << i;
            }
            hbits |= gb << (g * M);
        }
        float m[8];
        for (int t = 0; t < steps; ++t) {
            const float T = T0 * powf(rho, (float)t);
            const float beta = steps > 1 ? (float)t / (float)(steps - 1) : 1.0f;
            double acc = 0.0;
            for (int i = 0; i < ne; ++i) {
                const float g = 1.0f / (1.0f + expf(-z[i] / T));
                const float hv = ((hbits >> i) & 1u) ? 1.0f : 0.0f;
                m[i] = (1.0f - beta) * g + beta * hv;
                acc += (double)m[i] * (1.0 - (double)m[i]);
            }
            lm[t] += acc;
        }
        // final projection: top-N of m_{steps-1}
        uint32_t fbits = 0;
        for (int g = 0; g * M < ne; ++g) {
            float kk[8];
            for (int i = 0; i < M; ++i) kk[i] = rank_key(m[g * M + i]);
            uint32_t gb = 0;
            for (int i = 0; i < M; ++i) {
                int beaten = 0;
                for (int j = 0; j < M; ++j) {
                    if (j == i) continue;
                    beaten += ((j < i) ? (kk[j] >= kk[i]) : (kk[j] > kk[i])) ? 1 : 0;
                }
                if (beaten < N) gb |= 1u << i;
            }
            fbits |= gb << (g * M);
        }
        hard_mask[r * ldm + b] = (uint8_t)fbits;
        if (m_final)
            for (int i = 0; i < ne; ++i) m_final[r * ldf + k0 + i] = m[i];
    }
    for (int t = 0; t < steps; ++t) {
        const double v = block_sum(lm[t], sh);
        if (threadIdx.x == 0) part[(int64_t)t * kRedBlocks + blockIdx.x] = v;
    }
}

__global__ __launch_bounds__(kRedThreads) void gate_final_kernel(const double* __restrict__ part, int steps,
                                                                 double* __restrict__ lmid) {
    __shared__ double sh[kRedThreads];
    for (int t = 0; t < steps; ++t) {
        double acc = 0.0;
        for (int i = threadIdx.x; i < kRedBlocks; i += kRedThreads) acc += part[(int64_t)t * kRedBlocks + i];
        const double s = block_sum(acc, sh);
        if (threadIdx.x == 0) lmid[t] = s;
    }
}

size_t gate_ws(int64_t, int64_t, int steps) { return (size_t)kRedBlocks * (size_t)(steps > 0 ? steps : 1) * sizeof(double); }

void launch_gate(const float* S, int64_t R, int64_t K, int64_t lds, const double* stats, int N, int M, float T0,
                 float rho, int steps, float* m_final, int64_t ldf, uint8_t* hard_mask, int64_t ldm, double* lmid,
                 void* ws, hipStream_t s) {
    double* part = (double*)ws;
    hipLaunchKernelGGL(gate_kernel, dim3(kRedBlocks), dim3(kRedThreads), 0, s, S, R, K, lds, stats, N, M, T0, rho,
                       steps, m_final, ldf, hard_mask, ldm, part);
    hipLaunchKernelGGL(gate_final_kernel, dim3(1), dim3(kRedThreads), 0, s, (const double*)part, steps, lmid);
}

}  // namespace nm
