// Weight-side kernels of the N:M path: curvature column sums, importance
// scores, top-N group masks, packing, the fused score->mask->pack pass and the
// sliding-window (2N-2):2N decomposition.  All of them are bound by HBM
// bandwidth: each weight is read once and its packed form written once.
//
// Sources: "SparseForge" (Methodology 2: s = (H+eps) W^2), "Sparse-BitNet"
// (sections 1-2: N:M groups, magnitude top-N on master weights, quantise then
// mask), "SlideSparse" (section 2A: N-1 width-4 stride-2 windows per 2N group),
// "Sparsity Induction" (section 2C: diagonal Gauss-Newton proxy).
#include <mutex>

#include "nm_internal.h"

namespace nm {

// ------------------------------------------------------------------ generic element access
__device__ __forceinline__ float load_f32(const void* p, nm_dtype dt, int64_t i) {
    switch (dt) {
        case NM_F32: return ((const float*)p)[i];
        case NM_BF16: return bf16_bits_to_f32(((const uint16_t*)p)[i]);
        case NM_I8: return (float)((const int8_t*)p)[i];
        default: return (float)((const int32_t*)p)[i];
    }
}

// dst[j] (vdt) <- src[i] (sdt): same dtype copies bits, f32 -> bf16 rounds to nearest even.
__device__ __forceinline__ void store_conv(void* dst, nm_dtype vdt, int64_t j, const void* src, nm_dtype sdt,
                                           int64_t i) {
    if (vdt == NM_BF16) {
        ((uint16_t*)dst)[j] = (sdt == NM_BF16) ? ((const uint16_t*)src)[i]
                                                : (uint16_t)f32_to_bf16_bits(load_f32(src, sdt, i));
    } else if (vdt == NM_I8 || vdt == NM_FP8) {   // one-byte values are copied as they are
        ((int8_t*)dst)[j] = ((const int8_t*)src)[i];
    } else if (vdt == NM_F32) {
        ((float*)dst)[j] = load_f32(src, sdt, i);
    } else {
        ((int32_t*)dst)[j] = ((const int32_t*)src)[i];
    }
}

__device__ __forceinline__ void store_zero(void* dst, nm_dtype vdt, int64_t j) {
    if (vdt == NM_BF16) ((uint16_t*)dst)[j] = 0;
    else if (vdt == NM_I8 || vdt == NM_FP8) ((int8_t*)dst)[j] = 0;   // FP8 code 0 is +0
    else ((uint32_t*)dst)[j] = 0;
}

// Hessian-aware score with one rounding per operation: t = w*w, u = h+eps, s = u*t.
__device__ __forceinline__ float hess_score(float w, float h, float eps) {
    float t = __fmul_rn(w, w);
    float u = __fadd_rn(h, eps);
    return __fmul_rn(u, t);
}

__device__ __forceinline__ float score_at(const void* W, nm_dtype wdt, int64_t woff, const float* H, int64_t hoff,
                                          float eps, nm_score_mode mode) {
    float w = load_f32(W, wdt, woff);
    return mode == NM_SCORE_MAGNITUDE ? fabsf(w) : hess_score(w, H[hoff], eps);
}

// Runtime-M top-N bits (M <= 16) with the same rule as topn_bits<M>.
__device__ __forceinline__ uint32_t topn_bits_rt(const float* k, int M, int N) {
    uint32_t bits = 0;
    for (int i = 0; i < M; ++i) {
        int beaten = 0;
        for (int j = 0; j < M; ++j) {
            if (j == i) continue;
            beaten += ((j < i) ? (k[j] >= k[i]) : (k[j] > k[i])) ? 1 : 0;
        }
        if (beaten < N) bits |= 1u << i;
    }
    return bits;
}

__device__ __forceinline__ uint32_t mask_bits_at(const uint8_t* mask, int64_t ldm, int64_t r, int64_t k0, int M) {
    uint32_t b = 0;
    for (int i = 0; i < M; ++i) {
        int64_t k = k0 + i;
        b |= (uint32_t)((mask[r * ldm + (k >> 3)] >> (k & 7)) & 1u) << i;
    }
    return b;
}

// ------------------------------------------------------------------ A1: colsumsq
// One launch, no workspace.  A block owns CG column groups of 16 bytes (64 bf16 or 32
// fp32 columns) over all rows: lane (cg, rl) walks rows rl, rl + 32, ... with eight
// 16-byte loads in flight, then the 32 row-lane partials of each column are summed in
// row-lane order through LDS, so the result does not depend on scheduling.  Squares of
// bf16 or f32 values are exact in f64 and the sums are kept in f64 (exact for bf16 data of
// moderate range); the column sum is rounded to f32 once at the end.
constexpr int kColCG = 8, kColRL = 32;

template <typename T>
__global__ __launch_bounds__(256) void colsumsq_kernel(const T* __restrict__ X, int64_t n, int64_t K, int64_t ldx,
                                                       float* __restrict__ H) {
    constexpr int VEC = 16 / sizeof(T), CG = kColCG, RL = kColRL, U = 8;
    __shared__ double red[RL][CG * VEC + 1];
    const int cg = threadIdx.x % CG, rl = threadIdx.x / CG;
    const int64_t c0 = (int64_t)blockIdx.x * CG * VEC + cg * VEC;
    double acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0;
    auto add = [&](const uint4& q) __attribute__((always_inline)) {
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            float x;
            if constexpr (sizeof(T) == 2) x = bf16_bits_to_f32((u[v >> 1] >> (16 * (v & 1))) & 0xffffu);
            else x = __uint_as_float(u[v]);
            const double xd = (double)x;
            acc[v] = __fma_rn(xd, xd, acc[v]);   // the square is exact: one rounding, the sum's
        }
    };
    if (c0 < K) {
        int64_t r = rl;
        for (; r + (U - 1) * RL < n; r += U * RL) {
            uint4 q[U];
#pragma unroll
            for (int u = 0; u < U; ++u) q[u] = *(const uint4*)(X + (r + u * RL) * ldx + c0);
#pragma unroll
            for (int u = 0; u < U; ++u) add(q[u]);
        }
        for (; r < n; r += RL) add(*(const uint4*)(X + r * ldx + c0));
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[rl][cg * VEC + v] = acc[v];
    __syncthreads();
    if (threadIdx.x < CG * VEC) {
        const int64_t col = (int64_t)blockIdx.x * CG * VEC + threadIdx.x;
        if (col < K) {
            double s = 0.0;
            for (int i = 0; i < RL; ++i) s += red[i][threadIdx.x];
            H[col] = (float)s;
        }
    }
}

size_t colsumsq_ws(int64_t, int64_t) { return 0; }

void launch_colsumsq(const void* X, nm_dtype xdt, int64_t n, int64_t K, int64_t ldx, float* H, void*, hipStream_t s) {
    if (K == 0) return;
    if (xdt == NM_BF16)
        hipLaunchKernelGGL(colsumsq_kernel<uint16_t>, dim3((unsigned)ceil_div(K, kColCG * 8)), dim3(256), 0, s,
                           (const uint16_t*)X, n, K, ldx, H);
    else
        hipLaunchKernelGGL(colsumsq_kernel<float>, dim3((unsigned)ceil_div(K, kColCG * 4)), dim3(256), 0, s,
                           (const float*)X, n, K, ldx, H);
}

// ------------------------------------------------------------------ A3: score
__global__ __launch_bounds__(256) void score_kernel(const void* __restrict__ W, nm_dtype wdt, int64_t R, int64_t K,
                                                    int64_t ldw, const float* __restrict__ H, int64_t ldh, float eps,
                                                    nm_score_mode mode, float* __restrict__ S, int64_t lds) {
    const int64_t total = R * K;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / K, k = t - r * K;
        S[r * lds + k] = score_at(W, wdt, r * ldw + k, H, r * ldh + k, eps, mode);
    }
}

// bf16 fast path: lane = 8 consecutive weights of PR rows (16-byte loads, all PR rows'
// loads issued first), two 16-byte stores of S per row.
constexpr int kScoreRows = 4;

template <bool HESS, bool HFULL>
__global__ __launch_bounds__(256) void score8_kernel(const uint16_t* __restrict__ W, int64_t ldw,
                                                     const float* __restrict__ H, int64_t ldh, float eps, int64_t R,
                                                     int64_t K, float* __restrict__ S, int64_t lds, int64_t row_base) {
    constexpr int PR = kScoreRows;
    const int64_t k0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (k0 >= K) return;
    const int64_t r0 = row_base + (int64_t)blockIdx.y * PR;
    uint4 wq[PR];
    float4 hq[PR][2];
#pragma unroll
    for (int p = 0; p < PR; ++p) {
        const int64_t r = r0 + p < R ? r0 + p : R - 1;
        wq[p] = *(const uint4*)(W + r * ldw + k0);
        if constexpr (HESS) {
            if (HFULL || p == 0) {
                const float* hp = H + (HFULL ? r * ldh : 0) + k0;
                hq[p][0] = *(const float4*)hp;
                hq[p][1] = *(const float4*)(hp + 4);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < PR; ++p) {
        const int64_t r = r0 + p;
        if (r >= R) break;
        const uint32_t u[4] = {wq[p].x, wq[p].y, wq[p].z, wq[p].w};
        float o[8];
        const float4 h0 = HESS ? hq[HFULL ? p : 0][0] : float4{}, h1 = HESS ? hq[HFULL ? p : 0][1] : float4{};
        const float h[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float w = bf16_bits_to_f32((u[i >> 1] >> (16 * (i & 1))) & 0xffffu);
            o[i] = HESS ? hess_score(w, h[i], eps) : fabsf(w);
        }
        *(float4*)(S + r * lds + k0) = make_float4(o[0], o[1], o[2], o[3]);
        *(float4*)(S + r * lds + k0 + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
}

void launch_score(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const float* H, int64_t ldh,
                  float eps, nm_score_mode mode, float* S, int64_t lds, hipStream_t s) {
    const int64_t total = R * K;
    if (total == 0) return;
    const bool hess = mode == NM_SCORE_HESSIAN;
    if (wdt == NM_BF16 && (K % 8) == 0 && (((uintptr_t)W) & 15) == 0 && (ldw % 8) == 0 && (((uintptr_t)S) & 15) == 0 &&
        (lds % 4) == 0 && (!hess || ((((uintptr_t)H) & 15) == 0 && (ldh % 4) == 0))) {
        constexpr int64_t kRowsPerLaunch = 65535LL * kScoreRows;
        for (int64_t rb = 0; rb < R; rb += kRowsPerLaunch) {
            const int64_t nr = R - rb < kRowsPerLaunch ? R - rb : kRowsPerLaunch;
            const dim3 g((unsigned)ceil_div(K, 256 * 8), (unsigned)ceil_div(nr, kScoreRows)), b(256);
            if (!hess)
                hipLaunchKernelGGL((score8_kernel<false, false>), g, b, 0, s, (const uint16_t*)W, ldw, H, ldh, eps, R,
                                   K, S, lds, rb);
            else if (ldh)
                hipLaunchKernelGGL((score8_kernel<true, true>), g, b, 0, s, (const uint16_t*)W, ldw, H, ldh, eps, R, K,
                                   S, lds, rb);
            else
                hipLaunchKernelGGL((score8_kernel<true, false>), g, b, 0, s, (const uint16_t*)W, ldw, H, ldh, eps, R,
                                   K, S, lds, rb);
        }
        return;
    }
    hipLaunchKernelGGL(score_kernel, dim3(grid_cap(ceil_div(total, 256), 8192)), dim3(256), 0, s, W, wdt, R, K, ldw,
                       H, ldh, eps, mode, S, lds);
}

// ------------------------------------------------------------------ A7: mask
// One thread per mask byte (8 consecutive weights: two 4-groups or one 8-group).
__global__ __launch_bounds__(256) void mask_kernel(const float* __restrict__ S, int64_t R, int64_t K, int64_t lds,
                                                   int N, int M, uint8_t* __restrict__ mask, int64_t ldm) {
    const int64_t bpr = ceil_div(K, 8);
    const int64_t total = R * bpr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / bpr, b = t - r * bpr;
        const int64_t k0 = b * 8;
        uint32_t byte = 0;
        for (int g = 0; g < 8 / M; ++g) {
            const int64_t kg = k0 + g * M;
            if (kg >= K) break;
            float key[8];
            for (int i = 0; i < M; ++i) key[i] = rank_key(S[r * lds + kg + i]);
            byte |= topn_bits_rt(key, M, N) << (g * M);
        }
        mask[r * ldm + b] = (uint8_t)byte;
    }
}

void launch_mask(const float* S, int64_t R, int64_t K, int64_t lds, int N, int M, uint8_t* mask, int64_t ldm,
                 hipStream_t s) {
    const int64_t total = R * ceil_div(K, 8);
    if (total == 0) return;
    hipLaunchKernelGGL(mask_kernel, dim3(grid_cap(ceil_div(total, 256), 8192)), dim3(256), 0, s, S, R, K, lds, N, M,
                       mask, ldm);
}

// ------------------------------------------------------------------ A8: pack (generic N:M)
// A thread owns G consecutive groups of a row, G chosen so the chunk's index
// bits fill whole 32-bit words; it streams its fields LSB-first into words.
struct BitWriter {
    uint64_t acc = 0;
    int nbits = 0;
    uint32_t* out;
    __device__ BitWriter(uint32_t* o) : out(o) {}
    __device__ __forceinline__ void put(uint32_t v, int b) {
        acc |= (uint64_t)v << nbits;
        nbits += b;
        if (nbits >= 32) {
            *out++ = (uint32_t)acc;
            acc >>= 32;
            nbits -= 32;
        }
    }
    __device__ __forceinline__ void flush() {
        if (nbits > 0) *out++ = (uint32_t)acc;
        acc = 0;
        nbits = 0;
    }
};

// Streams mask bits LSB-first into whole bytes (chunks start on a byte boundary).
struct MaskWriter {
    uint32_t acc = 0;
    int nbits = 0;
    uint8_t* out;
    __device__ MaskWriter(uint8_t* o) : out(o) {}
    __device__ __forceinline__ void put(uint32_t v, int b) {
        if (!out) return;
        acc |= v << nbits;
        nbits += b;
        while (nbits >= 8) {
            *out++ = (uint8_t)acc;
            acc >>= 8;
            nbits -= 8;
        }
    }
    __device__ __forceinline__ void flush() {
        if (out && nbits > 0) *out++ = (uint8_t)acc;
        acc = 0;
        nbits = 0;
    }
};

inline int gcd_i(int a, int b) { return b == 0 ? a : gcd_i(b, a % b); }

// Select positions for one group: the first N set bits ascending, padded with
// the smallest unset positions; returns them ascending in pos[], and whether
// each carries a real value in real[] (bitmask).
__device__ __forceinline__ uint32_t select_positions(uint32_t bits, int M, int N, int* pos) {
    uint32_t chosen = 0, real = 0;
    int cnt = 0;
    for (int i = 0; i < M && cnt < N; ++i)
        if ((bits >> i) & 1u) { chosen |= 1u << i; real |= 1u << i; ++cnt; }
    for (int i = 0; i < M && cnt < N; ++i)
        if (!((chosen >> i) & 1u)) { chosen |= 1u << i; ++cnt; }
    int c = 0;
    for (int i = 0; i < M; ++i)
        if ((chosen >> i) & 1u) pos[c++] = i;
    return real;
}

// mode_sel: 0 = bits from mask_in; 1 = select from score of Wsc.
__global__ __launch_bounds__(256) void pack_generic_kernel(
    int mode_sel, const void* __restrict__ Wsc, nm_dtype sdt, int64_t ldsc, const float* __restrict__ H, int64_t ldh,
    float eps, nm_score_mode smode, const uint8_t* __restrict__ mask_in, uint8_t* __restrict__ mask_out, int64_t ldm,
    const void* __restrict__ Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K, int N, int M, int G, nm_dtype vdt,
    void* __restrict__ vals, int64_t ldv, uint32_t* __restrict__ idx, int64_t ldi) {
    const int b = (M == 4) ? 2 : 3;
    const int64_t groups = K / M;
    const int64_t cpr = ceil_div(groups, G);
    const int64_t total = R * cpr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / cpr, c = t - r * cpr;
        const int64_t g0 = c * G;
        const int64_t g1 = g0 + G < groups ? g0 + G : groups;
        BitWriter bw(idx + r * ldi + (g0 * N * b) / 32);
        MaskWriter mw(mode_sel ? (mask_out ? mask_out + r * ldm + (g0 * M) / 8 : nullptr) : nullptr);
        for (int64_t g = g0; g < g1; ++g) {
            const int64_t k0 = g * M;
            uint32_t bits;
            if (mode_sel == 0) {
                bits = mask_bits_at(mask_in, ldm, r, k0, M);
            } else {
                float key[8];
                for (int i = 0; i < M; ++i)
                    key[i] = rank_key(score_at(Wsc, sdt, r * ldsc + k0 + i, H, r * ldh + k0 + i, eps, smode));
                bits = topn_bits_rt(key, M, N);
                mw.put(bits, M);
            }
            int pos[8];
            const uint32_t real = select_positions(bits, M, N, pos);
            for (int j = 0; j < N; ++j) {
                const int64_t slot = g * N + j;
                if ((real >> pos[j]) & 1u) store_conv(vals, vdt, r * ldv + slot, Wv, wdt, r * ldwv + k0 + pos[j]);
                else store_zero(vals, vdt, r * ldv + slot);
                bw.put((uint32_t)pos[j], b);
            }
        }
        bw.flush();
        mw.flush();
    }
}

static int pack_chunk_groups(int N, int M) {
    const int b = index_bits(M);
    int G = 32 / gcd_i(N * b, 32);
    if (M == 4 && (G & 1)) G *= 2;  // keep 4-groups paired so mask bytes are owned by one thread
    return G;
}


// ------------------------------------------------------------------ fused 2:4 fast path
// Lane = 8 consecutive weights (two 4-groups) of PR rows; a quad of lanes = 32 weights =
// one 32-bit index word, assembled across the quad with two xor-shuffles.  Block
// (256 lanes) = 2048 columns x PR rows: the PR rows' loads are all issued before any
// selection, and the curvature H (one row, shared by all rows) is read once per lane.
// The lane writes its 4 kept values (8 bytes) and its mask byte directly.
// rows per thread: 2 measured faster than 1, 4 and 8 (28672 x 8192 from a mask: 132 us
// with 4, 127 with 2; 11008 x 4096 fused: 31.1 -> 30.1 us)
constexpr int kPP24Rows = 2;

// FM: the kept positions come from the mask (input) instead of the score: per group
// the first two set bits ascending, padded with the smallest unset positions (value 0).
template <typename TW, bool HESS, bool HFULL, bool FM = false>
__global__ __launch_bounds__(256) void prune_pack24_kernel(const TW* __restrict__ W, int64_t ldw,
                                                           const float* __restrict__ H, int64_t ldh, float eps,
                                                           int64_t R, int64_t K, uint8_t* __restrict__ mask,
                                                           int64_t ldm, uint16_t* __restrict__ vals, int64_t ldv,
                                                           uint32_t* __restrict__ idx, int64_t ldi, int64_t row_base) {
    constexpr int PR = kPP24Rows;
    const int q = threadIdx.x & 3;
    // a quad's mask bytes are one aligned word when the mask rows are word-aligned and the
    // quad's 32 columns lie inside the row
    const bool mask_words = (((uintptr_t)mask & 3u) == 0) && (ldm % 4) == 0 && (K % 32) == 0;
    const int64_t k0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    const int64_t r0 = row_base + (int64_t)blockIdx.y * PR;
    const bool col_ok = k0 < K;
    // the values' bf16 bit patterns as loaded (two per word, the lower column in the low
    // half), and their f32 values for the score
    uint32_t wu[PR][4];
    float w[PR][8];
    uint32_t mbin[PR];   // FM: the input mask byte of each row
#pragma unroll
    for (int p = 0; p < PR; ++p) {
        const int64_t r = r0 + p < R ? r0 + p : R - 1;   // rows past the end re-read the last row, never stored
        const int64_t kc = col_ok ? k0 : 0;
        if constexpr (FM) mbin[p] = mask[r * ldm + (kc >> 3)];
        if constexpr (sizeof(TW) == 2) {
            const uint4 v = *(const uint4*)(W + r * ldw + kc);
            wu[p][0] = v.x; wu[p][1] = v.y; wu[p][2] = v.z; wu[p][3] = v.w;
        } else {
            const float4 a = *(const float4*)(W + r * ldw + kc);
            const float4 c = *(const float4*)(W + r * ldw + kc + 4);
            w[p][0] = a.x; w[p][1] = a.y; w[p][2] = a.z; w[p][3] = a.w;
            w[p][4] = c.x; w[p][5] = c.y; w[p][6] = c.z; w[p][7] = c.w;
        }
    }
    float hsh[8];
    if constexpr (HESS && !HFULL) {
        const float* hp = H + (col_ok ? k0 : 0);
        const float4 h0 = *(const float4*)hp;
        const float4 h1 = *(const float4*)(hp + 4);
        hsh[0] = h0.x; hsh[1] = h0.y; hsh[2] = h0.z; hsh[3] = h0.w;
        hsh[4] = h1.x; hsh[5] = h1.y; hsh[6] = h1.z; hsh[7] = h1.w;
    }
#pragma unroll
    for (int p = 0; p < PR; ++p) {
        const int64_t r = r0 + p;
        if constexpr (sizeof(TW) == 2) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                w[p][i] = __uint_as_float((i & 1) ? (wu[p][i >> 1] & 0xffff0000u) : (wu[p][i >> 1] << 16));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) wu[p][j] = f32_to_bf16_bits(w[p][2 * j]) | (f32_to_bf16_bits(w[p][2 * j + 1]) << 16);
        }
        float key[8];
        if constexpr (FM) {
#pragma unroll
            for (int i = 0; i < 8; ++i) key[i] = 0.f;
        } else if constexpr (HESS) {
            float h[8];
            if constexpr (HFULL) {
                const float* hp = H + (r < R ? r : R - 1) * ldh + (col_ok ? k0 : 0);
                const float4 h0 = *(const float4*)hp;
                const float4 h1 = *(const float4*)(hp + 4);
                h[0] = h0.x; h[1] = h0.y; h[2] = h0.z; h[3] = h0.w;
                h[4] = h1.x; h[5] = h1.y; h[6] = h1.z; h[7] = h1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) h[i] = hsh[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) key[i] = rank_key(hess_score(w[p][i], h[i], eps));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) key[i] = rank_key(fabsf(w[p][i]));
        }
        uint32_t packed[2];
        uint32_t mbyte = 0, nib = 0;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            uint32_t bits, real;
            if constexpr (FM) {
                const uint32_t b4 = (mbin[p] >> (4 * gi)) & 0xFu;
                const uint32_t s1 = b4 & (0u - b4), s2 = (b4 ^ s1) & (0u - (b4 ^ s1));
                real = s1 | s2;                                   // first two set bits
                const uint32_t f = ~real & 0xFu, f1 = f & (0u - f), f2 = (f ^ f1) & (0u - (f ^ f1));
                const int have = (s1 != 0) + (s2 != 0);
                bits = real | (have < 2 ? f1 : 0u) | (have < 1 ? f2 : 0u);
            } else {
                const float kk[4] = {key[4 * gi], key[4 * gi + 1], key[4 * gi + 2], key[4 * gi + 3]};
                bits = top2of4_bits(kk);
                real = bits;
            }
            // exactly two bits: the kept positions p0 < p1; their 16-bit values are bytes
            // 2p, 2p+1 of the group's 8 bytes, picked by one byte permute (selector 12 gives
            // a zero byte: the value of a padded slot)
            const uint32_t p0 = __builtin_ctz(bits);
            const uint32_t p1 = 31u - __builtin_clz(bits);
            uint32_t s0 = 0x0100u + p0 * 0x0202u, s1 = 0x0100u + p1 * 0x0202u;
            if constexpr (FM) {
                s0 = ((real >> p0) & 1u) ? s0 : 0x0c0cu;
                s1 = ((real >> p1) & 1u) ? s1 : 0x0c0cu;
            }
            packed[gi] = __builtin_amdgcn_perm(wu[p][2 * gi + 1], wu[p][2 * gi], s0 | (s1 << 16));
            mbyte |= bits << (4 * gi);
            nib |= (p0 | (p1 << 2)) << (4 * gi);
        }
        const bool ok = col_ok && r < R;
        if (ok) {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u32x2_t{packed[0], packed[1]}, (u32x2_t*)(vals + r * ldv + (k0 >> 1)));
        }
        // the quad's four index bytes and four mask bytes are gathered into one word each
        // (lane q's byte at bits 8q) and stored by lane 0 of the quad
        uint32_t v = ok ? nib << (8 * q) : 0u;
        v |= (uint32_t)__shfl_xor((int)v, 1);
        v |= (uint32_t)__shfl_xor((int)v, 2);
        if (q == 0 && ok) __builtin_nontemporal_store(v, idx + r * ldi + (k0 >> 5));
        if constexpr (!FM) {
            if (mask) {
                uint32_t mw = ok ? mbyte << (8 * q) : 0u;
                mw |= (uint32_t)__shfl_xor((int)mw, 1);
                mw |= (uint32_t)__shfl_xor((int)mw, 2);
                if (mask_words) {
                    if (q == 0 && ok) __builtin_nontemporal_store(mw, (uint32_t*)(mask + r * ldm + (k0 >> 3)));
                } else if (ok) {
                    mask[r * ldm + (k0 >> 3)] = (uint8_t)mbyte;
                }
            }
        }
    }
}

// ------------------------------------------------------------------ pattern check of a caller's mask
// Groups of G consecutive mask bits of a row (G = M, or 2N for the slide; G <= 16) with
// more than cap set bits: an N:M group holds at most N nonzeros ("Sparse-BitNet",
// section 1), N-1 windows at most 2N-2 ("SlideSparse", section 2A), and the packers keep
// only the first cap of them.  One thread per group; a group's bits span at most three
// bytes, all inside the row's ceil(K/8).  The count lands in a per-device counter that
// only the validating calls use (serialised by the host, which reads it back).
__device__ unsigned long long g_overfull;

__global__ void overfull_reset_kernel() { g_overfull = 0ull; }

__global__ __launch_bounds__(256) void overfull_kernel(const uint8_t* __restrict__ mask, int64_t ldm, int64_t R,
                                                       int64_t K, int G, int cap) {
    const int64_t gpr = K / G, total = R * gpr;
    uint32_t cnt = 0;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total; u += (int64_t)gridDim.x * 256) {
        const int64_t r = u / gpr, g = u - r * gpr;
        const int64_t b0 = g * G, byte0 = b0 >> 3;
        const int sh = (int)(b0 & 7), nb = (sh + G + 7) >> 3;
        const uint8_t* row = mask + r * ldm + byte0;
        uint32_t w = 0;
        for (int i = 0; i < nb; ++i) w |= (uint32_t)row[i] << (8 * i);
        cnt += __popc((w >> sh) & ((1u << G) - 1u)) > cap ? 1u : 0u;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(&g_overfull, (unsigned long long)cnt);
}

nm_status count_overfull(const uint8_t* mask, int64_t ldm, int64_t R, int64_t K, int G, int cap, hipStream_t s,
                         int64_t* bad) {
    static std::mutex mu;   // one validating call per process at a time: they share the counter
    std::lock_guard<std::mutex> lock(mu);
    hipLaunchKernelGGL(overfull_reset_kernel, dim3(1), dim3(1), 0, s);
    const int64_t groups = R * (K / G);
    hipLaunchKernelGGL(overfull_kernel, dim3(grid_cap(ceil_div(groups, 256), 4096)), dim3(256), 0, s, mask, ldm, R, K,
                       G, cap);
    nm_status st = check_launch("pattern check");
    if (st != NM_OK) return st;
    unsigned long long n = 0;
    hipError_t e = hipMemcpyFromSymbolAsync(&n, HIP_SYMBOL(g_overfull), sizeof(n), 0, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return set_error(NM_ERR_DEVICE, "pattern check: %s", hipGetErrorString(e));
    *bad = (int64_t)n;
    return NM_OK;
}

void launch_pack(const void* W, nm_dtype wdt, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask, int64_t ldm,
                 int N, int M, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx, int64_t ldi, hipStream_t s) {
    const int64_t vec = wdt == NM_F32 ? 4 : 8;
    const bool fast = N == 2 && M == 4 && vdt == NM_BF16 && (wdt == NM_BF16 || wdt == NM_F32) && (K % 8) == 0 &&
                      (((uintptr_t)W) & 15) == 0 && (ldw % vec) == 0 && (((uintptr_t)vals) & 7) == 0 && (ldv % 4) == 0;
    if (fast) {
        if (R == 0 || K == 0) return;
        constexpr int64_t kRowsPerLaunch = 65535LL * kPP24Rows;  // grid.y limit
        for (int64_t rb = 0; rb < R; rb += kRowsPerLaunch) {
            const int64_t nr = R - rb < kRowsPerLaunch ? R - rb : kRowsPerLaunch;
            const dim3 g((unsigned)ceil_div(K, 256 * 8), (unsigned)ceil_div(nr, kPP24Rows)), b(256);
            if (wdt == NM_BF16)
                hipLaunchKernelGGL((prune_pack24_kernel<uint16_t, false, false, true>), g, b, 0, s, (const uint16_t*)W,
                                   ldw, (const float*)nullptr, (int64_t)0, 0.f, R, K, (uint8_t*)mask, ldm,
                                   (uint16_t*)vals, ldv, idx, ldi, rb);
            else
                hipLaunchKernelGGL((prune_pack24_kernel<float, false, false, true>), g, b, 0, s, (const float*)W, ldw,
                                   (const float*)nullptr, (int64_t)0, 0.f, R, K, (uint8_t*)mask, ldm, (uint16_t*)vals,
                                   ldv, idx, ldi, rb);
        }
        return;
    }
    const int G = pack_chunk_groups(N, M);
    const int64_t total = R * ceil_div(K / M, G);
    if (total == 0) return;
    hipLaunchKernelGGL(pack_generic_kernel, dim3(grid_cap(ceil_div(total, 256), 8192)), dim3(256), 0, s, 0,
                       (const void*)nullptr, NM_F32, (int64_t)0, (const float*)nullptr, (int64_t)0, 0.f,
                       NM_SCORE_MAGNITUDE, mask, (uint8_t*)nullptr, ldm, W, wdt, ldw, R, K, N, M, G, vdt, vals, ldv,
                       idx, ldi);
}

void launch_prune_pack(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh, float eps,
                       nm_score_mode mode, const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K, int N,
                       int M, uint8_t* mask, int64_t ldm, nm_dtype vdt, void* vals, int64_t ldv, uint32_t* idx,
                       int64_t ldi, hipStream_t s) {
    const bool fast = (N == 2 && M == 4 && Wsc == Wv && sdt == wdt && ldsc == ldwv && vdt == NM_BF16 &&
                       (sdt == NM_BF16 || sdt == NM_F32) && (K % 8) == 0);
    if (fast) {
        if (R == 0 || K == 0) return;
        const bool hess = mode == NM_SCORE_HESSIAN, hfull = ldh != 0;
        constexpr int64_t kRowsPerLaunch = 65535LL * kPP24Rows;  // grid.y limit
        for (int64_t rb = 0; rb < R; rb += kRowsPerLaunch) {
            const int64_t nr = R - rb < kRowsPerLaunch ? R - rb : kRowsPerLaunch;
            const dim3 g((unsigned)ceil_div(K, 256 * 8), (unsigned)ceil_div(nr, kPP24Rows)), b(256);
#define NM_PP24(TW, HS, HF)                                                                                    \
    hipLaunchKernelGGL((prune_pack24_kernel<TW, HS, HF>), g, b, 0, s, (const TW*)Wv, ldwv, H, ldh, eps, R, K, \
                       mask, ldm, (uint16_t*)vals, ldv, idx, ldi, rb)
            if (sdt == NM_BF16) {
                if (!hess) NM_PP24(uint16_t, false, false);
                else if (hfull) NM_PP24(uint16_t, true, true);
                else NM_PP24(uint16_t, true, false);
            } else {
                if (!hess) NM_PP24(float, false, false);
                else if (hfull) NM_PP24(float, true, true);
                else NM_PP24(float, true, false);
            }
#undef NM_PP24
        }
        return;
    }
    const int G = pack_chunk_groups(N, M);
    const int64_t total = R * ceil_div(K / M, G);
    if (total == 0) return;
    hipLaunchKernelGGL(pack_generic_kernel, dim3(grid_cap(ceil_div(total, 256), 8192)), dim3(256), 0, s, 1, Wsc, sdt,
                       ldsc, H, ldh, eps, mode, (const uint8_t*)nullptr, mask, ldm, Wv, wdt, ldwv, R, K, N, M, G, vdt,
                       vals, ldv, idx, ldi);
}

// ------------------------------------------------------------------ A9: slide decomposition
// A thread owns Gt consecutive 2N-groups of a row (Gt chosen so that the
// chunk's 4 index bits per window fill whole words).  Per group: kept
// positions ascending go to the earliest covering window with a free slot;
// windows are padded with value 0 at their smallest unused positions.
__global__ __launch_bounds__(256) void slide_kernel(int select, const void* __restrict__ Wsc, nm_dtype sdt,
                                                    int64_t ldsc, const float* __restrict__ H, int64_t ldh, float eps,
                                                    nm_score_mode smode, const uint8_t* __restrict__ mask_in,
                                                    uint8_t* __restrict__ mask_out, int64_t ldm,
                                                    const void* __restrict__ Wv, nm_dtype wdt, int64_t ldwv, int64_t R,
                                                    int64_t K, int Ns, int Gt, nm_dtype vdt, void* __restrict__ vals,
                                                    int64_t ldv, uint32_t* __restrict__ idx, int64_t ldi) {
    const int Mg = 2 * Ns, Wn = Ns - 1;
    const int64_t groups = K / Mg;
    const int64_t cpr = ceil_div(groups, Gt);
    const int64_t total = R * cpr;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / cpr, c = t - r * cpr;
        const int64_t g0 = c * Gt;
        const int64_t g1 = g0 + Gt < groups ? g0 + Gt : groups;
        BitWriter bw(idx + r * ldi + (g0 * Wn * 4) / 32);
        MaskWriter mw(select && mask_out ? mask_out + r * ldm + (g0 * Mg) / 8 : nullptr);
        for (int64_t g = g0; g < g1; ++g) {
            const int64_t k0 = g * Mg;
            uint32_t bits;
            if (select) {
                float key[16];
                for (int i = 0; i < Mg; ++i)
                    key[i] = rank_key(score_at(Wsc, sdt, r * ldsc + k0 + i, H, r * ldh + k0 + i, eps, smode));
                bits = topn_bits_rt(key, Mg, Mg - 2);
                mw.put(bits, Mg);
            } else {
                bits = mask_bits_at(mask_in, ldm, r, k0, Mg);
            }
            int wl[8][2];
            int wc[8];
            for (int w = 0; w < Wn; ++w) wc[w] = 0;
            for (int p = 0; p < Mg; ++p) {
                if (!((bits >> p) & 1u)) continue;
                const int wa = p / 2 - 1, wb = p / 2;
                if (wa >= 0 && wa < Wn && wc[wa] < 2) wl[wa][wc[wa]++] = p - 2 * wa;
                else if (wb < Wn && wc[wb] < 2) wl[wb][wc[wb]++] = p - 2 * wb;
            }
            for (int w = 0; w < Wn; ++w) {
                int loc[2], isv[2], cnt = 0;
                for (int q = 0; q < wc[w]; ++q) { loc[cnt] = wl[w][q]; isv[cnt] = 1; ++cnt; }
                for (int l = 0; l < 4 && cnt < 2; ++l) {
                    bool taken = false;
                    for (int q = 0; q < cnt; ++q) taken |= (loc[q] == l);
                    if (!taken) { loc[cnt] = l; isv[cnt] = 0; ++cnt; }
                }
                if (loc[0] > loc[1]) {
                    int tl = loc[0]; loc[0] = loc[1]; loc[1] = tl;
                    int tv = isv[0]; isv[0] = isv[1]; isv[1] = tv;
                }
                const int64_t wg = g * Wn + w;
                for (int j = 0; j < 2; ++j) {
                    const int64_t slot = wg * 2 + j;
                    if (isv[j]) store_conv(vals, vdt, r * ldv + slot, Wv, wdt, r * ldwv + k0 + 2 * w + loc[j]);
                    else store_zero(vals, vdt, r * ldv + slot);
                    bw.put((uint32_t)loc[j], 2);
                }
            }
        }
        bw.flush();
        mw.flush();
    }
}

// 6:8 fast path (Ns = 4, values copied without conversion).  Lane = one 8-group of
// PR rows; its 6 kept positions go to the 3 windows by the same greedy rule as
// slide_kernel, giving 6 values and 12 index bits per group.  The 12-bit fields of
// 8 consecutive groups (96 bits = 3 words) are assembled across the lanes with
// xor-shuffles.  SEL: 0 |W|, 1 Hessian with a row-vector H, 2 Hessian with a full
// H, 3 kept positions from the input mask.
constexpr int kS68Rows = 4;   // 1, 2 and 8 rows per thread measured slower (14336 x 4096: 62, 47, 48 against 43 us)

// The window assignment depends only on the group's 8 keep bits, so it is tabulated
// for all 256 masks at compile time (same greedy rule and zero padding as
// slide_kernel).  Entry: byte-permute selectors that cut each window's two values
// out of the group's raw bits (selector byte 0x0c gives a zero byte), and the
// group's 12 index bits.  bf16: window w reads elements 2w..2w+3 = words w, w+1
// of the group; int8: bytes 2w..2w+3 of the group's 8 bytes.
struct SlideWin {
    int loc[3][2];
    bool val[3][2];
};
constexpr SlideWin slide_windows(uint32_t bits) {
    SlideWin r{};
    int wc[3] = {0, 0, 0}, wl[3][2] = {{0, 0}, {0, 0}, {0, 0}};
    for (int q = 0; q < 8; ++q) {
        if (!((bits >> q) & 1u)) continue;
        const int wa = q / 2 - 1, wb = q / 2;
        if (wa >= 0 && wa < 3 && wc[wa] < 2) {
            wl[wa][wc[wa]] = q - 2 * wa;
            ++wc[wa];
        } else if (wb < 3 && wc[wb] < 2) {
            wl[wb][wc[wb]] = q - 2 * wb;
            ++wc[wb];
        }
    }
    for (int w = 0; w < 3; ++w) {
        int loc[2] = {wl[w][0], wl[w][1]};
        bool isv[2] = {wc[w] > 0, wc[w] > 1};
        int cnt = wc[w];
        for (int l = 0; l < 4 && cnt < 2; ++l) {
            const bool taken = (cnt > 0 && loc[0] == l) || (cnt > 1 && loc[1] == l);
            if (!taken) {
                loc[cnt] = l;
                isv[cnt] = false;
                ++cnt;
            }
        }
        if (loc[0] > loc[1]) {
            const int tl = loc[0]; loc[0] = loc[1]; loc[1] = tl;
            const bool tv = isv[0]; isv[0] = isv[1]; isv[1] = tv;
        }
        r.loc[w][0] = loc[0]; r.loc[w][1] = loc[1];
        r.val[w][0] = isv[0]; r.val[w][1] = isv[1];
    }
    return r;
}
struct SlideLut {
    uint32_t e[256][4];   // bf16: 3 selectors + index bits; int8: sel0 | sel1 << 16, sel2 | bits << 16
};
constexpr SlideLut make_slide_lut(bool bf16) {
    SlideLut t{};
    for (uint32_t m = 0; m < 256; ++m) {
        const SlideWin sw = slide_windows(m);
        uint32_t v12 = 0, sel[3] = {0, 0, 0};
        for (int w = 0; w < 3; ++w) {
            v12 |= (uint32_t)(sw.loc[w][0] | (sw.loc[w][1] << 2)) << (4 * w);
            for (int q = 0; q < 2; ++q) {
                const int p = sw.loc[w][q];
                if (bf16) {
                    const uint32_t b0 = sw.val[w][q] ? (uint32_t)(2 * p) : 0x0cu;
                    const uint32_t b1 = sw.val[w][q] ? (uint32_t)(2 * p + 1) : 0x0cu;
                    sel[w] |= (b0 | (b1 << 8)) << (16 * q);
                } else {
                    const uint32_t b = sw.val[w][q] ? (uint32_t)(2 * w + p) : 0x0cu;
                    sel[w] |= b << (8 * q);
                }
            }
            if (!bf16) sel[w] |= 0x0c0c0000u;
        }
        if (bf16) {
            t.e[m][0] = sel[0]; t.e[m][1] = sel[1]; t.e[m][2] = sel[2]; t.e[m][3] = v12;
        } else {
            t.e[m][0] = (sel[0] & 0xffffu) | (sel[1] << 16);
            t.e[m][1] = (sel[2] & 0xffffu) | (v12 << 16);
            t.e[m][2] = 0; t.e[m][3] = 0;
        }
    }
    return t;
}
__device__ const SlideLut kSlideLutBf16 = make_slide_lut(true);
__device__ const SlideLut kSlideLutI8 = make_slide_lut(false);

template <typename TS, typename TV, int SEL>
__global__ __launch_bounds__(256) void slide68_kernel(const TS* __restrict__ Wsc, int64_t ldsc,
                                                      const float* __restrict__ H, int64_t ldh, float eps,
                                                      const TV* __restrict__ Wv, int64_t ldwv, int64_t R, int64_t K,
                                                      const uint8_t* __restrict__ mask_in, uint8_t* __restrict__ mask_out,
                                                      int64_t ldm, TV* __restrict__ vals, int64_t ldv,
                                                      uint32_t* __restrict__ idx, int64_t ldi, int64_t row_base,
                                                      int gx) {
    // block: gx (256 or 64) consecutive groups of 256 / gx sets of PR rows; 64 when a row's
    // groups would leave most of a 256-wide block idle (6912 x 2560: 320 groups, 27.6 -> 23.4
    // us), 256 otherwise (14336 x 4096: 48.9 us against 52.9 with 64)
    constexpr int PR = kS68Rows;
    const int64_t groups = K / 8;
    const int64_t g = (int64_t)blockIdx.x * gx + (threadIdx.x % gx);
    const bool gok = g < groups;
    const int64_t k0 = (gok ? g : 0) * 8;
    const int64_t r0 = row_base + ((int64_t)blockIdx.y * (256 / gx) + threadIdx.x / gx) * PR;
    const int j8 = threadIdx.x & 7;
    __shared__ uint4 lut[256];
    lut[threadIdx.x] = *(const uint4*)(sizeof(TV) == 2 ? kSlideLutBf16.e[threadIdx.x] : kSlideLutI8.e[threadIdx.x]);
    __syncthreads();
    uint32_t vraw[PR][4];   // the 8 values' bits: bf16 -> 4 words, int8 -> 2 words
    float sc[PR][8];
    uint32_t mb[PR];
#pragma unroll
    for (int p = 0; p < PR; ++p) {
        const int64_t r = r0 + p < R ? r0 + p : R - 1;
        if constexpr (sizeof(TV) == 2) {
            const uint4 q = *(const uint4*)(Wv + r * ldwv + k0);
            vraw[p][0] = q.x; vraw[p][1] = q.y; vraw[p][2] = q.z; vraw[p][3] = q.w;
        } else {
            const uint2 q = *(const uint2*)(Wv + r * ldwv + k0);
            vraw[p][0] = q.x; vraw[p][1] = q.y; vraw[p][2] = 0; vraw[p][3] = 0;
        }
        if constexpr (SEL == 3) {
            mb[p] = mask_in[r * ldm + (k0 >> 3)];
        } else if constexpr (sizeof(TS) == 2) {
            const uint4 q = *(const uint4*)(Wsc + r * ldsc + k0);
            const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) sc[p][i] = bf16_bits_to_f32((u[i >> 1] >> (16 * (i & 1))) & 0xffffu);
        } else {
            const float4 a = *(const float4*)(Wsc + r * ldsc + k0);
            const float4 c = *(const float4*)(Wsc + r * ldsc + k0 + 4);
            sc[p][0] = a.x; sc[p][1] = a.y; sc[p][2] = a.z; sc[p][3] = a.w;
            sc[p][4] = c.x; sc[p][5] = c.y; sc[p][6] = c.z; sc[p][7] = c.w;
        }
    }
    float hrow[8];
    if constexpr (SEL == 1) {
        const float4 h0 = *(const float4*)(H + k0);
        const float4 h1 = *(const float4*)(H + k0 + 4);
        hrow[0] = h0.x; hrow[1] = h0.y; hrow[2] = h0.z; hrow[3] = h0.w;
        hrow[4] = h1.x; hrow[5] = h1.y; hrow[6] = h1.z; hrow[7] = h1.w;
    }
#pragma unroll
    for (int p = 0; p < PR; ++p) {
        const int64_t r = r0 + p;
        const bool ok = gok && r < R;
        uint32_t bits;
        if constexpr (SEL == 3) {
            bits = mb[p];
        } else {
            float h[8];
            if constexpr (SEL == 2) {
                const float* hp = H + (r < R ? r : R - 1) * ldh + k0;
                const float4 h0 = *(const float4*)hp;
                const float4 h1 = *(const float4*)(hp + 4);
                h[0] = h0.x; h[1] = h0.y; h[2] = h0.z; h[3] = h0.w;
                h[4] = h1.x; h[5] = h1.y; h[6] = h1.z; h[7] = h1.w;
            } else if constexpr (SEL == 1) {
#pragma unroll
                for (int i = 0; i < 8; ++i) h[i] = hrow[i];
            }
            float key[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                key[i] = rank_key(SEL == 0 ? fabsf(sc[p][i]) : hess_score(sc[p][i], h[i], eps));
            bits = top6of8_bits(key);
            if (mask_out && ok) mask_out[r * ldm + (k0 >> 3)] = (uint8_t)bits;
        }
        // kept positions ascending -> earliest covering window with a free slot (tabulated)
        const uint4 L = lut[bits & 0xffu];
        uint32_t v12, outv[3];
        if constexpr (sizeof(TV) == 2) {
            outv[0] = __builtin_amdgcn_perm(vraw[p][1], vraw[p][0], L.x);
            outv[1] = __builtin_amdgcn_perm(vraw[p][2], vraw[p][1], L.y);
            outv[2] = __builtin_amdgcn_perm(vraw[p][3], vraw[p][2], L.z);
            v12 = L.w;
        } else {
            outv[0] = __builtin_amdgcn_perm(vraw[p][1], vraw[p][0], (L.x & 0xffffu) | 0x0c0c0000u);
            outv[1] = __builtin_amdgcn_perm(vraw[p][1], vraw[p][0], (L.x >> 16) | 0x0c0c0000u);
            outv[2] = __builtin_amdgcn_perm(vraw[p][1], vraw[p][0], (L.y & 0xffffu) | 0x0c0c0000u);
            v12 = L.y >> 16;
        }
        if (ok) {
            if constexpr (sizeof(TV) == 2) {
                uint32_t* vp = (uint32_t*)(vals + r * ldv + 6 * g);
                vp[0] = outv[0]; vp[1] = outv[1]; vp[2] = outv[2];
            } else {
                uint16_t* vp = (uint16_t*)(vals + r * ldv + 6 * g);
                vp[0] = (uint16_t)outv[0]; vp[1] = (uint16_t)outv[1]; vp[2] = (uint16_t)outv[2];
            }
        }
        // 12 index bits at bit 12*j8 of the cluster's 3 words
        const uint32_t f = ok ? v12 : 0u;
        const int pos = 12 * j8, wd = pos >> 5, sh = pos & 31;
        const uint32_t lo = f << sh, hi = sh > 20 ? f >> (32 - sh) : 0u;
        uint32_t c0 = wd == 0 ? lo : 0u;
        uint32_t c1 = wd == 1 ? lo : (wd == 0 ? hi : 0u);
        uint32_t c2 = wd == 2 ? lo : (wd == 1 ? hi : 0u);
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) {
            c0 |= (uint32_t)__shfl_xor((int)c0, m);
            c1 |= (uint32_t)__shfl_xor((int)c1, m);
            c2 |= (uint32_t)__shfl_xor((int)c2, m);
        }
        if (j8 == 0 && gok && r < R) {
            const int64_t w0 = (g / 8) * 3, nbits = 12 * groups;
            uint32_t* ip = idx + r * ldi + w0;
            ip[0] = c0;
            if (32 * (w0 + 1) < nbits) ip[1] = c1;
            if (32 * (w0 + 2) < nbits) ip[2] = c2;
        }
    }
}

void launch_slide(const void* Wsc, nm_dtype sdt, int64_t ldsc, const float* H, int64_t ldh, float eps,
                  nm_score_mode mode, bool select, const void* Wv, nm_dtype wdt, int64_t ldwv, int64_t R, int64_t K,
                  int Ns, const uint8_t* mask_in, uint8_t* mask_out, int64_t ldm, nm_dtype vdt, void* vals,
                  int64_t ldv, uint32_t* idx, int64_t ldi, hipStream_t s) {
    if (Ns == 4 && (K % 8) == 0 && wdt == vdt && (wdt == NM_BF16 || wdt == NM_I8 || wdt == NM_FP8) &&
        (!select || sdt == NM_BF16 || sdt == NM_F32)) {
        const int64_t ev = wdt == NM_BF16 ? 2 : 1;
        const bool vals_ok = (((uintptr_t)vals) & (ev == 2 ? 3 : 1)) == 0 && (ldv % 2) == 0;
        const bool wv_ok = (((uintptr_t)Wv) & (ev == 2 ? 15 : 7)) == 0 && (ldwv % 8) == 0;
        const bool ws_ok = !select || ((((uintptr_t)Wsc) & 15) == 0 && (ldsc % (sdt == NM_F32 ? 4 : 8)) == 0);
        const bool h_ok = !select || mode == NM_SCORE_MAGNITUDE || ((((uintptr_t)H) & 15) == 0 && (ldh % 4) == 0);
        if (vals_ok && wv_ok && ws_ok && h_ok) {
            if (R == 0 || K == 0) return;
            const int sel = !select ? 3 : (mode == NM_SCORE_MAGNITUDE ? 0 : (ldh ? 2 : 1));
            const int gx = (K / 8) % 256 == 0 || K / 8 > 1024 ? 256 : 64;
            const int64_t rows_per_block = 256 / gx * kS68Rows, kRowsPerLaunch = 65535LL * rows_per_block;
            for (int64_t rb = 0; rb < R; rb += kRowsPerLaunch) {
                const int64_t nr = R - rb < kRowsPerLaunch ? R - rb : kRowsPerLaunch;
                const dim3 g((unsigned)ceil_div(K / 8, gx), (unsigned)ceil_div(nr, rows_per_block)), b(256);
#define NM_S68(TS, TV, SL)                                                                                         \
    hipLaunchKernelGGL((slide68_kernel<TS, TV, SL>), g, b, 0, s, (const TS*)Wsc, ldsc, H, ldh, eps, (const TV*)Wv, \
                       ldwv, R, K, mask_in, mask_out, ldm, (TV*)vals, ldv, idx, ldi, rb, gx)
#define NM_S68_SEL(TS, TV)                          \
    do {                                            \
        if (sel == 0) NM_S68(TS, TV, 0);            \
        else if (sel == 1) NM_S68(TS, TV, 1);       \
        else if (sel == 2) NM_S68(TS, TV, 2);       \
        else NM_S68(TS, TV, 3);                     \
    } while (0)
                if (wdt == NM_BF16) {
                    if (!select || sdt == NM_BF16) NM_S68_SEL(uint16_t, uint16_t);
                    else NM_S68_SEL(float, uint16_t);
                } else {
                    if (!select || sdt == NM_BF16) NM_S68_SEL(uint16_t, int8_t);
                    else NM_S68_SEL(float, int8_t);
                }
#undef NM_S68_SEL
#undef NM_S68
            }
            return;
        }
    }
    // chunk of Gt groups: Gt * (Ns-1) windows * 4 bits must be a multiple of 32,
    // and (for mask bytes written bit by bit) chunks never share a mask byte with
    // another thread: Gt * 2Ns must be a multiple of 8.
    int Gt = 8 / gcd_i(Ns - 1, 8);
    while ((Gt * 2 * Ns) % 8) Gt *= 2;
    const int64_t total = R * ceil_div(K / (2 * Ns), Gt);
    if (total == 0) return;
    hipLaunchKernelGGL(slide_kernel, dim3(grid_cap(ceil_div(total, 256), 8192)), dim3(256), 0, s, select ? 1 : 0, Wsc,
                       sdt, ldsc, H, ldh, eps, mode, mask_in, mask_out, ldm, Wv, wdt, ldwv, R, K, Ns, Gt, vdt, vals,
                       ldv, idx, ldi);
}

}  // namespace nm
