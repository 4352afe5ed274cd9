// Hutchinson estimate of the Hessian diagonal ("SparseForge", Methodology 2:
// the diagonal of the Hessian is estimated with Rademacher probes because the
// full Hessian is prohibitive).  For the layer's quadratic output energy
// L(W) = ||X W^T||_F^2 the Hessian-vector product of a probe V is
// 2 (V X^T) X, so with P probes
//     D = (1/P) sum_p V_p .* (2 (V_p X^T) X).
// Two dense bf16 MFMA GEMMs (v_mfma_f32_32x32x16_bf16, f32 accumulation):
//   gemm1: U_p = V_p X^T  [R, n] for all probes at once (probes stacked along
//          rows), V generated from a counter-based SplitMix64 and never stored
//          (into the LDS stages of the dense split ring, k_spmm.hip, or in
//          registers in hutch_gemm1_kernel below); U is rounded to bf16 into the
//          workspace.
//   gemm2: for a tile of D, loop over probes: G = U_p X (inner dimension n, from
//          a transposed copy of X), then D += V_p .* G with V_p regenerated for
//          the tile; D is written once, scaled by 2/P.  The dense split ring
//          (k_spmm.hip) runs it on 256 x 256 tiles; hutch_gemm2_kernel below (128 x
//          128 tiles) where that does not apply.
// Operand layout (gfx950, verified on hardware): lane l holds A row (l%32),
// K [8(l/32), +8); B column (l%32), K [8(l/32), +8); C column (l%32), rows
// 8(e/4) + 4(l/32) + e%4.
#include "nm_internal.h"

namespace nm {

typedef __bf16 bf16x8_h __attribute__((ext_vector_type(8)));
typedef float f32x16_h __attribute__((ext_vector_type(16)));

constexpr int HT = 128;          // tile rows and columns
constexpr int HK = 64;           // inner step
constexpr int HS = HK * 2 + 16;  // LDS row stride in bytes (128 + pad)



// Stage a [128 x 64] bf16 tile (rows row0.., columns col0..) of a row-major
// matrix into registers: 1024 16-byte chunks, 4 per thread; rows >= nrows load 0.
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ M, int64_t ld, int64_t nrows, int64_t row0,
                                          int64_t col0, uint4 (&r)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int c = threadIdx.x + p * 256;
        const int row = c >> 3, part = c & 7;
        const int64_t gr = row0 + row;
        r[p] = gr < nrows ? *(const uint4*)(M + gr * ld + col0 + part * 8) : make_uint4(0, 0, 0, 0);
    }
}

__device__ __forceinline__ void store_tile(uint8_t* s, const uint4 (&r)[4]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int c = threadIdx.x + p * 256;
        const int row = c >> 3, part = c & 7;
        *(uint4*)(s + row * HS + part * 16) = r[p];
    }
}

// ------------------------------------------------------------------ gemm1: U = V X^T
// grid.x: tiles of 64*SR stacked probe rows, grid.y: tiles of 128 over n.  V is made
// in registers, so only X is loaded; SR row sub-tiles per wave reuse each X fragment
// SR times.
template <int SR>
__global__ __launch_bounds__(256) void hutch_gemm1_kernel(const uint16_t* __restrict__ X, int64_t ldx, int64_t n,
                                                          int64_t K, int64_t R, int P, uint64_t seed,
                                                          uint16_t* __restrict__ U) {
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][HT * HS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wt = wave >> 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t row0 = (int64_t)blockIdx.x * (64 * SR);  // stacked row index p*R + o
    const int64_t col0 = (int64_t)blockIdx.y * HT;          // calibration row i
    const int64_t PR = (int64_t)P * R;
    const int64_t kblocks = K / 64;

    // the SR A sub-tile rows this lane generates
    int pr[SR];
    int64_t orow[SR];
    bool rvalid[SR];
#pragma unroll
    for (int i = 0; i < SR; ++i) {
        const int64_t sr = row0 + (wr * SR + i) * 32 + l32;
        rvalid[i] = sr < PR;
        const int64_t srr = rvalid[i] ? sr : 0;
        pr[i] = (int)(srr / R);
        orow[i] = srr - (int64_t)pr[i] * R;
    }

    f32x16_h acc[SR][2];
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_h{};

    uint4 rb[4];
    const int nsteps = (int)(K / HK);
    load_tile(X, ldx, n, col0, 0, rb);
    store_tile(sB[0], rb);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        const bool more = s + 1 < nsteps;
        if (more) load_tile(X, ldx, n, col0, (int64_t)(s + 1) * HK, rb);
        const uint8_t* b = sB[s & 1];
        uint64_t word[SR];
#pragma unroll
        for (int i = 0; i < SR; ++i) word[i] = rad_word(seed, pr[i], orow[i], s, kblocks);
#pragma unroll
        for (int d = 0; d < HK / 16; ++d) {
            uint4 fb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tok = (wt * 2 + j) * 32 + l32;
                fb[j] = *(const uint4*)(b + tok * HS + d * 32 + h * 16);
            }
#pragma unroll
            for (int i = 0; i < SR; ++i) {
                const uint32_t byte = (uint32_t)(word[i] >> (16 * d + 8 * h)) & 0xffu;
                const bf16x8_h av = __builtin_bit_cast(bf16x8_h, signs_to_bf16x8(byte));
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, __builtin_bit_cast(bf16x8_h, fb[j]),
                                                                        acc[i][j], 0, 0, 0);
            }
        }
        if (more) store_tile(sB[(s + 1) & 1], rb);
        __syncthreads();
    }
    // store U (bf16, round to nearest even): lane holds column i = l32, rows 8(e/4)+4h+e%4
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t ci = col0 + (wt * 2 + j) * 32 + l32;
            if (ci >= n) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t sr = row0 + (wr * SR + i) * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                if (sr < PR) U[sr * n + ci] = (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
            }
        }
}

// ------------------------------------------------------------------ transpose X [n, K] -> XT [K, n]
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ X, int64_t ldx, int64_t n,
                                                        int64_t K, uint16_t* __restrict__ XT) {
    __shared__ uint16_t t[64][65];
    const int64_t i0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;
        const int64_t i = i0 + r, k = k0 + c;
        t[r][c] = (i < n && k < K) ? X[i * ldx + k] : 0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;  // r: k offset, c: i offset
        const int64_t k = k0 + r, i = i0 + c;
        if (k < K && i < n) XT[k * n + i] = t[c][r];
    }
}

// ------------------------------------------------------------------ gemm2: D = (2/P) sum_p V_p .* (U_p X)
// grid.x: tiles over R, grid.y: tiles over K (output columns).  Two blocks per CU (the
// register budget is held to 256 per lane), so one block's tile loads hide behind the
// other's MFMAs.  One flat pipeline over
// (probe, inner step): the next step's tiles (the next probe's first ones at a probe's
// end) are loaded while the current step's MFMAs run.  At each probe's first step the
// block's 256 Rademacher words (128 rows x 2 blocks of 64 columns) are generated once,
// one per thread, into LDS (by probe parity, so that a wave still applying the previous
// probe's signs is never overwritten); the probe's end applies them to G and adds into D.
__global__ __launch_bounds__(256, 2) void hutch_gemm2_kernel(const uint16_t* __restrict__ U, const uint16_t* __restrict__ XT,
                                                          int64_t n, int64_t K, int64_t R, int P, uint64_t seed,
                                                          float* __restrict__ D, int64_t ldd) {
    __shared__ __attribute__((aligned(16))) uint8_t sm[2][2][HT * HS];  // [buf][A|B]
    __shared__ uint64_t sV[2][2 * HT];   // [probe parity][column block][row]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wt = wave >> 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t row0 = (int64_t)blockIdx.x * HT;  // weight row o
    const int64_t col0 = (int64_t)blockIdx.y * HT;  // weight column k
    const int64_t kblocks = K / 64;
    const int nsteps = (int)(n / HK);
    const int total = P * nsteps;

    f32x16_h dacc[2][2], acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            dacc[i][j] = f32x16_h{};
            acc[i][j] = f32x16_h{};
        }

    uint4 ra[4], rb[4];
    auto load = [&](int t) __attribute__((always_inline)) {
        const int p = t / nsteps, s = t - p * nsteps;
        load_tile(U + (int64_t)p * R * n, n, R, row0, (int64_t)s * HK, ra);
        load_tile(XT, n, K, col0, (int64_t)s * HK, rb);
    };
    load(0);
    store_tile(sm[0][0], ra);
    store_tile(sm[0][1], rb);
    for (int t = 0; t < total; ++t) {
        const int p = t / nsteps, s = t - p * nsteps;
        if (s == 0) {   // this probe's sign words (read at its last step, after at least one barrier)
            const int64_t o = row0 + (tid & (HT - 1)), oc = o < R ? o : R - 1;
            const int64_t kb = (col0 >> 6) + (tid >> 7);
            sV[p & 1][tid] = rad_word(seed, p, oc, kb < kblocks ? kb : kblocks - 1, kblocks);
        }
        __syncthreads();
        const bool more = t + 1 < total;
        if (more) load(t + 1);
        const uint8_t* a = sm[t & 1][0];
        const uint8_t* b = sm[t & 1][1];
#pragma unroll
        for (int d = 0; d < HK / 16; ++d) {
            uint4 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = *(const uint4*)(a + ((wr * 2 + i) * 32 + l32) * HS + d * 32 + h * 16);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = *(const uint4*)(b + ((wt * 2 + j) * 32 + l32) * HS + d * 32 + h * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_h, fa[i]),
                                                                        __builtin_bit_cast(bf16x8_h, fb[j]),
                                                                        acc[i][j], 0, 0, 0);
        }
        if (s == nsteps - 1) {
            // D += V_p .* G: lane holds columns k = col0 + wt*64 + j*32 + l32 (one 64-column
            // block per wave column: word block wt, bit j*32 + l32) and rows 8(e/4)+4h+e%4
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int orow = (wr * 2 + i) * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                    const uint64_t w = sV[p & 1][wt * HT + orow];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float g = acc[i][j][e];
                        dacc[i][j][e] += ((w >> (j * 32 + l32)) & 1ull) ? -g : g;
                    }
                }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_h{};
        }
        if (more) {
            store_tile(sm[(t + 1) & 1][0], ra);
            store_tile(sm[(t + 1) & 1][1], rb);
        }
    }
    const float scale = 2.0f / (float)P;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t k = col0 + (wt * 2 + j) * 32 + l32;
            if (k >= K) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t o = row0 + (wr * 2 + i) * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                if (o < R) D[o * ldd + k] = dacc[i][j][e] * scale;
            }
        }
}

size_t hutch_ws(int64_t n, int64_t K, int64_t R, int probes) {
    return (size_t)probes * (size_t)R * (size_t)n * 2 + (size_t)K * (size_t)n * 2;
}

void launch_hutchinson(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes, uint64_t seed,
                       float* D, int64_t ldd, void* ws, hipStream_t s) {
    uint16_t* U = (uint16_t*)ws;
    uint16_t* XT = U + (size_t)probes * (size_t)R * (size_t)n;
    const uint16_t* Xb = (const uint16_t*)X;
    // the dense split ring with the probe rows generated into LDS where it applies, else the
    // register-generating tile kernel
    constexpr int SR1 = 2;   // 128 stacked rows per block (256 measured no faster: the sign generation bounds it)
    if (launch_hutch_u_ring(Xb, ldx, n, K, R, probes, seed, U, s) == NM_ERR_SHAPE)
        hipLaunchKernelGGL(hutch_gemm1_kernel<SR1>, dim3((unsigned)ceil_div((int64_t)probes * R, 64 * SR1), (unsigned)ceil_div(n, HT)),
                           dim3(256), 0, s, Xb, ldx, n, K, R, probes, seed, U);
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)ceil_div(K, 64), (unsigned)ceil_div(n, 64)), dim3(256), 0, s,
                       Xb, ldx, n, K, XT);
    // the dense split ring where it applies (aligned workspace, 32-bit offsets), else 128 x 128 tiles
    if (launch_hutch_ring(U, XT, n, K, R, probes, seed, D, ldd, s, nullptr) == NM_ERR_SHAPE)
        hipLaunchKernelGGL(hutch_gemm2_kernel, dim3((unsigned)ceil_div(R, HT), (unsigned)ceil_div(K, HT)), dim3(256), 0, s,
                           (const uint16_t*)U, (const uint16_t*)XT, n, K, R, probes, seed, D, ldd);
}

// Fused diagonal -> score -> moments: the second product's epilogue writes
// S = (D + eps) W^2 instead of D (same arithmetic as nm_score on the stored D), and the
// per-block moments of S, which the final kernel combines into (mean, std).  Needs the
// dense split ring (checked by the caller): no fallback kernel carries the epilogue.
size_t hutch_score_ws(int64_t n, int64_t K, int64_t R, int probes) {
    const size_t h = (hutch_ws(n, K, R, probes) + 255) & ~(size_t)255;
    return h + (size_t)3 * (size_t)hutch_ring_blocks(K, R) * sizeof(double);
}

nm_status launch_hutchinson_score(const void* X, int64_t n, int64_t K, int64_t ldx, int64_t R, int probes,
                                  uint64_t seed, const uint16_t* W, int64_t ldw, float eps, float* S, int64_t lds,
                                  double* stats, void* ws, hipStream_t s) {
    uint16_t* U = (uint16_t*)ws;
    uint16_t* XT = U + (size_t)probes * (size_t)R * (size_t)n;
    double* mpart = (double*)((uint8_t*)ws + ((hutch_ws(n, K, R, probes) + 255) & ~(size_t)255));
    const uint16_t* Xb = (const uint16_t*)X;
    constexpr int SR1 = 2;
    if (launch_hutch_u_ring(Xb, ldx, n, K, R, probes, seed, U, s) == NM_ERR_SHAPE)
        hipLaunchKernelGGL(hutch_gemm1_kernel<SR1>, dim3((unsigned)ceil_div((int64_t)probes * R, 64 * SR1), (unsigned)ceil_div(n, HT)),
                           dim3(256), 0, s, Xb, ldx, n, K, R, probes, seed, U);
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)ceil_div(K, 64), (unsigned)ceil_div(n, 64)), dim3(256), 0, s,
                       Xb, ldx, n, K, XT);
    const HutchScore sc{W, ldw, eps, mpart};
    const nm_status st = launch_hutch_ring(U, XT, n, K, R, probes, seed, S, lds, s, &sc);
    if (st != NM_OK) return set_error(st, "nm_hutchinson_score: the dense split ring does not apply");
    if (stats) launch_moments_final(mpart, (int)hutch_ring_blocks(K, R), stats, s);
    return check_launch("nm_hutchinson_score");
}

}  // namespace nm
