// Per-token quantisation fused with the 6:8 activation lift ("SlideSparse",
// sections 2B-2C: the lift is a pure index remap, done inside the per-token
// quantisation kernel, so that the online step reads the bf16 activation once
// and writes the lifted one-byte codes the sparse product consumes; INT8 and
// FP8 are among the pages' precisions).  Token row m, in f32 (the quotients
// decide the codes):
//   int8: s = max|x| / 127, q = rint(x / s), ties to even;
//   fp8 : s = max|x| / 448, q = the OCP e4m3 code nearest x / s, ties to even;
// a zero row gives s = 0 and codes 0.  With the lift of a (2N-2):2N weight, lifted
// column 4(N-1)g + 4w + l holds the code of column 2Ng + 2w + l (windows at offsets
// 0, 2, .., 2N-4 of each group; for 6:8, 12g + 4w + l from 8g + 2w + l).
//
// One block of 256 threads per token row: pass 1 takes the absolute maximum over 16-byte
// loads of 8 columns and keeps up to 8 of them per thread in registers (K <= 16384 in one
// pass; longer rows re-read the rest, which is L2-resident by then); the maximum is reduced
// across the wave and then across the block's four waves; pass 2 rounds and writes each
// 8-column group as 12 lifted bytes (three dwords; 6:8) or, without the lift, 8 bytes.
// For other N, pass 2 takes one window per thread: its 4 columns (two column pairs from the
// row, L2-resident by then), rounded and written as one dword of the lifted row.
#include "nm_internal.h"

namespace nm {

constexpr int kQuantThreads = 256;   // one token row per block
constexpr int kQuantCache = 8;       // 8-column groups per thread kept in registers

// OCP e4m3 code of v, |v| <= 448, finite: nearest code, ties to even.  The f32
// exponent E picks the binade; (fraction - 1) * 8 and v * 2^9 are exact, so one
// rint per value gives round-half-even, and a mantissa that rounds up to 8 carries
// into the exponent field as the code arithmetic requires.  -0 keeps its sign.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const int E = (int)((bits >> 23) & 0xffu) - 127;
    uint32_t mag;
    if (E < -6) {   // subnormal codes m * 2^-9, m = 0..8 (8 is the smallest normal)
        mag = (uint32_t)rintf(__builtin_bit_cast(float, bits & 0x7fffffffu) * 512.0f);
    } else {
        const float frac = __builtin_bit_cast(float, (bits & 0x7fffffu) | 0x3f800000u);   // in [1, 2)
        mag = (uint32_t)((E + 7) * 8) + (uint32_t)rintf((frac - 1.0f) * 8.0f);
    }
    return sign | mag;
}

// LIFT: 0 no lift, 1 the 6:8 lift (Ns = 4), 2 the lift of any (2N-2):2N (runtime Ns)
template <int LIFT, bool FP8>
__global__ __launch_bounds__(kQuantThreads) void quant_lift_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                   int64_t Mtok, int64_t K, int Ns,
                                                                   int8_t* __restrict__ Xq, int64_t ldq,
                                                                   float* __restrict__ sx) {
    const int lane = threadIdx.x;   // the thread's place in the row
    const int64_t m = blockIdx.x;
    const uint16_t* xr = X + m * ldx;
    const int64_t groups = K / 8;
    uint4 cache[kQuantCache];
    float amax = 0.0f;
    auto absmax8 = [&](const uint4 v) __attribute__((always_inline)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // |bf16| as f32 bits: clear the sign, widen
            amax = fmaxf(amax, __builtin_bit_cast(float, (w[i] & 0x7fffu) << 16));
            amax = fmaxf(amax, __builtin_bit_cast(float, (w[i] >> 16 & 0x7fffu) << 16));
        }
    };
#pragma unroll
    for (int c = 0; c < kQuantCache; ++c) {
        const int64_t g = lane + kQuantThreads * c;
        cache[c] = g < groups ? *(const uint4*)(xr + 8 * g) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kQuantCache; ++c) absmax8(cache[c]);
    for (int64_t g = lane + kQuantThreads * kQuantCache; g < groups; g += kQuantThreads)
        absmax8(*(const uint4*)(xr + 8 * g));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    __shared__ float wmax[kQuantThreads / 64];
    if ((lane & 63) == 0) wmax[lane >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);   // max: order-free
    const float s = __fdiv_rn(amax, FP8 ? 448.0f : 127.0f);
    if (lane == 0) sx[m] = s;

    int8_t* qr = Xq + m * ldq;
    auto code = [&](float x) __attribute__((always_inline)) -> uint32_t {
        if constexpr (FP8) {
            return s > 0.0f ? e4m3_code(fminf(fmaxf(__fdiv_rn(x, s), -448.0f), 448.0f)) : 0u;
        } else {
            float q = 0.0f;
            if (s > 0.0f) q = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.0f), 127.0f);
            return (uint32_t)(int32_t)q & 0xffu;
        }
    };
    if constexpr (LIFT == 2) {
        // one window per lane: columns 2Ng + 2w .. +3 (two aligned column pairs)
        const int64_t wpr = K / (2 * Ns) * (Ns - 1);
        for (int64_t q = lane; q < wpr; q += kQuantThreads) {
            const int64_t g = q / (Ns - 1), w = q - g * (Ns - 1);
            const uint32_t* src = (const uint32_t*)(xr + 2 * Ns * g + 2 * w);
            const uint32_t p0 = src[0], p1 = src[1];
            const uint32_t b0 = code(__builtin_bit_cast(float, (p0 & 0xffffu) << 16));
            const uint32_t b1 = code(__builtin_bit_cast(float, (p0 >> 16) << 16));
            const uint32_t b2 = code(__builtin_bit_cast(float, (p1 & 0xffffu) << 16));
            const uint32_t b3 = code(__builtin_bit_cast(float, (p1 >> 16) << 16));
            *(uint32_t*)(qr + 4 * q) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
        return;
    }
    auto emit = [&](int64_t g, const uint4 v) __attribute__((always_inline)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = code(__builtin_bit_cast(float, ((w[i >> 1] >> (16 * (i & 1))) & 0xffffu) << 16));
        const uint32_t lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
        const uint32_t hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        if constexpr (LIFT == 1) {
            uint32_t* o = (uint32_t*)(qr + 12 * g);   // windows: bytes 0-3, 2-5, 4-7
            o[0] = lo;
            o[1] = (lo >> 16) | (hi << 16);
            o[2] = hi;
        } else {
            *(uint2*)(qr + 8 * g) = make_uint2(lo, hi);
        }
    };
#pragma unroll
    for (int c = 0; c < kQuantCache; ++c) {
        const int64_t g = lane + kQuantThreads * c;
        if (g < groups) emit(g, cache[c]);
    }
    for (int64_t g = lane + kQuantThreads * kQuantCache; g < groups; g += kQuantThreads)
        emit(g, *(const uint4*)(xr + 8 * g));
}

void launch_quant_lift(const void* X, int64_t Mtok, int64_t K, int64_t ldx, int Ns, nm_dtype qdt, void* Xq,
                       int64_t ldq, float* x_scale, hipStream_t s) {
    if (Mtok == 0) return;
    const dim3 g((unsigned)Mtok), b(kQuantThreads);
    const uint16_t* x = (const uint16_t*)X;
    int8_t* q = (int8_t*)Xq;
#define NM_QL(L, F8) hipLaunchKernelGGL((quant_lift_kernel<L, F8>), g, b, 0, s, x, ldx, Mtok, K, Ns, q, ldq, x_scale)
    const int lift = Ns == 0 ? 0 : (Ns == 4 ? 1 : 2);
    if (qdt == NM_FP8) {
        if (lift == 0) NM_QL(0, true);
        else if (lift == 1) NM_QL(1, true);
        else NM_QL(2, true);
    } else {
        if (lift == 0) NM_QL(0, false);
        else if (lift == 1) NM_QL(1, false);
        else NM_QL(2, false);
    }
#undef NM_QL
}

}  // namespace nm
