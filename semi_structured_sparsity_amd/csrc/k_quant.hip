// Per-token quantisation fused with the 6:8 activation lift ("SlideSparse",
// sections 2B-2C: the lift is a pure index remap, done inside the per-token
// quantisation kernel, so that the online step reads the bf16 activation once
// and writes the lifted one-byte codes the sparse product consumes; INT8 and
// FP8 are among the pages' precisions).  Token row m, in f32 (the quotients
// decide the codes):
//   int8: s = max|x| / 127, q = rint(x / s), ties to even;
//   fp8 : s = max|x| / 448, q = the OCP e4m3 code nearest x / s, ties to even;
// a zero row gives s = 0 and codes 0.  With the lift, lifted column 12g + 4w + l
// holds the code of column 8g + 2w + l (windows at offsets 0, 2, 4 of each group).
//
// One wave per token row, four rows per block: pass 1 takes the absolute maximum over
// 16-byte loads of 8 columns and keeps up to 8 of them per lane in registers (K <= 4096
// in one pass; longer rows re-read the rest, which is L2-resident by then); the maximum
// is reduced across the wave; pass 2 rounds and writes each 8-column group as 12 lifted
// bytes (three dwords) or, without the lift, 8 bytes.
#include "nm_internal.h"

namespace nm {

constexpr int kQuantThreads = 256;   // four waves, one token row each
constexpr int kQuantCache = 8;       // 8-column groups per lane kept in registers

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

template <bool LIFT, bool FP8>
__global__ __launch_bounds__(kQuantThreads) void quant_lift_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                   int64_t Mtok, int64_t K, int8_t* __restrict__ Xq,
                                                                   int64_t ldq, float* __restrict__ sx) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
    if (m >= Mtok) return;   // whole waves only: no barrier below
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
        const int64_t g = lane + 64 * c;
        cache[c] = g < groups ? *(const uint4*)(xr + 8 * g) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kQuantCache; ++c) absmax8(cache[c]);
    for (int64_t g = lane + 64 * kQuantCache; g < groups; g += 64) absmax8(*(const uint4*)(xr + 8 * g));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float s = __fdiv_rn(amax, FP8 ? 448.0f : 127.0f);
    if (lane == 0) sx[m] = s;

    int8_t* qr = Xq + m * ldq;
    auto emit = [&](int64_t g, const uint4 v) __attribute__((always_inline)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = __builtin_bit_cast(float, ((w[i >> 1] >> (16 * (i & 1))) & 0xffffu) << 16);
            if constexpr (FP8) {
                b[i] = s > 0.0f ? e4m3_code(fminf(fmaxf(__fdiv_rn(x, s), -448.0f), 448.0f)) : 0u;
            } else {
                float q = 0.0f;
                if (s > 0.0f) q = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.0f), 127.0f);
                b[i] = (uint32_t)(int32_t)q & 0xffu;
            }
        }
        const uint32_t lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
        const uint32_t hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        if constexpr (LIFT) {
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
        const int64_t g = lane + 64 * c;
        if (g < groups) emit(g, cache[c]);
    }
    for (int64_t g = lane + 64 * kQuantCache; g < groups; g += 64) emit(g, *(const uint4*)(xr + 8 * g));
}

void launch_quant_lift(const void* X, int64_t Mtok, int64_t K, int64_t ldx, int Ns, nm_dtype qdt, void* Xq,
                       int64_t ldq, float* x_scale, hipStream_t s) {
    if (Mtok == 0) return;
    const dim3 g((unsigned)ceil_div(Mtok, kQuantThreads / 64)), b(kQuantThreads);
    const uint16_t* x = (const uint16_t*)X;
    int8_t* q = (int8_t*)Xq;
    if (qdt == NM_FP8) {
        if (Ns) hipLaunchKernelGGL((quant_lift_kernel<true, true>), g, b, 0, s, x, ldx, Mtok, K, q, ldq, x_scale);
        else hipLaunchKernelGGL((quant_lift_kernel<false, true>), g, b, 0, s, x, ldx, Mtok, K, q, ldq, x_scale);
    } else {
        if (Ns) hipLaunchKernelGGL((quant_lift_kernel<true, false>), g, b, 0, s, x, ldx, Mtok, K, q, ldq, x_scale);
        else hipLaunchKernelGGL((quant_lift_kernel<false, false>), g, b, 0, s, x, ldx, Mtok, K, q, ldq, x_scale);
    }
}

}  // namespace nm
