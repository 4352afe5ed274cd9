// Per-token int8 quantisation fused with the 6:8 activation lift ("SlideSparse",
// sections 2B-2C: the lift is a pure index remap, done inside the per-token
// quantisation kernel, so that the online step of the int8 path reads the bf16
// activation once and writes the lifted int8 codes the sparse product consumes).
// Token row m: s = max|x| / 127 and q = rint(x / s), ties to even, in f32 (the
// quotients decide integers); a zero row gives s = 0 and codes 0.  With the lift,
// lifted column 12g + 4w + l holds the code of column 8g + 2w + l (windows at
// offsets 0, 2, 4 of each 8-column group).
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

template <bool LIFT>
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
    const float s = __fdiv_rn(amax, 127.0f);
    if (lane == 0) sx[m] = s;

    int8_t* qr = Xq + m * ldq;
    auto emit = [&](int64_t g, const uint4 v) __attribute__((always_inline)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = __builtin_bit_cast(float, ((w[i >> 1] >> (16 * (i & 1))) & 0xffffu) << 16);
            float q = 0.0f;
            if (s > 0.0f) q = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -127.0f), 127.0f);
            b[i] = (uint32_t)(int32_t)q & 0xffu;
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

void launch_quant_lift(const void* X, int64_t Mtok, int64_t K, int64_t ldx, int Ns, int8_t* Xq, int64_t ldq,
                       float* x_scale, hipStream_t s) {
    if (Mtok == 0) return;
    const dim3 g((unsigned)ceil_div(Mtok, kQuantThreads / 64));
    if (Ns) hipLaunchKernelGGL(quant_lift_kernel<true>, g, dim3(kQuantThreads), 0, s, (const uint16_t*)X, ldx, Mtok, K,
                               Xq, ldq, x_scale);
    else hipLaunchKernelGGL(quant_lift_kernel<false>, g, dim3(kQuantThreads), 0, s, (const uint16_t*)X, ldx, Mtok, K,
                            Xq, ldq, x_scale);
}

}  // namespace nm
