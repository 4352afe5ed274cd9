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
// One block of 256 threads per token row, or one wave per row for rows of up to 4096
// columns: pass 1 takes the absolute maximum over 16-byte loads of 8 columns and keeps up
// to 8 of them per thread in registers (K <= 16384 in one pass with 256 threads; longer
// rows re-read the rest, which is L2-resident by then); the maximum is reduced across the
// wave and then across the block's four waves; pass 2 rounds and writes each
// 8-column group as 12 lifted bytes (three dwords; 6:8) or, without the lift, 8 bytes.
// For other N, pass 2 takes one window per thread: its 4 columns (two column pairs from the
// row, L2-resident by then), rounded and written as one dword of the lifted row.
#include "nm_internal.h"

namespace nm {

constexpr int kQuantThreads = 256;   // one token row per block
constexpr int kQuantCache = 8;       // 8-column groups per thread kept in registers

// OCP e4m3 code of v, |v| <= 448, finite: nearest code, ties to even.  With t the
// biased f32 exponent of |v| raised to that of 2^-6 (below it the codes are the
// subnormals m 2^-9), y = |v| 2^(3 - (t - 127)) is exact and lies in [8, 16) in a normal
// binade, [0, 8) in the subnormal one; rint(y) (ties to even) is the code's 3-bit
// mantissa plus 8, counted from the binade's first code (t - 121) * 8 - 8, and a value
// that rounds up to 16 carries into the next binade as the code arithmetic requires.
// -0 keeps its sign.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, v);
    const float a = __builtin_bit_cast(float, bits & 0x7fffffffu);
    const int t = max((int)((bits >> 23) & 0xffu), 121);
    const uint32_t r = (uint32_t)rintf(__builtin_ldexpf(a, 130 - t));
    return ((bits >> 24) & 0x80u) | ((uint32_t)(t - 121) * 8u + r);
}

// x / s rounded to nearest f32 for one row's scale s (finite, > 0) without a division per
// element: s and x are scaled by the same power of two so that s lies in [1, 2) (exact),
// r = RN(1 / s) is formed once, q0 = RN(x r) is within an ulp of x / s, the residual
// x - q0 s is exact in one fma, and RN(q0 + (x - q0 s) r) is RN(x / s) (Markstein's
// correction step).  The quotient carries x's sign (also for x = -0).  A quotient that
// the scaling pushes below the normal range is below 2^-125 and gives code 0 either way.
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

struct RowDiv {
    int k;       // the scaling exponent
    float s1;    // s 2^k, in [1, 2)
    float r1;    // RN(1 / s1)
};
__device__ __forceinline__ RowDiv row_div(float s) {
    RowDiv d;
    d.k = 1 - __builtin_amdgcn_frexp_expf(s);
    d.s1 = __builtin_ldexpf(s, d.k);
    d.r1 = __fdiv_rn(1.0f, d.s1);
    return d;
}
__device__ __forceinline__ float row_quot(float x, const RowDiv& d) {
    const float xs = __builtin_ldexpf(x, d.k);
    const float q0 = xs * d.r1;
    const float rem = __builtin_fmaf(-q0, d.s1, xs);
    return __builtin_copysignf(__builtin_fmaf(rem, d.r1, q0), x);
}

// LIFT: 0 no lift, 1 the 6:8 lift (Ns = 4), 2 the lift of any (2N-2):2N (runtime Ns).
// RW: threads per token row, 256 (the block) or 64 (one wave per row, four rows per block:
// no block barrier, and four times the rows in flight; for rows of up to 4096 columns,
// which then sit in registers whole).
template <int LIFT, bool FP8, int RW>
__global__ __launch_bounds__(kQuantThreads) void quant_lift_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                   int64_t Mtok, int64_t K, int Ns,
                                                                   int8_t* __restrict__ Xq, int64_t ldq,
                                                                   float* __restrict__ sx) {
    static_assert(RW == 64 || RW == kQuantThreads, "a wave or the block per row");
    const int lane = threadIdx.x % RW;   // the thread's place in the row
    const int64_t m = RW == kQuantThreads ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * 4 + threadIdx.x / 64;
    if (RW == 64 && m >= Mtok) return;   // a whole wave; this form has no block barrier
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
        const int64_t g = lane + RW * c;
        cache[c] = g < groups ? *(const uint4*)(xr + 8 * g) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kQuantCache; ++c) absmax8(cache[c]);
    for (int64_t g = lane + RW * kQuantCache; g < groups; g += RW)
        absmax8(*(const uint4*)(xr + 8 * g));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if constexpr (RW == kQuantThreads) {
        __shared__ float wmax[kQuantThreads / 64];
        if ((lane & 63) == 0) wmax[lane >> 6] = amax;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, wmax[w]);   // max: order-free
    }
    // every lane holds the row's maximum: make it (and all that follows from it) uniform
    amax = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, amax)));
    const float s = __fdiv_rn(amax, FP8 ? 448.0f : 127.0f);
    if (lane == 0) sx[m] = s;

    int8_t* qr = Xq + m * ldq;
    // pass 2 with the quotient x / s formed by FD ? row_quot : a division per element (s
    // finite and > 0 on every ordinary row; an infinite absolute maximum keeps the division)
    auto pass2 = [&](auto fd) __attribute__((always_inline)) {
        constexpr bool FD = decltype(fd)::value;
        const RowDiv rd = row_div(FD ? s : 1.0f);
        // (FD implies s > 0; otherwise a zero row, s = 0, gives codes 0)
        auto code = [&](float x) __attribute__((always_inline)) -> uint32_t {
            if (!FD && !(s > 0.0f)) return 0u;
            const float v = FD ? row_quot(x, rd) : __fdiv_rn(x, s);
            if constexpr (FP8) return e4m3_code(fminf(fmaxf(v, -448.0f), 448.0f));
            else return (uint32_t)(int32_t)fminf(fmaxf(rintf(v), -127.0f), 127.0f) & 0xffu;
        };
        if constexpr (LIFT == 2) {
            // one window per lane: columns 2Ng + 2w .. +3 (two aligned column pairs)
            const int64_t wpr = K / (2 * Ns) * (Ns - 1);
            for (int64_t q = lane; q < wpr; q += RW) {
                const int64_t g = q / (Ns - 1), w = q - g * (Ns - 1);
                const uint32_t* src = (const uint32_t*)(xr + 2 * Ns * g + 2 * w);
                const uint32_t p0 = src[0], p1 = src[1];
                const uint32_t b0 = code(__builtin_bit_cast(float, (p0 & 0xffffu) << 16));
                const uint32_t b1 = code(__builtin_bit_cast(float, (p0 >> 16) << 16));
                const uint32_t b2 = code(__builtin_bit_cast(float, (p1 & 0xffffu) << 16));
                const uint32_t b3 = code(__builtin_bit_cast(float, (p1 >> 16) << 16));
                *(uint32_t*)(qr + 4 * q) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
            }
        } else {
            auto emit = [&](int64_t g, const uint4 v) __attribute__((always_inline)) {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                uint32_t b[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    b[i] = code(__builtin_bit_cast(float, ((w[i >> 1] >> (16 * (i & 1))) & 0xffffu) << 16));
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
                const int64_t g = lane + RW * c;
                if (g < groups) emit(g, cache[c]);
            }
            for (int64_t g = lane + RW * kQuantCache; g < groups; g += RW)
                emit(g, *(const uint4*)(xr + 8 * g));
        }
    };
    if (s > 0.0f && s <= 3.0e38f) pass2(BoolTag<true>{});
    else pass2(BoolTag<false>{});
}

void launch_quant_lift(const void* X, int64_t Mtok, int64_t K, int64_t ldx, int Ns, nm_dtype qdt, void* Xq,
                       int64_t ldq, float* x_scale, hipStream_t s) {
    if (Mtok == 0) return;
    const uint16_t* x = (const uint16_t*)X;
    int8_t* q = (int8_t*)Xq;
    // a wave per row when the row fits its registers and there are rows enough to fill the
    // chip with waves; a block per row otherwise
    const bool wave_rows = K <= 64 * 8 * kQuantCache && Mtok >= 256;
    const dim3 gb((unsigned)Mtok), gw((unsigned)((Mtok + 3) / 4)), b(kQuantThreads);
#define NM_QL(L, F8)                                                                                              \
    do {                                                                                                          \
        if (wave_rows)                                                                                            \
            hipLaunchKernelGGL((quant_lift_kernel<L, F8, 64>), gw, b, 0, s, x, ldx, Mtok, K, Ns, q, ldq, x_scale); \
        else                                                                                                      \
            hipLaunchKernelGGL((quant_lift_kernel<L, F8, kQuantThreads>), gb, b, 0, s, x, ldx, Mtok, K, Ns, q, ldq, \
                               x_scale);                                                                          \
    } while (0)
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
