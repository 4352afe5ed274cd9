// Bitmap-format sparse weights ("SALR", section 4): the pruned weight is stored as a
// bitmap of its kept positions, the kept values of each row in column order, and a
// lookup table of where each 64-column block's values start, so any sparsity pattern
// (unstructured, or (2N-2):2N without the sliding-window expansion) is carried at one
// bit per position plus the values.  The product runs in two stages per K step of a
// block's tile: stage 1 rebuilds the dense weight tile in LDS from the bitmap, the table
// and the values; stage 2 multiplies it with dense bf16 MFMA (v_mfma_f32_32x32x16_bf16).
// Up to 4 tokens the rows are streamed instead (one wave per row); from 512 tokens stage 1
// runs once over the whole weight into the workspace, and stage 2 is the dense split
// ring (k_spmm.hip) when the product has a 256 x 256 tile for every CU.
//
// Layout (the bitmap is the 1-bit mask of the other entry points):
//   mask [R, ldm] bytes, bit k%8 of byte k/8 = position k kept;
//   vals [R, ldv] bf16, row r's kept values in column order at 0 .. nnz_r - 1;
//   offs [R, ldo] int32, offs[r, b] = kept values of row r before column 64 b, and
//   offs[r, K/64] = nnz_r.  Kept values at a row position >= ldv are not stored and read
//   as zero.
#include "nm_internal.h"

namespace nm {

typedef __bf16 bm_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float bm_f32x16_t __attribute__((ext_vector_type(16)));
typedef int bm_i32x4_t __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ encode
// One wave per row, 512 columns per pass: lane l owns 8 columns (one bitmap byte, one
// 16-byte load of W, loaded a pass ahead).  The lanes' kept counts are scanned across the
// wave (inclusive prefix by shuffles), each lane places its kept values at its prefix in
// a per-wave LDS buffer, and the wave stores the pass's values with consecutive lanes on
// consecutive positions of the value row.  Lanes that start a 64-column block write its
// table entry.
__global__ __launch_bounds__(256) void bitmap_encode_kernel(const uint16_t* __restrict__ W, int64_t ldw, int64_t R,
                                                            int64_t K, const uint8_t* __restrict__ mask, int64_t ldm,
                                                            uint16_t* __restrict__ vals, int64_t ldv,
                                                            int32_t* __restrict__ offs, int64_t ldo) {
    // a pass's kept values, compacted in column order (a wave's LDS accesses run in order,
    // so only the compiler must keep the writes before the reads)
    __shared__ uint16_t sval[4][512];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r = (int64_t)blockIdx.x * 4 + wave;
    if (r >= R) return;   // the whole wave leaves together
    const int64_t nbytes = K / 8;
    uint16_t* sv = sval[wave];
    // the next pass's bitmap byte and 8 columns of W are loaded before this pass is stored
    auto load = [&](int64_t q, uint32_t& mb, uint4& v) __attribute__((always_inline)) {
        const bool in = q < nbytes;
        mb = in ? mask[r * ldm + q] : 0u;
        v = in ? *(const uint4*)(W + r * ldw + 8 * q) : make_uint4(0, 0, 0, 0);
    };
    uint32_t mbn;
    uint4 vn;
    load(lane, mbn, vn);
    int64_t base = 0;
    for (int64_t c0 = 0; c0 < nbytes; c0 += 64) {
        const int64_t q = c0 + lane;   // bitmap byte = 8-column group
        const uint32_t mb = mbn;
        const uint4 v = vn;
        if (c0 + 64 < nbytes) load(q + 64, mbn, vn);
        const int cnt = __popc(mb);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d, 64);
            if (lane >= d) incl += t;
        }
        const int rel = incl - cnt;   // this lane's first value within the pass
        if (q < nbytes && (q & 7) == 0) offs[r * ldo + q / 8] = (int32_t)(base + rel);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        int k = rel;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((mb >> e) & 1u) sv[k++] = (uint16_t)(e & 1 ? w4[e >> 1] >> 16 : w4[e >> 1] & 0xffffu);
        }
        asm volatile("" ::: "memory");
        const int total = __shfl(incl, 63, 64);
        // consecutive lanes store consecutive values of the row (positions past ldv are dropped)
        for (int t = lane; t < total; t += 64) {
            const int64_t j = base + t;
            if (j < ldv) vals[r * ldv + j] = sv[t];
        }
        asm volatile("" ::: "memory");
        base += total;
    }
    if (lane == 0) offs[r * ldo + K / 64] = (int32_t)base;
}

void launch_bitmap_encode(const void* W, int64_t R, int64_t K, int64_t ldw, const uint8_t* mask, int64_t ldm,
                          void* vals, int64_t ldv, int32_t* offs, int64_t ldo, hipStream_t s) {
    hipLaunchKernelGGL(bitmap_encode_kernel, dim3((unsigned)ceil_div(R, 4)), dim3(256), 0, s, (const uint16_t*)W, ldw, R,
                       K, mask, ldm, (uint16_t*)vals, ldv, offs, ldo);
}

// ------------------------------------------------------------------ decode + dense MFMA
// Block = 4 waves (2 x 2) on a 128-row x 128-token tile, K in stages of 64 columns,
// LDS double-buffered: the next stage's bitmap bytes, table entries, value windows and
// X chunks are loaded into registers while the current stage's MFMAs issue, then
// expanded and written to the other buffer.  Stage 1 (decode): a unit is one tile row's
// 8-column group (a bitmap byte); its kept values are consecutive in the value row,
// starting at offs[row, block] + the kept count of the block's earlier groups, so two
// aligned 16-byte loads cover them, and the expansion places them at the set bits.
// Requires 16-byte aligned value rows (ldv % 8 == 0).  Stage 2: each wave
// multiplies 64 rows x 64 tokens (2 x 2 sub-tiles of 32 x 32) over the stage's 64
// columns (4 MFMA depths of 16).  16-byte chunks of both LDS tiles are XOR-swizzled
// by (row % 8) so that the 16 lanes served together by a read hit distinct banks.
// gridDim.y splits the stages; with more than one split the f32 partials go to
// part[split][Mtok][R] and bitmap_reduce_kernel sums them in split order.  With many
// tokens the per-tile decode would repeat once per token tile, so stage 1 runs once as
// bitmap_decode_kernel into a dense copy of the weight in the workspace and the product
// kernel reads its tiles like those of X (the pages' two stages as two passes).
struct BitmapArgs {
    const uint16_t* X;
    const uint16_t* dense;   // many tokens: the decoded weight [R, K] in the workspace
    const uint16_t* vals;
    const uint8_t* mask;
    const int32_t* offs;
    void* Y;
    float* part;
    int64_t ldx, ldv, ldm, ldo, ldy;
    int64_t Mtok, K, R;
    int ydt;
    int nsteps, steps_per_split;
    int tiles_r;
};

constexpr int kBmBR = 128, kBmBT = 128, kBmKC = 64;

// Stage 1 for one 8-column group of a row: bits64 = the row's bitmap word of the group's
// 64-column block, off = offs[row, block], byte = the group within the block.  The
// group's kept values (at most 8) are consecutive in the value row from position
// j0 = off + (kept count of the block's earlier groups); the two aligned 16-byte chunks
// from the one holding j0 cover them (chunks past the row read as zero).  The expansion
// shifts that window so value j0 is the low half of the first word, then walks the 8
// columns and takes the next value for each set bit.  Returns the 8 dense bf16.
struct BmWindow {
    uint4 w0, w1;
    uint32_t mb, sh;
};
// Branch-free: both chunks are always loaded (at indices clamped into the row, vchunks
// >= 1) and zeroed when they lie outside it or the group keeps nothing.
__device__ __forceinline__ BmWindow bm_fetch(uint64_t bits64, int32_t off, int byte, const uint16_t* vrow,
                                             int64_t vchunks) {
    BmWindow r;
    const int b8 = 8 * byte;
    r.mb = (uint32_t)(bits64 >> b8) & 0xffu;
    const int64_t j0 = (int64_t)off + __popcll(bits64 & ((1ull << b8) - 1ull));
    const int64_t c = j0 >> 3;
    r.sh = (uint32_t)(j0 & 7);
    const int64_t ca = c < 0 ? 0 : (c < vchunks ? c : vchunks - 1);
    const int64_t cb = c + 1 < 0 ? 0 : (c + 1 < vchunks ? c + 1 : vchunks - 1);
    const uint4 a = *(const uint4*)(vrow + 8 * ca);
    const uint4 b = *(const uint4*)(vrow + 8 * cb);
    const uint32_t ka = (r.mb != 0u && c >= 0 && c < vchunks) ? 0xffffffffu : 0u;
    const uint32_t kb = (r.mb != 0u && c + 1 >= 0 && c + 1 < vchunks) ? 0xffffffffu : 0u;
    r.w0 = make_uint4(a.x & ka, a.y & ka, a.z & ka, a.w & ka);
    r.w1 = make_uint4(b.x & kb, b.y & kb, b.z & kb, b.w & kb);
    return r;
}
// The window shifted so that the group's first value is the low half of d[0]; then
// column c takes value (kept count of the group's columns before c) of d, selected by
// shifts without branches, or 0 when its bit is clear.
__device__ __forceinline__ uint4 bm_expand(const BmWindow& b) {
    const uint32_t w[8] = {b.w0.x, b.w0.y, b.w0.z, b.w0.w, b.w1.x, b.w1.y, b.w1.z, b.w1.w};
    // values s + 2i + {0, 1} (s = b.sh) sit in words ds + i and ds + i + 1 <= 7
    const uint32_t ds = b.sh >> 1, hs = (b.sh & 1u) * 16u;
    uint32_t d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = w[i], hi = w[i + 1];
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            lo = ds == (uint32_t)k ? w[i + k] : lo;
            hi = ds == (uint32_t)k ? w[i + k + 1] : hi;
        }
        d[i] = hs ? ((lo >> 16) | (hi << 16)) : lo;
    }
    // halfword rank (0..7) of d: pick the 64-bit half, shift by 16 (rank % 4), mask
    const uint64_t d01 = (uint64_t)d[0] | ((uint64_t)d[1] << 32), d23 = (uint64_t)d[2] | ((uint64_t)d[3] << 32);
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t r0 = __popc(b.mb & ((1u << (2 * p)) - 1u));
        const uint32_t bit0 = (b.mb >> (2 * p)) & 1u, bit1 = (b.mb >> (2 * p + 1)) & 1u;
        const uint32_t r1 = r0 + bit0;
        const uint64_t s0 = (r0 & 4u) ? d23 : d01, s1 = (r1 & 4u) ? d23 : d01;
        const uint32_t v0 = (uint32_t)(s0 >> (16u * (r0 & 3u))) & (0xffffu & (0u - bit0));
        const uint32_t v1 = (uint32_t)(s1 >> (16u * (r1 & 3u))) & (0xffffu & (0u - bit1));
        o[p] = v0 | (v1 << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// A wave's 2 x 2 sub-tiles (rows from rw, tokens from tw): the lane holds token column
// l32 and rows 8*(e/4) + 4*h + e%4 of each sub-tile; stored to Y (converted) or, with a
// K split, to the split's f32 partials.
__device__ __forceinline__ void bm_store(const BitmapArgs& a, const bm_f32x16_t (&acc)[2][2], int64_t rw, int64_t tw,
                                         int lane) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t tok = tw + j * 32 + l32;
            if (tok >= a.Mtok) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t r = rw + i * 32 + 8 * (e / 4) + 4 * h + (e % 4);
                if (r >= a.R) continue;
                const float v = acc[i][j][e];
                if (a.part) a.part[((int64_t)blockIdx.y * a.Mtok + tok) * a.R + r] = v;
                else if (a.ydt == NM_F32) ((float*)a.Y)[tok * a.ldy + r] = v;
                else ((uint16_t*)a.Y)[tok * a.ldy + r] = (uint16_t)f32_to_bf16_bits(v);
            }
        }
}

// Stage 1 as a pass of its own (many tokens): the dense weight [R, K] (row stride K) is
// rebuilt once into the workspace, one thread per 8-column group.
__global__ __launch_bounds__(256) void bitmap_decode_kernel(BitmapArgs a, uint16_t* __restrict__ Wd) {
    const int64_t groups = a.K / 8, total = a.R * groups, vchunks = a.ldv / 8;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / groups, g = i - r * groups, b = g >> 3;
        const uint64_t bits64 = *(const uint64_t*)(a.mask + r * a.ldm + 8 * b);
        const BmWindow w = bm_fetch(bits64, a.offs[r * a.ldo + b], (int)(g & 7), a.vals + r * a.ldv, vchunks);
        *(uint4*)(Wd + r * a.K + 8 * g) = bm_expand(w);
    }
}

__global__ __launch_bounds__(256, 2) void bitmap_spmm_kernel(BitmapArgs a) {
    // one array: [buffer][weight tile, X tile][64-column rows]
    __shared__ __attribute__((aligned(16))) uint16_t sm[2 * 2 * kBmBR * kBmKC];
    static_assert(kBmBR == kBmBT, "the two tiles share one layout");
    constexpr int kTile = kBmBR * kBmKC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wt = wave >> 1, h = lane >> 5, l32 = lane & 31;
    const int tr = blockIdx.x % a.tiles_r, tt = blockIdx.x / a.tiles_r;
    const int64_t r0 = (int64_t)tr * kBmBR, t0 = (int64_t)tt * kBmBT;
    const int s_begin = blockIdx.y * a.steps_per_split;
    const int s_end = s_begin + a.steps_per_split < a.nsteps ? s_begin + a.steps_per_split : a.nsteps;

    // weight role: four units of (tile row, 8-column group) per thread, q = tid + 256 u
    const uint8_t* mrow[4];
    const int32_t* orow[4];
    const uint16_t* vrow[4];
    int dlds[4], dbyte[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int q = tid + 256 * u, row = q >> 3, byte = q & 7;
        const int64_t gr = r0 + row < a.R ? r0 + row : a.R - 1;
        mrow[u] = a.mask + gr * a.ldm;
        orow[u] = a.offs + gr * a.ldo;
        vrow[u] = a.vals + gr * a.ldv;
        dbyte[u] = byte;
        dlds[u] = row * kBmKC + ((byte ^ (row & 7)) << 3);
    }
    const int64_t vchunks = a.ldv / 8;   // 16-byte chunks per value row
    // X role: four 16-byte chunks of the 128 x 64 X tile
    int64_t xoff[4];
    int xlds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i, tok = q >> 3, c = q & 7;
        const int64_t gt = t0 + tok < a.Mtok ? t0 + tok : a.Mtok - 1;
        xoff[i] = gt * a.ldx + 8 * c;
        xlds[i] = tok * kBmKC + ((c ^ (tok & 7)) << 3);
    }

    // The bitmap words and table entries of stage st+2 and the value windows of stage
    // st+1 are in flight while stage st multiplies: each stage waits for one round trip,
    // not for the two dependent ones (table, then values).
    uint64_t mbits[4];
    int32_t moff[4];
    BmWindow win[4];
    uint4 xv[4];
    auto load_meta = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            mbits[u] = *(const uint64_t*)(mrow[u] + 8 * (int64_t)st);
            moff[u] = orow[u][st];
        }
    };
    auto load = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            win[u] = bm_fetch(mbits[u], moff[u], dbyte[u], vrow[u], vchunks);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[i] = *(const uint4*)(a.X + xoff[i] + (int64_t)st * kBmKC);
    };
    auto store = [&](int buf) __attribute__((always_inline)) {
        uint16_t* sA = sm + (2 * buf) * kTile;
        uint16_t* sX = sA + kTile;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            *(uint4*)&sA[dlds[u]] = bm_expand(win[u]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) *(uint4*)(&sX[xlds[i]]) = xv[i];
    };

    bm_f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = bm_f32x16_t{};

    if (s_begin < s_end) {
        load_meta(s_begin);
        load(s_begin);
        if (s_begin + 1 < s_end) load_meta(s_begin + 1);
        store(0);
    }
    __syncthreads();
    for (int st = s_begin; st < s_end; ++st) {
        const int buf = (st - s_begin) & 1;
        const bool more = st + 1 < s_end;
        // past the range the last stage is loaded again (valid, never stored): the loads
        // stay unconditional so the compiler keeps their registers out of memory
        load(more ? st + 1 : st);
        load_meta(st + 2 < s_end ? st + 2 : s_end - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bm_i32x4_t af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wr * 64 + i * 32 + l32;
                af[i] = *(const bm_i32x4_t*)&sm[(2 * buf) * kTile + row * kBmKC + (((2 * s + h) ^ (row & 7)) << 3)];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tok = wt * 64 + j * 32 + l32;
                bf[j] = *(const bm_i32x4_t*)&sm[(2 * buf + 1) * kTile + tok * kBmKC + (((2 * s + h) ^ (tok & 7)) << 3)];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bm_bf16x8_t, af[i]),
                                                                       __builtin_bit_cast(bm_bf16x8_t, bf[j]),
                                                                       acc[i][j], 0, 0, 0);
        }
        if (more) store(buf ^ 1);
        __syncthreads();
    }

    bm_store(a, acc, r0 + wr * 64, t0 + wt * 64, lane);
}

// Stage 2 on the dense copy: the same tiling, with the weight tile read like X.
__global__ __launch_bounds__(256, 2) void bitmap_dense_kernel(BitmapArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBmBR * kBmKC];
    __shared__ __attribute__((aligned(16))) uint16_t sX[2][kBmBT * kBmKC];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wt = wave >> 1, h = lane >> 5, l32 = lane & 31;
    const int tr = blockIdx.x % a.tiles_r, tt = blockIdx.x / a.tiles_r;
    const int64_t r0 = (int64_t)tr * kBmBR, t0 = (int64_t)tt * kBmBT;
    const int s_begin = blockIdx.y * a.steps_per_split;
    const int s_end = s_begin + a.steps_per_split < a.nsteps ? s_begin + a.steps_per_split : a.nsteps;
    const uint16_t* wp[4];
    const uint16_t* xp[4];
    int ls[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i, row = q >> 3, c = q & 7;
        const int64_t gr = r0 + row < a.R ? r0 + row : a.R - 1;
        const int64_t gt = t0 + row < a.Mtok ? t0 + row : a.Mtok - 1;
        wp[i] = a.dense + gr * a.K + 8 * c;
        xp[i] = a.X + gt * a.ldx + 8 * c;
        ls[i] = row * kBmKC + ((c ^ (row & 7)) << 3);
    }
    uint4 w0, w1, w2, w3, x0, x1, x2, x3;
    bm_f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = bm_f32x16_t{};
    if (s_begin < s_end) {
        const int64_t o = (int64_t)s_begin * kBmKC;
        w0 = *(const uint4*)(wp[0] + o); w1 = *(const uint4*)(wp[1] + o);
        w2 = *(const uint4*)(wp[2] + o); w3 = *(const uint4*)(wp[3] + o);
        x0 = *(const uint4*)(xp[0] + o); x1 = *(const uint4*)(xp[1] + o);
        x2 = *(const uint4*)(xp[2] + o); x3 = *(const uint4*)(xp[3] + o);
        *(uint4*)&sA[0][ls[0]] = w0; *(uint4*)&sA[0][ls[1]] = w1; *(uint4*)&sA[0][ls[2]] = w2; *(uint4*)&sA[0][ls[3]] = w3;
        *(uint4*)&sX[0][ls[0]] = x0; *(uint4*)&sX[0][ls[1]] = x1; *(uint4*)&sX[0][ls[2]] = x2; *(uint4*)&sX[0][ls[3]] = x3;
    }
    __syncthreads();
    for (int st = s_begin; st < s_end; ++st) {
        const int buf = (st - s_begin) & 1;
        const bool more = st + 1 < s_end;
        const int64_t o = (int64_t)(more ? st + 1 : st) * kBmKC;   // past the range: reloaded, never stored
        w0 = *(const uint4*)(wp[0] + o); w1 = *(const uint4*)(wp[1] + o);
        w2 = *(const uint4*)(wp[2] + o); w3 = *(const uint4*)(wp[3] + o);
        x0 = *(const uint4*)(xp[0] + o); x1 = *(const uint4*)(xp[1] + o);
        x2 = *(const uint4*)(xp[2] + o); x3 = *(const uint4*)(xp[3] + o);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bm_i32x4_t af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wr * 64 + i * 32 + l32;
                af[i] = *(const bm_i32x4_t*)&sA[buf][row * kBmKC + (((2 * s + h) ^ (row & 7)) << 3)];
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tok = wt * 64 + j * 32 + l32;
                bf[j] = *(const bm_i32x4_t*)&sX[buf][tok * kBmKC + (((2 * s + h) ^ (tok & 7)) << 3)];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bm_bf16x8_t, af[i]),
                                                                       __builtin_bit_cast(bm_bf16x8_t, bf[j]),
                                                                       acc[i][j], 0, 0, 0);
        }
        if (more) {
            const int nb = buf ^ 1;
            *(uint4*)&sA[nb][ls[0]] = w0; *(uint4*)&sA[nb][ls[1]] = w1; *(uint4*)&sA[nb][ls[2]] = w2; *(uint4*)&sA[nb][ls[3]] = w3;
            *(uint4*)&sX[nb][ls[0]] = x0; *(uint4*)&sX[nb][ls[1]] = x1; *(uint4*)&sX[nb][ls[2]] = x2; *(uint4*)&sX[nb][ls[3]] = x3;
        }
        __syncthreads();
    }
    bm_store(a, acc, r0 + wr * 64, t0 + wt * 64, lane);
}

// ------------------------------------------------------------------ few tokens: row streaming
// With a handful of tokens the product is a stream over the weight: one wave per weight
// row, lane l expanding the row's 8-column groups l, l + 64, l + 128, ... (the stage-1
// window decode above: consecutive lanes take consecutive stretches of the value row, so
// a wave's loads cover it contiguously) and multiplying each with the tokens' 8 columns
// (f32 multiply-adds in column order, groups in lane order).  A step takes U groups per
// lane; a wave walks the (row, step) pairs of its rows in one sequence, and the next
// step's bitmap words, table entries and token columns are loaded while this step's value
// windows load and multiply, so a step waits for one memory round trip, not two
// (slide68 at one token 45 -> 41 us with U = 2; U = 4 held too many registers, 43.5 us,
// and without the overlap U = 4 was the best, U = 8 and 16 slower).  The lanes' sums are
// added by a butterfly across the wave, whose result is the same on every lane and run.
// The tokens' columns are read from memory for every row (they stay in L1): copying them
// into LDS once per block measured the same (slide68 at 1 token 42.2 against 42.0 us).
constexpr int kBmRowTokens = 4;

template <int MT, int U>
__global__ __launch_bounds__(256) void bitmap_rows_kernel(BitmapArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t groups = a.K / 8, vchunks = a.ldv / 8;
    const int64_t steps = (groups + 64 * U - 1) / (64 * U);   // per row, >= 1
    const int64_t wstride = (int64_t)gridDim.x * 4;
    const int mt = (int)a.Mtok;   // <= MT
    int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.R) return;   // the whole wave; this kernel has no barrier
    uint64_t bits[U], nbits[U];
    int32_t off[U], noff[U];
    uint4 xv[U][MT], nxv[U][MT];
    // step st of row rr: groups st * 64 U + lane + 64 u (past the row: its last group, unused)
    auto meta = [&](int64_t rr, int64_t st, uint64_t (&b)[U], int32_t (&o)[U], uint4 (&x)[U][MT])
                    __attribute__((always_inline)) {
        const uint8_t* mrow = a.mask + rr * a.ldm;
        const int32_t* orow = a.offs + rr * a.ldo;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = st * 64 * U + lane + 64 * u, gc = g < groups ? g : groups - 1;
            b[u] = g < groups ? *(const uint64_t*)(mrow + (gc >> 3) * 8) : 0ull;
            o[u] = orow[gc >> 3];
#pragma unroll
            for (int m = 0; m < MT; ++m) x[u][m] = *(const uint4*)(a.X + (m < mt ? m : 0) * a.ldx + gc * 8);
        }
    };
    meta(r, 0, bits, off, xv);
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
    int64_t st = 0;
    while (true) {
        const uint16_t* vrow = a.vals + r * a.ldv;
        BmWindow wnd[U];
#pragma unroll
        for (int u = 0; u < U; ++u) wnd[u] = bm_fetch(bits[u], off[u], lane & 7, vrow, vchunks);
        const bool last = st + 1 == steps;
        const int64_t rn = last ? r + wstride : r, sn = last ? 0 : st + 1;
        const bool more = rn < a.R;
        if (more) meta(rn, sn, nbits, noff, nxv);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (st * 64 * U + lane + 64 * u >= groups) continue;   // past the row
            const uint4 wv = bm_expand(wnd[u]);
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
            float w[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                w[2 * e] = __uint_as_float(ww[e] << 16);
                w[2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint32_t xx[4] = {xv[u][m].x, xv[u][m].y, xv[u][m].z, xv[u][m].w};
                float t = acc[m];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    t = __fmaf_rn(w[2 * e], __uint_as_float(xx[e] << 16), t);
                    t = __fmaf_rn(w[2 * e + 1], __uint_as_float(xx[e] & 0xffff0000u), t);
                }
                acc[m] = t;
            }
        }
        if (last) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) acc[m] += __shfl_xor(acc[m], o);
            if (lane == 0) {
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    if (m < mt) {
                        if (a.ydt == NM_F32) ((float*)a.Y)[m * a.ldy + r] = acc[m];
                        else ((uint16_t*)a.Y)[m * a.ldy + r] = (uint16_t)f32_to_bf16_bits(acc[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
        }
        if (!more) break;
        r = rn;
        st = sn;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            bits[u] = nbits[u];
            off[u] = noff[u];
#pragma unroll
            for (int m = 0; m < MT; ++m) xv[u][m] = nxv[u][m];
        }
    }
}

// Y[m, o] = sum of the splits' partials in split order, converted.
__global__ __launch_bounds__(256) void bitmap_reduce_kernel(const float* __restrict__ part, int KS, int64_t M,
                                                            int64_t R, void* Y, int ydt, int64_t ldy) {
    const int64_t total = M * R;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const float v = split_sum(part + i, KS, total);
        const int64_t m = i / R, o = i - m * R;
        if (ydt == NM_F32) ((float*)Y)[m * ldy + o] = v;
        else ((uint16_t*)Y)[m * ldy + o] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// Stage split over blocks while fewer than 512 blocks (two per CU) would run and every
// split keeps at least 4 stages.
static int bitmap_splits(int64_t Mtok, int64_t K, int64_t R) {
    const int64_t tiles = ceil_div(R, kBmBR) * ceil_div(Mtok, kBmBT), nsteps = K / kBmKC;
    int ks = 1;
    while (tiles * ks < 512 && nsteps >= 8 * ks) ks *= 2;
    return ks;
}

// From this many tokens (four token tiles or more) the weight is decoded once into the
// workspace instead of once per token tile.
constexpr int64_t kBmDenseTokens = 512;

static size_t bm_dense_bytes(int64_t Mtok, int64_t K, int64_t R) {
    return Mtok >= kBmDenseTokens ? (((size_t)R * (size_t)K * 2 + 255) & ~(size_t)255) : 0;
}

size_t bitmap_spmm_ws(int64_t Mtok, int64_t K, int64_t R) {
    if (Mtok <= 0 || K <= 0 || R <= 0 || Mtok <= kBmRowTokens) return 0;
    const int ks = bitmap_splits(Mtok, K, R);
    return bm_dense_bytes(Mtok, K, R) + (ks > 1 ? (size_t)ks * (size_t)Mtok * (size_t)R * 4 : 0);
}

nm_status launch_bitmap_spmm(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals, int64_t ldv,
                             const uint8_t* mask, int64_t ldm, const int32_t* offs, int64_t ldo, int64_t R, void* Y,
                             nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s) {
    BitmapArgs a{};
    a.X = (const uint16_t*)X;
    a.vals = (const uint16_t*)vals;
    a.mask = mask;
    a.offs = offs;
    a.Y = Y;
    a.ldx = ldx;
    a.ldv = ldv;
    a.ldm = ldm;
    a.ldo = ldo;
    a.ldy = ldy;
    a.Mtok = Mtok;
    a.K = K;
    a.R = R;
    a.ydt = (int)ydt;
    a.nsteps = (int)(K / kBmKC);
    if (Mtok <= kBmRowTokens) {
        // 4 waves (rows) per block, up to 8 blocks per CU
        const dim3 g((unsigned)grid_cap(ceil_div(R, 4), 2048));
        if (Mtok == 1) hipLaunchKernelGGL((bitmap_rows_kernel<1, 2>), g, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((bitmap_rows_kernel<kBmRowTokens, 2>), g, dim3(256), 0, s, a);
        return check_launch("nm_spmm_bitmap");
    }
    const size_t db = bm_dense_bytes(Mtok, K, R);
    if (db) {
        if (!ws || ws_bytes < db) return set_error(NM_ERR_WORKSPACE, "nm_spmm_bitmap: workspace of %zu bytes needed", db);
        const dim3 g(grid_cap(ceil_div(R * (K / 8), 256), 16384));
        hipLaunchKernelGGL(bitmap_decode_kernel, g, dim3(256), 0, s, a, (uint16_t*)ws);
        a.dense = (const uint16_t*)ws;
        ws = (uint8_t*)ws + db;
        ws_bytes -= db;
        // enough 256 x 256 tiles for every CU: the dense split ring on the decoded weight
        // (NM_ERR_SHAPE: it does not apply, nothing was launched; any other status is final)
        const nm_status dr = launch_dense_ring(a.dense, K, a.X, ldx, Mtok, K, R, Y, ydt, ldy, s);
        if (dr != NM_ERR_SHAPE) return dr;
    }
    const int ks = bitmap_splits(Mtok, K, R);
    a.steps_per_split = (int)ceil_div(a.nsteps, ks);
    const int ksn = (int)ceil_div(a.nsteps, a.steps_per_split);
    a.tiles_r = (int)ceil_div(R, kBmBR);
    if (ksn > 1) {
        const size_t need = (size_t)ksn * (size_t)Mtok * (size_t)R * 4;
        if (!ws || ws_bytes < need) return set_error(NM_ERR_WORKSPACE, "nm_spmm_bitmap: workspace of %zu bytes needed", need);
        a.part = (float*)ws;
    }
    const dim3 grid((unsigned)(a.tiles_r * ceil_div(Mtok, kBmBT)), (unsigned)ksn);
    if (db) hipLaunchKernelGGL(bitmap_dense_kernel, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(bitmap_spmm_kernel, grid, dim3(256), 0, s, a);
    if (ksn > 1) {
        const dim3 g(grid_cap(ceil_div(Mtok * R, 256), 8192));
        hipLaunchKernelGGL(bitmap_reduce_kernel, g, dim3(256), 0, s, (const float*)a.part, ksn, Mtok, R, Y, (int)ydt, ldy);
    }
    return check_launch("nm_spmm_bitmap");
}

}  // namespace nm
