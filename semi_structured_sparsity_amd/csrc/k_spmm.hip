// Structured-sparse linear layer Y = X * W_hat^T on packed 2:4 weights, on the
// gfx950 sparse matrix instructions (SMFMAC): the packed weight is the sparse
// A operand, X^T the dense B operand, Y^T the accumulator tile.
//
// "SlideSparse" (sections 2A-2C): a (2N-2):2N weight is stored as overlapping
// 2:4 windows over the lifted width K' = (2 - 2/N) K; the activation is lifted
// to match by a pure index remap (windows 0-3, 2-5, 4-7 of each 8-column group).
// Here lift_kernel writes the lifted activation once into the workspace (1.5x the
// bytes of X, small next to the product) and the plain 2:4 kernels multiply it;
// that measured faster than gathering lifted fragments inside the product kernels
// at every token count tried.
//
// Operand layouts of the two instructions (gfx950, verified on hardware with
// integer data):
//   v_smfmac_f32_32x32x32_bf16: lane l holds A row (l%32), 8 compressed bf16
//     that cover K [16*(l/32), +16) (two kept per 4-group), with their 2-bit
//     in-group positions in bits [2e+1:2e] of the index operand; B column
//     (l%32) as 16 bf16 at K = 16*(e/8) + 8*(l/32) + e%8; C column (l%32),
//     rows 8*(e/4) + 4*(l/32) + e%4.
//   v_smfmac_i32_32x32x64_i8: the same with 16 compressed int8 covering K
//     [32*(l/32), +32), B as 32 int8 at K = 32*(e/16) + 16*(l/32) + e%16.
// For both, the fragment of depth d (one instruction) is 16 bytes of
// compressed values at byte 32d + 16(l/32) of a row's step, and two 16-byte B
// reads at bytes 64d + 16(l/32) and 64d + 32 + 16(l/32) of a token's step.
#include "nm_internal.h"

namespace nm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

// OCP FP8 e4m3 code: one byte, multiplied by v_smfmac_f32_32x32x64_fp8_fp8 with the
// int8 instruction's operand layout and f32 accumulation.
struct fp8e4m3 {
    uint8_t v;
};

// Accumulator types and the sparse instruction of each operand type.  A is the
// lane's 16 bytes of compressed values, B its 32 bytes of the dense operand, idx
// its index bits (bf16: the lane's 16-bit half already selected).
template <typename T>
struct Mma {   // bf16
    using Acc = f32x16_t;
    using AccS = float;
    __device__ static Acc run(i32x4_t a, i32x8_t b, Acc c, int idx) {
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                         __builtin_bit_cast(bf16x16_t, b), c, idx, 0, 0);
    }
};
template <>
struct Mma<int8_t> {
    using Acc = i32x16_t;
    using AccS = int32_t;
    __device__ static Acc run(i32x4_t a, i32x8_t b, Acc c, int idx) {
        return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c, idx, 0, 0);
    }
};
template <>
struct Mma<fp8e4m3> {
    using Acc = f32x16_t;
    using AccS = float;
    __device__ static Acc run(i32x4_t a, i32x8_t b, Acc c, int idx) {
        return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a, b, c, idx, 0, 0);
    }
};

struct SpmmArgs {
    const uint8_t* X;      // [Mtok, ldx] elements of T
    const uint8_t* vals;   // [R, ldv] elements of T
    const uint32_t* idx;   // [R, ldi] words
    const float* x_scale;  // [Mtok] or null
    void* Y;               // [Mtok, ldy] of ydt
    void* part;            // split-K partials [KS][Mtok][R] (f32 or i32) or null
    int64_t ldx, ldv, ldi, ldy;
    int64_t Mtok, K, R;
    int64_t comp_bytes;    // packed value bytes per row (K'/2 * sizeof(T))
    int64_t idx_words;     // index words per row (ceil(K'/32): two 2-bit fields per 4 lifted columns)
    int64_t xrow_bytes;    // bytes of one row of the original (unlifted) X, for the in-kernel lift
    float w_scale;
    int scaled;
    int ydt;
    int nsteps, KS, steps_per_split;
    int tiles_r, tiles_t;
    int tile_rows;         // K-split ring: weight rows per row tile (0: the tile's height)
    // rank-r adapter term added to the accumulators (bf16 products only; rank 0: none):
    // u [Mtok, rank] (ldu) and the stacked up-projection B [R, rank] (ldb), both bf16
    const uint16_t* lr_u;
    const uint16_t* lr_b;
    int64_t ldu, ldb;
    int rank;
    // Hutchinson modes of the dense split ring: probes, their seed, stages per probe, rows
    // per probe
    uint64_t seed;
    int probes, pstages;
    int64_t prows;
    // score epilogue of the Hutchinson second product: W [rows of D, K] bf16 (ldw), eps, and
    // the per-block moments of the scores ([count | mean | m2][blocks])
    const uint16_t* sw;
    int64_t ldsw;
    float eps;
    double* mpart;
};

// Per-dtype step geometry of the register-staged kernel: a step stages 128 bytes of
// activation columns per token.
template <typename T>
struct Geo {
    static constexpr int KO = 128 / (int)sizeof(T);           // columns per step
    static constexpr int KL = KO;
    static constexpr int KDEP = sizeof(T) == 2 ? 32 : 64;      // K per instruction
    static constexpr int ND = KL / KDEP;                       // instructions per step
    static constexpr int AV = KL / 2 * (int)sizeof(T);         // compressed bytes per row per step
    static constexpr int AI = KL / 32;                         // index words per row per step
    static constexpr int BV = KL * (int)sizeof(T);             // bytes per token per step
    static constexpr int AVS = AV + 16;                        // LDS row strides (padded)
    static constexpr int AIS = AI | 1;
    static constexpr int BS = BV + 16;
};

template <typename T, int WR, int WT, int SR, int ST>
struct Tile {
    using G = Geo<T>;
    static constexpr int NT = WR * WT * 64;
    static constexpr int BR = WR * SR * 32;
    static constexpr int BT = WT * ST * 32;
    static constexpr int A_BYTES = BR * G::AVS;
    static constexpr int I_BYTES = BR * G::AIS * 4;
    static constexpr int B_BYTES = BT * G::BS;
    static constexpr int STAGE = A_BYTES + I_BYTES + B_BYTES;
    static constexpr int NA = BR * (G::AV / 16);               // A 16-byte chunks per step
    static constexpr int NI = BR * G::AI;                      // index words per step
    static constexpr int NB = BT * 8;                          // X 16-byte chunks per step
    static constexpr int PA = (NA + NT - 1) / NT;
    static constexpr int PI = (NI + NT - 1) / NT;
    static constexpr int PB = (NB + NT - 1) / NT;
};

// Block index -> (R tile, token tile).  Workgroups are dispatched round-robin
// over the 8 XCDs; the remap gives each XCD a contiguous range of tiles, and
// the range is walked in groups of 8 R tiles so that the blocks resident on one
// XCD at a time share their weight and activation tiles in that XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int nb, int tiles_r, int tiles_t, int& tr, int& tt) {
    const int xcd = bid & 7, loc = bid >> 3;
    const int base = nb >> 3, rem = nb & 7;
    const int id = xcd * base + (xcd < rem ? xcd : rem) + loc;
    const int GR = 8;
    const int per_group = GR * tiles_t;
    const int grp = id / per_group;
    const int first = grp * GR;
    const int gsz = (tiles_r - first) < GR ? (tiles_r - first) : GR;
    const int in = id - grp * per_group;
    tr = first + in % gsz;
    tt = in / gsz;
}

template <typename T, int WR, int WT, int SR, int ST>
__global__ __launch_bounds__(WR* WT * 64) void spmm_kernel(SpmmArgs a) {
    using G = Geo<T>;
    using TL = Tile<T, WR, WT, SR, ST>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave % WR, wt = wave / WR;
    const int nb = gridDim.x;
    int tr, tt;
    tile_of(blockIdx.x, nb, a.tiles_r, a.tiles_t, tr, tt);
    const int64_t r0 = (int64_t)tr * TL::BR, t0 = (int64_t)tt * TL::BT;
    const int split = blockIdx.y;
    const int s_begin = split * a.steps_per_split;
    const int s_end = (s_begin + a.steps_per_split) < a.nsteps ? (s_begin + a.steps_per_split) : a.nsteps;

    uint4 ra[TL::PA];
    uint32_t ri[TL::PI];
    uint4 rb[TL::PB];

    auto load_step = [&](int s) {
#pragma unroll
        for (int p = 0; p < TL::PA; ++p) {
            const int c = tid + p * TL::NT;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < TL::NA) {
                const int row = c / (G::AV / 16), part = c % (G::AV / 16);
                int64_t gr = r0 + row;
                gr = gr < a.R ? gr : a.R - 1;
                const int64_t off = (int64_t)s * G::AV + part * 16;
                if (off < a.comp_bytes)
                    v = *(const uint4*)(a.vals + gr * a.ldv * (int64_t)sizeof(T) + off);
            }
            ra[p] = v;
        }
#pragma unroll
        for (int p = 0; p < TL::PI; ++p) {
            const int c = tid + p * TL::NT;
            uint32_t v = 0x44444444u;  // padding groups: positions (0,1) with zero values
            if (c < TL::NI) {
                const int row = c / G::AI, part = c % G::AI;
                int64_t gr = r0 + row;
                gr = gr < a.R ? gr : a.R - 1;
                const int64_t w = (int64_t)s * G::AI + part;
                if (w < a.idx_words) v = a.idx[gr * a.ldi + w];
            }
            ri[p] = v;
        }
#pragma unroll
        for (int p = 0; p < TL::PB; ++p) {
            const int c = tid + p * TL::NT;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (c < TL::NB) {
                const int row = c / 8, part = c % 8;
                const int64_t gt = t0 + row;
                const int64_t col = (int64_t)s * G::KO + part * (16 / (int)sizeof(T));
                if (gt < a.Mtok && col < a.K)
                    v = *(const uint4*)(a.X + (gt * a.ldx + col) * (int64_t)sizeof(T));
            }
            rb[p] = v;
        }
    };

    auto store_step = [&](int buf) {
        uint8_t* sA = smem + buf * TL::STAGE;
        uint32_t* sI = (uint32_t*)(sA + TL::A_BYTES);
        uint8_t* sB = sA + TL::A_BYTES + TL::I_BYTES;
#pragma unroll
        for (int p = 0; p < TL::PA; ++p) {
            const int c = tid + p * TL::NT;
            if (c < TL::NA) {
                const int row = c / (G::AV / 16), part = c % (G::AV / 16);
                *(uint4*)(sA + row * G::AVS + part * 16) = ra[p];
            }
        }
#pragma unroll
        for (int p = 0; p < TL::PI; ++p) {
            const int c = tid + p * TL::NT;
            if (c < TL::NI) {
                const int row = c / G::AI, part = c % G::AI;
                sI[row * G::AIS + part] = ri[p];
            }
        }
#pragma unroll
        for (int p = 0; p < TL::PB; ++p) {
            const int c = tid + p * TL::NT;
            if (c < TL::NB) {
                const int row = c / 8, part = c % 8;
                *(uint4*)(sB + row * G::BS + part * 16) = rb[p];
            }
        }
    };

    using AccV = typename Mma<T>::Acc;
    AccV acc[SR][ST];
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[i][j] = AccV{};

    const int h = lane >> 5, l32 = lane & 31;

    if (s_begin < s_end) {
        load_step(s_begin);
        store_step(0);
        __syncthreads();
    }
    for (int s = s_begin; s < s_end; ++s) {
        const int buf = (s - s_begin) & 1;
        const bool more = (s + 1) < s_end;
        if (more) load_step(s + 1);
        const uint8_t* sA = smem + buf * TL::STAGE;
        const uint32_t* sI = (const uint32_t*)(sA + TL::A_BYTES);
        const uint8_t* sB = sA + TL::A_BYTES + TL::I_BYTES;
#pragma unroll
        for (int d = 0; d < G::ND; ++d) {
            uint4 fa[SR];
            uint32_t fi[SR];
            uint4 fb[ST][2];
#pragma unroll
            for (int i = 0; i < SR; ++i) {
                const int row = (wr * SR + i) * 32 + l32;
                fa[i] = *(const uint4*)(sA + row * G::AVS + d * 32 + h * 16);
                if constexpr (sizeof(T) == 2) fi[i] = sI[row * G::AIS + d] >> (16 * h);
                else fi[i] = sI[row * G::AIS + 2 * d + h];
            }
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                const int tok = (wt * ST + j) * 32 + l32;
                fb[j][0] = *(const uint4*)(sB + tok * G::BS + d * 64 + h * 16);
                fb[j][1] = *(const uint4*)(sB + tok * G::BS + d * 64 + 32 + h * 16);
            }
#pragma unroll
            for (int i = 0; i < SR; ++i)
#pragma unroll
                for (int j = 0; j < ST; ++j) {
                    const uint4 b0 = fb[j][0], b1 = fb[j][1];
                    const i32x8_t bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                                        (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
                    acc[i][j] = Mma<T>::run(__builtin_bit_cast(i32x4_t, fa[i]), bv, acc[i][j], (int)fi[i]);
                }
        }
        if (more) store_step(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds token column l32, rows 8*(e/4) + 4*h + e%4 of each sub-tile
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const int64_t tok = t0 + (wt * ST + j) * 32 + l32;
            if (tok >= a.Mtok) continue;
            const int64_t rbase = r0 + (wr * SR + i) * 32 + 4 * h;
            float xs = 1.0f;
            if (a.scaled && a.x_scale) xs = a.x_scale[tok];
            const float sc = __fmul_rn(a.w_scale, xs);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t rr = rbase + 8 * g;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t r = rr + e;
                    if (r >= a.R) continue;
                    const auto v = acc[i][j][4 * g + e];
                    if (a.part) {
                        const int64_t o = ((int64_t)split * a.Mtok + tok) * a.R + r;
                        ((typename Mma<T>::AccS*)a.part)[o] = v;
                        continue;
                    }
                    const int64_t o = tok * a.ldy + r;
                    if (a.ydt == NM_I32) {
                        ((int32_t*)a.Y)[o] = (int32_t)v;
                    } else {
                        const float f = a.scaled ? __fmul_rn(sc, (float)v) : (float)v;
                        if (a.ydt == NM_F32) ((float*)a.Y)[o] = f;
                        else ((uint16_t*)a.Y)[o] = (uint16_t)f32_to_bf16_bits(f);
                    }
                }
            }
        }
}


// ------------------------------------------------------------------ ring-pipelined kernel (plain 2:4, many tokens)
// Block tile WRN*SR*32 weight rows x WTN*ST*32 tokens, WRN x WTN waves, each wave
// SR x ST 32x32 SMFMAC tiles.  Operands stream from global memory straight into
// an NS-stage LDS ring with global_load_lds (16 bytes per lane, placed
// lane-major), so no registers stage them and NS-1 stages are in flight while
// one is consumed.  The loads are issued from inline assembly and counted by
// hand (s_waitcnt vmcnt), and the stage hand-off uses an LDS-only barrier, so
// the compiler never drains the whole ring.
// LDS layouts (16-byte chunks XOR-swizzled so that any 16 consecutive rows of
// a fragment read hit distinct banks):
//   A values: row r (64 B = 4 chunks), logical chunk c stored at c ^ ((r>>2)&3)
//   A index : row r, AI words, unswizzled
//   X       : token t (128 B = 8 chunks), logical chunk c stored at c ^ ((t>>1)&7)
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
__device__ __forceinline__ void dma16(uint32_t lds, const void* g) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// A block-uniform pointer, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// saddr form: uniform 64-bit base in SGPRs + per-lane 32-bit byte offset
__device__ __forceinline__ void dma16s(uint32_t lds, const void* base, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4s(uint32_t lds, const void* base, uint32_t off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const void* g) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// Wait until at most N vector-memory loads of this wave are in flight and all its LDS
// reads are done, then meet the other waves.  The wait is a compiler builtin, so the
// compiler's own wait-count bookkeeping knows that every earlier LDS read has completed;
// the barrier is an opaque statement that no memory access moves across.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_sched_barrier(0);  // SMFMACs written after the barrier stay after it
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));  // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Index words are read from LDS one dword per lane.  Such a read is served a half-wave
// (32 lanes) at a time over 32 dword banks (measured with an LDS probe and the bank-conflict
// counter), and the 32 lanes of a half-wave read one word from each of 32 consecutive rows.
// A row of W index words (W a power of two, at most 32) therefore keeps logical word w at
// w ^ iswz<W>(r), r counted from a multiple of 32: the 32 reads then hit 32 distinct banks.
// Rows padded to a whole number of 16-byte pieces and swizzled by piece instead reach only
// 8 banks (a 4-way conflict, 4x the read time).
template <int W>
__device__ __forceinline__ int iswz(int r) {
    static_assert(W >= 1 && W <= 32 && (W & (W - 1)) == 0, "W a power of two up to 32");
    return (r / (32 / W)) & (W - 1);
}

// A global_load_lds instruction costs about the same per 128-byte line it touches
// whatever part of the line it uses (measured on the hardware), and a row's index
// words for one stage fill only a few bytes of a line.  With IG > 1 the index
// words are therefore loaded for IG stages at once (IG consecutive 16-byte pieces
// of a row), into two group buffers after the ring: group h (stages h*IG ..
// h*IG+IG-1) is loaded in IG batches of rows, one batch with each of the stages
// (h-1)*IG+1 .. h*IG, so every stage issues the same number of loads.  Within a
// row of a group buffer, piece c is stored at c ^ ((r>>2) & (IG-1)), and a lane reads
// its row's piece of a stage (the index words of all its depths) with one 16-byte read
// at the stage's first depth: under that swizzle the 16 lanes served together hit
// distinct banks.  Without groups (IG == 1) the index words travel one dword per lane
// and each row of AI words is stored swizzled word by word (iswz), so that the
// per-depth dword reads are conflict-free.
template <typename T, int SR, int ST, int KB, int NS, int WRN, int WTN, int IG = 1>
struct Ring {
    static constexpr int NW = WRN * WTN;               // waves per block (WRN along rows, WTN along tokens)
    static constexpr int BR = WRN * SR * 32;           // weight rows per block
    static constexpr int BT = WTN * ST * 32;           // tokens per block
    static constexpr int KO = KB / (int)sizeof(T);     // original columns per stage (KB bytes of X per token)
    static constexpr int KL = KO;
    static constexpr int KDEP = sizeof(T) == 2 ? 32 : 64;
    static constexpr int ND = KL / KDEP;               // SMFMAC depths per stage
    static constexpr int AROW = KL / 2 * (int)sizeof(T);  // compressed bytes per weight row per stage
    static constexpr int ACH = AROW / 16;              // 16-byte chunks per weight row per stage
    static constexpr int AI = KL / 32;                 // index words per row per stage
    static constexpr int A_OFF = 0;
    static constexpr int I_OFF = BR * AROW;                           // IG == 1: index words in the stage
    static constexpr int B_OFF = I_OFF + (IG == 1 ? BR * AI * 4 : 0);
    static constexpr int STAGE = B_OFF + BT * KB;
    static constexpr int IGRP = BR * AI * 4 * IG;                     // IG > 1: bytes of one index group
    static constexpr int G_OFF = NS * STAGE;                          // IG > 1: the two group buffers
    static constexpr int LDS = NS * STAGE + (IG > 1 ? 2 * IGRP : 0);
    static constexpr int NA = BR * AROW / 1024 / NW;   // A wave-instructions per wave
    // index loads per wave: 16-byte pieces per batch (IG > 1), else dwords per stage
    static constexpr int NI = IG > 1 ? IGRP / 1024 / NW / IG : BR * AI * 4 / 256 / NW;
    static constexpr int NB = BT * KB / 1024 / NW;     // X wave-instructions per wave
    static constexpr int PER = NA + NI + NB;           // loads per wave per stage
    static_assert(LDS <= 160 * 1024, "LDS ring too large");
    static_assert(NA >= 1 && NI >= 1 && NB >= 1, "tile too small for its waves");
    static_assert(BR * AROW % (1024 * NW) == 0 && BT * KB % (1024 * NW) == 0, "loads must split evenly over the waves");
    static_assert(IG > 1 || BR * AI * 4 % (256 * NW) == 0, "index loads must split evenly over the waves");
    // grouped index loads: the ring waits for every load at each stage end (NS == 2), one
    // 16-byte piece per row per stage holding one word per depth (bf16), and a power-of-two
    // group
    static_assert(IG == 1 || (NS == 2 && AI * 4 == 16 && sizeof(T) == 2 && (IG & (IG - 1)) == 0 &&
                              IGRP % (1024 * NW * IG) == 0),
                  "grouped index loads need NS == 2, bf16 with 16 index bytes per row per stage, IG a power of two");
    static_assert(AI <= 32 && (AI & (AI - 1)) == 0, "index words per row a power of two");
    static_assert(ND % 2 == 0, "depth ping-pong needs an even depth count");
    static_assert(ACH == 4 || ACH == 8, "weight-row chunk count without a swizzle");
    // Swizzles of 16-byte chunks, so that the 16 lanes served together by a 16-byte LDS read
    // hit distinct banks (checked on the hardware with an LDS probe):
    //   weight rows: logical chunk c at c ^ swa(r);  X rows: logical chunk c at c ^ swb(t).
    __device__ static int swa(int r) { return AROW == 64 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
    __device__ static int achunk(int r, int c) { return c ^ swa(r); }      // physical chunk of logical c
    __device__ static int alogical(int r, int p) { return p ^ swa(r); }    // logical chunk at physical p
    __device__ static int swb(int t) { return KB == 128 ? ((t >> 1) & 7) : (t & 15); }
};

template <int SR, int ST>
struct RingFrag {          // fragments of one SMFMAC depth
    i32x4_t a[SR];         // compressed values per row sub-tile
    uint32_t iw[SR];       // index fields per row sub-tile
    i32x8_t b[ST];         // X fragment per token sub-tile
};

// Adds the adapter term sum_j u[t, j] B[o, j] to a wave's SR x ST accumulator tiles
// (rows from rw, tokens from tw) with dense bf16 MFMA (v_mfma_f32_32x32x16_bf16), whose
// accumulator layout equals the sparse instruction's: the B rows are the A operand (lane
// l: row l%32, 8 consecutive ranks from 8*(l/32)), the u rows the B operand.  rank is a
// multiple of 8, so each lane's 8 ranks are all inside or all past the end (then zero).
// Rows and tokens past the edges read the last valid one; their outputs are not stored.
template <int SR, int ST>
__device__ __forceinline__ void add_lowrank(const SpmmArgs& a, f32x16_t (&acc)[SR][ST], int64_t rw, int64_t tw,
                                            int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    for (int k0 = 0; k0 < a.rank; k0 += 16) {
        const bool ok = k0 + 8 * h < a.rank;
        i32x4_t bl[SR], uu[ST];
#pragma unroll
        for (int i = 0; i < SR; ++i) {
            const int64_t r = rw + i * 32 + l32 < a.R ? rw + i * 32 + l32 : a.R - 1;
            bl[i] = ok ? *(const i32x4_t*)(a.lr_b + r * a.ldb + k0 + 8 * h) : i32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const int64_t t = tw + j * 32 + l32 < a.Mtok ? tw + j * 32 + l32 : a.Mtok - 1;
            uu[j] = ok ? *(const i32x4_t*)(a.lr_u + t * a.ldu + k0 + 8 * h) : i32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < SR; ++i)
#pragma unroll
            for (int j = 0; j < ST; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bl[i]),
                                                                   __builtin_bit_cast(bf16x8_t, uu[j]), acc[i][j], 0, 0, 0);
    }
}

// Words of the wave-private LDS buffer store_tile needs: SR sub-tiles x 64 lanes x 16
// accumulators, each lane's 16 padded to 20 words (16-byte pieces of 16 consecutive lanes
// then fall on distinct banks).
template <int SR>
constexpr int kStageWords = SR * 64 * 20;

// Stores a wave's SR x ST accumulator tiles (rows from rw, tokens from tw).  A lane
// holds token column l32 and rows 8*(e/4) + 4*h + e%4 of each 32x32 sub-tile.
// bf16 tiles fully inside Y (inside) with 8-byte aligned rows are stored straight from
// the accumulators, four consecutive rows per 8-byte store (measured as fast as staging
// for them).  Everything else goes through a wave-private LDS buffer of kStageWords<SR>
// words (stage, 16-byte aligned), since 4-byte outputs stored straight would scatter
// every instruction over 32 token rows of Y: each 32-token column of sub-tiles is written
// to LDS as whole accumulator vectors (stores of single extracted elements have been
// miscompiled), read back as 4-row runs of one token (a lane's elements 4q..4q+3 are 4
// consecutive rows), and stored as whole runs of Y's rows (32 lanes per token, 4
// outputs per lane), scaled and converted on the way.  The caller has finished every
// other use of the buffer.
template <typename T, int SR, int ST>
__device__ __forceinline__ void store_tile(const SpmmArgs& a, const typename Mma<T>::Acc (&acc)[SR][ST], int64_t rw,
                                           int64_t tw, bool inside, uint32_t* stage, int lane) {
    using AccV = typename Mma<T>::Acc;
    using AccS = typename Mma<T>::AccS;
    static_assert(SR == 4, "one token row of the wave's tile (4 sub-tiles) per half-wave");
    const int h = lane >> 5, l32 = lane & 31;
    if (inside && a.ydt == NM_BF16 && ((uintptr_t)a.Y % 8) == 0 && (a.ldy % 4) == 0) {
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const int64_t tok = tw + j * 32 + l32;
            const float sc = a.scaled ? __fmul_rn(a.w_scale, a.x_scale ? a.x_scale[tok] : 1.0f) : 1.0f;
#pragma unroll
            for (int i = 0; i < SR; ++i) {
                uint16_t* yrow = (uint16_t*)a.Y + tok * a.ldy + rw + i * 32 + 4 * h;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float f[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = (float)acc[i][j][4 * g + e];
                        if (a.scaled) f[e] = __fmul_rn(sc, f[e]);
                    }
                    *(uint2*)(yrow + 8 * g) = make_uint2(f32_to_bf16_bits(f[0]) | (f32_to_bf16_bits(f[1]) << 16),
                                                         f32_to_bf16_bits(f[2]) | (f32_to_bf16_bits(f[3]) << 16));
                }
            }
        }
        return;
    }
    const int es = a.ydt == NM_BF16 ? 2 : 4;
    // 16-byte (4-byte outputs) or 8-byte (bf16) vector stores need aligned rows of Y
    const bool vec = ((uintptr_t)a.Y % (4 * es)) == 0 && (a.ldy * es) % (4 * es) == 0;
    // reader: lane l32 of a half-wave takes rows 4*l32 .. 4*l32+3 of the wave's 128, which
    // are elements 4q .. 4q+3 of lane (token + 32 h') in sub-tile i
    const int ri = l32 >> 3, rq = (l32 & 7) >> 1, rh = l32 & 1;
#pragma unroll
    for (int j = 0; j < ST; ++j) {
#pragma unroll
        for (int i = 0; i < SR; ++i) *(AccV*)&stage[(i * 64 + lane) * 20] = acc[i][j];
        // lgkmcnt(0): this wave's LDS writes are done before any lane reads another's
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll 4
        for (int p = 0; p < 16; ++p) {
            const int tk = 2 * p + h;   // lanes 0-31 and 32-63 take two tokens per pass
            const int64_t tok = tw + j * 32 + tk;
            const uint4 raw = *(const uint4*)&stage[(ri * 64 + tk + 32 * rh) * 20 + 4 * rq];
            const int64_t r = rw + 4 * l32;
            if (tok >= a.Mtok || r >= a.R) continue;
            const AccS v[4] = {__builtin_bit_cast(AccS, raw.x), __builtin_bit_cast(AccS, raw.y),
                               __builtin_bit_cast(AccS, raw.z), __builtin_bit_cast(AccS, raw.w)};
            const int64_t o = tok * a.ldy + r;
            const bool full = vec && r + 3 < a.R;
            if (a.ydt == NM_I32) {
                if (full) {
                    *(uint4*)((int32_t*)a.Y + o) = raw;
                } else {
                    for (int e = 0; e < 4 && r + e < a.R; ++e) ((int32_t*)a.Y)[o + e] = (int32_t)v[e];
                }
                continue;
            }
            float f[4];
            if (a.scaled) {
                const float sc = __fmul_rn(a.w_scale, a.x_scale ? a.x_scale[tok] : 1.0f);
#pragma unroll
                for (int e = 0; e < 4; ++e) f[e] = __fmul_rn(sc, (float)v[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) f[e] = (float)v[e];
            }
            if (a.ydt == NM_F32) {
                if (full) {
                    *(float4*)((float*)a.Y + o) = make_float4(f[0], f[1], f[2], f[3]);
                } else {
                    for (int e = 0; e < 4 && r + e < a.R; ++e) ((float*)a.Y)[o + e] = f[e];
                }
            } else {
                if (full) {
                    *(uint2*)((uint16_t*)a.Y + o) = make_uint2(f32_to_bf16_bits(f[0]) | (f32_to_bf16_bits(f[1]) << 16),
                                                               f32_to_bf16_bits(f[2]) | (f32_to_bf16_bits(f[3]) << 16));
                } else {
                    for (int e = 0; e < 4 && r + e < a.R; ++e) ((uint16_t*)a.Y)[o + e] = (uint16_t)f32_to_bf16_bits(f[e]);
                }
            }
        }
        // the next column of sub-tiles overwrites the buffer only after every lane has read it
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }
}

// NS-stage LDS ring of KB bytes of X per token per stage; see the comment block above.
template <typename T, int SR, int ST, int KB, int NS, int WRN, int WTN, int OCC = 1, int IG = 1>
__global__ __launch_bounds__(64 * WRN * WTN, OCC) void spmm_ring_kernel(SpmmArgs a) {
    using RG = Ring<T, SR, ST, KB, NS, WRN, WTN, IG>;
    using FR = RingFrag<SR, ST>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[RG::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % WRN, wt = wave / WRN;
    int tr, tt;
    tile_of(blockIdx.x, gridDim.x, a.tiles_r, a.tiles_t, tr, tt);
    const int64_t r0 = (int64_t)tr * RG::BR, t0 = (int64_t)tt * RG::BT;
    // gridDim.y > 1: the stages split over blocks (split blockIdx.y takes stages s_begin ..
    // s_begin + nsteps - 1 and writes f32 / i32 partials); stage indices below are local
    const int spp = gridDim.y > 1 ? a.steps_per_split : a.nsteps;
    const int split = blockIdx.y, s_begin = split * spp;
    const int nsteps = a.nsteps - s_begin < spp ? a.nsteps - s_begin : spp;
    const uint32_t sbase = lds_addr(smem);
    const int64_t es = sizeof(T);

    // per-lane byte offsets (from the block's base pointers, which live in SGPRs)
    // at stage 0; stage s adds s * (row bytes per stage)
    constexpr int ACH = RG::AROW / 16, BCH = KB / 16;  // 16-byte chunks per row
    const void* baseA = uniform_ptr(a.vals + r0 * a.ldv * es);
    const void* baseI = uniform_ptr(a.idx + r0 * a.ldi);
    const void* baseB = uniform_ptr(a.X + t0 * a.ldx * es);
    const int64_t rmax = a.R - 1 - r0, tmax = a.Mtok - 1 - t0;
    uint32_t oA[RG::NA], oI[RG::NI], oB[RG::NB];
    // IG > 1: per batch p and instruction i, the row's byte offset and the piece (stage of the group)
    uint32_t gI[IG > 1 ? IG : 1][RG::NI];
    int gC[IG > 1 ? IG : 1][RG::NI];
    if constexpr (IG > 1) {
#pragma unroll
        for (int p = 0; p < IG; ++p)
#pragma unroll
            for (int i = 0; i < RG::NI; ++i) {
                const int q = ((p * RG::NW + wave) * RG::NI + i) * 64 + lane;   // 16-byte slot of the group buffer
                const int row = q / IG, c = (q % IG) ^ ((row >> 2) & (IG - 1));
                const int64_t gr = row < rmax ? row : rmax;
                gI[p][i] = (uint32_t)(gr * a.ldi * 4);
                gC[p][i] = c;
            }
    }
#pragma unroll
    for (int i = 0; i < RG::NA; ++i) {
        const int q = (wave * RG::NA + i) * 64 + lane;       // 16-byte chunk of the block's stage, row-major
        const int row = q / ACH, c = RG::alogical(row, q % ACH);
        const int64_t gr = row < rmax ? row : rmax;
        oA[i] = (uint32_t)(gr * a.ldv * es + c * 16);
    }
#pragma unroll
    for (int i = 0; i < RG::NI; ++i) {
        const int q = (wave * RG::NI + i) * 64 + lane;  // dword slot of the stage's [BR, AI] index block
        const int row = q / RG::AI, lw = (q % RG::AI) ^ iswz<RG::AI>(row);
        const int64_t gr = row < rmax ? row : rmax;
        oI[i] = (uint32_t)(gr * a.ldi * 4 + lw * 4);
    }
#pragma unroll
    for (int i = 0; i < RG::NB; ++i) {
        const int row = (wave * RG::NB + i) * (64 / BCH) + lane / BCH;
        const int c = (lane % BCH) ^ RG::swb(row);
        const int64_t gt = row < tmax ? row : tmax;
        oB[i] = (uint32_t)(gt * a.ldx * es + c * 16);
    }
    // IG > 1: batch p of index group g (stages past the last are clamped to it: read, never used)
    auto issue_group = [&](int g, int p) __attribute__((always_inline)) {
        const uint32_t gb = sbase + (uint32_t)(RG::G_OFF + (g & 1) * RG::IGRP);
#pragma unroll
        for (int i = 0; i < RG::NI; ++i) {
            const int stg = g * IG + gC[p][i];
            const int sc = s_begin + (stg < nsteps ? stg : nsteps - 1);
            dma16s(gb + (uint32_t)(((p * RG::NW + wave) * RG::NI + i) * 1024), baseI, gI[p][i] + (uint32_t)(sc * 16));
        }
    };
    auto issue = [&](int s) __attribute__((always_inline)) {
        const uint32_t st = sbase + (uint32_t)((s % NS) * RG::STAGE);
        const int sg = s_begin + s;   // the stage's place in the whole K
#pragma unroll
        for (int i = 0; i < RG::NA; ++i)
            dma16s(st + RG::A_OFF + (wave * RG::NA + i) * 1024, baseA, oA[i] + (uint32_t)(sg * RG::AROW));
        if constexpr (IG > 1) {
            // stage s >= 1 carries batch (s-1) % IG of group (s-1) / IG + 1; group 0 is loaded up front
            if (s >= 1) issue_group((s - 1) / IG + 1, (s - 1) % IG);
        } else {
#pragma unroll
            for (int i = 0; i < RG::NI; ++i)
                dma4s(st + RG::I_OFF + (wave * RG::NI + i) * 256, baseI, oI[i] + (uint32_t)(sg * RG::AI * 4));
        }
#pragma unroll
        for (int i = 0; i < RG::NB; ++i)
            dma16s(st + RG::B_OFF + (wave * RG::NB + i) * 1024, baseB, oB[i] + (uint32_t)(sg * KB));
    };
    const int h = lane >> 5, l32 = lane & 31;
    i32x4_t ipc[SR];   // IG > 1: the current stage's index piece of each row sub-tile (one word per depth)
    auto read_depth = [&](int S, int d, FR& f) __attribute__((always_inline)) {
        const int slot = S % NS;
        const uint8_t* sA = smem + slot * RG::STAGE + RG::A_OFF;
        const uint32_t* sI = (const uint32_t*)(smem + slot * RG::STAGE + RG::I_OFF);
        const uint8_t* sB = smem + slot * RG::STAGE + RG::B_OFF;
        const uint32_t* sG = (const uint32_t*)(smem + RG::G_OFF + ((S / IG) & 1) * RG::IGRP);
#pragma unroll
        for (int i = 0; i < SR; ++i) {
            const int row = (wr * SR + i) * 32 + l32;
            f.a[i] = *(const i32x4_t*)(sA + row * RG::AROW + RG::achunk(row, 2 * d + h) * 16);
            // bf16: the lane's 16 index bits are selected (shifted by 16h) at the SMFMAC, so
            // that no VALU op waits on this read ahead of unrelated SMFMACs
            if constexpr (IG > 1) {
                if (d == 0) ipc[i] = *(const i32x4_t*)(sG + row * (4 * IG) + ((S % IG) ^ ((row >> 2) & (IG - 1))) * 4);
                f.iw[i] = (uint32_t)ipc[i][d];
            } else {
                f.iw[i] = sI[row * RG::AI + ((sizeof(T) == 2 ? d : 2 * d + h) ^ iswz<RG::AI>(row))];
            }
        }
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const int tok = (wt * ST + j) * 32 + l32;
            const uint8_t* trow = sB + tok * KB;
            const int sw = RG::swb(tok);
            const i32x4_t lo = *(const i32x4_t*)(trow + ((4 * d + h) ^ sw) * 16);
            const i32x4_t hi = *(const i32x4_t*)(trow + ((4 * d + 2 + h) ^ sw) * 16);
            f.b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    using AccV = typename Mma<T>::Acc;
    AccV acc[SR][ST];
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[i][j] = AccV{};

    const uint32_t ish = 16u * (uint32_t)h;
    auto mfmas = [&](const FR& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SR; ++i)
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                acc[i][j] = Mma<T>::run(f.a[i], f.b[j], acc[i][j], (int)(sizeof(T) == 2 ? f.iw[i] >> ish : f.iw[i]));
            }
    };

    // Prologue: stages 0..NS-1 fill the ring; wait for stage 0 (the other NS-1
    // may stay in flight) and read its depth 0.  Every depth step reads the next
    // depth's fragments before issuing the current depth's SMFMACs.  The last
    // depth of stage S waits for stage S+1 (stages S+2..S+NS-1 may stay in
    // flight), passes the barrier, reads depth 0 of stage S+1 and refills the
    // slot of stage S (fully read into registers by every wave) with stage S+NS.
    FR fa, fb;
    if constexpr (IG > 1) {
        if (nsteps > 0) {
#pragma unroll
            for (int p = 0; p < IG; ++p) issue_group(0, p);
        }
    }
#pragma unroll
    for (int p = 0; p < NS; ++p)
        if (p < nsteps) issue(p);
    if (nsteps >= NS) wait_vm_barrier<(NS - 1) * RG::PER>();
    else wait_vm_barrier<0>();
    if (nsteps > 0) read_depth(0, 0, fa);
    // One stage.  HasNext (all but the last stage) hands over to stage S+1 at its last
    // depth; the last stage is peeled off so that the steady-state loop carries no
    // branch around LDS reads, which keeps the compiler's wait counts exact.
    auto stage = [&](int S, auto has_next) __attribute__((always_inline)) {
#pragma unroll
        for (int d = 0; d < RG::ND; d += 2) {
            read_depth(S, d + 1, fb);
            mfmas(fa);
            if (d + 2 < RG::ND) {
                read_depth(S, d + 2, fa);
            } else if constexpr (decltype(has_next)::value) {
                if (S + NS - 1 < nsteps) wait_vm_barrier<(NS - 2) * RG::PER>();
                else wait_vm_barrier<0>();
                read_depth(S + 1, 0, fa);
                if (S + NS < nsteps) issue(S + NS);
            }
            mfmas(fb);
        }
    };
    int S = 0;
    for (; S + 1 < nsteps; ++S) stage(S, std::true_type{});
    if (S < nsteps) stage(S, std::false_type{});
    wait_vm_all();
    if constexpr (sizeof(T) == 2) {   // the adapter term once, in the first split
        if (a.rank > 0 && split == 0) add_lowrank<SR, ST>(a, acc, r0 + wr * SR * 32, t0 + wt * ST * 32, lane);
    }

    // every wave has finished reading the ring: its LDS becomes the output staging buffers
    __syncthreads();
    static_assert(RG::LDS >= RG::NW * kStageWords<SR> * 4, "staging buffers fit in the ring");
    if (a.part) {   // this split's partial tile, unscaled, into [split][Mtok][R]
        SpmmArgs b = a;
        using AccS = typename Mma<T>::AccS;
        b.Y = (AccS*)a.part + (int64_t)split * a.Mtok * a.R;
        b.ydt = std::is_same<AccS, float>::value ? NM_F32 : NM_I32;
        b.ldy = a.R;
        b.scaled = 0;
        store_tile<T, SR, ST>(b, acc, r0 + wr * SR * 32, t0 + wt * ST * 32, false, (uint32_t*)smem + wave * kStageWords<SR>,
                              lane);
        return;
    }
    store_tile<T, SR, ST>(a, acc, r0 + wr * SR * 32, t0 + wt * ST * 32, r0 + RG::BR <= a.R && t0 + RG::BT <= a.Mtok,
                          (uint32_t*)smem + wave * kStageWords<SR>, lane);
}

// ------------------------------------------------------------------ split ring kernel (256 x 256 tiles)
// A 256 x 256 tile moves about a third fewer bytes per multiply-add than the 256 x 128
// tile of the ring kernel, but a whole stage of it (256 bytes of X per token) does not
// fit twice in LDS, and a 128-byte stage leaves each weight row's values for the stage
// in half a line (a DMA instruction costs the same per line touched, whatever it uses).
// Here the operands travel in separate buffers, each loaded in whole 128-byte lines:
//   X      : a two-stage ring of 128 bytes per token per stage,
//   values : groups of two stages (128 bytes per weight row), double-buffered,
//   indices: groups of 64 bytes per weight row (IGS stages), double-buffered, each
//            loaded in IB batches of rows, one batch per value group.
// A loop iteration multiplies one value group (two stages).  At its top (after the
// barrier that ends the previous group) it issues X stage 2g+1, the next value group and
// one index batch; between its two stages it issues X stage 2g+2.  Every load is waited
// for with an exact s_waitcnt vmcnt count, as loads of a wave complete in order.  Eight
// waves (two per SIMD) of 128 x 64 each cover the tile; LDS holds exactly 160 KB.
// Requires an even stage count (K a multiple of 256 bytes of X per token).
template <typename T, int SR, int ST, int WRN, int WTN, int IP = 16>
struct Ring2 {
    static constexpr int NW = WRN * WTN;
    static constexpr int BR = WRN * SR * 32;           // weight rows per block
    static constexpr int BT = WTN * ST * 32;           // tokens per block
    static constexpr int KB = 128;                     // X bytes per token per stage
    static constexpr int KO = KB / (int)sizeof(T);     // columns per stage
    static constexpr int KDEP = sizeof(T) == 2 ? 32 : 64;
    static constexpr int ND = KO / KDEP;               // SMFMAC depths per stage (2)
    static constexpr int AROW = KO / 2 * (int)sizeof(T);   // value bytes per row per stage (64)
    static constexpr int AI = KO / 32;                 // index words per row per stage
    static constexpr int IGS = 64 / (AI * 4);          // stages per index group
    static constexpr int IB = IGS / 2;                 // index batches per group (one per value group)
    static constexpr int XSTAGE = BT * KB;
    static constexpr int AGRP = BR * 2 * AROW;         // one value group: two stages
    static constexpr int IGRP = BR * 64;               // one index group
    static constexpr int X_OFF = 0;
    static constexpr int A_OFF = 2 * XSTAGE;
    static constexpr int I_OFF = A_OFF + 2 * AGRP;
    static constexpr int LDS = I_OFF + 2 * IGRP;
    static constexpr int NBX = XSTAGE / 1024 / NW;     // X loads per wave per stage
    static constexpr int NAG = AGRP / 1024 / NW;       // value loads per wave per group
    static constexpr int NIG = IGRP / IB / (64 * IP) / NW;   // index loads (IP bytes per lane) per wave per batch
    static_assert(ND == 2 && AROW == 64 && 2 * AROW == 128, "two depths of 64 value bytes per stage");
    static_assert(IGS >= 2 && IGS % 2 == 0 && IB >= 1, "index groups cover whole value groups");
    static_assert(NBX >= 1 && NAG >= 1 && NIG >= 1, "tile too small for its waves");
    static_assert(XSTAGE % (1024 * NW) == 0 && AGRP % (1024 * NW) == 0 && IGRP % (IB * 64 * IP * NW) == 0,
                  "loads must split evenly over the waves");
    static_assert(IP == 16 || IP == 4, "index loads of 16 or 4 bytes per lane");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(NBX + NAG + NIG < 64, "vmcnt is a 6-bit field");
    // 16-byte chunk swizzles (conflict-free 16-lane LDS reads):
    //   value group row r (8 chunks): logical c at c ^ ((r >> 1) & 7)
    //   X token t (8 chunks): logical c at c ^ ((t >> 1) & 7)
    //   index group row r: IP == 4, 16 words, logical word w at w ^ iswz<16>(r) (conflict-free
    //   dword reads); IP == 16, 4 pieces, logical piece p at p ^ ((r >> 2) & 3)
    __device__ static int swa(int r) { return (r >> 1) & 7; }
    __device__ static int swb(int t) { return (t >> 1) & 7; }
    __device__ static int swi(int r) { return (r >> 2) & 3; }
};

template <typename T, int SR, int ST, int WRN, int WTN, int IP = 16>
__global__ __launch_bounds__(64 * WRN * WTN, 1) void spmm_ring2_kernel(SpmmArgs a) {
    using RG = Ring2<T, SR, ST, WRN, WTN, IP>;
    using FR = RingFrag<SR, ST>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[RG::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % WRN, wt = wave / WRN;
    int tr, tt;
    tile_of(blockIdx.x, gridDim.x, a.tiles_r, a.tiles_t, tr, tt);
    const int64_t r0 = (int64_t)tr * RG::BR, t0 = (int64_t)tt * RG::BT;
    const int nsteps = a.nsteps;              // even, >= 2
    const int NG = nsteps >> 1;               // value groups = loop iterations
    const int NIGR = (nsteps + RG::IGS - 1) / RG::IGS;   // index groups
    const uint32_t sbase = lds_addr(smem);
    const int64_t es = sizeof(T);
    // the last IP index bytes of a row (a partial last index group is clamped to them)
    const uint32_t ilast = (uint32_t)(nsteps * RG::AI * 4 - IP);

    const void* baseA = uniform_ptr(a.vals + r0 * a.ldv * es);
    const void* baseI = uniform_ptr(a.idx + r0 * a.ldi);
    const void* baseB = uniform_ptr(a.X + t0 * a.ldx * es);
    const int64_t rmax = a.R - 1 - r0, tmax = a.Mtok - 1 - t0;
    uint32_t oA[RG::NAG], oI[RG::NIG], oB[RG::NBX];
    int pI[RG::NIG];
#pragma unroll
    for (int i = 0; i < RG::NAG; ++i) {
        const int q = (wave * RG::NAG + i) * 64 + lane;   // 16-byte chunk of the group buffer, row-major
        const int row = q >> 3, c = (q & 7) ^ RG::swa(row);
        const int64_t gr = row < rmax ? row : rmax;
        oA[i] = (uint32_t)(gr * a.ldv * es + c * 16);
    }
#pragma unroll
    for (int i = 0; i < RG::NIG; ++i) {
        // IP-byte unit q of one batch; row within the batch (batches start at multiples of
        // 16 rows, so the swizzle of the batch-relative row equals that of the absolute row)
        // and the unit's logical byte offset in the row's 64 bytes
        const int q = (wave * RG::NIG + i) * 64 + lane;
        const int row = q / (64 / IP), u = q % (64 / IP);
        oI[i] = (uint32_t)row;
        if constexpr (IP == 4) {
            pI[i] = (u ^ iswz<16>(row)) * 4;                    // logical byte of physical word u
        } else {
            const int pb = u * IP;                              // physical byte in the row
            pI[i] = (((pb >> 4) ^ RG::swi(row)) << 4) | (pb & 15);
        }
    }
#pragma unroll
    for (int i = 0; i < RG::NBX; ++i) {
        const int row = (wave * RG::NBX + i) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ RG::swb(row);
        const int64_t gt = row < tmax ? row : tmax;
        oB[i] = (uint32_t)(gt * a.ldx * es + c * 16);
    }
    auto issue_x = [&](int s) __attribute__((always_inline)) {
        const uint32_t st = sbase + (uint32_t)(RG::X_OFF + (s & 1) * RG::XSTAGE);
#pragma unroll
        for (int i = 0; i < RG::NBX; ++i)
            dma16s(st + (wave * RG::NBX + i) * 1024, baseB, oB[i] + (uint32_t)(s * RG::KB));
    };
    auto issue_a = [&](int g) __attribute__((always_inline)) {
        const uint32_t st = sbase + (uint32_t)(RG::A_OFF + (g & 1) * RG::AGRP);
#pragma unroll
        for (int i = 0; i < RG::NAG; ++i)
            dma16s(st + (wave * RG::NAG + i) * 1024, baseA, oA[i] + (uint32_t)(g * 2 * RG::AROW));
    };
    // batch b of index group j: rows [b * BR / IB, (b + 1) * BR / IB)
    auto issue_i = [&](int j, int b) __attribute__((always_inline)) {
        const uint32_t st = sbase + (uint32_t)(RG::I_OFF + (j & 1) * RG::IGRP + b * (RG::IGRP / RG::IB));
#pragma unroll
        for (int i = 0; i < RG::NIG; ++i) {
            const int row = b * (RG::BR / RG::IB) + (int)oI[i];
            const int64_t gr = row < rmax ? row : rmax;
            uint32_t off = (uint32_t)(j * 64 + pI[i]);
            off = off < ilast ? off : ilast;
            if constexpr (IP == 16) dma16s(st + (wave * RG::NIG + i) * 1024, baseI, (uint32_t)(gr * a.ldi * 4) + off);
            else dma4s(st + (wave * RG::NIG + i) * 256, baseI, (uint32_t)(gr * a.ldi * 4) + off);
        }
    };

    const int h = lane >> 5, l32 = lane & 31;
    auto read_depth = [&](int s, int d, FR& f) __attribute__((always_inline)) {
        const int g = s >> 1, ss = s & 1, j = s / RG::IGS, si = s % RG::IGS;
        const uint8_t* sA = smem + RG::A_OFF + (g & 1) * RG::AGRP;
        const uint32_t* sI = (const uint32_t*)(smem + RG::I_OFF + (j & 1) * RG::IGRP);
        const uint8_t* sB = smem + RG::X_OFF + (s & 1) * RG::XSTAGE;
        // X pieces first: a depth's first SMFMAC then waits only for the earliest reads
#pragma unroll
        for (int jj = 0; jj < ST; ++jj) {
            const int tok = (wt * ST + jj) * 32 + l32;
            const uint8_t* trow = sB + tok * RG::KB;
            const int sw = RG::swb(tok);
            const i32x4_t lo = *(const i32x4_t*)(trow + ((4 * d + h) ^ sw) * 16);
            const i32x4_t hi = *(const i32x4_t*)(trow + ((4 * d + 2 + h) ^ sw) * 16);
            f.b[jj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < SR; ++i) {
            const int row = (wr * SR + i) * 32 + l32;
            f.a[i] = *(const i32x4_t*)(sA + row * 128 + ((4 * ss + 2 * d + h) ^ RG::swa(row)) * 16);
            // index word w of the row's group
            const int w = si * RG::AI + (sizeof(T) == 2 ? d : 2 * d + h);
            if constexpr (IP == 4) f.iw[i] = sI[row * 16 + (w ^ iswz<16>(row))];
            else f.iw[i] = sI[row * 16 + ((w >> 2) ^ RG::swi(row)) * 4 + (w & 3)];
        }
    };

    using AccV = typename Mma<T>::Acc;
    AccV acc[SR][ST];
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[i][j] = AccV{};
    const uint32_t ish = 16u * (uint32_t)h;
    auto mfmas = [&](const FR& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SR; ++i)
#pragma unroll
            for (int j = 0; j < ST; ++j)
                acc[i][j] = Mma<T>::run(f.a[i], f.b[j], acc[i][j], (int)(sizeof(T) == 2 ? f.iw[i] >> ish : f.iw[i]));
    };

    // Issue order: prologue [values 0, index group 0, X 0]; top(g) [X 2g+1, values g+1,
    // index batch g % IB of group g / IB + 1]; mid(g) [X 2g+2].  Loads past the end are
    // not issued; the waits count exactly the loads issued after the ones needed.  Each
    // depth's fragments are read from LDS while the previous depth's SMFMACs issue.
    constexpr int NAG = RG::NAG, NIG = RG::NIG;
    FR fa, fb;
    issue_a(0);
#pragma unroll
    for (int b = 0; b < RG::IB; ++b) issue_i(0, b);
    issue_x(0);
    wait_vm_barrier<0>();
    read_depth(0, 0, fa);
    // a depth's fragment reads (SR value pieces, SR index words, 2 ST X pieces) spread over
    // the first SMFMACs of the previous depth, in a scheduling region of their own
    auto interleave = [&]() __attribute__((always_inline)) {
        constexpr int NR = 2 * SR + 2 * ST, RPM = 3;
        static_assert(NR % RPM == 0 && NR / RPM <= SR * ST, "reads spread over the depth's SMFMACs");
#pragma unroll
        for (int i = 0; i < NR / RPM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, SR * ST - NR / RPM, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int g = 0; g < NG; ++g) {
        const int s0 = 2 * g;
        const bool more = g + 1 < NG;                     // X 2g+2, values g+1 exist
        const bool it = g / RG::IB + 1 < NIGR;            // a next index group exists
        issue_x(s0 + 1);
        if (more) issue_a(g + 1);
        if (it) issue_i(g / RG::IB + 1, g % RG::IB);
        read_depth(s0, 1, fb);
        mfmas(fa);
        interleave();
        // mid(g): X s0+1 done; the values and index batch of top(g) may stay in flight
        if (more && it) wait_vm_barrier<NAG + NIG>();
        else if (more) wait_vm_barrier<NAG>();
        else wait_vm_barrier<0>();
        if (more) issue_x(s0 + 2);
        read_depth(s0 + 1, 0, fa);
        mfmas(fb);
        interleave();
        read_depth(s0 + 1, 1, fb);
        mfmas(fa);
        interleave();
        // fb complete before the branch (the barrier in it waits for them anyway), so the
        // SMFMACs after the join wait for nothing
        __builtin_amdgcn_s_waitcnt(0xc07f);
        if (more) {
            // top(g+1): X s0+2 was the last load issued, so everything is waited for
            wait_vm_barrier<0>();
            read_depth(s0 + 2, 0, fa);
        }
        mfmas(fb);
    }
    wait_vm_all();
    if constexpr (sizeof(T) == 2) {
        if (a.rank > 0) add_lowrank<SR, ST>(a, acc, r0 + wr * SR * 32, t0 + wt * ST * 32, lane);
    }

    // every wave has finished reading the ring: its LDS becomes the output staging buffers
    __syncthreads();
    static_assert(RG::LDS >= RG::NW * kStageWords<SR> * 4, "staging buffers fit in the ring");
    store_tile<T, SR, ST>(a, acc, r0 + wr * SR * 32, t0 + wt * ST * 32, r0 + RG::BR <= a.R && t0 + RG::BT <= a.Mtok,
                          (uint32_t*)smem + wave * kStageWords<SR>, lane);
}

// Score epilogue of the Hutchinson second product (a fused diagonal -> score step): the
// tile's D values (acc * scale, rounded to f32 as D would be stored) become
// s = (d + eps) * (w * w) with one rounding per operation in the order t = w*w, u = d + eps,
// s = u*t -- the score of the per-weight curvature -- and are written to S (Y, ldy) as
// whole 16-byte runs of a row; each lane also folds its scores into moments (shifted sums
// in f64 about its first score) for the per-tensor statistics.  Rows of the tile are D's
// columns k (rw ..), tokens D's rows o (tw ..); K (a.R) is a multiple of 64.
template <int SR, int ST>
__device__ __forceinline__ Moments store_score_tile(const SpmmArgs& a, const f32x16_t (&acc)[SR][ST], int64_t rw,
                                                    int64_t tw, uint32_t* stage, int lane) {
    static_assert(SR == 4, "one token row of the wave's tile (4 sub-tiles) per half-wave");
    const int h = lane >> 5, l32 = lane & 31;
    const int ri = l32 >> 3, rq = (l32 & 7) >> 1, rh = l32 & 1;
    double n = 0.0, s1 = 0.0, s2 = 0.0, c = 0.0;
#pragma unroll
    for (int j = 0; j < ST; ++j) {
#pragma unroll
        for (int i = 0; i < SR; ++i) *(f32x16_t*)&stage[(i * 64 + lane) * 20] = acc[i][j];
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll 4
        for (int p = 0; p < 16; ++p) {
            const int tk = 2 * p + h;
            const int64_t o = tw + j * 32 + tk, k = rw + 4 * l32;
            const uint4 raw = *(const uint4*)&stage[(ri * 64 + tk + 32 * rh) * 20 + 4 * rq];
            if (o >= a.Mtok || k >= a.R) continue;
            const uint2 wq = *(const uint2*)(a.sw + o * a.ldsw + k);
            const uint32_t wb[4] = {wq.x & 0xffffu, wq.x >> 16, wq.y & 0xffffu, wq.y >> 16};
            const uint32_t v[4] = {raw.x, raw.y, raw.z, raw.w};
            float sc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float d = __fmul_rn(a.w_scale, __uint_as_float(v[e]));
                const float w = bf16_bits_to_f32(wb[e]);
                sc[e] = __fmul_rn(__fadd_rn(d, a.eps), __fmul_rn(w, w));
                if (n == 0.0) c = (double)sc[e];
                const double dd = (double)sc[e] - c;
                s1 += dd;
                s2 += dd * dd;
                n += 1.0;
            }
            *(float4*)((float*)a.Y + o * a.ldy + k) = make_float4(sc[0], sc[1], sc[2], sc[3]);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }
    Moments m{n, n > 0.0 ? c + s1 / n : 0.0, n > 0.0 ? s2 - s1 * (s1 / n) : 0.0};
    if (m.m2 < 0.0) m.m2 = 0.0;
    return m;
}

// ------------------------------------------------------------------ dense split ring (bf16)
// Y = X W^T for a dense bf16 weight W [R, K] (ldv) with the split ring's tile, waves,
// swizzles, DMA and epilogue, and dense MFMA (v_mfma_f32_32x32x16_bf16, whose operand and
// accumulator layouts are the sparse instruction's with 16-byte B fragments).  A stage is
// SK columns (SK * 2 bytes of W per row and of X per token, SK / 16 MFMA depths) in an
// NS-slot LDS ring: with a 64-column stage two slots fill 128 KB, with a 32-column stage
// five fill 160 KB and keep four stages in flight while one is multiplied.
// One barrier per stage, before its last depth: stage s+1 has landed and every wave has
// read stage s, whose slot then takes stage s+NS.  Used for the many-token product of
// weights decoded from the bitmap format and for both Hutchinson products.
// HUTCH: the Hutchinson second product D = (2/P) sum_p V_p .* (U_p X) (D [R, K] f32 as Y
// [Mtok = R rows, R = K columns]): the A operand is the transposed calibration rows XT [K, n]
// (vals), the B operand probe p's rows of U [P*R, n] (X); the stage index runs over
// (probe, stage of n).  With signs s_p = +-1 one set of accumulators carries the sum:
// before probe p's products it is multiplied by s_{p-1} s_p and after the last by
// s_{P-1}, so that after probe p it holds s_p .* (D_{p-1} + s_p .* G_p).  Each lane's
// signs are four Rademacher words per probe (its two rows of U, two 64-column blocks).
// GEN: the Hutchinson first product U [P*R, n] = V X^T: the A operand is the calibration
// rows X [n, K] (vals), the B operand the stacked probe rows q = p R + o of V, made in
// registers: a stage's 64 columns of a row are one Rademacher word, which each lane turns
// into its +-1 bf16 fragments with a few bit operations per depth.  The B operand never
// passes through LDS (measured: the whole Hutchinson call 6.62-6.74 -> 6.23-6.34 ms
// against signs written into LDS stages and read back as fragments; a 3- or 4-slot ring
// for the A stages then measured the same as 2).
// HUTCH_SCORE: HUTCH whose epilogue writes the score of D (store_score_tile) and the block's
// moments of it instead of D.
// MODE: 0 plain, 1 HUTCH, 2 GEN, 3 HUTCH_SCORE.
template <int SR, int ST, int WRN, int WTN, int MODE = 0, int SK = 64, int NS = 2>
__global__ __launch_bounds__(64 * WRN * WTN, 1) void dense_ring_kernel(SpmmArgs a) {
    constexpr bool HUTCH = MODE == 1 || MODE == 3, GEN = MODE == 2;
    constexpr int NW = WRN * WTN, BR = WRN * SR * 32, BT = WTN * ST * 32;
    constexpr int ROWB = SK * 2, CH = ROWB / 16, D = SK / 16;   // bytes and chunks per row per stage, depths
    static_assert(SK == 64 || SK == 32, "64- or 32-column stages");
    static_assert(D % 2 == 0, "depth ping-pong needs an even depth count");
    // GEN: the B operand is made in registers, so a slot holds the A stage alone
    constexpr int WSTAGE = BR * ROWB, XSTAGE = BT * ROWB, SLOT = WSTAGE + (GEN ? 0 : XSTAGE);
    constexpr int RING = NS * SLOT;
    constexpr int NWL = WSTAGE / 1024 / NW, NXL = XSTAGE / 1024 / NW;   // loads per wave per stage
    static_assert(WSTAGE % (1024 * NW) == 0 && XSTAGE % (1024 * NW) == 0 && NWL >= 1 && NXL >= 1, "loads per wave");
    constexpr int SMEM = RING > NW * kStageWords<SR> * 4 ? RING : NW * kStageWords<SR> * 4;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave % WRN, wt = wave / WRN;
    int tr, tt;
    tile_of(blockIdx.x, gridDim.x, a.tiles_r, a.tiles_t, tr, tt);
    const int64_t r0 = (int64_t)tr * BR, t0 = (int64_t)tt * BT;
    const int nsteps = a.nsteps;   // K / SK >= 1 (HUTCH: probes * stages per probe)
    const int PS = HUTCH ? a.pstages : nsteps;
    const uint32_t sbase = lds_addr(smem);
    // row / token r of CH chunks: logical chunk c at c ^ sw(r) (16 consecutive rows read by a
    // 16-byte LDS read then hit 64 distinct banks)
    auto sw = [](int r) { return CH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); };
    const void* baseW = uniform_ptr(a.vals + r0 * a.ldv * 2);
    const void* baseX = uniform_ptr(a.X + t0 * a.ldx * 2);
    const int64_t rmax = a.R - 1 - r0, tmax = a.Mtok - 1 - t0;
    uint32_t oW[NWL], oX[NXL];
    // GEN: half-wave h of a lane's B sub-tiles j = 0, 1 draws the Rademacher words of
    // sub-tile j = h's row (its stacked probe row q = p R + o); the counter of stage s is
    // gctr + s (64-column stages)
    static_assert(!GEN || (ST == 2 && SK == 64), "GEN: two token sub-tiles, one word per row and stage");
    uint64_t gctr = 0;
    if constexpr (GEN) {
        const int64_t q = t0 + (wt * ST + (lane >> 5)) * 32 + (lane & 31), qc = q < a.Mtok ? q : a.Mtok - 1;
        const int gp = (int)(qc / a.prows);
        const int64_t go = qc - (int64_t)gp * a.prows;
        gctr = ((uint64_t)gp << 40) + (uint64_t)go * (uint64_t)(a.K / 64);
    }
    constexpr int RPL = 64 / CH;   // rows per DMA instruction
#pragma unroll
    for (int i = 0; i < NWL; ++i) {
        const int row = (wave * NWL + i) * RPL + lane / CH;
        const int64_t gr = row < rmax ? row : rmax;
        oW[i] = (uint32_t)(gr * a.ldv * 2 + ((lane % CH) ^ sw(row)) * 16);
    }
#pragma unroll
    for (int i = 0; i < NXL; ++i) {
        const int row = (wave * NXL + i) * RPL + lane / CH;
        const int64_t gt = row < tmax ? row : tmax;
        oX[i] = (uint32_t)(gt * a.ldx * 2 + ((lane % CH) ^ sw(row)) * 16);
    }
    auto issue = [&](int s) __attribute__((always_inline)) {
        const uint32_t slot = sbase + (uint32_t)((s % NS) * SLOT);
        // HUTCH: stage s % PS of probe s / PS (the probe's U rows follow the previous probe's)
        const int ks = HUTCH ? s % PS : s;
        const uint32_t xp = HUTCH ? (uint32_t)(s / PS) * (uint32_t)(a.Mtok * a.ldx * 2) : 0u;
#pragma unroll
        for (int i = 0; i < NWL; ++i) dma16s(slot + (wave * NWL + i) * 1024, baseW, oW[i] + (uint32_t)(ks * ROWB));
        if constexpr (!GEN) {
#pragma unroll
            for (int i = 0; i < NXL; ++i)
                dma16s(slot + WSTAGE + (wave * NXL + i) * 1024, baseX, oX[i] + xp + (uint32_t)(ks * ROWB));
        }
    };
    struct Frag {
        i32x4_t a[SR], b[ST];
    };
    const int h = lane >> 5, l32 = lane & 31;
    auto read_depth = [&](int s, int d, Frag& f) __attribute__((always_inline)) {
        const uint8_t* sW = smem + (s % NS) * SLOT;
        const uint8_t* sX = sW + WSTAGE;
#pragma unroll
        for (int i = 0; i < SR; ++i) {
            const int row = (wr * SR + i) * 32 + l32;
            f.a[i] = *(const i32x4_t*)(sW + row * ROWB + ((2 * d + h) ^ sw(row)) * 16);
        }
        if constexpr (!GEN) {
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                const int tok = (wt * ST + j) * 32 + l32;
                f.b[j] = *(const i32x4_t*)(sX + tok * ROWB + ((2 * d + h) ^ sw(tok)) * 16);
            }
        }
    };
    // GEN: the stage's words of sub-tiles j = 0, 1 (as dword pairs) for every lane: this
    // half-wave's word and, across the halves, the other's
    auto gen_words = [&](int s, uint32_t (&w)[ST][2]) __attribute__((always_inline)) {
        const uint64_t z = splitmix64_at(a.seed, gctr + (uint64_t)s);
        const uint32_t lo = (uint32_t)z, hi = (uint32_t)(z >> 32);
        const uint32_t olo = (uint32_t)__shfl_xor((int)lo, 32), ohi = (uint32_t)__shfl_xor((int)hi, 32);
        w[0][0] = h ? olo : lo;
        w[0][1] = h ? ohi : hi;
        w[1][0] = h ? lo : olo;
        w[1][1] = h ? hi : ohi;
    };
    // GEN: depth d's B fragment of sub-tile j is columns 16 d + 8 h .. +8 of the stage, i.e.
    // sign byte 2 d + h of the row's word; bf16 pair e of it is 0x3F80 | sign << 15 for
    // columns 2e and 2e+1: with v = u | u << 15, v << (15 - 2e) carries bit 2e of u to bit
    // 15 and bit 2e+1 to bit 31
    auto make_b = [&](int d, const uint32_t (&w)[ST][2], Frag& f) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const uint32_t u = __builtin_amdgcn_ubfe(w[j][d >> 1], 16 * (d & 1) + 8 * h, 8);
            const uint32_t v = u | (u << 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) f.b[j][e] = (int)(((v << (15 - 2 * e)) & 0x80008000u) | 0x3F803F80u);
        }
    };
    f32x16_t acc[SR][ST];
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[i][j] = f32x16_t{};
    auto mfmas = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SR; ++i)
#pragma unroll
            for (int j = 0; j < ST; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.a[i]),
                                                                     __builtin_bit_cast(bf16x8_t, f.b[j]), acc[i][j], 0, 0, 0);
    };
    // HUTCH: a lane's sign words of a probe, per token sub-tile j (a row o of U) and 64-column
    // block of its A rows (sub-tiles 0-1 and 2-3), recomputed where needed rather than kept
    // live across the loop; flip multiplies acc by the signs of w
    // (element e of sub-tile i is column 64 m + 32 (i & 1) + 8 (e / 4) + 4 h + e % 4 of a
    // 64-column block m: bit 8 (e / 4) + e % 4 of the word's half i & 1 shifted down by 4 h;
    // adding bit << 31 toggles the sign bit)
    auto flip = [&](const uint64_t (&w)[ST][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SR; ++i)
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                const uint32_t x = (uint32_t)(w[j][i >> 1] >> (32 * (i & 1) + 4 * h));
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    // written out, or the compiler turns the extract and shift into a
                    // shift and a mask (three operations instead of two)
                    const uint32_t bit = __builtin_amdgcn_ubfe(x, 8 * (e / 4) + (e % 4), 1);
                    uint32_t r;
                    asm("v_lshl_add_u32 %0, %1, 31, %2" : "=v"(r) : "v"(bit), "v"(__float_as_uint(acc[i][j][e])));
                    acc[i][j][e] = __uint_as_float(r);
                }
            }
    };
    auto probe_words = [&](int p, uint64_t (&w)[ST][2]) __attribute__((always_inline)) {
        const int64_t kblocks = a.R / 64;
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const int64_t o = t0 + (wt * ST + j) * 32 + l32, oc = o < a.Mtok ? o : a.Mtok - 1;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int64_t kb = (r0 + wr * SR * 32) / 64 + b, kbc = kb < kblocks ? kb : kblocks - 1;
                w[j][b] = rad_word(a.seed, p, oc, kbc, kblocks);
            }
        }
    };
    constexpr int PER = NWL + (GEN ? 0 : NXL);   // DMA loads per stage
    // a depth's SR + ST fragment reads, one after each of its first SR + ST MFMAs (in the
    // scheduling region that holds them)
    constexpr int NRD = GEN ? SR : SR + ST;   // LDS fragment reads per depth
    auto interleave_reads_mfmas = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NRD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, SR * ST - NRD, 0);
        __builtin_amdgcn_sched_barrier(0);   // the next depth is a region of its own
    };
    // Prologue: stages 0..NS-1 fill the ring; wait for stage 0 (the others may stay in
    // flight) and read its depth 0.  Each depth's fragments are read while the previous
    // depth's MFMAs issue; the last depth of stage s waits for stage s+1 (stages s+2 ..
    // s+NS-1 may stay in flight), meets the other waves, refills stage s's slot with stage
    // s+NS and reads depth 0 of stage s+1.
    Frag fr[2];
#pragma unroll
    for (int p = 0; p < NS; ++p)
        if (p < nsteps) issue(p);
    if (nsteps >= NS) wait_vm_barrier<(NS - 1) * PER>();
    else wait_vm_barrier<0>();
    uint32_t gw[ST][2], gn[ST][2];   // GEN: the words of stages s and s + 1
    uint64_t wp[ST][2] = {};         // HUTCH: the sign words of the previous probe (none: 0)
    read_depth(0, 0, fr[0]);
    if constexpr (GEN) {
        gen_words(0, gw);
        make_b(0, gw, fr[0]);
    }
    for (int s = 0; s < nsteps; ++s) {
        if constexpr (GEN) {
            if (s + 1 < nsteps) gen_words(s + 1, gn);
        }
        if constexpr (HUTCH) {
            if (s % PS == 0) {   // probe p = s / PS begins: acc *= s_{p-1} s_p (s_p for p = 0)
                uint64_t wn[ST][2];
                probe_words(s / PS, wn);
#pragma unroll
                for (int j = 0; j < ST; ++j)
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        const uint64_t t = wn[j][b] ^ wp[j][b];
                        wp[j][b] = wn[j][b];
                        wn[j][b] = t;
                    }
                flip(wn);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d + 1 < D) {
                read_depth(s, d + 1, fr[(d + 1) & 1]);
                if constexpr (GEN) make_b(d + 1, gw, fr[(d + 1) & 1]);
            } else {
                // the last depth's fragments complete before the branch (the barrier below
                // waits for them anyway), so the MFMAs after the join wait for nothing
                __builtin_amdgcn_s_waitcnt(0xc07f);
                if (s + 1 < nsteps) {
                    // stage s+1 landed (the loads of s+2 .. s+NS-1 may stay in flight) and
                    // stage s read by every wave
                    if (s + NS - 1 < nsteps) wait_vm_barrier<(NS - 2) * PER>();
                    else wait_vm_barrier<0>();
                    if (s + NS < nsteps) issue(s + NS);
                    read_depth(s + 1, 0, fr[0]);
                    if constexpr (GEN) make_b(0, gn, fr[0]);
                }
            }
            mfmas(fr[d & 1]);
            if (d + 1 < D) interleave_reads_mfmas();
        }
        if constexpr (GEN) {
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                gw[j][0] = gn[j][0];
                gw[j][1] = gn[j][1];
            }
        }
    }
    if constexpr (HUTCH) flip(wp);   // acc *= s_{P-1}
    wait_vm_all();
    __syncthreads();
    if constexpr (MODE == 3) {
        Moments m = store_score_tile<SR, ST>(a, acc, r0 + wr * SR * 32, t0 + wt * ST * 32,
                                             (uint32_t*)smem + wave * kStageWords<SR>, lane);
        // the block's moments: a fixed-order tree over its threads through LDS
        __syncthreads();
        double* sh = (double*)smem;   // [3][64 * NW]
        constexpr int NT = 64 * NW;
        sh[tid] = m.n;
        sh[NT + tid] = m.mean;
        sh[2 * NT + tid] = m.m2;
        __syncthreads();
        for (int w = NT / 2; w > 0; w >>= 1) {
            if (tid < w) {
                const Moments o = moments_combine(Moments{sh[tid], sh[NT + tid], sh[2 * NT + tid]},
                                                  Moments{sh[tid + w], sh[NT + tid + w], sh[2 * NT + tid + w]});
                sh[tid] = o.n;
                sh[NT + tid] = o.mean;
                sh[2 * NT + tid] = o.m2;
            }
            __syncthreads();
        }
        if (tid < 3) a.mpart[(int64_t)tid * gridDim.x + blockIdx.x] = sh[tid * NT];
    } else {
        store_tile<uint16_t, SR, ST>(a, acc, r0 + wr * SR * 32, t0 + wt * ST * 32, r0 + BR <= a.R && t0 + BT <= a.Mtok,
                                     (uint32_t*)smem + wave * kStageWords<SR>, lane);
    }
}

// ------------------------------------------------------------------ K-split ring kernel (up to 256 tokens)
// With up to 256 tokens the 256-row tiles of the ring kernel are too few to fill the
// chip, and a weight-streaming kernel that loads SMFMAC fragments straight from
// memory touches a 128-byte line for every 32 bytes of weight (one row per lane).  Here a block of 4 waves owns a 32*SR x 32*ST tile; each stage (KB
// bytes of X per token, four SMFMAC depths) arrives in an NS-stage LDS ring by
// whole-line DMA as in the ring kernel, and wave w computes depth w of every stage
// over the whole tile.  The four partial tiles are summed through LDS in wave order.
// gridDim.y splits the stages over blocks (partials + the fixed-order reduce kernel).
// LIFT (6:8 weights, "SlideSparse" section 2B: the lifted activation is an index remap of
// X): the activation is never lifted in memory.  Stage s multiplies lifted columns whose
// windows lie in a run of at most 12 (bf16) or 23 (one-byte) 8-column groups of X; the X
// slot of a token holds 256 original bytes from the 16-byte-aligned start of that run
// (loaded by the same whole-line DMA, clamped to the row), and each lane assembles its
// lifted B fragment from the slot: window w of group q is original columns 8q + 2w .. +3,
// i.e. dwords w, w+1 of the group's 16 bytes (bf16) or bytes 2w .. 2w+3 of its 8 (one-
// byte codes: one byte-aligned funnel shift of the group's two dwords).
// Partial tiles summed through LDS: a lane's 16 accumulators at a stride of 20 floats, so
// the 16 lanes of a 16-byte store hit distinct banks (a 16-float stride puts them on 4)
constexpr int kRedStride = 20;

// XRES (up to 32 tokens, no lift): the block's X range -- its valid token rows, the
// columns of its stages -- is loaded into LDS once, ahead of the ring, and the ring carries
// the weight alone.  Under a full-chip weight stream a load from HBM takes about 4 us, so a
// CU's share of the bandwidth needs about 100 KB of weight in flight; with 32 token rows of
// X in every stage (one token valid at M = 1) a 6-stage ring held about 50 KB.  X rows sit
// 16 bytes apart beyond whole KB (16 lanes reading 16 tokens at one column hit distinct
// banks); token slots past the last valid token read the last valid row (their sums are
// never stored).
// Measured on 4096 x 4096 and 11008 x 4096 at 1 and 16 tokens: 6-8% faster than X in the
// ring.  A 14-stage weight ring with 16 KB of resident rows and no K split was slower (the
// 11008-row weight at one token: 17.8 against 16.2 us); reading that weight alone in the
// same stage order takes about 10 us.
constexpr int kXresBytes = 64 * 1024 + 32 * 16;

template <typename T, int SR, int ST, int KB, int NS, bool LIFT = false, int XRB_ = 0>
__global__ __launch_bounds__(256, 1) void spmm_ringk_kernel(SpmmArgs a) {
    constexpr bool XRES = XRB_ > 0;
    constexpr int es = sizeof(T);
    constexpr int KO = KB / es, KDEP = es == 2 ? 32 : 64;
    static_assert(KO / KDEP == 4, "one depth per wave per stage");
    static_assert(!(LIFT && XRES), "the resident X holds original columns of the unlifted product only");
    constexpr int BR = 32 * SR, BT = 32 * ST;
    constexpr int AROW = KO / 2 * es, ACH = AROW / 16, AI = KO / 32, BCH = KB / 16;
    static_assert(ACH == 8 && BCH == 16, "swizzles below are for 8-chunk weight rows and 16-chunk X rows");
    constexpr int I_OFF = BR * AROW, B_OFF = I_OFF + BR * AI * 4, STAGE = B_OFF + (XRES ? 0 : BT * KB);
    constexpr int NA = BR * AROW / 1024 / 4, NI = BR * AI * 4 / 256 / 4, NB = XRES ? 0 : BT * KB / 1024 / 4;
    constexpr int PER = NA + NI + NB;   // loads per wave per stage
    static_assert(NA >= 1 && NI >= 1 && (XRES || NB >= 1) && (BR * AROW) % 4096 == 0 && (BR * AI * 4) % 1024 == 0 &&
                      (BT * KB) % 4096 == 0,
                  "loads must split evenly over the 4 waves");
    static_assert(!XRES || ST == 1, "resident X for up to 32 tokens");
    constexpr int X_OFF = NS * STAGE, XRB = XRB_;
    constexpr int RED = 4 * 64 * kRedStride * 4;        // one sub-tile of all four waves
    constexpr int LDS = X_OFF + XRB > RED ? X_OFF + XRB : RED;
    static_assert(LDS <= 160 * 1024, "LDS ring too large");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    int tr, tt;
    tile_of(blockIdx.x, gridDim.x, a.tiles_r, a.tiles_t, tr, tt);
    // a row tile holds TRW <= BR weight rows; its other rows re-read the last one (their
    // sums are not stored)
    const int TRW = a.tile_rows > 0 && a.tile_rows < BR ? a.tile_rows : BR;
    const int64_t r0 = (int64_t)tr * TRW, t0 = (int64_t)tt * BT;
    const int split = blockIdx.y;
    const int s_begin = split * a.steps_per_split;
    const int s_end = (s_begin + a.steps_per_split) < a.nsteps ? (s_begin + a.steps_per_split) : a.nsteps;
    const int nloc = s_end > s_begin ? s_end - s_begin : 0;
    const uint32_t sbase = lds_addr(smem);
    auto swa = [](int r) { return (r >> 1) & 7; };   // weight row r: logical chunk c at c ^ swa(r)
    auto swb = [](int t) { return t & 15; };         // X token t: logical chunk c at c ^ swb(t)

    const void* baseA = uniform_ptr(a.vals + r0 * a.ldv * es);
    const void* baseI = uniform_ptr(a.idx + r0 * a.ldi);
    const void* baseB = uniform_ptr(a.X + t0 * a.ldx * es);
    const int64_t rmax = (a.R - 1 - r0) < (TRW - 1) ? (a.R - 1 - r0) : (TRW - 1), tmax = a.Mtok - 1 - t0;
    uint32_t oA[NA], oI[NI], oB[NB > 0 ? NB : 1], oBc[NB > 0 ? NB : 1];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int q = (wave * NA + i) * 64 + lane;
        const int row = q / ACH, c = (q % ACH) ^ swa(row);
        const int64_t gr = row < rmax ? row : rmax;
        oA[i] = (uint32_t)(gr * a.ldv * es + c * 16);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int q = (wave * NI + i) * 64 + lane;   // dword slot of the stage's [BR, AI] index block
        const int row = q / AI, lw = (q % AI) ^ iswz<AI>(row);
        const int64_t gr = row < rmax ? row : rmax;
        oI[i] = (uint32_t)(gr * a.ldi * 4 + lw * 4);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int row = (wave * NB + i) * (64 / BCH) + lane / BCH;
        const int c = (lane % BCH) ^ swb(row);
        const int64_t gt = row < tmax ? row : tmax;
        oB[i] = (uint32_t)(gt * a.ldx * es + (LIFT ? 0 : c * 16));
        oBc[i] = (uint32_t)(c * 16);
    }
    // LIFT: first original byte of stage sg's slot (a multiple of 16), and the last 16-byte
    // chunk of an X row (slot chunks past the row end load it; they are never used)
    auto slot_start = [](int sg) -> uint32_t {
        return es == 2 ? (uint32_t)(16 * ((32 * sg) / 3)) : (uint32_t)(8 * (((64 * sg) / 3) & ~1));
    };
    const uint32_t xlast = (uint32_t)(a.xrow_bytes - 16);
    auto issue = [&](int sl) __attribute__((always_inline)) {   // local stage sl of this block's range
        const int sg = s_begin + sl;
        const uint32_t st = sbase + (uint32_t)((sl % NS) * STAGE);
#pragma unroll
        for (int i = 0; i < NA; ++i) dma16s(st + (wave * NA + i) * 1024, baseA, oA[i] + (uint32_t)(sg * AROW));
#pragma unroll
        for (int i = 0; i < NI; ++i) dma4s(st + I_OFF + (wave * NI + i) * 256, baseI, oI[i] + (uint32_t)(sg * AI * 4));
        if constexpr (XRES) {
            // X is resident
        } else if constexpr (LIFT) {
            const uint32_t xs = slot_start(sg);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const uint32_t o = xs + oBc[i];
                dma16s(st + B_OFF + (wave * NB + i) * 1024, baseB, oB[i] + (o < xlast ? o : xlast));
            }
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i) dma16s(st + B_OFF + (wave * NB + i) * 1024, baseB, oB[i] + (uint32_t)(sg * KB));
        }
    };
    // XRES: valid token rows of the tile, padded LDS row bytes of the resident X
    const int xmv = XRES ? (int)(a.Mtok - t0 < BT ? a.Mtok - t0 : BT) : 0;
    const int xcpr = XRES ? (nloc * KB + 1023) / 1024 : 0;   // 1 KB loads per row
    const int xrowp = xcpr * 1024 + 16;
    struct Frag {
        i32x4_t a[SR];
        uint32_t iw[SR];
        i32x8_t b[ST];
    };
    const int d = wave;   // this wave's depth in every stage
    // LIFT: the lane's B fragment of depth d in stage sg from the token's slot of original
    // columns (trow, chunk swizzle sw).  The fragment's two 16-byte halves are lifted bytes
    // 64d + 16h + 32r (r = 0, 1) of the stage: lifted windows J .. (2 of 4 bf16 columns, or
    // 4 of 4 one-byte codes), window J = group J/3, offset J%3 of the 6:8 lift.
    auto lifted_frag = [&](const uint8_t* trow, int sw, int sg) __attribute__((always_inline)) -> i32x8_t {
        i32x8_t out;
        if constexpr (es == 2) {
            const int qb = (32 * sg) / 3;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int J = 32 * sg + 8 * d + 2 * h + 4 * r;   // first window of this half
                const int q = J / 3, w = J - 3 * q, ql = q - qb;
                const i32x4_t g0 = *(const i32x4_t*)(trow + ((ql ^ sw) * 16));
                const i32x4_t g1 = *(const i32x4_t*)(trow + (((ql + 1) ^ sw) * 16));
                // window J: dwords w, w+1 of group ql; window J+1: dwords w+1, w+2 of group ql
                // (w < 2) or dwords 0, 1 of group ql + 1 (w == 2)
                const int e0 = w == 0 ? g0[0] : (w == 1 ? g0[1] : g0[2]);
                const int e1 = w == 0 ? g0[1] : (w == 1 ? g0[2] : g0[3]);
                const int e2 = w == 0 ? g0[1] : (w == 1 ? g0[2] : g1[0]);
                const int e3 = w == 0 ? g0[2] : (w == 1 ? g0[3] : g1[1]);
                out[4 * r + 0] = e0;
                out[4 * r + 1] = e1;
                out[4 * r + 2] = e2;
                out[4 * r + 3] = e3;
            }
        } else {
            const int gb = ((64 * sg) / 3) & ~1;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int J = 64 * sg + 16 * d + 4 * h + 8 * r;   // windows J .. J+3
                const int q = J / 3, w = J - 3 * q, ql = q - gb;
                // groups ql and ql + 1 (8 bytes each, halves of 16-byte chunks)
                const uint2 ga = *(const uint2*)(trow + (((ql >> 1) ^ sw) * 16) + 8 * (ql & 1));
                const uint2 gc = *(const uint2*)(trow + ((((ql + 1) >> 1) ^ sw) * 16) + 8 * ((ql + 1) & 1));
                // window of group g at offset v: bytes 2v .. 2v+3 of the group (v_alignbyte takes
                // a byte shift of 0-3 only: offset 2 is the high dword itself)
                auto win = [](uint2 g, int v) {
                    return v == 2 ? (int)g.y : (int)__builtin_amdgcn_alignbyte(g.y, g.x, (uint32_t)(2 * v));
                };
                // windows J .. J+3 by the offset of J: (w = 0) g0 0,1,2 g1 0; (1) g0 1,2 g1 0,1; (2) g0 2 g1 0,1,2
                out[4 * r + 0] = win(ga, w);
                out[4 * r + 1] = w == 2 ? win(gc, 0) : win(ga, w + 1);
                out[4 * r + 2] = w == 0 ? win(ga, 2) : win(gc, w - 1);
                out[4 * r + 3] = win(gc, w);
            }
        }
        return out;
    };
    auto read = [&](int sl, Frag& f) __attribute__((always_inline)) {
        const uint8_t* sA = smem + (sl % NS) * STAGE;
        const uint32_t* sI = (const uint32_t*)(sA + I_OFF);
        const uint8_t* sB = sA + B_OFF;
#pragma unroll
        for (int i = 0; i < SR; ++i) {
            const int row = i * 32 + l32;
            f.a[i] = *(const i32x4_t*)(sA + row * AROW + ((2 * d + h) ^ swa(row)) * 16);
            f.iw[i] = sI[row * AI + ((es == 2 ? d : 2 * d + h) ^ iswz<AI>(row))];
        }
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            const int tok = j * 32 + l32;
            const uint8_t* trow = sB + tok * KB;
            if constexpr (XRES) {
                const uint8_t* xr = smem + X_OFF + (tok < xmv ? tok : xmv - 1) * xrowp + sl * KB;
                const i32x4_t lo = *(const i32x4_t*)(xr + (4 * d + h) * 16);
                const i32x4_t hi = *(const i32x4_t*)(xr + (4 * d + 2 + h) * 16);
                f.b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else if constexpr (LIFT) {
                f.b[j] = lifted_frag(trow, swb(tok), s_begin + sl);
            } else {
                const i32x4_t lo = *(const i32x4_t*)(trow + ((4 * d + h) ^ swb(tok)) * 16);
                const i32x4_t hi = *(const i32x4_t*)(trow + ((4 * d + 2 + h) ^ swb(tok)) * 16);
                f.b[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    };
    using AccV = typename Mma<T>::Acc;
    AccV acc[SR][ST];
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < ST; ++j) acc[i][j] = AccV{};
    const uint32_t ish = 16u * (uint32_t)h;
    auto mfmas = [&](const Frag& f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < SR; ++i)
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                acc[i][j] = Mma<T>::run(f.a[i], f.b[j], acc[i][j], (int)(es == 2 ? f.iw[i] >> ish : f.iw[i]));
            }
    };

    // Prologue fills the ring and reads stage 0.  Step S issues the SMFMACs of stage S,
    // waits for stage S+1 (stages S+2.. may stay in flight), meets the other waves (so
    // stage S's slot has been read by all), refills that slot with stage S+NS and reads
    // stage S+1 into the other fragment set.
    Frag fa, fb;
    if constexpr (XRES) {
        // the tile's X range ahead of the ring's first stages (so the wait for stage 0 covers
        // it): row t, 1 KB piece c; lanes past the range reload its last 16 bytes into the
        // row's padding.  The caller guarantees xmv * xrowp <= XRB; rows that would not fit
        // are not loaded.
        const int rows = xmv * xrowp <= XRB ? xmv : XRB / xrowp;
        const uint32_t kbytes = (uint32_t)(nloc * KB);
        for (int q = wave; q < rows * xcpr; q += 4) {
            const int t = q / xcpr, c = q - t * xcpr;
            uint32_t off = (uint32_t)(c * 1024 + lane * 16);
            off = off < kbytes - 16 ? off : kbytes - 16;
            dma16s(sbase + (uint32_t)(X_OFF + t * xrowp + c * 1024), baseB,
                   (uint32_t)(t * a.ldx * es) + (uint32_t)(s_begin * KB) + off);
        }
    }
#pragma unroll
    for (int p = 0; p < NS; ++p)
        if (p < nloc) issue(p);
    if (nloc >= NS) wait_vm_barrier<(NS - 1) * PER>();
    else wait_vm_barrier<0>();
    if (nloc > 0) read(0, fa);
    auto step = [&](int S, Frag& cur, Frag& nxt) __attribute__((always_inline)) {
        mfmas(cur);
        if (S + 1 < nloc) {
            if (S + NS - 1 < nloc) wait_vm_barrier<(NS - 2) * PER>();
            else wait_vm_barrier<0>();
            if (S + NS < nloc) issue(S + NS);
            read(S + 1, nxt);
        }
    };
    int S = 0;
    for (; S + 1 < nloc; S += 2) {
        step(S, fa, fb);
        step(S + 1, fb, fa);
    }
    if (S < nloc) step(S, fa, fb);
    wait_vm_all();

    // The four partial tiles are summed in wave order through LDS, one 32x32 sub-tile at a
    // time (whole-vector stores of the accumulators), by all 256 threads, which then write
    // the outputs along the rows (or the split's partials).
    float* red = (float*)smem;
#pragma unroll
    for (int i = 0; i < SR; ++i)
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            __syncthreads();
            *(AccV*)&red[(wave * 64 + lane) * kRedStride] = acc[i][j];
            __syncthreads();
            for (int q = tid; q < 1024; q += 256) {
                const int tk = q >> 5, row = q & 31;   // Y element (token, row) of the sub-tile
                const int src_lane = tk + 32 * ((row >> 2) & 1), e = 4 * (row >> 3) + (row & 3);
                const int64_t gt = t0 + 32 * j + tk, gr = r0 + 32 * i + row;
                using AccS = typename Mma<T>::AccS;
                AccS v = 0;
#pragma unroll
                for (int w = 0; w < 4; ++w) v += __builtin_bit_cast(AccS, red[(w * 64 + src_lane) * kRedStride + e]);
                if (gt >= a.Mtok || gr >= a.R || 32 * i + row >= TRW) continue;
                if (a.part) {
                    ((AccS*)a.part)[((int64_t)split * a.Mtok + gt) * a.R + gr] = v;
                    continue;
                }
                const int64_t o = gt * a.ldy + gr;
                if (a.ydt == NM_I32) {
                    ((int32_t*)a.Y)[o] = (int32_t)v;
                } else {
                    float f = (float)v;
                    if (a.scaled) {
                        const float xs = a.x_scale ? a.x_scale[gt] : 1.0f;
                        f = __fmul_rn(__fmul_rn(a.w_scale, xs), f);
                    }
                    if (a.ydt == NM_F32) ((float*)a.Y)[o] = f;
                    else ((uint16_t*)a.Y)[o] = (uint16_t)f32_to_bf16_bits(f);
                }
            }
        }
}

// ------------------------------------------------------------------ skinny kernel (few tokens: weight-streaming)
// For few tokens the product is bound by the HBM stream of the packed weight.
// A block of KSPLIT waves owns 32*SRk weight rows and 32*STk tokens; wave w
// walks its own slice of the SMFMAC depths, loading the packed values, their
// index words and the X fragments straight from global memory into registers
// (X is small and stays in L2).  The KSPLIT partial tiles are then summed
// through LDS in wave order (deterministic) and written out.
template <typename T>
__device__ __forceinline__ i32x8_t load_xfrag(const uint8_t* xrow, int Kbase, int h) {
    // element e of the fragment is column Kbase + KE*(e/(EL/2)) + (EL/2)*h + e%(EL/2), where
    // bf16: EL = 16 elements (KE = 16), int8: EL = 32 elements (KE = 32)
    constexpr int es = sizeof(T);
    constexpr int HALF = 16 / es;  // elements per 16-byte half
    const i32x4_t lo = *(const i32x4_t*)(xrow + (int64_t)(Kbase + HALF * h) * es);
    const i32x4_t hi = *(const i32x4_t*)(xrow + (int64_t)(Kbase + 2 * HALF + HALF * h) * es);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename T, int SRk, int STk, int KSPLIT, int U>
__global__ __launch_bounds__(KSPLIT * 64) void spmm_skinny_kernel(SpmmArgs a) {
    constexpr int es = sizeof(T);
    constexpr int KDEP = es == 2 ? 32 : 64;      // columns per SMFMAC
    __shared__ __attribute__((aligned(16))) float red[KSPLIT * 64 * kRedStride];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    // blockIdx.y splits the depths over blocks (partials then go to a.part); one block
    // column always covers every token (32 * STk >= Mtok)
    const int64_t r0 = (int64_t)blockIdx.x * (32 * SRk), t0 = 0;
    const int split = blockIdx.y;
    const int64_t Kl = a.comp_bytes * 2 / es;     // multiplied width
    const int D = (int)(Kl / KDEP);
    const int Db = (D + (int)gridDim.y - 1) / (int)gridDim.y;
    const int bd0 = split * Db < D ? split * Db : D, bd1 = bd0 + Db < D ? bd0 + Db : D;
    const int per = (bd1 - bd0 + KSPLIT - 1) / KSPLIT;
    const int d0 = bd0 + wave * per, d1 = d0 + per < bd1 ? d0 + per : bd1;

    const uint8_t* arow[SRk];
    const uint32_t* irow[SRk];
#pragma unroll
    for (int i = 0; i < SRk; ++i) {
        int64_t r = r0 + 32 * i + l32;
        r = r < a.R ? r : a.R - 1;
        arow[i] = a.vals + r * a.ldv * es + 16 * h;
        irow[i] = a.idx + r * a.ldi;
    }
    // B columns are independent in the product, so lanes past the last token load a valid
    // token's row and their (unwritten) output columns are simply discarded
    const uint8_t* xrow[STk];
#pragma unroll
    for (int j = 0; j < STk; ++j) {
        int64_t t = t0 + 32 * j + l32;
        t = t < a.Mtok ? t : a.Mtok - 1;
        xrow[j] = a.X + t * a.ldx * es;
    }
    using AccV = typename Mma<T>::Acc;
    AccV acc[SRk][STk];
#pragma unroll
    for (int i = 0; i < SRk; ++i)
#pragma unroll
        for (int j = 0; j < STk; ++j) acc[i][j] = AccV{};

    // U depths per batch: every load of a batch is issued before its first SMFMAC.  Every
    // batch has a compile-time depth count and runs branch-free (the depth bounds are
    // wave-uniform), so the compiler neither sinks loads into branches nor issues loads
    // for depths past the end.
    auto batch = [&](int d, auto nb) __attribute__((always_inline)) {
        constexpr int NB = decltype(nb)::value;   // depths in this batch (compile time)
        i32x4_t fa[NB][SRk];
        uint32_t fi[NB][SRk];
        i32x8_t fb[NB][STk];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int dd = d + u;
#pragma unroll
            for (int i = 0; i < SRk; ++i) {
                fa[u][i] = *(const i32x4_t*)(arow[i] + (int64_t)dd * 32);
                if constexpr (es == 2) fi[u][i] = irow[i][dd] >> (16 * h);
                else fi[u][i] = irow[i][2 * dd + h];
            }
#pragma unroll
            for (int j = 0; j < STk; ++j) fb[u][j] = load_xfrag<T>(xrow[j], dd * KDEP, h);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads ahead of the SMFMACs
#pragma unroll
        for (int u = 0; u < NB; ++u)
#pragma unroll
            for (int i = 0; i < SRk; ++i)
#pragma unroll
                for (int j = 0; j < STk; ++j) {
                    acc[i][j] = Mma<T>::run(fa[u][i], fb[u][j], acc[i][j], (int)fi[u][i]);
                }
    };
    // full batches of U, then the remainder as batches of U/2, U/4, ..., 1 (each branch-free)
    int d = d0;
    for (; d + U <= d1; d += U) batch(d, std::integral_constant<int, U>{});
    if constexpr (U > 8)
        if (d + 8 <= d1) { batch(d, std::integral_constant<int, 8>{}); d += 8; }
    if constexpr (U > 4)
        if (d + 4 <= d1) { batch(d, std::integral_constant<int, 4>{}); d += 4; }
    if constexpr (U > 2)
        if (d + 2 <= d1) { batch(d, std::integral_constant<int, 2>{}); d += 2; }
    if constexpr (U > 1)
        if (d < d1) batch(d, std::integral_constant<int, 1>{});

    // fixed-order reduction of the KSPLIT partial tiles, one 32x32 sub-tile at a time
#pragma unroll
    for (int i = 0; i < SRk; ++i)
#pragma unroll
        for (int j = 0; j < STk; ++j) {
            __syncthreads();
            // one vector store of the whole accumulator (storing its 16 elements one by one
            // through bit casts was compiled into four copies of the first 16 bytes)
            *(AccV*)&red[(wave * 64 + lane) * kRedStride] = acc[i][j];
            __syncthreads();
            for (int q = tid; q < 1024; q += KSPLIT * 64) {
                const int tok = q >> 5, row = q & 31;                      // Y element (token, row) of the sub-tile
                const int src_lane = tok + 32 * ((row >> 2) & 1), e = 4 * (row >> 3) + (row & 3);
                const int64_t gt = t0 + 32 * j + tok, gr = r0 + 32 * i + row;
                using AccS = typename Mma<T>::AccS;
                AccS v = 0;
                for (int w = 0; w < KSPLIT; ++w) v += __builtin_bit_cast(AccS, red[(w * 64 + src_lane) * kRedStride + e]);
                if (a.part) {
                    if (gt < a.Mtok && gr < a.R) ((AccS*)a.part)[((int64_t)split * a.Mtok + gt) * a.R + gr] = v;
                } else if (gt < a.Mtok && gr < a.R) {
                    const int64_t o = gt * a.ldy + gr;
                    if (a.ydt == NM_I32) {
                        ((int32_t*)a.Y)[o] = (int32_t)v;
                    } else {
                        float f = (float)v;
                        if (a.scaled) {
                            const float xs = a.x_scale ? a.x_scale[gt] : 1.0f;
                            f = __fmul_rn(__fmul_rn(a.w_scale, xs), f);
                        }
                        if (a.ydt == NM_F32) ((float*)a.Y)[o] = f;
                        else ((uint16_t*)a.Y)[o] = (uint16_t)f32_to_bf16_bits(f);
                    }
                }
            }
        }
}

// Split-K reduction: partials summed in split order, then the epilogue.
template <typename Acc>
__global__ __launch_bounds__(256) void spmm_reduce_kernel(SpmmArgs a) {
    const int64_t total = a.Mtok * a.R;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tok = t / a.R, r = t - tok * a.R;
        const Acc v = split_sum((const Acc*)a.part + t, a.KS, total);
        const int64_t o = tok * a.ldy + r;
        if (a.ydt == NM_I32) {
            ((int32_t*)a.Y)[o] = (int32_t)v;
        } else {
            float f = (float)v;
            if (a.scaled) {
                const float xs = a.x_scale ? a.x_scale[tok] : 1.0f;
                f = __fmul_rn(__fmul_rn(a.w_scale, xs), f);
            }
            if (a.ydt == NM_F32) ((float*)a.Y)[o] = f;
            else ((uint16_t*)a.Y)[o] = (uint16_t)f32_to_bf16_bits(f);
        }
    }
}

// ------------------------------------------------------------------ adapter term ("SALR", section 3)
// All low-rank adapters of a layer stacked along the rank: Y = X W_hat^T + u B^T with
// u = bf16(X A^T), A [rank, K], B [R, rank].  u is computed once per call here; the
// many-token product kernels add u B^T to their accumulators (add_lowrank), the others
// through lowrank_epilogue_kernel.

// Partial u over one K chunk per wave: block = 32 tokens x (32 RT ranks), four waves on
// four consecutive chunks of the block's K range (gridDim.y ranges); v_mfma_f32_32x32x16_bf16
// with the tokens as the A operand and the rank rows of A as the B operand.  Partials go
// to P[split][Mtok][rank] (split = 4 * blockIdx.y + wave).
template <int RT>
__global__ __launch_bounds__(256) void lowrank_u_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                        const uint16_t* __restrict__ A, int64_t lda, int64_t M,
                                                        int64_t K, int rank, int64_t kchunk, float* __restrict__ P) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5, l32 = lane & 31;
    const int64_t t0 = (int64_t)blockIdx.x * 32;
    const int split = blockIdx.y * 4 + wave;
    const int64_t kb = split * kchunk, ke = kb + kchunk < K ? kb + kchunk : K;
    const int64_t tok = t0 + l32 < M ? t0 + l32 : M - 1;
    const uint16_t* xr = X + tok * ldx + 8 * h;
    f32x16_t acc[RT];
#pragma unroll
    for (int q = 0; q < RT; ++q) acc[q] = f32x16_t{};
    const uint16_t* ar[RT];
    bool aok[RT];
#pragma unroll
    for (int q = 0; q < RT; ++q) {
        const int n = q * 32 + l32;
        aok[q] = n < rank;
        ar[q] = A + (int64_t)(aok[q] ? n : 0) * lda + 8 * h;
    }
#pragma unroll 4
    for (int64_t k = kb; k < ke; k += 16) {
        const i32x4_t xv = *(const i32x4_t*)(xr + k);
#pragma unroll
        for (int q = 0; q < RT; ++q) {
            const i32x4_t av = aok[q] ? *(const i32x4_t*)(ar[q] + k) : i32x4_t{0, 0, 0, 0};
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, xv),
                                                             __builtin_bit_cast(bf16x8_t, av), acc[q], 0, 0, 0);
        }
    }
    // lane holds rank column q*32 + l32 and token rows 8*(e/4) + 4*h + e%4
#pragma unroll
    for (int q = 0; q < RT; ++q) {
        const int n = q * 32 + l32;
        if (n >= rank) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t t = t0 + 8 * (e / 4) + 4 * h + (e % 4);
            if (t < M) P[((int64_t)split * M + t) * rank + n] = acc[q][e];
        }
    }
}

// u[m, n] = bf16(sum of the partials in split order)
__global__ __launch_bounds__(256) void lowrank_u_reduce_kernel(const float* __restrict__ P, int S, int64_t M, int rank,
                                                               uint16_t* __restrict__ U) {
    const int64_t total = M * rank;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const float v = split_sum(P + i, S, total);
        U[i] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// Y[m, o] = P[m, o] + sum_j u[m, j] B[o, j] (j ascending, f32), converted to a.ydt.
__global__ __launch_bounds__(256) void lowrank_epilogue_kernel(const float* __restrict__ P, SpmmArgs a) {
    const int64_t total = a.Mtok * a.R;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t m = i / a.R, o = i - m * a.R;
        const uint16_t* ur = a.lr_u + m * a.ldu;
        const uint16_t* br = a.lr_b + o * a.ldb;
        float lr = 0.0f;
        for (int j = 0; j < a.rank; ++j) lr = __fmaf_rn(bf16_bits_to_f32(ur[j]), bf16_bits_to_f32(br[j]), lr);
        const float v = P[i] + lr;
        if (a.ydt == NM_F32) ((float*)a.Y)[m * a.ldy + o] = v;
        else ((uint16_t*)a.Y)[m * a.ldy + o] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// K chunking of the u product: four chunks per block, blocks along K until the grid has
// about 256 blocks, chunks of at least 256 columns (a multiple of 16).
struct LowRankPlan {
    int ks;           // blocks along K
    int64_t kchunk;   // columns per wave
    int S() const { return 4 * ks; }
};
static LowRankPlan lowrank_plan(int64_t M, int64_t K) {
    LowRankPlan p{1, 0};
    const int64_t tiles = ceil_div(M, 32);
    while (tiles * p.ks < 256 && K / (4 * p.ks * 2) >= 256) p.ks *= 2;
    p.kchunk = ceil_div(ceil_div(K, (int64_t)p.S()), 16) * 16;
    return p;
}

// ------------------------------------------------------------------ host side
struct SpmmPlan {
    bool large, ring, big;
    int64_t split_rows;  // > 0: big tiles on rows [0, split_rows), narrow tiles on the rest
    int mid;     // K-split ring: 0 none, else 32-token sub-tiles per block (1, 2 or 4)
    int skinny;  // 0: none, 1: <=32 tokens, 2: <=64, 3: <=128
    int xres;    // K-split ring with X resident in LDS (up to 64 KB, 8-stage weight ring)
    int sr1;     // K-split ring on 32-row tiles (one-byte codes up to 32 tokens)
    int tile_rows;   // K-split ring: weight rows per row tile when fewer than the tile height
    int tiles_r, tiles_t, nsteps, KS, steps_per_split;
};

// Many-token tiles (6:8 products with many tokens run here on the lifted activation):
//   narrow: ring kernel (T, SR, ST, KB, NS, WRN, WTN), 256 x 128 tile, 4 waves (one per
//           SIMD), 2 stages of 256 B of X per token
//   big   : split ring kernel (T, SR, ST, WRN, WTN, IP), 256 x 256 tile, 8 waves (two per
//           SIMD); bf16 index batches load 4 bytes per lane (16 do not split over 8 waves)
#define NM_RING_NARROW T, 4, 2, 256, 2, 2, 2
#define NM_RING_BIG T, 4, 2, 2, 4, 4

// Compute units of the current device (cached per device).
static int64_t device_cus() {
    static int64_t cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        cache[dev] = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
    }
    return cache[dev];
}

template <typename T>
static SpmmPlan plan_for(int64_t Mtok, int64_t K, int64_t R, bool ring_ok, bool xres_ok = true) {
    using G = Geo<T>;
    SpmmPlan p{};
    // up to 256 tokens: the K-split ring kernel on 64 x 32, 64 x 64 or 64 x 128 tiles, with
    // the stages split over blocks while fewer than 160 tiles would run (each split keeps
    // >= 4 stages; measured on the 4096- and 11008-row layers: 64 tiles run best in 4
    // splits, 172 tiles unsplit, as the partials' reduce costs more than it gains there)
    {
        constexpr int KOm = 256 / (int)sizeof(T);
        const bool mid = ring_ok && Mtok <= 256 && (K % KOm) == 0;
        // token tile: the narrowest (32, 64 or 128 tokens) whose tiles fit one round on the
        // CUs, else the widest.  Narrow tiles carry less X per stage, so more of the ring is
        // weight in flight; the token tiles of a row tile share the weight through L2.
        // Measured: 4096 rows at 128 tokens 23.8 -> 18.9 us on 32-token tiles (256 tiles,
        // no K split); where 32-token tiles need 2.7-3.4 rounds (11008 rows at 128 tokens,
        // 14336 rows of 6:8 at 64, 6912 int8 rows at 256) they were 24-66% slower.
        p.mid = 0;
        if (mid) {
            const int64_t cus = device_cus(), rt = ceil_div(R, 64);
            p.mid = Mtok <= 32 ? 1 : (Mtok <= 64 ? 2 : 4);   // the widest tile the tokens need
            for (int m = 1; m < p.mid; m *= 2)
                if (rt * ceil_div(Mtok, 32 * m) <= cus) {
                    p.mid = m;
                    break;
                }
        }
        if (p.mid) {
            p.tiles_r = (int)ceil_div(R, 64);
            p.tiles_t = (int)ceil_div(Mtok, 32 * p.mid);
            p.nsteps = (int)(K / KOm);
            // Up to 64 tokens the product streams the weight.  Where 64-row tiles leave CUs
            // idle (or would split K, with a reduce launch after), each row tile takes
            // ceil(R / (CUs / token tiles)) rows, when that is at least 32: one round of equal
            // tiles and no split; a tile's rows past its share re-read its last row (L2 hits;
            // their sums are not stored).  Measured: 11008 rows at 16 tokens 18.9 -> 16.8 us,
            // at one token 16.6 -> 15.9 us (the stream is bound chip-wide as well as per CU).  One-byte codes whose share is 16-32 rows run on
            // 32-row tiles (their index rows fill whole DMA batches there; bf16 ones do not).
            // Shares of 16-31 rows (bf16, unlifted) re-read more of each tile from L2, which
            // pays only where the K split would not fill whole rounds of the CUs (measured at
            // one token: 5000 rows 16.7 -> 13.4 us against 316 split blocks; 4096 rows 12.4 ->
            // 13.2 us against 256; lifted products 1.7x slower).
            p.sr1 = 0;
            p.tile_rows = 0;
            if (p.mid <= 2) {
                const int64_t cus = device_cus(), per = cus / p.tiles_t;
                if (per >= 1 && (int64_t)p.tiles_r < per) {
                    const int64_t rows = ceil_div(R, per);
                    const bool one32 = sizeof(T) == 1 && p.mid == 1 && rows <= 32;
                    int64_t ks = 1;
                    while ((int64_t)p.tiles_r * p.tiles_t * ks < 160 && p.nsteps >= 8 * ks) ks *= 2;
                    const bool split_ragged = ((int64_t)p.tiles_r * p.tiles_t * ks) % cus != 0;
                    const bool small_ok = one32 || (xres_ok && split_ragged);
                    if (rows < 64 && (rows >= 32 || (small_ok && rows >= 16))) {
                        p.tile_rows = (int)rows;
                        p.tiles_r = (int)ceil_div(R, rows);
                        p.sr1 = one32 ? 1 : 0;
                    }
                }
            }
            int KS = 1;
            while ((int64_t)p.tiles_r * p.tiles_t * KS < 160 && p.nsteps >= 8 * KS) KS *= 2;
            p.steps_per_split = (int)ceil_div(p.nsteps, KS);
            p.KS = (int)ceil_div(p.nsteps, p.steps_per_split);
            // up to 32 tokens of an unlifted X whose range per block fits 64 KB: X resident in
            // LDS, an 8-stage weight ring
            p.xres = 0;
            if (xres_ok && p.mid == 1) {
                const int64_t rows = Mtok < 32 ? Mtok : 32;
                if (rows * (ceil_div((int64_t)p.steps_per_split * 256, 1024) * 1024 + 16) <= kXresBytes) p.xres = 1;
            }
            // bf16, 65-256 tokens on 128-token tiles (X not lifted in the kernel): a block of
            // the K-split ring takes 64 rows and reads its tokens' whole X range -- four times
            // the weight's bytes in every stage, which leaves the ring little weight in
            // flight.  The narrow ring's 256 x 128 tiles read a quarter of that per weight
            // byte; their stages are split over blocks until about one round runs, the
            // splits' partials summed by the reduce kernel.  Measured: 11008 rows at 128
            // tokens 38.9 -> 36.2 us; for int8 (6912 rows, 256 tokens, 15 stages) slower,
            // 30.9 -> 36.6 us, as each split holds only 4 stages of a 2-slot ring.
            using RNm = Ring<NM_RING_NARROW>;
            if (sizeof(T) == 2 && p.mid == 4 && xres_ok && ring_ok && (K % RNm::KO) == 0) {
                const int64_t cus = device_cus();
                const int64_t tiles = ceil_div(R, RNm::BR) * ceil_div(Mtok, RNm::BT);
                const int64_t ns = K / RNm::KO;
                int64_t ks = cus / tiles;
                if (ks > ns / 2) ks = ns / 2;
                if (ks < 1) ks = 1;
                SpmmPlan q{};
                q.ring = true;
                q.large = Mtok > 128;
                q.tiles_r = (int)ceil_div(R, RNm::BR);
                q.tiles_t = (int)ceil_div(Mtok, RNm::BT);
                q.nsteps = (int)ns;
                q.steps_per_split = (int)ceil_div(ns, ks);
                q.KS = (int)ceil_div(ns, q.steps_per_split);
                return q;
            }
            return p;
        }
    }
    p.large = Mtok > 128;
    using RB = Ring2<NM_RING_BIG>;
    using RN = Ring<NM_RING_NARROW>;
    p.ring = ring_ok && p.large && (K % RN::KO) == 0;
    // the big tile moves about a third fewer bytes per multiply-add; with fewer of its
    // tiles than CUs the narrow tile's finer grain fills the chip better (measured: 11008
    // rows x 2048 tokens (344 big tiles) run 7% faster big, 4096 x 2048 (128) 20% slower)
    // Tile choice by whole rounds of tiles over the CUs.  The big tile moves about a third
    // fewer bytes per multiply-add; a round of big tiles takes about 1.5x a round of
    // narrow ones (1.4x on 11008 rows x 2048 tokens, 1.8x on 28672 x 8192).  Candidates:
    // all narrow, all big, and whole rounds of big tiles over the first rows with the
    // remaining rows in narrow tiles (a second launch), so that a short last round of big
    // tiles becomes a round of half-size ones.
    p.big = false;
    p.split_rows = 0;
    if (p.ring && (K % (2 * RB::KO)) == 0) {
        const int64_t cus = device_cus();
        const int64_t ttb = ceil_div(Mtok, RB::BT), tb = ceil_div(R, RB::BR) * ttb;
        const int64_t ttn = ceil_div(Mtok, RN::BT), tn = ceil_div(R, RN::BR) * ttn;
        int64_t best = 2 * ceil_div(tn, cus);
        if (3 * ceil_div(tb, cus) < best) {
            best = 3 * ceil_div(tb, cus);
            p.big = true;
        }
        const int64_t rtb = (tb / cus) * cus / ttb;   // big row tiles that fill whole rounds
        if (rtb >= 1 && rtb * RB::BR < R) {
            const int64_t rest = R - rtb * RB::BR;
            const int64_t c = 3 * ceil_div(rtb * ttb, cus) + 2 * ceil_div(ceil_div(rest, RN::BR) * ttn, cus);
            if (c < best) {
                p.big = false;
                p.split_rows = rtb * RB::BR;
            }
        }
    }
    const int BR = p.ring ? (p.big ? RB::BR : RN::BR) : 128;
    const int BT = p.ring ? (p.big ? RB::BT : RN::BT) : (p.large ? 128 : 32);
    p.tiles_r = (int)ceil_div(R, BR);
    p.tiles_t = (int)ceil_div(Mtok, BT);
    {
        constexpr int KDEP = sizeof(T) == 2 ? 32 : 64;
        p.skinny = 0;
        if (!p.large && K % KDEP == 0) p.skinny = Mtok <= 32 ? 1 : (Mtok <= 64 ? 2 : 3);
    }
    p.nsteps = (int)ceil_div(K, p.ring ? (p.big ? RB::KO : RN::KO) : G::KO);
    if (p.skinny) {
        // K split over blocks (partials + a fixed-order reduce) where the row tiles alone
        // leave the chip short of blocks; measured on the 4096- and 11008-row layers
        p.KS = 1;
        if (p.skinny == 1 && sizeof(T) == 2 && ceil_div(R, 32) <= 512) p.KS = 2;
        if (p.skinny == 3 && ceil_div(R, 64) < 128) p.KS = 4;
        p.steps_per_split = 0;
        return p;
    }
    const int64_t blocks = (int64_t)p.tiles_r * p.tiles_t;
    int KS = 1;
    if (!p.large) {
        const int64_t target = 1024;
        while ((int64_t)KS * blocks < target && KS * 4 <= p.nsteps) KS *= 2;
    }
    if (p.nsteps == 0) {
        p.KS = 1;
        p.steps_per_split = 0;
        return p;
    }
    p.steps_per_split = (int)ceil_div(p.nsteps, KS);
    p.KS = (int)ceil_div(p.nsteps, p.steps_per_split);
    return p;
}

// ------------------------------------------------------------------ (2N-2):2N activation lift
// The N-1 overlapping 2:4 windows of a 2N-column group (offsets 0, 2, .., 2N-4) multiply
// the lifted activation XL[m, 4(N-1)q + 4w + j] = X[m, 2Nq + 2w + j].  Products that do
// not gather it inside the product kernel write it out once (memory-bound, (2-2/N)x the
// bytes of X) so that the product runs on the plain 2:4 kernels.
// 6:8: one lane = one 8-column group, three windows from one 16-byte (bf16) or 8-byte load.
template <typename T>
__global__ __launch_bounds__(256) void lift68_kernel(const T* __restrict__ X, int64_t ldx, int64_t Mtok, int64_t K,
                                                     T* __restrict__ XL, int64_t ldl) {
    const int64_t gpr = K / 8, total = Mtok * gpr;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total; u += stride) {
        const int64_t m = u / gpr, q = u - m * gpr;
        if constexpr (sizeof(T) == 2) {
            const uint4 v = *(const uint4*)(X + m * ldx + 8 * q);   // elements (0,1) (2,3) (4,5) (6,7)
            uint2* o = (uint2*)(XL + m * ldl + 12 * q);
            o[0] = make_uint2(v.x, v.y);
            o[1] = make_uint2(v.y, v.z);
            o[2] = make_uint2(v.z, v.w);
        } else {
            const uint2 v = *(const uint2*)(X + m * ldx + 8 * q);   // bytes 0-3, 4-7
            uint32_t* o = (uint32_t*)(XL + m * ldl + 12 * q);
            o[0] = v.x;
            o[1] = (v.x >> 16) | (v.y << 16);
            o[2] = v.y;
        }
    }
}

// Any N: one lane = one window (4 lifted columns), read as two pairs of columns (a pair
// starts at an even column, so it is 4-byte (bf16) or 2-byte (one-byte codes) aligned).
template <typename T>
__global__ __launch_bounds__(256) void lift_kernel(const T* __restrict__ X, int64_t ldx, int64_t Mtok, int64_t K,
                                                   int Ns, T* __restrict__ XL, int64_t ldl) {
    using P = typename std::conditional<sizeof(T) == 2, uint32_t, uint16_t>::type;   // a pair of columns
    const int64_t wpr = K / (2 * Ns) * (Ns - 1), total = Mtok * wpr;   // windows per row
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < total; u += stride) {
        const int64_t m = u / wpr, q = u - m * wpr;
        const int64_t g = q / (Ns - 1), w = q - g * (Ns - 1);
        const P* src = (const P*)(X + m * ldx + 2 * Ns * g + 2 * w);
        const P lo = src[0], hi = src[1];
        if constexpr (sizeof(T) == 2) *(uint2*)(XL + m * ldl + 4 * q) = make_uint2(lo, hi);
        else *(uint32_t*)(XL + m * ldl + 4 * q) = (uint32_t)lo | ((uint32_t)hi << 16);
    }
}

static int64_t lifted_cols(int64_t K, int Ns) { return Ns ? K / (2 * Ns) * 4 * (Ns - 1) : K; }

static size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

static size_t lift_bytes(int64_t Mtok, int64_t K, int Ns, int64_t es) {
    return round256((size_t)Mtok * (size_t)lifted_cols(K, Ns) * (size_t)es);
}

// Workspace of one nm_spmm / nm_spmm_lowrank call, in the order it is carved:
//   u, pu: the adapter's u = bf16(X A^T) and its K-split f32 partials (rank > 0),
//   xl   : the lifted activation (Ns >= 3),
//   f32  : the sparse product in f32 when the adapter term is added by its own kernel,
//   part : split-K partials of the product.
struct SpmmWs {
    size_t u = 0, pu = 0, xl = 0, f32 = 0, part = 0;
    size_t total() const { return u + pu + xl + f32 + part; }
};

// ring_ok: the product's operands allow the DMA ring kernels (decided by the caller from
// the actual pointers and leading dimensions; the query takes the larger of both plans).
// fused: the lift happens inside the K-split ring kernel (no lifted activation stored).
static SpmmWs spmm_ws_layout(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt, int rank, bool ring_ok,
                             bool fused);
// 6:8 products of up to 256 tokens on the K-split ring lift inside the kernel
static bool lift_fused(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt, bool ring_ok);

size_t spmm_ws(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt) {
    const size_t a = spmm_ws_layout(Mtok, K, R, Ns, xdt, 0, true, lift_fused(Mtok, K, R, Ns, xdt, true)).total();
    const size_t b = spmm_ws_layout(Mtok, K, R, Ns, xdt, 0, false, false).total();
    return a > b ? a : b;
}

// The DMA ring kernels take 16-byte pieces of the index rows and 32-bit per-lane offsets
// from a block's base pointers.
static bool ring_ok_for(const SpmmArgs& a, int64_t es) {
    return ((uintptr_t)a.idx & 15u) == 0 && (a.ldi % 4) == 0 && a.R * a.ldv * es < (1LL << 32) &&
           a.R * a.ldi * 4 < (1LL << 32) && a.Mtok * a.ldx * es < (1LL << 32);
}

static bool lift_fused(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt, bool ring_ok) {
    if (Ns != 4) return false;
    const int64_t Kl = lifted_cols(K, Ns);
    // the token tile of the K-split ring the lifted product would run on
    const SpmmPlan p = xdt == NM_BF16 ? plan_for<uint16_t>(Mtok, Kl, R, ring_ok, false)
                                      : plan_for<int8_t>(Mtok, Kl, R, ring_ok, false);
    // one-byte codes: the in-kernel gather (two 8-byte reads and a funnel shift per window
    // pair) costs more than a separate lift on the 128-token tiles (6912 x 2560 int8 at 256
    // tokens: 38.3 us fused against 32.7 us lifting first; at one token 14.6 against 16.2)
    return p.mid != 0 && (xdt == NM_BF16 || p.mid <= 2);
}

static SpmmWs spmm_ws_layout(int64_t Mtok, int64_t K, int64_t R, int Ns, nm_dtype xdt, int rank, bool ring_ok,
                             bool fused) {
    SpmmWs w;
    if (Mtok <= 0 || K <= 0 || R <= 0) return w;
    const int64_t Kl = lifted_cols(K, Ns), es = xdt == NM_BF16 ? 2 : 1;
    if (rank > 0) {
        const LowRankPlan lp = lowrank_plan(Mtok, K);
        w.u = round256((size_t)Mtok * rank * 2);
        w.pu = round256((size_t)lp.S() * Mtok * rank * 4);
    }
    if (Ns && !fused) w.xl = lift_bytes(Mtok, K, Ns, es);
    // the plan depends on the element size only (int8 and FP8 share it)
    const SpmmPlan p = es == 2 ? plan_for<uint16_t>(Mtok, Kl, R, ring_ok, !fused)
                               : plan_for<int8_t>(Mtok, Kl, R, ring_ok, !fused);
    if (rank > 0 && !p.ring) w.f32 = round256((size_t)Mtok * (size_t)R * 4);
    if (p.KS > 1) w.part = round256((size_t)p.KS * (size_t)Mtok * (size_t)R * 4);
    return w;
}

// plain 2:4 product of X [Mtok, K] (K = the lifted width for (2N-2):2N); part: the split-K
// partials, f32buf: the sparse product in f32 when an adapter term is added afterwards
// (both carved from the workspace by the caller, sized by spmm_ws_layout)
template <typename T>
static nm_status run_spmm(SpmmArgs a, bool ring_ok, bool lift, void* part, void* f32buf, hipStream_t s) {
    const SpmmPlan p = plan_for<T>(a.Mtok, a.K, a.R, ring_ok, !lift);
    a.nsteps = p.nsteps;
    a.KS = p.KS;
    a.steps_per_split = p.steps_per_split;
    a.tiles_r = p.tiles_r;
    a.tiles_t = p.tiles_t;
    a.tile_rows = p.tile_rows;
    a.part = p.KS > 1 ? part : nullptr;
    if (a.rank > 0 && !p.ring) {
        // the other kernels carry no adapter term: they write the sparse product in f32
        // into the workspace and lowrank_epilogue_kernel adds the term and converts
        SpmmArgs b = a;
        b.rank = 0;
        b.Y = f32buf;
        b.ydt = NM_F32;
        b.ldy = a.R;
        b.scaled = 0;
        const nm_status st = run_spmm<T>(b, ring_ok, lift, part, nullptr, s);
        if (st != NM_OK) return st;
        const dim3 g(grid_cap(ceil_div(a.Mtok * a.R, 256), 65536));
        hipLaunchKernelGGL(lowrank_epilogue_kernel, g, dim3(256), 0, s, (const float*)f32buf, a);
        return check_launch("nm_spmm_lowrank");
    }
    const dim3 grid((unsigned)(p.tiles_r * p.tiles_t), (unsigned)p.KS);
    if (p.mid) {
        // up to 32 tokens a 6-stage ring (17 KB a stage): more weight bytes in flight per CU
        // when the weight comes from HBM (measured 13-15% faster there at one token; a
        // 6-stage ring for 64 tokens measured no faster than 3 stages)
        if (p.sr1) {
            // 32-row tiles of one-byte codes: a 12-stage ring (13 KB a stage), 16 weight
            // stages beside a resident X
            if constexpr (sizeof(T) == 1) {
                if (lift) hipLaunchKernelGGL((spmm_ringk_kernel<T, 1, 1, 256, 12, true>), grid, dim3(256), 0, s, a);
                else if (p.xres)
                    hipLaunchKernelGGL((spmm_ringk_kernel<T, 1, 1, 256, 16, false, kXresBytes>), grid, dim3(256), 0, s, a);
                else hipLaunchKernelGGL((spmm_ringk_kernel<T, 1, 1, 256, 12, false>), grid, dim3(256), 0, s, a);
            } else {
                return set_error(NM_ERR_DEVICE, "nm_spmm: 32-row K-split tiles are for one-byte codes");
            }
        } else if (lift) {   // 6:8: the activation is lifted inside the kernel (one-byte codes: up to 64 tokens)
            if (p.mid == 1) hipLaunchKernelGGL((spmm_ringk_kernel<T, 2, 1, 256, 6, true>), grid, dim3(256), 0, s, a);
            else if (p.mid == 2) hipLaunchKernelGGL((spmm_ringk_kernel<T, 2, 2, 256, 3, true>), grid, dim3(256), 0, s, a);
            else if constexpr (sizeof(T) == 2)
                hipLaunchKernelGGL((spmm_ringk_kernel<T, 2, 4, 256, 3, true>), grid, dim3(256), 0, s, a);
            else
                return set_error(NM_ERR_DEVICE, "nm_spmm: no in-kernel lift for one-byte codes on 128-token tiles");
        } else {
            if (p.xres)
                hipLaunchKernelGGL((spmm_ringk_kernel<T, 2, 1, 256, 8, false, kXresBytes>), grid, dim3(256), 0, s, a);
            else if (p.mid == 1) hipLaunchKernelGGL((spmm_ringk_kernel<T, 2, 1, 256, 6>), grid, dim3(256), 0, s, a);
            else if (p.mid == 2) hipLaunchKernelGGL((spmm_ringk_kernel<T, 2, 2, 256, 3>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((spmm_ringk_kernel<T, 2, 4, 256, 3>), grid, dim3(256), 0, s, a);
        }
    } else if (p.skinny == 1) {
        // 32-row tiles, 4 waves split K, 16 depths in flight per wave
        hipLaunchKernelGGL((spmm_skinny_kernel<T, 1, 1, 4, 16>), dim3((unsigned)ceil_div(a.R, 32), p.KS), dim3(256), 0, s, a);
    } else if (p.skinny == 2) {
        // two 32-row tiles per wave share each X fragment when that still leaves >= 200 blocks
        if (ceil_div(a.R, 64) >= 200)
            hipLaunchKernelGGL((spmm_skinny_kernel<T, 2, 2, 4, 4>), dim3((unsigned)ceil_div(a.R, 64), p.KS), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((spmm_skinny_kernel<T, 1, 2, 4, 8>), dim3((unsigned)ceil_div(a.R, 32), p.KS), dim3(256), 0, s, a);
    } else if (p.skinny == 3) {
        hipLaunchKernelGGL((spmm_skinny_kernel<T, 2, 4, 4, 4>), dim3((unsigned)ceil_div(a.R, 64), p.KS), dim3(256), 0, s, a);
    } else if (p.ring) {
        using RB = Ring2<NM_RING_BIG>;
        using RN = Ring<NM_RING_NARROW>;
        // one launch on rows [r_begin, r_end) of the product
        auto launch = [&](bool big, int64_t r_begin, int64_t r_end) {
            SpmmArgs b = a;
            const int64_t es = sizeof(T), ys = a.ydt == NM_BF16 ? 2 : 4;
            b.vals = a.vals + r_begin * a.ldv * es;
            b.idx = a.idx + r_begin * a.ldi;
            b.Y = (uint8_t*)a.Y + r_begin * ys;
            if (a.rank > 0) b.lr_b = a.lr_b + r_begin * a.ldb;
            b.R = r_end - r_begin;
            b.tiles_r = (int)ceil_div(b.R, big ? RB::BR : RN::BR);
            b.tiles_t = (int)ceil_div(a.Mtok, big ? RB::BT : RN::BT);
            b.nsteps = (int)(a.K / (big ? RB::KO : RN::KO));
            // the narrow ring's stages split over blocks (few tokens): partials into the workspace
            const bool split = !big && p.KS > 1;
            b.part = split ? a.part : nullptr;
            b.KS = split ? p.KS : 1;
            b.steps_per_split = split ? p.steps_per_split : b.nsteps;
            const dim3 g((unsigned)(b.tiles_r * b.tiles_t), (unsigned)b.KS);
            if (big) hipLaunchKernelGGL((spmm_ring2_kernel<NM_RING_BIG>), g, dim3(512), 0, s, b);
            // bf16: index words loaded 4 stages at a time (whole 64-byte runs of a row)
            else hipLaunchKernelGGL((spmm_ring_kernel<NM_RING_NARROW, 1, sizeof(T) == 2 ? 4 : 1>), g, dim3(256), 0, s, b);
        };
        if (p.split_rows > 0) {
            launch(true, 0, p.split_rows);
            launch(false, p.split_rows, a.R);
        } else {
            launch(p.big, 0, a.R);
        }
        if (p.KS <= 1) return check_launch("nm_spmm");
    } else if (p.large)
        hipLaunchKernelGGL((spmm_kernel<T, 2, 2, 2, 2>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((spmm_kernel<T, 4, 1, 1, 1>), grid, dim3(256), 0, s, a);
    if (p.KS > 1) {
        const int64_t total = a.Mtok * a.R;
        const dim3 g(grid_cap(ceil_div(total, 256), 8192));
        if (std::is_same<typename Mma<T>::AccS, float>::value)
            hipLaunchKernelGGL(spmm_reduce_kernel<float>, g, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(spmm_reduce_kernel<int32_t>, g, dim3(256), 0, s, a);
    }
    return check_launch("nm_spmm");
}

size_t spmm_lowrank_ws(int64_t Mtok, int64_t K, int64_t R, int Ns, int rank) {
    const size_t a =
        spmm_ws_layout(Mtok, K, R, Ns, NM_BF16, rank, true, lift_fused(Mtok, K, R, Ns, NM_BF16, true)).total();
    const size_t b = spmm_ws_layout(Mtok, K, R, Ns, NM_BF16, rank, false, false).total();
    return a > b ? a : b;
}

// Every workspace need of the call is known (and checked) before the first launch.
static nm_status spmm_impl(const char* fn, const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx,
                           const void* vals, const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi, int Ns,
                           const float* x_scale, float w_scale, const LowRankIn* lr, void* Y, nm_dtype ydt,
                           int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s) {
    if (Mtok == 0 || R == 0) return NM_OK;
    SpmmArgs a{};
    a.X = (const uint8_t*)X;
    a.vals = (const uint8_t*)vals;
    a.idx = idx;
    a.x_scale = x_scale;
    a.Y = Y;
    a.ldx = ldx;
    a.ldv = ldv;
    a.ldi = ldi;
    a.ldy = ldy;
    a.Mtok = Mtok;
    a.K = K;
    a.R = R;
    const int64_t Kl = lifted_cols(K, Ns);
    const int64_t es = xdt == NM_BF16 ? 2 : 1;
    a.comp_bytes = Kl / 2 * es;
    a.idx_words = (Kl + 31) / 32;   // the bitstream's last word is partial when K' % 32 == 16
    a.w_scale = w_scale;
    a.scaled = (x_scale != nullptr || w_scale != 1.0f) ? 1 : 0;
    a.ydt = (int)ydt;
    // the 2:4 product runs over the lifted width, on X itself (lifted inside the kernel, up
    // to 256 tokens of 6:8) or on the lifted activation that the workspace holds (256-byte
    // aligned, row stride K')
    a.K = Kl;
    a.xrow_bytes = K * es;
    bool ring_ok = ring_ok_for(a, es);
    const bool fused = lift_fused(Mtok, K, R, Ns, xdt, ring_ok);
    if (Ns && !fused) {
        a.ldx = Kl;
        ring_ok = ring_ok_for(a, es);
    }
    const int rank = lr ? lr->rank : 0;
    const SpmmWs w = spmm_ws_layout(Mtok, K, R, Ns, xdt, rank, ring_ok, fused);
    if (w.total() && (!ws || ws_bytes < w.total()))
        return set_error(NM_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, w.total());
    uint8_t* wp = (uint8_t*)ws;
    uint16_t* U = (uint16_t*)wp;
    float* PU = (float*)(wp + w.u);
    uint8_t* XL = wp + w.u + w.pu;
    void* F32 = XL + w.xl;
    void* PART = (uint8_t*)F32 + w.f32;
    if (lr) {
        // u = bf16(X A^T) from the original X, into the front of the workspace
        const LowRankPlan lp = lowrank_plan(Mtok, K);
        const dim3 g((unsigned)ceil_div(Mtok, 32), (unsigned)lp.ks);
        const int RT = (int)ceil_div(lr->rank, 32);
        const uint16_t* Xb = (const uint16_t*)X;
        switch (RT) {
            case 1: hipLaunchKernelGGL(lowrank_u_kernel<1>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
            case 2: hipLaunchKernelGGL(lowrank_u_kernel<2>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
            case 3: hipLaunchKernelGGL(lowrank_u_kernel<3>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
            case 4: hipLaunchKernelGGL(lowrank_u_kernel<4>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
            case 5: hipLaunchKernelGGL(lowrank_u_kernel<5>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
            case 6: hipLaunchKernelGGL(lowrank_u_kernel<6>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
            case 7: hipLaunchKernelGGL(lowrank_u_kernel<7>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
            default: hipLaunchKernelGGL(lowrank_u_kernel<8>, g, dim3(256), 0, s, Xb, ldx, lr->A, lr->lda, Mtok, K, lr->rank, lp.kchunk, PU); break;
        }
        const dim3 gr(grid_cap(ceil_div(Mtok * lr->rank, 256), 4096));
        hipLaunchKernelGGL(lowrank_u_reduce_kernel, gr, dim3(256), 0, s, (const float*)PU, lp.S(), Mtok, lr->rank, U);
        a.lr_u = U;
        a.ldu = lr->rank;
        a.lr_b = lr->B;
        a.ldb = lr->ldb;
        a.rank = lr->rank;
    }
    if (Ns && !fused) {
        // (2N-2):2N: lift X into the workspace, then the plain product over the lifted width
        if (Ns == 4) {
            const dim3 g(grid_cap(ceil_div(Mtok * (K / 8), 256), 8192));
            if (es == 1)   // int8 or FP8 codes: the lift moves bytes
                hipLaunchKernelGGL(lift68_kernel<int8_t>, g, dim3(256), 0, s, (const int8_t*)X, ldx, Mtok, K, (int8_t*)XL, Kl);
            else
                hipLaunchKernelGGL(lift68_kernel<uint16_t>, g, dim3(256), 0, s, (const uint16_t*)X, ldx, Mtok, K,
                                   (uint16_t*)XL, Kl);
        } else {
            const dim3 g(grid_cap(ceil_div(Mtok * (Kl / 4), 256), 8192));
            if (es == 1)
                hipLaunchKernelGGL(lift_kernel<int8_t>, g, dim3(256), 0, s, (const int8_t*)X, ldx, Mtok, K, Ns, (int8_t*)XL, Kl);
            else
                hipLaunchKernelGGL(lift_kernel<uint16_t>, g, dim3(256), 0, s, (const uint16_t*)X, ldx, Mtok, K, Ns,
                                   (uint16_t*)XL, Kl);
        }
        a.X = XL;
    }
    if (xdt == NM_I8) return run_spmm<int8_t>(a, ring_ok, fused, PART, F32, s);
    if (xdt == NM_FP8) return run_spmm<fp8e4m3>(a, ring_ok, fused, PART, F32, s);
    return run_spmm<uint16_t>(a, ring_ok, fused, PART, F32, s);
}

nm_status launch_spmm(const void* X, nm_dtype xdt, int64_t Mtok, int64_t K, int64_t ldx, const void* vals,
                      const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi, int Ns, const float* x_scale,
                      float w_scale, void* Y, nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s) {
    return spmm_impl("nm_spmm", X, xdt, Mtok, K, ldx, vals, idx, R, ldv, ldi, Ns, x_scale, w_scale, nullptr, Y, ydt,
                     ldy, ws, ws_bytes, s);
}

nm_status launch_spmm_lowrank(const void* X, int64_t Mtok, int64_t K, int64_t ldx, const void* vals,
                              const uint32_t* idx, int64_t R, int64_t ldv, int64_t ldi, int Ns, const LowRankIn& lr,
                              void* Y, nm_dtype ydt, int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s) {
    return spmm_impl("nm_spmm_lowrank", X, NM_BF16, Mtok, K, ldx, vals, idx, R, ldv, ldi, Ns, nullptr, 1.0f, &lr, Y,
                     ydt, ldy, ws, ws_bytes, s);
}

// Stage width and ring depth of the dense split ring (Hutchinson's products, bitmap decode).
// Measured on the Hutchinson call at 28672 x 8192, n = 1024, 8 probes (same result bit for
// bit): 64-column stages in 2 slots 7.17 ms, 32-column stages in 4 slots 7.68 ms, in 5
// slots 7.73 ms -- more bytes in flight do not help; the extra barriers cost.  Neither did
// an L2 prefetch of the next stage's lines (one dword per line, 7.05 against 6.82 ms), nor
// four waves of 128 x 128 per tile with AGPR accumulators (a dense 28672 x 8192 product at
// 8192 tokens: 4.13 against 3.52 ms; one wave per SIMD leaves nothing to cover the waits).
// Nor a ping-pong schedule (waves w and w + 4 of a SIMD alternating a phase of fragment
// reads with a phase of 16 or 32 MFMAs, a block barrier after every phase, the second
// four waves one phase late): the same Hutchinson time, the U product 6% and the dense
// product 15% slower.  The one barrier per stage is not what holds the MFMA pipes idle.
// Under this load the clock falls to 1.6-1.8 GHz (GRBM cycles over the dispatch time); a
// copy that skips the stage loads runs at 1.9-2.1 GHz: the operand traffic costs power as
// well as issue slots, and a 256 x 256 tile is the largest two waves per SIMD can hold.
constexpr int kDenseSK = 64, kDenseNS = 2;

// Y [Mtok, R] (ydt bf16 or f32, ldy) = X [Mtok, K] (ldx) W^T, W [R, K] (ldw) dense bf16.
// NM_ERR_SHAPE (nothing launched) when the kernel does not apply: K % 64, unaligned rows,
// operands past 32-bit offsets, or fewer 256 x 256 tiles than CUs.
nm_status launch_dense_ring(const uint16_t* W, int64_t ldw, const uint16_t* X, int64_t ldx, int64_t Mtok, int64_t K,
                            int64_t R, void* Y, nm_dtype ydt, int64_t ldy, hipStream_t s) {
    constexpr int SR = 4, ST = 2, WRN = 2, WTN = 4, BR = WRN * SR * 32, BT = WTN * ST * 32;
    const int64_t tiles = ceil_div(R, BR) * ceil_div(Mtok, BT);
    if (K % 64 || ((uintptr_t)W & 15u) || ((uintptr_t)X & 15u) || ldw % 8 || ldx % 8 || R * ldw * 2 >= (1LL << 32) ||
        Mtok * ldx * 2 >= (1LL << 32) || tiles < device_cus())
        return NM_ERR_SHAPE;
    SpmmArgs a{};
    a.X = (const uint8_t*)X;
    a.vals = (const uint8_t*)W;
    a.Y = Y;
    a.ldx = ldx;
    a.ldv = ldw;
    a.ldy = ldy;
    a.Mtok = Mtok;
    a.K = K;
    a.R = R;
    a.ydt = (int)ydt;
    a.scaled = 0;
    a.rank = 0;
    a.nsteps = (int)(K / kDenseSK);
    a.tiles_r = (int)ceil_div(R, BR);
    a.tiles_t = (int)ceil_div(Mtok, BT);
    hipLaunchKernelGGL((dense_ring_kernel<SR, ST, WRN, WTN, 0, kDenseSK, kDenseNS>), dim3((unsigned)tiles),
                       dim3(64 * WRN * WTN), 0, s, a);
    return check_launch("dense product");
}

// D [R, K] (ldd) = (2/P) sum_p V_p .* (U_p X): U [P*R, n] and XT [K, n] bf16 in the workspace.
// With sc (score epilogue): S [R, K] (ldd) = (D + eps) W^2 instead of D, and the moments of S
// per block into sc->mpart ([3][hutch_ring_blocks(K, R)]).
nm_status launch_hutch_ring(const uint16_t* U, const uint16_t* XT, int64_t n, int64_t K, int64_t R, int probes,
                            uint64_t seed, float* D, int64_t ldd, hipStream_t s, const HutchScore* sc) {
    constexpr int SR = 4, ST = 2, WRN = 2, WTN = 4, BR = WRN * SR * 32, BT = WTN * ST * 32;
    if (n % 64 || K % 64 || ((uintptr_t)U & 15u) || ((uintptr_t)XT & 15u) || (int64_t)probes * R * n * 2 >= (1LL << 32) ||
        K * n * 2 >= (1LL << 32) || (int64_t)probes * (n / 64) >= (1LL << 31))
        return NM_ERR_SHAPE;
    SpmmArgs a{};
    a.vals = (const uint8_t*)XT;   // A: rows k of D's columns
    a.ldv = n;
    a.X = (const uint8_t*)U;       // B: rows o of U_p
    a.ldx = n;
    a.Y = D;
    a.ydt = NM_F32;
    a.ldy = ldd;
    a.Mtok = R;
    a.R = K;
    a.K = n;
    a.scaled = 1;
    a.w_scale = 2.0f / (float)probes;
    a.seed = seed;
    a.probes = probes;
    a.pstages = (int)(n / kDenseSK);
    a.nsteps = probes * a.pstages;
    a.tiles_r = (int)ceil_div(K, BR);
    a.tiles_t = (int)ceil_div(R, BT);
    const int64_t tiles = (int64_t)a.tiles_r * a.tiles_t;
    if (sc) {
        a.sw = sc->W;
        a.ldsw = sc->ldw;
        a.eps = sc->eps;
        a.mpart = sc->mpart;
        hipLaunchKernelGGL((dense_ring_kernel<SR, ST, WRN, WTN, 3, kDenseSK, kDenseNS>), dim3((unsigned)tiles),
                           dim3(64 * WRN * WTN), 0, s, a);
    } else {
        hipLaunchKernelGGL((dense_ring_kernel<SR, ST, WRN, WTN, 1, kDenseSK, kDenseNS>), dim3((unsigned)tiles),
                           dim3(64 * WRN * WTN), 0, s, a);
    }
    return check_launch("nm_hdiag_hutchinson");
}

int64_t hutch_ring_blocks(int64_t K, int64_t R) { return ceil_div(K, 256) * ceil_div(R, 256); }

// U [P*R, n] (bf16, row stride n) = V X^T, X [n, K] (ldx); V from the probes' Rademacher words.
nm_status launch_hutch_u_ring(const uint16_t* X, int64_t ldx, int64_t n, int64_t K, int64_t R, int probes,
                              uint64_t seed, uint16_t* U, hipStream_t s) {
    constexpr int SR = 4, ST = 2, WRN = 2, WTN = 4, BR = WRN * SR * 32, BT = WTN * ST * 32;
    // per-lane DMA offsets are 32-bit from the block's first row: 256 rows and a row's columns
    if (K % 64 || ((uintptr_t)X & 15u) || ldx % 8 || (256 * ldx + K) * 2 >= (1LL << 32)) return NM_ERR_SHAPE;
    SpmmArgs a{};
    a.vals = (const uint8_t*)X;   // A: rows i of the calibration set
    a.ldv = ldx;
    a.Y = U;
    a.ydt = NM_BF16;
    a.ldy = n;
    a.Mtok = (int64_t)probes * R;   // B: stacked probe rows
    a.R = n;
    a.K = K;
    a.seed = seed;
    a.probes = probes;
    a.prows = R;
    a.nsteps = (int)(K / kDenseSK);
    a.tiles_r = (int)ceil_div(n, BR);
    a.tiles_t = (int)ceil_div(a.Mtok, BT);
    const int64_t tiles = (int64_t)a.tiles_r * a.tiles_t;
    hipLaunchKernelGGL((dense_ring_kernel<SR, ST, WRN, WTN, 2, kDenseSK, kDenseNS>), dim3((unsigned)tiles),
                       dim3(64 * WRN * WTN), 0, s, a);
    return check_launch("nm_hdiag_hutchinson");
}

}  // namespace nm
