// Gathered 4-bit (or 8-bit) quantised matmuls over expert tiles: the kernels
// and their launchers, included by one translation unit per (group size,
// code width) pair (gemm_g*_b*.hip), which instantiates them.
//
//   gate|up  h[s, n] = act(x[tok(s)] . Wg[e, n]) * (x[tok(s)] . Wu[e, n]),
//            act = gelu_tanh (GeGLU), or silu with MOE_F_SWIGLU (SwiGLU)
//   down     y[perm[s], m] = w[perm[s]] * (h[s] . Wd[e, m])
//
// Prior art: the expert-tile QMM of the Layr-Labs/mlx PR #4 page ("What":
// expert tiles with short fallback tiles over sorted indices, one private row
// count per tile), the compiled gelu-product of SwiftLM issue #236 ("Still
// missing") and the direct weighted unsort of the PR #4 page ("Measured
// standing").  Design for gfx950:
//
//  * Every product runs on v_mfma_f32_16x16x32_bf16.  The weight operand is
//    the code itself, exactly (codes_as_bf16: OFF + q for 4-bit codes, OFF =
//    16 in the fp32 intermediate mode and 128 in the bf16 mode;
//    bytes_as_bf16: q for 8-bit ones), decoded in registers.  Per group (a
//    chain of 32 or 64 columns) the fp32 accumulator takes s * P (one FMA per
//    output per chain); the rest, sum_g (b - OFF s) X, is itself a
//    small contraction over groups, run on MFMAs once per tile after the
//    groups, with both factors split into bf16 hi + lo.  Rounding dequantised
//    weights to bf16 instead would cost the accuracy the fp32 path needs.
//  * Activations come pre-ordered (x_perm, from the route launch) with their
//    group sums, so nothing here reorders or sums activations on the fly.
//  * Skinny path, tiles of <= 16 rows (decode): one wave per workgroup, no
//    activation staging and no barrier; each wave streams its own weight
//    rows (16-byte coalesced loads, turned into operand order through a
//    small LDS buffer) with RING chunks of loads in flight, and issues the
//    MFMA chains of a chunk's groups and blocks together.
//  * Wide path, tiles of up to 64 rows (prefill): the activation tile is
//    staged in LDS, double-buffered; each wave owns 4 column blocks and all
//    row blocks, so a decoded weight word feeds every row block and an LDS
//    activation fragment feeds 4 MFMAs; weights go through a per-wave LDS
//    transpose as on the skinny path.
//  * Both paths do the same arithmetic in the same order for every output
//    element, so results do not depend on how rows are grouped into tiles
//    (hence not on the order of the tokens).
//  * Gate and up of an output column sit in the same lane: the GeGLU (or
//    SwiGLU) product is formed in registers and h is written once, already
//    in MFMA operand order, with its 16-column block sums, from which the
//    down matmul forms the group sums it needs.
//  * The down kernels scale each row by its routing weight and write it to
//    its original (token, slot) position: the weighted unsort.
//  * Each path reads its own tile list (experts of more than 16 rows, cut
//    into near-equal tiles; experts of 1..16 rows).  Grids are sized from
//    bounds the host knows (at most one skinny tile per expert, at most
//    max_tiles wide tiles) and workgroups past the list's device-side count
//    exit at once: the host never reads it back.
#pragma once

#include "moe_internal.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kThreads = 256;
// skinny paths (one wave per workgroup): 16-column weight blocks per wave
// and weight chunks in flight
constexpr int kSkinnyGateUpRing = 2;
constexpr int kSkinnyDownBlocks = 2, kSkinnyDownRing = 2;

// A buffer resource over n bytes at p (p the same in every lane): a 16-byte
// load through it at a byte offset at or past n returns zeros and reads no
// memory.  Word 3 = 0x00020000: 32-bit data format, no swizzle.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(n), 0x00020000);
}
// 16 bytes at byte offset voff + soff (soff the same in every lane).
__device__ __forceinline__ u32x4 load16(Rsrc r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Start of a skinny chunk: nothing moves across.  The memory counter a wave
// waits on retires loads in issue order, so a wait for one load is a wait for
// every earlier one.  Without the fence the scheduler lifts the weight reload
// above the next chunk's activation loads, or a chunk's LDS put (and the wait
// for its weights) above the previous chunk's arithmetic; either way a chunk
// waits for weights it needs only later, and the ring is shallower than it
// looks.
__device__ __forceinline__ void chunk_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Skinny work item blockIdx.x: tile blockIdx.x / ncb of the skinny list
// (tiles of at most kBmSmall rows), column block blockIdx.x % ncb; tile
// {-1, ..} past the list's device-side count.  Column blocks vary fastest, so
// the workgroups past the count are the last ones dispatched: the dispatcher
// hands runs of consecutive workgroups to one CU, and exiting workgroups
// spread through the grid left whole CUs without work.  The entry and the
// count are read together (the grid never exceeds the list's capacity, so the
// entry read stays inside it).
__device__ __forceinline__ int4 load_skinny_tile(const FfnArgs& a, int ncb, int& cb) {
    const int ti = static_cast<int>(blockIdx.x) / ncb;
    cb = static_cast<int>(blockIdx.x) - ti * ncb;
    const int4 t = reinterpret_cast<const int4*>(a.tiles_skinny)[ti];
    const int n = min(a.num_tiles[3], a.max_skinny);
    return ti < n ? t : int4{-1, 0, 0, 0};
}

// ------------------------------------------------------------ group geometry
// A chunk is 128 columns of K: four MFMA slices of 32 columns (one weight word
// per lane and slice).  The K loop scales products in chains of kChain
// columns: a chain's slices are chained from zero on the MFMA, then acc += s P
// with the scale of the chain's group.  A group of 32 or 64 columns is one
// chain; a group of 128 columns is two chains of 64 with the same scale (one
// chain of four slices would need twice the decoded weights in registers at
// once).  K may end in a half chunk of 64 columns (not with GS = 128, where H
// and I are multiples of 128).
template <int GS>
struct Geo {
    static_assert(GS == 32 || GS == 64 || GS == 128, "group size");
    static constexpr int kChain = GS < 64 ? GS : 64;    // columns per scaled chain
    static constexpr int kSlices = kChain / 32;         // MFMA slices per chain
    static constexpr int kChains = 128 / kChain;        // chains per chunk
    static constexpr int kShift = GS == 128 ? 1 : 0;    // chain index >> kShift = group
    static constexpr int kMaxG = kMaxDim / GS;          // groups per row, at most
    static constexpr int kSteps = (kMaxG + 31) / 32;    // bias-contraction MFMA steps
    // The chunk word (0..15) that lane group q feeds to slice s.  The four words
    // of a slice (q = 0..3) lie in one chain.  64-column chains: words 2q and
    // 2q + 1 of each chain; 32: word 4 s + q.
    static __device__ __forceinline__ constexpr int word(int s, int q) {
        return kChain == 64 ? 8 * (s >> 1) + 2 * q + (s & 1) : 4 * s + q;
    }
};

// --------------------------------------------------------------- bias term
// Operand of the bias contraction for one lane: 8 consecutive groups per MFMA
// step (group 32 st + 8 q + j in element j), split into bf16 hi and lo.
template <int NS>
struct BiasOp {
    u32x4 hi[NS];
    u32x4 lo[NS];
};

__device__ __forceinline__ void pack_split(const float (&v)[8], u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hi[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
        lo[j] = pack_bf16x2(v[2 * j] - __uint_as_float(hi[j] << 16),
                            v[2 * j + 1] - __uint_as_float(hi[j] & 0xFFFF0000u));
    }
}

// Column operand: c[g] = b[g] - OFF s[g] of one weight row (OFF the code
// offset), from its rows of the scale and bias tables.  Entries past G read
// whatever follows the row in LDS (the next row, or the next member of the
// shared-memory struct: at most 32 NS - 1 entries past the last row) at fixed
// offsets from one address, and are replaced by 0, so no bits read there
// reach the product.
template <int NS, int OFF = 16>
__device__ __forceinline__ void bias_from_table(BiasOp<NS>& o, const uint16_t* ts, const uint16_t* tb,
                                                int G, int q, int steps, bool active) {
    const uint16_t* const s8 = ts + 8 * q;
    const uint16_t* const b8 = tb + 8 * q;
    const int lim = active ? G - 8 * q : 0;  // entries j of step st valid while 32 st + j < lim
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        if (st < steps) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float c =
                    fmaf(-static_cast<float>(OFF), bf16_to_f32(s8[32 * st + j]), bf16_to_f32(b8[32 * st + j]));
                v[j] = 32 * st + j < lim ? c : 0.f;
            }
            pack_split(v, o.hi[st], o.lo[st]);
        }
    }
}

// Group sum g of h from its GS / 16 block sums of 16 columns (h_sums row
// X16), added in block order ((b0 + b1) + b2) + ..., the one order every path
// uses.
template <int GS>
__device__ __forceinline__ float group_of_blocks(const float* X16, int g) {
    if constexpr (GS == 32) {
        const f32x2 b = *reinterpret_cast<const f32x2*>(X16 + 2 * g);
        return b[0] + b[1];
    } else if constexpr (GS == 64) {
        const f32x4 b = *reinterpret_cast<const f32x4*>(X16 + 4 * g);
        return ((b[0] + b[1]) + b[2]) + b[3];
    } else {
        const f32x4 b = *reinterpret_cast<const f32x4*>(X16 + 8 * g);
        const f32x4 c = *reinterpret_cast<const f32x4*>(X16 + 8 * g + 4);
        return ((((((b[0] + b[1]) + b[2]) + b[3]) + c[0]) + c[1]) + c[2]) + c[3];
    }
}

// The GS / 16 block sums of one group, loaded now and added later in the
// order of group_of_blocks.
template <int GS>
struct BlockSums {
    float b[GS / 16];
    __device__ __forceinline__ void load(const float* X16, int g) {
        if constexpr (GS == 32) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(X16 + 2 * g);
            b[0] = v[0];
            b[1] = v[1];
        } else {
#pragma unroll
            for (int h = 0; h < GS / 64; ++h) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(X16 + (GS / 16) * g + 4 * h);
#pragma unroll
                for (int i = 0; i < 4; ++i) b[4 * h + i] = v[i];
            }
        }
    }
    __device__ __forceinline__ float sum() const {
        float v = b[0];
#pragma unroll
        for (int i = 1; i < GS / 16; ++i) v += b[i];
        return v;
    }
};

// The group sums of one activation row as the bias operand (NS steps).
template <int NS>
struct RowSums {
    float v[NS][8];

    __device__ __forceinline__ void load(const float* X, int G, int q) {
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int j = 0; j < 8; ++j) v[st][j] = X[min(32 * st + 8 * q + j, G - 1)];
    }
    // from the 16-column block sums of the row (G * GS / 16 floats); steps past
    // the ones used are left unread
    template <int GS>
    __device__ __forceinline__ void load_blocks(const float* X16, int G, int q, int steps) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            if (st < steps) {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[st][j] = group_of_blocks<GS>(X16, min(32 * st + 8 * q + j, G - 1));
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[st][j] = 0.f;
            }
        }
    }
    __device__ __forceinline__ void pack(BiasOp<NS>& o, int G, int q, int steps) const {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            if (st < steps) {
                float w[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) w[j] = (32 * st + 8 * q + j < G) ? v[st][j] : 0.f;
                pack_split(w, o.hi[st], o.lo[st]);
            }
        }
    }
};

// sum_g c[n, g] X[m, g] for one 16x16 block: hi*hi + hi*lo + lo*hi per step.
template <int NS>
__device__ __forceinline__ f32x4 bias_mfma(const BiasOp<NS>& A, const BiasOp<NS>& B, int steps) {
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        if (st < steps) {
            r = mfma16(A.hi[st], B.hi[st], r);
            r = mfma16(A.hi[st], B.lo[st], r);
            r = mfma16(A.lo[st], B.hi[st], r);
        }
    }
    return r;
}

// P of one group for one 16x16 block: the group's NSL slices chained from
// zero, in slice order (with P = 2 each slice's activation is hi + lo: the hi
// part first).  Then acc += s P.  Every path goes through exactly this.
template <int NSL, int P = 1>
__device__ __forceinline__ f32x4 group_step(f32x4 acc, const u32x4 (&x)[NSL][P], const u32x4 (&b)[NSL],
                                            float s16) {
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
        for (int pp = 0; pp < P; ++pp) p = mfma16(x[sl][pp], b[sl], p);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = fmaf(s16, p[v], acc[v]);
    return acc;
}

// A lane's weight words for the four slices of a chunk: one per slice for
// 4-bit codes, two (words 2 s and 2 s + 1) for 8-bit codes.
template <int BITS>
using WLane = std::conditional_t<BITS == 4, u32x4, u32x8>;

// Slice s's weight operand from the lane's words.
template <int BITS, int OFF>
__device__ __forceinline__ u32x4 slice_operand(const WLane<BITS>& w, int s, CodeConsts<OFF> kc) {
    if constexpr (BITS == 4) {
        return codes_as_bf16(w[s], kc);
    } else {
        return bytes_as_bf16(w[2 * s], w[2 * s + 1]);
    }
}

// The groups of one chunk (NSL = 4 slices, or 2 for a half chunk) for NB
// weight blocks: the MFMA chains of all (block, group) pairs are issued
// together, slice by slice, then each block takes its scaled products in group
// order -- group_step's arithmetic, pair by pair.  x[s]: slice s's activation
// operand; wv[b]: block b's weight words.
template <int GS, int NB, int NSL, int BITS, int OFF>
__device__ __forceinline__ void chunk_steps(f32x4 (&acc)[NB], const u32x4 (&x)[4], const WLane<BITS> (&wv)[NB],
                                            const float (&s16)[NB][Geo<GS>::kChains], CodeConsts<OFF> kc) {
    constexpr int MPG = Geo<GS>::kSlices, NG = NSL / MPG;
    static_assert(NSL % MPG == 0, "a chunk holds whole groups");
    f32x4 p[NB][NG];
#pragma unroll
    for (int m = 0; m < MPG; ++m)
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                p[b][j] = mfma16(x[j * MPG + m], slice_operand<BITS, OFF>(wv[b], j * MPG + m, kc),
                                 m == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : p[b][j]);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NG; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[b][v] = fmaf(s16[b][j], p[b][j][v], acc[b][v]);
}

// A bf16 scale as the factor of P.
__device__ __forceinline__ float scale16(uint16_t t) { return bf16_to_f32(t); }

// v from another lane of the same 16-lane row, by a DPP control (no LDS).
// Every control used here reads inside the row; with bound_ctrl set the move
// folds into the add that consumes it (one v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum over the 16 lanes of a 16-lane row (the same value in every lane): a
// butterfly, lane i adding lane i ^ 1, i ^ 2, i ^ 4, i ^ 8 in turn.  The first
// two are quad permutations; after them the value is the same across each
// quad, so the half-row mirror (lane i of 8 -> 7 - i) reads lane i ^ 4's
// value, and after that the row mirror (i -> 15 - i) reads lane i ^ 8's.
__device__ __forceinline__ float sum16(float v) {
    v += dpp_row<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_row<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_row<0x141>(v);  // row_half_mirror
    v += dpp_row<0x140>(v);  // row_mirror
    return v;
}

// h of the rows [row_begin, row_begin + rows) of a tile, stored once in
// operand order, and their 16-column block sums.  The stores go through
// buffer resources over exactly those rows (none for a wave without columns),
// so a store for a row past the tile falls outside and is dropped: no branch
// per store, 32-bit offsets.
template <bool kF32H>
struct HOut {
    Rsrc hi, lo, sums;
    int I;

    __device__ __forceinline__ void init(const FfnArgs& a, size_t A, int row_begin, int rows, bool active) {
        I = a.I;
        const uint32_t n = active ? static_cast<uint32_t>(rows) : 0u;
        uint16_t* const h = static_cast<uint16_t*>(a.h) + static_cast<size_t>(row_begin) * I;
        hi = make_rsrc(h, n * I * 2u);
        if constexpr (kF32H) lo = make_rsrc(h + A * I, n * I * 2u);
        sums = make_rsrc(a.hs + static_cast<size_t>(row_begin) * (I / 16), n * (I / 16) * 4u);
    }
    // h = act(g) * u for tile row r, column hcol (act = silu with kSilu, else
    // gelu_tanh); returns the value the down matmul will see (bf16 h, or hi + lo)
    template <bool kSilu>
    __device__ __forceinline__ float put(int r, int hcol, float g, float u) const {
        const float hv = (kSilu ? silu(g) : gelu_tanh(g)) * u;
        const uint32_t off = 2u * static_cast<uint32_t>(r * I + (hcol & ~7) + permuted_pos(hcol & 7));
        const uint16_t h16 = f32_to_bf16(hv);
        float seen = bf16_to_f32(h16);
        if constexpr (kF32H) {
            const uint16_t l16 = f32_to_bf16(hv - seen);
            seen += bf16_to_f32(l16);
            __builtin_amdgcn_raw_buffer_store_b16(l16, lo, off, 0, 0);
        }
        __builtin_amdgcn_raw_buffer_store_b16(h16, hi, off, 0, 0);
        return seen;
    }
    // the 16-column block sum of row r (its 16 lanes' values), block cb16
    __device__ __forceinline__ void put_sum(int r, int cb16, float seen, int lr) const {
        const float s = sum16(seen);
        const uint32_t off = lr == 0 ? 4u * static_cast<uint32_t>(r * (I / 16) + cb16) : 0xFFFFFFF0u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), sums, off, 0, 0);
    }
};

// ================================================== weights through LDS
// The MFMA operand wants lane (lr, q) to hold words 2q, 2q+1 of weight row lr
// for each group, so lanes next to each other would read rows 1.4 KB apart:
// every 4-lane quad would touch 4 cache lines and the vector L1 tag lookups,
// not HBM, would set the pace.  Instead each lane loads 16 contiguous bytes
// (4 lanes per row: a quad reads one line) and the chunk is turned into
// operand order through a small LDS buffer private to the wave (no barrier).
//
// A wave owns NCB blocks of 16 weight rows.  With 4-bit codes a chunk is 64
// bytes per row: 16 words w = 8 g + 2 q + p (g the 64-column half, p = 0, 1),
// word w at u32 offset 4 * (q ^ ((row >> 2) & 3)) + 2 g + p of a 16-u32 LDS
// row; the XOR keeps the 16 rows of a fragment read on distinct banks.  With
// 8-bit codes a chunk is 128 bytes per row, and the pair of words holding the
// columns of 4-bit word w sits where w would, in 8-byte units of a 32-u32 row.
template <int NCB, int GS = 64, int BITS = 4>
struct WaveW {
    static constexpr int kParts = BITS / 4;       // 16-byte loads per lane and block
    static constexpr int kRowU32 = 16 * kParts;   // u32 per LDS row
    uint32_t* lds;   // NCB * 16 rows x kRowU32 u32
    Rsrc blk[NCB];   // block cb: its 16 weight rows
    uint32_t voff;   // this lane's load row and piece, bytes

    // blocks at blk_ptr[cb] (the same in every lane), rows of row_words u32
    __device__ __forceinline__ void init(uint32_t* l, const uint32_t* const (&blk_ptr)[NCB],
                                         int row_words) {
        const int lane = threadIdx.x & 63;
        lds = l;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) blk[cb] = make_rsrc(blk_ptr[cb], 64u * row_words);
        voff = 4u * ((lane >> 2) * row_words + 4 * (lane & 3));
    }
    // Chunk c (part h at 64 h bytes).  Pieces past a row's end (the second half
    // of a half chunk, chunks past the last) read the next row or, past the
    // block, zeros; they are never used.
    __device__ __forceinline__ void load(int c, u32x4 (&v)[NCB][kParts]) const {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int h = 0; h < kParts; ++h) v[cb][h] = load16(blk[cb], voff, 64u * (kParts * c + h));
    }
    __device__ __forceinline__ void put(const u32x4 (&v)[NCB][kParts]) const {
        const int lane = threadIdx.x & 63;
        const int j = lane & 3, sw = (lane >> 4) & 3;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            uint32_t* row = lds + (16 * cb + (lane >> 2)) * kRowU32;
            if constexpr (BITS == 4) {
                const int g = j >> 1, qa = 2 * (j & 1);
                *reinterpret_cast<u32x2*>(row + 4 * (qa ^ sw) + 2 * g) = u32x2{v[cb][0][0], v[cb][0][1]};
                *reinterpret_cast<u32x2*>(row + 4 * ((qa + 1) ^ sw) + 2 * g) = u32x2{v[cb][0][2], v[cb][0][3]};
            } else {
                // part h: words 4 j .. 4 j + 3 of half h = the pairs of 4-bit
                // words 8 h + 2 j and 8 h + 2 j + 1
#pragma unroll
                for (int h = 0; h < 2; ++h) *reinterpret_cast<u32x4*>(row + 8 * (j ^ sw) + 4 * h) = v[cb][h];
            }
        }
    }
    // The words lane (lr, q) feeds to slices 0..3 (Geo<GS>::word) of row
    // 16 cb + lr; for 64-column chains one contiguous read ([g0 word 2q,
    // g0 word 2q+1, g1 word 2q, g1 word 2q+1], pairs of words for 8-bit codes).
    __device__ __forceinline__ WLane<BITS> get(int cb, int lr, int q) const {
        const uint32_t* row = lds + (16 * cb + lr) * kRowU32;
        const int sw = (lr >> 2) & 3;
        if constexpr (BITS == 4) {
            if constexpr (Geo<GS>::kChain == 64) {
                return *reinterpret_cast<const u32x4*>(row + 4 * (q ^ sw));
            } else {
                // word w sits at 4 ((w & 7) >> 1 ^ sw) + 2 (w >> 3) + (w & 1)
                u32x4 r;
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    const int w = Geo<GS>::word(sl, q);
                    r[sl] = row[4 * (((w & 7) >> 1) ^ sw) + 2 * (w >> 3) + (w & 1)];
                }
                return r;
            }
        } else {
            u32x8 r;
            if constexpr (Geo<GS>::kChain == 64) {
                const u32x4 lo = *reinterpret_cast<const u32x4*>(row + 8 * (q ^ sw));
                const u32x4 hi = *reinterpret_cast<const u32x4*>(row + 8 * (q ^ sw) + 4);
                r = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            } else {
#pragma unroll
                for (int sl = 0; sl < 4; ++sl) {
                    const int w = Geo<GS>::word(sl, q);
                    const u32x2 pr = *reinterpret_cast<const u32x2*>(
                        row + 2 * (4 * (((w & 7) >> 1) ^ sw) + 2 * (w >> 3) + (w & 1)));
                    r[2 * sl] = pr[0];
                    r[2 * sl + 1] = pr[1];
                }
            }
            return r;
        }
    }
};

// Scale and bias rows of NCB blocks of 16 weight rows, copied raw into a
// wave's LDS tables (entry (row, g) at row * G + g).  A block's 16 rows are
// contiguous, 32 G bytes, so they move as 16-byte pieces in row order: NP
// loads per lane and table cover G <= 32 NP.  The loads are issued early and the
// stores made later, so their latency overlaps the first weight loads.
// kBias = false: scales only (the wide paths read biases from HBM at the end).
template <int NCB, bool kBias = true, int NP = 2>
struct Tables {
    u32x4 vs[NCB][NP], vb[NCB][kBias ? NP : 1];  // NP pieces per lane cover G <= 32 NP

    __device__ __forceinline__ void load(const uint16_t* s, const uint16_t* b,
                                         const size_t (&row0)[NCB], int G) {
        const int lane = threadIdx.x & 63;
        const uint32_t n = 32u * G;  // 16 rows of G bf16; pieces past it read zeros
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const Rsrc rs = make_rsrc(s + row0[cb] * G, n);
#pragma unroll
            for (int j = 0; j < NP; ++j) vs[cb][j] = load16(rs, 16u * (lane + 64 * j), 0);
            if constexpr (kBias) {
                const Rsrc rb = make_rsrc(b + row0[cb] * G, n);
#pragma unroll
                for (int j = 0; j < NP; ++j) vb[cb][j] = load16(rb, 16u * (lane + 64 * j), 0);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* ts, uint16_t* tb, int G) const {
        const int lane = threadIdx.x & 63, np = 2 * G;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int idx = lane + 64 * j;
                if (idx < np) {
                    *reinterpret_cast<u32x4*>(ts + cb * 16 * G + 8 * idx) = vs[cb][j];
                    if constexpr (kBias)
                        *reinterpret_cast<u32x4*>(tb + cb * 16 * G + 8 * idx) = vb[cb][j];
                }
            }
    }
};

// =========================================================== skinny paths
// One wave's LDS: NB 16-row weight blocks.
template <int NB, int MAXG, int BITS>
struct alignas(16) SkinnySmem {
    uint32_t w[NB * 16 * 4 * BITS];  // weight transposition buffer (16 or 32 u32 per row)
    uint16_t ts[NB * 16 * MAXG];   // scales of the wave's weight rows
    uint16_t tb[NB * 16 * MAXG];   // biases
    int32_t dst[kBmSmall];         // down: destination slot of each row
    float wt[kBmSmall];            // down: its routing weight
};

// gate|up, tiles of <= 16 rows.  Grid: skinny tiles x I / 16 column blocks;
// one wave per workgroup owns 16 columns of h, i.e. weight block gate (rows
// n0 .. n0 + 15) and block up (rows I + n0 ..), and writes their 16-column
// block sums of h.
// RING chunks of weights are in flight.
template <bool kF32H, int RING, int GS, int BITS>
__global__ __launch_bounds__(64, GS == 32 || BITS == 8 ? 2 : 3) void moe_gateup_skinny(FfnArgs a) {
    constexpr int NB = 2, NS = Geo<GS>::kSteps, GPC = Geo<GS>::kChains, SH = Geo<GS>::kShift;
    constexpr int OFF = kCodeOffset<BITS, kF32H>;
    __shared__ SkinnySmem<NB, Geo<GS>::kMaxG, BITS> sm;
    int cb;
    const int4 tile = load_skinny_tile(a, a.I / 16, cb);
    if (tile.x < 0) return;
    const int e = tile.x, row_begin = tile.y, rows = tile.z;
    const int lane = threadIdx.x & 63, q = lane >> 4, lr = lane & 15;
    const int H = a.H, I = a.I, G = H / GS;
    const size_t A = static_cast<size_t>(a.T) * a.k;
    const int hcol0 = cb * 16;

    size_t row0[NB];
    const uint32_t* blk[NB];
    row0[0] = static_cast<size_t>(e) * 2 * I + hcol0;
    row0[1] = row0[0] + I;
#pragma unroll
    for (int b = 0; b < NB; ++b) blk[b] = a.w_gu + row0[b] * (H / 32 * BITS);
    // the row's token first: loads retire in issue order, so the activation
    // loads that depend on it can go out while the tables and weights are
    // still in flight (padding lanes, row >= rows, read row 0: their outputs
    // are never stored)
    const int tok = a.perm[row_begin + min(lr, rows - 1)] / a.k;
    Tables<NB, true, Geo<GS>::kMaxG / 32> tab;
    tab.load(a.s_gu, a.b_gu, row0, G);
    WaveW<NB, GS, BITS> ww;
    ww.init(sm.w, blk, H / 32 * BITS);
    u32x4 rv[RING][NB][BITS / 4];
#pragma unroll
    for (int i = 0; i < RING; ++i) ww.load(i, rv[i]);

    const uint32_t* xa = reinterpret_cast<const uint32_t*>(a.xp) + static_cast<size_t>(tok) * (H / 2);
    u32x4 ra[2][4];
    // slice s of chunk c: the activation piece of chunk word Geo<GS>::word(s, q),
    // in 64-column half 2 c + s / 2 (the same in every lane; past K the last
    // half is read again and never used)
    constexpr bool kC64 = Geo<GS>::kChain == 64;
    const uint32_t* const xq = xa + (kC64 ? 8 : 4) * q;
    auto load_a = [&](int c, int buf) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint32_t* const xg = xq + static_cast<uint32_t>(32 * min(2 * c + hf, H / 64 - 1));
#pragma unroll
            for (int s = 0; s < 2; ++s)
                ra[buf][2 * hf + s] = *reinterpret_cast<const u32x4*>(xg + (kC64 ? 4 : 16) * s);
        }
    };
    load_a(0, 0);
    // the bias term's row sums, loaded early; the term itself is formed as soon
    // as the tables are in place and added after the groups (the same
    // arithmetic as forming it there), so no load waits at the end
    const int steps = (G + 31) / 32;
    RowSums<NS> xsum;
    xsum.load(a.xs + static_cast<size_t>(tok) * G, G, q);

    tab.store(sm.ts, sm.tb, G);
    __builtin_amdgcn_wave_barrier();
    f32x4 bterm[NB];
    {
        BiasOp<NS> X;
        xsum.pack(X, G, q, steps);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            BiasOp<NS> C;
            bias_from_table<NS, OFF>(C, sm.ts + (16 * b + lr) * G, sm.tb + (16 * b + lr) * G, G, q,
                                                   steps, true);
            bterm[b] = bias_mfma(X, C, steps);
        }
    }

    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nfull = H / 128, nch = (H + 127) / 128;
    const CodeConsts<OFF> kc = code_consts<OFF>(a.zero);
    // chunk c: its weights go through LDS, the slot reloads with chunk c + RING
    // at once, then the MFMAs run (K may end in a half chunk of 64 columns)
    auto compute = [&](int slot, int abuf, int c, bool reload, bool full) {
        chunk_fence();
        ww.put(rv[slot]);
        if (reload) ww.load(c + RING, rv[slot]);
        __builtin_amdgcn_wave_barrier();
        WLane<BITS> wv[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) wv[b] = ww.get(b, lr, q);
        float s16[NB][GPC];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < GPC; ++j)
                s16[b][j] = scale16(sm.ts[(16 * b + lr) * G + min((GPC * c + j) >> SH, G - 1)]);
        if (full) {
            chunk_steps<GS, NB, 4, BITS>(acc, ra[abuf], wv, s16, kc);
        } else if constexpr (GS != 128) {
            chunk_steps<GS, NB, 2, BITS>(acc, ra[abuf], wv, s16, kc);
        }
        __builtin_amdgcn_wave_barrier();
    };
    // the loop runs full chunks only, U per trip (a multiple of the ring and
    // of the two activation buffers); the rest (at most U chunks, the last one
    // possibly a half chunk of 64 columns) follows
    constexpr int U = RING % 2 == 0 ? RING : 2 * RING;
    int c0 = 0;
    for (; c0 + U <= nfull; c0 += U) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            load_a(c0 + i + 1, (i + 1) & 1);
            compute(i % RING, i & 1, c0 + i, true, true);
        }
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
        if (c0 + i < nch) {
            load_a(c0 + i + 1, (i + 1) & 1);
            compute(i % RING, i & 1, c0 + i, c0 + i + RING < nch, c0 + i < nfull);
        }
    }

    // the bias term, added once after the groups
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] += bterm[b];

    // GeGLU, h once, and the 16-column block sum of h per row
    HOut<kF32H> ho;
    ho.init(a, A, row_begin, rows, true);
    auto epilogue = [&](auto silu_tag) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 4 * q + v;
            ho.put_sum(r, cb, ho.template put<decltype(silu_tag)::value>(r, hcol0 + lr, acc[0][v], acc[1][v]), lr);
        }
    };
    if (a.flags & MOE_F_SWIGLU)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

// down, tiles of <= 16 rows.  Grid: skinny tiles x H / (16 NB) column
// blocks; one wave per workgroup owns output columns 16 NB cb + [0, 16 NB),
// NB 16-row weight blocks.
template <bool kF32H, int NB, int RING, int GS, int BITS>
__global__ __launch_bounds__(64, kF32H || GS == 32 || BITS == 8 ? 2 : 3) void moe_down_skinny(FfnArgs a) {
    constexpr int P = kF32H ? 2 : 1, NS = Geo<GS>::kSteps, GPC = Geo<GS>::kChains, MPG = Geo<GS>::kSlices;
    constexpr int SH = Geo<GS>::kShift, OFF = kCodeOffset<BITS, kF32H>;
    constexpr bool kC64 = Geo<GS>::kChain == 64;
    __shared__ SkinnySmem<NB, Geo<GS>::kMaxG, BITS> sm;
    int cb;
    const int4 tile = load_skinny_tile(a, a.H / (16 * NB), cb);
    if (tile.x < 0) return;
    const int e = tile.x, row_begin = tile.y, rows = tile.z;
    const int lane = threadIdx.x & 63, q = lane >> 4, lr = lane & 15;
    const int H = a.H, I = a.I, G = I / GS;
    const size_t A = static_cast<size_t>(a.T) * a.k;
    const int cbase = cb * 16 * NB;
    const int nb = min(NB, (H - cbase) / 16);  // blocks inside H (H is a multiple of 64)

    size_t row0[NB];
    const uint32_t* blk[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        row0[b] = static_cast<size_t>(e) * H + cbase + 16 * min(b, nb - 1);
        blk[b] = a.w_d + row0[b] * (I / 32 * BITS);
    }
    Tables<NB, true, Geo<GS>::kMaxG / 32> tab;
    tab.load(a.s_d, a.b_d, row0, G);
    WaveW<NB, GS, BITS> ww;
    ww.init(sm.w, blk, I / 32 * BITS);
    u32x4 rv[RING][NB][BITS / 4];
#pragma unroll
    for (int i = 0; i < RING; ++i) ww.load(i, rv[i]);

    // padding lanes (row >= rows) read row 0: their outputs are never stored
    const int arow = row_begin + min(lr, rows - 1);
    // destination slot and routing weight of each row, read now and kept in
    // LDS for the epilogue
    if (lane < kBmSmall) {
        const int32_t d = a.perm[row_begin + min(lane, rows - 1)];
        sm.dst[lane] = d;
        sm.wt[lane] = a.topk_w[d];
    }
    const uint32_t* ha = reinterpret_cast<const uint32_t*>(a.h) + static_cast<size_t>(arow) * (I / 2);
    const size_t part = A * (I / 2);  // offset of the lo half, u32
    u32x4 ra[2][4][P];
    // slice s of chunk c, as in the gate|up kernel (64-column half 2 c + s / 2)
    const uint32_t* hq[P];
#pragma unroll
    for (int pp = 0; pp < P; ++pp) hq[pp] = ha + pp * part + (kC64 ? 8 : 4) * q;
    auto load_a = [&](int c, int buf) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint32_t goff = 32 * min(2 * c + hf, I / 64 - 1);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int pp = 0; pp < P; ++pp)
                    ra[buf][2 * hf + s][pp] =
                        *reinterpret_cast<const u32x4*>(hq[pp] + goff + (kC64 ? 4 : 16) * s);
        }
    };
    load_a(0, 0);
    // the bias term early, as in the gate|up kernel
    const int steps = (G + 31) / 32;
    RowSums<NS> hsum;
    hsum.template load_blocks<GS>(a.hs + static_cast<size_t>(arow) * (I / 16), G, q, steps);

    uint16_t* const ts = sm.ts;
    uint16_t* const tb = sm.tb;
    tab.store(ts, tb, G);
    __builtin_amdgcn_wave_barrier();
    f32x4 bterm[NB];
    {
        BiasOp<NS> X;
        hsum.pack(X, G, q, steps);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            BiasOp<NS> C;
            bias_from_table<NS, OFF>(C, ts + (16 * b + lr) * G, tb + (16 * b + lr) * G, G, q, steps,
                                                   true);
            bterm[b] = bias_mfma(X, C, steps);
        }
    }

    f32x4 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nfull = I / 128, nch = (I + 127) / 128;
    const CodeConsts<OFF> kc = code_consts<OFF>(a.zero);
    // chunk c: its weights go through LDS, the slot reloads with chunk c + RING
    // at once, then the MFMAs run (K may end in a half chunk of 64 columns)
    auto compute = [&](int slot, int abuf, int c, bool reload, bool full) {
        chunk_fence();
        ww.put(rv[slot]);
        if (reload) ww.load(c + RING, rv[slot]);
        __builtin_amdgcn_wave_barrier();
        WLane<BITS> wv[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) wv[b] = ww.get(b, lr, q);
        float s16[NB][GPC];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < GPC; ++j)
                s16[b][j] = scale16(ts[(16 * b + lr) * G + min((GPC * c + j) >> SH, G - 1)]);
        if constexpr (!kF32H) {
            u32x4 x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = ra[abuf][j][0];
            if (full) {
                chunk_steps<GS, NB, 4, BITS>(acc, x, wv, s16, kc);
            } else if constexpr (GS != 128) {
                chunk_steps<GS, NB, 2, BITS>(acc, x, wv, s16, kc);
            }
        } else {
            // groups in order, each with its hi and lo activation slices
#pragma unroll
            for (int j = 0; j < GPC; ++j) {
                if (j * MPG < 2 || full) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        u32x4 bw[MPG];
                        u32x4 xs2[MPG][P];
#pragma unroll
                        for (int m = 0; m < MPG; ++m) {
                            bw[m] = slice_operand<BITS, OFF>(wv[b], j * MPG + m, kc);
#pragma unroll
                            for (int pp = 0; pp < P; ++pp) xs2[m][pp] = ra[abuf][j * MPG + m][pp];
                        }
                        acc[b] = group_step<MPG, P>(acc[b], xs2, bw, s16[b][j]);
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    };
    // full chunks in the loop, U per trip, then the rest (as in gate|up)
    constexpr int U = RING % 2 == 0 ? RING : 2 * RING;
    int cc = 0;
    for (; cc + U <= nfull; cc += U) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            load_a(cc + i + 1, (i + 1) & 1);
            compute(i % RING, i & 1, cc + i, true, true);
        }
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
        if (cc + i < nch) {
            load_a(cc + i + 1, (i + 1) & 1);
            compute(i % RING, i & 1, cc + i, cc + i + RING < nch, cc + i < nfull);
        }
    }

    // the bias term, added once after the groups
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] += bterm[b];

    // weighted unsort (destinations and weights read before the K loop)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int r = 4 * q + v;
        if (r < rows) {
            float* yrow = a.y + static_cast<size_t>(sm.dst[r]) * H + cbase + lr;
            const float wt = sm.wt[r];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < nb) yrow[16 * b] = wt * acc[b][v];
        }
    }
}

// ============================================================= wide paths
// Tiles of at most 64 rows (32 with an fp32 h or 8-bit codes; 16 or more, as
// an expert of 33 rows gives 17 + 16 at 32); RB = 16-row blocks.  The activation tile (RB*16 rows) is staged in LDS in chunks of 128 columns
// (NBUF buffers); an LDS row is 16 pieces of 16 bytes plus 16 bytes of
// padding, so the 16 rows of a fragment read fall on distinct banks.  Each
// wave owns 4 blocks of 16 weight rows, moved through its own LDS buffer.
constexpr int kAStride = 2 * 32 + 4;  // u32 per staged activation row

// MAXG bounds the group count the scale tables hold: 48 keeps a workgroup's
// LDS under 80 KB, so that two workgroups share a CU.
template <int RB, int P, int NBUF, int MAXG, int BITS = 4>
struct alignas(16) WideSmem {
    uint32_t a[NBUF][P][RB * 16 * kAStride];  // after the K loop: group sums of the rows
    uint32_t w[4][64 * 4 * BITS];  // per-wave weight transposition buffer; after the K loop
                                // the wave's bias rows, one block at a time
    uint16_t ts[4][64 * MAXG];  // per-wave scales of its 64 weight rows
    int32_t dst[RB * 16];       // down: destination slot of each row
    float wt[RB * 16];          // down: its routing weight
};

// The down kernels' shared memory: the wide layout plus the group sums of
// the tile's rows, read in the prologue when a row has at most kPreG groups
// (704 columns at group size 32 or 64).  At 4 row blocks the bf16 layout then
// fills exactly half of a CU's LDS, so two workgroups still share a CU.
constexpr int kPreG = 22;
// Down rows of at most kLdsBiasG groups also read their bias rows in the
// prologue, into LDS beside the scales (the smaller tables leave room), so
// that the bias term after the K loop waits on no global load.
constexpr int kLdsBiasG = 16;
// per-wave biases of its 64 weight rows (64 N per wave), or nothing
template <int N>
struct DownBiasTable {
    uint16_t tb[4 * 64 * N];
    __device__ __forceinline__ uint16_t* wave_tb(int wave) { return tb + wave * 64 * N; }
};
template <>
struct DownBiasTable<0> {
    __device__ __forceinline__ uint16_t* wave_tb(int) { return nullptr; }
};
template <int RB, bool kF32H, int MAXG, int BITS>
struct alignas(16) DownSmem : WideSmem<RB, kF32H ? 2 : 1, kF32H ? 1 : 2, MAXG, BITS>,
                              DownBiasTable<MAXG <= kLdsBiasG ? MAXG : 0> {
    float xg[RB * 16 * kPreG];
};

// Bias rows of a wave's four weight blocks (16 rows x G bf16 each, contiguous),
// read raw as 16-byte pieces (lane l holds pieces l and l + 64 of each block)
// while the last chunk is multiplied, and turned into operand order through
// the wave's LDS buffer once the K loop is done.
template <int CB, int NP>
struct BiasRows {
    u32x4 v[CB][NP];  // NP pieces per lane cover G <= 32 NP

    // blk[cb]: the block's first bias (the same in every lane)
    __device__ __forceinline__ void load(const uint16_t* const (&blk)[CB], int G) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const Rsrc r = make_rsrc(blk[cb], 32u * G);  // pieces past the block read zeros
#pragma unroll
            for (int j = 0; j < NP; ++j) v[cb][j] = load16(r, 16u * (lane + 64 * j), 0);
        }
    }
    // block cb to buf as 16 rows of G (pieces past the block are not stored)
    __device__ __forceinline__ void store(uint16_t* buf, int cb, int G) const {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int j = 0; j < NP; ++j)
            if (lane + 64 * j < 2 * G) *reinterpret_cast<u32x4*>(buf + 8 * (lane + 64 * j)) = v[cb][j];
    }
};
// row stride (floats) of the group sums staged in a[] after the K loop: 16
// rows of a fragment read fall on distinct banks, and 8-group reads up to the
// last group the tables hold stay inside a row
template <int GS>
constexpr int kXStride = Geo<GS>::kMaxG + 4;
// One row-block count per kernel (a tile's unused row blocks are skipped at
// run time): a kernel that branches to several instantiations is allocated
// for all of them at once and overflows into accumulation registers.
constexpr int kWideRowBlocks = kBmBig / 16, kWideRowBlocksF32 = kBmBigF32 / 16;

// Thread t copies piece t % 16 of rows t / 16 + 16 i.  Rows past the tile
// read a real row and groups past G the last group: those values are never
// used, and the loads need no branch.
template <int RB, int P>
struct Stager {
    static constexpr int kPasses = RB;
    u32x4 v[kPasses][P];

    // chunk c of rows src[i]; nh = K / 64 halves of 64 columns (a half past K
    // reads the last one again, never used)
    __device__ __forceinline__ void load(const uint32_t* const (&src)[kPasses], size_t part, int c,
                                         int nh) {
        const int pc = threadIdx.x & 15;
        const int hf = min(2 * c + (pc >> 3), nh - 1);
        const int piece = 8 * hf + (pc & 7);
#pragma unroll
        for (int i = 0; i < kPasses; ++i)
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
                v[i][pp] = *reinterpret_cast<const u32x4*>(src[i] + pp * part + 4 * piece);
    }
    template <int NBUF, int MAXG, int BITS>
    __device__ __forceinline__ void store(WideSmem<RB, P, NBUF, MAXG, BITS>& sm, int buf) const {
        const int pc = threadIdx.x & 15, r0 = threadIdx.x >> 4;
#pragma unroll
        for (int i = 0; i < kPasses; ++i)
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
                *reinterpret_cast<u32x4*>(&sm.a[buf][pp][(r0 + 16 * i) * kAStride + 4 * pc]) = v[i][pp];
    }
};

template <int RB, int P, int NBUF, int MAXG, int BITS>
__device__ __forceinline__ u32x4 lds_frag(const WideSmem<RB, P, NBUF, MAXG, BITS>& sm, int buf, int pp, int row,
                                          int piece) {
    return *reinterpret_cast<const u32x4*>(&sm.a[buf][pp][row * kAStride + 4 * piece]);
}

// Shared K loop of the wide paths: acc[rb][cb] over all groups for the four
// 16-row weight blocks blk[cb] of this wave (row length K), activations staged
// from src (P parts, `part` apart); row blocks rb >= nrb are skipped.
template <int GS, int RB, int P, int NBUF, int MAXG, int BITS, int OFF, class Last>
__device__ __forceinline__ void wide_kloop(WideSmem<RB, P, NBUF, MAXG, BITS>& sm, Stager<RB, P>& st,
                                           const uint32_t* const (&src)[RB], size_t part,
                                           const uint32_t* const (&blk)[4], int K, bool active,
                                           int nrb, CodeConsts<OFF> kc, f32x4 (&acc)[RB][4], Last&& last) {
    constexpr int CB = 4, GPC = Geo<GS>::kChains, MPG = Geo<GS>::kSlices, SH = Geo<GS>::kShift;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, lr = lane & 15;
    const int G = K / GS, nh = K / 64;
    const int nch = (K + 127) / 128;
    WaveW<CB, GS, BITS> ww;
    ww.init(sm.w[wave], blk, K / 32 * BITS);
    // chunk c + 1's weights arrive in registers while chunk c is multiplied and
    // go to the wave's LDS buffer after it (chunk c's reads are done by then)
    u32x4 wn[CB][BITS / 4];
    ww.load(0, wn);
    ww.put(wn);
    __syncthreads();  // stage 0 and the scale tables are in place

    // chunk c; the last one (peeled, so that the next-chunk registers are free
    // for the epilogue's loads) issues no loads of its own
    auto chunk = [&](int c, auto last_tag) {
        constexpr bool kLast = decltype(last_tag)::value;
        const int buf = NBUF == 2 ? (c & 1) : 0;
        WLane<BITS> wq[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) wq[cb] = ww.get(cb, lr, q);
        // the next chunk's loads; during the last chunk, the epilogue's
        if constexpr (!kLast) {
            st.load(src, part, c + 1, nh);
            ww.load(c + 1, wn);
        } else {
            last();
        }
        if (active) {
#pragma unroll
            for (int j = 0; j < GPC; ++j) {
                const int ch = GPC * c + j;  // chain; its group is ch >> SH
                if (ch < K / Geo<GS>::kChain) {
                    const int g = ch >> SH;
                    u32x4 bw[CB][MPG];
                    float s16[CB];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                        for (int m = 0; m < MPG; ++m) bw[cb][m] = slice_operand<BITS, OFF>(wq[cb], j * MPG + m, kc);
                        s16[cb] = scale16(sm.ts[wave][(16 * cb + lr) * G + g]);
                    }
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        if (rb >= nrb) break;  // row blocks past the tile
                        const int row = 16 * rb + lr;
                        u32x4 xa[MPG][P];
#pragma unroll
                        for (int m = 0; m < MPG; ++m)
#pragma unroll
                            for (int pp = 0; pp < P; ++pp)
                                xa[m][pp] = lds_frag(sm, buf, pp, row, Geo<GS>::word(j * MPG + m, q));
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb)
                            acc[rb][cb] = group_step<MPG, P>(acc[rb][cb], xa, bw[cb], s16[cb]);
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        if constexpr (!kLast) ww.put(wn);
        if constexpr (NBUF == 2) {
            if constexpr (!kLast) st.store(sm, buf ^ 1);
            __syncthreads();
        } else {
            __syncthreads();
            if constexpr (!kLast) st.store(sm, 0);
            __syncthreads();
        }
    };
    for (int c = 0; c + 1 < nch; ++c) chunk(c, std::false_type{});
    chunk(nch - 1, std::true_type{});
}

// The group sums of the staged rows go to LDS for the bias term (the
// activation buffers are free once the K loop is done): thread t writes
// groups g = t % 16 + 16 j of rows t / 16 + 16 i, the value xsum(i, j, g)
// (G <= MAXG).
template <int GS, int RB, int P, int NBUF, int MAXG, int BITS, class XSum>
__device__ __forceinline__ void stage_group_sums(WideSmem<RB, P, NBUF, MAXG, BITS>& sm, int G, XSum&& xsum) {
    constexpr int XS = kXStride<GS>;
    static_assert(sizeof(float) * RB * 16 * XS <= sizeof(sm.a), "group sums must fit the activation buffer");
    float* xl = reinterpret_cast<float*>(&sm.a[0][0][0]);
    const int pc = threadIdx.x & 15, r0 = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < (MAXG + 15) / 16; ++j) {
            const int g = pc + 16 * j;
            if (g < G) xl[(r0 + 16 * i) * XS + g] = xsum(i, j, g);
        }
}

// The bias term of the wide paths, added once after the K loop, from the
// group sums stage_group_sums left in LDS.  rows(cb): the wave's bias rows of
// weight block cb in LDS (16 rows of G): from the tables, or staged from the
// registers that took them during the last chunk (wide_bias_rows).
template <int GS, int OFF, int RB, int P, int NBUF, int MAXG, int BITS, class Rows>
__device__ __forceinline__ void wide_bias(WideSmem<RB, P, NBUF, MAXG, BITS>& sm, Rows&& rows,
                                          int G, bool active, int nrb, f32x4 (&acc)[RB][4]) {
    constexpr int CB = 4, NS = Geo<GS>::kSteps, XS = kXStride<GS>;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, lr = lane & 15;
    const float* xl = reinterpret_cast<const float*>(&sm.a[0][0][0]);
    __syncthreads();
    const int steps = (G + 31) / 32;
    // the row operand of row block rb (8 consecutive groups per step; reads
    // past G stay inside the row stride and are replaced by 0)
    auto row_op = [&](int rb, BiasOp<NS>& X) {
        const float* xr = xl + (16 * rb + lr) * XS;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            if (st < steps) {
                const f32x4 v0 = *reinterpret_cast<const f32x4*>(xr + 32 * st + 8 * q);
                const f32x4 v1 = *reinterpret_cast<const f32x4*>(xr + 32 * st + 8 * q + 4);
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = j < 4 ? v0[j] : v1[j - 4];
                    v[j] = 32 * st + 8 * q + j < G ? x : 0.f;
                }
                pack_split(v, X.hi[st], X.lo[st]);
            }
        }
    };
    // up to two steps: the row operands once per row block; more (group size
    // 32): rebuilt per weight block, which keeps the registers low
    constexpr bool kKeepX = NS <= 2;
    BiasOp<NS> X[kKeepX ? RB : 1];
    if constexpr (kKeepX) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) row_op(rb, X[rb]);
    }
    const uint16_t* ts = sm.ts[wave];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        const uint16_t* const tb = rows(cb);
        BiasOp<NS> C;
        bias_from_table<NS, OFF>(C, ts + (16 * cb + lr) * G, tb + lr * G, G, q, steps, active);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (rb >= nrb) break;  // row blocks past the tile
            if constexpr (kKeepX) {
                acc[rb][cb] += bias_mfma(X[rb], C, steps);
            } else {
                row_op(rb, X[0]);
                acc[rb][cb] += bias_mfma(X[0], C, steps);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // one weight block at a time: registers stay low
    }
}

// Bias rows of block cb for wide_bias, from registers through the wave's
// weight buffer (free after the K loop).
template <int RB, int P, int NBUF, int MAXG, int BITS, int NP>
__device__ __forceinline__ auto wide_bias_rows(WideSmem<RB, P, NBUF, MAXG, BITS>& sm, const BiasRows<4, NP>& br,
                                               int G) {
    uint16_t* const wb = reinterpret_cast<uint16_t*>(sm.w[threadIdx.x >> 6]);
    return [&sm, &br, wb, G](int cb) -> const uint16_t* {
        (void)sm;
        __builtin_amdgcn_wave_barrier();  // the previous block's reads are done
        br.store(wb, cb, G);
        __builtin_amdgcn_wave_barrier();
        return wb;
    };
}

// gate|up wide, column block `by` of 128 h columns (ceil(I / 128) blocks).  Wave w owns h columns
// n0 + 32 w + [0, 32): weight blocks 0/1 = gate columns +0/+16, blocks 2/3 =
// the matching up columns.  Waves {0,1} cover h columns 128 by + [0, 64),
// waves {2,3} the next 64.
template <int GS, int RB, int MAXG, bool kF32H, int BITS>
__device__ __forceinline__ void gateup_wide(const FfnArgs& a, WideSmem<RB, 1, 2, MAXG, BITS>& sm, int e,
                                            int row_begin, int rows, int by) {
    constexpr int P = 1, NBUF = 2, CB = 4;
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, lr = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: weight rows are per wave
    const int H = a.H, I = a.I, G = H / GS;
    const size_t A = static_cast<size_t>(a.T) * a.k;
    const int n0 = by * 128;
    const bool active = n0 + 32 * wave < I;
    const int hbase = active ? n0 + 32 * wave : 0;

    size_t row0[CB];
    const uint32_t* blk[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        row0[cb] = static_cast<size_t>(e) * 2 * I + hbase + 16 * (cb & 1) + (cb >> 1) * I;
        blk[cb] = a.w_gu + row0[cb] * (H / 32 * BITS);
    }
    Tables<CB, false, (MAXG + 31) / 32> tab;
    tab.load(a.s_gu, a.b_gu, row0, G);

    int tok[RB];
    const uint32_t* src[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int r = (tid >> 4) + 16 * i;
        tok[i] = a.perm[row_begin + min(r, rows - 1)] / a.k;
        src[i] = reinterpret_cast<const uint32_t*>(a.xp) + static_cast<size_t>(tok[i]) * (H / 2);
    }
    Stager<RB, P> st;
    st.load(src, 0, 0, H / 64);
    tab.store(sm.ts[wave], nullptr, G);
    st.store(sm, 0);

    f32x4 acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* bblk[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) bblk[cb] = a.b_gu + row0[cb] * G;
    BiasRows<CB, Geo<GS>::kMaxG / 32> br;
    // the bias rows and the rows' group sums of x (thread t: groups t % 16 +
    // 16 j of rows t / 16 + 16 i) are read during the last chunk
    constexpr int XJ = (MAXG + 15) / 16;
    float xv[RB][XJ];
    auto last = [&] {
        br.load(bblk, G);
        const int pc = tid & 15;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const float* xrow = a.xs + static_cast<size_t>(tok[i]) * G;
#pragma unroll
            for (int j = 0; j < XJ; ++j) xv[i][j] = pc + 16 * j < G ? xrow[pc + 16 * j] : 0.f;
        }
    };
    wide_kloop<GS, RB, P, NBUF, MAXG, BITS>(sm, st, src, 0, blk, H, active, (rows + 15) / 16, code_consts<kCodeOffset<BITS, kF32H>>(a.zero), acc,
                                            last);

    stage_group_sums<GS>(sm, G, [&](int i, int j, int) { return xv[i][j]; });
    wide_bias<GS, kCodeOffset<BITS, kF32H>>(sm, wide_bias_rows(sm, br, G), G, active, (rows + 15) / 16, acc);

    // GeGLU epilogue and the 16-column block sums of h
    HOut<kF32H> ho;
    ho.init(a, A, row_begin, rows, active);
    auto epilogue = [&](auto silu_tag) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            if (rb >= (rows + 15) / 16) break;  // row blocks past the tile
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int hcol = hbase + 16 * half + lr;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = 16 * rb + 4 * q + v;
                    const float seen = ho.template put<decltype(silu_tag)::value>(r, hcol, acc[rb][half][v],
                                                                                  acc[rb][2 + half][v]);
                    ho.put_sum(r, hbase / 16 + half, seen, lr);
                }
            }
        }
    };
    if (a.flags & MOE_F_SWIGLU)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

// ================================================= wide gate|up, fp8 operands
// bf16 mode with 4-bit codes in 64-column chains (fp8_wide_gateup): the same
// product on the scaled 32x32x64 fp8 MFMA.  A code q as the e4m3 byte q reads
// exactly as q * 2^-9, so two masks of a code word give its eight codes as
// fp8 operands (even nibbles, then odd); the route left x as e4m3 hi + lo
// with one power-of-two scale per 32 columns (x 2^-e = hi + lo), which the
// MFMA applies per lane (its row and 32-column half), and the codes take the
// fixed scale 2^9 (the K order this needs: put_fp8).  Per chain of 64
// columns and 32x32 block:
//   P = x_hi . q + x_lo . q,   acc += s P
// and after the K loop the bias term sum_g b X_g (offset 0: q itself is the
// operand).  A wave owns 32 h columns: 32-row weight block 0 = the gate rows,
// block 1 = the matching up rows, so the GeGLU pairs stay in one lane; the
// 64 rows of a tile are two 32-row blocks.  Output element j of lane l (32x32
// layout): row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, 127 + 9);
}

// The lane's 32 codes (four words, see put_fp8) as an e4m3 operand: per
// word the even nibbles (columns 0, 2, 4, 6), then the odd ones.
__device__ __forceinline__ i32x8 codes_as_fp8(u32x4 w) {
    i32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[2 * i] = static_cast<int>(w[i] & 0x0F0F0F0Fu);
        r[2 * i + 1] = static_cast<int>((w[i] >> 4) & 0x0F0F0F0Fu);
    }
    return r;
}

// The wave's weight chunk in LDS.  The MFMA's K order: byte i of a lane in
// half kh (lane / 32) is K = 32 (i / 16) + 16 kh + i % 16, and the lane's
// A scale covers K block kh ([32 kh, 32 kh + 32)).  So for chain j (64
// columns, words 8 j .. 8 j + 7) the lane in half kh takes the words of
// columns 16 kh + [0, 16) and 32 + 16 kh + [0, 16): words 8 j + 2 kh, +1,
// 8 j + 4 + 2 kh, +1, kept together as slot 2 j + kh of the row (four
// 16-byte slots per row, slot s at s ^ ((r >> 1) & 3) so that the 32 rows an
// operand read touches fall on distinct banks).  A lane loaded words
// 4 pc .. 4 pc + 3 of its row: the pairs go to slots 2 (pc / 2) and
// 2 (pc / 2) + 1, at word 2 (pc % 2).
__device__ __forceinline__ void put_fp8(uint32_t* lds, const u32x4 (&v)[4][1]) {
    const int lane = threadIdx.x & 63, rr = lane >> 2, pc = lane & 3;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int r = 16 * cb + rr, sw = (r >> 1) & 3, s0 = 2 * (pc >> 1);
        uint32_t* const row = lds + 16 * r + 2 * (pc & 1);
        *reinterpret_cast<u32x2*>(row + 4 * (s0 ^ sw)) = u32x2{v[cb][0][0], v[cb][0][1]};
        *reinterpret_cast<u32x2*>(row + 4 * ((s0 + 1) ^ sw)) = u32x2{v[cb][0][2], v[cb][0][3]};
    }
}
__device__ __forceinline__ u32x4 get_fp8(const uint32_t* lds, int r, int p) {
    return *reinterpret_cast<const u32x4*>(lds + 16 * r + 4 * (p ^ ((r >> 1) & 3)));
}

// The wide gate|up LDS of the fp8 path: the bf16 layout plus the staged rows'
// block scales (one word per row: the chunk's four 32-column blocks), per
// activation buffer.
template <int MAXG>
struct alignas(16) GateupFp8Smem : WideSmem<4, 1, 2, MAXG, 4> {
    uint32_t sw8[2][64];
};

// Activation chunk c of the fp8 path: thread t copies piece t % 16 of rows
// t / 16 + 16 i -- pieces 0..7 the hi bytes of columns 128 c + 16 p .. + 15,
// pieces 8..15 the lo bytes -- into the same LDS rows as the bf16 staging
// (a half chunk past H reads the last half again, never used), and the
// rows' scale words.
template <int RB>
struct Stager8 {
    u32x4 v[RB];
    uint32_t w[RB];
    __device__ __forceinline__ void load(const uint8_t* const (&hi)[RB], const uint8_t* const (&lo)[RB],
                                         const uint32_t* const (&sc)[RB], int c, int nh) {
        const int pc = threadIdx.x & 15, q8 = pc & 7;
        const int col = 64 * min(2 * c + (q8 >> 2), nh - 1) + 16 * (q8 & 3);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            v[i] = *reinterpret_cast<const u32x4*>((pc < 8 ? hi[i] : lo[i]) + col);
            w[i] = sc[i][c];  // the row's 16 threads read the same word: no branch in the loop
        }
    }
    template <int MAXG>
    __device__ __forceinline__ void store(GateupFp8Smem<MAXG>& sm, int buf) const {
        const int pc = threadIdx.x & 15, r0 = threadIdx.x >> 4;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            *reinterpret_cast<u32x4*>(&sm.a[buf][0][(r0 + 16 * i) * kAStride + 4 * pc]) = v[i];
            sm.sw8[buf][r0 + 16 * i] = w[i];  // the same value from the row's 16 threads
        }
    }
};

// sum_g b[n, g] X[m, g] for the wave's four 32x32 blocks, accumulated onto
// acc by the MFMA: the bias rows of all four weight blocks go to the wave's
// scale table (free after the K loop: with offset 0 the bias term needs no
// scale), the group sums are in LDS (stage_group_sums); X enters as bf16
// hi + lo, b is bf16 already.  Entries past G are zero on the X side and
// replaced by zero on the b side (they read the next row or stale LDS).
template <int GS, int MAXG, int NP>
__device__ __forceinline__ void wide_bias_fp8(GateupFp8Smem<MAXG>& sm, const BiasRows<4, NP>& br, int G,
                                              int rows, f32x16 (&acc)[2][2]) {
    constexpr int NS = (Geo<GS>::kMaxG + 15) / 16, XS = kXStride<GS>;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, kh = lane >> 5;
    const float* xl = reinterpret_cast<const float*>(&sm.a[0][0][0]);
    uint16_t* const tb = sm.ts[wave];
    __builtin_amdgcn_wave_barrier();  // the wave's scale reads are done
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) br.store(tb + 16 * cb * G, cb, G);
    __syncthreads();  // the group sums and the bias rows are in place
    const int steps = (G + 15) / 16;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        if (st < steps) {
            const int g0 = 16 * st + 8 * kh;
            u32x4 b[2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const uint16_t* const br16 = tb + (32 * c2 + n) * G + g0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t lo = g0 + 2 * i < G ? br16[2 * i] : 0u;
                    const uint32_t hi = g0 + 2 * i + 1 < G ? br16[2 * i + 1] : 0u;
                    b[c2][i] = lo | (hi << 16);
                }
            }
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                if (32 * r2 < rows) {
                    const float* const xr = xl + (32 * r2 + n) * XS + g0;
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(xr);
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(xr + 4);
                    float v[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) v[k] = g0 + k < G ? (k < 4 ? x0[k] : x1[k - 4]) : 0.f;
                    u32x4 xh, xo;
                    pack_split(v, xh, xo);
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        acc[r2][c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xh), as_bf16x8(b[c2]),
                                                                              acc[r2][c2], 0, 0, 0);
                        acc[r2][c2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xo), as_bf16x8(b[c2]),
                                                                              acc[r2][c2], 0, 0, 0);
                    }
                }
            }
        }
    }
}

template <int GS, int MAXG>
__device__ __forceinline__ void gateup_wide_fp8(const FfnArgs& a, GateupFp8Smem<MAXG>& sm, int e, int row_begin,
                                                int rows, int by) {
    constexpr int RB = 4, CB = 4, SH = Geo<GS>::kShift;
    const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, kh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: weight rows are per wave
    const int H = a.H, I = a.I, G = H / GS, S8 = x8_stride(H);
    const size_t A = static_cast<size_t>(a.T) * a.k;
    const int n0 = by * 128;
    const bool active = n0 + 32 * wave < I;
    const int hbase = active ? n0 + 32 * wave : 0;

    // weight blocks: 0/1 the gate rows hbase + [0, 32), 2/3 the up rows
    size_t row0[CB];
    const uint32_t* blk[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        row0[cb] = static_cast<size_t>(e) * 2 * I + hbase + 16 * (cb & 1) + (cb >> 1) * I;
        blk[cb] = a.w_gu + row0[cb] * (H / 8);
    }
    Tables<CB, false, (MAXG + 31) / 32> tab;
    tab.load(a.s_gu, a.b_gu, row0, G);

    int tok[RB];
    const uint8_t* shi[RB];
    const uint8_t* slo[RB];
    const uint32_t* ssc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int r = (tid >> 4) + 16 * i;
        tok[i] = a.perm[row_begin + min(r, rows - 1)] / a.k;
        shi[i] = a.x8hi + static_cast<size_t>(tok[i]) * H;
        slo[i] = a.x8lo + static_cast<size_t>(tok[i]) * H;
        ssc[i] = reinterpret_cast<const uint32_t*>(a.x8s + static_cast<size_t>(tok[i]) * S8);
    }
    const int nh = H / 64, nch = (H + 127) / 128;
    Stager8<RB> st;
    st.load(shi, slo, ssc, 0, nh);
    tab.store(sm.ts[wave], nullptr, G);
    st.store(sm, 0);

    f32x16 acc[2][2];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) acc[r2][c2] = f32x16{};

    const uint16_t* bblk[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) bblk[cb] = a.b_gu + row0[cb] * G;
    BiasRows<CB, Geo<GS>::kMaxG / 32> br;
    constexpr int XJ = (MAXG + 15) / 16;
    float xv[RB][XJ];
    auto last = [&] {
        br.load(bblk, G);
        const int pc = tid & 15;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const float* xrow = a.xs + static_cast<size_t>(tok[i]) * G;
#pragma unroll
            for (int j = 0; j < XJ; ++j) xv[i][j] = pc + 16 * j < G ? xrow[pc + 16 * j] : 0.f;
        }
    };

    uint32_t* const wl = sm.w[wave];
    WaveW<CB, GS, 4> ww;
    ww.init(wl, blk, H / 8);
    u32x4 wn[CB][1];
    ww.load(0, wn);
    put_fp8(wl, wn);
    __syncthreads();  // chunk 0 and the scale tables are in place

    auto chunk = [&](int c, auto last_tag) {
        constexpr bool kLast = decltype(last_tag)::value;
        const int buf = c & 1;
        u32x4 wq[2][2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int j = 0; j < 2; ++j) wq[c2][j] = get_fp8(wl, 32 * c2 + n, 2 * j + kh);
        // the block scales of the lane's two rows (the chunk's four blocks)
        const uint32_t cur[2] = {sm.sw8[buf][n], sm.sw8[buf][32 + n]};
        if constexpr (!kLast) {
            st.load(shi, slo, ssc, c + 1, nh);
            ww.load(c + 1, wn);
        } else {
            last();
        }
        if (active) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ch = 2 * c + j;  // chain of 64 columns; its group is ch >> SH
                if (ch < nh) {
                    const int g = ch >> SH;
                    i32x8 b[2];
                    float s16[2];
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        b[c2] = codes_as_fp8(wq[c2][j]);
                        s16[c2] = scale16(sm.ts[wave][(32 * c2 + n) * G + g]);
                    }
                    // both 32-row halves, also in a tile of exactly 32 rows (its
                    // staged rows 32..63 repeat its last row and are never
                    // stored): with no branch between them the scheduler runs
                    // one half's scale FMAs beside the other half's MFMAs
#pragma unroll
                    for (int r2 = 0; r2 < 2; ++r2) {
                        {
                            // columns 16 kh + [0, 16) and 32 + 16 kh + [0, 16) of the chain
                            const int row = 32 * r2 + n, p0 = 4 * j + kh;
                            const u32x4 h0 = lds_frag(sm, buf, 0, row, p0), h1 = lds_frag(sm, buf, 0, row, p0 + 2);
                            const u32x4 l0 = lds_frag(sm, buf, 0, row, 8 + p0), l1 = lds_frag(sm, buf, 0, row, 10 + p0);
                            const i32x8 xh = {static_cast<int>(h0[0]), static_cast<int>(h0[1]), static_cast<int>(h0[2]),
                                              static_cast<int>(h0[3]), static_cast<int>(h1[0]), static_cast<int>(h1[1]),
                                              static_cast<int>(h1[2]), static_cast<int>(h1[3])};
                            const i32x8 xo = {static_cast<int>(l0[0]), static_cast<int>(l0[1]), static_cast<int>(l0[2]),
                                              static_cast<int>(l0[3]), static_cast<int>(l1[0]), static_cast<int>(l1[1]),
                                              static_cast<int>(l1[2]), static_cast<int>(l1[3])};
                            const int sa = static_cast<int>((cur[r2] >> (8 * (2 * j + kh))) & 0xFFu);
#pragma unroll
                            for (int c2 = 0; c2 < 2; ++c2) {
                                f32x16 pz = {};
                                pz = mfma_fp8(xh, b[c2], pz, sa);
                                pz = mfma_fp8(xo, b[c2], pz, sa);
#pragma unroll
                                for (int v = 0; v < 16; ++v) acc[r2][c2][v] = fmaf(s16[c2], pz[v], acc[r2][c2][v]);
                            }
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        if constexpr (!kLast) {
            put_fp8(wl, wn);
            st.store(sm, buf ^ 1);
        }
        __syncthreads();
    };
    for (int c = 0; c + 1 < nch; ++c) chunk(c, std::false_type{});
    chunk(nch - 1, std::true_type{});

    stage_group_sums<GS>(sm, G, [&](int i, int j, int) { return xv[i][j]; });
    wide_bias_fp8<GS>(sm, br, G, rows, acc);

    // GeGLU epilogue and the 16-column block sums of h
    HOut<false> ho;
    ho.init(a, A, row_begin, rows, active);
    auto epilogue = [&](auto silu_tag) {
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            if (32 * r2 >= rows) break;  // rows past the tile
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 32 * r2 + 8 * (v >> 2) + 4 * kh + (v & 3);
                const float seen = ho.template put<decltype(silu_tag)::value>(r, hbase + n, acc[r2][0][v],
                                                                              acc[r2][1][v]);
                ho.put_sum(r, hbase / 16 + (n >> 4), seen, lane & 15);
            }
        }
    };
    if (a.flags & MOE_F_SWIGLU)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

// down wide, column block `by` of 256 output columns (ceil(H / 256) blocks).  Wave w owns output columns
// n0 + 64 w + [0, 64): four 16-row weight blocks.
template <int GS, int RB, int MAXG, bool kF32H, int BITS>
__device__ __forceinline__ void down_wide(const FfnArgs& a, DownSmem<RB, kF32H, MAXG, BITS>& sm, int e,
                                          int row_begin, int rows, int by) {
    constexpr int P = kF32H ? 2 : 1, NBUF = kF32H ? 1 : 2, CB = 4;
    const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, lr = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: weight rows are per wave
    const int H = a.H, I = a.I, G = I / GS;
    const size_t A = static_cast<size_t>(a.T) * a.k;
    const int n0 = by * 256;
    const bool active = n0 + 64 * wave < H;  // H is a multiple of 64
    const int cbase = active ? n0 + 64 * wave : 0;

    size_t row0[CB];
    const uint32_t* blk[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        row0[cb] = static_cast<size_t>(e) * H + cbase + 16 * cb;
        blk[cb] = a.w_d + row0[cb] * (I / 32 * BITS);
    }
    constexpr bool kLdsBias = MAXG <= kLdsBiasG;
    Tables<CB, kLdsBias, (MAXG + 31) / 32> tab;
    tab.load(a.s_d, a.b_d, row0, G);

    int hrow[RB];
    const uint32_t* src[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int r = (tid >> 4) + 16 * i;
        hrow[i] = row_begin + min(r, rows - 1);
        src[i] = reinterpret_cast<const uint32_t*>(a.h) + static_cast<size_t>(hrow[i]) * (I / 2);
    }
    // destination slot and routing weight of each row, kept in LDS for the
    // epilogue (the K loop's first barrier publishes them)
    if (tid < RB * 16) {
        const int32_t d = a.perm[row_begin + min(tid, rows - 1)];
        sm.dst[tid] = d;
        sm.wt[tid] = a.topk_w[d];
    }
    const size_t part = A * (I / 2);
    Stager<RB, P> st;
    st.load(src, part, 0, I / 64);
    // rows of at most kPreG groups: their group sums (from the block sums of
    // h, in the one order) are read now, with the first stage, and kept in
    // LDS for the bias term, which then waits on no global load
    const bool pre = G <= kPreG;
    constexpr int PN = (RB * 16 * kPreG + kThreads - 1) / kThreads;
    BlockSums<GS> pb[PN];
    if (pre) {
#pragma unroll
        for (int n = 0; n < PN; ++n) {
            const int idx = tid + kThreads * n;
            if (idx < RB * 16 * G) {
                const int r = idx / G;
                pb[n].load(a.hs + static_cast<size_t>(row_begin + min(r, rows - 1)) * (I / 16), idx - r * G);
            }
        }
    }
    uint16_t* const tbw = sm.wave_tb(wave);
    tab.store(sm.ts[wave], kLdsBias ? tbw : nullptr, G);
    st.store(sm, 0);
    if (pre) {
#pragma unroll
        for (int n = 0; n < PN; ++n) {
            const int idx = tid + kThreads * n;
            if (idx < RB * 16 * G) sm.xg[idx] = pb[n].sum();
        }
    }

    f32x4 acc[RB][CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* bblk[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) bblk[cb] = a.b_d + row0[cb] * G;
    BiasRows<CB, Geo<GS>::kMaxG / 32> br;
    wide_kloop<GS, RB, P, NBUF, MAXG, BITS>(sm, st, src, part, blk, I, active, (rows + 15) / 16, code_consts<kCodeOffset<BITS, kF32H>>(a.zero), acc,
                                  [&] {
                                      if constexpr (!kLdsBias) br.load(bblk, G);
                                  });

    if (pre)
        stage_group_sums<GS>(sm, G, [&](int i, int, int g) { return sm.xg[((tid >> 4) + 16 * i) * G + g]; });
    else
        stage_group_sums<GS>(sm, G, [&](int i, int, int g) {
            return group_of_blocks<GS>(a.hs + static_cast<size_t>(hrow[i]) * (I / 16), g);
        });
    if constexpr (kLdsBias)
        wide_bias<GS, kCodeOffset<BITS, kF32H>>(sm, [&](int cb) -> const uint16_t* { return tbw + 16 * cb * G; }, G, active,
                      (rows + 15) / 16, acc);
    else
        wide_bias<GS, kCodeOffset<BITS, kF32H>>(sm, wide_bias_rows(sm, br, G), G, active, (rows + 15) / 16, acc);

    if (!active) return;
    // weighted unsort (destinations and weights read before the K loop)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * rb + 4 * q + v;
            if (r < rows) {
                const int32_t dst = sm.dst[r];
                const float wt = sm.wt[r];
                float* yrow = a.y + static_cast<size_t>(dst) * H + cbase + lr;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) yrow[16 * cb] = wt * acc[rb][cb][v];
            }
        }
    }
}

// XCD-aware order of the wide work.  Workgroups go to the 8 XCDs round-robin
// by linear id, and each XCD has its own L2: XCD x takes the contiguous run
// [x * share, (x + 1) * share) of the (tile, column block) items, column block
// fastest, so that a tile's column blocks (one activation tile) and an
// expert's consecutive tiles (one set of weights) meet in the same L2.  The
// share comes from the device-side tile count; the grid holds a multiple of 8
// workgroups, at least as many as items.
constexpr int kXcds = 8;

__device__ __forceinline__ bool wide_work(const FfnArgs& a, int ncol, int& tile, int& col) {
    const int total = min(a.num_tiles[2], a.max_tiles) * ncol;
    const int share = (total + kXcds - 1) / kXcds;
    const int L = blockIdx.x, i = L / kXcds;
    if (i >= share) return false;
    const int item = (L % kXcds) * share + i;
    if (item >= total) return false;
    tile = item / ncol;
    col = item - tile * ncol;
    return true;
}

// Two workgroups share a CU when their LDS fits in half of it.
template <class Smem>
constexpr int kWideWgsPerCu = sizeof(Smem) <= 80 * 1024 ? 2 : 1;
// Row blocks per wave: 4 (64-row tiles), or 2 (32-row tiles) with an fp32 h
// or 8-bit codes, whose extra operand registers would not fit beside four.
template <bool kF32H, int BITS>
constexpr int kWideRB = kF32H || BITS == 8 ? kWideRowBlocksF32 : kWideRowBlocks;
template <bool kF32H, int MAXG, int BITS>
using GateupWideSmem = WideSmem<kWideRB<kF32H, BITS>, 1, 2, MAXG, BITS>;
template <bool kF32H, int MAXG, int BITS>
using DownWideSmem = DownSmem<kWideRB<kF32H, BITS>, kF32H, MAXG, BITS>;
// The wide gate|up takes fp8 operands in bf16 mode with 4-bit codes in
// 64-column chains (the host prepares x for it under the same condition).
template <bool kF32H, int GS, int BITS>
constexpr bool kFp8Gateup = !kF32H && BITS == 4 && Geo<GS>::kChain == 64;
// Tiles of at least kFp8MinRows rows take the fp8 operands.  An expert of
// more than kBmBig rows is cut into tiles of at least (kBmBig + 1) / 2 rows,
// so all tiles of one expert take the same path and a row's bits do not
// depend on its place among its expert's rows.
constexpr int kFp8MinRows = 32;
static_assert((kBmBig + 1) / 2 >= kFp8MinRows, "an expert's tiles must share one operand path");
template <bool kF32H, int MAXG, int GS, int BITS>
using GateupSmem = std::conditional_t<kFp8Gateup<kF32H, GS, BITS>, GateupFp8Smem<MAXG>,
                                      GateupWideSmem<kF32H, MAXG, BITS>>;

template <bool kF32H, int MAXG, int GS, int BITS>
__global__ __launch_bounds__(kThreads, (kWideWgsPerCu<GateupSmem<kF32H, MAXG, GS, BITS>>)) void moe_gateup_wide(
    FfnArgs a) {
    int ti, by;
    if (!wide_work(a, (a.I + 127) / 128, ti, by)) return;
    const int4 tile = reinterpret_cast<const int4*>(a.tiles)[ti];
    if constexpr (kFp8Gateup<kF32H, GS, BITS>) {
        // tiles of fewer than 32 rows (one 32-row block) on the exact bf16
        // operand, which is faster there
        __shared__ GateupFp8Smem<MAXG> sm;
        if (tile.z >= kFp8MinRows)
            gateup_wide_fp8<GS, MAXG>(a, sm, tile.x, tile.y, tile.z, by);
        else
            gateup_wide<GS, kWideRowBlocks, MAXG, false, BITS>(a, sm, tile.x, tile.y, tile.z, by);
    } else {
        __shared__ GateupWideSmem<kF32H, MAXG, BITS> sm;
        gateup_wide<GS, kWideRB<kF32H, BITS>, MAXG, kF32H, BITS>(a, sm, tile.x, tile.y, tile.z, by);
    }
}

template <bool kF32H, int MAXG, int GS, int BITS>
__global__ __launch_bounds__(kThreads, (kWideWgsPerCu<DownWideSmem<kF32H, MAXG, BITS>>)) void moe_down_wide(
    FfnArgs a) {
    __shared__ DownWideSmem<kF32H, MAXG, BITS> sm;
    int ti, by;
    if (!wide_work(a, (a.H + 255) / 256, ti, by)) return;
    const int4 tile = reinterpret_cast<const int4*>(a.tiles)[ti];
    down_wide<GS, kWideRB<kF32H, BITS>, MAXG, kF32H, BITS>(a, sm, tile.x, tile.y, tile.z, by);
}

}  // namespace

// Grid widths, from bounds that hold for every routing.  A skinny tile is a
// whole expert of <= 16 rows (at most one per expert), or with skinny_only a
// piece of <= 16 rows of one (ceil(c / 16) <= floor(c / 16) + 1 pieces for an
// expert of c rows).  The wide list holds ceil(c / bm_big) tiles per expert of
// more than 16 rows, at most floor(A / bm_big) + min(E, A) = max_tiles in all
// (a sum of floors never exceeds the floor of the sum).  The height of a wide
// tile is no bound: with bm_big = 32 an expert of 33 rows gives tiles of 17
// and 16 rows.
static int skinny_grid(const FfnArgs& a) {
    const int A = a.T * a.k;
    return min(a.max_skinny, min(a.E, A) + (a.skinny_only ? A / kBmSmall : 0));
}
static int wide_grid(const FfnArgs& a) { return a.skinny_only ? 0 : a.max_tiles; }

// No tile can be wide: nothing to launch, but the timing events still mark
// the (empty) interval.
static hipError_t skip_launch(hipStream_t stream, const KTiming& t) {
    if (t.start != nullptr && t.stop != nullptr) {
        hipError_t e = hipEventRecord(t.start, stream);
        if (e == hipSuccess) e = hipEventRecord(t.stop, stream);
        return e;
    }
    return hipSuccess;
}

// The kernels take the group size and the code width as template
// parameters; a.gs and a.bits pick them.
template <int GS, int BITS>
static hipError_t gateup_skinny_gs(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    constexpr int RING = kSkinnyGateUpRing;
    const dim3 grid(skinny_grid(a) * (a.I / 16));
    if (a.flags & MOE_F_FP32_INTERMEDIATE)
        return launch_kernel(moe_gateup_skinny<true, RING, GS, BITS>, grid, dim3(64), stream, t, a);
    return launch_kernel(moe_gateup_skinny<false, RING, GS, BITS>, grid, dim3(64), stream, t, a);
}

// MAXG: groups per row the scale tables hold.  Rows of at most 3/4 of the
// largest group count take the smaller tables (two workgroups per CU at group
// size 64).
template <int GS, int BITS>
static hipError_t gateup_wide_gs(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    const int n = wide_grid(a);
    if (n == 0) return skip_launch(stream, t);
    const int items = n * ((a.I + 127) / 128);
    const dim3 grid((items + kXcds - 1) / kXcds * kXcds);
    constexpr int kBig = Geo<GS>::kMaxG, kSmall = 3 * kBig / 4;
    const bool f32 = a.flags & MOE_F_FP32_INTERMEDIATE, small = a.H / GS <= kSmall;
    if (f32)
        return small ? launch_kernel(moe_gateup_wide<true, kSmall, GS, BITS>, grid, dim3(kThreads), stream, t, a)
                     : launch_kernel(moe_gateup_wide<true, kBig, GS, BITS>, grid, dim3(kThreads), stream, t, a);
    return small ? launch_kernel(moe_gateup_wide<false, kSmall, GS, BITS>, grid, dim3(kThreads), stream, t, a)
                 : launch_kernel(moe_gateup_wide<false, kBig, GS, BITS>, grid, dim3(kThreads), stream, t, a);
}

template <int GS, int BITS>
static hipError_t down_skinny_gs(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    constexpr int NB = kSkinnyDownBlocks, RING = kSkinnyDownRing;
    static_assert(64 % (16 * NB) == 0, "H (a multiple of 64) must split into whole column blocks");
    const dim3 grid(skinny_grid(a) * (a.H / (16 * NB)));
    if (a.flags & MOE_F_FP32_INTERMEDIATE)
        return launch_kernel(moe_down_skinny<true, NB, RING, GS, BITS>, grid, dim3(64), stream, t, a);
    return launch_kernel(moe_down_skinny<false, NB, RING, GS, BITS>, grid, dim3(64), stream, t, a);
}

template <int GS, int BITS>
static hipError_t down_wide_gs(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    const int n = wide_grid(a);
    if (n == 0) return skip_launch(stream, t);
    const int items = n * ((a.H + 255) / 256);
    const dim3 grid((items + kXcds - 1) / kXcds * kXcds);
    constexpr int kBig = Geo<GS>::kMaxG, kSmall = 3 * kBig / 4, kTiny = kLdsBiasG;
    static_assert(kTiny < kSmall || GS == 128, "table sizes");
    const bool f32 = a.flags & MOE_F_FP32_INTERMEDIATE;
    const int G = a.I / GS;
    if (G <= kTiny)
        return f32 ? launch_kernel(moe_down_wide<true, kTiny, GS, BITS>, grid, dim3(kThreads), stream, t, a)
                   : launch_kernel(moe_down_wide<false, kTiny, GS, BITS>, grid, dim3(kThreads), stream, t, a);
    const bool small = G <= kSmall;
    if (f32)
        return small ? launch_kernel(moe_down_wide<true, kSmall, GS, BITS>, grid, dim3(kThreads), stream, t, a)
                     : launch_kernel(moe_down_wide<true, kBig, GS, BITS>, grid, dim3(kThreads), stream, t, a);
    return small ? launch_kernel(moe_down_wide<false, kSmall, GS, BITS>, grid, dim3(kThreads), stream, t, a)
                 : launch_kernel(moe_down_wide<false, kBig, GS, BITS>, grid, dim3(kThreads), stream, t, a);
}

// One entry per kernel of the pair (GS, BITS), defined by its translation unit.
#define MOE_GEMM_INSTANCE(GS, BITS)                                                                   \
    hipError_t launch_gemm_g##GS##_b##BITS(GemmOp op, const FfnArgs& a, hipStream_t stream,           \
                                           const KTiming& t) {                                        \
        switch (op) {                                                                                 \
            case GemmOp::kGateupSkinny: return gateup_skinny_gs<GS, BITS>(a, stream, t);              \
            case GemmOp::kGateupWide: return gateup_wide_gs<GS, BITS>(a, stream, t);                  \
            case GemmOp::kDownSkinny: return down_skinny_gs<GS, BITS>(a, stream, t);                  \
            case GemmOp::kDownWide: return down_wide_gs<GS, BITS>(a, stream, t);                      \
        }                                                                                             \
        return hipErrorInvalidValue;                                                                  \
    }

}  // namespace moe
