// Internal declarations shared by the libmoeffn translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ffn.h"

namespace moe {

// ------------------------------------------------------------------ types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// Tile heights used by the forward's own routing: an expert of at most 16
// rows is one skinny tile; a larger one is cut into ceil(rows / 64) wide
// tiles of near-equal height (17..64 rows each; with 32, 16..32: an expert of
// 33 rows gives 17 + 16), so no expert leaves a short tail that reads its
// weights once more.  64 rows = 4 row blocks per wave
// keeps the wide kernels within 256 vector registers (32 rows with fp32
// intermediates).
constexpr int kBmBig = 64;
constexpr int kBmBigF32 = 32;  // with MOE_F_FP32_INTERMEDIATE or 8-bit codes
constexpr int kBmSmall = 16;
// The fp8 operand path of the wide gate|up kernel: bf16 mode, 4-bit codes in
// groups of 64 or 128 columns, batches that can have wide tiles.  The code q
// as an e4m3 byte reads exactly as q * 2^-9 (subnormal below 8, and the
// normal binade from 8 on continues the same step), and x splits exactly into
// e4m3 hi + lo under a power-of-two scale per 32 columns.
inline bool fp8_wide_gateup(int64_t T, int gs, int bits, uint32_t flags) {
    return T > kBmSmall && bits == 4 && (gs == 64 || gs == 128) && !(flags & MOE_F_FP32_INTERMEDIATE);
}
// Bytes per row of the block scales: H / 32, rounded up to 4 (a chunk of 128
// columns reads its four scales as one word; a final half chunk reads two
// padding bytes, unused).
__host__ __device__ inline int x8_stride(int H) { return (H / 32 + 3) / 4 * 4; }
// Largest H and I the kernels take (the scale and bias tables in LDS and the
// bias contraction are sized for it).
constexpr int kMaxDim = 4096;

// ---------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even: the conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// a and b rounded to nearest-even bf16 and packed, a in the low half: one
// conversion instruction for the pair.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// ------------------------------------------------------------ dequant
// The eight 4-bit codes of one weight word as eight bf16 values OFF + q,
// exactly: with OFF = 16, q goes into the top four of the seven mantissa
// bits of 16.0; with OFF = 128, into the bottom four of 128.0, which needs no
// shift for the first pair (7 instructions per word instead of 8).  Element
// order in the MFMA operand is [q0, q4, q1, q5, q2, q6, q3, q7]; the
// activation operand is stored in the same order (permute8 below), so each
// code still meets its own column.  With P = sum_k x_k (OFF + q_k) and
// X = sum_k x_k over a group,
//   sum_k x_k (s q_k + b) = s P + (b - OFF s) X.
// A small offset keeps P close in size to the part that carries information,
// so little is lost when X is taken out: the fp32 intermediate mode uses 16;
// the bf16 mode, whose h is rounded to 8 bits anyway, uses 128.
//
// The two constants sit in registers (CodeConsts, built from a zero the
// compiler cannot see through): folded into literals, each AND-OR below would
// take two VALU instructions, because gfx9 VOP3 forms such as v_and_or_b32
// take no literal operand.
template <int OFF>
struct CodeConsts {
    uint32_t mask, one;
};
// The mask goes to a vector register (a per-lane select on a condition the
// compiler cannot fold) and the other constant stays scalar: one VOP3
// instruction may read only one scalar operand.  (OFF = 0, 8-bit codes: not
// used.)
template <int OFF>
__device__ __forceinline__ CodeConsts<OFF> code_consts(uint32_t zero) {
    static_assert(OFF == 0 || OFF == 16 || OFF == 128, "code offset");
    const uint32_t mask = (threadIdx.x & zero) ? 0u : (OFF == 128 ? 0x000F000Fu : 0x00780078u);
    return CodeConsts<OFF>{mask, (OFF == 128 ? 0x43004300u : 0x41804180u) | zero};
}
template <int OFF>
__device__ __forceinline__ u32x4 codes_as_bf16(uint32_t w, CodeConsts<OFF> k) {
    u32x4 r;
    if constexpr (OFF == 128) {
        r[0] = (w & k.mask) | k.one;          // q0, q4
        r[1] = ((w >> 4) & k.mask) | k.one;   // q1, q5
        r[2] = ((w >> 8) & k.mask) | k.one;   // q2, q6
        r[3] = ((w >> 12) & k.mask) | k.one;  // q3, q7
    } else {
        r[0] = ((w << 3) & k.mask) | k.one;  // q0, q4
        r[1] = ((w >> 1) & k.mask) | k.one;  // q1, q5
        r[2] = ((w >> 5) & k.mask) | k.one;  // q2, q6
        r[3] = ((w >> 9) & k.mask) | k.one;  // q3, q7
    }
    return r;
}
// 8-bit codes: the bf16 mantissa cannot take q under a fixed exponent, so
// each byte is converted (exactly: q <= 255 has 8 significant bits) and the
// operand is q itself, offset 0.  w0 holds columns 0..3 of the 8-column piece,
// w1 columns 4..7; element pairs come out in the permute8 order [q0, q4, q1,
// q5, q2, q6, q3, q7], as for the 4-bit codes.
__device__ __forceinline__ u32x4 bytes_as_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = pack_bf16x2(static_cast<float>((w0 >> (8 * i)) & 0xFFu), static_cast<float>((w1 >> (8 * i)) & 0xFFu));
    return r;
}
// The code offset of the exact operand: 16 + q (fp32 intermediate mode) or
// 128 + q (bf16 mode) for 4-bit codes, q for 8-bit.
template <int BITS, bool kF32H>
constexpr int kCodeOffset = BITS == 4 ? (kF32H ? 16 : 128) : 0;

// Position of column c (0..7) of an 8-column piece after permute8.
__device__ __forceinline__ int permuted_pos(int c) { return ((c & 3) << 1) | (c >> 2); }

// Reorder eight consecutive bf16 values [v0..v7] to [v0,v4,v1,v5,v2,v6,v3,v7].
__device__ __forceinline__ u32x4 permute8(u32x4 v) {
    u32x4 r;
    r[0] = (v[0] & 0xFFFFu) | (v[2] << 16);
    r[1] = (v[0] >> 16) | (v[2] & 0xFFFF0000u);
    r[2] = (v[1] & 0xFFFFu) | (v[3] << 16);
    r[3] = (v[1] >> 16) | (v[3] & 0xFFFF0000u);
    return r;
}

// Sum of the eight bf16 values packed in v, in index order, fp32.
__device__ __forceinline__ float sum8_bf16(u32x4 v) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s += __uint_as_float(v[i] << 16);
        s += __uint_as_float(v[i] & 0xFFFF0000u);
    }
    return s;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// tanh-approximate GELU in fp32: 0.5 v (1 + tanh(z)) = v / (1 + exp(-2 z)),
// z = sqrt(2/pi) (v + 0.044715 v^3).  exp(-2 z) is 2^(-2 z log2 e) on the
// hardware base-2 exponential and the quotient is v times the hardware
// reciprocal: each within a few ulp, far below the rounding of h that follows
// (bf16, or 16 bits as hi + lo).  Large |v| give v or -0 (the exponential
// saturates to 0 or +inf, whose reciprocal is 0).
__device__ __forceinline__ float gelu_tanh(float v) {
    const float z = 0.7978845608028654f * (v + 0.044715f * v * v * v);
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.8853900817779268f * z));
}

// SiLU in fp32: v * sigmoid(v) = v / (1 + exp(-v)), evaluated the same way.
__device__ __forceinline__ float silu(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * v));
}

// ---------------------------------------------------- kernel launchers
// Optional start/stop events of one kernel.  With events the kernel is
// launched through hipExtLaunchKernelGGL, which records them with the dispatch
// itself, so the interval is the kernel alone.
struct KTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

template <typename... Args, typename F = void (*)(Args...)>
inline hipError_t launch_kernel_lds(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                    const KTiming& t, Args... args) {
    if (t.start != nullptr && t.stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, t.start, t.stop, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
    return hipGetLastError();
}
template <typename... Args, typename F = void (*)(Args...)>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t stream,
                                const KTiming& t, Args... args) {
    return launch_kernel_lds(kernel, grid, block, 0, stream, t, args...);
}

struct RouteArgs {
    const int32_t* ids;
    int32_t A, E, bm_big, bm_small, max_tiles;
    int32_t *counts, *offsets, *perm, *inv_perm, *tiles, *num_tiles;
    // nullptr: one tile list in expert order, num_tiles [2].  Otherwise experts
    // of more than skinny_max_rows rows go to tiles (balanced, bm_big at
    // most), the others to tiles_skinny in tiles of bm_small (at most
    // max_skinny entries), each list in expert order; num_tiles [4] =
    // {total, invalid ids, wide, skinny}.
    int32_t* tiles_skinny;
    int32_t skinny_max_rows, max_skinny;
    // A caller's slot -> assignment order, sorted by expert (or nullptr).
    // Checked on the device: num_tiles[4] = 0 if used, 1 if not sorted or out
    // of range, 2 if not a permutation; in both failure cases the kernel sorts
    // by itself.
    const int32_t* presorted;
    // count_wgs > 0: the sort (or the check of a caller's order) spreads over
    // that many workgroups of kRouteSegment assignments, counts in hist
    // [count_wgs][E + 1], then one order status per segment (forward only);
    // 0: one workgroup sorts
    int32_t count_wgs;
    int32_t* hist;
    // activation preparation (forward only; x == nullptr skips it)
    const uint16_t* x;  // [T, H] bf16
    int32_t T, H;
    int32_t gs;         // quantisation group size: 32, 64 or 128
    uint16_t* xp;       // [T, H] bf16, pieces reordered by permute8
    float* xs;          // [T, H/gs] group sums
    // x as e4m3 hi + lo under a power-of-two scale per 32 columns (nullptr:
    // not written; see x8_stride)
    uint8_t* x8hi;      // [T, H] e4m3, each 8-column piece in the order 0,2,4,6,1,3,5,7
    uint8_t* x8lo;      // [T, H] e4m3, the remainder x * 2^-e - hi, same order
    uint8_t* x8s;       // [T, x8_stride(H)] e8m0 block scales (127 + e)
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream, const KTiming& t = {});
constexpr int kRouteSegment = kRouteThreads;  // assignments per counting workgroup
constexpr int64_t kRouteMultiMin = 2048;      // larger A sorts over several workgroups
int route_count_wgs(int64_t A);
size_t route_lds_bytes(int E);

struct FfnArgs {
    int32_t T, k, E, H, I, max_tiles;
    int32_t gs;           // quantisation group size: 32, 64 or 128
    int32_t bits;         // code width: 4 or 8 (8: skinny kernels only)
    int32_t max_skinny;   // capacity of tiles_skinny
    int32_t skinny_only;  // 1: every tile is skinny, the wide launches are skipped
    uint32_t flags;
    uint32_t zero;       // always 0 (see CodeConsts)
    const uint16_t* x;
    const uint16_t* xp;  // [T, H] x with pieces reordered by permute8
    const float* xs;     // [T, H/gs] group sums of x
    const uint8_t* x8hi;  // x split into e4m3 hi + lo with block scales (RouteArgs)
    const uint8_t* x8lo;
    const uint8_t* x8s;
    float* hs;           // [A, I/16] sums of h over 16-column blocks (as the down matmul sees it)
    const int32_t* ids;
    const float* topk_w;
    const uint32_t* w_gu;
    const uint16_t* s_gu;
    const uint16_t* b_gu;
    const uint32_t* w_d;
    const uint16_t* s_d;
    const uint16_t* b_d;
    const int32_t* perm;
    const int32_t* tiles;         // tiles of more than kBmSmall rows
    const int32_t* tiles_skinny;  // tiles of at most kBmSmall rows
    const int32_t* num_tiles;     // {total, invalid ids, wide, skinny}
    void* h;             // [A, I] bf16, or hi and lo [2, A, I] bf16; pieces permuted
    float* y;
    void* out;
};
// The four quantised matmul launches; each (group size, code width) pair is
// instantiated in a translation unit of its own.
enum class GemmOp { kGateupSkinny, kGateupWide, kDownSkinny, kDownWide };
hipError_t launch_gemm_g32_b4(GemmOp op, const FfnArgs& a, hipStream_t stream, const KTiming& t);
hipError_t launch_gemm_g32_b8(GemmOp op, const FfnArgs& a, hipStream_t stream, const KTiming& t);
hipError_t launch_gemm_g64_b4(GemmOp op, const FfnArgs& a, hipStream_t stream, const KTiming& t);
hipError_t launch_gemm_g64_b8(GemmOp op, const FfnArgs& a, hipStream_t stream, const KTiming& t);
hipError_t launch_gemm_g128_b4(GemmOp op, const FfnArgs& a, hipStream_t stream, const KTiming& t);
hipError_t launch_gemm_g128_b8(GemmOp op, const FfnArgs& a, hipStream_t stream, const KTiming& t);
hipError_t launch_gateup_skinny(const FfnArgs& a, hipStream_t stream, const KTiming& t = {});
hipError_t launch_gateup_wide(const FfnArgs& a, hipStream_t stream, const KTiming& t = {});
hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t stream, const KTiming& t = {});
hipError_t launch_down_wide(const FfnArgs& a, hipStream_t stream, const KTiming& t = {});
hipError_t launch_combine(const FfnArgs& a, hipStream_t stream, const KTiming& t = {});
hipError_t launch_router_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids,
                              float* weights, hipStream_t stream);
constexpr int kRouterMaxK = 64;

}  // namespace moe
