// Internal declarations shared by the libmoeffn translation units.
#pragma once

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

constexpr int kGroup = 64;      // quantisation group (columns per scale/bias)
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// Tile heights used by the forward's own routing.  32-row tiles run on
// 32x32x16 MFMAs; tiles of at most 16 rows run on 16x16x32 MFMAs.
constexpr int kBmBig = 32;
constexpr int kBmSmall = 16;

// ---------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------ dequant
// The eight 4-bit codes of one weight word as eight bf16 values 128 + q,
// which bf16 holds exactly (exponent 7, mantissa q).  Element order in the
// MFMA operand is [q0, q4, q1, q5, q2, q6, q3, q7]; the activation operand is
// stored in the same order (permute8 below), so the products still pair each
// code with its own column.  The +128 offset is removed in fp32 per group:
//   sum_k x_k (s q_k + b) = s * sum_k x_k (128 + q_k) + (b - 128 s) * sum_k x_k.
__device__ __forceinline__ u32x4 codes_as_bf16(uint32_t w) {
    u32x4 r;
    r[0] = (w & 0x000F000Fu) | 0x43004300u;
    r[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    r[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    r[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return r;
}
constexpr float kCodeOffset = 128.0f;

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
// z = sqrt(2/pi) (v + 0.044715 v^3).
__device__ __forceinline__ float gelu_tanh(float v) {
    const float z = 0.7978845608028654f * (v + 0.044715f * v * v * v);
    return v / (1.0f + expf(-2.0f * z));
}

// ---------------------------------------------------- kernel launchers
struct RouteArgs {
    const int32_t* ids;
    int32_t A, E, bm_big, bm_small, max_tiles;
    int32_t *counts, *offsets, *perm, *inv_perm, *tiles, *num_tiles;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

struct FfnArgs {
    int32_t T, k, E, H, I, max_tiles;
    uint32_t flags;
    const uint16_t* x;
    const int32_t* ids;
    const float* topk_w;
    const uint32_t* w_gu;
    const uint16_t* s_gu;
    const uint16_t* b_gu;
    const uint32_t* w_d;
    const uint16_t* s_d;
    const uint16_t* b_d;
    const int32_t* perm;
    const int32_t* tiles;
    const int32_t* num_tiles;
    void* h;
    float* y;
    void* out;
};
hipError_t launch_gateup(const FfnArgs& a, hipStream_t stream);
hipError_t launch_down(const FfnArgs& a, hipStream_t stream);
hipError_t launch_combine(const FfnArgs& a, hipStream_t stream);

}  // namespace moe
