// Device router: softmax top-k with renormalised weights, the step that feeds
// the route/sort kernel.  The pages do not define the router; this is the
// usual top-k softmax gate (the fused top-k candidate selection of the
// mlx-node PR #168 page is its nearest relative there).
//
// One wave per token.  Lane l holds logits l, l + 64, ... (E <= 1024: 16 per
// lane).  Each of the k rounds takes the wave-wide largest remaining logit,
// the lower expert id on ties, so ids come out in order of descending logit.
// Weights: w_j = exp(l_j - m) / sum over the k chosen of exp(l_i - m), with m
// the largest logit -- the softmax over all E experts renormalised over the
// chosen k (the full denominator cancels).  The sum runs in a fixed order, so
// results are deterministic.  NaN logits rank as -inf.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterPerLane = MOE_MAX_EXPERTS / 64;
constexpr int kRouterTokensPerBlock = 4;

__global__ __launch_bounds__(64 * kRouterTokensPerBlock) void moe_router_topk_kernel(
    const float* __restrict__ logits, int32_t T, int32_t E, int32_t k, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kRouterTokensPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave; no barrier follows
    const float* row = logits + static_cast<size_t>(t) * E;
    float v[kRouterPerLane];
#pragma unroll
    for (int i = 0; i < kRouterPerLane; ++i) {
        const int e = lane + 64 * i;
        const float x = e < E ? row[e] : -INFINITY;
        v[i] = x != x ? -INFINITY : x;
    }
    uint32_t taken = 0;  // bit i: logit lane + 64 i already chosen
    float my_v = -INFINITY;
    int32_t my_id = 0;
    float top = 0.f;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int32_t bi = INT32_MAX;
#pragma unroll
        for (int i = 0; i < kRouterPerLane; ++i) {
            const int e = lane + 64 * i;
            const bool cand = e < E && !((taken >> i) & 1u);
            if (cand && (v[i] > bv || (v[i] == bv && e < bi))) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int32_t oi = __shfl_xor(bi, off);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        if (j == 0) top = bv;
        if (lane == j) {
            my_v = bv;
            my_id = bi;
        }
    }
    // weights: lanes 0..k-1 hold the chosen logits in order
    const float ex = lane < k ? expf(my_v - top) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) sum += __shfl_xor(sum, off);
    sum = __shfl(sum, 0);  // one rounding of the sum for every lane
    if (lane < k) {
        ids[static_cast<size_t>(t) * k + lane] = my_id;
        weights[static_cast<size_t>(t) * k + lane] = ex / sum;
    }
}

}  // namespace

hipError_t launch_router_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids,
                              float* weights, hipStream_t stream) {
    const dim3 grid((T + kRouterTokensPerBlock - 1) / kRouterTokensPerBlock);
    hipLaunchKernelGGL(moe_router_topk_kernel, grid, dim3(64 * kRouterTokensPerBlock), 0, stream,
                       logits, T, E, k, ids, weights);
    return hipGetLastError();
}

}  // namespace moe
