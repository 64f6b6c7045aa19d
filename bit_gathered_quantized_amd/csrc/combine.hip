// Combine: out[t, m] = sum over j = 0..k-1 (ascending) of y[t*k + j, m].
//
// y already carries the routing weights (applied by the down kernel), so this
// is the weighted expert sum of SwiftLM issue #236 ("Already on main":
// weightedExpertSum).  Each thread sums four adjacent columns in fp32 in a
// fixed slot order, so the result does not depend on which tile produced
// which row.  Slots whose expert id is out of range were never written and
// are skipped.  HBM-bound: reads A*H*4 bytes, writes T*H*2 (or 4).
#include "moe_internal.h"

namespace moe {
namespace {

template <bool kF32Out>
__global__ __launch_bounds__(256) void moe_combine(FfnArgs a) {
    const int H4 = a.H / 4;
    const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t total = static_cast<size_t>(a.T) * H4;
    if (idx >= total) return;
    const int t = static_cast<int>(idx / H4);
    const int c4 = static_cast<int>(idx - static_cast<size_t>(t) * H4);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    // eight slots at a time: all their loads are issued before the first add
    // (rows of out-of-range slots are read but not added)
    for (int j0 = 0; j0 < a.k; j0 += 8) {
        float4 v[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            const size_t asg = static_cast<size_t>(t) * a.k + min(j, a.k - 1);
            const int32_t id = a.ids[asg];
            ok[u] = j < a.k && id >= 0 && id < a.E;
            v[u] = reinterpret_cast<const float4*>(a.y + asg * a.H)[c4];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (ok[u]) {
                s.x += v[u].x;
                s.y += v[u].y;
                s.z += v[u].z;
                s.w += v[u].w;
            }
        }
    }
    if constexpr (kF32Out) {
        reinterpret_cast<float4*>(static_cast<float*>(a.out) + static_cast<size_t>(t) * a.H)[c4] = s;
    } else {
        reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + static_cast<size_t>(t) * a.H)[c4] =
            u32x2{pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)};
    }
}

}  // namespace

hipError_t launch_combine(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    const size_t total = static_cast<size_t>(a.T) * (a.H / 4);
    const dim3 grid(static_cast<unsigned>((total + 255) / 256));
    if (a.flags & MOE_F_FP32_OUT)
        return launch_kernel(moe_combine<true>, grid, dim3(256), stream, t, a);
    else
        return launch_kernel(moe_combine<false>, grid, dim3(256), stream, t, a);
}

}  // namespace moe
