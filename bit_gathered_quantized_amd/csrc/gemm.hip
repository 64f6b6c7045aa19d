// Dispatch of the quantised matmul launches to the translation unit of the
// problem's group size and code width (gemm_g*_b*.hip).
#include "moe_internal.h"

namespace moe {

namespace {
hipError_t dispatch(GemmOp op, const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    const bool b8 = a.bits == 8;
    switch (a.gs) {
        case 32: return b8 ? launch_gemm_g32_b8(op, a, stream, t) : launch_gemm_g32_b4(op, a, stream, t);
        case 128: return b8 ? launch_gemm_g128_b8(op, a, stream, t) : launch_gemm_g128_b4(op, a, stream, t);
        default: return b8 ? launch_gemm_g64_b8(op, a, stream, t) : launch_gemm_g64_b4(op, a, stream, t);
    }
}
}  // namespace

hipError_t launch_gateup_skinny(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    return dispatch(GemmOp::kGateupSkinny, a, stream, t);
}
hipError_t launch_down_skinny(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    return dispatch(GemmOp::kDownSkinny, a, stream, t);
}
hipError_t launch_gateup_wide(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    return dispatch(GemmOp::kGateupWide, a, stream, t);
}
hipError_t launch_down_wide(const FfnArgs& a, hipStream_t stream, const KTiming& t) {
    return dispatch(GemmOp::kDownWide, a, stream, t);
}

}  // namespace moe
