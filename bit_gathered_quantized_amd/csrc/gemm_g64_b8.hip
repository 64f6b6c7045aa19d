// The quantised matmul kernels for groups of 64 columns and 8-bit codes.
#include "gemm_kernels.h"

namespace moe {
MOE_GEMM_INSTANCE(64, 8)
}  // namespace moe
