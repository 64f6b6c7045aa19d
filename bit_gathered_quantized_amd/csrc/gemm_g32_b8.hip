// The quantised matmul kernels for groups of 32 columns and 8-bit codes.
#include "gemm_kernels.h"

namespace moe {
MOE_GEMM_INSTANCE(32, 8)
}  // namespace moe
