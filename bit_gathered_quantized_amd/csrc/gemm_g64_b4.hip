// The quantised matmul kernels for groups of 64 columns and 4-bit codes.
#include "gemm_kernels.h"

namespace moe {
MOE_GEMM_INSTANCE(64, 4)
}  // namespace moe
