// The quantised matmul kernels for groups of 128 columns and 4-bit codes.
#include "gemm_kernels.h"

namespace moe {
MOE_GEMM_INSTANCE(128, 4)
}  // namespace moe
