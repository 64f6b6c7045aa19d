// The quantised matmul kernels for groups of 128 columns and 8-bit codes.
#include "gemm_kernels.h"

namespace moe {
MOE_GEMM_INSTANCE(128, 8)
}  // namespace moe
