// Instantiates the grouped-GEMM kernel for the 256 x 128 shape.
#include "gemm_kernel.h"

namespace moe {

hipError_t gemm_bf16_256n(const GemmArgs &g) { return launch_bf16_act<TileN256>(g); }

}  // namespace moe
