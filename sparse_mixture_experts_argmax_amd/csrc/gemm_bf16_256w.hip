// Instantiates the grouped-GEMM kernel for the 256 x 256 shape.
#include "gemm_kernel.h"

namespace moe {

hipError_t gemm_bf16_256w(const GemmArgs &g) { return launch_bf16_act<TileW256>(g); }

}  // namespace moe
