// Instantiates the grouped-GEMM kernel for the 128 x 128 shape.
#include "gemm_kernel.h"

namespace moe {

hipError_t gemm_bf16_128n(const GemmArgs &g) { return launch_bf16_act<TileN128>(g); }

}  // namespace moe
