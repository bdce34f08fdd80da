// Instantiates the grouped-GEMM kernel for the 128 x 256 shape.
#include "gemm_kernel.h"

namespace moe {

hipError_t gemm_bf16_128w(const GemmArgs &g) { return launch_bf16_act<TileW128>(g); }

}  // namespace moe
