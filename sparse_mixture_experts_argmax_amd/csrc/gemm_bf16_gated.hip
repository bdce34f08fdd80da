// Instantiates the grouped-GEMM kernel for the gated SwiGLU shapes (128 and 256 rows).
#include "gemm_kernel.h"

namespace moe {

hipError_t gemm_bf16_gated(const GemmArgs &g, int bm) {
    return bm == 256 ? launch_bf16_tile<TileG256, 2, false>(g) : launch_bf16_tile<TileG128, 2, false>(g);
}

}  // namespace moe
