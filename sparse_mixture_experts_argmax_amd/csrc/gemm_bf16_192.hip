// Instantiates the grouped-GEMM kernel for the 192-row shapes (experts of 129 to 192 rows).
#include "gemm_kernel.h"

namespace moe {

hipError_t gemm_bf16_192(const GemmArgs &g, bool wide) {
    return wide ? launch_bf16_act<TileW192>(g) : launch_bf16_act<TileN192>(g);
}

}  // namespace moe
