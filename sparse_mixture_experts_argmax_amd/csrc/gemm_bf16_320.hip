// Instantiates the grouped-GEMM kernel for the 320-row shapes (experts of 257 to 320 rows).
#include "gemm_kernel.h"

namespace moe {

hipError_t gemm_bf16_320(const GemmArgs &g, bool wide) {
    return wide ? launch_bf16_act<TileW320>(g) : launch_bf16_act<TileN320>(g);
}

}  // namespace moe
