// Combine and auxiliary load-balancing loss.
//
// y_t = sum over kept choices j (rank order) of gate[t,j] * ybuf[e_tj, slot_tj],
// fp32 sum, one rounding to the storage dtype ([CS25-L5] "Switch Layer":
// gate times expert output; [CMU-L16] section 2.3: y = G_0 E_0 + G_1 E_1).
// Dropped choices contribute nothing; the token rides the residual path,
// which the caller adds ([CS25-L5] "Capacity Factor"; [CMU-L16] 6.1).
//
// L_aux = alpha * N * sum_i f_i P_i, f_i = route_count_i / (k T),
// P_i = prob_sum_i / T ([SW-GLaM] "负载均衡"), fp64 on the device, by
// the first wave of block 0 in a fixed order.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(
    const uint8_t *__restrict__ ybuf, const int32_t *__restrict__ expert_idx,
    const int32_t *__restrict__ slot, const float *__restrict__ gate, int64_t T, int d, int E,
    int k, int64_t C, uint8_t *__restrict__ y, const float *__restrict__ prob_sum,
    const int32_t *__restrict__ route_count, float alpha, float *__restrict__ aux) {
    constexpr int EPP = BF16 ? 8 : 4;           // elements per 16-byte piece
    constexpr int ES = BF16 ? 2 : 4;            // element bytes
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    if (blockIdx.x == 0 && wave == 0) {
        const float a = aux_loss_wave<false>(route_count, prob_sum, E, T, k, alpha, lane);
        if (lane == 0) aux[0] = a;
    }

    const int pieces = d / EPP;
    const int64_t row_bytes = (int64_t)d * ES;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < T; t += nwaves) {
        for (int p = lane; p < pieces; p += 64) {
            float acc[EPP];
#pragma unroll
            for (int q = 0; q < EPP; ++q) acc[q] = 0.f;
            for (int j = 0; j < k; ++j) {
                const int64_t a = t * k + j;
                const int s = slot[a];
                const int e = expert_idx[a];
                if (s < 0 || s >= C || e < 0 || e >= E) continue;
                const float g = gate[a];
                const u32x4 v = ld16(ybuf + ((int64_t)e * C + s) * row_bytes + p * 16);
                if (BF16) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] = fmaf(g, bf2f((uint16_t)(v[q] & 0xFFFFu)), acc[2 * q]);
                        acc[2 * q + 1] = fmaf(g, bf2f((uint16_t)(v[q] >> 16)), acc[2 * q + 1]);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q] = fmaf(g, __uint_as_float(v[q]), acc[q]);
                }
            }
            u32x4 o;
            if (BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
            }
            st16(y + t * row_bytes + p * 16, o);
        }
    }
}

}  // namespace

hipError_t launch_combine(const void *ybuf, int dtype_bf16, const int32_t *expert_idx,
                          const int32_t *slot, const float *gate, const float *prob_sum,
                          const int32_t *route_count, int64_t T, int d, int E, int k, int64_t C,
                          float alpha, void *y, float *aux_loss, hipStream_t s) {
    int64_t blocks = (T + 3) / 4;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    const uint8_t *yb = reinterpret_cast<const uint8_t *>(ybuf);
    uint8_t *yo = reinterpret_cast<uint8_t *>(y);
    if (dtype_bf16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, yb,
                           expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum, route_count,
                           alpha, aux_loss);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, yb,
                           expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum, route_count,
                           alpha, aux_loss);
    return hipGetLastError();
}

}  // namespace moe
