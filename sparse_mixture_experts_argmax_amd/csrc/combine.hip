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

constexpr int CMB_MAXK = 8;

// One wave per token.  The token's choices (row offset of its expert row,
// or -1, and gate) are read once into registers, then each lane walks its
// 16-byte pieces of d U at a time, so the row loads of all U pieces and of
// every choice are in flight together instead of each waiting on the index
// loads of its own iteration.  KC >= k bounds the choices (register arrays).
template <bool BF16, int KC, int U>
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
        // the kept choices of token t, in rank order
        int64_t roff[KC];
        float g[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            roff[j] = -1;
            g[j] = 0.f;
            if (j < k) {
                const int64_t a = t * k + j;
                const int s = slot[a];
                const int e = expert_idx[a];
                const bool kept = !(s < 0 || s >= C || e < 0 || e >= E);
                roff[j] = kept ? ((int64_t)e * C + s) * row_bytes : -1;
                g[j] = gate[a];
            }
        }
        auto accum = [&](float (&acc)[EPP], const u32x4 &v, float gj) {
            if (BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[2 * q] = fmaf(gj, bf2f((uint16_t)(v[q] & 0xFFFFu)), acc[2 * q]);
                    acc[2 * q + 1] = fmaf(gj, bf2f((uint16_t)(v[q] >> 16)), acc[2 * q + 1]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = fmaf(gj, __uint_as_float(v[q]), acc[q]);
            }
        };
        auto out = [&](const float (&acc)[EPP], int p) {
            u32x4 o;
            if (BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
            }
            st16(y + t * row_bytes + p * 16, o);
        };
        int p = lane;
        for (; p + (U - 1) * 64 < pieces; p += U * 64) {
            float a[U][EPP];
            u32x4 v[U][KC];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < EPP; ++q) a[u][q] = 0.f;
#pragma unroll
            for (int j = 0; j < KC; ++j)
                if (roff[j] >= 0) {
#pragma unroll
                    for (int u = 0; u < U; ++u) v[u][j] = ld16(ybuf + roff[j] + (p + 64 * u) * 16);
                }
#pragma unroll
            for (int j = 0; j < KC; ++j)
                if (roff[j] >= 0) {
#pragma unroll
                    for (int u = 0; u < U; ++u) accum(a[u], v[u][j], g[j]);
                }
#pragma unroll
            for (int u = 0; u < U; ++u) out(a[u], p + 64 * u);
        }
        for (; p < pieces; p += 64) {
            float a0[EPP];
#pragma unroll
            for (int q = 0; q < EPP; ++q) a0[q] = 0.f;
#pragma unroll
            for (int j = 0; j < KC; ++j)
                if (roff[j] >= 0) accum(a0, ld16(ybuf + roff[j] + p * 16), g[j]);
            out(a0, p);
        }
    }
}

// pieces in flight per lane: about 8 row loads (U pieces of KC choices)
template <bool BF16, int KC>
void launch_combine_k(dim3 grid, hipStream_t s, const uint8_t *yb, const int32_t *expert_idx, const int32_t *slot,
                      const float *gate, int64_t T, int d, int E, int k, int64_t C, uint8_t *yo,
                      const float *prob_sum, const int32_t *route_count, float alpha, float *aux_loss) {
    constexpr int U = KC >= 8 ? 1 : 8 / KC;
    hipLaunchKernelGGL((combine_kernel<BF16, KC, U>), grid, dim3(256), 0, s, yb, expert_idx, slot, gate, T, d, E,
                       k, C, yo, prob_sum, route_count, alpha, aux_loss);
}
template <bool BF16>
void launch_combine_t(dim3 grid, hipStream_t s, const uint8_t *yb, const int32_t *expert_idx, const int32_t *slot,
                      const float *gate, int64_t T, int d, int E, int k, int64_t C, uint8_t *yo,
                      const float *prob_sum, const int32_t *route_count, float alpha, float *aux_loss) {
    if (k <= 1)
        launch_combine_k<BF16, 1>(grid, s, yb, expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum, route_count,
                                  alpha, aux_loss);
    else if (k <= 2)
        launch_combine_k<BF16, 2>(grid, s, yb, expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum, route_count,
                                  alpha, aux_loss);
    else if (k <= 4)
        launch_combine_k<BF16, 4>(grid, s, yb, expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum, route_count,
                                  alpha, aux_loss);
    else
        launch_combine_k<BF16, CMB_MAXK>(grid, s, yb, expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum,
                                         route_count, alpha, aux_loss);
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
    const dim3 grid((unsigned)blocks);
    if (k > CMB_MAXK) return hipErrorInvalidValue;
    if (dtype_bf16)
        launch_combine_t<true>(grid, s, yb, expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum, route_count, alpha,
                               aux_loss);
    else
        launch_combine_t<false>(grid, s, yb, expert_idx, slot, gate, T, d, E, k, C, yo, prob_sum, route_count, alpha,
                                aux_loss);
    return hipGetLastError();
}

}  // namespace moe
