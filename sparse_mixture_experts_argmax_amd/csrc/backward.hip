// Backward of the gate side of the layer: combine and router.
//
// Combine ([CS25-L5] "Switch Layer", y_t = sum over kept j of g_tj E_tj(x_t)):
// the output is linear in the gate and in the expert output, so
// dL/dg_tj = <dy_t, E_tj(x_t)> and dL/dE_tj = g_tj dy_t for kept choices,
// zero for dropped ones.
//
// Router: the loss reaches the logits z through the gates (the full-softmax
// probability of the choice for k = 1, the softmax over the kept logits for
// k >= 2), through the balance loss alpha N sum_i f_i P_i with f held
// constant ([CMU-L16] exercise 2: its gradient with respect to p_i(x_t) is
// alpha N f_i / T) and through the weighted z-loss (the gradient of
// (w / T) lse_t^2 is (2 w / T) lse_t p_t).  The top-k choice itself carries
// no gradient.  Then dW_r = dz^T x, db_r = sum_t dz_t and the router's part
// of dx is dz W_r, all accumulated in fp32 in a fixed order.
#include "common.h"
#include "launch.h"

#include <math.h>

namespace moe {

namespace {

template <bool BF16>
__device__ __forceinline__ void load8(const void *p, int64_t i, float (&v)[8]) {
    if (BF16) {
        const u32x4 q = ld16(reinterpret_cast<const uint16_t *>(p) + i);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[2 * h] = __uint_as_float(q[h] << 16);
            v[2 * h + 1] = __uint_as_float(q[h] & 0xFFFF0000u);
        }
    } else {
        const u32x4 a = ld16(reinterpret_cast<const float *>(p) + i);
        const u32x4 b = ld16(reinterpret_cast<const float *>(p) + i + 4);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            v[h] = __uint_as_float(a[h]);
            v[4 + h] = __uint_as_float(b[h]);
        }
    }
}

template <bool BF16>
__device__ __forceinline__ void store8(void *p, int64_t i, const float (&v)[8]) {
    if (BF16) {
        u32x4 q;
#pragma unroll
        for (int h = 0; h < 4; ++h) q[h] = (uint32_t)f2bf(v[2 * h]) | ((uint32_t)f2bf(v[2 * h + 1]) << 16);
        st16(reinterpret_cast<uint16_t *>(p) + i, q);
    } else {
        u32x4 a, b;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            a[h] = __float_as_uint(v[h]);
            b[h] = __float_as_uint(v[4 + h]);
        }
        st16(reinterpret_cast<float *>(p) + i, a);
        st16(reinterpret_cast<float *>(p) + i + 4, b);
    }
}

// One wave per (token, rank) choice; lanes take 8-element pieces of the row.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const void *__restrict__ dy, const void *__restrict__ ybuf, const int32_t *__restrict__ expert_idx,
    const int32_t *__restrict__ slot, const float *__restrict__ gate, int64_t T, int d, int E, int k,
    int64_t C, float *__restrict__ dgate, void *__restrict__ dybuf) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t a = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); a < T * k; a += nwaves) {
        const int e = expert_idx[a];
        const int s = slot[a];
        if (s < 0 || e < 0 || e >= E) {
            if (lane == 0) dgate[a] = 0.f;
            continue;
        }
        const int64_t t = a / k;
        const float g = gate[a];
        const int64_t yrow = ((int64_t)e * C + s) * d;
        float acc = 0.f;
        for (int c = lane * 8; c < d; c += 512) {
            float vd[8], vy[8], vo[8];
            load8<BF16>(dy, t * d + c, vd);
            load8<BF16>(ybuf, yrow + c, vy);
#pragma unroll
            for (int h = 0; h < 8; ++h) {
                acc = fmaf(vd[h], vy[h], acc);
                vo[h] = g * vd[h];
            }
            store8<BF16>(dybuf, yrow + c, vo);
        }
        for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        if (lane == 0) dgate[a] = acc;
    }
}

// dz for one token per wave: the gate path, the balance loss and the z-loss
// through the softmax Jacobian.  Lanes take experts n = lane, lane + 64, ...
__global__ __launch_bounds__(256) void router_bwd_dz_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ expert_idx, const float *__restrict__ gate,
    const float *__restrict__ dgate, const int32_t *__restrict__ route_count, int64_t T, int E, int k,
    float alpha, float zw, float *__restrict__ dz) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *z = logits + t * E;
    // balance-loss weights a_n = alpha N f_n / T with f_n = count_n / (k T)
    const float aw = (float)((double)alpha * E / ((double)k * (double)T * (double)T));
    float mx = -INFINITY;
    for (int n = lane; n < E; n += 64) mx = fmaxf(mx, z[n]);
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    float s = 0.f, pa = 0.f;
    for (int n = lane; n < E; n += 64) {
        const float ex = expf(z[n] - mx);
        s += ex;
        pa = fmaf(ex, aw * (float)route_count[n], pa);
    }
    for (int m = 32; m >= 1; m >>= 1) {
        s += __shfl_xor(s, m);
        pa += __shfl_xor(pa, m);
    }
    const float inv = 1.f / s;
    pa *= inv;                                       // sum_n p_n a_n
    const float lse = mx + logf(s);
    const float zc = 2.f * zw / (float)T * lse;
    // the gate path: k = 1, c1 (onehot - p) with c1 = dg p_e; k >= 2,
    // g_j (dg_j - sum_i g_i dg_i) on the kept experts
    const int32_t *ix = expert_idx + t * k;
    const float *gt = gate + t * k;
    const float *dg = dgate + t * k;
    float c1 = 0.f, sg = 0.f;
    if (k == 1) {
        const int e0 = ix[0];
        c1 = (e0 >= 0 && e0 < E) ? dg[0] * (expf(z[e0] - mx) * inv) : 0.f;
    } else {
        for (int j = 0; j < k; ++j) sg = fmaf(gt[j], dg[j], sg);
    }
    for (int n = lane; n < E; n += 64) {
        const float p = expf(z[n] - mx) * inv;
        float v = p * (aw * (float)route_count[n] - pa) + zc * p;
        if (k == 1) {
            v += c1 * ((n == ix[0] ? 1.f : 0.f) - p);
        } else {
            for (int j = 0; j < k; ++j)
                if (ix[j] == n) v += gt[j] * (dg[j] - sg);
        }
        dz[t * E + n] = v;
    }
}

// dx[t, :] = sum_n dz[t, n] W_r[n, :] (n in order), register-tiled: a
// block covers 64 tokens x 128 columns and steps over the experts 32 at a
// time through LDS; each thread owns 4 tokens x 8 columns, so an expert
// costs it 16 bytes of dz and 32 bytes of W_r from LDS for 32 FMAs.
constexpr int DX_TT = 64, DX_NC = 128, DX_KS = 32;
__global__ __launch_bounds__(256) void router_bwd_dx_kernel(const float *__restrict__ dz,
                                                            const float *__restrict__ Wr, int64_t T, int d,
                                                            int E, float *__restrict__ dx) {
    __shared__ __attribute__((aligned(16))) float s_a[DX_KS][DX_TT];     // dz, transposed
    __shared__ __attribute__((aligned(16))) float s_b[DX_KS][DX_NC];     // W_r rows
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int c0 = blockIdx.y * DX_NC;
    const int64_t t0 = (int64_t)blockIdx.x * DX_TT;
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    for (int n0 = 0; n0 < E; n0 += DX_KS) {
        for (int i = tid; i < DX_TT * DX_KS; i += 256) {
            const int r = i / DX_KS, q = i - r * DX_KS;
            const int64_t t = t0 + r;
            s_a[q][r] = (t < T && n0 + q < E) ? dz[t * E + n0 + q] : 0.f;
        }
        for (int i = tid; i < DX_KS * (DX_NC / 4); i += 256) {
            const int q = i / (DX_NC / 4), pc = i - q * (DX_NC / 4);
            const int c = c0 + pc * 4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (n0 + q < E && c < d) v = *reinterpret_cast<const float4 *>(Wr + (int64_t)(n0 + q) * d + c);
            *reinterpret_cast<float4 *>(&s_b[q][pc * 4]) = v;
        }
        __syncthreads();
#pragma unroll 4
        for (int q = 0; q < DX_KS; ++q) {
            const float4 av = *reinterpret_cast<const float4 *>(&s_a[q][ty * 4]);
            const float4 ba = *reinterpret_cast<const float4 *>(&s_b[q][tx * 8]);
            const float4 bb = *reinterpret_cast<const float4 *>(&s_b[q][tx * 8 + 4]);
            const float as[4] = {av.x, av.y, av.z, av.w};
            const float bs[8] = {ba.x, ba.y, ba.z, ba.w, bb.x, bb.y, bb.z, bb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(as[i], bs[j], acc[i][j]);
        }
        __syncthreads();
    }
    const int cc = c0 + tx * 8;
    if (cc < d)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = t0 + ty * 4 + i;
            if (t < T) {
                float4 *o = reinterpret_cast<float4 *>(dx + t * d + cc);
                o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
            }
        }
}

// Tokens per chunk (one partial row each): 512, halved down to 128 while the
// grid has fewer than 1024 blocks.  Few experts and a narrow d leave few
// blocks otherwise (Mixtral-shaped: 128 at 512 tokens), and each block
// stages its tokens in turn; at 128 the gate-side backward ran 291 -> 201 us
// there and 176 -> 137 us on switch_base.  With 256 experts the grid is
// large already and smaller chunks only grow the partial sums (+12 %).
int dw_expert_group(int E) { return E <= 16 ? 16 : 64; }
int dw_chunk_tokens(int64_t T, int d, int E) {
    const int eg = dw_expert_group(E);
    const int64_t blocks = (int64_t)((d + 8 * (1024 / eg) - 1) / (8 * (1024 / eg))) * ((E + eg - 1) / eg);
    int tc = 512;
    while (tc > 128 && blocks * ((T + tc - 1) / tc) < 1024) tc /= 2;
    return tc;
}

// part_w[chunk][n][c] = sum over the chunk's tokens t (in order) of
// dz[t, n] x[t, c], as a register-tiled product: a block covers EG experts
// and 8 (1024 / EG) columns; each thread owns 4 experts x 8 columns, so a
// staged token costs it 16 bytes of dz and 32 bytes of x from LDS for 32
// FMAs.  Column block 0 also writes part_b[chunk][n] = sum_t dz[t, n].
template <bool BF16, int EG>
__global__ __launch_bounds__(256) void router_bwd_dw_kernel(const float *__restrict__ dz,
                                                            const void *__restrict__ x, int64_t T, int d,
                                                            int E, int tc, float *__restrict__ part_w,
                                                            float *__restrict__ part_b) {
    constexpr int TY = EG / 4;                       // groups of 4 experts
    constexpr int TX = 256 / TY;                     // groups of 8 columns
    constexpr int NC = TX * 8;                       // columns per block
    constexpr int TS = EG == 64 ? 32 : 16;           // tokens staged at a time
    __shared__ __attribute__((aligned(16))) float s_dz[TS][EG];
    __shared__ __attribute__((aligned(16))) float s_x[TS][NC];
    const int tid = threadIdx.x;
    const int tx = tid % TX, ty = tid / TX;
    const int c0 = blockIdx.x * NC;
    const int n0 = blockIdx.y * EG;
    const int chunk = blockIdx.z;
    const int64_t ta = (int64_t)chunk * tc;
    const int64_t tb = ta + tc < T ? ta + tc : T;
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    float bacc = 0.f;
    for (int64_t t0 = ta; t0 < tb; t0 += TS) {
        for (int i = tid; i < TS * EG; i += 256) {
            const int r = i / EG, q = i - r * EG;
            const int64_t t = t0 + r;
            s_dz[r][q] = (t < tb && n0 + q < E) ? dz[t * E + n0 + q] : 0.f;
        }
        for (int i = tid; i < TS * (NC / 8); i += 256) {
            const int r = i / (NC / 8), pc = i - r * (NC / 8);
            const int64_t t = t0 + r;
            const int c = c0 + pc * 8;
            float v[8];
            if (t < tb && c < d) {
                load8<BF16>(x, t * d + c, v);
            } else {
#pragma unroll
                for (int h = 0; h < 8; ++h) v[h] = 0.f;
            }
            float4 *dst = reinterpret_cast<float4 *>(&s_x[r][pc * 8]);
            dst[0] = make_float4(v[0], v[1], v[2], v[3]);
            dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
        __syncthreads();
        for (int r = 0; r < TS; ++r) {
            const float4 zv = *reinterpret_cast<const float4 *>(&s_dz[r][ty * 4]);
            const float4 xa = *reinterpret_cast<const float4 *>(&s_x[r][tx * 8]);
            const float4 xb = *reinterpret_cast<const float4 *>(&s_x[r][tx * 8 + 4]);
            const float zs[4] = {zv.x, zv.y, zv.z, zv.w};
            const float xs[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(zs[i], xs[j], acc[i][j]);
        }
        if (blockIdx.x == 0 && tid < EG) {
            const int m = tb - t0 < TS ? (int)(tb - t0) : TS;
            for (int r = 0; r < m; ++r) bacc += s_dz[r][tid];
        }
        __syncthreads();
    }
    const int cc = c0 + tx * 8;
    if (cc < d)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + ty * 4 + i;
            if (n < E) {
                float4 *o = reinterpret_cast<float4 *>(part_w + ((int64_t)chunk * E + n) * d + cc);
                o[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                o[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
            }
        }
    if (blockIdx.x == 0 && tid < EG && n0 + tid < E) part_b[(int64_t)chunk * E + n0 + tid] = bacc;
}

// dW_r[n][c] = sum over chunks in order of part_w; db_r likewise.
__global__ __launch_bounds__(256) void router_bwd_dw_reduce_kernel(const float *__restrict__ part_w,
                                                                   const float *__restrict__ part_b, int nchunk,
                                                                   int E, int d, float *__restrict__ dW,
                                                                   float *__restrict__ db) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nw = (int64_t)E * d;
    if (i < nw) {
        float s = 0.f;
#pragma unroll 8
        for (int q = 0; q < nchunk; ++q) s += part_w[(int64_t)q * nw + i];
        dW[i] = s;
    }
    if (db != nullptr && i < E) {
        float s = 0.f;
        for (int q = 0; q < nchunk; ++q) s += part_b[(int64_t)q * E + i];
        db[i] = s;
    }
}

}  // namespace

int router_bwd_chunks(int64_t T, int d, int E) {
    const int tc = dw_chunk_tokens(T, d, E);
    return (int)((T + tc - 1) / tc);
}

hipError_t launch_combine_backward(const void *dy, int dtype_bf16, const void *ybuf, const int32_t *expert_idx,
                                   const int32_t *slot, const float *gate, int64_t T, int d, int E, int k,
                                   int64_t C, float *dgate, void *dybuf, hipStream_t s) {
    const int64_t n = T * k;
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    if (dtype_bf16)
        hipLaunchKernelGGL(combine_backward_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, dy, ybuf,
                           expert_idx, slot, gate, T, d, E, k, C, dgate, dybuf);
    else
        hipLaunchKernelGGL(combine_backward_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, dy, ybuf,
                           expert_idx, slot, gate, T, d, E, k, C, dgate, dybuf);
    return hipGetLastError();
}

hipError_t launch_router_backward(const void *x, int dtype_bf16, const float *W_r, const float *logits,
                                  const int32_t *expert_idx, const float *gate, const float *dgate,
                                  const int32_t *route_count, int64_t T, int d, int E, int k, float alpha,
                                  float z_weight, float *dz, float *dW, float *db, float *dx, float *part_w,
                                  float *part_b, hipStream_t s) {
    const int nchunk = router_bwd_chunks(T, d, E);
    const int tc = dw_chunk_tokens(T, d, E);
    if (nchunk > 65535) return hipErrorInvalidValue;      // the grid's z extent
    if (T > 0) {
        hipLaunchKernelGGL(router_bwd_dz_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits,
                           expert_idx, gate, dgate, route_count, T, E, k, alpha, z_weight, dz);
        if (dx != nullptr)
            hipLaunchKernelGGL(router_bwd_dx_kernel, dim3((unsigned)((T + DX_TT - 1) / DX_TT),
                                                          (unsigned)((d + DX_NC - 1) / DX_NC)),
                               dim3(256), 0, s, dz, W_r, T, d, E, dx);
#define MOE_DW(EGV)                                                                                      \
    do {                                                                                                 \
        const dim3 g((unsigned)((d + 8 * (1024 / EGV) - 1) / (8 * (1024 / EGV))),                        \
                     (unsigned)((E + EGV - 1) / EGV), (unsigned)nchunk);                                 \
        if (dtype_bf16)                                                                                  \
            hipLaunchKernelGGL((router_bwd_dw_kernel<true, EGV>), g, dim3(256), 0, s, dz, x, T, d, E,   \
                               tc, part_w, part_b);                                                      \
        else                                                                                             \
            hipLaunchKernelGGL((router_bwd_dw_kernel<false, EGV>), g, dim3(256), 0, s, dz, x, T, d, E,  \
                               tc, part_w, part_b);                                                      \
    } while (0)
        if (dw_expert_group(E) == 16) MOE_DW(16);
        else MOE_DW(64);
#undef MOE_DW
    }
    const int64_t nw = (int64_t)E * d;
    hipLaunchKernelGGL(router_bwd_dw_reduce_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, part_w,
                       part_b, nchunk, E, d, dW, db);
    return hipGetLastError();
}

}  // namespace moe
