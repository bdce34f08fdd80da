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

// dx[t, :] = sum_n dz[t, n] W_r[n, :] for TOK tokens per block; W_r is
// read from L2 once per block, four rows per step so the loads overlap.
template <int TOK>
__global__ __launch_bounds__(256) void router_bwd_dx_kernel(const float *__restrict__ dz,
                                                            const float *__restrict__ Wr, int64_t T, int d,
                                                            int E, float *__restrict__ dx) {
    extern __shared__ float s_dz[];                  // [TOK][E]
    const int64_t t0 = (int64_t)blockIdx.x * TOK;
    for (int i = threadIdx.x; i < TOK * E; i += 256) {
        const int r = i / E;
        s_dz[i] = t0 + r < T ? dz[(t0 + r) * E + (i - r * E)] : 0.f;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < d; c += 256) {
        float acc[TOK];
#pragma unroll
        for (int r = 0; r < TOK; ++r) acc[r] = 0.f;
        int n = 0;
        for (; n + 4 <= E; n += 4) {
            float w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = Wr[(int64_t)(n + u) * d + c];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int r = 0; r < TOK; ++r) acc[r] = fmaf(s_dz[r * E + n + u], w[u], acc[r]);
        }
        for (; n < E; ++n) {
            const float w = Wr[(int64_t)n * d + c];
#pragma unroll
            for (int r = 0; r < TOK; ++r) acc[r] = fmaf(s_dz[r * E + n], w, acc[r]);
        }
#pragma unroll
        for (int r = 0; r < TOK; ++r)
            if (t0 + r < T) dx[(t0 + r) * d + c] = acc[r];
    }
}

constexpr int DW_EG = 16;      // experts per block
constexpr int DW_TC = 512;     // tokens per chunk (one partial row each)
constexpr int DW_TS = 32;      // tokens staged in LDS at a time

// part_w[chunk][n][c] = sum over the chunk's tokens t of dz[t, n] x[t, c];
// column block 0 also writes part_b[chunk][n] = sum_t dz[t, n].
template <bool BF16>
__global__ __launch_bounds__(256) void router_bwd_dw_kernel(const float *__restrict__ dz,
                                                            const void *__restrict__ x, int64_t T, int d,
                                                            int E, float *__restrict__ part_w,
                                                            float *__restrict__ part_b) {
    __shared__ __attribute__((aligned(16))) float s_dz[DW_TS][DW_EG];
    const int c = blockIdx.x * 256 + threadIdx.x;
    const int n0 = blockIdx.y * DW_EG;
    const int chunk = blockIdx.z;
    const int64_t ta = (int64_t)chunk * DW_TC;
    const int64_t tb = ta + DW_TC < T ? ta + DW_TC : T;
    float acc[DW_EG];
#pragma unroll
    for (int i = 0; i < DW_EG; ++i) acc[i] = 0.f;
    float bacc = 0.f;
    for (int64_t t0 = ta; t0 < tb; t0 += DW_TS) {
        for (int i = threadIdx.x; i < DW_TS * DW_EG; i += 256) {
            const int r = i / DW_EG, q = i - r * DW_EG;
            const int64_t t = t0 + r;
            s_dz[r][q] = (t < tb && n0 + q < E) ? dz[t * E + n0 + q] : 0.f;
        }
        // this column's x for the staged tokens, all loads issued together
        // (rows past the chunk read as 0, and their dz rows are 0 too)
        float xv[DW_TS];
#pragma unroll
        for (int r = 0; r < DW_TS; ++r) {
            const int64_t xi = (t0 + r) * d + c;
            const bool in = c < d && t0 + r < tb;
            xv[r] = !in ? 0.f : BF16 ? bf2f(reinterpret_cast<const uint16_t *>(x)[xi])
                                     : reinterpret_cast<const float *>(x)[xi];
        }
        __syncthreads();
        const int m = tb - t0 < DW_TS ? (int)(tb - t0) : DW_TS;
#pragma unroll 4
        for (int r = 0; r < DW_TS; ++r) {
            const float4 *z4 = reinterpret_cast<const float4 *>(&s_dz[r][0]);
#pragma unroll
            for (int q = 0; q < DW_EG / 4; ++q) {
                const float4 v = z4[q];
                acc[4 * q] = fmaf(v.x, xv[r], acc[4 * q]);
                acc[4 * q + 1] = fmaf(v.y, xv[r], acc[4 * q + 1]);
                acc[4 * q + 2] = fmaf(v.z, xv[r], acc[4 * q + 2]);
                acc[4 * q + 3] = fmaf(v.w, xv[r], acc[4 * q + 3]);
            }
        }
        if (blockIdx.x == 0 && threadIdx.x < DW_EG)
            for (int r = 0; r < m; ++r) bacc += s_dz[r][threadIdx.x];
        __syncthreads();
    }
    if (c < d)
#pragma unroll
        for (int i = 0; i < DW_EG; ++i)
            if (n0 + i < E) part_w[((int64_t)chunk * E + n0 + i) * d + c] = acc[i];
    if (blockIdx.x == 0 && threadIdx.x < DW_EG && n0 + threadIdx.x < E)
        part_b[(int64_t)chunk * E + n0 + threadIdx.x] = bacc;
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

int router_bwd_chunks(int64_t T) { return (int)((T + DW_TC - 1) / DW_TC); }

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
    const int nchunk = router_bwd_chunks(T);
    if (T > 0) {
        hipLaunchKernelGGL(router_bwd_dz_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, logits,
                           expert_idx, gate, dgate, route_count, T, E, k, alpha, z_weight, dz);
        if (dx != nullptr && E <= 256)
            hipLaunchKernelGGL(router_bwd_dx_kernel<32>, dim3((unsigned)((T + 31) / 32)), dim3(256),
                               (size_t)32 * E * sizeof(float), s, dz, W_r, T, d, E, dx);
        else if (dx != nullptr)
            hipLaunchKernelGGL(router_bwd_dx_kernel<8>, dim3((unsigned)((T + 7) / 8)), dim3(256),
                               (size_t)8 * E * sizeof(float), s, dz, W_r, T, d, E, dx);
        const dim3 g((unsigned)((d + 255) / 256), (unsigned)((E + DW_EG - 1) / DW_EG), (unsigned)nchunk);
        if (dtype_bf16)
            hipLaunchKernelGGL(router_bwd_dw_kernel<true>, g, dim3(256), 0, s, dz, x, T, d, E, part_w, part_b);
        else
            hipLaunchKernelGGL(router_bwd_dw_kernel<false>, g, dim3(256), 0, s, dz, x, T, d, E, part_w, part_b);
    }
    const int64_t nw = (int64_t)E * d;
    hipLaunchKernelGGL(router_bwd_dw_reduce_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, part_w,
                       part_b, nchunk, E, d, dW, db);
    return hipGetLastError();
}

}  // namespace moe
