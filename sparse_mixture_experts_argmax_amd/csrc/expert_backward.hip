// Backward of the expert side: the gradients of the grouped expert FFN and the
// adjoint of the dispatch.
//
// [CMU-L16] exercise 2 and section 5: each expert is an ordinary FFN on the
// rows routed to it, so its backward is the chain rule through the two
// products and the activation ([SW-GLaM] "Dense Scaling 与 MoE 的核心差异":
// FFN(x) = W_2 sigma(W_1 x); [CMU-L16] 2.1 biases, 2.3 SwiGLU):
//   A = X W1^T (+ b1), G = X W3^T          (recomputed from the dispatch rows)
//   dH = dY W2;  dW2 = dY^T H;  db2 = column sums of dY
//   ReLU:   dA = dH * 1[A > 0]
//   SwiGLU: dA = dH * G * silu'(A),  dG = dH * silu(A)
//   dX = dA W1 (+ dG W3);  dW1 = dA^T X;  dW3 = dG^T X;  db1 = column sums of dA
// The dispatch copied x_t to row slot_tj of expert e_tj; its adjoint adds
// those rows back per token ([SW-GLaM] "All-to-All", the return trip).
//
// Every product runs on the forward's grouped GEMM (MFMA, K-contiguous
// operands), so the operands that are not K-contiguous are transposed first:
//   * W2 [E, d, f] -> W2t [E, f, d]                 (B of dH = dY W2)
//   * W1, W3 [E, f, d] -> W13t [E, d, f (+ f)]      (B of dX = [dA | dG] [W1; W3])
//   * dY, X [E, C, d] -> dYt, Xt [E, d, Cp]         (the weight gradients
//     contract over the rows of an expert, so both operands are transposed)
//   * H, dA, dG [E, C, f] -> Ht, dAt, dGt [E, f, Cp], written transposed by
//     the activation-backward kernel itself (one LDS tile, two layouts out)
// Cp is C rounded up to 64 and the rows at or beyond an expert's count are
// zero in every transposed activation, so the weight-gradient GEMMs sum over
// whole K tiles of real rows and zeros.  Intermediates are rounded to the
// storage dtype, as the forward's H is; sums are fp32.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int TT = 64;      // transpose tile

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
    using T = uint16_t;
    static __device__ __forceinline__ float ld(T v) { return bf2f(v); }
    static __device__ __forceinline__ T st(float v) { return f2bf(v); }
};
template <>
struct Elem<false> {
    using T = float;
    static __device__ __forceinline__ float ld(T v) { return v; }
    static __device__ __forceinline__ T st(float v) { return v; }
};

// dst[e][c][col0 + r] = src[e][r][c] for r < rcount[e] (all R rows when
// rcount is null) and 0 for the other r < R_pad; c < Cc.  One 64 x 64 tile per
// block, staged through LDS so that both the reads and the writes run along
// rows.  Grid (ceil(Cc / 64), ceil(R_pad / 64), E).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *__restrict__ src, int64_t src_es, int src_ld,
                                                        int R, int Cc, const int32_t *__restrict__ rcount,
                                                        T *__restrict__ dst, int64_t dst_es, int dst_ld,
                                                        int dst_col0, int R_pad) {
    __shared__ T tile[TT][TT + 1];
    const int e = blockIdx.z;
    const int c0 = blockIdx.x * TT;
    const int r0 = blockIdx.y * TT;
    int rc = R;
    if (rcount != nullptr) {
        rc = rcount[e];
        rc = rc < 0 ? 0 : (rc > R ? R : rc);
    }
    const T *s = src + (int64_t)e * src_es;
    T *d = dst + (int64_t)e * dst_es;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < TT; i += 4) {
        const int r = r0 + i, c = c0 + tx;
        T v = T(0);
        if (r < rc && c < Cc) v = s[(int64_t)r * src_ld + c];
        tile[i][tx] = v;
    }
    __syncthreads();
    for (int i = ty; i < TT; i += 4) {
        const int c = c0 + i, r = r0 + tx;
        if (c < Cc && r < R_pad) d[(int64_t)c * dst_ld + dst_col0 + r] = tile[tx][i];
    }
}

// The bf16 transpose with 16-byte accesses on both sides: a thread loads 8
// consecutive columns of one source row, and stores 8 consecutive source
// rows of one column as one 16-byte piece of its destination row (read from
// the LDS tile one element at a time).  Needs Cc, R_pad, src_ld, dst_ld and
// dst_col0 to be multiples of 8 (every use here: widths and the padded row
// count are); same result as transpose_kernel.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t *__restrict__ src, int64_t src_es,
                                                          int src_ld, int R, int Cc,
                                                          const int32_t *__restrict__ rcount,
                                                          uint16_t *__restrict__ dst, int64_t dst_es, int dst_ld,
                                                          int dst_col0, int R_pad) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[TT][TT + 8];
    const int e = blockIdx.z;
    const int c0 = blockIdx.x * TT;
    const int r0 = blockIdx.y * TT;
    int rc = R;
    if (rcount != nullptr) {
        rc = rcount[e];
        rc = rc < 0 ? 0 : (rc > R ? R : rc);
    }
    const uint16_t *s = src + (int64_t)e * src_es;
    uint16_t *d = dst + (int64_t)e * dst_es;
    const int t = threadIdx.x;
    // load: 64 rows x 8 pieces, two per thread
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = t + 256 * h;
        const int i = q >> 3, pc = (q & 7) * 8;
        const int r = r0 + i, c = c0 + pc;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < rc && c < Cc) v = ld16(s + (int64_t)r * src_ld + c);
        *reinterpret_cast<u32x4 *>(&tile[i][pc]) = v;
    }
    __syncthreads();
    // store: 64 destination rows (source columns) x 8 pieces of 8 source rows
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int q = t + 256 * h;
        const int j = q >> 3, pr = (q & 7) * 8;
        const int c = c0 + j, r = r0 + pr;
        if (c < Cc && r < R_pad) {
            u32x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = (uint32_t)tile[pr + 2 * u][j] | ((uint32_t)tile[pr + 2 * u + 1][j] << 16);
            st16(d + (int64_t)c * dst_ld + dst_col0 + r, v);
        }
    }
}

// The activation backward of one 64-row x 64-column tile of one expert, from
// the recomputed pre-activations A (and G) and dH = dY W2:
//   ReLU:   H = max(A, 0), dA = dH * 1[A > 0]
//   SwiGLU: s = silu(A), H = s G, dA = dH G silu'(A), dG = dH s
// dA (and dG) go out row-major into dAG [E, C, nf] (dG in columns f ..
// 2f - 1) for dX, and transposed into Ht, dAt (, dGt) [E, f, Cp] for the
// weight gradients, zero in the rows at or beyond the expert's count.
// silu through the hardware exp2 and reciprocal (about 1 ulp each), as in
// the forward's epilogue.  Grid (ceil(f / 64), Cp / 64, E).
template <bool BF16, bool SW>
__global__ __launch_bounds__(256) void act_backward_kernel(
    const typename Elem<BF16>::T *__restrict__ A, const typename Elem<BF16>::T *__restrict__ G,
    const typename Elem<BF16>::T *__restrict__ dH, const int32_t *__restrict__ count, int64_t C, int f, int Cp,
    typename Elem<BF16>::T *__restrict__ dAG, typename Elem<BF16>::T *__restrict__ Ht,
    typename Elem<BF16>::T *__restrict__ dAt, typename Elem<BF16>::T *__restrict__ dGt) {
    using El = Elem<BF16>;
    using T = typename El::T;
    __shared__ T sH[TT][TT + 1];
    __shared__ T sA[TT][TT + 1];
    __shared__ T sG[SW ? TT : 1][TT + 1];
    const int e = blockIdx.z;
    const int j0 = blockIdx.x * TT;
    const int m0 = blockIdx.y * TT;
    int cnt = count[e];
    cnt = cnt < 0 ? 0 : (cnt > C ? (int)C : cnt);
    const int nf = SW ? 2 * f : f;
    const int64_t rbase = (int64_t)e * C * f;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < TT; i += 4) {
        const int m = m0 + i, j = j0 + tx;
        float h = 0.f, da = 0.f, dg = 0.f;
        if (m < cnt && j < f) {
            const int64_t o = rbase + (int64_t)m * f + j;
            const float a = El::ld(A[o]);
            const float dh = El::ld(dH[o]);
            if (SW) {
                const float g = El::ld(G[o]);
                const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.44269504088896341f));
                const float s = a * sg;
                h = s * g;
                da = dh * g * (sg * (1.0f + a * (1.0f - sg)));
                dg = dh * s;
            } else {
                h = fmaxf(a, 0.f);
                da = a > 0.f ? dh : 0.f;
            }
            T *row = dAG + ((int64_t)e * C + m) * nf;
            row[j] = El::st(da);
            if (SW) row[f + j] = El::st(dg);
        }
        sH[i][tx] = El::st(h);
        sA[i][tx] = El::st(da);
        if (SW) sG[SW ? i : 0][tx] = El::st(dg);
    }
    __syncthreads();
    const int64_t tbase = (int64_t)e * f * Cp;
    for (int i = ty; i < TT; i += 4) {
        const int j = j0 + i, m = m0 + tx;
        if (j < f && m < Cp) {
            const int64_t o = tbase + (int64_t)j * Cp + m;
            Ht[o] = sH[tx][i];
            dAt[o] = sA[tx][i];
            if (SW) dGt[o] = sG[SW ? tx : 0][i];
        }
    }
}

// The bf16 activation backward with 16-byte accesses (the scheme of
// transpose16_kernel): a thread takes 8 consecutive columns of one row for
// the loads, the arithmetic and the row-major stores, then 8 consecutive
// rows of one column for the transposed stores (gathered from the LDS tiles
// one element at a time).  The same arithmetic element for element as
// act_backward_kernel.  Needs f % 8 == 0; Cp is a multiple of 64.
template <bool SW>
__global__ __launch_bounds__(256) void act_backward16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ G, const uint16_t *__restrict__ dH,
    const int32_t *__restrict__ count, int64_t C, int f, int Cp, uint16_t *__restrict__ dAG,
    uint16_t *__restrict__ Ht, uint16_t *__restrict__ dAt, uint16_t *__restrict__ dGt) {
    __shared__ __attribute__((aligned(16))) uint16_t sH[TT][TT + 8];
    __shared__ __attribute__((aligned(16))) uint16_t sA[TT][TT + 8];
    __shared__ __attribute__((aligned(16))) uint16_t sG[SW ? TT : 1][TT + 8];
    const int e = blockIdx.z;
    const int j0 = blockIdx.x * TT;
    const int m0 = blockIdx.y * TT;
    int cnt = count[e];
    cnt = cnt < 0 ? 0 : (cnt > C ? (int)C : cnt);
    const int nf = SW ? 2 * f : f;
    const int64_t rbase = (int64_t)e * C * f;
    const int t = threadIdx.x;
    // 64 rows x 8 pieces of 8 columns, two per thread
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int q = t + 256 * hh;
        const int i = q >> 3, pc = (q & 7) * 8;
        const int m = m0 + i, j = j0 + pc;
        u32x4 hv = {0u, 0u, 0u, 0u}, av = {0u, 0u, 0u, 0u}, gv = {0u, 0u, 0u, 0u};
        if (m < cnt && j < f) {
            const int64_t o = rbase + (int64_t)m * f + j;
            const u32x4 a8 = ld16(A + o);
            const u32x4 d8 = ld16(dH + o);
            u32x4 g8 = {0u, 0u, 0u, 0u};
            if (SW) g8 = ld16(G + o);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float h2[2], da2[2], dg2[2];
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const float a = bf2f((uint16_t)(a8[u] >> (16 * w)));
                    const float dh = bf2f((uint16_t)(d8[u] >> (16 * w)));
                    if (SW) {
                        const float g = bf2f((uint16_t)(g8[u] >> (16 * w)));
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.44269504088896341f));
                        const float sa = a * sg;
                        h2[w] = sa * g;
                        da2[w] = dh * g * (sg * (1.0f + a * (1.0f - sg)));
                        dg2[w] = dh * sa;
                    } else {
                        h2[w] = fmaxf(a, 0.f);
                        da2[w] = a > 0.f ? dh : 0.f;
                        dg2[w] = 0.f;
                    }
                }
                hv[u] = pack_bf16x2(h2[0], h2[1]);
                av[u] = pack_bf16x2(da2[0], da2[1]);
                gv[u] = pack_bf16x2(dg2[0], dg2[1]);
            }
            uint16_t *row = dAG + ((int64_t)e * C + m) * nf;
            st16(row + j, av);
            if (SW) st16(row + f + j, gv);
        }
        *reinterpret_cast<u32x4 *>(&sH[i][pc]) = hv;
        *reinterpret_cast<u32x4 *>(&sA[i][pc]) = av;
        if (SW) *reinterpret_cast<u32x4 *>(&sG[SW ? i : 0][pc]) = gv;
    }
    __syncthreads();
    // 64 destination rows (columns j) x 8 pieces of 8 rows m
    const int64_t tbase = (int64_t)e * f * Cp;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int q = t + 256 * hh;
        const int jj = q >> 3, pr = (q & 7) * 8;
        const int j = j0 + jj, m = m0 + pr;
        if (j < f && m < Cp) {
            const int64_t o = tbase + (int64_t)j * Cp + m;
            u32x4 vh, va, vg;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                vh[u] = (uint32_t)sH[pr + 2 * u][jj] | ((uint32_t)sH[pr + 2 * u + 1][jj] << 16);
                va[u] = (uint32_t)sA[pr + 2 * u][jj] | ((uint32_t)sA[pr + 2 * u + 1][jj] << 16);
                if (SW) vg[u] = (uint32_t)sG[SW ? pr + 2 * u : 0][jj] | ((uint32_t)sG[SW ? pr + 2 * u + 1 : 0][jj] << 16);
            }
            st16(Ht + o, vh);
            st16(dAt + o, va);
            if (SW) st16(dGt + o, vg);
        }
    }
}

// dst[r] = sum over c < Cp of src[r][c] (fp32, lane-strided then a butterfly:
// a fixed order), one wave per row, rounded to the storage dtype.
template <bool BF16>
__global__ __launch_bounds__(256) void rowsum_kernel(const typename Elem<BF16>::T *__restrict__ src, int64_t rows,
                                                     int Cp, typename Elem<BF16>::T *__restrict__ dst) {
    using El = Elem<BF16>;
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const typename El::T *p = src + r * Cp;
    float s = 0.f;
    for (int c = lane; c < Cp; c += 64) s += El::ld(p[c]);
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (lane == 0) dst[r] = El::st(s);
}

// n16 pieces of 16 bytes set to zero (a kernel, not hipMemsetAsync, so that
// the call can sit in a captured graph)
__global__ __launch_bounds__(256) void zero16_kernel(u32x4 *__restrict__ p, int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n16) p[i] = u32x4{0u, 0u, 0u, 0u};
}

hipError_t zero_bytes(void *p, size_t bytes, hipStream_t s) {
    if (p == nullptr || bytes == 0) return hipSuccess;
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, (u32x4 *)p, n16);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t *__restrict__ p, int n, int v) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// dx_t = dx_add_t + sum over kept choices j (rank order) of dxbuf[e_tj, slot_tj],
// fp32.  One wave per token, 16-byte pieces of the dxbuf rows per lane.
template <bool BF16>
__global__ __launch_bounds__(256) void dispatch_backward_kernel(
    const uint8_t *__restrict__ dxbuf, const int32_t *__restrict__ expert_idx, const int32_t *__restrict__ slot,
    int64_t T, int d, int E, int k, int64_t C, const float *__restrict__ dx_add, float *__restrict__ dx) {
    constexpr int EPP = BF16 ? 8 : 4;           // elements per 16-byte piece
    constexpr int ES = BF16 ? 2 : 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int pieces = d / EPP;
    const int64_t row_bytes = (int64_t)d * ES;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    for (int64_t t = (int64_t)blockIdx.x * 4 + wave; t < T; t += nwaves) {
        for (int p = lane; p < pieces; p += 64) {
            float acc[EPP];
            if (dx_add != nullptr) {
#pragma unroll
                for (int q = 0; q < EPP; q += 4) {
                    const u32x4 v = ld16(dx_add + t * d + p * EPP + q);
#pragma unroll
                    for (int u = 0; u < 4; ++u) acc[q + u] = __uint_as_float(v[u]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < EPP; ++q) acc[q] = 0.f;
            }
            for (int j = 0; j < k; ++j) {
                const int64_t a = t * k + j;
                const int s = slot[a];
                const int e = expert_idx[a];
                if (s < 0 || s >= C || e < 0 || e >= E) continue;
                const u32x4 v = ld16(dxbuf + ((int64_t)e * C + s) * row_bytes + p * 16);
                if (BF16) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[2 * q] += bf2f((uint16_t)(v[q] & 0xFFFFu));
                        acc[2 * q + 1] += bf2f((uint16_t)(v[q] >> 16));
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q] += __uint_as_float(v[q]);
                }
            }
#pragma unroll
            for (int q = 0; q < EPP; q += 4) {
                u32x4 o;
#pragma unroll
                for (int u = 0; u < 4; ++u) o[u] = __float_as_uint(acc[q + u]);
                st16(dx + t * d + p * EPP + q, o);
            }
        }
    }
}

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

template <typename T>
hipError_t transpose(const void *src, int64_t src_es, int src_ld, int R, int Cc, const int32_t *rcount, void *dst,
                     int64_t dst_es, int dst_ld, int dst_col0, int R_pad, int E, hipStream_t s) {
    if (R_pad <= 0 || Cc <= 0 || E <= 0) return hipSuccess;
    const dim3 grid((unsigned)((Cc + TT - 1) / TT), (unsigned)((R_pad + TT - 1) / TT), (unsigned)E);
    const bool vec16 = sizeof(T) == 2 && Cc % 8 == 0 && R_pad % 8 == 0 && src_ld % 8 == 0 && dst_ld % 8 == 0 &&
                       dst_col0 % 8 == 0;
    if (vec16)
        hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, s, (const uint16_t *)src, src_es, src_ld, R, Cc,
                           rcount, (uint16_t *)dst, dst_es, dst_ld, dst_col0, R_pad);
    else
        hipLaunchKernelGGL(transpose_kernel<T>, grid, dim3(256), 0, s, (const T *)src, src_es, src_ld, R, Cc, rcount,
                           (T *)dst, dst_es, dst_ld, dst_col0, R_pad);
    return hipGetLastError();
}

}  // namespace

ExpertBwdWs expert_backward_ws(int E, int64_t C, int d, int f, int dtype_bf16, int act) {
    const size_t es = dtype_bf16 ? 2 : 4;
    const bool sw = act == 2;
    const size_t nf = (size_t)f * (sw ? 2 : 1);
    const size_t Cp = (size_t)((C + 63) / 64 * 64);
    ExpertBwdWs w;
    size_t o = 0;
    w.tmap_r = o;  o += up256((size_t)tile_map_ints(E) * 4);
    w.tmap_d = o;  o += up256((size_t)tile_map_ints(E) * 4);
    w.tmap_f = o;  o += up256((size_t)tile_map_ints(E) * 4);
    w.cnt_d = o;   o += up256((size_t)E * 4);
    w.cnt_f = o;   o += up256((size_t)E * 4);
    w.a = o;       o += up256((size_t)E * C * f * es);
    w.g = o;       o += sw ? up256((size_t)E * C * f * es) : 0;
    w.dh = o;      o += up256((size_t)E * C * f * es);
    w.dag = o;     o += up256((size_t)E * C * nf * es);
    w.w2t = o;     o += up256((size_t)E * f * d * es);
    w.w13t = o;    o += up256((size_t)E * d * nf * es);
    w.dyt = o;     o += up256((size_t)E * d * Cp * es);
    w.xt = o;      o += up256((size_t)E * d * Cp * es);
    w.ht = o;      o += up256((size_t)E * f * Cp * es);
    w.dat = o;     o += up256((size_t)E * f * Cp * es);
    w.dgt = o;     o += sw ? up256((size_t)E * f * Cp * es) : 0;
    w.part = o;    o += up256(tail_split_bytes(dtype_bf16, C));   // the products over the experts' rows
    w.total = o;
    return w;
}

hipError_t launch_expert_backward(const void *xbuf, int dtype_bf16, const int32_t *expert_count, int E, int64_t C,
                                  int d, int f, const void *W1, const void *b1, const void *W3, const void *W2,
                                  int act, const void *dybuf, void *dxbuf, void *dW1, void *dW3, void *dW2,
                                  void *db1, void *db2, char *ws, hipStream_t s) {
    const ExpertBwdWs w = expert_backward_ws(E, C, d, f, dtype_bf16, act);
    const bool sw = act == 2;
    const int nf = sw ? 2 * f : f;
    const int Cp = (int)((C + 63) / 64 * 64);
    const size_t es = dtype_bf16 ? 2 : 4;
    int32_t *tmap_r = (int32_t *)(ws + w.tmap_r), *tmap_d = (int32_t *)(ws + w.tmap_d),
            *tmap_f = (int32_t *)(ws + w.tmap_f), *cnt_d = (int32_t *)(ws + w.cnt_d),
            *cnt_f = (int32_t *)(ws + w.cnt_f);
    void *Aa = ws + w.a, *Ga = ws + w.g, *dH = ws + w.dh, *dAG = ws + w.dag, *W2t = ws + w.w2t,
         *W13t = ws + w.w13t, *dYt = ws + w.dyt, *Xt = ws + w.xt, *Ht = ws + w.ht, *dAt = ws + w.dat,
         *dGt = ws + w.dgt;
    hipError_t err;
#define MOE_TRY(expr)                       \
    do {                                    \
        if ((err = (expr)) != hipSuccess) return err; \
    } while (0)
    if (C == 0) {
        // no expert rows: every weight and bias gradient is zero
        MOE_TRY(zero_bytes(dW1, (size_t)E * f * d * es, s));
        MOE_TRY(zero_bytes(dW2, (size_t)E * d * f * es, s));
        if (sw) MOE_TRY(zero_bytes(dW3, (size_t)E * f * d * es, s));
        MOE_TRY(zero_bytes(db1, (size_t)E * f * es, s));
        MOE_TRY(zero_bytes(db2, (size_t)E * d * es, s));
        return hipSuccess;
    }
    // row tiles over the experts' kept rows, and over the d / f rows of the
    // weight gradients (every expert holds all of them)
    const int bm_r = gemm_bm(dtype_bf16, C, 0);
    const int bm_d = gemm_bm(dtype_bf16, d, 0);
    const int bm_f = gemm_bm(dtype_bf16, f, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, cnt_d, E, d);
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, cnt_f, E, f);
    MOE_TRY(hipGetLastError());
    MOE_TRY(launch_tile_map(expert_count, E, bm_r, tmap_r, s));
    MOE_TRY(launch_tile_map(cnt_d, E, bm_d, tmap_d, s));
    MOE_TRY(launch_tile_map(cnt_f, E, bm_f, tmap_f, s));
    const int64_t rows = (int64_t)E * C;
    // the pre-activations, recomputed: A = X W1^T (+ b1), G = X W3^T
    float *part = w.part < w.total ? reinterpret_cast<float *>(ws + w.part) : nullptr;
    MOE_TRY(launch_grouped_gemm(xbuf, W1, nullptr, b1, dtype_bf16, 0, expert_count, tmap_r, bm_r, E, C, f, d, rows,
                                Aa, s, nullptr, 0, nullptr, nullptr, part));
    if (sw)
        MOE_TRY(launch_grouped_gemm(xbuf, W3, nullptr, nullptr, dtype_bf16, 0, expert_count, tmap_r, bm_r, E, C, f,
                                    d, rows, Ga, s, nullptr, 0, nullptr, nullptr, part));
    // the K-contiguous operands: W2t, W13t, dYt, Xt
    if (dtype_bf16) {
        MOE_TRY(transpose<uint16_t>(W2, (int64_t)d * f, f, d, f, nullptr, W2t, (int64_t)f * d, d, 0, d, E, s));
        MOE_TRY(transpose<uint16_t>(W1, (int64_t)f * d, d, f, d, nullptr, W13t, (int64_t)d * nf, nf, 0, f, E, s));
        if (sw)
            MOE_TRY(transpose<uint16_t>(W3, (int64_t)f * d, d, f, d, nullptr, W13t, (int64_t)d * nf, nf, f, f, E, s));
        MOE_TRY(transpose<uint16_t>(dybuf, C * d, d, (int)C, d, expert_count, dYt, (int64_t)d * Cp, Cp, 0, Cp, E, s));
        MOE_TRY(transpose<uint16_t>(xbuf, C * d, d, (int)C, d, expert_count, Xt, (int64_t)d * Cp, Cp, 0, Cp, E, s));
    } else {
        MOE_TRY(transpose<float>(W2, (int64_t)d * f, f, d, f, nullptr, W2t, (int64_t)f * d, d, 0, d, E, s));
        MOE_TRY(transpose<float>(W1, (int64_t)f * d, d, f, d, nullptr, W13t, (int64_t)d * nf, nf, 0, f, E, s));
        if (sw)
            MOE_TRY(transpose<float>(W3, (int64_t)f * d, d, f, d, nullptr, W13t, (int64_t)d * nf, nf, f, f, E, s));
        MOE_TRY(transpose<float>(dybuf, C * d, d, (int)C, d, expert_count, dYt, (int64_t)d * Cp, Cp, 0, Cp, E, s));
        MOE_TRY(transpose<float>(xbuf, C * d, d, (int)C, d, expert_count, Xt, (int64_t)d * Cp, Cp, 0, Cp, E, s));
    }
    // dH = dY W2
    MOE_TRY(launch_grouped_gemm(dybuf, W2t, nullptr, nullptr, dtype_bf16, 0, expert_count, tmap_r, bm_r, E, C, f, d,
                                rows, dH, s, nullptr, 0, nullptr, nullptr, part));
    // the activation backward: dA (and dG) row-major, H, dA (and dG) transposed
    {
        const dim3 grid((unsigned)((f + TT - 1) / TT), (unsigned)(Cp / TT), (unsigned)E);
#define MOE_ACTB(BF, SWV, T_)                                                                                  \
    hipLaunchKernelGGL((act_backward_kernel<BF, SWV>), grid, dim3(256), 0, s, (const T_ *)Aa, (const T_ *)Ga,   \
                       (const T_ *)dH, expert_count, C, f, Cp, (T_ *)dAG, (T_ *)Ht, (T_ *)dAt, (T_ *)dGt)
        if (C > 0) {
            if (dtype_bf16 && f % 8 == 0) {
                if (sw)
                    hipLaunchKernelGGL((act_backward16_kernel<true>), grid, dim3(256), 0, s, (const uint16_t *)Aa,
                                       (const uint16_t *)Ga, (const uint16_t *)dH, expert_count, C, f, Cp,
                                       (uint16_t *)dAG, (uint16_t *)Ht, (uint16_t *)dAt, (uint16_t *)dGt);
                else
                    hipLaunchKernelGGL((act_backward16_kernel<false>), grid, dim3(256), 0, s, (const uint16_t *)Aa,
                                       (const uint16_t *)Ga, (const uint16_t *)dH, expert_count, C, f, Cp,
                                       (uint16_t *)dAG, (uint16_t *)Ht, (uint16_t *)dAt, (uint16_t *)dGt);
            } else if (dtype_bf16) {
                if (sw) MOE_ACTB(true, true, uint16_t); else MOE_ACTB(true, false, uint16_t);
            } else {
                if (sw) MOE_ACTB(false, true, float); else MOE_ACTB(false, false, float);
            }
        }
#undef MOE_ACTB
        MOE_TRY(hipGetLastError());
    }
    // dX = [dA | dG] [W1; W3]
    MOE_TRY(launch_grouped_gemm(dAG, W13t, nullptr, nullptr, dtype_bf16, 0, expert_count, tmap_r, bm_r, E, C, d, nf,
                                rows, dxbuf, s, nullptr, 0, nullptr, nullptr, part));
    // the weight gradients, contracting over the (padded) rows of each expert
    // (bf16: each expert's sum stops after its own rows, in whole K tiles)
    const int32_t *kc = dtype_bf16 ? expert_count : nullptr;
    MOE_TRY(launch_grouped_gemm(dYt, Ht, nullptr, nullptr, dtype_bf16, 0, cnt_d, tmap_d, bm_d, E, d, f, Cp,
                                (int64_t)E * d, dW2, s, nullptr, 0, nullptr, kc));
    MOE_TRY(launch_grouped_gemm(dAt, Xt, nullptr, nullptr, dtype_bf16, 0, cnt_f, tmap_f, bm_f, E, f, d, Cp,
                                (int64_t)E * f, dW1, s, nullptr, 0, nullptr, kc));
    if (sw)
        MOE_TRY(launch_grouped_gemm(dGt, Xt, nullptr, nullptr, dtype_bf16, 0, cnt_f, tmap_f, bm_f, E, f, d, Cp,
                                    (int64_t)E * f, dW3, s, nullptr, 0, nullptr, kc));
    // the bias gradients: row sums of the transposed dA and dY
    if (db1 != nullptr && E * (int64_t)f > 0) {
        const unsigned g = (unsigned)(((int64_t)E * f + 3) / 4);
        if (dtype_bf16)
            hipLaunchKernelGGL(rowsum_kernel<true>, dim3(g), dim3(256), 0, s, (const uint16_t *)dAt, (int64_t)E * f, Cp,
                               (uint16_t *)db1);
        else
            hipLaunchKernelGGL(rowsum_kernel<false>, dim3(g), dim3(256), 0, s, (const float *)dAt, (int64_t)E * f, Cp,
                               (float *)db1);
        MOE_TRY(hipGetLastError());
    }
    if (db2 != nullptr) {
        const unsigned g = (unsigned)(((int64_t)E * d + 3) / 4);
        if (dtype_bf16)
            hipLaunchKernelGGL(rowsum_kernel<true>, dim3(g), dim3(256), 0, s, (const uint16_t *)dYt, (int64_t)E * d, Cp,
                               (uint16_t *)db2);
        else
            hipLaunchKernelGGL(rowsum_kernel<false>, dim3(g), dim3(256), 0, s, (const float *)dYt, (int64_t)E * d, Cp,
                               (float *)db2);
        MOE_TRY(hipGetLastError());
    }
#undef MOE_TRY
    return hipSuccess;
}

hipError_t launch_dispatch_backward(const void *dxbuf, int dtype_bf16, const int32_t *expert_idx, const int32_t *slot,
                                    int64_t T, int d, int E, int k, int64_t C, const float *dx_add, float *dx,
                                    hipStream_t s) {
    if (T == 0) return hipSuccess;
    int64_t blocks = (T + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(dxbuf);
    if (dtype_bf16)
        hipLaunchKernelGGL(dispatch_backward_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, xb, expert_idx,
                           slot, T, d, E, k, C, dx_add, dx);
    else
        hipLaunchKernelGGL(dispatch_backward_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, xb, expert_idx,
                           slot, T, d, E, k, C, dx_add, dx);
    return hipGetLastError();
}

}  // namespace moe
