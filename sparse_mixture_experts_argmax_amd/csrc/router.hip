// Router: fp32 logits h = W_r x, softmax, top-k with lowest-index ties,
// gates, and per-block partial sums of the probabilities and choice counts.
//
// [SW-GLaM] "Dense Scaling 与 MoE 的核心差异": h(x) = W_r x, p = softmax(h).
// [SW-GLaM] "Switch Transformer：把 MoE 做简单": i* = argmax p, gate p_{i*}.
// [CMU-L16] section 2.3: top-k keeps k logits, gate = softmax over them;
// an all-zero router picks the lowest indices (ties -> lower index).
// [CS25-L5] "稳定训练" / [SW-RES] section 2.1: the router runs in fp32.
//
// Two kernels:
//  * router_mfma  (bf16 x, E <= 256).  The fp32 router weight is split
//    exactly into three bf16 parts, w = hi + mid + lo (each part takes the
//    round-to-nearest bf16 of what the previous parts left, so the sum
//    reproduces all 24 significand bits).  bf16 x bf16 products are exact
//    in fp32, so three bf16 MFMAs with fp32 accumulation give an fp32 dot
//    product without any fp32 vector FMA.  One wave owns 16 tokens and all
//    experts; the W_r chunk is split once per block into LDS and shared by
//    the four waves.  Row softmax and top-k run on the MFMA output layout
//    with 16-lane butterflies.
//  * router_generic (fp32 x, or E > 256): fp32 FMA dot products into LDS,
//    then one wave per token row.
#include "common.h"
#include "launch.h"

#include <math.h>

namespace moe {

namespace {

constexpr int MAXK = 8;

// ---------------------------------------------------------------------------
// MFMA router
// ---------------------------------------------------------------------------
constexpr int RM_WAVES = 4;
constexpr int RM_TOK_WAVE = 16;
constexpr int RM_TOK_BLOCK = RM_WAVES * RM_TOK_WAVE;
constexpr int RM_KC = 32;                  // one 16x16x32 MFMA k-step per chunk
constexpr int RM_STRIDE = RM_KC + 8;       // padded LDS row (bf16 elements)

__device__ __forceinline__ void split3(float w, uint16_t &h, uint16_t &m, uint16_t &l) {
    h = f2bf(w);
    const float r1 = w - bf2f(h);      // exact
    m = f2bf(r1);
    const float r2 = r1 - bf2f(m);     // exact
    l = f2bf(r2);
}

// Register stage of one K chunk: this thread's share of the W_r chunk (fp32)
// and its x fragment.  Loads are never conditional (indices are clamped and
// out-of-range values zeroed when used) so that the compiler only waits for a
// stage when it is consumed, DEPTH chunks after its loads were issued.
template <int WPER>
struct RStage {
    float4 w[WPER];
    u32x4 x;
    bool xin;
};

template <int NB>
constexpr int router_depth() { return NB <= 4 ? 4 : (NB <= 8 ? 3 : 2); }

template <int NB>
__global__ __launch_bounds__(256) void router_mfma_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ Wr, const float *__restrict__ br,
    int64_t T, int d, int E, int k, int32_t *__restrict__ out_idx, float *__restrict__ out_gate,
    float *__restrict__ part_prob, int32_t *__restrict__ part_cnt) {
    constexpr int EP = NB * 16;
    constexpr int DEPTH = router_depth<NB>();
    __shared__ __attribute__((aligned(16))) uint16_t sW[3][EP * RM_STRIDE];
    __shared__ float sProb[RM_WAVES][EP];
    __shared__ int sCnt[EP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;      // expert column within a 16-block / token row of A
    const int kg = lane >> 4;       // k group (A/B operands) or row group (D)
    const int64_t tw = (int64_t)blockIdx.x * RM_TOK_BLOCK + wave * RM_TOK_WAVE;

    for (int i = tid; i < EP; i += 256) sCnt[i] = 0;

    constexpr int WPIECES = EP * (RM_KC / 4);           // float4 pieces per chunk
    constexpr int WPER = (WPIECES + 255) / 256;
    // this thread's W pieces: row p/8 (clamped to E-1), column (p%8)*4
    const float *wrow[WPER];
    bool wok[WPER];
#pragma unroll
    for (int q = 0; q < WPER; ++q) {
        const int p = tid + q * 256;
        int row = p >> 3;
        wok[q] = p < WPIECES && row < E;
        row = row < E ? row : E - 1;
        wrow[q] = Wr + (int64_t)row * d + (p & 7) * 4;
    }
    const int64_t txr = (tw + col < T) ? tw + col : T - 1;
    const uint16_t *xrow = x + txr * d + 8 * kg;
    const bool tok_in = tw + col < T;

    auto load = [&](RStage<WPER> &st, int c) {
        const int k0 = c * RM_KC;
#pragma unroll
        for (int q = 0; q < WPER; ++q) {
            const int kc = k0 + ((tid + q * 256) & 7) * 4;
            st.w[q] = *reinterpret_cast<const float4 *>(wrow[q] + (kc < d ? k0 : 0));
        }
        st.xin = tok_in && (k0 + 8 * kg < d);
        st.x = ld16(xrow + (k0 + 8 * kg < d ? k0 : 0));
    };
    auto store_w = [&](const RStage<WPER> &st, int c) {
        const int k0 = c * RM_KC;
#pragma unroll
        for (int q = 0; q < WPER; ++q) {
            const int p = tid + q * 256;
            if (p < WPIECES) {
                const int row = p >> 3;
                const int c4 = (p & 7) * 4;
                const bool ok = wok[q] && (k0 + c4 < d);
                const float w[4] = {ok ? st.w[q].x : 0.f, ok ? st.w[q].y : 0.f,
                                    ok ? st.w[q].z : 0.f, ok ? st.w[q].w : 0.f};
                uint16_t h[4], m[4], l[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) split3(w[j], h[j], m[j], l[j]);
                const int o = row * RM_STRIDE + c4;
                uint2 vh, vm, vl;
                vh.x = h[0] | ((uint32_t)h[1] << 16); vh.y = h[2] | ((uint32_t)h[3] << 16);
                vm.x = m[0] | ((uint32_t)m[1] << 16); vm.y = m[2] | ((uint32_t)m[3] << 16);
                vl.x = l[0] | ((uint32_t)l[1] << 16); vl.y = l[2] | ((uint32_t)l[3] << 16);
                *reinterpret_cast<uint2 *>(&sW[0][o]) = vh;
                *reinterpret_cast<uint2 *>(&sW[1][o]) = vm;
                *reinterpret_cast<uint2 *>(&sW[2][o]) = vl;
            }
        }
    };

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int boff = col * RM_STRIDE + 8 * kg;
    auto compute = [&](const RStage<WPER> &st) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const bf16x8 a = as_bf16x8(st.xin ? st.x : z);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int o = nb * 16 * RM_STRIDE + boff;
            const bf16x8 bh = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sW[0][o]));
            const bf16x8 bm = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sW[1][o]));
            const bf16x8 bl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&sW[2][o]));
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc[nb], 0, 0, 0);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm, acc[nb], 0, 0, 0);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc[nb], 0, 0, 0);
        }
    };

    // ring of DEPTH register stages; chunk c lives in stage c % DEPTH
    const int nchunk = (d + RM_KC - 1) / RM_KC;
    RStage<WPER> st[DEPTH];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) load(st[s], s < nchunk ? s : nchunk - 1);
    auto step = [&](RStage<WPER> &cur, int c) {
        lds_barrier();                       // the previous chunk's MFMAs are done with sW
        store_w(cur, c);
        lds_barrier();
        compute(cur);
        const int cn = c + DEPTH;
        load(cur, cn < nchunk ? cn : nchunk - 1);
    };
    int c0 = 0;
    for (; c0 + DEPTH <= nchunk; c0 += DEPTH) {      // whole rounds: no exits inside
#pragma unroll
        for (int s = 0; s < DEPTH; ++s) step(st[s], c0 + s);
    }
#pragma unroll
    for (int s = 0; s < DEPTH - 1; ++s)              // the last nchunk % DEPTH chunks
        if (c0 + s < nchunk) step(st[s], c0 + s);

    // ---- epilogue: lane holds logits of tokens tw + 4*kg + i, experts nb*16 + col
    float bias[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int n = nb * 16 + col;
        bias[nb] = (br != nullptr && n < E) ? br[n] : 0.f;
    }
    float psum[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) psum[nb] = 0.f;

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = tw + 4 * kg + i;
        const bool tok_ok = t < T;
        float v[NB];
        float mx = -INFINITY;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = nb * 16 + col;
            float z = acc[nb][i] + bias[nb];
            if (z != z) z = -INFINITY;          // NaN ranks as -inf: indices stay in range
            v[nb] = z;
            if (n < E) mx = fmaxf(mx, z);
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
        float ex[NB];
        float s = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int n = nb * 16 + col;
            ex[nb] = (n < E) ? expf(v[nb] - mx) : 0.f;
            s += ex[nb];
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m);
        if (tok_ok) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) psum[nb] += ex[nb] / s;
        }

        // top-k by k rounds of a 16-lane argmax over the not-yet-chosen experts
        uint32_t excl[(NB + 31) / 32];
#pragma unroll
        for (int q = 0; q < (NB + 31) / 32; ++q) excl[q] = 0u;
        float vsel[MAXK];
        int isel[MAXK];
#pragma unroll
        for (int j = 0; j < MAXK; ++j) {
            vsel[j] = -INFINITY;
            isel[j] = 0;
            if (j < k) {
                Cand c{-INFINITY, 0x7fffffff, 0};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int n = nb * 16 + col;
                    const bool taken = (excl[nb >> 5] >> (nb & 31)) & 1u;
                    if (n < E && !taken) {
                        const Cand o{v[nb], n, 1};
                        if (cand_better(o, c)) c = o;
                    }
                }
#pragma unroll
                for (int m = 8; m >= 1; m >>= 1) {
                    const Cand o = cand_shfl_xor(c, m);
                    if (cand_better(o, c)) c = o;
                }
                if ((c.i & 15) == col) {
                    const int nbw = c.i >> 4;
                    excl[nbw >> 5] |= 1u << (nbw & 31);
                }
                vsel[j] = c.v;
                isel[j] = c.i;
            }
        }
        if (tok_ok && col == 0) {
            if (k == 1) {
                out_idx[t] = isel[0];
                out_gate[t] = 1.0f / s;        // p_{i*} = exp(0) / sum
                atomicAdd(&sCnt[isel[0]], 1);
            } else {
                float ek[MAXK];
                float sk = 0.f;
#pragma unroll
                for (int j = 0; j < MAXK; ++j) {
                    ek[j] = (j < k) ? expf(vsel[j] - vsel[0]) : 0.f;
                    sk += ek[j];
                }
#pragma unroll
                for (int j = 0; j < MAXK; ++j) {
                    if (j < k) {
                        out_idx[t * k + j] = isel[j];
                        out_gate[t * k + j] = ek[j] / sk;
                        atomicAdd(&sCnt[isel[j]], 1);
                    }
                }
            }
        }
    }

    // ---- block partials: probability sums and choice counts per expert
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        psum[nb] += __shfl_xor(psum[nb], 16);
        psum[nb] += __shfl_xor(psum[nb], 32);
    }
    if (lane < 16) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sProb[wave][nb * 16 + lane] = psum[nb];
    }
    __syncthreads();
    for (int n = tid; n < E; n += 256) {
        const float s = ((sProb[0][n] + sProb[1][n]) + sProb[2][n]) + sProb[3][n];
        part_prob[(int64_t)blockIdx.x * E + n] = s;
        part_cnt[(int64_t)blockIdx.x * E + n] = sCnt[n];
    }
}

// ---------------------------------------------------------------------------
// generic router (fp32 FMA): any dtype, any E <= 1024
// ---------------------------------------------------------------------------
constexpr int RG_TOK = 8;   // tokens per block, two rows per wave

template <bool BF16>
__global__ __launch_bounds__(256) void router_generic_kernel(
    const void *__restrict__ xv, const float *__restrict__ Wr, const float *__restrict__ br,
    int64_t T, int d, int E, int k, int32_t *__restrict__ out_idx, float *__restrict__ out_gate,
    float *__restrict__ part_prob, int32_t *__restrict__ part_cnt) {
    extern __shared__ float smem[];
    float *sZ = smem;                                   // [RG_TOK][E]
    int *sCnt = reinterpret_cast<int *>(smem + RG_TOK * E);   // [E]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * RG_TOK;

    for (int n = tid; n < E; n += 256) sCnt[n] = 0;
    for (int p = tid; p < RG_TOK * E; p += 256) {
        const int r = p / E;
        const int n = p - r * E;
        const int64_t t = t0 + r;
        float z = 0.f;
        if (t < T) {
            const float *w = Wr + (int64_t)n * d;
            if (BF16) {
                const uint16_t *xr = reinterpret_cast<const uint16_t *>(xv) + t * d;
                for (int q = 0; q < d; ++q) z = fmaf(bf2f(xr[q]), w[q], z);
            } else {
                const float *xr = reinterpret_cast<const float *>(xv) + t * d;
                for (int q = 0; q < d; ++q) z = fmaf(xr[q], w[q], z);
            }
            if (br != nullptr) z += br[n];
            if (z != z) z = -INFINITY;
        }
        sZ[p] = z;
    }
    __syncthreads();

    for (int rr = 0; rr < 2; ++rr) {
        const int r = wave * 2 + rr;
        const int64_t t = t0 + r;
        float *row = sZ + r * E;
        if (t < T) {
            float mx = -INFINITY;
            for (int n = lane; n < E; n += 64) mx = fmaxf(mx, row[n]);
            for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
            float s = 0.f;
            for (int n = lane; n < E; n += 64) s += expf(row[n] - mx);
            for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
            float vsel[MAXK];
            int isel[MAXK];
            for (int j = 0; j < MAXK; ++j) {
                vsel[j] = -INFINITY;
                isel[j] = 0;
                if (j < k) {
                    Cand c{-INFINITY, 0x7fffffff, 0};
                    for (int n = lane; n < E; n += 64) {
                        bool taken = false;
                        for (int q = 0; q < j; ++q) taken |= (isel[q] == n);
                        if (!taken) {
                            const Cand o{row[n], n, 1};
                            if (cand_better(o, c)) c = o;
                        }
                    }
                    for (int m = 32; m >= 1; m >>= 1) {
                        const Cand o = cand_shfl_xor(c, m);
                        if (cand_better(o, c)) c = o;
                    }
                    vsel[j] = c.v;
                    isel[j] = c.i;
                }
            }
            // probabilities replace the logits (after every lane has read them)
            __builtin_amdgcn_wave_barrier();
            for (int n = lane; n < E; n += 64) row[n] = expf(row[n] - mx) / s;
            if (lane == 0) {
                if (k == 1) {
                    out_idx[t] = isel[0];
                    out_gate[t] = 1.0f / s;
                    atomicAdd(&sCnt[isel[0]], 1);
                } else {
                    float ek[MAXK];
                    float sk = 0.f;
                    for (int j = 0; j < MAXK; ++j) {
                        ek[j] = (j < k) ? expf(vsel[j] - vsel[0]) : 0.f;
                        sk += ek[j];
                    }
                    for (int j = 0; j < k; ++j) {
                        out_idx[t * k + j] = isel[j];
                        out_gate[t * k + j] = ek[j] / sk;
                        atomicAdd(&sCnt[isel[j]], 1);
                    }
                }
            }
        } else {
            for (int n = lane; n < E; n += 64) row[n] = 0.f;
        }
    }
    __syncthreads();
    for (int n = tid; n < E; n += 256) {
        float s = 0.f;
        for (int r = 0; r < RG_TOK; ++r) s += sZ[r * E + n];
        part_prob[(int64_t)blockIdx.x * E + n] = s;
        part_cnt[(int64_t)blockIdx.x * E + n] = sCnt[n];
    }
}

// ---------------------------------------------------------------------------
// reduction of the block partials: one wave per expert, fixed order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_reduce_kernel(
    const float *__restrict__ part_prob, const int32_t *__restrict__ part_cnt, int nblk, int E,
    float *__restrict__ prob_sum, int32_t *__restrict__ route_count) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    double s = 0.0;
    long long c = 0;
    for (int b = lane; b < nblk; b += 64) {
        s += (double)part_prob[(int64_t)b * E + e];
        c += part_cnt[(int64_t)b * E + e];
    }
    for (int m = 32; m >= 1; m >>= 1) {
        s += __shfl_xor(s, m);
        c += __shfl_xor(c, m);
    }
    if (lane == 0) {
        prob_sum[e] = (float)s;
        route_count[e] = (int32_t)c;
    }
}

bool use_mfma(int dtype_bf16, int E) { return dtype_bf16 && E <= 256; }

}  // namespace

int router_blocks(int64_t T, int dtype_bf16, int E) {
    const int per = use_mfma(dtype_bf16, E) ? RM_TOK_BLOCK : RG_TOK;
    return (int)((T + per - 1) / per);
}

hipError_t launch_router(const void *x, int dtype_bf16, const float *W_r, const float *b_r,
                         int64_t T, int d, int E, int k, int32_t *expert_idx, float *gate,
                         float *part_prob, int32_t *part_cnt, hipStream_t s) {
    const int nblk = router_blocks(T, dtype_bf16, E);
    if (nblk == 0) return hipSuccess;
    if (use_mfma(dtype_bf16, E)) {
        const uint16_t *xb = reinterpret_cast<const uint16_t *>(x);
        const int nb = (E + 15) / 16;
#define MOE_ROUTER_CASE(NBV)                                                                  \
    if (nb <= NBV) {                                                                          \
        hipLaunchKernelGGL(router_mfma_kernel<NBV>, dim3(nblk), dim3(256), 0, s, xb, W_r, b_r, \
                           T, d, E, k, expert_idx, gate, part_prob, part_cnt);                \
        return hipGetLastError();                                                             \
    }
        MOE_ROUTER_CASE(1)
        MOE_ROUTER_CASE(2)
        MOE_ROUTER_CASE(4)
        MOE_ROUTER_CASE(8)
        MOE_ROUTER_CASE(16)
#undef MOE_ROUTER_CASE
        return hipErrorInvalidValue;
    }
    const size_t shm = (size_t)(RG_TOK + 1) * E * sizeof(float);
    if (dtype_bf16)
        hipLaunchKernelGGL(router_generic_kernel<true>, dim3(nblk), dim3(256), shm, s, x, W_r,
                           b_r, T, d, E, k, expert_idx, gate, part_prob, part_cnt);
    else
        hipLaunchKernelGGL(router_generic_kernel<false>, dim3(nblk), dim3(256), shm, s, x, W_r,
                           b_r, T, d, E, k, expert_idx, gate, part_prob, part_cnt);
    return hipGetLastError();
}

hipError_t launch_router_reduce(const float *part_prob, const int32_t *part_cnt, int nblk,
                                int E, float *prob_sum, int32_t *route_count, hipStream_t s) {
    hipLaunchKernelGGL(router_reduce_kernel, dim3((E + 3) / 4), dim3(256), 0, s, part_prob,
                       part_cnt, nblk, E, prob_sum, route_count);
    return hipGetLastError();
}

}  // namespace moe
