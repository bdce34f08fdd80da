// Grouped GEMM of the experts: for every expert e and every kept row m < count[e]
//   out[e, m, n] = act( sum_k A[e, m, k] * B[e, n, k] (+ bias[e, n]) )
// with act = none, ReLU, or SwiGLU (silu(A B^T) * (A B3^T)).
//
// [SW-GLaM] "Dense Scaling 与 MoE 的核心差异": FFN(x) = W_2 sigma(W_1 x);
// [CMU-L16] section 2.1 (biases b, c) and 2.3 (SwiGLU expert, Swish beta = 1);
// [CMU-L16] section 5 / [CS25-L5] "Switch Layer": experts run as batched
// matrix products over their slot lists (a dedicated grouped-GEMM kernel).
//
// bf16 path (gfx950 MFMA v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   * 256 threads = 4 waves in a 2x2 grid; block tile 128 x 128 x 64, each
//     wave 64 x 64 = 4 x 4 MFMA tiles (two 16x16 accumulators sets for SwiGLU).
//   * A and B tiles are K-contiguous in HBM (x rows, nn.Linear-style weight
//     rows), so both are staged through LDS the same way: 16-byte global
//     loads into registers one K step ahead, stores into the other half of a
//     double-buffered, row-padded LDS tile (conflict-free 16-byte reads).
//   * Only real row tiles are launched work: tile_map holds the prefix sums
//     of ceil(count[e] / 128), read on the device, so an expert with few
//     rows costs few tiles and an empty expert none.
//   * Tile order is expert-major, then column tile, then row tile, so the
//     row tiles that share a weight tile run next to each other; the block
//     index is remapped so that each XCD (blocks are dealt to the 8 XCDs
//     round-robin) gets one contiguous range of that order and its own L2
//     keeps the weight and activation tiles it reuses.
//   * The epilogue adds the bias, applies the activation, rounds to bf16 and
//     stages the tile in LDS so that rows go out as coalesced 16-byte stores.
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 x 16 tiles).
#include "common.h"
#include "launch.h"

#include <math.h>

namespace moe {

namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDSK = BK + 8;          // padded row, bf16 elements (144 bytes)
constexpr int LOADS = (BM * BK / 8) / 256;   // 16-byte pieces per thread per tile = 4
constexpr int OUT_STRIDE = BN + 8;    // staged output row, bf16 elements

// Which tile this block computes.  Returns false if there is none.
__device__ __forceinline__ bool map_tile(const int32_t *__restrict__ tile_map, int E, int tiles_n,
                                         int &e, int &mt, int &nt) {
    const int total_m = tile_map[E];
    const int total = total_m * tiles_n;
    const int per_xcd = (total + 7) >> 3;
    const int b = blockIdx.x;
    const int slot = b >> 3;
    if (slot >= per_xcd) return false;
    const int L = (b & 7) * per_xcd + slot;
    if (L >= total) return false;
    // largest e with tile_map[e] * tiles_n <= L
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_map[mid] * tiles_n <= L) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int r = L - tile_map[e] * tiles_n;
    const int mtiles = tile_map[e + 1] - tile_map[e];
    nt = r / mtiles;
    mt = r - nt * mtiles;
    return true;
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

template <int ACT, bool BIAS>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, const uint16_t *__restrict__ B3,
    const uint16_t *__restrict__ bias, const int32_t *__restrict__ count,
    const int32_t *__restrict__ tile_map, int E, int64_t C, int N, int K, int tiles_n,
    uint16_t *__restrict__ out) {
    constexpr bool DUAL = (ACT == 2);
    constexpr int NBUF_B = DUAL ? 2 : 1;
    // [buffer][A | B | B3] tiles
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (1 + NBUF_B) * BM * LDSK];

    int e, mt, nt;
    if (!map_tile(tile_map, E, tiles_n, e, mt, nt)) return;
    const int cnt = count[e];
    const int m0 = mt * BM;
    const int n0 = nt * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    const uint16_t *Ae = A + (int64_t)e * C * K;
    const uint16_t *Be = B + (int64_t)e * N * K;
    const uint16_t *B3e = DUAL ? B3 + (int64_t)e * N * K : nullptr;

    // global -> register staging: piece q = tid + i*256, row q/8, column (q%8)*8
    const uint16_t *pa[LOADS];
    const uint16_t *pb[LOADS];
    const uint16_t *pb3[LOADS];
    int soff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int q = tid + i * 256;
        const int r = q >> 3;
        const int c = (q & 7) * 8;
        int am = m0 + r;
        if (am > cnt - 1) am = cnt - 1;                 // rows past the count: any valid row
        int bn = n0 + r;
        if (bn > N - 1) bn = N - 1;
        pa[i] = Ae + (int64_t)am * K + c;
        pb[i] = Be + (int64_t)bn * K + c;
        pb3[i] = DUAL ? B3e + (int64_t)bn * K + c : nullptr;
        soff[i] = r * LDSK + c;
    }
    u32x4 ra[LOADS], rb[LOADS], rb3[LOADS];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int c = ((tid + i * 256) & 7) * 8;
            const bool in = (k0 + c) < K;
            const u32x4 z = {0u, 0u, 0u, 0u};
            ra[i] = in ? ld16(pa[i] + k0) : z;
            rb[i] = in ? ld16(pb[i] + k0) : z;
            if (DUAL) rb3[i] = in ? ld16(pb3[i] + k0) : z;
        }
    };
    auto sstore = [&](int buf) {
        uint16_t *sa = smem + buf * (1 + NBUF_B) * BM * LDSK;
        uint16_t *sb = sa + BM * LDSK;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            *reinterpret_cast<u32x4 *>(sa + soff[i]) = ra[i];
            *reinterpret_cast<u32x4 *>(sb + soff[i]) = rb[i];
            if (DUAL) *reinterpret_cast<u32x4 *>(sb + BM * LDSK + soff[i]) = rb3[i];
        }
    };

    f32x4 acc[4][4];
    f32x4 acc3[DUAL ? 4 : 1][DUAL ? 4 : 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (DUAL) {
#pragma unroll
        for (int i = 0; i < (DUAL ? 4 : 1); ++i)
#pragma unroll
            for (int j = 0; j < (DUAL ? 4 : 1); ++j) acc3[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int arow = (wm * 64 + (lane & 15)) * LDSK + 8 * (lane >> 4);
    const int brow = (wn * 64 + (lane & 15)) * LDSK + 8 * (lane >> 4);
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const uint16_t *sa = smem + (kt & 1) * (1 + NBUF_B) * BM * LDSK;
        const uint16_t *sb = sa + BM * LDSK;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sa + arow + i * 16 * LDSK + ks * 32));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + brow + j * 16 * LDSK + ks * 32));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            if (DUAL) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + BM * LDSK + brow + j * 16 * LDSK + ks * 32));
#pragma unroll
                for (int i = 0; i < (DUAL ? 4 : 1); ++i)
#pragma unroll
                    for (int j = 0; j < (DUAL ? 4 : 1); ++j)
                        acc3[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc3[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) sstore((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: bias, activation, bf16, staged through LDS
    uint16_t *so = smem;   // [BM][OUT_STRIDE]; every wave is past its last LDS read
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int nl = wn * 64 + j * 16 + (lane & 15);
        const int n = n0 + nl;
        float bv = 0.f;
        if (BIAS && n < N) bv = bf2f(bias[(int64_t)e * N + n]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ml = wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                float v = acc[i][j][r] + bv;
                if (ACT == 1) v = fmaxf(v, 0.f);
                if (ACT == 2) v = silu(v) * acc3[DUAL ? i : 0][DUAL ? j : 0][r];
                so[ml * OUT_STRIDE + nl] = f2bf(v);
            }
        }
    }
    __syncthreads();
    uint16_t *oe = out + (int64_t)e * C * N;
    constexpr int PIECES = BM * BN / 8;
#pragma unroll
    for (int q = tid; q < PIECES; q += 256) {
        const int r = q / (BN / 8);
        const int c = (q % (BN / 8)) * 8;
        const int m = m0 + r;
        const int n = n0 + c;
        if (m < cnt && n < N)
            st16(oe + (int64_t)m * N + n, *reinterpret_cast<const u32x4 *>(so + r * OUT_STRIDE + c));
    }
}

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 16;

template <int ACT, bool BIAS>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float *__restrict__ A, const float *__restrict__ B, const float *__restrict__ B3,
    const float *__restrict__ bias, const int32_t *__restrict__ count,
    const int32_t *__restrict__ tile_map, int E, int64_t C, int N, int K, int tiles_n,
    float *__restrict__ out) {
    constexpr bool DUAL = (ACT == 2);
    __shared__ float sA[FBK][FBM + 1];
    __shared__ float sB[FBK][FBN + 1];
    __shared__ float sB3[DUAL ? FBK : 1][FBN + 1];

    int e, mt, nt;
    if (!map_tile(tile_map, E, tiles_n, e, mt, nt)) return;
    const int cnt = count[e];
    const int m0 = mt * FBM;
    const int n0 = nt * FBN;
    const int tid = threadIdx.x;
    const int tm = (tid >> 4) * 4;     // 4 rows
    const int tn = (tid & 15) * 4;     // 4 columns
    const float *Ae = A + (int64_t)e * C * K;
    const float *Be = B + (int64_t)e * N * K;
    const float *B3e = DUAL ? B3 + (int64_t)e * N * K : nullptr;

    float acc[4][4] = {};
    float acc3[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += FBK) {
        for (int q = tid; q < FBM * FBK; q += 256) {
            const int r = q / FBK, c = q % FBK;
            int am = m0 + r;
            if (am > cnt - 1) am = cnt - 1;
            int bn = n0 + r;
            if (bn > N - 1) bn = N - 1;
            const bool in = k0 + c < K;
            sA[c][r] = in ? Ae[(int64_t)am * K + k0 + c] : 0.f;
            sB[c][r] = in ? Be[(int64_t)bn * K + k0 + c] : 0.f;
            if (DUAL) sB3[c][r] = in ? B3e[(int64_t)bn * K + k0 + c] : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < FBK; ++kk) {
            float a[4], b[4], b3[4];
            for (int i = 0; i < 4; ++i) a[i] = sA[kk][tm + i];
            for (int j = 0; j < 4; ++j) b[j] = sB[kk][tn + j];
            if (DUAL) for (int j = 0; j < 4; ++j) b3[j] = sB3[kk][tn + j];
            for (int i = 0; i < 4; ++i)
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
                    if (DUAL) acc3[i][j] = fmaf(a[i], b3[j], acc3[i][j]);
                }
        }
        __syncthreads();
    }
    float *oe = out + (int64_t)e * C * N;
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + tm + i;
        if (m >= cnt) continue;
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tn + j;
            if (n >= N) continue;
            float v = acc[i][j];
            if (BIAS) v += bias[(int64_t)e * N + n];
            if (ACT == 1) v = fmaxf(v, 0.f);
            if (ACT == 2) v = silu(v) * acc3[i][j];
            oe[(int64_t)m * N + n] = v;
        }
    }
}

// tile_map[0] = 0, tile_map[e+1] = sum_{e' <= e} ceil(count[e'] / bm); one block
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t *__restrict__ count, int E, int bm,
                                                        int32_t *__restrict__ tile_map) {
    __shared__ int s[1024];
    const int t = threadIdx.x;
    s[t] = (t < E) ? (count[t] + bm - 1) / bm : 0;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = (t >= off) ? s[t - off] : 0;
        __syncthreads();
        s[t] += v;
        __syncthreads();
    }
    if (t < E) tile_map[t + 1] = s[t];
    if (t == 0) tile_map[0] = 0;
}

// Blocks for at most E * ceil(C / bm) row tiles, and at most
// ceil(rows_bound / bm) + E of them (each expert wastes at most one partial tile).
int64_t grid_for(int64_t C, int E, int bm, int tiles_n, int64_t rows_bound) {
    int64_t m = (int64_t)E * ((C + bm - 1) / bm);
    const int64_t m2 = (rows_bound + bm - 1) / bm + E;
    if (m2 < m) m = m2;
    const int64_t g = m * tiles_n;
    return ((g + 7) / 8) * 8;
}

}  // namespace

int gemm_bm(int dtype_bf16) { return dtype_bf16 ? BM : FBM; }

hipError_t launch_tile_map(const int32_t *expert_count, int E, int bm, int32_t *tile_map,
                           hipStream_t s) {
    hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(1024), 0, s, expert_count, E, bm, tile_map);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const void *A, const void *B, const void *B3, const void *bias,
                               int dtype_bf16, int act, const int32_t *expert_count,
                               const int32_t *tile_map, int E, int64_t C, int N, int K,
                               int64_t rows_bound, void *out, hipStream_t s) {
    if (C == 0 || rows_bound == 0) return hipSuccess;
    if (dtype_bf16) {
        const int tiles_n = (N + BN - 1) / BN;
        const dim3 grid((unsigned)grid_for(C, E, BM, tiles_n, rows_bound));
        const uint16_t *a = (const uint16_t *)A, *b = (const uint16_t *)B, *b3 = (const uint16_t *)B3,
                       *bi = (const uint16_t *)bias;
        uint16_t *o = (uint16_t *)out;
#define MOE_GEMM(ACTV, BIASV)                                                                  \
    hipLaunchKernelGGL((gemm_bf16_kernel<ACTV, BIASV>), grid, dim3(256), 0, s, a, b, b3, bi,   \
                       expert_count, tile_map, E, C, N, K, tiles_n, o)
        if (act == 0) { if (bias) MOE_GEMM(0, true); else MOE_GEMM(0, false); }
        else if (act == 1) { if (bias) MOE_GEMM(1, true); else MOE_GEMM(1, false); }
        else MOE_GEMM(2, false);
#undef MOE_GEMM
    } else {
        const int tiles_n = (N + FBN - 1) / FBN;
        const dim3 grid((unsigned)grid_for(C, E, FBM, tiles_n, rows_bound));
        const float *a = (const float *)A, *b = (const float *)B, *b3 = (const float *)B3,
                    *bi = (const float *)bias;
        float *o = (float *)out;
#define MOE_GEMM(ACTV, BIASV)                                                                 \
    hipLaunchKernelGGL((gemm_f32_kernel<ACTV, BIASV>), grid, dim3(256), 0, s, a, b, b3, bi,   \
                       expert_count, tile_map, E, C, N, K, tiles_n, o)
        if (act == 0) { if (bias) MOE_GEMM(0, true); else MOE_GEMM(0, false); }
        else if (act == 1) { if (bias) MOE_GEMM(1, true); else MOE_GEMM(1, false); }
        else MOE_GEMM(2, false);
#undef MOE_GEMM
    }
    return hipGetLastError();
}

}  // namespace moe
