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

constexpr int MAX_E_LDS = 1024;

// Which tile this block computes (tile_map staged in LDS).  Returns false if none.
// Order: expert-major, then column tile, then row tile; block b of XCD b % 8
// takes the (b / 8)-th tile of that XCD's contiguous share.
__device__ __forceinline__ bool map_tile(const int32_t *__restrict__ tile_map, int E, int tiles_n,
                                         int *s_map, int &e, int &mt, int &nt) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_map[i] = tile_map[i];
    __syncthreads();
    const int total = s_map[E] * tiles_n;
    const int per_xcd = (total + 7) >> 3;
    const int b = blockIdx.x;
    const int slot = b >> 3;
    if (slot >= per_xcd) return false;
    const int L = (b & 7) * per_xcd + slot;
    if (L >= total) return false;
    int lo = 0, hi = E - 1;           // largest e with s_map[e] * tiles_n <= L
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_map[mid] * tiles_n <= L) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int r = L - s_map[e] * tiles_n;
    const int mtiles = s_map[e + 1] - s_map[e];
    nt = r / mtiles;
    mt = r - nt * mtiles;
    return true;
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

// Tile shape: block BM x BN, K step 64; 4 waves in a 2 x 2 grid, each wave
// (BM/2) x (BN/2) = FM x FN 32x32 MFMA fragments (v_mfma_f32_32x32x16_bf16:
// on gfx950 one wave per SIMD keeps it issuing at nearly the full rate,
// which the 16x16x32 form does not reach).  LDS rows are 64 bf16 =
// 128 bytes = 8 pieces of 16 bytes; piece c of row r is stored at position
// c ^ (r % 8), so the 16 rows of a fragment read and the 8 rows of a staging
// write each touch every bank group once, with no padding.
template <int BM_, int BN_, int MINB_ = 1>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = 64;
    static constexpr int MINB = MINB_;                  // blocks per CU the registers are sized for
    static constexpr int FM = BM / 64, FN = BN / 64;    // 32x32 fragments per wave
    static constexpr int LA = BM * 8 / 256;             // 16-byte A pieces per thread per K tile
    static constexpr int LB = BN * 8 / 256;             // 16-byte B pieces per thread per K tile
    static constexpr int OUT_STRIDE = BN + 8;           // staged output row (bf16 elements)
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
    // element offset of logical piece c of row r
    static __device__ __forceinline__ int off(int r, int c) { return r * 64 + ((c ^ (r & 7)) << 3); }
};

// Register stage of one K tile: this thread's 16-byte pieces of A, B (and B3).
template <int LA, int LB, bool DUAL>
struct Stage {
    u32x4 a[LA];
    u32x4 b[LB];
    u32x4 b3[DUAL ? LB : 1];
    bool in;          // false: these columns lie past K and are stored as zeros
};

template <class TL, int ACT, bool BIAS, bool KTAIL>
__global__ __launch_bounds__(256, TL::MINB) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, const uint16_t *__restrict__ B3,
    const uint16_t *__restrict__ bias, const int32_t *__restrict__ count,
    const int32_t *__restrict__ tile_map, int E, int64_t C, int N, int K, int tiles_n,
    uint16_t *__restrict__ out) {
    constexpr int BM = TL::BM, BN = TL::BN;
    constexpr int LA = TL::LA, LB = TL::LB, FM = TL::FM, FN = TL::FN;
    constexpr bool DUAL = (ACT == 2);
    constexpr int NBT = DUAL ? 2 : 1;                    // weight tiles per stage
    constexpr int STAGE_ELEMS = (BM + NBT * BN) * 64;
    constexpr int OUT_ELEMS = BM * TL::OUT_STRIDE;
    constexpr int SMEM_ELEMS = 2 * STAGE_ELEMS > OUT_ELEMS ? 2 * STAGE_ELEMS : OUT_ELEMS;
    // two LDS stages of [A | B | B3] tiles; reused for the output tile at the end
    __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM_ELEMS];
    __shared__ int s_map[MAX_E_LDS + 1];

    int e, mt, nt;
    if (!map_tile(tile_map, E, tiles_n, s_map, e, mt, nt)) return;
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
    const int64_t b3off = DUAL ? (int64_t)(B3 - B) : 0;

    // staging: piece q = tid + i*256 -> row q / 8, logical piece q % 8 (rows past
    // the count / past N read a valid row whose result is discarded)
    const int pc = tid & 7;
    const uint16_t *pa[LA];
    const uint16_t *pb[LB];
    int soa[LA], sob[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int r = (tid >> 3) + i * 32;
        int am = m0 + r;
        am = am < cnt ? am : cnt - 1;
        pa[i] = Ae + (int64_t)am * K + pc * 8;
        soa[i] = TL::off(r, pc);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int r = (tid >> 3) + i * 32;
        int bn = n0 + r;
        bn = bn < N ? bn : N - 1;
        pb[i] = Be + (int64_t)bn * K + pc * 8;
        sob[i] = TL::off(r, pc);
    }

    using St = Stage<LA, LB, DUAL>;
    // loads of K tile kt.  With KTAIL (K not a multiple of 64) pieces past K
    // are read from column 0 and zeroed when stored (a select at load time
    // would make the wave wait for the load right away).
    auto gload = [&](St &st, int kt) {
        int kk = kt * 64;
        if (KTAIL) {
            st.in = kk + pc * 8 < K;
            kk = st.in ? kk : -pc * 8;
        }
#pragma unroll
        for (int i = 0; i < LA; ++i) st.a[i] = ld16(pa[i] + kk);
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            st.b[i] = ld16(pb[i] + kk);
            if (DUAL) st.b3[i] = ld16(pb[i] + b3off + kk);
        }
        __builtin_amdgcn_sched_barrier(0);     // issue the loads here, ahead of the MFMAs
    };
    auto sstore = [&](const St &st, int buf) {
        uint16_t *sa = smem + buf * STAGE_ELEMS;
        uint16_t *sb = sa + BM * 64;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const bool in = KTAIL ? st.in : true;
#pragma unroll
        for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4 *>(sa + soa[i]) = in ? st.a[i] : z;
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            *reinterpret_cast<u32x4 *>(sb + sob[i]) = in ? st.b[i] : z;
            if (DUAL) *reinterpret_cast<u32x4 *>(sb + BN * 64 + sob[i]) = in ? st.b3[i] : z;
        }
    };

    // accumulators hold C^T fragments: acc[i][j] = W rows (n) x X rows (m); lane
    // l holds output row m = l % 32 of the fragment and, for g = 0..3, the four
    // consecutive columns n = 8g + 4 (l / 32) + 0..3 in elements 4g .. 4g+3
    f32x16 acc[FM][FN];
    f32x16 acc3[DUAL ? FM : 1][DUAL ? FN : 1];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
#pragma unroll
    for (int i = 0; i < (DUAL ? FM : 1); ++i)
#pragma unroll
        for (int j = 0; j < (DUAL ? FN : 1); ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc3[i][j][q] = 0.f;

    // fragment reads (32x16 operands): row (base + lane%32), logical piece
    // 2 ks + lane/32; the fragment bases are multiples of 32, so the stored
    // piece is piece ^ (lane % 8)
    const int arow = (wm * (BM / 2) + (lane & 31)) * 64;
    const int brow = (wn * (BN / 2) + (lane & 31)) * 64;
    auto compute = [&](int buf) {
        const uint16_t *sa = smem + buf * STAGE_ELEMS;
        const uint16_t *sb = sa + BM * 64;
        // every fragment of the K tile is read first, into its own registers, so
        // the reads of later 16-wide k steps overlap the MFMAs of earlier ones
        bf16x8 af[4][FM], bfr[4][FN], bf3[DUAL ? 4 : 1][DUAL ? FN : 1];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int pofs = ((ks * 2 + (lane >> 5)) ^ (lane & 7)) << 3;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[ks][i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sa + arow + i * 32 * 64 + pofs));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[ks][j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + brow + j * 32 * 64 + pofs));
            if (DUAL) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bf3[DUAL ? ks : 0][DUAL ? j : 0] =
                        as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + BN * 64 + brow + j * 32 * 64 + pofs));
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks][j], af[ks][i], acc[i][j], 0, 0, 0);
            if (DUAL) {
#pragma unroll
                for (int i = 0; i < (DUAL ? FM : 1); ++i)
#pragma unroll
                    for (int j = 0; j < (DUAL ? FN : 1); ++j)
                        acc3[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf3[DUAL ? ks : 0][j], af[ks][i],
                                                                             acc3[i][j], 0, 0, 0);
            }
        }
    };

    // ---- pipeline: K tile kt is loaded into registers three steps ahead, stored
    // into LDS buffer kt % 2 one step ahead and consumed at step kt.  Register
    // stage r holds tiles r, r+3, ...; the steady-state loop (six steps, no
    // conditional memory operations) only waits for a load when its stage is
    // stored to LDS, two compute steps after the loads were issued.
    const int nk = (K + 63) >> 6;
    St r0, r1, r2;
    gload(r0, 0);
    if (nk > 1) gload(r1, 1);
    if (nk > 2) gload(r2, 2);
    sstore(r0, 0);
    __syncthreads();
#define MOE_STEP(KT, RFREE, RNEXT, CUR, NXT, LOAD)              \
    do {                                                       \
        if (LOAD) gload(RFREE, (KT) + 3);                      \
        compute(CUR);                                          \
        if ((KT) + 1 < nk) sstore(RNEXT, NXT);                 \
        __syncthreads();                                       \
    } while (0)
    int kt = 0;
    for (; kt + 9 <= nk; kt += 6) {
        MOE_STEP(kt + 0, r0, r1, 0, 1, true);
        MOE_STEP(kt + 1, r1, r2, 1, 0, true);
        MOE_STEP(kt + 2, r2, r0, 0, 1, true);
        MOE_STEP(kt + 3, r0, r1, 1, 0, true);
        MOE_STEP(kt + 4, r1, r2, 0, 1, true);
        MOE_STEP(kt + 5, r2, r0, 1, 0, true);
    }
    // tail: at most 8 steps, loads only while tiles remain
#define MOE_TAIL(S, RF, RN, CB, NB)                                       \
    if (kt + (S) < nk) MOE_STEP(kt + (S), RF, RN, CB, NB, kt + (S) + 3 < nk);
    MOE_TAIL(0, r0, r1, 0, 1)
    MOE_TAIL(1, r1, r2, 1, 0)
    MOE_TAIL(2, r2, r0, 0, 1)
    MOE_TAIL(3, r0, r1, 1, 0)
    MOE_TAIL(4, r1, r2, 0, 1)
    MOE_TAIL(5, r2, r0, 1, 0)
    MOE_TAIL(6, r0, r1, 0, 1)
    MOE_TAIL(7, r1, r2, 1, 0)
#undef MOE_TAIL
#undef MOE_STEP

    // ---- epilogue: bias, activation, bf16, staged through LDS
    constexpr int OS = TL::OUT_STRIDE;
    uint16_t *so = smem;    // [BM][OUT_STRIDE]; every wave is past its last LDS read
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int nl = wn * (BN / 2) + j * 32 + 8 * g + 4 * (lane >> 5);   // 4 consecutive columns
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (BIAS) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = n0 + nl + r;
                    bv[r] = (n < N) ? bf2f(bias[(int64_t)e * N + n]) : 0.f;
                }
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int ml = wm * (BM / 2) + i * 32 + (lane & 31);
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float t = acc[i][j][4 * g + r] + bv[r];
                    if (ACT == 1) t = fmaxf(t, 0.f);
                    if (ACT == 2) t = silu(t) * acc3[DUAL ? i : 0][DUAL ? j : 0][4 * g + r];
                    v[r] = t;
                }
                uint2 pk;
                pk.x = pack_bf16x2(v[0], v[1]);
                pk.y = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2 *>(so + ml * OS + nl) = pk;
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
            st16(oe + (int64_t)m * N + n, *reinterpret_cast<const u32x4 *>(so + r * OS + c));
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
    __shared__ int s_map[MAX_E_LDS + 1];

    int e, mt, nt;
    if (!map_tile(tile_map, E, tiles_n, s_map, e, mt, nt)) return;
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

// The tile shapes of the bf16 path: one BM for both expert GEMMs, so they share
// one tile map. The gated (two-matrix) variant holds twice the accumulators and
// runs one block per CU; the others fit two.
using TileBF16 = Tile<128, 128, 2>;
using TileBF16Gated = Tile<128, 128, 1>;
static_assert(TileBF16::BM == TileBF16Gated::BM && TileBF16::BN == TileBF16Gated::BN, "one tile map");

int gemm_bm(int dtype_bf16) { return dtype_bf16 ? TileBF16::BM : FBM; }

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
        const int tiles_n = (N + TileBF16::BN - 1) / TileBF16::BN;
        const dim3 grid((unsigned)grid_for(C, E, TileBF16::BM, tiles_n, rows_bound));
        const uint16_t *a = (const uint16_t *)A, *b = (const uint16_t *)B, *b3 = (const uint16_t *)B3,
                       *bi = (const uint16_t *)bias;
        uint16_t *o = (uint16_t *)out;
#define MOE_GEMM(TL, ACTV, BIASV)                                                              \
    do {                                                                                       \
        if (K % 64 == 0)                                                                       \
            hipLaunchKernelGGL((gemm_bf16_kernel<TL, ACTV, BIASV, false>), grid, dim3(256), 0, s, \
                               a, b, b3, bi, expert_count, tile_map, E, C, N, K, tiles_n, o);   \
        else                                                                                   \
            hipLaunchKernelGGL((gemm_bf16_kernel<TL, ACTV, BIASV, true>), grid, dim3(256), 0, s, \
                               a, b, b3, bi, expert_count, tile_map, E, C, N, K, tiles_n, o);   \
    } while (0)
        if (act == 0) { if (bias) MOE_GEMM(TileBF16, 0, true); else MOE_GEMM(TileBF16, 0, false); }
        else if (act == 1) { if (bias) MOE_GEMM(TileBF16, 1, true); else MOE_GEMM(TileBF16, 1, false); }
        else MOE_GEMM(TileBF16Gated, 2, false);
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
