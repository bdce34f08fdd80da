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

#define MOE_LDS_AS __attribute__((address_space(3)))
#define MOE_GLB_AS __attribute__((address_space(1)))

// s_waitcnt with vmcnt = V and lgkmcnt = 0 (expcnt left alone), gfx9 encoding.
template <int V>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Tile shape: block BM x BN, K step 64, STAGES-deep LDS ring; 4 waves in a
// 2 x 2 grid, each wave (BM/2) x (BN/2) = FM x FN MFMA 16x16 fragments.
// LDS rows are 64 bf16 = 128 bytes = 8 pieces of 16 bytes; piece c of row r
// is stored at position c ^ (r % 8), so the 16 rows of a fragment read and
// the 8 rows of a DMA write each touch every bank group once.
template <int BM_, int BN_, int STAGES_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = 64, STAGES = STAGES_;
    static constexpr int FM = BM / 32, FN = BN / 32;    // 16x16 fragments per wave
    static constexpr int AI = BM / 32, BI = BN / 32;    // DMA instructions per wave per stage
    static constexpr int OUT_STRIDE = BN + 8;           // staged output row (bf16 elements)
    static_assert(BM % 32 == 0 && BN % 32 == 0, "tile");
};

// Persistent grouped GEMM.  Each block walks a list of output tiles; the
// K tiles of all its output tiles form one stream that flows through a
// three-stage LDS ring filled by 16-byte DMA (global_load_lds), so the loads
// of the next output tile overlap the MFMAs of the current one.
template <class TL, int ACT, bool BIAS>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, const uint16_t *__restrict__ B3,
    const uint16_t *__restrict__ bias, const int32_t *__restrict__ count,
    const int32_t *__restrict__ tile_map, int E, int64_t C, int N, int K, int tiles_n,
    uint16_t *__restrict__ out) {
    constexpr int BM = TL::BM, BN = TL::BN, S = TL::STAGES;
    constexpr int FM = TL::FM, FN = TL::FN, AI = TL::AI, BI = TL::BI;
    constexpr bool DUAL = (ACT == 2);
    constexpr int NBT = DUAL ? 2 : 1;                    // weight tiles per stage
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
    constexpr int STAGE_BYTES = A_BYTES + NBT * B_BYTES;
    constexpr int PER = AI + NBT * BI;                   // DMA instructions per wave per stage
    static_assert(S == 3, "the ring below is written out for three stages");
    // one LDS array per stage: the compiler then sees that reads of one stage
    // cannot alias the DMA in flight into another and adds no wait of its own
    __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE_BYTES];
    __shared__ int s_map[MAX_E_LDS + 1];
    __shared__ int s_cnt[MAX_E_LDS];

    for (int i = threadIdx.x; i <= E; i += blockDim.x) {
        s_map[i] = tile_map[i];
        if (i < E) s_cnt[i] = count[i];
    }
    __syncthreads();

    // this block's output tiles: its XCD (blocks are dealt to the 8 XCDs
    // round-robin) owns one contiguous share of the tile order, and the
    // XCD's blocks take that share's tiles in turn
    const int total = s_map[E] * tiles_n;
    const int per_xcd_blocks = gridDim.x >> 3;
    const int share = (total + 7) >> 3;
    const int lo = (blockIdx.x & 7) * share + (blockIdx.x >> 3);
    const int hi = min(total, ((blockIdx.x & 7) + 1) * share);
    if (lo >= hi) return;
    const int my_tiles = (hi - lo + per_xcd_blocks - 1) / per_xcd_blocks;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (LDS DMA base)
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int64_t b3off = DUAL ? (int64_t)(B3 - B) : 0;

    // tile index -> (expert, first row, first column)
    auto locate = [&](int lt, int &e, int &m0, int &n0) {
        const int L = lo + lt * per_xcd_blocks;
        int a = 0, b = E - 1;                           // largest e with s_map[e] * tiles_n <= L
        while (a < b) {
            const int mid = (a + b + 1) >> 1;
            if (s_map[mid] * tiles_n <= L) a = mid; else b = mid - 1;
        }
        e = a;
        const int r = L - s_map[e] * tiles_n;
        const int mtiles = s_map[e + 1] - s_map[e];
        const int nt = r / mtiles;
        m0 = (r - nt * mtiles) * BM;
        n0 = nt * BN;
    };

    // DMA sources of the tile being loaded: wave instruction i fills LDS rows
    // [8 (wave*AI + i), +8); lane l lands at position l of that 1 KB block =
    // row l/8, piece l%8, which holds logical piece (l%8) ^ (l/8) of the row
    // (rows past the count / past N read a valid row whose result is dropped)
    const int lr = lane >> 3;
    const int lc = (lane & 7) ^ lr;
    const uint16_t *asrc[AI];
    const uint16_t *bsrc[BI];
    auto point = [&](int lt) {
        int e, m0, n0;
        locate(lt, e, m0, n0);
        const int cnt = s_cnt[e];
        const uint16_t *Ae = A + (int64_t)e * C * K;
        const uint16_t *Be = B + (int64_t)e * N * K;
#pragma unroll
        for (int i = 0; i < AI; ++i) {
            int am = m0 + (wave * AI + i) * 8 + lr;
            am = am < cnt ? am : cnt - 1;
            asrc[i] = Ae + (int64_t)am * K + lc * 8;
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            int bn = n0 + (wave * BI + j) * 8 + lr;
            bn = bn < N ? bn : N - 1;
            bsrc[j] = Be + (int64_t)bn * K + lc * 8;
        }
    };

    const int nk = (K + 63) >> 6;                       // K tiles per output tile
    const int steps = my_tiles * nk;
    // the last K tile of a tile with K % 64 != 0: pieces past K are cleared
    // in LDS after their DMA has landed (they were loaded from column 0)
    const bool ktail = (K & 63) != 0;
    const bool tail_piece = ktail && ((nk - 1) * 64 + lc * 8 >= K);

    // loads of step g (steps are issued in order; a tile's first K tile sets
    // up that tile's sources)
    auto issue = [&](uint8_t *base, int g) {
        g = g < steps ? g : steps - 1;                  // past the end: reload the last step
        const int lt = g / nk;
        const int kt = g - lt * nk;
        if (kt == 0) point(lt);
        const int k0 = (ktail && kt == nk - 1 && tail_piece) ? -lc * 8 : kt * 64;
#pragma unroll
        for (int i = 0; i < AI; ++i)
            __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)(asrc[i] + k0),
                                             (MOE_LDS_AS void *)(base + (wave * AI + i) * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < BI; ++j)
            __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)(bsrc[j] + k0),
                                             (MOE_LDS_AS void *)(base + A_BYTES + (wave * BI + j) * 1024), 16, 0, 0);
        if (DUAL) {
#pragma unroll
            for (int j = 0; j < BI; ++j)
                __builtin_amdgcn_global_load_lds((const MOE_GLB_AS void *)(bsrc[j] + b3off + k0),
                                                 (MOE_LDS_AS void *)(base + A_BYTES + B_BYTES + (wave * BI + j) * 1024),
                                                 16, 0, 0);
        }
    };
    auto clear_tail = [&](uint8_t *base) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (tail_piece) {
#pragma unroll
            for (int i = 0; i < AI; ++i) *reinterpret_cast<u32x4 *>(base + (wave * AI + i) * 1024 + lane * 16) = z;
#pragma unroll
            for (int j = 0; j < NBT * BI; ++j)
                *reinterpret_cast<u32x4 *>(base + A_BYTES + (wave * BI + (j % BI)) * 1024 + (j / BI) * B_BYTES + lane * 16) = z;
        }
    };

    // accumulators hold C^T fragments: acc[i][j] = W rows (n) x X rows (m), so
    // each lane ends with 4 consecutive output columns of one output row
    f32x4 acc[FM][FN];
    f32x4 acc3[DUAL ? FM : 1][DUAL ? FN : 1];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < (DUAL ? FM : 1); ++i)
#pragma unroll
            for (int j = 0; j < (DUAL ? FN : 1); ++j) acc3[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // fragment reads: row (base + lane%16), logical piece ks*4 + lane/16, stored at
    // piece ^ (row % 8) = piece ^ (lane % 8) (fragment bases are multiples of 16)
    const int arow = (wm * (BM / 2) + (lane & 15)) * 128;
    const int brow = (wn * (BN / 2) + (lane & 15)) * 128;
    auto compute = [&](const uint8_t *sa) {
        const uint8_t *sb = sa + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int pofs = (((ks * 4 + (lane >> 4)) ^ (lane & 7)) * 16);
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sa + arow + i * 16 * 128 + pofs));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + brow + j * 16 * 128 + pofs));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
            if (DUAL) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + B_BYTES + brow + j * 16 * 128 + pofs));
#pragma unroll
                for (int i = 0; i < (DUAL ? FM : 1); ++i)
#pragma unroll
                    for (int j = 0; j < (DUAL ? FN : 1); ++j)
                        acc3[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc3[i][j], 0, 0, 0);
            }
        }
    };

    // epilogue of local tile lt: bias, activation, bf16, 8-byte stores of the
    // 4 consecutive columns each lane holds (no LDS: the ring stays in flight)
    auto epilogue = [&](int lt) {
        int e, m0, n0;
        locate(lt, e, m0, n0);
        const int cnt = s_cnt[e];
        uint16_t *oe = out + (int64_t)e * C * N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * (BN / 2) + j * 16 + 4 * (lane >> 4);
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (BIAS && n < N) {
                const uint2 bb = *reinterpret_cast<const uint2 *>(bias + (int64_t)e * N + n);
                bv[0] = bf2f((uint16_t)(bb.x & 0xFFFFu)); bv[1] = bf2f((uint16_t)(bb.x >> 16));
                bv[2] = bf2f((uint16_t)(bb.y & 0xFFFFu)); bv[3] = bf2f((uint16_t)(bb.y >> 16));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int m = m0 + wm * (BM / 2) + i * 16 + (lane & 15);
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float t = acc[i][j][r] + bv[r];
                    if (ACT == 1) t = fmaxf(t, 0.f);
                    if (ACT == 2) t = silu(t) * acc3[DUAL ? i : 0][DUAL ? j : 0][r];
                    v[r] = t;
                }
                if (m < cnt && n < N) {
                    uint2 pk;
                    pk.x = pack_bf16x2(v[0], v[1]);
                    pk.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2 *>(oe + (int64_t)m * N + n) = pk;
                }
            }
        }
    };

    // ---- the stream: step g consumes K tile g % nk of local tile g / nk from
    // stage g % 3 after waiting for it (the newer stage stays in flight), and
    // refills the stage consumed at step g-1 with step g+2
    auto step = [&](uint8_t *cur, uint8_t *refill, int g) {
        const int ct = g / nk;                      // local output tile of this step
        const int ck = g - ct * nk;                 // its K tile
        wait_vm_lgkm0<(S - 2) * PER>();
        if (ktail && ck == nk - 1) {
            clear_tail(cur);
            wait_vm_lgkm0<(S - 2) * PER>();
        }
        __builtin_amdgcn_s_barrier();
        issue(refill, g + 2);
        if (ck == 0) zero_acc();
        compute(cur);
        if (ck == nk - 1) epilogue(ct);
    };
    issue(st0, 0);
    issue(st1, 1);
    int g = 0;
    for (; g + 3 <= steps; g += 3) {
        step(st0, st2, g);
        step(st1, st0, g + 1);
        step(st2, st1, g + 2);
    }
    if (g < steps) step(st0, st2, g);
    if (g + 1 < steps) step(st1, st0, g + 1);
    wait_vm_lgkm0<0>();          // no DMA may outlive the block
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

// The tile shape of the bf16 path (one shape for both expert GEMMs, so they
// share one tile map).
using TileBF16 = Tile<128, 128, 3>;

// Compute units of the current device (8 XCDs x 32 on MI355X), times 1 block each.
int persistent_blocks() {
    static thread_local int cached = 0;
    if (cached == 0) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            cached = ((cus + 7) / 8) * 8;
        else
            cached = 256;
    }
    return cached;
}

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
        // persistent: one block per CU (the LDS ring takes most of a CU), at most
        // as many blocks as tiles, a multiple of the 8 XCDs
        int64_t g = grid_for(C, E, TileBF16::BM, tiles_n, rows_bound);
        if (g > persistent_blocks()) g = persistent_blocks();
        const dim3 grid((unsigned)g);
        const uint16_t *a = (const uint16_t *)A, *b = (const uint16_t *)B, *b3 = (const uint16_t *)B3,
                       *bi = (const uint16_t *)bias;
        uint16_t *o = (uint16_t *)out;
#define MOE_GEMM(ACTV, BIASV)                                                                  \
    hipLaunchKernelGGL((gemm_bf16_kernel<TileBF16, ACTV, BIASV>), grid, dim3(256), 0, s, a, b, b3, bi, \
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
