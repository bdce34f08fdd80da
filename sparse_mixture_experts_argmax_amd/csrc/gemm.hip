// Grouped GEMM of the experts: for every expert e and every kept row m < count[e]
//   out[e, m, n] = act( sum_k A[e, m, k] * B[e, n, k] (+ bias[e, n]) )
// with act = none, ReLU, or SwiGLU (silu(A B^T) * (A B3^T)).
//
// [SW-GLaM] "Dense Scaling 与 MoE 的核心差异": FFN(x) = W_2 sigma(W_1 x);
// [CMU-L16] section 2.1 (biases b, c) and 2.3 (SwiGLU expert, Swish beta = 1);
// [CMU-L16] section 5 / [CS25-L5] "Switch Layer": experts run as batched
// matrix products over their slot lists (a dedicated grouped-GEMM kernel).
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * 256 threads = 4 waves in a 2x2 grid; block tiles of 128 to 320 rows by
//     128 to 256 columns (the shapes at the end of gemm_kernel.h), each wave
//     owning a quarter.
//   * A and B tiles are K-contiguous in HBM (x rows, nn.Linear-style weight
//     rows), so both are staged the same way: 16-byte LDS DMA
//     (global_load_lds) into a ring of LDS stages one to three K tiles ahead
//     of the MFMAs (the wide 320- and 192-row tiles keep the weights two
//     ahead and the activations one), 16-byte pieces of each LDS row
//     XOR-swizzled by row (conflict-free fragment reads, no padding).
//   * Only real row tiles are launched work: a tile that holds a whole
//     expert's capacity maps blocks to (expert, column tile) directly;
//     otherwise tile_map holds the prefix sums of ceil(count[e] / BM), built
//     on the device, so an expert with few rows costs few tiles and an empty
//     expert none.
//   * The first GEMM of the fused forward gathers its rows of x by token
//     index; the second scales each output row by its token's gate and
//     writes it to that token's row of y.
//   * Tile order is expert-major, then column tile, then row tile, so the
//     row tiles that share a weight tile run next to each other; the block
//     index is remapped so that each XCD (blocks are dealt to the 8 XCDs
//     round-robin) gets one contiguous range of that order and its own L2
//     keeps the weight and activation tiles it reuses.
//   * The epilogue adds the bias, applies the activation and rounds to bf16;
//     the tile goes out through LDS as coalesced 16-byte row stores when it
//     fits a stage buffer, else straight from registers.
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 x 32 tiles, the next K
// tile's loads in flight during the current one's FMAs).
#include "gemm_kernel.h"

#include <atomic>

namespace moe {

namespace {

// ---------------------------------------------------------------------------
// fp32 path
// ---------------------------------------------------------------------------
constexpr int FBM = 64, FBN = 64, FBK = 32;
constexpr int FLQ = FBM * FBK / 256;                 // values of each operand a thread stages per K tile

// The K loop keeps the next K tile's loads in flight (in registers) while the
// current tile is multiplied out of LDS, so that a step costs its FMAs rather
// than a global-memory round trip; each output still sums its K terms in
// ascending k, one fma at a time.
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
    SplitPart sp;
    if (!map_tile(tile_map, E, tiles_n, s_map, e, mt, nt, sp)) return;
    const int cnt = count[e];
    const int m0 = mt * FBM;
    const int n0 = nt * FBN;
    const int tid = threadIdx.x;
    const int tm = (tid >> 4) * 4;     // 4 rows
    const int tn = (tid & 15) * 4;     // 4 columns
    const float *Ae = A + (int64_t)e * C * K;
    const float *Be = B + (int64_t)e * N * K;
    const float *B3e = DUAL ? B3 + (int64_t)e * N * K : nullptr;

    // staged value l of this thread: tile row r = q / FBK, column c = q % FBK
    // (q = tid + 256 l), so 32 consecutive threads read 128 contiguous bytes
    // of one row; rows past the count or past N repeat the last one
    float ra[FLQ], rb[FLQ], rb3[DUAL ? FLQ : 1];
    auto load = [&](int k0) {
#pragma unroll
        for (int l = 0; l < FLQ; ++l) {
            const int q = tid + 256 * l;
            const int r = q / FBK, c = q % FBK;
            int am = m0 + r;
            if (am > cnt - 1) am = cnt - 1;
            int bn = n0 + r;
            if (bn > N - 1) bn = N - 1;
            const bool in = k0 + c < K;
            ra[l] = in ? Ae[(int64_t)am * K + k0 + c] : 0.f;
            rb[l] = in ? Be[(int64_t)bn * K + k0 + c] : 0.f;
            if (DUAL) rb3[DUAL ? l : 0] = in ? B3e[(int64_t)bn * K + k0 + c] : 0.f;
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int l = 0; l < FLQ; ++l) {
            const int q = tid + 256 * l;
            const int r = q / FBK, c = q % FBK;
            sA[c][r] = ra[l];
            sB[c][r] = rb[l];
            if (DUAL) sB3[DUAL ? c : 0][r] = rb3[DUAL ? l : 0];
        }
    };

    float acc[4][4] = {};
    float acc3[4][4] = {};
    load(0);
    for (int k0 = 0; k0 < K; k0 += FBK) {
        store();
        __syncthreads();
        if (k0 + FBK < K) load(k0 + FBK);
#pragma unroll 8
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

// tile_map[0] = 0, tile_map[e+1] = sum_{e' <= e} ceil(count[e'] / bm); one block.
// The split last wave's counters after it are cleared.
__global__ __launch_bounds__(1024) void tile_map_kernel(const int32_t *__restrict__ count, int E, int bm,
                                                        int32_t *__restrict__ tile_map) {
    __shared__ int s[1024];
    const int t = threadIdx.x;
    if (t < TAIL_SPLIT_SLOTS) tile_map[E + 1 + t] = 0;
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

}  // namespace

// Row-tile height of the bf16 path: one BM for both expert GEMMs, so they
// share one tile map.  When an expert's capacity fits one tile of 192 or 320
// rows, that tile covers all of its rows, so every weight tile is streamed
// once (experts of about 256 rows would otherwise pay a third, mostly empty
// 128-row tile and read their weights three times).  256 (half the LDS bytes
// per MFMA of 128) when experts hold at least 512 rows: a 256-row tile over a
// 257-row expert spends half its MFMAs on padding.  The gated SwiGLU tiles
// exist for 128 and 256 rows only.
int gemm_bm(int dtype_bf16, int64_t C, int act) {
    if (!dtype_bf16) return FBM;
    if (C >= 512) return 256;
    if (act != 2 && C > 256 && C <= 320) return 320;
    if (act != 2 && C > 128 && C <= 192) return 192;
    return 128;
}

size_t tail_split_bytes(int dtype_bf16, int64_t C) {
    // a bf16 launch takes the tile map (and may split its last wave) when
    // the capacity exceeds the row tile, which is at least 128 rows
    if (!dtype_bf16 || C <= 128) return 0;
    return (size_t)TAIL_SPLIT_SLOTS * TAIL_SPLIT_PART_FLOATS * sizeof(float);
}

// Compute units of the current device, read once per device; at most
// TAIL_SPLIT_SLOTS (the split last wave's counters and partial slots).
static int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
        v = n < TAIL_SPLIT_SLOTS ? n : TAIL_SPLIT_SLOTS;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

hipError_t launch_tile_map(const int32_t *expert_count, int E, int bm, int32_t *tile_map,
                           hipStream_t s) {
    hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(1024), 0, s, expert_count, E, bm, tile_map);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const void *A, const void *B, const void *B3, const void *bias,
                               int dtype_bf16, int act, const int32_t *expert_count,
                               const int32_t *tile_map, int bm, int E, int64_t C, int N, int K,
                               int64_t rows_bound, void *out, hipStream_t s, const int32_t *row_tok,
                               int64_t T, const float *gate, const int32_t *kcount, float *split_part) {
    if (C == 0 || rows_bound == 0) return hipSuccess;
    if (row_tok != nullptr && (!dtype_bf16 || T < 1 || (act == 0 && gate == nullptr)))
        return hipErrorInvalidValue;
    if (kcount != nullptr && (K % 64 != 0 || row_tok != nullptr)) return hipErrorInvalidValue;
    if (dtype_bf16) {
        // fused forward: the first GEMM gathers token rows, the second
        // scatters gated rows to y (out is then y)
        // tile order: consecutive blocks (the same XCD) share the panel of the
        // operand that is re-read more cheaply.  Column tile major shares the
        // weight panel across an expert's row tiles (the expert GEMMs: C rows
        // against N >= C columns); when an expert's rows outnumber the
        // columns (the weight gradients dW1, dW3: f rows against d columns)
        // the A panels are the large operand, and row tile major streams
        // each once while the small B panels are re-read from the caches.
        // Measured on the Mixtral-shaped expert backward: 17.6 -> 16.5 ms.
        FuseArgs fz{row_tok, T, gate, (uint16_t *)out, row_tok == nullptr ? 0 : (act == 0 ? 2 : 1), kcount,
                    nullptr, nullptr, 0, C > N ? 1 : 0};
        if (split_part != nullptr && C > bm) {
            // the split last wave (tile-map launches): partial sums in
            // split_part, counters after the tile map
            fz.ncu = device_cus();
            if (fz.ncu >= 8) {
                fz.part = split_part;
                fz.flags = const_cast<int32_t *>(tile_map) + E + 1;
            }
        }
        // the gated tiles exist for 128 and 256 rows only
        if ((bm != 128 && bm != 192 && bm != 256 && bm != 320) || (act == 2 && bm != 128 && bm != 256))
            return hipErrorInvalidValue;
        const uint16_t *a = (const uint16_t *)A, *b = (const uint16_t *)B, *b3 = (const uint16_t *)B3,
                       *bi = (const uint16_t *)bias;
        uint16_t *o = (uint16_t *)out;
        // row tiles an expert-parallel launch can expect (for the column-tile
        // choice): one per expert when a tile holds the whole capacity; with
        // the tile map, E ceil(C / bm) whatever rows_bound, so that the fused
        // forward and the split expert FFN pick the same column tiles and so
        // split the same last wave (the same sums, bit for bit)
        const int64_t mt_est = C <= bm ? (rows_bound < E ? rows_bound : E) : (int64_t)E * ((C + bm - 1) / bm);
        // a tile that holds the whole capacity goes by (expert, column tile)
        // without the tile map
        const bool expert = C <= bm;
        // expert-per-tile launches stream each weight tile once: they load it
        // non-temporal when the activation operand fits half the 256 MB
        // last-level cache (then it stays there, written by the previous
        // stage and read by several column tiles, instead of being evicted
        // by the weight stream; measured 18 % off the second switch_base
        // GEMM, and slower when the activations do not fit)
        const bool wnt = expert && rows_bound * (int64_t)K * 2 <= (int64_t(128) << 20);
        const GemmArgs g{a, b, b3, bi, expert_count, tile_map, E, C, N, K, rows_bound, o, s, fz, act,
                         expert, wnt};
        // wide column tiles unless that leaves fewer tiles than CUs
        if (act == 2) return gemm_bf16_gated(g, bm);
        if (bm == 320) return gemm_bf16_320(g, mt_est * ((N + 191) / 192) >= 256);
        if (bm == 192) return gemm_bf16_192(g, mt_est * ((N + 255) / 256) >= 256);
        const bool wide = mt_est * ((N + 255) / 256) >= 256;
        if (bm == 256) return wide ? gemm_bf16_256w(g) : gemm_bf16_256n(g);
        return wide ? gemm_bf16_128w(g) : gemm_bf16_128n(g);
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
