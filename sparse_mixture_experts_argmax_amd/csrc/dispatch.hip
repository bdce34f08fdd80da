// Dispatch: capacity slots in token order, drops, and the expert-major permutation.
//
// [CS25-L5] "Capacity Factor 与 Token Dropping": tokens, in order, take the
// next free slot of their expert while fewer than C are taken; the rest skip
// the expert.  [CMU-L16] section 6.1: every first choice is placed before
// any second choice.  The slot of choice (t, j) is therefore the number of
// choices of the same expert that come before it in the order
// (rank 0, token 0..T-1), (rank 1, token 0..T-1), ...
//
// That count is computed without atomics, so it is deterministic:
//   slot_rank  -- per block of 256 tokens and rank j: the position of each
//                 choice among same-expert choices of the block (wave ballots
//                 over the bits of the expert index, then the counts of the
//                 earlier waves) and the block's per-expert histogram.
//   slot_scan  -- per expert, an exclusive scan of the histograms in
//                 (rank, block) order: the slots taken before each block.
//                 In the fused forward it also sums the router's per-block
//                 partials (probability sums, choice counts).  On the f32
//                 path its last block builds the GEMM tile map from the kept
//                 counts; the bf16 forward leaves that to slot_index.
//   permute    -- slot = scan + in-block position; slots >= C drop; kept
//                 rows are copied x[t] -> xbuf[e, slot] with 16-byte moves.
//   slot_index -- the bf16 forward's alternative to permute: the same slots,
//                 but only the token of each expert row is recorded (the
//                 first GEMM gathers the rows from x itself).  Its block 0
//                 also writes the GEMM tile map and, when the second GEMM
//                 writes y, the auxiliary loss, from the totals the scan
//                 finished a launch earlier.
// [SW-GLaM] "All-to-All": the data-sharded -> expert-sharded relayout, done
// here as a permutation inside one GPU's memory.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

__global__ __launch_bounds__(DISPATCH_TOK_BLOCK) void slot_rank_kernel(
    const int32_t *__restrict__ expert_idx, int64_t T, int E, int k, int nbits,
    int32_t *__restrict__ rank, int32_t *__restrict__ hist, unsigned *__restrict__ done) {
    extern __shared__ int sc[];                     // [4 waves][E]
    const int tid = threadIdx.x;
    // the completion counter of the scan that follows starts at zero
    if (done != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *done = 0u;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int j = blockIdx.y;
    const int nblk = gridDim.x;
    const int64_t t = (int64_t)blockIdx.x * DISPATCH_TOK_BLOCK + tid;

    for (int q = tid; q < 4 * E; q += DISPATCH_TOK_BLOCK) sc[q] = 0;
    int e = (t < T) ? expert_idx[t * k + j] : -1;
    const bool ok = e >= 0 && e < E;               // out-of-range indices are treated as dropped
    if (!ok) e = 0;

    // lanes of this wave that chose the same expert
    uint64_t same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(ok && bit);
        same &= bit ? m : ~m;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rw = __popcll(same & below);
    __syncthreads();
    if (ok && rw == 0) sc[wave * E + e] = __popcll(same);
    __syncthreads();
    if (ok) {
        int r = rw;
        for (int w = 0; w < wave; ++w) r += sc[w * E + e];
        rank[(int64_t)j * T + t] = r;
    }
    // histogram, laid out [E][k * nblk] so that the scan reads it contiguously
    for (int n = tid; n < E; n += DISPATCH_TOK_BLOCK)
        hist[(int64_t)n * k * nblk + (int64_t)j * nblk + blockIdx.x] =
            ((sc[n] + sc[E + n]) + sc[2 * E + n]) + sc[3 * E + n];
}

// The GEMM tile map from the clipped counts, by one whole block of 256
// threads: thread t owns experts 4t .. 4t + 3 (E <= 1024), a wave scan, then
// the wave totals.  COHERENT: the counts come from other blocks of the same
// launch, so they are read from L2 (agent-scope atomic loads).
template <bool COHERENT>
__device__ void tile_map_block(const int32_t *expert_count, int E, int bm, int32_t *tile_map, int *s_wsum) {
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    if (t < TAIL_SPLIT_SLOTS) tile_map[E + 1 + t] = 0;    // the split last wave's counters
    static_assert(TAIL_SPLIT_SLOTS <= 256, "one counter per thread");
    int c[4];
    int local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int ee = 4 * t + q;
        int n = 0;
        if (ee < E)
            n = COHERENT ? __hip_atomic_load(expert_count + ee, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : expert_count[ee];
        c[q] = (n + bm - 1) / bm;
        local += c[q];
    }
    int inc = local;
    for (int m = 1; m < 64; m <<= 1) {
        const int u = __shfl_up(inc, m);
        if (lane >= m) inc += u;
    }
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    int run = inc - local;
    for (int i = 0; i < wave; ++i) run += s_wsum[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int ee = 4 * t + q;
        if (ee < E) tile_map[ee] = run;
        run += c[q];
    }
    if (E - 1 >= 4 * t && E - 1 < 4 * t + 4) tile_map[E] = run;
}

// One wave per expert: exclusive scan over (rank, block), in place.
// Optionally (the fused forward) also:
//  * the router's per-expert totals, in the same order and precision as its
//    own reduction, so that both give the same bits;
//  * the expert GEMMs' tile map (tile_map[e] = sum over e' < e of
//    ceil(expert_count[e'] / bm)), built by whichever block finishes last
//    (a completion counter that slot_rank zeroed).
__global__ __launch_bounds__(256) void slot_scan_kernel(int32_t *__restrict__ hist, int L, int E,
                                                        int64_t C, int32_t *__restrict__ expert_count,
                                                        const float *__restrict__ part_prob, int nblk_r,
                                                        float *__restrict__ prob_sum,
                                                        int32_t *__restrict__ route_count,
                                                        int32_t *__restrict__ tile_map, int bm,
                                                        unsigned *__restrict__ done, float alpha,
                                                        int64_t T, int k, float *__restrict__ aux,
                                                        const float *__restrict__ part_z,
                                                        float *__restrict__ z_loss) {
    __shared__ int s_last;
    __shared__ int s_wsum[4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int e = blockIdx.x * 4 + wave;
    if (e < E) {
        int32_t *h = hist + (int64_t)e * L;
        int run = 0;
        for (int b0 = 0; b0 < L; b0 += 64) {
            const int b = b0 + lane;
            const int v = (b < L) ? h[b] : 0;
            int inc = v;
            for (int m = 1; m < 64; m <<= 1) {
                const int u = __shfl_up(inc, m);
                if (lane >= m) inc += u;
            }
            if (b < L) h[b] = run + inc - v;
            run += __shfl(inc, 63);
        }
        if (lane == 0) expert_count[e] = (int32_t)((int64_t)run < C ? (int64_t)run : C);
        // run = number of choices of expert e before capacity
        if (part_prob != nullptr) {
            double sp = 0.0;
            for (int b = lane; b < nblk_r; b += 64) sp += (double)part_prob[(int64_t)b * E + e];
            for (int m = 32; m >= 1; m >>= 1) sp += __shfl_xor(sp, m);
            if (lane == 0) {
                prob_sum[e] = (float)sp;
                route_count[e] = run;
            }
            // the router's z-loss from its block partials (expert 0's wave)
            if (z_loss != nullptr && e == 0) {
                const float zl = z_loss_wave(part_z, nblk_r, T, lane);
                if (lane == 0) z_loss[0] = zl;
            }
        }
    }
    if (tile_map == nullptr) return;                 // uniform over the grid
    __threadfence();                                 // this block's counts are visible ...
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(done, 1u) == gridDim.x - 1;   // ... before it counts
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    tile_map_block<true>(expert_count, E, bm, tile_map, s_wsum);
    if (aux != nullptr && wave == 0) {
        const float a = aux_loss_wave<true>(route_count, prob_sum, E, T, k, alpha, lane);
        if (lane == 0) aux[0] = a;
    }
}

// One wave per (token, rank) choice; lanes move 16-byte pieces of the row.
__global__ __launch_bounds__(256) void permute_kernel(
    const uint8_t *__restrict__ x, int row_bytes, const int32_t *__restrict__ expert_idx,
    const int32_t *__restrict__ rank, const int32_t *__restrict__ base, int64_t T, int E, int k,
    int nblk, int64_t C, int32_t *__restrict__ slot, uint8_t *__restrict__ drop,
    uint8_t *__restrict__ xbuf) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int pieces = row_bytes >> 4;
    for (int64_t a = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); a < T * k; a += nwaves) {
        const int64_t t = a / k;
        const int j = (int)(a - t * k);
        const int e = expert_idx[a];
        int64_t s = -1;
        if (e >= 0 && e < E) {
            const int blk = (int)(t / DISPATCH_TOK_BLOCK);
            s = (int64_t)base[(int64_t)e * k * nblk + (int64_t)j * nblk + blk] + rank[(int64_t)j * T + t];
            if (s >= C) s = -1;
        }
        if (lane == 0) {
            slot[a] = (int32_t)s;
            drop[a] = (s < 0) ? 1 : 0;
        }
        if (s >= 0) {
            const uint8_t *src = x + t * row_bytes;
            uint8_t *dst = xbuf + ((int64_t)e * C + s) * row_bytes;
            for (int p = lane; p < pieces; p += 64) st16(dst + p * 16, ld16(src + p * 16));
        }
    }
}

// The fused forward's dispatch: slots and drops exactly as permute_kernel
// computes them, one choice per thread, but no row is copied: each kept
// choice records the token of its expert row (row_tok[e C + slot] = t), from
// which the first expert GEMM gathers x.  With one choice per token, y_zero
// (= y) gets the rows of dropped tokens cleared, since the second GEMM then
// writes only kept rows; the wave clears each such row together.
__global__ __launch_bounds__(256) void slot_index_kernel(
    const int32_t *__restrict__ expert_idx, const int32_t *__restrict__ rank,
    const int32_t *__restrict__ base, int64_t T, int E, int k, int nblk, int64_t C,
    int32_t *__restrict__ slot, uint8_t *__restrict__ drop, int32_t *__restrict__ row_tok,
    const float *__restrict__ gate, float *__restrict__ row_gate, uint8_t *__restrict__ y_zero,
    int row_bytes, const int32_t *__restrict__ expert_count, const float *__restrict__ prob_sum,
    const int32_t *__restrict__ route_count, int32_t *__restrict__ tile_map, int bm, float alpha,
    float *__restrict__ aux) {
    __shared__ int s_wsum[4];
    const int lane = threadIdx.x & 63;
    // block 0 also writes the GEMM tile map and the loss from the totals
    // the scan finished (a launch earlier, so plain loads see them)
    if (blockIdx.x == 0) {
        if (tile_map != nullptr) tile_map_block<false>(expert_count, E, bm, tile_map, s_wsum);
        if (aux != nullptr && threadIdx.x < 64) {
            const float av = aux_loss_wave<false>(route_count, prob_sum, E, T, k, alpha, lane);
            if (lane == 0) aux[0] = av;
        }
    }
    const int64_t a = (int64_t)blockIdx.x * 256 + threadIdx.x;
    bool dropped = false;
    if (a < T * k) {
        const int64_t t = a / k;
        const int j = (int)(a - t * k);
        const int e = expert_idx[a];
        int64_t s = -1;
        if (e >= 0 && e < E) {
            const int blk = (int)(t / DISPATCH_TOK_BLOCK);
            s = (int64_t)base[(int64_t)e * k * nblk + (int64_t)j * nblk + blk] + rank[(int64_t)j * T + t];
            if (s >= C) s = -1;
        }
        slot[a] = (int32_t)s;
        drop[a] = (s < 0) ? 1 : 0;
        if (s >= 0) {
            row_tok[(int64_t)e * C + s] = (int32_t)t;
            if (row_gate != nullptr) row_gate[(int64_t)e * C + s] = gate[a];
        }
        dropped = s < 0;
    }
    if (y_zero != nullptr) {
        // k = 1: choice a is token a
        uint64_t m = __ballot(dropped);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const int pieces = row_bytes >> 4;
        while (m != 0) {
            const int l = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            const int64_t t = a - lane + l;
            for (int p = lane; p < pieces; p += 64) st16(y_zero + t * row_bytes + p * 16, z);
        }
    }
}

int bits_for(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

}  // namespace

hipError_t launch_slot_rank(const int32_t *expert_idx, int64_t T, int E, int k, int32_t *rank,
                            int32_t *hist, unsigned *done, hipStream_t s) {
    const int nblk = dispatch_blocks(T);
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL(slot_rank_kernel, dim3(nblk, k), dim3(DISPATCH_TOK_BLOCK),
                       (size_t)4 * E * sizeof(int), s, expert_idx, T, E, k, bits_for(E), rank, hist,
                       done);
    return hipGetLastError();
}

hipError_t launch_slot_scan(int32_t *hist, int nblk, int E, int k, int64_t C,
                            int32_t *expert_count, const float *part_prob, int nblk_r,
                            float *prob_sum, int32_t *route_count, int32_t *tile_map, int bm,
                            unsigned *done, hipStream_t s, int64_t T, float alpha, float *aux,
                            const float *part_z, float *z_loss) {
    if (z_loss != nullptr && (part_prob == nullptr || part_z == nullptr)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(slot_scan_kernel, dim3((E + 3) / 4), dim3(256), 0, s, hist, nblk * k, E, C,
                       expert_count, part_prob, nblk_r, prob_sum, route_count, tile_map, bm, done,
                       alpha, T, k, aux, part_z, z_loss);
    return hipGetLastError();
}

hipError_t launch_slot_index(const int32_t *expert_idx, const int32_t *rank, const int32_t *base,
                             int64_t T, int E, int k, int64_t C, int32_t *slot, uint8_t *drop_mask,
                             int32_t *row_tok, const float *gate, float *row_gate, void *y_zero,
                             int row_bytes, hipStream_t s, const int32_t *expert_count,
                             const float *prob_sum, const int32_t *route_count, int32_t *tile_map,
                             int bm, float alpha, float *aux) {
    const int64_t n = T * k;
    if (n == 0) return hipSuccess;
    if (tile_map != nullptr && (E > 1024 || bm < 1 || expert_count == nullptr)) return hipErrorInvalidValue;
    if (aux != nullptr && (prob_sum == nullptr || route_count == nullptr)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(slot_index_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, expert_idx,
                       rank, base, T, E, k, dispatch_blocks(T), C, slot, drop_mask, row_tok, gate,
                       row_gate, reinterpret_cast<uint8_t *>(y_zero), row_bytes, expert_count, prob_sum,
                       route_count, tile_map, bm, alpha, aux);
    return hipGetLastError();
}

hipError_t launch_permute(const void *x, int elem_bytes, const int32_t *expert_idx,
                          const int32_t *rank, const int32_t *base, int64_t T, int d, int E,
                          int k, int64_t C, int32_t *slot, uint8_t *drop_mask, void *xbuf,
                          hipStream_t s) {
    const int64_t n = T * k;
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t *>(x), d * elem_bytes, expert_idx, rank, base,
                       T, E, k, dispatch_blocks(T), C, slot, drop_mask,
                       reinterpret_cast<uint8_t *>(xbuf));
    return hipGetLastError();
}

}  // namespace moe
