// Priority routing: capacity slots filled in descending score order.
//
// [CS25-L5], the V-MoE part after "什么是视觉 token": with a capacity factor
// below 1 the tokens are ranked by importance first and the high-priority
// ones take the expert slots.  The capacity rule of the plain dispatch with
// the token visit order replaced by descending score (equal scores: lower
// token index first; NaN scores last), still rank-major for k > 1: every
// first choice is placed before any second choice.
//
// Three launches after the plain rank and scan passes, which (run with an
// unbounded capacity) give every choice its position pos in its expert's
// list in (rank, token) order and every expert its choice count n_e:
//  * priority_list_kernel: each choice writes its order key at pos of its
//    expert's list, key = (descending score bits << 32) | token;
//  * priority_slot_kernel: one block per 256 entries of the lists laid end
//    to end; an entry's slot is the start of its rank's segment plus the
//    number of keys in that segment below its own (keys are distinct),
//    found by streaming the segment through LDS (with few experts split
//    over several blocks per entry block, whose counts a second pass of the
//    same kernel gathers);
//  * permute_slots_kernel: the rows of the kept choices into xbuf.
// Work is sum over experts of n_e^2 / 2 compares (rank segments bound it
// further): 4 M for 16384 tokens over 64 experts, and at most T^2 / 2 when
// every token picks one expert.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int PR_BLOCK = 256;

// Ascending order key of a score for "higher first": NaN last, -0 = +0.
__device__ __forceinline__ uint32_t desc_key(float v) {
    if (v != v) return 0xFFFFFFFFu;
    if (v == 0.f) v = 0.f;
    const uint32_t b = __float_as_uint(v);
    const uint32_t asc = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ~asc;
}

// Exclusive prefix of cnt[0 .. E) into off[0 .. E) (LDS), E <= 1024, 256 threads.
__device__ void block_offsets(const int32_t *__restrict__ cnt, int E, int32_t *off) {
    __shared__ int s_wave[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int v[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        v[i] = e < E ? cnt[e] : 0;
        sum += v[i];
    }
    int inc = sum;
    for (int m = 1; m < 64; m <<= 1) {
        const int u = __shfl_up(inc, m);
        if (lane >= m) inc += u;
    }
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    int base = inc - sum;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = tid * 4 + i;
        if (e < E) off[e] = base;
        base += v[i];
    }
    __syncthreads();
}

__global__ __launch_bounds__(PR_BLOCK) void priority_list_kernel(
    const int32_t *__restrict__ expert_idx, const float *__restrict__ priority,
    const int32_t *__restrict__ rank, const int32_t *__restrict__ base,
    const int32_t *__restrict__ n_e, int64_t T, int E, int k, int nblk,
    uint64_t *__restrict__ list, int32_t *__restrict__ off_out, int32_t *__restrict__ slot,
    uint8_t *__restrict__ drop, int32_t *__restrict__ pcnt) {
    __shared__ int32_t s_off[1024];
    block_offsets(n_e, E, s_off);
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e < E; e += PR_BLOCK) off_out[e] = s_off[e];
    const int64_t a = (int64_t)blockIdx.x * PR_BLOCK + threadIdx.x;
    if (a >= T * k) return;
    const int64_t t = a / k;
    const int j = (int)(a - t * k);
    const int e = expert_idx[a];
    if (e < 0 || e >= E) {          // not a choice: never placed
        slot[a] = -1;
        drop[a] = 1;
        return;
    }
    const int blk = (int)(t / DISPATCH_TOK_BLOCK);
    const int64_t pos = (int64_t)base[(int64_t)e * k * nblk + (int64_t)j * nblk + blk] + rank[(int64_t)j * T + t];
    list[s_off[e] + pos] = ((uint64_t)desc_key(priority[t]) << 32) | (uint64_t)(uint32_t)t;
    if (pcnt != nullptr) pcnt[s_off[e] + pos] = 0;    // the split count's sums start at zero
}

// Block b takes entries [256 b, 256 b + 256) of the experts' lists laid end
// to end (expert e's list starts at off[e]); each entry finds its expert by
// a binary search over off.  The block streams the union of its entries'
// rank segments through LDS; an entry counts the keys of its own segment
// (global positions [off[e] + lo, off[e] + hi), disjoint across experts)
// below its key.  With few experts (long segments) the stream is split over
// gridDim.y blocks: block (b, y) takes the y-th of every gridDim.y tiles of
// 256 keys and adds its counts to pcnt (integer sums: the same total in any
// order), and priority_final_kernel turns them into slots; with gridDim.y =
// 1 the block writes the slots itself.
__global__ __launch_bounds__(PR_BLOCK) void priority_slot_kernel(
    const uint64_t *__restrict__ list, const int32_t *__restrict__ off, const int32_t *__restrict__ n_e,
    const int32_t *__restrict__ base, int E, int k, int nblk, int64_t C, int32_t *__restrict__ slot,
    uint8_t *__restrict__ drop, int32_t *__restrict__ expert_count, int32_t *__restrict__ pcnt,
    int final_pass) {
    __shared__ __attribute__((aligned(16))) uint64_t s_key[PR_BLOCK];
    __shared__ int s_lo, s_hi;
    __shared__ int32_t s_off[1024];                  // the list offsets, searched in LDS
    const int tid = threadIdx.x;
    const int ny = gridDim.y, y = blockIdx.y;
    if (blockIdx.x == 0 && y == 0 && !final_pass)
        for (int e = tid; e < E; e += PR_BLOCK) {
            const int n = n_e[e];
            expert_count[e] = (int32_t)((int64_t)n < C ? (int64_t)n : C);
        }
    const int V = off[E - 1] + n_e[E - 1];           // entries in all lists
    const int p0 = blockIdx.x * PR_BLOCK;
    if (p0 >= V) return;                             // the whole block
    for (int e = tid; e < E; e += PR_BLOCK) s_off[e] = off[e];
    __syncthreads();
    const int p = p0 + tid;
    const bool ok = p < V;
    // the expert holding entry p: the largest e with off[e] <= p
    int e = 0;
    if (ok) {
        int lo_e = 0, hi_e = E - 1;
        while (lo_e < hi_e) {
            const int mid = (lo_e + hi_e + 1) >> 1;
            if (s_off[mid] <= p) lo_e = mid;
            else hi_e = mid - 1;
        }
        e = lo_e;
    }
    const int oe = ok ? s_off[e] : 0;
    const int pl = p - oe;                           // position in the expert's list
    // this entry's rank segment [lo, hi) of the expert's list
    const int32_t *b = base + (int64_t)e * k * nblk;
    int j = 0;
    int lo = 0, hi = 0;
    uint64_t my = 0;
    if (ok) {
        for (int r = 1; r < k; ++r)
            if (b[(int64_t)r * nblk] <= pl) j = r;
        lo = b[(int64_t)j * nblk];
        hi = j + 1 < k ? b[(int64_t)(j + 1) * nblk] : n_e[e];
        my = list[p];
    }
    if (final_pass) {
        // the split count's sums, gathered (one entry per thread)
        if (ok) {
            const int64_t s = (int64_t)lo + pcnt[p];
            const int64_t t = (int64_t)(uint32_t)(my & 0xFFFFFFFFull);
            const int64_t a = t * k + j;
            slot[a] = s < C ? (int32_t)s : -1;
            drop[a] = s < C ? 0 : 1;
        }
        return;
    }
    if (tid == 0) {
        s_lo = 0x7fffffff;
        s_hi = 0;
    }
    __syncthreads();
    if (ok) {
        atomicMin(&s_lo, oe + lo);
        atomicMax(&s_hi, oe + hi);
    }
    __syncthreads();
    const int blo = s_lo, bhi = s_hi;
    // a tile key i is in this entry's segment when (q0 + i - (oe + lo)) <
    // (hi - lo) as unsigned; full tiles read 16 keys per step with 16-byte
    // LDS loads, so that the loads are in flight together
    const uint32_t span = (uint32_t)(hi - lo);
    const int glo = oe + lo;
    int cnt = 0;
    for (int q0 = blo + y * PR_BLOCK; q0 < bhi; q0 += ny * PR_BLOCK) {
        const int q = q0 + tid;
        s_key[tid] = q < bhi ? list[q] : ~0ull;
        __syncthreads();
        const int rel = q0 - glo;
        if (bhi - q0 >= PR_BLOCK) {
            const u32x4 *s4 = reinterpret_cast<const u32x4 *>(s_key);
            for (int i0 = 0; i0 < PR_BLOCK; i0 += 16) {
                uint64_t kk[16];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const u32x4 v = s4[(i0 >> 1) + u];
                    kk[2 * u] = (uint64_t)v[0] | ((uint64_t)v[1] << 32);
                    kk[2 * u + 1] = (uint64_t)v[2] | ((uint64_t)v[3] << 32);
                }
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    cnt += ((uint32_t)(rel + i0 + u) < span && kk[u] < my) ? 1 : 0;
            }
        } else {
            const int m = bhi - q0;
            for (int i = 0; i < m; ++i)
                cnt += ((uint32_t)(rel + i) < span && s_key[i] < my) ? 1 : 0;
        }
        __syncthreads();
    }
    if (ok && ny > 1) {
        if (cnt > 0) atomicAdd(&pcnt[p], cnt);
    } else if (ok) {
        const int64_t s = (int64_t)lo + cnt;
        const int64_t t = (int64_t)(uint32_t)(my & 0xFFFFFFFFull);
        const int64_t a = t * k + j;
        slot[a] = s < C ? (int32_t)s : -1;
        drop[a] = s < C ? 0 : 1;
    }
}

// One wave per (token, rank) choice; lanes move 16-byte pieces of the row.
__global__ __launch_bounds__(256) void permute_slots_kernel(const uint8_t *__restrict__ x, int row_bytes,
                                                            const int32_t *__restrict__ expert_idx,
                                                            const int32_t *__restrict__ slot, int64_t T,
                                                            int k, int64_t C, uint8_t *__restrict__ xbuf) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * 4;
    const int pieces = row_bytes >> 4;
    for (int64_t a = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); a < T * k; a += nwaves) {
        const int s = slot[a];
        if (s < 0) continue;
        const int64_t t = a / k;
        const int e = expert_idx[a];
        const uint8_t *src = x + t * row_bytes;
        uint8_t *dst = xbuf + ((int64_t)e * C + s) * row_bytes;
        for (int q = lane; q < pieces; q += 64) st16(dst + q * 16, ld16(src + q * 16));
    }
}

}  // namespace

hipError_t launch_permute_slots(const void *x, int elem_bytes, const int32_t *expert_idx, const int32_t *slot,
                                int64_t T, int d, int k, int64_t C, void *xbuf, hipStream_t s) {
    const int64_t n = T * k;
    if (n == 0 || C == 0) return hipSuccess;
    int64_t blocks = (n + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(permute_slots_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t *>(x), d * elem_bytes, expert_idx, slot, T, k, C,
                       reinterpret_cast<uint8_t *>(xbuf));
    return hipGetLastError();
}

hipError_t launch_priority_slots(const void *x, int elem_bytes, const int32_t *expert_idx,
                                 const float *priority, const int32_t *rank, const int32_t *base,
                                 const int32_t *n_e, int64_t T, int d, int E, int k, int64_t C,
                                 uint64_t *list, int32_t *off, int32_t *slot, uint8_t *drop_mask,
                                 int32_t *expert_count, void *xbuf, hipStream_t s, int32_t *pcnt) {
    if (E > 1024) return hipErrorInvalidValue;
    const int64_t n = T * k;
    const int nblk = dispatch_blocks(T);
    const unsigned lb = (unsigned)((n + PR_BLOCK - 1) / PR_BLOCK);
    // split the key stream when the average segment is long (few experts):
    // about 512 keys of it per block, at most 8 blocks per entry block
    int64_t ny = n / E / 512;
    ny = ny < 1 ? 1 : ny > 8 ? 8 : ny;
    if (pcnt == nullptr) ny = 1;
    int32_t *pc = ny > 1 ? pcnt : nullptr;
    if (n > 0)
        hipLaunchKernelGGL(priority_list_kernel, dim3(lb), dim3(PR_BLOCK), 0, s, expert_idx, priority, rank,
                           base, n_e, T, E, k, nblk, list, off, slot, drop_mask, pc);
    else
        hipLaunchKernelGGL(priority_list_kernel, dim3(1), dim3(PR_BLOCK), 0, s, expert_idx, priority, rank,
                           base, n_e, T, E, k, nblk, list, off, slot, drop_mask, pc);
    // the lists hold at most T k entries
    hipLaunchKernelGGL(priority_slot_kernel, dim3(lb > 0 ? lb : 1, (unsigned)ny), dim3(PR_BLOCK), 0, s, list, off,
                       n_e, base, E, k, nblk, C, slot, drop_mask, expert_count, pc, 0);
    if (ny > 1)
        hipLaunchKernelGGL(priority_slot_kernel, dim3(lb > 0 ? lb : 1), dim3(PR_BLOCK), 0, s, list, off, n_e, base,
                           E, k, nblk, C, slot, drop_mask, expert_count, pc, 1);
    if (n == 0 || C == 0) return hipGetLastError();
    int64_t blocks = (n + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(permute_slots_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint8_t *>(x), d * elem_bytes, expert_idx, slot, T, k, C,
                       reinterpret_cast<uint8_t *>(xbuf));
    return hipGetLastError();
}

namespace {

// out[t] = gate[t k], the gate of each token's first choice (the default
// priority score of the fused forward)
__global__ __launch_bounds__(256) void first_gate_kernel(const float *__restrict__ gate, int64_t T, int k,
                                                          float *__restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t < T) out[t] = gate[t * k];
}

}  // namespace

hipError_t launch_first_gate(const float *gate, int64_t T, int k, float *out, hipStream_t s) {
    if (T > 0)
        hipLaunchKernelGGL(first_gate_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, gate, T, k, out);
    return hipGetLastError();
}

}  // namespace moe
