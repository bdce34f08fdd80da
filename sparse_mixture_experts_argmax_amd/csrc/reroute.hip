// Top-1 dispatch with multi-stage re-routing of the overflow.
//
// [CS25-L5] "“No Token Left Behind”为何没有成功": a token whose top-1 expert
// is full goes to its second choice, then its third, until it gets a slot
// (the page reports that this did not improve the model).  Stage s offers
// every token still without a slot its choice of rank s, in token order,
// and fills the experts from where the earlier stages left them; stage 0
// alone is the plain capacity rule.
//
// Each stage is the plain dispatch's rank and scan passes (one rank, an
// unbounded capacity) over a candidate array that holds the stage's choice
// of the unplaced tokens and -1 for the rest, then a placement pass
// (slot = fill[e] + position among the stage's candidates of e, kept while
// below C, with fill[e] folded from the earlier stages' counts as
// min(fill + n_e, C)), which also writes the next stage's candidates: three
// launches per stage.  A final pass writes the drop flags, the expert counts
// and each token's gate, the full-softmax probability of the expert it
// landed on.
#include "common.h"
#include "launch.h"

#include <math.h>

namespace moe {

namespace {

__global__ __launch_bounds__(256) void reroute_cand_kernel(const int32_t *__restrict__ pref, int R, int s,
                                                           int64_t T, int E, const int32_t *__restrict__ expert,
                                                           int32_t *__restrict__ cand) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    int e = -1;
    if (s == 0 || expert[t] < 0) {
        e = pref[t * R + s];
        if (e < 0 || e >= E) e = -1;
    }
    cand[t] = e;
}

// Stage s's placement: slot = (the expert's fill after the earlier stages) +
// the candidate's position among this stage's candidates of its expert, kept
// while below C.  The fill after stage q is min(fill after q - 1 + n_q, C),
// folded here from the per-stage counts n_e [stages][E] (no pass of its own).
// Unless this is the last stage, each thread then writes its token's next
// candidate in place: the next preference (or -1 past [0, E)) while the
// token has no slot, -1 once it has one.
__global__ __launch_bounds__(256) void reroute_place_kernel(int32_t *__restrict__ cand,
                                                            const int32_t *__restrict__ rank,
                                                            const int32_t *__restrict__ base,
                                                            const int32_t *__restrict__ n_hist, int64_t T, int nblk,
                                                            int64_t C, int s, int E, const int32_t *__restrict__ pref,
                                                            int R, bool last, int32_t *__restrict__ expert,
                                                            int32_t *__restrict__ slot) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const int e = cand[t];
    int64_t sl = -1;
    if (e >= 0) {
        int64_t f = 0;
        for (int q = 0; q < s; ++q) {
            f += n_hist[(int64_t)q * E + e];
            f = f < C ? f : C;
        }
        const int blk = (int)(t / DISPATCH_TOK_BLOCK);
        sl = f + base[(int64_t)e * nblk + blk] + rank[t];
        if (sl >= C) sl = -1;
    }
    int landed;
    if (sl >= 0) {
        expert[t] = e;
        slot[t] = (int32_t)sl;
        landed = e;
    } else if (s == 0) {
        expert[t] = -1;
        slot[t] = -1;
        landed = -1;
    } else {
        landed = expert[t];                          // placed at an earlier stage, or not yet
    }
    if (!last) {
        int nx = -1;
        if (landed < 0) {
            nx = pref[t * R + s + 1];
            if (nx < 0 || nx >= E) nx = -1;
        }
        cand[t] = nx;
    }
}

// One wave per token: drop flag and gate; block 0 also writes the counts
// (each expert's fill after the last stage, folded from the stage counts).
__global__ __launch_bounds__(256) void reroute_final_kernel(const float *__restrict__ logits,
                                                            const int32_t *__restrict__ expert,
                                                            const int32_t *__restrict__ n_hist, int stages,
                                                            int64_t C, int64_t T, int E,
                                                            uint8_t *__restrict__ drop, float *__restrict__ gate,
                                                            int32_t *__restrict__ expert_count) {
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e < E; e += 256) {
            int64_t f = 0;
            for (int q = 0; q < stages; ++q) {
                f += n_hist[(int64_t)q * E + e];
                f = f < C ? f : C;
            }
            expert_count[e] = (int32_t)f;
        }
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int e = expert[t];
    if (lane == 0) drop[t] = e < 0 ? 1 : 0;
    if (gate == nullptr) return;
    const float *z = logits + t * E;
    float mx = -INFINITY;
    for (int n = lane; n < E; n += 64) mx = fmaxf(mx, z[n]);
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
    float sum = 0.f;
    for (int n = lane; n < E; n += 64) sum += expf(z[n] - mx);
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m);
    if (lane == 0) gate[t] = e >= 0 ? expf(z[e] - mx) / sum : 0.f;
}

}  // namespace

hipError_t launch_reroute(const void *x, int elem_bytes, const int32_t *pref, const float *logits, int64_t T,
                          int d, int E, int R, int stages, int64_t C, int32_t *expert, int32_t *slot,
                          uint8_t *drop_mask, float *gate, int32_t *expert_count, void *xbuf, int32_t *rank,
                          int32_t *hist, int32_t *cand, int32_t *n_e, hipStream_t s) {
    if (stages < 1 || stages > R || stages > REROUTE_MAX_STAGES) return hipErrorInvalidValue;
    const int nblk = dispatch_blocks(T);
    const unsigned tb = (unsigned)((T + 255) / 256);
    // stage 0's candidates; each placement pass writes the next stage's
    if (T > 0) hipLaunchKernelGGL(reroute_cand_kernel, dim3(tb), dim3(256), 0, s, pref, R, 0, T, E, expert, cand);
    for (int st = 0; st < stages; ++st) {
        hipError_t err = launch_slot_rank(cand, T, E, 1, rank, hist, nullptr, s);
        if (err != hipSuccess) return err;
        // an unbounded capacity: n_e[st] = this stage's candidates per expert
        err = launch_slot_scan(hist, nblk, E, 1, T + 1, n_e + (int64_t)st * E, nullptr, 0, nullptr, nullptr,
                               nullptr, 0, nullptr, s);
        if (err != hipSuccess) return err;
        if (T > 0)
            hipLaunchKernelGGL(reroute_place_kernel, dim3(tb), dim3(256), 0, s, cand, rank, hist, n_e, T, nblk, C,
                               st, E, pref, R, st == stages - 1, expert, slot);
    }
    const unsigned fb = (unsigned)((T + 3) / 4);
    hipLaunchKernelGGL(reroute_final_kernel, dim3(fb > 0 ? fb : 1), dim3(256), 0, s, logits, expert, n_e, stages, C,
                       T, E, drop_mask, gate, expert_count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_permute_slots(x, elem_bytes, expert, slot, T, d, 1, C, xbuf, s);
}

namespace {

// counts[e] = number of tokens whose first preference is e (entries outside
// [0, E) count nowhere); an LDS histogram per block, added to counts, which
// the launcher clears first.  Integer sums: the same counts in any order.
__global__ __launch_bounds__(256) void first_choice_count_kernel(const int32_t *__restrict__ pref, int64_t T, int R,
                                                                  int E, int32_t *__restrict__ counts) {
    __shared__ int h[1024];
    for (int i = threadIdx.x; i < E; i += 256) h[i] = 0;
    __syncthreads();
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < T; t += (int64_t)gridDim.x * 256) {
        const int e = pref[t * R];
        if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += 256)
        if (h[i]) atomicAdd(&counts[i], h[i]);
}

__global__ __launch_bounds__(256) void clear_i32_kernel(int32_t *__restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_first_choice_count(const int32_t *pref, int64_t T, int R, int E, int32_t *counts, hipStream_t s) {
    hipLaunchKernelGGL(clear_i32_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, counts, E);
    if (T > 0) {
        int64_t b = (T + 255) / 256;
        if (b > 1024) b = 1024;
        hipLaunchKernelGGL(first_choice_count_kernel, dim3((unsigned)b), dim3(256), 0, s, pref, T, R, E, counts);
    }
    return hipGetLastError();
}

}  // namespace moe
