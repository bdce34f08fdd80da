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
// below C) and a pass that advances fill[e] = min(fill[e] + n_e, C).  A
// final pass writes the drop flags, the expert counts and each token's gate,
// the full-softmax probability of the expert it landed on.
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

__global__ __launch_bounds__(256) void reroute_place_kernel(const int32_t *__restrict__ cand,
                                                            const int32_t *__restrict__ rank,
                                                            const int32_t *__restrict__ base,
                                                            const int32_t *__restrict__ fill, int64_t T, int nblk,
                                                            int64_t C, int s, int32_t *__restrict__ expert,
                                                            int32_t *__restrict__ slot) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const int e = cand[t];
    int64_t sl = -1;
    if (e >= 0) {
        const int blk = (int)(t / DISPATCH_TOK_BLOCK);
        sl = (int64_t)(s == 0 ? 0 : fill[e]) + base[(int64_t)e * nblk + blk] + rank[t];
        if (sl >= C) sl = -1;
    }
    if (sl >= 0) {
        expert[t] = e;
        slot[t] = (int32_t)sl;
    } else if (s == 0) {
        expert[t] = -1;
        slot[t] = -1;
    }
}

__global__ __launch_bounds__(256) void reroute_fill_kernel(const int32_t *__restrict__ n_e,
                                                           int32_t *__restrict__ fill, int E, int64_t C, int s) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const int64_t f = (int64_t)(s == 0 ? 0 : fill[e]) + n_e[e];
    fill[e] = (int32_t)(f < C ? f : C);
}

// One wave per token: drop flag and gate; block 0 also copies the counts.
__global__ __launch_bounds__(256) void reroute_final_kernel(const float *__restrict__ logits,
                                                            const int32_t *__restrict__ expert,
                                                            const int32_t *__restrict__ fill, int64_t T, int E,
                                                            uint8_t *__restrict__ drop, float *__restrict__ gate,
                                                            int32_t *__restrict__ expert_count) {
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e < E; e += 256) expert_count[e] = fill[e];
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
                          int32_t *hist, int32_t *cand, int32_t *n_e, int32_t *fill, hipStream_t s) {
    if (stages < 1 || stages > R) return hipErrorInvalidValue;
    const int nblk = dispatch_blocks(T);
    const unsigned tb = (unsigned)((T + 255) / 256);
    const unsigned eb = (unsigned)((E + 255) / 256);
    for (int st = 0; st < stages; ++st) {
        if (T > 0) hipLaunchKernelGGL(reroute_cand_kernel, dim3(tb), dim3(256), 0, s, pref, R, st, T, E, expert, cand);
        hipError_t err = launch_slot_rank(cand, T, E, 1, rank, hist, nullptr, s);
        if (err != hipSuccess) return err;
        err = launch_slot_scan(hist, nblk, E, 1, T + 1, n_e, nullptr, 0, nullptr, nullptr, nullptr, 0, nullptr, s);
        if (err != hipSuccess) return err;
        if (T > 0)
            hipLaunchKernelGGL(reroute_place_kernel, dim3(tb), dim3(256), 0, s, cand, rank, hist, fill, T, nblk, C,
                               st, expert, slot);
        hipLaunchKernelGGL(reroute_fill_kernel, dim3(eb), dim3(256), 0, s, n_e, fill, E, C, st);
    }
    const unsigned fb = (unsigned)((T + 3) / 4);
    hipLaunchKernelGGL(reroute_final_kernel, dim3(fb > 0 ? fb : 1), dim3(256), 0, s, logits, expert, fill, T, E,
                       drop_mask, gate, expert_count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_permute_slots(x, elem_bytes, expert, slot, T, d, 1, C, xbuf, s);
}

}  // namespace moe
