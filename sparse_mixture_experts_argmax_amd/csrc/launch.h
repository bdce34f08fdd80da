// Internal launchers of the MoE kernels (called only by the C ABI layer).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---- router -----------------------------------------------------------
// Number of per-block partial rows the router writes for T tokens.
int router_blocks(int64_t T, int dtype_bf16, int E);
// w3: scratch of 3 * router_w3_rows(E) * d bf16 for the exact three-part
// split of W_r (or of the stacked noisy weight).
int router_w3_rows(int E);
// part_z [router_blocks]: each block's sum of its tokens' squared
// log-sum-exps (the router z-loss partials).  logits (may be null): the
// fp32 logits W_r x + b_r [T, E] as the softmax sees them (before the
// NaN-to-minus-infinity ranking rule).
hipError_t launch_router(const void *x, int dtype_bf16, const float *W_r, const float *b_r,
                         int64_t T, int d, int E, int k, int32_t *expert_idx, float *gate,
                         float *part_prob, int32_t *part_cnt, uint16_t *w3, hipStream_t s,
                         float *part_z, float *logits = nullptr);
// Noisy top-k router (any dtype and E; MFMA for bf16 x and E <= 256):
// logits H = W_r x (+ b_r) + eps * softplus(W_noise x), eps [T, E] given;
// partial rows as launch_router, router_noisy_blocks(T, dtype_bf16, E) of
// them; w3 as launch_router.
int router_noisy_blocks(int64_t T, int dtype_bf16, int E);
hipError_t launch_router_noisy(const void *x, int dtype_bf16, const float *W_r, const float *b_r,
                               const float *W_noise, const float *eps, int64_t T, int d, int E,
                               int k, int32_t *expert_idx, float *gate, float *part_prob,
                               int32_t *part_cnt, float *part_z, uint16_t *w3, hipStream_t s);
// z_loss (may be null): (1/T) sum of the part_z partials.
hipError_t launch_router_reduce(const float *part_prob, const int32_t *part_cnt, int nblk,
                                int E, float *prob_sum, int32_t *route_count, hipStream_t s,
                                const float *part_z, int64_t T, float *z_loss);

// ---- dispatch ---------------------------------------------------------
constexpr int DISPATCH_TOK_BLOCK = 256;
inline int dispatch_blocks(int64_t T) { return (int)((T + DISPATCH_TOK_BLOCK - 1) / DISPATCH_TOK_BLOCK); }
// done (may be null): zeroed here for the completion counter of the scan.
hipError_t launch_slot_rank(const int32_t *expert_idx, int64_t T, int E, int k, int32_t *rank,
                            int32_t *hist, unsigned *done, hipStream_t s);
// part_prob (nblk_r router partial rows) may be null; when given, the scan also
// writes the router's prob_sum and route_count (what launch_router_reduce
// would, bit for bit).  tile_map may be null; when given, the last block
// also writes the GEMM tile map for row tiles of bm (what launch_tile_map
// would), using the completion counter done that launch_slot_rank zeroed.
// aux (may be null; needs tile_map): the last block also writes the
// auxiliary loss from the totals it finished (what launch_combine would).
// z_loss (may be null; needs part_prob): the router's z-loss from its part_z
// partials (what launch_router_reduce would, bit for bit).
hipError_t launch_slot_scan(int32_t *hist, int nblk, int E, int k, int64_t C,
                            int32_t *expert_count, const float *part_prob, int nblk_r,
                            float *prob_sum, int32_t *route_count, int32_t *tile_map, int bm,
                            unsigned *done, hipStream_t s, int64_t T = 0, float alpha = 0.f,
                            float *aux = nullptr, const float *part_z = nullptr,
                            float *z_loss = nullptr);
// Slots and drops as launch_permute, but rows are not copied: row_tok[e C +
// slot] = token for every kept choice.  k = 1 only (both may be null):
// row_gate[e C + slot] = gate of that choice, and y_zero gets the rows
// (row_bytes each) of dropped tokens cleared.  tile_map (may be null): block
// 0 also writes the GEMM tile map for row tiles of bm from expert_count (what
// launch_tile_map would); aux (may be null): block 0 also writes the
// auxiliary loss from prob_sum and route_count (what launch_combine would).
// The totals come from the scan, a launch earlier.
hipError_t launch_slot_index(const int32_t *expert_idx, const int32_t *rank, const int32_t *base,
                             int64_t T, int E, int k, int64_t C, int32_t *slot, uint8_t *drop_mask,
                             int32_t *row_tok, const float *gate, float *row_gate, void *y_zero,
                             int row_bytes, hipStream_t s, const int32_t *expert_count = nullptr,
                             const float *prob_sum = nullptr, const int32_t *route_count = nullptr,
                             int32_t *tile_map = nullptr, int bm = 0, float alpha = 0.f,
                             float *aux = nullptr);
// Priority routing (priority.hip): after launch_slot_rank and a
// launch_slot_scan with an unbounded capacity (n_e = each expert's choice
// count), the slots of the capacity rule with tokens visited in descending
// priority[t] (ties: lower index; NaN last), rank-major; also drop_mask,
// expert_count = min(n_e, C) and the kept rows in xbuf.  list [T k] uint64,
// off [E] and pcnt [T k] int32 (may be null: no split count) are scratch.
// E <= 1024.
hipError_t launch_priority_slots(const void *x, int elem_bytes, const int32_t *expert_idx,
                                 const float *priority, const int32_t *rank, const int32_t *base,
                                 const int32_t *n_e, int64_t T, int d, int E, int k, int64_t C,
                                 uint64_t *list, int32_t *off, int32_t *slot, uint8_t *drop_mask,
                                 int32_t *expert_count, void *xbuf, hipStream_t s, int32_t *pcnt);
// Backward of the gate side (backward.hip).  Combine: dgate [T, k] fp32 and
// the kept rows of dybuf [E, C, d] (g dy, storage dtype).  Router: dz [T, E]
// from the logits, gates and dgate; dW [E, d], db [E] (may be null) and dx
// [T, d] (may be null), fp32; part_w [router_bwd_chunks(T, d, E)][E][d] and
// part_b [router_bwd_chunks(T, d, E)][E] are scratch.
int router_bwd_chunks(int64_t T, int d, int E);
hipError_t launch_combine_backward(const void *dy, int dtype_bf16, const void *ybuf, const int32_t *expert_idx,
                                   const int32_t *slot, const float *gate, int64_t T, int d, int E, int k,
                                   int64_t C, float *dgate, void *dybuf, hipStream_t s);
hipError_t launch_router_backward(const void *x, int dtype_bf16, const float *W_r, const float *logits,
                                  const int32_t *expert_idx, const float *gate, const float *dgate,
                                  const int32_t *route_count, int64_t T, int d, int E, int k, float alpha,
                                  float z_weight, float *dz, float *dW, float *db, float *dx, float *part_w,
                                  float *part_b, hipStream_t s);
// xbuf[expert_idx[a], slot[a]] = x[a / k] for every choice a with slot >= 0.
hipError_t launch_permute_slots(const void *x, int elem_bytes, const int32_t *expert_idx, const int32_t *slot,
                                int64_t T, int d, int k, int64_t C, void *xbuf, hipStream_t s);
// Top-1 dispatch with re-routing (reroute.hip): stage s offers the tokens
// still without a slot their choice pref[t, s] (pref [T, R]), stages <= R;
// expert [T] and slot [T] (-1 if dropped), drop_mask [T], gate [T] (the
// full-softmax probability of the landing expert from logits [T, E]; both
// may be null), expert_count [E] and the kept rows in xbuf.  rank [T], hist
// [E dispatch_blocks(T)], cand [T] and n_e [REROUTE_MAX_STAGES E] are
// scratch.  stages <= REROUTE_MAX_STAGES.
constexpr int REROUTE_MAX_STAGES = 8;
hipError_t launch_reroute(const void *x, int elem_bytes, const int32_t *pref, const float *logits, int64_t T,
                          int d, int E, int R, int stages, int64_t C, int32_t *expert, int32_t *slot,
                          uint8_t *drop_mask, float *gate, int32_t *expert_count, void *xbuf, int32_t *rank,
                          int32_t *hist, int32_t *cand, int32_t *n_e, hipStream_t s);
// counts [E] = how many tokens have e as their first preference pref[t, 0]
// (pref [T, R]); the fused re-routing forward's choice counts for the loss.
hipError_t launch_first_choice_count(const int32_t *pref, int64_t T, int R, int E, int32_t *counts, hipStream_t s);
// out [T] = gate[t, 0] of gate [T, k]: the default priority score.
hipError_t launch_first_gate(const float *gate, int64_t T, int k, float *out, hipStream_t s);
hipError_t launch_permute(const void *x, int elem_bytes, const int32_t *expert_idx,
                          const int32_t *rank, const int32_t *base, int64_t T, int d, int E,
                          int k, int64_t C, int32_t *slot, uint8_t *drop_mask, void *xbuf,
                          hipStream_t s);

// ---- experts ----------------------------------------------------------
// Row-tile height of the grouped GEMM (act: 0 none, 1 relu, 2 swiglu, the
// activation of the first GEMM; both GEMMs use the same height); tile_map
// holds E+1 prefix sums of ceil(expert_count / gemm_bm(dtype, C, act)),
// followed by TAIL_SPLIT_SLOTS completion counters of the split last wave
// (below), which every builder of the map clears.
int gemm_bm(int dtype_bf16, int64_t C, int act);
constexpr int TAIL_SPLIT_SLOTS = 256;
inline int64_t tile_map_ints(int E) { return (int64_t)E + 1 + TAIL_SPLIT_SLOTS; }
// The split last wave: a tile-map launch whose tiles leave a last wave at most
// half full splits each of those tiles' K loop over up to 8 blocks; each
// block stores its fp32 partial sums (TAIL_SPLIT_PART_FLOATS per block, at
// most TAIL_SPLIT_SLOTS blocks) and the last to finish adds them in part
// order and runs the epilogue.  Bytes of that partial buffer for a bf16
// launch over experts of capacity C (0 when none is needed: one tile per
// expert, or fp32).
constexpr int TAIL_SPLIT_PART_FLOATS = 256 * 256;
size_t tail_split_bytes(int dtype_bf16, int64_t C);
hipError_t launch_tile_map(const int32_t *expert_count, int E, int bm, int32_t *tile_map,
                           hipStream_t s);
// out[e, m, :] = act(A[e, m, :] . B[e]^T (+ bias[e]))  for m < count[e]
// act: 0 none, 1 relu, 2 swiglu (silu(A.B^T) * (A.B3^T)).
// tile_map was built for row tiles of bm = gemm_bm(dtype, C, act of the first GEMM).
// rows_bound: an upper bound of sum_e count[e] (sizes the grid).
// row_tok [E, C] (bf16 only; null = off): row m of expert e is token
// row_tok[e C + m].  With act != 0, A is x [T, K] and the expert rows are
// gathered from it; with act == 0, out is y [T, N] and each output row goes
// to its token's row scaled by row_gate[e C + m] (one choice per token).
// split_part: tail_split_bytes(dtype, C) bytes for the split last wave, or
// null (no split); the counters follow the tile map.
hipError_t launch_grouped_gemm(const void *A, const void *B, const void *B3, const void *bias,
                               int dtype_bf16, int act, const int32_t *expert_count,
                               const int32_t *tile_map, int bm, int E, int64_t C, int N, int K,
                               int64_t rows_bound, void *out, hipStream_t s,
                               const int32_t *row_tok = nullptr, int64_t T = 0,
                               const float *row_gate = nullptr, const int32_t *kcount = nullptr,
                               float *split_part = nullptr);

// ---- expert-side backward (expert_backward.hip) ----------------------------
// Byte offsets of the backward's scratch inside one workspace: tile maps and
// constant row counts, the recomputed pre-activations A (and G), dH, [dA | dG],
// the transposed weights W2t [E, f, d] and W13t [E, d, f (+ f)], and the
// transposed activations dYt, Xt [E, d, Cp], Ht, dAt (, dGt) [E, f, Cp],
// Cp = C rounded up to 64.
struct ExpertBwdWs {
    size_t tmap_r, tmap_d, tmap_f, cnt_d, cnt_f, a, g, dh, dag, w2t, w13t, dyt, xt, ht, dat, dgt, part, total;
};
ExpertBwdWs expert_backward_ws(int E, int64_t C, int d, int f, int dtype_bf16, int act);
// The gradients of the grouped expert FFN (act 1 ReLU, 2 SwiGLU) given dybuf
// = dL/d(expert output) [E, C, d]: dxbuf [E, C, d] (kept rows), dW1, dW3
// (SwiGLU), dW2 in the weights' layouts, db1 [E, f] and db2 [E, d] (may be
// null), all in the storage dtype.  ws holds expert_backward_ws(...).total bytes.
hipError_t launch_expert_backward(const void *xbuf, int dtype_bf16, const int32_t *expert_count, int E, int64_t C,
                                  int d, int f, const void *W1, const void *b1, const void *W3, const void *W2,
                                  int act, const void *dybuf, void *dxbuf, void *dW1, void *dW3, void *dW2,
                                  void *db1, void *db2, char *ws, hipStream_t s);
// dx [T, d] fp32 = dx_add (may be null) + the kept rows of dxbuf, per token.
hipError_t launch_dispatch_backward(const void *dxbuf, int dtype_bf16, const int32_t *expert_idx, const int32_t *slot,
                                    int64_t T, int d, int E, int k, int64_t C, const float *dx_add, float *dx,
                                    hipStream_t s);

// ---- combine ----------------------------------------------------------
hipError_t launch_combine(const void *ybuf, int dtype_bf16, const int32_t *expert_idx,
                          const int32_t *slot, const float *gate, const float *prob_sum,
                          const int32_t *route_count, int64_t T, int d, int E, int k, int64_t C,
                          float alpha, void *y, float *aux_loss, hipStream_t s);

}  // namespace moe
