/*
 * moe.h -- C ABI of the Switch-Transformer MoE layer forward on MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [CS25-L5]  "Lecture05", notes on Stanford CS25 lecture 5 "Scaling
 *              Transformers through Sparsity"
 *   [SW-RES]   "Training Stability, Results & Limitations" (Switch results)
 *   [SW-GLaM]  "从 Switch Transformer 到 GLaM"
 *   [CMU-L16]  "第 16 讲 · 混合专家（MoE）", notes on CMU 10-423 lecture 16
 *
 * Conventions shared by every entry point
 *   - Sizes: T tokens, d model width, dff expert hidden width, E experts,
 *     k experts per token, C capacity (slots per expert).
 *   - Every pointer argument is a DEVICE pointer (hipMalloc'd or a torch
 *     CUDA tensor) unless stated otherwise.  All arrays are dense, row-major,
 *     16-byte aligned.  The library never allocates, frees or synchronises;
 *     every buffer is owned by the caller.  It keeps no global mutable state
 *     and is safe to call from several threads on distinct streams; the one
 *     exception is moe_router_noalloc, whose scratch is a static array per
 *     GPU (see there).
 *   - dtype: MOE_F32 or MOE_BF16 names the storage type of x, W1, W3, W2,
 *     b1, b2, the dispatch buffer, the expert outputs and y.  The router
 *     weight W_r, its bias and the gates are always fp32 ([CS25-L5]
 *     "稳定训练" and [SW-RES] section 2.1: the router runs in float32 while
 *     the experts keep bfloat16).  bf16 expert arithmetic accumulates in fp32.
 *   - Weight orientation follows [SW-GLaM] "Dense Scaling 与 MoE 的核心差异":
 *     h = W_r x and FFN(x) = W_2 sigma(W_1 x), so W_r is [E, d],
 *     W1 and W3 are [E, dff, d], W2 is [E, d, dff] (out-features x
 *     in-features, the layout of torch.nn.Linear weights).
 *   - Errors: arguments are checked before anything is enqueued; a failed
 *     check returns MOE_ERR_* and writes nothing.  After each launch the
 *     HIP launch status is checked (MOE_ERR_HIP).  Faults inside kernels
 *     surface at the caller's next synchronisation.  After an error the
 *     contents of the outputs are unspecified.
 *   - Limits: 1 <= E <= 1024, 1 <= k <= min(E, 8), d and dff multiples of 8,
 *     T * k < 2^31, capacity_factor finite and > 0.  T = 0 is accepted:
 *     nothing is routed, per-expert counts and sums are zero and the
 *     auxiliary loss is 0.
 *   - All work is enqueued on `stream` (NULL = the null stream) and the
 *     call returns without waiting.  Results are deterministic: two calls on
 *     the same inputs give bitwise identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misaligned buffer */
    MOE_ERR_UNSUPPORTED = 2,        /* unknown dtype / activation, or a size past a limit */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4                 /* a HIP launch reported an error */
} moe_status;

/* The *_RANGE_ entries are not valid arguments: they make every 32-bit int a
 * value of the type, so that an unknown code passed by a C caller reaches the
 * argument checks (MOE_ERR_UNSUPPORTED) as a defined value in C++ as well. */
typedef enum {
    MOE_F32 = 0,
    MOE_BF16 = 1,
    MOE_DTYPE_RANGE_LO_ = -0x7fffffff - 1,
    MOE_DTYPE_RANGE_HI_ = 0x7fffffff
} moe_dtype;
typedef enum {
    MOE_ACT_RELU = 0,
    MOE_ACT_SWIGLU = 1,
    MOE_ACT_RANGE_LO_ = -0x7fffffff - 1,
    MOE_ACT_RANGE_HI_ = 0x7fffffff
} moe_act;

/* Overflow policy of moe_forward_policy (range markers as above). */
typedef enum {
    MOE_POLICY_PRIORITY = 1,
    MOE_POLICY_REROUTE = 2,
    MOE_POLICY_RANGE_LO_ = -0x7fffffff - 1,
    MOE_POLICY_RANGE_HI_ = 0x7fffffff
} moe_policy;

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_string(int status);

/*
 * The digest of the kernel sources this library was built from (16 hex
 * digits of a sha256 over the csrc/ files with comments and blank space
 * removed; static string, never NULL).  A caller that holds the sources can
 * compare it with their digest to tell a stale build; the Python binding
 * refuses to load a library whose digest differs from its tree's.
 */
const char *moe_source_digest(void);

/*
 * Expert capacity C = ceil(capacity_factor * k * T / E - 1e-9), clamped to
 * [0, T].  Host function, no GPU work.
 * [SW-GLaM] "Expert Capacity 与 Token Dropping": C = (T/N) x capacity factor;
 * [CMU-L16] exercise 3 scales it by k (1.25 x 2 x 1024 / 8 = 320).  Rounding
 * up keeps a factor of 1 covering the even split ([CS25-L5] "Capacity
 * Factor").  Returns -1 for invalid arguments (T < 0, E < 1, k < 1,
 * capacity_factor not finite or <= 0).
 */
int64_t moe_capacity(int64_t T, int32_t E, int32_t k, double capacity_factor);

/* Workspace bytes needed by moe_router / moe_dispatch / moe_expert_ffn /
 * moe_forward for the given sizes (host functions).  0 means "none";
 * SIZE_MAX means the sizes are invalid. */
size_t moe_router_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k);
size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k);
size_t moe_dispatch_priority_workspace_bytes(int64_t T, int32_t E, int32_t k);
size_t moe_router_backward_workspace_bytes(int64_t T, int32_t d, int32_t E);
size_t moe_dispatch_reroute_workspace_bytes(int64_t T, int32_t E);
size_t moe_expert_ffn_workspace_bytes(int32_t E, int64_t C, int32_t dff, moe_dtype dt);
size_t moe_workspace_bytes(int64_t T, int32_t d, int32_t dff, int32_t E, int32_t k,
                           int64_t C, moe_dtype dt, moe_act act);

/*
 * Where moe_forward keeps its intermediates inside `ws` (byte offsets), so
 * a caller can read them after the call: slot [T,k] int32, expert_count [E]
 * int32, route_count [E] int32, prob_sum [E] fp32, the dispatch buffer
 * xbuf [E,C,d] and the expert outputs ybuf [E,C,d] (storage dtype), and
 * row_tok [E,C] int32 (the token of each kept expert row).
 * With bf16 and T, C > 0 the forward does not write xbuf (the first expert
 * GEMM reads the token rows of x through row_tok); with bf16, T, C > 0 and
 * k = 1 it does not write ybuf either (the second GEMM writes each gated row
 * straight to y).  The f32 forward writes xbuf and ybuf, not row_tok.
 * Returns MOE_OK or MOE_ERR_INVALID_ARGUMENT.  Host function.
 */
typedef struct {
    size_t slot, expert_count, route_count, prob_sum, xbuf, ybuf, row_tok, total;
} moe_ws_layout;
moe_status moe_forward_workspace_layout(int64_t T, int32_t d, int32_t dff, int32_t E,
                                        int32_t k, int64_t C, moe_dtype dt, moe_act act,
                                        moe_ws_layout *out /* host pointer */);

/*
 * Router: logits, softmax, top-k selection and gates for every token.
 * [SW-GLaM] "Dense Scaling 与 MoE 的核心差异" (h(x) = W_r x, softmax) and
 * "Switch Transformer：把 MoE 做简单" (i* = argmax p, gate p_{i*});
 * [CMU-L16] section 2.3 (top-k keeps k logits, softmax over them).
 *   x           [T, d]  storage dtype
 *   W_r         [E, d]  fp32;  b_r [E] fp32 added to the logits, or NULL
 *   expert_idx  [T, k]  int32 out, best first; ties go to the lower index
 *                       ([CMU-L16] section 2.3: an all-zero router picks
 *                       the lowest-indexed experts)
 *   gate        [T, k]  fp32 out; k = 1: full-softmax probability of the
 *                       chosen expert; k >= 2: softmax over the k kept logits
 *   prob_sum    [E]     fp32 out, sum over tokens of the softmax p_i(x)
 *   route_count [E]     int32 out, number of (token, rank) choices per expert
 *                       (before capacity)
 *   z_loss      [1]     fp32 out, or NULL: the router z-loss
 *                       (1/T) sum_t (log sum_i exp z_ti)^2 over the fp32
 *                       logits z ([CMU-L16] section 4.2, the z-loss of Zoph
 *                       et al.; unweighted: the training loss multiplies it,
 *                       by 0.001 in OLMoE); 0 for T = 0
 *   logits      [T, E]  fp32 out, or NULL: the logits W_r x + b_r as the
 *                       softmax sees them (what moe_router_backward takes)
 *   ws          moe_router_workspace_bytes(T, d, E, k) bytes of device scratch
 *               (per-block partial sums, and for bf16 x with E <= 256 room
 *               for the exact three-part bf16 split of W_r, which the MFMA
 *               path makes there for E > 128)
 * Logits are fp32 ([SW-RES] section 2.1); non-finite inputs do not fault
 * and still give indices in [0, E).
 */
moe_status moe_router(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                      int64_t T, int32_t d, int32_t E, int32_t k,
                      int32_t *expert_idx, float *gate, float *prob_sum, int32_t *route_count,
                      float *z_loss, float *logits, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_router for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, outputs and kernels, with no workspace argument.  Its
 * scratch (the router's per-block partial rows and the three-part split of
 * W_r) lives in a static device array of moe_router_noalloc_scratch_bytes()
 * = 32 MiB that the library holds on each GPU it runs on until the process
 * ends.  The call allocates nothing: on its first call on a GPU it looks up
 * that GPU's copy of the array (hipGetSymbolAddress, with the GPU current)
 * and keeps the address.  Sizes whose router workspace,
 * moe_router_workspace_bytes(T, d, E, k), exceeds the array return
 * MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the five
 * workloads of this library need at most 10 MiB).  `stream` must belong to
 * the current device.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (two streams, or two threads) race
 * and give wrong results; calls in order on one stream are safe.  Each call
 * writes every scratch byte it reads, so nothing carries over between calls.
 * MOE_ERR_HIP if the array's address cannot be found.
 */
size_t moe_router_noalloc_scratch_bytes(void);
moe_status moe_router_noalloc(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                              int64_t T, int32_t d, int32_t E, int32_t k,
                              int32_t *expert_idx, float *gate, float *prob_sum, int32_t *route_count,
                              float *z_loss, float *logits, hipStream_t stream);

/*
 * Noisy top-k router: moe_router on the logits
 *   H = W_r x (+ b_r) + noise * softplus(W_noise x)
 * ([CMU-L16] section 2.3, the noisy top-k of Shazeer et al.: a learned,
 * input-dependent noise scale lets a token reach a lower choice; the page's
 * formula image is missing, and this is the form of the paper it cites).
 * H takes the place of the logits for the softmax, the selection and its
 * tie rule, the gates, prob_sum, route_count and z_loss.
 *   W_noise     [E, d]  fp32 noise weights
 *   noise       [T, E]  fp32 standard normal draws (the caller draws them)
 * Other arguments and the workspace as moe_router.  bf16 x with E <= 256
 * runs the MFMA router on W_r and W_noise (the same exact fp32 products as
 * moe_router); fp32 x, or E up to 1024, the fp32 FMA path.
 * The dispatch, expert and combine entry points take its outputs unchanged.
 */
moe_status moe_router_noisy(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                            const float *W_noise, const float *noise, int64_t T, int32_t d,
                            int32_t E, int32_t k, int32_t *expert_idx, float *gate,
                            float *prob_sum, int32_t *route_count, float *z_loss, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Dispatch: capacity slots in token order and the expert-major permutation.
 * [CS25-L5] "Capacity Factor 与 Token Dropping" (capacity-aware dispatch:
 * tokens in order fill their expert's C slots, overflow skips the expert);
 * [CMU-L16] section 6.1 (first choices of all tokens are placed before any
 * second choice); [SW-GLaM] "All-to-All" (data-sharded -> expert-sharded
 * layout, here a permutation inside one GPU's memory).
 *   expert_idx   [T, k]     int32 in, values in [0, E)
 *   C            capacity (0 <= C <= T), e.g. from moe_capacity
 *   slot         [T, k]     int32 out, slot within the expert or -1 if dropped
 *   drop_mask    [T, k]     uint8 out, 1 = this choice was dropped
 *   expert_count [E]        int32 out, kept choices per expert (<= C)
 *   xbuf         [E, C, d]  storage dtype out; row s of expert e holds x of the
 *                           token in slot s; rows >= expert_count[e] are
 *                           left untouched
 */
moe_status moe_dispatch(const void *x, moe_dtype dt, const int32_t *expert_idx,
                        int64_t T, int32_t d, int32_t E, int32_t k, int64_t C,
                        int32_t *slot, uint8_t *drop_mask, int32_t *expert_count, void *xbuf,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Priority dispatch: moe_dispatch with the capacity spent on the highest
 * scores first.  [CS25-L5], the V-MoE part after "什么是视觉 token" (with a
 * capacity factor below 1, tokens are ranked by importance and the
 * high-priority ones take the expert slots).  Tokens are visited in
 * descending priority[t] (equal scores: lower token index first; NaN scores
 * last; -0 equals +0), every first choice before any second choice; each
 * takes its expert's next free slot while fewer than C are taken.
 *   priority     [T]  fp32 in, the tokens' scores (the page leaves the score
 *                     open; the router's gate of each token's first choice,
 *                     gate[:, 0], is the plain one)
 * Other arguments as moe_dispatch; the workspace is
 * moe_dispatch_priority_workspace_bytes(T, E, k) bytes (8 T k + small).
 * E <= 1024.  Cost: about n_e^2 / 2 key compares per expert (n_e its
 * choices before capacity), at most (T k)^2 / 2 when all choices go to one
 * expert; T k is limited to 2^20 (MOE_ERR_UNSUPPORTED above it), which keeps
 * that worst case well under a second.
 */
moe_status moe_dispatch_priority(const void *x, moe_dtype dt, const int32_t *expert_idx,
                                 const float *priority, int64_t T, int32_t d, int32_t E, int32_t k,
                                 int64_t C, int32_t *slot, uint8_t *drop_mask, int32_t *expert_count,
                                 void *xbuf, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Top-1 dispatch with multi-stage re-routing of the overflow.
 * [CS25-L5] "“No Token Left Behind”为何没有成功" (a token whose expert is
 * full is sent to its second, then third choice until it gets a slot; the
 * page reports that this did not improve the model).  Stage s = 0 ..
 * stages-1 visits the tokens still without a slot in token order and offers
 * each its choice pref[t, s]; the experts fill from where the earlier stages
 * left them, C slots each.  One stage is moe_dispatch with k = 1.
 *   pref         [T, R]  int32 in, each token's experts in preference order
 *                        (moe_router's expert_idx with k = R), 1 <= stages <= R;
 *                        an entry outside [0, E) is no choice: the token stays
 *                        unplaced at that stage and is offered its next entry
 *                        at the next one (a shorter list, padded with -1)
 *   logits       [T, E]  fp32 in (moe_router's logits output), or NULL
 *   expert       [T]     int32 out, the expert the token landed on, -1 if dropped
 *   slot         [T]     int32 out, its slot, -1 if dropped
 *   drop_mask    [T]     uint8 out
 *   gate         [T]     fp32 out (NULL exactly when logits is NULL): the
 *                        full-softmax probability of the landing expert, 0
 *                        if dropped (the top-1 gate of that expert)
 *   expert_count [E]     int32 out; xbuf [E, C, d] out as moe_dispatch
 * expert and slot feed moe_expert_ffn / moe_combine as a k = 1 routing.
 * ws: moe_dispatch_reroute_workspace_bytes(T, E) bytes.
 */
moe_status moe_dispatch_reroute(const void *x, moe_dtype dt, const int32_t *pref, const float *logits, int64_t T,
                                int32_t d, int32_t E, int32_t R, int32_t stages, int64_t C, int32_t *expert,
                                int32_t *slot, uint8_t *drop_mask, float *gate, int32_t *expert_count, void *xbuf,
                                void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Combine backward: the gradients of moe_combine's y with respect to the
 * gates and the expert outputs, given dy = dL/dy.  y is linear in both
 * ([CS25-L5] "Switch Layer"): for a kept choice (t, j) at expert e, slot s,
 *   dgate[t, j]        = <dy_t, ybuf[e, s]>   (fp32 sum over d)
 *   dybuf[e, s, :]     = gate[t, j] * dy_t    (rounded to the storage dtype)
 * and a dropped choice gets dgate = 0 (its dybuf rows are not written).
 *   dy [T, d] and ybuf [E, C, d] in the storage dtype; expert_idx, slot,
 *   gate as moe_combine; dgate [T, k] fp32 out; dybuf [E, C, d] out, only
 *   the kept rows written (the caller clears it if it needs the rest).
 */
moe_status moe_combine_backward(const void *dy, moe_dtype dt, const void *ybuf, const int32_t *expert_idx,
                                const int32_t *slot, const float *gate, int64_t T, int32_t d, int32_t E,
                                int32_t k, int64_t C, float *dgate, void *dybuf, hipStream_t stream);

/*
 * Router backward: the gradient of
 *   L = sum_tj dgate[t, j] g_tj + alpha N sum_i f_i P_i + z_weight z_loss
 * with the choices held fixed, to the logits, W_r, b_r and x.  g are the
 * gates of moe_router (k = 1: full-softmax probability of the choice;
 * k >= 2: softmax over the kept logits), f_i = route_count_i / (k T) is a
 * constant ([CMU-L16] exercise 2: the balance loss's gradient with respect
 * to p_i(x_t) is alpha N f_i / T) and z_loss is moe_router's.  The top-k
 * choice carries no gradient.
 *   x [T, d] (storage dtype), W_r [E, d] fp32, logits [T, E] fp32 (from
 *   moe_router), expert_idx / gate / route_count from moe_router, dgate
 *   [T, k] fp32 (from moe_combine_backward), alpha and z_weight the loss
 *   weights (0 leaves a term out).
 *   dlogits [T, E] fp32 out, dL/dz
 *   dW_r    [E, d] fp32 out, dlogits^T x (fp32, fixed order: partial sums
 *           over chunks of 128, 256 or 512 tokens, the size fixed by T, d
 *           and E, then their sum in chunk order)
 *   db_r    [E] fp32 out or NULL, sum_t dlogits_t
 *   dx      [T, d] fp32 out or NULL, the router's part of dL/dx, dlogits W_r
 *   ws      moe_router_backward_workspace_bytes(T, d, E) bytes of scratch
 * W_r and dx must be 16-byte aligned; T up to 65535 * 512 tokens
 * (MOE_ERR_UNSUPPORTED beyond).
 */
moe_status moe_router_backward(const void *x, moe_dtype dt, const float *W_r, const float *logits,
                               const int32_t *expert_idx, const float *gate, const float *dgate,
                               const int32_t *route_count, int64_t T, int32_t d, int32_t E, int32_t k,
                               float alpha, float z_weight, float *dlogits, float *dW_r, float *db_r,
                               float *dx, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Expert FFN backward: the gradients of moe_expert_ffn given
 * dybuf = dL/d(expert output) (moe_combine_backward's dybuf).  [CMU-L16]
 * exercise 2 and section 5: each expert is an ordinary FFN on its routed
 * rows, so the backward is the chain rule through both products and the
 * activation, with the pre-activations A = W1 x + b1 (and G = W3 x)
 * recomputed from xbuf:
 *   dH = dY W2;  dW2 = dY^T H;  db2 = column sums of dY
 *   ReLU:   dA = dH * 1[A > 0]                (the derivative at A = 0 is 0)
 *   SwiGLU: dA = dH * G * silu'(A), dG = dH * silu(A)
 *   dX = dA W1 (+ dG W3);  dW1 = dA^T X;  dW3 = dG^T X;  db1 = column sums of dA
 *   xbuf, expert_count, W1, b1, W3, W2, act as moe_expert_ffn (the forward's
 *     inputs; b2 does not enter the backward)
 *   dybuf [E, C, d] in, rows < expert_count[e] read
 *   dxbuf [E, C, d] out, rows < expert_count[e] written (dL/d(expert input))
 *   dW1, dW3 [E, dff, d], dW2 [E, d, dff] out (dW3 exactly when W3 is given)
 *   db1 [E, dff], db2 [E, d] out or NULL (ReLU only)
 * Outputs in the storage dtype; sums in fp32; A, G, H, dH, dA and dG are
 * rounded to the storage dtype in between, as the forward rounds H.
 * ws: moe_expert_ffn_backward_workspace_bytes(E, C, d, dff, dt, act) bytes
 * (the transposed weights, the recomputed activations and their transposes).
 */
size_t moe_expert_ffn_backward_workspace_bytes(int32_t E, int64_t C, int32_t d, int32_t dff, moe_dtype dt,
                                              moe_act act);
moe_status moe_expert_ffn_backward(const void *xbuf, moe_dtype dt, const int32_t *expert_count, int32_t E,
                                   int64_t C, int32_t d, int32_t dff, const void *W1, const void *b1,
                                   const void *W3, const void *W2, moe_act act, const void *dybuf, void *dxbuf,
                                   void *dW1, void *dW3, void *dW2, void *db1, void *db2, void *ws,
                                   size_t ws_bytes, hipStream_t stream);

/*
 * Dispatch backward (the un-permute of the gradients): the adjoint of
 * moe_dispatch's copy.  The dispatch sent x_t to row slot[t, j] of expert
 * expert_idx[t, j] for every kept choice ([SW-GLaM] "All-to-All"); its
 * transpose gathers those rows back and adds them per token:
 *   dx_t = dx_add_t + sum over kept j (rank order) of dxbuf[e_tj, slot_tj]
 * in fp32; a dropped choice adds nothing (the token's residual path carries
 * its gradient).
 *   dxbuf [E, C, d] in (storage dtype; moe_expert_ffn_backward's dxbuf)
 *   expert_idx, slot [T, k] as moe_combine
 *   dx_add [T, d] fp32 in or NULL (moe_router_backward's dx, the router's share)
 *   dx [T, d] fp32 out (may be dx_add itself)
 */
moe_status moe_dispatch_backward(const void *dxbuf, moe_dtype dt, const int32_t *expert_idx, const int32_t *slot,
                                 int64_t T, int32_t d, int32_t E, int32_t k, int64_t C, const float *dx_add,
                                 float *dx, hipStream_t stream);

/*
 * Experts: every expert's FFN on its kept rows, as grouped GEMMs.
 * ReLU expert y = W_2 relu(W_1 x + b_1) + b_2 ([SW-GLaM] FFN equation;
 * [CMU-L16] section 2.1); SwiGLU expert y = W_2 (silu(W_1 x) * (W_3 x))
 * ([CMU-L16] section 2.3, Swish with beta = 1; b1 and b2 must be NULL).
 *   xbuf  [E, C, d] in, rows < expert_count[e] are read
 *   W1, W3 [E, dff, d]; W2 [E, d, dff]; b1 [E, dff] or NULL; b2 [E, d] or NULL
 *   ybuf  [E, C, d] out, rows < expert_count[e] written, others untouched
 * The hidden activations go through `ws` in the storage dtype.
 */
moe_status moe_expert_ffn(const void *xbuf, moe_dtype dt, const int32_t *expert_count,
                          int32_t E, int64_t C, int32_t d, int32_t dff,
                          const void *W1, const void *b1, const void *W3, const void *W2,
                          const void *b2, moe_act act,
                          void *ybuf, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Combine and auxiliary loss.
 * y_t = sum over kept choices j of gate[t,j] * ybuf[expert_idx[t,j], slot[t,j]]
 * ([CS25-L5] "Switch Layer": gate times expert output; [CMU-L16] section
 * 2.3), summed in fp32 in rank order and rounded once to the storage dtype.
 * A dropped choice contributes 0 and gates are not renormalised; a token
 * with every choice dropped gets y = 0 (it continues on the residual path,
 * which the caller adds: [CS25-L5] "Capacity Factor", [CMU-L16] section 6.1).
 * aux_loss[0] = alpha * E * sum_i f_i P_i with f_i = route_count_i / (k T)
 * and P_i = prob_sum_i / T ([SW-GLaM] "负载均衡"), fp32, computed on the
 * device in fp64.
 */
moe_status moe_combine(const void *ybuf, moe_dtype dt, const int32_t *expert_idx,
                       const int32_t *slot, const float *gate, const float *prob_sum,
                       const int32_t *route_count, int64_t T, int32_t d, int32_t E, int32_t k,
                       int64_t C, float alpha, void *y, float *aux_loss, hipStream_t stream);

/*
 * The whole layer: router, dispatch, experts, combine and loss, enqueued
 * back to back with C = moe_capacity(T, E, k, capacity_factor).  Outputs
 * y [T,d] (storage dtype, MoE branch only), aux_loss [1] fp32, z_loss [1]
 * fp32 or NULL (the router z-loss, as moe_router), expert_idx [T,k] int32,
 * gate [T,k] fp32, drop_mask [T,k] uint8; every other intermediate stays in
 * `ws` (see moe_forward_workspace_layout).
 * The results are those of moe_router, moe_dispatch, moe_expert_ffn and
 * moe_combine called in turn, bit for bit; with bf16 the forward fuses the
 * dispatch copy into the first expert GEMM (it reads the token rows of x
 * directly) and, with k = 1, the combine into the second (each expert row is
 * scaled by its gate and written to its token's row of y).
 */
moe_status moe_forward(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                       const void *W1, const void *b1, const void *W3, const void *W2,
                       const void *b2, moe_act act, int64_t T, int32_t d, int32_t dff,
                       int32_t E, int32_t k, double capacity_factor, float alpha,
                       void *y, float *aux_loss, float *z_loss, int32_t *expert_idx, float *gate,
                       uint8_t *drop_mask, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward with stage timing: identical work and results, plus HIP events
 * recorded on `stream` at the stage boundaries, for callers that time the
 * stages of the layer ([CS25-L5] "Capacity Factor" asks that dispatch
 * traffic and step time be logged alongside the routing statistics).
 * stage_events [MOE_STAGE_EVENTS] host array of caller-created events:
 *   [0] start  [1] after router  [2] after dispatch (slots, permutation or
 *   row index, GEMM tile map)  [3] after expert GEMM 1 (+activation)  [4]
 *   after expert GEMM 2 (+gated scatter to y when fused)  [5] after combine
 *   and loss (nothing is enqueued between [4] and [5] when the second GEMM
 *   wrote y).
 * NULL array or NULL entries -> MOE_ERR_INVALID_ARGUMENT, nothing enqueued.
 */
#define MOE_STAGE_EVENTS 6
/*
 * moe_forward with the noisy top-k router of moe_router_noisy: the logits
 * H = W_r x (+ b_r) + noise * softplus(W_noise x) drive the routing, the
 * gates, the loss and z_loss ([CMU-L16] section 2.3).  W_noise [E, d] fp32
 * (16-byte aligned), noise [T, E] fp32 standard normal draws; everything
 * else, the workspace included, as moe_forward.
 */
moe_status moe_forward_noisy(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                             const float *W_noise, const float *noise, const void *W1, const void *b1,
                             const void *W3, const void *W2, const void *b2, moe_act act, int64_t T, int32_t d,
                             int32_t dff, int32_t E, int32_t k, double capacity_factor, float alpha, void *y,
                             float *aux_loss, float *z_loss, int32_t *expert_idx, float *gate,
                             uint8_t *drop_mask, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The fused layer with an overflow policy in place of the plain capacity rule
 * (the same router, expert FFN, combine and losses as moe_forward, and the
 * dispatch of moe_dispatch_priority or moe_dispatch_reroute):
 *   MOE_POLICY_PRIORITY  [CS25-L5], the V-MoE part: the capacity
 *       C = moe_capacity(T, E, k, capacity_factor) is filled in descending
 *       priority[t] (NULL: each token's first gate, gate[t, 0]); any k.
 *       expert_idx, gate, drop_mask [T, k] as moe_forward.
 *   MOE_POLICY_REROUTE   [CS25-L5] "“No Token Left Behind”为何没有成功":
 *       k = 1; the router's top-`stages` choices are each token's
 *       preferences (1 <= stages <= min(E, 8)) and stage s offers the tokens
 *       still without a slot their choice s, C = moe_capacity(T, E, 1,
 *       capacity_factor) slots per expert.  expert_idx [T, 1] is the expert
 *       the token landed on (-1 if dropped), gate [T, 1] the full-softmax
 *       probability of that expert (0 if dropped), drop_mask [T, 1].  The
 *       loss counts each token's first choice (f_i over the top-1 choices,
 *       before capacity).  priority must be NULL.
 * aux_loss and z_loss as moe_forward (the z-loss over all logits).
 * ws: moe_forward_policy_workspace_bytes(...) bytes (it also holds xbuf and
 * the expert outputs: this path runs the split kernels, not the fused
 * gather / scatter of moe_forward).
 */
size_t moe_forward_policy_workspace_bytes(int64_t T, int32_t d, int32_t dff, int32_t E, int32_t k,
                                          double capacity_factor, moe_dtype dt, moe_act act, moe_policy policy,
                                          int32_t stages);
moe_status moe_forward_policy(const void *x, moe_dtype dt, const float *W_r, const float *b_r, const void *W1,
                              const void *b1, const void *W3, const void *W2, const void *b2, moe_act act,
                              int64_t T, int32_t d, int32_t dff, int32_t E, int32_t k, double capacity_factor,
                              float alpha, moe_policy policy, const float *priority, int32_t stages, void *y,
                              float *aux_loss, float *z_loss, int32_t *expert_idx, float *gate,
                              uint8_t *drop_mask, void *ws, size_t ws_bytes, hipStream_t stream);

moe_status moe_forward_staged(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                              const void *W1, const void *b1, const void *W3, const void *W2,
                              const void *b2, moe_act act, int64_t T, int32_t d, int32_t dff,
                              int32_t E, int32_t k, double capacity_factor, float alpha,
                              void *y, float *aux_loss, float *z_loss, int32_t *expert_idx,
                              float *gate, uint8_t *drop_mask, void *ws, size_t ws_bytes,
                              hipStream_t stream, hipEvent_t *stage_events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
