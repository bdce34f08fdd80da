// C ABI of the MoE layer forward: argument checks, workspace carving and the
// launch sequence of every entry point.  See include/moe.h for the contract.
#include "moe.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "launch.h"

// Scratch of moe_router_noalloc: one copy per GPU, held for the life of the
// process.  Host code never uses this name as an address (on the host it is
// a stand-in); noalloc_scratch() returns the device address of the current
// GPU's copy.
#define MOE_NOALLOC_SCRATCH_BYTES (size_t(32) << 20)
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_E = 1024;
constexpr int MAX_K = 8;
constexpr int64_t MAX_DIM = 1 << 20;
constexpr int64_t PRIORITY_MAX_CHOICES = int64_t(1) << 20;   // T k of moe_dispatch_priority

size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
size_t esize(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }
bool act_ok(int a) { return a == MOE_ACT_RELU || a == MOE_ACT_SWIGLU; }

// Router partial rows are sized for the smaller token tile of the two router kernels.
constexpr int64_t ROUTER_MIN_TOK = 8;

struct RouterWs {
    size_t part_prob, part_cnt, part_z, w3, total;
};
RouterWs router_ws(int64_t T, int d, int E) {
    RouterWs w;
    const int64_t nblk = (T + ROUTER_MIN_TOK - 1) / ROUTER_MIN_TOK;
    w.part_prob = 0;
    w.part_cnt = up((size_t)nblk * E * 4);
    w.part_z = w.part_cnt + up((size_t)nblk * E * 4);
    w.w3 = w.part_z + up((size_t)nblk * 4);
    // three bf16 parts of W_r, or of the stacked noisy weight
    w.total = w.w3 + up((size_t)3 * moe::router_w3_rows(E) * d * 2);
    return w;
}

struct DispatchWs {
    size_t rank, hist, done, total;
};
DispatchWs dispatch_ws(int64_t T, int E, int k) {
    DispatchWs w;
    w.rank = 0;
    w.hist = up((size_t)T * k * 4);
    w.done = w.hist + up((size_t)E * k * moe::dispatch_blocks(T) * 4);
    w.total = w.done + up(4);
    return w;
}

// Priority dispatch: the plain dispatch's rank and scan scratch, then the
// per-expert order-key lists, the choice counts and the list offsets.
struct PriorityWs {
    DispatchWs d;
    size_t list, cnt, off, pcnt, total;
};
PriorityWs priority_ws(int64_t T, int E, int k) {
    PriorityWs w;
    w.d = dispatch_ws(T, E, k);
    w.list = w.d.total;
    w.cnt = w.list + up((size_t)T * k * 8);
    w.off = w.cnt + up((size_t)E * 4);
    w.pcnt = w.off + up((size_t)E * 4);
    w.total = w.pcnt + up((size_t)T * k * 4);
    return w;
}

// The expert FFN's scratch: the tile map (with the split last wave's
// counters after it), the hidden activations H, and the split last wave's
// partial sums.
struct FfnWs {
    size_t tile_map, h, part, total;
};
FfnWs ffn_ws(int E, int64_t C, int dff, moe_dtype dt) {
    FfnWs w;
    w.tile_map = 0;
    w.h = up((size_t)moe::tile_map_ints(E) * 4);
    w.part = w.h + up((size_t)E * C * dff * esize(dt));
    w.total = w.part + up(moe::tail_split_bytes(dt == MOE_BF16, C));
    return w;
}

struct ForwardWs {
    RouterWs r;
    DispatchWs dsp;
    FfnWs f;
    size_t router, prob_sum, route_count, dispatch, expert_count, slot, xbuf, ffn, ybuf, row_tok,
        row_gate, total;
};
ForwardWs forward_ws(int64_t T, int d, int dff, int E, int k, int64_t C, moe_dtype dt) {
    ForwardWs w;
    w.r = router_ws(T, d, E);
    w.dsp = dispatch_ws(T, E, k);
    w.f = ffn_ws(E, C, dff, dt);
    size_t o = 0;
    w.router = o;        o += w.r.total;
    w.prob_sum = o;      o += up((size_t)E * 4);
    w.route_count = o;   o += up((size_t)E * 4);
    w.dispatch = o;      o += w.dsp.total;
    w.expert_count = o;  o += up((size_t)E * 4);
    w.slot = o;          o += up((size_t)T * k * 4);
    w.xbuf = o;          o += up((size_t)E * C * d * esize(dt));
    w.ffn = o;           o += w.f.total;
    w.ybuf = o;          o += up((size_t)E * C * d * esize(dt));
    w.row_tok = o;       o += up((size_t)E * C * 4);
    w.row_gate = o;      o += up((size_t)E * C * 4);
    w.total = o;
    return w;
}

// Size limits shared by the entry points.
moe_status check_sizes(int64_t T, int32_t E, int32_t k) {
    if (T < 0 || E < 1 || k < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (E > MAX_E || k > MAX_K || k > E) return MOE_ERR_UNSUPPORTED;
    if (T * (int64_t)k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}
moe_status check_width(int64_t w) {
    if (w < 8 || (w % 8) != 0) return MOE_ERR_INVALID_ARGUMENT;
    if (w > MAX_DIM) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}
// A pointer that must be present (or may be NULL when its array is empty).
bool ptr_ok(const void *p, bool empty_ok) { return (p == nullptr) ? empty_ok : aligned16(p); }
bool opt_ok(const void *p) { return p == nullptr || aligned16(p); }
// Scalars/small arrays only need natural alignment.
bool ptr4_ok(const void *p, bool empty_ok) {
    return (p == nullptr) ? empty_ok : (((uintptr_t)p & 3u) == 0);
}

#define MOE_CHECK(expr)                          \
    do {                                         \
        const moe_status st_ = (expr);           \
        if (st_ != MOE_OK) return st_;           \
    } while (0)
#define MOE_HIP(expr)                            \
    do {                                         \
        if ((expr) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

moe_status check_ffn_args(moe_dtype dt, moe_act act, const void *W1, const void *b1,
                          const void *W3, const void *W2, const void *b2) {
    if (!dtype_ok(dt) || !act_ok(act)) return MOE_ERR_UNSUPPORTED;
    if (!ptr_ok(W1, false) || !ptr_ok(W2, false)) return MOE_ERR_INVALID_ARGUMENT;
    if (!opt_ok(b1) || !opt_ok(b2) || !opt_ok(W3)) return MOE_ERR_INVALID_ARGUMENT;
    if (act == MOE_ACT_SWIGLU) {
        if (W3 == nullptr) return MOE_ERR_INVALID_ARGUMENT;
        if (b1 != nullptr || b2 != nullptr) return MOE_ERR_UNSUPPORTED;
    } else if (W3 != nullptr) {
        return MOE_ERR_INVALID_ARGUMENT;
    }
    return MOE_OK;
}

// reduce = false leaves prob_sum / route_count / z_loss to the dispatch scan
// (the fused forward), which reads the router's partials from ws.
moe_status run_router(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                      int64_t T, int32_t d, int32_t E, int32_t k, int32_t *expert_idx,
                      float *gate, float *prob_sum, int32_t *route_count, float *z_loss, char *ws,
                      hipStream_t stream, bool reduce = true, float *logits = nullptr,
                      const float *W_noise = nullptr, const float *noise = nullptr) {
    const RouterWs w = router_ws(T, d, E);
    float *part_prob = reinterpret_cast<float *>(ws + w.part_prob);
    int32_t *part_cnt = reinterpret_cast<int32_t *>(ws + w.part_cnt);
    float *part_z = reinterpret_cast<float *>(ws + w.part_z);
    uint16_t *w3 = reinterpret_cast<uint16_t *>(ws + w.w3);
    const int bf16 = dt == MOE_BF16;
    if (W_noise != nullptr)
        MOE_HIP(moe::launch_router_noisy(x, bf16, W_r, b_r, W_noise, noise, T, d, E, k, expert_idx, gate,
                                         part_prob, part_cnt, part_z, w3, stream));
    else
        MOE_HIP(moe::launch_router(x, bf16, W_r, b_r, T, d, E, k, expert_idx, gate, part_prob,
                                   part_cnt, w3, stream, part_z, logits));
    const int nblk = W_noise != nullptr ? moe::router_noisy_blocks(T, bf16, E) : moe::router_blocks(T, bf16, E);
    if (reduce)
        MOE_HIP(moe::launch_router_reduce(part_prob, part_cnt, nblk, E, prob_sum, route_count, stream, part_z, T,
                                          z_loss));
    return MOE_OK;
}

// part_prob != null (the fused forward): the scan also finishes the router's
// prob_sum / route_count from its nblk_r partial rows; tile_map != null: it
// also writes the GEMM tile map for row tiles of bm.
moe_status run_dispatch(const void *x, moe_dtype dt, const int32_t *expert_idx, int64_t T,
                        int32_t d, int32_t E, int32_t k, int64_t C, int32_t *slot,
                        uint8_t *drop_mask, int32_t *expert_count, void *xbuf, char *ws,
                        hipStream_t stream, const float *part_prob = nullptr, int nblk_r = 0,
                        float *prob_sum = nullptr, int32_t *route_count = nullptr,
                        int32_t *tile_map = nullptr, int bm = 0, int32_t *row_tok = nullptr,
                        void *y_zero = nullptr, float alpha = 0.f, float *aux = nullptr,
                        const float *gate = nullptr, float *row_gate = nullptr,
                        const float *part_z = nullptr, float *z_loss = nullptr) {
    const DispatchWs w = dispatch_ws(T, E, k);
    int32_t *rank = reinterpret_cast<int32_t *>(ws + w.rank);
    int32_t *hist = reinterpret_cast<int32_t *>(ws + w.hist);
    unsigned *done = reinterpret_cast<unsigned *>(ws + w.done);
    // with row_tok the index pass (a launch after the scan) writes the tile
    // map and the loss, so the scan needs no completion counter
    const bool late = row_tok != nullptr;
    MOE_HIP(moe::launch_slot_rank(expert_idx, T, E, k, rank, hist, tile_map && !late ? done : nullptr,
                                  stream));
    MOE_HIP(moe::launch_slot_scan(hist, moe::dispatch_blocks(T), E, k, C, expert_count, part_prob,
                                  nblk_r, prob_sum, route_count, late ? nullptr : tile_map, bm, done,
                                  stream, T, alpha, late ? nullptr : aux, part_z, z_loss));
    if (late)
        MOE_HIP(moe::launch_slot_index(expert_idx, rank, hist, T, E, k, C, slot, drop_mask, row_tok,
                                       gate, row_gate, y_zero, d * (int)esize(dt), stream, expert_count,
                                       prob_sum, route_count, tile_map, bm, alpha, aux));
    else
        MOE_HIP(moe::launch_permute(x, (int)esize(dt), expert_idx, rank, hist, T, d, E, k, C, slot,
                                    drop_mask, xbuf, stream));
    return MOE_OK;
}

moe_status run_ffn(const void *xbuf, moe_dtype dt, const int32_t *expert_count, int32_t E,
                   int64_t C, int32_t d, int32_t dff, const void *W1, const void *b1,
                   const void *W3, const void *W2, const void *b2, moe_act act, void *ybuf,
                   int64_t rows_bound, char *ws, hipStream_t stream) {
    if (C == 0) return MOE_OK;
    const FfnWs w = ffn_ws(E, C, dff, dt);
    int32_t *tile_map = reinterpret_cast<int32_t *>(ws + w.tile_map);
    void *H = ws + w.h;
    float *part = w.part < w.total ? reinterpret_cast<float *>(ws + w.part) : nullptr;
    const int bf16 = dt == MOE_BF16;
    const int act1 = (act == MOE_ACT_SWIGLU) ? 2 : 1;
    const int bm = moe::gemm_bm(bf16, C, act1);
    MOE_HIP(moe::launch_tile_map(expert_count, E, bm, tile_map, stream));
    MOE_HIP(moe::launch_grouped_gemm(xbuf, W1, W3, b1, bf16, act1, expert_count, tile_map, bm, E, C,
                                     dff, d, rows_bound, H, stream, nullptr, 0, nullptr, nullptr, part));
    MOE_HIP(moe::launch_grouped_gemm(H, W2, nullptr, b2, bf16, 0, expert_count, tile_map, bm, E, C,
                                     d, dff, rows_bound, ybuf, stream, nullptr, 0, nullptr, nullptr, part));
    return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

int64_t moe_capacity(int64_t T, int32_t E, int32_t k, double capacity_factor) {
    if (T < 0 || E < 1 || k < 1 || !isfinite(capacity_factor) || capacity_factor <= 0.0)
        return -1;
    const double c = ceil((double)k * (double)T * capacity_factor / (double)E - 1e-9);
    if (c <= 0.0) return 0;
    if (c >= (double)T) return T;
    return (int64_t)c;
}

size_t moe_router_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k) {
    if (check_sizes(T, E, k) != MOE_OK || check_width(d) != MOE_OK) return SIZE_MAX;
    return router_ws(T, d, E).total;
}

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k) {
    if (check_sizes(T, E, k) != MOE_OK) return SIZE_MAX;
    return dispatch_ws(T, E, k).total;
}

size_t moe_expert_ffn_workspace_bytes(int32_t E, int64_t C, int32_t dff, moe_dtype dt) {
    if (E < 1 || E > MAX_E || C < 0 || check_width(dff) != MOE_OK || !dtype_ok(dt)) return SIZE_MAX;
    return ffn_ws(E, C, dff, dt).total;
}

size_t moe_workspace_bytes(int64_t T, int32_t d, int32_t dff, int32_t E, int32_t k, int64_t C,
                           moe_dtype dt, moe_act act) {
    if (check_sizes(T, E, k) != MOE_OK || check_width(d) != MOE_OK ||
        check_width(dff) != MOE_OK || !dtype_ok(dt) || !act_ok(act) || C < 0 || C > T)
        return SIZE_MAX;
    return forward_ws(T, d, dff, E, k, C, dt).total;
}

moe_status moe_forward_workspace_layout(int64_t T, int32_t d, int32_t dff, int32_t E, int32_t k,
                                        int64_t C, moe_dtype dt, moe_act act, moe_ws_layout *out) {
    if (out == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (moe_workspace_bytes(T, d, dff, E, k, C, dt, act) == SIZE_MAX) return MOE_ERR_INVALID_ARGUMENT;
    const ForwardWs w = forward_ws(T, d, dff, E, k, C, dt);
    out->slot = w.slot;
    out->expert_count = w.expert_count;
    out->route_count = w.route_count;
    out->prob_sum = w.prob_sum;
    out->xbuf = w.xbuf;
    out->ybuf = w.ybuf;
    out->row_tok = w.row_tok;
    out->total = w.total;
    return MOE_OK;
}

moe_status moe_router(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                      int64_t T, int32_t d, int32_t E, int32_t k, int32_t *expert_idx,
                      float *gate, float *prob_sum, int32_t *route_count, float *z_loss,
                      float *logits, void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr_ok(W_r, false) || !opt_ok(b_r) || !ptr4_ok(expert_idx, empty) ||
        !ptr4_ok(gate, empty) || !ptr4_ok(prob_sum, false) || !ptr4_ok(route_count, false) ||
        !(z_loss == nullptr || ptr4_ok(z_loss, false)) || !(logits == nullptr || ptr4_ok(logits, empty)))
        return MOE_ERR_INVALID_ARGUMENT;
    const size_t need = router_ws(T, d, E).total;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    return run_router(x, dt, W_r, b_r, T, d, E, k, expert_idx, gate, prob_sum, route_count, z_loss,
                      static_cast<char *>(ws), stream, true, logits);
}

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::once_flag g_scratch_once[NOALLOC_MAX_DEVICES];
void *g_scratch_ptr[NOALLOC_MAX_DEVICES];
hipError_t g_scratch_err[NOALLOC_MAX_DEVICES];

// The device address of the current GPU's scratch array, looked up once per
// device (with that device current) and kept.
moe_status noalloc_scratch(char **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return MOE_ERR_HIP;
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return MOE_ERR_HIP;
    *out = static_cast<char *>(g_scratch_ptr[dev]);
    return MOE_OK;
}

}  // namespace

size_t moe_router_noalloc_scratch_bytes(void) { return MOE_NOALLOC_SCRATCH_BYTES; }

moe_status moe_router_noalloc(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                              int64_t T, int32_t d, int32_t E, int32_t k, int32_t *expert_idx,
                              float *gate, float *prob_sum, int32_t *route_count, float *z_loss,
                              float *logits, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr_ok(W_r, false) || !opt_ok(b_r) || !ptr4_ok(expert_idx, empty) ||
        !ptr4_ok(gate, empty) || !ptr4_ok(prob_sum, false) || !ptr4_ok(route_count, false) ||
        !(z_loss == nullptr || ptr4_ok(z_loss, false)) || !(logits == nullptr || ptr4_ok(logits, empty)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (router_ws(T, d, E).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
    char *ws = nullptr;
    MOE_CHECK(noalloc_scratch(&ws));
    // every scratch byte the router reads (per-block partial rows, the
    // three-part split of W_r) is written earlier in the same call, so the
    // previous call's contents need no clearing
    return run_router(x, dt, W_r, b_r, T, d, E, k, expert_idx, gate, prob_sum, route_count, z_loss, ws,
                      stream, true, logits);
}

moe_status moe_router_noisy(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                            const float *W_noise, const float *noise, int64_t T, int32_t d,
                            int32_t E, int32_t k, int32_t *expert_idx, float *gate,
                            float *prob_sum, int32_t *route_count, float *z_loss, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr_ok(W_r, false) || !opt_ok(b_r) || !ptr_ok(W_noise, false) ||
        !ptr4_ok(noise, empty) || !ptr4_ok(expert_idx, empty) || !ptr4_ok(gate, empty) ||
        !ptr4_ok(prob_sum, false) || !ptr4_ok(route_count, false) ||
        !(z_loss == nullptr || ptr4_ok(z_loss, false)))
        return MOE_ERR_INVALID_ARGUMENT;
    const RouterWs w = router_ws(T, d, E);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    char *base = static_cast<char *>(ws);
    float *part_prob = reinterpret_cast<float *>(base + w.part_prob);
    int32_t *part_cnt = reinterpret_cast<int32_t *>(base + w.part_cnt);
    float *part_z = reinterpret_cast<float *>(base + w.part_z);
    uint16_t *w3 = reinterpret_cast<uint16_t *>(base + w.w3);
    const int bf16 = dt == MOE_BF16;
    MOE_HIP(moe::launch_router_noisy(x, bf16, W_r, b_r, W_noise, noise, T, d, E, k, expert_idx, gate,
                                     part_prob, part_cnt, part_z, w3, stream));
    MOE_HIP(moe::launch_router_reduce(part_prob, part_cnt, moe::router_noisy_blocks(T, bf16, E), E, prob_sum,
                                      route_count, stream, part_z, T, z_loss));
    return MOE_OK;
}

moe_status moe_dispatch(const void *x, moe_dtype dt, const int32_t *expert_idx, int64_t T,
                        int32_t d, int32_t E, int32_t k, int64_t C, int32_t *slot,
                        uint8_t *drop_mask, int32_t *expert_count, void *xbuf, void *ws,
                        size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    if (C < 0 || C > T) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr4_ok(expert_idx, empty) || !ptr4_ok(slot, empty) ||
        (drop_mask == nullptr && !empty) || !ptr4_ok(expert_count, false) || !ptr_ok(xbuf, C == 0))
        return MOE_ERR_INVALID_ARGUMENT;
    const size_t need = dispatch_ws(T, E, k).total;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    return run_dispatch(x, dt, expert_idx, T, d, E, k, C, slot, drop_mask, expert_count, xbuf,
                        static_cast<char *>(ws), stream);
}

namespace {
moe_status run_priority_dispatch(const void *x, moe_dtype dt, const int32_t *expert_idx, const float *priority,
                                 int64_t T, int32_t d, int32_t E, int32_t k, int64_t C, int32_t *slot,
                                 uint8_t *drop_mask, int32_t *expert_count, void *xbuf, char *base,
                                 hipStream_t stream) {
    const PriorityWs w = priority_ws(T, E, k);
    int32_t *rank = reinterpret_cast<int32_t *>(base + w.d.rank);
    int32_t *hist = reinterpret_cast<int32_t *>(base + w.d.hist);
    int32_t *n_e = reinterpret_cast<int32_t *>(base + w.cnt);
    MOE_HIP(moe::launch_slot_rank(expert_idx, T, E, k, rank, hist, nullptr, stream));
    // an unbounded capacity: the scan's counts are the experts' choice counts
    MOE_HIP(moe::launch_slot_scan(hist, moe::dispatch_blocks(T), E, k, T * k + 1, n_e, nullptr, 0, nullptr,
                                  nullptr, nullptr, 0, nullptr, stream));
    MOE_HIP(moe::launch_priority_slots(x, (int)esize(dt), expert_idx, priority, rank, hist, n_e, T, d, E, k,
                                       C, reinterpret_cast<uint64_t *>(base + w.list),
                                       reinterpret_cast<int32_t *>(base + w.off), slot, drop_mask,
                                       expert_count, xbuf, stream, reinterpret_cast<int32_t *>(base + w.pcnt)));
    return MOE_OK;
}
}  // namespace

size_t moe_dispatch_priority_workspace_bytes(int64_t T, int32_t E, int32_t k) {
    if (check_sizes(T, E, k) != MOE_OK) return SIZE_MAX;
    return priority_ws(T, E, k).total;
}

moe_status moe_dispatch_priority(const void *x, moe_dtype dt, const int32_t *expert_idx,
                                 const float *priority, int64_t T, int32_t d, int32_t E, int32_t k,
                                 int64_t C, int32_t *slot, uint8_t *drop_mask, int32_t *expert_count,
                                 void *xbuf, void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    // the per-expert ranking is quadratic in the choices at one expert
    if (T * (int64_t)k > PRIORITY_MAX_CHOICES) return MOE_ERR_UNSUPPORTED;
    if (C < 0 || C > T) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr4_ok(expert_idx, empty) || !ptr4_ok(priority, empty) ||
        !ptr4_ok(slot, empty) || (drop_mask == nullptr && !empty) || !ptr4_ok(expert_count, false) ||
        !ptr_ok(xbuf, C == 0))
        return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < priority_ws(T, E, k).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    return run_priority_dispatch(x, dt, expert_idx, priority, T, d, E, k, C, slot, drop_mask, expert_count, xbuf,
                                 static_cast<char *>(ws), stream);
}

moe_status moe_combine_backward(const void *dy, moe_dtype dt, const void *ybuf, const int32_t *expert_idx,
                                const int32_t *slot, const float *gate, int64_t T, int32_t d, int32_t E,
                                int32_t k, int64_t C, float *dgate, void *dybuf, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    if (C < 0 || C > T) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(dy, empty) || !ptr_ok(ybuf, C == 0) || !ptr4_ok(expert_idx, empty) || !ptr4_ok(slot, empty) ||
        !ptr4_ok(gate, empty) || !ptr4_ok(dgate, empty) || !ptr_ok(dybuf, C == 0))
        return MOE_ERR_INVALID_ARGUMENT;
    MOE_HIP(moe::launch_combine_backward(dy, dt == MOE_BF16, ybuf, expert_idx, slot, gate, T, d, E, k, C, dgate,
                                         dybuf, stream));
    return MOE_OK;
}

// rank [T], hist, done (the plain dispatch's scratch for one rank), then
// cand [T], n_e [E], fill [E].
// Re-routing: the plain dispatch's rank and scan scratch, the candidates and
// every stage's per-expert candidate counts.
struct RerouteWs {
    DispatchWs d;
    size_t cand, cnt, total;
};
RerouteWs reroute_ws(int64_t T, int E) {
    RerouteWs w;
    w.d = dispatch_ws(T, E, 1);
    w.cand = w.d.total;
    w.cnt = w.cand + up((size_t)T * 4);
    w.total = w.cnt + up((size_t)moe::REROUTE_MAX_STAGES * E * 4);
    return w;
}

size_t moe_dispatch_reroute_workspace_bytes(int64_t T, int32_t E) {
    if (check_sizes(T, E, 1) != MOE_OK) return SIZE_MAX;
    return reroute_ws(T, E).total;
}

moe_status moe_dispatch_reroute(const void *x, moe_dtype dt, const int32_t *pref, const float *logits, int64_t T,
                                int32_t d, int32_t E, int32_t R, int32_t stages, int64_t C, int32_t *expert,
                                int32_t *slot, uint8_t *drop_mask, float *gate, int32_t *expert_count, void *xbuf,
                                void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, R));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    if (C < 0 || C > T || stages < 1 || stages > R) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr4_ok(pref, empty) || !ptr4_ok(expert, empty) || !ptr4_ok(slot, empty) ||
        (drop_mask == nullptr && !empty) || !ptr4_ok(expert_count, false) || !ptr_ok(xbuf, C == 0) ||
        ((logits == nullptr) != (gate == nullptr)) || !(logits == nullptr || ptr4_ok(logits, empty)) ||
        !(gate == nullptr || ptr4_ok(gate, empty)))
        return MOE_ERR_INVALID_ARGUMENT;
    const RerouteWs w = reroute_ws(T, E);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    char *base = static_cast<char *>(ws);
    MOE_HIP(moe::launch_reroute(x, (int)esize(dt), pref, logits, T, d, E, R, stages, C, expert, slot, drop_mask,
                                gate, expert_count, xbuf, reinterpret_cast<int32_t *>(base + w.d.rank),
                                reinterpret_cast<int32_t *>(base + w.d.hist),
                                reinterpret_cast<int32_t *>(base + w.cand), reinterpret_cast<int32_t *>(base + w.cnt),
                                stream));
    return MOE_OK;
}

size_t moe_router_backward_workspace_bytes(int64_t T, int32_t d, int32_t E) {
    if (check_sizes(T, E, 1) != MOE_OK || check_width(d) != MOE_OK) return SIZE_MAX;
    const size_t nc = (size_t)moe::router_bwd_chunks(T, d, E);
    return up(nc * E * d * 4) + up(nc * E * 4);
}

moe_status moe_router_backward(const void *x, moe_dtype dt, const float *W_r, const float *logits,
                               const int32_t *expert_idx, const float *gate, const float *dgate,
                               const int32_t *route_count, int64_t T, int32_t d, int32_t E, int32_t k,
                               float alpha, float z_weight, float *dlogits, float *dW_r, float *db_r,
                               float *dx, void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    const bool empty = T == 0;
    if (moe::router_bwd_chunks(T, d, E) > 65535) return MOE_ERR_UNSUPPORTED;
    if (!ptr_ok(x, empty) || !ptr_ok(W_r, false) || !ptr4_ok(logits, empty) || !ptr4_ok(expert_idx, empty) ||
        !ptr4_ok(gate, empty) || !ptr4_ok(dgate, empty) || !ptr4_ok(route_count, false) ||
        !ptr4_ok(dlogits, empty) || !ptr4_ok(dW_r, false) || !(db_r == nullptr || ptr4_ok(db_r, false)) ||
        !(dx == nullptr || ptr_ok(dx, empty)) || !isfinite(alpha) || !isfinite(z_weight))
        return MOE_ERR_INVALID_ARGUMENT;
    const size_t nc = (size_t)moe::router_bwd_chunks(T, d, E);
    if (ws_bytes < up(nc * E * d * 4) + up(nc * E * 4)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    float *part_w = static_cast<float *>(ws);
    float *part_b = reinterpret_cast<float *>(static_cast<char *>(ws) + up(nc * E * d * 4));
    MOE_HIP(moe::launch_router_backward(x, dt == MOE_BF16, W_r, logits, expert_idx, gate, dgate, route_count, T, d,
                                        E, k, alpha, z_weight, dlogits, dW_r, db_r, dx, part_w, part_b, stream));
    return MOE_OK;
}

moe_status moe_expert_ffn(const void *xbuf, moe_dtype dt, const int32_t *expert_count, int32_t E,
                          int64_t C, int32_t d, int32_t dff, const void *W1, const void *b1,
                          const void *W3, const void *W2, const void *b2, moe_act act,
                          void *ybuf, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (E < 1 || C < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (E > MAX_E) return MOE_ERR_UNSUPPORTED;
    MOE_CHECK(check_width(d));
    MOE_CHECK(check_width(dff));
    MOE_CHECK(check_ffn_args(dt, act, W1, b1, W3, W2, b2));
    if (!ptr_ok(xbuf, C == 0) || !ptr4_ok(expert_count, false) || !ptr_ok(ybuf, C == 0))
        return MOE_ERR_INVALID_ARGUMENT;
    const size_t need = ffn_ws(E, C, dff, dt).total;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    return run_ffn(xbuf, dt, expert_count, E, C, d, dff, W1, b1, W3, W2, b2, act, ybuf,
                   (int64_t)E * C, static_cast<char *>(ws), stream);
}

size_t moe_expert_ffn_backward_workspace_bytes(int32_t E, int64_t C, int32_t d, int32_t dff, moe_dtype dt,
                                              moe_act act) {
    if (E < 1 || E > MAX_E || C < 0 || check_width(d) != MOE_OK || check_width(dff) != MOE_OK ||
        !dtype_ok(dt) || !act_ok(act))
        return SIZE_MAX;
    return moe::expert_backward_ws(E, C, d, dff, dt == MOE_BF16, act == MOE_ACT_SWIGLU ? 2 : 1).total;
}

moe_status moe_expert_ffn_backward(const void *xbuf, moe_dtype dt, const int32_t *expert_count, int32_t E,
                                   int64_t C, int32_t d, int32_t dff, const void *W1, const void *b1,
                                   const void *W3, const void *W2, moe_act act, const void *dybuf, void *dxbuf,
                                   void *dW1, void *dW3, void *dW2, void *db1, void *db2, void *ws,
                                   size_t ws_bytes, hipStream_t stream) {
    if (E < 1 || C < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (E > MAX_E) return MOE_ERR_UNSUPPORTED;
    MOE_CHECK(check_width(d));
    MOE_CHECK(check_width(dff));
    // the forward's weight arguments, and their gradients alike
    MOE_CHECK(check_ffn_args(dt, act, W1, b1, W3, W2, nullptr));
    if ((dW3 == nullptr) != (W3 == nullptr) || !ptr_ok(dW1, false) || !ptr_ok(dW2, false) || !opt_ok(dW3) ||
        !opt_ok(db1) || !opt_ok(db2))
        return MOE_ERR_INVALID_ARGUMENT;
    if (act == MOE_ACT_SWIGLU && (db1 != nullptr || db2 != nullptr)) return MOE_ERR_UNSUPPORTED;
    if (!ptr_ok(xbuf, C == 0) || !ptr4_ok(expert_count, false) || !ptr_ok(dybuf, C == 0) ||
        !ptr_ok(dxbuf, C == 0))
        return MOE_ERR_INVALID_ARGUMENT;
    const size_t need = moe::expert_backward_ws(E, C, d, dff, dt == MOE_BF16, act == MOE_ACT_SWIGLU ? 2 : 1).total;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    MOE_HIP(moe::launch_expert_backward(xbuf, dt == MOE_BF16, expert_count, E, C, d, dff, W1, b1, W3, W2,
                                        act == MOE_ACT_SWIGLU ? 2 : 1, dybuf, dxbuf, dW1, dW3, dW2, db1, db2,
                                        static_cast<char *>(ws), stream));
    return MOE_OK;
}

moe_status moe_dispatch_backward(const void *dxbuf, moe_dtype dt, const int32_t *expert_idx, const int32_t *slot,
                                 int64_t T, int32_t d, int32_t E, int32_t k, int64_t C, const float *dx_add,
                                 float *dx, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    if (C < 0 || C > T) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(dxbuf, empty || C == 0) || !ptr4_ok(expert_idx, empty) || !ptr4_ok(slot, empty) ||
        !opt_ok(dx_add) || !ptr_ok(dx, empty))
        return MOE_ERR_INVALID_ARGUMENT;
    MOE_HIP(moe::launch_dispatch_backward(dxbuf, dt == MOE_BF16, expert_idx, slot, T, d, E, k, C, dx_add, dx,
                                          stream));
    return MOE_OK;
}

moe_status moe_combine(const void *ybuf, moe_dtype dt, const int32_t *expert_idx,
                       const int32_t *slot, const float *gate, const float *prob_sum,
                       const int32_t *route_count, int64_t T, int32_t d, int32_t E, int32_t k,
                       int64_t C, float alpha, void *y, float *aux_loss, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    if (!dtype_ok(dt)) return MOE_ERR_UNSUPPORTED;
    if (C < 0 || C > T || !isfinite(alpha)) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(ybuf, empty || C == 0) || !ptr4_ok(expert_idx, empty) || !ptr4_ok(slot, empty) ||
        !ptr4_ok(gate, empty) || !ptr4_ok(prob_sum, false) || !ptr4_ok(route_count, false) ||
        !ptr_ok(y, empty) || !ptr4_ok(aux_loss, false))
        return MOE_ERR_INVALID_ARGUMENT;
    MOE_HIP(moe::launch_combine(ybuf, dt == MOE_BF16, expert_idx, slot, gate, prob_sum,
                                route_count, T, d, E, k, C, alpha, y, aux_loss, stream));
    return MOE_OK;
}

}  // extern "C"

namespace {

moe_status forward_impl(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                        const void *W1, const void *b1, const void *W3, const void *W2,
                        const void *b2, moe_act act, int64_t T, int32_t d, int32_t dff, int32_t E,
                        int32_t k, double capacity_factor, float alpha, void *y, float *aux_loss,
                        float *z_loss, int32_t *expert_idx, float *gate, uint8_t *drop_mask,
                        void *ws, size_t ws_bytes, hipStream_t stream, hipEvent_t *ev,
                        const float *W_noise = nullptr, const float *noise = nullptr) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    MOE_CHECK(check_width(dff));
    MOE_CHECK(check_ffn_args(dt, act, W1, b1, W3, W2, b2));
    if (!isfinite(alpha)) return MOE_ERR_INVALID_ARGUMENT;
    const int64_t C = moe_capacity(T, E, k, capacity_factor);
    if (C < 0) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr_ok(W_r, false) || !opt_ok(b_r) || !ptr_ok(y, empty) ||
        !ptr4_ok(aux_loss, false) || !(z_loss == nullptr || ptr4_ok(z_loss, false)) || !ptr4_ok(expert_idx, empty) ||
        !ptr4_ok(gate, empty) || (drop_mask == nullptr && !empty) ||
        (W_noise != nullptr && (!ptr_ok(W_noise, false) || !ptr4_ok(noise, empty))))
        return MOE_ERR_INVALID_ARGUMENT;
    if (ev != nullptr) {
        for (int i = 0; i < MOE_STAGE_EVENTS; ++i)
            if (ev[i] == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    }
    const ForwardWs w = forward_ws(T, d, dff, E, k, C, dt);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    char *base = static_cast<char *>(ws);
    float *prob_sum = reinterpret_cast<float *>(base + w.prob_sum);
    int32_t *route_count = reinterpret_cast<int32_t *>(base + w.route_count);
    int32_t *expert_count = reinterpret_cast<int32_t *>(base + w.expert_count);
    int32_t *slot = reinterpret_cast<int32_t *>(base + w.slot);
    void *xbuf = base + w.xbuf;
    void *ybuf = base + w.ybuf;
    const int bf16 = dt == MOE_BF16;
    int32_t *tile_map = reinterpret_cast<int32_t *>(base + w.ffn + w.f.tile_map);
    void *H = base + w.ffn + w.f.h;
    float *part = w.f.part < w.f.total ? reinterpret_cast<float *>(base + w.ffn + w.f.part) : nullptr;
    const int64_t rows = T * (int64_t)k;
    const int act1 = (act == MOE_ACT_SWIGLU) ? 2 : 1;
    const int bm = moe::gemm_bm(bf16, C, act1);
    auto mark = [&](int i) -> bool { return ev == nullptr || hipEventRecord(ev[i], stream) == hipSuccess; };

    if (!mark(0)) return MOE_ERR_HIP;
    // the router's per-expert totals are finished by the dispatch scan (one
    // launch fewer); with T = 0 there is no dispatch work, so the router does it
    const bool fuse_reduce = T > 0;
    // bf16 with work to do: no dispatch copy (the first GEMM gathers the
    // token rows through row_tok) and, with one choice per token, no combine
    // pass (the second GEMM writes gated rows straight to y; the index pass
    // writes the auxiliary loss and clears the rows of dropped tokens)
    const bool gather = bf16 && T > 0 && C > 0;
    const bool scatter = gather && k == 1;
    int32_t *row_tok = gather ? reinterpret_cast<int32_t *>(base + w.row_tok) : nullptr;
    float *row_gate = scatter ? reinterpret_cast<float *>(base + w.row_gate) : nullptr;
    MOE_CHECK(run_router(x, dt, W_r, b_r, T, d, E, k, expert_idx, gate, prob_sum, route_count,
                         z_loss, base + w.router, stream, !fuse_reduce, nullptr, W_noise, noise));
    const int nblk_r = W_noise != nullptr ? moe::router_noisy_blocks(T, bf16, E) : moe::router_blocks(T, bf16, E);
    if (!mark(1)) return MOE_ERR_HIP;
    MOE_CHECK(run_dispatch(x, dt, expert_idx, T, d, E, k, C, slot, drop_mask, expert_count, xbuf,
                           base + w.dispatch, stream,
                           fuse_reduce ? reinterpret_cast<const float *>(base + w.router + w.r.part_prob)
                                       : nullptr,
                           nblk_r, prob_sum, route_count,
                           T > 0 && C > 0 ? tile_map : nullptr, bm, row_tok, scatter ? y : nullptr,
                           alpha, scatter ? aux_loss : nullptr, gate, row_gate,
                           fuse_reduce ? reinterpret_cast<const float *>(base + w.router + w.r.part_z)
                                       : nullptr,
                           fuse_reduce ? z_loss : nullptr));
    if (!mark(2)) return MOE_ERR_HIP;
    if (C > 0)
        MOE_HIP(moe::launch_grouped_gemm(gather ? x : xbuf, W1, W3, b1, bf16, act1, expert_count, tile_map,
                                         bm, E, C, dff, d, rows, H, stream, row_tok, T, nullptr, nullptr, part));
    if (!mark(3)) return MOE_ERR_HIP;
    if (C > 0)
        MOE_HIP(moe::launch_grouped_gemm(H, W2, nullptr, b2, bf16, 0, expert_count, tile_map, bm, E, C, d,
                                         dff, rows, scatter ? y : ybuf, stream, scatter ? row_tok : nullptr,
                                         T, row_gate, nullptr, part));
    if (!mark(4)) return MOE_ERR_HIP;
    if (!scatter)
        MOE_HIP(moe::launch_combine(ybuf, bf16, expert_idx, slot, gate, prob_sum, route_count, T, d, E,
                                    k, C, alpha, y, aux_loss, stream));
    if (!mark(5)) return MOE_ERR_HIP;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                       const void *W1, const void *b1, const void *W3, const void *W2,
                       const void *b2, moe_act act, int64_t T, int32_t d, int32_t dff,
                       int32_t E, int32_t k, double capacity_factor, float alpha, void *y,
                       float *aux_loss, float *z_loss, int32_t *expert_idx, float *gate,
                       uint8_t *drop_mask, void *ws, size_t ws_bytes, hipStream_t stream) {
    return forward_impl(x, dt, W_r, b_r, W1, b1, W3, W2, b2, act, T, d, dff, E, k,
                        capacity_factor, alpha, y, aux_loss, z_loss, expert_idx, gate, drop_mask, ws,
                        ws_bytes, stream, nullptr);
}

moe_status moe_forward_noisy(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                             const float *W_noise, const float *noise, const void *W1, const void *b1,
                             const void *W3, const void *W2, const void *b2, moe_act act, int64_t T, int32_t d,
                             int32_t dff, int32_t E, int32_t k, double capacity_factor, float alpha, void *y,
                             float *aux_loss, float *z_loss, int32_t *expert_idx, float *gate,
                             uint8_t *drop_mask, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (W_noise == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    return forward_impl(x, dt, W_r, b_r, W1, b1, W3, W2, b2, act, T, d, dff, E, k, capacity_factor, alpha, y,
                        aux_loss, z_loss, expert_idx, gate, drop_mask, ws, ws_bytes, stream, nullptr, W_noise,
                        noise);
}

moe_status moe_forward_staged(const void *x, moe_dtype dt, const float *W_r, const float *b_r,
                              const void *W1, const void *b1, const void *W3, const void *W2,
                              const void *b2, moe_act act, int64_t T, int32_t d, int32_t dff,
                              int32_t E, int32_t k, double capacity_factor, float alpha, void *y,
                              float *aux_loss, float *z_loss, int32_t *expert_idx, float *gate,
                              uint8_t *drop_mask, void *ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t *stage_events) {
    if (stage_events == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    return forward_impl(x, dt, W_r, b_r, W1, b1, W3, W2, b2, act, T, d, dff, E, k,
                        capacity_factor, alpha, y, aux_loss, z_loss, expert_idx, gate, drop_mask, ws,
                        ws_bytes, stream, stage_events);
}

// ---- the fused forward with an overflow policy -------------------------------

namespace {

// Workspace of moe_forward_policy: the router's scratch and totals, the
// policy's inputs (priority: the first-rank gates as scores; re-routing: the
// router's top-`stages` preferences, their gates and the logits), the
// policy dispatch's scratch, then slot, expert_count, xbuf, the FFN scratch
// and ybuf.
struct PolicyWs {
    RouterWs r;
    size_t router, prob_sum, route_count, count1, score, pref, pgate, logits, pdisp, slot, expert_count, xbuf, ffn,
        ybuf, total;
};
PolicyWs policy_ws(int64_t T, int d, int dff, int E, int k, int64_t C, moe_dtype dt, int policy, int stages) {
    PolicyWs w{};
    w.r = router_ws(T, d, E);
    const bool rr = policy == MOE_POLICY_REROUTE;
    const int kr = rr ? stages : k;                      // the router's choices per token
    size_t o = 0;
    w.router = o;       o += w.r.total;
    w.prob_sum = o;     o += up((size_t)E * 4);
    w.route_count = o;  o += up((size_t)E * 4);
    w.count1 = o;       o += up((size_t)E * 4);
    w.score = o;        o += rr ? 0 : up((size_t)T * 4);
    w.pref = o;         o += rr ? up((size_t)T * kr * 4) : 0;
    w.pgate = o;        o += rr ? up((size_t)T * kr * 4) : 0;
    w.logits = o;       o += rr ? up((size_t)T * E * 4) : 0;
    w.pdisp = o;        o += rr ? reroute_ws(T, E).total : priority_ws(T, E, k).total;
    w.slot = o;         o += up((size_t)T * (rr ? 1 : k) * 4);
    w.expert_count = o; o += up((size_t)E * 4);
    w.xbuf = o;         o += up((size_t)E * C * d * esize(dt));
    w.ffn = o;          o += ffn_ws(E, C, dff, dt).total;
    w.ybuf = o;         o += up((size_t)E * C * d * esize(dt));
    w.total = o;
    return w;
}

bool policy_ok(int policy, int k, int32_t stages, int E) {
    if (policy == MOE_POLICY_PRIORITY) return true;
    if (policy == MOE_POLICY_REROUTE) return k == 1 && stages >= 1 && stages <= E && stages <= MAX_K;
    return false;
}

}  // namespace

size_t moe_forward_policy_workspace_bytes(int64_t T, int32_t d, int32_t dff, int32_t E, int32_t k,
                                          double capacity_factor, moe_dtype dt, moe_act act, moe_policy policy,
                                          int32_t stages) {
    if (check_sizes(T, E, k) != MOE_OK || check_width(d) != MOE_OK || check_width(dff) != MOE_OK ||
        !dtype_ok(dt) || !act_ok(act) || !policy_ok(policy, k, stages, E))
        return SIZE_MAX;
    if (policy == MOE_POLICY_PRIORITY && T * (int64_t)k > PRIORITY_MAX_CHOICES) return SIZE_MAX;
    if (policy == MOE_POLICY_REROUTE && check_sizes(T, E, stages) != MOE_OK) return SIZE_MAX;
    const int64_t C = moe_capacity(T, E, k, capacity_factor);
    if (C < 0) return SIZE_MAX;
    return policy_ws(T, d, dff, E, k, C, dt, policy, stages).total;
}

moe_status moe_forward_policy(const void *x, moe_dtype dt, const float *W_r, const float *b_r, const void *W1,
                              const void *b1, const void *W3, const void *W2, const void *b2, moe_act act,
                              int64_t T, int32_t d, int32_t dff, int32_t E, int32_t k, double capacity_factor,
                              float alpha, moe_policy policy, const float *priority, int32_t stages, void *y,
                              float *aux_loss, float *z_loss, int32_t *expert_idx, float *gate,
                              uint8_t *drop_mask, void *ws, size_t ws_bytes, hipStream_t stream) {
    MOE_CHECK(check_sizes(T, E, k));
    MOE_CHECK(check_width(d));
    MOE_CHECK(check_width(dff));
    MOE_CHECK(check_ffn_args(dt, act, W1, b1, W3, W2, b2));
    if (policy != MOE_POLICY_PRIORITY && policy != MOE_POLICY_REROUTE) return MOE_ERR_UNSUPPORTED;
    if (!policy_ok(policy, k, stages, E)) return MOE_ERR_INVALID_ARGUMENT;
    if (policy == MOE_POLICY_PRIORITY && T * (int64_t)k > PRIORITY_MAX_CHOICES) return MOE_ERR_UNSUPPORTED;
    if (policy == MOE_POLICY_REROUTE && priority != nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (!isfinite(alpha)) return MOE_ERR_INVALID_ARGUMENT;
    const int64_t C = moe_capacity(T, E, k, capacity_factor);
    if (C < 0) return MOE_ERR_INVALID_ARGUMENT;
    const bool empty = T == 0;
    if (!ptr_ok(x, empty) || !ptr_ok(W_r, false) || !opt_ok(b_r) || !ptr_ok(y, empty) ||
        !ptr4_ok(aux_loss, false) || !(z_loss == nullptr || ptr4_ok(z_loss, false)) ||
        !ptr4_ok(expert_idx, empty) || !ptr4_ok(gate, empty) || (drop_mask == nullptr && !empty) ||
        !(priority == nullptr || ptr4_ok(priority, empty)))
        return MOE_ERR_INVALID_ARGUMENT;
    const PolicyWs w = policy_ws(T, d, dff, E, k, C, dt, policy, stages);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (!ptr_ok(ws, false)) return MOE_ERR_INVALID_ARGUMENT;
    char *base = static_cast<char *>(ws);
    float *prob_sum = reinterpret_cast<float *>(base + w.prob_sum);
    int32_t *route_count = reinterpret_cast<int32_t *>(base + w.route_count);
    int32_t *count1 = reinterpret_cast<int32_t *>(base + w.count1);
    int32_t *slot = reinterpret_cast<int32_t *>(base + w.slot);
    int32_t *expert_count = reinterpret_cast<int32_t *>(base + w.expert_count);
    void *xbuf = base + w.xbuf;
    void *ybuf = base + w.ybuf;
    const int bf16 = dt == MOE_BF16;
    const int32_t *loss_count = route_count;
    if (policy == MOE_POLICY_PRIORITY) {
        // [CS25-L5], the V-MoE part: the router's top-k, then the capacity
        // spent on the highest scores first (the caller's, or each token's
        // first gate)
        MOE_CHECK(run_router(x, dt, W_r, b_r, T, d, E, k, expert_idx, gate, prob_sum, route_count, z_loss,
                             base + w.router, stream, true));
        const float *score = priority;
        if (score == nullptr) {
            float *sc = reinterpret_cast<float *>(base + w.score);
            MOE_HIP(moe::launch_first_gate(gate, T, k, sc, stream));
            score = sc;
        }
        MOE_CHECK(run_priority_dispatch(x, dt, expert_idx, score, T, d, E, k, C, slot, drop_mask, expert_count,
                                        xbuf, base + w.pdisp, stream));
    } else {
        // [CS25-L5] "No Token Left Behind": the router's top-`stages` choices
        // are the preferences; stage s offers the unplaced tokens their
        // choice s.  The loss counts each token's first choice (k = 1).
        int32_t *pref = reinterpret_cast<int32_t *>(base + w.pref);
        float *pgate = reinterpret_cast<float *>(base + w.pgate);
        float *logits = reinterpret_cast<float *>(base + w.logits);
        MOE_CHECK(run_router(x, dt, W_r, b_r, T, d, E, stages, pref, pgate, prob_sum, route_count, z_loss,
                             base + w.router, stream, true, logits));
        MOE_HIP(moe::launch_first_choice_count(pref, T, stages, E, count1, stream));
        loss_count = count1;
        const RerouteWs rw = reroute_ws(T, E);
        char *rb = base + w.pdisp;
        MOE_HIP(moe::launch_reroute(x, (int)esize(dt), pref, logits, T, d, E, stages, stages, C, expert_idx, slot,
                                    drop_mask, gate, expert_count, xbuf, reinterpret_cast<int32_t *>(rb + rw.d.rank),
                                    reinterpret_cast<int32_t *>(rb + rw.d.hist),
                                    reinterpret_cast<int32_t *>(rb + rw.cand), reinterpret_cast<int32_t *>(rb + rw.cnt),
                                    stream));
    }
    const int kc = policy == MOE_POLICY_REROUTE ? 1 : k;
    MOE_CHECK(run_ffn(xbuf, dt, expert_count, E, C, d, dff, W1, b1, W3, W2, b2, act, ybuf, T * (int64_t)kc,
                      base + w.ffn, stream));
    MOE_HIP(moe::launch_combine(ybuf, bf16, expert_idx, slot, gate, prob_sum, loss_count, T, d, E, kc, C, alpha, y,
                                aux_loss, stream));
    return MOE_OK;
}

}  // extern "C"
