// Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built by tests/test_abi_sanitize.py with the ABI translation unit compiled
// with host-only sanitizers; run on the CPU with no GPU work: every entry
// point call here is one its argument checks reject before anything is
// enqueued (stand-in device addresses that are never dereferenced), plus the
// host helpers (capacity, workspace sizes and layout, status strings) at
// ordinary and extreme sizes.  A sanitizer report aborts the process; the
// checks themselves print a line and exit 1 on a wrong status.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                   \
    do {                                                                                     \
        const long long got_ = (long long)(expr);                                            \
        if (got_ != (long long)(want)) {                                                     \
            printf("FAIL %s:%d %s = %lld, expected %lld\n", __FILE__, __LINE__, #expr, got_, \
                   (long long)(want));                                                       \
            ++failures;                                                                      \
        }                                                                                    \
    } while (0)

int main() {
    void *P = (void *)(uintptr_t)4096;          // aligned stand-in address, never dereferenced
    void *M = (void *)(uintptr_t)4098;          // misaligned stand-in
    const size_t BIG = (size_t)1 << 40;

    // host helpers
    EXPECT(moe_capacity(8192, 8, 2, 1.25), 2560);
    EXPECT(moe_capacity(1024, 8, 2, 1.25), 320);
    EXPECT(moe_capacity(-1, 8, 1, 1.0), -1);
    EXPECT(moe_capacity(10, 8, 1, NAN), -1);
    // a pure function: C is clamped to T; the T k limit belongs to the entry points
    EXPECT(moe_capacity(INT64_MAX / 2, 1, 8, 1e300), INT64_MAX / 2);
    EXPECT(moe_capacity((int64_t)1 << 40, 1024, 8, 1.0), (int64_t)1 << 33);
    EXPECT(strcmp(moe_status_string(MOE_ERR_HIP), "MOE_ERR_HIP"), 0);
    EXPECT(strcmp(moe_status_string(-7), "MOE_ERR_UNKNOWN"), 0);
    EXPECT(moe_workspace_bytes(16384, 768, 3072, 64, 1, 320, MOE_BF16, MOE_ACT_RELU) > 0, 1);
    EXPECT(moe_workspace_bytes((int64_t)1 << 40, 768, 3072, 64, 8, 320, MOE_BF16, MOE_ACT_RELU), SIZE_MAX);
    EXPECT(moe_workspace_bytes(16384, 1 << 21, 3072, 64, 1, 320, MOE_BF16, MOE_ACT_RELU), SIZE_MAX);
    EXPECT(moe_workspace_bytes(16384, 768, 3072, 64, 1, 16385, MOE_BF16, MOE_ACT_RELU), SIZE_MAX);
    EXPECT(moe_router_workspace_bytes(32768, 1024, 1024, 8) > 0, 1);
    EXPECT(moe_dispatch_workspace_bytes(((int64_t)1 << 31) - 1, 1024, 1) > 0, 1);
    EXPECT(moe_dispatch_priority_workspace_bytes(100, 2000, 1), SIZE_MAX);
    EXPECT(moe_expert_ffn_workspace_bytes(1024, (int64_t)1 << 30, 1 << 20, MOE_BF16) > 0, 1);
    EXPECT(moe_expert_ffn_backward_workspace_bytes(8, 2560, 4096, 14336, MOE_BF16, MOE_ACT_SWIGLU) > 0, 1);
    EXPECT(moe_expert_ffn_backward_workspace_bytes(8, 2560, 4095, 14336, MOE_BF16, MOE_ACT_SWIGLU), SIZE_MAX);
    EXPECT(moe_router_noalloc_scratch_bytes(), (size_t)32 << 20);
    moe_ws_layout lay;
    EXPECT(moe_forward_workspace_layout(8192, 4096, 14336, 8, 2, 2560, MOE_BF16, MOE_ACT_SWIGLU, &lay), MOE_OK);
    EXPECT(lay.total, moe_workspace_bytes(8192, 4096, 14336, 8, 2, 2560, MOE_BF16, MOE_ACT_SWIGLU));
    EXPECT(moe_forward_workspace_layout(8192, 4096, 14336, 8, 2, 2560, MOE_BF16, MOE_ACT_SWIGLU, nullptr),
           MOE_ERR_INVALID_ARGUMENT);

    // entry points: rejected before anything is enqueued
    EXPECT(moe_router(P, MOE_BF16, (float *)P, nullptr, 64, 64, 8, 9, (int32_t *)P, (float *)P, (float *)P,
                      (int32_t *)P, nullptr, nullptr, P, BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_router(M, MOE_BF16, (float *)P, nullptr, 64, 64, 8, 1, (int32_t *)P, (float *)P, (float *)P,
                      (int32_t *)P, nullptr, nullptr, P, BIG, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_router(P, MOE_BF16, (float *)P, nullptr, 64, 64, 8, 1, (int32_t *)P, (float *)P, (float *)P,
                      (int32_t *)P, nullptr, nullptr, P, 0, nullptr), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_router_noalloc(P, MOE_BF16, (float *)P, nullptr, (int64_t)1 << 20, 64, 1024, 1, (int32_t *)P,
                              (float *)P, (float *)P, (int32_t *)P, nullptr, nullptr, nullptr),
           MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_router_noisy(P, MOE_BF16, (float *)P, nullptr, nullptr, (float *)P, 64, 64, 8, 1, (int32_t *)P,
                            (float *)P, (float *)P, (int32_t *)P, nullptr, P, BIG, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_dispatch(P, MOE_BF16, (int32_t *)P, 64, 64, 8, 1, 65, (int32_t *)P, (uint8_t *)P, (int32_t *)P, P, P,
                        BIG, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_dispatch(P, (moe_dtype)7, (int32_t *)P, 64, 64, 8, 1, 16, (int32_t *)P, (uint8_t *)P, (int32_t *)P,
                        P, P, BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_dispatch(P, (moe_dtype)-3, (int32_t *)P, 64, 64, 8, 1, 16, (int32_t *)P, (uint8_t *)P, (int32_t *)P,
                        P, P, BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_expert_ffn(P, MOE_BF16, (int32_t *)P, 8, 16, 64, 128, P, nullptr, nullptr, P, nullptr, (moe_act)9, P,
                          P, BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_dispatch_priority(P, MOE_BF16, (int32_t *)P, (float *)P, ((int64_t)1 << 19) + 1, 64, 8, 2, 16,
                                 (int32_t *)P, (uint8_t *)P, (int32_t *)P, P, P, BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_dispatch_reroute(P, MOE_BF16, (int32_t *)P, (float *)P, 64, 64, 16, 3, 4, 16, (int32_t *)P,
                                (int32_t *)P, (uint8_t *)P, (float *)P, (int32_t *)P, P, P, BIG, nullptr),
           MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_expert_ffn(P, MOE_BF16, (int32_t *)P, 8, 16, 64, 100, P, nullptr, nullptr, P, nullptr, MOE_ACT_RELU, P,
                          P, BIG, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_expert_ffn(P, MOE_BF16, (int32_t *)P, 8, 16, 64, 128, P, P, P, P, nullptr, MOE_ACT_SWIGLU, P, P, BIG,
                          nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_expert_ffn_backward(P, MOE_BF16, (int32_t *)P, 8, 16, 64, 128, P, nullptr, P, P, MOE_ACT_SWIGLU, P, P,
                                   P, nullptr, P, nullptr, nullptr, P, BIG, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_expert_ffn_backward(P, MOE_BF16, (int32_t *)P, 8, 16, 64, 128, P, nullptr, nullptr, P, MOE_ACT_RELU,
                                   P, P, P, nullptr, P, nullptr, nullptr, P, 1, nullptr), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_dispatch_backward(P, MOE_BF16, (int32_t *)P, (int32_t *)P, 64, 64, 8, 1, 65, nullptr, (float *)P,
                                 nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_combine(P, MOE_BF16, (int32_t *)P, (int32_t *)P, (float *)P, (float *)P, (int32_t *)P, 64, 64, 8, 1,
                       16, INFINITY, P, (float *)P, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_combine_backward(P, MOE_BF16, P, (int32_t *)P, (int32_t *)P, (float *)P, 64, 64, 8, 1, 65, (float *)P,
                                P, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_router_backward(P, MOE_BF16, (float *)P, (float *)P, (int32_t *)P, (float *)P, (float *)P,
                               (int32_t *)P, 64, 64, 8, 9, 0.01f, 0.f, (float *)P, (float *)P, nullptr, nullptr, P,
                               BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_forward(P, MOE_BF16, (float *)P, nullptr, P, nullptr, nullptr, P, nullptr, MOE_ACT_RELU,
                       (int64_t)1 << 30, 64, 128, 8, 2, 1.25, 0.01f, P, (float *)P, nullptr, (int32_t *)P,
                       (float *)P, (uint8_t *)P, P, BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_forward(P, MOE_BF16, (float *)P, nullptr, P, nullptr, nullptr, P, nullptr, MOE_ACT_RELU, 64, 64, 128,
                       8, 1, 1.25, 0.01f, P, (float *)P, nullptr, (int32_t *)P, (float *)P, (uint8_t *)P, P, 1024,
                       nullptr), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_forward_noisy(P, MOE_BF16, (float *)P, nullptr, nullptr, (float *)P, P, nullptr, nullptr, P, nullptr,
                             MOE_ACT_RELU, 64, 64, 128, 8, 1, 1.25, 0.01f, P, (float *)P, nullptr, (int32_t *)P,
                             (float *)P, (uint8_t *)P, P, BIG, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_forward_policy(P, MOE_BF16, (float *)P, nullptr, P, nullptr, nullptr, P, nullptr, MOE_ACT_RELU, 64,
                              64, 128, 8, 2, 1.25, 0.01f, MOE_POLICY_REROUTE, nullptr, 2, P, (float *)P, nullptr,
                              (int32_t *)P, (float *)P, (uint8_t *)P, P, BIG, nullptr), MOE_ERR_INVALID_ARGUMENT);
    EXPECT(moe_forward_policy(P, MOE_BF16, (float *)P, nullptr, P, nullptr, nullptr, P, nullptr, MOE_ACT_RELU, 64,
                              64, 128, 8, 1, 1.25, 0.01f, (moe_policy)7, nullptr, 2, P, (float *)P, nullptr,
                              (int32_t *)P, (float *)P, (uint8_t *)P, P, BIG, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_forward_policy(P, MOE_BF16, (float *)P, nullptr, P, nullptr, nullptr, P, nullptr, MOE_ACT_RELU, 64,
                              64, 128, 8, 1, 1.25, 0.01f, MOE_POLICY_PRIORITY, nullptr, 0, P, (float *)P, nullptr,
                              (int32_t *)P, (float *)P, (uint8_t *)P, P, 16, nullptr), MOE_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(moe_forward_policy_workspace_bytes(64, 64, 128, 8, 1, 1.0, MOE_BF16, MOE_ACT_RELU, MOE_POLICY_REROUTE, 9),
           SIZE_MAX);
    EXPECT(moe_forward_policy_workspace_bytes(64, 64, 128, 8, 1, 1.0, MOE_BF16, MOE_ACT_RELU, MOE_POLICY_REROUTE, 4) >
           0, 1);
    if (failures) return 1;
    printf("abi checks passed\n");
    return 0;
}
