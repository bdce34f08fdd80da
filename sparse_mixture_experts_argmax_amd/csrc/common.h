// Device helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 values to a packed pair of bf16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte global load / store through the vector memory path.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// The router z-loss (1/T) sum_t (log sum_i exp z_ti)^2 from per-block
// partial sums of the squared log-sum-exps ([CMU-L16] section 4.2), in fp64
// by one whole wave in a fixed order (lane-strided sums, then a butterfly),
// so the router's own reduction and the dispatch scan give the same bits;
// 0 for T = 0.  Every lane returns the value.
__device__ __forceinline__ float z_loss_wave(const float *part_z, int nblk, int64_t T, int lane) {
    double s = 0.0;
    for (int b = lane; b < nblk; b += 64) s += (double)part_z[b];
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    return T > 0 ? (float)(s / (double)T) : 0.f;
}

// Auxiliary load-balancing loss alpha * E * sum_i f_i P_i with
// f_i = route_count_i / (k T) and P_i = prob_sum_i / T ([SW-GLaM] "负载均衡"),
// in fp64 by one whole wave in a fixed order (lane l sums experts l, l + 64,
// ..., then a butterfly), so every caller gets the same bits.  COHERENT reads
// totals that other blocks of the running kernel wrote.
template <bool COHERENT>
__device__ __forceinline__ float aux_loss_wave(const int32_t *route_count, const float *prob_sum, int E,
                                               int64_t T, int k, float alpha, int lane) {
    double s = 0.0;
    for (int e = lane; e < E; e += 64) {
        int32_t rc;
        float ps;
        if (COHERENT) {
            rc = __hip_atomic_load(route_count + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ps = __hip_atomic_load(prob_sum + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            rc = route_count[e];
            ps = prob_sum[e];
        }
        s += (double)rc * (double)ps;
    }
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    const double Td = (double)T;
    return (T > 0) ? (float)((double)alpha * (double)E * s / ((double)k * Td * Td)) : 0.0f;
}

#define MOE_LDS_AS __attribute__((address_space(3)))
#define MOE_GLB_AS __attribute__((address_space(1)))

// s_waitcnt vmcnt(V) lgkmcnt(0) (expcnt left alone), gfx9 encoding.  The
// 16-byte LDS DMA (global_load_lds) is counted by vmcnt; a waitcnt of our own
// lets a stage be waited for while the newer stages stay in flight.
template <int V>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier for LDS rings filled by DMA.  The caller has already
// waited (wait_vm_lgkm0) for its own LDS accesses and for the DMA of the stage
// it needs; the barrier then makes every wave's part visible.  No fence: an
// LDS fence would also wait for the DMA of the newer stages (the compiler
// counts LDS DMA as LDS writes), draining the ring.  The empty asm statements
// keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup barrier that orders LDS accesses only (waits lgkmcnt, not vmcnt):
// global loads issued ahead for later steps stay in flight across it, which
// __syncthreads (a full fence) would drain.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Argmax candidate: larger value wins, equal values go to the lower index.
// `ok` false means "no candidate" and loses to any real one.
struct Cand {
    float v;
    int i;
    int ok;
};

__device__ __forceinline__ bool cand_better(const Cand &a, const Cand &b) {
    if (a.ok != b.ok) return a.ok > b.ok;
    if (a.v != b.v) return a.v > b.v;
    return a.i < b.i;
}

// Reductions over each row of 16 lanes with DPP lane moves (no LDS round
// trip): swap neighbours, swap pairs, mirror within 8, mirror within 16.
// After the four steps every lane of the row holds the same result (each
// step combines two groups that already agree internally).
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<DPP_XOR1>(v));
    v = fmaxf(v, dpp_f<DPP_XOR2>(v));
    v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
    return fmaxf(v, dpp_f<DPP_MIRROR>(v));
}
__device__ __forceinline__ int row16_min(int v) {
    v = min(v, dpp_i<DPP_XOR1>(v));
    v = min(v, dpp_i<DPP_XOR2>(v));
    v = min(v, dpp_i<DPP_HALF_MIRROR>(v));
    return min(v, dpp_i<DPP_MIRROR>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<DPP_XOR1>(v);
    v += dpp_f<DPP_XOR2>(v);
    v += dpp_f<DPP_HALF_MIRROR>(v);
    return v + dpp_f<DPP_MIRROR>(v);
}

__device__ __forceinline__ Cand cand_shfl_xor(const Cand &c, int m) {
    Cand o;
    o.v = __shfl_xor(c.v, m);
    o.i = __shfl_xor(c.i, m);
    o.ok = __shfl_xor(c.ok, m);
    return o;
}

}  // namespace moe
