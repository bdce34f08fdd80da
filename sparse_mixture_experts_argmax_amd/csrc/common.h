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

__device__ __forceinline__ Cand cand_shfl_xor(const Cand &c, int m) {
    Cand o;
    o.v = __shfl_xor(c.v, m);
    o.i = __shfl_xor(c.i, m);
    o.ok = __shfl_xor(c.ok, m);
    return o;
}

}  // namespace moe
