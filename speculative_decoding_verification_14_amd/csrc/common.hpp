// Shared device helpers for the gfx950 verify-step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specverify {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load as raw dwords (global_load_dwordx4).
__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

// Butterfly reductions across a 64-lane wavefront (fixed order, hence deterministic).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Release (writer) / acquire (reader) ordering at device (agent) scope, so
// workgroups on different XCDs see each other's partial results.
__device__ __forceinline__ unsigned arrive_acq_rel(unsigned* counter) {
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void counter_reset(unsigned* counter) {
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void fence_acquire_agent() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ void fence_release_agent() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}

}  // namespace specverify
