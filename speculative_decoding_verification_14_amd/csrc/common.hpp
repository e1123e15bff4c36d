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

// 16-byte streaming load (nontemporal hint): for data read once per call, such
// as the KV cache, it streams past the caches instead of displacing them.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
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

// Wavefront reductions on the DPP network (VALU lane moves, no LDS round trip):
// quad swaps, then row shifts by 4 and 8 leave each 16-lane row's total in its
// lane 15; row broadcasts of lanes 15 and 31 fold the four rows into lane 63,
// which readlane hands to every lane. Lanes whose DPP source is out of range
// read the identity. The reduction order is fixed, so results are deterministic.
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ int dpp_move(int v, int identity) {
    return __builtin_amdgcn_update_dpp(identity, v, kCtrl, kRowMask, 0xF, false);
}

__device__ __forceinline__ float dpp_wave_max(float v) {
    const int id = __builtin_bit_cast(int, -INFINITY);
    auto step = [&](int moved) { v = fmaxf(v, __builtin_bit_cast(float, moved)); };
    step(dpp_move<0xB1>(__builtin_bit_cast(int, v), id));        // quad_perm [1,0,3,2]
    step(dpp_move<0x4E>(__builtin_bit_cast(int, v), id));        // quad_perm [2,3,0,1]
    step(dpp_move<0x114>(__builtin_bit_cast(int, v), id));       // row_shr:4
    step(dpp_move<0x118>(__builtin_bit_cast(int, v), id));       // row_shr:8
    step(dpp_move<0x142, 0xA>(__builtin_bit_cast(int, v), id));  // row_bcast:15 into rows 1, 3
    step(dpp_move<0x143, 0xC>(__builtin_bit_cast(int, v), id));  // row_bcast:31 into rows 2, 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ double dpp_move_f64(double v) {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const int lo = dpp_move<kCtrl, kRowMask>(static_cast<int>(u & 0xFFFFFFFFull), 0);
    const int hi = dpp_move<kCtrl, kRowMask>(static_cast<int>(u >> 32), 0);
    return __builtin_bit_cast(double, (static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                                          static_cast<unsigned>(lo));
}

__device__ __forceinline__ double dpp_wave_sum(double v) {
    v += dpp_move_f64<0xB1>(v);
    v += dpp_move_f64<0x4E>(v);
    v += dpp_move_f64<0x114>(v);
    v += dpp_move_f64<0x118>(v);
    v += dpp_move_f64<0x142, 0xA>(v);
    v += dpp_move_f64<0x143, 0xC>(v);
    const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
    const unsigned lo = __builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFull), 63);
    const unsigned hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), 63);
    return __builtin_bit_cast(double, (static_cast<unsigned long long>(hi) << 32) | lo);
}

// Inclusive prefix sum across the wavefront on the DPP network: Hillis-Steele
// shifts by 1, 2, 4, 8 inside each 16-lane row (lanes without a source add 0),
// then the row totals are carried into rows 1, 3 (lane 15 / 47) and 2, 3 (lane 31).
// No lane-id compares, fixed order, so deterministic.
__device__ __forceinline__ double dpp_wave_incl_scan(double v) {
    v += dpp_move_f64<0x111>(v);        // row_shr:1
    v += dpp_move_f64<0x112>(v);        // row_shr:2
    v += dpp_move_f64<0x114>(v);        // row_shr:4
    v += dpp_move_f64<0x118>(v);        // row_shr:8
    v += dpp_move_f64<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    v += dpp_move_f64<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
    return v;
}

// The value of the next-lower lane (0 in lane 0): the exclusive prefix when
// applied to an inclusive one.
__device__ __forceinline__ double dpp_wave_shr1(double v) { return dpp_move_f64<0x138>(v); }   // wave_shr:1

// The lane index within the wavefront behind an empty asm, so that lane-id
// compares are computed where they are used instead of being hoisted out of loops
// (a hoisted compare pins a 64-bit lane mask in scalar registers for the whole loop).
__device__ __forceinline__ int lane_id() {
    int l = static_cast<int>(threadIdx.x & 63u);
    asm volatile("" : "+v"(l));
    return l;
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
