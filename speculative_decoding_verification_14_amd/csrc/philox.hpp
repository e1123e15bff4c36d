// Philox4x32-10 counter-based generator (Salmon, Moraes, Dror & Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, Philox section):
// ten rounds; each round takes the 32x32->64-bit products of counter words 0
// and 2 with two fixed odd multipliers, and forms the new counter from the
// high halves xor the other two words xor the round key, and the low halves;
// the key is advanced by two Weyl constants between rounds.
//
// Verify-step keying: key = (seed lo, seed hi), counter = (position,
// seq_id lo, seq_id hi, 0). A uniform is the top 24 bits of a word times 2^-24.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specverify {

struct PhiloxWords {
    uint32_t w[4];
};

__host__ __device__ __forceinline__ PhiloxWords philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                              uint32_t c3, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;
    constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t prod0 = static_cast<uint64_t>(kMul0) * c0;
        const uint64_t prod1 = static_cast<uint64_t>(kMul1) * c2;
        const uint32_t n0 = static_cast<uint32_t>(prod1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = static_cast<uint32_t>(prod1);
        const uint32_t n2 = static_cast<uint32_t>(prod0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = static_cast<uint32_t>(prod0);
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += kWeyl0;
        k1 += kWeyl1;
    }
    PhiloxWords out;
    out.w[0] = c0; out.w[1] = c1; out.w[2] = c2; out.w[3] = c3;
    return out;
}

__host__ __device__ __forceinline__ double word_to_unit(uint32_t w) {
    return static_cast<double>(w >> 8) * (1.0 / 16777216.0);
}

// Words 0 and 1 as uniforms for counter (pos, seq_id lo, seq_id hi, stream).
__host__ __device__ __forceinline__ void stream_uniforms(uint64_t seed, int64_t seq_id, int64_t pos, uint32_t stream,
                                                         double* u0, double* u1) {
    const uint64_t sid = static_cast<uint64_t>(seq_id);
    const PhiloxWords w = philox4x32_10(static_cast<uint32_t>(pos), static_cast<uint32_t>(sid),
                                        static_cast<uint32_t>(sid >> 32), stream,
                                        static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
    *u0 = word_to_unit(w.w[0]);
    *u1 = word_to_unit(w.w[1]);
}

// (u_acc, u_smp) for the token decided at absolute position `pos` of sequence `seq_id`
// (stream 0). Tree verification draws the acceptance uniform of a node's i-th
// candidate, i >= 2, from word 0 of stream i (stream 1 belongs to draft sampling).
__host__ __device__ __forceinline__ void verify_uniforms(uint64_t seed, int64_t seq_id, int64_t pos,
                                                         double* u_acc, double* u_smp) {
    stream_uniforms(seed, seq_id, pos, 0u, u_acc, u_smp);
}

}  // namespace specverify
