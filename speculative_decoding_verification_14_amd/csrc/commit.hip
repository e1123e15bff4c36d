// Cache-length commit after a verify step (gfx950).
//
// "Accelerating RL Post-Training Rollouts via System-Integrated Speculative
// Decoding" (gist.science explainer): the accepted drafts plus the verifier's
// own token are adopted together; "ReSpec: Towards Optimizing Speculative
// Decoding in Reinforcement Learning Systems" (talk notes), "Adaptive Server":
// speculation extends the KV cache in place. After a accepted drafts the
// committed length grows by a + 1, unless that passes the cache capacity.
#include "common.hpp"
#include "kernels.hpp"

namespace specverify {
namespace {

__global__ __launch_bounds__(256) void commit_kernel(int32_t* seq_lens, const int32_t* num_accepted, int B,
                                                     int capacity, int32_t* overflow_flags) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const long long proposed = static_cast<long long>(seq_lens[b]) + num_accepted[b] + 1;
    const bool over = proposed > capacity;
    if (!over) seq_lens[b] = static_cast<int32_t>(proposed);
    if (overflow_flags) overflow_flags[b] = over ? 1 : 0;
}

}  // namespace

hipError_t launch_commit(int32_t* seq_lens, const int32_t* num_accepted, int B, int capacity,
                         int32_t* overflow_flags, hipStream_t stream) {
    hipLaunchKernelGGL(commit_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, seq_lens, num_accepted, B,
                       capacity, overflow_flags);
    return hipGetLastError();
}

}  // namespace specverify
