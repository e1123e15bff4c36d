// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace specverify {

// Per-device cache of a launch parameter derived from the device (CU count,
// resident workgroups of a kernel), 0 until filled. Relaxed atomics: host threads
// calling on different streams may fill an entry at the same time, always with the
// same value, without a data race.
struct DeviceMemo {
    std::atomic<int> v[64];
    int get(int dev) const { return (dev >= 0 && dev < 64) ? v[dev].load(std::memory_order_relaxed) : 0; }
    void put(int dev, int x) {
        if (dev >= 0 && dev < 64) v[dev].store(x, std::memory_order_relaxed);
    }
};

struct AttnLaunch {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* cu_drafts;   // [B+1] draft-count offsets (ragged k), or NULL: k drafts each
    const int32_t* parents;     // tree: [B][k] parent of node n at [n-1] (tree mask), or NULL
    void* out;
    int B, k, Hq, Hkv, D, block_size, max_blocks, num_blocks, max_seq_len;   // k: the largest k_b
    float sm_scale;
    void* workspace;
};

struct AttnGeometry {
    int rows;          // (k+1) * G query rows per KV head
    int tiles;         // 16-row MFMA tiles per row group (1 or 2)
    int row_groups;    // groups of up to 32 rows
    int chunk;         // keys per workgroup (multiple of 128)
    int splits;        // max KV splits per (sequence, KV head)
    size_t workspace;  // bytes
};

AttnGeometry attn_geometry(int B, int k, int Hq, int Hkv, int D, int max_seq_len);
hipError_t launch_attn(const AttnLaunch& p, const AttnGeometry& g, hipStream_t stream);

struct RejectLaunch {
    const float* target_logits;
    const float* draft_logits;
    const int32_t* draft_tokens;
    const int64_t* seq_ids;
    const int32_t* seq_lens;
    const int32_t* cu_drafts;   // [B+1] draft-count offsets (ragged k), or NULL: k drafts each
    const int32_t* parents;     // tree: [B][k] parent of node n at [n-1] (k = nodes), else NULL
    int32_t* out_nodes;         // tree: [B][k] accepted nodes, or NULL
    int B, k, V;                // k: the largest k_b (tree: the number of draft nodes)
    float temperature;
    uint64_t seed;
    int32_t* out_tokens;
    int32_t* num_accepted;
    float* out_probs;
    float* accept_probs;
    void* workspace;
};

size_t reject_workspace_bytes(int B, int k, int V);
int reject_max_vocab();   // largest V the reject kernel accepts
hipError_t launch_reject(const RejectLaunch& p, hipStream_t stream);
// How launch_reject runs a call of this shape on the current device: every level of every
// sequence at once, or the chain with W-wavefront workgroups (W = 4 or 8).
struct RejectPlan {
    bool levels;
    int W;
};
RejectPlan reject_plan(int B, int k, int V);
// The library's own sampling workspace for callers that cannot allocate: its size, and the
// current device's copy (looked up on the first call on each device; allocates nothing).
size_t reject_noalloc_scratch_bytes();
hipError_t reject_noalloc_scratch(void** ptr_out);
// The error word of a reject (chain or tree) workspace, copied to *flag_out and cleared.
hipError_t launch_reject_error_flag(void* workspace, int32_t* flag_out, hipStream_t stream);
size_t reject_tree_workspace_bytes(int B, int nodes, int V);
int reject_tree_max_branch();   // children per tree node the walk supports
hipError_t launch_reject_tree(const RejectLaunch& p, hipStream_t stream);

hipError_t launch_commit(int32_t* seq_lens, const int32_t* num_accepted, int B, int capacity,
                         int32_t* overflow_flags, hipStream_t stream);

struct TreeCommitLaunch {
    void* k_cache;
    void* v_cache;
    const int32_t* block_table;
    int32_t* seq_lens;
    const int32_t* accepted_nodes;   // [B][nodes]
    const int32_t* num_accepted;
    int32_t* overflow_flags;
    int B, nodes, Hkv, D, block_size, max_blocks, num_blocks, capacity;
};

// Moves the accepted path's KV rows to L+1 .. L+a, then commits the lengths.
hipError_t launch_tree_commit(const TreeCommitLaunch& p, hipStream_t stream);

struct RopeLaunch {
    void* q;                    // [B][k+1][Hq][D] bf16, rotated in place
    const void* k_new;          // [B][k+1][Hkv][D] bf16
    const void* v_new;          // [B][k+1][Hkv][D] bf16
    void* k_cache;
    void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* parents;     // tree: [B][k], or NULL
    int B, k, Hq, Hkv, D, block_size, max_blocks, num_blocks;
    double theta;
};

hipError_t launch_rope_append(const RopeLaunch& p, hipStream_t stream);

struct LmHeadLaunch {
    const void* hidden;   // [R][H] bf16
    const void* weight;   // [V][H] bf16
    float* logits;        // [R][V]
    int R, H, V;
};

int lm_head_k_multiple();
// false when the launch grid for R rows and V columns would exceed 2^23 workgroups
bool lm_head_grid_ok(int R, int V);   // H must be a multiple of this
hipError_t launch_lm_head(const LmHeadLaunch& p, hipStream_t stream);

}  // namespace specverify
