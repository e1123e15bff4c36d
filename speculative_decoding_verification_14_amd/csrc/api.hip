// C-ABI of libspecverify.so: argument validation, launch geometry, status codes.
// The entry points and their contracts are declared in include/specverify.h.
#include <atomic>
#include <cmath>
#include <cstring>

#include "kernels.hpp"
#include "specverify.h"

using namespace specverify;

namespace {

// Per-device memo of the gfx950 check (0 unknown, 1 gfx950, 2 other); immutable once set.
std::atomic<int> g_arch_ok[64];

spec_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return SPEC_ERR_NO_DEVICE;
    }
    if (dev < 64) {
        const int memo = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (memo == 1) return SPEC_OK;
        if (memo == 2) return SPEC_ERR_NO_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return SPEC_ERR_NO_DEVICE;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? SPEC_OK : SPEC_ERR_NO_DEVICE;
}

bool is_pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

spec_status attn_shape_check(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len) {
    if (B < 1 || B > 65535) return SPEC_ERR_BAD_SHAPE;
    if (k < 0 || k > 15) return SPEC_ERR_BAD_SHAPE;   // k = 0: plain decode, one query row
    if (Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return SPEC_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return SPEC_ERR_BAD_SHAPE;
    if (max_seq_len < k + 1) return SPEC_ERR_BAD_SHAPE;
    const long long rows = static_cast<long long>(k + 1) * (Hq / Hkv);
    if (static_cast<long long>(Hkv) * ((rows + 31) / 32) > 65535) return SPEC_ERR_BAD_SHAPE;
    // the per-sequence work prefix (128-key iterations x row groups x KV heads) is kept in int32
    if (static_cast<long long>(B) * Hkv * ((rows + 31) / 32) * ((static_cast<long long>(max_seq_len) + 127) / 128) >
        0x7FFFFFFFLL)
        return SPEC_ERR_BAD_SHAPE;
    return SPEC_OK;
}

spec_status from_hip(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP; }

}  // namespace

namespace {

spec_status verify_attn_impl(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* cu_drafts, const int32_t* parents, void* out,
                             int32_t B, int32_t k,
                             int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks,
                             int32_t num_blocks, int32_t max_seq_len, float sm_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return SPEC_ERR_NULL_POINTER;
    spec_status s = attn_shape_check(B, k, Hq, Hkv, D, max_seq_len);
    if (s != SPEC_OK) return s;
    if (!is_pow2_in(block_size, 16, 64)) return SPEC_ERR_BAD_SHAPE;
    if (max_blocks < 1 || num_blocks < 1) return SPEC_ERR_BAD_SHAPE;
    if (!(std::isfinite(sm_scale) && sm_scale > 0.0f)) return SPEC_ERR_BAD_VALUE;
    const AttnGeometry geo = attn_geometry(B, k, Hq, Hkv, D, max_seq_len);
    if (geo.workspace > 0 && !workspace) return SPEC_ERR_NULL_POINTER;
    if (workspace_bytes < geo.workspace) return SPEC_ERR_WORKSPACE_TOO_SMALL;
    if ((s = check_device()) != SPEC_OK) return s;
    AttnLaunch p;
    p.q = q; p.k_cache = k_cache; p.v_cache = v_cache;
    p.block_table = block_table; p.seq_lens = seq_lens; p.cu_drafts = cu_drafts; p.parents = parents; p.out = out;
    p.B = B; p.k = k; p.Hq = Hq; p.Hkv = Hkv; p.D = D;
    p.block_size = block_size; p.max_blocks = max_blocks; p.num_blocks = num_blocks;
    p.max_seq_len = max_seq_len; p.sm_scale = sm_scale;
    p.workspace = workspace;
    return from_hip(launch_attn(p, geo, static_cast<hipStream_t>(stream)));
}

spec_status reject_impl(const float* target_logits, const float* draft_logits, const int32_t* draft_tokens,
                        const int32_t* cu_drafts, const int64_t* seq_ids, const int32_t* seq_lens, int32_t B,
                        int32_t k, int32_t V, float temperature, uint64_t seed, int32_t* out_tokens,
                        int32_t* num_accepted, float* out_probs, float* accept_probs, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (B < 1 || B > 65535 || k < 0 || k > 15 || V < 2 || V > reject_max_vocab()) return SPEC_ERR_BAD_SHAPE;
    // k = 0 (plain decode: the bonus draw from p_0 only) reads no draft rows or tokens
    if (!target_logits || (k > 0 && (!draft_logits || !draft_tokens)) || !seq_ids || !seq_lens || !out_tokens ||
        !num_accepted || !workspace)
        return SPEC_ERR_NULL_POINTER;
    if (!(std::isfinite(temperature) && temperature > 0.0f)) return SPEC_ERR_BAD_VALUE;
    if (workspace_bytes < reject_workspace_bytes(B, k, V)) return SPEC_ERR_WORKSPACE_TOO_SMALL;
    spec_status s = check_device();
    if (s != SPEC_OK) return s;
    RejectLaunch p;
    p.target_logits = target_logits; p.draft_logits = draft_logits; p.draft_tokens = draft_tokens;
    p.seq_ids = seq_ids; p.seq_lens = seq_lens; p.cu_drafts = cu_drafts; p.parents = nullptr; p.out_nodes = nullptr;
    p.B = B; p.k = k; p.V = V; p.temperature = temperature; p.seed = seed;
    p.out_tokens = out_tokens; p.num_accepted = num_accepted;
    p.out_probs = out_probs; p.accept_probs = accept_probs;
    p.workspace = workspace;
    return from_hip(launch_reject(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* spec_status_string(spec_status s) {
    switch (s) {
        case SPEC_OK: return "ok";
        case SPEC_ERR_NULL_POINTER: return "a required pointer argument is NULL";
        case SPEC_ERR_BAD_SHAPE: return "a size argument is outside the supported range";
        case SPEC_ERR_BAD_VALUE: return "a scalar argument (temperature or scale) is invalid";
        case SPEC_ERR_WORKSPACE_TOO_SMALL: return "workspace is smaller than the reported size";
        case SPEC_ERR_NO_DEVICE: return "no HIP device, or the current device is not gfx950";
        case SPEC_ERR_HIP: return "a HIP runtime call or kernel launch failed";
        case SPEC_ERR_UNIMPLEMENTED: return "shape combination not built into this library";
        default: return "unknown status";
    }
}

int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }

spec_status spec_verify_attn_workspace_size(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t max_seq_len, size_t* bytes_out) {
    if (!bytes_out) return SPEC_ERR_NULL_POINTER;
    const spec_status s = attn_shape_check(B, k, Hq, Hkv, D, max_seq_len);
    if (s != SPEC_OK) return s;
    *bytes_out = attn_geometry(B, k, Hq, Hkv, D, max_seq_len).workspace;
    return SPEC_OK;
}


spec_status spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, void* out,
                             int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t block_size, int32_t max_blocks, int32_t num_blocks,
                             int32_t max_seq_len, float sm_scale,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return verify_attn_impl(q, k_cache, v_cache, block_table, seq_lens, nullptr, nullptr, out, B, k, Hq, Hkv, D,
                            block_size, max_blocks, num_blocks, max_seq_len, sm_scale, workspace, workspace_bytes,
                            stream);
}

spec_status spec_verify_attn_ragged(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_drafts,
                                    void* out, int32_t B, int32_t max_k, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t block_size, int32_t max_blocks, int32_t num_blocks,
                                    int32_t max_seq_len, float sm_scale,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_drafts) return SPEC_ERR_NULL_POINTER;
    return verify_attn_impl(q, k_cache, v_cache, block_table, seq_lens, cu_drafts, nullptr, out, B, max_k, Hq, Hkv,
                            D, block_size, max_blocks, num_blocks, max_seq_len, sm_scale, workspace, workspace_bytes,
                            stream);
}

spec_status spec_verify_attn_tree(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, const int32_t* parents,
                                  void* out, int32_t B, int32_t nodes, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t block_size, int32_t max_blocks, int32_t num_blocks,
                                  int32_t max_seq_len, float sm_scale,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (!parents) return SPEC_ERR_NULL_POINTER;
    if (nodes < 1) return SPEC_ERR_BAD_SHAPE;
    return verify_attn_impl(q, k_cache, v_cache, block_table, seq_lens, nullptr, parents, out, B, nodes, Hq, Hkv, D,
                            block_size, max_blocks, num_blocks, max_seq_len, sm_scale, workspace, workspace_bytes,
                            stream);
}

spec_status spec_reject_sample_workspace_size(int32_t B, int32_t k, int32_t V, size_t* bytes_out) {
    if (!bytes_out) return SPEC_ERR_NULL_POINTER;
    if (B < 1 || B > 65535 || k < 0 || k > 15 || V < 2 || V > reject_max_vocab()) return SPEC_ERR_BAD_SHAPE;
    *bytes_out = reject_workspace_bytes(B, k, V);
    return SPEC_OK;
}

spec_status spec_reject_sample(const float* target_logits, const float* draft_logits,
                               const int32_t* draft_tokens, const int64_t* seq_ids,
                               const int32_t* seq_lens, int32_t B, int32_t k, int32_t V,
                               float temperature, uint64_t seed,
                               int32_t* out_tokens, int32_t* num_accepted,
                               float* out_probs, float* accept_probs,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return reject_impl(target_logits, draft_logits, draft_tokens, nullptr, seq_ids, seq_lens, B, k, V, temperature,
                       seed, out_tokens, num_accepted, out_probs, accept_probs, workspace, workspace_bytes, stream);
}

spec_status spec_reject_sample_noalloc(const float* target_logits, const float* draft_logits,
                                       const int32_t* draft_tokens, const int64_t* seq_ids,
                                       const int32_t* seq_lens, int32_t B, int32_t k, int32_t V,
                                       float temperature, uint64_t seed,
                                       int32_t* out_tokens, int32_t* num_accepted,
                                       float* out_probs, float* accept_probs, void* stream) {
    if (B < 1 || B > 65535 || k < 0 || k > 15 || V < 2 || V > reject_max_vocab()) return SPEC_ERR_BAD_SHAPE;
    if (reject_workspace_bytes(B, k, V) > reject_noalloc_scratch_bytes()) return SPEC_ERR_WORKSPACE_TOO_SMALL;
    // the rest of the host validation happens in reject_impl, before anything is enqueued
    if (!target_logits || (k > 0 && (!draft_logits || !draft_tokens)) || !seq_ids || !seq_lens || !out_tokens ||
        !num_accepted)
        return SPEC_ERR_NULL_POINTER;
    if (!(std::isfinite(temperature) && temperature > 0.0f)) return SPEC_ERR_BAD_VALUE;
    spec_status s = check_device();
    if (s != SPEC_OK) return s;
    void* scratch = nullptr;
    if (reject_noalloc_scratch(&scratch) != hipSuccess) {
        (void)hipGetLastError();
        return SPEC_ERR_HIP;
    }
    return reject_impl(target_logits, draft_logits, draft_tokens, nullptr, seq_ids, seq_lens, B, k, V, temperature,
                       seed, out_tokens, num_accepted, out_probs, accept_probs, scratch,
                       reject_noalloc_scratch_bytes(), stream);
}

spec_status spec_reject_sample_ragged(const float* target_logits, const float* draft_logits,
                                      const int32_t* draft_tokens, const int32_t* cu_drafts,
                                      const int64_t* seq_ids, const int32_t* seq_lens, int32_t B, int32_t max_k,
                                      int32_t V, float temperature, uint64_t seed,
                                      int32_t* out_tokens, int32_t* num_accepted,
                                      float* out_probs, float* accept_probs,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_drafts) return SPEC_ERR_NULL_POINTER;
    return reject_impl(target_logits, draft_logits, draft_tokens, cu_drafts, seq_ids, seq_lens, B, max_k, V,
                       temperature, seed, out_tokens, num_accepted, out_probs, accept_probs, workspace,
                       workspace_bytes, stream);
}

spec_status spec_reject_sample_tree_workspace_size(int32_t B, int32_t nodes, int32_t V, size_t* bytes_out) {
    if (!bytes_out) return SPEC_ERR_NULL_POINTER;
    if (B < 1 || B > 65535 || nodes < 1 || nodes > 15 || V < 2 || V > reject_max_vocab()) return SPEC_ERR_BAD_SHAPE;
    *bytes_out = reject_tree_workspace_bytes(B, nodes, V);
    return SPEC_OK;
}

spec_status spec_reject_sample_tree(const float* target_logits, const float* draft_logits,
                                    const int32_t* draft_tokens, const int32_t* parents, const int64_t* seq_ids,
                                    const int32_t* seq_lens, int32_t B, int32_t nodes, int32_t V,
                                    float temperature, uint64_t seed, int32_t* out_tokens, int32_t* num_accepted,
                                    int32_t* accepted_nodes, float* out_probs, float* accept_probs,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 1 || B > 65535 || nodes < 1 || nodes > 15 || V < 2 || V > reject_max_vocab()) return SPEC_ERR_BAD_SHAPE;
    if (!target_logits || !draft_logits || !draft_tokens || !parents || !seq_ids || !seq_lens || !out_tokens ||
        !num_accepted || !workspace)
        return SPEC_ERR_NULL_POINTER;
    if (!(std::isfinite(temperature) && temperature > 0.0f)) return SPEC_ERR_BAD_VALUE;
    if (workspace_bytes < reject_tree_workspace_bytes(B, nodes, V)) return SPEC_ERR_WORKSPACE_TOO_SMALL;
    spec_status s = check_device();
    if (s != SPEC_OK) return s;
    RejectLaunch p;
    p.target_logits = target_logits; p.draft_logits = draft_logits; p.draft_tokens = draft_tokens;
    p.seq_ids = seq_ids; p.seq_lens = seq_lens; p.cu_drafts = nullptr; p.parents = parents;
    p.out_nodes = accepted_nodes;
    p.B = B; p.k = nodes; p.V = V; p.temperature = temperature; p.seed = seed;
    p.out_tokens = out_tokens; p.num_accepted = num_accepted;
    p.out_probs = out_probs; p.accept_probs = accept_probs;
    p.workspace = workspace;
    return from_hip(launch_reject_tree(p, static_cast<hipStream_t>(stream)));
}

spec_status spec_reject_error_flag(void* workspace, int32_t* flag_out, void* stream) {
    if (!workspace || !flag_out) return SPEC_ERR_NULL_POINTER;
    const spec_status s = check_device();
    if (s != SPEC_OK) return s;
    return from_hip(launch_reject_error_flag(workspace, flag_out, static_cast<hipStream_t>(stream)));
}

spec_status spec_reject_sample_plan(int32_t B, int32_t k, int32_t V, int32_t* mode_out) {
    if (!mode_out) return SPEC_ERR_NULL_POINTER;
    if (B < 1 || B > 65535 || k < 0 || k > 15 || V < 2 || V > (1 << 20)) return SPEC_ERR_BAD_SHAPE;
    const spec_status s = check_device();
    if (s != SPEC_OK) return s;
    const RejectPlan plan = reject_plan(B, k, V);
    *mode_out = plan.levels ? 2 : (plan.W == 4 ? 1 : 0);
    return SPEC_OK;
}

spec_status spec_commit_lengths(int32_t* seq_lens, const int32_t* num_accepted, int32_t B, int32_t k,
                                int32_t capacity_tokens, int32_t* overflow_flags, void* stream) {
    if (!seq_lens || !num_accepted) return SPEC_ERR_NULL_POINTER;
    if (B < 1 || k < 0 || k > 15 || capacity_tokens < 1) return SPEC_ERR_BAD_SHAPE;
    const spec_status s = check_device();
    if (s != SPEC_OK) return s;
    return from_hip(launch_commit(seq_lens, num_accepted, B, capacity_tokens, overflow_flags,
                                  static_cast<hipStream_t>(stream)));
}

spec_status spec_commit_tree(void* k_cache, void* v_cache, const int32_t* block_table, int32_t* seq_lens,
                             const int32_t* accepted_nodes, const int32_t* num_accepted, int32_t B,
                             int32_t nodes, int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks,
                             int32_t num_blocks, int32_t capacity_tokens, int32_t* overflow_flags, void* stream) {
    if (!k_cache || !v_cache || !block_table || !seq_lens || !accepted_nodes || !num_accepted)
        return SPEC_ERR_NULL_POINTER;
    if (B < 1 || B > 65535 || nodes < 1 || nodes > 15 || Hkv < 1 || Hkv > 65535) return SPEC_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return SPEC_ERR_BAD_SHAPE;
    if (!is_pow2_in(block_size, 16, 64) || max_blocks < 1 || num_blocks < 1 || capacity_tokens < 1)
        return SPEC_ERR_BAD_SHAPE;
    const spec_status s = check_device();
    if (s != SPEC_OK) return s;
    TreeCommitLaunch p;
    p.k_cache = k_cache; p.v_cache = v_cache; p.block_table = block_table; p.seq_lens = seq_lens;
    p.accepted_nodes = accepted_nodes; p.num_accepted = num_accepted; p.overflow_flags = overflow_flags;
    p.B = B; p.nodes = nodes; p.Hkv = Hkv; p.D = D; p.block_size = block_size; p.max_blocks = max_blocks;
    p.num_blocks = num_blocks; p.capacity = capacity_tokens;
    return from_hip(launch_tree_commit(p, static_cast<hipStream_t>(stream)));
}

spec_status spec_rope_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, const int32_t* parents,
                             int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                             int32_t max_blocks, int32_t num_blocks, double rope_theta, void* stream) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !block_table || !seq_lens) return SPEC_ERR_NULL_POINTER;
    if (B < 1 || B > 65535 || k < 0 || k > 15 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0) return SPEC_ERR_BAD_SHAPE;
    if (parents && k < 1) return SPEC_ERR_BAD_SHAPE;
    if (D != 64 && D != 128) return SPEC_ERR_BAD_SHAPE;
    if (!is_pow2_in(block_size, 16, 64) || max_blocks < 1 || num_blocks < 1) return SPEC_ERR_BAD_SHAPE;
    if (!(std::isfinite(rope_theta) && rope_theta > 1.0)) return SPEC_ERR_BAD_VALUE;
    const spec_status s = check_device();
    if (s != SPEC_OK) return s;
    RopeLaunch p;
    p.q = q; p.k_new = k_new; p.v_new = v_new; p.k_cache = k_cache; p.v_cache = v_cache;
    p.block_table = block_table; p.seq_lens = seq_lens; p.parents = parents;
    p.B = B; p.k = k; p.Hq = Hq; p.Hkv = Hkv; p.D = D; p.block_size = block_size; p.max_blocks = max_blocks;
    p.num_blocks = num_blocks; p.theta = rope_theta;
    return from_hip(launch_rope_append(p, static_cast<hipStream_t>(stream)));
}

spec_status spec_lm_head(const void* hidden, const void* weight, float* logits, int32_t R, int32_t H, int32_t V,
                         void* stream) {
    if (!hidden || !weight || !logits) return SPEC_ERR_NULL_POINTER;
    if (R < 1 || R > 65535 * 256 || V < 1 || H < lm_head_k_multiple() || H % lm_head_k_multiple() != 0)
        return SPEC_ERR_BAD_SHAPE;
    if (H > (1 << 20) || static_cast<long long>(V) * H > (1LL << 40) || !lm_head_grid_ok(R, V))
        return SPEC_ERR_BAD_SHAPE;
    const spec_status s = check_device();
    if (s != SPEC_OK) return s;
    LmHeadLaunch p;
    p.hidden = hidden; p.weight = weight; p.logits = logits; p.R = R; p.H = H; p.V = V;
    return from_hip(launch_lm_head(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
