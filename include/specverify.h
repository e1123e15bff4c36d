/*
 * specverify.h - C-ABI of libspecverify.so: the target-side verify step of
 * lossless speculative decoding on one AMD Instinct MI355X (gfx950).
 *
 * One verify step of a batch of B sequences is three calls on one stream:
 *   spec_verify_attn     paged-KV attention of the k+1 verify rows
 *   spec_reject_sample   vocab-wide softmax + acceptance chain + residual / bonus sample
 *   spec_commit_lengths  the accepted length rolls each cache length forward
 *
 * Conventions shared by every call:
 *  - All data pointers are device pointers owned by the caller, contiguous and
 *    row-major as documented per argument. The library allocates nothing and
 *    never synchronises: work is enqueued on `stream` (a hipStream_t; NULL means
 *    the default stream) and the caller synchronises. Its only global state is a
 *    per-device cache of launch parameters read from the device (CU count,
 *    resident workgroups per kernel, whether it is gfx950), filled on first use
 *    with atomic stores, so host threads may call concurrently. Calls on
 *    different streams may run concurrently if they use different workspaces and
 *    outputs; spec_reject_sample* additionally needs the device to itself while
 *    it runs (see there).
 *  - Host-side arguments are validated before anything is enqueued; on any
 *    error nothing is enqueued and an error code is returned. Device-resident
 *    data (token ids, block ids, lengths) is a documented precondition and is
 *    not checked.
 *  - Workspaces are caller-allocated device memory of at least the size the
 *    matching *_workspace_size call reports, ZERO-FILLED ONCE after allocation.
 *    Every call leaves a workspace ready for the next one (the reject
 *    workspace carries a call counter that tags its exchange slots), so a
 *    workspace is reused across calls without clearing; two calls in flight
 *    at the same time must not share one.
 *  - No C++ exception crosses this interface.
 *  - k, the number of drafted tokens, is chosen per call, 0 <= k <= 15. k = 0
 *    is plain (non-speculative) decoding through the same three calls: one
 *    query row, one token drawn from the target distribution, the length
 *    advanced by one. This is the switch between speculative and plain decoding
 *    that [RESP] (adaptive server) and [EFR] (speculation toggled by regime)
 *    make at run time, without a separate decode kernel.
 *
 * Beyond the plain three-call interface, by design:
 *  - V pages are [num_blocks][Hkv][D][block_size] (key index fastest), not the K
 *    pages' [num_blocks][Hkv][block_size][D]: a 16-byte load of a V page row is
 *    then eight consecutive keys of one dimension, the B-operand fragment of the
 *    P.V matrix product, so V streams from memory straight into matrix-core
 *    registers. The caller's append writes V in this layout (spec_rope_append does).
 *  - spec_reject_sample takes a workspace (and spec_reject_sample_workspace_size
 *    sizes it): the workgroups that share a sequence's vocabulary exchange partial
 *    statistics through it while the kernel runs.
 *  - spec_reject_error_flag reports whether a sampling call had to give up a wait;
 *    spec_reject_sample_plan says which way a sampling call of a given shape runs.
 *  - Ragged draft lengths, tree verification and the upstream steps (RoPE with the
 *    KV append, the LM head) have calls of their own.
 *
 * Sources for what is computed (page titles; the pages print no API):
 *  [ACC]  "Accelerating RL Post-Training Rollouts via System-Integrated
 *         Speculative Decoding" (gist.science summary), section 2 "Method",
 *         core mechanism: the draft proposes k tokens, the target verifies all
 *         of them in one forward pass, rejection sampling against the target's
 *         distribution keeps the rollout distribution identical to the policy.
 *  [ODC]  "Online Draft Co-Training for Speculative Decoding in Large-Scale,
 *         Long-Context RL Post-Training" (ta-paperlens commentary), metaphor
 *         section: the verifier rewrites from the first draft token that misses.
 *  [RESP] "ReSpec: Towards Optimizing Speculative Decoding in Reinforcement
 *         Learning Systems" (talk notes), "Adaptive Server": speculation
 *         extends the KV cache; accepted length is the progress measure (GAP 2).
 *  [EFR]  "EfficientRollout: System-Aware Self-Speculative Decoding for RL
 *         Rollouts", abstract: long, high-temperature generations; the active
 *         batch shrinks during a rollout.
 *  The acceptance rule itself is standard speculative sampling (Leviathan et
 *  al. 2023; Chen et al. 2023); Philox4x32-10 is from Salmon et al., SC'11.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t spec_status;

#define SPEC_OK                       0
#define SPEC_ERR_NULL_POINTER         1  /* a required pointer argument is NULL            */
#define SPEC_ERR_BAD_SHAPE            2  /* a size argument is out of the supported range  */
#define SPEC_ERR_BAD_VALUE            3  /* a scalar (temperature, scale) is invalid       */
#define SPEC_ERR_WORKSPACE_TOO_SMALL  4  /* workspace_bytes below the reported size        */
#define SPEC_ERR_NO_DEVICE            5  /* no HIP device, or the current device is not gfx950 */
#define SPEC_ERR_HIP                  6  /* a HIP runtime call or kernel launch failed     */
#define SPEC_ERR_UNIMPLEMENTED        7  /* shape combination not built into this library  */

#define SPEC_ABI_VERSION 1

/* Static string for a status code (never NULL). */
const char* spec_status_string(spec_status s);

/* SPEC_ABI_VERSION of the loaded library. */
int32_t spec_abi_version(void);

/* ------------------------------------------------------------------------
 * Verify attention  [ACC]: all k drafted tokens are checked in one target pass.
 *
 * For every sequence b the cache already holds its L_b committed tokens plus
 * the k+1 verify tokens [x_last, d_0 .. d_{k-1}] at positions L_b .. L_b+k
 * (the caller appends their K/V rows before this call). Query row i
 * (0 <= i <= k) attends to keys 0 .. L_b+i (causal inside the draft);
 * query head h reads KV head h / (Hq/Hkv). Scores are sm_scale * q.k, softmax
 * in fp32, output in bf16 (round to nearest even).
 *
 *  q            bf16  [B][k+1][Hq][D]
 *  k_cache      bf16  [num_blocks][Hkv][block_size][D]
 *  v_cache      bf16  [num_blocks][Hkv][D][block_size]   (key index fastest)
 *  block_table  int32 [B][max_blocks]   logical page -> physical page
 *  seq_lens     int32 [B]   committed length L_b (keys read: L_b + k + 1)
 *  out          bf16  [B][k+1][Hq][D]
 *
 * Shapes: 1 <= B <= 65535; 0 <= k <= 15; Hkv >= 1; Hq % Hkv == 0; D in {64, 128};
 * block_size in {16, 32, 64}; max_blocks >= 1; num_blocks >= 1;
 * max_seq_len >= k + 1; sm_scale finite and > 0.
 * Device preconditions: L_b + k + 1 <= min(max_seq_len, max_blocks*block_size);
 * the first ceil((L_b+k+1)/block_size) block-table entries of b are < num_blocks.
 * Entries past that are never read. Cache slots past key L_b+k are never read
 * into the result (their contents may be anything, NaN included).
 * Workspace: spec_verify_attn_workspace_size(B, k, Hq, Hkv, D, max_seq_len).
 * ---------------------------------------------------------------------- */
spec_status spec_verify_attn_workspace_size(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t max_seq_len, size_t* bytes_out);

spec_status spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, void* out,
                             int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t D,
                             int32_t block_size, int32_t max_blocks, int32_t num_blocks,
                             int32_t max_seq_len, float sm_scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Verify attention with ragged draft lengths  [EFR] (abstract: the draft length
 * adapts to acceptance), [RESP] (GAP 1 and the Adaptive Server: the speculation
 * configuration is chosen per batch as it shrinks).
 *
 * As spec_verify_attn, except that sequence b has its own draft count
 * k_b = cu_drafts[b+1] - cu_drafts[b] (0 <= k_b <= max_k) and the query and
 * output rows are packed: sequence b's rows i = 0 .. k_b are rows
 * cu_drafts[b] + b + i of
 *
 *  q    bf16 [R][Hq][D],  out  bf16 [R][Hq][D],  R = cu_drafts[B] + B
 *  cu_drafts  int32 [B+1] device array, cu_drafts[0] = 0, non-decreasing
 *
 * Row i of sequence b attends keys 0 .. L_b + i; L_b + k_b + 1 keys are read.
 * The offsets are a device-side precondition (not checked; k_b is clamped into
 * [0, max_k]). Shapes and workspace are those of spec_verify_attn with k = max_k
 * (spec_verify_attn_workspace_size(B, max_k, ...)); SPEC_ERR_NULL_POINTER if
 * cu_drafts is NULL. With every k_b = max_k the result equals spec_verify_attn's.
 * ---------------------------------------------------------------------- */
spec_status spec_verify_attn_ragged(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, const int32_t* cu_drafts,
                                    void* out, int32_t B, int32_t max_k, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t block_size, int32_t max_blocks, int32_t num_blocks,
                                    int32_t max_seq_len, float sm_scale,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Rejection sampling  [ACC], [ODC], [EFR].
 *
 * p_j = softmax(target_logits[b][j] / T), q_j = softmax(draft_logits[b][j] / T).
 * For j = 0 .. k-1, at position P = L_b + 1 + j with (u_acc, u_smp) =
 * Philox4x32-10(counter = (P, seq_id lo, seq_id hi, 0), key = (seed lo, seed hi)),
 * u = (word >> 8) * 2^-24 from words 0 and 1: accept d_j iff u_acc < p_j(d_j)/q_j(d_j)
 * (q_j(d_j) = 0 counts as +inf when p_j(d_j) > 0). The first rejection at j emits
 * a sample of max(0, p_j - q_j) (normalised) and stops; if all k are accepted a
 * bonus token is drawn from p_k with u_smp at P = L_b + 1 + k. Sampling is
 * inverse-CDF in ascending token id: the smallest y with C(y) > u_smp * C(V-1).
 *
 *  target_logits fp32 [B][k+1][V]      draft_logits fp32 [B][k][V]
 *  draft_tokens  int32 [B][k]  (each < V)
 *  seq_ids       int64 [B]  stable per-sequence ids (batch-slot independent)
 *  seq_lens      int32 [B]  committed lengths L_b (read only)
 *  out_tokens    int32 [B][k+1]  accepted drafts, then the sampled token at index
 *                num_accepted[b], then -1
 *  num_accepted  int32 [B]  a_b in [0, k]
 *  out_probs     fp32 [B][k+1] or NULL: p_i(out_tokens[b][i]) for i <= a_b, 0 after
 *  accept_probs  fp32 [B][k]   or NULL: min(1, p_j/q_j) at d_j for tested j, -1 for untested
 *
 * Shapes: 1 <= B <= 65535; 0 <= k <= 15; 2 <= V <= 1048576; temperature finite
 * and > 0. Logits are finite (padding of -inf is allowed; NaN is not).
 * k = 0: no draft is tested; out_tokens[b][0] is drawn from p_0 with u_smp at
 * P = L_b + 1 and num_accepted[b] = 0. draft_logits, draft_tokens and
 * accept_probs are not read or written and may be NULL.
 * Rows read: when the levels run one after another (the usual case) a row after
 * a sequence's first rejection is not read and no row is read twice (the heavy
 * logits, probability above 2^-14, are re-read for fp64 weights). When every
 * level of every sequence fits the device at once (small batches: B (k+1)
 * ceil(V / 16384) <= the CU count, or twice that for k <= 3) the levels run at
 * once and all 2k+1 rows of each sequence are read; the outputs are the same bits.
 * Residency: the workgroups of one sequence (ceil(V / 32768) of 512 threads, or
 * ceil(V / 16384) of 256 threads) exchange partial sums while running, so the grid
 * is sized to what the device holds at once and a plain launch assumes all of it
 * is resident together (SPEC_ERR_HIP if the device cannot hold one sequence's
 * workgroups). The call therefore needs the device to itself while it runs:
 * another kernel running beside it can leave part of the grid waiting for a CU.
 * Every wait is bounded (2^20 polls, about 10 ms): should one give up, the kernel
 * still ends, the affected sequences report num_accepted = -1 (their other
 * outputs are not written) and the workspace's error word is set; read it with
 * spec_reject_error_flag. The outputs of a call do not depend on timing, so a call
 * with any -1 can be repeated on an otherwise idle device for the intended result.
 * Workspace: spec_reject_sample_workspace_size(B, k, V).
 * ---------------------------------------------------------------------- */
spec_status spec_reject_sample_workspace_size(int32_t B, int32_t k, int32_t V, size_t* bytes_out);

spec_status spec_reject_sample(const float* target_logits, const float* draft_logits,
                               const int32_t* draft_tokens, const int64_t* seq_ids,
                               const int32_t* seq_lens, int32_t B, int32_t k, int32_t V,
                               float temperature, uint64_t seed,
                               int32_t* out_tokens, int32_t* num_accepted,
                               float* out_probs, float* accept_probs,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Rejection sampling without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Computes exactly what spec_reject_sample computes, with the same arguments and
 * outputs, but uses the library's own workspace: a 16 MiB device array of the
 * library, one copy per GPU, zero when the library is loaded and held until the
 * process ends. Nothing is allocated: the array's device address is looked up
 * (hipGetSymbolAddress) on the first call on each device and kept.
 * Limit: spec_reject_sample_workspace_size(B, k, V) must not exceed 16 MiB
 * (SPEC_ERR_WORKSPACE_TOO_SMALL otherwise; e.g. B = 1024 at k = 3, V = 128256
 * fits, B = 4096 does not). Every call on a GPU shares that GPU's array, which
 * carries the call counter from one call to the next, so no clearing is needed
 * between calls; calls that overlap on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller. As for
 * spec_reject_sample, a sequence whose bounded wait gave up reports
 * num_accepted = -1.
 * ---------------------------------------------------------------------- */
spec_status spec_reject_sample_noalloc(const float* target_logits, const float* draft_logits,
                                       const int32_t* draft_tokens, const int64_t* seq_ids,
                                       const int32_t* seq_lens, int32_t B, int32_t k, int32_t V,
                                       float temperature, uint64_t seed,
                                       int32_t* out_tokens, int32_t* num_accepted,
                                       float* out_probs, float* accept_probs, void* stream);

/* ------------------------------------------------------------------------
 * Error word of a sampling workspace (spec_reject_sample, _ragged or _tree).
 *
 * Copies the workspace's error word to *flag_out (a device int32) and clears it,
 * in one single-thread launch on `stream` (no memset, so it may be captured in a
 * graph). The word is nonzero if, since the last read, a bounded wait of a sampling
 * call on this workspace gave up (see spec_reject_sample) or a tree broke its
 * documented shape. Every sequence that reports num_accepted = -1 sets it; a
 * sequence whose other workgroups completed it despite one giving up has correct
 * outputs, though the word is set. Setting the
 * environment variable SPECVERIFY_SPIN_LIMIT (polls per wait, 0 .. 2^20) before the
 * first sampling call of a process shortens every wait; it exists to exercise this
 * path in tests.
 * ---------------------------------------------------------------------- */
spec_status spec_reject_error_flag(void* workspace, int32_t* flag_out, void* stream);

/* ------------------------------------------------------------------------
 * How spec_reject_sample (or _ragged, with k = the largest k_b) runs a call of
 * shape (B, k, V) on the current device, so that a caller can account for the rows
 * it reads (see "Rows read" under spec_reject_sample):
 *   *mode_out = 0  the levels one after another, workgroups of 512 threads
 *               (rows after a sequence's first rejection are not read);
 *   *mode_out = 1  the same with workgroups of 256 threads;
 *   *mode_out = 2  every level of every sequence at once (all 2k+1 rows read).
 * Host only: enqueues nothing. Errors: SPEC_ERR_NULL_POINTER, SPEC_ERR_BAD_SHAPE
 * (the shape spec_reject_sample accepts), SPEC_ERR_HIP / SPEC_ERR_NO_DEVICE.
 * ---------------------------------------------------------------------- */
spec_status spec_reject_sample_plan(int32_t B, int32_t k, int32_t V, int32_t* mode_out);

/* ------------------------------------------------------------------------
 * Rejection sampling with ragged draft lengths  [EFR] (acceptance-aware draft
 * length), [RESP] (GAP 1, Adaptive Server).
 *
 * As spec_reject_sample, with sequence b's k_b = cu_drafts[b+1] - cu_drafts[b]
 * (0 <= k_b <= max_k) and its rows packed (T = cu_drafts[B] + B, K = cu_drafts[B]):
 *
 *  target_logits fp32 [T][V]   rows cu_drafts[b] + b + j, j = 0 .. k_b
 *  draft_logits  fp32 [K][V]   rows cu_drafts[b] + j,     j = 0 .. k_b - 1
 *  draft_tokens  int32 [K]     same indexing as draft_logits
 *  out_tokens    int32 [T], out_probs fp32 [T] or NULL: same indexing as target_logits
 *  accept_probs  fp32 [K] or NULL: same indexing as draft_logits
 *  num_accepted  int32 [B]: a_b in [0, k_b]
 *
 * The chain of sequence b runs over its own k_b drafts (positions L_b + 1 + j);
 * k_b = 0 is plain decoding for that sequence. Shapes and workspace are those of
 * spec_reject_sample with k = max_k (spec_reject_sample_workspace_size(B, max_k,
 * V)); draft_logits and draft_tokens may be NULL when max_k = 0. The offsets are
 * a device-side precondition (not checked; k_b is clamped into [0, max_k]).
 * With every k_b = max_k the outputs equal spec_reject_sample's.
 * ---------------------------------------------------------------------- */
spec_status spec_reject_sample_ragged(const float* target_logits, const float* draft_logits,
                                      const int32_t* draft_tokens, const int32_t* cu_drafts,
                                      const int64_t* seq_ids, const int32_t* seq_lens, int32_t B, int32_t max_k,
                                      int32_t V, float temperature, uint64_t seed,
                                      int32_t* out_tokens, int32_t* num_accepted,
                                      float* out_probs, float* accept_probs,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Tree verification  [RESP] (GAP 1: speculation with a branching factor t; the
 * drafts form a tree that one target pass checks). The pages give neither the
 * mask nor the acceptance rule; the ones below are multi-candidate speculative
 * sampling (SpecInfer, Miao et al. 2024), which keeps the output distribution
 * equal to the target's when each node's children were drawn independently from
 * the draft distribution at that node.
 *
 * Tree of one sequence: node 0 is the last committed token (position L_b), nodes
 * 1 .. N (N = nodes) are drafts; parents[b][n-1] in [0, n) is node n's parent, and
 * node n sits at position L_b + depth(n). The children of a node, in index order,
 * are its candidates; at most 4 per node.
 *
 * spec_verify_attn_tree: as spec_verify_attn with k = N (q, out [B][N+1][Hq][D];
 * the caller has appended the KV rows of nodes 0 .. N at cache slots
 * L_b .. L_b + N), except that node n attends the committed keys 0 .. L_b - 1 and
 * the slots L_b + m of its ancestors m and itself (the tree mask). Workspace:
 * spec_verify_attn_workspace_size(B, N, ...). 1 <= N <= 15. Parents are a
 * device-side precondition: an index outside [0, n) is read as the nearest one
 * inside (so every read stays within the sequence's slots), while
 * spec_reject_sample_tree reports such a tree with num_accepted = -1.
 *
 * spec_reject_sample_tree: the walk. At node v (from the root) with children
 * c_1 .. c_m: r = p_v; for i = 1 .. m accept c_i's token x iff u_i < r(x)/q_v(x)
 * (q_v(x) = 0: +inf if r(x) > 0, else 0), u_1 = word 0 of Philox(P, seq, stream 0)
 * and u_i = word 0 of stream i for i >= 2, P = L_b + depth(v) + 1; an accepted
 * child continues the walk; after a rejection r = max(0, r - q_v) normalised (left
 * unchanged if it sums to zero). If every child is rejected, the token at P is drawn
 * from r with u_smp (word 1 of stream 0) and the walk stops; at a leaf, a bonus
 * token is drawn from p_v with u_smp. A chain-shaped tree reproduces
 * spec_reject_sample.
 *
 *  target_logits fp32 [B][N+1][V]  row n: target logits at node n
 *  draft_logits  fp32 [B][N+1][V]  row v: draft logits at node v (the distribution
 *                                  v's children were drawn from; rows of leaves unused)
 *  draft_tokens  int32 [B][N]      token of node n at [n-1] (each < V)
 *  parents       int32 [B][N]
 *  out_tokens    int32 [B][N+1]    the accepted path's tokens, then the drawn token,
 *                                  then -1
 *  num_accepted  int32 [B]         a_b = depth of the last accepted node
 *  accepted_nodes int32 [B][N] or NULL: the accepted nodes in path order, then -1
 *                (their KV rows are the ones to keep at L_b+1 .. L_b+a_b;
 *                spec_commit_tree moves them and commits L' = L + a + 1)
 *  out_probs     fp32 [B][N+1] or NULL: p at the deciding node of each emitted token
 *  accept_probs  fp32 [B][N]   or NULL: min(1, r(x)/q(x)) at each tested node, -1 else
 *
 * Shapes: 1 <= B <= 65535; 1 <= N <= 15; V as for spec_reject_sample. The parents
 * are a device-side precondition (a node with more than 4 children, or a parent
 * index out of range, ends that sequence with num_accepted = -1). Workspace:
 * spec_reject_sample_tree_workspace_size(B, N, V).
 * Runs as spec_reject_sample's chain does: the walk of a sequence reads only the
 * rows of the nodes it visits, its workgroups (of 512 threads, or of 256 when each
 * can have a CU of its own) exchange partial sums while running, with the same
 * residency requirement, bounded waits and error word; the outputs do not depend on
 * the workgroup size.
 * ---------------------------------------------------------------------- */
spec_status spec_verify_attn_tree(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, const int32_t* parents,
                                  void* out, int32_t B, int32_t nodes, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t block_size, int32_t max_blocks, int32_t num_blocks,
                                  int32_t max_seq_len, float sm_scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

spec_status spec_reject_sample_tree_workspace_size(int32_t B, int32_t nodes, int32_t V, size_t* bytes_out);

spec_status spec_reject_sample_tree(const float* target_logits, const float* draft_logits,
                                    const int32_t* draft_tokens, const int32_t* parents, const int64_t* seq_ids,
                                    const int32_t* seq_lens, int32_t B, int32_t nodes, int32_t V,
                                    float temperature, uint64_t seed, int32_t* out_tokens, int32_t* num_accepted,
                                    int32_t* accepted_nodes, float* out_probs, float* accept_probs,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Commit  [ACC] (accepted length per step), [RESP] (KV cache extended in place).
 *
 * seq_lens[b] <- seq_lens[b] + num_accepted[b] + 1, unless that exceeds
 * capacity_tokens: then seq_lens[b] is left unchanged and overflow_flags[b] = 1
 * (overflow_flags[b] = 0 otherwise; overflow_flags may be NULL).
 *
 *  seq_lens int32 [B] in/out;  num_accepted int32 [B] in [0, k];  overflow_flags int32 [B] or NULL
 * Shapes: B >= 1; 0 <= k <= 15; capacity_tokens >= 1.
 * ---------------------------------------------------------------------- */
spec_status spec_commit_lengths(int32_t* seq_lens, const int32_t* num_accepted, int32_t B, int32_t k,
                                int32_t capacity_tokens, int32_t* overflow_flags, void* stream);

/* ------------------------------------------------------------------------
 * Tree commit  [RESP] (GAP 1: a tree of drafts checked in one pass; "Adaptive
 * Server": the KV cache is extended in place). After spec_reject_sample_tree the
 * committed prefix is the root and the accepted path n_1 .. n_a, whose KV rows sit
 * at slots L_b + n_j. For every sequence whose commit fits, slot L_b + j takes the
 * K and V rows (all KV heads) that slot L_b + n_j held before the call, j = 1 .. a
 * (the root stays at L_b), then seq_lens[b] += a + 1 as in spec_commit_lengths. A
 * commit past capacity_tokens moves nothing (overflow_flags[b] = 1); a_b <= 0
 * moves nothing. Slots past L_b + a_b keep their old rows (they lie beyond the new
 * length). Two launches on `stream`: the move, then the length commit.
 *
 *  k_cache / v_cache  bf16 paged caches, as for spec_verify_attn (in/out)
 *  block_table        int32 [B][max_blocks]; slots L_b .. L_b + nodes must map to
 *                     pages that no other sequence's slots L .. L + nodes use
 *  seq_lens           int32 [B] in/out (the lengths the tree step ran at)
 *  accepted_nodes     int32 [B][nodes]: the accepted nodes in path order (as written
 *                     by spec_reject_sample_tree); entry j-1 must lie in [j, nodes]
 *  num_accepted       int32 [B]: a_b (-1, an error of the walk, moves nothing)
 *  overflow_flags     int32 [B] or NULL
 *
 * Shapes: 1 <= B <= 65535; 1 <= nodes <= 15; 1 <= Hkv <= 65535; D in {64, 128};
 * block_size a power of two in [16, 64]. A node index or page id out of range
 * leaves that sequence's cache untouched (a device-side precondition: the length
 * commit still runs).
 * ---------------------------------------------------------------------- */
spec_status spec_commit_tree(void* k_cache, void* v_cache, const int32_t* block_table, int32_t* seq_lens,
                             const int32_t* accepted_nodes, const int32_t* num_accepted, int32_t B,
                             int32_t nodes, int32_t Hkv, int32_t D, int32_t block_size, int32_t max_blocks,
                             int32_t num_blocks, int32_t capacity_tokens, int32_t* overflow_flags, void* stream);

/* ------------------------------------------------------------------------
 * Upstream of the verify step  [ACC] (section 2: the target checks all k drafts in
 * one forward pass, whose output distribution the sampler reads); [RESP] ("Adaptive
 * Server": the KV cache is extended in place). The pages name no position encoding
 * or output head; the readings here are rotate-half RoPE and a plain LM head.
 *
 * spec_rope_append: for the k+1 new rows of every sequence (row 0 the last committed
 * token, rows 1..k the drafts; for a tree, row n is node n), rotate q (in place) and
 * k_new by RoPE at position P = L_b + i (tree: L_b + depth(n)), then write the
 * rotated K and the given V into cache slot L_b + i (tree: L_b + n). For each pair
 * j in [0, D/2) the elements (x_j, x_{j+D/2}) turn by the angle P * theta^(-2j/D);
 * the rotation is computed in float64 and rounded once to bfloat16 (nearest even).
 *
 *  q       bf16 [B][k+1][Hq][D] in/out    k_new, v_new  bf16 [B][k+1][Hkv][D]
 *  k_cache, v_cache, block_table   as for spec_verify_attn (the cache is written)
 *  seq_lens int32 [B] (L_b, before the step)
 *  parents  int32 [B][k] (a tree, positions by depth) or NULL (a chain)
 *  rope_theta > 1 (500000 for the 8B shape, 1000000 for the Qwen shapes)
 * Shapes: 1 <= B <= 65535; 0 <= k <= 15 (k >= 1 with parents); Hq a multiple of
 * Hkv; D in {64, 128}; block_size a power of two in [16, 64]. A row whose slot lies
 * outside the block table, or on a page id out of range, is rotated but not
 * appended (a device-side precondition). One launch.
 *
 * spec_lm_head: logits[r][v] = sum_h hidden[r][h] * weight[v][h], bf16 operands with
 * float32 accumulation (each bf16 product is exact in float32; the sum is within
 * H * 2^-24 / (1 - H * 2^-24) of sum_h |hidden[r][h] weight[v][h]|), no bias. The
 * rows are the verify rows in spec_reject_sample's order, so `logits` is its
 * target_logits as written.
 *
 *  hidden  bf16 [R][H]   weight  bf16 [V][H]   logits  fp32 [R][V] (written)
 * Shapes: 1 <= R <= 65535 * 256; V >= 1; H a positive multiple of 128, at most 2^20;
 * V * H <= 2^40; ceil(V / 256) rounded up to a multiple of 8, times ceil(R / 256), at
 * most 2^23 (the workgroups of the launch).
 * One launch.
 * ---------------------------------------------------------------------- */
spec_status spec_rope_append(void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, const int32_t* parents,
                             int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t D, int32_t block_size,
                             int32_t max_blocks, int32_t num_blocks, double rope_theta, void* stream);

spec_status spec_lm_head(const void* hidden, const void* weight, float* logits, int32_t R, int32_t H, int32_t V,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
