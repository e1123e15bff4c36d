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

// ---------------------------------------------------------------- tree commit
//
// "ReSpec: Towards Optimizing Speculative Decoding in Reinforcement Learning
// Systems" (talk notes), GAP 1 and "Adaptive Server": a tree of drafts is checked
// in one pass and the KV cache grows in place. The committed prefix after a tree
// step is the root and the accepted path n_1 .. n_a, so slot L+j must hold the row
// that node n_j's slot L+n_j held; the length commit follows as for the chain.

constexpr int kMoveThreads = 256;
constexpr int kMaxNodes = 15;

struct TreeMoveArgs {
    uint16_t* kc;   // [pages][Hkv][bs][D]
    uint16_t* vc;   // [pages][Hkv][D][bs]
    const int32_t* bt;
    const int32_t* seq_lens;
    const int32_t* nodes;   // [B][N] accepted nodes in path order
    const int32_t* num_accepted;
    int N, Hkv, bs_log2, max_blocks, num_blocks, capacity;
};

// One workgroup per (KV head, sequence). Every row of the path is read into LDS
// before any is written: slot L+j can be both the destination of step j and the
// source of an earlier step (n_i = j for i < j).
template <int D>
__global__ __launch_bounds__(kMoveThreads) void tree_move_kernel(TreeMoveArgs a) {
    __shared__ uint16_t s_k[kMaxNodes][D];
    __shared__ uint16_t s_v[kMaxNodes][D];
    __shared__ size_t s_src[kMaxNodes], s_dst[kMaxNodes];   // element offset of (page, head) + slot
    __shared__ int s_so[kMaxNodes], s_do[kMaxNodes];          // slot offsets inside the page
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = a.seq_lens[b];
    const int acc = a.num_accepted[b];
    if (acc <= 0 || acc > a.N || L < 0) return;                              // nothing accepted, or an error
    if (static_cast<long long>(L) + acc + 1 > a.capacity) return;            // the commit is refused
    const int bs = 1 << a.bs_log2;
    const size_t head_elems = size_t(D) << a.bs_log2;
    int bad = 0;
    if (tid < acc) {
        const int j = tid + 1;
        const int node = a.nodes[size_t(b) * a.N + tid];
        bad = node < j || node > a.N;   // the j-th node of a path has index >= j
        if (!bad) {
            const long long src = static_cast<long long>(L) + node, dst = static_cast<long long>(L) + j;
            const long long ps = src >> a.bs_log2, pd = dst >> a.bs_log2;
            bad = ps >= a.max_blocks || pd >= a.max_blocks;
            if (!bad) {
                const int pgs = a.bt[size_t(b) * a.max_blocks + ps];
                const int pgd = a.bt[size_t(b) * a.max_blocks + pd];
                bad = pgs < 0 || pgs >= a.num_blocks || pgd < 0 || pgd >= a.num_blocks;
                s_src[tid] = (size_t(pgs) * a.Hkv + g) * head_elems;
                s_dst[tid] = (size_t(pgd) * a.Hkv + g) * head_elems;
                s_so[tid] = static_cast<int>(src & (bs - 1));
                s_do[tid] = static_cast<int>(dst & (bs - 1));
            }
        }
    }
    if (__syncthreads_or(bad)) return;   // an out-of-range node or page: this sequence is left as it was
    for (int e = tid; e < acc * D; e += kMoveThreads) {
        const int j = e / D, d = e % D;
        s_k[j][d] = a.kc[s_src[j] + size_t(s_so[j]) * D + d];
        s_v[j][d] = a.vc[s_src[j] + (size_t(d) << a.bs_log2) + s_so[j]];
    }
    __syncthreads();
    for (int e = tid; e < acc * D; e += kMoveThreads) {
        const int j = e / D, d = e % D;
        a.kc[s_dst[j] + size_t(s_do[j]) * D + d] = s_k[j][d];
        a.vc[s_dst[j] + (size_t(d) << a.bs_log2) + s_do[j]] = s_v[j][d];
    }
}

}  // namespace

hipError_t launch_tree_commit(const TreeCommitLaunch& p, hipStream_t stream) {
    TreeMoveArgs a;
    a.kc = static_cast<uint16_t*>(p.k_cache);
    a.vc = static_cast<uint16_t*>(p.v_cache);
    a.bt = p.block_table;
    a.seq_lens = p.seq_lens;
    a.nodes = p.accepted_nodes;
    a.num_accepted = p.num_accepted;
    a.N = p.nodes;
    a.Hkv = p.Hkv;
    a.bs_log2 = __builtin_ctz(static_cast<unsigned>(p.block_size));
    a.max_blocks = p.max_blocks;
    a.num_blocks = p.num_blocks;
    a.capacity = p.capacity;
    const dim3 grid(p.Hkv, p.B);
    if (p.D == 128)
        hipLaunchKernelGGL(tree_move_kernel<128>, grid, dim3(kMoveThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(tree_move_kernel<64>, grid, dim3(kMoveThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_commit(p.seq_lens, p.num_accepted, p.B, p.capacity, p.overflow_flags, stream);
}

hipError_t launch_commit(int32_t* seq_lens, const int32_t* num_accepted, int B, int capacity,
                         int32_t* overflow_flags, hipStream_t stream) {
    hipLaunchKernelGGL(commit_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, seq_lens, num_accepted, B,
                       capacity, overflow_flags);
    return hipGetLastError();
}

}  // namespace specverify
