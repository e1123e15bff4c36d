// Paged-KV verify attention for the k+1 verify rows of every sequence (gfx950).
//
// What is computed: "Accelerating RL Post-Training Rollouts via System-Integrated
// Speculative Decoding" (gist.science summary), section 2 "Method", core mechanism:
// the target checks all k drafted tokens in one forward pass. For one layer, row
// i (0..k) of sequence b attends to keys 0 .. L_b+i of its paged cache (causal
// inside the draft), query head h reads KV head h / G.
//
// How (one MI355X):
//  * MFMA tiles. The (k+1) x G query rows of a KV head are packed into 16-row
//    tiles, so both products are dense 16-wide contractions on
//    v_mfma_f32_16x16x32_bf16:
//      S^T = K Q^T    (A = 16 keys x 32 dims from the K page, B = Q^T in registers)
//      O^T += V^T P^T (A = 16 dims x 32 keys from the V page, B = P^T in registers)
//    Computing the transposes puts the softmax statistics of query row r and the
//    accumulators of O^T[., r] on the same lanes (lane % 16 == r), so the online
//    softmax needs only a 4-lane max. Operands are 16-byte global loads straight
//    into MFMA registers: K pages are [block][Hkv][slot][D], V pages are
//    [block][Hkv][D][slot]. Each K/V byte is read once, with streaming
//    (nontemporal) loads; LDS holds only the block-table slice and the
//    cross-wave combine.
//  * Persistent, balanced grid. Contexts are ragged, so a grid of fixed-size KV
//    splits leaves half its workgroups empty and a ragged tail. Instead the work
//    of all (sequence, KV head, 128-key iteration) triples is laid out in one
//    flat order and P = CUs x occupancy workgroups each take an equal contiguous
//    share. A share covers whole (sequence, head) segments, whose output is
//    written directly, plus at most one partial segment at each end, written as
//    fp32 (max, sum, O) partials; a merge launch combines the pieces of a split
//    segment in workgroup order (deterministic).
//  * Inside a piece the four waves take interleaved 32-key blocks; at the end the
//    waves' (max, sum, O) are combined through LDS.
//  * Tree verification ("ReSpec: Towards Optimizing Speculative Decoding in
//    Reinforcement Learning Systems", GAP 1: speculation with a branching factor)
//    replaces the causal mask inside the draft by the tree mask: node n's row sees
//    the committed keys and the slots L + m of its ancestors m (and itself).
//  * Ragged draft lengths (k_b per sequence, rows packed by an offsets array) use
//    the same kernels: a sequence contributes (k_b+1) x G rows, ceil of that / the
//    row-group size per KV head, and L_b + k_b + 1 keys to the flat work order, so
//    short drafts cost no padding work.
//  * Row groups hold 16, 32 or 64 query rows (one, two or four MFMA tiles, chosen
//    from the largest (k+1) x G of the call), so up to 64 rows per KV head read the
//    KV once.
#include "common.hpp"
#include "kernels.hpp"

namespace specverify {
namespace {

constexpr int kAT = 256;
constexpr int kAWaves = kAT / kWave;
constexpr int kBlockKeys = 32;
constexpr int kIterKeys = kAWaves * kBlockKeys;     // keys per workgroup iteration
constexpr int kBtSpan = 4096;                       // keys whose block-table entries sit in LDS at once
constexpr int kBtEntries = kBtSpan / 16;
constexpr int kLdsPrefix = 4096;                    // batch sizes whose work prefix each workgroup builds in LDS
constexpr int kMaxP = 1024;                         // workgroups of the persistent grid (workspace is sized for this)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMergeBatch = 8;                      // split pieces whose loads the merge issues together

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* bt;
    const int32_t* seq_lens;
    const int32_t* cu;   // [B+1] draft-count offsets, or null: every sequence has k drafts
    const int32_t* parents;   // tree: [B][k] parent of node n at [n-1], or null (causal chain)
    uint16_t* out;
    float* part_o;     // [kMaxP][2][rg_rows][D]
    float* part_ml;    // [kMaxP][2][rg_rows][2]
    int32_t* prefix;   // [B+1] exclusive prefix of work (iterations x row groups x KV heads) per sequence
    int B, k, Hq, Hkv, G, rows, row_groups, U, max_blocks, bs_log2, P;   // rows, row_groups, U: at k
    int rg_rows;       // query rows per row group: 16 x the tiles of the launched kernel
    float scale_log2;
};

// Per-sequence shape: k_b drafts, its first query row in the packed [rows][Hq][D]
// layout, its query rows per KV head and its row groups. Without offsets every
// sequence has k drafts and starts at b (k+1).
struct SeqShape {
    int kb, row0, rows, row_groups;
};

__device__ __forceinline__ SeqShape seq_shape(const int32_t* cu, int b, int k, int G, int rg_rows) {
    SeqShape s;
    if (cu) {
        const int c0 = cu[b], c1 = cu[b + 1];
        s.kb = min(max(c1 - c0, 0), k);
        s.row0 = c0 + b;
    } else {
        s.kb = k;
        s.row0 = b * (k + 1);
    }
    s.rows = (s.kb + 1) * G;
    s.row_groups = (s.rows + rg_rows - 1) / rg_rows;
    return s;
}

// The values of this lane and of lane l ^ 16 (pair16) or l ^ 32 (pair32), in either
// order, through v_permlane16_swap / v_permlane32_swap: VALU instructions, where a
// __shfl_xor compiles to an LDS permute and a wait for it. Given the same register
// twice, the 16-lane swap exchanges odd rows of 16 lanes with even ones and the 32-lane
// swap the upper half with the lower, so each lane ends up holding its own value and
// its partner's. Sums and maxima of the pair are then the shuffle's, bit for bit.
__device__ __forceinline__ void pair16(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    const __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&p)[8]) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(p[i]);
    return r;
}

// Zero the bf16 elements of a 16-byte V fragment whose key index is >= limit
// (element i holds key key0 + i).
__device__ __forceinline__ uint4 zero_keys_from(uint4 v, int key0, int limit) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (key0 + 2 * i < limit) ? 0x0000FFFFu : 0u;
        const uint32_t hi = (key0 + 2 * i + 1 < limit) ? 0xFFFF0000u : 0u;
        w[i] &= (lo | hi);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ int iters_of(int seq_len, int k) {
    const int n = seq_len + k + 1;
    return n <= 0 ? 0 : (n + kIterKeys - 1) / kIterKeys;
}

// Flat work of sequence b: 128-key iterations x row groups x KV heads.
__device__ __forceinline__ int work_of(const int32_t* seq_lens, const int32_t* cu, int b, int k, int G, int Hkv,
                                       int rg_rows) {
    const SeqShape sh = seq_shape(cu, b, k, G, rg_rows);
    return iters_of(seq_lens[b], sh.kb) * sh.row_groups * Hkv;
}

// Workgroup w of P owns flat positions [range_start(w), range_start(w+1)).
__device__ __forceinline__ long long range_start(int w, long long total, int P) {
    const long long q = total / P, r = total % P;
    return w * q + (w < r ? w : r);
}

// Workgroups that share the work: all P launched, or fewer when there is little work,
// so that each takes at least kMinIters iterations and a segment is cut into fewer
// pieces for the merge. Both launches derive it from the same total. (7B shape at
// B = 4: 32.0 us per call with 4, 30.2 with 2, 36.2 with 1, where the merge's extra
// pieces outweigh the shorter walks; larger batches fill the grid with any of them.)
constexpr int kMinIters = 2;
__device__ __forceinline__ int sharing_workgroups(long long total, int P) {
    const long long want = total / kMinIters;
    return static_cast<int>(want < 1 ? 1 : (want < P ? want : P));
}

__device__ __forceinline__ int range_owner(long long x, long long total, int P) {
    const long long q = total / P, r = total % P;
    if (x < r * (q + 1)) return static_cast<int>(x / (q + 1));
    return static_cast<int>(r + (x - r * (q + 1)) / q);
}

// Exclusive prefix of work per sequence, built by one 256-thread workgroup into
// `dst` (LDS or global); dst[B] is the total.
__device__ void build_prefix(const int32_t* seq_lens, const int32_t* cu, int B, int k, int G, int Hkv, int rg_rows,
                             int32_t* dst, int* s_wave) {
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    int carry = 0;
    for (int base = 0; base < B; base += kAT) {
        const int b = base + tid;
        int v = (b < B) ? work_of(seq_lens, cu, b, k, G, Hkv, rg_rows) : 0;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int y = __shfl_up(v, o, kWave);
            if (lane >= o) v += y;
        }
        if (lane == kWave - 1) s_wave[wave] = v;
        __syncthreads();
        int before = carry;
        for (int i = 0; i < wave; ++i) before += s_wave[i];
        if (b < B) dst[b + 1] = before + v;
        int tot = carry;
        for (int i = 0; i < kAWaves; ++i) tot += s_wave[i];
        __syncthreads();
        carry = tot;
    }
    if (tid == 0) dst[0] = 0;
    __syncthreads();
}

__global__ __launch_bounds__(kAT) void attn_plan_kernel(const int32_t* seq_lens, const int32_t* cu, int B, int k,
                                                        int G, int Hkv, int rg_rows, int32_t* prefix) {
    __shared__ int s_wave[kAWaves];
    build_prefix(seq_lens, cu, B, k, G, Hkv, rg_rows, prefix, s_wave);
}

template <int D, int NT, bool kTree>
__global__ __launch_bounds__(kAT) void attn_streamk_kernel(AttnArgs a) {
    constexpr int DS = D / 32;   // k-steps of S^T = K Q^T
    constexpr int DJ = D / 16;   // 16-dim blocks of O^T
    constexpr int kRG = 16 * NT; // query rows per row group
    __shared__ int s_bt[kBtEntries];
    __shared__ int32_t s_prefix[kLdsPrefix + 1];
    __shared__ int s_wave[kAWaves];
    __shared__ float s_m[kAWaves][NT][16];
    __shared__ float s_l[kAWaves][NT][16];
    __shared__ float s_o[kAWaves][16][D + 4];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane & 15, lg = lane >> 4;
    const int bs = 1 << a.bs_log2;
    const int w = blockIdx.x;

    const int32_t* prefix = a.prefix;
    if (a.B <= kLdsPrefix) {
        build_prefix(a.seq_lens, a.cu, a.B, a.k, a.G, a.Hkv, kRG, s_prefix, s_wave);
        if (w == 0)
            for (int i = tid; i <= a.B; i += kAT) a.prefix[i] = s_prefix[i];
        prefix = s_prefix;
    }
    const long long total = prefix[a.B];
    const int P = sharing_workgroups(total, a.P);
    if (w >= P) return;
    const long long r0 = range_start(w, total, P), r1 = range_start(w + 1, total, P);
    if (r0 >= r1) return;

    // segment (b, u) starts at prefix[b] + u * iters_b; find the last b whose start is <= r0
    // (sequences without work have equal prefixes and are passed over)
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= r0) lo = mid; else hi = mid - 1;
    }
    int b = lo;
    SeqShape sh = seq_shape(a.cu, b, a.k, a.G, kRG);
    int U_b = sh.row_groups * a.Hkv;
    int iters_b = (prefix[b + 1] - prefix[b]) / U_b;
    const long long off = r0 - prefix[b];
    int u = static_cast<int>(off / iters_b);
    int it0 = static_cast<int>(off % iters_b);

    const size_t head_stride = size_t(D) << a.bs_log2;   // elements per (block, KV head)
    long long cur = r0;
    bool first_piece = true;
    while (cur < r1) {
        const int it1 = static_cast<int>(min(static_cast<long long>(iters_b), it0 + (r1 - cur)));
        const int g = u / sh.row_groups, rg = u % sh.row_groups;
        const int L = a.seq_lens[b];
        const int N = L + sh.kb + 1;
        const int c0 = it0 * kIterKeys;
        const int c1 = min(N, it1 * kIterKeys);

        // Tree: ancestor-or-self masks of the nodes (bit m: slot L + m is visible),
        // built from the parents with uniform loads; the chain sees every slot <= L + i.
        unsigned anc_all[16];
        if (kTree) {
            anc_all[0] = 1u;
#pragma unroll
            for (int n = 1; n < 16; ++n) {
                unsigned m = 1u << n;
                if (n <= sh.kb) {
                    int par = a.parents[size_t(b) * a.k + n - 1];
                    par = par < 0 ? 0 : (par >= n ? n - 1 : par);   // a broken tree stays in range
#pragma unroll
                    for (int j = 0; j < n; ++j)
                        if (j == par) m |= anc_all[j];
                }
                anc_all[n] = m;
            }
        }

        // Q^T operands and the last visible key of this lane's query row in each tile.
        bf16x8 qop[NT][DS];
        int lim[NT];
        unsigned anc[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            const int r = rg * kRG + n * 16 + l16;
            if (r < sh.rows) {
                const int i = r / a.G;
                const int h = g * a.G + r % a.G;
                const uint16_t* qp = a.q + ((size_t(sh.row0) + i) * a.Hq + h) * D + 8 * lg;
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) qop[n][ds] = as_bf16x8(load16(qp + 32 * ds));
                lim[n] = L + i;
                anc[n] = ~0u;
                if (kTree) {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (j == i) anc[n] = anc_all[j];
                }
            } else {
#pragma unroll
                for (int ds = 0; ds < DS; ++ds) qop[n][ds] = as_bf16x8(make_uint4(0, 0, 0, 0));
                lim[n] = N - 1;   // padding rows: harmless finite result, never stored
                anc[n] = ~0u;
            }
        }

        float m_run[NT], l_run[NT];
        f32x4 o[NT][DJ];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            m_run[n] = -INFINITY;
            l_run[n] = 0.0f;
#pragma unroll
            for (int j = 0; j < DJ; ++j) o[n][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }

        for (int s0 = c0; s0 < c1; s0 += kBtSpan) {
            // s0 and every sub-range end below c1 are multiples of 128: no 32-key block straddles s1
            const int s1 = min(c1, s0 + kBtSpan);
            const int p0 = s0 >> a.bs_log2;
            const int np = ((s1 - 1) >> a.bs_log2) - p0 + 1;
            __syncthreads();
            for (int i = tid; i < np; i += kAT) s_bt[i] = a.bt[size_t(b) * a.max_blocks + p0 + i];
            __syncthreads();

            // K: tile t, lane row l16 holds key t0 + 8*(l16/4) + 4t + l16%4, dims 32*ds + 8*lg .. +7.
            // V: lane holds keys t0 + 8*lg .. +7 of dims 16j + l16. Addresses are clamped into
            // the sub-range so the loads are unconditional; keys >= s1 are masked (scores) or
            // zeroed (values) when the block is consumed.
            for (int t0 = s0 + wave * kBlockKeys; t0 < s1; t0 += kIterKeys) {
                uint4 kr[2][DS], vr[DJ];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int key = min(t0 + 8 * (l16 >> 2) + 4 * t + (l16 & 3), s1 - 1);
                    const int pg = s_bt[(key >> a.bs_log2) - p0];
                    const uint16_t* kp = a.kc + (size_t(pg) * a.Hkv + g) * head_stride +
                                         size_t(key & (bs - 1)) * D + 8 * lg;
#pragma unroll
                    for (int ds = 0; ds < DS; ++ds) kr[t][ds] = load16_nt(kp + 32 * ds);
                }
                {
                    const int vkey0 = min(t0 + 8 * lg, (s1 - 1) & ~7);
                    const int pg = s_bt[(vkey0 >> a.bs_log2) - p0];
                    const uint16_t* vp = a.vc + (size_t(pg) * a.Hkv + g) * head_stride + (vkey0 & (bs - 1));
                    if (a.bs_log2 >= 6) {
                        // 64-key pages: a V page row (one dimension) is a whole 128-byte line,
                        // half of which is this block's; the other half belongs to the next
                        // block, which another wave of the workgroup reads at the same time.
                        // Cached loads let that read find the line in the L2 (streaming loads
                        // fetched every such line twice: 1.26x the algorithmic bytes at 262K).
#pragma unroll
                        for (int j = 0; j < DJ; ++j) vr[j] = load16(vp + size_t(16 * j + l16) * bs);
                    } else {
#pragma unroll
                        for (int j = 0; j < DJ; ++j) vr[j] = load16_nt(vp + size_t(16 * j + l16) * bs);
                    }
                }
                if (t0 + kBlockKeys > s1) {
                    // tail block: values of keys >= s1 (past the sequence, or another piece's) become 0
#pragma unroll
                    for (int j = 0; j < DJ; ++j) vr[j] = zero_keys_from(vr[j], t0 + 8 * lg, s1);
                }
                const bool full = (t0 + kBlockKeys <= s1) && (t0 + kBlockKeys - 1 <= L);
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    f32x4 st[2];
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                        for (int ds = 0; ds < DS; ++ds)
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[t][ds]), qop[n][ds], acc,
                                                                         0, 0, 0);
                        st[t] = acc;
                    }
                    // lane's scores: row l16 of tile n, keys t0 + 8*lg + i (i = 4t + e)
                    float sv[8];
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e) sv[4 * t + e] = st[t][e] * a.scale_log2;
                    if (!full) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            const int key = t0 + 8 * lg + i;
                            bool hide;
                            if constexpr (kTree) {
                                // draft slot L + m is visible iff bit m of the ancestor mask is set; the
                                // bits stop at the node itself, which covers the causal limit, and every
                                // key < s1 lies below L + 16. Branch-free, with an in-range shift.
                                const unsigned rel = static_cast<unsigned>(key - L);
                                hide = (key >= s1) | ((rel < 32u) & (((anc[n] >> (rel & 31u)) & 1u) == 0u));
                            } else {
                                hide = key >= s1 || key > lim[n];
                            }
                            if (hide) sv[i] = -INFINITY;
                        }
                    }
                    float bmax = sv[0];
#pragma unroll
                    for (int i = 1; i < 8; ++i) bmax = fmaxf(bmax, sv[i]);
                    {
                        float x0, x1;
                        pair16(bmax, x0, x1);
                        bmax = fmaxf(x0, x1);
                        pair32(bmax, x0, x1);
                        bmax = fmaxf(x0, x1);
                    }
                    const float m_new = fmaxf(m_run[n], bmax);
                    const float m_ref = (m_new == -INFINITY) ? 0.0f : m_new;
                    const float alpha = __builtin_amdgcn_exp2f(m_run[n] - m_ref);
                    float p[8];
                    float psum = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        p[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref);
                        psum += p[i];
                    }
                    l_run[n] = l_run[n] * alpha + psum;
                    const bool moved = __any(m_new != m_run[n]);
                    m_run[n] = m_new;
                    const bf16x8 pop = pack_bf16x8(p);
                    // alpha is exactly 1 in every row whose maximum did not move: once the
                    // running maxima settle, most blocks skip the rescale (a wave-uniform branch)
                    if (moved) {
#pragma unroll
                        for (int j = 0; j < DJ; ++j) o[n][j] *= alpha;
                    }
#pragma unroll
                    for (int j = 0; j < DJ; ++j)
                        o[n][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[j]), pop, o[n][j], 0, 0, 0);
                }
            }
        }

        // ---- combine the four waves: per row, M = max over waves, weights 2^(m_w - M).
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float x0, x1;
            pair16(l_run[n], x0, x1);
            float lt = x0 + x1;
            pair32(lt, x0, x1);
            lt = x0 + x1;
            if (lg == 0) {
                s_m[wave][n][l16] = m_run[n];
                s_l[wave][n][l16] = lt;
            }
        }
        __syncthreads();
        const bool whole = (it0 == 0) && (it1 == iters_b);
        const size_t slot = size_t(w) * 2 + (first_piece ? 0 : 1);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float M = s_m[0][n][l16];
#pragma unroll
            for (int v = 1; v < kAWaves; ++v) M = fmaxf(M, s_m[v][n][l16]);
            const float M_ref = (M == -INFINITY) ? 0.0f : M;
            const float wself = __builtin_amdgcn_exp2f(m_run[n] - M_ref);
#pragma unroll
            for (int j = 0; j < DJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) s_o[wave][l16][16 * j + 4 * lg + e] = o[n][j][e] * wself;
            __syncthreads();
            {   // 256 threads: row r = tid / 16, dims (tid % 16) * (D/16) .. +D/16
                const int r = tid / 16;
                const int d0 = (tid % 16) * (D / 16);
                float Mr = s_m[0][n][r];
#pragma unroll
                for (int v = 1; v < kAWaves; ++v) Mr = fmaxf(Mr, s_m[v][n][r]);
                const float Mr_ref = (Mr == -INFINITY) ? 0.0f : Mr;
                float lsum = 0.0f;
#pragma unroll
                for (int v = 0; v < kAWaves; ++v) lsum += s_l[v][n][r] * __builtin_amdgcn_exp2f(s_m[v][n][r] - Mr_ref);
                float acc[D / 16];
#pragma unroll
                for (int dd = 0; dd < D / 16; ++dd) {
                    float x = 0.0f;
#pragma unroll
                    for (int v = 0; v < kAWaves; ++v) x += s_o[v][r][d0 + dd];
                    acc[dd] = x;
                }
                const int row = rg * kRG + n * 16 + r;
                if (whole) {
                    if (row < sh.rows) {
                        const int i = row / a.G;
                        const int h = g * a.G + row % a.G;
                        uint16_t* op = a.out + ((size_t(sh.row0) + i) * a.Hq + h) * D + d0;
                        const float inv = 1.0f / lsum;
#pragma unroll
                        for (int dd = 0; dd < D / 16; ++dd) op[dd] = f32_to_bf16_bits(acc[dd] * inv);
                    }
                } else {
                    const size_t prow = slot * kRG + n * 16 + r;
                    float* po = a.part_o + prow * D + d0;
#pragma unroll
                    for (int dd = 0; dd < D / 16; ++dd) po[dd] = acc[dd];
                    if ((tid % 16) == 0) {
                        a.part_ml[prow * 2 + 0] = Mr;
                        a.part_ml[prow * 2 + 1] = lsum;
                    }
                }
            }
            __syncthreads();
        }

        cur += it1 - it0;
        first_piece = false;
        it0 = 0;
        if (++u == U_b) {
            u = 0;
            do {   // the next sequence with work (its share starts where this one ended)
                if (++b >= a.B) break;
            } while (prefix[b + 1] == prefix[b]);
            if (b >= a.B) break;
            sh = seq_shape(a.cu, b, a.k, a.G, kRG);
            U_b = sh.row_groups * a.Hkv;
            iters_b = (prefix[b + 1] - prefix[b]) / U_b;
        }
    }
}

// One row (dims d0 .. d0 + D/16) of a split segment: M = max over the pieces w0 .. w1,
// then their sums and outputs weighted by 2^(m - M), folded in workgroup order.
// The loads of KB pieces (max, sum and output row) are issued together, in one round
// trip: addresses clamped to the last piece, weights past it 0. The running maximum
// moves only between batches, so with at most KB pieces the weights are 2^(m_j - M) for
// the pieces' own maximum M, the same bits as a separate pass for M would give; with
// more, the sums so far are rescaled when a batch raises it. Returns 1 / sum.
template <int D, int KB, typename PR>
__device__ __forceinline__ float merge_row(const AttnArgs& a, PR&& prow_of, int w0, int w1, int n, int r, int d0,
                                           float (&acc)[D / 16]) {
    float M = -INFINITY, lsum = 0.0f;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) acc[dd] = 0.0f;
    for (int wb = w0; wb <= w1; wb += KB) {
        float ms[KB], ls[KB], po[KB][D / 16];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            const size_t prow = prow_of(min(wb + j, w1), n, r);
            ms[j] = a.part_ml[prow * 2];
            ls[j] = a.part_ml[prow * 2 + 1];
#pragma unroll
            for (int dd = 0; dd < D / 16; ++dd) po[j][dd] = a.part_o[prow * D + d0 + dd];
        }
        float bm = M;
#pragma unroll
        for (int j = 0; j < KB; ++j) bm = fmaxf(bm, (wb + j <= w1) ? ms[j] : -INFINITY);
        // scale of the sums so far: 0 before the first finite maximum (they are 0), else
        // 2^(M - bm), exactly 1 when the batch does not raise M
        const float sc = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - bm);
        lsum *= sc;
#pragma unroll
        for (int dd = 0; dd < D / 16; ++dd) acc[dd] *= sc;
        M = bm;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            // branch-free, so that all of the batch's loads stay in flight together
            const float wt = (wb + j > w1 || ms[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms[j] - M);
            lsum += wt * ls[j];
#pragma unroll
            for (int dd = 0; dd < D / 16; ++dd) acc[dd] += wt * po[j][dd];
        }
    }
    return 1.0f / lsum;
}

// Combine the pieces of every (sequence, KV head, row group) segment that was
// split between workgroups, in workgroup order. One workgroup per 16-row tile of a
// segment (blockIdx.z), so that the tiles of a row group merge side by side rather
// than one after another: a merge is a chain of dependent round trips, one per
// batch of pieces.
template <int D>
__global__ __launch_bounds__(kAT) void attn_merge_kernel(AttnArgs a, int tiles) {
    const int u = blockIdx.x, b = blockIdx.y, n = blockIdx.z;
    const int rgr = 16 * tiles;
    const SeqShape sh = seq_shape(a.cu, b, a.k, a.G, rgr);
    const int U_b = sh.row_groups * a.Hkv;
    if (u >= U_b) return;
    const long long total = a.prefix[a.B];
    const int iters_b = (a.prefix[b + 1] - a.prefix[b]) / U_b;
    if (iters_b <= 0) return;
    const long long S = static_cast<long long>(a.prefix[b]) + static_cast<long long>(u) * iters_b;
    const long long E = S + iters_b;
    const int P = sharing_workgroups(total, a.P);
    const int w0 = range_owner(S, total, P), w1 = range_owner(E - 1, total, P);
    if (w0 == w1) return;                      // one workgroup wrote the output directly
    const int first_slot = (S == range_start(w0, total, P)) ? 0 : 1;
    const int g = u / sh.row_groups, rg = u % sh.row_groups;
    const int tid = threadIdx.x;
    // piece ww's partial row for tile n: workgroup w0's piece sits in slot first_slot,
    // every later one in slot 0 of its workgroup
    auto prow_of = [&](int ww, int n, int r) {
        return (size_t(ww) * 2 + (ww == w0 ? first_slot : 0)) * rgr + n * 16 + r;
    };
    {
        const int r = tid / 16;
        const int d0 = (tid % 16) * (D / 16);
        const int row = rg * rgr + n * 16 + r;
        if (row >= sh.rows) return;
        float acc[D / 16];
        const float inv = (w1 - w0 < 2) ? merge_row<D, 2>(a, prow_of, w0, w1, n, r, d0, acc)
                                        : merge_row<D, kMergeBatch>(a, prow_of, w0, w1, n, r, d0, acc);
        const int i = row / a.G;
        const int h = g * a.G + row % a.G;
        uint16_t* op = a.out + ((size_t(sh.row0) + i) * a.Hq + h) * D + d0;
#pragma unroll
        for (int dd = 0; dd < D / 16; ++dd) op[dd] = f32_to_bf16_bits(acc[dd] * inv);
    }
}

// Persistent-grid size per (device, kernel instantiation): CUs x resident workgroups.
DeviceMemo g_grid_memo[16];

template <int D, int NT, bool kTree>
int persistent_grid(int slot) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    DeviceMemo& memo = g_grid_memo[slot];
    if (memo.get(dev) > 0) return memo.get(dev);
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_streamk_kernel<D, NT, kTree>, kAT, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    int P = cus * (per_cu > 0 ? per_cu : 1);
    if (P > kMaxP) P = kMaxP;
    if (P < 1) P = 1;
    memo.put(dev, P);
    return P;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

AttnGeometry attn_geometry(int B, int k, int Hq, int Hkv, int D, int max_seq_len) {
    AttnGeometry g;
    const int G = Hq / Hkv;
    g.rows = (k + 1) * G;
    g.tiles = g.rows <= 16 ? 1 : (g.rows <= 32 ? 2 : 4);
    g.row_groups = (g.rows + 16 * g.tiles - 1) / (16 * g.tiles);
    g.chunk = kIterKeys;
    g.splits = (max_seq_len + kIterKeys - 1) / kIterKeys;
    const size_t prefix_bytes = align256(sizeof(int32_t) * (size_t(B) + 1));
    const size_t part = size_t(kMaxP) * 2 * 16 * g.tiles;
    g.workspace = prefix_bytes + part * size_t(D) * sizeof(float) + part * 2 * sizeof(float);
    return g;
}

hipError_t launch_attn(const AttnLaunch& p, const AttnGeometry& geo, hipStream_t stream) {
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.kc = static_cast<const uint16_t*>(p.k_cache);
    a.vc = static_cast<const uint16_t*>(p.v_cache);
    a.bt = p.block_table;
    a.seq_lens = p.seq_lens;
    a.cu = p.cu_drafts;
    a.parents = p.parents;
    a.out = static_cast<uint16_t*>(p.out);
    char* ws = static_cast<char*>(p.workspace);
    a.prefix = reinterpret_cast<int32_t*>(ws);
    a.part_o = reinterpret_cast<float*>(ws + align256(sizeof(int32_t) * (size_t(p.B) + 1)));
    a.part_ml = a.part_o + size_t(kMaxP) * 2 * 16 * geo.tiles * p.D;
    a.B = p.B;
    a.k = p.k;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.G = p.Hq / p.Hkv;
    a.rows = geo.rows;
    a.row_groups = geo.row_groups;
    a.rg_rows = 16 * geo.tiles;
    a.U = p.Hkv * geo.row_groups;
    a.max_blocks = p.max_blocks;
    int lg = 0;
    while ((1 << lg) < p.block_size) ++lg;
    a.bs_log2 = lg;
    a.scale_log2 = p.sm_scale * kLog2e;

    if (p.B > kLdsPrefix) {
        hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kAT), 0, stream, p.seq_lens, p.cu_drafts, p.B, p.k, a.G,
                           p.Hkv, a.rg_rows, a.prefix);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 block(kAT);
    const bool tree = p.parents != nullptr;
    const int slot = (p.D == 128 ? 0 : 6) + (geo.tiles == 1 ? 0 : (geo.tiles == 2 ? 2 : 4)) + (tree ? 1 : 0);
#define SPEC_ATTN_LAUNCH(DD, NN, TT)                                                               \
    do {                                                                                           \
        a.P = persistent_grid<DD, NN, TT>(slot);                                                   \
        hipLaunchKernelGGL((attn_streamk_kernel<DD, NN, TT>), dim3(a.P), block, 0, stream, a);     \
    } while (0)
    if (p.D == 128) {
        if (geo.tiles == 1) { if (tree) SPEC_ATTN_LAUNCH(128, 1, true); else SPEC_ATTN_LAUNCH(128, 1, false); }
        else if (geo.tiles == 2) { if (tree) SPEC_ATTN_LAUNCH(128, 2, true); else SPEC_ATTN_LAUNCH(128, 2, false); }
        else { if (tree) SPEC_ATTN_LAUNCH(128, 4, true); else SPEC_ATTN_LAUNCH(128, 4, false); }
    } else {
        if (geo.tiles == 1) { if (tree) SPEC_ATTN_LAUNCH(64, 1, true); else SPEC_ATTN_LAUNCH(64, 1, false); }
        else if (geo.tiles == 2) { if (tree) SPEC_ATTN_LAUNCH(64, 2, true); else SPEC_ATTN_LAUNCH(64, 2, false); }
        else { if (tree) SPEC_ATTN_LAUNCH(64, 4, true); else SPEC_ATTN_LAUNCH(64, 4, false); }
    }
#undef SPEC_ATTN_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid(a.U, p.B, geo.tiles);
    if (p.D == 128) hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, block, 0, stream, a, geo.tiles);
    else hipLaunchKernelGGL(attn_merge_kernel<64>, mgrid, block, 0, stream, a, geo.tiles);
    return hipGetLastError();
}

}  // namespace specverify
