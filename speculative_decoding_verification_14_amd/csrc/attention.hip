// Paged-KV verify attention for the k+1 verify rows of every sequence (gfx950).
//
// What is computed: "Accelerating RL Post-Training Rollouts via System-Integrated
// Speculative Decoding" (gist.science summary), section 2 "Method", core mechanism:
// the target checks all k drafted tokens in one forward pass. For one layer, row
// i (0..k) of sequence b attends to keys 0 .. L_b+i of its paged cache (causal
// inside the draft), query head h reads KV head h / G.
//
// How (one MI355X):
//  * One workgroup (4 waves) per (sequence, KV head, row group, KV split). The
//    (k+1) x G query rows of a KV head are packed into 16-row tiles, so both
//    products are dense 16-wide contractions and run on v_mfma_f32_16x16x32_bf16:
//      S^T = K Q^T   (A = 16 keys x 32 dims from the K page, B = Q^T from registers)
//      O^T += V^T P^T (A = 16 dims x 32 keys from the V page, B = P^T from registers)
//    Computing the transposes puts the softmax statistics of query row r and the
//    accumulators of O^T[., r] on the same lanes (lane % 16 == r), so the online
//    softmax needs no cross-lane traffic beyond a 4-lane max.
//  * Every operand fetch is a 16-byte global load straight into MFMA registers:
//    K pages are [block][Hkv][slot][D] (8 consecutive dims of a key), V pages are
//    [block][Hkv][D][slot] (8 consecutive keys of a dim). Each K/V byte of a
//    sequence is read exactly once; there is no reuse for LDS to exploit, so LDS
//    holds only the block-table slice of the chunk and the cross-wave combine.
//  * Waves take interleaved 32-key blocks of the workgroup's chunk; at the end the
//    four waves' (max, sum, O) are combined through LDS. A sequence that fits one
//    chunk writes its bf16 output directly; longer ones write fp32 partials that
//    the merge kernel combines in split order (deterministic).
#include "common.hpp"
#include "kernels.hpp"

namespace specverify {
namespace {

constexpr int kAT = 256;
constexpr int kAWaves = kAT / kWave;
constexpr int kBlockKeys = 32;
constexpr int kMaxChunk = 16384;
constexpr int kMaxChunkPages = kMaxChunk / 16;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* bt;
    const int32_t* seq_lens;
    uint16_t* out;
    float* part_o;     // [B][Hkv][RG][splits][32 rows][D]
    float* part_ml;    // [B][Hkv][RG][splits][32 rows][2]
    int k, Hq, Hkv, G, rows, row_groups, max_blocks, bs_log2, chunk, splits;
    float scale_log2;
};

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

template <int D, int NT>
__global__ __launch_bounds__(kAT) void attn_partial_kernel(AttnArgs a) {
    constexpr int DS = D / 32;   // k-steps of S^T = K Q^T
    constexpr int DJ = D / 16;   // 16-dim blocks of O^T
    __shared__ int s_bt[kMaxChunkPages];
    __shared__ float s_m[kAWaves][NT][16];
    __shared__ float s_l[kAWaves][NT][16];
    __shared__ float s_o[kAWaves][16][D + 4];

    const int split = blockIdx.x;
    const int g = blockIdx.y / a.row_groups, rg = blockIdx.y % a.row_groups;
    const int b = blockIdx.z;
    const int L = a.seq_lens[b];
    const int N = L + a.k + 1;
    const int c0 = split * a.chunk;
    if (c0 >= N) return;
    const int c1 = min(N, c0 + a.chunk);
    // clamped to the grid: lengths past max_seq_len (a broken precondition) lose keys, never fault
    const int n_splits_b = min(a.splits, (N + a.chunk - 1) / a.chunk);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int l16 = lane & 15, lg = lane >> 4;
    const int bs = 1 << a.bs_log2;

    const int p0 = c0 >> a.bs_log2;
    const int np = ((c1 - 1) >> a.bs_log2) - p0 + 1;
    for (int i = tid; i < np; i += kAT) s_bt[i] = a.bt[size_t(b) * a.max_blocks + p0 + i];

    // Q^T operands and the last visible key of this lane's query row in each tile.
    bf16x8 qop[NT][DS];
    int lim[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int r = rg * 32 + n * 16 + l16;
        if (r < a.rows) {
            const int i = r / a.G;
            const int h = g * a.G + r % a.G;
            const uint16_t* qp = a.q + ((size_t(b) * (a.k + 1) + i) * a.Hq + h) * D + 8 * lg;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) qop[n][ds] = as_bf16x8(load16(qp + 32 * ds));
            lim[n] = L + i;
        } else {
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) qop[n][ds] = as_bf16x8(make_uint4(0, 0, 0, 0));
            lim[n] = N - 1;   // padding rows: harmless finite result, never stored
        }
    }
    __syncthreads();

    float m_run[NT], l_run[NT];
    f32x4 o[NT][DJ];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        m_run[n] = -INFINITY;
        l_run[n] = 0.0f;
#pragma unroll
        for (int j = 0; j < DJ; ++j) o[n][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const size_t head_stride = size_t(D) << a.bs_log2;   // elements per (block, KV head)

    // Fragments of one 32-key block. K: tile t, lane row l16 holds key
    // t0 + 8*(l16/4) + 4t + l16%4, dims 32*ds + 8*lg .. +7. V: lane holds keys
    // t0 + 8*lg .. +7 of dims 16j + l16. Addresses are clamped into the chunk so
    // the loads are unconditional and can all be in flight; keys >= c1 are masked
    // (scores) or zeroed (values) when the block is consumed.
    auto load_block = [&](int t0, uint4 (&kr)[2][DS], uint4 (&vr)[DJ]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int key = min(t0 + 8 * (l16 >> 2) + 4 * t + (l16 & 3), c1 - 1);
            const int pg = s_bt[(key >> a.bs_log2) - p0];
            const uint16_t* kp = a.kc + (size_t(pg) * a.Hkv + g) * head_stride + size_t(key & (bs - 1)) * D + 8 * lg;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) kr[t][ds] = load16(kp + 32 * ds);
        }
        const int vkey0 = min(t0 + 8 * lg, (c1 - 1) & ~7);
        const int pg = s_bt[(vkey0 >> a.bs_log2) - p0];
        const uint16_t* vp = a.vc + (size_t(pg) * a.Hkv + g) * head_stride + (vkey0 & (bs - 1));
#pragma unroll
        for (int j = 0; j < DJ; ++j) vr[j] = load16(vp + size_t(16 * j + l16) * bs);
    };

    auto compute_block = [&](int t0, uint4 (&kr)[2][DS], uint4 (&vr)[DJ]) {
        const bool full = (t0 + kBlockKeys <= c1) && (t0 + kBlockKeys - 1 <= L);
        if (t0 + kBlockKeys > c1) {
            // tail block: values of keys >= c1 (other splits' keys or garbage) become 0
#pragma unroll
            for (int j = 0; j < DJ; ++j) vr[j] = zero_keys_from(vr[j], t0 + 8 * lg, c1);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            f32x4 st[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int ds = 0; ds < DS; ++ds)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[t][ds]), qop[n][ds], acc, 0, 0, 0);
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
                    if (key >= c1 || key > lim[n]) sv[i] = -INFINITY;
                }
            }
            float bmax = sv[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) bmax = fmaxf(bmax, sv[i]);
            bmax = fmaxf(bmax, __shfl_xor(bmax, 16, kWave));
            bmax = fmaxf(bmax, __shfl_xor(bmax, 32, kWave));
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
            m_run[n] = m_new;
            const bf16x8 pop = pack_bf16x8(p);
#pragma unroll
            for (int j = 0; j < DJ; ++j) {
                o[n][j] *= alpha;
                o[n][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vr[j]), pop, o[n][j], 0, 0, 0);
            }
        }
    };

    constexpr int kStep = kAWaves * kBlockKeys;
    for (int t0 = c0 + wave * kBlockKeys; t0 < c1; t0 += kStep) {
        uint4 kr[2][DS], vr[DJ];
        load_block(t0, kr, vr);
        compute_block(t0, kr, vr);
    }

    // ---- combine the four waves: per row, M = max over waves, weights 2^(m_w - M).
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        float lt = l_run[n] + __shfl_xor(l_run[n], 16, kWave);
        lt += __shfl_xor(lt, 32, kWave);
        if (lg == 0) {
            s_m[wave][n][l16] = m_run[n];
            s_l[wave][n][l16] = lt;
        }
    }
    __syncthreads();

    const bool single = (n_splits_b == 1);
    const size_t unit = (size_t(b) * a.Hkv + g) * a.row_groups + rg;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        // this lane's row l16: scale own accumulators by 2^(m_wave - M)
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
        // 256 threads: row r = tid / 16, dims (tid % 16) * (D/16) .. +D/16
        {
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
            const int row = rg * 32 + n * 16 + r;
            if (single) {
                if (row < a.rows) {
                    const int i = row / a.G;
                    const int h = g * a.G + row % a.G;
                    uint16_t* op = a.out + ((size_t(b) * (a.k + 1) + i) * a.Hq + h) * D + d0;
                    const float inv = 1.0f / lsum;
#pragma unroll
                    for (int dd = 0; dd < D / 16; ++dd) op[dd] = f32_to_bf16_bits(acc[dd] * inv);
                }
            } else {
                const size_t slot = (unit * a.splits + split) * 32 + n * 16 + r;
                float* po = a.part_o + slot * D + d0;
#pragma unroll
                for (int dd = 0; dd < D / 16; ++dd) po[dd] = acc[dd];
                if ((tid % 16) == 0) {
                    a.part_ml[slot * 2 + 0] = Mr;
                    a.part_ml[slot * 2 + 1] = lsum;
                }
            }
        }
        __syncthreads();
    }
}

// Merge the split partials of one (sequence, KV head, row group) in split order.
template <int D>
__global__ __launch_bounds__(kAT) void attn_merge_kernel(AttnArgs a, int tiles) {
    const int g = blockIdx.x / a.row_groups, rg = blockIdx.x % a.row_groups;
    const int b = blockIdx.y;
    const int N = a.seq_lens[b] + a.k + 1;
    const int ns = min(a.splits, (N + a.chunk - 1) / a.chunk);
    if (ns <= 1) return;
    const int tid = threadIdx.x;
    const size_t unit = (size_t(b) * a.Hkv + g) * a.row_groups + rg;
    for (int n = 0; n < tiles; ++n) {
        const int r = tid / 16;
        const int d0 = (tid % 16) * (D / 16);
        const int row = rg * 32 + n * 16 + r;
        if (row >= a.rows) continue;
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[((unit * a.splits + s) * 32 + n * 16 + r) * 2]);
        float lsum = 0.0f;
        float acc[D / 16];
#pragma unroll
        for (int dd = 0; dd < D / 16; ++dd) acc[dd] = 0.0f;
        for (int s = 0; s < ns; ++s) {
            const size_t slot = (unit * a.splits + s) * 32 + n * 16 + r;
            const float ms = a.part_ml[slot * 2];
            const float w = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
            lsum += w * a.part_ml[slot * 2 + 1];
            const float* po = a.part_o + slot * D + d0;
#pragma unroll
            for (int dd = 0; dd < D / 16; ++dd) acc[dd] += w * po[dd];
        }
        const int i = row / a.G;
        const int h = g * a.G + row % a.G;
        uint16_t* op = a.out + ((size_t(b) * (a.k + 1) + i) * a.Hq + h) * D + d0;
        const float inv = 1.0f / lsum;
#pragma unroll
        for (int dd = 0; dd < D / 16; ++dd) op[dd] = f32_to_bf16_bits(acc[dd] * inv);
    }
}

int floor_pow2(long long x) {
    int p = 1;
    while (2LL * p <= x) p *= 2;
    return p;
}

}  // namespace

AttnGeometry attn_geometry(int B, int k, int Hq, int Hkv, int D, int max_seq_len) {
    AttnGeometry g;
    const int G = Hq / Hkv;
    g.rows = (k + 1) * G;
    g.tiles = g.rows <= 16 ? 1 : 2;
    g.row_groups = (g.rows + 31) / 32;
    // Aim for ~4096 workgroups at the longest context, with at most 64 splits per
    // sequence (bounds the merge), chunks a power of two in [256, kMaxChunk].
    const long long units = static_cast<long long>(B) * Hkv * g.row_groups;
    long long target = static_cast<long long>(max_seq_len) * units / 4096;
    int chunk = floor_pow2(target < 256 ? 256 : target);
    while (chunk < kMaxChunk && (max_seq_len + chunk - 1) / chunk > 64) chunk *= 2;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    if (chunk < 256) chunk = 256;
    g.chunk = chunk;
    g.splits = (max_seq_len + chunk - 1) / chunk;
    // a single split never writes partials
    g.workspace = g.splits > 1 ? units * size_t(g.splits) * 32 * (size_t(D) + 2) * sizeof(float) : 0;
    return g;
}

hipError_t launch_attn(const AttnLaunch& p, const AttnGeometry& geo, hipStream_t stream) {
    AttnArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.kc = static_cast<const uint16_t*>(p.k_cache);
    a.vc = static_cast<const uint16_t*>(p.v_cache);
    a.bt = p.block_table;
    a.seq_lens = p.seq_lens;
    a.out = static_cast<uint16_t*>(p.out);
    const size_t units = size_t(p.B) * p.Hkv * geo.row_groups;
    a.part_o = static_cast<float*>(p.workspace);
    a.part_ml = a.part_o + units * geo.splits * 32 * size_t(p.D);
    a.k = p.k;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.G = p.Hq / p.Hkv;
    a.rows = geo.rows;
    a.row_groups = geo.row_groups;
    a.max_blocks = p.max_blocks;
    int lg = 0;
    while ((1 << lg) < p.block_size) ++lg;
    a.bs_log2 = lg;
    a.chunk = geo.chunk;
    a.splits = geo.splits;
    a.scale_log2 = p.sm_scale * kLog2e;

    const dim3 grid(geo.splits, p.Hkv * geo.row_groups, p.B), block(kAT);
    if (p.D == 128) {
        if (geo.tiles == 1) hipLaunchKernelGGL((attn_partial_kernel<128, 1>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_partial_kernel<128, 2>), grid, block, 0, stream, a);
    } else {
        if (geo.tiles == 1) hipLaunchKernelGGL((attn_partial_kernel<64, 1>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_partial_kernel<64, 2>), grid, block, 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || geo.splits <= 1) return e;
    const dim3 mgrid(p.Hkv * geo.row_groups, p.B);
    if (p.D == 128) hipLaunchKernelGGL(attn_merge_kernel<128>, mgrid, block, 0, stream, a, geo.tiles);
    else hipLaunchKernelGGL(attn_merge_kernel<64>, mgrid, block, 0, stream, a, geo.tiles);
    return hipGetLastError();
}

}  // namespace specverify
