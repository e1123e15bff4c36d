// The verify pass's upstream steps (gfx950): RoPE and KV append of the new rows,
// and the LM head that produces the logits the sampler reads.
//
// "Accelerating RL Post-Training Rollouts via System-Integrated Speculative
// Decoding" (gist.science summary), section 2: the target checks all k drafts in
// one forward pass; "ReSpec" (talk notes), Adaptive Server: the KV cache is
// extended in place. The pages name neither the position encoding nor the output
// head. This file implements rotate-half RoPE with a caller-given theta (pair j
// with j + D/2, angle pos * theta^(-2j/D)), the append of the rotated K and raw V
// at slot L + i (tree node n: position L + depth(n), slot L + n), and
// logits = hidden x W^T with bf16 operands and fp32 accumulation.
#include "common.hpp"
#include "kernels.hpp"

namespace specverify {
namespace {

// ---------------------------------------------------------------- RoPE + append

constexpr int kRopeThreads = 256;

// float64 -> bfloat16 bits, round to nearest even, in one rounding: the value is
// scaled by a power of two (exact) so that its 8 significant bits are the integer
// part, and rint (nearest even) rounds it.
__device__ __forceinline__ uint16_t bf16_rne(double x) {
    const uint16_t sign = signbit(x) ? 0x8000u : 0u;
    const double a = fabs(x);
    if (a == 0.0) return sign;
    if (!(a < 0x1.0p128)) return sign | 0x7F80u;
    int e;
    (void)frexp(a, &e);
    e -= 1;                                    // 2^e <= a < 2^(e+1)
    if (e < -126) return sign | static_cast<uint16_t>(rint(ldexp(a, 133)));   // subnormal: quantum 2^-133
    double n = rint(ldexp(a, 7 - e));          // in [128, 256]
    if (n == 256.0) {
        n = 128.0;
        e += 1;
    }
    if (e > 127) return sign | 0x7F80u;
    return sign | static_cast<uint16_t>((e + 127) << 7) | static_cast<uint16_t>(n - 128.0);
}

__device__ __forceinline__ double bf16_bits_to_f64(uint16_t h) {
    return static_cast<double>(__builtin_bit_cast(float, static_cast<uint32_t>(h) << 16));
}

struct RopeArgs {
    uint16_t* q;              // [B][k+1][Hq][D], rotated in place
    const uint16_t* k_new;    // [B][k+1][Hkv][D]
    const uint16_t* v_new;    // [B][k+1][Hkv][D]
    uint16_t* kc;             // [pages][Hkv][bs][D]
    uint16_t* vc;             // [pages][Hkv][D][bs]
    const int32_t* bt;
    const int32_t* seq_lens;
    const int32_t* parents;   // [B][k] or null (a chain)
    int k, Hq, Hkv, bs_log2, max_blocks, num_blocks;
    double log2_theta;
};

// One workgroup per new row (sequence b, row i).
template <int D>
__global__ __launch_bounds__(kRopeThreads) void rope_append_kernel(RopeArgs a) {
    constexpr int H2 = D / 2;
    __shared__ double s_cos[H2], s_sin[H2];
    const int i = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int L = a.seq_lens[b];
    int depth = i;
    if (a.parents && i > 0) {   // walk to the root; a broken parent index is clamped into [0, n)
        depth = 0;
        int n = i;
        for (int step = 0; step < a.k && n > 0; ++step) {
            int par = a.parents[size_t(b) * a.k + n - 1];
            par = par < 0 ? 0 : (par >= n ? n - 1 : par);
            n = par;
            ++depth;
        }
    }
    const double pos = static_cast<double>(L) + depth;
    if (tid < H2) {
        const double inv_freq = exp2(-(2.0 * tid / D) * a.log2_theta);
        double sn, cs;
        sincos(pos * inv_freq, &sn, &cs);
        s_cos[tid] = cs;
        s_sin[tid] = sn;
    }
    __syncthreads();

    const size_t row = size_t(b) * (a.k + 1) + i;
    uint16_t* qrow = a.q + row * a.Hq * D;
    for (int p = tid; p < a.Hq * H2; p += kRopeThreads) {
        const int h = p / H2, j = p % H2;
        uint16_t* x = qrow + size_t(h) * D;
        const double x0 = bf16_bits_to_f64(x[j]), x1 = bf16_bits_to_f64(x[j + H2]);
        x[j] = bf16_rne(x0 * s_cos[j] - x1 * s_sin[j]);
        x[j + H2] = bf16_rne(x1 * s_cos[j] + x0 * s_sin[j]);
    }

    // the cache slot of this row; a slot outside the block table or a page id out of
    // range leaves the cache untouched for this row
    const long long slot = static_cast<long long>(L) + i;
    const long long pidx = slot >> a.bs_log2;
    if (L < 0 || pidx >= a.max_blocks) return;
    const int page = a.bt[size_t(b) * a.max_blocks + pidx];
    if (page < 0 || page >= a.num_blocks) return;
    const int off = static_cast<int>(slot & ((1 << a.bs_log2) - 1));
    const uint16_t* krow = a.k_new + row * a.Hkv * D;
    const uint16_t* vrow = a.v_new + row * a.Hkv * D;
    for (int p = tid; p < a.Hkv * H2; p += kRopeThreads) {
        const int g = p / H2, j = p % H2;
        const uint16_t* x = krow + size_t(g) * D;
        const double x0 = bf16_bits_to_f64(x[j]), x1 = bf16_bits_to_f64(x[j + H2]);
        uint16_t* dst = a.kc + ((size_t(page) * a.Hkv + g) * (size_t(1) << a.bs_log2) + off) * D;
        dst[j] = bf16_rne(x0 * s_cos[j] - x1 * s_sin[j]);
        dst[j + H2] = bf16_rne(x1 * s_cos[j] + x0 * s_sin[j]);
    }
    for (int p = tid; p < a.Hkv * D; p += kRopeThreads) {
        const int g = p / D, d = p % D;
        a.vc[((size_t(page) * a.Hkv + g) * D + d) * (size_t(1) << a.bs_log2) + off] = vrow[size_t(g) * D + d];
    }
}

// ---------------------------------------------------------------- LM head
//
// logits[r][v] = sum_h hidden[r][h] W[v][h]: M = R rows (small: the verify rows),
// N = V (large), K = H. The weight is the stream (1 GB at the 8B shape), so each
// W element is loaded from HBM once, straight into MFMA registers; the hidden
// rows, read by every workgroup, are staged through LDS.
//
// Workgroup: NWM x NWN waves over a 256-row M block and NWN * 16 * NT vocabulary
// columns; wave (wm, wn) owns row tiles wm * MT .. + MT - 1 (MT = 16 / NWM) and 16 NT
// columns, so MT * NT v_mfma_f32_16x16x32_bf16 accumulators. K runs in chunks of 64.
// Inside a chunk the k order is permuted (the same way for both operands, so the sum
// is unchanged): lane group lg of MFMA step s holds k = 16 lg + 8 s + j, j < 8. A lane
// then reads 32 contiguous bytes of a W row per chunk, and the four lane groups cover
// the row's 128-byte line; the NWM waves that share columns read the same lines, the
// later ones from the cache.

constexpr int kGemmM = 256;                    // rows per M block, at most
constexpr int kGemmKC = 64;                    // K chunk
constexpr int kAStride = kGemmKC * 2 + 16;     // LDS bytes per staged row (padded)
// Loads of chunk j are issued RING chunks before the chunk that uses them, hidden
// rows and W alternating in one order (hidden j, W j, hidden j+1, ...). Vector loads
// complete in issue order, so the wait for a staged hidden chunk also covers the W
// loads issued before it; with both rings equally deep that costs W no lead.

constexpr int kLmRing = 2;

struct GemmArgs {
    const uint16_t* A;   // [R][H]
    const uint16_t* W;   // [V][H]
    float* C;            // [R][V]
    int R, H, V;
};

template <int NWM, int NWN, int NT, int RING, int MB>
__global__ __launch_bounds__(NWM * NWN * kWave) void lm_head_kernel(GemmArgs a) {
    constexpr int kRing = RING;
    static_assert(MB == 64 || MB == 128 || MB == 256, "M block: 64, 128 or 256 rows");
    constexpr int kThreads = NWM * NWN * kWave;
    constexpr int MT = MB / 16 / NWM;                     // row tiles per wave
    constexpr int kCols = NWN * 16 * NT;                  // columns per workgroup
    constexpr int AQ = MB * kGemmKC * 2 / 16 / kThreads;   // 16-byte pieces of the hidden chunk per thread
    constexpr int kPartsPerRow = 8 / AQ;                  // threads per 128-byte chunk row
    static_assert(AQ >= 1 && AQ * kPartsPerRow == 8 && MT * NWM * 16 == MB, "tile shape");
    struct WChunk { uint4 w[NT][2]; };
    struct AChunk { uint4 v[AQ]; };

    __shared__ __attribute__((aligned(16))) unsigned char s_a[2][MB * kAStride];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int wm = wave / NWN, wn = wave % NWN;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * kCols + wn * 16 * NT;
    const int m0 = blockIdx.y * MB;
    const int chunks = a.H / kGemmKC;

    // this lane's W rows (clamped into range: columns >= V are computed, never stored)
    const uint16_t* wrow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = min(n0 + 16 * t + l16, a.V - 1);
        wrow[t] = a.W + size_t(n) * a.H + 16 * lg;
    }
    auto load_w = [&](WChunk& c, int kc) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint16_t* p = wrow[t] + size_t(kc) * kGemmKC;
            c.w[t][0] = load16_nt(p);
            c.w[t][1] = load16_nt(p + 8);
        }
    };

    // hidden staging: thread -> (row, part of the 128-byte chunk row). Rows >= R stage a copy of
    // row R-1: output row m depends on hidden row m alone, and rows >= R are never written out.
    const int arow = tid / kPartsPerRow, apart = tid % kPartsPerRow;
    const uint16_t* asrc = a.A + size_t(min(m0 + arow, a.R - 1)) * a.H + 8 * AQ * apart;
    auto load_a = [&](AChunk& c, int kc) {
#pragma unroll
        for (int q = 0; q < AQ; ++q) c.v[q] = load16(asrc + size_t(kc) * kGemmKC + 8 * q);
    };
    auto store_a = [&](const AChunk& c, int buf) {
        unsigned char* dst = s_a[buf] + arow * kAStride + 16 * AQ * apart;
#pragma unroll
        for (int q = 0; q < AQ; ++q) *reinterpret_cast<uint4*>(dst + 16 * q) = c.v[q];
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Every load is issued unconditionally (chunk indices clamped at the end; the extra loads
    // re-read the last chunk and are never used), so the wait counts before each use are exact
    // and never drain the loads still in flight. The prologue issues in the loop's own order, so
    // the wait counts at the loop head are the same from both paths into it.
    WChunk wr[kRing];
    AChunk ar[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
        load_a(ar[j], min(j, chunks - 1));
        load_w(wr[j], min(j, chunks - 1));
    }
    store_a(ar[0], 0);
    __syncthreads();

    for (int c0 = 0; c0 < chunks; c0 += kRing) {   // chunks is a multiple of kRing
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            const int c = c0 + u;
            const unsigned char* abase = s_a[c & 1] + (wm * MT * 16 + l16) * kAStride + 32 * lg;
            const WChunk& w = wr[u];
            // A fragments read kPF row tiles ahead of their MFMAs (the order pinned), so the LDS
            // latency overlaps the MFMAs of the tiles before
            constexpr int kPF = MT < 4 ? MT : 4;
            uint4 af[kPF][2];
#pragma unroll
            for (int j = 0; j < kPF; ++j) {
                const unsigned char* ap = abase + j * 16 * kAStride;
                af[j][0] = *reinterpret_cast<const uint4*>(ap);
                af[j][1] = *reinterpret_cast<const uint4*>(ap + 16);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 a0 = af[mt % kPF][0], a1 = af[mt % kPF][1];
                if (mt + kPF < MT) {
                    const unsigned char* ap = abase + (mt + kPF) * 16 * kAStride;
                    af[mt % kPF][0] = *reinterpret_cast<const uint4*>(ap);
                    af[mt % kPF][1] = *reinterpret_cast<const uint4*>(ap + 16);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(w.w[t][0]),
                                                                        acc[mt][t], 0, 0, 0);
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(w.w[t][1]),
                                                                        acc[mt][t], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            load_a(ar[u], min(c + kRing, chunks - 1));
            load_w(wr[u], min(c + kRing, chunks - 1));
            store_a(ar[(u + 1) % kRing], (c + 1) & 1);   // after the last chunk: a copy nobody reads
            __syncthreads();
        }
    }

    // C tile: lane holds rows 16 (wm MT + mt) + 4 lg + e of column n0 + 16 t + l16
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = n0 + 16 * t + l16;
        if (n >= a.V) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 16 * (wm * MT + mt) + 4 * lg + e;
                if (m < a.R) a.C[size_t(m) * a.V + n] = acc[mt][t][e];
            }
    }
}

}  // namespace

hipError_t launch_rope_append(const RopeLaunch& p, hipStream_t stream) {
    RopeArgs a;
    a.q = static_cast<uint16_t*>(p.q);
    a.k_new = static_cast<const uint16_t*>(p.k_new);
    a.v_new = static_cast<const uint16_t*>(p.v_new);
    a.kc = static_cast<uint16_t*>(p.k_cache);
    a.vc = static_cast<uint16_t*>(p.v_cache);
    a.bt = p.block_table;
    a.seq_lens = p.seq_lens;
    a.parents = p.parents;
    a.k = p.k;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.bs_log2 = __builtin_ctz(static_cast<unsigned>(p.block_size));
    a.max_blocks = p.max_blocks;
    a.num_blocks = p.num_blocks;
    a.log2_theta = std::log2(p.theta);
    const dim3 grid(p.k + 1, p.B);
    if (p.D == 128)
        hipLaunchKernelGGL(rope_append_kernel<128>, grid, dim3(kRopeThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(rope_append_kernel<64>, grid, dim3(kRopeThreads), 0, stream, a);
    return hipGetLastError();
}

int lm_head_k_multiple() { return kGemmKC * kLmRing; }

hipError_t launch_lm_head(const LmHeadLaunch& p, hipStream_t stream) {
    GemmArgs a;
    a.A = static_cast<const uint16_t*>(p.hidden);
    a.W = static_cast<const uint16_t*>(p.weight);
    a.C = p.logits;
    a.R = p.R;
    a.H = p.H;
    a.V = p.V;
    // one row of 8 waves, two 16-column tiles each (256 columns per workgroup), rings of two; the
    // M block is the smallest of 64, 128 and 256 rows that holds R (256-row blocks beyond that)
    constexpr int WM = 1, WN = 8, NT = 2, RING = kLmRing;
    const int gx = (p.V + WN * 16 * NT - 1) / (WN * 16 * NT);
    if (p.R <= 64)
        hipLaunchKernelGGL((lm_head_kernel<WM, WN, NT, RING, 64>), dim3(gx, 1), dim3(WM * WN * kWave), 0, stream, a);
    else if (p.R <= 128)
        hipLaunchKernelGGL((lm_head_kernel<WM, WN, NT, RING, 128>), dim3(gx, 1), dim3(WM * WN * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL((lm_head_kernel<WM, WN, NT, RING, kGemmM>), dim3(gx, (p.R + kGemmM - 1) / kGemmM),
                           dim3(WM * WN * kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace specverify
