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

#include <utility>

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
// W element is loaded from HBM once, straight into MFMA registers; the hidden rows,
// read by every workgroup, are staged through LDS.
//
// Workgroup: 8 waves over an MB-row block (MB = 64, 128 or 256) and 256 vocabulary
// columns; each wave owns 32 columns (two 16-column tiles) and all MB rows, so
// MB / 16 x 2 v_mfma_f32_16x16x32_bf16 accumulators, 128 registers at MB = 256, which
// leaves room for two waves per SIMD. K runs in chunks of 64. Inside a chunk the k
// order is permuted (the same way for both operands, so the sum is unchanged): lane
// group lg of MFMA step s holds k = 16 lg + 8 s + j, j < 8, so that a lane reads 32
// contiguous bytes of its W row per chunk and the four lane groups cover the row's
// 128 bytes.
//
// The hidden rows reach LDS by buffer-to-LDS loads (no register staging) into two
// slots. A chunk row is 128 bytes; its eight 16-byte pieces are stored XOR-swizzled by
// sw(row) = (row % 8) ^ ((row / 8) % 2). A 16-byte LDS read is served eight lanes at a
// time, and the eight rows 8i .. 8i + 7 of a fragment read then fetch eight different
// pieces, i.e. eight distinct 16-byte bank groups of the 128-byte bank row; the 16 rows
// of the fragment also fall in 16 distinct (row parity, piece) pairs, so a 256-byte
// bank row would serve them without conflict too. (Swizzling by (row / 2) % 8 gave
// pairs of rows the same piece: half of the LDS busy cycles were bank conflicts.)
// The slots are two separate LDS arrays, each named by a compile-time index: the
// compiler can then tell a read of one slot from a load into the other, and waits only
// for the latter's own loads instead of draining every load in flight before each read
// (which, with one array, it did: that wait serialised the W prefetch). W is loaded two
// chunks ahead of its MFMAs.
//
// Each workgroup starts its walk over the K chunks at its own chunk (5 x its column
// block, wrapping): W rows lie 8 KB apart, and with every workgroup at the same chunk
// the requests in flight share their low address bits and pile onto a few HBM
// channels; staggering the start took the 8B-shape call from 331 us to 294 us.

constexpr int kGemmKC = 64;                    // K chunk
constexpr int kLmWaves = 8;                    // waves per workgroup, one 32-column strip each
constexpr int kLmNT = 2;                       // 16-column tiles per wave
constexpr int kLmCols = kLmWaves * 16 * kLmNT; // columns per workgroup
constexpr int kLmStagger = 5;                  // starting chunk = 5 x column block (mod chunks)

struct GemmArgs {
    const uint16_t* A;   // [R][H]
    const uint16_t* W;   // [V][H]
    float* C;            // [R][V]
    int R, H, V;
    int gx, gy;          // column blocks, row blocks
};

// f(std::integral_constant<int, i>) for i = 0 .. N - 1, each with its index as a constant.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at lds + 16 l
// (the LDS address must be the same in every lane); a read past the buffer's size
// yields zeros.
__device__ __forceinline__ void load_to_lds16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

template <int MB>
__global__ __launch_bounds__(kLmWaves * kWave) void lm_head_kernel(GemmArgs a) {
    static_assert(MB == 64 || MB == 128 || MB == 256, "M block: 64, 128 or 256 rows");
    constexpr int NT = kLmNT;
    constexpr int MT = MB / 16;                                    // row tiles per wave
    constexpr int kChunkBytes = MB * kGemmKC * 2;
    constexpr int kDma = kChunkBytes / (kWave * 16) / kLmWaves;    // 1 KB loads per wave per chunk
    static_assert(kDma >= 1, "chunk split");
    constexpr int kWOps = 2 * NT;                                  // W loads per wave per chunk
    // Issue order: hidden chunk 0, W chunks 0 and 1, then per chunk c: wait, hidden chunk
    // c + 1, MFMAs of c, W chunk c + 2. Between hidden chunk c and chunk c's wait come W
    // chunk c + 1's loads alone (W chunks 0 and 1 for c = 0), and vector loads complete in
    // issue order, so waiting until kWOps loads are outstanding completes hidden chunk c.
    constexpr int kAfter = kWOps;
    struct WChunk { uint4 w[NT][2]; };

    // one array per slot, each addressed only through a compile-time slot number
    __shared__ __attribute__((aligned(1024))) unsigned char s_a0[kChunkBytes];
    __shared__ __attribute__((aligned(1024))) unsigned char s_a1[kChunkBytes];
    auto slot = [&](auto S) __attribute__((always_inline)) -> unsigned char* {
        if constexpr (decltype(S)::value == 0) return s_a0;
        else return s_a1;
    };

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int l16 = lane & 15, lg = lane >> 4;
    // workgroup -> (column block, row block). Workgroups are dealt to the 8 XCDs in turn; the
    // row blocks of one column block (R > 256) go to one XCD one after another, so that they
    // tend to run together and find W in that XCD's L2.
    const unsigned id = blockIdx.x, xcd = id % 8u, sx = id / 8u;
    const int rb = static_cast<int>(sx % static_cast<unsigned>(a.gy));
    const int cb = static_cast<int>(sx / static_cast<unsigned>(a.gy)) * 8 + static_cast<int>(xcd);
    if (cb >= a.gx) return;   // padding of the grid to whole rounds of 8
    const int n0 = cb * kLmCols + wave * 16 * NT;
    const int m0 = rb * MB;
    const int chunks = a.H / kGemmKC;   // even
    const int k_start = static_cast<int>((static_cast<unsigned>(cb) * kLmStagger) % static_cast<unsigned>(chunks));
    auto rot = [&](int kc) { kc += k_start; return kc >= chunks ? kc - chunks : kc; };

    // this lane's W rows (clamped into range: columns >= V are computed, never stored)
    const uint16_t* wrow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wrow[t] = a.W + size_t(min(n0 + 16 * t + l16, a.V - 1)) * a.H + 16 * lg;
    auto load_w = [&](WChunk& c, int kc) {
        kc = rot(kc);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint16_t* p = wrow[t] + size_t(kc) * kGemmKC;
            c.w[t][0] = load16(p);
            c.w[t][1] = load16(p + 8);
        }
    };

    // hidden rows m0 .. m0 + MB - 1 through a buffer resource: rows >= R read as zero (their
    // outputs are never stored). Load i of this wave fills LDS slots (wave kDma + i) 64 + lane:
    // row r = slot / 8, physical piece slot % 8, holding logical piece (slot % 8) ^ sw(r).
    const int rows_here = min(MB, a.R - m0);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.A + size_t(m0) * a.H), static_cast<short>(0), rows_here * a.H * 2, 0x00020000);
    int voff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int r = (wave * kDma + i) * 8 + (lane >> 3);
        voff[i] = r * a.H * 2 + (((lane & 7) ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
    }
    auto dma = [&](int chunk, unsigned char* buf) {
        const int kc = rot(min(chunk, chunks - 1));   // past the last chunk: a copy nobody reads
#pragma unroll
        for (int i = 0; i < kDma; ++i)
            load_to_lds16(ra, buf + (wave * kDma + i) * (kWave * 16), voff[i], kc * kGemmKC * 2);
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    WChunk wr[2];
    dma(0, s_a0);
    load_w(wr[0], 0);
    load_w(wr[1], min(1, chunks - 1));

    // fragment reads: row 16 mt + l16, logical pieces 2 lg and 2 lg + 1 (sw depends on the row
    // modulo 16 only, so it is the same for every row tile)
    const int sw = (l16 & 7) ^ (l16 >> 3);
    const int rd0 = l16 * 128 + (((2 * lg) ^ sw) << 4);
    const int rd1 = l16 * 128 + (((2 * lg + 1) ^ sw) << 4);

    for (int c0 = 0; c0 < chunks; c0 += 2) {
        static_for<2>([&](auto U) __attribute__((always_inline)) {
            constexpr int u = decltype(U)::value;
            const int c = c0 + u;
            // this wave's loads of chunk c have landed and its reads of chunk c - 1 are done; after
            // the barrier, every wave's are, so chunk c is readable and c - 1's slot refillable
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kAfter) : "memory");
            dma(c + 1, slot(std::integral_constant<int, 1 - u>{}));
            const unsigned char* buf = slot(std::integral_constant<int, u>{});
            const WChunk& w = wr[u];
            // A fragments read kPF row tiles ahead of their MFMAs (the order pinned), so the LDS
            // latency overlaps the MFMAs of the tiles before
            constexpr int kPF = MT < 4 ? MT : 4;
            uint4 af[kPF][2];
#pragma unroll
            for (int j = 0; j < kPF; ++j) {
                af[j][0] = *reinterpret_cast<const uint4*>(buf + j * 2048 + rd0);
                af[j][1] = *reinterpret_cast<const uint4*>(buf + j * 2048 + rd1);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint4 a0 = af[mt % kPF][0], a1 = af[mt % kPF][1];
                if (mt + kPF < MT) {
                    af[mt % kPF][0] = *reinterpret_cast<const uint4*>(buf + (mt + kPF) * 2048 + rd0);
                    af[mt % kPF][1] = *reinterpret_cast<const uint4*>(buf + (mt + kPF) * 2048 + rd1);
                }
                __builtin_amdgcn_sched_barrier(0);
                // step 0 of every tile, then step 1: back-to-back MFMAs on one accumulator stall
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(w.w[t][0]),
                                                                        acc[mt][t], 0, 0, 0);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(w.w[t][1]),
                                                                        acc[mt][t], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            load_w(wr[u], min(c + 2, chunks - 1));
        });
    }
    // the surplus loads past the last chunk land before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // C tile: lane holds rows 16 mt + 4 lg + e of column n0 + 16 t + l16; streaming stores (the
    // logits are written once here and read once by the sampler, from HBM either way)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int n = n0 + 16 * t + l16;
        if (n >= a.V) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + 16 * mt + 4 * lg + e;
                if (m < a.R) __builtin_nontemporal_store(acc[mt][t][e], a.C + size_t(m) * a.V + n);
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

int lm_head_k_multiple() { return 2 * kGemmKC; }

bool lm_head_grid_ok(int R, int V) {
    const long long mb = R <= 64 ? 64 : (R <= 128 ? 128 : 256);
    const long long gx = (static_cast<long long>(V) + kLmCols - 1) / kLmCols;
    const long long gy = (R + mb - 1) / mb;
    return (gx + 7) / 8 * 8 * gy <= (1LL << 23);
}

hipError_t launch_lm_head(const LmHeadLaunch& p, hipStream_t stream) {
    GemmArgs a;
    a.A = static_cast<const uint16_t*>(p.hidden);
    a.W = static_cast<const uint16_t*>(p.weight);
    a.C = p.logits;
    a.R = p.R;
    a.H = p.H;
    a.V = p.V;
    // the M block is the smallest of 64, 128 and 256 rows that holds R (256-row blocks beyond that)
    const int mb = p.R <= 64 ? 64 : (p.R <= 128 ? 128 : 256);
    a.gx = (p.V + kLmCols - 1) / kLmCols;
    a.gy = (p.R + mb - 1) / mb;
    const dim3 grid(static_cast<unsigned>((a.gx + 7) / 8) * 8u * static_cast<unsigned>(a.gy));
    if (mb == 64)
        hipLaunchKernelGGL(lm_head_kernel<64>, grid, dim3(kLmWaves * kWave), 0, stream, a);
    else if (mb == 128)
        hipLaunchKernelGGL(lm_head_kernel<128>, grid, dim3(kLmWaves * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL(lm_head_kernel<256>, grid, dim3(kLmWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace specverify
