// Vocab-wide softmax + lossless acceptance chain + residual / bonus sampling (gfx950).
//
// What is computed: "Accelerating RL Post-Training Rollouts via System-Integrated
// Speculative Decoding" (gist.science summary), section 2 "Method", core mechanism
// (verify the k drafts against the target distribution by rejection sampling, so
// the rollout distribution equals the target policy's); "Online Draft Co-Training
// for Speculative Decoding ..." (ta-paperlens), metaphor section (rewrite from the
// first miss). The rule is standard speculative sampling: accept d_j iff
// u_acc < p_j(d_j)/q_j(d_j); at the first rejection sample max(0, p_j - q_j);
// after full acceptance sample p_k. Sampling is inverse CDF in ascending token id.
//
// How (one MI355X):
//  * The vocab of a row is cut into slices of kSlice = 4096 logits. Every launch
//    is a grid of (W slices) x (B sequences) workgroups of 256 threads, so even
//    B = 64 puts 2048 workgroups on the 256 CUs; a thread holds 16 logits per row
//    in registers, fetched by 16-byte loads that are all in flight together.
//  * Launch j = 0..k. Workgroups never talk to each other inside a launch: the
//    kernel boundary is the only synchronisation (no atomics, no cache flushes).
//    Launch j first re-derives decision j-1 of its sequence from the slice
//    partials launch j-1 stored (a fixed-order combine, so every workgroup of the
//    sequence reaches the same decision), then does one of:
//      - accepted, j < k: max and sum of exps of its slice of rows p_j and q_j;
//      - rejected at j-1: fp64 sub-chunk sums of max(0, p - q) of its slice;
//      - accepted, j = k: sub-chunk sums of exps of its slice of the bonus row.
//    Sequences that left the chain return at once, so rows after a sequence's
//    first rejection are never read.
//  * A final launch, one wavefront per sequence, finds the sub-chunk (256 logits)
//    where the running sum crosses u_smp * total, rescans that sub-chunk with a
//    wavefront prefix scan, and writes the sample and the padding.
//  * Precision: exps of logits within kTheta nats of a slice maximum are taken
//    in fp64, all others in fp32, and every sum is accumulated in fp64, so the
//    normalisers and the CDF match an fp64 reference to ~1e-10 of their mass.
#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace specverify {
namespace {

constexpr int kRT = 256;                     // threads per workgroup
constexpr int kWavesRT = kRT / kWave;        // 4
constexpr int kEPT = 16;                     // logits per thread per row
constexpr int kSlice = kRT * kEPT;           // 4096 logits per slice
constexpr int kSub = 4 * kWave;              // 256 logits: one wave's 16-byte load
constexpr int kSubPerSlice = kSlice / kSub;  // 16
constexpr float kTheta = 8.0f;

enum : int { kModeResidual = 0, kModeBonus = 1 };

struct FinalRecord {       // written once per sequence, when its chain ends
    int mode;
    int a;
    int pad0, pad1;
    double Mp, Zp, Mq, Zq; // residual mode: normalisers of the rejected pair
};

constexpr int kChainPart = 4;                          // m_p, Z_p, m_q, Z_q
constexpr int kSamplePart = 2 + 2 * kSubPerSlice + 2;  // m_w, R_w, S_r[16], P_w, S_p[16], pad
constexpr int kOffR = 1, kOffSr = 2, kOffP = 2 + kSubPerSlice, kOffSp = 3 + kSubPerSlice;

struct RejectArgs {
    const float* target;
    const float* draft;
    const int32_t* draft_tokens;
    const int64_t* seq_ids;
    const int32_t* seq_lens;
    int32_t* out_tokens;
    int32_t* num_accepted;
    float* out_probs;
    float* accept_probs;
    int32_t* active;       // [2][B], parity-double-buffered by launch index
    FinalRecord* final_rec;
    double* chain_part;    // [B][k][W][kChainPart]
    double* sample_part;   // [B][W][kSamplePart]
    int B, k, V, W;
    float invT;
    double invT64;
    uint64_t seed;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct RejectLayout {
    size_t active, final_rec, chain_part, sample_part, total;
};

RejectLayout reject_layout(int B, int k, int W) {
    RejectLayout L;
    size_t o = 0;
    L.active = o;      o = align256(o + sizeof(int32_t) * 2 * size_t(B));
    L.final_rec = o;   o = align256(o + sizeof(FinalRecord) * size_t(B));
    L.chain_part = o;  o = align256(o + sizeof(double) * size_t(B) * k * W * kChainPart);
    L.sample_part = o; o = align256(o + sizeof(double) * size_t(B) * W * kSamplePart);
    L.total = o;
    return L;
}

// Slice element e of this thread: e = i*1024 + tid*4 + c (i, c in 0..3), so each
// (i, wave) pair is a contiguous run of 256 logits: the sub-chunk i*4 + wave.
// Loads are unconditional (clamped addresses) so all of them are in flight together.
template <bool kVec4>
__device__ __forceinline__ void load_slice(const float* row, int V, int w, float (&v)[kEPT]) {
    const int tid = threadIdx.x;
    if (kVec4) {
        float4 f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int x0 = w * kSlice + i * (kRT * 4) + tid * 4;
            f[i] = *reinterpret_cast<const float4*>(row + min(x0, V - 4));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = w * kSlice + i * (kRT * 4) + tid * 4 < V;
            v[4 * i + 0] = ok ? f[i].x : -INFINITY;
            v[4 * i + 1] = ok ? f[i].y : -INFINITY;
            v[4 * i + 2] = ok ? f[i].z : -INFINITY;
            v[4 * i + 3] = ok ? f[i].w : -INFINITY;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int x = w * kSlice + i * (kRT * 4) + tid * 4 + c;
                const float val = row[min(x, V - 1)];
                v[4 * i + c] = (x < V) ? val : -INFINITY;
            }
    }
}

template <bool kVec4>
__device__ __forceinline__ void load_sub(const float* row, int V, int x0, float (&v)[4]) {
    if (kVec4) {
        const float4 f = *reinterpret_cast<const float4*>(row + min(x0, V - 4));
        const bool ok = x0 < V;
        v[0] = ok ? f.x : -INFINITY; v[1] = ok ? f.y : -INFINITY;
        v[2] = ok ? f.z : -INFINITY; v[3] = ok ? f.w : -INFINITY;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float val = row[min(x0 + c, V - 1)];
            v[c] = (x0 + c < V) ? val : -INFINITY;
        }
    }
}

// e^{(z - m)/T} in fp64 for one logit.
__device__ __forceinline__ double exp_f64(float z, double m, double invT64) {
    return exp((static_cast<double>(z) - m) * invT64);
}

// e^{(z - m)/T} for N logits: fp32 for terms more than kTheta nats below m, fp64
// otherwise. The fp64 terms are visited by a per-lane loop over a bitmask, so a
// wave pays for max-over-lanes of its flagged count, not for every slot.
template <int N>
__device__ __forceinline__ void exps_mixed(const float (&z)[N], float m, float invT, double invT64,
                                           double (&out)[N]) {
    unsigned flags = 0;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float x = (z[e] - m) * invT;
        const bool near = x > -kTheta;
        flags |= static_cast<unsigned>(near) << e;
        out[e] = near ? 0.0 : static_cast<double>(expf(x));
    }
    const double m64 = static_cast<double>(m);
    while (flags) {
        const int e = __builtin_ctz(flags);
        flags &= flags - 1;
        float ze = 0.0f;
#pragma unroll
        for (int s = 0; s < N; ++s) ze = (s == e) ? z[s] : ze;
        const double val = exp_f64(ze, m64, invT64);
#pragma unroll
        for (int s = 0; s < N; ++s) out[s] = (s == e) ? val : out[s];
    }
}

template <int N>
__device__ __forceinline__ double sum_exps_mixed(const float (&z)[N], float m, float invT, double invT64) {
    unsigned flags = 0;
    float tail = 0.0f;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float x = (z[e] - m) * invT;
        const bool near = x > -kTheta;
        flags |= static_cast<unsigned>(near) << e;
        tail += near ? 0.0f : expf(x);
    }
    double acc = static_cast<double>(tail);
    const double m64 = static_cast<double>(m);
    while (flags) {
        const int e = __builtin_ctz(flags);
        flags &= flags - 1;
        float ze = 0.0f;
#pragma unroll
        for (int s = 0; s < N; ++s) ze = (s == e) ? z[s] : ze;
        acc += exp_f64(ze, m64, invT64);
    }
    return acc;
}

__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kWavesRT; ++i) r = fmaxf(r, red[i]);
    return r;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
    v = wave_sum(v);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double r = red[0];
#pragma unroll
    for (int i = 1; i < kWavesRT; ++i) r += red[i];
    return r;
}

// Inclusive prefix sum across the wavefront (Hillis-Steele, fixed order).
__device__ __forceinline__ double wave_incl_scan(double v) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double y = __shfl_up(v, o, kWave);
        if (lane >= o) v += y;
    }
    return v;
}

__device__ __forceinline__ double wave_excl_from_incl(double incl) {
    const double e = __shfl_up(incl, 1, kWave);
    return (threadIdx.x % kWave) == 0 ? 0.0 : e;
}

// Combine W slice partials (max m_w, sum of exps Z_w relative to m_w) into the row's
// (M, Z) inside one wavefront: lanes take slices, butterflies reduce in a fixed order.
__device__ void combine_row(const double* part, int stride, int offset, int W, double invT64,
                            double* M_out, double* Z_out) {
    const int lane = threadIdx.x % kWave;
    double m = -INFINITY;
    for (int w = lane; w < W; w += kWave) m = fmax(m, part[size_t(w) * stride + offset]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, kWave));
    double z = 0.0;
    for (int w = lane; w < W; w += kWave) {
        const double mw = part[size_t(w) * stride + offset];
        const double zw = part[size_t(w) * stride + offset + 1];
        z += (zw > 0.0) ? zw * exp((mw - m) * invT64) : 0.0;
    }
    *M_out = m;
    *Z_out = wave_sum(z);
}

// Sampling weights of a residual: max(0, p - q), also returning e^{(z_p - M_p)/T}
// (the weights of the p-fallback).
struct ResidualCtx {
    float mp, mq;            // row maxima (exactly representable logits)
    double invZp, invZq;
};

template <int N>
__device__ __forceinline__ void residual_weights(const float (&zp)[N], const float (&zq)[N], const ResidualCtx& c,
                                                 float invT, double invT64, double (&r)[N], double (&ep)[N]) {
    double eq[N];
    exps_mixed(zp, c.mp, invT, invT64, ep);
    exps_mixed(zq, c.mq, invT, invT64, eq);
#pragma unroll
    for (int e = 0; e < N; ++e) r[e] = fmax(0.0, ep[e] * c.invZp - eq[e] * c.invZq);
}

struct Decision {
    int accepted;
    double Mp, Zp, Mq, Zq;
};

// Decision j of sequence b from the slice partials of launch j (one wavefront);
// lane 0 also writes the outputs of that decision when `write` is set.
__device__ Decision decide(const RejectArgs& a, int b, int j, bool write) {
    const double* part = a.chain_part + (size_t(b) * a.k + j) * a.W * kChainPart;
    Decision d;
    combine_row(part, kChainPart, 0, a.W, a.invT64, &d.Mp, &d.Zp);
    combine_row(part, kChainPart, 2, a.W, a.invT64, &d.Mq, &d.Zq);
    const float* prow = a.target + (size_t(b) * (a.k + 1) + j) * a.V;
    const float* qrow = a.draft + (size_t(b) * a.k + j) * a.V;
    const int tok = a.draft_tokens[size_t(b) * a.k + j];
    const bool ok = tok >= 0 && tok < a.V;   // out-of-range ids (a broken precondition) are rejected
    const double p_d = ok ? exp((static_cast<double>(prow[ok ? tok : 0]) - d.Mp) * a.invT64) / d.Zp : 0.0;
    const double q_d = ok ? exp((static_cast<double>(qrow[ok ? tok : 0]) - d.Mq) * a.invT64) / d.Zq : 0.0;
    const double ratio = (q_d > 0.0) ? p_d / q_d : (p_d > 0.0 ? INFINITY : 0.0);
    double u_acc, u_smp;
    verify_uniforms(a.seed, a.seq_ids[b], int64_t(a.seq_lens[b]) + 1 + j, &u_acc, &u_smp);
    d.accepted = u_acc < ratio;
    if (write && (threadIdx.x % kWave) == 0) {
        if (a.accept_probs) a.accept_probs[size_t(b) * a.k + j] = static_cast<float>(fmin(1.0, ratio));
        if (d.accepted) {
            a.out_tokens[size_t(b) * (a.k + 1) + j] = tok;
            if (a.out_probs) a.out_probs[size_t(b) * (a.k + 1) + j] = static_cast<float>(p_d);
        }
    }
    return d;
}

enum : int { kWorkStats = 0, kWorkResidual = 1, kWorkBonus = 2 };

template <bool kVec4>
__global__ __launch_bounds__(kRT) void reject_level_kernel(RejectArgs a, int j) {
    __shared__ float red_f[kWavesRT];
    __shared__ double red_d[kWavesRT];
    __shared__ double s_sub[2][kSubPerSlice];
    __shared__ int s_work;
    __shared__ double s_norm[4];
    const int w = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    int32_t* active_in = a.active + size_t((j + 1) & 1) * a.B;
    int32_t* active_out = a.active + size_t(j & 1) * a.B;
    const bool leader = (w == 0);

    int work = kWorkStats;
    if (j > 0) {
        if (active_in[b] == 0) {
            if (leader && tid == 0) active_out[b] = 0;
            return;
        }
        if (wave == 0) {
            const Decision d = decide(a, b, j - 1, leader);
            if (lane == 0) {
                s_work = d.accepted ? (j < a.k ? kWorkStats : kWorkBonus) : kWorkResidual;
                s_norm[0] = d.Mp; s_norm[1] = d.Zp; s_norm[2] = d.Mq; s_norm[3] = d.Zq;
                if (leader) {
                    active_out[b] = (d.accepted && j < a.k) ? 1 : 0;
                    if (!d.accepted) {
                        FinalRecord r;
                        r.mode = kModeResidual; r.a = j - 1; r.pad0 = r.pad1 = 0;
                        r.Mp = d.Mp; r.Zp = d.Zp; r.Mq = d.Mq; r.Zq = d.Zq;
                        a.final_rec[b] = r;
                    } else if (j == a.k) {
                        FinalRecord r;
                        r.mode = kModeBonus; r.a = a.k; r.pad0 = r.pad1 = 0;
                        r.Mp = r.Zp = r.Mq = r.Zq = 0.0;
                        a.final_rec[b] = r;
                    }
                }
            }
        }
        __syncthreads();
        work = s_work;
    } else if (leader && tid == 0) {
        active_out[b] = 1;
    }

    if (work == kWorkStats) {
        const float* prow = a.target + (size_t(b) * (a.k + 1) + j) * a.V;
        const float* qrow = a.draft + (size_t(b) * a.k + j) * a.V;
        float vp[kEPT], vq[kEPT];
        load_slice<kVec4>(prow, a.V, w, vp);
        load_slice<kVec4>(qrow, a.V, w, vq);
        float tp = -INFINITY, tq = -INFINITY;
#pragma unroll
        for (int e = 0; e < kEPT; ++e) { tp = fmaxf(tp, vp[e]); tq = fmaxf(tq, vq[e]); }
        const float mp = block_max(tp, red_f);
        const float mq = block_max(tq, red_f);
        // a slice of -inf logits contributes nothing (and must not form -inf - -inf)
        const double zp = block_sum(mp == -INFINITY ? 0.0 : sum_exps_mixed(vp, mp, a.invT, a.invT64), red_d);
        const double zq = block_sum(mq == -INFINITY ? 0.0 : sum_exps_mixed(vq, mq, a.invT, a.invT64), red_d);
        if (tid == 0) {
            double* part = a.chain_part + ((size_t(b) * a.k + j) * a.W + w) * kChainPart;
            part[0] = mp; part[1] = zp; part[2] = mq; part[3] = zq;
        }
        return;
    }

    // Sampling work: sub-chunk sums of the weights over this slice.
    double sr[4], sp[4];
    double mw = 0.0;
    if (work == kWorkResidual) {
        const int r = j - 1;
        const float* prow = a.target + (size_t(b) * (a.k + 1) + r) * a.V;
        const float* qrow = a.draft + (size_t(b) * a.k + r) * a.V;
        float vp[kEPT], vq[kEPT];
        load_slice<kVec4>(prow, a.V, w, vp);
        load_slice<kVec4>(qrow, a.V, w, vq);
        ResidualCtx c;
        c.mp = static_cast<float>(s_norm[0]);
        c.mq = static_cast<float>(s_norm[2]);
        c.invZp = 1.0 / s_norm[1];
        c.invZq = 1.0 / s_norm[3];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float zp4[4], zq4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) { zp4[e] = vp[4 * i + e]; zq4[e] = vq[4 * i + e]; }
            double rr[4], ep[4];
            residual_weights(zp4, zq4, c, a.invT, a.invT64, rr, ep);
            sr[i] = ((rr[0] + rr[1]) + rr[2]) + rr[3];
            sp[i] = ((ep[0] + ep[1]) + ep[2]) + ep[3];
        }
    } else {
        const float* prow = a.target + (size_t(b) * (a.k + 1) + a.k) * a.V;
        float vp[kEPT];
        load_slice<kVec4>(prow, a.V, w, vp);
        float t = -INFINITY;
#pragma unroll
        for (int e = 0; e < kEPT; ++e) t = fmaxf(t, vp[e]);
        const float m = block_max(t, red_f);
        mw = m;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float z4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) z4[e] = vp[4 * i + e];
            double ex[4] = {0.0, 0.0, 0.0, 0.0};
            if (m != -INFINITY) exps_mixed(z4, m, a.invT, a.invT64, ex);
            sr[i] = ((ex[0] + ex[1]) + ex[2]) + ex[3];
            sp[i] = 0.0;
        }
    }
    // sub-chunk (i, wave) = logits [i*1024 + wave*256, +256) of the slice
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double r = wave_sum(sr[i]);
        const double p = wave_sum(sp[i]);
        if (lane == 0) { s_sub[0][i * kWavesRT + wave] = r; s_sub[1][i * kWavesRT + wave] = p; }
    }
    __syncthreads();
    if (tid == 0) {
        double* part = a.sample_part + (size_t(b) * a.W + w) * kSamplePart;
        double R = 0.0, P = 0.0;
        for (int s = 0; s < kSubPerSlice; ++s) {
            part[kOffSr + s] = s_sub[0][s];
            part[kOffSp + s] = s_sub[1][s];
            R += s_sub[0][s];
            P += s_sub[1][s];
        }
        part[0] = mw;
        part[kOffR] = R;
        part[kOffP] = P;
    }
}

// One wavefront per sequence: locate and write the residual / bonus sample.
// Slices, then sub-chunks, then logits are searched with wavefront prefix scans
// in a fixed order; at each level the crossing is the first positive weight
// whose running sum exceeds t = u_smp * total. If rounding leaves no crossing,
// the last positive weight is taken (at the slice level: the largest token with
// positive weight).
template <bool kVec4>
__global__ __launch_bounds__(kWave) void reject_finalize_kernel(RejectArgs a) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const FinalRecord rec = a.final_rec[b];
    const int mode = rec.mode, aa = rec.a;
    const float* prow = a.target + (size_t(b) * (a.k + 1) + aa) * a.V;
    const float* qrow = a.draft + (size_t(b) * a.k + (aa < a.k ? aa : 0)) * a.V;
    const double* part = a.sample_part + size_t(b) * a.W * kSamplePart;

    double M = 0.0;
    if (mode == kModeBonus) {
        double m = -INFINITY;
        for (int ww = lane; ww < a.W; ww += kWave) m = fmax(m, part[size_t(ww) * kSamplePart]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, kWave));
        M = m;
    }
    auto slice_weight = [&](int ww, int off) -> double {
        if (ww >= a.W) return 0.0;
        const double* pw = part + size_t(ww) * kSamplePart;
        const double s = pw[off];
        if (mode != kModeBonus) return s;
        return (s > 0.0) ? s * exp((pw[0] - M) * a.invT64) : 0.0;
    };
    auto row_total = [&](int off) -> double {
        double tot = 0.0;
        for (int base = 0; base < a.W; base += kWave)
            tot += __shfl(wave_incl_scan(slice_weight(base + lane, off)), kWave - 1, kWave);
        return tot;
    };
    int use_p = 0;
    double total = row_total(kOffR);
    if (mode == kModeResidual && !(total > 0.0)) {   // zero residual: sample p_j instead
        use_p = 1;
        total = row_total(kOffP);
    }
    const int sum_off = use_p ? kOffP : kOffR;
    const int sub_off = use_p ? kOffSp : kOffSr;
    double u_acc, u_smp;
    verify_uniforms(a.seed, a.seq_ids[b], int64_t(a.seq_lens[b]) + 1 + aa, &u_acc, &u_smp);
    const double t = u_smp * total;

    // slice level
    int ws = -1, last_pos = -1;
    bool exact = true;
    double run = 0.0;
    {
        double carry = 0.0;
        for (int base = 0; base < a.W; base += kWave) {
            const double s = slice_weight(base + lane, sum_off);
            const double incl = wave_incl_scan(s);
            const double excl = wave_excl_from_incl(incl);
            const unsigned long long pos = __ballot(s > 0.0);
            if (pos) last_pos = base + 63 - __builtin_clzll(pos);
            const unsigned long long cross = __ballot(s > 0.0 && carry + incl > t);
            if (cross) {
                const int l0 = __ffsll(static_cast<long long>(cross)) - 1;
                ws = base + l0;
                run = carry + __shfl(excl, l0, kWave);
                break;
            }
            carry += __shfl(incl, kWave - 1, kWave);
        }
        if (ws < 0) { ws = last_pos < 0 ? 0 : last_pos; exact = false; }
    }
    const double scale = (mode == kModeBonus) ? exp((part[size_t(ws) * kSamplePart] - M) * a.invT64) : 1.0;
    // sub-chunk level (16 sums on lanes 0..15)
    int subc;
    {
        const double s = (lane < kSubPerSlice) ? part[size_t(ws) * kSamplePart + sub_off + lane] * scale : 0.0;
        const double incl = wave_incl_scan(s);
        const double excl = wave_excl_from_incl(incl);
        const unsigned long long pos = __ballot(s > 0.0);
        const unsigned long long cross = exact ? __ballot(s > 0.0 && run + incl > t) : 0ull;
        if (cross) {
            subc = __ffsll(static_cast<long long>(cross)) - 1;
            run = run + __shfl(excl, subc, kWave);
        } else {
            subc = pos ? 63 - __builtin_clzll(pos) : 0;
            exact = false;
        }
    }
    // logit level: the 256 logits of the crossing sub-chunk, 4 per lane
    const int i_row = subc / kWavesRT, i_wave = subc % kWavesRT;
    const int sub_base = ws * kSlice + i_row * (kRT * 4) + i_wave * kSub;
    const int x0 = sub_base + lane * 4;
    float zp4[4], zq4[4];
    load_sub<kVec4>(prow, a.V, x0, zp4);
    double wt[4];
    if (mode == kModeResidual) {
        load_sub<kVec4>(qrow, a.V, x0, zq4);
        ResidualCtx c;
        c.mp = static_cast<float>(rec.Mp);
        c.mq = static_cast<float>(rec.Mq);
        c.invZp = 1.0 / rec.Zp;
        c.invZq = 1.0 / rec.Zq;
        double r[4], ep[4];
        residual_weights(zp4, zq4, c, a.invT, a.invT64, r, ep);
#pragma unroll
        for (int e = 0; e < 4; ++e) wt[e] = use_p ? ep[e] : r[e];
    } else {
        const float m = static_cast<float>(part[size_t(ws) * kSamplePart]);
        exps_mixed(zp4, m, a.invT, a.invT64, wt);
#pragma unroll
        for (int e = 0; e < 4; ++e) wt[e] *= scale;
    }
    double pre[4];
    pre[0] = wt[0];
    pre[1] = pre[0] + wt[1];
    pre[2] = pre[1] + wt[2];
    pre[3] = pre[2] + wt[3];
    const double incl = wave_incl_scan(pre[3]);
    const double excl = wave_excl_from_incl(incl);
    int hit = 4, lastc = -1;
#pragma unroll
    for (int e = 3; e >= 0; --e)
        if (exact && wt[e] > 0.0 && (run + excl) + pre[e] > t) hit = e;
#pragma unroll
    for (int e = 0; e < 4; ++e) if (wt[e] > 0.0) lastc = e;
    const unsigned long long mhit = __ballot(hit < 4);
    int y;
    if (mhit) {
        const int l0 = __ffsll(static_cast<long long>(mhit)) - 1;
        y = sub_base + l0 * 4 + __shfl(hit, l0, kWave);
    } else {
        const unsigned long long mpos = __ballot(lastc >= 0);
        const int l1 = mpos ? (63 - __builtin_clzll(mpos)) : 0;
        const int c1 = __shfl(lastc, l1, kWave);
        y = sub_base + l1 * 4 + (c1 < 0 ? 0 : c1);
    }
    if (lane != 0) return;
    if (y >= a.V) y = a.V - 1;   // only reachable when every weight is zero

    double py;
    if (mode == kModeBonus) py = exp((static_cast<double>(prow[y]) - M) * a.invT64) / total;
    else py = exp((static_cast<double>(prow[y]) - rec.Mp) * a.invT64) / rec.Zp;
    const size_t ob = size_t(b) * (a.k + 1);
    a.out_tokens[ob + aa] = y;
    if (a.out_probs) a.out_probs[ob + aa] = static_cast<float>(py);
    for (int i = aa + 1; i <= a.k; ++i) {
        a.out_tokens[ob + i] = -1;
        if (a.out_probs) a.out_probs[ob + i] = 0.0f;
    }
    if (a.accept_probs)
        for (int i = aa + 1; i < a.k; ++i) a.accept_probs[size_t(b) * a.k + i] = -1.0f;
    a.num_accepted[b] = aa;
}

}  // namespace

size_t reject_workspace_bytes(int B, int k, int V) {
    const int W = (V + kSlice - 1) / kSlice;
    return reject_layout(B, k, W).total;
}

hipError_t launch_reject(const RejectLaunch& p, hipStream_t stream) {
    const int W = (p.V + kSlice - 1) / kSlice;
    const RejectLayout lay = reject_layout(p.B, p.k, W);
    char* ws = static_cast<char*>(p.workspace);
    RejectArgs a;
    a.target = p.target_logits;
    a.draft = p.draft_logits;
    a.draft_tokens = p.draft_tokens;
    a.seq_ids = p.seq_ids;
    a.seq_lens = p.seq_lens;
    a.out_tokens = p.out_tokens;
    a.num_accepted = p.num_accepted;
    a.out_probs = p.out_probs;
    a.accept_probs = p.accept_probs;
    a.active = reinterpret_cast<int32_t*>(ws + lay.active);
    a.final_rec = reinterpret_cast<FinalRecord*>(ws + lay.final_rec);
    a.chain_part = reinterpret_cast<double*>(ws + lay.chain_part);
    a.sample_part = reinterpret_cast<double*>(ws + lay.sample_part);
    a.B = p.B; a.k = p.k; a.V = p.V; a.W = W;
    a.invT = 1.0f / p.temperature;
    a.invT64 = 1.0 / static_cast<double>(p.temperature);
    a.seed = p.seed;
    const dim3 grid(W, p.B), block(kRT);
    const bool vec4 = (p.V % 4) == 0;
    for (int j = 0; j <= p.k; ++j) {
        if (vec4) hipLaunchKernelGGL(reject_level_kernel<true>, grid, block, 0, stream, a, j);
        else hipLaunchKernelGGL(reject_level_kernel<false>, grid, block, 0, stream, a, j);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (vec4) hipLaunchKernelGGL(reject_finalize_kernel<true>, dim3(p.B), dim3(kWave), 0, stream, a);
    else hipLaunchKernelGGL(reject_finalize_kernel<false>, dim3(p.B), dim3(kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace specverify
