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
//  * The vocab of a row is cut into slices of kSlice = 4096 logits; a grid of
//    (W slices) x (B sequences) workgroups of 256 threads covers one level of the
//    chain for the whole batch, so even B = 64 puts 2048 workgroups on 256 CUs.
//    Each thread holds 16 logits per row in registers (four 16-byte loads).
//  * Level j (one launch per j < k) reads only rows p_j, q_j of sequences still
//    in the chain; a workgroup writes its slice partial (max, sum of exps) and
//    bumps a per-sequence counter with agent-scope acquire/release. The workgroup
//    that arrives last combines the partials in slice order (deterministic),
//    takes the acceptance decision and records the next level. Nothing waits.
//  * The sampling launch re-reads exactly one row pair (or the bonus row) per
//    sequence, computes fp64 sub-chunk sums of the sampling weights; the last
//    workgroup locates the crossing slice, then sub-chunk (256 logits), and
//    rescans that one sub-chunk with a wavefront prefix scan.
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
constexpr int kLevelSample = 1 << 20;

struct SeqState {
    int next_level;
    int mode;
    int a;
    int pad;
    double Mp, Zp, Mq, Zq;   // normalisers of the rejected pair: logits max and sum of exps
};

constexpr int kChainPart = 4;                         // m_p, Z_p, m_q, Z_q
constexpr int kSamplePart = 2 + 2 * kSubPerSlice + 2; // m_w, R_w, S_r[16], P_w, S_p[16], pad

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
    unsigned* cnt_chain;
    unsigned* cnt_sample;
    SeqState* state;
    double* chain_part;
    double* sample_part;
    int B, k, V, W;
    float invT;
    double invT64;
    uint64_t seed;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct RejectLayout {
    size_t cnt_chain, cnt_sample, state, chain_part, sample_part, total;
};

RejectLayout reject_layout(int B, int W) {
    RejectLayout L;
    size_t o = 0;
    L.cnt_chain = o;   o = align256(o + sizeof(unsigned) * B);
    L.cnt_sample = o;  o = align256(o + sizeof(unsigned) * B);
    L.state = o;       o = align256(o + sizeof(SeqState) * B);
    L.chain_part = o;  o = align256(o + sizeof(double) * size_t(B) * W * kChainPart);
    L.sample_part = o; o = align256(o + sizeof(double) * size_t(B) * W * kSamplePart);
    L.total = o;
    return L;
}

// Slice element e of this thread: e = i*1024 + tid*4 + c (i, c in 0..3), so each
// (i, wave) pair is a contiguous run of 256 logits: the sub-chunk i*4 + wave.
template <bool kVec4>
__device__ __forceinline__ void load_slice(const float* row, int V, int w, float (&v)[kEPT]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int x0 = w * kSlice + i * (kRT * 4) + tid * 4;
        if (kVec4 && x0 + 3 < V) {
            const float4 f = *reinterpret_cast<const float4*>(row + x0);
            v[4 * i + 0] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) v[4 * i + c] = (x0 + c < V) ? row[x0 + c] : -INFINITY;
        }
    }
}

template <bool kVec4>
__device__ __forceinline__ void load_sub(const float* row, int V, int x0, float (&v)[4]) {
    if (kVec4 && x0 + 3 < V) {
        const float4 f = *reinterpret_cast<const float4*>(row + x0);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (x0 + c < V) ? row[x0 + c] : -INFINITY;
    }
}

// e^{(z - m)/T} in fp64 (exact exp) for one logit.
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
// (M, Z) with wave 0: lanes take slices, butterflies reduce in a fixed order.
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
    z = wave_sum(z);
    *M_out = m;
    *Z_out = z;
}

// ---------------------------------------------------------------------------- chain level j

template <bool kVec4>
__global__ __launch_bounds__(kRT) void reject_chain_kernel(RejectArgs a, int j) {
    __shared__ float red_f[kWavesRT];
    __shared__ double red_d[kWavesRT];
    __shared__ int s_last;
    const int w = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    if (j > 0 && a.state[b].next_level != j) return;

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
    // A slice that is entirely -inf (only possible past V, never for a whole slice) contributes 0.
    const double zp = block_sum(mp == -INFINITY ? 0.0 : sum_exps_mixed(vp, mp, a.invT, a.invT64), red_d);
    const double zq = block_sum(mq == -INFINITY ? 0.0 : sum_exps_mixed(vq, mq, a.invT, a.invT64), red_d);

    if (tid == 0) {
        double* part = a.chain_part + (size_t(b) * a.W + w) * kChainPart;
        part[0] = mp; part[1] = zp; part[2] = mq; part[3] = zq;
        s_last = (arrive_acq_rel(a.cnt_chain + b) == unsigned(a.W - 1));
    }
    __syncthreads();
    if (!s_last) return;
    fence_acquire_agent();
    if (tid >= kWave) return;

    // ---- last workgroup of this sequence: wave 0 combines and decides.
    const double* part = a.chain_part + size_t(b) * a.W * kChainPart;
    double Mp, Zp, Mq, Zq;
    combine_row(part, kChainPart, 0, a.W, a.invT64, &Mp, &Zp);
    combine_row(part, kChainPart, 2, a.W, a.invT64, &Mq, &Zq);
    if (tid != 0) return;

    const int d = a.draft_tokens[size_t(b) * a.k + j];
    const bool d_ok = d >= 0 && d < a.V;   // out-of-range ids (a broken precondition) are rejected
    const double p_d = d_ok ? exp((static_cast<double>(prow[d]) - Mp) * a.invT64) / Zp : 0.0;
    const double q_d = d_ok ? exp((static_cast<double>(qrow[d]) - Mq) * a.invT64) / Zq : 0.0;
    const double ratio = (q_d > 0.0) ? p_d / q_d : (p_d > 0.0 ? INFINITY : 0.0);
    const int L = a.seq_lens[b];
    double u_acc, u_smp;
    verify_uniforms(a.seed, a.seq_ids[b], int64_t(L) + 1 + j, &u_acc, &u_smp);
    if (a.accept_probs) a.accept_probs[size_t(b) * a.k + j] = static_cast<float>(fmin(1.0, ratio));

    SeqState* st = a.state + b;
    if (u_acc < ratio) {
        a.out_tokens[size_t(b) * (a.k + 1) + j] = d;
        if (a.out_probs) a.out_probs[size_t(b) * (a.k + 1) + j] = static_cast<float>(p_d);
        if (j + 1 < a.k) {
            st->next_level = j + 1;
        } else {
            st->next_level = kLevelSample;
            st->mode = kModeBonus;
            st->a = a.k;
        }
    } else {
        st->next_level = kLevelSample;
        st->mode = kModeResidual;
        st->a = j;
        st->Mp = Mp; st->Zp = Zp; st->Mq = Mq; st->Zq = Zq;
    }
    counter_reset(a.cnt_chain + b);
}

// ---------------------------------------------------------------------------- sampling level

// Sampling weights of 4 consecutive logits (kind: 0 residual, 1 bonus, 2 p-fallback).
struct WeightCtx {
    int mode;
    float mp_f, mq_f;    // reference maxima (float) for the mixed-precision exps
    double invZp, invZq; // residual normalisers
};

template <int N>
__device__ __forceinline__ void residual_weights(const float (&zp)[N], const float (&zq)[N], const WeightCtx& c,
                                                 float invT, double invT64, double (&r)[N], double (&ep)[N]) {
    double eq[N];
    exps_mixed(zp, c.mp_f, invT, invT64, ep);
    exps_mixed(zq, c.mq_f, invT, invT64, eq);
#pragma unroll
    for (int e = 0; e < N; ++e) r[e] = fmax(0.0, ep[e] * c.invZp - eq[e] * c.invZq);
}

template <bool kVec4>
__global__ __launch_bounds__(kRT) void reject_sample_kernel(RejectArgs a) {
    __shared__ float red_f[kWavesRT];
    __shared__ double s_sub[2][kSubPerSlice];
    __shared__ int s_last;
    const int w = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const SeqState st = a.state[b];
    const int mode = st.mode;
    const int aa = st.a;

    const float* prow = a.target + (size_t(b) * (a.k + 1) + aa) * a.V;
    const float* qrow = a.draft + (size_t(b) * a.k + (aa < a.k ? aa : 0)) * a.V;
    float vp[kEPT], vq[kEPT];
    load_slice<kVec4>(prow, a.V, w, vp);
    WeightCtx c;
    c.mode = mode;
    double mw = 0.0;
    double sr[4], sp[4];
    if (mode == kModeResidual) {
        load_slice<kVec4>(qrow, a.V, w, vq);
        c.mp_f = static_cast<float>(st.Mp);
        c.mq_f = static_cast<float>(st.Mq);
        c.invZp = 1.0 / st.Zp;
        c.invZq = 1.0 / st.Zq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float zp4[4], zq4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) { zp4[e] = vp[4 * i + e]; zq4[e] = vq[4 * i + e]; }
            double r[4], ep[4];
            residual_weights(zp4, zq4, c, a.invT, a.invT64, r, ep);
            sr[i] = ((r[0] + r[1]) + r[2]) + r[3];
            sp[i] = ((ep[0] + ep[1]) + ep[2]) + ep[3];
        }
    } else {
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
            double ex[4];
            if (m == -INFINITY) { ex[0] = ex[1] = ex[2] = ex[3] = 0.0; }
            else exps_mixed(z4, m, a.invT, a.invT64, ex);
            sr[i] = ((ex[0] + ex[1]) + ex[2]) + ex[3];
            sp[i] = 0.0;
        }
    }
    // Sub-chunk sums: sub-chunk (i, wave) = logits [i*1024 + wave*256, +256) of the slice.
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
            part[2 + s] = s_sub[0][s];
            part[2 + kSubPerSlice + 1 + s] = s_sub[1][s];
            R += s_sub[0][s];
            P += s_sub[1][s];
        }
        part[0] = mw;
        part[1] = R;
        part[2 + kSubPerSlice] = P;
        s_last = (arrive_acq_rel(a.cnt_sample + b) == unsigned(a.W - 1));
    }
    __syncthreads();
    if (!s_last) return;
    fence_acquire_agent();
    if (wave != 0) return;

    // ---- last workgroup: wave 0 locates the sample. Slices, then sub-chunks, then
    // logits are searched with wavefront prefix scans in a fixed order; at each level
    // the crossing is the first positive weight whose running sum exceeds t. If
    // rounding leaves no crossing, the last positive weight is taken (which, at the
    // slice level, is the largest token with positive weight).
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
    double total = row_total(1);
    if (mode == kModeResidual && !(total > 0.0)) {   // zero residual: sample p_j instead
        use_p = 1;
        total = row_total(2 + kSubPerSlice);
    }
    const int sum_off = use_p ? (2 + kSubPerSlice) : 1;
    const int sub_off = sum_off + 1;
    double u_acc, u_smp;
    verify_uniforms(a.seed, a.seq_ids[b], int64_t(a.seq_lens[b]) + 1 + aa, &u_acc, &u_smp);
    const double t = u_smp * total;

    // slice level
    int ws = -1, last_pos = -1;
    bool exact = true;          // false: no crossing found, take last positive below
    double run = 0.0;           // running sum before the chosen slice
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
    const double scale = (mode == kModeBonus)
        ? exp((part[size_t(ws) * kSamplePart] - M) * a.invT64) : 1.0;
    // sub-chunk level (16 sums, lanes 0..15)
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
    // logit level: rescan the 256 logits of the crossing sub-chunk (4 per lane)
    const int i_row = subc / kWavesRT, i_wave = subc % kWavesRT;
    const int sub_base = ws * kSlice + i_row * (kRT * 4) + i_wave * kSub;
    const int x0 = sub_base + lane * 4;
    float zp4[4], zq4[4];
    load_sub<kVec4>(prow, a.V, x0, zp4);
    double wt[4];
    if (mode == kModeResidual) {
        load_sub<kVec4>(qrow, a.V, x0, zq4);
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
    for (int e = 3; e >= 0; --e) {
        if (exact && wt[e] > 0.0 && (run + excl) + pre[e] > t) hit = e;
    }
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
    else py = exp((static_cast<double>(prow[y]) - st.Mp) * a.invT64) / st.Zp;
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
    counter_reset(a.cnt_sample + b);
}

}  // namespace

size_t reject_workspace_bytes(int B, int k, int V) {
    (void)k;
    const int W = (V + kSlice - 1) / kSlice;
    return reject_layout(B, W).total;
}

hipError_t launch_reject(const RejectLaunch& p, hipStream_t stream) {
    const int W = (p.V + kSlice - 1) / kSlice;
    const RejectLayout lay = reject_layout(p.B, W);
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
    a.cnt_chain = reinterpret_cast<unsigned*>(ws + lay.cnt_chain);
    a.cnt_sample = reinterpret_cast<unsigned*>(ws + lay.cnt_sample);
    a.state = reinterpret_cast<SeqState*>(ws + lay.state);
    a.chain_part = reinterpret_cast<double*>(ws + lay.chain_part);
    a.sample_part = reinterpret_cast<double*>(ws + lay.sample_part);
    a.B = p.B; a.k = p.k; a.V = p.V; a.W = W;
    a.invT = 1.0f / p.temperature;
    a.invT64 = 1.0 / static_cast<double>(p.temperature);
    a.seed = p.seed;
    const dim3 grid(W, p.B), block(kRT);
    const bool vec4 = (p.V % 4) == 0;
    for (int j = 0; j < p.k; ++j) {
        if (vec4) hipLaunchKernelGGL(reject_chain_kernel<true>, grid, block, 0, stream, a, j);
        else hipLaunchKernelGGL(reject_chain_kernel<false>, grid, block, 0, stream, a, j);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (vec4) hipLaunchKernelGGL(reject_sample_kernel<true>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(reject_sample_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace specverify
