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
// How (one MI355X, one launch for the whole batch):
//  * A row of V logits is cut into units of 4096; each unit of the current row
//    (pair) is held in the registers of one wavefront (16 x 16-byte loads per
//    lane per row, all in flight together). Eight unit wavefronts form a
//    512-thread workgroup (one per CU); the Q = ceil(U / 8) workgroups of a
//    sequence form a group, and groups take sequences in turn.
//  * Level j: every wavefront reduces its units of p_j and q_j to (max, sum of
//    exps) with an online softmax on the DPP network; wave 0 of the workgroup
//    combines the eight through LDS and publishes the workgroup's pair; then it
//    gathers the Q pairs of the group, combines them in a fixed order and takes
//    the acceptance test. Every workgroup computes the same decision from the
//    same published bits, so one cross-CU exchange per level suffices.
//  * Exchange is fence-free: each published 32-bit value travels in a 64-bit
//    atomic slot together with the call's epoch, so a slot is either stale (old
//    epoch, keep polling) or complete. No cache write-back or invalidation is
//    needed and the workspace never has to be cleared between calls.
//  * On the first rejection (or after k acceptances, on row p_k) the rows still
//    in registers are turned into sampling weights: nothing is read twice. Unit
//    sums go through LDS to the workgroup leader, one exchange gives every
//    leader the workgroup totals, the leaders find the crossing workgroup, and
//    that workgroup's leader finds the crossing unit, whose wavefront scans its
//    per-load sums in LDS for the token.
//  * Precision: the chain statistics use fp32 exps (relative error ~1e-7, ample
//    for an acceptance test). The sampling pass takes logits whose probability
//    exceeds 2^-14 in fp64 and the rest with an error-compensated fp32 exp,
//    accumulating in fp64, so the sampling CDF is within ~1e-9 of an fp64 one.
//  * Co-residency of a group is required: the grid is sized to what the device
//    holds at once, and every wait is bounded so that a wavefront always
//    terminates (a timed-out sequence reports num_accepted = -1).
#include "common.hpp"
#include "fastexp.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace specverify {
namespace {

constexpr int kVecs = 16;                  // 16-byte loads per lane per row
constexpr int kUnit = kWave * kVecs * 4;   // 4096 logits: one wavefront's share of a row
constexpr int kStep = 4;                   // loads per online-softmax step (16 logits per lane)
constexpr int kStatSlots = 6;              // M_p, M_q, Z_p (hi, lo), Z_q (hi, lo)
constexpr int kSampSlots = 8;              // A, B, P, Q (hi, lo each); bonus row: weight sum, max
constexpr int kUnitWaves = 8;              // unit wavefronts per workgroup
constexpr int kRT = kUnitWaves * kWave;    // 512 threads
constexpr int kMaxQ = 32;                  // workgroups per sequence: U <= 256, i.e. V <= 2^20
constexpr float kLnTau = -9.70406052783923f;  // ln 2^-14: logits above this probability share use fp64
constexpr unsigned kSpinLimit = 1u << 20;

enum : unsigned { kCtlEpoch = 0, kCtlDone = 1, kCtlError = 2 };

typedef float f4 __attribute__((ext_vector_type(4)));

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
    unsigned* ctl;                     // epoch of the last finished call, finished-wave count, error flag
    unsigned long long* stat_slots;    // [B][k+1][kStatSlots][Q]: workgroup statistics per level
    unsigned long long* samp_slots;    // [B][kSampSlots][Q]: workgroup sampling sums
    int B, k, V, U, Q, groups;
    float invT;                        // 1 / T
    float c2;                          // log2(e) / T
    double invT64;
    uint64_t seed;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct RejectLayout {
    size_t ctl, stat, samp, total;
};

RejectLayout reject_layout(int B, int k, int Q) {
    RejectLayout L;
    size_t o = 0;
    L.ctl = o;  o = align256(o + 4 * sizeof(unsigned));
    L.stat = o; o = align256(o + sizeof(unsigned long long) * size_t(B) * (k + 1) * Q * kStatSlots);
    L.samp = o; o = align256(o + sizeof(unsigned long long) * size_t(B) * Q * kSampSlots);
    L.total = o;
    return L;
}

// ---------------------------------------------------------------- slots

__device__ __forceinline__ void slot_store(unsigned long long* p, unsigned payload, unsigned epoch) {
    const unsigned long long v = (static_cast<unsigned long long>(payload) << 32) | epoch;
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long slot_load(unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned hi32(double d) {
    return static_cast<unsigned>(__builtin_bit_cast(unsigned long long, d) >> 32);
}
__device__ __forceinline__ unsigned lo32(double d) {
    return static_cast<unsigned>(__builtin_bit_cast(unsigned long long, d));
}
__device__ __forceinline__ double join64(unsigned hi, unsigned lo) {
    return __builtin_bit_cast(double, (static_cast<unsigned long long>(hi) << 32) | lo);
}

// Lane 0 publishes the N payloads (N back-to-back single-lane stores) to
// slots[s * stride], s = 0 .. N-1.
template <int N>
__device__ __forceinline__ void publish(unsigned long long* slots, const unsigned (&payload)[N], unsigned epoch,
                                        int stride = 1) {
    if (lane_id() == 0) {
#pragma unroll
        for (int s = 0; s < N; ++s) slot_store(slots + size_t(s) * stride, payload[s], epoch);
    }
}

// Waits until the N slots of each of the Q workgroups carry `epoch` and returns
// their payloads: lane l gets workgroup l (lanes >= Q read zero). Slot s of
// workgroup l is slots[s * Q + l], so each read instruction covers consecutive
// words. Returns false if the bounded wait ran out (only possible if the group
// were not resident at once).
template <int N>
__device__ __forceinline__ bool gather(unsigned long long* slots, int Q, unsigned epoch, unsigned (&out)[N]) {
    const int lane = lane_id();
    for (unsigned it = 0; it < kSpinLimit; ++it) {
        bool ok = true;
#pragma unroll
        for (int s = 0; s < N; ++s) {
            unsigned long long v = 0;
            if (lane < Q) {
                v = slot_load(slots + size_t(s) * Q + lane);
                ok = ok && static_cast<unsigned>(v) == epoch;
            }
            out[s] = static_cast<unsigned>(v >> 32);
        }
        if (__all(ok)) return true;
        __builtin_amdgcn_s_sleep(4);
    }
    return false;
}

// Values that are equal in every lane (read by all lanes from one address, or
// derived from wavefront reductions) made provably uniform, so that control flow
// depending on them stays scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ int64_t uniform(int64_t v) {
    const int lo = __builtin_amdgcn_readfirstlane(static_cast<int>(v & 0xFFFFFFFFll));
    const int hi = __builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(static_cast<unsigned>(hi)) << 32) | static_cast<unsigned>(lo));
}
__device__ __forceinline__ double uniform(double v) {
    return __builtin_bit_cast(double, uniform(__builtin_bit_cast(int64_t, v)));
}

// ---------------------------------------------------------------- loads

// Four consecutive logits from x (x a multiple of 4 when kVec4), -inf past the
// row. Lanes past the row issue no load (loads of one clamped address from many
// lanes and waves serialise in the memory pipeline).
template <bool kVec4>
__device__ __forceinline__ f4 load4(const float* row, int V, int x) {
    f4 f = f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (kVec4) {
        if (x < V) f = __builtin_nontemporal_load(reinterpret_cast<const f4*>(row + x));
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (x + c < V) f[c] = __builtin_nontemporal_load(row + x + c);
    }
    return f;
}

// Element (i, c) of lane l in unit u is logit u*4096 + i*256 + 4*l + c: each load
// of a wavefront is one contiguous 1 KB run. p and q loads are interleaved so the
// online softmax can start on the first step while the rest are in flight. Only
// the last unit of a row can reach past V; the others load without bounds tests.
template <bool kVec4, bool kTwo>
__device__ __forceinline__ void load_unit(const float* prow, const float* qrow, int V, int u,
                                          f4 (&xp)[kVecs], f4 (&xq)[kVecs]) {
    const int base = u * kUnit + lane_id() * 4;
    if (kVec4 && (u + 1) * kUnit <= V) {
#pragma unroll
        for (int i = 0; i < kVecs; ++i) {
            xp[i] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(prow + base + i * (kWave * 4)));
            if (kTwo) xq[i] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(qrow + base + i * (kWave * 4)));
        }
    } else {
#pragma unroll
        for (int i = 0; i < kVecs; ++i) {
            xp[i] = load4<kVec4>(prow, V, base + i * (kWave * 4));
            if (kTwo) xq[i] = load4<kVec4>(qrow, V, base + i * (kWave * 4));
        }
    }
}

// ---------------------------------------------------------------- chain statistics

// One online-softmax step over loads 4s..4s+3 of this lane: running max m and
// running sum s of e^{(x - m)/T}, the exps as hardware exp2 of (x - m) * log2(e)/T.
__device__ __forceinline__ void online_step(const f4 (&x)[kVecs], int s, float c2, float& m, double& acc) {
    float gm = -INFINITY;
#pragma unroll
    for (int i = kStep * s; i < kStep * s + kStep; ++i)
        gm = fmaxf(gm, fmaxf(fmaxf(x[i].x, x[i].y), fmaxf(x[i].z, x[i].w)));
    const float mn = fmaxf(m, gm);
    const float ref = (mn == -INFINITY) ? 0.0f : mn;   // all -inf so far: every term is 0
    const float rescale = __builtin_amdgcn_exp2f((m - ref) * c2);
    float part[kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
        const f4 v = x[kStep * s + i];
        const float e0 = __builtin_amdgcn_exp2f((v.x - ref) * c2);
        const float e1 = __builtin_amdgcn_exp2f((v.y - ref) * c2);
        const float e2 = __builtin_amdgcn_exp2f((v.z - ref) * c2);
        const float e3 = __builtin_amdgcn_exp2f((v.w - ref) * c2);
        part[i] = (e0 + e1) + (e2 + e3);
    }
    const float sum = (part[0] + part[1]) + (part[2] + part[3]);
    acc = acc * static_cast<double>(rescale) + static_cast<double>(sum);
    m = mn;
}

struct RowStats {
    float Mp, Mq;     // row maxima (logits)
    double Zp, Zq;    // sum of e^{(z - M)/T} over the row
};

// Combines per-lane partials (M_i, Z_i), lanes without one holding (-inf, 0),
// into (M, Z) of their union, identically in every wavefront that holds the same
// partials in the same lanes.
__device__ __forceinline__ void combine_pair(float m, double z, double invT64, float& M, double& Z) {
    M = dpp_wave_max(m);
    Z = dpp_wave_sum((z > 0.0) ? z * exp_nonpos_f64((static_cast<double>(m) - M) * invT64) : 0.0);
}

// ---------------------------------------------------------------- sampling weights

struct SampleCtx {
    float Mp, Mq, invT;
    float hp, hq;        // ln(tau * Z): log-weights above these are taken in fp64
    float dn;            // ln Z_p - ln Z_q: x in the residual support iff lp - lq > dn
    double Mp64, Mq64, invT64;
};

// Log-weight of a logit in nats, (z - M) / T, and the residual-support test. The
// operations are written with the no-contraction intrinsics so that every call
// site rounds identically (the support must be the same set wherever it is judged).
__device__ __forceinline__ float log_weight(float z, float M, float invT) { return __fmul_rn(__fsub_rn(z, M), invT); }
__device__ __forceinline__ bool in_support(float xp, float xq, float dn) { return __fsub_rn(xp, xq) > dn; }

// Light part of the unnormalised weights a = e^{(z_p - M_p)/T}, b = e^{(z_q - M_q)/T}
// of the four logits of one load: compensated fp32 exps, zeroed (by a product, so
// the exp is never moved into a branch) for heavy logits, whose probability under
// the chain's normalisers exceeds tau. Their bits are set in `hmask` (bit 4*i + e)
// and they are taken in fp64 by heavy_pass. Membership of the residual support
// {p > q} is judged with the chain's normalisers.
__device__ __forceinline__ void light_weights(bool residual, const f4& vp, const f4& vq, const SampleCtx& c, int i,
                                              float (&la)[4], float (&lb)[4], bool (&in_s)[4],
                                              unsigned long long& hmask) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float xp = log_weight(vp[e], c.Mp, c.invT);
        const float xq = residual ? log_weight(vq[e], c.Mq, c.invT) : -INFINITY;
        const bool h = (xp > c.hp) || (xq > c.hq);   // xq = -inf never passes
        in_s[e] = residual ? in_support(xp, xq, c.dn) : true;   // NaN for padding: not in the support
        const float keep = h ? 0.0f : 1.0f;
        la[e] = exp_small_f32(xp) * keep;
        lb[e] = residual ? exp_small_f32(xq) * keep : 0.0f;
        hmask |= static_cast<unsigned long long>(h) << (4 * i + e);
    }
}

// fp64 weights of this lane's heavy logits. They are re-read from memory (four
// per lane per round trip; there are few, typically 0..4 per lane) rather than
// picked out of the register arrays, which would need dynamic indexing and
// force the arrays out of registers. `f` receives (load index, a, b, in support)
// for each; the trip count is the largest per-lane count in the wavefront.
template <bool kVec4, typename F>
__device__ __forceinline__ void heavy_pass(bool residual, const float* prow, const float* qrow, int base,
                                           const SampleCtx& c, unsigned long long hmask, F&& f) {
    while (__any(hmask != 0ull)) {
        int idx[4];
        bool has[4];
        float zp[4], zq[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            has[r] = hmask != 0ull;
            idx[r] = has[r] ? __builtin_ctzll(hmask) : 0;
            hmask &= has[r] ? hmask - 1 : hmask;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // heavy logits are never padding (-inf), so x < V; lanes without one read logit 0
            const int x = has[r] ? base + (idx[r] >> 2) * (kWave * 4) + (idx[r] & 3) : 0;
            zp[r] = prow[x];
            zq[r] = residual ? qrow[x] : -INFINITY;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const double va = exp_nonpos_f64((static_cast<double>(zp[r]) - c.Mp64) * c.invT64);
            const double vb = residual ? exp_nonpos_f64((static_cast<double>(zq[r]) - c.Mq64) * c.invT64) : 0.0;
            const bool ins = residual
                ? in_support(log_weight(zp[r], c.Mp, c.invT), log_weight(zq[r], c.Mq, c.invT), c.dn) : true;
            if (has[r]) f(idx[r] >> 2, va, vb, ins);
        }
    }
}

struct UnitSums {
    double A, B, P, Q;   // sums over the support of a, b; sums over all logits of a, b
};

// Per-lane sums of a and b over the support for each of the lane's sixteen loads,
// kept in LDS ([load][lane], 16 KB per wavefront) for the final scan. For the
// bonus row only the a-sums are meaningful.
typedef double2 LoadSums[kVecs][kWave];

// Unit sums of the sampling weights and, in `ls`, the per-load sums.
template <bool kVec4, bool kResidual>
__device__ __forceinline__ UnitSums unit_sums(const f4 (&xp)[kVecs], const f4 (&xq)[kVecs], const SampleCtx& c,
                                              const float* prow, const float* qrow, int base, LoadSums& ls) {
    const int lane = lane_id();
    double A = 0.0, Bs = 0.0, P = 0.0, Q = 0.0;
    unsigned long long hmask = 0ull;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        float la[4], lb[4];
        bool in_s[4];
        light_weights(kResidual, xp[i], xq[i], c, i, la, lb, in_s, hmask);
        float fa = 0.0f, fb = 0.0f, fp = 0.0f, fq = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            fp += la[e];
            fa += in_s[e] ? la[e] : 0.0f;
            if (kResidual) {
                fq += lb[e];
                fb += in_s[e] ? lb[e] : 0.0f;
            }
        }
        A += static_cast<double>(fa);
        P += static_cast<double>(fp);
        if (kResidual) {
            Bs += static_cast<double>(fb);
            Q += static_cast<double>(fq);
        }
        ls[i][lane] = make_double2(fa, fb);
    }
    heavy_pass<kVec4>(kResidual, prow, qrow, base, c, hmask, [&](int i, double va, double vb, bool ins) {
        P += va;
        A += ins ? va : 0.0;
        double2 g = ls[i][lane];
        g.x += ins ? va : 0.0;
        if (kResidual) {
            Q += vb;
            Bs += ins ? vb : 0.0;
            g.y += ins ? vb : 0.0;
        }
        ls[i][lane] = g;
    });
    UnitSums s;
    s.A = dpp_wave_sum(A);
    s.P = dpp_wave_sum(P);
    s.B = kResidual ? dpp_wave_sum(Bs) : 0.0;
    s.Q = kResidual ? dpp_wave_sum(Q) : 0.0;
    return s;
}

// Sampling weight of one logit from its unnormalised a, b: the residual
// max(0, a/Z_p - b/Z_q) on the support, else a itself (p_j, or the bonus row).
__device__ __forceinline__ double sample_weight(bool residual, bool in_s, double a, double b, double invZp,
                                                double invZq) {
    if (!residual) return a;
    return in_s ? fmax(0.0, a * invZp - b * invZq) : 0.0;
}

// Weights of the four logits of one load, fp64 for the heavy ones.
__device__ __forceinline__ void load_weights(bool two_rows, bool residual, const f4& vp, const f4& vq,
                                             const SampleCtx& c, double invZp, double invZq, double (&w)[4]) {
    float la[4], lb[4];
    bool in_s[4];
    unsigned long long hm = 0ull;
    light_weights(two_rows, vp, vq, c, 0, la, lb, in_s, hm);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool heavy = (hm >> e) & 1ull;
        const double va = heavy ? exp_nonpos_f64((static_cast<double>(vp[e]) - c.Mp64) * c.invT64) : la[e];
        const double vb = (heavy && two_rows) ? exp_nonpos_f64((static_cast<double>(vq[e]) - c.Mq64) * c.invT64)
                                              : lb[e];
        w[e] = sample_weight(residual, in_s[e], va, vb, invZp, invZq);
    }
}

// ---------------------------------------------------------------- per-sequence pieces

struct SeqCtx {
    int b;
    int u;                    // unit of this wavefront: q * kUnitWaves + wave
    int q;                    // workgroup of the group
    int wave;                 // wavefront of the workgroup
    unsigned epoch;
    const float* prow_base;   // target logits of the sequence, [k+1][V]
    const float* qrow_base;   // draft logits of the sequence, [k][V]
    int64_t sid;
    int32_t L;
};

// Draft token j and its target / draft logits (wave-uniform).
struct TokenLogits {
    int tok;
    bool ok;           // 0 <= tok < V (out-of-range ids, a broken precondition, are rejected)
    float zp, zq;
    double u_acc;      // the test's uniform, computed before the group's statistics arrive
};

// Workgroup-shared state: per-wavefront partials going to wave 0, and wave 0's
// results going back to all eight wavefronts.
struct UnitStat {
    float Mp, Mq;
    double Zp, Zq;
};
struct LevelRes {
    unsigned flags;
    float Mp, Mq;
    double Zp, Zq;
};
struct SampRes {
    int owner;         // wavefront holding the crossing unit, -1 if in another workgroup
    unsigned flags;    // kSampUseP, kSampExact, kSampError
    double run, t, Z1, Z2;
};
struct Shared {
    LoadSums ls[kUnitWaves];
    UnitStat unit[kUnitWaves];
    double4 usum[kUnitWaves];
    LevelRes res;
    SampRes samp;
};

enum : unsigned { kResAccepted = 1u, kResError = 2u };
enum : unsigned { kSampUseP = 1u, kSampExact = 2u, kSampError = 4u };

__device__ __forceinline__ void flag_error(const RejectArgs& a, const SeqCtx& s) {
    if (s.wave == 0 && lane_id() == 0) {
        __hip_atomic_fetch_or(a.ctl + kCtlError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.num_accepted[s.b] = -1;
    }
}

// The first group to see all its workgroups' first slots records it; the last
// of all groups stores this call's epoch for the next call. By then every
// wavefront of the grid has read the epoch (each workgroup publishes only after
// a barrier that follows its wavefronts' reads).
__device__ __forceinline__ void count_group(const RejectArgs& a, const SeqCtx& s, bool& counted) {
    if (counted) return;
    counted = true;
    if (lane_id() == 0) {
        const unsigned n = __hip_atomic_fetch_add(a.ctl + kCtlDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n + 1 == static_cast<unsigned>(a.groups)) {
            __hip_atomic_store(a.ctl + kCtlDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.ctl + kCtlEpoch, s.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The first lane with positive weight w whose running sum carry + (inclusive
// prefix of w) exceeds t, and the running sum before it. If rounding leaves no
// such lane, the last lane with positive weight (lane 0 if none) and exact = false.
__device__ __forceinline__ int find_crossing(double w, double carry, double t, double& run, bool& exact) {
    const double incl = dpp_wave_incl_scan(w);
    const double excl = dpp_wave_shr1(incl);
    const unsigned long long cross = __ballot(w > 0.0 && carry + incl > t);
    const unsigned long long pos = __ballot(w > 0.0);
    int l;
    if (cross) {
        l = __ffsll(static_cast<long long>(cross)) - 1;
        exact = true;
    } else {
        l = pos ? 63 - __builtin_clzll(pos) : 0;
        exact = false;
    }
    run = carry + __shfl(excl, l, kWave);
    return l;
}

// Draw from the weights of this unit (residual of row `row`; p_row when `use_p` or
// for the bonus row), given the running sum `run` before this unit and the
// target t. Only the wavefront owning the crossing unit calls this; lane 0 writes
// the token, its probability and the padding of the sequence's outputs.
template <bool kVec4>
__device__ __forceinline__ void final_scan(const RejectArgs& a, const SeqCtx& s, int row, bool two_rows,
                                           const float* prow, const float* qrow, const SampleCtx& c,
                                           const LoadSums& ls, bool use_p, bool exact, double run, double t,
                                           double invZp, double invZq, double Zp_true, double wscale,
                                           double M_ref) {
    // wscale maps this unit's weights onto the scale of run and t (1, except for
    // the bonus row, whose unit weights are relative to the unit's own maximum);
    // M_ref is the row maximum the emitted probability is taken against.
    const int lane = lane_id();
    const int base = s.u * kUnit + lane * 4;
    const bool residual = two_rows && !use_p;
    // load level (each load of a wavefront is 256 consecutive tokens)
    bool found = false;
    int istar = 0, ilast = -1;
    double run_i = run;
#pragma unroll 1
    for (int i = 0; i < kVecs; ++i) {
        double v;
        if (!use_p) {
            const double2 g = ls[i][lane];
            v = (residual ? g.x * invZp - g.y * invZq : g.x) * wscale;
        } else {                 // zero residual (rare): p-weights of this load, recomputed
            double w[4];
            const f4 vp = load4<kVec4>(prow, a.V, base + i * (kWave * 4));
            load_weights(false, false, vp, vp, c, invZp, invZq, w);
            v = ((w[0] + w[1]) + (w[2] + w[3])) * wscale;
        }
        const double Ti = dpp_wave_sum(v);
        if (Ti > 0.0) ilast = i;
        if (exact && !found && Ti > 0.0) {
            if (run_i + Ti > t) {
                found = true;
                istar = i;
            } else {
                run_i += Ti;
            }
        }
    }
    if (!found) {          // rounding left no crossing here: take the last positive weight
        exact = false;
        istar = ilast < 0 ? 0 : ilast;
    }
    double w[4];
    const f4 vp = load4<kVec4>(prow, a.V, base + istar * (kWave * 4));
    const f4 vq = two_rows ? load4<kVec4>(qrow, a.V, base + istar * (kWave * 4)) : vp;
    load_weights(two_rows, residual, vp, vq, c, invZp, invZq, w);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] *= wscale;
    const double lsum = (w[0] + w[1]) + (w[2] + w[3]);
    const double incl = dpp_wave_incl_scan(lsum);
    const double excl = dpp_wave_shr1(incl);
    int lstar, estar = -1;
    const unsigned long long cross = exact ? __ballot(lsum > 0.0 && run_i + incl > t) : 0ull;
    int elast = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) if (w[e] > 0.0) elast = e;
    if (cross) {
        lstar = __ffsll(static_cast<long long>(cross)) - 1;
        double r = run_i + excl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (w[e] > 0.0) {
                r += w[e];
                if (estar < 0 && r > t) estar = e;
            }
        }
        if (estar < 0) estar = elast;
    } else {
        const unsigned long long pos = __ballot(lsum > 0.0);
        lstar = pos ? 63 - __builtin_clzll(pos) : 0;
        estar = elast;
    }
    estar = __shfl(estar, lstar, kWave);
    if (lane != 0) return;
    if (estar < 0) estar = 0;
    int y = s.u * kUnit + istar * (kWave * 4) + lstar * 4 + estar;
    if (y >= a.V) y = a.V - 1;   // only reachable when every weight is zero
    const double py = exp_nonpos_f64((static_cast<double>(prow[y]) - M_ref) * c.invT64) / Zp_true;
    const int k = a.k, b = s.b;
    const size_t ob = size_t(b) * (k + 1);
    a.out_tokens[ob + row] = y;
    if (a.out_probs) a.out_probs[ob + row] = static_cast<float>(py);
    for (int i = row + 1; i <= k; ++i) {
        a.out_tokens[ob + i] = -1;
        if (a.out_probs) a.out_probs[ob + i] = 0.0f;
    }
    if (a.accept_probs)
        for (int i = row + 1; i < k; ++i) a.accept_probs[size_t(b) * k + i] = -1.0f;
    a.num_accepted[b] = row;
}

// Reads wave 0's sampling decision and runs the final scan in the owning
// wavefront (every wavefront of the workgroup calls this after the barrier).
__device__ __forceinline__ bool read_samp(const RejectArgs& a, const SeqCtx& s, const Shared& sh, bool& use_p,
                                          bool& exact, double& run, double& t, double& Z1, double& Z2) {
    const unsigned flags = static_cast<unsigned>(uniform(static_cast<int>(sh.samp.flags)));
    if (flags & kSampError) {
        flag_error(a, s);
        return false;
    }
    if (uniform(sh.samp.owner) != s.wave) return false;
    use_p = flags & kSampUseP;
    exact = flags & kSampExact;
    run = uniform(sh.samp.run);
    t = uniform(sh.samp.t);
    Z1 = uniform(sh.samp.Z1);
    Z2 = uniform(sh.samp.Z2);
    return true;
}

// Sampling from the residual of row `row` after its draft was rejected; `st`
// holds the chain statistics of that row. Each wavefront turns its unit (still in
// registers) into weights; wave 0 sums the workgroup's units, one exchange gives
// it every workgroup's sums, it finds the crossing workgroup and, if that is its
// own, the crossing unit, whose wavefront then scans it for the token.
template <bool kVec4>
__device__ __forceinline__ void sample_row(const RejectArgs& a, const SeqCtx& s, int row, const f4 (&xp)[kVecs],
                                           const f4 (&xq)[kVecs], const RowStats& st, Shared& sh) {
    const float* prow = s.prow_base + size_t(row) * a.V;
    const float* qrow = s.qrow_base + size_t(row) * a.V;
    SampleCtx c;
    c.Mp = st.Mp;
    c.Mq = st.Mq;
    c.invT = a.invT;
    c.Mp64 = st.Mp;
    c.Mq64 = st.Mq;
    c.invT64 = a.invT64;
    const double lzp = log(st.Zp), lzq = log(st.Zq);
    c.hp = static_cast<float>(kLnTau + lzp);
    c.hq = static_cast<float>(kLnTau + lzq);
    c.dn = static_cast<float>(lzp - lzq);

    const int lane = lane_id();
    const UnitSums us = unit_sums<kVec4, true>(xp, xq, c, prow, qrow, s.u * kUnit + lane * 4, sh.ls[s.wave]);
    if (lane == 0) sh.usum[s.wave] = make_double4(us.A, us.B, us.P, us.Q);
    __syncthreads();
    if (s.wave == 0) {
        double Au = 0.0, Bu = 0.0, Pu = 0.0, Qu = 0.0;
        if (lane < kUnitWaves) {
            const double4 v = sh.usum[lane];
            Au = v.x; Bu = v.y; Pu = v.z; Qu = v.w;
        }
        const double Aw = dpp_wave_sum(Au), Bw = dpp_wave_sum(Bu), Pw = dpp_wave_sum(Pu), Qw = dpp_wave_sum(Qu);
        unsigned long long* slots = a.samp_slots + size_t(s.b) * a.Q * kSampSlots;
        const unsigned pay[kSampSlots] = {hi32(Aw), lo32(Aw), hi32(Bw), lo32(Bw),
                                          hi32(Pw), lo32(Pw), hi32(Qw), lo32(Qw)};
        publish(slots + s.q, pay, s.epoch, a.Q);
        double u_acc, u_smp;
        verify_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + row, &u_acc, &u_smp);
        unsigned v[kSampSlots];
        const bool ok = gather<kSampSlots>(slots, a.Q, s.epoch, v);
        // lane l < Q: workgroup l's sums (zero in the other lanes)
        const double Ag = join64(v[0], v[1]), Bg = join64(v[2], v[3]);
        const double Pg = join64(v[4], v[5]), Qg = join64(v[6], v[7]);
        const double Zp = dpp_wave_sum(Pg), Zq = dpp_wave_sum(Qg);
        const double invZp = 1.0 / Zp, invZq = 1.0 / Zq;
        double Rg = fmax(0.0, Ag * invZp - Bg * invZq);
        double total = dpp_wave_sum(Rg);
        bool use_p = false;
        if (!(total > 0.0)) {      // zero residual: draw from p_j instead
            use_p = true;
            Rg = Pg;
            total = Zp;
        }
        const double t = u_smp * total;
        double run;
        bool exact;
        const int qstar = find_crossing(Rg, 0.0, t, run, exact);
        int owner = -1;
        if (qstar == s.q) {        // the crossing workgroup: find the crossing unit
            const double Ru = use_p ? Pu : fmax(0.0, Au * invZp - Bu * invZq);
            bool exact_u;
            owner = find_crossing(Ru, run, t, run, exact_u);
            exact = exact && exact_u;
        }
        if (lane == 0) {
            sh.samp.owner = owner;
            sh.samp.flags = (use_p ? kSampUseP : 0u) | (exact ? kSampExact : 0u) | (ok ? 0u : kSampError);
            sh.samp.run = run;
            sh.samp.t = t;
            sh.samp.Z1 = Zp;
            sh.samp.Z2 = Zq;
        }
    }
    __syncthreads();
    bool use_p, exact;
    double run, t, Zp, Zq;
    if (!read_samp(a, s, sh, use_p, exact, run, t, Zp, Zq)) return;
    final_scan<kVec4>(a, s, row, true, prow, qrow, c, sh.ls[s.wave], use_p, exact, run, t, 1.0 / Zp, 1.0 / Zq, Zp,
                      1.0, c.Mp64);
}

// Acceptance test of draft j from the combined statistics and the draft token's
// two logits (loaded while the group was exchanging statistics); workgroup 0
// writes the outputs of the test.
__device__ __forceinline__ bool accept_test(const RejectArgs& a, const SeqCtx& s, int j, const RowStats& st,
                                            const TokenLogits& tl) {
    const int k = a.k, b = s.b;
    double p_d = 0.0, q_d = 0.0;
    if (tl.ok) {
        p_d = exp_nonpos_f64((static_cast<double>(tl.zp) - st.Mp) * a.invT64) / st.Zp;
        q_d = exp_nonpos_f64((static_cast<double>(tl.zq) - st.Mq) * a.invT64) / st.Zq;
    }
    const double ratio = (q_d > 0.0) ? p_d / q_d : (p_d > 0.0 ? INFINITY : 0.0);
    const bool accepted = uniform(static_cast<int>(tl.u_acc < ratio)) != 0;
    if (s.q == 0 && lane_id() == 0) {
        if (a.accept_probs) a.accept_probs[size_t(b) * k + j] = static_cast<float>(fmin(1.0, ratio));
        if (accepted) {
            a.out_tokens[size_t(b) * (k + 1) + j] = tl.tok;
            if (a.out_probs) a.out_probs[size_t(b) * (k + 1) + j] = static_cast<float>(p_d);
        }
    }
    return accepted;
}

// Level `row` of the chain (rows p_row and q_row): every wavefront reduces its
// unit, wave 0 combines the workgroup's eight, publishes the pair and gathers the
// group's, combines those in workgroup order and takes the acceptance test; every
// workgroup reaches the same decision from the same bits. Returns the result flags
// (kResAccepted, kResError) and the row's statistics in `st`.
template <bool kVec4>
__device__ __forceinline__ unsigned level_step(const RejectArgs& a, const SeqCtx& s, int row, f4 (&xp)[kVecs],
                                               f4 (&xq)[kVecs], RowStats& st, const TokenLogits& tok, Shared& sh,
                                               bool& counted) {
    const float* prow = s.prow_base + size_t(row) * a.V;
    const float* qrow = s.qrow_base + size_t(row) * a.V;
    // wave 0 takes the acceptance test: the draft token's two logits are loaded
    // first, so they have long arrived when the group's statistics are in
    float ztp = 0.0f, ztq = 0.0f;
    if (s.wave == 0 && tok.ok) {
        ztp = prow[tok.tok];
        ztq = qrow[tok.tok];
    }
    load_unit<kVec4, true>(prow, qrow, a.V, s.u, xp, xq);
    float mp = -INFINITY, mq = -INFINITY;
    double sp = 0.0, sq = 0.0;
#pragma unroll
    for (int g = 0; g < kVecs / kStep; ++g) {
        online_step(xp, g, a.c2, mp, sp);
        online_step(xq, g, a.c2, mq, sq);
    }
    {
        float Mp_u, Mq_u;
        double Zp_u, Zq_u;
        combine_pair(mp, sp, a.invT64, Mp_u, Zp_u);
        combine_pair(mq, sq, a.invT64, Mq_u, Zq_u);
        if (lane_id() == 0) sh.unit[s.wave] = UnitStat{Mp_u, Mq_u, Zp_u, Zq_u};
    }
    __syncthreads();
    if (s.wave == 0) {
        const int lane = lane_id();
        float mpw = -INFINITY, mqw = -INFINITY;
        double zpw = 0.0, zqw = 0.0;
        if (lane < kUnitWaves) {
            const UnitStat u = sh.unit[lane];
            mpw = u.Mp; mqw = u.Mq; zpw = u.Zp; zqw = u.Zq;
        }
        float Mp_w, Mq_w;
        double Zp_w, Zq_w;
        combine_pair(mpw, zpw, a.invT64, Mp_w, Zp_w);
        combine_pair(mqw, zqw, a.invT64, Mq_w, Zq_w);
        const size_t level = size_t(s.b) * (a.k + 1) + row;
        unsigned long long* slots = a.stat_slots + level * a.Q * kStatSlots;
        const unsigned pay[kStatSlots] = {__builtin_bit_cast(unsigned, Mp_w), __builtin_bit_cast(unsigned, Mq_w),
                                          hi32(Zp_w), lo32(Zp_w), hi32(Zq_w), lo32(Zq_w)};
        publish(slots + s.q, pay, s.epoch, a.Q);
        TokenLogits tl = tok;
        double u_smp;
        verify_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + row, &tl.u_acc, &u_smp);
        unsigned v[kStatSlots];
        unsigned flags = 0;
        if (gather<kStatSlots>(slots, a.Q, s.epoch, v)) {
            count_group(a, s, counted);
            tl.zp = uniform(ztp);
            tl.zq = uniform(ztq);
            const bool have = lane < a.Q;
            combine_pair(have ? __builtin_bit_cast(float, v[0]) : -INFINITY, have ? join64(v[2], v[3]) : 0.0,
                         a.invT64, st.Mp, st.Zp);
            combine_pair(have ? __builtin_bit_cast(float, v[1]) : -INFINITY, have ? join64(v[4], v[5]) : 0.0,
                         a.invT64, st.Mq, st.Zq);
            if (accept_test(a, s, row, st, tl)) flags |= kResAccepted;
        } else {
            count_group(a, s, counted);
            st.Mp = st.Mq = 0.0f;
            st.Zp = st.Zq = 1.0;
            flags |= kResError;
        }
        if (lane == 0) sh.res = LevelRes{flags, st.Mp, st.Mq, st.Zp, st.Zq};
    }
    __syncthreads();
    st.Mp = uniform(sh.res.Mp);
    st.Mq = uniform(sh.res.Mq);
    st.Zp = uniform(sh.res.Zp);
    st.Zq = uniform(sh.res.Zq);
    return static_cast<unsigned>(uniform(static_cast<int>(sh.res.flags)));
}

// The bonus row p_k after k acceptances, with one exchange: each wavefront weighs
// its unit against the unit's own maximum M_u (heavy logits judged with the
// unit's own normaliser, a superset of the row's heavy set); wave 0 rescales its
// units to the workgroup maximum and publishes (sum, maximum); the gathered pairs
// are rescaled to the row maximum M, which also gives the row's Z.
template <bool kVec4>
__device__ __forceinline__ void bonus_row(const RejectArgs& a, const SeqCtx& s, f4 (&xp)[kVecs], f4 (&xq)[kVecs],
                                          Shared& sh, bool& counted) {
    const int row = a.k;
    const float* prow = s.prow_base + size_t(row) * a.V;
    load_unit<kVec4, false>(prow, prow, a.V, s.u, xp, xq);
    float m = -INFINITY;
    double acc = 0.0;
#pragma unroll
    for (int g = 0; g < kVecs / kStep; ++g) online_step(xp, g, a.c2, m, acc);
    float Mu;
    double Zu;
    combine_pair(m, acc, a.invT64, Mu, Zu);
    SampleCtx c;
    c.Mp = Mu;
    c.Mq = 0.0f;
    c.invT = a.invT;
    c.Mp64 = Mu;
    c.Mq64 = 0.0;
    c.invT64 = a.invT64;
    c.hp = static_cast<float>(kLnTau + log(Zu));
    c.hq = kLnTau;
    c.dn = 0.0f;
    const int lane = lane_id();
    const UnitSums us = unit_sums<kVec4, false>(xp, xq, c, prow, prow, s.u * kUnit + lane * 4, sh.ls[s.wave]);
    const double Mu64 = Mu;
    if (lane == 0) sh.usum[s.wave] = make_double4(us.P, Mu64, 0.0, 0.0);
    __syncthreads();
    if (s.wave == 0) {
        double Pu = 0.0, Mv = -INFINITY;
        if (lane < kUnitWaves) {
            const double4 v = sh.usum[lane];
            Pu = v.x;
            Mv = v.y;
        }
        const double Mw = dpp_wave_max(static_cast<float>(Mv));
        const double Ww = dpp_wave_sum((Pu > 0.0) ? Pu * exp_nonpos_f64((Mv - Mw) * a.invT64) : 0.0);
        unsigned long long* slots = a.samp_slots + size_t(s.b) * a.Q * kSampSlots;
        const unsigned pay[4] = {hi32(Ww), lo32(Ww), hi32(Mw), lo32(Mw)};
        publish(slots + s.q, pay, s.epoch, a.Q);
        double u_acc, u_smp;
        verify_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + row, &u_acc, &u_smp);
        unsigned v[4];
        const bool ok = gather<4>(slots, a.Q, s.epoch, v);
        count_group(a, s, counted);
        const bool have = lane < a.Q;
        const double Wg = have ? join64(v[0], v[1]) : 0.0;
        const double Mg = have ? join64(v[2], v[3]) : -INFINITY;
        const double M = dpp_wave_max(static_cast<float>(Mg));
        const double Wr = (Wg > 0.0) ? Wg * exp_nonpos_f64((Mg - M) * a.invT64) : 0.0;
        const double Z = dpp_wave_sum(Wr);
        const double t = u_smp * Z;
        double run;
        bool exact;
        const int qstar = find_crossing(Wr, 0.0, t, run, exact);
        int owner = -1;
        if (qstar == s.q) {
            const double Wu = (Pu > 0.0) ? Pu * exp_nonpos_f64((Mv - M) * a.invT64) : 0.0;
            bool exact_u;
            owner = find_crossing(Wu, run, t, run, exact_u);
            exact = exact && exact_u;
        }
        if (lane == 0) {
            sh.samp.owner = owner;
            sh.samp.flags = (exact ? kSampExact : 0u) | (ok ? 0u : kSampError);
            sh.samp.run = run;
            sh.samp.t = t;
            sh.samp.Z1 = Z;
            sh.samp.Z2 = M;
        }
    }
    __syncthreads();
    bool use_p, exact;
    double run, t, Z, M;
    if (!read_samp(a, s, sh, use_p, exact, run, t, Z, M)) return;
    const double wscale = exp_nonpos_f64((Mu64 - M) * a.invT64);
    final_scan<kVec4>(a, s, row, false, prow, prow, c, sh.ls[s.wave], false, exact, run, t, 1.0 / Z, 1.0, Z, wscale,
                      M);
}

template <bool kVec4>
__global__ __launch_bounds__(kRT) __attribute__((amdgpu_waves_per_eu(2, 2))) void reject_kernel(RejectArgs a) {
    // Workgroups go to the eight XCDs round-robin; with a multiple of eight groups,
    // group g takes the Q workgroups on XCD g % 8 (they start together and share
    // an L2). Any other count uses the plain mapping. Both are bijections.
    const int w = blockIdx.x;
    int group, q;
    if (a.groups % 8 == 0) {
        const int l = w / 8;
        group = (w % 8) + 8 * (l / a.Q);
        q = l % a.Q;
    } else {
        group = w / a.Q;
        q = w % a.Q;
    }
    SeqCtx s;
    s.q = q;
    s.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    s.u = q * kUnitWaves + s.wave;
    {
        const unsigned last = __hip_atomic_load(a.ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.epoch = (last + 1u == 0u) ? 1u : last + 1u;
    }
    bool counted = q != 0;   // workgroup 0's wave 0 counts the group
    __shared__ Shared sh;
    f4 xp[kVecs], xq[kVecs];
    for (int b = group; b < a.B; b += a.groups) {
        s.b = b;
        s.prow_base = a.target + size_t(b) * (a.k + 1) * a.V;
        s.qrow_base = a.draft + size_t(b) * a.k * a.V;
        // per-lane copies (equal in every lane), first needed at the first acceptance
        // test, so that no wait for them precedes the loads of the first level
        s.sid = a.seq_ids[b];
        s.L = a.seq_lens[b];
        // the draft tokens of the sequence, lane j holding token j
        const int lane = lane_id();
        const int tok_lane = (lane < a.k) ? a.draft_tokens[size_t(b) * a.k + lane] : 0;
        RowStats st;
        bool done = false;
        for (int j = 0; j < a.k && !done; ++j) {
            TokenLogits tl;
            tl.tok = __builtin_amdgcn_readlane(tok_lane, j);
            tl.ok = tl.tok >= 0 && tl.tok < a.V;
            tl.zp = tl.zq = 0.0f;
            tl.u_acc = 0.0;
            const unsigned res = level_step<kVec4>(a, s, j, xp, xq, st, tl, sh, counted);
            if (res & kResError) {
                flag_error(a, s);
                done = true;
            } else if (!(res & kResAccepted)) {
                sample_row<kVec4>(a, s, j, xp, xq, st, sh);
                done = true;
            }
        }
        if (done) continue;
        bonus_row<kVec4>(a, s, xp, xq, sh, counted);
    }
}

template <bool kVec4>
hipError_t co_resident(int dev, int* wgs) {
    static int memo[64];
    if (dev >= 0 && dev < 64 && memo[dev] > 0) {
        *wgs = memo[dev];
        return hipSuccess;
    }
    int per_cu = 0, cus = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reject_kernel<kVec4>, kRT, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    *wgs = per_cu * cus;
    if (dev >= 0 && dev < 64) memo[dev] = *wgs;
    return hipSuccess;
}

template <bool kVec4>
hipError_t launch_variant(RejectArgs& a, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int wgs = 0;
    e = co_resident<kVec4>(dev, &wgs);
    if (e != hipSuccess) return e;
    int groups = min(a.B, wgs / a.Q);
    if (groups < 1) return hipErrorInvalidConfiguration;
    if (groups > 8) groups -= groups % 8;   // a multiple of 8 (one XCD per group); rounds take the rest
    a.groups = groups;
    // A plain launch: the grid never exceeds what the device holds at once, so on
    // a GPU not shared with other streams every group is resident together. (A
    // cooperative launch would guarantee it, at ~13 us of extra launch latency
    // per call on this stack; should residency ever be partial, the waits are
    // bounded and the affected sequences report an error instead of hanging.)
    hipLaunchKernelGGL((reject_kernel<kVec4>), dim3(groups * a.Q), dim3(kRT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t reject_workspace_bytes(int B, int k, int V) {
    const int U = (V + kUnit - 1) / kUnit;
    const int Q = (U + kUnitWaves - 1) / kUnitWaves;
    return reject_layout(B, k, Q).total;
}

int reject_max_vocab() { return kUnit * kUnitWaves * kMaxQ; }

hipError_t launch_reject(const RejectLaunch& p, hipStream_t stream) {
    const int U = (p.V + kUnit - 1) / kUnit;
    const int Q = (U + kUnitWaves - 1) / kUnitWaves;
    if (Q > kMaxQ) return hipErrorInvalidValue;
    const RejectLayout lay = reject_layout(p.B, p.k, Q);
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
    a.ctl = reinterpret_cast<unsigned*>(ws + lay.ctl);
    a.stat_slots = reinterpret_cast<unsigned long long*>(ws + lay.stat);
    a.samp_slots = reinterpret_cast<unsigned long long*>(ws + lay.samp);
    a.B = p.B; a.k = p.k; a.V = p.V; a.U = U; a.Q = Q; a.groups = 0;
    a.invT = 1.0f / p.temperature;
    a.c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(p.temperature));
    a.invT64 = 1.0 / static_cast<double>(p.temperature);
    a.seed = p.seed;
    return (p.V % 4) == 0 ? launch_variant<true>(a, stream) : launch_variant<false>(a, stream);
}

}  // namespace specverify
