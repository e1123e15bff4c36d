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
//  * A row of V logits is cut into U units of 4096; each unit of the current row
//    (pair) is held in the registers of one wavefront (16 x 16-byte loads per
//    lane per row, all in flight together). W unit wavefronts form a workgroup:
//    eight (one workgroup per CU) when the batch fills the device in one round of
//    them, four otherwise: a sequence over twice as many CUs (one workgroup on
//    each) when B * ceil(U/4) workgroups fit one per CU, which shortens each step
//    of a sequence's serial chain at small batches, and two workgroups of
//    different sequences per CU when the batch takes several rounds. The
//    Q = ceil(U / W) workgroups of a sequence form a group, and groups take
//    sequences in turn.
//  * Level j: every wavefront reduces its units of p_j and q_j to (max, sum of
//    exps) with an online softmax on the DPP network; wave 0 of the workgroup
//    combines them four at a time (quads of consecutive units) and publishes one
//    entry per quad; then it gathers the ceil(U / 4) quads of the sequence,
//    combines them in quad order and takes the acceptance test. Every workgroup
//    computes the same decision from the same published bits, so one cross-CU
//    exchange per level suffices; and as the quads are the same for W = 4 and
//    W = 8, so are all results: a sequence's outputs do not depend on the batch.
//  * Exchange is fence-free: each published 32-bit value travels in a 64-bit
//    atomic slot together with the call's epoch, so a slot is either stale (old
//    epoch, keep polling) or complete. No cache write-back or invalidation is
//    needed and the workspace never has to be cleared between calls.
//  * On the first rejection (or after k acceptances, on row p_k) the rows still
//    in registers are turned into sampling weights: nothing is read twice. Unit
//    sums go through LDS to the workgroup leader, one exchange gives every
//    leader the quad totals, the leaders find the crossing quad, and the leader
//    of the workgroup holding it finds the crossing unit, whose wavefront scans
//    its per-load sums in LDS for the token.
//  * Precision: the chain statistics use fp32 exps (relative error ~1e-7, ample
//    for an acceptance test). The sampling pass takes logits whose probability
//    exceeds 2^-14 in fp64 and the rest with an error-compensated fp32 exp,
//    accumulating in fp64, so the sampling CDF is within ~1e-9 of an fp64 one.
//  * Co-residency of a group is required: the grid is sized to what the device
//    holds at once, and every wait is bounded so that a wavefront always
//    terminates (a timed-out sequence reports num_accepted = -1).
#include <atomic>
#include <cstdlib>

#include "common.hpp"
#include "fastexp.hpp"
#include "heavy.hpp"
#include "softmax_step.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace specverify {
namespace {

constexpr int kVecs = 16;                  // 16-byte loads per lane per row
constexpr int kUnit = kWave * kVecs * 4;   // 4096 logits: one wavefront's share of a row
constexpr int kStep = 4;                   // loads per online-softmax step (16 logits per lane)
constexpr int kStatSlots = 6;              // M_p, M_q, Z_p (hi, lo), Z_q (hi, lo)
constexpr int kSampSlots = 8;              // A, B, P, Q (hi, lo each); bonus row: weight sum, max
constexpr int kUnitWaves = 8;              // unit wavefronts per workgroup at most (4 where the batch is small)
constexpr int kRT = kUnitWaves * kWave;    // 512 threads
constexpr int kMaxQ = 64;                  // workgroups per sequence: U <= 256 (V <= 2^20), four units each
constexpr int kMaxBranch = 4;              // tree: children per node
constexpr int kTreeEx = 24;                // tree: exchanges per sequence (levels, passes, the draw)
constexpr unsigned kSpinLimit = 1u << 20;    // polls per wait (see reject_spin_limit)
constexpr int kMaxLevels = 16;             // decision slots per sequence (k <= 15)
constexpr int kDecSlots = 3;               // per level: decision, p of the draft, min(1, p/q)

enum : unsigned { kCtlEpoch = 0, kCtlDone = 1, kCtlError = 2, kCtlQueue = 3, kCtlFinished = 4 };
constexpr int kMaxGroups = 1024;           // groups of one launch (the device holds at most 512 workgroups)

typedef float f4 __attribute__((ext_vector_type(4)));

struct RejectArgs {
    const float* target;
    const float* draft;
    const int32_t* draft_tokens;
    const int64_t* seq_ids;
    const int32_t* seq_lens;
    const int32_t* cu;                 // [B+1] draft-count offsets, or null: k drafts each
    int32_t* out_tokens;
    int32_t* num_accepted;
    float* out_probs;
    float* accept_probs;
    unsigned* ctl;                     // epoch of the last finished call, finished-wave count, error flag
    unsigned long long* stat_slots;    // [B][k+1][kStatSlots][U]: unit statistics per level
    unsigned long long* samp_slots;    // [B][kSampSlots][U]: unit sampling sums
    const int32_t* parents;            // tree: [B][k] parent of node n at [n-1]; null for a chain
    int32_t* out_nodes;                // tree: [B][k] accepted node indices, or null
    unsigned long long* tree_slots;    // tree: [B][kTreeEx][kSampSlots][U], one block per exchange
    unsigned long long* dec_slots;     // level-parallel: [B][kDecSlots][kMaxLevels] each level's decision,
                                       // the probability of its draft and min(1, p/q)
    unsigned long long* bonus_slots;   // level-parallel: [B][4][U] the bonus row's exchange
    unsigned long long* next_slots;    // chain: [kMaxGroups] each group's next sequence
    unsigned spin;                     // polls before a wait gives up
    int B, k, V, U, Q, groups;
    float invT;                        // 1 / T
    float c2;                          // log2(e) / T
    double invT64;
    float T;
    uint64_t seed;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct RejectLayout {
    size_t ctl, stat, samp, dec, bonus, next, total;
};

RejectLayout reject_layout(int B, int k, int U) {
    RejectLayout L;
    size_t o = 0;
    L.ctl = o;  o = align256(o + 8 * sizeof(unsigned));
    L.stat = o; o = align256(o + sizeof(unsigned long long) * size_t(B) * (k + 1) * U * kStatSlots);
    L.samp = o; o = align256(o + sizeof(unsigned long long) * size_t(B) * U * kSampSlots);
    L.dec = o;  o = align256(o + sizeof(unsigned long long) * size_t(B) * kDecSlots * kMaxLevels);
    L.bonus = o; o = align256(o + sizeof(unsigned long long) * size_t(B) * U * 4);
    L.next = o; o = align256(o + sizeof(unsigned long long) * kMaxGroups);
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
// words. Returns false if the bounded wait ran out after `spin` polls (only
// possible if the group were not resident at once).
template <int N>
__device__ __forceinline__ bool gather_at(unsigned long long* slots, int stride, int first, int count, unsigned epoch,
                                          unsigned spin, unsigned (&out)[N]) {
    // Two polls in flight: the next one is issued before the previous one is looked at,
    // so a slot is seen about half a round trip sooner than with one poll at a time
    // (on the 8B rows the call takes ~1.5 us less).
    const int lane = lane_id();
    unsigned long long va[N], vb[N];
    auto issue = [&](unsigned long long (&v)[N]) {
#pragma unroll
        for (int s = 0; s < N; ++s) v[s] = lane < count ? slot_load(slots + size_t(s) * stride + first + lane) : 0ull;
    };
    auto take = [&](const unsigned long long (&v)[N]) {
        bool ok = true;
#pragma unroll
        for (int s = 0; s < N; ++s) {
            if (lane < count) ok = ok && static_cast<unsigned>(v[s]) == epoch;
            out[s] = static_cast<unsigned>(v[s] >> 32);
        }
        return __all(ok);
    };
    if (spin == 0) return false;
    issue(va);
    for (unsigned it = 0; it + 1 < spin; it += 2) {
        issue(vb);
        if (take(va)) return true;
        issue(va);
        if (take(vb)) return true;
    }
    return take(va);
}

template <int N>
__device__ __forceinline__ bool gather(unsigned long long* slots, int Q, unsigned epoch, unsigned spin,
                                       unsigned (&out)[N]) {
    return gather_at<N>(slots, Q, 0, Q, epoch, spin, out);
}

// The first two steps of the DPP wavefront reductions (dpp_wave_max / dpp_wave_sum) alone: every lane ends with the
// maximum / sum of its group of four lanes (lanes 4j .. 4j+3), with the same bits as
// the full reduction gives when all other lanes hold the identity.
__device__ __forceinline__ float dpp_quad_max(float v) {
    const int id = __builtin_bit_cast(int, -INFINITY);
    v = fmaxf(v, __builtin_bit_cast(float, dpp_move<0xB1>(__builtin_bit_cast(int, v), id)));
    v = fmaxf(v, __builtin_bit_cast(float, dpp_move<0x4E>(__builtin_bit_cast(int, v), id)));
    return v;
}

__device__ __forceinline__ double dpp_quad_sum(double v) {
    v += dpp_move_f64<0xB1>(v);
    v += dpp_move_f64<0x4E>(v);
    return v;
}

// Exchanges go through quads: four consecutive units, combined in lanes 0..3 of the
// workgroup's wave 0 and published as one entry. A workgroup of W unit wavefronts
// holds W / 4 quads, and a sequence's nq = ceil(U / 4) quads are combined in quad
// order, so every result is the same whatever W is.
constexpr int kQuad = 4;

__device__ __forceinline__ int quads_of(int U) { return (U + kQuad - 1) / kQuad; }

// combine_pair over each group of four lanes: lane 4j .. 4j+3 end with the (M, Z) of
// the units in those lanes (the same bits as combine_pair over them alone).
__device__ __forceinline__ void combine_quad(float m, double z, double invT64, float& M, double& Z) {
    M = dpp_quad_max(m);
    Z = dpp_quad_sum((z > 0.0) ? z * exp_nonpos_f64((static_cast<double>(m) - M) * invT64) : 0.0);
}

// Lane 4j (j < lanes / 4) of wave 0 publishes the quad in its lanes, quad index
// first + j of the sequence when below nq: payload s to slots[s * nq + quad].
template <int N>
__device__ __forceinline__ void publish_quads(unsigned long long* slots, const unsigned (&payload)[N], unsigned epoch,
                                              int first, int lanes, int nq) {
    const int lane = lane_id();
    const int qd = first + lane / kQuad;
    if ((lane & (kQuad - 1)) == 0 && lane < lanes && qd < nq) {
#pragma unroll
        for (int s = 0; s < N; ++s) slot_store(slots + size_t(s) * nq + qd, payload[s], epoch);
    }
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

// Element i of a read-only input at a wave-uniform address, through the constant
// address space: a scalar load, counted apart from the vector loads in flight.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p, size_t i) {
    typedef const __attribute__((address_space(4))) T CT;
    return ((CT*)p)[i];
}

// ---------------------------------------------------------------- loads

// Logits rows are read through buffer resources: a load at an offset past the
// row's V * 4 bytes returns zero without touching memory, so every lane loads
// unconditionally. Without per-lane branches around the loads the compiler counts
// the loads in flight exactly and can start on the first ones as they arrive.
constexpr int kRsrcFlags = 0x00020000;   // raw 32-bit data, no swizzle
constexpr int kNonTemporal = 2;          // streamed once: do not keep in the caches

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* row, int V) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), static_cast<short>(0), V * 4, kRsrcFlags);
}

// Four consecutive logits from x (x a multiple of 4 when kVec4), without padding.
template <bool kVec4>
__device__ __forceinline__ f4 load4_raw(__amdgpu_buffer_rsrc_t r, int x) {
    if (kVec4) return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, x * 4, 0, kNonTemporal));
    f4 f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        f[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (x + c) * 4, 0, kNonTemporal));
    return f;
}

// -inf for the logits of f (from x) at or past V.
__device__ __forceinline__ void pad4(f4& f, int x, int V) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (x + c >= V) f[c] = -INFINITY;
}

template <bool kVec4>
__device__ __forceinline__ f4 load4(__amdgpu_buffer_rsrc_t r, int V, int x) {
    f4 f = load4_raw<kVec4>(r, x);
    pad4(f, x, V);
    return f;
}

// Element (i, c) of lane l in unit u is logit u*4096 + i*256 + 4*l + c: each load
// of a wavefront is one contiguous 1 KB run. p and q loads are interleaved so the
// online softmax can start on the first step while the rest are in flight. Only
// the last unit of a row can reach past V; its padding is set after the loads.
template <bool kVec4, bool kTwo>
__device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t rp, __amdgpu_buffer_rsrc_t rq, int V, int u,
                                          f4 (&xp)[kVecs], f4 (&xq)[kVecs]) {
    const int base = u * kUnit + lane_id() * 4;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        xp[i] = load4_raw<kVec4>(rp, base + i * (kWave * 4));
        if (kTwo) xq[i] = load4_raw<kVec4>(rq, base + i * (kWave * 4));
    }
    if ((u + 1) * kUnit > V) {   // uniform
#pragma unroll
        for (int i = 0; i < kVecs; ++i) {
            pad4(xp[i], base + i * (kWave * 4), V);
            if (kTwo) pad4(xq[i], base + i * (kWave * 4), V);
        }
    }
}

// ---------------------------------------------------------------- chain statistics

// One online-softmax step over loads 4s..4s+3 of this lane: running max m and
// running sum s of 2^{(x - m) c2}, c2 = log2(e)/T, the terms as hardware exp2 of
// one fma each. The statistics feed the acceptance ratio u < p/q, whose decisions
// the fp64 oracle reproduces except within a small margin of u, so the sum must
// carry no error common to all its terms (softmax_step.hpp): the rounding of the
// step's offset -ref c2 is put back into the step's sum, and the sum so far moves
// onto the new maximum with an exponent that is exactly 0 when the maximum did not
// move. (Without this the error compounded over the steps to ~2e-6 of the sum; fp64
// for the same corrections measured 4% slower.) What remains is the rounding of
// each term's own argument and exp2, independent from term to term.
__device__ __forceinline__ void online_step(const f4 (&x)[kVecs], int s, float c2, float& m, double& acc) {
    // maximum() rather than fmaxf(): the inputs are never NaN, and it takes loaded
    // values without a canonicalising instruction each (three-input form on gfx950)
    float gm = -INFINITY;
#pragma unroll
    for (int i = kStep * s; i < kStep * s + kStep; ++i)
        gm = __builtin_elementwise_maximum(gm, __builtin_elementwise_maximum(
                 __builtin_elementwise_maximum(x[i].x, x[i].y), __builtin_elementwise_maximum(x[i].z, x[i].w)));
    const float mn = __builtin_elementwise_maximum(m, gm);
    const float ref = (mn == -INFINITY) ? 0.0f : mn;   // all -inf so far: every term is 0
    const StepOffset off = step_offset(ref, c2);       // exps as exp2(x * c2 + off.nr), one fma each
    const float rescale = __builtin_amdgcn_exp2f(rescale_exponent(m, c2, off));   // 1 if no move, 0 from -inf
    float part[kStep];
#pragma unroll
    for (int i = 0; i < kStep; ++i) {
        const f4 v = x[kStep * s + i];
        const float e0 = __builtin_amdgcn_exp2f(fmaf(v.x, c2, off.nr));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(v.y, c2, off.nr));
        const float e2 = __builtin_amdgcn_exp2f(fmaf(v.z, c2, off.nr));
        const float e3 = __builtin_amdgcn_exp2f(fmaf(v.w, c2, off.nr));
        part[i] = (e0 + e1) + (e2 + e3);
    }
    const float sum = corrected_sum((part[0] + part[1]) + (part[2] + part[3]), off);
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
    float tp, tq;        // heavy thresholds on the raw logits (probability above tau)
    float dn;            // ln Z_p - ln Z_q: x in the residual support iff lp - lq > dn
    double Mp64, Mq64, invT64;
};

// Log-weight of a logit in nats, (z - M) / T, and the residual-support test. Each
// operation rounds on its own: contraction is switched off here, because HIP's
// __fmul_rn / __fsub_rn are plain operators that the compiler may fuse, and it
// fused the support test's subtraction with one of the two products at one call
// site but not necessarily at another. The support must be the same set wherever
// it is judged (the unit sums, the heavy re-reads, the final scan).
__device__ __forceinline__ float log_weight(float z, float M, float invT) {
#pragma clang fp contract(off)
    return (z - M) * invT;
}
__device__ __forceinline__ bool in_support(float xp, float xq, float dn) {
#pragma clang fp contract(off)
    return xp - xq > dn;
}
__device__ __forceinline__ bool is_heavy(bool residual, float zp, float zq, const SampleCtx& c) {
    return static_cast<int>(heavy_sign(residual, zp, zq, c.tp, c.tq)) < 0;
}

// Light part of the unnormalised weights a = e^{(z_p - M_p)/T}, b = e^{(z_q - M_q)/T}
// of the four logits of one load: compensated fp32 exps, zeroed (by a product, so
// the exp is never moved into a branch) for heavy logits, which are taken in fp64
// separately. Membership of the residual support {p > q} is judged with the
// chain's normalisers.
__device__ __forceinline__ void light_weights(bool residual, const f4& vp, const f4& vq, const SampleCtx& c,
                                              float (&la)[4], float (&lb)[4], bool (&in_s)[4], bool (&h)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float xp = log_weight(vp[e], c.Mp, c.invT);
        const float xq = residual ? log_weight(vq[e], c.Mq, c.invT) : -INFINITY;
        h[e] = is_heavy(residual, vp[e], vq[e], c);
        in_s[e] = residual ? in_support(xp, xq, c.dn) : true;   // NaN for padding: not in the support
        const float keep = h[e] ? 0.0f : 1.0f;
        la[e] = exp_small_f32(xp) * keep;
        lb[e] = residual ? exp_small_f32(xq) * keep : 0.0f;
    }
}

// Up to four heavy logits of the lane, re-read from memory (rather than picked out
// of the register arrays, which would need dynamic indexing and force the arrays
// out of registers). Issued before the light pass so that the loads are in by the
// time they are weighed.
struct HeavyRound {
    unsigned ks;         // element index in the unit per byte (0xFF: none)
    float zp[4], zq[4];
};

__device__ __forceinline__ int round_k(const HeavyRound& r, int j) {
    const unsigned b = (r.ks >> (8 * j)) & 0xFFu;
    return b == 0xFFu ? -1 : static_cast<int>(b);
}

__device__ __forceinline__ void heavy_fetch(bool residual, __amdgpu_buffer_rsrc_t rp, __amdgpu_buffer_rsrc_t rq,
                                            int V, int base, HeavyBits& hb, HeavyRound& r) {
    r.ks = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = take_heavy(hb);
        r.ks |= static_cast<unsigned>(k & 0xFF) << (8 * j);
        // Through the rows' buffer resources, like every other read of the logits: an
        // offset past the row returns 0 without touching memory, so the read stays in
        // bounds whatever the classification said. An element at or past V (padding,
        // never heavy under the thresholds used, see heavy.hpp) is then taken as -inf,
        // weight 0. Lanes without a heavy element read logit 0. Cached loads: the row
        // was streamed moments ago.
        const int x = k >= 0 ? heavy_element(base, k) : 0;
        const bool pad = x >= V;
        const float zp = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, x * 4, 0, 0));
        const float zq = residual ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rq, x * 4, 0, 0))
                                  : -INFINITY;
        r.zp[j] = pad ? -INFINITY : zp;
        r.zq[j] = pad ? -INFINITY : zq;
    }
}

// fp64 weights of one round of heavy logits; `f` receives (load index, a, b, in
// support) for each.
template <typename F>
__device__ __forceinline__ void heavy_weigh(bool residual, const SampleCtx& c, const HeavyRound& r, F&& f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double va = exp_nonpos_f64((static_cast<double>(r.zp[j]) - c.Mp64) * c.invT64);
        const double vb = residual ? exp_nonpos_f64((static_cast<double>(r.zq[j]) - c.Mq64) * c.invT64) : 0.0;
        const bool ins = residual
            ? in_support(log_weight(r.zp[j], c.Mp, c.invT), log_weight(r.zq[j], c.Mq, c.invT), c.dn) : true;
        const int k = round_k(r, j);
        if (k >= 0) f(k >> 2, va, vb, ins);
    }
}

struct UnitSums {
    double A, B, P, Q;   // sums over the support of a, b; sums over all logits of a, b
};

// Per-lane sums of a and b over the support for each of the lane's sixteen loads,
// kept in LDS ([load][lane], 16 KB per wavefront) for the final scan. For the
// bonus row only the a-sums are meaningful.
typedef double2 LoadSums[kVecs][kWave];

// Unit sums of the sampling weights and, in `ls`, the per-load sums. The heavy
// logits are found first and their re-reads issued; the light pass over the
// registers then hides the loads' latency.
template <bool kVec4, bool kResidual>
__device__ __forceinline__ UnitSums unit_sums(const f4 (&xp)[kVecs], const f4 (&xq)[kVecs], const SampleCtx& c,
                                              const float* prow, const float* qrow, int V, int base, LoadSums& ls) {
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rp = row_rsrc(prow, V), rq = row_rsrc(qrow, V);
    HeavyBits hb = heavy_bits<kVecs>(kResidual, xp, xq, c.tp, c.tq);
    HeavyRound hr;
    heavy_fetch(kResidual, rp, rq, V, base, hb, hr);
    double A = 0.0, Bs = 0.0, P = 0.0, Q = 0.0;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        float la[4], lb[4];
        bool in_s[4], h[4];
        light_weights(kResidual, xp[i], xq[i], c, la, lb, in_s, h);
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
    auto add = [&](int i, double va, double vb, bool ins) {
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
    };
    heavy_weigh(kResidual, c, hr, add);
    while (__any((hb.lo | hb.hi) != 0u)) {   // lanes with more than four (rare)
        heavy_fetch(kResidual, rp, rq, V, base, hb, hr);
        heavy_weigh(kResidual, c, hr, add);
    }
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
    bool in_s[4], h[4];
    light_weights(two_rows, vp, vq, c, la, lb, in_s, h);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double va = h[e] ? exp_nonpos_f64((static_cast<double>(vp[e]) - c.Mp64) * c.invT64) : la[e];
        const double vb = (h[e] && two_rows) ? exp_nonpos_f64((static_cast<double>(vq[e]) - c.Mq64) * c.invT64)
                                             : lb[e];
        w[e] = sample_weight(residual, in_s[e], va, vb, invZp, invZq);
    }
}

// ---------------------------------------------------------------- per-sequence pieces

struct SeqCtx {
    int b;
    int kb;                   // drafts of this sequence
    size_t tb, db;            // its first target (and output) row, its first draft row
    int u;                    // unit of this wavefront: q * (unit wavefronts per workgroup) + wave
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
// results going back to all of the workgroup's wavefronts.
struct UnitStat {
    float Mp, Mq;
    double Zp, Zq;
};
struct LevelRes {
    unsigned flags;
    float Mp, Mq;
    double Zp, Zq;
    int tok;              // the candidate, its probability and min(1, p/q), for outputs written later
    float pd, ratio;
};
struct SampRes {
    int owner;         // wavefront holding the crossing unit, -1 if in another workgroup
    unsigned flags;    // kSampUseP, kSampExact, kSampError
    double run, t, Z1, Z2;
    double W;          // a residual round: the residual's mass sum max(0, p - q)
};
template <int W>
struct SharedT {
    static constexpr int kW = W;   // unit wavefronts of the workgroup
    LoadSums ls[W];
    UnitStat unit[W];
    double4 usum[W];
    int next;             // the group's next sequence
    LevelRes res;
    SampRes samp;
};
using Shared = SharedT<kUnitWaves>;

enum : unsigned { kResAccepted = 1u, kResError = 2u };
enum : unsigned { kSampUseP = 1u, kSampExact = 2u, kSampError = 4u, kSampAbort = 8u };
enum : unsigned { kDecRejected = 1u, kDecAccepted = 2u };   // payloads of the decision slots

// Level-parallel sampling: the outputs of accepted level i (its draft token, p of it and
// min(1, p/q)), written by the group that draws the sequence's last token once it has
// seen every earlier level's published decision. A level never writes its own outputs:
// one whose wait for the earlier decisions gave up would leave them unwritten while a
// later group, trusting its published acceptance, completed the sequence.
__device__ __forceinline__ void level_outputs(const RejectArgs& a, const SeqCtx& s, int i, unsigned pd_bits,
                                              unsigned ratio_bits) {
    a.out_tokens[s.tb + i] = a.draft_tokens[s.db + i];
    if (a.out_probs) a.out_probs[s.tb + i] = __builtin_bit_cast(float, pd_bits);
    if (a.accept_probs) a.accept_probs[s.db + i] = __builtin_bit_cast(float, ratio_bits);
}

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

// Inverse CDF inside the crossing unit, given the running sum `run` before the
// unit and the target t. lv(i, j0) returns the sum of the sampling weights of
// load i over lanes j0 .. j0+15 (from the LDS slab, or recomputed); wf(vp, vq, w)
// the weights of four logits, on the same scale as run and t. Returns true on the
// one lane that holds the drawn token, with its id in y and its target logit in zy.
template <bool kVec4, typename LV, typename WF>
__device__ __forceinline__ bool scan_unit(const RejectArgs& a, const SeqCtx& s, const float* prow,
                                          const float* qrow, bool two_rows, bool exact, double run, double t,
                                          LV&& lv, WF&& wf, int& y, float& zy) {
    const int lane = lane_id();
    const int base = s.u * kUnit + lane * 4;
    // Load level (each load of a wavefront is 256 consecutive tokens): load i's
    // total T_i is summed by the four lanes 4i..4i+3, sixteen per-lane sums each.
    double Ti = lv(lane >> 2, (lane & 3) * (kWave / 4));
    Ti += __shfl_xor(Ti, 1, kWave);
    Ti += __shfl_xor(Ti, 2, kWave);
    const bool head = (lane & 3) == 3;   // one lane per load carries its total
    const double incl = dpp_wave_incl_scan(head ? Ti : 0.0);
    const unsigned long long pos_i = __ballot(head && Ti > 0.0);
    const unsigned long long cross_i = exact ? __ballot(head && Ti > 0.0 && run + incl > t) : 0ull;
    int istar;
    double run_i;
    if (cross_i) {
        const int l = __ffsll(static_cast<long long>(cross_i)) - 1;
        istar = l >> 2;
        run_i = run + __shfl(incl - Ti, l, kWave);
    } else {               // rounding left no crossing here: take the last positive weight
        exact = false;
        istar = pos_i ? (63 - __builtin_clzll(pos_i)) >> 2 : 0;
        run_i = run;
    }
    double w[4];
    const f4 vp = load4<kVec4>(row_rsrc(prow, a.V), a.V, base + istar * (kWave * 4));
    const f4 vq = two_rows ? load4<kVec4>(row_rsrc(qrow, a.V), a.V, base + istar * (kWave * 4)) : vp;
    wf(vp, vq, w);
    const double lsum = (w[0] + w[1]) + (w[2] + w[3]);
    const double lincl = dpp_wave_incl_scan(lsum);
    const double lexcl = dpp_wave_shr1(lincl);
    int lstar, estar = -1;
    const unsigned long long cross = exact ? __ballot(lsum > 0.0 && run_i + lincl > t) : 0ull;
    int elast = -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) if (w[e] > 0.0) elast = e;
    if (cross) {
        lstar = __ffsll(static_cast<long long>(cross)) - 1;
        double r = run_i + lexcl;
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
    if (lane != lstar) return false;
    if (estar < 0) estar = 0;
    y = s.u * kUnit + istar * (kWave * 4) + lstar * 4 + estar;
    zy = estar == 0 ? vp.x : (estar == 1 ? vp.y : (estar == 2 ? vp.z : vp.w));
    if (y >= a.V) {        // only reachable when every weight is zero
        y = a.V - 1;
        zy = prow[y];
    }
    return true;
}

// The chain's outputs after the draw of token y (probability py) at index `row`:
// the token, its probability, and the padding of the sequence's outputs.
__device__ __forceinline__ void emit_chain(const RejectArgs& a, const SeqCtx& s, int row, int y, double py) {
    const int k = s.kb;
    const size_t ob = s.tb;
    a.out_tokens[ob + row] = y;
    if (a.out_probs) a.out_probs[ob + row] = static_cast<float>(py);
    for (int i = row + 1; i <= k; ++i) {
        a.out_tokens[ob + i] = -1;
        if (a.out_probs) a.out_probs[ob + i] = 0.0f;
    }
    if (a.accept_probs)
        for (int i = row + 1; i < k; ++i) a.accept_probs[s.db + i] = -1.0f;
    a.num_accepted[s.b] = row;
}

// Draw from the weights of this unit (the residual of rows prow, qrow; p when `use_p`
// or for the bonus row), given the running sum `run` before this unit and the
// target t. Only the wavefront owning the crossing unit calls this; emit(y, p(y))
// runs on the lane holding the drawn token.
template <bool kVec4, typename E>
__device__ __forceinline__ void final_scan(const RejectArgs& a, const SeqCtx& s, bool two_rows,
                                           const float* prow, const float* qrow, const SampleCtx& c,
                                           const LoadSums& ls, bool use_p, bool exact, double run, double t,
                                           double invZp, double invZq, double Zp_true, double wscale,
                                           double M_ref, E&& emit) {
    // wscale maps this unit's weights onto the scale of run and t (1, except for
    // the bonus row, whose unit weights are relative to the unit's own maximum);
    // M_ref is the row maximum the emitted probability is taken against.
    const bool residual = two_rows && !use_p;
    auto lv = [&](int i, int j0) -> double {
        double v = 0.0;
        if (!use_p) {
#pragma unroll
            for (int j = 0; j < kWave / 4; ++j) {
                const double2 g = ls[i][j0 + j];
                v += residual ? g.x * invZp - g.y * invZq : g.x;
            }
        } else {                 // zero residual (rare): p-weights of this load, recomputed
#pragma unroll 1
            for (int j = 0; j < kWave / 4; ++j) {
                const int x = s.u * kUnit + i * (kWave * 4) + (j0 + j) * 4;
                double w[4];
                load_weights(two_rows, false, load4<kVec4>(row_rsrc(prow, a.V), a.V, x),
                             two_rows ? load4<kVec4>(row_rsrc(qrow, a.V), a.V, x)
                             : f4{-INFINITY, -INFINITY, -INFINITY, -INFINITY}, c, invZp, invZq, w);
                v += (w[0] + w[1]) + (w[2] + w[3]);
            }
        }
        return v * wscale;
    };
    auto wf = [&](const f4& vp, const f4& vq, double (&w)[4]) {
        load_weights(two_rows, residual, vp, vq, c, invZp, invZq, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] *= wscale;
    };
    int y;
    float zy;
    if (!scan_unit<kVec4>(a, s, prow, qrow, two_rows, exact, run, t, lv, wf, y, zy)) return;
    emit(y, exp_nonpos_f64((static_cast<double>(zy) - M_ref) * c.invT64) / Zp_true);
}

// Reads wave 0's sampling decision and runs the final scan in the owning
// wavefront (every wavefront of the workgroup calls this after the barrier).
template <typename SH>
__device__ __forceinline__ bool read_samp(const RejectArgs& a, const SeqCtx& s, const SH& sh, bool& use_p,
                                          bool& exact, double& run, double& t, double& Z1, double& Z2) {
    const unsigned flags = static_cast<unsigned>(uniform(static_cast<int>(sh.samp.flags)));
    if (flags & kSampAbort) return false;   // the row is not reached: another level draws
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

// SampleCtx of a row pair from its chain statistics: the normalisers the residual
// support and the heavy thresholds are judged with.
__device__ __forceinline__ SampleCtx residual_ctx(const RejectArgs& a, const RowStats& st) {
    SampleCtx c;
    c.Mp = st.Mp;
    c.Mq = st.Mq;
    c.invT = a.invT;
    c.Mp64 = st.Mp;
    c.Mq64 = st.Mq;
    c.invT64 = a.invT64;
    c.tp = heavy_threshold(st.Mp, st.Zp, a.T);
    c.tq = heavy_threshold(st.Mq, st.Zq, a.T);
    c.dn = ln_approx(st.Zp) - ln_approx(st.Zq);
    return c;
}

// The residual round of a rejected candidate's rows p = prow, q = qrow (still in
// registers). Each wavefront turns its unit into the sums A, B of a and b over the
// support {p > q} (judged with the chain statistics in c) and the totals P, Q; wave 0
// sums the workgroup's units by quads, and one exchange gives every workgroup all
// quads' sums, hence the exact normalisers Z_p = sum P, Z_q = sum Q and the residual's
// mass W = sum over quads of max(0, A/Z_p - B/Z_q). With `draw` the draw follows: u_smp
// at position L + 1 + pos, from the residual, or from p when it sums to zero; the
// workgroup holding the crossing quad finds the crossing unit, whose wavefront scans it,
// and emit(y, p(y)) runs on the lane holding the token. Returns false if a wait gave up
// (the error is flagged); Zp, Zq and W come back in every wavefront.
template <bool kVec4, typename SH, typename E>
__device__ __forceinline__ bool residual_round(const RejectArgs& a, const SeqCtx& s, const float* prow,
                                               const float* qrow, int pos, unsigned long long* slots,
                                               const f4 (&xp)[kVecs], const f4 (&xq)[kVecs], const SampleCtx& c,
                                               SH& sh, bool draw, E&& emit, double& Zp_out, double& Zq_out,
                                               double& W_out) {
    const int lane = lane_id();
    const UnitSums us = unit_sums<kVec4, true>(xp, xq, c, prow, qrow, a.V, s.u * kUnit + lane * 4, sh.ls[s.wave]);
    if (lane == 0) sh.usum[s.wave] = make_double4(us.A, us.B, us.P, us.Q);
    __syncthreads();
    if (s.wave == 0) {
        const int nq = quads_of(a.U);
        {   // the workgroup's quads, all at once
            double Au = 0.0, Bu = 0.0, Pu = 0.0, Qu = 0.0;
            if (lane < SH::kW) {
                const double4 v = sh.usum[lane];
                Au = v.x; Bu = v.y; Pu = v.z; Qu = v.w;
            }
            const double Aw = dpp_quad_sum(Au), Bw = dpp_quad_sum(Bu), Pw = dpp_quad_sum(Pu), Qw = dpp_quad_sum(Qu);
            const unsigned pay[kSampSlots] = {hi32(Aw), lo32(Aw), hi32(Bw), lo32(Bw),
                                              hi32(Pw), lo32(Pw), hi32(Qw), lo32(Qw)};
            publish_quads(slots, pay, s.epoch, s.q * (SH::kW / kQuad), SH::kW, nq);
        }
        double u_acc, u_smp;
        verify_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + pos, &u_acc, &u_smp);
        unsigned v[kSampSlots];
        const bool ok = gather<kSampSlots>(slots, nq, s.epoch, a.spin, v);
        // lane l < nq: quad l's sums (zero in the other lanes)
        const double Ag = join64(v[0], v[1]), Bg = join64(v[2], v[3]);
        const double Pg = join64(v[4], v[5]), Qg = join64(v[6], v[7]);
        const double Zp = dpp_wave_sum(Pg), Zq = dpp_wave_sum(Qg);
        const double invZp = 1.0 / Zp, invZq = 1.0 / Zq;
        double Rg = fmax(0.0, Ag * invZp - Bg * invZq);
        double total = dpp_wave_sum(Rg);
        const double W = total;
        bool use_p = false;
        if (!(total > 0.0)) {      // zero residual: draw from p instead
            use_p = true;
            Rg = Pg;
            total = Zp;
        }
        const double t = u_smp * total;
        double run = 0.0;
        bool exact = false;
        int owner = -1;
        if (draw) {
            const int qstar = find_crossing(Rg, 0.0, t, run, exact);
            if (qstar / (SH::kW / kQuad) == s.q) {   // the crossing quad is this workgroup's: find its unit
                const int j = qstar % (SH::kW / kQuad);
                double Ru = 0.0;
                if (lane < kQuad) {
                    const double4 v4 = sh.usum[kQuad * j + lane];
                    Ru = use_p ? v4.z : fmax(0.0, v4.x * invZp - v4.y * invZq);
                }
                bool exact_u;
                owner = kQuad * j + find_crossing(Ru, run, t, run, exact_u);
                exact = exact && exact_u;
            }
        }
        if (lane == 0) {
            sh.samp.owner = owner;
            sh.samp.flags = (use_p ? kSampUseP : 0u) | (exact ? kSampExact : 0u) | (ok ? 0u : kSampError);
            sh.samp.run = run;
            sh.samp.t = t;
            sh.samp.Z1 = Zp;
            sh.samp.Z2 = Zq;
            sh.samp.W = W;
        }
    }
    __syncthreads();
    Zp_out = uniform(sh.samp.Z1);
    Zq_out = uniform(sh.samp.Z2);
    W_out = uniform(sh.samp.W);
    bool use_p, exact;
    double run, t, Zp, Zq;
    if (!read_samp(a, s, sh, use_p, exact, run, t, Zp, Zq)) {
        return !(static_cast<unsigned>(uniform(static_cast<int>(sh.samp.flags))) & kSampError);
    }
    if (draw)
        final_scan<kVec4>(a, s, true, prow, qrow, c, sh.ls[s.wave], use_p, exact, run, t, 1.0 / Zp, 1.0 / Zq, Zp,
                          1.0, c.Mp64, emit);
    return true;
}

// Sampling from the residual of row `row` after its draft was rejected; `st` holds
// the chain statistics of that row.
template <bool kVec4, typename SH>
__device__ __forceinline__ void sample_row(const RejectArgs& a, const SeqCtx& s, int row, const f4 (&xp)[kVecs],
                                           const f4 (&xq)[kVecs], const RowStats& st, SH& sh) {
    const float* prow = s.prow_base + size_t(row) * a.V;
    const float* qrow = s.qrow_base + size_t(row) * a.V;
    double Zp, Zq, W;
    (void)residual_round<kVec4>(a, s, prow, qrow, row, a.samp_slots + size_t(s.b) * a.U * kSampSlots, xp, xq,
                                residual_ctx(a, st), sh, true,
                                [&](int y, double py) { emit_chain(a, s, row, y, py); }, Zp, Zq, W);
}

// One acceptance test: the rows it reads, the candidate, where its uniform comes
// from and where its outputs go (a chain level, or the first child of a tree node).
struct LevelRef {
    const float* prow;
    const float* qrow;
    size_t tok_idx;               // the candidate is draft_tokens[tok_idx]
    int pos;                      // decided position L + 1 + pos
    unsigned stream;              // Philox stream of the acceptance uniform
    unsigned long long* slots;    // this exchange's slots
    size_t acc_idx, out_idx;      // accept_probs index; out_tokens / out_probs index
    long long node_idx;           // out_nodes index (tree), -1: none
    int node;
    bool defer;                   // leave the outputs to the caller (the level may not be reached)
};

// Acceptance test of one candidate from the combined statistics and its two
// logits (loaded while the group was exchanging statistics); workgroup 0 writes
// the outputs of the test.
__device__ __forceinline__ bool accept_test(const RejectArgs& a, const SeqCtx& s, const LevelRef& r,
                                            const RowStats& st, const TokenLogits& tl, float& pd_out,
                                            float& ratio_out) {
    double ep = 0.0, eq = 0.0;   // p and q of the token times Z_p and Z_q
    if (tl.ok) {
        ep = exp_nonpos_f64((static_cast<double>(tl.zp) - st.Mp) * a.invT64);
        eq = exp_nonpos_f64((static_cast<double>(tl.zq) - st.Mq) * a.invT64);
    }
    // u < p/q without a division on the way to the decision: u q Z_p Z_q < p Z_p Z_q.
    // (q = 0 makes the ratio +inf when p > 0 and 0 when p = 0, as the product form does.)
    const bool accepted = uniform(static_cast<int>(tl.u_acc * (eq * st.Zp) < ep * st.Zq)) != 0;
    const double p_d = ep / st.Zp, q_d = eq / st.Zq;
    const double ratio = (q_d > 0.0) ? p_d / q_d : (p_d > 0.0 ? INFINITY : 0.0);
    pd_out = static_cast<float>(p_d);
    ratio_out = static_cast<float>(fmin(1.0, ratio));
    if (!r.defer && s.q == 0 && lane_id() == 0) {
        if (a.accept_probs) a.accept_probs[r.acc_idx] = static_cast<float>(fmin(1.0, ratio));
        if (accepted) {
            a.out_tokens[r.out_idx] = tl.tok;
            if (a.out_probs) a.out_probs[r.out_idx] = static_cast<float>(p_d);
            if (r.node_idx >= 0 && a.out_nodes) a.out_nodes[r.node_idx] = r.node;
        }
    }
    return accepted;
}

// Level `row` of the chain (rows p_row and q_row): every wavefront reduces its
// unit, wave 0 combines the workgroup's units by quads, publishes one pair per quad
// and gathers the sequence's quads, combines those in quad order and takes the
// acceptance test; every workgroup reaches the same decision from the same bits.
// Returns the result flags (kResAccepted, kResError) and the row's statistics in
// `st`; with r.defer the outputs of the test are left in sh.res for the caller.
// kSeq: the workgroup's quads one after another in lanes 0..3 instead of all at
// once (the same bits; it leaves the tree walk, which is short of registers, with
// fewer spills).
template <bool kVec4, bool kSeq = false, typename SH>
__device__ __forceinline__ unsigned level_core(const RejectArgs& a, const SeqCtx& s, const LevelRef& r,
                                               f4 (&xp)[kVecs], f4 (&xq)[kVecs], RowStats& st, SH& sh,
                                               bool& counted) {
    const float* prow = r.prow;
    const float* qrow = r.qrow;
    load_unit<kVec4, true>(row_rsrc(prow, a.V), row_rsrc(qrow, a.V), a.V, s.u, xp, xq);
    // wave 0 takes the acceptance test: the draft token and its two logits are read
    // behind the unit's loads, through the scalar cache (uniform addresses into
    // read-only inputs), so that waiting for them waits for no vector load and
    // holds none back; they have long arrived when the group's statistics are in
    TokenLogits tok;
    tok.tok = 0;
    tok.ok = false;
    float ztp = 0.0f, ztq = 0.0f;
    if (s.wave == 0) {
        tok.tok = load_uniform(a.draft_tokens, r.tok_idx);
        tok.ok = tok.tok >= 0 && tok.tok < a.V;
        if (tok.ok) {
            ztp = load_uniform(prow, tok.tok);
            ztq = load_uniform(qrow, tok.tok);
        }
    }
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
        const int nq = quads_of(a.U);
        constexpr int kLanes = kSeq ? kQuad : SH::kW;
#pragma unroll 1
        for (int j = 0; j < SH::kW / kLanes; ++j) {   // unit j * kLanes + i in lane i, a quad's pair in lane 4m
            float mpw = -INFINITY, mqw = -INFINITY;
            double zpw = 0.0, zqw = 0.0;
            if (lane < kLanes) {
                const UnitStat u = sh.unit[j * kLanes + lane];
                mpw = u.Mp; mqw = u.Mq; zpw = u.Zp; zqw = u.Zq;
            }
            float Mp_w, Mq_w;
            double Zp_w, Zq_w;
            combine_quad(mpw, zpw, a.invT64, Mp_w, Zp_w);
            combine_quad(mqw, zqw, a.invT64, Mq_w, Zq_w);
            const unsigned pay[kStatSlots] = {__builtin_bit_cast(unsigned, Mp_w), __builtin_bit_cast(unsigned, Mq_w),
                                              hi32(Zp_w), lo32(Zp_w), hi32(Zq_w), lo32(Zq_w)};
            publish_quads(r.slots, pay, s.epoch, s.q * (SH::kW / kQuad) + j * (kLanes / kQuad), kLanes, nq);
        }
        TokenLogits tl = tok;
        double u_smp;
        stream_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + r.pos, r.stream, &tl.u_acc, &u_smp);
        unsigned v[kStatSlots];
        unsigned flags = 0;
        float pd = 0.0f, ratio = 0.0f;
        if (gather<kStatSlots>(r.slots, nq, s.epoch, a.spin, v)) {
            count_group(a, s, counted);
            tl.zp = uniform(ztp);
            tl.zq = uniform(ztq);
            const bool have = lane < nq;
            combine_pair(have ? __builtin_bit_cast(float, v[0]) : -INFINITY, have ? join64(v[2], v[3]) : 0.0,
                         a.invT64, st.Mp, st.Zp);
            combine_pair(have ? __builtin_bit_cast(float, v[1]) : -INFINITY, have ? join64(v[4], v[5]) : 0.0,
                         a.invT64, st.Mq, st.Zq);
            if (accept_test(a, s, r, st, tl, pd, ratio)) flags |= kResAccepted;
        } else {
            count_group(a, s, counted);
            st.Mp = st.Mq = 0.0f;
            st.Zp = st.Zq = 1.0;
            flags |= kResError;
        }
        if (lane == 0) sh.res = LevelRes{flags, st.Mp, st.Mq, st.Zp, st.Zq, tl.tok, pd, ratio};
    }
    __syncthreads();
    st.Mp = uniform(sh.res.Mp);
    st.Mq = uniform(sh.res.Mq);
    st.Zp = uniform(sh.res.Zp);
    st.Zq = uniform(sh.res.Zq);
    return static_cast<unsigned>(uniform(static_cast<int>(sh.res.flags)));
}

// Level `row` of the chain (rows p_row and q_row, draft row, position L + 1 + row).
template <bool kVec4, typename SH>
__device__ __forceinline__ unsigned level_step(const RejectArgs& a, const SeqCtx& s, int row, f4 (&xp)[kVecs],
                                               f4 (&xq)[kVecs], RowStats& st, SH& sh, bool& counted,
                                               bool defer = false) {
    LevelRef r;
    r.prow = s.prow_base + size_t(row) * a.V;
    r.qrow = s.qrow_base + size_t(row) * a.V;
    r.tok_idx = s.db + row;
    r.pos = row;
    r.stream = 0u;
    r.slots = a.stat_slots + (size_t(s.b) * (a.k + 1) + row) * a.U * kStatSlots;
    r.acc_idx = s.db + row;
    r.out_idx = s.tb + row;
    r.node_idx = -1;
    r.node = 0;
    r.defer = defer;
    return level_core<kVec4>(a, s, r, xp, xq, st, sh, counted);
}

// The bonus row p_k after k acceptances, with one exchange: each wavefront weighs
// its unit against the unit's own maximum M_u (heavy logits judged with the
// unit's own normaliser, a superset of the row's heavy set); wave 0 rescales its
// units to each quad's maximum and publishes (sum, maximum) per quad; the gathered
// pairs are rescaled to the row maximum M, which also gives the row's Z.
// With gate_dec, the row is drawn only if the decisions of levels 0 .. gate_levels - 1
// (published by other groups) all accept; otherwise the call returns without output.
template <bool kVec4, bool kSeq = false, typename SH, typename E>
__device__ __forceinline__ void bonus_core(const RejectArgs& a, const SeqCtx& s, const float* prow, int pos,
                                           unsigned long long* slots, f4 (&xp)[kVecs], f4 (&xq)[kVecs],
                                           SH& sh, bool& counted, E&& emit,
                                           unsigned long long* gate_dec = nullptr, int gate_levels = 0) {
    const __amdgpu_buffer_rsrc_t rp = row_rsrc(prow, a.V);
    load_unit<kVec4, false>(rp, rp, a.V, s.u, xp, xq);
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
    // A unit with no finite logit (all past V) has Z_u = 0: its threshold is +inf, so that
    // no padding element is classified heavy.
    c.tp = unit_heavy_threshold(Mu, Zu, a.T);
    c.tq = INFINITY;
    c.dn = 0.0f;
    const int lane = lane_id();
    const UnitSums us = unit_sums<kVec4, false>(xp, xq, c, prow, prow, a.V, s.u * kUnit + lane * 4, sh.ls[s.wave]);
    const double Mu64 = Mu;
    if (lane == 0) sh.usum[s.wave] = make_double4(us.P, Mu64, 0.0, 0.0);
    __syncthreads();
    if (s.wave == 0) {
        const int nq = quads_of(a.U);
        constexpr int kLanes = kSeq ? kQuad : SH::kW;
#pragma unroll 1
        for (int j = 0; j < SH::kW / kLanes; ++j) {   // (weight sum, maximum) of each quad
            double Pu = 0.0, Mv = -INFINITY;
            if (lane < kLanes) {
                const double4 v4 = sh.usum[j * kLanes + lane];
                Pu = v4.x;
                Mv = v4.y;
            }
            const double Mw = dpp_quad_max(static_cast<float>(Mv));
            const double Ww = dpp_quad_sum((Pu > 0.0) ? Pu * exp_nonpos_f64((Mv - Mw) * a.invT64) : 0.0);
            const unsigned pay[4] = {hi32(Ww), lo32(Ww), hi32(Mw), lo32(Mw)};
            publish_quads(slots, pay, s.epoch, s.q * (SH::kW / kQuad) + j * (kLanes / kQuad), kLanes, nq);
        }
        double u_acc, u_smp;
        verify_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + pos, &u_acc, &u_smp);
        unsigned v[4];
        bool ok = gather<4>(slots, nq, s.epoch, a.spin, v);
        count_group(a, s, counted);
        bool reached = true;
        if (gate_dec) {
            unsigned dv[kDecSlots];
            ok = gather_at<kDecSlots>(gate_dec, kMaxLevels, 0, gate_levels, s.epoch, a.spin, dv) && ok;
            reached = __all(lane >= gate_levels || dv[0] == kDecAccepted);
            if (ok && reached && s.q == 0 && lane < gate_levels) level_outputs(a, s, lane, dv[1], dv[2]);
        }
        const bool have = lane < nq;
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
        if (qstar / (SH::kW / kQuad) == s.q) {   // the crossing quad is this workgroup's: find its unit
            const int j = qstar % (SH::kW / kQuad);
            double Wu = 0.0;
            if (lane < kQuad) {
                const double4 v4 = sh.usum[kQuad * j + lane];
                Wu = (v4.x > 0.0) ? v4.x * exp_nonpos_f64((v4.y - M) * a.invT64) : 0.0;
            }
            bool exact_u;
            owner = kQuad * j + find_crossing(Wu, run, t, run, exact_u);
            exact = exact && exact_u;
        }
        if (lane == 0) {
            sh.samp.owner = owner;
            sh.samp.flags = (exact ? kSampExact : 0u) | (ok ? 0u : kSampError) | (ok && !reached ? kSampAbort : 0u);
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
    const LoadSums& ls = sh.ls[s.wave];
    auto lv = [&](int i, int j0) -> double {
        double v = 0.0;
#pragma unroll
        for (int j = 0; j < kWave / 4; ++j) v += ls[i][j0 + j].x;
        return v * wscale;
    };
    auto wf = [&](const f4& vp, const f4& vq, double (&w)[4]) {
        load_weights(false, false, vp, vq, c, 1.0 / Z, 1.0, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] *= wscale;
    };
    int y;
    float zy;
    if (!scan_unit<kVec4>(a, s, prow, prow, false, exact, run, t, lv, wf, y, zy)) return;
    emit(y, exp_nonpos_f64((static_cast<double>(zy) - M) * c.invT64) / Z);
}

// The bonus row p_k after k acceptances.
template <bool kVec4, typename SH>
__device__ __forceinline__ void bonus_row(const RejectArgs& a, const SeqCtx& s, f4 (&xp)[kVecs], f4 (&xq)[kVecs],
                                          SH& sh, bool& counted) {
    const int row = s.kb;
    bonus_core<kVec4>(a, s, s.prow_base + size_t(row) * a.V, row,
                      a.samp_slots + size_t(s.b) * a.U * kSampSlots, xp, xq, sh, counted,
                      [&](int y, double py) { emit_chain(a, s, row, y, py); });
}


// ---------------------------------------------------------------- tree verification
//
// "ReSpec: Towards Optimizing Speculative Decoding in Reinforcement Learning
// Systems" (talk notes), GAP 1: speculation with a branching factor, the drafts
// forming a tree that one target pass checks. The walk is multi-candidate
// speculative sampling (SpecInfer, Miao et al. 2024): at node v the children are
// tested in index order against a running residual r (r = p_v first, then
// r = max(0, r - q_v) normalised after each rejection, unchanged if that sums to
// zero); an accepted child continues the walk, a node whose children are all
// rejected ends it with a draw from r, and a leaf ends it with a bonus draw from
// p_v. The first child is an ordinary level of the chain (same uniform, same
// statistics); candidate i >= 2 takes word 0 of Philox stream i.

// The residual of a node after its first child was rejected, in closed form. The
// candidates of a node share the draft distribution q = q_v, so if r = max(0, p - c q) / W
// (with W its sum), max(0, r - q) = max(0, p - (c + W) q) / W on every logit (where
// p <= c q both sides are 0): after each rejection the residual is max(0, p - c q)
// normalised, with c_1 = 1 and c_{j+1} = c_j + W_j, W_j = sum max(0, p - c_j q); a
// residual that sums to zero leaves (c, W) as they were. c = 0, W = 1 is r = p.
struct TreeRounds {
    double iZp, iZq;   // exact normalisers of the node's rows
    double c, W, iW;   // r = max(0, p - c q) / W
};

// r for one logit with unnormalised weights a (p) and b (q).
__device__ __forceinline__ double tree_r(const TreeRounds& R, double a, double b) {
    return fmax(0.0, a * R.iZp - R.c * (b * R.iZq)) * R.iW;
}

// One pass over the unit in registers (rows p_v, q_v): f(a, b) -> (w1, w2) for every
// logit, with a = e^{(z_p - M_p)/T}, b = e^{(z_q - M_q)/T} (fp64 for heavy logits,
// compensated fp32 otherwise, as for the chain's residual); the per-load w1 sums go
// to the wavefront's LDS slab. Returns the wavefront's (sum w1, sum w2).
template <bool kVec4, typename F>
__device__ __forceinline__ double2 tree_unit_pass(const f4 (&xp)[kVecs], const f4 (&xq)[kVecs], const SampleCtx& c,
                                                  const float* prow, const float* qrow, int V, int base,
                                                  LoadSums& ls, F&& f) {
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rp = row_rsrc(prow, V), rq = row_rsrc(qrow, V);
    HeavyBits hb = heavy_bits<kVecs>(true, xp, xq, c.tp, c.tq);
    HeavyRound hr;
    heavy_fetch(true, rp, rq, V, base, hb, hr);
    double S1 = 0.0, S2 = 0.0;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
        float la[4], lb[4];
        bool in_s[4], h[4];
        light_weights(true, xp[i], xq[i], c, la, lb, in_s, h);   // heavy logits come out as 0
        double l1 = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double2 w = f(static_cast<double>(la[e]), static_cast<double>(lb[e]));
            l1 += w.x;
            S2 += w.y;
        }
        S1 += l1;
        ls[i][lane] = make_double2(l1, 0.0);
    }
    auto add = [&](int i, double va, double vb, bool) {
        const double2 w = f(va, vb);
        S1 += w.x;
        S2 += w.y;
        ls[i][lane].x += w.x;
    };
    heavy_weigh(true, c, hr, add);
    while (__any((hb.lo | hb.hi) != 0u)) {
        heavy_fetch(true, rp, rq, V, base, hb, hr);
        heavy_weigh(true, c, hr, add);
    }
    return make_double2(dpp_wave_sum(S1), dpp_wave_sum(S2));
}

enum : int { kDrawn = 0, kDrawZero = 1, kDrawError = 2 };

// One pass and one exchange: the group's totals (T1, T2) of f's two weights, in
// every wavefront; with `draw`, also the draw from the w1 weights with u_smp at
// position L + 1 + pos (emit(y, p_v(y)) runs on the lane holding the token), or
// kDrawZero, without drawing, if they sum to zero. The exchange goes through quads
// of units, as the chain's does, so the result is the same for any workgroup size.
template <bool kVec4, typename SH, typename F, typename E>
__device__ __forceinline__ int tree_round(const RejectArgs& a, const SeqCtx& s, const f4 (&xp)[kVecs],
                                          const f4 (&xq)[kVecs], const SampleCtx& c, double iZp, const float* prow,
                                          const float* qrow, unsigned long long* slots, int pos, SH& sh,
                                          bool draw, F&& f, E&& emit, double& T1, double& T2) {
    const int lane = lane_id();
    const double2 ws = tree_unit_pass<kVec4>(xp, xq, c, prow, qrow, a.V, s.u * kUnit + lane * 4, sh.ls[s.wave], f);
    if (lane == 0) sh.usum[s.wave] = make_double4(ws.x, ws.y, 0.0, 0.0);
    __syncthreads();
    if (s.wave == 0) {
        const int nq = quads_of(a.U);
        double u1 = 0.0, u2 = 0.0;
        if (lane < SH::kW) {
            const double4 v = sh.usum[lane];
            u1 = v.x;
            u2 = v.y;
        }
        const double w1 = dpp_quad_sum(u1), w2 = dpp_quad_sum(u2);
        const unsigned pay[4] = {hi32(w1), lo32(w1), hi32(w2), lo32(w2)};
        publish_quads(slots, pay, s.epoch, s.q * (SH::kW / kQuad), SH::kW, nq);
        double u_acc, u_smp;
        verify_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + pos, &u_acc, &u_smp);
        unsigned v[4];
        const bool ok = gather<4>(slots, nq, s.epoch, a.spin, v);
        const double Wg = join64(v[0], v[1]);      // lane l < nq: quad l's sums (zero in the others)
        const double t1 = dpp_wave_sum(Wg), t2 = dpp_wave_sum(join64(v[2], v[3]));
        const double t = u_smp * t1;
        double run = 0.0;
        bool exact = false;
        int owner = -1;
        unsigned flags = ok ? 0u : kSampError;
        if (draw) {
            if (!(t1 > 0.0)) {
                flags |= kSampUseP;                   // nothing to draw from
            } else {
                const int qstar = find_crossing(Wg, 0.0, t, run, exact);
                if (qstar / (SH::kW / kQuad) == s.q) {   // the crossing quad is this workgroup's: find its unit
                    const int j = qstar % (SH::kW / kQuad);
                    const double Ru = (lane < kQuad) ? sh.usum[kQuad * j + lane].x : 0.0;
                    bool exact_u;
                    owner = kQuad * j + find_crossing(Ru, run, t, run, exact_u);
                    exact = exact && exact_u;
                }
            }
        }
        if (lane == 0) {
            sh.samp.owner = owner;
            sh.samp.flags = flags | (exact ? kSampExact : 0u);
            sh.samp.run = run;
            sh.samp.t = t;
            sh.samp.Z1 = t1;
            sh.samp.Z2 = t2;
        }
    }
    __syncthreads();
    const unsigned flags = static_cast<unsigned>(uniform(static_cast<int>(sh.samp.flags)));
    T1 = uniform(sh.samp.Z1);
    T2 = uniform(sh.samp.Z2);
    if (flags & kSampError) return kDrawError;
    if (!draw) return kDrawn;
    if (flags & kSampUseP) return kDrawZero;
    if (uniform(sh.samp.owner) != s.wave) return kDrawn;
    const double run = uniform(sh.samp.run), t = uniform(sh.samp.t);
    const LoadSums& ls = sh.ls[s.wave];
    auto lv = [&](int i, int j0) -> double {
        double v = 0.0;
#pragma unroll
        for (int j = 0; j < kWave / 4; ++j) v += ls[i][j0 + j].x;
        return v;
    };
    auto wf = [&](const f4& vp, const f4& vq, double (&w)[4]) {
        float la[4], lb[4];
        bool in_s[4], h[4];
        light_weights(true, vp, vq, c, la, lb, in_s, h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double va = h[e] ? exp_nonpos_f64((static_cast<double>(vp[e]) - c.Mp64) * c.invT64) : la[e];
            const double vb = h[e] ? exp_nonpos_f64((static_cast<double>(vq[e]) - c.Mq64) * c.invT64) : lb[e];
            w[e] = f(va, vb).x;
        }
    };
    int y;
    float zy;
    if (scan_unit<kVec4>(a, s, prow, qrow, true, (flags & kSampExact) != 0u, run, t, lv, wf, y, zy))
        emit(y, exp_nonpos_f64((static_cast<double>(zy) - c.Mp64) * c.invT64) * iZp);
    return kDrawn;
}

// The test of a node's i-th child (i >= 2) against the residual the rounds leave:
// accept iff u < r(x) / q(x), u = word 0 of stream i. Every workgroup takes it from
// the same bits; workgroup 0 writes its outputs. Returns the decision.
template <typename SH>
__device__ __forceinline__ bool tree_candidate(const RejectArgs& a, const SeqCtx& s, const SampleCtx& c,
                                               const TreeRounds& R, const float* prow, const float* qrow, int node,
                                               int i, int depth, SH& sh) {
    if (s.wave == 0) {
        const int N = a.k;
        const size_t nb = size_t(s.b) * N;
        const int x = load_uniform(a.draft_tokens, nb + node - 1);
        const bool ok = x >= 0 && x < a.V;
        double av = 0.0, bv = 0.0;   // out-of-range ids (a broken precondition) are rejected
        if (ok) {
            av = exp_nonpos_f64((static_cast<double>(load_uniform(prow, x)) - c.Mp64) * c.invT64);
            bv = exp_nonpos_f64((static_cast<double>(load_uniform(qrow, x)) - c.Mq64) * c.invT64);
        }
        const double rx = tree_r(R, av, bv), qx = bv * R.iZq;
        double u0, u1;
        stream_uniforms(a.seed, s.sid, int64_t(s.L) + 1 + depth, static_cast<uint32_t>(i), &u0, &u1);
        const bool accepted = u0 * qx < rx;   // q = 0: accepted iff r > 0, as a ratio of +inf
        if (s.q == 0 && lane_id() == 0) {
            const double ratio = (qx > 0.0) ? rx / qx : (rx > 0.0 ? INFINITY : 0.0);
            if (a.accept_probs) a.accept_probs[nb + node - 1] = static_cast<float>(fmin(1.0, ratio));
            if (accepted) {
                const size_t ob = size_t(s.b) * (N + 1);
                a.out_tokens[ob + depth] = x;
                if (a.out_probs) a.out_probs[ob + depth] = static_cast<float>(av * R.iZp);
                if (a.out_nodes) a.out_nodes[nb + depth] = node;
            }
        }
        if (lane_id() == 0) sh.res.flags = accepted ? kResAccepted : 0u;
    }
    __syncthreads();
    return (static_cast<unsigned>(uniform(static_cast<int>(sh.res.flags))) & kResAccepted) != 0u;
}

// The tree's outputs after the final draw of token y (probability py) at index
// `depth`: the token, the padding, the untested nodes and the accepted length.
__device__ __forceinline__ void emit_tree(const RejectArgs& a, const SeqCtx& s, int depth, unsigned tested, int y,
                                          double py) {
    const int N = a.k;
    const size_t ob = size_t(s.b) * (N + 1), nb = size_t(s.b) * N;
    a.out_tokens[ob + depth] = y;
    if (a.out_probs) a.out_probs[ob + depth] = static_cast<float>(py);
    for (int i = depth + 1; i <= N; ++i) {
        a.out_tokens[ob + i] = -1;
        if (a.out_probs) a.out_probs[ob + i] = 0.0f;
    }
    if (a.out_nodes)
        for (int i = depth; i < N; ++i) a.out_nodes[nb + i] = -1;
    if (a.accept_probs)
        for (int n = 1; n <= N; ++n)
            if (!((tested >> n) & 1u)) a.accept_probs[nb + n - 1] = -1.0f;
    a.num_accepted[s.b] = depth;
}

// The walk of one sequence's tree (nodes 0 .. N, rows [N+1][V] of target and draft).
template <bool kVec4, typename SH>
__device__ __forceinline__ void tree_walk(const RejectArgs& a, SeqCtx& s, f4 (&xp)[kVecs], f4 (&xq)[kVecs],
                                          SH& sh, bool& counted) {
    const int N = a.k;
    const size_t b = s.b;
    const float* tbase = a.target + b * (N + 1) * a.V;
    const float* dbase = a.draft + b * (N + 1) * a.V;
    // one block of kSampSlots x U slots per exchange (unit-level exchanges fill it,
    // workgroup-level ones use its first kSampSlots x Q)
    unsigned long long* slots0 = a.tree_slots + b * kTreeEx * kSampSlots * a.U;
    auto slot = [&](int e) { return slots0 + size_t(e) * kSampSlots * a.U; };
    int ex = 0, v = 0, depth = 0;
    unsigned tested = 0u;
    // A broken tree ends the sequence with num_accepted = -1. A failure before the group's first
    // exchange must still count the group when this is its last sequence, or the call's epoch
    // would never be stored (every workgroup of the group fails alike, so none exchanges after).
    auto fail = [&]() {
        flag_error(a, s);
        if (s.wave == 0 && s.b + a.groups >= a.B) count_group(a, s, counted);   // wave 0 counts, as after a gather
    };
    for (int n = 1; n <= N; ++n) {   // every parent precedes its node
        const int par = load_uniform(a.parents, b * N + n - 1);
        if (par < 0 || par >= n) {
            fail();
            return;
        }
    }
    for (;;) {
        // children of v in index order, four bits each (scalar loads of the parents)
        unsigned chp = 0u;
        int m = 0;
        for (int n = v + 1; n <= N; ++n) {
            if (load_uniform(a.parents, b * N + n - 1) == v) {
                if (m < kMaxBranch) chp |= static_cast<unsigned>(n) << (4 * m);
                ++m;
            }
        }
        if (m > kMaxBranch || ex + 4 + m > kTreeEx) {   // outside the documented shapes
            fail();
            return;
        }
        const float* prow = tbase + size_t(v) * a.V;
        auto emit = [&](int y, double py) { emit_tree(a, s, depth, tested, y, py); };
        if (m == 0) {   // a leaf: the bonus draw from p_v
            bonus_core<kVec4, true>(a, s, prow, depth, slot(ex++), xp, xq, sh, counted, emit);
            return;
        }
        const float* qrow = dbase + size_t(v) * a.V;
        const int c1 = static_cast<int>(chp & 15u);
        LevelRef r;
        r.prow = prow;
        r.qrow = qrow;
        r.tok_idx = b * N + c1 - 1;
        r.pos = depth;
        r.stream = 0u;
        r.slots = slot(ex++);
        r.acc_idx = b * N + c1 - 1;
        r.out_idx = b * (N + 1) + depth;
        r.node_idx = static_cast<long long>(b * N + depth);
        r.node = c1;
        r.defer = false;
        RowStats st;
        const unsigned res = level_core<kVec4, true>(a, s, r, xp, xq, st, sh, counted);
        tested |= 1u << c1;
        if (res & kResError) {
            flag_error(a, s);
            return;
        }
        if (res & kResAccepted) {
            v = c1;
            ++depth;
            continue;
        }
        // The first child was rejected. The chain's residual round gives the exact
        // normalisers and W_1 = sum max(0, p - q) in one pass and one exchange; with a single
        // child it also draws (as a rejected chain level does). Each later rejection costs one
        // pass over the unit for the next residual's mass, and the draw after the last child
        // one more (two if that residual sums to zero, which leaves r as it was).
        const SampleCtx c = residual_ctx(a, st);
        double Zp, Zq, W1;
        if (!residual_round<kVec4>(a, s, prow, qrow, depth, slot(ex++), xp, xq, c, sh, m == 1, emit, Zp, Zq, W1))
            return;
        if (m == 1) return;
        TreeRounds R;
        R.iZp = 1.0 / Zp;
        R.iZq = 1.0 / Zq;
        R.c = (W1 > 0.0) ? 1.0 : 0.0;
        R.W = (W1 > 0.0) ? W1 : 1.0;
        R.iW = 1.0 / R.W;
        bool moved = false;
        for (int i = 2;; ++i) {   // candidate i, 1-based; i = m + 1 is the draw
            if (i <= m) {
                const int ci = static_cast<int>((chp >> (4 * (i - 1))) & 15u);
                tested |= 1u << ci;
                if (tree_candidate(a, s, c, R, prow, qrow, ci, i, depth, sh)) {
                    v = ci;
                    ++depth;
                    moved = true;
                    break;
                }
            }
            const bool draw = i >= m;
            const double cn = R.c + R.W;
            auto f = [&](double av, double bv) { return make_double2(fmax(0.0, av * R.iZp - cn * (bv * R.iZq)), 0.0); };
            double T1, T2;
            int d = tree_round<kVec4>(a, s, xp, xq, c, R.iZp, prow, qrow, slot(ex++), depth, sh, draw, f, emit, T1,
                                      T2);
            if (d == kDrawZero) {   // the residual after the last rejection sums to zero: draw from r
                auto g = [&](double av, double bv) {
                    return make_double2(fmax(0.0, av * R.iZp - R.c * (bv * R.iZq)), 0.0);
                };
                d = tree_round<kVec4>(a, s, xp, xq, c, R.iZp, prow, qrow, slot(ex++), depth, sh, true, g, emit, T1,
                                      T2);
                if (d == kDrawZero) d = kDrawError;   // r has positive mass: cannot happen
            }
            if (d == kDrawError) {
                flag_error(a, s);
                return;
            }
            if (draw) return;
            if (T1 > 0.0) {
                R.c = cn;
                R.W = T1;
                R.iW = 1.0 / T1;
            }
        }
        if (moved) continue;
        return;
    }
}

template <bool kVec4, int W>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void reject_tree_kernel(RejectArgs a) {
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
    s.u = q * W + s.wave;
    {
        const unsigned last = __hip_atomic_load(a.ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.epoch = (last + 1u == 0u) ? 1u : last + 1u;
    }
    bool counted = q != 0;
    __shared__ SharedT<W> sh;
    f4 xp[kVecs], xq[kVecs];
    for (int b = group; b < a.B; b += a.groups) {
        s.b = b;
        s.kb = a.k;
        s.tb = size_t(b) * (a.k + 1);
        s.db = size_t(b) * a.k;
        s.sid = load_uniform(a.seq_ids, b);
        s.L = load_uniform(a.seq_lens, b);
        tree_walk<kVec4>(a, s, xp, xq, sh, counted);
    }
}

// W unit wavefronts per workgroup: 8 (one workgroup per CU) when the batch fills the
// device in one round of them, 4 otherwise (a sequence over twice as many CUs when
// there are CUs to spare, which shortens every step of a sequence's serial chain;
// two sequences' workgroups per CU when the batch takes several rounds).
template <bool kVec4, int W>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void reject_kernel(RejectArgs a) {
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
    s.u = q * W + s.wave;
    {
        const unsigned last = __hip_atomic_load(a.ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.epoch = (last + 1u == 0u) ? 1u : last + 1u;
    }
    bool counted = q != 0;   // workgroup 0's wave 0 counts the group
    __shared__ SharedT<W> sh;
    f4 xp[kVecs], xq[kVecs];
    // Sequence g first; the sequences past the first `groups` go to the groups as
    // they finish (a sequence's chain takes one to four levels, so a fixed share
    // could pair two long chains): wave 0 of a group's workgroup 0 takes a ticket
    // from a call-wide counter and publishes the group's next sequence in its slot,
    // tagged with the call's epoch and the round; the group's other workgroups read
    // it there. The last group to finish resets the counters for the next call.
    const bool queued = a.B > a.groups;
    int b = group;
    for (int round = 1; b < a.B; ++round) {
        s.b = b;
        if (a.cu) {   // ragged: k_b drafts, rows packed by the offsets
            const int c0 = load_uniform(a.cu, b), c1 = load_uniform(a.cu, size_t(b) + 1);
            s.kb = min(max(c1 - c0, 0), a.k);
            s.db = static_cast<size_t>(c0);
            s.tb = static_cast<size_t>(c0) + b;
        } else {
            s.kb = a.k;
            s.db = size_t(b) * a.k;
            s.tb = size_t(b) * (a.k + 1);
        }
        s.prow_base = a.target + s.tb * a.V;
        s.qrow_base = a.draft + s.db * a.V;
        // scalar loads, first waited for at the first acceptance test
        s.sid = load_uniform(a.seq_ids, b);
        s.L = load_uniform(a.seq_lens, b);
        RowStats st;
        bool done = false;
        for (int j = 0; j < s.kb && !done; ++j) {
            const unsigned res = level_step<kVec4>(a, s, j, xp, xq, st, sh, counted);
            if (res & kResError) {
                flag_error(a, s);
                done = true;
            } else if (!(res & kResAccepted)) {
                sample_row<kVec4>(a, s, j, xp, xq, st, sh);
                done = true;
            }
        }
        if (!done) bonus_row<kVec4>(a, s, xp, xq, sh, counted);
        if (!queued) break;
        if (s.wave == 0) {
            const int lane = lane_id();
            unsigned long long* slot = a.next_slots + group;
            int nb = -1;
            if (q == 0) {
                unsigned t = 0;
                if (lane == 0) t = __hip_atomic_fetch_add(a.ctl + kCtlQueue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                t = static_cast<unsigned>(uniform(static_cast<int>(t)));
                nb = (static_cast<long long>(a.groups) + t < a.B) ? a.groups + static_cast<int>(t) : a.B;
                if (lane == 0) slot_store(slot, (static_cast<unsigned>(round) << 16) | static_cast<unsigned>(nb), s.epoch);
            } else {
                for (unsigned it = 0; it < a.spin; ++it) {
                    const unsigned long long v = slot_load(slot);
                    const unsigned pay = static_cast<unsigned>(v >> 32);
                    if (static_cast<unsigned>(v) == s.epoch && (pay >> 16) == static_cast<unsigned>(round)) {
                        nb = static_cast<int>(pay & 0xFFFFu);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(4);
                }
                nb = uniform(nb);
            }
            if (lane == 0) sh.next = nb;
        }
        __syncthreads();
        b = uniform(sh.next);
        if (b < 0) {   // the wait ran out (only if the group were not resident at once)
            if (s.wave == 0 && lane_id() == 0)
                __hip_atomic_fetch_or(a.ctl + kCtlError, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
    if (queued && q == 0 && s.wave == 0 && lane_id() == 0) {
        const unsigned f = __hip_atomic_fetch_add(a.ctl + kCtlFinished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (f + 1 == static_cast<unsigned>(a.groups)) {   // every group has taken its last ticket
            __hip_atomic_store(a.ctl + kCtlQueue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.ctl + kCtlFinished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Small batches, k >= 1: the levels of a sequence run at once instead of one after
// another, each on a group of its own (group g: sequence g / (k + 1), level
// g % (k + 1); level k_b is the bonus row, and with ragged draft lengths the
// groups past a sequence's k_b only count themselves). Every group computes its row pair's
// statistics and takes its acceptance test exactly as the chain does, then
// publishes the decision; a level drawn from is the first rejected one, or the
// bonus row if none is, and only the group of that level samples. The other groups
// of levels past the first rejection finish without output. Rows after the first
// rejection are read, which the chain avoids, but at these batch sizes the device
// is far from its bandwidth and the serial exchanges are what cost. The arithmetic
// of every level is the chain's, so the outputs are the same bits.
template <bool kVec4, int W>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void reject_levels_kernel(
    RejectArgs a) {
    const int w = blockIdx.x;
    const int group = w / a.Q, q = w % a.Q;
    const int b = group / (a.k + 1), j = group % (a.k + 1);
    SeqCtx s;
    s.q = q;
    s.wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    s.u = q * W + s.wave;
    {
        const unsigned last = __hip_atomic_load(a.ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s.epoch = (last + 1u == 0u) ? 1u : last + 1u;
    }
    bool counted = q != 0;   // workgroup 0's wave 0 counts the group
    __shared__ SharedT<W> sh;
    __shared__ int s_reached;
    f4 xp[kVecs], xq[kVecs];
    s.b = b;
    if (a.cu) {   // ragged: k_b drafts, rows packed by the offsets (groups j > k_b have no level)
        const int c0 = load_uniform(a.cu, b), c1 = load_uniform(a.cu, size_t(b) + 1);
        s.kb = min(max(c1 - c0, 0), a.k);
        s.db = static_cast<size_t>(c0);
        s.tb = static_cast<size_t>(c0) + b;
    } else {
        s.kb = a.k;
        s.db = size_t(b) * a.k;
        s.tb = size_t(b) * (a.k + 1);
    }
    s.prow_base = a.target + s.tb * a.V;
    s.qrow_base = a.draft + s.db * a.V;
    s.sid = load_uniform(a.seq_ids, b);
    s.L = load_uniform(a.seq_lens, b);
    unsigned long long* dec = a.dec_slots + size_t(b) * kDecSlots * kMaxLevels;
    const int lane = lane_id();
    if (j > s.kb) {   // past this sequence's drafts: nothing to do but be counted
        if (s.wave == 0) count_group(a, s, counted);
        return;
    }
    if (j == s.kb) {   // the bonus row, drawn if every level accepts
        bonus_core<kVec4>(a, s, s.prow_base + size_t(j) * a.V, j, a.bonus_slots + size_t(b) * a.U * 4, xp, xq, sh,
                          counted, [&](int y, double py) { emit_chain(a, s, j, y, py); }, dec, s.kb);
        return;
    }
    RowStats st;
    const unsigned res = level_step<kVec4>(a, s, j, xp, xq, st, sh, counted, true);
    const float pd = uniform(sh.res.pd), ratio = uniform(sh.res.ratio);
    const bool accepted = (res & kResAccepted) != 0;   // false on an error
    if (s.q == 0 && s.wave == 0 && lane == 0) {        // published even on an error, so later levels stop
        slot_store(dec + j, accepted ? kDecAccepted : kDecRejected, s.epoch);
        slot_store(dec + kMaxLevels + j, __builtin_bit_cast(unsigned, pd), s.epoch);
        slot_store(dec + 2 * kMaxLevels + j, __builtin_bit_cast(unsigned, ratio), s.epoch);
    }
    if (res & kResError) {
        flag_error(a, s);
        return;
    }
    if (accepted) return;   // its outputs are written by the group that draws the last token
    if (s.wave == 0) {      // the first rejection draws: did every earlier level accept?
        unsigned dv[kDecSlots];
        const bool ok = gather_at<kDecSlots>(dec, kMaxLevels, 0, j, s.epoch, a.spin, dv);
        const bool reached = __all(lane >= j || dv[0] == kDecAccepted);
        if (ok && reached && s.q == 0) {   // the outputs the chain writes at the earlier levels and this one
            if (lane < j) level_outputs(a, s, lane, dv[1], dv[2]);
            if (lane == 0 && a.accept_probs) a.accept_probs[s.db + j] = ratio;
        }
        if (lane == 0) s_reached = ok ? (reached ? 1 : 0) : -1;
    }
    __syncthreads();
    const int reached = uniform(s_reached);
    if (reached < 0) {
        flag_error(a, s);
        return;
    }
    if (!reached) return;   // an earlier level rejected: this one is never tested
    sample_row<kVec4>(a, s, j, xp, xq, st, sh);
}

// Workgroups of the kernel the device holds at once, and its CU count.
template <bool kVec4, bool kTree, int W>
hipError_t co_resident(int dev, int* wgs, int* cus_out) {
    static DeviceMemo memo_wgs, memo_cus;
    if (memo_wgs.get(dev) > 0 && memo_cus.get(dev) > 0) {
        *wgs = memo_wgs.get(dev);
        *cus_out = memo_cus.get(dev);
        return hipSuccess;
    }
    int per_cu = 0, cus = 0;
    hipError_t e = kTree
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reject_tree_kernel<kVec4, W>, W * kWave, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reject_kernel<kVec4, W>, W * kWave, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    *wgs = per_cu * cus;
    *cus_out = cus;
    memo_wgs.put(dev, *wgs);
    memo_cus.put(dev, cus);
    return hipSuccess;
}

template <bool kVec4, bool kTree, int W>
hipError_t launch_variant(RejectArgs& a, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int wgs = 0, cus = 0;
    e = co_resident<kVec4, kTree, W>(dev, &wgs, &cus);
    if (e != hipSuccess) return e;
    int groups = min(a.B, wgs / a.Q);
    if (groups < 1) return hipErrorInvalidConfiguration;
    // Not rounded down to a multiple of eight (which would keep each group on one
    // XCD): that would send the last sequences of a batch that fits into a second
    // serial round, and with the work queue it leaves CUs idle (152K vocabulary,
    // B = 256: 208 us with 51 groups, 214 us with 48).
    a.groups = groups;
    // A plain launch: the grid never exceeds what the device holds at once, so on
    // a GPU not shared with other streams every group is resident together. (A
    // cooperative launch would guarantee it, at ~13 us of extra launch latency
    // per call on this stack; should residency ever be partial, the waits are
    // bounded and the affected sequences report an error instead of hanging.)
    if (kTree) hipLaunchKernelGGL((reject_tree_kernel<kVec4, W>), dim3(groups * a.Q), dim3(W * kWave), 0, stream, a);
    else hipLaunchKernelGGL((reject_kernel<kVec4, W>), dim3(groups * a.Q), dim3(W * kWave), 0, stream, a);
    return hipGetLastError();
}

// Workgroups of the level kernel the current device holds at once (-1 if the device
// cannot be queried).
template <bool kVec4>
int levels_capacity() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return -1;
    }
    static DeviceMemo memo;
    int wgs = memo.get(dev);
    if (wgs <= 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reject_levels_kernel<kVec4, 4>, 4 * kWave, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            return -1;
        }
        wgs = per_cu * cus;
        memo.put(dev, wgs);
    }
    return wgs;
}

// The level-parallel kernel: B (k + 1) groups of Q four-wavefront workgroups, all
// resident at once (the groups wait for each other's decisions). If the device
// would not hold them all, the chain with the same workgroups runs instead (the
// same bits).
template <bool kVec4>
hipError_t launch_levels(RejectArgs& a, hipStream_t stream) {
    // Every group waits for the decisions of the levels before it, so all of them
    // must be resident at once: the kernel's own occupancy decides.
    const int wgs = levels_capacity<kVec4>();
    if (wgs < 0) return hipErrorInvalidDevice;
    if (static_cast<long long>(a.B) * (a.k + 1) * a.Q > wgs) return launch_variant<kVec4, false, 4>(a, stream);
    a.groups = a.B * (a.k + 1);
    hipLaunchKernelGGL((reject_levels_kernel<kVec4, 4>), dim3(a.groups * a.Q), dim3(4 * kWave), 0, stream, a);
    return hipGetLastError();
}

// CUs of the current device (0 if it cannot be read).
int device_cus() {
    static DeviceMemo memo;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    if (memo.get(dev) > 0) return memo.get(dev);
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    memo.put(dev, cus);
    return cus;
}

// Polls per bounded wait: 2^20 (~10 ms of polling, far beyond any wait of a
// resident group), or the value of the environment variable SPECVERIFY_SPIN_LIMIT
// when it is set the first time this is called. A small limit makes the waits
// give up early, so that tests can exercise the error path from the host; every
// wait still ends.
unsigned reject_spin_limit() {
    static std::atomic<long long> cached{-1};
    long long v = cached.load(std::memory_order_relaxed);
    if (v < 0) {
        v = kSpinLimit;
        if (const char* e = std::getenv("SPECVERIFY_SPIN_LIMIT")) {
            char* end = nullptr;
            const long long x = std::strtoll(e, &end, 10);
            if (end != e && x >= 0 && x <= kSpinLimit) v = x;
        }
        cached.store(v, std::memory_order_relaxed);
    }
    return static_cast<unsigned>(v);
}

// Copies the workspace's error word into *flag_out and clears it. One thread; a
// kernel rather than a memset or copy, so that it can sit in a captured graph.
__global__ void reject_error_flag_kernel(unsigned* ctl, int32_t* flag_out) {
    const unsigned v = __hip_atomic_exchange(ctl + kCtlError, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag_out = static_cast<int32_t>(v);
}

// Workgroups per sequence with W unit wavefronts each.
int groups_of(int V, int W) {
    const int U = (V + kUnit - 1) / kUnit;
    return (U + W - 1) / W;
}

// The sampling workspace of spec_reject_sample_noalloc: a file-scope device array, one
// copy per GPU, zero at module load and kept until the process ends. Its name is a
// host-side stand-in in host code; the device address comes from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char g_reject_scratch[kNoAllocScratchBytes];

// Device address of this GPU's copy of g_reject_scratch, looked up once per device (with
// that device current) and kept; nullptr until then.
std::atomic<void*> g_reject_scratch_ptr[64];

}  // namespace

size_t reject_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t reject_noalloc_scratch(void** ptr_out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* ptr = g_reject_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_reject_scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_reject_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    *ptr_out = ptr;
    return hipSuccess;
}

size_t reject_workspace_bytes(int B, int k, int V) {
    return reject_layout(B, k, (V + kUnit - 1) / kUnit).total;
}

int reject_max_vocab() { return kUnit * 256; }

hipError_t launch_reject_error_flag(void* workspace, int32_t* flag_out, hipStream_t stream) {
    hipLaunchKernelGGL(reject_error_flag_kernel, dim3(1), dim3(1), 0, stream, static_cast<unsigned*>(workspace),
                       flag_out);
    return hipGetLastError();
}

RejectPlan reject_plan(int B, int k, int V) {
    const int cus = device_cus();
    const long long q4 = groups_of(V, 4), q8 = groups_of(V, 8);
    const long long level_cap = static_cast<long long>(cus) * (k <= 3 ? 2 : 1);
    RejectPlan r;
    r.levels = k >= 1 && cus > 0 && static_cast<long long>(B) * (k + 1) * q4 <= level_cap;
    const bool one_round8 = static_cast<long long>(B) * q8 <= cus;
    const bool own_cu4 = static_cast<long long>(B) * q4 <= cus;
    r.W = (r.levels || own_cu4 || !one_round8) ? 4 : 8;
    if (r.levels) {   // the level kernel's own residency decides in the end (launch_levels)
        const int wgs = (V % 4) == 0 ? levels_capacity<true>() : levels_capacity<false>();
        if (wgs <= 0 || static_cast<long long>(B) * (k + 1) * groups_of(V, 4) > wgs) r.levels = false;
    }
    return r;
}

hipError_t launch_reject(const RejectLaunch& p, hipStream_t stream) {
    const int U = (p.V + kUnit - 1) / kUnit;
    // The levels of each sequence at once when all of them fit one workgroup per CU,
    // or two per CU for drafts of at most three tokens (k >= 1; ragged calls take
    // k_max + 1 groups per sequence); else the chain. Two per CU made the 8B rows at
    // B = 16 (k = 3) faster but the long-tail shape, k = 7 with few acceptances,
    // slower: all its levels are computed where the chain mostly stops at the first,
    // and the longer the draft, the more of them go unused. The chain takes eight-wave workgroups
    // only when the batch fills the device in one round of them (one per CU), and
    // four-wave ones otherwise: when each can have a CU to itself, and when the
    // sequences are handed out over several rounds, where two workgroups of
    // different sequences share each CU (152K vocabulary, B = 256, inside the full
    // step: 210 us instead of 215 us; at B = 64 the same time). The outputs do not
    // depend on it.
    const RejectPlan plan = reject_plan(p.B, p.k, p.V);
    const bool levels = plan.levels;
    const int W = plan.W;
    const int Q = groups_of(p.V, W);
    if (Q > kMaxQ) return hipErrorInvalidValue;
    const RejectLayout lay = reject_layout(p.B, p.k, U);
    char* ws = static_cast<char*>(p.workspace);
    RejectArgs a;
    a.target = p.target_logits;
    a.draft = p.draft_logits;
    a.draft_tokens = p.draft_tokens;
    a.seq_ids = p.seq_ids;
    a.seq_lens = p.seq_lens;
    a.cu = p.cu_drafts;
    a.out_tokens = p.out_tokens;
    a.num_accepted = p.num_accepted;
    a.out_probs = p.out_probs;
    a.accept_probs = p.accept_probs;
    a.ctl = reinterpret_cast<unsigned*>(ws + lay.ctl);
    a.stat_slots = reinterpret_cast<unsigned long long*>(ws + lay.stat);
    a.samp_slots = reinterpret_cast<unsigned long long*>(ws + lay.samp);
    a.dec_slots = reinterpret_cast<unsigned long long*>(ws + lay.dec);
    a.bonus_slots = reinterpret_cast<unsigned long long*>(ws + lay.bonus);
    a.next_slots = reinterpret_cast<unsigned long long*>(ws + lay.next);
    a.parents = nullptr;
    a.out_nodes = nullptr;
    a.tree_slots = nullptr;
    a.B = p.B; a.k = p.k; a.V = p.V; a.U = U; a.Q = Q; a.groups = 0;
    a.invT = 1.0f / p.temperature;
    a.c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(p.temperature));
    a.invT64 = 1.0 / static_cast<double>(p.temperature);
    a.T = p.temperature;
    a.seed = p.seed;
    a.spin = reject_spin_limit();
    if (levels) return (p.V % 4) == 0 ? launch_levels<true>(a, stream) : launch_levels<false>(a, stream);
    if (W == 4)
        return (p.V % 4) == 0 ? launch_variant<true, false, 4>(a, stream) : launch_variant<false, false, 4>(a, stream);
    return (p.V % 4) == 0 ? launch_variant<true, false, 8>(a, stream) : launch_variant<false, false, 8>(a, stream);
}

size_t reject_tree_workspace_bytes(int B, int nodes, int V) {
    const int U = (V + kUnit - 1) / kUnit;
    (void)nodes;
    return align256(4 * sizeof(unsigned)) + sizeof(unsigned long long) * size_t(B) * kTreeEx * kSampSlots * U;
}

int reject_tree_max_branch() { return kMaxBranch; }

hipError_t launch_reject_tree(const RejectLaunch& p, hipStream_t stream) {
    const int U = (p.V + kUnit - 1) / kUnit;
    // Four-wave workgroups when each can have a CU of its own (a tree's serial walk then
    // spreads over twice the CUs, as the chain's does at such batches), eight otherwise.
    // The exchanges go through quads, so the outputs do not depend on it.
    const int cus = device_cus();
    const int W = (cus > 0 && static_cast<long long>(p.B) * groups_of(p.V, 4) <= cus) ? 4 : kUnitWaves;
    const int Q = groups_of(p.V, W);
    if (Q > kMaxQ) return hipErrorInvalidValue;
    char* ws = static_cast<char*>(p.workspace);
    RejectArgs a;
    a.target = p.target_logits;
    a.draft = p.draft_logits;
    a.draft_tokens = p.draft_tokens;
    a.seq_ids = p.seq_ids;
    a.seq_lens = p.seq_lens;
    a.cu = nullptr;
    a.out_tokens = p.out_tokens;
    a.num_accepted = p.num_accepted;
    a.out_probs = p.out_probs;
    a.accept_probs = p.accept_probs;
    a.ctl = reinterpret_cast<unsigned*>(ws);
    a.stat_slots = nullptr;
    a.samp_slots = nullptr;
    a.dec_slots = nullptr;
    a.bonus_slots = nullptr;
    a.next_slots = nullptr;
    a.parents = p.parents;
    a.out_nodes = p.out_nodes;
    a.tree_slots = reinterpret_cast<unsigned long long*>(ws + align256(4 * sizeof(unsigned)));
    a.B = p.B; a.k = p.k; a.V = p.V; a.U = U; a.Q = Q; a.groups = 0;
    a.invT = 1.0f / p.temperature;
    a.c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(p.temperature));
    a.invT64 = 1.0 / static_cast<double>(p.temperature);
    a.T = p.temperature;
    a.seed = p.seed;
    a.spin = reject_spin_limit();
    if (W == 4)
        return (p.V % 4) == 0 ? launch_variant<true, true, 4>(a, stream) : launch_variant<false, true, 4>(a, stream);
    return (p.V % 4) == 0 ? launch_variant<true, true, kUnitWaves>(a, stream)
                          : launch_variant<false, true, kUnitWaves>(a, stream);
}

}  // namespace specverify
