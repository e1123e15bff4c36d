// Classification of "heavy" logits for the sampling pass of the verify step.
//
// The draw from the residual max(0, p - q) (or from p for the bonus token) sums
// fp32 weights for most logits but takes those whose probability exceeds
// tau = 2^-14 in fp64, so that the few large terms, which place every later CDF
// boundary, carry no fp32 rounding. A logit is heavy when its raw value lies
// above a per-row threshold; the heavy ones of a lane are packed into bit masks
// and their values re-read from memory.
//
// Everything here is __host__ __device__ so that a host build can check the
// classification and the re-read indices on the CPU; the device build is what
// the sampling kernels run.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace specverify {

namespace heavy {
constexpr int kLanes = 64;                    // lanes of a wavefront
constexpr int kLoadSpan = kLanes * 4;         // logits covered by one 16-byte load of the wavefront
constexpr float kLnTau = -9.70406052783923f;  // ln 2^-14
}  // namespace heavy

// ln Z from the hardware log2 (a few ulp) on the device, the C library's on the
// host: it only places the heavy thresholds and the support boundary, where any
// consistent value is correct and an error of 1e-7 moves only logits whose
// weight is that small.
__host__ __device__ inline float ln_approx(double Z) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_logf(static_cast<float>(Z)) * 0.693147180559945f;
#else
    return log2f(static_cast<float>(Z)) * 0.693147180559945f;
#endif
}

// Raw-logit threshold above which a logit's probability under (M, Z) exceeds tau:
// p > tau  <=>  z > M + T (ln tau + ln Z). Monotone, so one compare per logit;
// only its consistency matters (every site classifies with the same float).
// Requires Z > 0: with Z = 0 (no finite logit) it returns -inf.
__host__ __device__ inline float heavy_threshold(float M, double Z, float T) {
    return fmaf(T, heavy::kLnTau + ln_approx(Z), M);
}

// The threshold of a unit weighed against its own statistics (M_u, Z_u), as the
// bonus pass does. A unit lying wholly past V has M_u = -inf and Z_u = 0; its
// threshold is +inf, so that none of its -inf padding is heavy. (Through
// heavy_threshold it would be -inf, and the heavy test on the padding would
// compute -inf - (-inf), a NaN whose sign bit decides.)
__host__ __device__ inline float unit_heavy_threshold(float Mu, double Zu, float T) {
    return (Zu > 0.0) ? heavy_threshold(Mu, Zu, T) : INFINITY;
}

// Heavy test as a sign bit: t - z < 0 exactly when z > t (the difference of two
// distinct floats is never zero), so the bit is set iff z_p > t_p or z_q > t_q.
// Kept in a vector register rather than as a lane mask, so that the 64 tests of a
// unit can be packed into bits without tying up scalar registers. -inf padding is
// never heavy under a finite or +inf threshold.
__host__ __device__ inline unsigned heavy_sign(bool residual, float zp, float zq, float tp, float tq) {
    const float d = residual ? fminf(tp - zp, tq - zq) : tp - zp;
    return __builtin_bit_cast(unsigned, d);
}

// (mask << 1) | (sign bit of d): one funnel shift on the device.
__host__ __device__ inline unsigned shift_in_sign(unsigned mask, unsigned d) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_alignbit(mask, d, 31u);
#else
    return (mask << 1) | (d >> 31);
#endif
}

// The lane's heavy logits as two 32-bit masks: element k = 4i + e of the unit
// (load i, component e) is bit 31 - k of lo for k < 32 and bit 63 - k of hi
// otherwise (each mask is built by shifting in one bit per element).
struct HeavyBits {
    unsigned lo, hi;
};

// kN loads of four logits each (element [i][e] = load i, component e); zq is read
// only for the residual (two rows).
template <int kN, typename V4>
__host__ __device__ inline HeavyBits heavy_bits(bool residual, const V4 (&xp)[kN], const V4 (&xq)[kN], float tp,
                                                float tq) {
    static_assert(kN * 4 == 64, "a lane holds 64 logits of its unit");
    HeavyBits hb{0u, 0u};
#pragma unroll
    for (int i = 0; i < kN; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned d = heavy_sign(residual, xp[i][e], residual ? xq[i][e] : -INFINITY, tp, tq);
            if (i < kN / 2) hb.lo = shift_in_sign(hb.lo, d);
            else hb.hi = shift_in_sign(hb.hi, d);
        }
    }
    return hb;
}

// Takes one heavy element off the masks: its index k in the lane's 64, or -1.
__host__ __device__ inline int take_heavy(HeavyBits& hb) {
    if (hb.lo != 0u) {
        const int p = __builtin_ctz(hb.lo);
        hb.lo &= hb.lo - 1u;
        return 31 - p;
    }
    if (hb.hi != 0u) {
        const int p = __builtin_ctz(hb.hi);
        hb.hi &= hb.hi - 1u;
        return 63 - p;
    }
    return -1;
}

// Token index of the lane's element k (load k / 4, component k % 4), `base` the
// lane's first token in the unit (unit * 4096 + 4 * lane).
__host__ __device__ inline int heavy_element(int base, int k) {
    return base + (k >> 2) * heavy::kLoadSpan + (k & 3);
}

}  // namespace specverify
