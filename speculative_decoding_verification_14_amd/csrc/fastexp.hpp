// Exponentials for the softmax and sampling arithmetic of the verify step.
#pragma once

#include <hip/hip_runtime.h>

namespace specverify {

// e^x in fp64 for x <= 0 (down to the fp64 underflow range).
// Range reduction by the nearest integer n of x / ln 2, with ln 2 split in two
// (the high part has 24 trailing zero bits, so n * hi is exact), leaves
// |r| <= ln2 / 2; e^r is its Taylor series to degree 12, whose truncation error
// is below 2.5e-16 relative there; the result is scaled by 2^n. About 16 fp64
// operations, all FMA or add, against ~50 for a general-purpose exp.
__host__ __device__ inline double exp_nonpos_f64(double x) {
    constexpr double kLog2e = 0x1.71547652b82fep+0;
    constexpr double kLn2Hi = 0x1.62e42ff000000p-1;
    constexpr double kLn2Lo = -0x1.718432a1b0e26p-35;
    // Branch-free (a select at the end), so that inlined copies add no control
    // flow: arguments at or below -745, -inf and NaN give 0.
    const bool in_range = x > -745.0;
    const double xc = in_range ? x : -745.0;
    const double n = rint(xc * kLog2e);
    double r = fma(-n, kLn2Hi, xc);
    r = fma(-n, kLn2Lo, r);
    double p = 1.0 / 479001600.0;           // 1/12!
    p = fma(p, r, 1.0 / 39916800.0);        // 1/11!
    p = fma(p, r, 1.0 / 3628800.0);
    p = fma(p, r, 1.0 / 362880.0);
    p = fma(p, r, 1.0 / 40320.0);
    p = fma(p, r, 1.0 / 5040.0);
    p = fma(p, r, 1.0 / 720.0);
    p = fma(p, r, 1.0 / 120.0);
    p = fma(p, r, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    const double v = ldexp(p, static_cast<int>(n));
    return in_range ? v : 0.0;
}

// e^x in fp32 for the small terms of a softmax sum (x well below 0): the product
// x * log2(e) is carried as hi + lo (hi rounded, lo its rounding error plus the
// contribution of log2(e)'s own fp32 rounding), then 2^hi comes from the hardware
// exp2 and the factor 2^lo ~ 1 + lo ln2. Relative error is a few fp32 ulp, the
// same class as a library expf, in 6 instructions.
__device__ __forceinline__ float exp_small_f32(float x) {
    constexpr float kL = 0x1.715476p+0f;            // log2(e) rounded to fp32
    constexpr float kLLo = 1.9259630335e-08f;       // log2(e) - kL
    constexpr float kLn2 = 0.69314718f;
    x = fmaxf(x, -150.0f);                  // e^-150 is 0 in fp32; keeps -inf out of the fma
    const float hi = x * kL;
    const float lo = fmaf(x, kL, -hi) + x * kLLo;
    const float e = __builtin_amdgcn_exp2f(hi);
    return fmaf(e, kLn2 * lo, e);
}

}  // namespace specverify
