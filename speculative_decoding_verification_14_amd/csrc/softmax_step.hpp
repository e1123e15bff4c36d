// Offset arithmetic of one online-softmax step of the sampling pass's row statistics.
//
// A step sums terms exp2(x c2 + nr) for the logits x of four loads, c2 = log2(e)/T,
// with nr = -ref c2 rounded to fp32, ref the running maximum after the step. The
// rounding of nr is common to all the step's terms: -ref c2 = nr + eps exactly, and
// every term is 2^{(x - ref) c2} 2^-eps up to its own rounding. These helpers take
// eps exactly and put it back, so that the row's normaliser carries no error common
// to its terms. They are __host__ __device__ so that a host build can check them.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace specverify {

struct StepOffset {
    float nr;    // -ref c2 rounded to fp32
    float eps;   // -ref c2 - nr, exactly (the rounding error of a product is a float)
};

__host__ __device__ inline StepOffset step_offset(float ref, float c2) {
#pragma clang fp contract(off)
    StepOffset o;
    o.nr = -ref * c2;
    o.eps = fmaf(-ref, c2, -o.nr);
    return o;
}

// Base-2 exponent of the factor that moves a sum kept relative to m onto ref,
// (m - ref) c2, as fma(m, c2, nr) + eps. For m == ref the fma returns -eps exactly
// (a float), so the exponent is exactly 0 and the factor exactly 1; for m = -inf it
// is -inf (factor 0). exp2(fma(m, c2, nr)) alone would be 2^-eps where it should be
// 1, applied again at every step in which the maximum does not move.
__host__ __device__ inline float rescale_exponent(float m, float c2, const StepOffset& o) {
#pragma clang fp contract(off)
    return fmaf(m, c2, o.nr) + o.eps;
}

// The step's sum of exp2(x c2 + nr) times 2^eps = 1 + eps ln 2 (|eps| <= 2^-18 for
// |ref c2| < 64, so the dropped eps^2 term is below 1e-11).
__host__ __device__ inline float corrected_sum(float sum, const StepOffset& o) {
#pragma clang fp contract(off)
    return fmaf(sum, o.eps * 0.69314718f, sum);
}

}  // namespace specverify
