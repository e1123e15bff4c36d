// Host build of the sampling pass's online-softmax step offsets (softmax_step.hpp), for
// a CPU check that a lane's running sum carries no error common to all its terms.
// stdout, one line each:
//   "zero_exponent BAD"   count of (m, c2) for which rescale_exponent(m, c2, step_offset(m, c2))
//                         is not exactly 0 (over random m and c2)
//   "neg_inf BAD"         count for which m = -inf does not give an exponent of -inf
//   "rows N OLD_MAX OLD_MEAN NEW_MAX NEW_MEAN"
//                         relative error of a lane's sum over N rows of 64 logits, each summed
//                         as the pass does (four steps of 16, exp2f per term, fp64 running
//                         sum), against the same sum in fp64 with exp2 of the exact exponents:
//                         OLD with the offset rounding left in (rescale exp2(fma(m, c2, nr)),
//                         uncorrected step sums), NEW with the helpers
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "softmax_step.hpp"

using namespace specverify;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {   // splitmix64
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform01() { return (next_u64() >> 11) * (1.0 / 9007199254740992.0); }
static double normal() {   // Box-Muller
    const double u1 = uniform01() + 1e-300, u2 = uniform01();
    return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
}

// one lane's 64 logits in four steps of 16, as the pass sums them
static double lane_sum(const float* x, float c2, bool corrected, float& m_out) {
    float m = -std::numeric_limits<float>::infinity();
    double acc = 0.0;
    for (int s = 0; s < 4; ++s) {
        float gm = -std::numeric_limits<float>::infinity();
        for (int i = 0; i < 16; ++i) gm = std::fmax(gm, x[16 * s + i]);
        const float mn = std::fmax(m, gm);
        const float ref = std::isinf(mn) && mn < 0 ? 0.0f : mn;
        const StepOffset off = step_offset(ref, c2);
        const float rescale = corrected ? std::exp2f(rescale_exponent(m, c2, off)) : std::exp2f(std::fmaf(m, c2, off.nr));
        float sum = 0.0f;
        for (int i = 0; i < 16; ++i) sum += std::exp2f(std::fmaf(x[16 * s + i], c2, off.nr));
        if (corrected) sum = corrected_sum(sum, off);
        acc = acc * static_cast<double>(rescale) + static_cast<double>(sum);
        m = mn;
    }
    m_out = m;
    return acc;
}

int main() {
    // exponent exactly 0 when the maximum does not move, -inf from m = -inf
    long bad0 = 0, badinf = 0;
    for (int i = 0; i < 1000000; ++i) {
        const float m = static_cast<float>((uniform01() * 2.0 - 1.0) * std::ldexp(1.0, static_cast<int>(next_u64() % 12)));
        const float c2 = static_cast<float>(1.4426950408889634 / (0.25 + 2.0 * uniform01()));
        if (rescale_exponent(m, c2, step_offset(m, c2)) != 0.0f) ++bad0;
        const float e = rescale_exponent(-std::numeric_limits<float>::infinity(), c2, step_offset(m, c2));
        if (!(std::isinf(e) && e < 0)) ++badinf;
    }
    std::printf("zero_exponent %ld\n", bad0);
    std::printf("neg_inf %ld\n", badinf);

    // rows shaped like the workloads' logits: N(0, 3) around an offset, 1% boosted by 8,
    // offsets 0..40 so that |ref c2| spans several binades, T = 1 and 0.7
    const int N = 20000;
    double omax = 0, osum = 0, nmax = 0, nsum = 0;
    float x[64];
    for (int r = 0; r < N; ++r) {
        const double offset = 40.0 * uniform01();
        const float T = (r % 2) ? 1.0f : 0.7f;
        const float c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(T));
        for (int i = 0; i < 64; ++i) {
            double z = offset + 3.0 * normal();
            if (uniform01() < 0.01) z += 8.0;
            x[i] = static_cast<float>(z);
        }
        float m_old, m_new;
        const double s_old = lane_sum(x, c2, false, m_old);
        const double s_new = lane_sum(x, c2, true, m_new);
        double exact = 0.0;   // sum of 2^{(x - m) c2}, exponents exact in fp64
        for (int i = 0; i < 64; ++i)
            exact += std::exp2((static_cast<double>(x[i]) - static_cast<double>(m_new)) * static_cast<double>(c2));
        const double eo = std::fabs(s_old / exact - 1.0), en = std::fabs(s_new / exact - 1.0);
        omax = std::fmax(omax, eo); osum += eo;
        nmax = std::fmax(nmax, en); nsum += en;
    }
    std::printf("rows %d %.3e %.3e %.3e %.3e\n", N, omax, osum / N, nmax, nsum / N);
    return 0;
}
