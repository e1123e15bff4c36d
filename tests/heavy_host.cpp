// Host build of the sampling pass's heavy-logit classification (heavy.hpp), for
// a CPU check of which elements the pass re-reads.
// stdin : lines "V W T mode"; mode 0: a bonus-row unit's threshold through
//         heavy_threshold on the unit's own (M_u, Z_u) (the form the bonus pass used
//         before units wholly past V got a threshold of +inf), 1: through
//         unit_heavy_threshold (the form it uses), 2: the residual's thresholds,
//         which come from the whole row's (finite) statistics.
// stdout: per unit of the row ("W" unit wavefronts per workgroup, so the row is
//         covered by ceil(ceil(V/4096)/W)*W units): "u count min max", count the
//         re-read elements of the unit over its 64 lanes and min / max their token
//         indices (-1 -1 if none); then a line "end".
// Logits of the row are 0 for tokens below V and -inf padding past V, as the
// kernel's loads leave them.
#include <cmath>
#include <cstdio>
#include <limits>

#include "heavy.hpp"

using specverify::HeavyBits;

typedef float f4 __attribute__((ext_vector_type(4)));

int main() {
    int V, W, mode;
    float T;
    const float ninf = -std::numeric_limits<float>::infinity();
    while (std::scanf("%d %d %f %d", &V, &W, &T, &mode) == 4) {
        const int U = (V + 4095) / 4096;
        const int units = (U + W - 1) / W * W;
        for (int u = 0; u < units; ++u) {
            // the unit's own statistics, as the online softmax leaves them: an all
            // -inf unit has M_u = -inf and Z_u = 0
            float Mu = ninf;
            for (int x = u * 4096; x < (u + 1) * 4096; ++x) Mu = std::fmax(Mu, x < V ? 0.0f : ninf);
            double Zu = 0.0;
            for (int x = u * 4096; x < (u + 1) * 4096; ++x)
                if (x < V) Zu += std::exp(0.0 - static_cast<double>(Mu));
            float tp, tq;
            bool residual = false;
            if (mode == 0) {
                tp = specverify::heavy_threshold(Mu, Zu, T);
                tq = std::numeric_limits<float>::infinity();
            } else if (mode == 1) {
                tp = specverify::unit_heavy_threshold(Mu, Zu, T);
                tq = std::numeric_limits<float>::infinity();
            } else {   // the whole row's statistics: M = 0, Z = V (every logit 0)
                residual = true;
                tp = specverify::heavy_threshold(0.0f, static_cast<double>(V), T);
                tq = tp;
            }
            long count = 0;
            int lo = -1, hi = -1;
            for (int lane = 0; lane < 64; ++lane) {
                const int base = u * 4096 + 4 * lane;
                f4 xp[16], xq[16];
                for (int i = 0; i < 16; ++i)
                    for (int e = 0; e < 4; ++e) {
                        const int x = base + i * specverify::heavy::kLoadSpan + e;
                        xp[i][e] = x < V ? 0.0f : ninf;
                        xq[i][e] = xp[i][e];
                    }
                HeavyBits hb = specverify::heavy_bits<16>(residual, xp, xq, tp, tq);
                for (int k = specverify::take_heavy(hb); k >= 0; k = specverify::take_heavy(hb)) {
                    const int x = specverify::heavy_element(base, k);
                    ++count;
                    lo = (lo < 0 || x < lo) ? x : lo;
                    hi = x > hi ? x : hi;
                }
            }
            std::printf("%d %ld %d %d\n", u, count, lo, hi);
        }
        std::printf("end\n");
        std::fflush(stdout);
    }
    return 0;
}
