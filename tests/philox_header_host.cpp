// Host build of the library's device Philox header, for a CPU comparison with
// the oracle's independent implementation.
// stdin : lines "seed seq_id pos stream"  (decimal; seed as uint64, seq_id as int64)
// stdout: lines "w0 w1 w2 w3 u0_bits u1_bits" (u as 2^24 multiples; stream 0 through
//         verify_uniforms, other streams through stream_uniforms)
#include <cstdio>
#include "philox.hpp"

int main() {
    unsigned long long seed;
    long long sid, pos;
    unsigned stream;
    while (std::scanf("%llu %lld %lld %u", &seed, &sid, &pos, &stream) == 4) {
        const unsigned long long s = static_cast<unsigned long long>(sid);
        const specverify::PhiloxWords w = specverify::philox4x32_10(
            static_cast<uint32_t>(pos), static_cast<uint32_t>(s), static_cast<uint32_t>(s >> 32), stream,
            static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
        double ua, us;
        if (stream == 0) specverify::verify_uniforms(seed, sid, pos, &ua, &us);
        else specverify::stream_uniforms(seed, sid, pos, stream, &ua, &us);
        std::printf("%u %u %u %u %.0f %.0f\n", w.w[0], w.w[1], w.w[2], w.w[3], ua * 16777216.0, us * 16777216.0);
    }
    return 0;
}
