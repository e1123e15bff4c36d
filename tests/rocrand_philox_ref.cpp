// Host-side reference for Philox4x32-10: rocRAND's installed engine (a library
// routine, used here only to pin the oracle's own implementation).
//
// stdin : lines "key0 key1 c0 c1 c2 c3" (decimal uint32; c1 < 2^30)
// stdout: lines "w0 w1 w2 w3" = Philox4x32-10(counter=(c0,c1,c2,c3), key=(key0,key1))
//
// The engine is seeded with seed = key0 | key1<<32, subsequence = c2 | c3<<32 and
// offset = 4 * (c0 | c1<<32), which puts its counter at (c0, c1, c2, c3); its
// next four outputs are then the four words of that block.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
    unsigned long long k0, k1, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu %llu", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        const unsigned long long seed = k0 | (k1 << 32);
        const unsigned long long subsequence = c2 | (c3 << 32);
        const unsigned long long offset = 4ull * (c0 | (c1 << 32));
        rocrand_device::philox4x32_10_engine eng(seed, subsequence, offset);
        unsigned int w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
        std::printf("%u %u %u %u\n", w0, w1, w2, w3);
    }
    return 0;
}
