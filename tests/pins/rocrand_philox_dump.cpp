// Prints Philox4x32-10 blocks computed by rocRAND's host-callable engine, as an
// independent implementation to pin the oracle's generator against.
// Input lines: "seed c0 c1 c2 c3"; output lines: "w0 w1 w2 w3" for the block at
// counter (c0, c1, c2, c3) under key (seed lo, seed hi).
// The engine places a counter through its (subsequence, offset) arguments:
// offset 4 * (c0 + 2^32 c1) advances words 0-1, subsequence c2 + 2^32 c3 sets
// words 2-3 (so c1 must stay below 2^30).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
        const unsigned long long offset = 4ull * (c0 | (c1 << 32));
        const unsigned long long subsequence = c2 | (c3 << 32);
        rocrand_device::philox4x32_10_engine eng(seed, subsequence, offset);
        unsigned int w[4];
        for (int i = 0; i < 4; ++i) w[i] = eng();
        std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
    }
    return 0;
}
