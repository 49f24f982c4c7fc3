// Independent Philox4x32-10 reference for the oracle's tests: rocRAND's
// open-source engine (rocrand_philox4x32_10.h), run on the host.
//
// rocRAND keys the engine with the 64-bit seed (low word first), puts the
// subsequence in counter words 2..3 and advances counter words 0..1 by
// offset / 4, so counter (c0, c1, c2, c3) is reached with
// subsequence = c2 | c3 << 32 and an advance of x = c0 | c1 << 32 blocks.  The
// advance is given in elements (4 per block) and must fit in 64 bits, so it is
// applied in pieces of at most 2^62 - 1 blocks.
//
// stdin: lines "c0 c1 c2 c3 seed" (decimal); stdout: the 4 words in hex.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
    unsigned long long c0, c1, c2, c3, seed;
    while (std::scanf("%llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &seed) == 5) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, c2 | (c3 << 32), 0ULL, &st);
        const unsigned long long x = c0 | (c1 << 32);
        for (int i = 0; i < 4; ++i) skipahead(4ULL * (x >> 2), &st);
        skipahead(4ULL * (x & 3ULL), &st);
        unsigned int w[4];
        for (int i = 0; i < 4; ++i) w[i] = rocrand(&st);
        std::printf("%08x %08x %08x %08x\n", w[0], w[1], w[2], w[3]);
    }
    return 0;
}
