// Host-side reference for the oracle's Philox-4x32-10: AMD's open-source
// rocRAND engine (rocrand_philox4x32_10.h), an implementation independent of
// both the oracle and the GPU library. Test infrastructure only.
//
// Reads lines "seed b h i j" on stdin and prints the four output words of the
// block function at counter (b, h, i, j) under key (seed low word, seed high word).
// rocRAND's seed() puts the seed into the key, the offset/4 into counter words
// (0, 1) and the subsequence into counter words (2, 3); the first next() is word 0.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
    unsigned long long seed, b, h, i, j;
    while (std::scanf("%llu %llu %llu %llu %llu", &seed, &b, &h, &i, &j) == 5) {
        rocrand_device::philox4x32_10_engine eng(seed, i | (j << 32), 4ull * (b | (h << 32)));
        unsigned w0 = eng.next(), w1 = eng.next(), w2 = eng.next(), w3 = eng.next();
        std::printf("%u %u %u %u\n", w0, w1, w2, w3);
    }
    return 0;
}
