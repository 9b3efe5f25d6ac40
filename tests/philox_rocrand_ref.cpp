// Known-answer generator for the Philox4x32-10 pin: prints the four output
// words of rocRAND's Philox4x32-10 engine (an independent implementation of
// Salmon et al., SC'11) for each "seed subsequence offset" triple read from
// stdin.  The engine's key is (seed low, seed high) and its counter is
// (offset/4 low, offset/4 high, subsequence low, subsequence high).
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
    unsigned long long seed, subseq, offset;
    while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
        rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
        unsigned int w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
        std::printf("%u %u %u %u\n", w0, w1, w2, w3);
    }
    return 0;
}
