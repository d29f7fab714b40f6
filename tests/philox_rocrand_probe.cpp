// Host-side reference stream for the oracle's Philox4x32-10: rocRAND's engine,
// an implementation independent of the oracle.  Reads lines
// "seed subsequence block" and prints the four output words of counter block
// `block` of subsequence `subsequence` under key `seed`.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>

int main()
{
    unsigned long long seed, sub, block;
    while (std::scanf("%llu %llu %llu", &seed, &sub, &block) == 3) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, sub, 4ULL * block, &st);
        uint4 v = rocrand4(&st);
        std::printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
    }
    return 0;
}
