// Comparator for the oracle's Philox4x32-10: prints the four 32-bit words of
// blocks first_block .. first_block+n_blocks-1 from rocRAND's Philox4x32-10
// engine, initialised with (seed, subsequence = step, offset = 4 * block), which
// places the block index in counter words 0-1 and the step in words 2-3.
// Host-only use of the library's engine; built by the tests.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
    if (argc != 5) return 2;
    unsigned long long seed = strtoull(argv[1], nullptr, 0);
    unsigned long long step = strtoull(argv[2], nullptr, 0);
    unsigned long long first = strtoull(argv[3], nullptr, 0);
    unsigned long long n = strtoull(argv[4], nullptr, 0);
    for (unsigned long long q = 0; q < n; ++q) {
        const unsigned long long b = first + q;  // 4*b must stay below 2^64
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, step, 4ull * b, &st);
        uint4 v = rocrand4(&st);
        printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
    }
    return 0;
}
