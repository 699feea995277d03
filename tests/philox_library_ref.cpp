// Philox4x32-10 block outputs from rocRAND's header-only host engine: an
// implementation of the published generator (Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) that shares nothing
// with the float64 oracle's, used only to pin the oracle's round function.
//
// stdin: lines "seed subsequence offset"; stdout: the four 32-bit words of
// the first block.  rocRAND keys the generator with (seed lo, seed hi), puts
// the subsequence in counter words 2..3 and offset/4 in counter words 0..1,
// so counter (x, y, z, w) is reached with subsequence = w:z and
// offset = 4 * (y:x) for y < 2^30.
#include <rocrand/rocrand_kernel.h>

#include <cstdio>

int main() {
    unsigned long long seed, sub, off;
    while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, sub, off, &st);
        const uint4 r = rocrand4(&st);
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
