// Host-side dump of rocRAND's Philox4x32-10 engine output, used only by the
// oracle's pin test.  Reads lines "seed subsequence offset" from stdin and
// prints the four 32-bit words the engine returns next, in hex.
#include <cstdio>
#include <rocrand/rocrand_kernel.h>

int main() {
    unsigned long long seed, subseq, offset;
    while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, subseq, offset, &st);
        uint4 r = rocrand4(&st);
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
