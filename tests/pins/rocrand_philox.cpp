// Prints rocRAND's Philox4x32-10 output block for given (seed, counter).
// Used only as an external pin for the oracle's Philox; built for the host.
// Input lines:  seed c0 c1 c2 c3   (decimal; c1 < 2^30)
// Output lines: w0 w1 w2 w3        (hex)
//
// rocrand_init(seed, subsequence, offset) keys the engine with the seed's
// two 32-bit halves; the subsequence sets counter words 2..3 and offset/4
// sets counter words 0..1, so (c0, c1, c2, c3) is reached with
// subsequence = c2 + c3 * 2^32 and offset = 4 * (c0 + c1 * 2^32).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, c2 + (c3 << 32), 4ULL * (c0 + (c1 << 32)), &st);
        uint4 r = rocrand4(&st);
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
