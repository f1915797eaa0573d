// Test helper: prints Philox4x32-10 outputs computed by rocRAND's own engine
// (an implementation independent of the oracle), to pin the oracle's Philox.
// stdin: lines "key_lo key_hi c0 c1 c2 c3" (hex); stdout: "w0 w1 w2 w3" (hex).
// rocRAND's engine(seed, subsequence, offset) sets key = seed and counter
// words (0,1) = offset/4, (2,3) = subsequence; with offset a multiple of 4 the
// first next4() is the block for exactly that counter.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main()
{
    unsigned klo, khi, c0, c1, c2, c3;
    while (std::scanf("%x %x %x %x %x %x", &klo, &khi, &c0, &c1, &c2, &c3) == 6) {
        unsigned long long seed = ((unsigned long long)khi << 32) | klo;
        unsigned long long ctr01 = ((unsigned long long)c1 << 32) | c0;
        unsigned long long subseq = ((unsigned long long)c3 << 32) | c2;
        rocrand_device::philox4x32_10_engine e(seed, subseq, ctr01 * 4ull);
        uint4 r = e.next4();
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
