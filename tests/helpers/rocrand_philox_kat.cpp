// Prints rocRAND's Philox4x32-10 output block for each (seed, counter) line
// read from stdin, so that the oracle's Philox can be checked against an
// independent library implementation.  Host-only: no GPU is touched.
// Input lines:  seed_hex c0 c1 c2 c3   (counter words, hex)
// Output lines: w0 w1 w2 w3            (hex)
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main()
{
    unsigned long long seed;
    unsigned c0, c1, c2, c3;
    while (std::scanf("%llx %x %x %x %x", &seed, &c0, &c1, &c2, &c3) == 5) {
        // rocRAND maps (subsequence, offset) onto the 128-bit counter as
        // counter = (lo(offset/4), hi(offset/4), lo(subseq), hi(subseq)).
        unsigned long long block = ((unsigned long long)c1 << 32) | c0;
        unsigned long long subseq = ((unsigned long long)c3 << 32) | c2;
        rocrand_device::philox4x32_10_engine eng(seed, subseq, 0);
        // discard() counts single 32-bit outputs (4 per counter step); feed
        // it in pieces so that 4 * block never overflows 64 bits.
        for (unsigned long long t = 0; t < 2 * (block >> 62); ++t)
            eng.discard(1ull << 63);
        eng.discard(4ull * (block & ((1ull << 62) - 1)));
        uint4 r = eng.next4();
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
