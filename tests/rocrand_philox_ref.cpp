// Reference Philox4x32-10 outputs from rocRAND's engine (an independent library
// implementation), for pinning the oracle.  Reads lines "c0 c1 c2 c3 k0 k1" (hex)
// on stdin and prints the four output words (hex) per line.
//
// rocRAND's engine keeps key = seed and counter = {offset/4 (words 0,1),
// subsequence (words 2,3)}; seeding with those values makes next4() return the
// bijection applied to exactly (counter, key).
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main()
{
    unsigned c[4], k[2];
    while (std::scanf("%x %x %x %x %x %x", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
        unsigned long long seed = (unsigned long long)k[0] | ((unsigned long long)k[1] << 32);
        unsigned long long subseq = (unsigned long long)c[2] | ((unsigned long long)c[3] << 32);
        unsigned long long offset = ((unsigned long long)c[0] | ((unsigned long long)c[1] << 32)) * 4ull;
        rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
        uint4 r = eng.next4();
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
