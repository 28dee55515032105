// Host-side reference for Philox4x32-10 outputs from rocRAND's engine
// (a library routine), used only to pin the CPU oracle's Philox.
// Reads lines "c0 c1 c2 c3 k0 k1" and prints the 4 output words.
// rocRAND maps: key = seed, counter words 2..3 = subsequence,
// counter words 0..1 = offset / 4 (offset counted in 32-bit outputs).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
        unsigned long long subseq = ((unsigned long long)c3 << 32) | c2;
        unsigned long long offset = 4ull * (((unsigned long long)c1 << 32) | c0);
        rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
        uint4 r = eng.next4();
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
