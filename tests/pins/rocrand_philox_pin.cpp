// Runs rocRAND's Philox4x32-10 engine on the host as an independent reference for the
// oracle's Philox.  Reads lines "key0 key1 c0 c1 c2 c3" (hex) on stdin and prints the four
// output words of the block at that counter under that key (hex), one line per input.
// rocRAND maps (seed, subsequence, offset) to key = seed, counter = (offset/4 as the low
// 64 bits, subsequence as the high 64 bits); the block at the counter is the first result.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdint>

int main() {
    unsigned k0, k1, c0, c1, c2, c3;
    while (std::scanf("%x %x %x %x %x %x", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
        unsigned long long subseq = ((unsigned long long)c3 << 32) | c2;
        unsigned long long block = ((unsigned long long)c1 << 32) | c0;
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, subseq, 0, &st);
        // advance by whole blocks: offset counts 32-bit outputs, 4 per block
        if (block) {
            // skipahead takes an element count; split to stay exact for any 64-bit block
            unsigned long long hi = block >> 60, lo = block & ((1ull << 60) - 1);
            skipahead(lo * 4ull, &st);
            for (unsigned long long i = 0; i < hi; ++i) {
                skipahead((1ull << 60) * 2ull, &st);
                skipahead((1ull << 60) * 2ull, &st);
            }
        }
        uint4 w = rocrand4(&st);
        std::printf("%08x %08x %08x %08x\n", w.x, w.y, w.z, w.w);
    }
    return 0;
}
