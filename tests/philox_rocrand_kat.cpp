// Known-answer helper: prints rocRAND's Philox4x32-10 block for (seed, group, stream)
// triples.  rocRAND's engine seeded with (seed, subsequence s, offset 4*g) yields, from
// its first next4(), the block at counter (lo32(g), hi32(g), lo32(s), hi32(s)) under key
// (lo32(seed), hi32(seed)): the subsequence fills counter words 2 and 3.  Reads
// "seed group stream" triples (decimal) from stdin, prints 4 hex words each.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, g, sub;
    while (std::scanf("%llu %llu %llu", &seed, &g, &sub) == 3) {
        rocrand_device::philox4x32_10_engine eng(seed, sub, 4ull * g);
        uint4 r = eng.next4();
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
