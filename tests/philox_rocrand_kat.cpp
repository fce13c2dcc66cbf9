// Known-answer helper: prints rocRAND's Philox4x32-10 block for (seed, group) pairs.
// rocRAND's engine seeded with (seed, subsequence 0, offset 4*g) yields, from its first
// next4(), the block at counter (lo32(g), hi32(g), 0, 0) under key (lo32(seed),
// hi32(seed)).  Reads "seed group" pairs (decimal) from stdin, prints 4 hex words each.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, g;
    while (std::scanf("%llu %llu", &seed, &g) == 2) {
        rocrand_device::philox4x32_10_engine eng(seed, 0ull, 4ull * g);
        uint4 r = eng.next4();
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
