// Host program for the Philox pin: prints rocRAND's Philox4x32-10 block for
// each (key0 key1 c0 c1 c2 c3) line read on stdin. rocRAND's engine is an
// implementation independent of the oracle (numpy) and of the GPU library.
// The engine is seeded with key = seed, counter words (c2, c3) through the
// subsequence and (c0, c1) through skips that add up to 4 * (c1:c0) outputs
// (in pieces, so no skip overflows 64 bits), so its current block is the one
// for counter (c0, c1, c2, c3).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned k0, k1, c0, c1, c2, c3;
  while (std::scanf("%u %u %u %u %u %u", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
    const unsigned long long seed = (static_cast<unsigned long long>(k1) << 32) | k0;
    const unsigned long long subsequence = (static_cast<unsigned long long>(c3) << 32) | c2;
    const unsigned long long blocks = (static_cast<unsigned long long>(c1) << 32) | c0;
    rocrand_device::philox4x32_10_engine engine(seed, subsequence, 0);
    for (int i = 0; i < 4; ++i) engine.discard((blocks >> 2) * 4ull);
    engine.discard((blocks & 3ull) * 4ull);
    const uint4 r = engine.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
