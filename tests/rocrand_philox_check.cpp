// Test helper: evaluates Philox4x32-10 with rocRAND's host-callable engine
// (an independent library implementation) for (counter, key) pairs read from
// stdin, one "c0 c1 c2 c3 k0 k1" line each (hex), printing the four output
// words.  rocRAND's engine places seed = key, the subsequence in counter
// words 2-3 and offset / 4 in counter words 0-1, so c1 must be < 2^30 here.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
    unsigned long long sub = ((unsigned long long)c3 << 32) | c2;
    unsigned long long off = 4ull * (((unsigned long long)c1 << 32) | c0);
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    uint4 r = e.next4();
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
