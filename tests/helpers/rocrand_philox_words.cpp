// Independent Philox-4x32-10 reference for the oracle's tests: calls rocRAND's
// host-callable engine (its ten-round function) on counters and a key read
// from stdin, and prints the four output words.  Nothing here is compiled
// into the library or the oracle.
//
// stdin:  n  k0 k1  then n lines "c0 c1 c2 c3" (decimal)
// stdout: n lines "x0 x1 x2 x3"
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct Probe : rocrand_device::philox4x32_10_engine {
  uint4 run(uint4 c, uint2 k) { return ten_rounds(c, k); }
};

int main() {
  unsigned long n; unsigned k0, k1;
  if (std::scanf("%lu %u %u", &n, &k0, &k1) != 3) return 1;
  Probe p;
  uint2 key; key.x = k0; key.y = k1;
  for (unsigned long i = 0; i < n; ++i) {
    uint4 c;
    if (std::scanf("%u %u %u %u", &c.x, &c.y, &c.z, &c.w) != 4) return 2;
    uint4 r = p.run(c, key);
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
