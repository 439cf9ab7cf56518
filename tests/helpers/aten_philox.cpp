// Test helper: runs ATen's header-only Philox4x32-10 engine (an
// implementation independent of the oracle) on counter/key blocks read from
// stdin, one "c0 c1 c2 c3 k0 k1" line per block, and prints the four output
// words.  ATen's engine takes key = seed, counter[2..3] = subsequence,
// counter[0..1] = offset.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>
#include <cstdio>

int main() {
  unsigned c[4], k[2];
  while (std::scanf("%x %x %x %x %x %x", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    uint64_t seed = (uint64_t)k[0] | ((uint64_t)k[1] << 32);
    uint64_t sub = (uint64_t)c[2] | ((uint64_t)c[3] << 32);
    uint64_t off = (uint64_t)c[0] | ((uint64_t)c[1] << 32);
    at::Philox4_32 e(seed, sub, off);
    uint32_t o0 = e(), o1 = e(), o2 = e(), o3 = e();
    std::printf("%08x %08x %08x %08x\n", o0, o1, o2, o3);
  }
  return 0;
}
