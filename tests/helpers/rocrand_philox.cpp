// Host-side driver around rocRAND's Philox-4x32-10 engine, used only to cross-check the
// oracle's own Philox implementation. Reads lines "c0 c1 c2 c3 k0 k1" (decimal uint32) on
// stdin and prints the four output words of the block (counter, key) for each.
//
// rocRAND's engine is addressed through its public seeding API: the 64-bit seed is the key,
// the subsequence index fills counter words 2-3, and the offset (in 32-bit outputs, four per
// block) fills counter words 0-1.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned int c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    if (c1 >= (1u << 30)) { std::printf("ERR\n"); continue; }
    const unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
    const unsigned long long subseq = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    const unsigned long long offset = 4ull * ((unsigned long long)c0 | ((unsigned long long)c1 << 32));
    rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
    uint4 r = eng.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
