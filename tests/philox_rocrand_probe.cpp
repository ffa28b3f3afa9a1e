// Host-only known-answer source for the oracle's Philox4x32-10: rocRAND's
// Philox engine (its header source, compiled for the host; no GPU is used).
//
// stdin, one query per line:
//   w c0 c1 c2 c3 k0 k1   -> the four output words of the 4x32 counter
//                            (c0..c3) under the 2x32 key (k0, k1)
//   u seed offset         -> the first 32-bit output of the stream
//                            rocrand_init(seed, subsequence 0, 4 * offset)
// rocRAND places the seed in the key (low word first), a subsequence in
// counter words 2-3 and an offset, counted in single outputs, in words 0-1
// (four outputs per counter value).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstring>

static uint4 block_at(unsigned long long c01, unsigned long long c23, unsigned long long key) {
  rocrand_state_philox4x32_10 st;
  rocrand_init(key, c23, 0, &st);
  // advance the counter by c01 blocks of four outputs, in steps that keep
  // the output count within 64 bits
  const unsigned long long step = 1ull << 61;
  while (c01 >= step) {
    skipahead(step * 4ull, &st);
    c01 -= step;
  }
  if (c01) skipahead(c01 * 4ull, &st);
  return rocrand4(&st);
}

int main() {
  char kind[4];
  while (std::scanf("%3s", kind) == 1) {
    if (std::strcmp(kind, "w") == 0) {
      unsigned c0, c1, c2, c3, k0, k1;
      if (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) != 6) return 2;
      const uint4 r = block_at(((unsigned long long)c1 << 32) | c0,
                               ((unsigned long long)c3 << 32) | c2,
                               ((unsigned long long)k1 << 32) | k0);
      std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    } else if (std::strcmp(kind, "u") == 0) {
      unsigned long long seed, offset;
      if (std::scanf("%llu %llu", &seed, &offset) != 2) return 2;
      rocrand_state_philox4x32_10 st;
      rocrand_init(seed, 0, 4ull * offset, &st);
      std::printf("%u\n", rocrand(&st));
    } else {
      return 2;
    }
  }
  return 0;
}
