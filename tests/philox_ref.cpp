// Reference values of Philox4x32-10 from rocRAND's engine (a library
// implementation, header-only, built for the host), used to pin the oracle's
// own generator and its dropout convention.  Test helper; no GPU code.
//
//   philox_ref words   reads "k0 k1 c0 c1 c2 c3" lines (c1 < 2^30), prints the
//                      four output words of counter (c0,c1,c2,c3) under key (k0,k1)
//   philox_ref keep    reads "seed offset thr bh i j" lines, prints 1 if element
//                      (bh, i, j) is kept: of word j%4 of counter (j/4, i/2, bh,
//                      offset) under key (seed low, seed high), the low 16 bits
//                      for even i and the high 16 bits for odd i, are >= thr
//
// The engine's state is (key = seed, counter = (offset/4 as 64 bits,
// subsequence as 64 bits)), and next() returns word offset%4 of it.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstring>

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  if (!strcmp(argv[1], "words")) {
    unsigned long long k0, k1, c0, c1, c2, c3;
    while (scanf("%llu %llu %llu %llu %llu %llu", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
      if (c1 >= (1ull << 30)) return 3;
      rocrand_device::philox4x32_10_engine e(k0 | (k1 << 32), c2 | (c3 << 32), 4ull * (c0 | (c1 << 32)));
      const uint4 r = e.next4();
      printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
  }
  if (!strcmp(argv[1], "keep")) {
    unsigned long long seed, off, thr, bh, i, j;
    while (scanf("%llu %llu %llu %llu %llu %llu", &seed, &off, &thr, &bh, &i, &j) == 6) {
      if (i / 2 >= (1ull << 30)) return 3;
      rocrand_device::philox4x32_10_engine e(seed, bh | (off << 32), 4ull * ((j / 4) | ((i / 2) << 32)) + j % 4);
      const unsigned long long half = ((unsigned long long)e.next() >> (16 * (i % 2))) & 0xFFFFull;
      printf("%d\n", half >= thr ? 1 : 0);
    }
    return 0;
  }
  return 2;
}
