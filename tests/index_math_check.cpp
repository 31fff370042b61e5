// Host check of the kernels' integer index helpers (built with g++ by
// tests/test_index_math.py): multiply-high division against '/', and the
// block -> tile map being a bijection onto the tile grid.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "index_math.hpp"

using namespace baim;

static int check_div(uint32_t d, uint32_t n) {
  const FastDiv f = make_fastdiv(d);
  if (fdiv(n, f) != n / d) {
    printf("fdiv wrong: n=%u d=%u got %u want %u\n", n, d, fdiv(n, f), n / d);
    return 1;
  }
  return 0;
}

int main() {
  int bad = 0;
  // every divisor up to 4096 against every n up to 2^16, plus edges
  for (uint32_t d = 1; d <= 4096 && !bad; ++d) {
    for (uint32_t n = 0; n < (1u << 16); ++n) bad += check_div(d, n);
    const uint32_t edges[] = {d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7FFFFFFFu, 0x80000000u,
                              0xFFFFFFFEu, 0xFFFFFFFFu, (0xFFFFFFFFu / d) * d,
                              (0xFFFFFFFFu / d) * d - 1};
    for (uint32_t n : edges) bad += check_div(d, n);
  }
  // large and power-of-two divisors, pseudo-random numerators
  uint64_t s = 88172645463325252ull;
  for (int t = 0; t < 2000000 && !bad; ++t) {
    s ^= s << 13; s ^= s >> 7; s ^= s << 17;
    uint32_t d = (uint32_t)(s >> 32);
    if (t % 3 == 0) d = 1u << (s % 32);
    if (t % 3 == 1) d = (uint32_t)(s % 100000) + 1;
    if (d == 0) d = 1;
    bad += check_div(d, (uint32_t)s);
  }
  // tile map: every (tm, tn) exactly once, for many grids and group sizes
  for (int tiles_m = 1; tiles_m <= 70 && !bad; ++tiles_m)
    for (int tiles_n = 1; tiles_n <= 70 && !bad; tiles_n += (tiles_n < 20 ? 1 : 7))
      for (int group_m : {1, 2, 4, 8, 16}) {
        const int nb = tiles_m * tiles_n;
        std::vector<int> seen(nb, 0);
        for (int bid = 0; bid < nb; ++bid) {
          int tm, tn;
          tile_coords(bid, nb, tiles_m, tiles_n, group_m, tm, tn);
          if (tm < 0 || tm >= tiles_m || tn < 0 || tn >= tiles_n) {
            printf("tile out of range: %d %d (grid %dx%d g%d bid %d)\n", tm, tn, tiles_m,
                   tiles_n, group_m, bid);
            return 1;
          }
          seen[tm * tiles_n + tn]++;
        }
        for (int i = 0; i < nb; ++i)
          if (seen[i] != 1) {
            printf("tile %d seen %d times (grid %dx%d g%d)\n", i, seen[i], tiles_m, tiles_n,
                   group_m);
            return 1;
          }
      }
  if (bad) return 1;
  printf("OK\n");
  return 0;
}
