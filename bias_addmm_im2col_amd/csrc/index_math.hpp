// index_math.hpp -- integer index helpers shared by host and device code:
// division by a run-time invariant divisor, and the block -> output-tile
// map.  Plain C++ with no HIP dependency, so the host test-suite can build
// and check it with g++.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BAIM_HD __host__ __device__
#else
#define BAIM_HD
#endif

namespace baim {

// Division by a run-time invariant divisor d >= 1 for 0 <= n < 2^32
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994, Fig. 4.1): with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l,
// the sum taken in 64 bits.  Uniform operands keep it on the scalar unit.
struct FastDiv {
  uint32_t d, m, l;
};

BAIM_HD inline uint32_t fdiv(uint32_t n, FastDiv f) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (uint32_t)(((uint64_t)t + n) >> f.l);
}

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((((1ull << l) - d) << 32) / d) + 1;
  return FastDiv{d, (uint32_t)m, l};
}

// Block -> output tile, in two steps.  The hardware hands workgroup i to
// XCD i % 8; xcd_linear gives each XCD a contiguous run of logical ids.
// grouped_tile then walks group_m tile-rows at a time, so neighbouring
// tiles (which share A rows and B columns) run on the same XCD and share
// its L2.
BAIM_HD inline int xcd_linear(int bid, int nblocks) {
  const int q = nblocks >> 3, r = nblocks & 7;
  const int x = bid & 7, i = bid >> 3;
  return x * q + (x < r ? x : r) + i;
}

BAIM_HD inline void grouped_tile(int lid, int tiles_m, int tiles_n, int group_m, int& tm,
                                 int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = lid / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gsz = rows_left < group_m ? rows_left : group_m;
  const int in_g = lid - g * per_group;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

BAIM_HD inline void tile_coords(int bid, int nblocks, int tiles_m, int tiles_n, int group_m,
                                int& tm, int& tn) {
  grouped_tile(xcd_linear(bid, nblocks), tiles_m, tiles_n, group_m, tm, tn);
}

}  // namespace baim
