// tile_select.hpp -- host-side choice of block tile and K split for one
// GEMM problem (M, N, K).  Plain C++ (no HIP), checked on the host.
#pragma once

#include <stdint.h>

namespace baim {

// Block-tile configurations compiled into the library.  The _K2/_K4
// variants split every k-tile over 2 or 4 groups of waves (more waves per
// output tile, partial tiles summed through LDS in group order).
enum TileCfg {
  TILE_128x128 = 0,     // BK 32, 8 waves, 64x32 per wave
  TILE_128x64 = 1,      // BK 32, 8 waves, 32x32 per wave
  TILE_64x128 = 2,      // BK 32, 8 waves, 32x32 per wave
  TILE_64x64 = 3,       // BK 32, 4 waves, 32x32 per wave
  TILE_128x128_K2 = 4,  // BK 64, 16 waves
  TILE_128x64_K2 = 5,   // BK 64, 16 waves
  TILE_64x64_K2 = 6,    // BK 64, 8 waves
  TILE_64x64_K4 = 7,    // BK 128, 16 waves
  TILE_NCFG = 8
};

constexpr int kTileBM[TILE_NCFG] = {128, 128, 64, 64, 128, 128, 64, 64};
constexpr int kTileBN[TILE_NCFG] = {128, 64, 128, 64, 128, 64, 64, 64};
constexpr int kTileBK[TILE_NCFG] = {32, 32, 32, 32, 64, 64, 64, 128};
constexpr int kTileWaves[TILE_NCFG] = {8, 8, 8, 4, 16, 16, 8, 16};
constexpr int kTileKGroups[TILE_NCFG] = {1, 1, 1, 1, 2, 2, 2, 4};
constexpr int kNumCUs = 256;  // MI355X

struct GemmPlan {
  int cfg;           // TileCfg
  int tiles_m, tiles_n;
  int splits;        // K slices (1: no split); every slice is non-empty
  int kt_per_split;  // k-tiles per slice
};

// Plan for problem (M, N, K) with every dimension >= 0.  `override_spec`
// (may be NULL) is "cfg" or "cfg,splits" and forces the choice; an
// unparsable or out-of-range spec is ignored.
GemmPlan plan_gemm(int M, int N, int K, const char* override_spec);

// The block count of a plan.
inline int64_t plan_blocks(const GemmPlan& p) {
  return (int64_t)p.tiles_m * p.tiles_n * p.splits;
}

}  // namespace baim
