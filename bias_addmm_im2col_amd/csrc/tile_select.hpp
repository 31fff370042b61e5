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
  TILE_32x128 = 8,      // BK 32, 4 waves, 32x32 per wave: GEMMs with M <= 32
  TILE_256x256 = 9,     // BK 16, 8 waves, 128x64 per wave: large addmm (own kernel)
  TILE_NCFG = 10
};

constexpr int kTileBM[TILE_NCFG] = {128, 128, 64, 64, 128, 128, 64, 64, 32, 256};
constexpr int kTileBN[TILE_NCFG] = {128, 64, 128, 64, 128, 64, 64, 64, 128, 256};
constexpr int kTileBK[TILE_NCFG] = {32, 32, 32, 32, 64, 64, 64, 128, 32, 16};
constexpr int kTileWaves[TILE_NCFG] = {8, 8, 8, 4, 16, 16, 8, 16, 4, 8};
constexpr int kTileKGroups[TILE_NCFG] = {1, 1, 1, 1, 2, 2, 2, 4, 1, 1};
// Configurations compiled with the K-slice and stream schedules (the
// others would exceed their register budget with the extra state).
constexpr bool kTileSlices[TILE_NCFG] = {true, true, true, true, false, true, true, true, true, false};
constexpr bool kTileStream[TILE_NCFG] = {true, true, true, true, false, true, true, false, true, false};
// Configurations the tile-core kernels run (addmm's other instances,
// linear, the im2col convs): the 256x256 tile has a kernel of its own for
// addmm, and plan_core_tile maps it to the 128x128 tile for the others.
constexpr bool kTileCore[TILE_NCFG] = {true, true, true, true, true, true, true, true, true, false};
constexpr int kNumCUs = 256;  // MI355X

// How blocks map to work (the kernels' scheduling modes).
enum PlanMode {
  MODE_TILE = 0,    // one output tile per block
  MODE_SLICES = 1,  // tiles x splits blocks, one K slice each
  MODE_STREAM = 2,  // `workers` blocks share the (tile, k-tile) units evenly
};

struct GemmPlan {
  int cfg;  // TileCfg
  int tiles_m, tiles_n;
  int nkt;           // k-tiles of the tile's BK per tile
  int mode;          // PlanMode
  int splits;        // MODE_SLICES: K slices (>= 2, none empty); else 1
  int kt_per_split;  // MODE_SLICES: k-tiles per slice
  int workers;       // MODE_STREAM: blocks (< tiles, so a tile has at most 2 pieces)
};

// Plan for problem (M, N, K) with every dimension >= 0.  `override_spec`
// (may be NULL) forces the choice: "cfg" (one tile per block), "cfg,S" (S
// K slices) or "cfg,sP" (stream over P blocks); an unparsable or
// out-of-range spec is ignored.
GemmPlan plan_gemm(int M, int N, int K, const char* override_spec);

// The same tile configuration with one tile per block.
GemmPlan plan_tiles_only(const GemmPlan& p, int M, int N, int K);

// `p` for a tile-core kernel: the 256x256 configuration, which only the
// dedicated addmm kernel runs, becomes the 128x128 tile, one tile per
// block (what the planner chose for such sizes before the 256x256 tile
// existed).
GemmPlan plan_core_tile(const GemmPlan& p, int M, int N, int K);

// Whether the 256x256 kernel's 32-bit offsets reach all of mat2 [K, N] and
// a 256-row panel of mat1 [M, K].
inline bool plan_big_fits(int N, int K) {
  return (int64_t)K * N < ((int64_t)1 << 29) && (int64_t)256 * K < ((int64_t)1 << 29);
}

// Whether a B tile read from a row-major [K, N] matrix (mat2) keeps every
// in-tile byte offset below 2^31: the tile spans BK rows of N floats, so
// (BK - 1) * N + BN floats must stay addressable by a 32-bit offset.
bool plan_col_tile_fits(int cfg, int N);

// `p` with its configuration replaced, if its B tile over a row-major
// [K, N] matrix would not fit 32-bit offsets, by the 64x64x64 tile (BK 64),
// in the same mode (slices or stream) where that tile allows it.
GemmPlan plan_fit_col_operand(const GemmPlan& p, int M, int N, int K);

inline int64_t plan_tiles(const GemmPlan& p) { return (int64_t)p.tiles_m * p.tiles_n; }

// The block count of a plan.
inline int64_t plan_blocks(const GemmPlan& p) {
  if (p.mode == MODE_STREAM) return p.workers;
  return plan_tiles(p) * (p.mode == MODE_SLICES ? p.splits : 1);
}

// Whether out must be initialised before the GEMM kernel, and whether the
// split tiles are combined by the two-piece exchange (else atomic adds).
inline bool plan_needs_init(const GemmPlan& p) { return p.mode != MODE_TILE; }
inline bool plan_uses_exchange(const GemmPlan& p) {
  return p.mode == MODE_STREAM || (p.mode == MODE_SLICES && p.splits == 2);
}

}  // namespace baim
