// tile_select.cpp -- see tile_select.hpp.
//
// The choice follows how the chip fills (256 CUs) and how deep K is; the
// thresholds come from timing every configuration on the workload shapes
// (large / down / up projections, FFN, ragged 577-row, 3x3 and 7x7 convs):
//  * >= 256 tiles of 256x256 that fill the CUs evenly, K >= 512: the
//    256x256 tile (8 waves of 128x64; a third of the LDS reads per MFMA
//    of the 128x128 tile's 64x32 waves).  addmm only: its kernel indexes
//    the whole of mat2 and a 256-row panel of mat1 with 32-bit offsets.
//  * >= 512 tiles of 128x128: the 128x128 tile (most reuse per byte).
//  * >= 192 such tiles and deep K: 128x128 with each k-tile split over two
//    wave groups (16 waves per block: one block per CU still keeps four
//    waves per SIMD); below 256 tiles, 128x64 pieces streamed over exactly
//    one block per CU instead, so no CU idles.
//  * >= 256 such tiles and moderate K: half-size tiles (more blocks).
//  * many 64x64 tiles, or very shallow K: 64x64.
//  * few tiles and deep K: 64x64 with 2 or 4 wave groups per tile.
//  * so few tiles that one per CU is out of reach, with deep K: K is split
//    across blocks, which add partial tiles into a pre-initialised output
//    with atomics.  Only this last case is not bit-reproducible run to run.
#include "tile_select.hpp"

#include <stdlib.h>

namespace baim {

namespace {

int cdiv(int a, int b) { return (a + b - 1) / b; }

GemmPlan make(int cfg, int M, int N, int K, int splits) {
  GemmPlan p;
  p.cfg = cfg;
  p.tiles_m = cdiv(M, kTileBM[cfg]);
  p.tiles_n = cdiv(N, kTileBN[cfg]);
  p.nkt = cdiv(K, kTileBK[cfg]);
  p.mode = MODE_TILE;
  p.splits = 1;
  p.kt_per_split = p.nkt;
  p.workers = 0;
  if (splits > p.nkt) splits = p.nkt;
  if (splits >= 2 && kTileSlices[cfg]) {
    p.kt_per_split = cdiv(p.nkt, splits);
    // drop slices that would be empty after rounding up the slice length
    p.splits = cdiv(p.nkt, p.kt_per_split);
    if (p.splits >= 2) {
      p.mode = MODE_SLICES;
    } else {
      p.splits = 1;
      p.kt_per_split = p.nkt;
    }
  }
  return p;
}

GemmPlan make_stream(int cfg, int M, int N, int K, int64_t workers) {
  GemmPlan p = make(cfg, M, N, K, 1);
  // fewer workers than tiles keeps every tile in at most two pieces
  if (kTileStream[cfg] && p.nkt >= 2 && workers >= 1 && workers < plan_tiles(p)) {
    p.mode = MODE_STREAM;
    p.workers = (int)workers;
  }
  return p;
}

int64_t tiles_of(int cfg, int M, int N) {
  return (int64_t)cdiv(M, kTileBM[cfg]) * cdiv(N, kTileBN[cfg]);
}

// "cfg", "cfg,S" or "cfg,sP"
bool parse_override(const char* s, int* cfg, int* splits, int* workers) {
  if (!s || !*s) return false;
  char* end = nullptr;
  const long c = strtol(s, &end, 10);
  if (end == s || c < 0 || c >= TILE_NCFG) return false;
  long k = 1, w = 0;
  if (*end == ',') {
    const char* t = end + 1;
    if (*t == 's') {
      ++t;
      w = strtol(t, &end, 10);
      if (end == t || w < 1 || w > (1 << 20)) return false;
    } else {
      k = strtol(t, &end, 10);
      if (end == t || k < 1 || k > 64) return false;
    }
  }
  if (*end != '\0') return false;
  *cfg = (int)c;
  *splits = (int)k;
  *workers = (int)w;
  return true;
}

}  // namespace

GemmPlan plan_gemm(int M, int N, int K, const char* override_spec) {
  int cfg = 0, splits = 1, workers = 0;
  if (parse_override(override_spec, &cfg, &splits, &workers))
    return workers > 0 ? make_stream(cfg, M, N, K, workers) : make(cfg, M, N, K, splits);

  const int nkt = cdiv(K, 32);  // k-tiles of depth 32
  if (M <= 32) {
    // A 64-row tile would leave at least half its rows idle: 32 x 128
    // tiles, with K split across blocks only when they cannot give half
    // the CUs a block and K is deep (at least 8 k-tiles per slice).
    const int64_t t = tiles_of(TILE_32x128, M, N);
    if (t >= kNumCUs / 2 || nkt <= 8) return make(TILE_32x128, M, N, K, 1);
    int s = (int)((kNumCUs + t - 1) / t);
    if (s > nkt / 8) s = nkt / 8;
    return make(TILE_32x128, M, N, K, s < 1 ? 1 : s);
  }
  const int64_t t256 = tiles_of(TILE_256x256, M, N);
  if (t256 >= kNumCUs && (t256 % kNumCUs == 0 || t256 >= 4 * kNumCUs) && K >= 512 &&
      plan_big_fits(N, K))
    return make(TILE_256x256, M, N, K, 1);
  const int64_t t128 = tiles_of(TILE_128x128, M, N);
  if (t128 >= 2 * kNumCUs) return make(TILE_128x128, M, N, K, 1);
  if (t128 >= (3 * kNumCUs) / 4 && nkt >= 48) {
    // 192..255 tiles leave CUs idle; stream 128x64 pieces over exactly one
    // block per CU instead (at most two pieces per tile, combined
    // deterministically).  On the 3x3 conv: 174 -> 167 us.
    if (t128 < kNumCUs && tiles_of(TILE_128x64_K2, M, N) >= kNumCUs)
      return make_stream(TILE_128x64_K2, M, N, K, kNumCUs);
    return make(TILE_128x128_K2, M, N, K, 1);
  }
  if (t128 >= kNumCUs && nkt > 8) {
    // Half-size tiles: the orientation that wastes less of a ragged edge;
    // on a tie the 64-row tile.
    const int64_t t_wide = tiles_of(TILE_128x64, M, N), t_tall = tiles_of(TILE_64x128, M, N);
    return make(t_wide < t_tall ? TILE_128x64 : TILE_64x128, M, N, K, 1);
  }
  const int64_t t64 = tiles_of(TILE_64x64, M, N);
  if (t64 >= 2 * kNumCUs || nkt <= 8) return make(TILE_64x64, M, N, K, 1);
  if (t64 >= kNumCUs / 4 || nkt < 64)
    return make(nkt >= 64 ? TILE_64x64_K4 : (nkt >= 32 ? TILE_64x64_K2 : TILE_64x64), M, N, K, 1);
  // Fewer than a quarter of the CUs would get a tile: split K (depth-128
  // k-tiles of the 4-group 64x64 tile) so tiles * splits covers the CUs,
  // keeping at least 8 k-tiles per slice.
  const int nkt128 = cdiv(K, 128);
  int s = (int)((kNumCUs + t64 - 1) / t64);
  if (s > nkt128 / 8) s = nkt128 / 8;
  return make(TILE_64x64_K4, M, N, K, s < 1 ? 1 : s);
}

GemmPlan plan_tiles_only(const GemmPlan& p, int M, int N, int K) {
  return make(p.cfg, M, N, K, 1);
}

GemmPlan plan_core_tile(const GemmPlan& p, int M, int N, int K) {
  return kTileCore[p.cfg] ? p : make(TILE_128x128, M, N, K, 1);
}

bool plan_col_tile_fits(int cfg, int N) {
  return ((int64_t)(kTileBK[cfg] - 1) * N + kTileBN[cfg]) * 4 < ((int64_t)1 << 31);
}

GemmPlan plan_fit_col_operand(const GemmPlan& p, int M, int N, int K) {
  if (plan_col_tile_fits(p.cfg, N)) return p;
  if (p.mode == MODE_STREAM) return make_stream(TILE_64x64_K2, M, N, K, p.workers);
  return make(TILE_64x64_K2, M, N, K, p.mode == MODE_SLICES ? p.splits : 1);
}

}  // namespace baim
