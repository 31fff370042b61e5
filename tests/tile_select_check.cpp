// Host check of plan_gemm (built with g++ by tests/test_index_math.py):
// every plan covers the problem, has no empty K slice, and honours a valid
// override while ignoring a malformed one.
#include <stdio.h>

#include <initializer_list>

#include "tile_select.hpp"

using namespace baim;

static int check(int M, int N, int K, const char* spec) {
  const GemmPlan p = plan_gemm(M, N, K, spec);
  const int nkt = (K + kTileBK[p.cfg] - 1) / kTileBK[p.cfg];
  if (p.cfg < 0 || p.cfg >= TILE_NCFG) return printf("bad cfg %d\n", p.cfg), 1;
  if ((int64_t)p.tiles_m * kTileBM[p.cfg] < M || (int64_t)(p.tiles_m - 1) * kTileBM[p.cfg] >= M)
    return printf("tiles_m %d wrong for M=%d\n", p.tiles_m, M), 1;
  if ((int64_t)p.tiles_n * kTileBN[p.cfg] < N || (int64_t)(p.tiles_n - 1) * kTileBN[p.cfg] >= N)
    return printf("tiles_n %d wrong for N=%d\n", p.tiles_n, N), 1;
  if (p.splits < 1) return printf("splits %d\n", p.splits), 1;
  if ((p.mode == MODE_SLICES) != (p.splits > 1)) return printf("mode/splits mismatch\n"), 1;
  if (p.mode == MODE_STREAM && (p.workers < 1 || p.workers >= plan_tiles(p) || p.nkt < 2))
    return printf("stream workers %d for %lld tiles\n", p.workers, (long long)plan_tiles(p)), 1;
  if (p.nkt != nkt) return printf("nkt %d != %d\n", p.nkt, nkt), 1;
  if (p.splits > 1) {
    if ((int64_t)p.splits * p.kt_per_split < nkt || (int64_t)(p.splits - 1) * p.kt_per_split >= nkt)
      return printf("slices %d x %d do not tile %d k-tiles\n", p.splits, p.kt_per_split, nkt), 1;
  }
  if (plan_blocks(p) >= (1ll << 31)) return printf("too many blocks\n"), 1;
  return 0;
}

int main() {
  int bad = 0;
  const int sizes[] = {1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 577, 1000, 1024,
                       2048, 3072, 3364, 4096, 12544, 36864};
  const char* specs[] = {nullptr, "", "0", "1", "2", "3", "0,4", "3,2", "1,64", "9", "x", "0,",
                         "0,0", "2,7x", "-1", "1,s256", "4,s1", "3,s100000", "0,s", "2,s0"};
  for (int M : sizes)
    for (int N : sizes)
      for (int K : {0, 1, 31, 32, 147, 768, 1024, 2304, 4096, 100000})
        for (const char* s : specs) bad += check(M, N, K, s);
  // a valid override is honoured
  const GemmPlan f = plan_gemm(4096, 4096, 4096, "3,4");
  if (f.cfg != TILE_64x64 || f.splits != 4) bad += printf("override not honoured\n") > 0;
  // a malformed override is ignored (same as no override)
  const GemmPlan g = plan_gemm(300, 500, 700, "2,7x"), h = plan_gemm(300, 500, 700, nullptr);
  if (g.cfg != h.cfg || g.splits != h.splits) bad += printf("bad override not ignored\n") > 0;
  // a stream override keeps fewer workers than tiles, else falls back to tiles
  const GemmPlan st = plan_gemm(256, 12544, 2304, "1,s256");
  if (st.mode != MODE_STREAM || st.workers != 256) bad += printf("stream override\n") > 0;
  if (plan_gemm(64, 64, 2304, "1,s256").mode != MODE_TILE) bad += printf("stream fallback\n") > 0;
  // M <= 32 takes the 32-row tile
  if (plan_gemm(32, 12544, 288, nullptr).cfg != TILE_32x128) bad += printf("32-row tile\n") > 0;
  if (plan_gemm(7, 4096, 4096, nullptr).cfg != TILE_32x128) bad += printf("32-row tile 2\n") > 0;
  if (plan_gemm(33, 4096, 4096, nullptr).cfg == TILE_32x128) bad += printf("33 rows\n") > 0;
  // a B tile of mat2 [K, N] keeps 32-bit offsets: the 128-row tile moves to
  // a 64-row tile at large N, in the same mode; plans that fit stay
  for (int N : {1, 4096, 4227300, 4227400, 8388607})
    for (const char* s : {"7", "7,3", "7,s9", "0", "6,s5", "4,2"}) {
      const GemmPlan p0 = plan_gemm(64, N, 4096, s);
      const GemmPlan p1 = plan_fit_col_operand(p0, 64, N, 4096);
      if (!plan_col_tile_fits(p1.cfg, N)) bad += printf("col tile N=%d %s\n", N, s) > 0;
      if (plan_col_tile_fits(p0.cfg, N) && (p1.cfg != p0.cfg || p1.mode != p0.mode))
        bad += printf("fitting plan changed N=%d %s\n", N, s) > 0;
      if (p1.mode != p0.mode && !(p0.mode == MODE_STREAM && p1.mode == MODE_TILE))
        bad += printf("mode changed N=%d %s\n", N, s) > 0;
      bad += check(64, N, 4096, s);
    }
  if (plan_col_tile_fits(TILE_64x64_K4, 4227400) || !plan_col_tile_fits(TILE_64x64_K4, 4227300))
    bad += printf("128-row tile limit\n") > 0;
  // K == 0 never splits
  if (plan_gemm(8, 8, 0, "0,4").splits != 1) bad += printf("K=0 split\n") > 0;
  if (bad) return 1;
  printf("OK\n");
  return 0;
}
