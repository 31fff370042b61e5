// conv_window_plan.cpp -- see conv_window_plan.hpp.
#include "conv_window_plan.hpp"

#include <stdlib.h>
#include <string.h>

#include "tile_select.hpp"

namespace baim {

namespace {

bool geom_fits(int g, const WinShape& s) {
  if (s.KH != kWinKH[g] || s.KW != kWinKW[g] || s.sH != kWinSH[g] || s.sW != kWinSW[g] ||
      s.dH != kWinDH[g] || s.dW != kWinDW[g])
    return false;
  // rows copied as whole 16-byte quads, plus a 4-byte tail where compiled
  if (kWinTail[g] ? s.W / 4 > kWinMaxQ[g] : s.W % 4 != 0) return false;
  // output rows a run of kWinBN pixels can touch, and the window rows they need
  const int rows = (kWinBN[g] - 1 + s.OW - 1) / s.OW + 1;
  if ((rows - 1) * s.sH + (s.KH - 1) * s.dH + 1 > kWinWR[g]) return false;
  // every column read, [CL - pW, CL + W + pW), lies in a window row
  return s.pW <= kWinCL && s.W + s.pW + kWinCL <= kWinRS;
}

}  // namespace

WinPlan plan_conv_window(const WinShape& s, bool aligned, const char* spec) {
  WinPlan p{};
  p.geom = -1;
  p.mode = MODE_TILE;
  p.splits = 1;
  if (spec && strcmp(spec, "off") == 0) return p;
  // 16-byte loads of input rows and of weight rows (K = IC*9)
  if (s.groups != 1 || s.IC % 4 != 0 || !aligned) return p;
  if (s.B < 1 || s.IC < 1 || s.OC < 1 || s.OH < 1 || s.OW < 1) return p;
  for (int g = 0; g < WIN_NGEOM; ++g)
    if (geom_fits(g, s)) {
      p.geom = g;
      break;
    }
  if (p.geom < 0) return p;
  const int P = s.OH * s.OW;
  p.tpi = (P + kWinBN[p.geom] - 1) / kWinBN[p.geom];
  p.tiles_m = (s.OC + kWinBM[p.geom] - 1) / kWinBM[p.geom];
  p.tiles_n = s.B * p.tpi;
  p.nkt = (s.IC + kWinCI - 1) / kWinCI;
  p.kt_per_split = p.nkt;
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  // Between one and two blocks per CU, one tile per block would leave most
  // CUs idle in the second round: stream the (tile, k-tile) units over one
  // block per CU instead (fewer blocks than tiles keeps every tile in at
  // most two pieces, combined by the deterministic exchange).
  if (kWinStream[p.geom] && tiles > kNumCUs && tiles < 2 * kNumCUs && p.nkt >= 2) {
    p.mode = MODE_STREAM;
    p.workers = kNumCUs;
  }
  if (spec && spec[0]) {
    p.mode = MODE_TILE;
    p.workers = 0;
    if (spec[0] == 's') {
      char* end = nullptr;
      const long w = strtol(spec + 1, &end, 10);
      if (end != spec + 1 && *end == '\0' && w >= 1 && w < tiles && p.nkt >= 2 &&
          kWinStream[p.geom]) {
        p.mode = MODE_STREAM;
        p.workers = (int)w;
      }
    } else if (strcmp(spec, "2") == 0 && p.nkt >= 2) {
      p.mode = MODE_SLICES;
      p.splits = 2;
      p.kt_per_split = (p.nkt + 1) / 2;
    }
  }
  return p;
}

bool plan_conv_stem(const WinShape& s, bool aligned, const char* spec) {
  if (spec && strcmp(spec, "off") == 0) return false;
  return aligned && s.groups == 1 && s.IC == kStemIC && s.KH == kStemK && s.KW == kStemK &&
         s.sH == kStemS && s.sW == kStemS && s.dH == 1 && s.dW == 1 && s.OW >= kStemBN &&
         s.W % 4 == 0 && s.OC % 4 == 0 && s.B >= 1 && s.OH >= 1;
}

}  // namespace baim
