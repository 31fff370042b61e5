// conv_window_plan.hpp -- host-side choice for the LDS-window conv kernel
// (conv_window.hip): whether a conv's geometry is one of the compiled
// window instances and fits its LDS window, and how its tiles map to
// blocks.  Plain C++ (no HIP), checked on the host.
#pragma once

#include <stdint.h>

namespace baim {

// Compiled window geometries: kernel KH x KW, stride, dilation, and WR, the
// window rows held per input channel (enough for the four output rows a
// run of kWinBN pixels touches at OW >= 43).
enum WinGeom { WIN_3x3_S1_D1 = 0, WIN_3x3_S1_D2 = 1, WIN_NGEOM = 2 };
constexpr int kWinKH[WIN_NGEOM] = {3, 3};
constexpr int kWinKW[WIN_NGEOM] = {3, 3};
constexpr int kWinSH[WIN_NGEOM] = {1, 1};
constexpr int kWinSW[WIN_NGEOM] = {1, 1};
constexpr int kWinDH[WIN_NGEOM] = {1, 2};
constexpr int kWinDW[WIN_NGEOM] = {1, 2};
constexpr int kWinWR[WIN_NGEOM] = {6, 8};
// Block tile (output channels x output pixels of one image), input
// channels per k-tile, LDS window row stride and the column of iw = 0.
constexpr int kWinBM = 64, kWinBN = 128, kWinCI = 16, kWinRS = 64, kWinCL = 4;
constexpr int kWinWaves = 16, kWinKGroups = 2;

// The stem kernel (conv_stem.hip): IC = 3, 7 x 7 kernel, stride 4,
// dilation 1, a block of 128 output channels x 144 output pixels in one
// pass over K.  It needs OW >= 144 (a pixel run spans at most two output
// rows), W % 4 == 0 and OC % 4 == 0 (16-byte input and weight loads).
constexpr int kStemIC = 3, kStemK = 7, kStemS = 4, kStemBM = 128, kStemBN = 144, kStemWaves = 16;

struct WinShape {
  int B, IC, H, W, OC, KH, KW, sH, sW, pH, pW, dH, dW, OH, OW, groups;
};

struct WinPlan {
  int geom;  // WinGeom, or -1 when the window kernel does not apply
  int mode;  // PlanMode (tile_select.hpp)
  int workers, splits, kt_per_split;
  int tiles_m, tiles_n, tpi, nkt;  // tpi: kWinBN-pixel tiles per image
};

// Plan for `s`; `aligned` says input and weight start 16-byte aligned.
// `spec` (may be NULL) is the BAIM_CONV_WIN override: "off" (never the
// window kernel), "tile" (one tile per block), "2" (two K slices) or "sP"
// (stream over P blocks, P below the tile count); an override the problem
// cannot take falls back to one tile per block.
WinPlan plan_conv_window(const WinShape& s, bool aligned, const char* spec);

// Whether the stem kernel computes `s` (`aligned`: input and weight start
// 16-byte aligned; `spec` as for plan_conv_window, "off" declines).
bool plan_conv_stem(const WinShape& s, bool aligned, const char* spec);

inline int64_t win_plan_blocks(const WinPlan& p) {
  if (p.mode == 2) return p.workers;
  return (int64_t)p.tiles_m * p.tiles_n * (p.mode == 1 ? p.splits : 1);
}

}  // namespace baim
