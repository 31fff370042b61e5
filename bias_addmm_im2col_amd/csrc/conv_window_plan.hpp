// conv_window_plan.hpp -- host-side choice for the LDS-window conv kernel
// (conv_window.hip): whether a conv's geometry is one of the compiled
// window instances and fits its LDS window, and how its tiles map to
// blocks.  Plain C++ (no HIP), checked on the host.
#pragma once

#include <stdint.h>

namespace baim {

// Compiled window geometries: kernel KH x KW, stride, dilation, and WR, the
// window rows held per input channel (enough for the output rows a run of
// the geometry's kWinBN pixels touches: four at stride 1 with OW >= 43, four
// at stride 2 with 64 pixels and OW >= 21).
enum WinGeom { WIN_3x3_S1_D1 = 0, WIN_3x3_S1_D2 = 1, WIN_3x3_S2_D1 = 2, WIN_NGEOM = 3 };
constexpr int kWinKH[WIN_NGEOM] = {3, 3, 3};
constexpr int kWinKW[WIN_NGEOM] = {3, 3, 3};
constexpr int kWinSH[WIN_NGEOM] = {1, 1, 2};
constexpr int kWinSW[WIN_NGEOM] = {1, 1, 2};
constexpr int kWinDH[WIN_NGEOM] = {1, 2, 1};
constexpr int kWinDW[WIN_NGEOM] = {1, 2, 1};
constexpr int kWinWR[WIN_NGEOM] = {6, 8, 9};
// Block tile per geometry (output channels x output pixels of one image) and
// its wave groups splitting each k-tile.  The stride-2 conv has a quarter of
// the pixels of a stride-1 conv of the same input, so it takes half the tile
// width to keep about one tile per CU.
constexpr int kWinBM[WIN_NGEOM] = {64, 64, 64};
constexpr int kWinBN[WIN_NGEOM] = {128, 128, 64};
constexpr int kWinKGroups[WIN_NGEOM] = {2, 2, 4};
// Input rows: the stride-1 instances copy rows of W % 4 == 0 floats as
// 16-byte quads; the stride-2 instance also takes any other W, copying the
// W / 4 whole quads (at most kWinMaxQ) 16 bytes at a time from wherever the
// row starts and the last W % 4 columns 4 bytes at a time.
constexpr bool kWinTail[WIN_NGEOM] = {false, false, true};
constexpr int kWinMaxQ[WIN_NGEOM] = {15, 15, 14};
// Whether the geometry has a streamed (two-piece) kernel: the stride-2
// instance's would not fit its registers, so its tiles always run one per
// block (or in two K slices when forced).
constexpr bool kWinStream[WIN_NGEOM] = {true, true, false};
// Input channels per k-tile, LDS window row stride, the column of iw = 0.
constexpr int kWinCI = 16, kWinRS = 64, kWinCL = 4;
constexpr int kWinWaves = 16;

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
  int tiles_m, tiles_n, tpi, nkt;  // tpi: kWinBN[geom]-pixel tiles per image
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
