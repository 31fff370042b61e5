// sdpa_plan.hpp -- host-side choice of the attention kernel's block shape.
// Plain C++ (no HIP), checked on the host.
#pragma once

#include <stdint.h>

namespace baim {

// A block of the attention kernel is four (or eight) waves arranged as QW
// query groups (32 query rows each) x KW key groups; per key tile each wave
// takes NB 32-key blocks, so a tile holds 32*NB*KW keys.  Key groups keep
// separate running softmaxes and are merged at the end of the block, in
// group order.
enum SdpaCfg {
  SDPA_Q4 = 0,   // QW 4, KW 1, NB 2 (NB 1 for D <= 64): 128 query rows
  SDPA_Q2K2 = 1, // QW 2, KW 2, NB 1:  64 query rows, 64-key tiles
  SDPA_K4 = 2,   // QW 1, KW 4, NB 1:  32 query rows, 128-key tiles
  SDPA_K8 = 3,   // QW 1, KW 8, NB 1:  32 query rows, 256-key tiles, eight
                 // waves (two per SIMD); D <= kSdpaK8MaxD only
  SDPA_NCFG = 4
};
constexpr int kSdpaQW[SDPA_NCFG] = {4, 2, 1, 1};
constexpr int kSdpaKW[SDPA_NCFG] = {1, 2, 4, 8};
// Above this head dim the eight-wave shape's registers (two waves per SIMD)
// do not fit its k/v prefetch and O accumulators.
constexpr int kSdpaK8MaxD = 64;

// Key blocks per wave and tile.  The 128-row shape takes one 32-key block
// for head dims up to 64: its registers then fit three blocks per CU
// instead of two (measured 6% faster on 197x197, D 64); above 64 it takes
// two, which keeps fewer, longer tiles where occupancy is one block anyway.
constexpr int sdpa_nb(int cfg, int64_t D) { return cfg == SDPA_Q4 ? (D <= 64 ? 1 : 2) : 1; }

// Configuration for BH (batch x head) slices of Sq queries over Skv keys of
// head dim D: the one with the least estimated time, counting a block's
// time as its key tiles times (key blocks per SIMD + a fixed per-tile cost)
// and the blocks as ceil(blocks / CUs) rounds; an eight-wave tile has two
// waves' key blocks per SIMD, and the eight-wave shape is only considered
// when BH * ceil(Sq / 32) blocks fit one round.  override_spec ("0".."3",
// e.g. from an environment variable) forces a configuration; the
// eight-wave one is ignored above kSdpaK8MaxD.
int plan_sdpa(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const char* override_spec);

}  // namespace baim
