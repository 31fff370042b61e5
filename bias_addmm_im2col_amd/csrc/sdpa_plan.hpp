// sdpa_plan.hpp -- host-side choice of the attention kernel's block shape.
// Plain C++ (no HIP), checked on the host.
#pragma once

#include <stdint.h>

namespace baim {

// A block of the attention kernel is four waves arranged as QW query groups
// (32 query rows each) x KW key groups; per key tile each wave takes NB
// 32-key blocks, so a tile holds 32*NB*KW keys.  Key groups keep separate
// running softmaxes and are merged at the end of the block, in group order.
enum SdpaCfg {
  SDPA_Q4 = 0,   // QW 4, KW 1, NB 2 (NB 1 for D <= 64): 128 query rows
  SDPA_Q2K2 = 1, // QW 2, KW 2, NB 1:  64 query rows, 64-key tiles
  SDPA_K4 = 2,   // QW 1, KW 4, NB 1:  32 query rows, 128-key tiles
  SDPA_NCFG = 3
};
constexpr int kSdpaQW[SDPA_NCFG] = {4, 2, 1};
constexpr int kSdpaKW[SDPA_NCFG] = {1, 2, 4};

// Key blocks per wave and tile.  The 128-row shape takes one 32-key block
// for head dims up to 64: its registers then fit three blocks per CU
// instead of two (measured 6% faster on 197x197, D 64); above 64 it takes
// two, which keeps fewer, longer tiles where occupancy is one block anyway.
constexpr int sdpa_nb(int cfg, int64_t D) { return cfg == SDPA_Q4 ? (D <= 64 ? 1 : 2) : 1; }

// Configuration for BH (batch x head) slices of Sq queries over Skv keys of
// head dim D: the one with the least estimated time, counting a block's
// time as its key tiles times (blocks per wave + a fixed per-tile cost) and
// the blocks as ceil(blocks / CUs) rounds.  override_spec ("0".."2", e.g.
// from an environment variable) forces a configuration.
int plan_sdpa(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const char* override_spec);

}  // namespace baim
