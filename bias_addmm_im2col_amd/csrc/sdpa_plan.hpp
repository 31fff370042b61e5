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
  SDPA_Q4 = 0,   // QW 4, KW 1, NB 2: 128 query rows, 64-key tiles
  SDPA_Q2K2 = 1, // QW 2, KW 2, NB 1:  64 query rows, 64-key tiles
  SDPA_K4 = 2,   // QW 1, KW 4, NB 1:  32 query rows, 128-key tiles
  SDPA_NCFG = 3
};
constexpr int kSdpaQW[SDPA_NCFG] = {4, 2, 1};
constexpr int kSdpaKW[SDPA_NCFG] = {1, 2, 4};
constexpr int kSdpaNB[SDPA_NCFG] = {2, 1, 1};

// Configuration for BH (batch x head) slices of Sq queries over Skv keys:
// the one with the least estimated time, counting a block's time as its
// key tiles times (blocks per wave + a fixed per-tile cost) and the blocks
// as ceil(blocks / CUs) rounds.  override_spec ("0".."2", e.g. from an
// environment variable) forces a configuration.
int plan_sdpa(int64_t BH, int64_t Sq, int64_t Skv, const char* override_spec);

}  // namespace baim
