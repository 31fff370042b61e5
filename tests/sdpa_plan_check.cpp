// Host check of the attention block-shape choice (sdpa_plan.cpp): every
// plan is a valid configuration whose grid fits, overrides are honoured or
// ignored as documented, and the estimate prefers more blocks when the
// query range alone cannot fill the chip.
#include <stdio.h>

#include <initializer_list>

#include "sdpa_plan.hpp"

using namespace baim;

int main() {
  int bad = 0;
  const long sizes[] = {1, 2, 31, 32, 33, 64, 65, 127, 128, 129, 197, 577, 1024, 4096, 100000};
  for (long BH : {1L, 3L, 12L, 96L, 384L, 4096L})
    for (long Sq : sizes)
      for (long Skv : sizes)
        for (long D : {4L, 32L, 64L, 65L, 128L})
          for (const char* s : {(const char*)nullptr, "", "0", "1", "2", "3", "x", "01", "-1"}) {
            const int c = plan_sdpa(BH, Sq, Skv, D, s);
            if (c < 0 || c >= SDPA_NCFG) bad += printf("bad cfg %d\n", c) > 0;
            if (sdpa_nb(c, D) < 1 || sdpa_nb(c, D) > 2) bad += printf("bad key blocks\n") > 0;
            if (kSdpaQW[c] * kSdpaKW[c] != (c == SDPA_K8 ? 8 : 4)) bad += printf("wave count\n") > 0;
            if (c == SDPA_K8 && D > kSdpaK8MaxD) bad += printf("eight waves above D %d\n", kSdpaK8MaxD) > 0;
            if (c == SDPA_K8 && !(s && s[0] == '3' && !s[1]) && BH * ((Sq + 31) / 32) > 256)
              bad += printf("eight waves over several rounds\n") > 0;
            const long bq = 32 * kSdpaQW[c];
            if (BH * ((Sq + bq - 1) / bq) >= (1L << 31)) bad += printf("grid too large\n") > 0;
          }
  for (int c = 0; c < SDPA_NCFG; ++c) {
    const char spec[2] = {(char)('0' + c), 0};
    if (plan_sdpa(384, 197, 197, 64, spec) != c) bad += printf("override %d ignored\n", c) > 0;
  }
  if (plan_sdpa(96, 64, 577, 64, "7") != plan_sdpa(96, 64, 577, 64, nullptr))
    bad += printf("bad override not ignored\n") > 0;
  // the eight-wave shape is not compiled above D 64: its override falls back
  if (plan_sdpa(8, 1024, 4096, 128, "3") != plan_sdpa(8, 1024, 4096, 128, nullptr) ||
      plan_sdpa(8, 1024, 4096, 128, nullptr) == SDPA_K8)
    bad += printf("eight waves at D 128\n") > 0;
  // few (batch, head) slices with few queries: split the keys four ways,
  // or eight ways (two waves per SIMD) over a long key range
  if (plan_sdpa(8, 1024, 4096, 64, nullptr) != SDPA_K8) bad += printf("pooled\n") > 0;
  if (plan_sdpa(16, 256, 2048, 64, nullptr) != SDPA_K8) bad += printf("long keys\n") > 0;
  if (plan_sdpa(96, 64, 577, 64, nullptr) != SDPA_K4) bad += printf("cross-attention\n") > 0;
  // enough query blocks to fill the chip: 128-row blocks
  if (plan_sdpa(64, 1024, 1024, 128, nullptr) != SDPA_Q4) bad += printf("long self-attention\n") > 0;
  // 197-token self-attention, head dim 64: the 128-row shape with one key block
  if (plan_sdpa(384, 197, 197, 64, nullptr) != SDPA_Q4 || sdpa_nb(SDPA_Q4, 64) != 1)
    bad += printf("vit\n") > 0;
  if (bad) return 1;
  printf("OK\n");
  return 0;
}
