// sdpa_plan.cpp -- see sdpa_plan.hpp.
#include "sdpa_plan.hpp"

namespace baim {

namespace {
constexpr int kCUs = 256;  // MI355X
}  // namespace

int plan_sdpa(int64_t BH, int64_t Sq, int64_t Skv, int64_t D, const char* override_spec) {
  if (override_spec && override_spec[0] >= '0' && override_spec[0] < '0' + SDPA_NCFG &&
      override_spec[1] == 0 && (override_spec[0] - '0' != SDPA_K8 || D <= kSdpaK8MaxD))
    return override_spec[0] - '0';
  int best = SDPA_Q4;
  double best_t = 0.0;
  for (int cfg = 0; cfg < SDPA_NCFG; ++cfg) {
    // An eight-wave block takes most of a CU's LDS, so it runs one block per
    // CU: it pays only where the 32-row blocks fit one round anyway and each
    // CU's single block is short of waves.
    if (cfg == SDPA_K8 && (D > kSdpaK8MaxD || BH * ((Sq + 31) / 32) > kCUs)) continue;
    const int nb = sdpa_nb(cfg, D);
    const int64_t bq = 32 * kSdpaQW[cfg], bkv = 32 * nb * kSdpaKW[cfg];
    const int64_t blocks = BH * ((Sq + bq - 1) / bq);
    const int64_t tiles = (Skv + bkv - 1) / bkv;
    const int64_t rounds = (blocks + kCUs - 1) / kCUs;
    const int per_simd = kSdpaQW[cfg] * kSdpaKW[cfg] / 4;  // waves per SIMD
    const double t = (double)rounds * (double)tiles * (per_simd * nb + 0.3);
    if (cfg == 0 || t < best_t) {
      best = cfg;
      best_t = t;
    }
  }
  return best;
}

}  // namespace baim
