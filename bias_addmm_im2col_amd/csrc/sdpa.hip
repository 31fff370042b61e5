// sdpa.hip -- non-causal scaled-dot-product attention, fp32, on the gfx950
// matrix cores.
//
// "[ExecuTorch][WebGPU] Add optimized SDPA op" (pytorch/executorch PR
// #20851), Problem and Solution paragraphs: over row-major [B,H,S,D]
// tensors, out = softmax(q @ k^T * scale + attn_mask) @ v, with an optional
// additive [B,H,Sq,Skv] mask, Sq and Skv free to differ, and scale 1/sqrt(D)
// when not given.  The page chains three dispatches through two
// B*H*Sq*Skv scratch buffers (scores, then softmax).  Here one kernel
// streams 64-key tiles of k and v through LDS and keeps a running softmax
// per query row (maximum and sum rescaled as the maximum grows), so the
// scores stay in registers and nothing is allocated.
//
// Work split: a block of four (or eight) waves owns 32*QW query rows of one
// (batch, head): QW query groups of 32 rows times KW key groups (QW*KW = 4,
// or 1 x 8).  The block stages tiles of 32*NB*KW keys; in each, key group g
// takes the NB 32-key blocks g*NB .. g*NB+NB-1, and keeps its own running
// softmax, so a short query range still keeps every wave busy.  At the end
// the key groups' (maximum, sum, O) are merged through LDS in group order.
// The eight-wave shape puts two waves on each SIMD of a block; to fit their
// registers it reads Q from LDS instead of holding it.  Per 32-key block a
// wave computes
//   S^T[kv, q] = K[kv, :] . Q[q, :]        (a 32x32 block, k = d)
// on v_mfma_f32_32x32x2_f32 with K as the A operand (16-byte LDS reads) and
// Q as the B operand (kept in registers for the whole pass), then
//   O[q, d] += P[q, kv] V[kv, d]           (DP/32 blocks, k = kv)
// with P as the A operand.  In the MFMA lane layout (lane l, c = l % 32,
// h = l / 32) accumulator register j of S^T holds key 8*(j/4) + 4*h + j%4
// of query c, and the A operand of step s is row c, k-index h; visiting the
// keys of a 32-key block in the order 8*(s/4) + 4*h + s%4 makes step s of
// the second product take register s of the first as its A value: the
// probabilities never move between lanes.  Each query's row statistics
// (maximum, sum) live in lanes c and c+32; the per-row rescale factors the
// O rows need are passed through a 32-float LDS slot per wave.
//
// Ragged edges: q rows past Sq load as 0 and are not stored; keys past Skv
// get the logit -inf (weight 0) and their k/v rows load as 0; d past D (D
// is padded to DP, a multiple of 32) loads as 0 and is not stored.  A row
// whose logits are all -inf ends with sum 0 and gives 0 * (1/0) = NaN, the
// value of the plain definition.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>

#include <type_traits>

#include "gemm_core.hpp"
#include "index_math.hpp"
#include "launch.hpp"
#include "sdpa_plan.hpp"

namespace baim {

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

struct SdpaArgs {
  const float* q;
  const float* k;
  const float* v;
  const float* mask;
  float* out;
  int Sq, Skv, D;
  int qblocks, nblocks;
  float scale2;  // scale * log2(e): the logits are kept in base 2
};

template <int DP, int QW, int KW, int NB>
struct SdpaShape {
  static constexpr int NT = 64 * QW * KW;
  static constexpr int BQ = 32 * QW;        // query rows per block
  static constexpr int BKV = 32 * NB * KW;  // keys per tile
  static constexpr int KS = DP + 4;         // LDS row stride (floats) of the k and v tiles
  static constexpr int CH = DP / 4;         // 16-byte chunks per row
  static constexpr int NCH = BKV * CH / NT; // chunks per thread and tile
  static constexpr int ND = DP / 32;        // 32-wide d blocks of O
  static constexpr int NQ = DP / 8;         // Q chunks per lane
  static constexpr int TILE_FLOATS = 2 * BKV * KS;
  // merge of the key groups: partial O of groups 1..KW-1, then (max, sum)
  // of every group, both over the (dead) tile area
  static constexpr int RED_FLOATS = (KW - 1) * QW * 32 * DP;
  static constexpr int STAT_FLOATS = 2 * KW * BQ;
  static constexpr int MERGE_FLOATS = RED_FLOATS + STAT_FLOATS;
  static constexpr int SLOT_OFS = TILE_FLOATS > MERGE_FLOATS ? TILE_FLOATS : MERGE_FLOATS;
  // eight-wave blocks keep the block's Q rows in LDS (stride KS)
  static constexpr bool QLDS = QW * KW == 8;
  static constexpr int Q_OFS = SLOT_OFS + 32 * QW * KW;
  static constexpr int LDS_FLOATS = Q_OFS + (QLDS ? BQ * KS : 0);
  // their merge: every wave's partial O, the groups' (maximum, sum) and the
  // rows' 1/sum, over the tile area
  static constexpr int RED8_FLOATS = KW * QW * 32 * DP + 2 * KW * BQ + BQ;
  static_assert(DP % 32 == 0 && DP <= 128, "D is padded to 32, 64, 96 or 128");
  static_assert(QW * KW == 4 || (QW == 1 && KW == 8 && DP <= 64), "four waves, or 1 x 8 for D <= 64");
  static_assert(!QLDS || (RED8_FLOATS <= TILE_FLOATS && (ND * 16) % KW == 0), "eight-wave merge");
  static_assert((BKV * CH) % NT == 0, "tile splits evenly");
};

// Multiply row r = 8*(j/4) + 4*h + j%4 of a wave's 32x32 O blocks by f[r],
// where f[q] is held by lanes q and q + 32.
template <int ND>
__device__ __forceinline__ void scale_rows(f32x16 (&o)[ND], float f, float* slot, int c, int h) {
  if (h == 0) slot[c] = f;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  f32x4 r[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) r[g] = *reinterpret_cast<const f32x4*>(slot + 8 * g + 4 * h);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] *= r[j / 4][j % 4];
}

// The mask tile of a key tile, for the shapes with several key groups (a
// wave's lanes then read 32 different mask rows at a few keys each, which
// as direct loads touch a cache line per lane): the block's BQ query rows x
// BKV keys, loaded along the keys (coalesced: MV floats per load, 16 bytes
// where the rows allow) one tile ahead like k and v, and staged in LDS with
// row stride BKV + 4 (an odd multiple of 4 floats mod 32), from where each
// lane reads its four keys per 16-byte read.  The 128-row shape keeps
// direct loads: its registers are spent on three blocks per CU.
template <int BQ, int BKV, int NT, int MV>
struct SdpaMaskTile {
  static constexpr int MS = BKV + 4;
  static constexpr int ITEMS = BQ * BKV / MV;
  static constexpr int NQ = (ITEMS + NT - 1) / NT;  // loads per thread and tile
  static constexpr int FLOATS = BQ * MS;
  static_assert(BKV % 32 == 0 && MS % 8 == 4, "mask tile rows");
};

template <int DP, int QW, int KW, int NB, bool MASK, int MV>
__global__ __launch_bounds__(64 * QW * KW, QW * KW == 8 ? 1 : DP <= 64 ? (QW == 4 && NB == 1 ? 3 : 2) : 1)
void sdpa_kernel(SdpaArgs a) {
  using S = SdpaShape<DP, QW, KW, NB>;
  using MT = SdpaMaskTile<S::BQ, S::BKV, S::NT, MV>;
  // mask tile staged through LDS (the eight-wave shape's tiles leave no room)
  constexpr bool MSTAGE = MASK && KW > 1 && !S::QLDS;
  __shared__ __attribute__((aligned(16))) float smem[S::LDS_FLOATS + (MSTAGE ? MT::FLOATS : 0)];
  float* Ks = smem;
  float* Vs = smem + S::BKV * S::KS;
  float* Ms = smem + S::LDS_FLOATS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = wave % QW, kg = wave / QW;  // query group, key group
  float* slot = smem + S::SLOT_OFS + 32 * wave;
  const int c = lane & 31, h = lane >> 5;

  const int lid = xcd_linear(blockIdx.x, a.nblocks);
  const int bh = lid / a.qblocks, qb = lid - bh * a.qblocks;
  const int Sq = a.Sq, Skv = a.Skv, D = a.D;
  const int qrow0 = qb * S::BQ + qg * 32;  // first query row of this wave
  const int q = qrow0 + c;                 // this lane's query (column of S^T)
  const bool active = qrow0 < Sq;          // wave-uniform
  const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + (size_t)bh * Sq * D, (int64_t)Sq * D);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.k + (size_t)bh * Skv * D, (int64_t)Skv * D);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.v + (size_t)bh * Skv * D, (int64_t)Skv * D);
  __amdgpu_buffer_rsrc_t mr;
  if constexpr (MASK) mr = make_rsrc(a.mask + (size_t)bh * Sq * Skv, (int64_t)Sq * Skv);

  // Q fragments: chunk t holds Q[q][8t + 4h .. 8t + 4h + 3], in registers,
  // or (eight waves) read from the block's Q rows in LDS, which the first
  // tile's barrier publishes.
  f32x4 qf[S::QLDS ? 1 : S::NQ];
  float* Qs = smem + S::Q_OFS;
  if constexpr (S::QLDS) {
#pragma unroll
    for (int i = 0; i < (S::BQ * S::CH + S::NT - 1) / S::NT; ++i) {
      const int idx = i * S::NT + tid;
      const int row = idx / S::CH, d = 4 * (idx - row * S::CH);
      const int qq = qb * S::BQ + row;
      const bool in = (S::BQ * S::CH) % S::NT == 0 || row < S::BQ;
      const uint32_t off = (in && qq < Sq && d < D) ? (uint32_t)(qq * D + d) * 4u : kOOB;
      const f32x4 v4 = Vec<4>::load(qr, off);
      if (in) *reinterpret_cast<f32x4*>(Qs + row * S::KS + d) = v4;
    }
  } else {
#pragma unroll
    for (int t = 0; t < S::NQ; ++t) {
      const int d = 8 * t + 4 * h;
      const uint32_t off = (q < Sq && d < D) ? (uint32_t)(q * D + d) * 4u : kOOB;
      qf[t] = Vec<4>::load(qr, off);
    }
  }

  // k/v tile loads: chunk i of thread tid is row idx / CH, column 4*(idx % CH).
  // Mask tile loads: item i of thread tid is query row idx / (BKV/MV) of the
  // block, keys MV*(idx % (BKV/MV)) .. +MV-1 of the tile.
  f32x4 kreg[S::NCH], vreg[S::NCH];
  typename Vec<MV>::T mreg[MSTAGE ? MT::NQ : 1];
  auto fetch = [&](int kv0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::NCH; ++i) {
      const int idx = i * S::NT + tid;
      const int row = idx / S::CH, d = 4 * (idx - row * S::CH);
      const int kv = kv0 + row;
      const uint32_t off = (kv < Skv && d < D) ? (uint32_t)(kv * D + d) * 4u : kOOB;
      kreg[i] = Vec<4>::load(kr, off);
      vreg[i] = Vec<4>::load(vr, off);
    }
    if constexpr (MSTAGE) {
#pragma unroll
      for (int i = 0; i < MT::NQ; ++i) {
        const int idx = i * S::NT + tid;
        const int row = idx / (S::BKV / MV), col = MV * (idx - row * (S::BKV / MV));
        const int qq = qb * S::BQ + row, kv = kv0 + col;
        // keys past Skv get -inf later; with MV == 4, Skv % 4 == 0 keeps a
        // whole group inside the row
        const bool ok = idx < MT::ITEMS && qq < Sq && kv < Skv;
        mreg[i] = Vec<MV>::load(mr, ok ? (uint32_t)(qq * Skv + kv) * 4u : kOOB);
      }
    }
  };
  auto put = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::NCH; ++i) {
      const int idx = i * S::NT + tid;
      const int row = idx / S::CH, d = 4 * (idx - row * S::CH);
      *reinterpret_cast<f32x4*>(Ks + row * S::KS + d) = kreg[i];
      *reinterpret_cast<f32x4*>(Vs + row * S::KS + d) = vreg[i];
    }
    if constexpr (MSTAGE) {
#pragma unroll
      for (int i = 0; i < MT::NQ; ++i) {
        const int idx = i * S::NT + tid;
        if (MT::ITEMS % S::NT != 0 && idx >= MT::ITEMS) continue;
        const int row = idx / (S::BKV / MV), col = MV * (idx - row * (S::BKV / MV));
        *reinterpret_cast<typename Vec<MV>::T*>(Ms + row * MT::MS + col) = mreg[i];
      }
    }
  };

  f32x16 o[S::ND];
#pragma unroll
  for (int db = 0; db < S::ND; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.0f;
  float m_run = -INFINITY, l_lane = 0.0f;
  const int ntiles = (Skv + S::BKV - 1) / S::BKV;

  fetch(0);
  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * S::BKV;
    if (t > 0) __syncthreads();  // every wave is done with the previous tile
    put();
    __syncthreads();
    if (t + 1 < ntiles) fetch(kv0 + S::BKV);

    // This wave's key blocks: keys kb0 + 32*kb + (0..31) of the tile, in
    // the order 8*(j/4) + 4*h + j%4 (register j of S^T).
    const int kb0 = 32 * NB * kg;
    bool blk[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) blk[kb] = active && kv0 + kb0 + 32 * kb < Skv;

    f32x4 mk[NB][4];
    if constexpr (MSTAGE) {
      const float* mrow = Ms + (32 * qg + c) * MT::MS + kb0 + 4 * h;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          mk[kb][g] = *reinterpret_cast<const f32x4*>(mrow + 32 * kb + 8 * g);
    } else if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int kv = kv0 + kb0 + 32 * kb + 8 * g + 4 * h;
          const bool row_ok = blk[kb] && q < Sq;
          if constexpr (MV == 4) {
            const uint32_t off = (row_ok && kv < Skv) ? (uint32_t)(q * Skv + kv) * 4u : kOOB;
            mk[kb][g] = Vec<4>::load(mr, off);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t off =
                  (row_ok && kv + r < Skv) ? (uint32_t)(q * Skv + kv + r) * 4u : kOOB;
              mk[kb][g][r] = Vec<1>::load(mr, off);
            }
          }
        }
    }

    // S^T = K Q^T per key block.
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) s[kb][j] = 0.0f;
      if (blk[kb]) {
        const float* krow = Ks + (kb0 + 32 * kb + c) * S::KS + 4 * h;
        const float* qrow = Qs + (32 * qg + c) * S::KS + 4 * h;
#pragma unroll
        for (int t2 = 0; t2 < S::NQ; ++t2) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(krow + 8 * t2);
          f32x4 b4;
          if constexpr (S::QLDS)
            b4 = *reinterpret_cast<const f32x4*>(qrow + 8 * t2);
          else
            b4 = qf[S::QLDS ? 0 : t2];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[r], b4[r], s[kb], 0, 0, 0);
        }
      }
    }

    // Logits in base 2 (scale2 = scale * log2(e), the mask times log2(e)),
    // running maximum and sum.  Keys past Skv only occur in the last tile;
    // only there does each logit need the -inf test.
    float mt = -INFINITY;
    auto logits = [&](auto tail_tag) __attribute__((always_inline)) {
      constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float x;
          if constexpr (MASK)
            x = fmaf(mk[kb][j / 4][j % 4], kLog2e, s[kb][j] * a.scale2);
          else
            x = s[kb][j] * a.scale2;
          if constexpr (TAIL) {
            const int kv = kv0 + kb0 + 32 * kb + 8 * (j / 4) + 4 * h + (j % 4);
            x = (blk[kb] && kv < Skv) ? x : -INFINITY;
          }
          s[kb][j] = x;
          mt = fmaxf(mt, x);
        }
    };
    if (kv0 + S::BKV > Skv)
      logits(std::true_type{});
    else
      logits(std::false_type{});
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    float ps = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(s[kb][j] - m_use);
        s[kb][j] = p;
        ps += p;
      }
    // Rescale only when some row's maximum moved (rare after the first
    // tiles); otherwise the factor is exactly 1.
    if (__any(m_new != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_lane *= alpha;
      scale_rows(o, alpha, slot, c, h);
    }
    l_lane += ps;
    m_run = m_new;

    // O += P V: step st of key block kb takes key kb0 + 32*kb + 8*(st/4) + 4*h + st%4.
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
      if (blk[kb]) {
#pragma unroll
        for (int db = 0; db < S::ND; ++db)
#pragma unroll
          for (int st = 0; st < 16; ++st) {
            const int kv = kb0 + 32 * kb + 8 * (st / 4) + 4 * h + (st % 4);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(s[kb][st], Vs[kv * S::KS + 32 * db + c],
                                                         o[db], 0, 0, 0);
          }
      }
  }

  float inv;
  if constexpr (S::QLDS) {
    // Eight key groups: every wave stores its partial O scaled by
    // e^(m_g - M), then each wave sums one slice of the O registers over the
    // groups in group order (the same sums as one wave adding the others to
    // its own) and writes it.
    float* red = smem;
    float* stat_m = red + KW * QW * 32 * DP;
    float* stat_l = stat_m + KW * S::BQ;
    float* inv_row = stat_l + KW * S::BQ;
    const float l_w = l_lane + __shfl_xor(l_lane, 32);
    __syncthreads();  // the tile area is reused below
    if (h == 0) {
      stat_m[kg * S::BQ + 32 * qg + c] = m_run;
      stat_l[kg * S::BQ + 32 * qg + c] = l_w;
    }
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < KW; ++g) mx = fmaxf(mx, stat_m[g * S::BQ + 32 * qg + c]);
    const float m_use = mx == -INFINITY ? 0.0f : mx;
    scale_rows(o, __builtin_amdgcn_exp2f(m_run - m_use), slot, c, h);
    float* mine = red + (kg * QW + qg) * 32 * DP;
#pragma unroll
    for (int db = 0; db < S::ND; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) mine[(db * 16 + j) * 64 + lane] = o[db][j];
    if (kg == 0 && h == 0) {
      float L = 0.0f;
#pragma unroll
      for (int g = 0; g < KW; ++g)
        L += stat_l[g * S::BQ + 32 * qg + c] *
             __builtin_amdgcn_exp2f(stat_m[g * S::BQ + 32 * qg + c] - m_use);
      inv_row[32 * qg + c] = 1.0f / L;
    }
    __syncthreads();
    constexpr int SL = S::ND * 16 / KW;  // O registers per wave's slice
    float* out = a.out + (size_t)bh * Sq * D;
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      const int r = kg * SL + i, db = r / 16, j = r % 16;
      float acc = red[(0 * QW + qg) * 32 * DP + r * 64 + lane];
#pragma unroll
      for (int g = 1; g < KW; ++g) acc += red[(g * QW + qg) * 32 * DP + r * 64 + lane];
      const int rr = 8 * (j / 4) + 4 * h + (j % 4);  // row within the query group
      const int row = qrow0 + rr, d = 32 * db + c;
      if (row < Sq && d < D) out[(size_t)row * D + d] = acc * inv_row[32 * qg + rr];
    }
    return;
  } else if constexpr (KW == 1) {
    inv = 1.0f / (l_lane + __shfl_xor(l_lane, 32));
  } else {
    // Merge the key groups of each query row: with M the largest group
    // maximum, O = sum_g O_g e^(m_g - M) / sum_g l_g e^(m_g - M), summed in
    // group order.
    float* red = smem;
    float* stat_m = smem + S::RED_FLOATS;
    float* stat_l = stat_m + KW * S::BQ;
    const float l_w = l_lane + __shfl_xor(l_lane, 32);
    __syncthreads();  // the tile area is reused below
    if (h == 0) {
      stat_m[kg * S::BQ + 32 * qg + c] = m_run;
      stat_l[kg * S::BQ + 32 * qg + c] = l_w;
    }
    __syncthreads();
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < KW; ++g) mx = fmaxf(mx, stat_m[g * S::BQ + 32 * qg + c]);
    const float m_use = mx == -INFINITY ? 0.0f : mx;
    float L = 0.0f;
#pragma unroll
    for (int g = 0; g < KW; ++g)
      L += stat_l[g * S::BQ + 32 * qg + c] *
           __builtin_amdgcn_exp2f(stat_m[g * S::BQ + 32 * qg + c] - m_use);
    scale_rows(o, __builtin_amdgcn_exp2f(m_run - m_use), slot, c, h);
    if (kg > 0) {
      float* mine = red + ((kg - 1) * QW + qg) * 32 * DP;
#pragma unroll
      for (int db = 0; db < S::ND; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) mine[(db * 16 + j) * 64 + lane] = o[db][j];
    }
    __syncthreads();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KW; ++g) {
      const float* other = red + ((g - 1) * QW + qg) * 32 * DP;
#pragma unroll
      for (int db = 0; db < S::ND; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] += other[(db * 16 + j) * 64 + lane];
    }
    inv = 1.0f / L;
  }
  scale_rows(o, inv, slot, c, h);
  float* out = a.out + (size_t)bh * Sq * D;
  if (qrow0 + 32 <= Sq && D == DP) {
    // a whole block of 32 rows and every d: no test per element (the
    // masked 64 x 577 cross-attention 25.1 -> 24.4 us), non-temporal (the
    // output is not read back; 197-token ViT 53.6 -> 52.4 us)
#pragma unroll
    for (int db = 0; db < S::ND; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        __builtin_nontemporal_store(o[db][j], &out[(size_t)(qrow0 + 8 * (j / 4) + 4 * h + (j % 4)) * DP + 32 * db + c]);
    return;
  }
#pragma unroll
  for (int db = 0; db < S::ND; ++db) {
    const int d = 32 * db + c;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int row = qrow0 + 8 * (j / 4) + 4 * h + (j % 4);
      if (row < Sq && d < D) out[(size_t)row * D + d] = o[db][j];
    }
  }
}

template <int DP, int QW, int KW, int NB>
hipError_t launch_cfg(SdpaArgs a, bool mask_vec, hipStream_t s) {
  using S = SdpaShape<DP, QW, KW, NB>;
  a.qblocks = (a.Sq + S::BQ - 1) / S::BQ;
  a.nblocks = (int)((int64_t)(a.nblocks) * a.qblocks);  // nblocks carries BH in
  const dim3 grid(a.nblocks), block(S::NT);
  if (!a.mask)
    hipLaunchKernelGGL((sdpa_kernel<DP, QW, KW, NB, false, 4>), grid, block, 0, s, a);
  else if (mask_vec)
    hipLaunchKernelGGL((sdpa_kernel<DP, QW, KW, NB, true, 4>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((sdpa_kernel<DP, QW, KW, NB, true, 1>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int DP>
hipError_t launch_dp(const SdpaArgs& a, int cfg, bool mask_vec, hipStream_t s) {
  constexpr int NBQ4 = sdpa_nb(SDPA_Q4, DP);
  static_assert(kSdpaQW[SDPA_Q4] == 4 && kSdpaKW[SDPA_Q4] == 1, "");
  static_assert(kSdpaQW[SDPA_Q2K2] == 2 && kSdpaKW[SDPA_Q2K2] == 2 && sdpa_nb(SDPA_Q2K2, DP) == 1, "");
  static_assert(kSdpaQW[SDPA_K4] == 1 && kSdpaKW[SDPA_K4] == 4 && sdpa_nb(SDPA_K4, DP) == 1, "");
  static_assert(kSdpaQW[SDPA_K8] == 1 && kSdpaKW[SDPA_K8] == 8 && sdpa_nb(SDPA_K8, DP) == 1, "");
  switch (cfg) {
    case SDPA_Q2K2: return launch_cfg<DP, 2, 2, 1>(a, mask_vec, s);
    case SDPA_K4: return launch_cfg<DP, 1, 4, 1>(a, mask_vec, s);
    case SDPA_K8:
      if constexpr (DP <= kSdpaK8MaxD) return launch_cfg<DP, 1, 8, 1>(a, mask_vec, s);
      else return hipErrorInvalidValue;  // the planner never picks it above
    default: return launch_cfg<DP, 4, 1, NBQ4>(a, mask_vec, s);
  }
}

}  // namespace

hipError_t launch_sdpa(const SdpaProblem& p, hipStream_t stream) {
  SdpaArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.mask = p.mask;
  a.out = p.out;
  a.Sq = p.Sq;
  a.Skv = p.Skv;
  a.D = p.D;
  a.scale2 = p.scale * kLog2e;
  a.qblocks = 0;
  a.nblocks = p.BH;
  const int cfg = plan_sdpa(p.BH, p.Sq, p.Skv, p.D, getenv("BAIM_SDPA"));
  // 16-byte mask loads need rows that start on 16-byte boundaries.
  const bool mask_vec = p.mask && p.Skv % 4 == 0 && ((uintptr_t)p.mask & 15) == 0;
  if (p.D <= 32) return launch_dp<32>(a, cfg, mask_vec, stream);
  if (p.D <= 64) return launch_dp<64>(a, cfg, mask_vec, stream);
  if (p.D <= 96) return launch_dp<96>(a, cfg, mask_vec, stream);
  return launch_dp<128>(a, cfg, mask_vec, stream);
}

}  // namespace baim
