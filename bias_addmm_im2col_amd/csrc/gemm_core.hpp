// gemm_core.hpp -- device side of the fp32 tiled GEMM for gfx950 (CDNA4).
//
// The method ("[ExecuTorch][WebGPU] Add optimized addmm op", Solution
// paragraph) stages tiles of both operands in on-chip shared memory, syncs
// the workgroup, and accumulates over ceil(K/BK) k-tiles so that each
// coalesced tile load is reused by the whole output tile.  On gfx950 that
// becomes:
//   * a BM x BN block tile computed by WM x WN wavefronts (64 lanes each);
//     every wave owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 blocks;
//   * the contraction runs on the fp32 matrix cores,
//     v_mfma_f32_32x32x2_f32 (A 32x2, B 2x32, C 32x32, fp32 accumulate);
//   * both operand tiles are double-buffered in LDS; the next k-tile is
//     fetched from HBM into registers while the current one feeds the
//     matrix cores, then written to the other LDS buffer: one barrier per
//     k-tile;
//   * global reads are raw buffer loads: an offset past the buffer's range
//     returns 0, which gives the ragged M/N/K edges and the conv's zero
//     padding without branches.
//
// Lane layout of v_mfma_f32_32x32x2_f32 (lane l, c = l % 32, h = l / 32):
//   A operand: A[row c][k h];  B operand: B[k h][col c];
//   accumulator register j: C[row 8*(j/4) + 4*h + (j%4)][col c].
//
// K order: any fp32 summation order is acceptable, so inside a k-tile the
// MFMA step s (0 <= s < BK/2) of lane-half h uses k = 8*(s/4) + 4*h + s%4.
// Each lane then finds its A values for four consecutive steps in four
// consecutive LDS floats (one 16-byte read), and the two lane-halves read B
// rows four apart, which land in disjoint LDS banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "index_math.hpp"
#include "tile_select.hpp"

namespace baim {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource for gfx9-family: stride 0, 32-bit data format bits.
constexpr int kBufferFlags = 0x00020000;
// Offset used for a masked element: it is past the range of every
// resource built here (all ranges are below 2^31 bytes), so the load
// returns 0 without touching memory.
constexpr uint32_t kOOB = 0x80000000u;

// Resource over the `elems` floats starting at p (clamped to 2^31 - 1
// bytes).  The range is exact, so even a wrong offset cannot read past the
// tensor: the hardware returns 0 instead.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const float* p, int64_t elems) {
  const int64_t bytes = elems * 4 < 0x7FFFFFFF ? elems * 4 : 0x7FFFFFFF;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, (int)bytes, kBufferFlags);
}

template <int VEC> struct Vec;
template <> struct Vec<1> {
  typedef float T;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
};
template <> struct Vec<4> {
  typedef f32x4 T;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
};

// Block tile BM x BN x BK computed by WM x WN x WK waves: WM x WN waves
// split the output tile, and WK groups of them split each k-tile (group g
// takes k in [g*BK/WK, (g+1)*BK/WK)); the groups' partial tiles are summed
// through LDS at the end, in group order.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int WK_ = 1, int PF_ = 1>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, WK = WK_;
  static constexpr int PF = PF_;  // global->register prefetch depth in k-tiles (1 or 2)
  static constexpr int NT = 64 * WM * WN * WK;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int BKW = BK / WK;  // k per wave group and k-tile
  // LDS row strides (floats).  A is [BM][BK+4]: 16-byte reads of 32
  // consecutive rows spread over all banks.  B is [BK][BN+8]: rows four
  // apart start 32 banks apart.
  static constexpr int AS = BK + 4, BS = BN + 8;
  // A loader may instead keep B transposed, [BN][BK+4] like A, so that the
  // MFMA B fragments are 16-byte reads too.
  static constexpr int BTS = BK + 4;
  static constexpr int A_FLOATS = BM * AS;
  static constexpr int B_FLOATS = BK * BS > BN * BTS ? BK * BS : BN * BTS;
  static constexpr int STAGE = A_FLOATS + B_FLOATS;
  // Per-k-tile loader metadata (four slots of BK int4 entries) after the
  // two operand stages.
  static constexpr int META_SLOTS = 4;
  static constexpr int META_INTS = META_SLOTS * BK * 4;
  static constexpr int SMEM_FLOATS = 2 * STAGE + META_INTS;
  static_assert(BKW % 8 == 0, "each wave group needs a multiple of 8 k per tile");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32x32 blocks");
  static_assert(BN % 16 == 0, "B padding assumes BN % 16 == 0");
  static_assert(NT <= 1024, "at most 1024 threads per block");
  static_assert(PF == 1 || PF == 2, "prefetch depth 1 or 2");
  static_assert((WK - 1) * BM * BN <= 2 * STAGE, "k-group reduction must fit in the stages");
};

// Where a wave works: its output sub-tile origin and its k offset.
struct WaveSlot {
  int wm0, wn0, kofs, kgroup;
};

template <class T>
__device__ inline WaveSlot wave_slot() {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave / (T::WM * T::WN), wmn = wave % (T::WM * T::WN);
  return WaveSlot{(wmn / T::WN) * T::WTM, (wmn % T::WN) * T::WTN, kg * T::BKW, kg};
}

// ---------------------------------------------------------------- loaders

// ROWS x BK tile of a row-major matrix whose contiguous dim is K, stored in
// LDS as [ROWS][BK+4].  As the A operand: rows m of mat1 [M,K] or of the
// conv weight viewed as [OC, IC*KH*KW].  As the B operand (AS_B): rows n
// of a [N,K] weight, which is B already transposed.
template <class T, int VEC, int ROWS, bool AS_B>
struct KRowLoader {
  static constexpr bool kHasMeta = false;
  static constexpr bool kBTransposed = AS_B;
  static constexpr int CPR = T::BK / VEC;
  static constexpr int NCH = ROWS * CPR / T::NT;
  static_assert((ROWS * CPR) % T::NT == 0, "tile must split evenly over threads");
  static_assert(T::AS == T::BTS, "A and transposed-B rows share one stride");
  typedef typename Vec<VEC>::T V;
  const float* base;  // first row of the block
  int K, rows_left;
  V reg[2][NCH];  // two register slots (prefetch depth up to 2)

  __device__ void init(const float* A, int r0, int R, int K_) {
    base = A + (size_t)r0 * K_;
    K = K_;
    rows_left = R - r0;
  }
  template <int S>
  __device__ void load(int k0) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0, (int64_t)rows_left * K - k0);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + T::NT * i;
      const int r = q / CPR, c = (q % CPR) * VEC;
      const bool ok = r < rows_left && k0 + c < K;
      reg[S][i] = Vec<VEC>::load(rs, ok ? (uint32_t)(r * K + c) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* dst) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + T::NT * i;
      const int r = q / CPR, c = (q % CPR) * VEC;
      *reinterpret_cast<V*>(&dst[r * T::AS + c]) = reg[S][i];
    }
  }
  __device__ void meta(int) {}
};

template <class T, int VEC>
using RowTileLoader = KRowLoader<T, VEC, T::BM, false>;

// B tile from a row-major [K][N] matrix (mat2, read as mat2[k*N + n]).
template <class T, int VEC>
struct ColTileLoader {
  static constexpr bool kHasMeta = false;
  static constexpr bool kBTransposed = false;
  static constexpr int CPR = T::BN / VEC;
  static constexpr int NCH = T::BK * CPR / T::NT;
  static_assert((T::BK * CPR) % T::NT == 0, "B tile must split evenly over threads");
  typedef typename Vec<VEC>::T V;
  const float* base;  // column n0 of row 0
  int N, K, cols_left;
  V reg[2][NCH];

  __device__ void init(const float* B, int n0, int N_, int K_) {
    base = B + n0;
    N = N_;
    K = K_;
    cols_left = N_ - n0;
  }
  template <int S>
  __device__ void load(int k0) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + (size_t)k0 * N, (int64_t)(K - k0) * N - (N - cols_left));
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + T::NT * i;
      const int r = q / CPR, c = (q % CPR) * VEC;
      const bool ok = k0 + r < K && c < cols_left;
      reg[S][i] = Vec<VEC>::load(rs, ok ? (uint32_t)(r * N + c) * 4u : kOOB);
    }
  }
  template <int S>
  __device__ void store(float* Bs) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = threadIdx.x + T::NT * i;
      const int r = q / CPR, c = (q % CPR) * VEC;
      *reinterpret_cast<V*>(&Bs[r * T::BS + c]) = reg[S][i];
    }
  }
  __device__ void meta(int) {}
};

// ----------------------------------------------------------- contraction

template <class T>
struct Accum {
  f32x16 c[T::FM][T::FN];
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[i][j][r] = 0.0f;
  }
};

// One k-tile: for the wave's k range [kofs, kofs + BKW), BKW/2 MFMA steps
// for every 32x32 block of the wave's sub-tile.  B is read from [BK][BN+8]
// (four 4-byte reads per lane and 4 steps) or, with BT, from the transposed
// [BN][BK+4] (one 16-byte read).
template <class T, bool BT>
__device__ __forceinline__ void mma_tile(Accum<T>& acc, const float* As, const float* Bs,
                                         const WaveSlot& ws, int lane) {
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int g = 0; g < T::BKW / 8; ++g) {
    const int k = ws.kofs + 8 * g + 4 * h;
    f32x4 a[T::FM];
    f32x4 b[T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
      a[i] = *reinterpret_cast<const f32x4*>(&As[(ws.wm0 + 32 * i + c) * T::AS + k]);
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      if (BT) {
        b[j] = *reinterpret_cast<const f32x4*>(&Bs[(ws.wn0 + 32 * j + c) * T::BTS + k]);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) b[j][s] = Bs[(k + s) * T::BS + ws.wn0 + 32 * j + c];
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc.c[i][j], 0, 0, 0);
  }
}

// Sum the k groups' partial tiles into group 0 (group order, so the result
// does not depend on timing).  Returns true for the waves that hold the
// final tile and run the epilogue.  Called by every thread after mainloop.
template <class T>
__device__ __forceinline__ bool reduce_k_groups(Accum<T>& acc, float* smem, const WaveSlot& ws,
                                       int lane) {
  if (T::WK == 1) return true;
  constexpr int REGS = T::FM * T::FN * 16;
  constexpr int WAVE_FLOATS = REGS * 64;  // one wave's accumulators
  constexpr int GROUP_FLOATS = T::WM * T::WN * WAVE_FLOATS;
  const int wmn = (threadIdx.x >> 6) % (T::WM * T::WN);
  if (ws.kgroup > 0) {
    float* dst = smem + (ws.kgroup - 1) * GROUP_FLOATS + wmn * WAVE_FLOATS + lane;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[((i * T::FN + j) * 16 + r) * 64] = acc.c[i][j][r];
  }
  __syncthreads();
  if (ws.kgroup > 0) return false;
#pragma unroll 1
  for (int g = 1; g < T::WK; ++g) {
    const float* src = smem + (g - 1) * GROUP_FLOATS + wmn * WAVE_FLOATS + lane;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc.c[i][j][r] += src[((i * T::FN + j) * 16 + r) * 64];
  }
  return true;
}

// The k loop over k-tiles [t_begin, t_end).  Tile t is fetched from global
// memory into register slot (t - t_begin) % 2 PF iterations before it is
// needed; each iteration runs the MFMAs on tile t from one LDS buffer,
// writes tile t+1 from its register slot into the other buffer, and ends
// with one barrier.  With PF = 2 the loads of tile t+2 are in flight during
// the whole of iteration t and the wait before writing tile t+1 covers only
// loads issued an iteration earlier.  The loop is unrolled by two so that
// register slots are compile-time indices.
//
// That wait is only exact when no branch skips the loads: the compiler
// counts outstanding loads per path and, where a path may have issued fewer,
// waits for all of them, i.e. also for tile t+2.  Row and column loaders
// therefore always fetch; the last two iterations of a range fetch tile
// t_end - 1 again into a slot that is never written to LDS.  The im2col
// gathers keep the skipping form: their ranges are short pieces of a
// tile (stream scheduling), where the extra loads cost more than the
// exact wait gains (measured on the 3x3 convs).
//
// A loader may also keep per-k-tile metadata in LDS: meta(t) writes the
// metadata of tile t into slot t % 4 and is called PF + 1 tiles ahead of
// load(t).  The slot it overwrites was last read by load(t - 4), several
// barriers earlier, and load(t) runs after the next barrier.
template <class T, class AL, class BL>
struct MainLoop {
  AL& al;
  BL& bl;
  Accum<T>& acc;
  float* smem;
  const WaveSlot& ws;
  int lane, t_end;

  template <int S>
  __device__ __forceinline__ void fetch(int t) {
    al.template load<S>(t * T::BK);
    bl.template load<S>(t * T::BK);
  }
  template <int S>
  __device__ __forceinline__ void put(int t, float* buf) {
    (void)t;
    al.template store<S>(buf);
    bl.template store<S>(buf + T::A_FLOATS);
  }
  // One iteration for tile t held in register slot S (S = (t - t_begin) % 2).
  template <int S>
  __device__ __forceinline__ void step(int t, int i) {
    float* cur = smem + (i & 1) * T::STAGE;
    float* nxt = smem + ((i + 1) & 1) * T::STAGE;
    // PF = 1 needs a single register slot: tile t+1 is fetched and written
    // within the same iteration.
    constexpr int NEXT = T::PF == 2 ? 1 - S : 0;
    if (T::PF == 2) {
      if (!BL::kHasMeta)
        fetch<S>(t + 2 < t_end ? t + 2 : t_end - 1);
      else if (t + 2 < t_end)
        fetch<S>(t + 2);
      if (BL::kHasMeta && t + 3 < t_end) bl.meta(t + 3);
    } else {
      if (!BL::kHasMeta)
        fetch<0>(t + 1 < t_end ? t + 1 : t_end - 1);
      else if (t + 1 < t_end)
        fetch<0>(t + 1);
      if (BL::kHasMeta && t + 2 < t_end) bl.meta(t + 2);
    }
    mma_tile<T, BL::kBTransposed>(acc, cur, cur + T::A_FLOATS, ws, lane);
    // Loaders without metadata fetch every iteration (the last ones again
    // fetch tile t_end - 1), so their write to the idle stage can be
    // unconditional: nothing reads that stage before the next barrier.
    if (!BL::kHasMeta || t + 1 < t_end) put<NEXT>(t + 1, nxt);
    __syncthreads();
  }
};

// With PF = 2 the loop body runs both register slots' iterations and a lone
// last iteration is peeled after the loop, so every path into the loop
// header carries the same outstanding loads.  (With the second iteration
// under an `if`, the path that skips it reaches the header with the other
// slot's loads in flight, and the compiler then waits for every load --
// including the prefetch just issued -- before the first LDS read of each
// iteration.)  PEEL = false keeps the unpeeled loop, for instances whose
// registers the duplicated iteration would spill.
template <class T, class AL, class BL, bool PEEL = true>
__device__ __forceinline__ void mainloop(Accum<T>& acc, AL& al, BL& bl, int t_begin, int t_end,
                                         float* smem, const WaveSlot& ws, int lane) {
  acc.zero();
  if (t_begin >= t_end) return;
  MainLoop<T, AL, BL> ml{al, bl, acc, smem, ws, lane, t_end};
  if (BL::kHasMeta) {
#pragma unroll
    for (int d = 0; d <= T::PF; ++d)
      if (t_begin + d < t_end) bl.meta(t_begin + d);
    __syncthreads();
  }
  ml.template fetch<0>(t_begin);
  if (T::PF == 2 && (!BL::kHasMeta || t_begin + 1 < t_end))
    ml.template fetch<1>(t_begin + 1 < t_end ? t_begin + 1 : t_begin);
  ml.template put<0>(t_begin, smem);
  __syncthreads();
  if (T::PF == 2 && PEEL) {
    int t = t_begin;
    for (; t + 1 < t_end; t += 2) {
      ml.template step<0>(t, t - t_begin);
      ml.template step<1>(t + 1, t + 1 - t_begin);
    }
    if (t < t_end) ml.template step<0>(t, t - t_begin);
  } else if (T::PF == 2) {
    for (int t = t_begin; t < t_end; t += 2) {
      ml.template step<0>(t, t - t_begin);
      if (t + 1 < t_end) ml.template step<1>(t + 1, t + 1 - t_begin);
    }
  } else {
    for (int t = t_begin; t < t_end; ++t) ml.template step<0>(t, t - t_begin);
  }
}

// ------------------------------------------------------------ scheduling
//
// How blocks map to work:
//  MODE_TILE    one output tile per block, all of K.
//  MODE_SLICES  tiles x splits blocks; block (tile, z) computes K slice z.
//  MODE_STREAM  P blocks share the (tile, k-tile) units evenly: block w
//               takes units [w*U/P, (w+1)*U/P) in tile-major order, so a
//               tile is either whole in one block or cut into pieces.
// Block ids are XCD-remapped and tiles follow the grouped raster, so
// neighbouring tiles share an XCD's L2.
// How a (piece of a) tile writes its result.
enum {
  EPI_STORE = 0,     // whole tile: fused epilogue, plain stores
  EPI_ATOMIC = 1,    // one of several K slices: atomic add into an initialised out
  EPI_EXCHANGE = 2,  // one of exactly two pieces: swap in, the second combines
};

// Bit pattern written into out before two-piece tiles are combined: a
// signalling NaN, which no arithmetic produces (results are quiet NaNs), so
// it cannot be mistaken for a partial sum.
constexpr uint32_t kPieceSentinel = 0x7FA5A5A5u;

struct Sched {
  int tiles_m, tiles_n, group_m;
  int nkt;                     // k-tiles per tile
  int splits, kt_per_split;    // MODE_SLICES
};

template <int MODE, class F>
__device__ __forceinline__ void for_each_piece(const Sched& s, int BM, int BN, F&& f) {
  const int lid = xcd_linear(blockIdx.x, gridDim.x);
  const int ntiles = s.tiles_m * s.tiles_n;
  int tm, tn;
  if (MODE == MODE_STREAM) {
    const int64_t total = (int64_t)ntiles * s.nkt;
    const int64_t P = gridDim.x;
    const int64_t base = total / P, rem = total % P;
    int64_t u = lid * base + (lid < rem ? lid : rem);
    const int64_t ue = u + base + (lid < rem ? 1 : 0);
    while (u < ue) {
      const int tile = (int)(u / s.nkt);
      const int kb = (int)(u - (int64_t)tile * s.nkt);
      const int ke = (int)(s.nkt < kb + (ue - u) ? s.nkt : kb + (ue - u));
      grouped_tile(tile, s.tiles_m, s.tiles_n, s.group_m, tm, tn);
      f(tm * BM, tn * BN, kb, ke, (kb == 0 && ke == s.nkt) ? EPI_STORE : EPI_EXCHANGE);
      u += ke - kb;
      __syncthreads();  // LDS is reused by the next piece
    }
  } else {
    const int z = lid / ntiles;
    grouped_tile(lid - z * ntiles, s.tiles_m, s.tiles_n, s.group_m, tm, tn);
    if (MODE == MODE_SLICES) {
      const int tb = z * s.kt_per_split;
      const int te = s.nkt < tb + s.kt_per_split ? s.nkt : tb + s.kt_per_split;
      f(tm * BM, tn * BN, tb, te, s.splits == 2 ? EPI_EXCHANGE : EPI_ATOMIC);
    } else {
      f(tm * BM, tn * BN, 0, s.nkt, EPI_STORE);
    }
  }
}

// Row of accumulator register j of a 32x32 block, relative to the block.
__device__ inline int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

}  // namespace baim
