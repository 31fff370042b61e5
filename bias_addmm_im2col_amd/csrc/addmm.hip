// addmm.hip -- out = beta*self + alpha*(mat1 @ mat2) on the gfx950 matrix
// cores ("[ExecuTorch][WebGPU] Add optimized addmm op", Solution and
// Implementation paragraphs: mat1 [M,K] and mat2 [K,N] row-major, the
// epilogue picks self[r*N + c] for a full self and the broadcast self[c]
// otherwise, and writes beta*self + alpha*acc).  The same kernel computes
// linear, out = x @ weight^T + bias with weight [N,K] (the page's
// linear_fp32 reads that transposed weight), when instantiated with WNK:
// the weight's K-contiguous rows load straight into the transposed B tile.
// With WNK and AK = A_NHWC it computes the channels-last conv: the A tile is
// then gathered from the NHWC input as rows of the implicit im2col matrix
// (im2col_nhwc.hpp), the weight [OC,KH,KW,IC] is the [N,K] B operand and
// the bias is self [N].
//
// Work split (see gemm_core.hpp): one tile per block; or K slices; or
// stream pieces.  A tile cut into exactly two pieces is combined without a
// workspace: out starts as a sentinel, each piece swaps its partial in, and
// the piece that gets the other's partial back adds the two (an order-free
// sum) and writes the fused epilogue, so the result is the same bits on
// every run.  With more than two K slices (grids too small for anything
// else) out starts as beta*self and the slices add alpha*partial with
// hardware fp32 atomics.
#include <stdlib.h>

#include <type_traits>

#include "gemm_core.hpp"
#include "im2col_nhwc.hpp"
#include "launch.hpp"
#include "tile_select.hpp"

namespace baim {

struct AddmmArgs {
  float* out;
  const float* self;
  const float* A;
  const float* B;
  int M, N, K;
  int self_mode;  // 0: beta == 0 (self not read); 1: self [N]; 2: self [M,N]
  float beta, alpha;
  Sched sched;
  NhwcGeom g;  // A_NHWC only
};

// Where the A tile comes from.
enum { A_ROWS = 0, A_NHWC = 1 };

template <class T, int VA, int VB, bool WNK, int AK>
__device__ __forceinline__ void addmm_piece(const AddmmArgs& p, float* smem, int m0, int n0, int tb,
                                   int te, int epi) {
  const int lane = threadIdx.x & 63;
  const WaveSlot ws = wave_slot<T>();
  typename std::conditional<AK == A_NHWC, NhwcRowLoader<T, VA>, RowTileLoader<T, VA>>::type al;
  if constexpr (AK == A_NHWC)
    al.init(p.A, p.g, m0, p.M, p.K);
  else
    al.init(p.A, m0, p.M, p.K);
  typename std::conditional<WNK, KRowLoader<T, VB, T::BN, true>, ColTileLoader<T, VB>>::type bl;
  bl.init(p.B, n0, p.N, p.K);
  const int c = lane & 31;
  // A whole tile with a full self [M,N] and one 32 x 32 block per wave:
  // its 16 self values per lane are loaded before the k loop, so the
  // epilogue does not wait for them (they arrive with the first k-tile).
  constexpr bool kSelfAhead = T::FM * T::FN == 1 && T::WK < 4;  // registers to spare
  float sv[16];
  const bool self_ahead = kSelfAhead && epi == EPI_STORE && p.self_mode == 2 && ws.kgroup == 0;
  if (kSelfAhead && self_ahead) {
    const int n = n0 + ws.wn0 + c;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + ws.wm0 + acc_row(r, lane);
      sv[r] = (m < p.M && n < p.N) ? p.self[(size_t)m * p.N + n] : 0.0f;
    }
  }
  Accum<T> acc;
  // 16 waves with 4-byte loads on both operands: the peeled loop would spill
  mainloop<T, decltype(al), decltype(bl), !(T::NT == 1024 && VA == 1 && VB == 1)>(
      acc, al, bl, tb, te, smem, ws, lane);
  if (!reduce_k_groups<T>(acc, smem, ws, lane)) return;

  // Fused epilogue: beta*self + alpha*acc, self broadcast from [N] or full.
  if (epi == EPI_EXCHANGE) {
    // Two-piece tile: swap every partial in first (all swaps in flight at
    // once), then finish the elements whose other piece had already landed.
    uint32_t other[T::FM][T::FN][16];
#pragma unroll
    for (int j = 0; j < T::FN; ++j)
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = n0 + ws.wn0 + 32 * j + c, m = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          other[i][j][r] = kPieceSentinel;
          if (n < p.N && m < p.M)
            other[i][j][r] = atomicExch(reinterpret_cast<unsigned int*>(&p.out[(size_t)m * p.N + n]),
                                        __float_as_uint(acc.c[i][j][r]));
        }
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int n = n0 + ws.wn0 + 32 * j + c;
      if (n >= p.N) continue;
      const float srow = p.self_mode == 1 ? p.self[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          if (m >= p.M || other[i][j][r] == kPieceSentinel) continue;
          const size_t o = (size_t)m * p.N + n;
          const float v = __uint_as_float(other[i][j][r]) + acc.c[i][j][r];
          if (p.self_mode == 0) {
            p.out[o] = p.alpha * v;
          } else {
            const float sv = p.self_mode == 1 ? srow : p.self[o];
            p.out[o] = fmaf(p.alpha, v, p.beta * sv);
          }
        }
    }
    return;
  }
  if (epi == EPI_STORE && p.self_mode == 1 && m0 + T::BM <= p.M && n0 + T::BN <= p.N) {
    // A whole tile with self [N]: no bounds tests and no mode choice per
    // element (with them, the epilogue cost 3.7 us of the 4096 x 4096 x
    // 1024 down-projection and 3.3 us of the 2048 x 768 x 3072 FFN).
    // Non-temporal: the output is not read back (FFN 80 -> 77 us; the
    // 256x256 kernel's stores got slower that way and stay plain).
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int n = n0 + ws.wn0 + 32 * j + c;
        const float bs = p.beta * p.self[n];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
          __builtin_nontemporal_store(fmaf(p.alpha, acc.c[i][j][r], bs), &p.out[(size_t)m * p.N + n]);
        }
      }
    return;
  }
  if (epi == EPI_STORE && p.self_mode == 2 && m0 + T::BM <= p.M && n0 + T::BN <= p.N) {
    // the same with a full self (ragged-577 addmm 56.8 -> 55.6 us; 55.0
    // -> 54.4 us with non-temporal stores)
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int n = n0 + ws.wn0 + 32 * j + c;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const size_t o = (size_t)(m0 + ws.wm0 + 32 * i + acc_row(r, lane)) * p.N + n;
          const float s = (kSelfAhead && self_ahead) ? sv[r] : p.self[o];
          __builtin_nontemporal_store(fmaf(p.alpha, acc.c[i][j][r], p.beta * s), &p.out[o]);
        }
      }
    return;
  }
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = n0 + ws.wn0 + 32 * j + c;
    if (n >= p.N) continue;
    const float srow = p.self_mode == 1 && epi == EPI_STORE ? p.self[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + ws.wm0 + 32 * i + acc_row(r, lane);
        if (m >= p.M) continue;
        const size_t o = (size_t)m * p.N + n;
        const float v = acc.c[i][j][r];
        if (epi == EPI_ATOMIC) {
          unsafeAtomicAdd(&p.out[o], p.alpha * v);
        } else if (p.self_mode == 0) {
          p.out[o] = p.alpha * v;
        } else {
          const float s = p.self_mode == 1 ? srow : ((kSelfAhead && self_ahead) ? sv[r] : p.self[o]);
          p.out[o] = fmaf(p.alpha, v, p.beta * s);
        }
      }
  }
}

template <class T, int VA, int VB, int MODE, bool WNK, int AK>
__global__ __launch_bounds__(T::NT) void addmm_kernel(AddmmArgs p) {
  __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];
  for_each_piece<MODE>(p.sched, T::BM, T::BN, [&](int m0, int n0, int tb, int te, int epi) __attribute__((always_inline)) {
    addmm_piece<T, VA, VB, WNK, AK>(p, smem, m0, n0, tb, te, epi);
  });
}

// Output initialisation before a split tile's pieces land: the sentinel
// (two-piece combine, 16-byte stores) or beta*self / 0 (atomic K slices).
__global__ __launch_bounds__(256) void addmm_init_kernel(float* out, const float* self,
                                                         int self_mode, float beta,
                                                         int sentinel, uint32_t total,
                                                         FastDiv div_n) {
  const uint32_t stride = gridDim.x * 256u;
  if (sentinel) {
    const float s = __uint_as_float(kPieceSentinel);
    const f32x4 s4 = {s, s, s, s};
    const uint32_t head = (uint32_t)((16u - ((uintptr_t)out & 15u)) & 15u) / 4u;
    const uint32_t h = head < total ? head : total;
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < h; i += stride) out[i] = s;
    const uint32_t nvec = (total - h) / 4u;
    f32x4* o4 = reinterpret_cast<f32x4*>(out + h);
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < nvec; i += stride) o4[i] = s4;
    for (uint32_t i = h + nvec * 4u + blockIdx.x * 256u + threadIdx.x; i < total; i += stride)
      out[i] = s;
    return;
  }
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += stride) {
    float v = 0.0f;
    if (self_mode == 1) {
      const uint32_t m = fdiv(i, div_n);
      v = beta * self[i - m * div_n.d];
    } else if (self_mode == 2) {
      v = beta * self[i];
    }
    out[i] = v;
  }
}

// Every tile prefetches two k-tiles ahead (see mainloop).
typedef Tile<128, 128, 32, 2, 4, 1, 2> T128x128;
typedef Tile<128, 64, 32, 4, 2, 1, 2> T128x64;
typedef Tile<64, 128, 32, 2, 4, 1, 2> T64x128;
typedef Tile<64, 64, 32, 2, 2, 1, 2> T64x64;
typedef Tile<128, 128, 64, 2, 4, 2, 2> T128x128K2;
typedef Tile<128, 64, 64, 4, 2, 2, 2> T128x64K2;
typedef Tile<64, 64, 64, 2, 2, 2, 2> T64x64K2;
typedef Tile<64, 64, 128, 2, 2, 4, 2> T64x64K4;
typedef Tile<32, 128, 32, 1, 4, 1, 2> T32x128;

// The host planner's table must describe exactly these tiles.
template <class T>
constexpr bool same_tile(int cfg) {
  return T::BM == kTileBM[cfg] && T::BN == kTileBN[cfg] && T::BK == kTileBK[cfg] &&
         T::NT == 64 * kTileWaves[cfg] && T::WK == kTileKGroups[cfg];
}
static_assert(same_tile<T128x128>(TILE_128x128) && same_tile<T128x64>(TILE_128x64) &&
                  same_tile<T64x128>(TILE_64x128) && same_tile<T64x64>(TILE_64x64) &&
                  same_tile<T128x128K2>(TILE_128x128_K2) && same_tile<T128x64K2>(TILE_128x64_K2) &&
                  same_tile<T64x64K2>(TILE_64x64_K2) && same_tile<T64x64K4>(TILE_64x64_K4) &&
                  same_tile<T32x128>(TILE_32x128),
              "tile table out of sync with the compiled tiles");

// ------------------------------------------------------ the 256x256 tile
// Large addmm, one 256x256 output tile per block: 8 waves of 128x64
// outputs (4 x 2 blocks of 32x32, 128 accumulator registers, two waves per
// SIMD), k-tiles of 16 with two k-tiles of register prefetch and
// double-buffered LDS, as in the tile core (same LDS layouts and MFMA
// step order).  Per MFMA a wave reads a third of what a 64x32 wave of the
// 128x128 tile reads.  It is a kernel of its own: built from the tile core
// (per-k-tile buffer descriptors, the schedule hooks) the same tile held
// about 20 more registers through the k loop, the compiler then issued
// each B read right before its MFMAs, and it ran 262 us against 244 us in
// this form on the 4096 x 1024 x 4096 up-projection.
//
// mat1 rows of the block and all of mat2 (from the block's first column)
// are addressed with 32-bit offsets: the planner takes this tile only with
// 256*K and K*N below 2^29.  Rows past M or K read past the buffer ranges
// (0); columns past K (mat1) or N (mat2) are masked per load.
namespace big {
constexpr int BM = 256, BN = 256, BK = 16, NT = 512, WTM = 128, WTN = 64;
constexpr int FM = WTM / 32, FN = WTN / 32;
constexpr int AS = BK + 4, BS = BN + 8;  // LDS row strides, as in Tile
constexpr int A_FLOATS = BM * AS, B_FLOATS = BK * BS, STAGE = A_FLOATS + B_FLOATS;
static_assert(BM == kTileBM[TILE_256x256] && BN == kTileBN[TILE_256x256] &&
                  BK == kTileBK[TILE_256x256] && NT == 64 * kTileWaves[TILE_256x256] &&
                  kTileKGroups[TILE_256x256] == 1,
              "tile table out of sync with the 256x256 kernel");
}  // namespace big

template <int VA, int VB>
__global__ __launch_bounds__(big::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void addmm_big_kernel(AddmmArgs p) {
  using namespace big;
  __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, h = lane >> 5;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, p.sched.tiles_m, p.sched.tiles_n, p.sched.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm0 = (wave / (BN / WTN)) * WTM, wn0 = (wave % (BN / WTN)) * WTN;
  const int K = p.K, N = p.N;
  const int rows = min(BM, p.M - m0), cols = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (size_t)m0 * K, (int64_t)rows * K);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + n0, (int64_t)(K - 1) * N + cols);
  constexpr int A_NQ = BM * BK / VA / NT, B_NQ = BK * BN / VB / NT;
  typedef typename Vec<VA>::T TA;
  typedef typename Vec<VB>::T TB;
  TA xa0[A_NQ], xa1[A_NQ];
  TB xb0[B_NQ], xb1[B_NQ];
  auto fetch = [&](TA* xa, TB* xb, int t) __attribute__((always_inline)) {
    const int k0 = t * BK;
#pragma unroll
    for (int q = 0; q < A_NQ; ++q) {
      const int i = tid + NT * q, r = i / (BK / VA), cc = (i % (BK / VA)) * VA;
      xa[q] = Vec<VA>::load(ra, k0 + cc < K ? (uint32_t)(r * K + k0 + cc) * 4u : kOOB);
    }
#pragma unroll
    for (int q = 0; q < B_NQ; ++q) {
      const int i = tid + NT * q, r = i / (BN / VB), cc = (i % (BN / VB)) * VB;
      xb[q] = Vec<VB>::load(rb, cc < cols ? (uint32_t)((k0 + r) * N + cc) * 4u : kOOB);
    }
  };
  auto put = [&](const TA* xa, const TB* xb, float* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < A_NQ; ++q) {
      const int i = tid + NT * q, r = i / (BK / VA), cc = (i % (BK / VA)) * VA;
      *reinterpret_cast<TA*>(&buf[r * AS + cc]) = xa[q];
    }
#pragma unroll
    for (int q = 0; q < B_NQ; ++q) {
      const int i = tid + NT * q, r = i / (BN / VB), cc = (i % (BN / VB)) * VB;
      *reinterpret_cast<TB*>(&buf[A_FLOATS + r * BS + cc]) = xb[q];
    }
  };
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // one k-tile: step s of lane half h takes k = 8g + 4h + s (the tile
  // core's order), A four k at a time from [BM][BK+4], B from [BK][BN+8]
  auto mma = [&](const float* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < BK / 8; ++g) {
      const int k = 8 * g + 4 * h;
      f32x4 a[FM];
      float b[FN][4];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const f32x4*>(&buf[(wm0 + 32 * i + c) * AS + k]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) b[j][s] = buf[A_FLOATS + (k + s) * BS + wn0 + 32 * j + c];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
    }
  };
  // the k loop: both register slots' iterations per trip and a lone last
  // one after it (every path into the loop header carries the same loads);
  // the last fetches reload tile nkt - 1 into a slot never written to LDS
  const int nkt = (K + BK - 1) / BK;
  fetch(xa0, xb0, 0);
  fetch(xa1, xb1, nkt > 1 ? 1 : 0);
  put(xa0, xb0, smem);
  __syncthreads();
  int t = 0;
  for (; t + 1 < nkt; t += 2) {
    fetch(xa0, xb0, t + 2 < nkt ? t + 2 : nkt - 1);
    mma(smem);
    put(xa1, xb1, smem + STAGE);
    __syncthreads();
    fetch(xa1, xb1, t + 3 < nkt ? t + 3 : nkt - 1);
    mma(smem + STAGE);
    put(xa0, xb0, smem);
    __syncthreads();
  }
  if (t < nkt) mma(smem);

  // beta*self + alpha*acc, self broadcast from [N] or full [M,N].  The
  // self mode is uniform: with self [N] (the bias case) a tile wholly
  // inside out has a loop of its own without bounds tests.  With the
  // tests and the mode choice inside the innermost loop this epilogue cost
  // 11 us of the 4096 x 1024 x 4096 up-projection's 256.  (Loops of their
  // own for the other modes hoisted their loads or addresses and spilled.)
  const float alpha = p.alpha, beta = p.beta;
  float* const out = p.out;
  const float* const self = p.self;
  if (rows == BM && cols == BN && p.self_mode == 1) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn0 + 32 * j + c;
        const float bs = beta * self[n];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm0 + 32 * i + acc_row(r, lane);
          out[(size_t)m * N + n] = fmaf(alpha, acc[i][j][r], bs);
        }
      }
    return;
  }
  // no self, a full self or an edge tile: every element tested
  // against M and N
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn0 + 32 * j + c;
    if (n >= N) continue;
    const float srow = p.self_mode == 1 ? self[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm0 + 32 * i + acc_row(r, lane);
        if (m >= p.M) continue;
        const size_t o = (size_t)m * N + n;
        const float v = acc[i][j][r];
        if (p.self_mode == 0) {
          out[o] = alpha * v;
        } else {
          const float sv = p.self_mode == 1 ? srow : self[o];
          out[o] = fmaf(alpha, v, beta * sv);
        }
      }
  }
}

static hipError_t launch_big(const AddmmArgs& a, int nblocks, bool va, bool vb, hipStream_t s) {
  if (va && vb)
    hipLaunchKernelGGL((addmm_big_kernel<4, 4>), dim3(nblocks), dim3(big::NT), 0, s, a);
  else if (va)
    hipLaunchKernelGGL((addmm_big_kernel<4, 1>), dim3(nblocks), dim3(big::NT), 0, s, a);
  else if (vb)
    hipLaunchKernelGGL((addmm_big_kernel<1, 4>), dim3(nblocks), dim3(big::NT), 0, s, a);
  else
    hipLaunchKernelGGL((addmm_big_kernel<1, 1>), dim3(nblocks), dim3(big::NT), 0, s, a);
  return hipGetLastError();
}

template <class T, int VA, int VB, int MODE, bool WNK = false, int AK = A_ROWS>
static hipError_t launch_t(const AddmmArgs& a, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((addmm_kernel<T, VA, VB, MODE, WNK, AK>), dim3(nblocks), dim3(T::NT), 0, s, a);
  return hipGetLastError();
}

// Stream pieces are compiled for aligned operands only (the launcher falls
// back to one tile per block otherwise).
// Linear (WNK) is compiled with 16-byte loads of both operands or with
// 4-byte loads of both (its x and weight rows share K); so is the
// channels-last conv.
template <class T, int CFG, int MODE, bool WNK, int AK>
static hipError_t launch_vec(const AddmmArgs& a, int nblocks, bool va, bool vb, hipStream_t s) {
  if constexpr (MODE == MODE_STREAM) {
    if constexpr (kTileStream[CFG]) return launch_t<T, 4, 4, MODE_STREAM, WNK, AK>(a, nblocks, s);
    return hipErrorInvalidValue;  // never planned
  } else if constexpr (MODE == MODE_SLICES && !kTileSlices[CFG]) {
    return hipErrorInvalidValue;  // never planned
  } else if constexpr (WNK) {
    if (va && vb) return launch_t<T, 4, 4, MODE, true, AK>(a, nblocks, s);
    // The 4-byte channels-last gather does not fit the 16-wave 128x128
    // tile's registers; the launcher never plans it.
    if constexpr (AK == A_NHWC && CFG == TILE_128x128_K2) return hipErrorInvalidValue;
    else return launch_t<T, 1, 1, MODE, true, AK>(a, nblocks, s);
  } else {
    if (va && vb) return launch_t<T, 4, 4, MODE>(a, nblocks, s);
    if (va) return launch_t<T, 4, 1, MODE>(a, nblocks, s);
    if (vb) return launch_t<T, 1, 4, MODE>(a, nblocks, s);
    return launch_t<T, 1, 1, MODE>(a, nblocks, s);
  }
}

template <int MODE, bool WNK, int AK = A_ROWS>
static hipError_t launch_cfg(int cfg, const AddmmArgs& a, int nblocks, bool va, bool vb,
                             hipStream_t s) {
  switch (cfg) {
    case TILE_128x64:
      return launch_vec<T128x64, TILE_128x64, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_64x128:
      return launch_vec<T64x128, TILE_64x128, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_64x64:
      return launch_vec<T64x64, TILE_64x64, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_128x128_K2:
      return launch_vec<T128x128K2, TILE_128x128_K2, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_128x64_K2:
      return launch_vec<T128x64K2, TILE_128x64_K2, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_64x64_K2:
      return launch_vec<T64x64K2, TILE_64x64_K2, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_64x64_K4:
      return launch_vec<T64x64K4, TILE_64x64_K4, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_32x128:
      return launch_vec<T32x128, TILE_32x128, MODE, WNK, AK>(a, nblocks, va, vb, s);
    case TILE_256x256:
      // addmm, one tile per block (the other callers plan with plan_core_tile)
      if constexpr (AK == A_ROWS && !WNK && MODE == MODE_TILE) return launch_big(a, nblocks, va, vb, s);
      return hipErrorInvalidValue;
    default:
      return launch_vec<T128x128, TILE_128x128, MODE, WNK, AK>(a, nblocks, va, vb, s);
  }
}

// Plan, initialise out if the plan splits tiles, and launch.
template <int AK>
static hipError_t launch_gemm(const AddmmProblem& p, AddmmArgs& a, bool va, bool vb,
                              hipStream_t stream) {
  GemmPlan plan = plan_gemm(p.M, p.N, p.K, getenv("BAIM_TILE"));
  // mat2 [K, N] is read BK rows at a time with 32-bit offsets
  if (AK == A_ROWS && !p.weight_nk) plan = plan_fit_col_operand(plan, p.M, p.N, p.K);
  if (plan.mode == MODE_STREAM && !(va && vb)) plan = plan_tiles_only(plan, p.M, p.N, p.K);
  if (AK == A_NHWC || p.weight_nk || !plan_big_fits(p.N, p.K))
    plan = plan_core_tile(plan, p.M, p.N, p.K);
  if (AK == A_NHWC && !(va && vb) && plan.cfg == TILE_128x128_K2)
    plan = plan_gemm(p.M, p.N, p.K, "0");  // same block tile, 8 waves
  a.out = p.out;
  a.self = p.self;
  a.A = p.mat1;
  a.B = p.mat2;
  a.M = p.M;
  a.N = p.N;
  a.K = p.K;
  a.self_mode = p.self_mode;
  a.beta = p.beta;
  a.alpha = p.alpha;
  a.sched = Sched{plan.tiles_m, plan.tiles_n, 8, plan.nkt, plan.splits, plan.kt_per_split};
  const int nblocks = (int)plan_blocks(plan);
  if (plan_needs_init(plan)) {
    const uint32_t total = (uint32_t)p.M * (uint32_t)p.N;
    const int gb = (int)((total + 255u) / 256u < 4096u ? (total + 255u) / 256u : 4096u);
    hipLaunchKernelGGL(addmm_init_kernel, dim3(gb), dim3(256), 0, stream, p.out, p.self,
                       p.self_mode, p.beta, plan_uses_exchange(plan) ? 1 : 0, total,
                       make_fastdiv((uint32_t)p.N));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (AK == A_NHWC || p.weight_nk) {
    switch (plan.mode) {
      case MODE_SLICES:
        return launch_cfg<MODE_SLICES, true, AK>(plan.cfg, a, nblocks, va, vb, stream);
      case MODE_STREAM:
        return launch_cfg<MODE_STREAM, true, AK>(plan.cfg, a, nblocks, va, vb, stream);
      default:
        return launch_cfg<MODE_TILE, true, AK>(plan.cfg, a, nblocks, va, vb, stream);
    }
  }
  if constexpr (AK == A_ROWS) {
    switch (plan.mode) {
      case MODE_SLICES:
        return launch_cfg<MODE_SLICES, false>(plan.cfg, a, nblocks, va, vb, stream);
      case MODE_STREAM:
        return launch_cfg<MODE_STREAM, false>(plan.cfg, a, nblocks, va, vb, stream);
      default:
        return launch_cfg<MODE_TILE, false>(plan.cfg, a, nblocks, va, vb, stream);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_addmm(const AddmmProblem& p, hipStream_t stream) {
  // 16-byte vector loads need the contiguous dim (K for mat1 and for a
  // [N,K] weight, N for mat2 [K,N]) divisible by 4 and aligned bases.
  const bool va = p.K % 4 == 0 && ((uintptr_t)p.mat1 & 15) == 0;
  const bool vb = (p.weight_nk ? p.K : p.N) % 4 == 0 && ((uintptr_t)p.mat2 & 15) == 0;
  AddmmArgs a{};
  return launch_gemm<A_ROWS>(p, a, va, vb, stream);
}

hipError_t launch_conv2d_nhwc(const ConvProblem& q, hipStream_t stream) {
  // the 3-channel 7x7 stride-4 stem has its own kernel (16-byte stores of
  // four output channels need an aligned out as well)
  const bool stem_aligned = ((uintptr_t)q.x & 15) == 0 && ((uintptr_t)q.w & 15) == 0 &&
                            ((uintptr_t)q.out & 15) == 0;
  if (plan_conv_stem(win_shape(q), stem_aligned, getenv("BAIM_CONV_WIN")))
    return launch_conv2d_stem(q, true, stream);
  // out[B*OH*OW, OC] = im2col_nhwc(x)[B*OH*OW, KH*KW*IC] @ w[OC, KH*KW*IC]^T + bias
  AddmmProblem p;
  p.out = q.out;
  p.self = q.bias;
  p.mat1 = q.x;
  p.mat2 = q.w;
  p.weight_nk = true;
  p.M = q.B * q.OH * q.OW;
  p.N = q.OC;
  p.K = q.KH * q.KW * q.IC;
  p.self_mode = q.bias ? 1 : 0;
  p.beta = 1.0f;
  p.alpha = 1.0f;
  AddmmArgs a{};
  a.g.H = q.H;
  a.g.W = q.W;
  a.g.IC = q.IC;
  a.g.KW = q.KW;
  a.g.OH = q.OH;
  a.g.OW = q.OW;
  a.g.sH = q.sH;
  a.g.sW = q.sW;
  a.g.pH = q.pH;
  a.g.pW = q.pW;
  a.g.dH = q.dH;
  a.g.dW = q.dW;
  a.g.x_elems = q.B * q.H * q.W * q.IC;
  a.g.div_ow = make_fastdiv((uint32_t)q.OW);
  a.g.div_oh = make_fastdiv((uint32_t)q.OH);
  a.g.div_ic = make_fastdiv((uint32_t)q.IC);
  a.g.div_kw = make_fastdiv((uint32_t)q.KW);
  // 16-byte gathers need whole taps of four channels and an aligned input;
  // the weight rows are K = KH*KW*IC long.
  const bool va = q.IC % 4 == 0 && ((uintptr_t)q.x & 15) == 0;
  const bool vb = p.K % 4 == 0 && ((uintptr_t)q.w & 15) == 0;
  return launch_gemm<A_NHWC>(p, a, va, vb, stream);
}

}  // namespace baim
