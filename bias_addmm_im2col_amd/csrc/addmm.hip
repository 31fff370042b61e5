// addmm.hip -- out = beta*self + alpha*(mat1 @ mat2) on the gfx950 matrix
// cores ("[ExecuTorch][WebGPU] Add optimized addmm op", Solution and
// Implementation paragraphs: mat1 [M,K] and mat2 [K,N] row-major, the
// epilogue picks self[r*N + c] for a full self and the broadcast self[c]
// otherwise, and writes beta*self + alpha*acc).
//
// With a K split (chosen for grids too small to fill the chip), a first
// kernel writes beta*self (or 0) into out and every K slice then adds its
// alpha*partial with a hardware fp32 atomic add.
#include <stdlib.h>

#include "gemm_core.hpp"
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
  int tiles_m, tiles_n, group_m, splits, kt_per_split;
};

template <class T, int VA, int VB, bool SPLIT>
__global__ __launch_bounds__(T::NT) void addmm_kernel(AddmmArgs p) {
  __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE];
  const BlockWork w = block_work(p.tiles_m, p.tiles_n, p.group_m, SPLIT ? p.splits : 1,
                                 p.kt_per_split, p.K, T::BM, T::BN, T::BK);
  const int lane = threadIdx.x & 63;
  const WaveSlot ws = wave_slot<T>();
  const int wm0 = ws.wm0, wn0 = ws.wn0;

  RowTileLoader<T, VA> al;
  al.init(p.A, w.m0, p.M, p.K);
  ColTileLoader<T, VB> bl;
  bl.init(p.B, w.n0, p.N, p.K);
  Accum<T> acc;
  mainloop<T>(acc, al, bl, w.t_begin, w.t_end, smem, ws, lane);
  if (!reduce_k_groups<T>(acc, smem, ws, lane)) return;

  // Fused epilogue: beta*self + alpha*acc, self broadcast from [N] or full.
  const int c = lane & 31;
#pragma unroll
  for (int j = 0; j < T::FN; ++j) {
    const int n = w.n0 + wn0 + 32 * j + c;
    if (n >= p.N) continue;
    const float srow = !SPLIT && p.self_mode == 1 ? p.self[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = w.m0 + wm0 + 32 * i + acc_row(r, lane);
        if (m >= p.M) continue;
        const size_t o = (size_t)m * p.N + n;
        const float v = acc.c[i][j][r];
        if (SPLIT) {
          unsafeAtomicAdd(&p.out[o], p.alpha * v);
        } else if (p.self_mode == 0) {
          p.out[o] = p.alpha * v;
        } else {
          const float s = p.self_mode == 1 ? srow : p.self[o];
          p.out[o] = fmaf(p.alpha, v, p.beta * s);
        }
      }
  }
}

// out = beta*self (self_mode 1 or 2) or 0 (self_mode 0), before the K slices
// add their partial products.
__global__ __launch_bounds__(256) void addmm_init_kernel(float* out, const float* self,
                                                         int self_mode, float beta,
                                                         uint32_t total, FastDiv div_n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += gridDim.x * 256u) {
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

typedef Tile<128, 128, 32, 2, 4> T128x128;
typedef Tile<128, 64, 32, 4, 2> T128x64;
typedef Tile<64, 128, 32, 2, 4> T64x128;
typedef Tile<64, 64, 32, 2, 2> T64x64;
typedef Tile<128, 128, 64, 2, 4, 2> T128x128K2;
typedef Tile<128, 64, 64, 4, 2, 2> T128x64K2;
typedef Tile<64, 64, 64, 2, 2, 2> T64x64K2;
typedef Tile<64, 64, 128, 2, 2, 4> T64x64K4;

// The host planner's table must describe exactly these tiles.
template <class T>
constexpr bool same_tile(int cfg) {
  return T::BM == kTileBM[cfg] && T::BN == kTileBN[cfg] && T::BK == kTileBK[cfg] &&
         T::NT == 64 * kTileWaves[cfg] && T::WK == kTileKGroups[cfg];
}
static_assert(same_tile<T128x128>(TILE_128x128) && same_tile<T128x64>(TILE_128x64) &&
                  same_tile<T64x128>(TILE_64x128) && same_tile<T64x64>(TILE_64x64) &&
                  same_tile<T128x128K2>(TILE_128x128_K2) && same_tile<T128x64K2>(TILE_128x64_K2) &&
                  same_tile<T64x64K2>(TILE_64x64_K2) && same_tile<T64x64K4>(TILE_64x64_K4),
              "tile table out of sync with the compiled tiles");

template <class T, int VA, int VB, bool SPLIT>
static hipError_t launch_t(const AddmmArgs& a, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((addmm_kernel<T, VA, VB, SPLIT>), dim3(nblocks), dim3(T::NT), 0, s, a);
  return hipGetLastError();
}

template <class T, bool SPLIT>
static hipError_t launch_vec(const AddmmArgs& a, int nblocks, bool va, bool vb, hipStream_t s) {
  if (va && vb) return launch_t<T, 4, 4, SPLIT>(a, nblocks, s);
  if (va) return launch_t<T, 4, 1, SPLIT>(a, nblocks, s);
  if (vb) return launch_t<T, 1, 4, SPLIT>(a, nblocks, s);
  return launch_t<T, 1, 1, SPLIT>(a, nblocks, s);
}

template <bool SPLIT>
static hipError_t launch_cfg(int cfg, const AddmmArgs& a, int nblocks, bool va, bool vb,
                             hipStream_t s) {
  switch (cfg) {
    case TILE_128x64:
      return launch_vec<T128x64, SPLIT>(a, nblocks, va, vb, s);
    case TILE_64x128:
      return launch_vec<T64x128, SPLIT>(a, nblocks, va, vb, s);
    case TILE_64x64:
      return launch_vec<T64x64, SPLIT>(a, nblocks, va, vb, s);
    case TILE_128x128_K2:
      return launch_vec<T128x128K2, SPLIT>(a, nblocks, va, vb, s);
    case TILE_128x64_K2:
      return launch_vec<T128x64K2, SPLIT>(a, nblocks, va, vb, s);
    case TILE_64x64_K2:
      return launch_vec<T64x64K2, SPLIT>(a, nblocks, va, vb, s);
    case TILE_64x64_K4:
      return launch_vec<T64x64K4, SPLIT>(a, nblocks, va, vb, s);
    default:
      return launch_vec<T128x128, SPLIT>(a, nblocks, va, vb, s);
  }
}

hipError_t launch_addmm(const AddmmProblem& p, hipStream_t stream) {
  const GemmPlan plan = plan_gemm(p.M, p.N, p.K, getenv("BAIM_TILE"));
  AddmmArgs a;
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
  a.tiles_m = plan.tiles_m;
  a.tiles_n = plan.tiles_n;
  a.group_m = 8;
  a.splits = plan.splits;
  a.kt_per_split = plan.kt_per_split;
  const int nblocks = (int)plan_blocks(plan);
  // 16-byte vector loads need K (resp. N) divisible by 4 and aligned bases.
  const bool va = p.K % 4 == 0 && ((uintptr_t)p.mat1 & 15) == 0;
  const bool vb = p.N % 4 == 0 && ((uintptr_t)p.mat2 & 15) == 0;
  if (plan.splits > 1) {
    const uint32_t total = (uint32_t)p.M * (uint32_t)p.N;
    const int gb = (int)((total + 255u) / 256u < 4096u ? (total + 255u) / 256u : 4096u);
    hipLaunchKernelGGL(addmm_init_kernel, dim3(gb), dim3(256), 0, stream, p.out, p.self,
                       p.self_mode, p.beta, total, make_fastdiv((uint32_t)p.N));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_cfg<true>(plan.cfg, a, nblocks, va, vb, stream);
  }
  return launch_cfg<false>(plan.cfg, a, nblocks, va, vb, stream);
}

}  // namespace baim
