// Large-M bf16 GEMM on MFMA for the column- and row-parallel linears.
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]          (Y = X W with W stored [N, K])
//
// Both operands are K-contiguous (activations [M, K], nn.Linear weights
// [N, K]), so every global load is a 16-byte vector of 8 consecutive k and
// every LDS read feeds one v_mfma_f32_32x32x16_bf16 operand directly.
//
// Tiling: a workgroup owns a BM x BN output tile and walks K in steps of BK.
// Tiles of X and W go global -> registers -> LDS (double-buffered, one
// barrier per K step); the next K step's global loads are in flight while the
// current step's MFMAs run.  LDS rows are BK bf16 = 128 bytes; the 16-byte
// chunk index inside a row is XOR-swizzled with the row index so that the
// rows read by one MFMA operand fetch spread over all LDS banks.
// Workgroup ids are remapped so that tiles sharing X rows / W rows run on the
// same XCD (one L2 per XCD) in groups of 8 M-tiles.
#include "common.h"

namespace tpl {

template <int BM_, int BN_, int WM_, int WN_>
struct MfmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;   // per-wave sub-tile
  static constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA blocks per wave
  static constexpr int KC = BK / 8;                  // 16-byte chunks per row (8)
  static constexpr int A_LD = BM * KC / NT;          // 16-byte loads per thread, X
  static constexpr int B_LD = BN * KC / NT;          // 16-byte loads per thread, W
  static constexpr int LDS_A = BM * BK, LDS_B = BN * BK;   // bf16 elements per buffer
  static_assert(BM % (WM * 32) == 0 && BN % (WN * 32) == 0, "tile/wave mismatch");
  static_assert((BM * KC) % NT == 0 && (BN * KC) % NT == 0, "load split");
};

// Rows are 128 bytes, so two rows share one 256-byte sweep of the 64 LDS
// banks; XOR-ing the chunk index with (row / 2) % 8 makes the 16 rows that
// one quarter-wave reads in an MFMA operand fetch land on 16 distinct 16-byte
// bank groups.
__device__ __forceinline__ int swz(int row, int kc) { return kc ^ ((row >> 1) & 7); }

// Load 8 consecutive bf16 of row `r` starting at column `k` (element path:
// any alignment, zero outside [0,rows) x [0,K)).
__device__ __forceinline__ u32x4 load8_guarded(const uint16_t* __restrict__ p, int64_t ld,
                                               int r, int rows, int k, int K, bool aligned) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r >= rows) return v;
  const uint16_t* src = p + (int64_t)r * ld;
  if (aligned) {
    if (k < K) v = *reinterpret_cast<const u32x4*>(src + k);
    return v;
  }
  uint16_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = (k + i < K) ? src[k + i] : (uint16_t)0;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
  return v;
}

template <class C, bool OUT_F32, bool ALIGNED>
__global__ __launch_bounds__(C::NT) void gemm_bf16_mfma_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * (C::LDS_A + C::LDS_B)];

  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + C::BN - 1) / C::BN;
  const int ntile = tiles_m * tiles_n;
  const int pid = xcd_remap(blockIdx.x, ntile);
  constexpr int GROUP_M = 8;
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (pid / in_group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % in_group) % gsize;
  const int tn = (pid % in_group) / gsize;
  const int m0 = tm * C::BM, n0 = tn * C::BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[C::A_LD], rb[C::B_LD];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int c = tid + i * C::NT, row = c / C::KC, kc = c % C::KC;
      ra[i] = load8_guarded(X, K, m0 + row, M, k0 + kc * 8, K, ALIGNED);
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int c = tid + i * C::NT, row = c / C::KC, kc = c % C::KC;
      rb[i] = load8_guarded(W, K, n0 + row, N, k0 + kc * 8, K, ALIGNED);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* la = lds + buf * (C::LDS_A + C::LDS_B);
    uint16_t* lb = la + C::LDS_A;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int c = tid + i * C::NT, row = c / C::KC, kc = c % C::KC;
      *reinterpret_cast<u32x4*>(la + row * C::BK + swz(row, kc) * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int c = tid + i * C::NT, row = c / C::KC, kc = c % C::KC;
      *reinterpret_cast<u32x4*>(lb + row * C::BK + swz(row, kc) * 8) = rb[i];
    }
  };

  const int nk = (K + C::BK - 1) / C::BK;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < nk; ++t) {
    if (t + 1 < nk) gload((t + 1) * C::BK);
    const uint16_t* la = lds + (t & 1) * (C::LDS_A + C::LDS_B);
    const uint16_t* lb = la + C::LDS_A;
#pragma unroll
    for (int kk = 0; kk < C::BK / 16; ++kk) {
      const int kc = kk * 2 + (lane >> 5);
      bf16x8 a[C::FM], b[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::TM + i * 32 + (lane & 31);
        a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(la + row * C::BK + swz(row, kc) * 8));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int row = wn * C::TN + j * 32 + (lane & 31);
        b[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(lb + row * C::BK + swz(row, kc) * 8));
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (t + 1 < nk) lstore((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane holds column (lane & 31) and
  // rows 8*(r/4) + 4*(lane/32) + (r%4), r = 0..15.
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int n = n0 + wn * C::TN + j * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * C::TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M) {
          if constexpr (OUT_F32)
            reinterpret_cast<float*>(Y)[(int64_t)m * N + n] = acc[i][j][r];
          else
            reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = (uint16_t)f2bf_bits(acc[i][j][r]);
        }
      }
    }
  }
}

using Tile256x256 = MfmaTile<256, 256, 2, 2>;
using Tile256x128 = MfmaTile<256, 128, 2, 2>;
using Tile128x128 = MfmaTile<128, 128, 2, 2>;

template <class C>
static tp_status launch_tile(const void* x, const void* w, void* y, int M, int N, int K,
                             bool out_f32, bool aligned, hipStream_t s) {
  const int ntile = ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  dim3 grid(ntile), block(C::NT);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
  if (out_f32) {
    if (aligned) hipLaunchKernelGGL((gemm_bf16_mfma_kernel<C, true, true>), grid, block, 0, s, X, Wp, y, M, N, K);
    else hipLaunchKernelGGL((gemm_bf16_mfma_kernel<C, true, false>), grid, block, 0, s, X, Wp, y, M, N, K);
  } else {
    if (aligned) hipLaunchKernelGGL((gemm_bf16_mfma_kernel<C, false, true>), grid, block, 0, s, X, Wp, y, M, N, K);
    else hipLaunchKernelGGL((gemm_bf16_mfma_kernel<C, false, false>), grid, block, 0, s, X, Wp, y, M, N, K);
  }
  TPL_LAUNCH_CHECK("gemm_bf16_mfma");
  return TP_OK;
}

// Pick the tile with the lowest estimated time: number of full-chip rounds of
// workgroups (256 CUs, one 256-thread workgroup per CU at these register
// counts) times the per-tile cost relative to the 256x256 tile.
int gemm_mfma_pick_tile(int M, int N) {
  struct Opt { int bm, bn; double cost; } opts[3] = {
      {256, 256, 1.00}, {256, 128, 0.56}, {128, 128, 0.31}};
  int best = 0;
  double best_t = 1e300;
  for (int i = 0; i < 3; ++i) {
    const double tiles = (double)((M + opts[i].bm - 1) / opts[i].bm) * ((N + opts[i].bn - 1) / opts[i].bn);
    const double rounds = ceil(tiles / 256.0);
    const double t = rounds * opts[i].cost;
    if (t < best_t - 1e-12) { best_t = t; best = i; }
  }
  return best;
}

tp_status gemm_bf16_mfma(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                         bool out_f32, bool aligned, hipStream_t s, int force_tile) {
  const int pick = force_tile >= 0 ? force_tile : gemm_mfma_pick_tile((int)M, (int)N);
  switch (pick) {
    case 0: return launch_tile<Tile256x256>(x, w, y, (int)M, (int)N, (int)K, out_f32, aligned, s);
    case 1: return launch_tile<Tile256x128>(x, w, y, (int)M, (int)N, (int)K, out_f32, aligned, s);
    default: return launch_tile<Tile128x128>(x, w, y, (int)M, (int)N, (int)K, out_f32, aligned, s);
  }
}

}  // namespace tpl
