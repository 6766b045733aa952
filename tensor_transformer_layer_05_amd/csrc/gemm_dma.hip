// Large-M bf16 GEMM on MFMA with direct global->LDS tile loads (gfx950).
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]          (Y = X W with W stored [N, K])
//
// This is the path of the column- and row-parallel linears at prefill sizes
// (M > 64) when the operands allow 16-byte loads.  Design points for CDNA4:
//
//  * Tiles reach LDS through `buffer_load_dwordx4 ... lds`: each wave-level
//    load writes 1 KB (8 rows of 64 bf16) straight into LDS, so tile staging
//    costs no VGPRs and no ds_write instructions.  The buffer resource is
//    bounded to the tile's valid rows and out-of-range lanes get an offset
//    past that bound, so ragged edges (rows >= M or N, k >= K) read as zero
//    without any branch.
//  * LDS rows are 128 bytes (BK = 64); the 16-byte chunk index is XOR-ed with
//    (row / 2) % 8.  The loads realise the swizzle by choosing which global
//    chunk each lane fetches, and the MFMA fragment reads (16 lanes = 16 rows
//    of one chunk column) land on 16 distinct 16-byte bank groups.
//  * The W tile is the A operand and the X tile the B operand of
//    v_mfma_f32_32x32x16_bf16, so a lane's accumulators hold 4 consecutive
//    output features of one token: the epilogue writes 16-byte (fp32) or
//    8-byte (bf16) vectors.
//  * Two LDS stages.  8-wave tiles of at most 256 columns run a ping-pong
//    loop: each wave alternates a phase that reads a whole stage's fragments
//    (and issues tile loads) with a phase that issues the stage's MFMAs, and
//    the two waves of a SIMD run half a step apart, so one wave's MFMAs run
//    while the other reads.  The 256x320 tile (too many fragment registers
//    for that) and the 4-wave 128x128 tile run one barrier per 64-k step,
//    the step's body pinned by scheduling barriers: fragment reads for
//    sub-step kk+1 are issued before the MFMAs of sub-step kk, the next
//    step's tile loads go out in the first two sub-steps, and the last
//    sub-step's MFMAs are split around the barrier so that the next step's
//    first fragment reads overlap them.
//  * 256x256 tiles run 8 waves (2 per SIMD, 128x64 per wave, accumulators in
//    128 VGPRs); 128x128 tiles run 4 waves with 2 workgroups per CU, and
//    256x320 and 256x192 tiles 8 waves of 64x160 and 64x96, for grids that
//    256x256 tiles would leave with a partly empty last round.
//  * SwiGLU: the W tile holds BN/2 gate rows then the matching BN/2 up rows.
//    With an even number of W fragments per wave, each wave reads gate and up
//    fragments of the same outputs and applies the activation in registers.
//  * Workgroup ids are remapped so that consecutive tile ids share an XCD
//    (one L2 per XCD), walking groups of 4 M-tiles (measured: 4 and 8 within
//    1%, 2 and 16 slower).
#include "common.h"

namespace tpl {

#define TPL_LDS __attribute__((address_space(3)))

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14])
constexpr int kWaitVm0 = 0x0F70;   // vmcnt(0), others unconstrained

template <int BM_, int BN_, int WM_, int WN_>
struct DmaTile {
  static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_;
  static constexpr int NW = WM * WN, NT = NW * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;  // per-wave extents (tokens, features)
  static constexpr int FB = TM / 32, FA = TN / 32;  // 32-row fragments: B = X side, A = W side
  static constexpr int XL = BM / 8 / NW, WL = BN / 8 / NW;  // 1 KB loads per wave per step
  static constexpr int STAGE = (BM + BN) * BK;              // bf16 elements per LDS stage
  static_assert(XL * NW * 8 == BM && WL * NW * 8 == BN, "load split");
  static_assert(FA >= 2, "the last sub-step splits the A fragments in two");
};

__device__ __forceinline__ int dswz(int row, int kc) { return kc ^ ((row >> 1) & 7); }

// EPI: 0 = plain product; 1 = SwiGLU on a paired tile (W rows [0, I) gate,
// [I, 2I) up; the tile's first BN/2 W rows are gate rows n0.., the rest the
// matching up rows; output [M, I]); 2 = GELU on each output.  The fused
// epilogues apply the activation to the float32 accumulators, so the gate and
// up products are never rounded; only the activation's result is stored bf16.
template <class C, bool OUT_F32, bool VEC_OUT, int EPI>
__global__ __launch_bounds__(C::NT) void gemm_bf16_dma_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int M, int N, int K) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * C::STAGE];
  // SwiGLU: N is the intermediate size I, each tile covers BN/2 outputs.
  constexpr int OUT_BN = EPI == 1 ? C::BN / 2 : C::BN;
  // SwiGLU with an even number of W fragments per wave pairs gate and up rows
  // inside each wave; otherwise up-row waves hand their sums to gate-row waves
  // through LDS.
  constexpr bool kPairInWave = EPI == 1 && C::FA % 2 == 0;

  const int tiles_m = (M + C::BM - 1) / C::BM;
  const int tiles_n = (N + OUT_BN - 1) / OUT_BN;
  const int ntile = tiles_m * tiles_n;
  const int pid = xcd_remap(blockIdx.x, ntile);
  constexpr int GROUP_M = 4;
  const int in_group = GROUP_M * tiles_n;
  const int first_m = (pid / in_group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int tm = first_m + (pid % in_group) % gsize;
  const int tn = (pid % in_group) / gsize;
  const int m0 = tm * C::BM, n0 = tn * OUT_BN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;

  // Buffer resources based at the tile's first row, bounded to its valid rows.
  // SwiGLU: the waves loading W-tile rows [BN/2, BN) read the up rows I + n0..
  // (the split is wave-uniform: a wave's loads cover WL*8 consecutive rows).
  const uint32_t xrows = (uint32_t)min(C::BM, M - m0);
  const bool up_rows = EPI == 1 && wave * C::WL * 8 >= C::BN / 2;
  const uint32_t wrows = (uint32_t)min(OUT_BN, N - n0);
  const int wbase = up_rows ? N + n0 : n0;
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + (int64_t)m0 * K), 0, xrows * (uint32_t)K * 2u, 0x00020000);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)wbase * K), 0, wrows * (uint32_t)K * 2u, 0x00020000);
  const int wrow_shift = up_rows ? C::BN / 2 : 0;   // W-tile row -> row of the resource

  // Load i of this wave fills LDS rows (wave*L + i)*8 .. +7; lane -> row lane/8,
  // LDS chunk lane%8, which holds global chunk dswz(row, lane%8).
  const int lrow = lane >> 3, lpos = lane & 7;
  // 4-wave (128x128) tiles: one offset register per load.  8-wave tiles: the
  // swizzle (row/2) % 8 depends only on the parity of wave*L + i, so two base
  // offsets per operand plus a multiple of 16 rows address every load (fewer
  // registers and VALU instructions; the same addresses).
  constexpr bool kParity = C::NW == 8;
  uint32_t xoff[kParity ? 2 : C::XL], woff[kParity ? 2 : C::WL];
  int xk[kParity ? 2 : C::XL], wk[kParity ? 2 : C::WL];
#pragma unroll
  for (int i = 0; i < (kParity ? 2 : C::XL); ++i) {
    const int row = (wave * C::XL + i) * 8 + lrow;
    xk[i] = 8 * dswz(row, lpos);
    xoff[i] = (uint32_t)(row * K + xk[i]) * 2u;
  }
#pragma unroll
  for (int i = 0; i < (kParity ? 2 : C::WL); ++i) {
    const int row = (wave * C::WL + i) * 8 + lrow;
    wk[i] = 8 * dswz(row, lpos);
    woff[i] = (uint32_t)((row - wrow_shift) * K + wk[i]) * 2u;
  }
  const uint32_t rows16 = (uint32_t)K * 32u;   // bytes of 16 rows
  // Load i at k0: byte offset from the resource base, or past the bound when
  // its k is past K.
  auto load_x = [&](int k0, int stage) {
    TPL_LDS uint16_t* base = (TPL_LDS uint16_t*)lds + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::XL; ++i) {
      const int e = kParity ? (i & 1) : i;
      const uint32_t rows = kParity ? (uint32_t)(i >> 1) * rows16 : 0u;
      const uint32_t off = (k0 + xk[e] < K) ? xoff[e] + rows + (uint32_t)k0 * 2u : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (TPL_LDS void*)(base + (wave * C::XL + i) * 8 * C::BK), 16, off, 0, 0, 0);
    }
  };
  auto load_w = [&](int k0, int stage) {
    TPL_LDS uint16_t* base = (TPL_LDS uint16_t*)lds + stage * C::STAGE + C::BM * C::BK;
#pragma unroll
    for (int i = 0; i < C::WL; ++i) {
      const int e = kParity ? (i & 1) : i;
      const uint32_t rows = kParity ? (uint32_t)(i >> 1) * rows16 : 0u;
      const uint32_t off = (k0 + wk[e] < K) ? woff[e] + rows + (uint32_t)k0 * 2u : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (TPL_LDS void*)(base + (wave * C::WL + i) * 8 * C::BK), 16, off, 0, 0, 0);
    }
  };

  f32x16 acc[C::FA][C::FB];
#pragma unroll
  for (int i = 0; i < C::FA; ++i)
#pragma unroll
    for (int j = 0; j < C::FB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragment of sub-step kk: lane reads row (lane & 31) of its 32-row block,
  // 16-byte chunk 2*kk + lane/32.
  const int frow = lane & 31, fh = lane >> 5;
  bf16x8 fa[2][C::FA], fb[2][C::FB];
  // Every fragment row is frow plus a multiple of 16, so the chunk swizzle
  // (row/2) % 8 is the lane's (frow/2) % 8 for all of them: one chunk offset
  // per sub-step addresses every read (8-wave tiles; the 4-wave tile keeps
  // per-row addressing).
  static_assert(C::TM % 16 == 0 && C::TN % 32 == 0 && C::BN % 32 == 0 && C::BM % 16 == 0,
                "fragment rows keep the lane's swizzle");
  const int fsw = (frow >> 1) & 7;
  const int a_row0 = kPairInWave ? wn * (C::TN / 2) : wn * C::TN;
  const int b_row0 = wm * C::TM;
  auto read_frags = [&](int stage, int kk, int buf) {
    const int kc = 2 * kk + fh;
    if constexpr (kParity) {
      const char* sbase = reinterpret_cast<const char*>(lds) + stage * C::STAGE * 2;
      const char* abase = sbase + (C::BM + a_row0 + frow) * C::BK * 2;
      const char* bbase = sbase + (b_row0 + frow) * C::BK * 2;
      const int cofs = (kc ^ fsw) * 16;
#pragma unroll
      for (int i = 0; i < C::FA; ++i) {
        // In-wave SwiGLU pairing: fragments i < FA/2 are gate rows and i + FA/2
        // the up rows of the same outputs, so the epilogue pairs them in registers.
        const int r = !kPairInWave ? i * 32 : i < C::FA / 2 ? i * 32 : C::BN / 2 + (i - C::FA / 2) * 32;
        fa[buf][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(abase + r * C::BK * 2 + cofs));
      }
#pragma unroll
      for (int j = 0; j < C::FB; ++j)
        fb[buf][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(bbase + j * 32 * C::BK * 2 + cofs));
    } else {
      const uint16_t* base = lds + stage * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::FA; ++i) {
        const int row = !kPairInWave ? wn * C::TN + i * 32 + frow
                        : i < C::FA / 2 ? wn * (C::TN / 2) + i * 32 + frow
                                        : C::BN / 2 + wn * (C::TN / 2) + (i - C::FA / 2) * 32 + frow;
        fa[buf][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            base + C::BM * C::BK + row * C::BK + dswz(row, kc) * 8));
      }
#pragma unroll
      for (int j = 0; j < C::FB; ++j) {
        const int row = wm * C::TM + j * 32 + frow;
        fb[buf][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(base + row * C::BK + dswz(row, kc) * 8));
      }
    }
  };
  auto mfmas = [&](int buf, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < C::FB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };
  auto pin = []() { __builtin_amdgcn_sched_barrier(0); };

  const int nk = (K + C::BK - 1) / C::BK;
  // Ping-pong loop (8 waves, 256 rows, at most 256 columns; wider tiles have
  // no registers for a whole stage of fragments): each wave reads all of a
  // stage's fragments in one phase and issues the stage's MFMAs in the next,
  // with a workgroup barrier after each phase.  Waves 4-7, the second wave of
  // each SIMD, pass one extra barrier first (waves 0-3 one at the end), so
  // they run one phase later: one wave's MFMAs run while the other wave of
  // its SIMD reads fragments and issues tile loads.  At the end of its read
  // phase, each wave of 0-3 loads its share of the next stage's X tile (into
  // the slot the stage before left) and each wave of 4-7 its share of the W
  // tile two stages ahead (into the slot it has just read); each group waits
  // for its own loads before the barrier that precedes the first read of
  // them.  The accumulation order is the in-step loop's, so the results are
  // the same.
  constexpr bool kPP = C::NW == 8 && C::BM == 256 && C::BN <= 256;
  if constexpr (kPP) {
    const int lag = wave >> 2, q = wave & 3;
    constexpr int LX = C::BM / 32, LW = C::BN / 32;   // loads per wave per stage (rows / 4 waves / 8 rows)
    const int L8 = lag ? LW : LX;
    uint32_t o8[2];
    int k8[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = (q * L8 + e) * 8 + lrow;
      k8[e] = 8 * dswz(row, lpos);
      o8[e] = (uint32_t)(row * K + k8[e]) * 2u;
    }
    // Rows of this wave's loads: X rows (q LX + i) * 8 + lrow for waves 0-3,
    // W rows (q LW + i) * 8 + lrow for waves 4-7 (SwiGLU up rows when they
    // lie in [BN/2, BN): the resource then starts at row N + n0).
    const bool up8 = EPI == 1 && q * LW * 8 >= C::BN / 2;
    const uint32_t wrows8 = (uint32_t)min(OUT_BN, N - n0);
    const __amdgpu_buffer_rsrc_t wr8 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (int64_t)(up8 ? N + n0 : n0) * K), 0, wrows8 * (uint32_t)K * 2u, 0x00020000);
    const uint32_t shift8 = up8 ? (uint32_t)(C::BN / 2) * (uint32_t)K * 2u : 0u;
    auto load8 = [&](int k0, int stage) {
      TPL_LDS uint16_t* base = (TPL_LDS uint16_t*)lds + stage * C::STAGE;
      if (lag) {
#pragma unroll
        for (int i = 0; i < LW; ++i) {
          const int e = i & 1;
          const uint32_t off = (k0 + k8[e] < K) ? o8[e] + (uint32_t)(i >> 1) * rows16 + (uint32_t)k0 * 2u - shift8
                                                : 0x80000000u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              wr8, (TPL_LDS void*)(base + C::BM * C::BK + (q * LW + i) * 8 * C::BK), 16, off, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < LX; ++i) {
          const int e = i & 1;
          const uint32_t off = (k0 + k8[e] < K) ? o8[e] + (uint32_t)(i >> 1) * rows16 + (uint32_t)k0 * 2u
                                                : 0x80000000u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (TPL_LDS void*)(base + (q * LX + i) * 8 * C::BK), 16, off, 0, 0, 0);
        }
      }
    };
    bf16x8 fa4[4][C::FA], fb4[4][C::FB];
    auto read4 = [&](int stage) {
      const char* sbase = reinterpret_cast<const char*>(lds) + stage * C::STAGE * 2;
      const char* abase = sbase + (C::BM + a_row0 + frow) * C::BK * 2;
      const char* bbase = sbase + (b_row0 + frow) * C::BK * 2;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int cofs = ((2 * kk + fh) ^ fsw) * 16;
#pragma unroll
        for (int i = 0; i < C::FA; ++i) {
          const int r = !kPairInWave ? i * 32 : i < C::FA / 2 ? i * 32 : C::BN / 2 + (i - C::FA / 2) * 32;
          fa4[kk][i] = as_bf16x8(*reinterpret_cast<const u32x4*>(abase + r * C::BK * 2 + cofs));
        }
#pragma unroll
        for (int j = 0; j < C::FB; ++j)
          fb4[kk][j] = as_bf16x8(*reinterpret_cast<const u32x4*>(bbase + j * 32 * C::BK * 2 + cofs));
      }
    };
    auto phase_barrier = [&]() {
      pin();
      __builtin_amdgcn_s_barrier();
      pin();
    };
    load8(0, 0);
    if (lag && nk > 1) load8(C::BK, 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (lag) phase_barrier();
    for (int t = 0; t < nk; ++t) {
      const int st = t & 1;
      // read phase: after their reads of stage t, waves 0-3 load X of stage
      // t+1 (into the slot stage t-1 left, read by waves 4-7 one phase ago)
      // and waves 4-7 load W of stage t+2 (into the slot of stage t, read by
      // waves 0-3 one phase ago)
      read4(st);
      if (lag == 0 && t + 1 < nk) load8((t + 1) * C::BK, st ^ 1);
      if (lag) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this stage's fragments are in registers
        __builtin_amdgcn_s_waitcnt(kWaitVm0); // W of stage t+1 has landed
        if (t + 2 < nk) load8((t + 2) * C::BK, st);
      }
      phase_barrier();
      // MFMA phase
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < C::FA; ++i)
#pragma unroll
          for (int j = 0; j < C::FB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa4[kk][i], fb4[kk][j], acc[i][j], 0, 0, 0);
      if (lag == 0) __builtin_amdgcn_s_waitcnt(kWaitVm0);   // X of stage t+1 has landed
      phase_barrier();
    }
    if (!lag) phase_barrier();
  } else {
  load_x(0, 0);
  load_w(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  read_frags(0, 0, 0);
  pin();
  for (int t = 0; t < nk; ++t) {
    const int st = t & 1;
    const bool more = t + 1 < nk;
    // sub-step 0 (stage st+1 was last read before the previous barrier)
    read_frags(st, 1, 1);
    if (more) load_x((t + 1) * C::BK, st ^ 1);
    mfmas(0, 0, C::FA);
    pin();
    // sub-step 1
    read_frags(st, 2, 0);
    if (more) load_w((t + 1) * C::BK, st ^ 1);
    mfmas(1, 0, C::FA);
    pin();
    // sub-step 2
    read_frags(st, 3, 1);
    mfmas(0, 0, C::FA);
    pin();
    // sub-step 3, split around the barrier that publishes the next stage
    mfmas(1, 0, C::FA / 2);
    pin();
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_s_barrier();
    pin();
    if (more) read_frags(st ^ 1, 0, 0);
    mfmas(1, C::FA / 2, C::FA);
    pin();
  }
  }

  // Epilogue.  acc[i][j] lane holds token m = wm*TM + 32j + (lane&31) and
  // features n = wn*TN + 32i + 8*(r/4) + 4*(lane/32) + r%4, r = 0..15.
  // Full tiles of the ping-pong loop store through LDS, whose stages are free
  // once the loop has passed its last barrier: a direct store from the
  // accumulator layout writes 32 rows x 32 bytes per instruction, so the L2
  // takes four partial writes per 128-byte line, and at the end of a round the
  // 32 CUs of an XCD store at once.  Staged, every store instruction writes
  // whole lines (8 rows x 128 bytes for float32 from each wave's slab; whole
  // output rows from the workgroup's bf16 tile).  Measured, same bits: o_proj
  // 213.7 -> 208.3 us, down 689 -> 680, fc2 246 -> 240, the plain gate|up
  // 1388 -> 1347 us; the 4096-token prefill step 2.916 -> 2.897 ms.
  if constexpr (kPP && OUT_F32 && EPI == 0 && VEC_OUT) {
    static_assert(C::NW * C::TM * 32 * 4 <= 2 * C::STAGE * 2, "epilogue slabs fit in the stages");
    if (m0 + C::BM <= M && n0 + C::BN <= N) {
      float* sl = reinterpret_cast<float*>(lds) + wave * (C::TM * 32);
#pragma unroll
      for (int i = 0; i < C::FA; ++i) {
#pragma unroll
        for (int j = 0; j < C::FB; ++j) {
          const int row = 32 * j + frow;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = (2 * q + fh) ^ (row & 7);
            *reinterpret_cast<f32x4*>(sl + row * 32 + ch * 4) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          }
        }
        const int c = lane & 7;
#pragma unroll
        for (int s8 = 0; s8 < C::TM / 8; ++s8) {
          const int row = 8 * s8 + (lane >> 3);
          const f32x4 v = *reinterpret_cast<const f32x4*>(sl + row * 32 + ((c ^ (row & 7)) * 4));
          const int m = m0 + wm * C::TM + row;
          const int n = n0 + wn * C::TN + 32 * i + 4 * c;
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Y) + (int64_t)m * N + n) = v;
        }
      }
      return;
    }
  }
  if constexpr (kPP && !OUT_F32 && VEC_OUT && (kPairInWave || EPI != 1)) {
    constexpr int OB = kPairInWave ? C::BN / 2 : C::BN;   // outputs per tile row
    constexpr int CPR = OB / 8;                           // 16-byte chunks per row
    constexpr int NI = kPairInWave ? C::FA / 2 : C::FA;
    constexpr int WO = kPairInWave ? C::TN / 2 : C::TN;   // outputs per wave row
    static_assert(C::BM * OB * 2 <= 2 * C::STAGE * 2, "output tile fits in the stages");
    static_assert(CPR % 8 == 0 && (C::BM * CPR) % C::NT == 0, "swizzle groups, store rounds");
    if (m0 + C::BM <= M && n0 + OB <= N) {
      uint16_t* ot = lds;   // [BM][OB]; 16-byte chunk c of row r at c ^ (r & 7)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int j = 0; j < C::FB; ++j) {
          const int row = wm * C::TM + 32 * j + frow;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (kPairInWave)
                v[e] = act_fn<TP_ACT_SWIGLU>(acc[i][j][4 * q + e], acc[i + C::FA / 2][j][4 * q + e]);
              else if constexpr (EPI == 2)
                v[e] = act_fn<TP_ACT_GELU>(acc[i][j][4 * q + e], 0.f);
              else
                v[e] = acc[i][j][4 * q + e];
            }
            const int col = wn * WO + 32 * i + 8 * q + 4 * fh;
            const int ch = (col >> 3) ^ (row & 7);
            *reinterpret_cast<u32x2*>(ot + row * OB + ch * 8 + (col & 7)) =
                u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < C::BM * CPR / C::NT; ++it) {
        const int idx = it * C::NT + threadIdx.x;
        const int row = idx / CPR, c = idx % CPR;
        const u32x4 val = *reinterpret_cast<const u32x4*>(ot + row * OB + (c ^ (row & 7)) * 8);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(Y) + (int64_t)(m0 + row) * N + n0 + c * 8) = val;
      }
      return;
    }
  }
  // The in-step loop's 8-wave tiles (256x320): the bf16 output tile is larger
  // than the LDS, so it goes through in row groups of whole waves.
  if constexpr (!kPP && C::NW == 8 && !OUT_F32 && VEC_OUT && EPI != 1) {
    constexpr int OB = C::BN, CPR = OB / 8;
    constexpr int H = (C::BM * OB * 2 + 2 * C::STAGE * 2 - 1) / (2 * C::STAGE * 2);   // row groups
    constexpr int RG = C::BM / H;
    static_assert(C::BM % H == 0 && RG % C::TM == 0 && CPR % 8 == 0 && (RG * CPR) % C::NT == 0,
                  "row groups of whole waves, swizzle groups, store rounds");
    if (m0 + C::BM <= M && n0 + OB <= N) {
      uint16_t* ot = lds;   // [RG][OB]; 16-byte chunk c of row r at c ^ (r & 7)
#pragma unroll
      for (int hg = 0; hg < H; ++hg) {
        if ((wm * C::TM) / RG == hg) {
#pragma unroll
          for (int i = 0; i < C::FA; ++i) {
#pragma unroll
            for (int j = 0; j < C::FB; ++j) {
              const int row = wm * C::TM + 32 * j + frow - hg * RG;
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  if constexpr (EPI == 2) v[e] = act_fn<TP_ACT_GELU>(acc[i][j][4 * q + e], 0.f);
                  else v[e] = acc[i][j][4 * q + e];
                }
                const int col = wn * C::TN + 32 * i + 8 * q + 4 * fh;
                const int ch = (col >> 3) ^ (row & 7);
                *reinterpret_cast<u32x2*>(ot + row * OB + ch * 8 + (col & 7)) =
                    u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
              }
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < RG * CPR / C::NT; ++it) {
          const int idx = it * C::NT + threadIdx.x;
          const int row = idx / CPR, c = idx % CPR;
          const u32x4 val = *reinterpret_cast<const u32x4*>(ot + row * OB + (c ^ (row & 7)) * 8);
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(Y) + (int64_t)(m0 + hg * RG + row) * N + n0 +
                                    c * 8) = val;
        }
        if (hg + 1 < H) __syncthreads();
      }
      return;
    }
  }
  if constexpr (kPairInWave) {
    // acc[i] holds gate sums and acc[i + FA/2] the up sums of the same outputs
    // n = n0 + wn*TN/2 + 32i + 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
    for (int i = 0; i < C::FA / 2; ++i) {
#pragma unroll
      for (int j = 0; j < C::FB; ++j) {
        const int m = m0 + wm * C::TM + j * 32 + frow;
        if (m >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + wn * (C::TN / 2) + i * 32 + 8 * q + 4 * fh;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = act_fn<TP_ACT_SWIGLU>(acc[i][j][4 * q + e], acc[i + C::FA / 2][j][4 * q + e]);
          }
          if (VEC_OUT && n + 3 < N) {
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(Y) + (int64_t)m * N + n) =
                u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n + e] = (uint16_t)f2bf_bits(v[e]);
          }
        }
      }
    }
    return;
  } else if constexpr (EPI == 1) {
    // Up-row waves (wn >= WN/2) park their accumulators in LDS; the gate-row
    // wave with the same lane layout (wn - WN/2) combines them.
    constexpr int PER_WAVE = C::FA * C::FB * 16 * 64;   // floats
    float* xch = reinterpret_cast<float*>(lds);
    static_assert((C::NW / 2) * PER_WAVE * 4 <= 2 * C::STAGE * 2, "exchange fits in the stages");
    __syncthreads();
    const int pair = wm * (C::WN / 2) + (wn % (C::WN / 2));
    if (wn >= C::WN / 2) {
#pragma unroll
      for (int i = 0; i < C::FA; ++i)
#pragma unroll
        for (int j = 0; j < C::FB; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            xch[pair * PER_WAVE + ((i * C::FB + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if (wn < C::WN / 2) {
#pragma unroll
      for (int i = 0; i < C::FA; ++i) {
#pragma unroll
        for (int j = 0; j < C::FB; ++j) {
          const int m = m0 + wm * C::TM + j * 32 + frow;
          if (m >= M) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * C::TN + i * 32 + 8 * q + 4 * fh;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = act_fn<TP_ACT_SWIGLU>(
                  acc[i][j][4 * q + e], xch[pair * PER_WAVE + ((i * C::FB + j) * 16 + 4 * q + e) * 64 + lane]);
            }
            if (VEC_OUT && n + 3 < N) {
              *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(Y) + (int64_t)m * N + n) =
                  u32x2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n + e] = (uint16_t)f2bf_bits(v[e]);
            }
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::FA; ++i) {
#pragma unroll
    for (int j = 0; j < C::FB; ++j) {
      const int m = m0 + wm * C::TM + j * 32 + frow;
      if (m >= M) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * C::TN + i * 32 + 8 * q + 4 * fh;
        float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
        if constexpr (EPI == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = act_fn<TP_ACT_GELU>(v[e], 0.f);
        }
        if (VEC_OUT && n + 3 < N) {
          if constexpr (OUT_F32) {
            const f32x4 o = {v[0], v[1], v[2], v[3]};
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Y) + (int64_t)m * N + n) = o;
          } else {
            const u32x2 o = {pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(Y) + (int64_t)m * N + n) = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e < N) {
              if constexpr (OUT_F32)
                reinterpret_cast<float*>(Y)[(int64_t)m * N + n + e] = v[e];
              else
                reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n + e] = (uint16_t)f2bf_bits(v[e]);
            }
          }
        }
      }
    }
  }
}

using Dma256 = DmaTile<256, 256, 2, 4>;   // 8 waves, one workgroup per CU
using Dma128 = DmaTile<128, 128, 2, 2>;   // 4 waves, two workgroups per CU
// 256x320: 8 waves of 64x160 (144 KB of LDS for two stages).  For N where
// 256x256 tiles leave a mostly empty last round, e.g. the fused QKV at
// N = 5120: 16 x 16 tiles fill 256 CUs exactly once.
using Dma320 = DmaTile<256, 320, 4, 2>;
// 256x192: 8 waves of 64x96 (112 KB).  For grids that 256x256 tiles fill only
// partly, e.g. a 2048 x 6144 output: 8 x 32 tiles fill 256 CUs once where
// 8 x 24 tiles of 256x256 would leave a quarter of them idle.
using Dma192 = DmaTile<256, 192, 4, 2>;

template <class C, int EPI>
static tp_status launch_dma(const void* x, const void* w, void* y, int M, int N, int K,
                            bool out_f32, bool vec_out, hipStream_t s) {
  constexpr int OUT_BN = EPI == 1 ? C::BN / 2 : C::BN;
  const int ntile = ((M + C::BM - 1) / C::BM) * ((N + OUT_BN - 1) / OUT_BN);
  dim3 grid(ntile), block(C::NT);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
  if constexpr (EPI == 0) {
    if (out_f32) {
      if (vec_out) hipLaunchKernelGGL((gemm_bf16_dma_kernel<C, true, true, 0>), grid, block, 0, s, X, Wp, y, M, N, K);
      else hipLaunchKernelGGL((gemm_bf16_dma_kernel<C, true, false, 0>), grid, block, 0, s, X, Wp, y, M, N, K);
    } else {
      if (vec_out) hipLaunchKernelGGL((gemm_bf16_dma_kernel<C, false, true, 0>), grid, block, 0, s, X, Wp, y, M, N, K);
      else hipLaunchKernelGGL((gemm_bf16_dma_kernel<C, false, false, 0>), grid, block, 0, s, X, Wp, y, M, N, K);
    }
  } else {
    if (vec_out) hipLaunchKernelGGL((gemm_bf16_dma_kernel<C, false, true, EPI>), grid, block, 0, s, X, Wp, y, M, N, K);
    else hipLaunchKernelGGL((gemm_bf16_dma_kernel<C, false, false, EPI>), grid, block, 0, s, X, Wp, y, M, N, K);
  }
  TPL_LAUNCH_CHECK("gemm_bf16_dma");
  return TP_OK;
}

// 0 = 256x256 (8 waves), 1 = 128x128 (4 waves), 2 = 256x320 (8 waves),
// 3 = 256x192 (8 waves).
// Estimated time = full-chip rounds x round time in units of a 256x256 round:
// a round of 128x128 tiles (two per CU) does half that work at ~85% of its
// efficiency, a round of 256x320 tiles does 1.25x the work at the same
// efficiency, a round of 256x192 tiles takes 0.85 (measured on gate|up-, qkv-,
// o_proj-, down- and GELU-FFN-shaped problems).
// `wide` allows the 256x320 tile (its epilogue has no room for the SwiGLU
// exchange).
int gemm_dma_pick_tile(int M, int N, bool wide) {
  const double t256 = ceil((double)((M + 255) / 256) * ((N + 255) / 256) / 256.0);
  const double t128 = ceil((double)((M + 127) / 128) * ((N + 127) / 128) / 512.0) * 0.5 / 0.85;
  const double t320 = wide ? ceil((double)((M + 255) / 256) * ((N + 319) / 320) / 256.0) * 1.25 : 1e30;
  const double t192 = ceil((double)((M + 255) / 256) * ((N + 191) / 192) / 256.0) * 0.85;
  if (t320 < t256 && t320 < t128 && t320 < t192) return 2;
  if (t192 < t256 && t192 < t128) return 3;
  return t128 < t256 ? 1 : 0;
}

tp_status gemm_bf16_dma(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                        bool out_f32, bool vec_out, hipStream_t s, int force_tile) {
  const int pick = force_tile >= 0 ? force_tile : gemm_dma_pick_tile((int)M, (int)N, true);
  if (pick == 0) return launch_dma<Dma256, 0>(x, w, y, (int)M, (int)N, (int)K, out_f32, vec_out, s);
  if (pick == 2) return launch_dma<Dma320, 0>(x, w, y, (int)M, (int)N, (int)K, out_f32, vec_out, s);
  if (pick == 3) return launch_dma<Dma192, 0>(x, w, y, (int)M, (int)N, (int)K, out_f32, vec_out, s);
  return launch_dma<Dma128, 0>(x, w, y, (int)M, (int)N, (int)K, out_f32, vec_out, s);
}

// Column-parallel linear with the rank-local activation fused into the
// epilogue, bf16 output [M, I]: act = TP_ACT_SWIGLU (w is [2I, K], gate rows
// then up rows) or TP_ACT_GELU (w is [I, K]).  Same requirements as above.
tp_status gemm_bf16_dma_act(const void* x, const void* w, void* h, int64_t M, int64_t I, int64_t K,
                            int act, bool vec_out, hipStream_t s) {
  if (act == TP_ACT_SWIGLU) {
    // a paired 256-wide tile yields 128 outputs: pick the tile on the doubled width
    const int pick = gemm_dma_pick_tile((int)M, (int)(2 * I), false);
    if (pick == 0) return launch_dma<Dma256, 1>(x, w, h, (int)M, (int)I, (int)K, false, vec_out, s);
    if (pick == 3) return launch_dma<Dma192, 1>(x, w, h, (int)M, (int)I, (int)K, false, vec_out, s);
    return launch_dma<Dma128, 1>(x, w, h, (int)M, (int)I, (int)K, false, vec_out, s);
  }
  const int pick = gemm_dma_pick_tile((int)M, (int)I, true);
  if (pick == 0) return launch_dma<Dma256, 2>(x, w, h, (int)M, (int)I, (int)K, false, vec_out, s);
  if (pick == 2) return launch_dma<Dma320, 2>(x, w, h, (int)M, (int)I, (int)K, false, vec_out, s);
  if (pick == 3) return launch_dma<Dma192, 2>(x, w, h, (int)M, (int)I, (int)K, false, vec_out, s);
  return launch_dma<Dma128, 2>(x, w, h, (int)M, (int)I, (int)K, false, vec_out, s);
}

}  // namespace tpl
