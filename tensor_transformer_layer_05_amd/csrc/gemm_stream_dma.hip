// Decode bf16 linear for 4..64 tokens through LDS: weight streaming.
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]
//
// At decode the weight matrix is read once per call and dominates the HBM
// bytes, but with several tokens the token rows are re-read from L2 by every
// workgroup and make up most of a workgroup's load traffic.  Loads whose 64
// lanes each take 16 bytes of a different row (the MFMA operand layout) use
// only half of every 128-byte line they touch, and measured per-CU load
// throughput is then what bounds these shapes.  So both operands go through
// LDS:
//   * a workgroup owns up to RT tiles of 16 consecutive weight rows (fewer
//     rows when that fills more CUs), MT tiles of 16 tokens and all of K; its
//     WAVES waves split K into contiguous 128-k-aligned ranges;
//   * every wave streams its weight rows AND the token rows of its k range
//     through a private S-stage LDS ring with buffer_load_dwordx4 ... lds: one
//     wave-level load writes 4 rows x 256 contiguous bytes (two whole lines
//     per row), for weights and tokens alike;
//   * weight loads are non-temporal (each weight byte is read once per call);
//     token loads keep the default policy, since every workgroup re-reads
//     the token rows from L2;
//   * 256-byte LDS rows keep 16-byte chunk c of row r at c ^ (r % 16), so the
//     fragment reads of v_mfma_f32_16x16x32_bf16 (16 rows x one chunk per
//     quarter-wave) hit 16 distinct bank groups;
//   * out-of-range rows, tokens and k read as zero through the buffer bounds,
//     so the loop is branch-free and waits for exactly the chunk it uses;
//   * no workgroup barrier in the loop (the rings are per wave); the WAVES
//     partial tiles are summed in LDS in wave order at the end, so the result
//     depends only on WAVES, the k ranges and (with several token tiles) the
//     workgroup id that sets the chunk order, not on timing or S.
#include "common.h"

namespace tpl {

namespace {

constexpr uint32_t kSOob = 0x80000000u;   // offset past any buffer bound -> reads 0
#define TPL_LDS __attribute__((address_space(3)))

// s_waitcnt with only vmcnt constrained (gfx9 encoding)
#define TPL_VMCNT(n) ((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)
#define TPL_LGKM0 0xC07F

}  // namespace

// EPI: 0 plain, 1 SwiGLU (RT = 2: row tile 0 = gate rows n0.., tile 1 = the
// matching up rows N + n0.. of a [2N, K] weight; output [M, N]), 2 GELU.  The
// fused epilogues apply the activation to the float32 sums; only its result is
// rounded to bf16.
template <int WAVES, int MT, int RT, int S, bool OUT_F32, int EPI, int TG>
__global__ __launch_bounds__(WAVES * 64) void gemm_stream_dma_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int M, int N, int K, int kw, int rows_wg) {
  static_assert(EPI != 1 || RT == 2, "SwiGLU pairs a gate and an up row tile");
  static_assert(RT == 1 || RT == 2, "one or two row tiles");
  constexpr int WROWS = 16 * RT, XROWS = 16 * MT, ROWS = WROWS + XROWS;
  constexpr int STAGE = ROWS * 128;                   // bf16 elements per stage (256-byte rows)
  constexpr int RING = S * STAGE;                     // per wave
  static_assert(TG >= 1 && TG <= 4 * MT, "token row groups of 4 that are loaded");
  constexpr int DPC = WROWS / 4 + TG;                 // DMA instructions per chunk
  constexpr int RED = WAVES * RT * MT * 256;          // floats for the final reduction
  constexpr int LDS_E = (WAVES * RING * 2 > RED * 4) ? WAVES * RING : RED * 2;
  static_assert(S >= 3 && (S - 2) * DPC <= 63, "ring depth within the vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_E];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this workgroup's output rows n0 .. n0 + nrows - 1 (rows_wg <= 16 RT, or
  // <= 16 gate|up pairs): fewer than a full tile when that fills more CUs
  const int n0 = blockIdx.x * rows_wg;
  const int nrows = min(rows_wg, N - n0);
  const int g = lane >> 4;         // k-group of this lane inside a 32-k step
  const int i16 = lane & 15;       // weight row / token inside a 16-tile
  // blockIdx.y selects this workgroup's MT token tiles; the rest of the kernel
  // sees them as tokens 0 .. M-1 of X and Y.
  const int m0 = blockIdx.y * XROWS;
  X += (int64_t)m0 * K;
  Y = OUT_F32 ? (void*)((float*)Y + (int64_t)m0 * N) : (void*)((uint16_t*)Y + (int64_t)m0 * N);
  M = min(M - m0, XROWS);

  // one resource per weight row tile, based at its first row and bounded to its valid rows
  __amdgpu_buffer_rsrc_t wr[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int base = EPI == 1 ? (r == 0 ? n0 : N + n0) : n0 + 16 * r;
    const int rows = EPI == 1 ? nrows : max(0, min(16, nrows - 16 * r));
    wr[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)base * K), 0,
                                              (uint32_t)rows * (uint32_t)K * 2u, 0x00020000);
  }
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)X, 0, (uint32_t)M * (uint32_t)K * 2u, 0x00020000);

  const int kb = wave * kw;
  const int ke = min(K, kb + kw);
  const int nc = ke > kb ? (ke - kb + 127) / 128 : 0;   // 128-k chunks of this wave

  // DMA lane mapping: load d of a chunk covers stage rows 4d .. 4d+3 (weight
  // rows first, then token rows); lane -> row 4d + lane/16, LDS chunk position
  // lane%16 holding logical chunk (lane%16) ^ (row % 16).
  const int drow = lane >> 4, dpos = lane & 15;
  TPL_LDS uint16_t* ring = (TPL_LDS uint16_t*)lds + wave * RING;
  // With more than one 16-token tile, token rows are most of a workgroup's
  // loads, and workgroups that walk their k ranges in step all read the same
  // token lines of L2 at once.  So workgroups on one XCD (every 8th id) start
  // at different chunks and wrap around (gate|up + SwiGLU [7168, 8192] at 64
  // tokens: 34.8 -> 31.9 us, at 48 tokens 32.1 -> 28.8 us; at 8 tokens the
  // rotation measured 1% slower and is off).  The order of a wave's chunk sums
  // then depends on its workgroup id, deterministically.
  const int rot = (MT > 1 || gridDim.y > 1) && nc > 0 ? (int)((blockIdx.x >> 3) % (unsigned)nc) : 0;
  auto issue = [&](int c) {   // chunk c of this wave into stage c % S
    const int k0 = kb + (c < nc ? (c + rot) % nc : c) * 128;
    TPL_LDS uint16_t* dst = ring + (c % S) * STAGE;
#pragma unroll
    for (int d = 0; d < DPC; ++d) {
      const int row = 4 * d + drow;
      const int k = k0 + 8 * (dpos ^ (row & 15));
      if (d < WROWS / 4) {       // weight rows: tile d / 4, row row % 16 in it
        const __amdgpu_buffer_rsrc_t rs = d < 4 ? wr[0] : wr[RT - 1];
        const uint32_t off = k < ke ? (uint32_t)((row & 15) * K + k) * 2u : kSOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (TPL_LDS void*)(dst + d * 4 * 128), 16, off, 0, 0, kLoadStream);
      } else {                   // token rows
        const uint32_t off = k < ke ? (uint32_t)((row - WROWS) * K + k) * 2u : kSOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (TPL_LDS void*)(dst + d * 4 * 128), 16, off, 0, 0, 0);
      }
    }
  };

  f32x4 acc[RT][MT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Memory operations complete in issue order.  Before step c the chunks
  // c .. c+S-2 are in flight (prologue: 0 .. S-2; each step adds c+S-1), so
  // waiting until at most (S-2) chunks' loads are pending lands chunk c.  The
  // step copies its fragments to registers, then refills the stage of chunk
  // c-1, read by the previous step.  Chunks past the end read as zero.
  auto step = [&](int c) {
    __builtin_amdgcn_s_waitcnt(TPL_VMCNT((S - 2) * DPC));
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* st = lds + wave * RING + (c % S) * STAGE;
    u32x4 wv[RT][4], xv[MT][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int row = r * 16 + i16;
        wv[r][q] = *reinterpret_cast<const u32x4*>(st + row * 128 + ((4 * q + g) ^ (row & 15)) * 8);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = WROWS + t * 16 + i16;
        xv[t][q] = *reinterpret_cast<const u32x4*>(st + row * 128 + ((4 * q + g) ^ (row & 15)) * 8);
      }
    }
    __builtin_amdgcn_s_waitcnt(TPL_LGKM0);
    __builtin_amdgcn_sched_barrier(0);
    issue(c + S - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[r][q]), as_bf16x8(xv[t][q]),
                                                              acc[r][t], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  if constexpr (TG < 4 * MT) {   // zero the token rows that are never loaded, in every stage
    constexpr int ZROWS = XROWS - 4 * TG;
    for (int e = lane; e < S * ZROWS * 16; e += 64) {
      const int st = e / (ZROWS * 16), rr = (e / 16) % ZROWS, ch = e % 16;
      *reinterpret_cast<u32x4*>(lds + wave * RING + st * STAGE + (WROWS + 4 * TG + rr) * 128 + ch * 8) =
          u32x4{0u, 0u, 0u, 0u};
    }
  }
  if (nc > 0) {
#pragma unroll
    for (int c = 0; c < S - 1; ++c) issue(c);
    __builtin_amdgcn_sched_barrier(0);
    for (int c = 0; c < nc; ++c) step(c);
  }
  // Drain the trailing (out-of-range) loads before the LDS is reused.
  __builtin_amdgcn_s_waitcnt(TPL_VMCNT(0));
  __syncthreads();

  // 16x16 accumulator layout: lane holds column (token) lane & 15 and rows
  // (lane >> 4) * 4 + e.  Park every wave's partial in LDS, sum in wave order.
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(((wave * RT + r) * MT + t) * 64 + lane) * 4 + e] = acc[r][t][e];
  __syncthreads();

  constexpr int PER = RT * MT * 256;
  if constexpr (EPI == 1) {
    for (int v = threadIdx.x; v < MT * 256; v += WAVES * 64) {
      float sg = 0.f, su = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) { sg += red[w * PER + v]; su += red[w * PER + MT * 256 + v]; }
      const int t = v / 256, l = (v >> 2) & 63, e = v & 3;
      const int m = t * 16 + (l & 15);
      const int nl = (l >> 4) * 4 + e, n = n0 + nl;
      if (m < M && nl < nrows)
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = (uint16_t)f2bf_bits(
            act_fn<TP_ACT_SWIGLU>(sg, su));
    }
    return;
  }
  for (int v = threadIdx.x; v < PER; v += WAVES * 64) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[w * PER + v];
    const int rt = v / (MT * 256), t = (v / 256) % MT, l = (v >> 2) & 63, e = v & 3;
    const int m = t * 16 + (l & 15);
    const int nl = rt * 16 + (l >> 4) * 4 + e, n = n0 + nl;
    if (m < M && nl < nrows) {
      if constexpr (EPI == 2)
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] =
            (uint16_t)f2bf_bits(act_fn<TP_ACT_GELU>(s, 0.f));
      else if constexpr (OUT_F32)
        reinterpret_cast<float*>(Y)[(int64_t)m * N + n] = s;
      else
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = (uint16_t)f2bf_bits(s);
    }
  }
}

static int stream_dma_kw(int64_t K, int waves) {
  int kw = (int)((K + waves - 1) / waves);
  return (kw + 127) & ~127;
}

constexpr int64_t kStreamCUs = 256;   // compute units of an MI355X

// Output rows per workgroup: a full tile, or, when full tiles cover half the
// CUs or more but not all, the fewest rows that give about one workgroup per
// CU (rows past them read as zero through the buffer bound and are not
// stored; the K split does not change).  Every workgroup
// streams all of its token rows, so thinner tiles re-read the activations:
// below half the CUs that costs more than the idle CUs (SwiGLU on a [2048,
// 4096] weight, 32 tokens: 8.8 -> 9.0 us).  Kernel trace: gate|up SwiGLU on
// [7168, 8192], 64 tokens 36.8 -> 34.2 us, 48 tokens 33.4 -> 30.4 us.
static int stream_dma_rows(int64_t nout, int out_rows, int ty) {
  const int64_t tiles = (nout + out_rows - 1) / out_rows;
  if (tiles * ty >= kStreamCUs || 2 * tiles * ty < kStreamCUs) return out_rows;
  const int64_t per = kStreamCUs / ty;   // workgroups per token group
  return (int)((nout + per - 1) / per);
}

// One workgroup per (rows_wg output features, MT token tiles); the WAVES
// waves split K into 128-aligned ranges of stream_dma_kw(K, WAVES).
template <int WAVES, int MT, int RT, int S, int EPI = 0, int TG = 4 * MT>
static void launch_stream_dma(const void* x, const void* w, void* y, int M, int N, int K,
                              bool out_f32, hipStream_t s) {
  constexpr int OUT_ROWS = EPI == 1 ? 16 : 16 * RT;
  const int kw = stream_dma_kw(K, WAVES);
  const int ty = (M + 16 * MT - 1) / (16 * MT);
  const int rows_wg = stream_dma_rows(N, OUT_ROWS, ty);
  dim3 grid((N + rows_wg - 1) / rows_wg, ty), block(WAVES * 64);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
  if constexpr (EPI == 0) {
    if (out_f32)
      hipLaunchKernelGGL((gemm_stream_dma_kernel<WAVES, MT, RT, S, true, 0, TG>), grid, block, 0, s, X, Wp, y, M, N, K, kw, rows_wg);
    else
      hipLaunchKernelGGL((gemm_stream_dma_kernel<WAVES, MT, RT, S, false, 0, TG>), grid, block, 0, s, X, Wp, y, M, N, K, kw, rows_wg);
  } else {
    hipLaunchKernelGGL((gemm_stream_dma_kernel<WAVES, MT, RT, S, false, EPI, TG>), grid, block, 0, s, X, Wp, y, M, N, K, kw, rows_wg);
  }
}

// One token tile: load only the 4-row token groups that hold a token (M <=
// 4 TG); the other token rows of the ring are zeroed once per launch.  Rows
// past M read as zero either way, so the sums keep their bits.  Kernel trace,
// 8 tokens: SwiGLU on [2048, 4096] 8.36 -> 7.64 us, [8192, 3584] 12.3 -> 11.9
// us, [1536, 4096] 12.6 -> 12.2 us; the lm_head [16032, 8192] unchanged.
// These shapes are bound by the chain of chunk latencies of each wave (16
// chunks of 128 k per wave at K = 4096, three in flight), not by idle CUs:
// cutting the [1536, 4096] rows to fill all 256 CUs left it at 12.5 us.
template <int WAVES, int RT, int S, int EPI>
static void launch_stream_dma_tg(const void* x, const void* w, void* y, int M, int N, int K,
                                 bool out_f32, hipStream_t s) {
  const int tg = (M + 3) / 4;
  if (tg == 1) launch_stream_dma<WAVES, 1, RT, S, EPI, 1>(x, w, y, M, N, K, out_f32, s);
  else if (tg == 2) launch_stream_dma<WAVES, 1, RT, S, EPI, 2>(x, w, y, M, N, K, out_f32, s);
  else if (tg == 3) launch_stream_dma<WAVES, 1, RT, S, EPI, 3>(x, w, y, M, N, K, out_f32, s);
  else launch_stream_dma<WAVES, 1, RT, S, EPI, 4>(x, w, y, M, N, K, out_f32, s);
}

// Requires 4 <= M <= 64, K % 8 == 0, 16-byte aligned X and W, and M*K and
// 32*K elements addressable with 32-bit byte offsets.
// Waves per workgroup by token tiles (the K split; the fused-activation
// variant uses the same): 2 for 4..16 tokens, 3 for 17..32, 2 for 33..64.
// The sums depend only on the waves and their k ranges, not on how rows and
// tokens are tiled over workgroups.  LDS per workgroup = WAVES x S x (16 RT +
// 16 MT) x 256 bytes <= 144 KB.
tp_status gemm_bf16_stream_dma(const void* x, const void* w, void* y, int64_t M, int64_t N,
                               int64_t K, bool out_f32, hipStream_t s) {
  const int mt = (int)((M + 15) / 16);
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K;
  // 17..32 tokens (three waves and one K split whatever the tiling): the
  // tiling whose grid comes closest to filling the 256 CUs once without a
  // second round.  Short weights take one token tile per workgroup (twice the
  // grid, half the token rows re-read per workgroup), tall ones two row tiles
  // per workgroup (half the grid).  Kernel durations at 32 tokens:
  // [1536, 4096] 10.0 -> 8.1 us and [2048, 4096] 8.8 -> 7.9 us split;
  // [4096, 1024] 5.7 us as is (7.7 split); [7168, 8192] 35.3 -> 26.9 us and
  // [8192, 3584] 16.0 -> 12.7 us with two row tiles.
  const int64_t tiles16 = (N + 15) / 16;
  if (mt == 1) launch_stream_dma_tg<2, 2, 4, 0>(x, w, y, Mi, Ni, Ki, out_f32, s);
  else if (mt == 2 && 2 * tiles16 <= kStreamCUs) launch_stream_dma<3, 1, 1, 4>(x, w, y, Mi, Ni, Ki, out_f32, s);
  else if (mt == 2 && tiles16 > kStreamCUs) launch_stream_dma<3, 2, 2, 3>(x, w, y, Mi, Ni, Ki, out_f32, s);
  else if (mt == 2) launch_stream_dma<3, 2, 1, 4>(x, w, y, Mi, Ni, Ki, out_f32, s);
  else if (mt == 3) launch_stream_dma<2, 3, 2, 3>(x, w, y, Mi, Ni, Ki, out_f32, s);
  else launch_stream_dma<2, 4, 2, 3>(x, w, y, Mi, Ni, Ki, out_f32, s);
  TPL_LAUNCH_CHECK("gemm_bf16_stream_dma");
  return TP_OK;
}

// The same kernel with the rank-local activation fused (bf16 output [M, I])
// on the float32 sums; the waves split K as in the plain call for the same
// token count.
tp_status gemm_bf16_stream_dma_act(const void* x, const void* w, void* h, int64_t M, int64_t I,
                                   int64_t K, int act, hipStream_t s) {
  const int mt = (int)((M + 15) / 16);
  const int Mi = (int)M, Ii = (int)I, Ki = (int)K;
  if (act == TP_ACT_SWIGLU) {
    if (mt == 1) launch_stream_dma_tg<2, 2, 4, 1>(x, w, h, Mi, Ii, Ki, false, s);
    else if (mt == 2) launch_stream_dma<3, 2, 2, 3, 1>(x, w, h, Mi, Ii, Ki, false, s);
    else if (mt == 3) launch_stream_dma<2, 3, 2, 3, 1>(x, w, h, Mi, Ii, Ki, false, s);
    else launch_stream_dma<2, 4, 2, 3, 1>(x, w, h, Mi, Ii, Ki, false, s);
  } else {
    if (mt == 1) launch_stream_dma<2, 1, 1, 4, 2>(x, w, h, Mi, Ii, Ki, false, s);
    else if (mt == 2) launch_stream_dma<3, 2, 1, 4, 2>(x, w, h, Mi, Ii, Ki, false, s);
    else if (mt == 3) launch_stream_dma<2, 3, 2, 3, 2>(x, w, h, Mi, Ii, Ki, false, s);
    else launch_stream_dma<2, 4, 2, 3, 2>(x, w, h, Mi, Ii, Ki, false, s);
  }
  TPL_LAUNCH_CHECK("gemm_bf16_stream_dma_act");
  return TP_OK;
}

}  // namespace tpl
