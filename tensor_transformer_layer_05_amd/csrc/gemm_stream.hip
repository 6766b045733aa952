// Decode bf16 linear for 4..16 tokens on long-K weights (and 1..3 tokens where
// K is too long for the dot-product kernel's token stage): weight streaming.
// The entry points below route 1..3 tokens, and 4..8 on tall weights, to the
// dot-product kernel (gemv_dot.hip) and the rest of 4..64 tokens to the
// LDS-ring kernel (gemm_stream_dma.hip).
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]
//
// At decode the weight matrix is read once per call and dominates the bytes
// (the "mostly GEMV" regime of decode), so the kernel is organised around
// keeping many weight loads in flight:
//   * a workgroup owns up to RT tiles of 16 consecutive weight rows (output
//     features; fewer rows when that fills more CUs) and all of K; its WAVES
//     waves split K into contiguous ranges;
//   * each wave multiplies its (16 RT) x krange slice of W by the matching
//     slice of X^T on v_mfma_f32_16x16x32_bf16 (W rows are the A operand, 16
//     tokens per token tile the B operand); every X fragment feeds RT MFMAs;
//   * all loads are buffer loads whose resource is bounded to the valid rows
//     (tokens), and lanes outside the wave's k range get an offset past the
//     bound, so the loop has no per-lane branches: out-of-range data reads as
//     zero and the compiler can wait for exactly the chunk it is about to use
//     while the next 128-k chunk is in flight;
//   * the WAVES partial tiles are summed in LDS in a fixed order, so the
//     result does not depend on timing.
#include "common.h"

namespace tpl {

namespace {

constexpr uint32_t kOob = 0x80000000u;   // offset past any buffer bound -> reads 0

__device__ __forceinline__ u32x4 bload(const __amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

}  // namespace

// EPI: 0 = plain product; 1 = SwiGLU (RT = 2: row tile 0 = gate rows n0..,
// tile 1 = the matching up rows N + n0.. of a [2N, K] weight; output [M, N]);
// 2 = GELU on each output.  Fused epilogues apply the activation to the
// float32 sums; only the activation's result is rounded to bf16.
template <int WAVES, int MT, int RT, bool OUT_F32, int EPI>
__global__ __launch_bounds__(WAVES * 64) void gemm_stream_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int M, int N, int K, int kw, int rows_wg) {
  __shared__ float red[WAVES * RT * MT * 256];
  static_assert(EPI != 1 || RT == 2, "SwiGLU pairs a gate and an up row tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this workgroup's output rows n0 .. n0 + nrows - 1 (rows_wg <= 16 RT, or
  // <= 16 gate|up pairs): fewer than a full tile when that fills more CUs
  const int n0 = blockIdx.x * rows_wg;
  const int nrows = min(rows_wg, N - n0);
  const int g = lane >> 4;         // k-group of this lane inside a 32-k step
  const int i16 = lane & 15;       // weight row / token inside a 16-tile

  // one resource per row tile, based at its first row and bounded to its valid rows
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

  uint32_t woff[RT], xoff[MT];
#pragma unroll
  for (int r = 0; r < RT; ++r) woff[r] = (uint32_t)(i16 * K) * 2u;
#pragma unroll
  for (int t = 0; t < MT; ++t) xoff[t] = (uint32_t)((t * 16 + i16) * K) * 2u;

  f32x4 acc[RT][MT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wa[RT][4], xa[MT][4], wb[RT][4], xb[MT][4];
  auto load = [&](int c, u32x4 (&wv)[RT][4], u32x4 (&xv)[MT][4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kb + c * 128 + j * 32 + g * 8;
      const bool ok = k < ke;
      const uint32_t kbytes = (uint32_t)k * 2u;
#pragma unroll
      for (int r = 0; r < RT; ++r) wv[r][j] = bload(wr[r], ok ? woff[r] + kbytes : kOob);
#pragma unroll
      for (int t = 0; t < MT; ++t) xv[t][j] = bload(xr, ok ? xoff[t] + kbytes : kOob);
    }
  };
  auto compute = [&](const u32x4 (&wv)[RT][4], const u32x4 (&xv)[MT][4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[r][j]), as_bf16x8(xv[t][j]),
                                                              acc[r][t], 0, 0, 0);
  };

  // Double buffer, unrolled by two so both buffers stay in registers.  The
  // loop body has no early exit: past the last chunk every offset is out of
  // range, so those loads return zeros without memory traffic and their
  // MFMAs add nothing.  This keeps each chunk's loads in the same basic block
  // as, and (through the scheduling barriers) ahead of, the previous chunk's
  // MFMAs.
  if (nc > 0) {
    load(0, wa, xa);
    for (int c = 0; c < nc; c += 2) {
      load(c + 1, wb, xb);
      __builtin_amdgcn_sched_barrier(0);
      compute(wa, xa);
      __builtin_amdgcn_sched_barrier(0);
      load(c + 2, wa, xa);
      __builtin_amdgcn_sched_barrier(0);
      compute(wb, xb);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // 16x16 accumulator layout: lane holds column (token) lane & 15 and rows
  // (lane >> 4) * 4 + e.  Park every wave's partial in LDS, sum in wave order.
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

constexpr int64_t kStreamRegCUs = 256;   // compute units of an MI355X

// Output rows per workgroup: a full tile (16 RT rows, or 16 gate|up pairs),
// or, when full tiles would leave CUs idle, the fewest rows that still give
// one workgroup per CU (rows past them read as zero through the buffer bound
// and are not stored).  The K split does not depend on it, so neither do the
// sums.  Kernel trace, same bits: the decode gate|up + SwiGLU [7168, 8192] on
// 256 workgroups of 14 pairs instead of 224 of 16, 23.6 -> 22.4 us at one
// token and 24.3 -> 22.9 us at eight; a one-token QKV [1536, 4096] on 256
// workgroups of 6 rows instead of 96 of 16, 7.5 -> 5.8 us.
static int stream_rows(int64_t nout, int out_rows) {
  const int64_t tiles = (nout + out_rows - 1) / out_rows;
  if (tiles >= kStreamRegCUs) return out_rows;
  return (int)((nout + kStreamRegCUs - 1) / kStreamRegCUs);
}

template <int WAVES, int MT, int RT, int EPI = 0>
static void launch_stream(const void* x, const void* w, void* y, int M, int N, int K, int kw,
                          bool out_f32, hipStream_t s) {
  constexpr int OUT_ROWS = EPI == 1 ? 16 : 16 * RT;
  const int rows_wg = stream_rows(N, OUT_ROWS);
  dim3 grid((N + rows_wg - 1) / rows_wg), block(WAVES * 64);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
  if constexpr (EPI == 0) {
    if (out_f32)
      hipLaunchKernelGGL((gemm_stream_kernel<WAVES, MT, RT, true, 0>), grid, block, 0, s, X, Wp, y, M, N, K, kw, rows_wg);
    else
      hipLaunchKernelGGL((gemm_stream_kernel<WAVES, MT, RT, false, 0>), grid, block, 0, s, X, Wp, y, M, N, K, kw, rows_wg);
  } else {
    hipLaunchKernelGGL((gemm_stream_kernel<WAVES, MT, RT, false, EPI>), grid, block, 0, s, X, Wp, y, M, N, K, kw, rows_wg);
  }
}

tp_status gemm_bf16_stream_dma(const void* x, const void* w, void* y, int64_t M, int64_t N,
                               int64_t K, bool out_f32, hipStream_t s);
bool gemv_dot_fits(int64_t M, int64_t rows, int64_t K);
tp_status gemv_dot(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                   bool out_f32, hipStream_t s);
tp_status gemv_dot_act(const void* x, const void* w, void* h, int64_t M, int64_t I, int64_t K,
                       int act, hipStream_t s);

// Waves per workgroup of the one-token-tile decode linear on an [N, K]
// weight: 16 waves (1024 threads) when there are few row tiles to spread over
// the chip, fewer until every wave streams >= 512 k (four 128-k chunks, so
// its double-buffered loads have a run to overlap; one token, kernel trace:
// [1536, 4096] 8.22 -> 7.38 us with 8 waves instead of 16, [8192, 3584]
// 14.0 -> 13.9 us with 4 instead of 8).  The fused-activation variant takes
// the same split (hence the same float sums) as the plain linear on the full
// weight.
static int stream_waves(int64_t N, int64_t K) {
  const int64_t nblk = (N + 15) / 16;
  int waves = nblk < 384 ? 16 : 8;
  while (waves > 4 && K / waves < 512) waves >>= 1;
  return waves;
}

static int stream_kw(int64_t K, int waves) {
  int kw = (int)((K + waves - 1) / waves);
  return (kw + 31) & ~31;
}

// The LDS-ring kernel (gemm_stream_dma.hip) serves 4..64 tokens, except that
// up to 16 tokens stay on this kernel for weights of at most 8192 rows on
// which each of its waves streams at least eight 128-k chunks (K / waves >=
// 1024).  That is the decode gate|up weight (7168 x 8192): with SwiGLU fused,
// this kernel's eight waves per workgroup ran 26.1 / 26.3 / 28.4 us at 4 / 8 /
// 16 tokens against the ring's 32.6 / 32.8 / 34.1 us.  On taller weights the
// ring wins (lm_head 16032 x 8192 at 8 and 16 tokens: 58.6 and 59.5 us
// against 61.0 and 75.0), and on shorter K too (8192 x 3584: 13.7 against
// 15.4 us at 8 tokens).  Short weights stay here too: under 64 workgroups of
// 32 rows the ring has little data in flight, while this kernel cuts rows to
// give every CU a workgroup of eight waves (QKV 1536 x 4096 at 4 / 8 / 16
// tokens: 6.3 / 6.9 / 8.2 us against 12.6 / 12.3 / 12.8; 2048 x 4096, 64
// workgroups, stays on the ring at 7.6 / 7.3 against 7.7 / 8.3 us).  The
// choice depends only on (M, N, K) of the weight, and the fused-activation
// call counts the same workgroups (16 gate|up pairs or 32 rows each), so it
// takes the same kernel and K split as the plain call on the same weight, and
// the two give the same bits.
static bool stream_regs(int64_t M, int64_t N, int64_t K) {
  if (M <= 3) return true;
  return M <= 16 && N <= 8192 && (K / stream_waves(N, K) >= 1024 || (N + 31) / 32 < 64);
}

tp_status gemm_bf16_stream(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                           bool out_f32, hipStream_t s) {
  if (gemv_dot_fits(M, N, K)) return gemv_dot(x, w, y, M, N, K, out_f32, s);
  if (!stream_regs(M, N, K)) return gemm_bf16_stream_dma(x, w, y, M, N, K, out_f32, s);
  const int waves = stream_waves(N, K);
  const int kw = stream_kw(K, waves);
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K;
  if (waves == 16) launch_stream<16, 1, 1>(x, w, y, Mi, Ni, Ki, kw, out_f32, s);
  else if (waves == 8) launch_stream<8, 1, 1>(x, w, y, Mi, Ni, Ki, kw, out_f32, s);
  else launch_stream<4, 1, 1>(x, w, y, Mi, Ni, Ki, kw, out_f32, s);
  TPL_LAUNCH_CHECK("gemm_bf16_stream");
  return TP_OK;
}

tp_status gemm_bf16_stream_dma_act(const void* x, const void* w, void* h, int64_t M, int64_t I,
                                   int64_t K, int act, hipStream_t s);

// Decode linear with the rank-local activation fused (bf16 output [M, I]):
// act = TP_ACT_SWIGLU (w is [2I, K], gate rows then up rows) or TP_ACT_GELU
// (w is [I, K]).  Same requirements as gemm_bf16_stream; the K split is the
// one gemm_bf16_stream takes on the same weight, so the results equal the
// plain linear followed by the activation bit for bit.
tp_status gemm_bf16_stream_act(const void* x, const void* w, void* h, int64_t M, int64_t I,
                               int64_t K, int act, hipStream_t s) {
  const int64_t rows = act == TP_ACT_SWIGLU ? 2 * I : I;
  if (gemv_dot_fits(M, rows, K)) return gemv_dot_act(x, w, h, M, I, K, act, s);
  if (!stream_regs(M, rows, K)) return gemm_bf16_stream_dma_act(x, w, h, M, I, K, act, s);
  const int waves = stream_waves(rows, K);
  const int kw = stream_kw(K, waves);
  const int Mi = (int)M, Ii = (int)I, Ki = (int)K;
#define TPL_SACT(WV)                                                                         \
  do {                                                                                       \
    if (act == TP_ACT_SWIGLU) launch_stream<WV, 1, 2, 1>(x, w, h, Mi, Ii, Ki, kw, false, s); \
    else launch_stream<WV, 1, 1, 2>(x, w, h, Mi, Ii, Ki, kw, false, s);                     \
  } while (0)
  if (waves == 16) TPL_SACT(16);
  else if (waves == 8) TPL_SACT(8);
  else TPL_SACT(4);
#undef TPL_SACT
  TPL_LAUNCH_CHECK("gemm_bf16_stream_act");
  return TP_OK;
}

}  // namespace tpl
