// Small-M (decode, M <= 64 tokens) bf16 linear: weight streaming.
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]
//
// At decode the weight matrix is read once per call and dominates the bytes
// (the "mostly GEMV" regime of decode), so the kernel is organised around
// keeping many weight loads in flight:
//   * a workgroup owns RT tiles of 16 consecutive weight rows (output
//     features) and all of K; its WAVES waves split K into contiguous ranges;
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

template <int WAVES, int MT, int RT, bool OUT_F32>
__global__ __launch_bounds__(WAVES * 64) void gemm_stream_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int M, int N, int K, int kw) {
  __shared__ float red[WAVES * RT * MT * 256];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * 16 * RT;
  const int g = lane >> 4;         // k-group of this lane inside a 32-k step
  const int i16 = lane & 15;       // weight row / token inside a 16-tile

  const int wrows = min(16 * RT, N - n0);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * K), 0, (uint32_t)wrows * (uint32_t)K * 2u, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)X, 0, (uint32_t)M * (uint32_t)K * 2u, 0x00020000);

  const int kb = wave * kw;
  const int ke = min(K, kb + kw);
  const int nc = ke > kb ? (ke - kb + 127) / 128 : 0;   // 128-k chunks of this wave

  uint32_t woff[RT], xoff[MT];
#pragma unroll
  for (int r = 0; r < RT; ++r) woff[r] = (uint32_t)((r * 16 + i16) * K) * 2u;
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
      for (int r = 0; r < RT; ++r) wv[r][j] = bload(wr, ok ? woff[r] + kbytes : kOob);
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
  for (int v = threadIdx.x; v < PER; v += WAVES * 64) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[w * PER + v];
    const int rt = v / (MT * 256), t = (v / 256) % MT, l = (v >> 2) & 63, e = v & 3;
    const int m = t * 16 + (l & 15);
    const int n = n0 + rt * 16 + (l >> 4) * 4 + e;
    if (m < M && n < N) {
      if constexpr (OUT_F32)
        reinterpret_cast<float*>(Y)[(int64_t)m * N + n] = s;
      else
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = (uint16_t)f2bf_bits(s);
    }
  }
}

template <int WAVES, int MT, int RT>
static void launch_stream(const void* x, const void* w, void* y, int M, int N, int K, int kw,
                          bool out_f32, hipStream_t s) {
  dim3 grid((N + 16 * RT - 1) / (16 * RT)), block(WAVES * 64);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
  if (out_f32)
    hipLaunchKernelGGL((gemm_stream_kernel<WAVES, MT, RT, true>), grid, block, 0, s, X, Wp, y, M, N, K, kw);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<WAVES, MT, RT, false>), grid, block, 0, s, X, Wp, y, M, N, K, kw);
}

// Requires 1 <= M <= 64 (M > 32 goes to the LDS-ring kernel), K % 8 == 0, 16-byte aligned X and W, M*K and
// 32*K elements addressable with 32-bit byte offsets.
tp_status gemm_bf16_stream_dma(const void* x, const void* w, void* y, int64_t M, int64_t N,
                               int64_t K, bool out_f32, hipStream_t s);

tp_status gemm_bf16_stream(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                           bool out_f32, hipStream_t s) {
  const int mt = (int)((M + 15) / 16);
  // Three or four token tiles: the LDS-ring kernel (coalesced weight stream,
  // two row tiles per wave) is faster; measured on 64-token decode shards.
  if (mt >= 3) return gemm_bf16_stream_dma(x, w, y, M, N, K, out_f32, s);
  // Two row tiles per wave when there are several token tiles (each X
  // fragment then feeds two MFMAs) and enough row tiles to fill the chip.
  const int rt = (mt >= 2 && N >= 16 * 2 * 224) ? 2 : 1;
  const int64_t nblk = (N + 16 * rt - 1) / (16 * rt);
  // Waves per workgroup: split K so that every wave streams >= 256 k; 16
  // waves (1024 threads, <= 128 VGPRs each) only for the lightest register
  // footprints and when there are few row tiles to spread over the chip.
  int waves = (nblk < 384 && mt * rt <= 2) ? 16 : 8;
  while (waves > 4 && K / waves < 256) waves >>= 1;
  int kw = (int)((K + waves - 1) / waves);
  kw = (kw + 31) & ~31;
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K;
#define TPL_STREAM(WV, MTV, RTV) launch_stream<WV, MTV, RTV>(x, w, y, Mi, Ni, Ki, kw, out_f32, s)
#define TPL_STREAM_MT(WV, RTV)                  \
  if (mt == 1) TPL_STREAM(WV, 1, RTV);          \
  else TPL_STREAM(WV, 2, RTV);
  if (waves == 16) {
    if (rt == 1 && mt == 1) TPL_STREAM(16, 1, 1);
    else if (rt == 1) TPL_STREAM(16, 2, 1);
    else TPL_STREAM(16, 1, 2);
  } else if (rt == 1) {
    if (waves == 8) { TPL_STREAM_MT(8, 1); } else { TPL_STREAM_MT(4, 1); }
  } else {
    if (waves == 8) { TPL_STREAM_MT(8, 2); } else { TPL_STREAM_MT(4, 2); }
  }
#undef TPL_STREAM_MT
#undef TPL_STREAM
  TPL_LAUNCH_CHECK("gemm_bf16_stream");
  return TP_OK;
}

}  // namespace tpl
