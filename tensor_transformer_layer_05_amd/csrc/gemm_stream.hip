// Small-M (decode, M <= 64 tokens) bf16 linear: weight streaming.
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]
//
// At decode the weight matrix is read once per call and dominates the bytes
// (the "mostly GEMV" regime of decode), so the kernel is organised around
// streaming W from HBM with many 16-byte loads in flight:
//   * a workgroup owns 16 consecutive weight rows (output features) and all of
//     K; its WAVES waves split K into WAVES contiguous ranges;
//   * each wave multiplies its 16 x krange slice of W by the matching slice of
//     X^T on v_mfma_f32_16x16x32_bf16 (W rows are the MFMA A operand, up to 16
//     tokens per token tile are the B operand; unused token lanes carry zeros);
//   * per 32-k MFMA step a lane loads 16 bytes of its weight row; the loads of
//     the next 128-k chunk are issued before the current chunk's MFMAs;
//   * the WAVES partial 16 x M tiles are summed in LDS in a fixed order, so the
//     result does not depend on timing.
#include "common.h"

namespace tpl {

template <int WAVES, int MT, bool OUT_F32>
__global__ __launch_bounds__(WAVES * 64) void gemm_stream_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int M, int N, int K, int kw) {
  __shared__ float red[WAVES * MT * 256];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int g = lane >> 4;         // k-group of this lane inside a 32-k step
  const int row = n0 + (lane & 15);
  const int tok = lane & 15;
  const bool row_ok = row < N;
  const uint16_t* wrow = W + (int64_t)(row_ok ? row : 0) * K;

  const int kb = wave * kw;
  const int ke = min(K, kb + kw);

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wv[4], xv[MT][4];
  auto load_chunk = [&](int k0, u32x4 (&wr)[4], u32x4 (&xr)[MT][4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + j * 32 + g * 8;
      const bool ok = row_ok && k < ke;
      wr[j] = ok ? *reinterpret_cast<const u32x4*>(wrow + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = t * 16 + tok;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = k0 + j * 32 + g * 8;
        xr[t][j] = (m < M && k < ke) ? *reinterpret_cast<const u32x4*>(X + (int64_t)m * K + k)
                                     : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  if (kb < ke) {
    load_chunk(kb, wv, xv);
    for (int k0 = kb; k0 < ke; k0 += 128) {
      u32x4 wn[4], xn[MT][4];
      const bool more = k0 + 128 < ke;
      if (more) load_chunk(k0 + 128, wn, xn);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wv[j]), as_bf16x8(xv[t][j]),
                                                           acc[t], 0, 0, 0);
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wv[j] = wn[j];
#pragma unroll
          for (int t = 0; t < MT; ++t) xv[t][j] = xn[t][j];
        }
      }
    }
  }

  // 16x16 accumulator layout: lane holds column (token) lane & 15 and rows
  // (lane >> 4) * 4 + i.  Park every wave's partial in LDS, then sum them in
  // wave order.
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * MT + t) * 64 + lane) * 4 + i] = acc[t][i];
  __syncthreads();

  for (int v = threadIdx.x; v < MT * 256; v += WAVES * 64) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[w * MT * 256 + v];
    const int t = v >> 8, l = (v >> 2) & 63, i = v & 3;
    const int m = t * 16 + (l & 15);
    const int n = n0 + (l >> 4) * 4 + i;
    if (m < M && n < N) {
      if constexpr (OUT_F32)
        reinterpret_cast<float*>(Y)[(int64_t)m * N + n] = s;
      else
        reinterpret_cast<uint16_t*>(Y)[(int64_t)m * N + n] = (uint16_t)f2bf_bits(s);
    }
  }
}

template <int WAVES, int MT>
static void launch_stream(const void* x, const void* w, void* y, int M, int N, int K, int kw,
                          bool out_f32, hipStream_t s) {
  dim3 grid((N + 15) / 16), block(WAVES * 64);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
  if (out_f32)
    hipLaunchKernelGGL((gemm_stream_kernel<WAVES, MT, true>), grid, block, 0, s, X, Wp, y, M, N, K, kw);
  else
    hipLaunchKernelGGL((gemm_stream_kernel<WAVES, MT, false>), grid, block, 0, s, X, Wp, y, M, N, K, kw);
}

template <int WAVES>
static void launch_stream_mt(const void* x, const void* w, void* y, int M, int N, int K, int kw,
                             bool out_f32, hipStream_t s) {
  const int mt = (M + 15) / 16;
  switch (mt) {
    case 1: launch_stream<WAVES, 1>(x, w, y, M, N, K, kw, out_f32, s); break;
    case 2: launch_stream<WAVES, 2>(x, w, y, M, N, K, kw, out_f32, s); break;
    default:
      if constexpr (WAVES <= 8) {
        if (mt == 3) launch_stream<WAVES, 3>(x, w, y, M, N, K, kw, out_f32, s);
        else launch_stream<WAVES, 4>(x, w, y, M, N, K, kw, out_f32, s);
      }
      break;
  }
}

// Requires 1 <= M <= 64, K % 8 == 0, 16-byte aligned X and W.
tp_status gemm_bf16_stream(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                           bool out_f32, hipStream_t s) {
  const int nblk = (int)((N + 15) / 16);
  // Enough waves to keep ~8-16 per CU streaming, but at least 256 k per wave.
  // 16-wave workgroups cap registers at 128 per lane, too few for more than
  // two token tiles of double-buffered operands.
  int waves = M > 32 ? 8 : 16;
  while (waves > 4 && (K / waves < 256 || (int64_t)nblk * waves > 8192)) waves >>= 1;
  int kw = (int)((K + waves - 1) / waves);
  kw = (kw + 7) & ~7;
  switch (waves) {
    case 16: launch_stream_mt<16>(x, w, y, (int)M, (int)N, (int)K, kw, out_f32, s); break;
    case 8: launch_stream_mt<8>(x, w, y, (int)M, (int)N, (int)K, kw, out_f32, s); break;
    default: launch_stream_mt<4>(x, w, y, (int)M, (int)N, (int)K, kw, out_f32, s); break;
  }
  TPL_LAUNCH_CHECK("gemm_bf16_stream");
  return TP_OK;
}

}  // namespace tpl
