// float32 linear for fp32-stored shards (the integer-valued toy MLP runs on
// this path).  Plain LDS-tiled FMA kernel: 64x64 output tile per 256-thread
// workgroup, 4x4 outputs per thread, K in steps of 16.  Each output is the
// sum over k in increasing order, one fused multiply-add per term.
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]
#include "common.h"

namespace tpl {

__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W,
                                                       float* __restrict__ Y, int M, int N, int K) {
  __shared__ float xs[16][64 + 1];
  __shared__ float ws[16][64 + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    // 64 rows x 16 k for each operand: 1024 values, 4 per thread.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x + i * 256;
      const int r = e >> 4, kk = e & 15;
      const int k = k0 + kk;
      xs[kk][r] = (m0 + r < M && k < K) ? X[(int64_t)(m0 + r) * K + k] : 0.f;
      ws[kk][r] = (n0 + r < N && k < K) ? W[(int64_t)(n0 + r) * K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n < N) Y[(int64_t)m * N + n] = acc[i][j];
    }
  }
}

tp_status gemm_f32(const float* x, const float* w, float* y, int64_t M, int64_t N, int64_t K,
                   hipStream_t s) {
  dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64)), block(256);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, block, 0, s, x, w, y, (int)M, (int)N, (int)K);
  TPL_LAUNCH_CHECK("gemm_f32");
  return TP_OK;
}

}  // namespace tpl
