// Greedy token choice of a vocab-parallel lm_head (page P1 "Tensor Parallel：
// 当一张 GPU 放不下一个大模型", section "lm_head 怎么处理": the lm_head is split
// by vocab rows like any column-parallel linear, each rank finds the largest
// logit of its own vocab block, and an all-gather / all-reduce of the
// (value, index) pairs picks the global one).
//
// Order used everywhere (local scan, wave and workgroup combine, cross-rank
// combine): a NaN logit counts as -inf; a larger value wins; equal values go
// to the lower vocab id.  This is a total order on (value, id), so the result
// does not depend on how the work is split or in which order partial results
// meet, and it equals a sequential first-maximum scan of the full vocab.
#include <math.h>

#include "common.h"

namespace tpl {

namespace {

__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void take(float v, int i, float& bv, int& bi) {
  v = isnan(v) ? -INFINITY : v;
  if (beats(v, i, bv, bi)) { bv = v; bi = i; }
}

}  // namespace

// One workgroup of 1024 threads per token row.  Each thread issues up to
// kArgUnroll loads (16-byte ones when the row is 16-byte aligned) before it
// scans any of them, so a 16032-entry row costs one memory round trip rather
// than one per 1024 entries; then the waves combine by shuffles and LDS.
constexpr int kArgThreads = 1024, kArgWaves = kArgThreads / 64, kArgUnroll = 8;

__global__ __launch_bounds__(kArgThreads) void vocab_argmax_kernel(const float* __restrict__ logits, int V,
                                                                   int64_t offset, float* __restrict__ mv,
                                                                   int64_t* __restrict__ mi, int vec) {
  __shared__ float sv[kArgWaves];
  __shared__ int si[kArgWaves];
  const int64_t m = blockIdx.x;
  const float* row = logits + m * (int64_t)V;
  float bv = -INFINITY;
  int bi = INT32_MAX;
  if (vec) {   // V % 4 == 0, row 16-byte aligned
    const int n4 = V >> 2;
    for (int c0 = threadIdx.x; c0 < n4; c0 += kArgThreads * kArgUnroll) {
      f32x4 x[kArgUnroll];
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u) {
        const int c = c0 + u * kArgThreads;
        if (c < n4) x[u] = reinterpret_cast<const f32x4*>(row)[c];
      }
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u) {
        const int c = c0 + u * kArgThreads;
        if (c < n4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) take(x[u][e], 4 * c + e, bv, bi);
        }
      }
    }
  } else {
    for (int c0 = threadIdx.x; c0 < V; c0 += kArgThreads * kArgUnroll) {
      float x[kArgUnroll];
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u) {
        const int c = c0 + u * kArgThreads;
        if (c < V) x[u] = row[c];
      }
#pragma unroll
      for (int u = 0; u < kArgUnroll; ++u) {
        const int c = c0 + u * kArgThreads;
        if (c < V) take(x[u], c, bv, bi);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, kWave);
    const int oi = __shfl_xor(bi, o, kWave);
    if (beats(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kArgWaves; ++w)
      if (beats(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    mv[m] = bv;
    mi[m] = offset + bi;
  }
}

tp_status vocab_argmax_local(const float* logits, int64_t M, int64_t V, int64_t offset, float* mv,
                             int64_t* mi, bool vec, hipStream_t s) {
  hipLaunchKernelGGL(vocab_argmax_kernel, dim3((unsigned)M), dim3(kArgThreads), 0, s, logits, (int)V, offset,
                     mv, mi, (int)vec);
  TPL_LAUNCH_CHECK("vocab_argmax_local");
  return TP_OK;
}

struct RankPairs {
  const float* v[kMaxArgmaxRanks];
  const int64_t* i[kMaxArgmaxRanks];
};

// One thread per token row: the ranks' (value, id) pairs in rank order.
__global__ __launch_bounds__(256) void vocab_argmax_reduce_kernel(RankPairs P, int R, int64_t M,
                                                                  float* __restrict__ ov,
                                                                  int64_t* __restrict__ oi) {
  const int64_t m = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (m >= M) return;
  float bv = P.v[0][m];
  int64_t bi = P.i[0][m];
  for (int r = 1; r < R; ++r) {
    const float v = P.v[r][m];
    const int64_t i = P.i[r][m];
    if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
  }
  ov[m] = bv;
  oi[m] = bi;
}

tp_status vocab_argmax_reduce(const float* const* vals, const int64_t* const* idxs, int R, int64_t M,
                              float* ov, int64_t* oi, hipStream_t s) {
  RankPairs P = {};
  for (int r = 0; r < R; ++r) { P.v[r] = vals[r]; P.i[r] = idxs[r]; }
  const unsigned grid = (unsigned)((M + 255) / 256);
  hipLaunchKernelGGL(vocab_argmax_reduce_kernel, dim3(grid), dim3(256), 0, s, P, R, M, ov, oi);
  TPL_LAUNCH_CHECK("vocab_argmax_reduce");
  return TP_OK;
}

}  // namespace tpl
