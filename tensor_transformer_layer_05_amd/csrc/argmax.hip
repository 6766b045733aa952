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

// One workgroup per token row: 256 threads scan the row (16-byte loads when
// the row is 16-byte aligned), then combine across the wave and the 4 waves.
__global__ __launch_bounds__(256) void vocab_argmax_kernel(const float* __restrict__ logits, int V,
                                                           int64_t offset, float* __restrict__ mv,
                                                           int64_t* __restrict__ mi, int vec) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int64_t m = blockIdx.x;
  const float* row = logits + m * (int64_t)V;
  float bv = -INFINITY;
  int bi = INT32_MAX;
  if (vec) {
    for (int c = threadIdx.x * 4; c < V; c += 256 * 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(row + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) take(x[e], c + e, bv, bi);
    }
  } else {
    for (int c = threadIdx.x; c < V; c += 256) take(row[c], c, bv, bi);
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
    for (int w = 1; w < 4; ++w)
      if (beats(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    mv[m] = bv;
    mi[m] = offset + bi;
  }
}

tp_status vocab_argmax_local(const float* logits, int64_t M, int64_t V, int64_t offset, float* mv,
                             int64_t* mi, bool vec, hipStream_t s) {
  hipLaunchKernelGGL(vocab_argmax_kernel, dim3((unsigned)M), dim3(256), 0, s, logits, (int)V, offset,
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
