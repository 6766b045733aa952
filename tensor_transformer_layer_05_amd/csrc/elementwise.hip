// HBM-bound epilogue kernels: the rank-local activation, the in-HBM sum of
// rank partials (the arithmetic of the all-reduce), RMSNorm and the KV-cache
// append.  Each streams its operands once with 16-byte accesses where the
// layout allows and falls back to element accesses otherwise.
#include "common.h"

namespace tpl {

// ---- activation ------------------------------------------------------------

// One thread per 8 consecutive outputs of a row (vector path).
template <int ACT, bool BF16>
__global__ __launch_bounds__(256) void act_vec_kernel(const void* __restrict__ gate,
                                                      const void* __restrict__ up,
                                                      void* __restrict__ h, int64_t M, int64_t I,
                                                      int64_t ld) {
  const int64_t per_row = I / 8;
  const int64_t total = M * per_row;
  for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = v / per_row, c = (v % per_row) * 8;
    float g[8], u[8] = {0, 0, 0, 0, 0, 0, 0, 0}, o[8];
    if constexpr (BF16) {
      unpack8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(gate) + m * ld + c), g);
      if constexpr (ACT == TP_ACT_SWIGLU)
        unpack8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(up) + m * ld + c), u);
    } else {
      const float* gp = static_cast<const float*>(gate) + m * ld + c;
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp), g1 = *reinterpret_cast<const f32x4*>(gp + 4);
      for (int i = 0; i < 4; ++i) { g[i] = g0[i]; g[4 + i] = g1[i]; }
      if constexpr (ACT == TP_ACT_SWIGLU) {
        const float* upp = static_cast<const float*>(up) + m * ld + c;
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(upp), u1 = *reinterpret_cast<const f32x4*>(upp + 4);
        for (int i = 0; i < 4; ++i) { u[i] = u0[i]; u[4 + i] = u1[i]; }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = act_fn<ACT>(g[i], u[i]);
    if constexpr (BF16) {
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(h) + m * I + c) = pack8(o);
    } else {
      float* hp = static_cast<float*>(h) + m * I + c;
      *reinterpret_cast<f32x4*>(hp) = f32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<f32x4*>(hp + 4) = f32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

template <int ACT, bool BF16>
__global__ __launch_bounds__(256) void act_elem_kernel(const void* __restrict__ gate,
                                                       const void* __restrict__ up,
                                                       void* __restrict__ h, int64_t M, int64_t I,
                                                       int64_t ld) {
  const int64_t total = M * I;
  for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = v / I, i = v % I;
    float g, u = 0.f;
    if constexpr (BF16) {
      g = bf2f(static_cast<const uint16_t*>(gate)[m * ld + i]);
      if constexpr (ACT == TP_ACT_SWIGLU) u = bf2f(static_cast<const uint16_t*>(up)[m * ld + i]);
      static_cast<uint16_t*>(h)[v] = (uint16_t)f2bf_bits(act_fn<ACT>(g, u));
    } else {
      g = static_cast<const float*>(gate)[m * ld + i];
      if constexpr (ACT == TP_ACT_SWIGLU) u = static_cast<const float*>(up)[m * ld + i];
      static_cast<float*>(h)[v] = act_fn<ACT>(g, u);
    }
  }
}

static unsigned grid_for(int64_t work, int per_block = 256) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

template <int ACT>
static void launch_act(const void* g, const void* u, void* h, int64_t M, int64_t I, int64_t ld,
                       bool bf16, bool vec, hipStream_t s) {
  if (vec) {
    const unsigned gr = grid_for(M * (I / 8));
    if (bf16) hipLaunchKernelGGL((act_vec_kernel<ACT, true>), dim3(gr), dim3(256), 0, s, g, u, h, M, I, ld);
    else hipLaunchKernelGGL((act_vec_kernel<ACT, false>), dim3(gr), dim3(256), 0, s, g, u, h, M, I, ld);
  } else {
    const unsigned gr = grid_for(M * I);
    if (bf16) hipLaunchKernelGGL((act_elem_kernel<ACT, true>), dim3(gr), dim3(256), 0, s, g, u, h, M, I, ld);
    else hipLaunchKernelGGL((act_elem_kernel<ACT, false>), dim3(gr), dim3(256), 0, s, g, u, h, M, I, ld);
  }
}

tp_status act_local(const void* g, const void* u, void* h, int64_t M, int64_t I, int64_t ld,
                    int act, bool bf16, bool vec, hipStream_t s) {
  switch (act) {
    case TP_ACT_SWIGLU: launch_act<TP_ACT_SWIGLU>(g, u, h, M, I, ld, bf16, vec, s); break;
    case TP_ACT_GELU: launch_act<TP_ACT_GELU>(g, u, h, M, I, ld, bf16, vec, s); break;
    default: launch_act<TP_ACT_NONE>(g, u, h, M, I, ld, bf16, vec, s); break;
  }
  TPL_LAUNCH_CHECK("act_local");
  return TP_OK;
}

// ---- sum of rank partials --------------------------------------------------

struct PartialPtrs {
  const float* p[16];
};

template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void reduce_kernel(PartialPtrs P, int R,
                                                     const void* __restrict__ residual,
                                                     void* __restrict__ y, int64_t total) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if constexpr (VEC) {
    const int64_t nv = total / 4;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nv; v += stride) {
      f32x4 acc = *reinterpret_cast<const f32x4*>(P.p[0] + 4 * v);
      for (int r = 1; r < R; ++r) acc += *reinterpret_cast<const f32x4*>(P.p[r] + 4 * v);
      if constexpr (BF16) {
        if (residual) {
          const u32x2 rv = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(residual) + 4 * v);
          acc[0] += bf_lo(rv[0]); acc[1] += bf_hi(rv[0]);
          acc[2] += bf_lo(rv[1]); acc[3] += bf_hi(rv[1]);
        }
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + 4 * v) =
            u32x2{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3])};
      } else {
        if (residual) acc += *reinterpret_cast<const f32x4*>(static_cast<const float*>(residual) + 4 * v);
        *reinterpret_cast<f32x4*>(static_cast<float*>(y) + 4 * v) = acc;
      }
    }
  } else {
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < total; v += stride) {
      float acc = P.p[0][v];
      for (int r = 1; r < R; ++r) acc += P.p[r][v];
      if constexpr (BF16) {
        if (residual) acc += bf2f(static_cast<const uint16_t*>(residual)[v]);
        static_cast<uint16_t*>(y)[v] = (uint16_t)f2bf_bits(acc);
      } else {
        if (residual) acc += static_cast<const float*>(residual)[v];
        static_cast<float*>(y)[v] = acc;
      }
    }
  }
}

tp_status reduce_partials(const float* const* partials, int R, const void* residual, void* y,
                          int64_t total, bool bf16, bool vec, hipStream_t s) {
  PartialPtrs P = {};
  for (int r = 0; r < R; ++r) P.p[r] = partials[r];
  const unsigned gr = grid_for(vec ? total / 4 : total);
  if (bf16) {
    if (vec) hipLaunchKernelGGL((reduce_kernel<true, true>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
    else hipLaunchKernelGGL((reduce_kernel<true, false>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
  } else {
    if (vec) hipLaunchKernelGGL((reduce_kernel<false, true>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
    else hipLaunchKernelGGL((reduce_kernel<false, false>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
  }
  TPL_LAUNCH_CHECK("reduce_partials");
  return TP_OK;
}

// ---- RMSNorm -----------------------------------------------------------------

// One 256-thread workgroup per row.  Sum of squares in fp32: per-thread partial
// sums, a wave reduction, then the 4 wave sums in wave order.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x,
                                                      const void* __restrict__ gamma,
                                                      void* __restrict__ y, int64_t N, float eps) {
  __shared__ float wsum[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.f;
  if constexpr (BF16 && VEC) {
    const uint16_t* xr = static_cast<const uint16_t*>(x) + m * N;
    for (int64_t c = tid * 8; c < N; c += 256 * 8) {
      float f[8];
      unpack8(*reinterpret_cast<const u32x4*>(xr + c), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    }
  } else {
    for (int64_t c = tid; c < N; c += 256) {
      const float f = BF16 ? bf2f(static_cast<const uint16_t*>(x)[m * N + c])
                           : static_cast<const float*>(x)[m * N + c];
      ss = fmaf(f, f, ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = rsqrtf(tot / (float)N + eps);
  if constexpr (BF16 && VEC) {
    const uint16_t* xr = static_cast<const uint16_t*>(x) + m * N;
    const uint16_t* gr = static_cast<const uint16_t*>(gamma);
    uint16_t* yr = static_cast<uint16_t*>(y) + m * N;
    for (int64_t c = tid * 8; c < N; c += 256 * 8) {
      float f[8], gm[8], o[8];
      unpack8(*reinterpret_cast<const u32x4*>(xr + c), f);
      unpack8(*reinterpret_cast<const u32x4*>(gr + c), gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = f[i] * inv * gm[i];
      *reinterpret_cast<u32x4*>(yr + c) = pack8(o);
    }
  } else {
    for (int64_t c = tid; c < N; c += 256) {
      if constexpr (BF16) {
        const float f = bf2f(static_cast<const uint16_t*>(x)[m * N + c]);
        const float gm = bf2f(static_cast<const uint16_t*>(gamma)[c]);
        static_cast<uint16_t*>(y)[m * N + c] = (uint16_t)f2bf_bits(f * inv * gm);
      } else {
        const float f = static_cast<const float*>(x)[m * N + c];
        const float gm = static_cast<const float*>(gamma)[c];
        static_cast<float*>(y)[m * N + c] = f * inv * gm;
      }
    }
  }
}

// Rows of at most 8 x 2048 bf16 elements: the same arithmetic in the same order
// as rmsnorm_kernel<true, true>, with the row held in registers between the
// two passes and every load of the row issued before the first use.
template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gamma,
                                                          uint16_t* __restrict__ y, int64_t N, float eps) {
  __shared__ float wsum[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* xr = x + m * N;
  u32x4 xv[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = tid * 8 + k * 2048;
    xv[k] = c < N ? *reinterpret_cast<const u32x4*>(xr + c) : u32x4{0u, 0u, 0u, 0u};
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    if (tid * 8 + k * 2048 < N) {
      float f[8];
      unpack8(xv[k], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = rsqrtf(tot / (float)N + eps);
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = tid * 8 + k * 2048;
    if (c < N) {
      float f[8], gm[8], o[8];
      unpack8(xv[k], f);
      unpack8(*reinterpret_cast<const u32x4*>(gamma + c), gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = f[i] * inv * gm[i];
      *reinterpret_cast<u32x4*>(y + m * N + c) = pack8(o);
    }
  }
}

tp_status rmsnorm(const void* x, const void* gamma, void* y, int64_t M, int64_t N, float eps,
                  bool bf16, bool vec, hipStream_t s) {
  dim3 grid((unsigned)M), block(256);
  const int ch = (int)((N + 2047) / 2048);
  if (bf16 && vec && ch <= 8) {
    auto X = static_cast<const uint16_t*>(x);
    auto G = static_cast<const uint16_t*>(gamma);
    auto Y = static_cast<uint16_t*>(y);
#define TPL_RMS(C) hipLaunchKernelGGL((rmsnorm_reg_kernel<C>), grid, block, 0, s, X, G, Y, N, eps)
    switch (ch) {
      case 1: TPL_RMS(1); break;
      case 2: TPL_RMS(2); break;
      case 3: TPL_RMS(3); break;
      case 4: TPL_RMS(4); break;
      case 5: TPL_RMS(5); break;
      case 6: TPL_RMS(6); break;
      case 7: TPL_RMS(7); break;
      default: TPL_RMS(8); break;
    }
#undef TPL_RMS
    TPL_LAUNCH_CHECK("rmsnorm");
    return TP_OK;
  }
  if (bf16) {
    if (vec) hipLaunchKernelGGL((rmsnorm_kernel<true, true>), grid, block, 0, s, x, gamma, y, N, eps);
    else hipLaunchKernelGGL((rmsnorm_kernel<true, false>), grid, block, 0, s, x, gamma, y, N, eps);
  } else {
    hipLaunchKernelGGL((rmsnorm_kernel<false, false>), grid, block, 0, s, x, gamma, y, N, eps);
  }
  TPL_LAUNCH_CHECK("rmsnorm");
  return TP_OK;
}

// ---- sum of rank partials + residual, then RMSNorm (fused) ------------------------

// One 256-thread workgroup per row, bf16 storage, N % 8 == 0, 16-byte aligned
// rows.  Pass 1 forms h = residual + sum_r partials[r] exactly as reduce_kernel
// does (fp32, rank order, residual last, RNE to bf16), stores it and
// accumulates the squares of the stored bf16 values in rmsnorm_kernel's order;
// pass 2 re-reads this thread's own h values (still in L2) and normalises them
// exactly as rmsnorm_kernel does.  So y and yn equal the two unfused calls bit
// for bit, with one launch and one less pass over h in HBM.
__global__ __launch_bounds__(256) void reduce_rmsnorm_kernel(PartialPtrs P, int R,
                                                             const uint16_t* residual,
                                                             uint16_t* y,   // may alias residual
                                                             const uint16_t* __restrict__ gamma,
                                                             uint16_t* __restrict__ yn, int64_t N,
                                                             float eps) {
  __shared__ float wsum[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int64_t c = tid * 8; c < N; c += 256 * 8) {
    const int64_t o = m * N + c;
    float h[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 acc = *reinterpret_cast<const f32x4*>(P.p[0] + o + 4 * half);
      for (int r = 1; r < R; ++r) acc += *reinterpret_cast<const f32x4*>(P.p[r] + o + 4 * half);
      if (residual) {
        const u32x2 rv = *reinterpret_cast<const u32x2*>(residual + o + 4 * half);
        acc[0] += bf_lo(rv[0]); acc[1] += bf_hi(rv[0]);
        acc[2] += bf_lo(rv[1]); acc[3] += bf_hi(rv[1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) h[4 * half + i] = acc[i];
    }
    const u32x4 hb = pack8(h);
    *reinterpret_cast<u32x4*>(y + o) = hb;
    float f[8];
    unpack8(hb, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = rsqrtf(tot / (float)N + eps);
  for (int64_t c = tid * 8; c < N; c += 256 * 8) {
    float f[8], gm[8], o[8];
    unpack8(*reinterpret_cast<const u32x4*>(y + m * N + c), f);
    unpack8(*reinterpret_cast<const u32x4*>(gamma + c), gm);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f[i] * inv * gm[i];
    *reinterpret_cast<u32x4*>(yn + m * N + c) = pack8(o);
  }
}

// Rows of at most 8 x 2048 elements: reduce_rmsnorm_kernel's arithmetic in the
// same order, with each rank's loads for the whole row issued together and h
// kept in registers for the second pass.
template <int CH>
__global__ __launch_bounds__(256) void reduce_rmsnorm_reg_kernel(PartialPtrs P, int R,
                                                                 const uint16_t* residual,
                                                                 uint16_t* y,   // may alias residual
                                                                 const uint16_t* __restrict__ gamma,
                                                                 uint16_t* __restrict__ yn, int64_t N,
                                                                 float eps) {
  __shared__ float wsum[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  f32x4 acc[CH][2];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = tid * 8 + k * 2048;
#pragma unroll
    for (int half = 0; half < 2; ++half)
      acc[k][half] = c < N ? *reinterpret_cast<const f32x4*>(P.p[0] + m * N + c + 4 * half)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int r = 1; r < R; ++r) {
    f32x4 v[CH][2];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int64_t c = tid * 8 + k * 2048;
#pragma unroll
      for (int half = 0; half < 2; ++half)
        v[k][half] = c < N ? *reinterpret_cast<const f32x4*>(P.p[r] + m * N + c + 4 * half)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      acc[k][0] += v[k][0];
      acc[k][1] += v[k][1];
    }
  }
  u32x4 hb[CH];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = tid * 8 + k * 2048;
    if (c < N) {
      const int64_t o = m * N + c;
      float h[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x4 a = acc[k][half];
        if (residual) {
          const u32x2 rv = *reinterpret_cast<const u32x2*>(residual + o + 4 * half);
          a[0] += bf_lo(rv[0]); a[1] += bf_hi(rv[0]);
          a[2] += bf_lo(rv[1]); a[3] += bf_hi(rv[1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) h[4 * half + i] = a[i];
      }
      hb[k] = pack8(h);
      *reinterpret_cast<u32x4*>(y + o) = hb[k];
      float f[8];
      unpack8(hb[k], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = rsqrtf(tot / (float)N + eps);
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = tid * 8 + k * 2048;
    if (c < N) {
      float f[8], gm[8], o[8];
      unpack8(hb[k], f);
      unpack8(*reinterpret_cast<const u32x4*>(gamma + c), gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = f[i] * inv * gm[i];
      *reinterpret_cast<u32x4*>(yn + m * N + c) = pack8(o);
    }
  }
}

tp_status reduce_rmsnorm(const float* const* partials, int R, const void* residual, void* y,
                         const void* gamma, void* yn, int64_t M, int64_t N, float eps,
                         hipStream_t s) {
  PartialPtrs P = {};
  for (int r = 0; r < R; ++r) P.p[r] = partials[r];
  const int ch = (int)((N + 2047) / 2048);
  if (ch <= 8) {
    auto Rs = static_cast<const uint16_t*>(residual);
    auto Y = static_cast<uint16_t*>(y);
    auto G = static_cast<const uint16_t*>(gamma);
    auto YN = static_cast<uint16_t*>(yn);
#define TPL_RRMS(C) hipLaunchKernelGGL((reduce_rmsnorm_reg_kernel<C>), dim3((unsigned)M), dim3(256), 0, s, \
                                       P, R, Rs, Y, G, YN, N, eps)
    switch (ch) {
      case 1: TPL_RRMS(1); break;
      case 2: TPL_RRMS(2); break;
      case 3: TPL_RRMS(3); break;
      case 4: TPL_RRMS(4); break;
      case 5: TPL_RRMS(5); break;
      case 6: TPL_RRMS(6); break;
      case 7: TPL_RRMS(7); break;
      default: TPL_RRMS(8); break;
    }
#undef TPL_RRMS
    TPL_LAUNCH_CHECK("reduce_rmsnorm");
    return TP_OK;
  }
  hipLaunchKernelGGL(reduce_rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, s, P, R,
                     static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(y),
                     static_cast<const uint16_t*>(gamma), static_cast<uint16_t*>(yn), N, eps);
  TPL_LAUNCH_CHECK("reduce_rmsnorm");
  return TP_OK;
}

// ---- KV-cache append -----------------------------------------------------------

__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ kn,
                                                        const uint16_t* __restrict__ vn,
                                                        int64_t new_stride, uint16_t* __restrict__ kc,
                                                        uint16_t* __restrict__ vc, int64_t cs0,
                                                        int64_t cs1, int64_t cs2, int64_t B,
                                                        int64_t H, int64_t D, int64_t pos) {
  const int64_t total = B * H * D;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t d = e % D, j = (e / D) % H, b = e / (D * H);
    const int64_t src = b * new_stride + j * D + d;
    const int64_t dst = b * cs0 + pos * cs1 + j * cs2 + d;
    kc[dst] = kn[src];
    vc[dst] = vn[src];
  }
}

tp_status kv_append(const void* kn, const void* vn, int64_t new_stride, void* kc, void* vc,
                    const int64_t cs[3], int64_t B, int64_t H, int64_t D, int64_t pos,
                    hipStream_t s) {
  const unsigned gr = grid_for(B * H * D);
  hipLaunchKernelGGL(kv_append_kernel, dim3(gr), dim3(256), 0, s,
                     static_cast<const uint16_t*>(kn), static_cast<const uint16_t*>(vn), new_stride,
                     static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vc), cs[0], cs[1], cs[2], B,
                     H, D, pos);
  TPL_LAUNCH_CHECK("kv_append");
  return TP_OK;
}

}  // namespace tpl
