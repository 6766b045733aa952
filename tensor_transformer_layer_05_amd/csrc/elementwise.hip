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

// ---- 8-element row chunks in either storage type ------------------------------

// Non-temporal (streaming) loads, for rows read once.  In the 4096-token
// prefill step they shortened the first RMSNorm (33.5 -> 31.8 us) and the
// final sum of the MLP partials (83 -> 74 us), same bits; in the fused
// reduce + RMSNorm after o_proj they measured slower (96.5 -> 100.5 us), so
// that kernel keeps plain loads.
template <class T>
__device__ __forceinline__ T ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

template <bool F32>
__device__ __forceinline__ void load8_nt(const void* base, int64_t off, float* f) {
  if constexpr (F32) {
    const float* p = static_cast<const float*>(base) + off;
    const f32x4 a = ld_nt<f32x4>(p);
    const f32x4 b = ld_nt<f32x4>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  } else {
    unpack8(ld_nt<u32x4>(static_cast<const uint16_t*>(base) + off), f);
  }
}

template <bool F32>
__device__ __forceinline__ void load8(const void* base, int64_t off, float* f) {
  if constexpr (F32) {
    const float* p = static_cast<const float*>(base) + off;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  } else {
    unpack8(*reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off), f);
  }
}

// Stores 8 values and replaces them by what was stored (the bf16 rounding).
template <bool F32>
__device__ __forceinline__ void store8(void* base, int64_t off, float* f) {
  if constexpr (F32) {
    float* p = static_cast<float*>(base) + off;
    *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
  } else {
    const u32x4 b = pack8(f);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + off) = b;
    unpack8(b, f);
  }
}

__device__ __forceinline__ float load1(const void* base, int64_t i, bool f32) {
  return f32 ? static_cast<const float*>(base)[i] : bf2f(static_cast<const uint16_t*>(base)[i]);
}

// Residual operand of the sums: none, bfloat16 or float32 storage.
enum { kResNone = 0, kResBf16 = 1, kResF32 = 2 };

// ---- sum of rank partials --------------------------------------------------

struct PartialPtrs {
  const float* p[16];
};

// y = sum_r P[r] (+ residual): float32 sums in rank order 0..R-1, the residual
// added last, one rounding to y's storage type.
template <int RES, bool OUT_BF16, bool VEC>
__global__ __launch_bounds__(256) void reduce_kernel(PartialPtrs P, int R,
                                                     const void* __restrict__ residual,
                                                     void* __restrict__ y, int64_t total) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if constexpr (VEC) {
    const int64_t nv = total / 4;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nv; v += stride) {
      f32x4 acc = ld_nt<f32x4>(P.p[0] + 4 * v);
      for (int r = 1; r < R; ++r) acc += ld_nt<f32x4>(P.p[r] + 4 * v);
      if constexpr (RES == kResBf16) {
        const u32x2 rv = ld_nt<u32x2>(static_cast<const uint16_t*>(residual) + 4 * v);
        acc[0] += bf_lo(rv[0]); acc[1] += bf_hi(rv[0]);
        acc[2] += bf_lo(rv[1]); acc[3] += bf_hi(rv[1]);
      } else if constexpr (RES == kResF32) {
        acc += ld_nt<f32x4>(static_cast<const float*>(residual) + 4 * v);
      }
      if constexpr (OUT_BF16)
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + 4 * v) =
            u32x2{pack_bf2(acc[0], acc[1]), pack_bf2(acc[2], acc[3])};
      else
        *reinterpret_cast<f32x4*>(static_cast<float*>(y) + 4 * v) = acc;
    }
  } else {
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < total; v += stride) {
      float acc = P.p[0][v];
      for (int r = 1; r < R; ++r) acc += P.p[r][v];
      if constexpr (RES != kResNone) acc += load1(residual, v, RES == kResF32);
      if constexpr (OUT_BF16)
        static_cast<uint16_t*>(y)[v] = (uint16_t)f2bf_bits(acc);
      else
        static_cast<float*>(y)[v] = acc;
    }
  }
}

template <int RES>
static void launch_reduce(const PartialPtrs& P, int R, const void* residual, void* y,
                          int64_t total, bool bf16, bool vec, hipStream_t s) {
  const unsigned gr = grid_for(vec ? total / 4 : total);
  if (bf16) {
    if (vec) hipLaunchKernelGGL((reduce_kernel<RES, true, true>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
    else hipLaunchKernelGGL((reduce_kernel<RES, true, false>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
  } else {
    if (vec) hipLaunchKernelGGL((reduce_kernel<RES, false, true>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
    else hipLaunchKernelGGL((reduce_kernel<RES, false, false>), dim3(gr), dim3(256), 0, s, P, R, residual, y, total);
  }
}

tp_status reduce_partials(const float* const* partials, int R, const void* residual, bool res_f32,
                          void* y, int64_t total, bool bf16, bool vec, hipStream_t s) {
  PartialPtrs P = {};
  for (int r = 0; r < R; ++r) P.p[r] = partials[r];
  if (!residual) launch_reduce<kResNone>(P, R, residual, y, total, bf16, vec, s);
  else if (res_f32) launch_reduce<kResF32>(P, R, residual, y, total, bf16, vec, s);
  else launch_reduce<kResBf16>(P, R, residual, y, total, bf16, vec, s);
  TPL_LAUNCH_CHECK("reduce_partials");
  return TP_OK;
}

// ---- RMSNorm -----------------------------------------------------------------

// One 256-thread workgroup per row; x in float32 (XF32) or in the output type,
// gamma and y in the output type (bf16 when BF16).  Sum of squares in fp32:
// per-thread partial sums (the vector path: chunks of 8 consecutive elements
// at a stride of 2048, each chunk in order), a wave reduction, then the 4
// wave sums in wave order.
template <bool XF32, bool BF16, bool VEC>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x,
                                                      const void* __restrict__ gamma,
                                                      void* __restrict__ y, int64_t N, float eps) {
  static_assert(!VEC || BF16, "the vector path stores bf16");
  __shared__ float wsum[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.f;
  if constexpr (VEC) {
    for (int64_t c = tid * 8; c < N; c += 256 * 8) {
      float f[8];
      load8<XF32>(x, m * N + c, f);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    }
  } else {
    for (int64_t c = tid; c < N; c += 256) {
      const float f = load1(x, m * N + c, XF32);
      ss = fmaf(f, f, ss);
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = rsqrtf(tot / (float)N + eps);
  if constexpr (VEC) {
    const uint16_t* gr = static_cast<const uint16_t*>(gamma);
    for (int64_t c = tid * 8; c < N; c += 256 * 8) {
      float f[8], gm[8], o[8];
      load8<XF32>(x, m * N + c, f);
      unpack8(*reinterpret_cast<const u32x4*>(gr + c), gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = f[i] * inv * gm[i];
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + m * N + c) = pack8(o);
    }
  } else {
    for (int64_t c = tid; c < N; c += 256) {
      const float f = load1(x, m * N + c, XF32);
      const float gm = load1(gamma, c, !BF16);
      if constexpr (BF16)
        static_cast<uint16_t*>(y)[m * N + c] = (uint16_t)f2bf_bits(f * inv * gm);
      else
        static_cast<float*>(y)[m * N + c] = f * inv * gm;
    }
  }
}

// Rows of at most 8 x 2048 elements, bf16 gamma and y: the same arithmetic in
// the same order as rmsnorm_kernel's vector path, with the row held in
// registers between the two passes and every load of the row issued before
// the first use.
template <int CH, bool XF32>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(const void* __restrict__ x,
                                                          const uint16_t* __restrict__ gamma,
                                                          uint16_t* __restrict__ y, int64_t N, float eps) {
  __shared__ float wsum[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  float xv[CH][8];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = tid * 8 + k * 2048;
    if (c < N) {
      load8_nt<XF32>(x, m * N + c, xv[k]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[k][i] = 0.f;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    if (tid * 8 + k * 2048 < N) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(xv[k][i], xv[k][i], ss);
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
      float gm[8], o[8];
      unpack8(*reinterpret_cast<const u32x4*>(gamma + c), gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = xv[k][i] * inv * gm[i];
      *reinterpret_cast<u32x4*>(y + m * N + c) = pack8(o);
    }
  }
}

template <bool XF32>
static void launch_rmsnorm_reg(int ch, const void* x, const void* gamma, void* y, int64_t M,
                               int64_t N, float eps, hipStream_t s) {
  dim3 grid((unsigned)M), block(256);
  auto G = static_cast<const uint16_t*>(gamma);
  auto Y = static_cast<uint16_t*>(y);
#define TPL_RMS(C) hipLaunchKernelGGL((rmsnorm_reg_kernel<C, XF32>), grid, block, 0, s, x, G, Y, N, eps)
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
}

// x_f32: x is float32 storage; bf16: gamma and y are bf16 (x too unless x_f32).
tp_status rmsnorm(const void* x, bool x_f32, const void* gamma, void* y, int64_t M, int64_t N,
                  float eps, bool bf16, bool vec, hipStream_t s) {
  dim3 grid((unsigned)M), block(256);
  const int ch = (int)((N + 2047) / 2048);
  if (bf16 && vec && ch <= 8) {
    if (x_f32) launch_rmsnorm_reg<true>(ch, x, gamma, y, M, N, eps, s);
    else launch_rmsnorm_reg<false>(ch, x, gamma, y, M, N, eps, s);
  } else if (bf16 && vec) {
    if (x_f32) hipLaunchKernelGGL((rmsnorm_kernel<true, true, true>), grid, block, 0, s, x, gamma, y, N, eps);
    else hipLaunchKernelGGL((rmsnorm_kernel<false, true, true>), grid, block, 0, s, x, gamma, y, N, eps);
  } else if (bf16) {
    if (x_f32) hipLaunchKernelGGL((rmsnorm_kernel<true, true, false>), grid, block, 0, s, x, gamma, y, N, eps);
    else hipLaunchKernelGGL((rmsnorm_kernel<false, true, false>), grid, block, 0, s, x, gamma, y, N, eps);
  } else {
    if (x_f32) hipLaunchKernelGGL((rmsnorm_kernel<true, false, false>), grid, block, 0, s, x, gamma, y, N, eps);
    else hipLaunchKernelGGL((rmsnorm_kernel<false, false, false>), grid, block, 0, s, x, gamma, y, N, eps);
  }
  TPL_LAUNCH_CHECK("rmsnorm");
  return TP_OK;
}

// ---- sum of rank partials + residual, then RMSNorm (fused) ------------------------

// One 256-thread workgroup per row; gamma and yn bf16, y bf16 or float32
// (YF32), N % 8 == 0, 16-byte aligned rows.  Pass 1 forms y = residual +
// sum_r partials[r] exactly as reduce_kernel does (fp32, rank order, residual
// last, one rounding to y's type), stores it and accumulates the squares of
// the stored values in the order of rmsnorm_kernel's vector path; pass 2
// re-reads this thread's own y values (still in L2) and normalises them
// exactly as rmsnorm_kernel does.  So y and yn equal the two unfused calls bit
// for bit, with one launch and one less pass over y in HBM.
template <int RES, bool YF32>
__device__ __forceinline__ void sum_chunk(const PartialPtrs& P, int R, const void* residual,
                                          int64_t o, float* h) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(P.p[0] + o + 4 * half);
    for (int r = 1; r < R; ++r) acc += *reinterpret_cast<const f32x4*>(P.p[r] + o + 4 * half);
    if constexpr (RES == kResBf16) {
      const u32x2 rv = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(residual) + o + 4 * half);
      acc[0] += bf_lo(rv[0]); acc[1] += bf_hi(rv[0]);
      acc[2] += bf_lo(rv[1]); acc[3] += bf_hi(rv[1]);
    } else if constexpr (RES == kResF32) {
      acc += *reinterpret_cast<const f32x4*>(static_cast<const float*>(residual) + o + 4 * half);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) h[4 * half + i] = acc[i];
  }
}

template <int RES, bool YF32>
__global__ __launch_bounds__(256) void reduce_rmsnorm_kernel(PartialPtrs P, int R,
                                                             const void* residual,
                                                             void* y,   // may alias residual
                                                             const uint16_t* __restrict__ gamma,
                                                             uint16_t* __restrict__ yn, int64_t N,
                                                             float eps) {
  __shared__ float wsum[4];
  const int64_t m = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int64_t c = tid * 8; c < N; c += 256 * 8) {
    float h[8];
    sum_chunk<RES, YF32>(P, R, residual, m * N + c, h);
    store8<YF32>(y, m * N + c, h);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(h[i], h[i], ss);
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = rsqrtf(tot / (float)N + eps);
  for (int64_t c = tid * 8; c < N; c += 256 * 8) {
    float f[8], gm[8], o[8];
    load8<YF32>(y, m * N + c, f);
    unpack8(*reinterpret_cast<const u32x4*>(gamma + c), gm);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f[i] * inv * gm[i];
    *reinterpret_cast<u32x4*>(yn + m * N + c) = pack8(o);
  }
}

// Rows of at most 8 x 2048 elements: reduce_rmsnorm_kernel's arithmetic in the
// same order, with each rank's loads for the whole row issued together and y
// kept in registers for the second pass.
template <int CH, int RES, bool YF32>
__global__ __launch_bounds__(256) void reduce_rmsnorm_reg_kernel(PartialPtrs P, int R,
                                                                 const void* residual,
                                                                 void* y,   // may alias residual
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
  float h[CH][8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int64_t c = tid * 8 + k * 2048;
    if (c < N) {
      const int64_t o = m * N + c;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x4 a = acc[k][half];
        if constexpr (RES == kResBf16) {
          const u32x2 rv = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(residual) + o + 4 * half);
          a[0] += bf_lo(rv[0]); a[1] += bf_hi(rv[0]);
          a[2] += bf_lo(rv[1]); a[3] += bf_hi(rv[1]);
        } else if constexpr (RES == kResF32) {
          a += *reinterpret_cast<const f32x4*>(static_cast<const float*>(residual) + o + 4 * half);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) h[k][4 * half + i] = a[i];
      }
      store8<YF32>(y, o, h[k]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(h[k][i], h[k][i], ss);
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
      float gm[8], o[8];
      unpack8(*reinterpret_cast<const u32x4*>(gamma + c), gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = h[k][i] * inv * gm[i];
      *reinterpret_cast<u32x4*>(yn + m * N + c) = pack8(o);
    }
  }
}

template <int RES, bool YF32>
static void launch_reduce_rmsnorm(const PartialPtrs& P, int R, const void* residual, void* y,
                                  const void* gamma, void* yn, int64_t M, int64_t N, float eps,
                                  hipStream_t s) {
  auto G = static_cast<const uint16_t*>(gamma);
  auto YN = static_cast<uint16_t*>(yn);
  const int ch = (int)((N + 2047) / 2048);
  if (ch > 8) {
    hipLaunchKernelGGL((reduce_rmsnorm_kernel<RES, YF32>), dim3((unsigned)M), dim3(256), 0, s, P, R,
                       residual, y, G, YN, N, eps);
    return;
  }
#define TPL_RRMS(C) hipLaunchKernelGGL((reduce_rmsnorm_reg_kernel<C, RES, YF32>), dim3((unsigned)M), \
                                       dim3(256), 0, s, P, R, residual, y, G, YN, N, eps)
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
}

// gamma and yn bf16; residual bf16 or float32 (res_f32) or none; y bf16 or
// float32 (y_f32).
tp_status reduce_rmsnorm(const float* const* partials, int R, const void* residual, bool res_f32,
                         void* y, bool y_f32, const void* gamma, void* yn, int64_t M, int64_t N,
                         float eps, hipStream_t s) {
  PartialPtrs P = {};
  for (int r = 0; r < R; ++r) P.p[r] = partials[r];
#define TPL_RR(RES) \
  (y_f32 ? launch_reduce_rmsnorm<RES, true>(P, R, residual, y, gamma, yn, M, N, eps, s) \
         : launch_reduce_rmsnorm<RES, false>(P, R, residual, y, gamma, yn, M, N, eps, s))
  if (!residual) TPL_RR(kResNone);
  else if (res_f32) TPL_RR(kResF32);
  else TPL_RR(kResBf16);
#undef TPL_RR
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
