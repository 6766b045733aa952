// Internal helpers shared by the HIP sources of libtplayer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tplayer.h"

namespace tpl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kNumXcd = 8;    // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kMaxArgmaxRanks = 64;   // ranks combined by one vocab argmax reduce call
// Cache-policy operand of buffer loads: non-temporal (streaming).  For bytes
// read once per call (decode weights, the KV cache) whose loads cover whole
// 128-byte lines, a plain read of 1 GiB measured 6.7 TB/s with it against
// 5.9 TB/s without; loads that take half a line per instruction slowed down.
constexpr int kLoadStream = 2;

// ---- bf16 <-> fp32 ---------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even with gfx950's v_cvt_pk_bf16_f32 (one instruction
// per pair; NaN stays a NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f2bf_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// 8 bf16 packed in a u32x4 -> 8 floats
__device__ __forceinline__ void unpack8(const u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(v[i]);
    f[2 * i + 1] = bf_hi(v[i]);
  }
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf2(f[2 * i], f[2 * i + 1]);
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- rank-local activation (shared by the elementwise kernel and the fused
// GEMM epilogues, so both round and evaluate identically) --------------------

template <int ACT>
__device__ __forceinline__ float act_fn(float g, float u) {
  // SiLU(g) = g / (1 + e^-g) from the hardware base-2 exponential and
  // reciprocal (about 1 ulp each), e^-g = 2^(-g log2 e): a few instructions
  // where expf and an IEEE division take some twenty, which is the fused
  // gate|up epilogue's cost.  Below g of about -88 the exponential is +inf and
  // the reciprocal 0, giving -0 (the limit); a NaN stays NaN.
  if constexpr (ACT == TP_ACT_SWIGLU)
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
  // GELU(g) = g * Phi(g) with Phi(g) = erfc(-g / sqrt 2) / 2: the erfc form
  // keeps full relative accuracy for negative g, where 1 + erf(.) cancels.
  else if constexpr (ACT == TP_ACT_GELU) return 0.5f * g * erfcf(-g * 0.70710678118654752f);
  else return g;
}

// ---- wave reductions ---------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---- XCD-aware block index ---------------------------------------------------
// Workgroups are dealt to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Remap so that consecutive logical tile ids land on the same XCD and share
// its L2.  The map is a bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = (n + kNumXcd - 1) / kNumXcd;
  const int tall = (n % kNumXcd == 0) ? kNumXcd : (n % kNumXcd);
  const int xcd = b % kNumXcd, local = b / kNumXcd;
  if (xcd < tall) return xcd * per + local;
  return tall * per + (xcd - tall) * (per - 1) + local;
}

}  // namespace tpl

// ---- host-side launch plumbing (used by the api TU and the kernels' launchers)

namespace tpl {
void set_hip_error(const char* where, hipError_t e);
}

#define TPL_LAUNCH_CHECK(where)                                   \
  do {                                                            \
    hipError_t e_ = hipGetLastError();                            \
    if (e_ != hipSuccess) {                                       \
      ::tpl::set_hip_error(where, e_);                            \
      return TP_ERR_HIP;                                          \
    }                                                             \
  } while (0)
