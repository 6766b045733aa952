// Decode bf16 linear for 1..3 tokens (1..8 on tall weights): weight streaming
// with whole-line loads.
//
//   Y[m, n] = sum_k X[m, k] * W[n, k]
//
// With one to three tokens the weight bytes are the whole cost (the "mostly
// GEMV" regime of decode; page P2, section 三, the prefill/decode table), and
// the arithmetic is a few dot products per weight byte, so this kernel does
// not use the matrix cores at all:
//   * a workgroup of 8 waves owns up to 8 GROUPS consecutive output rows and
//     all of K; its waves split K into contiguous ranges of 64-k steps;
//   * lane l takes row (l >> 3) of an 8-row group and the 16 bytes at k
//     offset 8 (l & 7) of each 64-k step, so one load instruction reads 8
//     rows x 128 contiguous bytes: every 128-byte line it touches is read
//     whole by that one instruction.  That is what lets the weight loads use
//     the non-temporal policy (kLoadStream); the matrix-core layout (16 rows x
//     64 bytes per instruction) takes each line in two halves and slowed down
//     with it;
//   * the token rows are staged once in LDS; each lane multiplies its 8
//     weights with the matching 8 token values by v_dot2c_f32_bf16 into one
//     float32 partial per (row, token), in k order;
//   * at the end the 8 lanes of a row are summed by a fixed DPP tree and the
//     8 waves' sums in wave order, so the result depends only on K (through
//     the waves' k ranges), not on the row tiling or on timing.  The fused
//     SwiGLU / GELU variants apply the activation to these float32 sums, so
//     they equal the plain linear followed by the activation bit for bit.
#include "common.h"

namespace tpl {

namespace {

constexpr uint32_t kDotOob = 0x80000000u;   // offset past any buffer bound -> reads 0
constexpr int kDotWaves = 8;
constexpr int kDotMaxTokens = 8;           // calls with more tokens take the MFMA kernels
// Longest K whose MT token rows are staged in LDS (at most 96 KB of them).
constexpr int dot_max_k(int mt) { return mt <= 3 ? 16384 : 8192; }
// Zeroed k past the last 64-k step: a wave's last two batches of T steps may
// read up to 2 T - 1 steps past its range.
constexpr int dot_pad(int t) { return (2 * t + 1) * 64; }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// The vector elements go through scalar copies: a __builtin_bit_cast applied
// to the subscript w[i] itself compiled to element 0 for every i.
__device__ __forceinline__ float dot8(const u32x4 w, const u32x4 x, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wi = w[i], xi = x[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, wi),
                                          __builtin_bit_cast(bf16x2v, xi), acc, false);
  }
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over the 8 lanes 8r..8r+7 (every one of them gets the sum): swap
// neighbours, swap pairs, then mirror each half-row of 8.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp<0x141>(v);   // row_half_mirror
  return v;
}

// M <= MT tokens (token rows M..MT-1 read as zero); GROUPS 8-row groups per workgroup; PARTS = 2 pairs gate rows n
// with up rows N + n of a [2N, K] weight (SwiGLU), else 1; EPI: 0 plain,
// 1 SwiGLU, 2 GELU.  ksw = 64-k steps per wave; rows_wg = output rows per
// workgroup (<= 8 GROUPS).
template <int MT, int GROUPS, int PARTS, int EPI, bool OUT_F32>
__global__ __launch_bounds__(kDotWaves * 64) void gemv_dot_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, void* __restrict__ Y,
    int M, int N, int K, int ksw, int rows_wg) {
  static_assert(GROUPS * PARTS <= 8 && 8 % (GROUPS * PARTS) == 0, "8 loads per batch");
  static_assert(EPI != 1 || PARTS == 2, "SwiGLU pairs gate and up rows");
  constexpr int T = 8 / (GROUPS * PARTS);     // 64-k steps per batch of 8 loads
  constexpr int kPad = dot_pad(T);
  __shared__ __attribute__((aligned(16))) uint16_t xs[MT * (dot_max_k(MT) + kPad)];
  __shared__ float red[kDotWaves * GROUPS * 8 * PARTS * MT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * rows_wg;
  const int nrows = min(rows_wg, N - n0);
  const int slot = lane >> 3, kq = lane & 7;
  const int KP = (K + 63) / 64 * 64 + kPad;   // LDS row pitch of the staged tokens

  // one resource per part, based at its first row and bounded to the valid rows
  __amdgpu_buffer_rsrc_t wr[PARTS];
#pragma unroll
  for (int p = 0; p < PARTS; ++p)
    wr[p] = __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)(p ? N + n0 : n0) * K), 0,
                                              (uint32_t)nrows * (uint32_t)K * 2u, 0x00020000);
  uint32_t roff[GROUPS];
#pragma unroll
  for (int g = 0; g < GROUPS; ++g) roff[g] = (uint32_t)((g * 8 + slot) * K) * 2u;

  const int nsteps = (K + 63) / 64;
  const int s0 = wave * ksw;                       // this wave's first 64-k step
  const int ns = max(0, min(ksw, nsteps - s0));    // its steps
  const int nb = (ns + T - 1) / T;                 // its batches

  auto load = [&](int b, u32x4 (&v)[8]) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int s = b * T + t;
      const int k = (s0 + s) * 64 + kq * 8;
      const bool ok = s < ns && k < K;
#pragma unroll
      for (int g = 0; g < GROUPS; ++g)
#pragma unroll
        for (int p = 0; p < PARTS; ++p)
          v[(t * GROUPS + g) * PARTS + p] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr[p], ok ? roff[g] + (uint32_t)k * 2u : kDotOob,
                                                           0, kLoadStream));
    }
  };

  float acc[GROUPS][PARTS][MT];
#pragma unroll
  for (int g = 0; g < GROUPS; ++g)
#pragma unroll
    for (int p = 0; p < PARTS; ++p)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[g][p][m] = 0.f;

  auto compute = [&](int b, const u32x4 (&v)[8]) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      // past this wave's range the weights read as zero and the staged tokens
      // are finite (the next range, or the zeroed pad past K)
      const int k = (s0 + b * T + t) * 64 + kq * 8;
      u32x4 xf[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) xf[m] = *reinterpret_cast<const u32x4*>(xs + m * KP + k);
#pragma unroll
      for (int g = 0; g < GROUPS; ++g)
#pragma unroll
        for (int p = 0; p < PARTS; ++p)
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[g][p][m] = dot8(v[(t * GROUPS + g) * PARTS + p], xf[m], acc[g][p][m]);
    }
  };

  // Stage the tokens (first loads in flight before the first weight batch),
  // zero the pad, then stream: two batches of 8 loads in flight per wave.
  u32x4 wa[8], wb[8];
  {
    const int per_row = K / 8;                      // 16-byte pieces per token row
    const int total = MT * per_row;
    constexpr int kMaxPieces = MT * dot_max_k(MT) / 8 / (kDotWaves * 64);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)X, 0, (uint32_t)M * (uint32_t)per_row * 16u, 0x00020000);
    u32x4 xv[kMaxPieces];
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i)
      xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            xr, (uint32_t)(threadIdx.x + i * kDotWaves * 64) * 16u, 0, 0));
    load(0, wa);
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
      const int q = threadIdx.x + i * kDotWaves * 64;
      if (q < total) {
        const int m = q / per_row, c = q - m * per_row;
        *reinterpret_cast<u32x4*>(xs + m * KP + c * 8) = xv[i];
      }
    }
    for (int q = threadIdx.x; q < MT * (KP - K) / 8; q += kDotWaves * 64) {
      const int m = q / ((KP - K) / 8), c = q - m * ((KP - K) / 8);
      *reinterpret_cast<u32x4*>(xs + m * KP + K + c * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }
  // Unrolled by two so both buffers stay in registers; past the last batch
  // every offset is out of range, so those loads read zeros without memory
  // traffic and add nothing.
  for (int b = 0; b < nb; b += 2) {
    load(b + 1, wb);
    __builtin_amdgcn_sched_barrier(0);
    compute(b, wa);
    __builtin_amdgcn_sched_barrier(0);
    load(b + 2, wa);
    __builtin_amdgcn_sched_barrier(0);
    compute(b + 1, wb);
    __builtin_amdgcn_sched_barrier(0);
  }

  // lane sums of each row, then the waves' sums in wave order
#pragma unroll
  for (int g = 0; g < GROUPS; ++g)
#pragma unroll
    for (int p = 0; p < PARTS; ++p)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float s = sum8(acc[g][p][m]);
        if (kq == 0) red[(((wave * GROUPS + g) * 8 + slot) * PARTS + p) * MT + m] = s;
      }
  __syncthreads();
  for (int v = threadIdx.x; v < nrows * MT; v += kDotWaves * 64) {
    const int r = v / MT, m = v - r * MT;
    if (m >= M) continue;
    float s[PARTS];
#pragma unroll
    for (int p = 0; p < PARTS; ++p) {
      s[p] = 0.f;
#pragma unroll
      for (int w = 0; w < kDotWaves; ++w) s[p] += red[((w * GROUPS * 8 + r) * PARTS + p) * MT + m];
    }
    const int64_t o = (int64_t)m * N + n0 + r;
    if constexpr (EPI == 1)
      reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f2bf_bits(act_fn<TP_ACT_SWIGLU>(s[0], s[PARTS - 1]));
    else if constexpr (EPI == 2)
      reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f2bf_bits(act_fn<TP_ACT_GELU>(s[0], 0.f));
    else if constexpr (OUT_F32)
      reinterpret_cast<float*>(Y)[o] = s[0];
    else
      reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f2bf_bits(s[0]);
  }
}

constexpr int kDotCUs = 256;   // compute units of an MI355X

template <int MT, int PARTS, int EPI, bool OUT_F32>
static void launch_dot(const void* x, const void* w, void* y, int M, int N, int K, hipStream_t s) {
  // rows per workgroup: one workgroup per CU while that needs at most 64 rows
  // (32 gate|up pairs); 8-row groups, at most 8 loads per 64-k step
  constexpr int kMaxRows = 64 / PARTS;
  const int per_cu = (N + kDotCUs - 1) / kDotCUs;
  const int rows_wg = per_cu < kMaxRows ? per_cu : kMaxRows;
  const int groups = (rows_wg + 7) / 8;
  const int nsteps = (K + 63) / 64;
  const int ksw = (nsteps + kDotWaves - 1) / kDotWaves;
  dim3 grid((N + rows_wg - 1) / rows_wg), block(kDotWaves * 64);
  auto X = static_cast<const uint16_t*>(x);
  auto Wp = static_cast<const uint16_t*>(w);
#define TPL_DOT(G) hipLaunchKernelGGL((gemv_dot_kernel<MT, G, PARTS, EPI, OUT_F32>), grid, block, 0, s, X, Wp, y, M, N, K, ksw, rows_wg)
  if (groups <= 1) TPL_DOT(1);
  else if (groups <= 2) TPL_DOT(2);
  else if constexpr (PARTS == 1) {
    if (groups <= 4) TPL_DOT(4);
    else TPL_DOT(8);
  } else {
    TPL_DOT(4);
  }
#undef TPL_DOT
}

}  // namespace

// Whether gemv_dot serves a call on a weight of `rows` x K: 1..3 tokens, or
// 4..8 tokens on weights of more than 8192 rows, with token rows that fit the
// LDS stage.  Measured per call over weight copies larger than the Infinity
// Cache: the lm_head vocab shard [16032, 8192] at 4 / 5 / 8 tokens took 45.9 /
// 49.0 / 49.2 us here against 54.8 / 53.6 / 54.0 on the LDS-ring kernel,
// while the decode down projection [8192, 3584] at 5 and 8 tokens took 16.6
// and 16.7 us against 13.6 (and QKV [1536, 4096] 14.5 against 13.5).  The
// rule looks only at the weight's shape, so a fused-activation call and the
// plain call on the same weight take the same kernel.  K % 8 == 0 and 16-byte
// aligned x and w are the caller's conditions.
bool gemv_dot_fits(int64_t M, int64_t rows, int64_t K) {
  if (M < 1 || K < 8) return false;
  if (M <= 3) return K <= dot_max_k((int)M);
  return M <= kDotMaxTokens && rows > 8192 && K <= dot_max_k(8);
}

tp_status gemv_dot(const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
                   bool out_f32, hipStream_t s) {
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K;
#define TPL_DOTM(MT)                                                         \
  do {                                                                       \
    if (out_f32) launch_dot<MT, 1, 0, true>(x, w, y, Mi, Ni, Ki, s);         \
    else launch_dot<MT, 1, 0, false>(x, w, y, Mi, Ni, Ki, s);                \
  } while (0)
  if (M == 1) TPL_DOTM(1);
  else if (M == 2) TPL_DOTM(2);
  else if (M == 3) TPL_DOTM(3);
  else if (M == 4) TPL_DOTM(4);
  else TPL_DOTM(8);
#undef TPL_DOTM
  TPL_LAUNCH_CHECK("gemv_dot");
  return TP_OK;
}

// act = TP_ACT_SWIGLU (w is [2I, K], gate rows then up rows) or TP_ACT_GELU
// (w is [I, K]); output bf16 [M, I].
tp_status gemv_dot_act(const void* x, const void* w, void* h, int64_t M, int64_t I, int64_t K,
                       int act, hipStream_t s) {
  const int Mi = (int)M, Ii = (int)I, Ki = (int)K;
#define TPL_DOTA(MT)                                                                \
  do {                                                                              \
    if (act == TP_ACT_SWIGLU) launch_dot<MT, 2, 1, false>(x, w, h, Mi, Ii, Ki, s);  \
    else launch_dot<MT, 1, 2, false>(x, w, h, Mi, Ii, Ki, s);                       \
  } while (0)
  if (M == 1) TPL_DOTA(1);
  else if (M == 2) TPL_DOTA(2);
  else if (M == 3) TPL_DOTA(3);
  else if (M == 4) TPL_DOTA(4);
  else TPL_DOTA(8);
#undef TPL_DOTA
  TPL_LAUNCH_CHECK("gemv_dot_act");
  return TP_OK;
}

}  // namespace tpl
