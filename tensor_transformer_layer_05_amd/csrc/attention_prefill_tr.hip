// Prefill attention over a rank's local heads (many query rows), gfx950.
//
// Flash-attention structure: a workgroup owns 256 query rows of one q head
// (8 waves x 32 rows, two waves per SIMD) and walks the key span in tiles of
// 64 keys with an online softmax, so scores never reach HBM.
//
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    (A = K rows straight from LDS, B = the wave's Q^T fragments kept in
//    registers).  A lane then owns one query and 32 of the tile's 64 keys;
//    the other 32 sit in lane ^ 32, so row statistics are an in-register
//    reduction plus one v_permlane32_swap.
//  * The probabilities are already in the B-operand layout of O^T = V^T P^T
//    (8 keys per lane per 16-key step).  The matching V^T operand comes from
//    V stored naturally ([key][d]) in LDS through ds_read_b64_tr_b16: within
//    each 16-lane group, lane s addresses the 4 d of row k0 + s/4 starting at
//    d0 + 4 (s % 4), and lane j receives V[k0 + e][d0 + j], e = 0..3.
//  * Each wave alternates an MFMA step (the O product of tile t and the
//    scores of tile t+1) and a VALU step (the softmax of tile t+1 and the
//    rescale of O), with a workgroup barrier after each step.  The two waves
//    of a SIMD (w and w + 4) run half a tile apart, so one wave's MFMAs run
//    while the other works through its softmax: waves 4-7 pass one extra
//    barrier before the loop and waves 0-3 one after it.
//  * K and V tiles reach LDS through buffer_load_dwordx4 ... lds (1 KB = 4
//    key rows per wave-level load), in two slots each; K runs two tiles ahead
//    of the O product and V one.  Inside the loop only waves 0-3 load (at the
//    end of their MFMA step) and they wait for the loads before
//    the barrier that ends their next VALU step; the transposing V reads wait
//    for every load their wave has in flight, so waves 4-7 issue none.  Rows
//    past the key span read as zero through the buffer bound.  LDS rows are
//    256 bytes; K's 16-byte chunks are XOR-ed with (key % 16) so that the 16
//    rows of an A-fragment read hit distinct banks, V's with 4 (key % 4) so
//    that the 4 rows x 4 chunks of a transposed read do.
//  * A positive softmax scale is applied inside the exponent's FMA; the
//    running maximum is kept on unscaled scores.
//  * Causal masking is aligned to the end of the key span; tiles entirely
//    above a wave's last query are skipped by that wave.  Workgroups are
//    ordered longest first across all heads to balance the causal triangle.
#include <type_traits>

#include "common.h"

namespace tpl {

namespace {

constexpr int kD = 128;         // head dimension
constexpr int kBQ = 256;        // query rows per workgroup
constexpr int kQW = 32;         // query rows per wave
constexpr int kBK = 64;         // keys per tile
constexpr int kRowB = kD * 2;   // bytes per K/V row
constexpr int kTileE = kBK * kD;  // bf16 elements per K (or V) tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define TPL_LDS __attribute__((address_space(3)))

struct TrArgs {
  const uint16_t* q; int64_t qs0, qs1, qs2;
  const uint16_t* k; const uint16_t* v; int64_t ks0, ks1, ks2;
  uint16_t* o; int64_t os0, os1, os2;
  int B, Sq, Skv, Hq, Hkv, causal;
  float scale_log2;
};

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// a ^ IMM in a VALU op the compiler does not hoist out of the loop (one op per
// fragment address instead of a register held per address)
template <uint32_t IMM>
__device__ __forceinline__ uint32_t xor_late(uint32_t a) {
  uint32_t r;
  asm volatile("v_xor_b32_e32 %0, %1, %2" : "=v"(r) : "i"(IMM), "v"(a));
  return r;
}

}  // namespace

__global__ __launch_bounds__(512) void attn_prefill_tr_kernel(TrArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * kTileE];  // K slots 0, 1, V slots 0, 1

  // longest-first over (query block, head, batch)
  const int nqb = (a.Sq + kBQ - 1) / kBQ;
  const int hb = a.Hq * a.B;
  const int id = blockIdx.x;
  const int qblk = nqb - 1 - id / hb;
  const int h = (id % hb) % a.Hq, b = (id % hb) / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int off = a.Skv - a.Sq;
  const int s0 = qblk * kBQ;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c32 = lane & 31, hl = lane >> 5;
  const int qw0 = s0 + wave * kQW;

  // Q^T fragments: query qw0 + c32, d = 16 kk + 8 hl .. +7
  const uint16_t* qbase = a.q + b * a.qs0 + h * a.qs2;
  bf16x8 qf[8];
  {
    const int s = qw0 + c32;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v4 = {0u, 0u, 0u, 0u};
      if (s < a.Sq) v4 = *reinterpret_cast<const u32x4*>(qbase + (int64_t)s * a.qs1 + kk * 16 + hl * 8);
      qf[kk] = as_bf16x8(v4);
    }
  }

  // key span of the workgroup and of this wave
  int kv_end = a.Skv;
  if (a.causal) kv_end = min(a.Skv, min(s0 + kBQ, a.Sq) + off);
  const int nkt = (kv_end + kBK - 1) / kBK;
  const int wave_last_key = a.causal ? min(a.Skv - 1, min(qw0 + kQW, a.Sq) - 1 + off) : a.Skv - 1;
  const bool wave_active = qw0 < a.Sq;

  // DMA tile loads: 4 per wave per tile (2 K, 2 V), each 4 key rows x 256 B.
  const uint32_t nrec = (uint32_t)(((int64_t)(a.Skv - 1) * a.ks1 + kD) * 2);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + b * a.ks0 + hk * a.ks2), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v + b * a.ks0 + hk * a.ks2), 0, nrec, 0x00020000);
  const int lr = lane >> 4, lp = lane & 15;   // row within the 4-row load, LDS chunk
  const uint32_t row_bytes = (uint32_t)(a.ks1 * 2);
  // LDS: K slots 0,1 then V slots 0,1 (64 keys x 256 B each).  K runs two
  // tiles ahead of the O product, V one.
  // Tile loads: one wave-level load = 4 key rows x 256 B.  Before the loop
  // every wave loads rows (2 wave + i) * 4 + lr of a tile (i < 2); inside
  // it, waves 0-3 load rows (4 wave + i) * 4 + lr (i < 4) and waves 4-7 none,
  // so the latter never wait for loads in flight (the transposing V reads
  // wait for every load the wave has in flight).
  auto issue_rows = [&](const __amdgpu_buffer_rsrc_t& rs, int slot, int kt, int row, bool is_v) {
    const int t = kt * kBK + row;
    const int ch = is_v ? (lp ^ (4 * (row & 3))) : (lp ^ (row & 15));
    const bool ok = t < a.Skv;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (TPL_LDS void*)((TPL_LDS uint16_t*)lds + slot * kTileE + (row - lr) * kD), 16,
        ok ? (uint32_t)t * row_bytes + (uint32_t)ch * 16u : 0x80000000u, 0, 0, 0);
  };
  auto issue_k = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) issue_rows(kr, kt & 1, kt, (wave * 2 + i) * 4 + lr, false);
  };
  auto issue_v = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) issue_rows(vr, 2 + (kt & 1), kt, (wave * 2 + i) * 4 + lr, true);
  };
  auto issue_k4 = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_rows(kr, kt & 1, kt, (wave * 4 + i) * 4 + lr, false);
  };
  auto issue_v4 = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_rows(vr, 2 + (kt & 1), kt, (wave * 4 + i) * 4 + lr, true);
  };

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  // transposed-read addressing (per 16-lane group g16 = lane/16): lane s of the
  // group reads row k0 + s/4, d = d0 + 4 (s % 4) with d0 = 32 db + 16 (g16 & 1)
  const int g16 = lane >> 4, sidx = lane & 15;
  const int tr_row = sidx >> 2;                      // + k0
  const int tr_d = 16 * (g16 & 1) + 4 * (sidx & 3);  // + 32 db

  // tiles this wave takes part in (causal: up to its last query's last key)
  const int nw = (wave_active && wave_last_key >= 0) ? min(nkt, wave_last_key / kBK + 1) : 0;

  // S^T[key, query] of tile kt, 2 blocks of 32 keys (K from slot kt & 1)
  f32x16 st[2];
  // chunk (2 kk + hl) ^ (row % 16) of K row `row` (row % 16 = c32 % 16) is the
  // byte offset ((hl ^ row % 16) * 16) ^ (32 kk): one base address serves all kk
  const uint32_t y16 = (uint32_t)((hl ^ (c32 & 15)) * 16);
  auto s_tile = [&](int kt) {
    const uint32_t kaddr0 =
        (uint32_t)reinterpret_cast<uintptr_t>((TPL_LDS uint16_t*)lds + (kt & 1) * kTileE + c32 * kD) | y16;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
    auto step = [&](auto kkc) {
      constexpr int kk = decltype(kkc)::value;
      const uint32_t ka = xor_late<32u * kk>(kaddr0);
      const bf16x8 qk = qf[kk];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 af = as_bf16x8(*reinterpret_cast<const TPL_LDS u32x4*>((TPL_LDS uint8_t*)(uintptr_t)ka + kb * 8192));
        st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qk, st[kb], 0, 0, 0);
      }
    };
    step(std::integral_constant<int, 0>{}); step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{}); step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{}); step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{}); step(std::integral_constant<int, 7>{});
    // K reads three steps ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int g = 0; g < 5; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
  };
  // scores into the log2 domain, then the mask behind one wave-uniform branch
  // (only diagonal and ragged tiles need it): key t = t_first + 4 hl + 32 kb +
  // 8 (r / 4) + r % 4 is valid while t < lim
  // A positive scale is folded into the exponent's FMA (the running max is
  // kept on unscaled scores); otherwise the scores are scaled first.
  const bool fold = a.scale_log2 > 0.f;
  const float csc = fold ? a.scale_log2 : 1.f;
  auto softmax_a = [&](int kt) {
    const int t_first = kt * kBK;
    if (!fold) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] *= a.scale_log2;
    }
    const bool need_mask = (t_first + kBK > a.Skv) ||
                           (a.causal && t_first + kBK - 1 > qw0 + off);
    if (need_mask) {
      const int qpos = qw0 + c32 + off;
      const int lim = a.causal ? min(a.Skv, qpos + 1) : a.Skv;
      const int rel = lim - (t_first + 4 * hl);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= rel) st[kb][r] = -INFINITY;
    }
  };
  // online softmax for query c32: probabilities into pb (bf16, the B operand of
  // the O product), running max and sum updated; returns the factor that
  // rescales the older O sums.  v_exp_f32 is called directly: its arguments
  // are <= 0, and results below 2^-126 may flush to zero.
  auto softmax_b = [&](bf16x8* pb) -> float {
    // max over four independent chains, then across the pair of lanes
    float m4[4] = {st[0][0], st[0][8], st[1][0], st[1][8]};
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int r = 1; r < 8; ++r) m4[g] = fmaxf(m4[g], st[g >> 1][(g & 1) * 8 + r]);
    float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    mx = pair_max(mx);
    const float mnew = fmaxf(mrun, mx);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew * csc;
    const float alpha = __builtin_amdgcn_exp2f(fmaf(mrun, csc, -muse));
    mrun = mnew;
    float ps[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(st[kb][half * 8 + e], csc, -muse));
        ps[kb * 2 + half] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pb[kb * 2 + half] = as_bf16x8(pack8(p));
      }
    lrun = lrun * alpha + ((ps[0] + ps[1]) + (ps[2] + ps[3]));
    return alpha;
  };
  // O^T[d, query] += V^T[d, keys] P^T[keys, query], 16 keys per step (V from
  // slot kt & 1).  Step (kb, half) covers keys kb*32 + 16 half + {4 hl + 0..3,
  // 8 + 4 hl + 0..3} (the P^T register order).
  auto o_tile = [&](int kt, const bf16x8* pb) {
    const uint16_t* vs = lds + (2 + (kt & 1)) * kTileE;
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const int k0 = (step >> 1) * 32 + (step & 1) * 16 + 4 * hl;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + tr_d;
        s16x4 lo, hi;
        {
          const int row = k0 + tr_row;
          const int pos = ((d >> 3) ^ (4 * (row & 3))) * 8 + (d & 7);
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (TPL_LDS s16x4*)((TPL_LDS uint16_t*)vs + row * kD + pos));
        }
        {
          const int row = k0 + 8 + tr_row;
          const int pos = ((d >> 3) ^ (4 * (row & 3))) * 8 + (d & 7);
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (TPL_LDS s16x4*)((TPL_LDS uint16_t*)vs + row * kD + pos));
        }
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const bf16x8 af = as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]});
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[step], oacc[db], 0, 0, 0);
      }
    }
    // transposing reads four MFMAs ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int g = 0; g < 12; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
  };

  bf16x8 pb[4];
  if (nkt > 0) { issue_k(0); issue_v(0); }
  if (nkt > 1) issue_k(1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  // Ping-pong: step M(j) is the MFMA work (O product of tile j, scores of
  // tile j+1), step V(j) the VALU work (softmax of tile j+1, O rescale).
  // Waves 4-7 (the second wave of each SIMD) run every step one phase after
  // waves 0-3, so one wave's MFMAs run beside the other wave's softmax.
  const int lag = wave >> 2;
  auto phase_barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // Every wave runs the same steps M(j), barrier, V(j), barrier for j = -1 ..
  // nkt - 1; waves 4-7 pass one extra barrier first and waves 0-3 one at the
  // end, so waves 4-7 run each step one phase after waves 0-3.  Waves 0-3
  // issue the tile loads at the end of their M step (K(j+2) and V(j+1) into
  // the slots that K(j) and V(j-1) left; both groups finished reading those
  // one phase earlier) and wait for them before the barrier after their V
  // step, which precedes every read of those tiles.
  if (lag) phase_barrier();
  for (int j = -1; j < nkt; ++j) {
    if (j >= 0 && j < nw) o_tile(j, pb);
    if (j + 1 < nw) s_tile(j + 1);
    if (lag == 0 && j >= 0) {
      if (j + 2 < nkt) issue_k4(j + 2);
      if (j + 1 < nkt) issue_v4(j + 1);
    }
    phase_barrier();
    if (j + 1 < nw) {
      softmax_a(j + 1);
      const float alpha = softmax_b(pb);
      rescale(alpha);
    }
    if (lag == 0) __builtin_amdgcn_s_waitcnt(0x0F70);
    phase_barrier();
  }
  if (!lag) phase_barrier();

  // normalise and store O[s, h, d]; lane holds query c32 and, per 32-d block,
  // d = 8 (r/4) + 4 hl + r%4
  const float ltot = pair_sum(lrun);
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
  const bool o16 = ((a.os0 | a.os1 | a.os2) & 7) == 0 && (reinterpret_cast<uintptr_t>(a.o) & 15) == 0;
  if (o16) {
    // the wave's 32 rows go through LDS (free once every wave has passed the
    // last barrier), so that each store instruction writes 4 whole rows of
    // 256 bytes; 16-byte chunk c of row r sits at c ^ (r % 16)
    uint16_t* sl = lds + wave * (kQW * 128);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int ch = (db * 4 + grp) ^ (c32 & 15);
        *reinterpret_cast<u32x2*>(sl + c32 * 128 + ch * 8 + 4 * hl) =
            u32x2{pack_bf2(oacc[db][grp * 4 + 0] * inv, oacc[db][grp * 4 + 1] * inv),
                  pack_bf2(oacc[db][grp * 4 + 2] * inv, oacc[db][grp * 4 + 3] * inv)};
      }
#pragma unroll
    for (int it = 0; it < kQW / 4; ++it) {
      const int row = 4 * it + (lane >> 4), c = lane & 15;
      const int sr = qw0 + row;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sl + row * 128 + ((c ^ (row & 15)) * 8));
      if (sr < a.Sq)
        *reinterpret_cast<u32x4*>(a.o + b * a.os0 + (int64_t)sr * a.os1 + h * a.os2 + c * 8) = v;
    }
    return;
  }
  const int s = qw0 + c32;
  if (s < a.Sq) {
    uint16_t* orow = a.o + b * a.os0 + (int64_t)s * a.os1 + h * a.os2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = db * 32 + grp * 8 + 4 * hl;
        *reinterpret_cast<u32x2*>(orow + d) =
            u32x2{pack_bf2(oacc[db][grp * 4 + 0] * inv, oacc[db][grp * 4 + 1] * inv),
                  pack_bf2(oacc[db][grp * 4 + 2] * inv, oacc[db][grp * 4 + 3] * inv)};
      }
  }
}

// Requires D == 128, key/value row stride >= D, and the key span addressable
// with 32-bit offsets (checked by the caller).
tp_status attn_prefill_tr(const void* q, const int64_t qs[3], const void* k, const void* v,
                          const int64_t kvs[3], void* o, const int64_t os[3], int64_t B,
                          int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv, int causal, float scale,
                          hipStream_t s) {
  TrArgs a;
  a.q = static_cast<const uint16_t*>(q); a.qs0 = qs[0]; a.qs1 = qs[1]; a.qs2 = qs[2];
  a.k = static_cast<const uint16_t*>(k); a.v = static_cast<const uint16_t*>(v);
  a.ks0 = kvs[0]; a.ks1 = kvs[1]; a.ks2 = kvs[2];
  a.o = static_cast<uint16_t*>(o); a.os0 = os[0]; a.os1 = os[1]; a.os2 = os[2];
  a.B = (int)B; a.Sq = (int)Sq; a.Skv = (int)Skv; a.Hq = (int)Hq; a.Hkv = (int)Hkv;
  a.causal = causal;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int64_t nblk = ((Sq + kBQ - 1) / kBQ) * Hq * B;
  hipLaunchKernelGGL(attn_prefill_tr_kernel, dim3((unsigned)nblk), dim3(512), 0, s, a);
  TPL_LAUNCH_CHECK("attn_prefill_tr");
  return TP_OK;
}

bool attn_prefill_tr_ok(const int64_t kvs[3], int64_t Skv, int64_t D) {
  if (D != kD) return false;
  if (kvs[1] < D) return false;
  const int64_t span = ((Skv - 1) * kvs[1] + D) * 2;
  return span < (int64_t{1} << 31);
}

}  // namespace tpl
