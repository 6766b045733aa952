// Prefill (many query rows) attention over a rank's local heads, on MFMA.
//
// Flash-attention style: a workgroup owns 256 query rows of one head (4 waves
// x 64 rows) and walks the key span in tiles of 64 keys, keeping a running
// row maximum, a running sum of exponentials and an unnormalised output in
// registers (online softmax), so scores never touch HBM.
//
// Layout choice for CDNA's 64-wide MFMA: the kernel computes the TRANSPOSED
// score block S^T = K Q^T with v_mfma_f32_32x32x16_bf16.  In the accumulator
// layout a lane then owns one query (column) and 16 keys (rows), so the
// softmax statistics of a query are an in-register reduction plus one
// exchange between the two half-waves, and rescaling the output (also kept
// transposed, O^T = V^T P^T) is one multiplier per lane.  The probabilities
// are already in the register layout of the B operand of the O^T product;
// only V needs transposing, which is done while staging V tiles into LDS
// (V^T rows padded to 68 keys to spread LDS banks).
//
// Causal masking is aligned to the end of the key span; only tiles crossing
// the diagonal or the end of the span evaluate the mask.  Query blocks are
// issued longest-first to shorten the tail of the causal triangle.
#include "common.h"

namespace tpl {

constexpr int kPD = 128;        // head dimension
constexpr int kPBQ = 256;       // query rows per workgroup
constexpr int kPBK = 64;        // keys per tile
constexpr int kVtLd = 68;       // V^T row length in LDS (64 keys + pad)

struct PreArgs {
  const uint16_t* q; int64_t qs0, qs1, qs2;
  const uint16_t* k; const uint16_t* v; int64_t ks0, ks1, ks2;
  uint16_t* o; int64_t os0, os1, os2;
  int Sq, Skv, Hq, Hkv, causal;
  float scale_log2;
};

__device__ __forceinline__ int kswz(int row, int ch) { return ch ^ (row & 15); }

__global__ __launch_bounds__(256) void attn_prefill_kernel(PreArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kPBK * kPD];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kPD * kVtLd];

  const int nqb = (a.Sq + kPBQ - 1) / kPBQ;
  const int qblk = nqb - 1 - (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (a.Hq / a.Hkv);
  const int off = a.Skv - a.Sq;
  const int s0 = qblk * kPBQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5;            // half-wave
  const int c32 = lane & 31;
  const int qw0 = s0 + wave * 64;      // first query row of this wave

  const uint16_t* qbase = a.q + b * a.qs0 + h * a.qs2;
  const uint16_t* kbase = a.k + b * a.ks0 + hk * a.ks2;
  const uint16_t* vbase = a.v + b * a.ks0 + hk * a.ks2;

  // Q^T fragments (B operand of S^T = K Q^T): query column c32, d = 16*kk + 8*hl.
  bf16x8 qf[2][8];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int s = qw0 + qb * 32 + c32;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v4 = {0u, 0u, 0u, 0u};
      if (s < a.Sq) v4 = *reinterpret_cast<const u32x4*>(qbase + (int64_t)s * a.qs1 + kk * 16 + hl * 8);
      qf[qb][kk] = as_bf16x8(v4);
    }
  }

  int kv_end = a.Skv;
  if (a.causal) kv_end = min(a.Skv, min(s0 + kPBQ, a.Sq) + off);
  const int nkt = (kv_end + kPBK - 1) / kPBK;

  f32x16 oacc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][j][r] = 0.f;
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

  // Staging: K tile as 16 threads per key row (16-byte chunks); V tile as
  // thread (dg = tid % 16, kg = tid / 16) holding keys 4kg..4kg+3, d 8dg..8dg+7.
  u32x4 kr[4], vr[4];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256, row = c >> 4, ch = c & 15;
      const int t = kt * kPBK + row;
      kr[i] = t < a.Skv ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)t * a.ks1 + ch * 8)
                        : u32x4{0u, 0u, 0u, 0u};
    }
    const int dg = tid & 15, kg = tid >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = kt * kPBK + kg * 4 + i;
      vr[i] = t < a.Skv ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)t * a.ks1 + dg * 8)
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256, row = c >> 4, ch = c & 15;
      *reinterpret_cast<u32x4*>(&ks[buf][row * kPD + kswz(row, ch) * 8]) = kr[i];
    }
    const int dg = tid & 15, kg = tid >> 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // element e of each of the 4 key rows -> 4 consecutive keys of V^T row 8dg+e
      const int w = e >> 1;
      const bool hi = e & 1;
      uint32_t k0 = hi ? (vr[0][w] >> 16) : (vr[0][w] & 0xffffu);
      uint32_t k1 = hi ? (vr[1][w] >> 16) : (vr[1][w] & 0xffffu);
      uint32_t k2 = hi ? (vr[2][w] >> 16) : (vr[2][w] & 0xffffu);
      uint32_t k3 = hi ? (vr[3][w] >> 16) : (vr[3][w] & 0xffffu);
      *reinterpret_cast<u32x2*>(&vt[buf][(dg * 8 + e) * kVtLd + kg * 4]) =
          u32x2{k0 | (k1 << 16), k2 | (k3 << 16)};
    }
  };

  if (nkt > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) gload(kt + 1);
    const int buf = kt & 1;

    // S^T[key, query] for 64 keys (kb) x 64 queries (qb)
    f32x16 st[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[i][j][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      bf16x8 af[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + c32;
        af[kb] = as_bf16x8(*reinterpret_cast<const u32x4*>(&ks[buf][row * kPD + kswz(row, kk * 2 + hl) * 8]));
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          st[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kb], qf[qb][kk], st[kb][qb], 0, 0, 0);
    }

    // scale into the log2 domain and mask
    const int t_first = kt * kPBK;
    const bool need_mask = (t_first + kPBK > a.Skv) || (a.causal && t_first + kPBK - 1 > qw0 + off);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = st[kb][qb][r] * a.scale_log2;
          if (need_mask) {
            const int t = t_first + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const int qpos = qw0 + qb * 32 + c32 + off;
            if (t >= a.Skv || (a.causal && t > qpos)) x = -INFINITY;
          }
          st[kb][qb][r] = x;
        }

    // online softmax per query column; P^T packed to bf16 as the B operand
    bf16x8 pb[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][qb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrun[qb], mx);
      const float muse = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = exp2f(mrun[qb] - muse);
      mrun[qb] = mnew;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = exp2f(st[kb][qb][half * 8 + e] - muse);
            psum += p[e];
          }
          pb[qb][kb * 2 + half] = as_bf16x8(pack8(p));
        }
      }
      lrun[qb] = lrun[qb] * alpha + psum;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
    }

    // O^T[d, query] += V^T[d, keys] P^T[keys, query]
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const int kb = kstep >> 1, half = kstep & 1;
      const int kofs = kb * 32 + half * 16 + 4 * hl;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = db * 32 + c32;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(&vt[buf][d * kVtLd + kofs]);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(&vt[buf][d * kVtLd + kofs + 8]);
        const bf16x8 af = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pb[qb][kstep], oacc[db][qb], 0, 0, 0);
      }
    }

    if (kt + 1 < nkt) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // normalise and store O[s, h, d]: lane holds query c32, d rows
  // 8*(r/4) + 4*hl + (r%4) of each 32-row block -> 4 consecutive d per group
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ltot = lrun[qb] + __shfl_xor(lrun[qb], 32, 64);
    const float inv = 1.0f / ltot;
    const int s = qw0 + qb * 32 + c32;
    if (s >= a.Sq) continue;
    uint16_t* orow = a.o + b * a.os0 + (int64_t)s * a.os1 + h * a.os2;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = db * 32 + grp * 8 + 4 * hl;
        const f32x16& acc = oacc[db][qb];
        *reinterpret_cast<u32x2*>(orow + d) =
            u32x2{pack_bf2(acc[grp * 4 + 0] * inv, acc[grp * 4 + 1] * inv),
                  pack_bf2(acc[grp * 4 + 2] * inv, acc[grp * 4 + 3] * inv)};
      }
  }
}

tp_status attn_prefill(const void* q, const int64_t qs[3], const void* k, const void* v,
                       const int64_t kvs[3], void* o, const int64_t os[3], int64_t B, int64_t Sq,
                       int64_t Skv, int64_t Hq, int64_t Hkv, int causal, float scale,
                       hipStream_t s) {
  PreArgs a;
  a.q = static_cast<const uint16_t*>(q); a.qs0 = qs[0]; a.qs1 = qs[1]; a.qs2 = qs[2];
  a.k = static_cast<const uint16_t*>(k); a.v = static_cast<const uint16_t*>(v);
  a.ks0 = kvs[0]; a.ks1 = kvs[1]; a.ks2 = kvs[2];
  a.o = static_cast<uint16_t*>(o); a.os0 = os[0]; a.os1 = os[1]; a.os2 = os[2];
  a.Sq = (int)Sq; a.Skv = (int)Skv; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.causal = causal;
  a.scale_log2 = scale * 1.4426950408889634f;
  dim3 grid((unsigned)((Sq + kPBQ - 1) / kPBQ), (unsigned)Hq, (unsigned)B), block(256);
  hipLaunchKernelGGL(attn_prefill_kernel, grid, block, 0, s, a);
  TPL_LAUNCH_CHECK("attn_prefill");
  return TP_OK;
}

}  // namespace tpl
