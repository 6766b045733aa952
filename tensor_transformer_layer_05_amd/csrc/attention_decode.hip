// Decode attention over a rank's local heads (one query token per sequence).
//
// At decode the key/value cache is the dominant byte stream.  With grouped KV
// heads, the G = Hq/Hkv query heads of one KV head read the same cached keys
// and values, so one workgroup serves all G heads of one (sequence, KV head)
// pair over a chunk of the key span and every cached byte is read once.  The
// span is split into chunks so that about one workgroup per CU runs
// (flash-decoding split-KV); each chunk writes an unnormalised partial (max,
// sum of exponentials, weighted value sum) and a second pass combines the
// chunks with log-sum-exp rescaling, in chunk order.
//
// The G heads are the query columns of a small attention problem: S^T = K Q^T
// on v_mfma_f32_32x32x16_bf16 with the heads padded to 32 columns (the MFMA
// work is far below the chip's rate at these byte counts), so a lane owns one
// head and 16 of a tile's 32 keys, and the softmax statistics are an
// in-register reduction plus one v_permlane32_swap.  The probabilities feed
// O^T = V^T P^T directly, with V^T read from V ([key][d] in LDS) by
// ds_read_b64_tr_b16 (the layouts of the prefill kernel).
//
// Each of the 4 waves streams its own contiguous run of 32-key tiles through
// a private two-stage LDS ring with buffer_load_dwordx4 ... lds (1 KB = 4 key
// rows per load, rows past the span reading as zero): the next tile's K and V
// are in flight while the current one is computed, with an online softmax
// across tiles.  There is no barrier in the loop; the waves' (max, sum, O^T)
// are merged through LDS at the end.
#include "common.h"

namespace tpl {

constexpr int kDecD = 128;           // head dimension handled
constexpr int kDecTile = 32;         // keys per tile
constexpr int kDecMaxG = 32;         // query heads per KV head (MFMA columns)

struct DecArgs {
  const uint16_t* q; int64_t qs0, qs2;          // (b, h) strides (s = 0)
  const uint16_t* k; const uint16_t* v; int64_t ks0, ks1, ks2;
  uint16_t* o; int64_t os0, os2;
  float* ws;                                    // partials, or nullptr if one chunk
  int Skv, Hq, Hkv, G, nsplit, chunk;           // chunk: keys per workgroup (multiple of 4*32)
  float scale_log2;                             // softmax scale * log2(e)
};

namespace {
typedef short dec_s16x4 __attribute__((ext_vector_type(4)));
#define TPL_DLDS __attribute__((address_space(3)))

__device__ __forceinline__ float dec_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float dec_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
}  // namespace

__global__ __launch_bounds__(256) void attn_decode_kernel(DecArgs a) {
  constexpr int TE = kDecTile * kDecD;                 // bf16 elements of one K (or V) tile
  constexpr int WRING = 2 * 2 * TE;                    // per wave: 2 stages x (K, V)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * WRING];   // 128 KB
  __shared__ float wstat[4][kDecMaxG][2];

  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, hl = lane >> 5;
  const int G = a.G;
  const int wkeys = a.chunk / 4;                       // keys per wave (multiple of 32)
  const int tw = split * a.chunk + wave * wkeys;       // first key of this wave
  const int nt = max(0, min(wkeys, a.Skv - tw) + kDecTile - 1) / kDecTile;   // tiles with keys

  const uint32_t nrec = (uint32_t)(((int64_t)(a.Skv - 1) * a.ks1 + kDecD) * 2);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + b * a.ks0 + j * a.ks2), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v + b * a.ks0 + j * a.ks2), 0, nrec, 0x00020000);
  TPL_DLDS uint16_t* ring = (TPL_DLDS uint16_t*)lds + wave * WRING;
  const int lr = lane >> 4, lp = lane & 15;
  // tile i of this wave -> stage i & 1: 8 loads of 4 rows for K, 8 for V
  auto issue = [&](int i) {
    TPL_DLDS uint16_t* kd = ring + (i & 1) * 2 * TE;
    TPL_DLDS uint16_t* vd = kd + TE;
#pragma unroll
    for (int u = 0; u < kDecTile / 4; ++u) {
      const int row = 4 * u + lr;
      const int t = tw + i * kDecTile + row;
      const bool ok = t < a.Skv && i < nt;
      const uint32_t rb = (uint32_t)((int64_t)t * a.ks1 * 2);
      const int kc = lp ^ (row & 15), vc = lp ^ (4 * (row & 3));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (TPL_DLDS void*)(kd + u * 4 * kDecD), 16,
                                               ok ? rb + (uint32_t)kc * 16u : 0x80000000u, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (TPL_DLDS void*)(vd + u * 4 * kDecD), 16,
                                               ok ? rb + (uint32_t)vc * 16u : 0x80000000u, 0, 0, 0);
    }
  };
  issue(0);

  // Q^T fragments: column c32 = query head j*G + c32 (zero past G), d = 16 kk + 8 hl .. +7
  bf16x8 qf[8];
  {
    const bool hv = c32 < G;
    const uint16_t* qrow = a.q + b * a.qs0 + (int64_t)(j * G + (hv ? c32 : 0)) * a.qs2;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v4 = *reinterpret_cast<const u32x4*>(qrow + kk * 16 + hl * 8);
      if (!hv) v4 = u32x4{0u, 0u, 0u, 0u};
      qf[kk] = as_bf16x8(v4);
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const int g16 = lane >> 4, sidx = lane & 15;
  const int tr_row = sidx >> 2, tr_d = 16 * (g16 & 1) + 4 * (sidx & 3);

  for (int i = 0; i < nt; ++i) {
    // the other stage was last read by tile i-1, whose reads completed before its MFMAs
    issue(i + 1);
    __builtin_amdgcn_s_waitcnt((16 & 15) | ((16 >> 4) << 14) | 0x0F70);   // tile i landed; tile i+1 (16 loads) may pend
    const uint16_t* ks = lds + wave * WRING + (i & 1) * 2 * TE;
    const uint16_t* vs = ks + TE;
    f32x16 st;
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int ch = (2 * kk + hl) ^ (c32 & 15);
      const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + c32 * kDecD + ch * 8));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], st, 0, 0, 0);
    }
    // online softmax for column c32 over this tile's 32 keys (16 here, 16 in lane ^ 32)
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = tw + i * kDecTile + 8 * (r >> 2) + 4 * hl + (r & 3);
      const float x = t < a.Skv ? st[r] * a.scale_log2 : -INFINITY;
      st[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = dec_pair_max(mx);
    const float mnew = fmaxf(mrun, mx);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = exp2f(mrun - muse);
    mrun = mnew;
    bf16x8 pb[2];
    float psum = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2f(st[half * 8 + e] - muse);
        psum += p[e];
      }
      pb[half] = as_bf16x8(pack8(p));
    }
    lrun = lrun * alpha + psum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    // O^T[d, col] += V^T[d, keys] P^T[keys, col]; step `half` covers keys
    // 16 half + {4 hl + 0..3, 8 + 4 hl + 0..3} (the P^T register order)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k0 = half * 16 + 4 * hl;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + tr_d;
        const int r0 = k0 + tr_row, r1 = k0 + 8 + tr_row;
        const dec_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (TPL_DLDS dec_s16x4*)((TPL_DLDS uint16_t*)vs + r0 * kDecD + ((d >> 3) ^ (4 * (r0 & 3))) * 8 + (d & 7)));
        const dec_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (TPL_DLDS dec_s16x4*)((TPL_DLDS uint16_t*)vs + r1 * kDecD + ((d >> 3) ^ (4 * (r1 & 3))) * 8 + (d & 7)));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{l2[0], l2[1], h2[0], h2[1]}),
                                                           pb[half], oacc[db], 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // the trailing (out-of-range) DMA has landed
  const float lsum = dec_pair_sum(lrun);

  // merge the 4 waves: per column, O = sum_w 2^(m_w - m) O_w, L = sum_w 2^(m_w - m) l_w
  __syncthreads();   // every wave is done with its ring
  float* red = reinterpret_cast<float*>(lds);   // [4 waves][32 cols][128 d]
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = db * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
      red[(wave * kDecMaxG + c32) * kDecD + d] = oacc[db][r];
    }
  if (hl == 0) { wstat[wave][c32][0] = mrun; wstat[wave][c32][1] = lsum; }
  __syncthreads();
  for (int e = tid; e < G * kDecD; e += 256) {
    const int c = e / kDecD, d = e % kDecD;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, wstat[w][c][0]);
    const float mu = (m == -INFINITY) ? 0.f : m;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = exp2f(wstat[w][c][0] - mu);
      num = fmaf(sc, red[(w * kDecMaxG + c) * kDecD + d], num);
      den = fmaf(sc, wstat[w][c][1], den);
    }
    const int h = j * G + c;
    if (a.ws == nullptr) {
      a.o[b * a.os0 + h * a.os2 + d] = (uint16_t)f2bf_bits(num / den);
    } else {
      // ws layout: [B][Hq][nsplit] x {m, l} followed by [B][Hq][nsplit][D]
      const int64_t row = ((int64_t)b * a.Hq + h) * a.nsplit + split;
      float* ml = a.ws;
      float* ov = a.ws + (int64_t)gridDim.z * a.Hq * a.nsplit * 2;
      ov[row * kDecD + d] = num;
      if (d == 0) { ml[row * 2] = m; ml[row * 2 + 1] = den; }
    }
  }
}

// Combine the chunk partials of one (sequence, head): 128 threads, one per
// output element, chunks visited in order.  Partials are loaded 8 chunks at a
// time (indices clamped into range and masked afterwards, so the loads carry
// no branches and are all in flight together).
__global__ __launch_bounds__(128) void attn_decode_combine_kernel(DecArgs a, int B) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* ml = a.ws;
  const float* ov = a.ws + (int64_t)B * a.Hq * a.nsplit * 2;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.nsplit;
  const int ns = a.nsplit;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float m[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = ml[(row0 + min(s0 + u, ns - 1)) * 2];
#pragma unroll
    for (int u = 0; u < 8; ++u) mx = fmaxf(mx, m[u]);   // clamped duplicates do not change the max
  }
  float num = 0.f, den = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float m[8], l[8], o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t r = row0 + min(s0 + u, ns - 1);
      m[u] = ml[r * 2];
      l[u] = ml[r * 2 + 1];
      o[u] = ov[r * kDecD + d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool use = s0 + u < ns && l[u] != 0.f;   // past the end, or an empty chunk
      const float w = use ? exp2f(m[u] - mx) : 0.f;
      num = fmaf(w, use ? o[u] : 0.f, num);
      den = fmaf(w, use ? l[u] : 0.f, den);
    }
  }
  a.o[b * a.os0 + h * a.os2 + d] = (uint16_t)f2bf_bits(num / den);
}

// Chunks of whole 4 x 32-key tiles per workgroup, about one workgroup per CU
// (256) over all (sequence, KV head) pairs.
static int dec_chunk(int64_t B, int64_t Hkv, int64_t Skv) {
  const int64_t pairs = B * Hkv;
  int64_t ns = (256 + pairs - 1) / pairs;
  const int64_t max_ns = (Skv + 4 * kDecTile - 1) / (4 * kDecTile);
  if (ns > max_ns) ns = max_ns;
  if (ns < 1) ns = 1;
  int64_t chunk = (Skv + ns - 1) / ns;
  chunk = (chunk + 4 * kDecTile - 1) / (4 * kDecTile) * (4 * kDecTile);
  return (int)chunk;
}

int attn_decode_nsplit(int64_t B, int64_t Hkv, int64_t Skv) {
  const int64_t chunk = dec_chunk(B, Hkv, Skv);
  return (int)((Skv + chunk - 1) / chunk);
}

size_t attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv) {
  const int ns = attn_decode_nsplit(B, Hkv, Skv);
  if (ns == 1) return 0;
  return (size_t)(B * Hq * ns) * (2 + kDecD) * sizeof(float);
}

tp_status attn_decode(const void* q, const int64_t qs[3], const void* k, const void* v,
                      const int64_t kvs[3], void* o, const int64_t os[3], int64_t B, int64_t Skv,
                      int64_t Hq, int64_t Hkv, float scale, void* ws, hipStream_t s) {
  DecArgs a;
  a.q = static_cast<const uint16_t*>(q); a.qs0 = qs[0]; a.qs2 = qs[2];
  a.k = static_cast<const uint16_t*>(k); a.v = static_cast<const uint16_t*>(v);
  a.ks0 = kvs[0]; a.ks1 = kvs[1]; a.ks2 = kvs[2];
  a.o = static_cast<uint16_t*>(o); a.os0 = os[0]; a.os2 = os[2];
  a.Skv = (int)Skv; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / Hkv);
  if (a.G > kDecMaxG) return TP_ERR_UNSUPPORTED;
  a.chunk = dec_chunk(B, Hkv, Skv);
  a.nsplit = attn_decode_nsplit(B, Hkv, Skv);
  a.ws = a.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_decode_kernel, dim3(a.nsplit, a.Hkv, B), dim3(256), 0, s, a);
  if (a.ws) hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.Hq, B), dim3(128), 0, s, a, (int)B);
  TPL_LAUNCH_CHECK("attn_decode");
  return TP_OK;
}

}  // namespace tpl
