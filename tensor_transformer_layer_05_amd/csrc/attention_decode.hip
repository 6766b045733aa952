// Decode attention over a rank's local heads (one query token per sequence).
//
// At decode the key/value cache is the dominant byte stream.  With grouped KV
// heads, G = Hq/Hkv query heads read the same cached keys and values, so one
// workgroup handles ALL G query heads of one (sequence, KV head) pair over a
// contiguous chunk of keys: every cached byte is read exactly once.  The key
// span is split into chunks to give the chip enough workgroups (flash-decoding
// split-KV); each chunk writes an unnormalised partial (running max, sum of
// exponentials, weighted value sum) and a second pass combines the chunks
// with the usual log-sum-exp rescaling, in chunk order.
//
// Inside a workgroup (4 waves): 16 lanes cover one 128-element key row (16
// bytes each), so a wave reads 4 whole rows per load; scores are reduced over
// the 16 lanes with shuffles, kept in LDS, exponentiated per head, and the
// value pass accumulates 8 output elements per lane per head.
#include "common.h"

namespace tpl {

constexpr int kDecD = 128;           // head dimension handled
constexpr int kDecMaxChunk = 512;    // keys per workgroup (LDS score buffer)

struct DecArgs {
  const uint16_t* q; int64_t qs0, qs2;          // (b, h) strides (s = 0)
  const uint16_t* k; const uint16_t* v; int64_t ks0, ks1, ks2;
  uint16_t* o; int64_t os0, os2;
  float* ws;                                    // partials, or nullptr if one chunk
  int Skv, Hq, Hkv, chunk, nsplit;
  float scale_log2;                             // softmax scale * log2(e)
};

template <int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(DecArgs a) {
  __shared__ float qf[G][kDecD];
  __shared__ float sc[G][kDecMaxChunk];
  __shared__ float red[4][G][kDecD];
  __shared__ float stat[G][2];

  const int split = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = split * a.chunk;
  const int t1 = min(a.Skv, t0 + a.chunk);
  const int n = t1 - t0;

  // q of the G heads of this group, scaled into the log2 domain.
  for (int e = tid; e < G * kDecD; e += 256) {
    const int g = e / kDecD, d = e % kDecD;
    const int h = j * G + g;
    qf[g][d] = bf2f(a.q[b * a.qs0 + h * a.qs2 + d]) * a.scale_log2;
  }
  __syncthreads();

  const int sub = lane >> 4;        // which of the 4 rows this lane's group reads
  const int dc = (lane & 15) * 8;   // 8 head elements per lane
  const uint16_t* kb = a.k + b * a.ks0 + j * a.ks2;
  const uint16_t* vb = a.v + b * a.ks0 + j * a.ks2;

  // scores
  for (int base = wave * 4; base < n; base += 16) {
    const int t = base + sub;
    float kf[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (t < n) unpack8(*reinterpret_cast<const u32x4*>(kb + (int64_t)(t0 + t) * a.ks1 + dc), kf);
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(qf[g][dc + e], kf[e], acc);
      s[g] = acc;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) s[g] += __shfl_xor(s[g], o, 16);
    }
    if ((lane & 15) == 0 && t < n) {
#pragma unroll
      for (int g = 0; g < G; ++g) sc[g][t] = s[g];
    }
  }
  __syncthreads();

  // per-head max and exponentials (wave w handles heads w, w+4, ...)
  for (int g = wave; g < G; g += 4) {
    float mx = -INFINITY;
    for (int t = lane; t < n; t += 64) mx = fmaxf(mx, sc[g][t]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int t = lane; t < n; t += 64) {
      const float p = exp2f(sc[g][t] - mx);
      sc[g][t] = p;
      sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) { stat[g][0] = mx; stat[g][1] = sum; }
  }
  __syncthreads();

  // weighted value sum: lane group `sub` of wave `wave` takes rows t = 4*wave + sub (mod 16)
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  for (int t = wave * 4 + sub; t < n; t += 16) {
    float vf[8];
    unpack8(*reinterpret_cast<const u32x4*>(vb + (int64_t)(t0 + t) * a.ks1 + dc), vf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = sc[g][t];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
    }
  }
  // reduce the 4 row groups of a wave (lanes l, l^16, l^32, l^48), then the 4 waves
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[g][e];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      acc[g][e] = x;
    }
  if (sub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][g][dc + e] = acc[g][e];
  }
  __syncthreads();

  for (int e = tid; e < G * kDecD; e += 256) {
    const int g = e / kDecD, d = e % kDecD;
    const float s = ((red[0][g][d] + red[1][g][d]) + red[2][g][d]) + red[3][g][d];
    const int h = j * G + g;
    if (a.ws == nullptr) {
      a.o[b * a.os0 + h * a.os2 + d] = (uint16_t)f2bf_bits(s / stat[g][1]);
    } else {
      // ws layout: [B][Hq][nsplit] x {m, l} followed by [B][Hq][nsplit][D]
      const int64_t row = ((int64_t)b * a.Hq + h) * a.nsplit + split;
      float* ml = a.ws;
      float* ov = a.ws + (int64_t)gridDim.z * a.Hq * a.nsplit * 2;
      ov[row * kDecD + d] = s;
      if (d == 0) { ml[row * 2] = stat[g][0]; ml[row * 2 + 1] = stat[g][1]; }
    }
  }
}

// Combine the chunk partials of one (sequence, head): 128 threads, one per
// output element, chunks visited in order.
__global__ __launch_bounds__(128) void attn_decode_combine_kernel(DecArgs a, int B) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* ml = a.ws;
  const float* ov = a.ws + (int64_t)B * a.Hq * a.nsplit * 2;
  const int64_t row0 = ((int64_t)b * a.Hq + h) * a.nsplit;
  float mx = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) mx = fmaxf(mx, ml[(row0 + s) * 2]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float m = ml[(row0 + s) * 2];
    const float l = ml[(row0 + s) * 2 + 1];
    if (l == 0.f) continue;   // empty chunk
    const float w = exp2f(m - mx);
    num = fmaf(w, ov[(row0 + s) * kDecD + d], num);
    den = fmaf(w, l, den);
  }
  a.o[b * a.os0 + h * a.os2 + d] = (uint16_t)f2bf_bits(num / den);
}

int attn_decode_nsplit(int64_t B, int64_t Hkv, int64_t Skv) {
  const int64_t pairs = B * Hkv;
  int64_t ns = (1024 + pairs - 1) / pairs;                     // aim for ~1024 workgroups
  const int64_t min_ns = (Skv + kDecMaxChunk - 1) / kDecMaxChunk;
  const int64_t max_ns = (Skv + 63) / 64;                      // at least 64 keys per chunk
  if (ns > max_ns) ns = max_ns;
  if (ns < min_ns) ns = min_ns;
  if (ns < 1) ns = 1;
  return (int)ns;
}

size_t attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv) {
  const int ns = attn_decode_nsplit(B, Hkv, Skv);
  if (ns == 1) return 0;
  return (size_t)(B * Hq * ns) * (2 + kDecD) * sizeof(float);
}

template <int G>
static void launch_dec(const DecArgs& a, int B, hipStream_t s) {
  dim3 grid(a.nsplit, a.Hkv, B), block(256);
  hipLaunchKernelGGL((attn_decode_kernel<G>), grid, block, 0, s, a);
  if (a.ws) hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.Hq, B), dim3(128), 0, s, a, B);
}

tp_status attn_decode(const void* q, const int64_t qs[3], const void* k, const void* v,
                      const int64_t kvs[3], void* o, const int64_t os[3], int64_t B, int64_t Skv,
                      int64_t Hq, int64_t Hkv, float scale, void* ws, hipStream_t s) {
  DecArgs a;
  a.q = static_cast<const uint16_t*>(q); a.qs0 = qs[0]; a.qs2 = qs[2];
  a.k = static_cast<const uint16_t*>(k); a.v = static_cast<const uint16_t*>(v);
  a.ks0 = kvs[0]; a.ks1 = kvs[1]; a.ks2 = kvs[2];
  a.o = static_cast<uint16_t*>(o); a.os0 = os[0]; a.os2 = os[2];
  a.Skv = (int)Skv; a.Hq = (int)Hq; a.Hkv = (int)Hkv;
  a.nsplit = attn_decode_nsplit(B, Hkv, Skv);
  a.chunk = (int)((Skv + a.nsplit - 1) / a.nsplit);
  a.ws = a.nsplit > 1 ? static_cast<float*>(ws) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  switch (Hq / Hkv) {
    case 1: launch_dec<1>(a, (int)B, s); break;
    case 2: launch_dec<2>(a, (int)B, s); break;
    case 4: launch_dec<4>(a, (int)B, s); break;
    case 8: launch_dec<8>(a, (int)B, s); break;
    default: return TP_ERR_UNSUPPORTED;
  }
  TPL_LAUNCH_CHECK("attn_decode");
  return TP_OK;
}

}  // namespace tpl
