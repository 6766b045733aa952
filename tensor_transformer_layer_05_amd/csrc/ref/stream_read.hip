// Attainable HBM read bandwidth reference (measurement infrastructure, not a
// step of the layer): a read-only stream with the decode weight-streaming
// kernels' access shape, so their rates can be set against what a plain read
// of the same width reaches on this GPU.
//
//   * every lane issues 16-byte buffer loads (the GEMV's load width), a wave
//     covering 1 KB per load instruction;
//   * each wave streams its own contiguous slice in chunks of U loads per lane
//     (U KB per wave), double-buffered: the next chunk's loads are issued
//     before the current chunk is consumed, so up to 2 U KB per wave are in
//     flight (the register GEMV keeps two 8 KB chunks per wave in flight:
//     U = 8 with 8 waves per workgroup, one workgroup per CU);
//   * the loaded words are folded with XOR into one word per lane, stored once,
//     so no load can be dropped; the store traffic is negligible.
// Two options: non-temporal loads (the streaming cache policy), and chunks
// interleaved over all waves (wave w reads chunks w, w + nw, w + 2 nw, ... of
// the whole buffer) instead of one contiguous slice per wave.  On MI355X the
// non-temporal loads read 1 GiB at 6.7 TB/s against 5.9 without them.
// Loads past the wave's slice use an offset beyond the buffer resource's bound
// and return zero without touching memory, so the loop has no per-lane branch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/tpref.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOob = 0x80000000u;

template <int U, int AUX, bool SPREAD>
__global__ __launch_bounds__(1024) void stream_read_kernel(const uint8_t* __restrict__ src,
                                                           uint64_t per_wave, uint64_t bytes,
                                                           uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const uint64_t nw = (uint64_t)gridDim.x * (blockDim.x >> 6);
  const uint64_t gw = (uint64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  constexpr uint32_t kChunk = U * 1024u;
  uint64_t begin, len;
  uint32_t nc;
  if constexpr (SPREAD) {   // the whole buffer (below 2 GiB); chunks gw, gw + nw, ...
    begin = 0;
    len = bytes;
    const uint64_t total = (bytes + kChunk - 1) / kChunk;
    nc = gw < total ? (uint32_t)((total - gw + nw - 1) / nw) : 0;
  } else {
    begin = gw * per_wave;
    len = begin < bytes ? (bytes - begin < per_wave ? bytes - begin : per_wave) : 0;
    nc = (uint32_t)((len + kChunk - 1) / kChunk);
  }
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(src + (begin < bytes ? begin : 0)), 0, (uint32_t)len, 0x00020000);
  u32x4 a[U], b[U];
  uint32_t acc = 0;
  auto load = [&](uint32_t c, u32x4 (&v)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t cc = SPREAD ? (uint64_t)c * nw + gw : (uint64_t)c;
      const uint64_t off = cc * kChunk + (uint32_t)u * 1024u + (uint32_t)lane * 16u;
      v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            r, off < len ? (uint32_t)off : kOob, 0, AUX));
    }
  };
  auto fold = [&](const u32x4 (&v)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  };
  if (nc > 0) {
    load(0, a);
    for (uint32_t c = 0; c < nc; c += 2) {
      load(c + 1, b);
      __builtin_amdgcn_sched_barrier(0);
      fold(a);
      __builtin_amdgcn_sched_barrier(0);
      load(c + 2, a);
      __builtin_amdgcn_sched_barrier(0);
      fold(b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  out[gw * 64 + lane] = acc;
}

}  // namespace

template <int U>
static void launch_u(const uint8_t* src, uint64_t per, uint64_t bytes, uint32_t* out, int flags,
                     dim3 grid, dim3 block, hipStream_t s) {
  switch (flags) {
    case 0: hipLaunchKernelGGL((stream_read_kernel<U, 0, false>), grid, block, 0, s, src, per, bytes, out); break;
    case 1: hipLaunchKernelGGL((stream_read_kernel<U, 2, false>), grid, block, 0, s, src, per, bytes, out); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<U, 0, true>), grid, block, 0, s, src, per, bytes, out); break;
    default: hipLaunchKernelGGL((stream_read_kernel<U, 2, true>), grid, block, 0, s, src, per, bytes, out); break;
  }
}

extern "C" int tpref_stream_read(const void* buf, uint64_t bytes, uint32_t* out, int workgroups,
                                 int waves, int loads_per_lane, int flags, void* stream) {
  if (!buf || !out) return 1;
  if (workgroups <= 0 || workgroups > 65536 || (waves != 4 && waves != 8 && waves != 16)) return 2;
  if (bytes == 0 || (reinterpret_cast<uintptr_t>(buf) % 16) != 0) return 2;
  if (flags < 0 || flags > 3 || ((flags & 2) && bytes >= (uint64_t{1} << 31))) return 2;
  const uint64_t nw = (uint64_t)workgroups * waves;
  // each wave's slice is a whole number of 1 KB wave loads, below 2^31 bytes
  const uint64_t per = ((bytes + nw - 1) / nw + 1023) / 1024 * 1024;
  if (per >= (uint64_t{1} << 31)) return 2;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((unsigned)workgroups), block((unsigned)(waves * 64));
  auto src = static_cast<const uint8_t*>(buf);
  switch (loads_per_lane) {
    case 4: launch_u<4>(src, per, bytes, out, flags, grid, block, s); break;
    case 8: launch_u<8>(src, per, bytes, out, flags, grid, block, s); break;
    case 16: launch_u<16>(src, per, bytes, out, flags, grid, block, s); break;
    default: return 2;
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
