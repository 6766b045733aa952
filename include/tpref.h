/*
 * tpref.h -- measurement reference kernels (libtpref.so), not part of the
 * tensor-parallel layer's boundary.  They give the rates the layer's kernels
 * are compared with on the same GPU.
 */
#ifndef TPREF_H
#define TPREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of device memory at `buf` once, as the decode
 * weight-streaming kernels read their weights: 16-byte loads per lane, each
 * wave streaming its own contiguous slice in chunks of `loads_per_lane` KB
 * with the next chunk in flight.  `workgroups` x `waves` waves; one XOR of the
 * loaded words per lane goes to out[wave * 64 + lane] (out holds
 * workgroups * waves * 64 uint32, device).
 * flags: bit 0 = non-temporal loads (streaming cache policy); bit 1 = chunks
 * interleaved over all waves (wave w reads chunks w, w + nw, ... of the whole
 * buffer, nw = workgroups * waves) instead of one contiguous slice per wave.
 *   waves in {4, 8, 16}; loads_per_lane in {4, 8, 16}; buf 16-byte aligned;
 *   1 <= workgroups <= 65536; each wave's slice below 2 GiB; with bit 1 the
 *   whole buffer below 2 GiB; flags in 0..3.
 * Returns 0, 1 (NULL pointer), 2 (bad size or configuration) or 6 (launch
 * failure); asynchronous on `stream` (a hipStream_t, NULL: default stream).
 */
int tpref_stream_read(const void* buf, uint64_t bytes, uint32_t* out, int workgroups, int waves,
                      int loads_per_lane, int flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPREF_H */
