/*
 * kv4_roof.h -- read-bandwidth ceilings of the GPU (libkv4_roof.so), the
 * measured second denominator of the KV4 decode's HBM roofline.  Not part of
 * the decode method: plain read kernels that fold what they read into a value
 * and write nothing in practice.  Device pointers, asynchronous on `stream`
 * (a hipStream_t, NULL = the default stream); return 0 on success, 1 on an
 * invalid argument or launch error.
 */
#ifndef KV4_ROOF_H
#define KV4_ROOF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Grid-stride read of `bytes` (a multiple of 16, buf 16-byte aligned) with
 * `grid` workgroups of 256 lanes, 16 bytes per lane and 8 loads in flight per
 * lane, nontemporal policy.  sink: device buffer of >= 4 bytes.
 */
int kv4_roof_stream_read(const void* buf, size_t bytes, int grid, void* sink, void* stream);

/*
 * The decode's access pattern without its arithmetic: `waves` one-wave
 * workgroups; wave w reads blocks ids[w * blocks_per_wave ..
 * (w + 1) * blocks_per_wave) of `block_bytes` bytes each (a multiple of 16,
 * at most 4096) from `pool`, two blocks in flight, 16 bytes per lane,
 * nontemporal policy.  ids (device, int32, waves * blocks_per_wave entries)
 * are clamped into [0, pool_bytes / block_bytes); blocks_per_wave is even.
 * sink: device buffer of >= 4 * waves bytes.
 */
int kv4_roof_block_read(const void* pool, size_t pool_bytes, const int32_t* ids, int waves,
                        int blocks_per_wave, int block_bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KV4_ROOF_H */
