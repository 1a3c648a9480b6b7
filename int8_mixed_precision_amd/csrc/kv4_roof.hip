// kv4_roof.hip -- read-bandwidth ceilings of the GPU the decode runs on
// (libkv4_roof.so; include/kv4_roof.h).  Not part of the method: two plain
// read kernels whose achieved rates are the measured second denominator of
// the decode's roofline, next to the published HBM peak.
//
//   stream: a grid-stride read of one contiguous buffer, 16 bytes per lane and
//     8 loads in flight per lane;
//   blocks: every wave reads its list of blocks of `block_bytes` (for the
//     decode: 2,560 B, one (page, kv head) block of the INT4 pool) at ids
//     given by the caller (for the decode: a random permutation), two blocks
//     in flight, 16 bytes per lane -- the decode's own access pattern with
//     no arithmetic.
// Both read with the nontemporal policy, as the decode's tile loads do, and
// fold the data into a value that is written only if it equals a constant
// the data never produces (so the loads are not optimised away and nothing
// is written in practice).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kv4_roof.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ldnt(const u32x4* p)
{
    return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ uint32_t fold(u32x4 v)
{
    return v[0] ^ v[1] ^ v[2] ^ v[3];
}

constexpr uint32_t kNever = 0x9E3779B9u;   // the sink is written only on this value

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, uint64_t n,
                                                          uint32_t* __restrict__ sink)
{
    constexpr int U = 8;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ldnt(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
    }
    for (; i < n; i += stride) acc ^= fold(ldnt(p + i));
    if (acc == kNever) sink[0] = acc;
}

// One wave per workgroup; wave w reads blocks ids[w * per .. (w + 1) * per)
// (per even), two per step, the next step's loads issued before the current
// blocks are folded.  A block is `nu` 16-byte units (at most 64 * 4 = 256).
__global__ __launch_bounds__(64) void block_read_kernel(const uint8_t* __restrict__ pool,
                                                        const int32_t* __restrict__ ids, int per,
                                                        int nu, int nblocks, uint32_t* __restrict__ sink)
{
    constexpr int L = 4;                       // 16-byte loads per lane per block
    const int lane = threadIdx.x;
    const int32_t* my = ids + (size_t)blockIdx.x * per;
    uint32_t acc = 0;
    u32x4 cur[2][L], nxt[2][L];
    auto load = [&](u32x4 (&buf)[2][L], int i) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int id = min(max(my[i + s], 0), nblocks - 1);   // ids are clamped into the pool
            const u32x4* base = reinterpret_cast<const u32x4*>(pool + (size_t)id * (size_t)nu * 16);
#pragma unroll
            for (int k = 0; k < L; ++k) {
                const int idx = lane + 64 * k;
                buf[s][k] = idx < nu ? ldnt(base + idx) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    load(cur, 0);
    for (int i = 0; i < per; i += 2) {
        if (i + 2 < per) load(nxt, i + 2);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int k = 0; k < L; ++k) acc ^= fold(cur[s][k]);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int k = 0; k < L; ++k) cur[s][k] = nxt[s][k];
    }
    if (acc == kNever) sink[blockIdx.x] = acc;
}

int status()
{
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

int kv4_roof_stream_read(const void* buf, size_t bytes, int grid, void* sink, void* stream)
{
    if (buf == nullptr || sink == nullptr || grid < 1 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0)
        return 1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                       (uint64_t)(bytes / 16), static_cast<uint32_t*>(sink));
    return status();
}

int kv4_roof_block_read(const void* pool, size_t pool_bytes, const int32_t* ids, int waves,
                        int blocks_per_wave, int block_bytes, void* sink, void* stream)
{
    if (pool == nullptr || ids == nullptr || sink == nullptr || waves < 1 || blocks_per_wave < 2 ||
        blocks_per_wave % 2 != 0 || block_bytes < 16 || block_bytes % 16 != 0 ||
        block_bytes > 64 * 4 * 16 || reinterpret_cast<uintptr_t>(pool) % 16 != 0)
        return 1;
    const size_t nblocks = pool_bytes / (size_t)block_bytes;
    if (nblocks < 1 || nblocks > (size_t)INT32_MAX) return 1;
    hipLaunchKernelGGL(block_read_kernel, dim3((unsigned)waves), dim3(64), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(pool), ids,
                       blocks_per_wave, block_bytes / 16, (int)nblocks, static_cast<uint32_t*>(sink));
    return status();
}

}  // extern "C"
