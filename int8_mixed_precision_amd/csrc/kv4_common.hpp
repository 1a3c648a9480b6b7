// kv4_common.hpp -- geometry of the pools and small device helpers shared by
// the KV4 kernels.  Layouts are documented in include/kv4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv4.h"

namespace kv4 {

constexpr int kPage = 16;        // tokens per page
constexpr int kHalf = 8;         // tokens per V code word
constexpr int kHeadDim = 128;    // head dimension this build supports

// Byte geometry of one cache, derived once on the host and passed by value.
struct Geo {
    int Hq, Hkv, gqa, d, G, ng, S, R, SR;
    int num_layers, num_pages, max_slots, max_pages;
    int kind;
    int64_t pb;              // bytes per (page, kv head) block
    int64_t layer_pages;     // bytes of one layer of the page pool
    int64_t rb;              // bytes per (slot, kv head) ring block
    int SR32;                // ring entries, padded to a multiple of 32
    int64_t layer_side;      // bytes of one layer of the side pool
    // offsets inside a KV4 (page, head) block: K codes, V codes, K (Delta, m)
    // token-major, V m token-major, V Delta group-major
    int off_kc, off_vc, off_kdm, off_vm, off_vd;
};

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

inline Geo make_geo(const kv4_cache_desc& c)
{
    Geo g{};
    g.Hq = c.num_q_heads;
    g.Hkv = c.num_kv_heads;
    g.gqa = c.num_q_heads / c.num_kv_heads;
    g.d = c.head_dim;
    g.G = c.group_size;
    g.ng = c.head_dim / c.group_size;
    g.kind = c.kind;
    g.S = c.kind == KV4_KIND_MIXED ? c.sink : 0;
    g.R = c.kind == KV4_KIND_MIXED ? c.recent : 0;
    g.SR = g.S + g.R;
    g.num_layers = c.num_layers;
    g.num_pages = c.num_pages;
    g.max_slots = c.max_slots;
    g.max_pages = c.max_pages_per_seq;
    if (c.kind == KV4_KIND_MIXED) {
        g.off_kc = 0;
        g.off_vc = kPage * g.d / 2;
        g.off_kdm = kPage * g.d;
        g.off_vm = g.off_kdm + 4 * kPage * g.ng;
        g.off_vd = g.off_vm + 2 * kPage * g.ng;
        g.pb = g.off_vd + 2 * kPage * g.ng;
        g.SR32 = (int)round_up(g.SR, 32);
        g.rb = g.SR > 0 ? (int64_t)g.SR32 * (2 * g.d + 4) : 0;
    } else {
        g.pb = (int64_t)kPage * g.d * 2 * 2;
        g.rb = 0;
        g.SR32 = 0;
    }
    g.layer_pages = (int64_t)g.num_pages * g.Hkv * g.pb;
    g.layer_side = (int64_t)g.max_slots * g.Hkv * g.rb;
    return g;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// Index of channel c's code word inside one 8-token half of a page's V code
// block (d = 128): the four words a lane loads with one 16-byte access belong
// to four 16-channel column blocks of the PV product, and each column block
// lies inside one 32-channel group.
__host__ __device__ __forceinline__ int vpos(int c)
{
    return 64 * (c >> 6) + 4 * (c & 15) + 2 * ((c >> 5) & 1) + ((c >> 4) & 1);
}

// Position of K code word n (channels 8n .. 8n+7, d = 128) inside a token's
// 64-byte code row: word 4 kb + b holds channels 32 b + 8 kb .. +7, so the
// words of the four 32-channel blocks that one lane feeds to the QK product
// are one 16-byte access.
__host__ __device__ __forceinline__ int kpos(int n)
{
    return 4 * (n & 3) + (n >> 2);
}

// Byte of channel c of ring entry e inside the V code region of a ring block:
// entries in blocks of 8, channel-major, channels ordered c%16 then c/16, so
// one lane's eight channels 16 s + n (s = 0..7) of 8 entries are 64
// contiguous bytes.
__host__ __device__ __forceinline__ int ring_vbyte(int e, int c)
{
    return (e >> 3) * (8 * kHeadDim) + ((c & 15) * 8 + (c >> 4)) * 8 + (e & 7);
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

}  // namespace kv4
