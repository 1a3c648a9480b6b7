// kv4_common.hpp -- geometry of the pools and small device helpers shared by
// the KV4 kernels.  Layouts are documented in include/kv4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv4.h"

namespace kv4 {

constexpr int kPage = 16;        // tokens per page
constexpr int kHalf = 8;         // tokens per V code word
constexpr int kHeadDim = 128;    // head dimension the library supports

// Byte geometry of one cache, derived once on the host and passed by value.
struct Geo {
    int Hq, Hkv, gqa, d, G, ng, S, R, SR;
    int num_layers, num_pages, max_slots, max_pages;
    int kind;
    int rot;                 // 1: keys stored, and queries attended, in the rotated basis
    int intp;                // 1: decode takes the integer path (INT8 q, 8-bit P operand)
    int valu;                // 1: decode on the vector-ALU kernels at every q/kv ratio
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

// The fixed normalized Hadamard transform y = x H / sqrt(128) of a 128-channel
// key or query (Sylvester H; KV4-RL Section 5.1, Appendix A.3 "Encoding and
// allocation"; eq. 3.4 keeps the unquantized scores), in one fixed binary32
// order that every kernel follows so that the stored codes are reproducible:
// butterfly stages of span h = 1, 2, 4, ..., 64, each replacing every channel
// pair (c, c + h), c & h == 0, by (z_c + z_{c+h}, z_c - z_{c+h}), then every
// channel times the binary32 value nearest 1/sqrt(128).  Channels are spread
// over registers and lanes in each kernel's own layout: wht_local runs the
// stages over the channel bits held in one lane's N registers (the low bits),
// wht_lanes one stage whose channel bit is the lane bit `mask`.
constexpr float kWhtScale = 0x1.6a09e6p-4f;

template <int N>
__device__ __forceinline__ void wht_local(float (&v)[N])
{
#pragma unroll
    for (int h = 1; h < N; h <<= 1)
#pragma unroll
        for (int i = 0; i < N; ++i)
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

template <int N>
__device__ __forceinline__ void wht_lanes(float (&v)[N], int mask)
{
    const bool upper = (threadIdx.x & mask) != 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float p = __shfl_xor(v[i], mask);
        v[i] = upper ? p - v[i] : v[i] + p;
    }
}

template <int N>
__device__ __forceinline__ void wht_scale(float (&v)[N])
{
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] *= kWhtScale;
}

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
    g.rot = (c.flags & KV4_FLAG_ROTATE_K) != 0;
    g.intp = (c.flags & KV4_FLAG_INT_PATH) != 0;
    g.valu = (c.flags & KV4_FLAG_VALU_DECODE) != 0;
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
    } else if (c.kind == KV4_KIND_KV8) {
        g.off_kc = 0;                            // K int8 [16][d]
        g.off_vc = kPage * g.d;                  // V int8, 2 channel-major blocks of 8 tokens
        g.off_kdm = 2 * kPage * g.d;             // K scales [16] fp16
        g.off_vm = g.off_kdm + 2 * kPage;        // V scales [16] fp16
        g.off_vd = g.off_vm + 2 * kPage;
        g.pb = g.off_vd;
        g.rb = 0;
        g.SR32 = 0;
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

// ---- binary16 rounding and the INT8 code decision (side entries, KV8 pages
// and the integer path's query).  s = fp16(fp32(amax / 127)); the code is the
// integer in [-127, 127] nearest to the exact x / s, ties to even.
__device__ __forceinline__ uint16_t plus_zero16(uint16_t h) { return h == 0x8000u ? (uint16_t)0 : h; }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f)
{
    _Float16 h = (_Float16)f;     // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Exact decision: a binary64 estimate corrected by the exact binary64
// midpoints (c +- 1/2) s (exact because s is a binary16 value).
__device__ __forceinline__ int int8_code_exact(float x, double S, uint16_t sb)
{
    if (sb == 0) return 0;
    double a = fabs((double)x);
    int c = (int)fmin(fmax(rint(a / S), 0.0), 127.0);
    if (c > 0) {
        double mid = ((double)c - 0.5) * S;
        if (a < mid || (a == mid && (c & 1))) c -= 1;
    }
    if (c < 127) {
        double mid = ((double)c + 0.5) * S;
        if (a > mid || (a == mid && ((c + 1) & 1) == 0)) c += 1;
    }
    return x < 0.0f ? -c : c;
}

// Binary32 fast path: u = |x| rcp(s) has a relative error below 2^-22, so
// farther than 2^-11 from a midpoint (|u| < 128) its nearest integer is the
// exact code; near a midpoint, or for non-finite operands, the exact test decides.
__device__ __forceinline__ int int8_code(float x, float Sf, uint16_t sb)
{
    if (sb == 0) return 0;
    const float u = fabsf(x) * __builtin_amdgcn_rcpf(Sf);
    const float fl = floorf(u);
    const bool near = fabsf(u - fl - 0.5f) < 0x1p-11f && fl <= 126.0f;
    if (near || !(u < 256.0f) || !(Sf < 65536.0f)) return int8_code_exact(x, (double)Sf, sb);
    const int c = (int)fminf(rintf(u), 127.0f);
    return x < 0.0f ? -c : c;
}


// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

}  // namespace kv4
