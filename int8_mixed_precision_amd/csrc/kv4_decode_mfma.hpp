// kv4_decode_mfma.hpp -- matrix-core (MFMA) decode attention for GQA group 4.
//
// One wave per work item (sequence, kv head, context split); the split is
// walked in 32-token tiles (two pages).  Both contractions of a tile run on
// 16x16x32 MFMAs with fp32 accumulation:
//
//   QK (INT4 keys, v_mfma_f32_16x16x32_f16): rows = (q head j, 32-channel
//     block g), k = the 32 channels of one block, columns = 16 tokens.  Row
//     (j, g) carries q_j only when g is the block of the k-slots, so four
//     MFMAs leave every per-block product q_{j,g} . c_{t,g} in one
//     accumulator, and the affine identity q.k^ = sum_g Delta_g (q_g . c_g) +
//     m_g sum(q_g) (KV4-RL eq. 5.1, applied per group) gives the scores in-lane.
//   PV (INT4 values, v_mfma_f32_16x16x32_bf16): rows = (q head j, block g),
//     k = 32 tokens, columns = 16 channels of one block.  Row (j, g) carries
//     p_{j,t} Delta_{t,g}, so the per-token, per-group scale of eq. 3.3 is
//     applied exactly before the token sum; the offset term sum_t p m is
//     accumulated on the vector ALU.
//
// Exactness: codes enter the matrix core as subnormal numbers whose mantissa
// is the code (K: fp16, code * 2^-24 or 16 code * 2^-24; V: bf16, code *
// 2^-133), so widening is a mask (and one shift per two pairs) and needs no
// bias.  q is scaled by a power of two per head and is exact in fp16 (a query
// rotated into the keys' basis is a binary32 value, rounded to fp16); the
// bf16 A operand of PV is split as hi + lo (both rounded to nearest), which
// carries p*Delta to about 2^-18 relative.  The power-of-two scales are
// undone in the score factor and in the epilogue.
//
// Masking: tokens outside the work item (and never-written slots of a page)
// get score -inf and weight exactly 0 by selection, so garbage bytes can
// never reach the result.
#pragma once

#include <type_traits>

#include "kv4_decode.hpp"

namespace kv4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_f16(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Eight 4-bit K codes (code e in bits 4e..4e+3) -> four fp16 pairs whose bit
// patterns are subnormal numbers, exact multiples of 2^-24: pair 0 = codes
// (0, 4) and pair 2 = codes (2, 6) hold code * 2^-24, pairs 1 = (1, 5) and
// 3 = (3, 7) hold 16 code * 2^-24 (the nibble sits in mantissa bits 4..7).
// The A operand carries q / 16 in the k-slots of pairs 1 and 3.  One shift and
// four ands per word; the matrix core keeps fp16 subnormal inputs.
__device__ __forceinline__ u32x4_t widen_k16(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    u32x4_t r;
    r[0] = w & 0x000F000Fu;
    r[1] = w & 0x00F000F0u;
    r[2] = w8 & 0x000F000Fu;
    r[3] = w8 & 0x00F000F0u;
    return r;
}

// Eight 4-bit V codes -> four bf16 pairs holding code * 2^-133 exactly (bf16
// subnormals, mantissa = code); pair i = (code i, code i+4).  The A operand is
// pre-scaled so that the products are normal fp32 numbers.
__device__ __forceinline__ u32x4_t widen_v(uint32_t w)
{
    const uint32_t M = 0x000F000Fu;
    u32x4_t r;
    r[0] = w & M;
    r[1] = (w >> 4) & M;
    r[2] = (w >> 8) & M;
    r[3] = (w >> 12) & M;
    return r;
}

// Sum over the 4 lanes of a quad (lanes 4k..4k+3).
__device__ __forceinline__ float quad_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    return x;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float x, float y)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}

// Two fp32 values -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16(float x, float y)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, f16x2_t));
}

// Split (x, y) into bf16 high parts (nearest) and bf16 remainders (nearest):
// x = hi + lo + O(2^-18 |x|).
__device__ __forceinline__ void split_bf16(float x, float y, uint32_t& hi, uint32_t& lo)
{
    hi = pack_bf16(x, y);
    lo = pack_bf16(x - __uint_as_float(hi << 16), y - __uint_as_float(hi & 0xFFFF0000u));
}

// x where the lane's bit of `lanes` is set, else 0 (v_cndmask_b32).  Volatile:
// the QK loop rebuilds its block-diagonal operand from 4 registers every tile
// instead of keeping four 4-register copies, three of them zero, alive.
__device__ __forceinline__ uint32_t keep_lanes(uint32_t x, uint64_t lanes)
{
    uint32_t r;
    asm volatile("v_cndmask_b32_e64 %0, 0, %1, %2" : "=v"(r) : "v"(x), "s"(lanes));
    return r;
}

// Maximum over the four 16-lane rows, for every column (v_permlane*_swap).
__device__ __forceinline__ float rows_max(float x)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float x)
{
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float h2f(uint32_t w, int k)
{
    return (float)__builtin_bit_cast(f16x2_t, w)[k];
}

// DPP move inside a 16-lane row (bound_ctrl: every source lane is in the row).
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Maximum and sum over the 16 lanes of a row (quad swaps, then row rotations).
// The maximum is one v_max_f32 with a DPP source per step (a separate DPP move
// would need an extra canonicalising max); s_nop 1 covers the VALU-write to
// DPP-read hazard.  Inputs are finite or -inf.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ float row16_max(float x)
{
    asm volatile("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
                 "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
                 "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
                 "s_nop 1\n\tv_max_f32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
                 "s_nop 1"
                 : "+v"(x));
    return x;
}
#pragma clang diagnostic pop

__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x124>(x);
    return x + dpp<0x128>(x);
}

// The exponentials of an INT4 work item use a reference maximum m_ref that is
// raised only when a tile's maximum exceeds it by more than kSlack (base-2
// units), so accumulators are rescaled rarely; the running sum uses the same
// reference, which keeps the result exact.  The weights are also carried
// scaled by 2^kPScale (p' = 2^(s - m_ref + kPScale) <= 2^64), so that the
// products p' Delta code 2^-133 of the value contraction are normal fp32
// numbers whenever p Delta code >= 2^-41; p' Delta <= 2^80 stays inside bf16
// and every sum over 2^24 tokens inside fp32.
constexpr float kSlack = 16.0f;
constexpr float kPScale = 48.0f;

// One lane's loads for one 32-token tile (pages P0 = tokens 0..15 and
// P1 = tokens 16..31).  The tile's metadata (K (Delta, m), V m, V Delta of
// both pages: 2 x 128 NG bytes) is loaded once, 16 bytes per lane, and
// shared through LDS, instead of each lane loading the copies it needs.
// The registers are only the landing zone of the loads: at the start of the
// tile they belong to they are copied to a per-wave LDS stage and refilled
// with the next tile at once, so every load has a whole tile to arrive.
struct Kv4Tile {
    uint4 kc[2];              // K code words of token n16 of each page, channels 8 kb + 32 b (word b)
    uint4 vc0, vc1;           // V code words of channels 16 s + n16 for tokens 8 kb .. 8 kb + 7
    uint4 meta;               // 16-byte chunk lane % 32 of the metadata of page lane / 32
};

// Loads of one page block through a buffer descriptor: wave-uniform base in
// SGPRs, 32-bit lane offset, and a range of exactly one page block (reads
// past it return zero).
typedef __amdgpu_buffer_rsrc_t Page;

__device__ __forceinline__ Page page_rsrc(const uint8_t* p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0, bytes, 0x00020000);
}

// The INT4 tiles' bytes are read once per step, so their loads carry the
// nontemporal policy (the nt bit, cache-policy immediate 2 on gfx950): random
// 2.5 KB page blocks then stream at about 6.6-6.8 TB/s on MI355X, against
// about 5.7 TB/s with the default policy.  Each of those loads covers whole
// 128-byte lines.  The INT8 parts (protected ring, KV8 pages) keep the default
// policy: a lane there reads 32 contiguous bytes in two 16-byte loads, each of
// which covers half of every line it touches, and with the nontemporal policy
// that pattern measured much slower (KV8 decode 522 -> 682 us).
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ uint4 ld16(Page r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// A 16-byte global load of cache bytes with the nontemporal policy.
__device__ __forceinline__ uint4 ldg_stream(const void* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Per-lane byte offsets of the loads inside a page block.
struct Kv4Offs {
    uint32_t kc, vc, meta;
};

__device__ __forceinline__ void load_k_codes(Kv4Tile& t, Page P0, Page P1, const Kv4Offs& o)
{
    t.kc[0] = ld16(P0, o.kc);
    t.kc[1] = ld16(P1, o.kc);
}

// Per-lane pages (an ordinary per-lane address: a buffer descriptor would
// have to be wave-uniform): PV-role V codes of page kb / 2, metadata chunk
// of page lane / 32.
__device__ __forceinline__ void load_v_codes(Kv4Tile& t, const uint8_t* PM, const Kv4Offs& o)
{
    t.vc0 = ldg_stream(PM + o.vc);
    t.vc1 = ldg_stream(PM + o.vc + 4 * 64);
}

__device__ __forceinline__ void load_meta(Kv4Tile& t, const uint8_t* PH, const Kv4Offs& o)
{
    t.meta = ldg_stream(PH + o.meta);
}

// ---------------------------------------------------------------------------
// INT4 context split of the mixed cache, GQA group 4.  Lane roles
// (n16 = lane % 16, kb = lane / 16):
//   QK, transposed: A = scaled q in fp16, block-diagonal, row n16 = (head
//     n16/4, block n16%4) holding q of that head on that 32-channel block,
//     k = the 32 channels of block b (so only b = n16%4 is non-zero); B = K
//     codes of block b as fp16 subnormals, column = token n16 of a page,
//     k = channels 32 b + 8 kb ...  The four blocks accumulate into one D, so
//     lane l holds q_{kb,r} . c over block r of token n16 in D[r], for head
//     kb, and the score follows in-lane.
//   PV: A = w = p' Delta_V, row n16 = (head n16/4, block n16%4), k = tile
//     tokens 8 kb .. 8 kb + 7, split into bf16 hi + lo; B = V codes as bf16
//     subnormals.  Only D row (head, block r) of the accumulator for channels
//     32 r + 16 h + n16 is wanted, so each of the four blocks keeps the A rows
//     of its own block (the rest are zeroed) and two accumulators E[0], E[1]
//     cover all 128 channels: lane l holds head kb, channel 32 r + 16 h + n16
//     in E[h][r];
//     the m_V term sum p' m is accumulated on the vector ALU in the QK layout.
//   Probabilities move from the QK layout to the PV layout through LDS.
// Masking: tokens outside the work item (and never-written slots of a page)
// get score -inf, probability 0 and weight exactly 0 by selection, so garbage
// bytes never reach the result.
// ---------------------------------------------------------------------------
// A rotated query (ROT) is a binary32 value; its fp16 operand is then split
// into hi + lo (both rounded to nearest, ~22 significant bits together) and
// QK runs both halves, since one fp16 rounding costs ~3e-4 of a score.
__device__ __forceinline__ uint2 split_f16(float x, float y)
{
    const uint32_t hi = pack_f16(x, y);
    return make_uint2(hi, pack_f16(x - h2f(hi, 0), y - h2f(hi, 1)));
}

// NH = 2 (q/kv ratio 8): the wave runs the tile's QK, softmax and PV for q
// heads 0-3 and then 4-7 of the group on the same staged K/V tile, each half
// with its own query operands, softmax state and accumulators.
template <int G, bool ROT, int NH = 1>
__device__ __forceinline__ void mfma_item_kv4(const DecodeArgs& a, int b, int h, int t_lo, int t_hi,
                                              float* rec, Pace& pace)
{
    constexpr int NG = kHeadDim / G;
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int jq = n16 >> 2, gq = n16 & 3;       // A row (head, block) of this lane
    if (t_hi <= t_lo) return;

    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    const uint8_t* hbase = a.pages + (int64_t)a.layer * g.layer_pages + (int64_t)h * g.pb;
    const int64_t page_stride = (int64_t)g.Hkv * g.pb;

    // ---- q: block-diagonal A operands and block sums
    // A carries q_j scaled by 2^sc_j, with sc_j chosen so that max |q_j| * 2^sc_j
    // lies in [2^14, 2^15): every bf16 element of q above 2^-31 max |q_j| is then
    // exact in fp16 (a power-of-two scale; a rotated query is rounded to its
    // 11 significant bits), and the k-slots facing codes stored at 16 times
    // their value get a further 2^-4.
    u32x4_t aqv[NH];                             // scaled q of head jq on block gq (k-slot pairs)
    u32x4_t aql[NH];                             // its low half (rotated queries only)
    float sqm[NH][NG];                           // m-term factors and score factor of head kb
    float c2[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        float sq_part;
        int sc;                                  // scale exponent of head jq
        aql[hf] = u32x4_t{0u, 0u, 0u, 0u};
        {
            // rows of heads past the q/kv ratio (GQA 1 and 2 run in the four-head
            // layout) carry q = 0; their results are not written
            const int jh = 4 * hf + jq;
            const bool qreal = jh < g.gqa;
            const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * g.gqa + (qreal ? jh : 0)) * g.d;
            uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * gq + 8 * kb);
            if (!qreal) u = make_uint4(0u, 0u, 0u, 0u);
            float q[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                          bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
            if constexpr (ROT) {
                // query into the keys' basis: channel bits 3-4 are lane bits 4-5
                // (kb), bits 5-6 lane bits 0-1 (gq)
                wht_local(q);
                wht_lanes(q, 16);
                wht_lanes(q, 32);
                wht_lanes(q, 1);
                wht_lanes(q, 2);
                wht_scale(q);
            }
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(q[c]));
            amax = fmaxf(amax, dpp<0xB1>(amax));                 // over the quad (blocks) ...
            amax = rows_max(fmaxf(amax, dpp<0x4E>(amax)));       // ... and the rows: head jq
            sc = 15 - __builtin_amdgcn_frexp_expf(amax);
            // k-slot pairs (c, c + 4) of channels 32 gq + 8 kb + c, as widen_k16() pairs codes
            if constexpr (ROT) {
                const uint2 s0 = split_f16(ldexpf(q[0], sc), ldexpf(q[4], sc));
                const uint2 s1 = split_f16(ldexpf(q[1], sc - 4), ldexpf(q[5], sc - 4));
                const uint2 s2 = split_f16(ldexpf(q[2], sc), ldexpf(q[6], sc));
                const uint2 s3 = split_f16(ldexpf(q[3], sc - 4), ldexpf(q[7], sc - 4));
                aqv[hf] = u32x4_t{s0.x, s1.x, s2.x, s3.x};
                aql[hf] = u32x4_t{s0.y, s1.y, s2.y, s3.y};
            } else {
                aqv[hf][0] = pack_f16(ldexpf(q[0], sc), ldexpf(q[4], sc));
                aqv[hf][1] = pack_f16(ldexpf(q[1], sc - 4), ldexpf(q[5], sc - 4));
                aqv[hf][2] = pack_f16(ldexpf(q[2], sc), ldexpf(q[6], sc));
                aqv[hf][3] = pack_f16(ldexpf(q[3], sc - 4), ldexpf(q[7], sc - 4));
            }
            // the sum of q as the matrix core sees it, so that the offset term
            // m sum(q) matches the products
            auto opsum = [&](const u32x4_t& o, int i, int j) {
                return (h2f(o[i], 0) + h2f(o[i], 1)) + (h2f(o[j], 0) + h2f(o[j], 1));
            };
            float e0 = opsum(aqv[hf], 0, 2), e1 = opsum(aqv[hf], 1, 3);
            if constexpr (ROT) {
                e0 += opsum(aql[hf], 0, 2);
                e1 += opsum(aql[hf], 1, 3);
            }
            sq_part = ldexpf(fmaf(16.0f, e1, e0), -sc);
        }
        // sum of q over block gq of head jq (the four lanes of A row n16), then
        // the sums of head kb over each block r, for this lane's D rows
        const float sq_blk = rows_sum(sq_part);
        float sqr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sqr[r] = __shfl(sq_blk, 4 * kb + r);
        // D rows of this lane belong to head kb: its products come scaled by
        // 2^(sc_kb - 24); the offset term is scaled alike and the score factor
        // undoes it.
        const int sc_d = __shfl(sc, 4 * kb) - 24;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            sqm[hf][gg] = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if ((32 * r) / G == gg) sqm[hf][gg] += sqr[r];
            sqm[hf][gg] = ldexpf(sqm[hf][gg], sc_d);
        }
        c2[hf] = ldexpf(a.scale2, -sc_d);
    }

    // E[hf][h]: rows (head, block r), channels 32 r + 16 h + n16 (block-diagonal PV)
    f32x4_t E[NH][2];
    float accm[NH][NG];
    float m_sh[NH], l_run[NH];                   // m_sh = m_ref - kPScale
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        E[hf][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        E[hf][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) accm[hf][gg] = 0.f;
        m_sh[hf] = -INFINITY;
        l_run[hf] = 0.f;
    }

    // fixed per-lane offsets inside a page block
    constexpr int MB = 128 * NG;                 // metadata bytes per page
    Kv4Offs o;
    o.kc = (uint32_t)(g.off_kc + n16 * (kHeadDim / 2) + 16 * kb);
    o.vc = (uint32_t)(g.off_vc + 4 * ((kb & 1) * g.d + 4 * n16));
    const int chunk = lane & 31;                 // metadata chunk of this lane
    const bool chunk_ok = 16 * chunk < MB;
    o.meta = (uint32_t)(g.off_kdm + 16 * (chunk_ok ? chunk : 0));
    // byte offsets of this lane's metadata inside the LDS copy of a page's
    const int m_kdm = n16 * 4 * NG;                              // K (Delta, m) of token n16
    const int m_vm = 64 * NG + n16 * 2 * NG;                     // V m of token n16
    const int m_vd = (kb >> 1) * MB + 96 * NG + 2 * (((32 * gq) / G) * kPage + 8 * (kb & 1));

    // Page ids come through the scalar cache (the block table is read-only
    // during the kernel), ahead of their use.
    const int tile_first = t_lo / 32, tile_end = (t_hi + 31) / 32;
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    const const_i32 btc = (const_i32)bt;
    const int pb_bytes = (int)g.pb;
    auto page = [&](int pi) -> const uint8_t* {
        const int p = clampi(btc[min(pi, g.max_pages - 1)], 0, g.num_pages - 1);
        return hbase + (int64_t)p * page_stride;
    };
    const bool upper = kb >> 1;                  // lanes 32-63: PV tokens and metadata chunk in page 2

    __shared__ __attribute__((aligned(16))) float pbuf[NH][4][32];
    __shared__ __attribute__((aligned(16))) uint8_t mbuf[2 * 512];
    __shared__ uint4 stage[4][64];               // K codes of both pages, V codes, per lane

    auto load_tile = [&](Kv4Tile& t, const uint8_t* N0, const uint8_t* N1) {
        load_k_codes(t, page_rsrc(N0, pb_bytes), page_rsrc(N1, pb_bytes), o);
        const uint8_t* PM = upper ? N1 : N0;
        load_v_codes(t, PM, o);
        load_meta(t, PM, o);
    };

    // One tile: stage tile tl from the landing registers t into LDS, refill t
    // from pages (N0, N1), then compute from the stage.
    auto step = [&](Kv4Tile& t, int tl, const uint8_t* N0, const uint8_t* N1, auto full_tag) {
        constexpr bool full = decltype(full_tag)::value;
        // ---- this tile's data to LDS, then refill the landing registers
        stage[0][lane] = t.kc[0];
        stage[1][lane] = t.kc[1];
        stage[2][lane] = t.vc0;
        stage[3][lane] = t.vc1;
        if (chunk_ok) *reinterpret_cast<uint4*>(&mbuf[(lane >> 5) * MB + 16 * chunk]) = t.meta;
        __builtin_amdgcn_wave_barrier();
        load_tile(t, N0, N1);
        const uint4 kc0 = stage[0][lane], kc1 = stage[1][lane];
        uint32_t kdm[2][NG];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint8_t* src = &mbuf[hh * MB + m_kdm];
            if constexpr (NG == 4) {
                const uint4 u = *reinterpret_cast<const uint4*>(src);
                kdm[hh][0] = u.x; kdm[hh][1] = u.y; kdm[hh][2] = u.z; kdm[hh][3] = u.w;
            } else if constexpr (NG == 2) {
                const uint2 u = *reinterpret_cast<const uint2*>(src);
                kdm[hh][0] = u.x; kdm[hh][1] = u.y;
            } else {
                kdm[hh][0] = *reinterpret_cast<const uint32_t*>(src);
            }
        }

        // ---- QK, block by block: D_hh[r] = q_{kb,r} . c over block r, token
        // n16 of page hh; each block's widened K codes serve every half of the
        // q heads (one half below ratio 8)
        f32x4_t D0[NH], D1[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            D0[hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            D1[hf] = D0[hf];
        }
        {
            const uint32_t k0w[4] = {kc0.x, kc0.y, kc0.z, kc0.w};
            const uint32_t k1w[4] = {kc1.x, kc1.y, kc1.z, kc1.w};
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                // block-diagonal A: only rows of block bb (lanes with lane % 4 == bb) carry q
                const uint64_t rows = 0x1111111111111111ull << bb;
                const u32x4_t B0 = widen_k16(k0w[bb]), B1 = widen_k16(k1w[bb]);
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    const u32x4_t A = {keep_lanes(aqv[hf][0], rows), keep_lanes(aqv[hf][1], rows),
                                       keep_lanes(aqv[hf][2], rows), keep_lanes(aqv[hf][3], rows)};
                    D0[hf] = mfma_f16(A, B0, D0[hf]);
                    D1[hf] = mfma_f16(A, B1, D1[hf]);
                    if constexpr (ROT) {
                        const u32x4_t Al = {keep_lanes(aql[hf][0], rows), keep_lanes(aql[hf][1], rows),
                                            keep_lanes(aql[hf][2], rows), keep_lanes(aql[hf][3], rows)};
                        D0[hf] = mfma_f16(Al, B0, D0[hf]);
                        D1[hf] = mfma_f16(Al, B1, D1[hf]);
                    }
                }
            }
        }

        // ---- per half: scores, softmax and the PV operand
        u32x4_t ahi[NH], alo[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            float x0 = 0.f, x1 = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gg = (32 * r) / G;
                x0 = fmaf(h2f(kdm[0][gg], 0), D0[hf][r], x0);
                x1 = fmaf(h2f(kdm[1][gg], 0), D1[hf][r], x1);
            }
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                x0 = fmaf(h2f(kdm[0][gg], 1), sqm[hf][gg], x0);
                x1 = fmaf(h2f(kdm[1][gg], 1), sqm[hf][gg], x1);
            }
            float s0 = x0 * c2[hf], s1 = x1 * c2[hf];
            const int tok0 = 32 * tl + n16;
            const bool ok0 = full || (tok0 >= t_lo && tok0 < t_hi);
            const bool ok1 = full || (tok0 + 16 >= t_lo && tok0 + 16 < t_hi);
            if constexpr (!full) {
                s0 = ok0 ? s0 : -INFINITY;
                s1 = ok1 ? s1 : -INFINITY;
            }
            const float mx = row16_max(fmaxf(s0, s1));

            // ---- raise the reference maximum of head kb when the tile exceeds it
            // by more than kSlack.  The branch is wave-uniform and rarely taken;
            // lanes that do not grow scale by exactly 1.
            {
                const bool grow = mx > m_sh[hf] + (kPScale + kSlack);
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float m_new = grow ? mx - kPScale : m_sh[hf];
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_sh[hf] - m_new) : 1.0f;
                    m_sh[hf] = m_new;
                    l_run[hf] *= alpha;
#pragma unroll
                    for (int gg = 0; gg < NG; ++gg) accm[hf][gg] *= alpha;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) E[hf][hh] *= alpha;
                }
            }

            // ---- probabilities of head kb for tokens n16 and 16 + n16
            const float p0 = __builtin_amdgcn_exp2f(s0 - m_sh[hf]);
            const float p1 = __builtin_amdgcn_exp2f(s1 - m_sh[hf]);
            l_run[hf] += p0 + p1;
            {
                const uint8_t* v0p = &mbuf[m_vm];
                const uint8_t* v1p = &mbuf[MB + m_vm];
                uint32_t vm0[(NG + 1) / 2], vm1[(NG + 1) / 2];
                if constexpr (NG == 4) {
                    const uint2 u0 = *reinterpret_cast<const uint2*>(v0p);
                    const uint2 u1 = *reinterpret_cast<const uint2*>(v1p);
                    vm0[0] = u0.x; vm0[1] = u0.y; vm1[0] = u1.x; vm1[1] = u1.y;
                } else if constexpr (NG == 2) {
                    vm0[0] = *reinterpret_cast<const uint32_t*>(v0p);
                    vm1[0] = *reinterpret_cast<const uint32_t*>(v1p);
                } else {
                    vm0[0] = *reinterpret_cast<const uint16_t*>(v0p);
                    vm1[0] = *reinterpret_cast<const uint16_t*>(v1p);
                }
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) {
                    if constexpr (full) {
                        accm[hf][gg] = fmaf(p0, h2f(vm0[gg >> 1], gg & 1), fmaf(p1, h2f(vm1[gg >> 1], gg & 1), accm[hf][gg]));
                    } else {
                        // never-written slots may hold NaN: select, do not multiply
                        const float v0 = ok0 ? h2f(vm0[gg >> 1], gg & 1) : 0.f;
                        const float v1 = ok1 ? h2f(vm1[gg >> 1], gg & 1) : 0.f;
                        accm[hf][gg] = fmaf(p0, v0, fmaf(p1, v1, accm[hf][gg]));
                    }
                }
            }
            // A work item is one wave (64-thread workgroup) and one wave's LDS
            // accesses execute in issue order, so the reads below see these
            // writes; the barrier only keeps the compiler from reordering them.
            pbuf[hf][kb][n16] = p0;
            pbuf[hf][kb][16 + n16] = p1;
            __builtin_amdgcn_wave_barrier();
            const float4 pa = *reinterpret_cast<const float4*>(&pbuf[hf][jq][8 * kb]);
            const float4 pb = *reinterpret_cast<const float4*>(&pbuf[hf][jq][8 * kb + 4]);
            const uint4 vd = *reinterpret_cast<const uint4*>(&mbuf[m_vd]);

            // ---- PV: A = w = p Delta_V of head jq, block gq, tokens 8 kb + e
            const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
            const uint32_t vdw[4] = {vd.x, vd.y, vd.z, vd.w};
            float wv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) wv[e] = fmaf(pr[e], h2f(vdw[e >> 1], e & 1), 0.0f);
            if constexpr (!full) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tok = 32 * tl + 8 * kb + e;
                    wv[e] = (tok >= t_lo && tok < t_hi) ? wv[e] : 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hw, lw;
                split_bf16(wv[i], wv[i + 4], hw, lw);
                ahi[hf][i] = hw;
                alo[hf][i] = lw;
            }
        }

        // ---- PV, block by block; each block's widened V codes serve every half
        const uint4 vc0 = stage[2][lane], vc1 = stage[3][lane];
        const uint32_t vcw[8] = {vc0.x, vc0.y, vc0.z, vc0.w, vc1.x, vc1.y, vc1.z, vc1.w};
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            // rows of block blk only: each accumulator row gathers its own block
            const uint64_t rows = 0x1111111111111111ull << blk;
            const u32x4_t b0 = widen_v(vcw[2 * blk]), b1 = widen_v(vcw[2 * blk + 1]);
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
                const u32x4_t bh = {keep_lanes(ahi[hf][0], rows), keep_lanes(ahi[hf][1], rows),
                                    keep_lanes(ahi[hf][2], rows), keep_lanes(ahi[hf][3], rows)};
                const u32x4_t bl = {keep_lanes(alo[hf][0], rows), keep_lanes(alo[hf][1], rows),
                                    keep_lanes(alo[hf][2], rows), keep_lanes(alo[hf][3], rows)};
                E[hf][0] = mfma_bf16(bh, b0, E[hf][0]);
                E[hf][1] = mfma_bf16(bh, b1, E[hf][1]);
                E[hf][0] = mfma_bf16(bl, b0, E[hf][0]);
                E[hf][1] = mfma_bf16(bl, b1, E[hf][1]);
            }
        }
    };

    // Tiles in order; the landing registers always hold the next tile.
    // Refills past the last tile re-read the current pages (cache hits), so
    // every load is unconditional; page ids are read one tile ahead.
    {
        Kv4Tile t;
        const uint8_t* T0 = page(2 * tile_first);       // pages of the tile in t
        const uint8_t* T1 = page(2 * tile_first + 1);
        load_tile(t, T0, T1);
        const uint8_t* C0 = page(2 * tile_first + 2);   // pages of the next tile
        const uint8_t* C1 = page(2 * tile_first + 3);
        // one tile: refill pointers, then the step (full tiles need no masks)
        auto advance = [&](int tl, auto full_tag) {
            pace.tile(tile_end - tl);
            const bool more = tl + 1 < tile_end;
            const uint8_t* N0 = more ? C0 : T0;
            const uint8_t* N1 = more ? C1 : T1;
            C0 = page(2 * tl + 4);
            C1 = page(2 * tl + 5);
            step(t, tl, N0, N1, full_tag);
            T0 = N0;
            T1 = N1;
        };
        // only the first and the last tile of an item can be partial
        int tl = tile_first;
        if (32 * tl < t_lo || 32 * tl + 32 > t_hi) advance(tl++, std::false_type{});
        const int full_end = t_hi / 32;          // tiles [tl, full_end) are full
        for (; tl < full_end; ++tl) advance(tl, std::true_type{});
        if (tl < tile_end) advance(tl, std::false_type{});
    }

    // ---- epilogue: lane l holds head 4 hf + kb, channels 32 r + 16 h + n16 in E[hf][h][r]
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const float l = row16_sum(l_run[hf]);
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) accm[hf][gg] = row16_sum(accm[hf][gg]);
        const float inv = 1.0f / l;
        if (4 * hf + kb >= g.gqa) continue;      // a head past the q/kv ratio
        float* dst = rec + (4 * hf + kb) * (g.d + kPartPad);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dst[32 * r + n16] = (ldexpf(E[hf][0][r], 133) + accm[hf][(32 * r) / G]) * inv;
            dst[32 * r + 16 + n16] = (ldexpf(E[hf][1][r], 133) + accm[hf][(32 * r) / G]) * inv;
        }
        if (n16 == 0) dst[g.d] = m_sh[hf] + log2f(l);
    }
}

// Four int8 codes per word (byte i = code i) -> bf16 or fp16 pairs whose bit
// patterns are the subnormal numbers (code + 128) * 2^-133 (bf16) or
// (code + 128) * 2^-24 (fp16): pair 0 = codes (0, 2), pair 1 = (1, 3) of w0,
// pairs 2, 3 the same of w1.  The +128 bias is removed with the sum of the
// operand it multiplies.
__device__ __forceinline__ u32x4_t widen_i8(uint32_t w0, uint32_t w1)
{
    const uint32_t M = 0x00FF00FFu;
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    u32x4_t r;
    r[0] = x0 & M;
    r[1] = (x0 >> 8) & M;
    r[2] = x1 & M;
    r[3] = (x1 >> 8) & M;
    return r;
}

// ---------------------------------------------------------------------------
// Protected part of the mixed cache (sink + recent positions, INT8 with one
// fp16 scale per entry and kv head, KV4-RL Section 5.2), GQA group 4, on the
// matrix core.  The protected positions occupy ring entries [0, n8); they are
// walked in tiles of 32 entries (the ring is padded to a multiple of 32).
//   QK, transposed as for INT4: A = scaled q in fp16, block-diagonal, row n16 =
//     (head n16/4, block n16%4); MFMA b covers channels 32 kb + 8 b + i of
//     k-slot (kb, i), so a lane's K operand for all four MFMAs is the 32
//     contiguous bytes [32 kb, 32 kb + 32) of its token's row.  The score is
//     s_K * sum_b D[b] (one scale per token, no groups).
//   PV: A = w = p' s_V (the same for every block row), k = tile entries 8 kb ..
//     8 kb + 7, split into bf16 hi + lo; B = V codes (ring blocks of 8 entries,
//     channel-major).  The accumulators are compacted as in the INT4 item:
//     block r's MFMAs keep the A rows of block r and cover channels 32 r +
//     16 h + n16 in E[h][r].
// ---------------------------------------------------------------------------
// NH = 2 (q/kv ratio 8): q heads 0-3 and 4-7 of the group in turn on each
// tile's loads, as in the INT4 item.
template <bool ROT, int NH = 1>
__device__ __forceinline__ void mfma_prot_kv4(const DecodeArgs& a, int b, int h, float* rec)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int jq = n16 >> 2, gq = n16 & 3;
    const int n8 = regions_of(seq_len(a, b), g.S, g.R).n8;
    if (n8 <= 0) return;
    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const uint8_t* ring = a.side + (int64_t)a.layer * g.layer_side + ((int64_t)slot * g.Hkv + h) * g.rb;
    const uint8_t* vreg = ring + (int64_t)g.SR32 * g.d;
    const uint16_t* ksc = reinterpret_cast<const uint16_t*>(ring + (int64_t)2 * g.SR32 * g.d);
    const uint16_t* vsc = ksc + g.SR32;

    u32x4_t aqv[NH];
    u32x4_t aql[NH];                             // low half of a rotated query
    f32x4_t dinit[NH];
    float c2[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        aql[hf] = u32x4_t{0u, 0u, 0u, 0u};
        // ---- q of head jq, channels 32 kb + 8 gq + i, scaled by 2^sc into fp16
        int sc;
        {
            // rows of heads past the q/kv ratio (GQA 1 and 2 run in the four-head
            // layout) carry q = 0; their results are not written
            const int jh = 4 * hf + jq;
            const bool qreal = jh < g.gqa;
            const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * g.gqa + (qreal ? jh : 0)) * g.d;
            uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * kb + 8 * gq);
            if (!qreal) u = make_uint4(0u, 0u, 0u, 0u);
            float q[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                          bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
            if constexpr (ROT) {
                // channel bits 3-4 are lane bits 0-1 (gq), bits 5-6 lane bits 4-5 (kb)
                wht_local(q);
                wht_lanes(q, 1);
                wht_lanes(q, 2);
                wht_lanes(q, 16);
                wht_lanes(q, 32);
                wht_scale(q);
            }
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(q[c]));
            amax = fmaxf(amax, dpp<0xB1>(amax));
            amax = rows_max(fmaxf(amax, dpp<0x4E>(amax)));
            sc = 15 - __builtin_amdgcn_frexp_expf(amax);
            // k-slot pairs as widen_i8 pairs codes: (0, 2), (1, 3), (4, 6), (5, 7)
            constexpr int pe[4][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (ROT) {
                    const uint2 hl = split_f16(ldexpf(q[pe[i][0]], sc), ldexpf(q[pe[i][1]], sc));
                    aqv[hf][i] = hl.x;
                    aql[hf][i] = hl.y;
                } else {
                    aqv[hf][i] = pack_f16(ldexpf(q[pe[i][0]], sc), ldexpf(q[pe[i][1]], sc));
                }
            }
        }
        float qpart = 0.f;                       // the sum of exactly the operand used
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qpart += h2f(aqv[hf][i], 0) + h2f(aqv[hf][i], 1);
            if constexpr (ROT) qpart += h2f(aql[hf][i], 0) + h2f(aql[hf][i], 1);
        }
        // sum of the operand over MFMA block gq's 32 k-slots (row n16), then per D
        // row (head kb, block r): D starts at -128 * 2^-24 * that sum
        const float qblk = rows_sum(qpart);
#pragma unroll
        for (int r = 0; r < 4; ++r) dinit[hf][r] = -0x1p-17f * __shfl(qblk, 4 * kb + r);
        c2[hf] = ldexpf(a.scale2, 24 - __shfl(sc, 4 * kb));
    }

    // E[hf][h]: rows (head, block r), channels 32 r + 16 h + n16 (block-diagonal PV)
    f32x4_t E[NH][2], W[NH];
    float m_sh[NH], l_run[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        E[hf][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        E[hf][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        W[hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_sh[hf] = -INFINITY;
        l_run[hf] = 0.f;
    }
    __shared__ __attribute__((aligned(16))) float pbuf8[NH][4][32];
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0

    for (int e0 = 0; e0 < n8; e0 += 32) {
        // ---- loads: K rows of entries e0 + n16, e0 + 16 + n16 (bytes 32 kb ..),
        // V codes of entries e0 + 8 kb .. + 7 (this lane's 8 channels), scales
        const uint8_t* kr = ring + (int64_t)(e0 + n16) * g.d + 32 * kb;
        const uint4 k00 = *reinterpret_cast<const uint4*>(kr);
        const uint4 k01 = *reinterpret_cast<const uint4*>(kr + 16);
        const uint4 k10 = *reinterpret_cast<const uint4*>(kr + 16 * g.d);
        const uint4 k11 = *reinterpret_cast<const uint4*>(kr + 16 * g.d + 16);
        const uint8_t* vb = vreg + (int64_t)((e0 >> 3) + kb) * (8 * kHeadDim) + 64 * n16;
        const uint4 v0 = *reinterpret_cast<const uint4*>(vb);
        const uint4 v1 = *reinterpret_cast<const uint4*>(vb + 16);
        const uint4 v2 = *reinterpret_cast<const uint4*>(vb + 32);
        const uint4 v3 = *reinterpret_cast<const uint4*>(vb + 48);
        const float sk0 = half_bits_to_float(ksc[e0 + n16]);
        const float sk1 = half_bits_to_float(ksc[e0 + 16 + n16]);
        const uint4 svp = *reinterpret_cast<const uint4*>(vsc + e0 + 8 * kb);

        // ---- QK, block by block; each block's widened codes serve every half
        f32x4_t D0[NH], D1[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            D0[hf] = dinit[hf];
            D1[hf] = dinit[hf];
        }
        {
            const uint32_t kw0[8] = {k00.x, k00.y, k00.z, k00.w, k01.x, k01.y, k01.z, k01.w};
            const uint32_t kw1[8] = {k10.x, k10.y, k10.z, k10.w, k11.x, k11.y, k11.z, k11.w};
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint64_t rows = 0x1111111111111111ull << bb;
                const u32x4_t B0 = widen_i8(kw0[2 * bb], kw0[2 * bb + 1]);
                const u32x4_t B1 = widen_i8(kw1[2 * bb], kw1[2 * bb + 1]);
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    const u32x4_t A = {keep_lanes(aqv[hf][0], rows), keep_lanes(aqv[hf][1], rows),
                                       keep_lanes(aqv[hf][2], rows), keep_lanes(aqv[hf][3], rows)};
                    D0[hf] = mfma_f16(A, B0, D0[hf]);
                    D1[hf] = mfma_f16(A, B1, D1[hf]);
                    if constexpr (ROT) {
                        const u32x4_t Al = {keep_lanes(aql[hf][0], rows), keep_lanes(aql[hf][1], rows),
                                            keep_lanes(aql[hf][2], rows), keep_lanes(aql[hf][3], rows)};
                        D0[hf] = mfma_f16(Al, B0, D0[hf]);
                        D1[hf] = mfma_f16(Al, B1, D1[hf]);
                    }
                }
            }
        }
        // ---- per half: scores, softmax and the PV operand
        u32x4_t ahi[NH], alo[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            const bool ok0 = e0 + n16 < n8, ok1 = e0 + 16 + n16 < n8;
            float s0 = ((D0[hf][0] + D0[hf][1]) + (D0[hf][2] + D0[hf][3])) * sk0 * c2[hf];
            float s1 = ((D1[hf][0] + D1[hf][1]) + (D1[hf][2] + D1[hf][3])) * sk1 * c2[hf];
            s0 = ok0 ? s0 : -INFINITY;
            s1 = ok1 ? s1 : -INFINITY;
            const float mx = row16_max(fmaxf(s0, s1));
            {
                const bool grow = mx > m_sh[hf] + (kPScale + kSlack);
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float m_new = grow ? mx - kPScale : m_sh[hf];
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_sh[hf] - m_new) : 1.0f;
                    m_sh[hf] = m_new;
                    l_run[hf] *= alpha;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) E[hf][hh] *= alpha;
                    W[hf] *= alpha;
                }
            }
            const float p0 = __builtin_amdgcn_exp2f(s0 - m_sh[hf]);
            const float p1 = __builtin_amdgcn_exp2f(s1 - m_sh[hf]);
            l_run[hf] += p0 + p1;
            pbuf8[hf][kb][n16] = p0;
            pbuf8[hf][kb][16 + n16] = p1;
            __builtin_amdgcn_wave_barrier();
            const float4 pa = *reinterpret_cast<const float4*>(&pbuf8[hf][jq][8 * kb]);
            const float4 pb = *reinterpret_cast<const float4*>(&pbuf8[hf][jq][8 * kb + 4]);

            // ---- PV: w = p' s_V of head jq, entries e0 + 8 kb + e
            const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
            const uint32_t svw[4] = {svp.x, svp.y, svp.z, svp.w};
            float wv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // entries past the end may hold garbage scales: select, do not multiply
                const float w = fmaf(pr[e], h2f(svw[e >> 1], e & 1), 0.0f);
                wv[e] = e0 + 8 * kb + e < n8 ? w : 0.0f;
            }
            constexpr int pe[4][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hw, lw;
                split_bf16(wv[pe[i][0]], wv[pe[i][1]], hw, lw);
                ahi[hf][i] = hw;
                alo[hf][i] = lw;
            }
            W[hf] = mfma_bf16(ahi[hf], ones, W[hf]);
            W[hf] = mfma_bf16(alo[hf], ones, W[hf]);
        }
        // ---- PV, block by block; each block's widened codes serve every half
        {
            const uint32_t vw[16] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                                     v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const uint64_t rows = 0x1111111111111111ull << blk;
                const u32x4_t b0 = widen_i8(vw[4 * blk], vw[4 * blk + 1]);
                const u32x4_t b1 = widen_i8(vw[4 * blk + 2], vw[4 * blk + 3]);
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    const u32x4_t bh = {keep_lanes(ahi[hf][0], rows), keep_lanes(ahi[hf][1], rows),
                                        keep_lanes(ahi[hf][2], rows), keep_lanes(ahi[hf][3], rows)};
                    const u32x4_t bl = {keep_lanes(alo[hf][0], rows), keep_lanes(alo[hf][1], rows),
                                        keep_lanes(alo[hf][2], rows), keep_lanes(alo[hf][3], rows)};
                    E[hf][0] = mfma_bf16(bh, b0, E[hf][0]);
                    E[hf][1] = mfma_bf16(bh, b1, E[hf][1]);
                    E[hf][0] = mfma_bf16(bl, b0, E[hf][0]);
                    E[hf][1] = mfma_bf16(bl, b1, E[hf][1]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- epilogue: lane l holds head 4 hf + kb, channels 32 r + 16 h + n16 in E[hf][h][r]
    // (every block row of W carries the same sum; row 0 is used)
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const float l = row16_sum(l_run[hf]);
        const float inv = 1.0f / l;
        if (4 * hf + kb >= g.gqa) continue;      // a head past the q/kv ratio
        float* dst = rec + (4 * hf + kb) * (g.d + kPartPad);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dst[32 * r + n16] = (ldexpf(E[hf][0][r], 133) - 128.0f * W[hf][0]) * inv;
            dst[32 * r + 16 + n16] = (ldexpf(E[hf][1][r], 133) - 128.0f * W[hf][0]) * inv;
        }
        if (n16 == 0) dst[g.d] = m_sh[hf] + log2f(l);
    }
}

// ---------------------------------------------------------------------------
// KV8 kind: positions [t_lo, t_hi) of (b, h) from INT8 pages, in 32-token
// tiles (pages 2t and 2t + 1), with the protected part's matrix-core compute:
// fp16 QK on (code + 128) subnormals with D started at -128 2^-24 sum(q),
// score s_K sum D; bf16 PV with w = p' s_V on (code + 128) subnormals and the
// +128 removed by a ones-column product.  A lane's loads for a tile land in
// registers and move to a per-wave LDS stage at the start of the tile, so the
// next tile's loads are in flight during the compute.
// ---------------------------------------------------------------------------
template <int NH = 1>
__device__ __forceinline__ void mfma_item_kv8(const DecodeArgs& a, int b, int h, int t_lo, int t_hi,
                                              float* rec, Pace& pace)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int jq = n16 >> 2, gq = n16 & 3;
    if (t_hi <= t_lo) return;
    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    const uint8_t* hbase = a.pages + (int64_t)a.layer * g.layer_pages + (int64_t)h * g.pb;
    const int64_t page_stride = (int64_t)g.Hkv * g.pb;
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    const const_i32 btc = (const_i32)bt;
    auto page = [&](int pi) -> const uint8_t* {
        const int p = clampi(btc[min(pi, g.max_pages - 1)], 0, g.num_pages - 1);
        return hbase + (int64_t)p * page_stride;
    };

    // ---- q of head 4 hf + jq, channels 32 kb + 8 gq + i, scaled by 2^sc into
    // fp16, per half of the q heads (one half up to ratio 4)
    u32x4_t aqv[NH];
    f32x4_t dinit[NH];
    float c2[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        int sc;
        // rows of heads past the q/kv ratio (GQA 1 and 2 run in the four-head
        // layout) carry q = 0; their results are not written
        const int jh = 4 * hf + jq;
        const bool qreal = jh < g.gqa;
        const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * g.gqa + (qreal ? jh : 0)) * g.d;
        uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * kb + 8 * gq);
        if (!qreal) u = make_uint4(0u, 0u, 0u, 0u);
        const float q[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                            bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(q[c]));
        amax = fmaxf(amax, dpp<0xB1>(amax));
        amax = rows_max(fmaxf(amax, dpp<0x4E>(amax)));
        sc = 15 - __builtin_amdgcn_frexp_expf(amax);
        aqv[hf][0] = pack_f16(ldexpf(q[0], sc), ldexpf(q[2], sc));
        aqv[hf][1] = pack_f16(ldexpf(q[1], sc), ldexpf(q[3], sc));
        aqv[hf][2] = pack_f16(ldexpf(q[4], sc), ldexpf(q[6], sc));
        aqv[hf][3] = pack_f16(ldexpf(q[5], sc), ldexpf(q[7], sc));
        float qpart = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) qpart += h2f(aqv[hf][i], 0) + h2f(aqv[hf][i], 1);
        const float qblk = rows_sum(qpart);
#pragma unroll
        for (int r = 0; r < 4; ++r) dinit[hf][r] = -0x1p-17f * __shfl(qblk, 4 * kb + r);
        c2[hf] = ldexpf(a.scale2, 24 - __shfl(sc, 4 * kb));
    }

    f32x4_t E[NH][2], W[NH];
    float m_sh[NH], l_run[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        E[hf][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        E[hf][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        W[hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_sh[hf] = -INFINITY;
        l_run[hf] = 0.f;
    }
    __shared__ uint4 stage8[8][64];
    __shared__ __attribute__((aligned(16))) float pbuf8[NH][4][32];
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0

    // landing registers of one tile
    uint4 lk0, lk1, lk2, lk3, lv0, lv1, lv2, lv3, lsv;
    uint32_t lsk0, lsk1;
    const uint32_t kofs = (uint32_t)(g.off_kc + n16 * g.d + 32 * kb);
    const uint32_t vofs = (uint32_t)(g.off_vc + (kb & 1) * 8 * g.d + 64 * n16);
    const uint32_t svofs = (uint32_t)(g.off_vm + 16 * (kb & 1));
    auto load = [&](const uint8_t* P0, const uint8_t* P1) {
        lk0 = *reinterpret_cast<const uint4*>(P0 + kofs);
        lk1 = *reinterpret_cast<const uint4*>(P0 + kofs + 16);
        lk2 = *reinterpret_cast<const uint4*>(P1 + kofs);
        lk3 = *reinterpret_cast<const uint4*>(P1 + kofs + 16);
        const uint8_t* PV = (kb >> 1) ? P1 : P0;
        lv0 = *reinterpret_cast<const uint4*>(PV + vofs);
        lv1 = *reinterpret_cast<const uint4*>(PV + vofs + 16);
        lv2 = *reinterpret_cast<const uint4*>(PV + vofs + 32);
        lv3 = *reinterpret_cast<const uint4*>(PV + vofs + 48);
        lsk0 = reinterpret_cast<const uint16_t*>(P0 + g.off_kdm)[n16];
        lsk1 = reinterpret_cast<const uint16_t*>(P1 + g.off_kdm)[n16];
        lsv = *reinterpret_cast<const uint4*>(PV + svofs);
    };

    const int tile_first = t_lo / 32, tile_end = (t_hi + 31) / 32;
    const uint8_t* T0 = page(2 * tile_first);
    const uint8_t* T1 = page(2 * tile_first + 1);
    load(T0, T1);
    const uint8_t* C0 = page(2 * tile_first + 2);
    const uint8_t* C1 = page(2 * tile_first + 3);
    for (int tl = tile_first; tl < tile_end; ++tl) {
        pace.tile(tile_end - tl);
        // ---- this tile to the stage, then the next tile's loads (the last
        // tile re-reads its own pages: cache hits)
        stage8[0][lane] = lk0;
        stage8[1][lane] = lk1;
        stage8[2][lane] = lk2;
        stage8[3][lane] = lk3;
        stage8[4][lane] = lv0;
        stage8[5][lane] = lv1;
        stage8[6][lane] = lv2;
        stage8[7][lane] = lv3;
        const float sk0 = half_bits_to_float((uint16_t)lsk0);
        const float sk1 = half_bits_to_float((uint16_t)lsk1);
        const uint4 svp = lsv;
        __builtin_amdgcn_wave_barrier();
        const bool more = tl + 1 < tile_end;
        const uint8_t* N0 = more ? C0 : T0;
        const uint8_t* N1 = more ? C1 : T1;
        C0 = page(2 * tl + 4);
        C1 = page(2 * tl + 5);
        load(N0, N1);
        T0 = N0;
        T1 = N1;

        // ---- QK, block by block; each block's widened codes serve every half
        f32x4_t D0[NH], D1[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            D0[hf] = dinit[hf];
            D1[hf] = dinit[hf];
        }
        {
            const uint4 k00 = stage8[0][lane], k01 = stage8[1][lane];
            const uint4 k10 = stage8[2][lane], k11 = stage8[3][lane];
            const uint32_t kw0[8] = {k00.x, k00.y, k00.z, k00.w, k01.x, k01.y, k01.z, k01.w};
            const uint32_t kw1[8] = {k10.x, k10.y, k10.z, k10.w, k11.x, k11.y, k11.z, k11.w};
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint64_t rows = 0x1111111111111111ull << bb;
                const u32x4_t B0 = widen_i8(kw0[2 * bb], kw0[2 * bb + 1]);
                const u32x4_t B1 = widen_i8(kw1[2 * bb], kw1[2 * bb + 1]);
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    const u32x4_t A = {keep_lanes(aqv[hf][0], rows), keep_lanes(aqv[hf][1], rows),
                                       keep_lanes(aqv[hf][2], rows), keep_lanes(aqv[hf][3], rows)};
                    D0[hf] = mfma_f16(A, B0, D0[hf]);
                    D1[hf] = mfma_f16(A, B1, D1[hf]);
                }
            }
        }
        const int tok0 = 32 * tl + n16;
        const bool ok0 = tok0 >= t_lo && tok0 < t_hi;
        const bool ok1 = tok0 + 16 >= t_lo && tok0 + 16 < t_hi;

        // ---- per half: scores, softmax and the PV operand
        u32x4_t ahi[NH], alo[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            float s0 = ((D0[hf][0] + D0[hf][1]) + (D0[hf][2] + D0[hf][3])) * sk0 * c2[hf];
            float s1 = ((D1[hf][0] + D1[hf][1]) + (D1[hf][2] + D1[hf][3])) * sk1 * c2[hf];
            s0 = ok0 ? s0 : -INFINITY;
            s1 = ok1 ? s1 : -INFINITY;
            const float mx = row16_max(fmaxf(s0, s1));
            {
                const bool grow = mx > m_sh[hf] + (kPScale + kSlack);
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float m_new = grow ? mx - kPScale : m_sh[hf];
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_sh[hf] - m_new) : 1.0f;
                    m_sh[hf] = m_new;
                    l_run[hf] *= alpha;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) E[hf][hh] *= alpha;
                    W[hf] *= alpha;
                }
            }
            const float p0 = __builtin_amdgcn_exp2f(s0 - m_sh[hf]);
            const float p1 = __builtin_amdgcn_exp2f(s1 - m_sh[hf]);
            l_run[hf] += p0 + p1;
            pbuf8[hf][kb][n16] = p0;
            pbuf8[hf][kb][16 + n16] = p1;
            __builtin_amdgcn_wave_barrier();
            const float4 pa = *reinterpret_cast<const float4*>(&pbuf8[hf][jq][8 * kb]);
            const float4 pb = *reinterpret_cast<const float4*>(&pbuf8[hf][jq][8 * kb + 4]);

            // ---- PV operand: w = p' s_V of head 4 hf + jq, tokens 32 tl + 8 kb + e
            const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
            const uint32_t svw[4] = {svp.x, svp.y, svp.z, svp.w};
            float wv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // tokens outside the run may have garbage scales: select, do not multiply
                const float w = fmaf(pr[e], h2f(svw[e >> 1], e & 1), 0.0f);
                const int tok = 32 * tl + 8 * kb + e;
                wv[e] = tok >= t_lo && tok < t_hi ? w : 0.0f;
            }
            constexpr int pe[4][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hw, lw;
                split_bf16(wv[pe[i][0]], wv[pe[i][1]], hw, lw);
                ahi[hf][i] = hw;
                alo[hf][i] = lw;
            }
            W[hf] = mfma_bf16(ahi[hf], ones, W[hf]);
            W[hf] = mfma_bf16(alo[hf], ones, W[hf]);
        }

        // ---- PV, block by block; each block's widened codes serve every half
        {
            const uint4 v0 = stage8[4][lane], v1 = stage8[5][lane];
            const uint4 v2 = stage8[6][lane], v3 = stage8[7][lane];
            const uint32_t vw[16] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                                     v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const uint64_t rows = 0x1111111111111111ull << blk;
                const u32x4_t b0 = widen_i8(vw[4 * blk], vw[4 * blk + 1]);
                const u32x4_t b1 = widen_i8(vw[4 * blk + 2], vw[4 * blk + 3]);
#pragma unroll
                for (int hf = 0; hf < NH; ++hf) {
                    const u32x4_t bh = {keep_lanes(ahi[hf][0], rows), keep_lanes(ahi[hf][1], rows),
                                        keep_lanes(ahi[hf][2], rows), keep_lanes(ahi[hf][3], rows)};
                    const u32x4_t bl = {keep_lanes(alo[hf][0], rows), keep_lanes(alo[hf][1], rows),
                                        keep_lanes(alo[hf][2], rows), keep_lanes(alo[hf][3], rows)};
                    E[hf][0] = mfma_bf16(bh, b0, E[hf][0]);
                    E[hf][1] = mfma_bf16(bh, b1, E[hf][1]);
                    E[hf][0] = mfma_bf16(bl, b0, E[hf][0]);
                    E[hf][1] = mfma_bf16(bl, b1, E[hf][1]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- epilogue: lane l holds head 4 hf + kb, channels 32 r + 16 h + n16 in E[hf][h][r]
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const float l = row16_sum(l_run[hf]);
        const float inv = 1.0f / l;
        if (4 * hf + kb >= g.gqa) continue;      // a head past the q/kv ratio
        float* dst = rec + (4 * hf + kb) * (g.d + kPartPad);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dst[32 * r + n16] = (ldexpf(E[hf][0][r], 133) - 128.0f * W[hf][0]) * inv;
            dst[32 * r + 16 + n16] = (ldexpf(E[hf][1][r], 133) - 128.0f * W[hf][0]) * inv;
        }
        if (n16 == 0) dst[g.d] = m_sh[hf] + log2f(l);
    }
}

// ---------------------------------------------------------------------------
// BF16 comparator split (same tiling; keys and values used as stored).
//   QK: rows = 16 tokens, k = 8 consecutive channels per k-block, columns =
//       (head j, 0): only column block 0 of each head is non-zero.
//   PV: rows = (head j, part): part 0 = bf16(p), part 1 = bf16(p - part 0),
//       parts 2-3 zero;
//       columns = channels 16 s + n16; k = tokens 8 kb .. 8 kb + 7 in order.
// ---------------------------------------------------------------------------
template <int NH = 1>
__device__ __forceinline__ void mfma_item_bf16(const DecodeArgs& a, int b, int h, int t_lo, int t_hi,
                                               float* rec, Pace& pace)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int jq = n16 >> 2, gq = n16 & 3;
    if (t_hi <= t_lo) return;
    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    const uint8_t* hbase = a.pages + (int64_t)a.layer * g.layer_pages + (int64_t)h * g.pb;
    const int64_t page_stride = (int64_t)g.Hkv * g.pb;

    // columns of heads past the q/kv ratio (GQA 1 and 2 run in the four-head
    // layout) carry q = 0; their results are not written
    // (NH = 2: q heads 0-3 and 4-7 of the group as two halves on the same loads)
    u32x4_t bq[NH][4];
    f32x4_t O[NH][8];
    float m_run[NH], l_run[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const int jh = 4 * hf + jq;
        const bool qreal = jh < g.gqa;
        const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * g.gqa + (qreal ? jh : 0)) * g.d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * i + 8 * kb);
            u32x4_t v = {u.x, u.y, u.z, u.w}, z = {0u, 0u, 0u, 0u};
            bq[hf][i] = gq == 0 && qreal ? v : z;
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) O[hf][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_run[hf] = -INFINITY;
        l_run[hf] = 0.f;
    }
    const float c2 = a.scale2;
    const int rq = n16 >> 2, rr = n16 & 3;
    const int k_off0 = 2 * ((8 * (rq & 1) + rr) * g.d + 8 * kb);
    const int k_off1 = k_off0 + 2 * 4 * g.d;
    const int v_off = kPage * g.d * 2 + 2 * (((kb & 1) * g.d + n16) * kHalf);

    for (int ts = (t_lo / 32) * 32; ts < t_hi; ts += 32) {
        pace.tile((t_hi + 31) / 32 - ts / 32);
        const int pi = ts / kPage;
        const int p0 = clampi(bt[min(pi, g.max_pages - 1)], 0, g.num_pages - 1);
        const int p1 = clampi(bt[min(pi + 1, g.max_pages - 1)], 0, g.num_pages - 1);
        const uint8_t* P0 = hbase + p0 * page_stride;
        const uint8_t* P1 = hbase + p1 * page_stride;
        const uint8_t* PK = (rq >> 1) ? P1 : P0;
        const uint8_t* PM = (kb >> 1) ? P1 : P0;
        f32x4_t D0[NH], D1[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) D0[hf] = D1[hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 k0 = *reinterpret_cast<const uint4*>(PK + k_off0 + 64 * i);
            uint4 k1 = *reinterpret_cast<const uint4*>(PK + k_off1 + 64 * i);
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) {
                D0[hf] = mfma_bf16(u32x4_t{k0.x, k0.y, k0.z, k0.w}, bq[hf][i], D0[hf]);
                D1[hf] = mfma_bf16(u32x4_t{k1.x, k1.y, k1.z, k1.w}, bq[hf][i], D1[hf]);
            }
        }
        bool valid[8];
        u32x4_t ap[NH];
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            float sc[8], mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tok = ts + 8 * kb + e;
                valid[e] = tok >= t_lo && tok < t_hi;
                float s = quad_sum(e < 4 ? D0[hf][e] : D1[hf][e - 4]);
                sc[e] = valid[e] ? s * c2 : -INFINITY;
                mx = fmaxf(mx, sc[e]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[hf], mx);
            const float alpha = exp2f(m_run[hf] - m_new);
            m_run[hf] = m_new;
            float pv[8], ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = valid[e] ? exp2f(sc[e] - m_new) : 0.f;
                ps += pv[e];
            }
            l_run[hf] = fmaf(l_run[hf], alpha, ps);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hw, lw;
                split_bf16(pv[2 * i], pv[2 * i + 1], hw, lw);
                ap[hf][i] = gq == 0 ? hw : (gq == 1 ? lw : 0u);
            }
            const float alpha_d = __shfl(alpha, 4 * kb);
            if (__any(alpha_d != 1.0f)) {
#pragma unroll
                for (int s = 0; s < 8; ++s) { O[hf][s][0] *= alpha_d; O[hf][s][1] *= alpha_d; }
            }
        }
        // values of tokens outside the item may be any bit pattern (NaN, Inf):
        // zero them in partial tiles, since 0 * NaN would reach the sum
        const bool full = ts >= t_lo && ts + 32 <= t_hi;
        u32x4_t vmask;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vmask[i] = (valid[2 * i] ? 0x0000FFFFu : 0u) | (valid[2 * i + 1] ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            // 16 lanes read 256 contiguous bytes: whole lines, streamed
            uint4 v = ldg_stream(PM + v_off + 2 * 16 * s * kHalf);
            u32x4_t bv = {v.x, v.y, v.z, v.w};
            if (!full) bv &= vmask;
#pragma unroll
            for (int hf = 0; hf < NH; ++hf) O[hf][s] = mfma_bf16(ap[hf], bv, O[hf][s]);
        }
    }
    __shared__ float sh_l[NH][4], sh_m[NH][4];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        float lr = l_run[hf];
        lr += __shfl_xor(lr, 16);
        lr += __shfl_xor(lr, 32);
        if (kb == 0 && gq == 0) { sh_l[hf][jq] = lr; sh_m[hf][jq] = m_run[hf]; }
    }
    __syncthreads();
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const float lj = sh_l[hf][kb];
        const float inv = 1.0f / lj;
        if (4 * hf + kb >= g.gqa) continue;      // a head past the q/kv ratio
        float* dst = rec + (4 * hf + kb) * (g.d + kPartPad);
#pragma unroll
        for (int s = 0; s < 8; ++s) dst[16 * s + n16] = (O[hf][s][0] + O[hf][s][1]) * inv;
        if (n16 == 0) dst[g.d] = sh_m[hf][kb] + log2f(lj);
    }
}

// Grid = W one-wave workgroups, each walking its range of the balanced unit
// partition: protected parts on the vector ALU, runs of INT4 tiles on the
// matrix core.
// ROT: keys stored in the rotated basis (the query is rotated at load).
template <int G, bool ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void decode_kv4_mfma_kernel(DecodeArgs a)
{
    walk_units(a, [&](int b, int h) { mfma_prot_kv4<ROT>(a, b, h, prot_ptr(a, b * a.g.Hkv + h)); },
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_kv4<G, ROT>(a, b, h, lo, hi, rec, pace);
               });
}

// q/kv ratio 8 on the matrix core: the four-head layout twice per tile (q
// heads 0-3, then 4-7) on one load of the tile.  The second half's operands
// and softmax state need more registers: three waves per SIMD.
template <int G, bool ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void decode_kv4_mfma8_kernel(DecodeArgs a)
{
    walk_units(a, [&](int b, int h) { mfma_prot_kv4<ROT, 2>(a, b, h, prot_ptr(a, b * a.g.Hkv + h)); },
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_kv4<G, ROT, 2>(a, b, h, lo, hi, rec, pace);
               });
}

// q/kv ratio 16: the four-head layout four times per tile, two waves per SIMD.
template <int G, bool ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kv4_mfma16_kernel(DecodeArgs a)
{
    walk_units(a, [&](int b, int h) { mfma_prot_kv4<ROT, 4>(a, b, h, prot_ptr(a, b * a.g.Hkv + h)); },
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_kv4<G, ROT, 4>(a, b, h, lo, hi, rec, pace);
               });
}

// ---------------------------------------------------------------------------
// Integer path on the matrix core (KV4_FLAG_INT_PATH, GQA 4): the tiles, loads, LDS stage and partition of mfma_item_kv4 with
// integer products.  Lane roles (n16 = lane % 16, kb = lane / 16):
//   QK: v_mfma_i32_16x16x64_i8.  A = the INT8 query codes, block-diagonal:
//     row n16 = (head n16/4, 32-channel block n16%4); the lane's 16 k-slots
//     are its K code words b, b + 1 (channels 32 b + 8 kb + [0, 8)), b = 0 in
//     the first product and 2 in the second, non-zero only for b = n16%4.
//     B = those words widened to bytes, column = token n16 of a page.  Lane l
//     then holds the integer sums of head kb over each block r for its token
//     in D[r], and the score follows in-lane from Delta, m, Q and s_q.
//   PV: v_mfma_i32_16x16x32_i8 per 16 value channels.  A = the 8-bit codes u
//     of w = p' Delta_V, row n16 = (head n16/4, 8-token block n16%4), k-slots
//     = tile tokens 8 kb .. 8 kb + 7, non-zero only for block kb, so that each
//     block keeps its own scale; B = the V code word widened to bytes.  Lane l
//     holds, for head kb and its channel, the integer sum of each block r in
//     D[r]; the blocks' scales combine them in-lane.  The codes of (head j,
//     block b, group g) are formed by lane (4 j + b, g) and moved to lane
//     (4 j + b, b) by a lane shuffle; the scales go through LDS.
//   The offsets' term sum p' m_V is accumulated on the vector ALU as in the
//   floating-point item.
// ---------------------------------------------------------------------------
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t mfma_i8_64(u32x4_t a, u32x4_t b, i32x4_t c)
{
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a), __builtin_bit_cast(i32x4_t, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ i32x4_t mfma_i8_32(uint32_t alo, uint32_t ahi, uint32_t blo, uint32_t bhi, i32x4_t c)
{
    const long A = (long)(((uint64_t)ahi << 32) | alo), B = (long)(((uint64_t)bhi << 32) | blo);
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, c, 0, 0, 0);
}

// Nibbles of a code word as bytes: channels (tokens) 0, 2, 4, 6 and 1, 3, 5, 7.
__device__ __forceinline__ uint32_t nib_lo(uint32_t w) { return w & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t w) { return (w >> 4) & 0x0F0F0F0Fu; }

// INT8 codes of one head's query (Q-4 encoding) for this lane's 8 channels
// c0 .. c0 + 7; the scale comes from the head's maximum over all its lanes.
struct QCodes {
    uint32_t lo, hi;          // codes of channels c0 + 0, 2, 4, 6 and c0 + 1, 3, 5, 7
    int sum;
};

__device__ __forceinline__ QCodes quant_q8(const float (&q)[8], float S, uint16_t sb)
{
    QCodes r;
    int c[8];
    r.sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        c[i] = int8_code(q[i], S, sb);
        r.sum += c[i];
    }
    r.lo = pack_i8x4(c[0], c[2], c[4], c[6]);
    r.hi = pack_i8x4(c[1], c[3], c[5], c[7]);
    return r;
}

// NH = 2 (q/kv ratio 8): q heads 0-3 and then 4-7 of the group on each staged
// tile, as in mfma_item_kv4.
template <int G, bool ROT, int NH = 1>
__device__ __forceinline__ void mfma_item_int(const DecodeArgs& a, int b, int h, int t_lo, int t_hi,
                                              float* rec, Pace& pace)
{
    constexpr int NG = kHeadDim / G;
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int jq = n16 >> 2, gq = n16 & 3;       // A row (head, block) of this lane
    if (t_hi <= t_lo) return;

    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    const uint8_t* hbase = a.pages + (int64_t)a.layer * g.layer_pages + (int64_t)h * g.pb;
    const int64_t page_stride = (int64_t)g.Hkv * g.pb;

    // ---- INT8 query: head jq's codes on channels 32 gq + 8 kb + [0, 8)
    u32x4_t A1[NH], A2[NH];                      // block-diagonal QK operands
    float Qg[NH][NG];                            // code sums of head kb per group
    float c2[NH];                                // score factor of head kb
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        // rows of heads past the q/kv ratio (GQA 1 and 2 run in the four-head
        // layout) carry q = 0; their results are not written
        const int jh = 4 * hf + jq;
        const bool qreal = jh < g.gqa;
        const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * g.gqa + (qreal ? jh : 0)) * g.d;
        uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * gq + 8 * kb);
        if (!qreal) u = make_uint4(0u, 0u, 0u, 0u);
        float q[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                      bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
        if constexpr (ROT) {
            // into the keys' basis in the fixed span order 1, 2, ..., 64: channel
            // bits 3-4 are lane bits 4-5 (kb), bits 5-6 lane bits 0-1 (gq)
            wht_local(q);
            wht_lanes(q, 16);
            wht_lanes(q, 32);
            wht_lanes(q, 1);
            wht_lanes(q, 2);
            wht_scale(q);
        }
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(q[c]));
        amax = fmaxf(amax, dpp<0xB1>(amax));                 // over the quad (blocks) ...
        amax = rows_max(fmaxf(amax, dpp<0x4E>(amax)));       // ... and the rows: head jq
        const uint16_t sb = plus_zero16(f32_to_f16_bits(__fdiv_rn(amax, 127.0f)));
        const float S = half_bits_to_float(sb);
        const QCodes qc = quant_q8(q, S, sb);
        A1[hf] = u32x4_t{gq == 0 ? qc.lo : 0u, gq == 0 ? qc.hi : 0u, gq == 1 ? qc.lo : 0u, gq == 1 ? qc.hi : 0u};
        A2[hf] = u32x4_t{gq == 2 ? qc.lo : 0u, gq == 2 ? qc.hi : 0u, gq == 3 ? qc.lo : 0u, gq == 3 ? qc.hi : 0u};
        // code sum of head jq over block gq (the four rows), then head kb's blocks
        const float qblk = rows_sum((float)qc.sum);          // integers below 2^13: exact
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) Qg[hf][gg] = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) Qg[hf][(32 * r) / G] += __shfl(qblk, 4 * kb + r);
        c2[hf] = a.scale2 * __shfl(S, 4 * kb);
    }

    // O[hf][r][hh]: head 4 hf + kb, channel 32 r + 16 hh + n16
    float O[NH][4][2];
    float accm[NH][NG];
    float m_sh[NH], l_run[NH];                   // m_sh = m_ref - kPScale
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
#pragma unroll
        for (int r = 0; r < 4; ++r) O[hf][r][0] = O[hf][r][1] = 0.f;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) accm[hf][gg] = 0.f;
        m_sh[hf] = -INFINITY;
        l_run[hf] = 0.f;
    }

    constexpr int MB = 128 * NG;                 // metadata bytes per page
    Kv4Offs o;
    o.kc = (uint32_t)(g.off_kc + n16 * (kHeadDim / 2) + 16 * kb);
    o.vc = (uint32_t)(g.off_vc + 4 * ((kb & 1) * g.d + 4 * n16));
    const int chunk = lane & 31;
    const bool chunk_ok = 16 * chunk < MB;
    o.meta = (uint32_t)(g.off_kdm + 16 * (chunk_ok ? chunk : 0));
    const int m_kdm = n16 * 4 * NG;                              // K (Delta, m) of token n16
    const int m_vm = 64 * NG + n16 * 2 * NG;                     // V m of token n16
    // V Delta of group kb for the tokens of block gq (page gq / 2, half gq % 2)
    const int m_vdu = (gq >> 1) * MB + 96 * NG + 2 * ((kb < NG ? kb : 0) * kPage + 8 * (gq & 1));

    const int tile_first = t_lo / 32, tile_end = (t_hi + 31) / 32;
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    const const_i32 btc = (const_i32)bt;
    const int pb_bytes = (int)g.pb;
    auto page = [&](int pi) -> const uint8_t* {
        const int p = clampi(btc[min(pi, g.max_pages - 1)], 0, g.num_pages - 1);
        return hbase + (int64_t)p * page_stride;
    };
    const bool upper = kb >> 1;

    __shared__ __attribute__((aligned(16))) float pbuf[NH][4][32];
    __shared__ __attribute__((aligned(16))) float sbuf[NH][4][4][4]; // [half][group][head][block]
    __shared__ __attribute__((aligned(16))) uint8_t mbuf[2 * 512];
    __shared__ uint4 stage[4][64];

    auto load_tile = [&](Kv4Tile& t, const uint8_t* N0, const uint8_t* N1) {
        load_k_codes(t, page_rsrc(N0, pb_bytes), page_rsrc(N1, pb_bytes), o);
        const uint8_t* PM = upper ? N1 : N0;
        load_v_codes(t, PM, o);
        load_meta(t, PM, o);
    };

    auto step = [&](Kv4Tile& t, int tl, const uint8_t* N0, const uint8_t* N1, auto full_tag) {
        constexpr bool full = decltype(full_tag)::value;
        stage[0][lane] = t.kc[0];
        stage[1][lane] = t.kc[1];
        stage[2][lane] = t.vc0;
        stage[3][lane] = t.vc1;
        if (chunk_ok) *reinterpret_cast<uint4*>(&mbuf[(lane >> 5) * MB + 16 * chunk]) = t.meta;
        __builtin_amdgcn_wave_barrier();
        load_tile(t, N0, N1);
        const uint4 kc0 = stage[0][lane], kc1 = stage[1][lane];
        uint32_t kdm[2][NG];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint8_t* src = &mbuf[hh * MB + m_kdm];
            if constexpr (NG == 4) {
                const uint4 u = *reinterpret_cast<const uint4*>(src);
                kdm[hh][0] = u.x; kdm[hh][1] = u.y; kdm[hh][2] = u.z; kdm[hh][3] = u.w;
            } else if constexpr (NG == 2) {
                const uint2 u = *reinterpret_cast<const uint2*>(src);
                kdm[hh][0] = u.x; kdm[hh][1] = u.y;
            } else {
                kdm[hh][0] = *reinterpret_cast<const uint32_t*>(src);
            }
        }

        // ---- per half of the q heads (one half below ratio 8)
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            // ---- QK: integer sums of head kb over block r, token n16 of page hh
            const i32x4_t z = {0, 0, 0, 0};
            i32x4_t D0 = mfma_i8_64(A1[hf], u32x4_t{nib_lo(kc0.x), nib_hi(kc0.x), nib_lo(kc0.y), nib_hi(kc0.y)}, z);
            D0 = mfma_i8_64(A2[hf], u32x4_t{nib_lo(kc0.z), nib_hi(kc0.z), nib_lo(kc0.w), nib_hi(kc0.w)}, D0);
            i32x4_t D1 = mfma_i8_64(A1[hf], u32x4_t{nib_lo(kc1.x), nib_hi(kc1.x), nib_lo(kc1.y), nib_hi(kc1.y)}, z);
            D1 = mfma_i8_64(A2[hf], u32x4_t{nib_lo(kc1.z), nib_hi(kc1.z), nib_lo(kc1.w), nib_hi(kc1.w)}, D1);
            float x0 = 0.f, x1 = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gg = (32 * r) / G;
                x0 = fmaf(h2f(kdm[0][gg], 0), (float)D0[r], x0);
                x1 = fmaf(h2f(kdm[1][gg], 0), (float)D1[r], x1);
            }
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                x0 = fmaf(h2f(kdm[0][gg], 1), Qg[hf][gg], x0);
                x1 = fmaf(h2f(kdm[1][gg], 1), Qg[hf][gg], x1);
            }
            float s0 = x0 * c2[hf], s1 = x1 * c2[hf];
            const int tok0 = 32 * tl + n16;
            const bool ok0 = full || (tok0 >= t_lo && tok0 < t_hi);
            const bool ok1 = full || (tok0 + 16 >= t_lo && tok0 + 16 < t_hi);
            if constexpr (!full) {
                s0 = ok0 ? s0 : -INFINITY;
                s1 = ok1 ? s1 : -INFINITY;
            }
            const float mx = row16_max(fmaxf(s0, s1));
            {
                const bool grow = mx > m_sh[hf] + (kPScale + kSlack);
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float m_new = grow ? mx - kPScale : m_sh[hf];
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_sh[hf] - m_new) : 1.0f;
                    m_sh[hf] = m_new;
                    l_run[hf] *= alpha;
#pragma unroll
                    for (int gg = 0; gg < NG; ++gg) accm[hf][gg] *= alpha;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        O[hf][r][0] *= alpha;
                        O[hf][r][1] *= alpha;
                    }
                }
            }
            const float p0 = __builtin_amdgcn_exp2f(s0 - m_sh[hf]);
            const float p1 = __builtin_amdgcn_exp2f(s1 - m_sh[hf]);
            l_run[hf] += p0 + p1;
            {
                const uint8_t* v0p = &mbuf[m_vm];
                const uint8_t* v1p = &mbuf[MB + m_vm];
                uint32_t vm0[(NG + 1) / 2], vm1[(NG + 1) / 2];
                if constexpr (NG == 4) {
                    const uint2 u0 = *reinterpret_cast<const uint2*>(v0p);
                    const uint2 u1 = *reinterpret_cast<const uint2*>(v1p);
                    vm0[0] = u0.x; vm0[1] = u0.y; vm1[0] = u1.x; vm1[1] = u1.y;
                } else if constexpr (NG == 2) {
                    vm0[0] = *reinterpret_cast<const uint32_t*>(v0p);
                    vm1[0] = *reinterpret_cast<const uint32_t*>(v1p);
                } else {
                    vm0[0] = *reinterpret_cast<const uint16_t*>(v0p);
                    vm1[0] = *reinterpret_cast<const uint16_t*>(v1p);
                }
#pragma unroll
                for (int gg = 0; gg < NG; ++gg) {
                    // never-written slots may hold NaN: select, do not multiply
                    const float v0 = ok0 ? h2f(vm0[gg >> 1], gg & 1) : 0.f;
                    const float v1 = ok1 ? h2f(vm1[gg >> 1], gg & 1) : 0.f;
                    accm[hf][gg] = fmaf(p0, v0, fmaf(p1, v1, accm[hf][gg]));
                }
            }
            pbuf[hf][kb][n16] = p0;
            pbuf[hf][kb][16 + n16] = p1;
            __builtin_amdgcn_wave_barrier();

            // ---- 8-bit operand of (head jq, block gq, group kb): w = p' Delta_V of
            // tokens 32 tl + 8 gq + e, its scale max w / 255 and codes
            float sig = 0.f;
            uint32_t ulo = 0u, uhi = 0u;
            if (kb < NG) {
                const float4 pa = *reinterpret_cast<const float4*>(&pbuf[hf][jq][8 * gq]);
                const float4 pb = *reinterpret_cast<const float4*>(&pbuf[hf][jq][8 * gq + 4]);
                const uint4 vd = *reinterpret_cast<const uint4*>(&mbuf[m_vdu]);
                const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
                const uint32_t vdw[4] = {vd.x, vd.y, vd.z, vd.w};
                float w[8], wmax = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = pr[e] * h2f(vdw[e >> 1], e & 1);
                    const int tok = 32 * tl + 8 * gq + e;
                    w[e] = (full || (tok >= t_lo && tok < t_hi)) ? x : 0.f;
                    wmax = __builtin_elementwise_maximum(wmax, w[e]);   // no NaN: no canonicalising
                }
                const float rr = wmax > kTinyW ? 255.0f * __builtin_amdgcn_rcpf(wmax) : 0.f;
                int uc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) uc[e] = (int)fminf(rintf(w[e] * rr), 255.0f);
                // the matrix core multiplies signed bytes: carry u - 128 (exact in
                // [-128, 127]) and add 128 sum c back through the ones product
                ulo = pack_i8x4(uc[0] - 128, uc[2] - 128, uc[4] - 128, uc[6] - 128);
                uhi = pack_i8x4(uc[1] - 128, uc[3] - 128, uc[5] - 128, uc[7] - 128);
                sig = wmax * (1.0f / 255.0f);
            }
            sbuf[hf][kb][jq][gq] = sig;
            uint32_t Alo[NG], Ahi[NG];
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                const uint32_t sl = (uint32_t)__shfl((int)ulo, 16 * gg + n16);
                const uint32_t sh = (uint32_t)__shfl((int)uhi, 16 * gg + n16);
                Alo[gg] = kb == gq ? sl : 0u;
                Ahi[gg] = kb == gq ? sh : 0u;
            }
            __builtin_amdgcn_wave_barrier();
            float4 sg[NG];
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) sg[gg] = *reinterpret_cast<const float4*>(&sbuf[hf][gg][kb][0]);

            // ---- PV: integer sums per 8-token block, sum u c = sum (u - 128) c +
            // 128 sum c (the ones operand sums the codes of block kb), combined by
            // the blocks' scales
            const uint32_t ones = kb == gq ? 0x01010101u : 0u;
            const uint4 vc0 = stage[2][lane], vc1 = stage[3][lane];
            const uint32_t vcw[8] = {vc0.x, vc0.y, vc0.z, vc0.w, vc1.x, vc1.y, vc1.z, vc1.w};
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int gg = (32 * blk) / G;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint32_t vw = vcw[2 * blk + hh];
                    const i32x4_t Dc = mfma_i8_32(ones, ones, nib_lo(vw), nib_hi(vw), z);
                    const i32x4_t Dp = mfma_i8_32(Alo[gg], Ahi[gg], nib_lo(vw), nib_hi(vw), z);
                    const float d0 = (float)(Dp[0] + 128 * Dc[0]), d1 = (float)(Dp[1] + 128 * Dc[1]);
                    const float d2 = (float)(Dp[2] + 128 * Dc[2]), d3 = (float)(Dp[3] + 128 * Dc[3]);
                    O[hf][blk][hh] += (sg[gg].x * d0 + sg[gg].y * d1) + (sg[gg].z * d2 + sg[gg].w * d3);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    };

    {
        Kv4Tile t;
        const uint8_t* T0 = page(2 * tile_first);
        const uint8_t* T1 = page(2 * tile_first + 1);
        load_tile(t, T0, T1);
        const uint8_t* C0 = page(2 * tile_first + 2);
        const uint8_t* C1 = page(2 * tile_first + 3);
        auto advance = [&](int tl, auto full_tag) {
            pace.tile(tile_end - tl);
            const bool more = tl + 1 < tile_end;
            const uint8_t* N0 = more ? C0 : T0;
            const uint8_t* N1 = more ? C1 : T1;
            C0 = page(2 * tl + 4);
            C1 = page(2 * tl + 5);
            step(t, tl, N0, N1, full_tag);
            T0 = N0;
            T1 = N1;
        };
        int tl = tile_first;
        if (32 * tl < t_lo || 32 * tl + 32 > t_hi) advance(tl++, std::false_type{});
        const int full_end = t_hi / 32;
        for (; tl < full_end; ++tl) advance(tl, std::true_type{});
        if (tl < tile_end) advance(tl, std::false_type{});
    }

#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const float l = row16_sum(l_run[hf]);
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) accm[hf][gg] = row16_sum(accm[hf][gg]);
        const float inv = 1.0f / l;
        if (4 * hf + kb >= g.gqa) continue;      // a head past the q/kv ratio
        float* dst = rec + (4 * hf + kb) * (g.d + kPartPad);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dst[32 * r + n16] = (O[hf][r][0] + accm[hf][(32 * r) / G]) * inv;
            dst[32 * r + 16 + n16] = (O[hf][r][1] + accm[hf][(32 * r) / G]) * inv;
        }
        if (n16 == 0) dst[g.d] = m_sh[hf] + log2f(l);
    }
}

// Protected part of the integer path: integer QK of the INT8 query against
// the ring's INT8 keys on the matrix core (v_mfma_i32_16x16x64_i8; A = the
// query codes of head n16/4 on channels 32 kb + 8 (n16%4) + [0, 8), in the
// product that covers those bytes only; B = 16 key bytes of entry n16), then
// the PV of mfma_prot_kv4: binary32-accurate products with the dequantized
// INT8 values, no probability quantization.
// NH = 2 (q/kv ratio 8): q heads 0-3 and then 4-7 on each tile's loads.
template <bool ROT, int NH = 1>
__device__ __forceinline__ void mfma_prot_int(const DecodeArgs& a, int b, int h, float* rec)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int jq = n16 >> 2, gq = n16 & 3;
    const int n8 = regions_of(seq_len(a, b), g.S, g.R).n8;
    if (n8 <= 0) return;
    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const uint8_t* ring = a.side + (int64_t)a.layer * g.layer_side + ((int64_t)slot * g.Hkv + h) * g.rb;
    const uint8_t* vreg = ring + (int64_t)g.SR32 * g.d;
    const uint16_t* ksc = reinterpret_cast<const uint16_t*>(ring + (int64_t)2 * g.SR32 * g.d);
    const uint16_t* vsc = ksc + g.SR32;

    u32x4_t A1[NH], A2[NH];
    float c2[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        // rows of heads past the q/kv ratio (GQA 1 and 2 run in the four-head
        // layout) carry q = 0; their results are not written
        const int jh = 4 * hf + jq;
        const bool qreal = jh < g.gqa;
        const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * g.gqa + (qreal ? jh : 0)) * g.d;
        uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * kb + 8 * gq);
        if (!qreal) u = make_uint4(0u, 0u, 0u, 0u);
        float q[8] = {bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y),
                      bf16_lo(u.z), bf16_hi(u.z), bf16_lo(u.w), bf16_hi(u.w)};
        if constexpr (ROT) {
            // channel bits 3-4 are lane bits 0-1 (gq), bits 5-6 lane bits 4-5 (kb)
            wht_local(q);
            wht_lanes(q, 1);
            wht_lanes(q, 2);
            wht_lanes(q, 16);
            wht_lanes(q, 32);
            wht_scale(q);
        }
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(q[c]));
        amax = fmaxf(amax, dpp<0xB1>(amax));
        amax = rows_max(fmaxf(amax, dpp<0x4E>(amax)));
        const uint16_t sb = plus_zero16(f32_to_f16_bits(__fdiv_rn(amax, 127.0f)));
        const float S = half_bits_to_float(sb);
        int c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = int8_code(q[i], S, sb);
        const uint32_t w0 = pack_i8x4(c[0], c[1], c[2], c[3]), w1 = pack_i8x4(c[4], c[5], c[6], c[7]);
        A1[hf] = u32x4_t{gq == 0 ? w0 : 0u, gq == 0 ? w1 : 0u, gq == 1 ? w0 : 0u, gq == 1 ? w1 : 0u};
        A2[hf] = u32x4_t{gq == 2 ? w0 : 0u, gq == 2 ? w1 : 0u, gq == 3 ? w0 : 0u, gq == 3 ? w1 : 0u};
        c2[hf] = a.scale2 * __shfl(S, 4 * kb);
    }

    // E[hf][h]: rows (head, block r), channels 32 r + 16 h + n16 (block-diagonal PV)
    f32x4_t E[NH][2], W[NH];
    float m_sh[NH], l_run[NH];
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        E[hf][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        E[hf][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        W[hf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_sh[hf] = -INFINITY;
        l_run[hf] = 0.f;
    }
    __shared__ __attribute__((aligned(16))) float pbuf8[NH][4][32];
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0

    for (int e0 = 0; e0 < n8; e0 += 32) {
        // ---- loads: K rows of entries e0 + n16, e0 + 16 + n16 (bytes 32 kb ..),
        // V codes of entries e0 + 8 kb .. + 7 (this lane's 8 channels), scales
        const uint8_t* kr = ring + (int64_t)(e0 + n16) * g.d + 32 * kb;
        const uint4 k00 = *reinterpret_cast<const uint4*>(kr);
        const uint4 k01 = *reinterpret_cast<const uint4*>(kr + 16);
        const uint4 k10 = *reinterpret_cast<const uint4*>(kr + 16 * g.d);
        const uint4 k11 = *reinterpret_cast<const uint4*>(kr + 16 * g.d + 16);
        const uint8_t* vb = vreg + (int64_t)((e0 >> 3) + kb) * (8 * kHeadDim) + 64 * n16;
        const uint4 v0 = *reinterpret_cast<const uint4*>(vb);
        const uint4 v1 = *reinterpret_cast<const uint4*>(vb + 16);
        const uint4 v2 = *reinterpret_cast<const uint4*>(vb + 32);
        const uint4 v3 = *reinterpret_cast<const uint4*>(vb + 48);
        const float sk0 = half_bits_to_float(ksc[e0 + n16]);
        const float sk1 = half_bits_to_float(ksc[e0 + 16 + n16]);
        const uint4 svp = *reinterpret_cast<const uint4*>(vsc + e0 + 8 * kb);

#pragma unroll
        for (int hf = 0; hf < NH; ++hf) {
            // ---- QK: integer sums of head kb over sub-block r of each lane's 32 channels
            const i32x4_t z = {0, 0, 0, 0};
            i32x4_t D0 = mfma_i8_64(A1[hf], u32x4_t{k00.x, k00.y, k00.z, k00.w}, z);
            D0 = mfma_i8_64(A2[hf], u32x4_t{k01.x, k01.y, k01.z, k01.w}, D0);
            i32x4_t D1 = mfma_i8_64(A1[hf], u32x4_t{k10.x, k10.y, k10.z, k10.w}, z);
            D1 = mfma_i8_64(A2[hf], u32x4_t{k11.x, k11.y, k11.z, k11.w}, D1);
            const bool ok0 = e0 + n16 < n8, ok1 = e0 + 16 + n16 < n8;
            float s0 = (float)((D0[0] + D0[1]) + (D0[2] + D0[3])) * sk0 * c2[hf];
            float s1 = (float)((D1[0] + D1[1]) + (D1[2] + D1[3])) * sk1 * c2[hf];
            s0 = ok0 ? s0 : -INFINITY;
            s1 = ok1 ? s1 : -INFINITY;
            const float mx = row16_max(fmaxf(s0, s1));
            {
                const bool grow = mx > m_sh[hf] + (kPScale + kSlack);
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float m_new = grow ? mx - kPScale : m_sh[hf];
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_sh[hf] - m_new) : 1.0f;
                    m_sh[hf] = m_new;
                    l_run[hf] *= alpha;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) E[hf][hh] *= alpha;
                    W[hf] *= alpha;
                }
            }
            const float p0 = __builtin_amdgcn_exp2f(s0 - m_sh[hf]);
            const float p1 = __builtin_amdgcn_exp2f(s1 - m_sh[hf]);
            l_run[hf] += p0 + p1;
            pbuf8[hf][kb][n16] = p0;
            pbuf8[hf][kb][16 + n16] = p1;
            __builtin_amdgcn_wave_barrier();
            const float4 pa = *reinterpret_cast<const float4*>(&pbuf8[hf][jq][8 * kb]);
            const float4 pb = *reinterpret_cast<const float4*>(&pbuf8[hf][jq][8 * kb + 4]);

            // ---- PV: w = p' s_V of head jq, entries e0 + 8 kb + e
            const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
            const uint32_t svw[4] = {svp.x, svp.y, svp.z, svp.w};
            float wv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // entries past the end may hold garbage scales: select, do not multiply
                const float w = fmaf(pr[e], h2f(svw[e >> 1], e & 1), 0.0f);
                wv[e] = e0 + 8 * kb + e < n8 ? w : 0.0f;
            }
            u32x4_t ahi, alo;
            constexpr int pe[4][2] = {{0, 2}, {1, 3}, {4, 6}, {5, 7}};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hw, lw;
                split_bf16(wv[pe[i][0]], wv[pe[i][1]], hw, lw);
                ahi[i] = hw;
                alo[i] = lw;
            }
            const uint32_t vw[16] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                                     v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w};
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const uint64_t rows = 0x1111111111111111ull << blk;
                const u32x4_t bh = {keep_lanes(ahi[0], rows), keep_lanes(ahi[1], rows),
                                    keep_lanes(ahi[2], rows), keep_lanes(ahi[3], rows)};
                const u32x4_t bl = {keep_lanes(alo[0], rows), keep_lanes(alo[1], rows),
                                    keep_lanes(alo[2], rows), keep_lanes(alo[3], rows)};
                const u32x4_t b0 = widen_i8(vw[4 * blk], vw[4 * blk + 1]);
                const u32x4_t b1 = widen_i8(vw[4 * blk + 2], vw[4 * blk + 3]);
                E[hf][0] = mfma_bf16(bh, b0, E[hf][0]);
                E[hf][1] = mfma_bf16(bh, b1, E[hf][1]);
                E[hf][0] = mfma_bf16(bl, b0, E[hf][0]);
                E[hf][1] = mfma_bf16(bl, b1, E[hf][1]);
            }
            W[hf] = mfma_bf16(ahi, ones, W[hf]);
            W[hf] = mfma_bf16(alo, ones, W[hf]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- epilogue: lane l holds head 4 hf + kb, channels 32 r + 16 h + n16 in E[hf][h][r]
    // (every block row of W carries the same sum; row 0 is used)
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
        const float l = row16_sum(l_run[hf]);
        const float inv = 1.0f / l;
        if (4 * hf + kb >= g.gqa) continue;      // a head past the q/kv ratio
        float* dst = rec + (4 * hf + kb) * (g.d + kPartPad);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dst[32 * r + n16] = (ldexpf(E[hf][0][r], 133) - 128.0f * W[hf][0]) * inv;
            dst[32 * r + 16 + n16] = (ldexpf(E[hf][1][r], 133) - 128.0f * W[hf][0]) * inv;
        }
        if (n16 == 0) dst[g.d] = m_sh[hf] + log2f(l);
    }
}

// Integer path, q/kv ratios 1, 2 and 4.
template <int G, bool ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void decode_int_mfma_kernel(DecodeArgs a)
{
    walk_units(a, [&](int b, int h) { mfma_prot_int<ROT>(a, b, h, prot_ptr(a, b * a.g.Hkv + h)); },
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_int<G, ROT>(a, b, h, lo, hi, rec, pace);
               });
}

// Integer path, q/kv ratio 8: two four-head halves per tile.  The integer
// operands of the second half need more registers than three waves per SIMD
// leave without spilling inside the tile loop: two waves per SIMD.
template <int G, bool ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_int_mfma8_kernel(DecodeArgs a)
{
    walk_units(a, [&](int b, int h) { mfma_prot_int<ROT, 2>(a, b, h, prot_ptr(a, b * a.g.Hkv + h)); },
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_int<G, ROT, 2>(a, b, h, lo, hi, rec, pace);
               });
}

// KV8 kind: every position from INT8 pages (no protected parts).
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void decode_kv8_mfma_kernel(DecodeArgs a)
{
    walk_units(a, [&](int, int) {},
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_kv8(a, b, h, lo, hi, rec, pace);
               });
}

// KV8 kind, q/kv ratios 5 to 8: two four-head halves per staged tile.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kv8_mfma8_kernel(DecodeArgs a)
{
    walk_units(a, [&](int, int) {},
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_kv8<2>(a, b, h, lo, hi, rec, pace);
               });
}

__global__ __launch_bounds__(64) void decode_bf16_mfma_kernel(DecodeArgs a)
{
    walk_units(a, [&](int, int) {},
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_bf16(a, b, h, lo, hi, rec, pace);
               });
}

// BF16 comparator, q/kv ratios 5 to 8: two four-head halves on each tile's loads.
__global__ __launch_bounds__(64) void decode_bf16_mfma8_kernel(DecodeArgs a)
{
    walk_units(a, [&](int, int) {},
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   mfma_item_bf16<2>(a, b, h, lo, hi, rec, pace);
               });
}

}  // namespace kv4
