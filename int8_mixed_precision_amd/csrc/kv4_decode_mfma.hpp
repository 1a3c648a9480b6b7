// kv4_decode_mfma.hpp -- matrix-core (MFMA) decode attention for GQA group 4.
//
// One wave per work item (sequence, kv head, context split); the split is
// walked in 32-token tiles (two pages).  Both contractions of a tile run on
// v_mfma_f32_16x16x32_bf16 (A rows x 32 k-slots x 16 columns, fp32 accumulate):
//
//   QK (INT4 keys): rows = 16 tokens, k = 32 channels of one 32-channel block,
//     columns = (q head j, channel block g).  The B operand holds q_j only in
//     the k-slots of block g, so one tile of four MFMAs yields, per token, the
//     partial products q_{j,g} . c_{t,g} of every block separately; the affine
//     identity q.k^ = Delta (q.c) + m sum(q) (KV4-RL eq. 5.1, applied per group)
//     then turns them into scores.
//   PV (INT4 values): rows = (q head j, channel block g), k = 32 tokens,
//     columns = 16 channels of one block.  Row (j, g) carries p_{j,t} Delta_{t,g}
//     so that the per-token, per-group scale of eq. 3.3 is applied exactly
//     before the token sum; the offset term sum_t p m is accumulated on the
//     vector ALU.
//
// Exactness: 4-bit codes are widened to the bf16 values 16 + c (exact; one
// shift and one and-or per pair), q is used at its bf16 value, and the bf16 A
// operand of PV is split as hi + lo (both rounded to nearest), which carries
// p*Delta to about 2^-18 relative; accumulation is fp32 throughout.  The +16
// bias is removed with sum(q) on the QK side and, on the PV side, with the sum
// of exactly the A operand used (one more MFMA against a column of ones).
//
// Masking: tokens outside the work item (and never-written slots of a page)
// get score -inf and weight exactly 0 by selection, so garbage bytes can
// never reach the result.
#pragma once

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

// Eight 4-bit codes (code e in bits 4e..4e+3) -> four bf16 pairs holding the
// exact values 16 + code; pair i = (code i, code i+4).
__device__ __forceinline__ u32x4_t widen_codes(uint32_t w)
{
    const uint32_t M = 0x00780078u, B16 = 0x41804180u;
    u32x4_t r;
    r[0] = ((w << 3) & M) | B16;
    r[1] = ((w >> 1) & M) | B16;
    r[2] = ((w >> 5) & M) | B16;
    r[3] = ((w >> 9) & M) | B16;
    return r;
}

__device__ __forceinline__ float dpp_f(float x, int ctrl);

// Sum over the 4 lanes of a quad (lanes 4k..4k+3).
__device__ __forceinline__ float quad_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
    return x;
}

__device__ __forceinline__ float half_of(uint32_t w, int hi) { return half_bits_to_float(hi ? (w >> 16) : (w & 0xFFFFu)); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float x, float y)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}

// Split (x, y) into bf16 high parts (nearest) and bf16 remainders (nearest):
// x = hi + lo + O(2^-18 |x|).
__device__ __forceinline__ void split_bf16(float x, float y, uint32_t& hi, uint32_t& lo)
{
    hi = pack_bf16(x, y);
    lo = pack_bf16(x - __uint_as_float(hi << 16), y - __uint_as_float(hi & 0xFFFF0000u));
}

// (x & m) | o in one VOP3 instruction (the constants live in registers).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
    return r;
}

// Eight 4-bit codes -> four bf16 pairs 16 + code (pair i = codes i, i+4).
__device__ __forceinline__ u32x4_t widen(uint32_t w, uint32_t bias)
{
    const uint32_t M = 0x00780078u;
    u32x4_t r;
    r[0] = and_or(w << 3, M, bias);
    r[1] = and_or(w >> 1, M, bias);
    r[2] = and_or(w >> 5, M, bias);
    r[3] = and_or(w >> 9, M, bias);
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

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint32_t w, int k)
{
    return (float)__builtin_bit_cast(f16x2_t, w)[k];
}

// Online-softmax state of one INT4 work item.  The exponentials use a
// reference maximum m_ref that is raised only when a tile's maximum exceeds it
// by more than kSlack (base-2 units), so accumulators are rescaled rarely;
// l_run uses the same reference, which keeps the result exact.  With p <=
// 2^64, w (16 + c) <= 2^64 * 65504 * 31 and sums over any context stay far
// below the fp32 range.
constexpr float kSlack = 64.0f;

struct Kv4Acc {
    f32x4_t O[8];       // PV accumulators (rows = (head kb, block r) of this lane)
    f32x4_t W;          // sums over tokens of the PV A operand, per (head, block)
    float m_ref, l_run, accm;
};

// The 16-byte loads one lane makes for one 32-token tile: the K part (read by
// QK) and the V part (read by PV), loaded separately so that each can be
// refilled for the next tile as soon as the current one is consumed.
struct Kv4K {
    uint4 kc0, kc1;     // K codes of this lane's QK rows (tokens +0..3 and +4..7), its block
    uint4 kd, km;       // K Delta, m of its (block, 8 tokens)
};
struct Kv4V {
    uint4 vc0, vc1;     // V code words of its column blocks (tokens of its k-block)
    uint4 vd, vm;       // V Delta, m of its (block, 8 tokens)
};

__device__ __forceinline__ void kv4_load_k(Kv4K& t, const uint8_t* PK, const uint8_t* PM,
                                           const Geo& g, int kc_off0, int meta_off)
{
    t.kc0 = *reinterpret_cast<const uint4*>(PK + kc_off0);
    t.kc1 = *reinterpret_cast<const uint4*>(PK + kc_off0 + 4 * (kHeadDim / 2));
    t.kd = *reinterpret_cast<const uint4*>(PM + g.off_kd + meta_off);
    t.km = *reinterpret_cast<const uint4*>(PM + g.off_km + meta_off);
}

__device__ __forceinline__ void kv4_load_v(Kv4V& t, const uint8_t* PM, const Geo& g, int meta_off,
                                           int vc_off)
{
    t.vc0 = *reinterpret_cast<const uint4*>(PM + vc_off);
    t.vc1 = *reinterpret_cast<const uint4*>(PM + vc_off + 4 * 64);
    t.vd = *reinterpret_cast<const uint4*>(PM + g.off_vd + meta_off);
    t.vm = *reinterpret_cast<const uint4*>(PM + g.off_vm + meta_off);
}

// Scores of one 32-token tile for head jq: sc[e] = log2-scaled q.k^ of token
// tok0 + e (-inf outside [t_lo, t_hi) when the tile is partial).  Returns the
// tile maximum of head jq (the same in every lane of that head).
__device__ __forceinline__ float kv4_scores(float (&sc)[8], const Kv4K& t, const u32x4_t (&bq)[4],
                                            float sq, float sq16, float c2, bool full, int tok0,
                                            int t_lo, int t_hi)
{
    const uint32_t bias = 0x41804180u;
    // QK: tokens tok0 + e, e = 0..3 in D0 and 4..7 in D1, column (jq, gq)
    f32x4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
    D0 = mfma_bf16(widen(t.kc0.x, bias), bq[0], D0);
    D1 = mfma_bf16(widen(t.kc1.x, bias), bq[0], D1);
    D0 = mfma_bf16(widen(t.kc0.y, bias), bq[1], D0);
    D1 = mfma_bf16(widen(t.kc1.y, bias), bq[1], D1);
    D0 = mfma_bf16(widen(t.kc0.z, bias), bq[2], D0);
    D1 = mfma_bf16(widen(t.kc1.z, bias), bq[2], D1);
    D0 = mfma_bf16(widen(t.kc0.w, bias), bq[3], D0);
    D1 = mfma_bf16(widen(t.kc1.w, bias), bq[3], D1);
    const uint32_t kdw[4] = {t.kd.x, t.kd.y, t.kd.z, t.kd.w};
    const uint32_t kmw[4] = {t.km.x, t.km.y, t.km.z, t.km.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float acc = e < 4 ? D0[e] : D1[e - 4];
        // block partial of q.k^ = Delta (q.c) + m sum(q), summed over the 4 blocks
        const float v = fmaf(h2f(kdw[e >> 1], e & 1), acc - sq16, h2f(kmw[e >> 1], e & 1) * sq);
        sc[e] = quad_sum(v) * c2;
    }
    if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tok = tok0 + e;
            sc[e] = (tok >= t_lo && tok < t_hi) ? sc[e] : -INFINITY;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                     fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    return rows_max(mx);
}

// PV part of one tile with the reference maximum m_ref of head jq.
__device__ __forceinline__ void kv4_pv(Kv4Acc& st, const float (&sc)[8], const Kv4V& t, bool full,
                                       int tok0, int t_lo, int t_hi)
{
    const uint32_t bias = 0x41804180u;
    // A operand: w = p * Delta_V (exactly 0 outside the item), split hi + lo
    const uint32_t vdw[4] = {t.vd.x, t.vd.y, t.vd.z, t.vd.w};
    const uint32_t vmw[4] = {t.vm.x, t.vm.y, t.vm.z, t.vm.w};
    float wv[8], pm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(sc[e] - st.m_ref);
        wv[e] = fmaf(p, h2f(vdw[e >> 1], e & 1), 0.0f);
        pm[e] = fmaf(p, h2f(vmw[e >> 1], e & 1), 0.0f);
        st.l_run += p;
    }
    if (!full) {                          // metadata of slots outside the item may be NaN
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tok = tok0 + e;
            const bool ok = tok >= t_lo && tok < t_hi;
            wv[e] = ok ? wv[e] : 0.0f;
            pm[e] = ok ? pm[e] : 0.0f;
        }
    }
    st.accm += ((pm[0] + pm[1]) + (pm[2] + pm[3])) + ((pm[4] + pm[5]) + (pm[6] + pm[7]));
    u32x4_t ahi, alo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t hw, lw;
        split_bf16(wv[i], wv[i + 4], hw, lw);
        ahi[i] = hw;
        alo[i] = lw;
    }
    // column block s = channels 32 (s/2) + 16 (s%2) + n16
    const uint32_t vcw[8] = {t.vc0.x, t.vc0.y, t.vc0.z, t.vc0.w, t.vc1.x, t.vc1.y, t.vc1.z, t.vc1.w};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const u32x4_t bv = widen(vcw[s], bias);
        st.O[s] = mfma_bf16(ahi, bv, st.O[s]);
        st.O[s] = mfma_bf16(alo, bv, st.O[s]);
    }
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0
    st.W = mfma_bf16(ahi, ones, st.W);
    st.W = mfma_bf16(alo, ones, st.W);
}

// Raise the reference maximum of every head whose tile maximum mx exceeds it
// by more than kSlack, rescaling what was accumulated against the old one
// (alpha = 1 for the other heads).
__device__ __forceinline__ void kv4_raise(Kv4Acc& st, float mx)
{
    const int kb = threadIdx.x >> 4;
    const bool grow = mx > st.m_ref + kSlack;
    const float m_new = grow ? mx : st.m_ref;
    const float alpha = grow ? __builtin_amdgcn_exp2f(st.m_ref - m_new) : 1.0f;
    st.m_ref = m_new;
    st.l_run *= alpha;
    st.accm *= alpha;
    const float alpha_d = __shfl(alpha, 4 * kb);      // head kb of the D rows held here
#pragma unroll
    for (int s = 0; s < 8; ++s) st.O[s][s >> 1] *= alpha_d;
    st.W *= alpha_d;
}

// ---------------------------------------------------------------------------
// INT4 context split of the mixed cache.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mfma_item_kv4(const DecodeArgs& a, int b, int h, int split)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;   // MFMA column (or A row) and k-block
    const int jq = n16 >> 2, gq = n16 & 3;       // (head, 32-channel block) of that row/column
    const int n = clampi(a.seq_lens[b], 0, a.max_ctx);
    const Regions rg = regions_of(n, g.S, g.R);
    const int t_lo = max(split * a.split, g.S);
    const int t_hi = min((split + 1) * a.split, rg.rec_start);
    if (t_hi <= t_lo) return;

    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    const uint8_t* hbase = a.pages + (int64_t)a.layer * g.layer_pages + (int64_t)h * g.pb;
    const int64_t page_stride = (int64_t)g.Hkv * g.pb;
    const int mg = (32 * gq) / g.G;              // metadata group of block gq

    // ---- q operands: lane (column (jq, gq), k-block kb) holds q_jq on block gq
    const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * 4 + jq) * g.d;
    u32x4_t bq[4];
    float sq = 0.f;
    {
        const uint4* q4 = reinterpret_cast<const uint4*>(qrow + 32 * gq);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 u = q4[i];
            sq += bf16_lo(u.x) + bf16_hi(u.x) + bf16_lo(u.y) + bf16_hi(u.y) +
                  bf16_lo(u.z) + bf16_hi(u.z) + bf16_lo(u.w) + bf16_hi(u.w);
            // k-slot pairs (c, c+4) of channels 32 gq + 8 i + c
            u32x4_t v;
            v[0] = (u.x & 0xFFFFu) | (u.z << 16);
            v[1] = (u.x >> 16) | (u.z & 0xFFFF0000u);
            v[2] = (u.y & 0xFFFFu) | (u.w << 16);
            v[3] = (u.y >> 16) | (u.w & 0xFFFF0000u);
            u32x4_t z = {0u, 0u, 0u, 0u};
            bq[i] = (gq == kb) ? v : z;
        }
    }
    const float sq16 = 16.0f * sq;
    const float c2 = a.scale2;

    Kv4Acc st;
#pragma unroll
    for (int s = 0; s < 8; ++s) st.O[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.W = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m_ref = -INFINITY;
    st.l_run = 0.f;
    st.accm = 0.f;

    // fixed per-lane offsets inside a 32-token tile
    const int rq = n16 >> 2, rr = n16 & 3;       // QK row n16 -> tokens 8 rq + rr (+4)
    const int kc_off0 = g.off_kc + (8 * (rq & 1) + rr) * (g.d / 2) + 16 * kb;
    const int meta_off = 2 * (mg * kPage + 8 * (kb & 1));
    const int vc_off = g.off_vc + 4 * ((kb & 1) * g.d + 4 * n16);

    // Page ids of the item's tiles, two per lane: lane l holds the pages of
    // relative index l and l + 64 from the item's first page.  Context splits
    // are at most kMaxSplit = 2048 tokens (64 tiles), so this covers the item.
    int tbase = t_lo / 32;
    int pid_a = 0, pid_b = 0;
    auto load_pids = [&](int tb) {
        tbase = tb;
        const int pi = 2 * tb + lane;
        pid_a = clampi(bt[min(pi, g.max_pages - 1)], 0, g.num_pages - 1);
        pid_b = clampi(bt[min(pi + 64, g.max_pages - 1)], 0, g.num_pages - 1);
    };
    auto page_ptrs = [&](int tl, const uint8_t*& PK, const uint8_t*& PM) {
        const int rel = 2 * (tl - tbase);            // < 128: an item spans <= 64 tiles
        const int p0 = rel < 64 ? __builtin_amdgcn_readlane(pid_a, rel)
                                : __builtin_amdgcn_readlane(pid_b, rel - 64);
        const int p1 = rel + 1 < 64 ? __builtin_amdgcn_readlane(pid_a, rel + 1)
                                    : __builtin_amdgcn_readlane(pid_b, rel + 1 - 64);
        const uint8_t* P0 = hbase + p0 * page_stride;
        const uint8_t* P1 = hbase + p1 * page_stride;
        PK = (rq >> 1) ? P1 : P0;                // page of this lane's QK rows
        PM = (kb >> 1) ? P1 : P0;                // page of this lane's k-block tokens
    };
    const int tile_first = t_lo / 32, tile_end = (t_hi + 31) / 32;
    load_pids(tile_first);
    // Software pipeline over tiles, in registers: the K part of tile t+1 is
    // requested as soon as QK(t) has read the K part of tile t, and the V part
    // as soon as PV(t) has read the V part, so each load overlaps about half a
    // tile of compute without a second register set.
    Kv4K kt;
    Kv4V vt;
    {
        const uint8_t *PK, *PM;
        page_ptrs(tile_first, PK, PM);
        kv4_load_k(kt, PK, PM, g, kc_off0, meta_off);
        kv4_load_v(vt, PM, g, meta_off, vc_off);
    }
    for (int tl = tile_first; tl < tile_end; ++tl) {
        const bool full = 32 * tl >= t_lo && 32 * tl + 32 <= t_hi;
        const int tok0 = 32 * tl + 8 * kb;
        const bool more = tl + 1 < tile_end;
        const uint8_t *PK = nullptr, *PM = nullptr;
        if (more) page_ptrs(tl + 1, PK, PM);
        float sc[8];
        const float mx = kv4_scores(sc, kt, bq, sq, sq16, c2, full, tok0, t_lo, t_hi);
        if (more) kv4_load_k(kt, PK, PM, g, kc_off0, meta_off);
        kv4_raise(st, mx);
        kv4_pv(st, sc, vt, full, tok0, t_lo, t_hi);
        if (more) kv4_load_v(vt, PM, g, meta_off, vc_off);
    }

    // ---- reduce the per-k-block partial sums and hand them to the output lanes
    const float l_run = rows_sum(st.l_run);
    const float accm = rows_sum(st.accm);
    __shared__ float sh_c[16], sh_l[4], sh_m[4];
    if (kb == 0) {
        sh_c[n16] = accm;
        if (gq == 0) { sh_l[jq] = l_run; sh_m[jq] = st.m_ref; }
    }
    __syncthreads();
    const float lj = sh_l[kb];
    const float inv = 1.0f / lj;
    float* dst = part_ptr(a, b, h, split, kb);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int c = 32 * (s >> 1) + 16 * (s & 1) + n16;
        dst[c] = (st.O[s][s >> 1] - 16.0f * st.W[s >> 1] + sh_c[4 * kb + (s >> 1)]) * inv;
    }
    if (n16 == 0) dst[g.d] = sh_m[kb] + log2f(lj);
}

// ---------------------------------------------------------------------------
// BF16 comparator split (same tiling; keys and values used as stored).
//   QK: rows = 16 tokens, k = 8 consecutive channels per k-block, columns =
//       (head j, 0): only column block 0 of each head is non-zero.
//   PV: rows = (head j, part): part 0 = bf16(p), part 1 = bf16(p - part 0),
//       parts 2-3 zero;
//       columns = channels 16 s + n16; k = tokens 8 kb .. 8 kb + 7 in order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mfma_item_bf16(const DecodeArgs& a, int b, int h, int split)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int jq = n16 >> 2, gq = n16 & 3;
    const int n = clampi(a.seq_lens[b], 0, a.max_ctx);
    const int t_lo = split * a.split;
    const int t_hi = min((split + 1) * a.split, n);
    if (t_hi <= t_lo) return;
    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    const uint8_t* hbase = a.pages + (int64_t)a.layer * g.layer_pages + (int64_t)h * g.pb;
    const int64_t page_stride = (int64_t)g.Hkv * g.pb;

    const uint16_t* qrow = a.q + ((int64_t)b * g.Hq + h * 4 + jq) * g.d;
    u32x4_t bq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * i + 8 * kb);
        u32x4_t v = {u.x, u.y, u.z, u.w}, z = {0u, 0u, 0u, 0u};
        bq[i] = gq == 0 ? v : z;
    }
    const float c2 = a.scale2;
    f32x4_t O[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) O[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const int rq = n16 >> 2, rr = n16 & 3;
    const int k_off0 = 2 * ((8 * (rq & 1) + rr) * g.d + 8 * kb);
    const int k_off1 = k_off0 + 2 * 4 * g.d;
    const int v_off = kPage * g.d * 2 + 2 * (((kb & 1) * g.d + n16) * kHalf);

    for (int ts = (t_lo / 32) * 32; ts < t_hi; ts += 32) {
        const int pi = ts / kPage;
        const int p0 = clampi(bt[min(pi, g.max_pages - 1)], 0, g.num_pages - 1);
        const int p1 = clampi(bt[min(pi + 1, g.max_pages - 1)], 0, g.num_pages - 1);
        const uint8_t* P0 = hbase + p0 * page_stride;
        const uint8_t* P1 = hbase + p1 * page_stride;
        const uint8_t* PK = (rq >> 1) ? P1 : P0;
        const uint8_t* PM = (kb >> 1) ? P1 : P0;
        f32x4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 k0 = *reinterpret_cast<const uint4*>(PK + k_off0 + 64 * i);
            uint4 k1 = *reinterpret_cast<const uint4*>(PK + k_off1 + 64 * i);
            D0 = mfma_bf16(u32x4_t{k0.x, k0.y, k0.z, k0.w}, bq[i], D0);
            D1 = mfma_bf16(u32x4_t{k1.x, k1.y, k1.z, k1.w}, bq[i], D1);
        }
        float sc[8], mx = -INFINITY;
        bool valid[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tok = ts + 8 * kb + e;
            valid[e] = tok >= t_lo && tok < t_hi;
            float s = quad_sum(e < 4 ? D0[e] : D1[e - 4]);
            sc[e] = valid[e] ? s * c2 : -INFINITY;
            mx = fmaxf(mx, sc[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        float pv[8], ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            pv[e] = valid[e] ? exp2f(sc[e] - m_new) : 0.f;
            ps += pv[e];
        }
        l_run = fmaf(l_run, alpha, ps);
        u32x4_t ap;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t hw, lw;
            split_bf16(pv[2 * i], pv[2 * i + 1], hw, lw);
            ap[i] = gq == 0 ? hw : (gq == 1 ? lw : 0u);
        }
        const float alpha_d = __shfl(alpha, 4 * kb);
        if (__any(alpha_d != 1.0f)) {
#pragma unroll
            for (int s = 0; s < 8; ++s) { O[s][0] *= alpha_d; O[s][1] *= alpha_d; }
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
            uint4 v = *reinterpret_cast<const uint4*>(PM + v_off + 2 * 16 * s * kHalf);
            u32x4_t bv = {v.x, v.y, v.z, v.w};
            if (!full) bv &= vmask;
            O[s] = mfma_bf16(ap, bv, O[s]);
        }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    __shared__ float sh_l[4], sh_m[4];
    if (kb == 0 && gq == 0) { sh_l[jq] = l_run; sh_m[jq] = m_run; }
    __syncthreads();
    const float lj = sh_l[kb];
    const float inv = 1.0f / lj;
    float* dst = part_ptr(a, b, h, split, kb);
#pragma unroll
    for (int s = 0; s < 8; ++s) dst[16 * s + n16] = (O[s][0] + O[s][1]) * inv;
    if (n16 == 0) dst[g.d] = sh_m[kb] + log2f(lj);
}

// One 1-D grid over work items, split-major: all first splits of every
// (sequence, kv head), then all second splits, ..., and the protected parts
// last, where their short runs fill the tail of the grid.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) void decode_kv4_mfma_kernel(DecodeArgs a)
{
    const int nbh = a.batch * a.g.Hkv;
    const int split = blockIdx.x / nbh, bh = blockIdx.x % nbh;
    const int b = bh / a.g.Hkv, h = bh % a.g.Hkv;
    if (split < a.nsplit) mfma_item_kv4(a, b, h, split);
    else valu_item_kv4<4>(a, b, h, a.nsplit);
}

__global__ __launch_bounds__(64) void decode_bf16_mfma_kernel(DecodeArgs a)
{
    const int nbh = a.batch * a.g.Hkv;
    const int split = blockIdx.x / nbh, bh = blockIdx.x % nbh;
    mfma_item_bf16(a, bh / a.g.Hkv, bh % a.g.Hkv, split);
}

}  // namespace kv4
