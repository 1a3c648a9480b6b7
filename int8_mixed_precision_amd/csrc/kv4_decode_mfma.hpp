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

    f32x4_t O[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) O[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    f32x4_t Wsum = {0.f, 0.f, 0.f, 0.f};
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0
    float m_run = -INFINITY, l_run = 0.f, accm = 0.f;

    // fixed per-lane offsets inside a 32-token tile
    const int rq = n16 >> 2, rr = n16 & 3;       // QK row n16 -> tokens 8 rq + rr (+4)
    const int kc_off0 = g.off_kc + (8 * (rq & 1) + rr) * (g.d / 2) + 16 * kb;
    const int kc_off1 = kc_off0 + 4 * (g.d / 2);
    const int meta_off = 2 * (mg * kPage + 8 * (kb & 1));
    const int vc_off = g.off_vc + 4 * ((kb & 1) * g.d + 4 * n16);

    for (int ts = (t_lo / 32) * 32; ts < t_hi; ts += 32) {
        const int pi = ts / kPage;
        const int p0 = clampi(bt[min(pi, g.max_pages - 1)], 0, g.num_pages - 1);
        const int p1 = clampi(bt[min(pi + 1, g.max_pages - 1)], 0, g.num_pages - 1);
        const uint8_t* P0 = hbase + p0 * page_stride;
        const uint8_t* P1 = hbase + p1 * page_stride;
        const uint8_t* PK = (rq >> 1) ? P1 : P0;     // page of this lane's QK rows
        const uint8_t* PM = (kb >> 1) ? P1 : P0;     // page of this lane's k-block tokens
        const uint4 kc0 = *reinterpret_cast<const uint4*>(PK + kc_off0);
        const uint4 kc1 = *reinterpret_cast<const uint4*>(PK + kc_off1);
        const uint4 kd = *reinterpret_cast<const uint4*>(PM + g.off_kd + meta_off);
        const uint4 km = *reinterpret_cast<const uint4*>(PM + g.off_km + meta_off);
        const uint4 vc0 = *reinterpret_cast<const uint4*>(PM + vc_off);
        const uint4 vc1 = *reinterpret_cast<const uint4*>(PM + vc_off + 4 * 64);
        const uint4 vd = *reinterpret_cast<const uint4*>(PM + g.off_vd + meta_off);
        const uint4 vm = *reinterpret_cast<const uint4*>(PM + g.off_vm + meta_off);

        // ---- QK: tokens 8 kb + r (D0) and 8 kb + 4 + r (D1) of column (jq, gq)
        f32x4_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
        D0 = mfma_bf16(widen_codes(kc0.x), bq[0], D0);
        D0 = mfma_bf16(widen_codes(kc0.y), bq[1], D0);
        D0 = mfma_bf16(widen_codes(kc0.z), bq[2], D0);
        D0 = mfma_bf16(widen_codes(kc0.w), bq[3], D0);
        D1 = mfma_bf16(widen_codes(kc1.x), bq[0], D1);
        D1 = mfma_bf16(widen_codes(kc1.y), bq[1], D1);
        D1 = mfma_bf16(widen_codes(kc1.z), bq[2], D1);
        D1 = mfma_bf16(widen_codes(kc1.w), bq[3], D1);
        const uint32_t kdw[4] = {kd.x, kd.y, kd.z, kd.w}, kmw[4] = {km.x, km.y, km.z, km.w};
        float sc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = e < 4 ? D0[e] : D1[e - 4];
            float del = half_of(kdw[e >> 1], e & 1), off = half_of(kmw[e >> 1], e & 1);
            sc[e] = quad_sum(fmaf(del, acc - sq16, off * sq));
        }
        // ---- online softmax for head jq over this tile (base 2)
        float mx = -INFINITY;
        bool valid[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int tok = ts + 8 * kb + e;
            valid[e] = tok >= t_lo && tok < t_hi;
            sc[e] = valid[e] ? sc[e] * c2 : -INFINITY;
            mx = fmaxf(mx, sc[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);     // finite: every tile holds a valid token
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        // ---- PV A operand: w = p * Delta_V (exactly 0 off the item), split hi + lo
        const uint32_t vdw[4] = {vd.x, vd.y, vd.z, vd.w}, vmw[4] = {vm.x, vm.y, vm.z, vm.w};
        float wv[8], ps = 0.f, am = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float p = exp2f(sc[e] - m_new);
            ps += p;
            float del = half_of(vdw[e >> 1], e & 1), off = half_of(vmw[e >> 1], e & 1);
            wv[e] = valid[e] ? p * del : 0.f;
            am += valid[e] ? p * off : 0.f;
        }
        l_run = fmaf(l_run, alpha, ps);
        accm = fmaf(accm, alpha, am);
        u32x4_t ahi, alo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t hw, lw;
            split_bf16(wv[i], wv[i + 4], hw, lw);
            ahi[i] = hw;
            alo[i] = lw;
        }
        // ---- rescale accumulators of head kb (the D rows this lane holds)
        const float alpha_d = __shfl(alpha, 4 * kb);
        if (__any(alpha_d != 1.0f)) {
#pragma unroll
            for (int s = 0; s < 8; ++s) O[s][s >> 1] *= alpha_d;
            Wsum *= alpha_d;
        }
        // ---- PV: column block s = channels 32 (s/2) + 16 (s%2) + n16
        const uint32_t vcw[8] = {vc0.x, vc0.y, vc0.z, vc0.w, vc1.x, vc1.y, vc1.z, vc1.w};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            u32x4_t bv = widen_codes(vcw[s]);
            O[s] = mfma_bf16(ahi, bv, O[s]);
            O[s] = mfma_bf16(alo, bv, O[s]);
        }
        // sum over tokens of the A operand actually used, per (head kb, block r)
        Wsum = mfma_bf16(ahi, ones, Wsum);
        Wsum = mfma_bf16(alo, ones, Wsum);
    }

    // ---- reduce the per-k-block partial sums and hand them to the output lanes
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    accm += __shfl_xor(accm, 16);
    accm += __shfl_xor(accm, 32);
    __shared__ float sh_c[16], sh_l[4], sh_m[4];
    if (kb == 0) {
        sh_c[n16] = accm;
        if (gq == 0) { sh_l[jq] = l_run; sh_m[jq] = m_run; }
    }
    __syncthreads();
    const float lj = sh_l[kb];
    const float inv = 1.0f / lj;
    float* dst = part_ptr(a, b, h, split, kb);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int c = 32 * (s >> 1) + 16 * (s & 1) + n16;
        dst[c] = (O[s][s >> 1] - 16.0f * Wsum[s >> 1] + sh_c[4 * kb + (s >> 1)]) * inv;
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
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint4 v = *reinterpret_cast<const uint4*>(PM + v_off + 2 * 16 * s * kHalf);
            O[s] = mfma_bf16(ap, u32x4_t{v.x, v.y, v.z, v.w}, O[s]);
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
__global__ __launch_bounds__(64) void decode_kv4_mfma_kernel(DecodeArgs a)
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
