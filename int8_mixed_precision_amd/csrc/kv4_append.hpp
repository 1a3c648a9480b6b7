// kv4_append.hpp -- append kernels: quantize each new token's K and V into the
// paged INT4 cache and, for protected positions, into the INT8 side ring.
//
// KV4-RL (arXiv 2610.14448): affine INT4 x^ = Delta*c + m with FP16 Delta and
// m (Section 3 eq. 3.3; Section 5.1; Appendix A.3 "Encoding and allocation");
// INT8 side entries with symmetric per-token/head scaling, computed from the
// source vector (Appendix A.3); both produced when the token is generated, so
// leaving the recent window needs no requantization (Section 5.3).
//
// Quantizer readings (the pages fix only the affine form and FP16 metadata):
//   m = fp16(min x), r = fp32(max x - m), Delta = fp16(fp32(r / 15)), Delta = 0
//   when r <= 0 or it rounds to 0; c = nearest integer in [0,15] to the exact
//   (x - m)/Delta, ties to even.  INT8: s = fp16(fp32(amax / 127)),
//   c = nearest integer to the exact x/s, ties to even, in [-127, 127].
//   Stored zeros are +0.  Exactness: the code is first estimated in binary64
//   and then checked against the exact binary64 midpoints m + (c +- 1/2)Delta
//   (exact because m and Delta are binary16 values), so the result is the
//   exact nearest code for every finite bf16 input.
#pragma once

#include "kv4_common.hpp"

namespace kv4 {

struct AppendArgs {
    Geo g;
    int layer;
    const uint16_t* k;           // [total_new][Hkv][d] bf16
    const uint16_t* v;
    const int32_t* cu_new;       // [batch+1]
    const int32_t* ctx_before;   // [batch]
    const int32_t* slot_ids;     // [batch]
    const int32_t* block_tables; // [max_slots][max_pages]
    int batch, total_new;
    uint8_t* pages;
    uint8_t* side;
};

// DPP move inside a 16-lane row (every lane active, every source in the row).
template <int CTRL>
__device__ __forceinline__ int row_mov(int x)
{
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}

// Order-preserving integer key of a binary32 value: for non-NaN a and b,
// a < b exactly when fkey(a) < fkey(b) as signed integers (-0 sorts just
// below +0).  The reductions compare keys, which needs no canonicalisation of
// the moved operands and lets each DPP move fuse into its min or max.
__device__ __forceinline__ int fkey(float x)
{
    const int i = __float_as_int(x);
    return i ^ ((i >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float fkey_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// Minimum and maximum over aligned groups of LANES (16, 32 or 64) lanes: quad
// swaps and row rotations inside each 16-lane row, then the row swaps of
// v_permlane16_swap / v_permlane32_swap.  Exact for any order.
template <int LANES>
__device__ __forceinline__ void group_minmax_keys(int& lo, int& hi)
{
    static_assert(LANES == 16 || LANES == 32 || LANES == 64, "group of 16, 32 or 64 lanes");
    lo = min(lo, row_mov<0xB1>(lo));            // quad_perm [1,0,3,2]
    hi = max(hi, row_mov<0xB1>(hi));
    lo = min(lo, row_mov<0x4E>(lo));            // quad_perm [2,3,0,1]
    hi = max(hi, row_mov<0x4E>(hi));
    lo = min(lo, row_mov<0x124>(lo));           // row_ror 4
    hi = max(hi, row_mov<0x124>(hi));
    lo = min(lo, row_mov<0x128>(lo));           // row_ror 8
    hi = max(hi, row_mov<0x128>(hi));
    if constexpr (LANES >= 32) {
        auto a = __builtin_amdgcn_permlane16_swap((unsigned)lo, (unsigned)lo, false, false);
        lo = min((int)a[0], (int)a[1]);
        auto b = __builtin_amdgcn_permlane16_swap((unsigned)hi, (unsigned)hi, false, false);
        hi = max((int)b[0], (int)b[1]);
    }
    if constexpr (LANES == 64) {
        auto a = __builtin_amdgcn_permlane32_swap((unsigned)lo, (unsigned)lo, false, false);
        lo = min((int)a[0], (int)a[1]);
        auto b = __builtin_amdgcn_permlane32_swap((unsigned)hi, (unsigned)hi, false, false);
        hi = max((int)b[0], (int)b[1]);
    }
}

// Correctly rounded binary32 quotient a / B for a constant B (15 or 127) and
// any a >= 0: q0 = a * RN(1/B), the residual a - B q0 taken exactly by an fma,
// and one correction step q0 + residual * RN(1/B), rounded once (Markstein's
// correction theorem: a correctly rounded reciprocal and a quotient within
// one ulp give the correctly rounded quotient).  Checked against the binary64
// quotient rounded to binary32 for every finite a >= 0, subnormals included,
// for B = 15 and 127; a = +inf (an offset that overflowed binary16) gives +inf.
template <int B>
__device__ __forceinline__ float div_rn_const(float a)
{
    constexpr float y = 1.0f / (float)B;
    const float q0 = __fmul_rn(a, y);
    const float e = __builtin_fmaf(-(float)B, q0, a);
    const float q = __builtin_fmaf(e, y, q0);
    return a == __builtin_inff() ? a : q;
}

// INT4 parameters of a group whose values are spread over `lanes` consecutive
// lanes (two channels per lane).  Returns Delta and m bit patterns.
template <int LANES>
__device__ __forceinline__ void int4_params(float x0, float x1, uint16_t& db, uint16_t& mb)
{
    const int k0 = fkey(x0), k1 = fkey(x1);
    int lo = min(k0, k1), hi = max(k0, k1);
    group_minmax_keys<LANES>(lo, hi);
    mb = plus_zero16(f32_to_f16_bits(fkey_value(lo)));
    float mf = half_bits_to_float(mb);
    float r = fkey_value(hi) - mf;
    db = 0;
    if (r > 0.0f) db = plus_zero16(f32_to_f16_bits(div_rn_const<15>(r)));
}

__device__ __forceinline__ uint32_t int4_code_exact(float x, double D, double M, uint16_t db)
{
    if (db == 0) return 0u;
    double xv = (double)x;
    int c = (int)fmin(fmax(rint((xv - M) / D), 0.0), 15.0);
    if (c > 0) {
        double mid = M + ((double)c - 0.5) * D;
        if (xv < mid || (xv == mid && (c & 1))) c -= 1;
    }
    if (c < 15) {
        double mid = M + ((double)c + 0.5) * D;
        if (xv > mid || (xv == mid && ((c + 1) & 1) == 0)) c += 1;
    }
    return (uint32_t)c;
}

// Binary32 fast path of the INT4 code decision, with the same results (the
// INT8 one, int8_code, is in kv4_common.hpp).  With
// x, m and Delta (or s) exact binary32 values, u = fl(x - m) * rcp(Delta) has a
// relative error below 2^-22 (one rounding in the difference, 1 ulp in
// v_rcp_f32, one in the product), i.e. below 4e-6 for |u| < 16 and below 3.1e-5
// for |u| < 128.  Away from a midpoint between two admissible codes by more than
// 2^-14 (INT4) or 2^-11 (INT8) the nearest integer to u is therefore the exact
// nearest code; near a midpoint, or for non-finite operands, the binary64 test
// above decides.
// The binary32 candidate of int4_code, without a branch: the code, and
// whether the binary64 test must decide instead.  u - rint(u) is exact, so
// |u - rint(u)| >= 1/2 - 2^-14 (or a NaN) marks u as within 2^-14 of a
// half-integer; the test does not look at which half-integer, since taking the
// binary64 decision where the binary32 one would also do is always correct.
__device__ __forceinline__ uint32_t int4_code_fast(float x, float Df, float Mf, uint16_t db, bool& exact)
{
    const float u = (x - Mf) * __builtin_amdgcn_rcpf(Df);
    const float r = rintf(u);
    const bool near = !(fabsf(u - r) < 0.5f - 0x1p-14f);
    exact = db != 0 && (near || !(fabsf(u) < 64.0f) || !(Df < 65536.0f));
    return db == 0 ? 0u : (uint32_t)fminf(fmaxf(r, 0.0f), 15.0f);
}

__device__ __forceinline__ uint32_t int4_code(float x, float Df, float Mf, uint16_t db)
{
    bool exact;
    const uint32_t c = int4_code_fast(x, Df, Mf, db, exact);
    return exact ? int4_code_exact(x, (double)Df, (double)Mf, db) : c;
}

// Full-wave (64 lanes, 128 channels) INT8 scale.
__device__ __forceinline__ uint16_t int8_scale(float x0, float x1)
{
    // the key of a value >= 0 is its bit pattern
    int a = max(__float_as_int(fabsf(x0)), __float_as_int(fabsf(x1))), unused = a;
    group_minmax_keys<64>(unused, a);
    return plus_zero16(f32_to_f16_bits(div_rn_const<127>(__int_as_float(a))));
}

// Partner value of lane ^ MASK (MASK = 1, 2 or 4: inside groups of 8 lanes),
// through ds_swizzle's bit mode (and-mask 0x1F, xor-mask MASK), which leaves
// the vector ALU free.
template <int MASK>
__device__ __forceinline__ float lane_xor(float x)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (MASK << 10) | 0x1F));
}

// Minimum and maximum of 16 values in IEEE minimum / maximum (no NaN in the
// inputs; -0 below +0), three operands per instruction.
__device__ __forceinline__ void minmax16(const float (&x)[16], float& lo, float& hi)
{
    lo = __builtin_elementwise_minimum(x[0], x[1]);
    hi = __builtin_elementwise_maximum(x[0], x[1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) {
        lo = __builtin_elementwise_minimum(__builtin_elementwise_minimum(lo, x[j]), x[j + 1]);
        hi = __builtin_elementwise_maximum(__builtin_elementwise_maximum(hi, x[j]), x[j + 1]);
    }
}

// INT4 parameters from a group's minimum and maximum (the rule of int4_params).
__device__ __forceinline__ void int4_params_from(float lo, float hi, uint16_t& db, uint16_t& mb)
{
    mb = plus_zero16(f32_to_f16_bits(lo));
    const float r = hi - half_bits_to_float(mb);
    db = r > 0.0f ? plus_zero16(f32_to_f16_bits(div_rn_const<15>(r))) : (uint16_t)0;
}

// Codes of 16 values under (Delta, m); nibble k of word w[k / 8] is value k.
// The binary32 decision of int4_code_fast with two simplifications that give
// the same codes: a zero Delta takes the reciprocal 0 (u = 0, code 0), and
// there is no test on |u| or Delta, because where |u| >= 64 (or Delta is
// infinite and m finite, u = 0) the clamped nearest integer of u is already
// the exact code.  Only the largest |u - rint(u)| of the 16 values is tested:
// when it lies within 2^-14 of 1/2 (or is a NaN) each value is tested again
// and the binary64 decision replaces the codes of those that need it.
__device__ __forceinline__ void int4_codes16(const float (&x)[16], uint16_t db, uint16_t mb, uint32_t (&w)[2])
{
    const float D = half_bits_to_float(db), M = half_bits_to_float(mb);
    const float rD = db != 0 ? __builtin_amdgcn_rcpf(D) : 0.0f;
    constexpr float kMargin = 0.5f - 0x1p-14f;
    float c[16], dev = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float u = (x[j] - M) * rD;
        c[j] = rintf(u);
        dev = __builtin_elementwise_maximum(dev, fabsf(u - c[j]));
    }
    if (!(dev < kMargin)) {                      // rare: near a midpoint
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float u = (x[j] - M) * rD;
            if (!(fabsf(u - rintf(u)) < kMargin))
                c[j] = (float)int4_code_exact(x[j], (double)D, (double)M, db);
        }
    }
    // two codes per byte, 16 c1 + c0, converted and placed by v_cvt_pk_u8_f32
    w[0] = w[1] = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float c0 = __builtin_amdgcn_fmed3f(c[2 * i], 0.0f, 15.0f);
        const float c1 = __builtin_amdgcn_fmed3f(c[2 * i + 1], 0.0f, 15.0f);
        w[i >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(c1, 16.0f, c0), i & 3, w[i >> 2]);
    }
}

// The bf16 K and V of a whole half page in the layout of append_half_page:
// lane 8t + b holds channels 16 b .. 16 b + 15 of token t (row `row` + t).
struct HalfPageIn {
    uint4 k0, k1, v0, v1;
};

__device__ __forceinline__ HalfPageIn load_half_page(const AppendArgs& a, int64_t row, int h)
{
    const int lane = threadIdx.x, t = lane >> 3, b = lane & 7;
    const int64_t src = ((row + t) * a.g.Hkv + h) * a.g.d + 16 * b;
    HalfPageIn in;
    in.k0 = *reinterpret_cast<const uint4*>(a.k + src);
    in.k1 = *reinterpret_cast<const uint4*>(a.k + src + 8);
    in.v0 = *reinterpret_cast<const uint4*>(a.v + src);
    in.v1 = *reinterpret_cast<const uint4*>(a.v + src + 8);
    return in;
}

// A whole half page of new tokens (8 positions pos0 .. pos0 + 7, pos0 a
// multiple of 8) for one kv head, one wave: lane 8 t + b holds channels
// 16 b .. 16 b + 15 of token t, so a group's range, Delta and m are formed
// from 16 values per lane (G / 16 lanes per group) and a token's K code row
// is written as whole words.  The V code words, one per channel over the 8
// tokens, take a byte transpose through LDS.  Positions protected at the new
// length also get their INT8 side entries.
template <int G>
__device__ __forceinline__ void append_half_page(const AppendArgs& a, const HalfPageIn& in, uint8_t* pb,
                                                 int pos0, int p1, uint8_t* ring)
{
    static_assert(G == 32 || G == 64 || G == 128, "group of 32, 64 or 128 channels");
    constexpr int LB = G / 16;                   // lanes per group
    __shared__ uint8_t vt[8][64];                // [b][token-pair byte j][t]
    const Geo& g = a.g;
    const int lane = threadIdx.x, t = lane >> 3, b = lane & 7;
    const uint32_t kw[8] = {in.k0.x, in.k0.y, in.k0.z, in.k0.w, in.k1.x, in.k1.y, in.k1.z, in.k1.w};
    const uint32_t vw[8] = {in.v0.x, in.v0.y, in.v0.z, in.v0.w, in.v1.x, in.v1.y, in.v1.z, in.v1.w};
    float kx[16], vx[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        kx[2 * i] = bf16_lo(kw[i]);
        kx[2 * i + 1] = bf16_hi(kw[i]);
        vx[2 * i] = bf16_lo(vw[i]);
        vx[2 * i + 1] = bf16_hi(vw[i]);
    }
    if (g.rot) {
        // channel bits 0-3 in the lane, bits 4-6 on lane bits 0-2: the
        // stages in the order of the channel bits, as everywhere else
        // (the first two lane stages through DPP quad permutes: no LDS round
        // trip in the chain of 16 dependent stages per value)
        wht_local(kx);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = __int_as_float(row_mov<0xB1>(__float_as_int(kx[j])));   // lane ^ 1
            kx[j] = (b & 1) ? p - kx[j] : kx[j] + p;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = __int_as_float(row_mov<0x4E>(__float_as_int(kx[j])));   // lane ^ 2
            kx[j] = (b & 2) ? p - kx[j] : kx[j] + p;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = lane_xor<4>(kx[j]);
            kx[j] = (b & 4) ? p - kx[j] : kx[j] + p;
        }
        wht_scale(kx);
    }
    // ---- INT4 parameters: the group's range over LB lanes
    float klo, khi, vlo, vhi;
    minmax16(kx, klo, khi);
    minmax16(vx, vlo, vhi);
    if constexpr (LB >= 2) {
        klo = __builtin_elementwise_minimum(klo, lane_xor<1>(klo));
        khi = __builtin_elementwise_maximum(khi, lane_xor<1>(khi));
        vlo = __builtin_elementwise_minimum(vlo, lane_xor<1>(vlo));
        vhi = __builtin_elementwise_maximum(vhi, lane_xor<1>(vhi));
    }
    if constexpr (LB >= 4) {
        klo = __builtin_elementwise_minimum(klo, lane_xor<2>(klo));
        khi = __builtin_elementwise_maximum(khi, lane_xor<2>(khi));
        vlo = __builtin_elementwise_minimum(vlo, lane_xor<2>(vlo));
        vhi = __builtin_elementwise_maximum(vhi, lane_xor<2>(vhi));
    }
    if constexpr (LB >= 8) {
        klo = __builtin_elementwise_minimum(klo, lane_xor<4>(klo));
        khi = __builtin_elementwise_maximum(khi, lane_xor<4>(khi));
        vlo = __builtin_elementwise_minimum(vlo, lane_xor<4>(vlo));
        vhi = __builtin_elementwise_maximum(vhi, lane_xor<4>(vhi));
    }
    uint16_t kdb, kmb, vdb, vmb;
    int4_params_from(klo, khi, kdb, kmb);
    int4_params_from(vlo, vhi, vdb, vmb);
    uint32_t kc[2], vc[2];
    int4_codes16(kx, kdb, kmb, kc);
    int4_codes16(vx, vdb, vmb, vc);

    const int tp = pos0 % kPage + t, grp = b / LB;
    // K codes: words 2b and 2b + 1 of the token's row
    uint32_t* krow = reinterpret_cast<uint32_t*>(pb + g.off_kc + tp * (g.d / 2));
    krow[kpos(2 * b)] = kc[0];
    krow[kpos(2 * b + 1)] = kc[1];
    if (b % LB == 0) {
        reinterpret_cast<uint32_t*>(pb + g.off_kdm)[tp * g.ng + grp] = (uint32_t)kdb | ((uint32_t)kmb << 16);
        reinterpret_cast<uint16_t*>(pb + g.off_vd)[grp * kPage + tp] = vdb;
        reinterpret_cast<uint16_t*>(pb + g.off_vm)[tp * g.ng + grp] = vmb;
    }
    // V codes: byte j of lane (t, b) holds channels 16 b + 2 j, + 1 of token
    // t; after the transpose lane (t, b) holds byte t of every token, i.e.
    // channels 16 b + 2 t and 16 b + 2 t + 1 for tokens 0..7, and unzips the
    // nibbles into the two channels' code words.
#pragma unroll
    for (int j = 0; j < 8; ++j) vt[b][8 * j + t] = (uint8_t)(vc[j >> 2] >> (8 * (j & 3)));
    __syncthreads();
    const uint2 col = *reinterpret_cast<const uint2*>(&vt[b][8 * t]);
    __syncthreads();                             // vt is free for the next half page
    // byte t' = lo | hi << 4 (lo: channel 2t, hi: channel 2t + 1, token t')
    const uint32_t x0 = col.x, x1 = col.y;
    const uint32_t sel = 0x000F000Fu;
    const uint32_t l0 = (x0 & sel) | ((x0 >> 4) & ~sel), l1 = (x1 & sel) | ((x1 >> 4) & ~sel);
    const uint32_t h0 = ((x0 >> 4) & sel) | ((x0 >> 8) & ~sel), h1 = ((x1 >> 4) & sel) | ((x1 >> 8) & ~sel);
    // bytes 0 and 2 of each hold two tokens' nibbles
    const uint32_t lo_word = __builtin_amdgcn_perm(l1, l0, 0x06040200u);
    const uint32_t hi_word = __builtin_amdgcn_perm(h1, h0, 0x06040200u);
    uint32_t* vwords = reinterpret_cast<uint32_t*>(pb + g.off_vc) + ((pos0 / kHalf) & 1) * g.d;
    vwords[vpos(16 * b + 2 * t)] = lo_word;
    vwords[vpos(16 * b + 2 * t + 1)] = hi_word;

    // ---- INT8 side entries of protected positions
    if (ring != nullptr && (pos0 < g.S || pos0 + kHalf > p1 - g.R)) {
        const int pos = pos0 + t;
        float ka = 0.0f, va = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            ka = __builtin_elementwise_maximum(ka, fabsf(kx[j]));
            va = __builtin_elementwise_maximum(va, fabsf(vx[j]));
        }
        ka = __builtin_elementwise_maximum(ka, lane_xor<1>(ka));
        va = __builtin_elementwise_maximum(va, lane_xor<1>(va));
        ka = __builtin_elementwise_maximum(ka, lane_xor<2>(ka));
        va = __builtin_elementwise_maximum(va, lane_xor<2>(va));
        ka = __builtin_elementwise_maximum(ka, lane_xor<4>(ka));
        va = __builtin_elementwise_maximum(va, lane_xor<4>(va));
        if (pos < g.S || pos >= p1 - g.R) {
            const int e = pos < g.S ? pos : g.S + (pos - g.S) % g.R;
            const uint16_t sk = plus_zero16(f32_to_f16_bits(div_rn_const<127>(ka)));
            const uint16_t sv = plus_zero16(f32_to_f16_bits(div_rn_const<127>(va)));
            const float Sk = half_bits_to_float(sk), Sv = half_bits_to_float(sv);
            uint32_t kb[4] = {0u, 0u, 0u, 0u};
            uint8_t* vr = ring + (int64_t)g.SR32 * g.d;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                kb[j >> 2] |= (uint32_t)(int8_code(kx[j], Sk, sk) & 0xFF) << (8 * (j & 3));
                vr[ring_vbyte(e, 16 * b + j)] = (uint8_t)int8_code(vx[j], Sv, sv);
            }
            *reinterpret_cast<uint4*>(ring + (int64_t)e * g.d + 16 * b) = make_uint4(kb[0], kb[1], kb[2], kb[3]);
            if (b == 0) {
                uint16_t* sc = reinterpret_cast<uint16_t*>(ring + (int64_t)2 * g.SR32 * g.d);
                sc[e] = sk;
                sc[g.SR32 + e] = sv;
            }
        }
    }
}

// Grid (x, Hkv, batch): the whole half pages of a sequence's new tokens are
// strided over x (append_half_page); an unaligned first half page goes to
// wave x = 0 and an unaligned last one to the last wave, which quantize its
// tokens one at a time with lane l holding channels 2l, 2l + 1.  Each half
// page belongs to one wave, which owns its V code words, so the
// read-modify-write of a partial half page's nibbles is race-free.
template <int G>
__global__ __launch_bounds__(64) void append_kv4_kernel(AppendArgs a)
{
    const Geo& g = a.g;
    const int b = blockIdx.z, h = blockIdx.y, lane = threadIdx.x;
    int row0 = clampi(a.cu_new[b], 0, a.total_new);
    int row1 = clampi(a.cu_new[b + 1], row0, a.total_new);
    const int cap = g.max_pages * kPage;
    int p0 = clampi(a.ctx_before[b], 0, cap);
    int p1 = min(p0 + (row1 - row0), cap);
    if (p1 <= p0) return;
    int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    // page ids through the scalar cache (the block table is read-only during
    // the kernel), so that waiting for one never waits for the vector loads
    // issued after it
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    const const_i32 bt = (const_i32)(a.block_tables + (int64_t)slot * g.max_pages);
    constexpr int LPG = G / 2;                 // lanes per group
    const int grp = (2 * lane) / G;

    uint8_t* ring = g.SR > 0 ? a.side + (int64_t)a.layer * g.layer_side +
                                   ((int64_t)slot * g.Hkv + h) * g.rb
                             : nullptr;

    // whole half pages [f0, f1), strided over blockIdx.x; the next one's
    // loads (and block-table entry) are in flight while this one is
    // quantized.  The loads are unconditional (past the last half page the
    // current one is read again, from the cache), so the wait for this half
    // page's data never waits for the next one's.
    const int f0 = (p0 + kHalf - 1) / kHalf, f1 = p1 / kHalf;
    int hp = f0 + (int)blockIdx.x;
    if (hp < f1) {
        HalfPageIn cur = load_half_page(a, (int64_t)row0 + (hp * kHalf - p0), h);
        int page = bt[hp / 2];
        for (;;) {
            const int hn = hp + (int)gridDim.x;
            const bool more = hn < f1;
            const int hl = more ? hn : hp;
            const HalfPageIn nxt = load_half_page(a, (int64_t)row0 + (hl * kHalf - p0), h);
            const int page_n = bt[hl / 2];
            uint8_t* pb = a.pages + (int64_t)a.layer * g.layer_pages +
                          ((int64_t)clampi(page, 0, g.num_pages - 1) * g.Hkv + h) * g.pb;
            append_half_page<G>(a, cur, pb, hp * kHalf, p1, ring);
            if (!more) break;
            cur = nxt;
            page = page_n;
            hp = hn;
        }
    }
    // the partial half pages: an unaligned start (wave 0) and end (the last wave)
    const int head = (p0 % kHalf) ? p0 / kHalf : -1;
    const int tail = (p1 % kHalf && p1 / kHalf != head) ? p1 / kHalf : -1;
    for (int k = 0; k < 2; ++k) {
        const int hpp = k == 0 ? (blockIdx.x == 0 ? head : -1) : (blockIdx.x == gridDim.x - 1 ? tail : -1);
        if (hpp < 0) continue;
        const int t_lo = max(hpp * kHalf, p0), t_hi = min(hpp * kHalf + kHalf, p1);
        const int pg = clampi(bt[hpp / 2], 0, g.num_pages - 1);
        uint8_t* pb = a.pages + (int64_t)a.layer * g.layer_pages + ((int64_t)pg * g.Hkv + h) * g.pb;
        uint32_t* vw = reinterpret_cast<uint32_t*>(pb + g.off_vc) + (hpp & 1) * g.d;
        const int q0 = vpos(2 * lane), q1 = vpos(2 * lane + 1);
        uint32_t kkr[kHalf], vvr[kHalf];
        uint32_t w0 = vw[q0], w1 = vw[q1];
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
            if (t_lo + i < t_hi) {
                const int64_t src = ((int64_t)(row0 + (t_lo + i - p0)) * g.Hkv + h) * g.d;
                kkr[i] = *reinterpret_cast<const uint32_t*>(a.k + src + 2 * lane);
                vvr[i] = *reinterpret_cast<const uint32_t*>(a.v + src + 2 * lane);
            }
        }
#pragma unroll
        for (int i = 0; i < kHalf; ++i) {
            const int t = t_lo + i;
            if (t >= t_hi) break;
            const uint32_t kk = kkr[i], vv = vvr[i];
            float k0 = bf16_lo(kk), k1 = bf16_hi(kk), v0 = bf16_lo(vv), v1 = bf16_hi(vv);
            if (g.rot) {
                // keys in the rotated basis; lane l holds channels 2l, 2l + 1
                float kr[2] = {k0, k1};
                wht_local(kr);
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) wht_lanes(kr, m);
                wht_scale(kr);
                k0 = kr[0];
                k1 = kr[1];
            }
            int tp = t % kPage;
            // ---- INT4, keys
            uint16_t db, mb;
            int4_params<LPG>(k0, k1, db, mb);
            float D = half_bits_to_float(db), M = half_bits_to_float(mb);
            uint32_t c0 = int4_code(k0, D, M, db), c1 = int4_code(k1, D, M, db);
            pb[g.off_kc + tp * (g.d / 2) + 4 * kpos(lane >> 2) + (lane & 3)] = (uint8_t)(c0 | (c1 << 4));
            if ((lane % LPG) == 0) {
                uint16_t* kdm = reinterpret_cast<uint16_t*>(pb + g.off_kdm) + tp * 2 * g.ng + 2 * grp;
                kdm[0] = db;
                kdm[1] = mb;
            }
            // ---- INT4, values
            int4_params<LPG>(v0, v1, db, mb);
            D = half_bits_to_float(db);
            M = half_bits_to_float(mb);
            c0 = int4_code(v0, D, M, db);
            c1 = int4_code(v1, D, M, db);
            int sh = 4 * (t % kHalf);
            w0 = (w0 & ~(0xFu << sh)) | (c0 << sh);
            w1 = (w1 & ~(0xFu << sh)) | (c1 << sh);
            if ((lane % LPG) == 0) {
                reinterpret_cast<uint16_t*>(pb + g.off_vd)[grp * kPage + tp] = db;
                reinterpret_cast<uint16_t*>(pb + g.off_vm)[tp * g.ng + grp] = mb;
            }
            // ---- INT8 side entry for positions protected at the new length
            if (ring != nullptr && (t < g.S || t >= p1 - g.R)) {
                int e = t < g.S ? t : g.S + (t - g.S) % g.R;
                uint16_t sk = int8_scale(k0, k1), sv = int8_scale(v0, v1);
                const float Sk = half_bits_to_float(sk), Sv = half_bits_to_float(sv);
                int a0 = int8_code(k0, Sk, sk), a1 = int8_code(k1, Sk, sk);
                int b0 = int8_code(v0, Sv, sv), b1 = int8_code(v1, Sv, sv);
                reinterpret_cast<uint16_t*>(ring + (int64_t)e * g.d)[lane] =
                    (uint16_t)((a0 & 0xFF) | ((a1 & 0xFF) << 8));
                uint8_t* vr = ring + (int64_t)g.SR32 * g.d;
                vr[ring_vbyte(e, 2 * lane)] = (uint8_t)b0;
                vr[ring_vbyte(e, 2 * lane + 1)] = (uint8_t)b1;
                if (lane == 0) {
                    uint16_t* sc = reinterpret_cast<uint16_t*>(ring + (int64_t)2 * g.SR32 * g.d);
                    sc[e] = sk;
                    sc[g.SR32 + e] = sv;
                }
            }
        }
        vw[q0] = w0;
        vw[q1] = w1;
    }
}

// KV8 kind: INT8 codes and binary16 scales of every new token's K and V (the
// side entries' encoding, KV4-RL Appendix A.3) into its page.  Grid (x, Hkv,
// batch), tokens strided over x; lane l holds channels 2l and 2l + 1.  Every
// byte written belongs to one token, so tokens never race.
__global__ __launch_bounds__(64) void append_kv8_kernel(AppendArgs a)
{
    const Geo& g = a.g;
    const int b = blockIdx.z, h = blockIdx.y, lane = threadIdx.x;
    int row0 = clampi(a.cu_new[b], 0, a.total_new);
    int row1 = clampi(a.cu_new[b + 1], row0, a.total_new);
    const int cap = g.max_pages * kPage;
    int p0 = clampi(a.ctx_before[b], 0, cap);
    int p1 = min(p0 + (row1 - row0), cap);
    int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    for (int t = p0 + blockIdx.x; t < p1; t += gridDim.x) {
        int page = clampi(bt[t / kPage], 0, g.num_pages - 1);
        uint8_t* pb = a.pages + (int64_t)a.layer * g.layer_pages + ((int64_t)page * g.Hkv + h) * g.pb;
        int64_t src = ((int64_t)(row0 + (t - p0)) * g.Hkv + h) * g.d;
        const int tp = t % kPage;
        uint32_t kk = *reinterpret_cast<const uint32_t*>(a.k + src + 2 * lane);
        uint32_t vv = *reinterpret_cast<const uint32_t*>(a.v + src + 2 * lane);
        const float k0 = bf16_lo(kk), k1 = bf16_hi(kk), v0 = bf16_lo(vv), v1 = bf16_hi(vv);
        const uint16_t sk = int8_scale(k0, k1), sv = int8_scale(v0, v1);
        const float Sk = half_bits_to_float(sk), Sv = half_bits_to_float(sv);
        const int a0 = int8_code(k0, Sk, sk), a1 = int8_code(k1, Sk, sk);
        const int b0 = int8_code(v0, Sv, sv), b1 = int8_code(v1, Sv, sv);
        reinterpret_cast<uint16_t*>(pb + g.off_kc + (int64_t)tp * g.d)[lane] =
            (uint16_t)((a0 & 0xFF) | ((a1 & 0xFF) << 8));
        uint8_t* vr = pb + g.off_vc;
        vr[ring_vbyte(tp, 2 * lane)] = (uint8_t)b0;
        vr[ring_vbyte(tp, 2 * lane + 1)] = (uint8_t)b1;
        if (lane == 0) {
            reinterpret_cast<uint16_t*>(pb + g.off_kdm)[tp] = sk;
            reinterpret_cast<uint16_t*>(pb + g.off_vm)[tp] = sv;
        }
    }
}

// BF16 comparator: copy the new tokens into bf16 pages.  Grid (x, Hkv, batch),
// tokens strided over x.
__global__ __launch_bounds__(64) void append_bf16_kernel(AppendArgs a)
{
    const Geo& g = a.g;
    const int b = blockIdx.z, h = blockIdx.y, lane = threadIdx.x;
    int row0 = clampi(a.cu_new[b], 0, a.total_new);
    int row1 = clampi(a.cu_new[b + 1], row0, a.total_new);
    const int cap = g.max_pages * kPage;
    int p0 = clampi(a.ctx_before[b], 0, cap);
    int p1 = min(p0 + (row1 - row0), cap);
    int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    for (int t = p0 + blockIdx.x; t < p1; t += gridDim.x) {
        int page = clampi(bt[t / kPage], 0, g.num_pages - 1);
        uint8_t* pb = a.pages + (int64_t)a.layer * g.layer_pages + ((int64_t)page * g.Hkv + h) * g.pb;
        int64_t src = ((int64_t)(row0 + (t - p0)) * g.Hkv + h) * g.d;
        int tp = t % kPage;
        uint32_t kk = *reinterpret_cast<const uint32_t*>(a.k + src + 2 * lane);
        uint32_t vv = *reinterpret_cast<const uint32_t*>(a.v + src + 2 * lane);
        reinterpret_cast<uint32_t*>(pb)[tp * (g.d / 2) + lane] = kk;
        // V element (t, c) at [(t%16)/8][c][t%8]: 8 tokens of a channel are contiguous
        uint16_t* vb = reinterpret_cast<uint16_t*>(pb + (int64_t)kPage * g.d * 2) + (tp / kHalf) * g.d * kHalf;
        vb[(2 * lane) * kHalf + tp % kHalf] = (uint16_t)(vv & 0xFFFFu);
        vb[(2 * lane + 1) * kHalf + tp % kHalf] = (uint16_t)(vv >> 16);
    }
}

}  // namespace kv4
