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
__device__ __forceinline__ float row_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Minimum and maximum over aligned groups of LANES (16, 32 or 64) lanes: quad
// swaps and row rotations inside each 16-lane row, then the row swaps of
// v_permlane16_swap / v_permlane32_swap.  Exact for any order.
template <int LANES>
__device__ __forceinline__ void group_minmax(float& lo, float& hi)
{
    static_assert(LANES == 16 || LANES == 32 || LANES == 64, "group of 16, 32 or 64 lanes");
    lo = fminf(lo, row_mov<0xB1>(lo));          // quad_perm [1,0,3,2]
    hi = fmaxf(hi, row_mov<0xB1>(hi));
    lo = fminf(lo, row_mov<0x4E>(lo));          // quad_perm [2,3,0,1]
    hi = fmaxf(hi, row_mov<0x4E>(hi));
    lo = fminf(lo, row_mov<0x124>(lo));         // row_ror 4
    hi = fmaxf(hi, row_mov<0x124>(hi));
    lo = fminf(lo, row_mov<0x128>(lo));         // row_ror 8
    hi = fmaxf(hi, row_mov<0x128>(hi));
    if constexpr (LANES >= 32) {
        auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(lo), false, false);
        lo = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
        auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(hi), __float_as_uint(hi), false, false);
        hi = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    }
    if constexpr (LANES == 64) {
        auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(lo), false, false);
        lo = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
        auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(hi), __float_as_uint(hi), false, false);
        hi = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
    }
}

// INT4 parameters of a group whose values are spread over `lanes` consecutive
// lanes (two channels per lane).  Returns Delta and m bit patterns.
template <int LANES>
__device__ __forceinline__ void int4_params(float x0, float x1, uint16_t& db, uint16_t& mb)
{
    float lo = fminf(x0, x1), hi = fmaxf(x0, x1);
    group_minmax<LANES>(lo, hi);
    mb = plus_zero16(f32_to_f16_bits(lo));
    float mf = half_bits_to_float(mb);
    float r = hi - mf;
    db = 0;
    if (r > 0.0f) db = plus_zero16(f32_to_f16_bits(__fdiv_rn(r, 15.0f)));
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
// whether the binary64 test must decide instead.
__device__ __forceinline__ uint32_t int4_code_fast(float x, float Df, float Mf, uint16_t db, bool& exact)
{
    const float u = (x - Mf) * __builtin_amdgcn_rcpf(Df);
    const float fl = floorf(u);
    const bool near = fabsf(u - fl - 0.5f) < 0x1p-14f && fl >= 0.0f && fl <= 14.0f;
    exact = db != 0 && (near || !(fabsf(u) < 64.0f) || !(Df < 65536.0f));
    return db == 0 ? 0u : (uint32_t)fminf(fmaxf(rintf(u), 0.0f), 15.0f);
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
    float a = fmaxf(fabsf(x0), fabsf(x1)), unused = a;
    group_minmax<64>(unused, a);
    return plus_zero16(f32_to_f16_bits(__fdiv_rn(a, 127.0f)));
}

// Tokens of a whole half page quantized side by side.  One at a time measured
// fastest: at the bulk populate of 145,101 tokens, groups of 2, 4 and 8
// overlap their dependency chains but hold more registers, and the fewer waves
// per SIMD cost more (413 us for 1, 455 us for 2, 862 us for 8).
constexpr int kAppendGroup = 1;

// One wave per (sequence, kv head, 8-token half page) of new tokens; the wave
// owns the half page's V code words, so read-modify-write of nibbles is
// race-free.  Grid: (x, Hkv, batch); half pages are strided over x.
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
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    constexpr int LPG = G / 2;                 // lanes per group
    const int grp = (2 * lane) / G;

    uint8_t* ring = g.SR > 0 ? a.side + (int64_t)a.layer * g.layer_side +
                                   ((int64_t)slot * g.Hkv + h) * g.rb
                             : nullptr;

    for (int hp = p0 / kHalf + blockIdx.x; hp <= (p1 - 1) / kHalf; hp += gridDim.x) {
        int t_lo = max(hp * kHalf, p0), t_hi = min(hp * kHalf + kHalf, p1);
        int page = clampi(bt[hp / 2], 0, g.num_pages - 1);
        uint8_t* pb = a.pages + (int64_t)a.layer * g.layer_pages + ((int64_t)page * g.Hkv + h) * g.pb;
        uint32_t* vw = reinterpret_cast<uint32_t*>(pb + g.off_vc) + (hp & 1) * g.d;
        const int q0 = vpos(2 * lane), q1 = vpos(2 * lane + 1);
        // every token of the half page is loaded before the first is quantized
        // (one load latency per half page in a bulk append)
        uint32_t kkr[kHalf], vvr[kHalf];
        if (t_hi - t_lo == kHalf && !(ring != nullptr && (t_lo < g.S || t_hi > p1 - g.R))) {
            // A whole half page with no INT8 side entry (the bulk of a
            // populate): no test per token, the binary64 decision only for
            // the lanes that need it (after the binary32 codes of a group of
            // kAppendGroup tokens), and the V code words written whole, with
            // no read: the half page owns every nibble of them.
#pragma unroll
            for (int i = 0; i < kHalf; ++i) {
                const int64_t src = ((int64_t)(row0 + (t_lo + i - p0)) * g.Hkv + h) * g.d;
                kkr[i] = *reinterpret_cast<const uint32_t*>(a.k + src + 2 * lane);
                vvr[i] = *reinterpret_cast<const uint32_t*>(a.v + src + 2 * lane);
            }
            uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
            for (int i0 = 0; i0 < kHalf; i0 += kAppendGroup) {
                float kx[kAppendGroup][2], vx[kAppendGroup][2];
#pragma unroll
                for (int j = 0; j < kAppendGroup; ++j) {
                    kx[j][0] = bf16_lo(kkr[i0 + j]);
                    kx[j][1] = bf16_hi(kkr[i0 + j]);
                    vx[j][0] = bf16_lo(vvr[i0 + j]);
                    vx[j][1] = bf16_hi(vvr[i0 + j]);
                    if (g.rot) {
                        wht_local(kx[j]);
#pragma unroll
                        for (int m = 1; m < 64; m <<= 1) wht_lanes(kx[j], m);
                        wht_scale(kx[j]);
                    }
                }
                uint16_t kdb[kAppendGroup], kmb[kAppendGroup], vdb[kAppendGroup], vmb[kAppendGroup];
#pragma unroll
                for (int j = 0; j < kAppendGroup; ++j) {
                    int4_params<LPG>(kx[j][0], kx[j][1], kdb[j], kmb[j]);
                    int4_params<LPG>(vx[j][0], vx[j][1], vdb[j], vmb[j]);
                }
                uint32_t kc[kAppendGroup][2], vc[kAppendGroup][2];
                bool any_exact = false;
#pragma unroll
                for (int j = 0; j < kAppendGroup; ++j) {
                    const float KD = half_bits_to_float(kdb[j]), KM = half_bits_to_float(kmb[j]);
                    const float VD = half_bits_to_float(vdb[j]), VM = half_bits_to_float(vmb[j]);
                    bool e0, e1, e2, e3;
                    kc[j][0] = int4_code_fast(kx[j][0], KD, KM, kdb[j], e0);
                    kc[j][1] = int4_code_fast(kx[j][1], KD, KM, kdb[j], e1);
                    vc[j][0] = int4_code_fast(vx[j][0], VD, VM, vdb[j], e2);
                    vc[j][1] = int4_code_fast(vx[j][1], VD, VM, vdb[j], e3);
                    any_exact |= e0 | e1 | e2 | e3;
                }
                if (__builtin_amdgcn_ballot_w64(any_exact)) {        // rare: near a midpoint
#pragma unroll
                    for (int j = 0; j < kAppendGroup; ++j) {
                        const float KD = half_bits_to_float(kdb[j]), KM = half_bits_to_float(kmb[j]);
                        const float VD = half_bits_to_float(vdb[j]), VM = half_bits_to_float(vmb[j]);
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            bool ek, ev;
                            (void)int4_code_fast(kx[j][e], KD, KM, kdb[j], ek);
                            (void)int4_code_fast(vx[j][e], VD, VM, vdb[j], ev);
                            if (ek) kc[j][e] = int4_code_exact(kx[j][e], (double)KD, (double)KM, kdb[j]);
                            if (ev) vc[j][e] = int4_code_exact(vx[j][e], (double)VD, (double)VM, vdb[j]);
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < kAppendGroup; ++j) {
                    const int i = i0 + j, tp = (t_lo + i) % kPage;
                    pb[g.off_kc + tp * (g.d / 2) + 4 * kpos(lane >> 2) + (lane & 3)] =
                        (uint8_t)(kc[j][0] | (kc[j][1] << 4));
                    w0 |= vc[j][0] << (4 * i);
                    w1 |= vc[j][1] << (4 * i);
                    if ((lane % LPG) == 0) {
                        uint16_t* kdm = reinterpret_cast<uint16_t*>(pb + g.off_kdm) + tp * 2 * g.ng + 2 * grp;
                        kdm[0] = kdb[j];
                        kdm[1] = kmb[j];
                        reinterpret_cast<uint16_t*>(pb + g.off_vd)[grp * kPage + tp] = vdb[j];
                        reinterpret_cast<uint16_t*>(pb + g.off_vm)[tp * g.ng + grp] = vmb[j];
                    }
                }
            }
            vw[q0] = w0;
            vw[q1] = w1;
            continue;
        }
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
