// kv4_prefill.hpp -- prefill attention: causal softmax attention of every
// packed prompt position over its sequence's prefix, on the bf16 q, k, v the
// model computes (KV4-RL Appendix A.3, "Protected path and reconstruction":
// prefill and carried-prefix reconstruction run BF16 attention over the newly
// computed K/V, whose INT4 and INT8 copies kv4_append then writes).
#pragma once

#include "kv4_decode_mfma.hpp"

namespace kv4 {

struct PrefillArgs {
    const uint16_t* q;           // [total][Hq][d] bf16
    const uint16_t* k;           // [total][Hkv][d] bf16
    const uint16_t* v;
    const int32_t* cu;           // [batch + 1] row offsets
    void* out;                   // [total][Hq][d]
    int out_bf16;
    int batch, total, max_len, Hq, Hkv, gqa;
    float scale2;                // sm_scale * log2(e)
};

// One wave per (16-query tile, q head, sequence).  Lane roles (n16 = lane % 16,
// kb = lane / 16), 32-key tiles:
//   QK: bf16 MFMA 16x16x32, A = q rows (query n16 of the tile), B = k columns
//     (key 16 c + n16 of the key tile), k-slots = channels 32 bb + 8 kb + [0, 8)
//     for bb = 0..3.  Lane l then holds the scores of queries 4 kb + r against
//     key 16 c + n16 in S_c[r].
//   PV: bf16 MFMA 16x16x32 per 16 channels, A = p (query n16, keys 8 kb + e) in
//     bf16 hi + lo, B = V^T (channel 16 m + n16, keys 8 kb + e) read from an
//     LDS copy of the tile transposed on its way in.  Lane l holds queries
//     4 kb + r, channel 16 m + n16 in O[m][r]: the rows of the scores, so the
//     online-softmax rescale applies in-lane.
__global__ __launch_bounds__(64) void prefill_attn_kernel(PrefillArgs a)
{
    const int lane = threadIdx.x;
    const int n16 = lane & 15, kb = lane >> 4;
    const int b = blockIdx.z, j = blockIdx.y, qt = blockIdx.x;
    const int t0 = clampi(a.cu[b], 0, a.total);
    const int L = min(clampi(a.cu[b + 1], t0, a.total) - t0, a.max_len);
    if (16 * qt >= L) return;
    const int h = j / a.gqa;
    constexpr int d = kHeadDim;

    // ---- q rows of the tile (rows past the end read the last row: discarded)
    u32x4_t aq[4];
    {
        const int qi = min(16 * qt + n16, L - 1);
        const uint16_t* qr = a.q + ((int64_t)(t0 + qi) * a.Hq + j) * d;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const uint4 u = *reinterpret_cast<const uint4*>(qr + 32 * bb + 8 * kb);
            aq[bb] = u32x4_t{u.x, u.y, u.z, u.w};
        }
    }

    f32x4_t O[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) O[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_r[4], l_r[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_r[r] = -INFINITY;
        l_r[r] = 0.f;
    }
    __shared__ __attribute__((aligned(16))) float P[16][32];
    __shared__ __attribute__((aligned(16))) uint16_t VT[d][32];

    const int q_last = min(16 * qt + 15, L - 1);          // last valid query of the tile
    const int kt_end = q_last / 32 + 1;
    for (int kt = 0; kt < kt_end; ++kt) {
        // ---- loads: keys and values 16 c + n16 of the tile, channels 32 bb + 8 kb + [0, 8)
        uint4 kc[2][4], vc[2][4];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int ki = min(32 * kt + 16 * c + n16, L - 1);
            const int64_t row = ((int64_t)(t0 + ki) * a.Hkv + h) * d;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                kc[c][bb] = *reinterpret_cast<const uint4*>(a.k + row + 32 * bb + 8 * kb);
                vc[c][bb] = *reinterpret_cast<const uint4*>(a.v + row + 32 * bb + 8 * kb);
            }
        }
        // V transposed into LDS: VT[channel][key]
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint32_t w[4] = {vc[c][bb].x, vc[c][bb].y, vc[c][bb].z, vc[c][bb].w};
                const int ch = 32 * bb + 8 * kb, key = 16 * c + n16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    VT[ch + 2 * e][key] = (uint16_t)(w[e] & 0xFFFFu);
                    VT[ch + 2 * e + 1][key] = (uint16_t)(w[e] >> 16);
                }
            }

        // ---- scores
        float x[2][4];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
                S = mfma_bf16(aq[bb], u32x4_t{kc[c][bb].x, kc[c][bb].y, kc[c][bb].z, kc[c][bb].w}, S);
            const int key = 32 * kt + 16 * c + n16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int qpos = min(16 * qt + 4 * kb + r, L - 1);
                x[c][r] = key <= qpos ? S[r] * a.scale2 : -INFINITY;
            }
        }
        // ---- online softmax per query row (every row has key 0 in the first tile)
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float mx = row16_max(fmaxf(x[0][r], x[1][r]));
            const float mn = fmaxf(m_r[r], mx);
            alpha[r] = __builtin_amdgcn_exp2f(m_r[r] - mn);
            m_r[r] = mn;
            const float p0 = __builtin_amdgcn_exp2f(x[0][r] - mn);
            const float p1 = __builtin_amdgcn_exp2f(x[1][r] - mn);
            l_r[r] = l_r[r] * alpha[r] + (p0 + p1);
            P[4 * kb + r][n16] = p0;
            P[4 * kb + r][16 + n16] = p1;
        }
        // one-wave workgroup: its LDS accesses run in order
        __builtin_amdgcn_wave_barrier();
        const float4 pa = *reinterpret_cast<const float4*>(&P[n16][8 * kb]);
        const float4 pb = *reinterpret_cast<const float4*>(&P[n16][8 * kb + 4]);
        const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
        u32x4_t ahi, alo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t hw, lw;
            split_bf16(pr[2 * e], pr[2 * e + 1], hw, lw);
            ahi[e] = hw;
            alo[e] = lw;
        }
        // ---- PV
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint4 bv = *reinterpret_cast<const uint4*>(&VT[16 * m + n16][8 * kb]);
            const u32x4_t B = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) O[m][r] *= alpha[r];
            O[m] = mfma_bf16(ahi, B, O[m]);
            O[m] = mfma_bf16(alo, B, O[m]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- epilogue: queries 4 kb + r, channels 16 m + n16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int qi = 16 * qt + 4 * kb + r;
        const float l = row16_sum(l_r[r]);
        if (qi >= L) continue;
        const float inv = 1.0f / l;
        const int64_t o = ((int64_t)(t0 + qi) * a.Hq + j) * d;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float val = O[m][r] * inv;
            if (a.out_bf16)
                reinterpret_cast<uint16_t*>(a.out)[o + 16 * m + n16] = (uint16_t)f32_to_bf16_rne(val);
            else
                reinterpret_cast<float*>(a.out)[o + 16 * m + n16] = val;
        }
    }
}

}  // namespace kv4
