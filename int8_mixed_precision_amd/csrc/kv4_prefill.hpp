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

// One workgroup of four waves per (64-query block, q head, sequence); wave w
// takes queries 16 w .. 16 w + 15 of the block.  The 32-key tiles up to the
// block's last query are loaded once per workgroup into LDS (K row-major, V
// transposed), the next tile's loads in flight in registers during the
// compute.  Lane roles inside a wave (n16 = lane % 16, kb = (lane / 16) % 4):
//   QK: bf16 MFMA 16x16x32, A = q rows (query n16 of the wave's 16), B = K
//     columns (key 16 c + n16 of the tile) from LDS, k-slots = channels
//     32 bb + 8 kb + [0, 8), bb = 0..3.  Lane l then holds the scores of
//     queries 4 kb + r against key 16 c + n16 in S_c[r].
//   PV: bf16 MFMA 16x16x32 per 16 channels, A = p (query n16, keys 8 kb + e)
//     in bf16 hi + lo through the wave's LDS rows, B = V^T (channel 16 m + n16,
//     keys 8 kb + e).  Lane l holds queries 4 kb + r, channel 16 m + n16 in
//     O[m][r]: the rows of the scores, so the online-softmax rescale is in-lane.
constexpr int kPreQ = 64;        // queries per workgroup
constexpr int kPreK = 32;        // keys per tile
// LDS row strides, padded so that the 16 lanes of a row read at most two
// lanes per bank (rows stay 16-byte aligned): K rows of 136 halfs, V^T rows
// of 40 halfs, probability rows of 36 floats.
constexpr int kKs = kHeadDim + 8, kVt = kPreK + 8, kPs = kPreK + 4;

__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a)
{
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n16 = lane & 15, kb = lane >> 4;
    const int b = blockIdx.z, j = blockIdx.y, qb = blockIdx.x;
    const int t0 = clampi(a.cu[b], 0, a.total);
    const int L = min(clampi(a.cu[b + 1], t0, a.total) - t0, a.max_len);
    if (kPreQ * qb >= L) return;                          // uniform over the workgroup
    const int h = j / a.gqa;
    constexpr int d = kHeadDim;
    const int qw = kPreQ * qb + 16 * w;                   // first query of this wave

    // ---- q rows of the wave (rows past the end read the last row: discarded)
    u32x4_t aq[4];
    {
        const int qi = min(qw + n16, L - 1);
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
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kPreK][kKs];
    __shared__ __attribute__((aligned(16))) uint16_t VT[d][kVt];
    __shared__ __attribute__((aligned(16))) float P[4][16][kPs];

    // cooperative tile loads, two 16-byte chunks of K and two of V per thread:
    // K chunk (key idx / 16, channels 8 (idx % 16) ..), V keys 2 kp, 2 kp + 1
    // (kp = tid % 16) at channels 8 (tid / 16) .., so that each V^T store is one
    // 32-bit word holding a key pair
    const int kp = tid & 15, vch = 8 * (tid >> 4);
    auto load = [&](int kt, uint4 (&kr)[2], uint4 (&vr)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, key = idx >> 4, ch = 8 * (idx & 15);
            const int ki = min(kPreK * kt + key, L - 1);
            kr[i] = *reinterpret_cast<const uint4*>(a.k + ((int64_t)(t0 + ki) * a.Hkv + h) * d + ch);
            const int vi = min(kPreK * kt + 2 * kp + i, L - 1);
            vr[i] = *reinterpret_cast<const uint4*>(a.v + ((int64_t)(t0 + vi) * a.Hkv + h) * d + vch);
        }
    };
    auto store = [&](const uint4 (&kr)[2], const uint4 (&vr)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, key = idx >> 4, ch = 8 * (idx & 15);
            *reinterpret_cast<uint4*>(&Ks[key][ch]) = kr[i];
        }
        const uint32_t w0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};   // key 2 kp
        const uint32_t w1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};   // key 2 kp + 1
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<uint32_t*>(&VT[vch + 2 * e][2 * kp]) = (w0[e] & 0xFFFFu) | (w1[e] << 16);
            *reinterpret_cast<uint32_t*>(&VT[vch + 2 * e + 1][2 * kp]) = (w0[e] >> 16) | (w1[e] & 0xFFFF0000u);
        }
    };

    const int q_last_b = min(kPreQ * qb + kPreQ - 1, L - 1);   // last query of the block
    const int q_last_w = min(qw + 15, L - 1);                  // ... and of this wave
    const int kt_end = q_last_b / kPreK + 1;
    uint4 kr[2], vr[2];
    load(0, kr, vr);
    store(kr, vr);
    __syncthreads();
    for (int kt = 0; kt < kt_end; ++kt) {
        const bool more = kt + 1 < kt_end;
        if (more) load(kt + 1, kr, vr);                       // in flight during the compute
        if (kPreK * kt <= q_last_w) {                         // uniform per wave
            // ---- scores
            float x[2][4];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint4 kc = *reinterpret_cast<const uint4*>(&Ks[16 * c + n16][32 * bb + 8 * kb]);
                    S = mfma_bf16(aq[bb], u32x4_t{kc.x, kc.y, kc.z, kc.w}, S);
                }
                const int key = kPreK * kt + 16 * c + n16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qpos = min(qw + 4 * kb + r, L - 1);
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
                P[w][4 * kb + r][n16] = p0;
                P[w][4 * kb + r][16 + n16] = p1;
            }
            // the wave's own LDS rows: its LDS accesses run in order
            __builtin_amdgcn_wave_barrier();
            const float4 pa = *reinterpret_cast<const float4*>(&P[w][n16][8 * kb]);
            const float4 pb = *reinterpret_cast<const float4*>(&P[w][n16][8 * kb + 4]);
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
        }
        __syncthreads();                                      // the tile is consumed
        if (more) {
            store(kr, vr);
            __syncthreads();
        }
    }

    // ---- epilogue: queries 4 kb + r of the wave, channels 16 m + n16
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int qi = qw + 4 * kb + r;
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
