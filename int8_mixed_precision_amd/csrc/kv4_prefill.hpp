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
// Keys per tile: 32 (152 VGPRs and 53 KB of LDS at 64 keys leave 3 waves per
// SIMD instead of 4, and measured 4% slower).
constexpr int kPrefillKeys = 32;
// 16-query row blocks per wave: RB blocks share every K and V operand the wave
// reads from LDS.
constexpr int kPrefillRows = 2;                  // 198 VGPRs, 2 waves per SIMD: 28.8 -> 26.4 ms
constexpr int kPreQ = 4 * 16 * kPrefillRows;   // queries per workgroup

// KT keys per tile (32 or 64), RB row blocks per wave.  LDS row strides are
// padded so that the 16 lanes of a row read at most two lanes per bank (rows
// stay 16-byte aligned).
template <int KT, int RB>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a)
{
    constexpr int kPreK = KT, NC = KT / 16, NL = KT / 32;      // key blocks, 16-byte loads per thread / 2
    constexpr int kKs = kHeadDim + 8, kVt = KT + 8, kPs = KT + 4;
    constexpr int QB = 4 * 16 * RB;                            // queries per workgroup
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n16 = lane & 15, kb = lane >> 4;
    const int b = blockIdx.z, j = blockIdx.y, qb = blockIdx.x;
    const int t0 = clampi(a.cu[b], 0, a.total);
    const int L = min(clampi(a.cu[b + 1], t0, a.total) - t0, a.max_len);
    if (QB * qb >= L) return;                             // uniform over the workgroup
    const int h = j / a.gqa;
    constexpr int d = kHeadDim;
    const int qw = QB * qb + 16 * RB * w;                 // first query of this wave

    // ---- q rows of the wave's blocks (rows past the end read the last row: discarded)
    u32x4_t aq[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int qi = min(qw + 16 * rb + n16, L - 1);
        const uint16_t* qr = a.q + ((int64_t)(t0 + qi) * a.Hq + j) * d;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const uint4 u = *reinterpret_cast<const uint4*>(qr + 32 * bb + 8 * kb);
            aq[rb][bb] = u32x4_t{u.x, u.y, u.z, u.w};
        }
    }

    f32x4_t O[RB][8];
    float m_r[RB][4], l_r[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int m = 0; m < 8; ++m) O[rb][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            m_r[rb][r] = -INFINITY;
            l_r[rb][r] = 0.f;
        }
    }
    // two buffers of each tile: the tile after next is stored while this one is read
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kPreK][kKs];
    __shared__ __attribute__((aligned(16))) uint16_t VT[2][d][kVt];
    __shared__ __attribute__((aligned(16))) float P[4][RB][16][kPs];

    // cooperative tile loads, 2 NL 16-byte chunks of K and of V per thread:
    // K chunk (key idx / 16, channels 8 (idx % 16) ..); V keys 2 kp, 2 kp + 1 of
    // each 32-key half (kp = tid % 16) at channels 8 (tid / 16) .., so that each
    // V^T store is one 32-bit word holding a key pair
    const int kp = tid & 15, vch = 8 * (tid >> 4);
    auto load = [&](int kt, uint4 (&kr)[2 * NL], uint4 (&vr)[2 * NL]) {
#pragma unroll
        for (int i = 0; i < 2 * NL; ++i) {
            const int idx = tid + 256 * i, key = idx >> 4, ch = 8 * (idx & 15);
            const int ki = min(kPreK * kt + key, L - 1);
            kr[i] = *reinterpret_cast<const uint4*>(a.k + ((int64_t)(t0 + ki) * a.Hkv + h) * d + ch);
            const int vi = min(kPreK * kt + 32 * (i >> 1) + 2 * kp + (i & 1), L - 1);
            vr[i] = *reinterpret_cast<const uint4*>(a.v + ((int64_t)(t0 + vi) * a.Hkv + h) * d + vch);
        }
    };
    auto store = [&](int buf, const uint4 (&kr)[2 * NL], const uint4 (&vr)[2 * NL]) {
#pragma unroll
        for (int i = 0; i < 2 * NL; ++i) {
            const int idx = tid + 256 * i, key = idx >> 4, ch = 8 * (idx & 15);
            *reinterpret_cast<uint4*>(&Ks[buf][key][ch]) = kr[i];
        }
#pragma unroll
        for (int hh = 0; hh < NL; ++hh) {
            const uint4 a0 = vr[2 * hh], a1 = vr[2 * hh + 1];
            const uint32_t w0[4] = {a0.x, a0.y, a0.z, a0.w};   // key 32 hh + 2 kp
            const uint32_t w1[4] = {a1.x, a1.y, a1.z, a1.w};   // key 32 hh + 2 kp + 1
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                *reinterpret_cast<uint32_t*>(&VT[buf][vch + 2 * e][32 * hh + 2 * kp]) = (w0[e] & 0xFFFFu) | (w1[e] << 16);
                *reinterpret_cast<uint32_t*>(&VT[buf][vch + 2 * e + 1][32 * hh + 2 * kp]) =
                    (w0[e] >> 16) | (w1[e] & 0xFFFF0000u);
            }
        }
    };

    const int q_last_b = min(QB * qb + QB - 1, L - 1);         // last query of the block
    const int q_last_w = min(qw + 16 * RB - 1, L - 1);         // ... and of this wave
    const int kt_end = q_last_b / kPreK + 1;
    // Tile kt is read from buffer kt % 2 while tile kt + 1 (in registers since
    // the previous step) is stored to the other buffer and tile kt + 2 is
    // loaded.  One barrier per tile: every wave has passed the barrier that
    // ended tile kt - 1, i.e. finished reading the buffer that tile kt + 1
    // overwrites.
    uint4 kr[2 * NL], vr[2 * NL];
    load(0, kr, vr);
    store(0, kr, vr);
    if (kt_end > 1) load(1, kr, vr);
    __syncthreads();
    for (int kt = 0; kt < kt_end; ++kt) {
        const int buf = kt & 1;
        if (kPreK * kt <= q_last_w) {                         // uniform per wave
            // ---- scores: every K operand read once for the RB row blocks
            f32x4_t S[RB][NC];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int c = 0; c < NC; ++c) S[rb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const uint4 kc = *reinterpret_cast<const uint4*>(&Ks[buf][16 * c + n16][32 * bb + 8 * kb]);
                    const u32x4_t B = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) S[rb][c] = mfma_bf16(aq[rb][bb], B, S[rb][c]);
                }
            u32x4_t ahi[RB][NL], alo[RB][NL];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int qf = qw + 16 * rb;                  // first query of the block
                float x[NC][4];
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const int key = kPreK * kt + 16 * c + n16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int qpos = min(qf + 4 * kb + r, L - 1);
                        // tiles wholly at or below the block's first query need no mask
                        x[c][r] = (kPreK * kt + kPreK - 1 <= qf || key <= qpos) ? S[rb][c][r] * a.scale2
                                                                                : -INFINITY;
                    }
                }
                // online softmax per query row against a reference maximum raised
                // only when a row exceeds it by more than kSlack (exact for any
                // reference; every row has key 0 in the first tile)
                float mx[4];
                bool grow_any = false;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float xm = x[0][r];
#pragma unroll
                    for (int c = 1; c < NC; ++c) xm = fmaxf(xm, x[c][r]);
                    mx[r] = row16_max(xm);
                    grow_any |= mx[r] > m_r[rb][r] + kSlack;
                }
                if (__builtin_amdgcn_ballot_w64(grow_any)) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool grow = mx[r] > m_r[rb][r] + kSlack;
                        const float mn = grow ? mx[r] : m_r[rb][r];
                        const float alpha = grow ? __builtin_amdgcn_exp2f(m_r[rb][r] - mn) : 1.0f;
                        m_r[rb][r] = mn;
                        l_r[rb][r] *= alpha;
#pragma unroll
                        for (int m = 0; m < 8; ++m) O[rb][m][r] *= alpha;
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float ps = 0.f;
#pragma unroll
                    for (int c = 0; c < NC; ++c) {
                        const float pc = __builtin_amdgcn_exp2f(x[c][r] - m_r[rb][r]);
                        ps += pc;
                        P[w][rb][4 * kb + r][16 * c + n16] = pc;
                    }
                    l_r[rb][r] += ps;
                }
                // the wave's own LDS rows: its LDS accesses run in order
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int hh = 0; hh < NL; ++hh) {
                    const float4 pa = *reinterpret_cast<const float4*>(&P[w][rb][n16][32 * hh + 8 * kb]);
                    const float4 pb = *reinterpret_cast<const float4*>(&P[w][rb][n16][32 * hh + 8 * kb + 4]);
                    const float pr[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t hw, lw;
                        split_bf16(pr[2 * e], pr[2 * e + 1], hw, lw);
                        ahi[rb][hh][e] = hw;
                        alo[rb][hh][e] = lw;
                    }
                }
            }
            // ---- PV: every V operand read once for the RB row blocks
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int hh = 0; hh < NL; ++hh) {
                    const uint4 bv = *reinterpret_cast<const uint4*>(&VT[buf][16 * m + n16][32 * hh + 8 * kb]);
                    const u32x4_t B = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        O[rb][m] = mfma_bf16(ahi[rb][hh], B, O[rb][m]);
                        O[rb][m] = mfma_bf16(alo[rb][hh], B, O[rb][m]);
                    }
                }
        }
        if (kt + 1 < kt_end) {
            store(buf ^ 1, kr, vr);
            if (kt + 2 < kt_end) load(kt + 2, kr, vr);        // in flight during the next tile
        }
        __syncthreads();
    }

    // ---- epilogue: queries 16 rb + 4 kb + r of the wave, channels 16 m + n16
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int qi = qw + 16 * rb + 4 * kb + r;
            const float l = row16_sum(l_r[rb][r]);
            if (qi >= L) continue;
            const float inv = 1.0f / l;
            const int64_t o = ((int64_t)(t0 + qi) * a.Hq + j) * d;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const float val = O[rb][m][r] * inv;
                if (a.out_bf16)
                    reinterpret_cast<uint16_t*>(a.out)[o + 16 * m + n16] = (uint16_t)f32_to_bf16_rne(val);
                else
                    reinterpret_cast<float*>(a.out)[o + 16 * m + n16] = val;
            }
        }
}

}  // namespace kv4
