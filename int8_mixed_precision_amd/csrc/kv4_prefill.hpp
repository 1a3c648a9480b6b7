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

// One workgroup of four waves per (128-query block, q head, sequence); wave w
// takes queries 32 w .. 32 w + 31 of the block (RB = 2 row blocks of 16).  The
// 32-key tiles up to the block's last query are loaded once per workgroup into
// LDS (K row-major, V transposed), triple-buffered (the next tile's scores
// are computed during this tile's softmax), the loads of the tile after that
// in flight in registers.
//
// Everything is computed transposed, so that a lane owns one query of each of
// its row blocks (n16 = lane % 16, kb = lane / 16 picks 4 of the 16 keys or
// channels of a block):
//   QK: S^T = K Q^T on bf16 MFMA 16x16x32: A = K rows (key 16 c + n16 of the
//     tile) from LDS, B = the query rows (query n16, channels 32 bb + 8 kb +
//     [0, 8)) in registers.  Lane l holds the scores of query n16 against keys
//     16 c + 4 kb + r in S[c][r].
//   softmax: a query's tile maximum is the maximum of its lane's 8 scores and
//     of the other three lanes of its column (two row swaps); the running sum
//     is kept per lane and reduced once at the end.  The reference maximum is
//     raised only when a query exceeds it by more than kSlack (base 2), which
//     keeps every sum exact.
//   PV: O^T = V^T P^T on bf16 MFMA 16x16x32: A = V^T rows (channel 16 m + n16,
//     keys 8 kb + [0, 8)) from LDS; B = P^T (keys 8 kb + [0, 8), query n16) as
//     bf16 hi + lo (fp32-level accuracy).  The B operand of lane (n16, kb)
//     holds keys that lanes (n16, 2 (kb % 2)) and (n16, 2 (kb % 2) + 1) computed
//     in key block c = kb / 2: one v_permlane32_swap and one v_permlane16_swap
//     per register pair move them (no LDS).  Lane l then holds query n16,
//     channels 16 m + 4 kb + r in O[m][r]: the rescale and the final
//     normalisation are in-lane, and each lane stores 16 contiguous bytes.
constexpr int kPrefillKeys = 32;
constexpr int kPrefillRows = 2;
constexpr int kPreQ = 4 * 16 * kPrefillRows;   // queries per workgroup

// A pair of 32-bit registers after v_permlane32_swap then v_permlane16_swap:
// with x0 from key block 0 and x1 from key block 1 of every lane, lane row kb
// receives (row 2 (kb % 2) of block kb / 2, row 2 (kb % 2) + 1 of block kb / 2).
__device__ __forceinline__ void gather_rows(uint32_t x0, uint32_t x1, uint32_t& lo, uint32_t& hi)
{
    const auto s = __builtin_amdgcn_permlane32_swap(x0, x1, false, false);
    const auto t = __builtin_amdgcn_permlane16_swap(s[0], s[1], false, false);
    lo = t[0];
    hi = t[1];
}

// KT keys per tile (32), RB row blocks per wave.  LDS row strides are padded
// so that the 16 lanes of a row read at most two lanes per bank (rows stay
// 16-byte aligned).
template <int KT, int RB>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a)
{
    static_assert(KT == 32, "the P^T row exchange is written for 32-key tiles");
    constexpr int kPreK = KT, NC = KT / 16, NL = KT / 32;      // key blocks, 16-byte loads per thread / 2
    constexpr int kKs = kHeadDim + 8, kVt = KT + 8;
    constexpr int QB = 4 * 16 * RB;                            // queries per workgroup
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n16 = lane & 15, kb = lane >> 4;
    // grid (q head, sequence, query block) with the query blocks in reverse:
    // workgroups are dispatched x fastest, so the last (heaviest: the most
    // causal key tiles) query blocks of every sequence and head start first
    // and the cheap early blocks fill the tail
    const int b = blockIdx.y, j = blockIdx.x, qb = (int)gridDim.z - 1 - (int)blockIdx.z;
    const int t0 = clampi(a.cu[b], 0, a.total);
    const int L = min(clampi(a.cu[b + 1], t0, a.total) - t0, a.max_len);
    if (QB * qb >= L) return;                             // uniform over the workgroup
    const int h = j / a.gqa;
    constexpr int d = kHeadDim;
    const int qw = QB * qb + 16 * RB * w;                 // first query of this wave

    // ---- query rows of the wave's blocks (rows past the end read the last row:
    // discarded), negated when the scale is negative so that scores scale by
    // sc2 = |sm_scale| log2(e) >= 0
    const float sc2 = fabsf(a.scale2);
    const uint32_t qsign = a.scale2 < 0.f ? 0x80008000u : 0u;
    u32x4_t bq[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int qi = min(qw + 16 * rb + n16, L - 1);
        const uint16_t* qr = a.q + ((int64_t)(t0 + qi) * a.Hq + j) * d;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const uint4 u = *reinterpret_cast<const uint4*>(qr + 32 * bb + 8 * kb);
            bq[rb][bb] = u32x4_t{u.x ^ qsign, u.y ^ qsign, u.z ^ qsign, u.w ^ qsign};
        }
    }

    f32x4_t O[RB][8];
    float m_r[RB], l_r[RB];                               // per query n16; l_r: this lane's part
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int m = 0; m < 8; ++m) O[rb][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_r[rb] = -INFINITY;
        l_r[rb] = 0.f;
    }
    // three buffers of each tile: tiles kt and kt + 1 are read (this tile's
    // values, the next tile's scores) while tile kt + 2 is stored
    __shared__ __attribute__((aligned(16))) uint16_t Ks[3][kPreK][kKs];
    __shared__ __attribute__((aligned(16))) uint16_t VT[3][d][kVt];

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
        // (buf < 3)
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
    const int kt_end = q_last_b / kPreK + 1;                   // tiles of the workgroup
    const int kt_w = q_last_w / kPreK + 1;                     // tiles this wave computes

    // scores S^T of tile kt into S: every K operand read once for the RB row blocks
    auto scores = [&](int kt, f32x4_t (&S)[RB][NC]) {
        const int buf = kt % 3;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int c = 0; c < NC; ++c) S[rb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint4 kc = *reinterpret_cast<const uint4*>(&Ks[buf][16 * c + n16][32 * bb + 8 * kb]);
                const u32x4_t A = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) S[rb][c] = mfma_bf16(A, bq[rb][bb], S[rb][c]);
            }
    };

    // Software pipeline: in step kt the scores of tile kt + 1 are issued to
    // the matrix core before the softmax of tile kt runs on the vector ALU,
    // then tile kt's values are accumulated.  Tile t lives in buffer t % 3:
    // step kt reads buffers kt % 3 (values) and (kt + 1) % 3 (keys) and
    // stores tile kt + 2 into buffer (kt + 2) % 3, last read in step kt - 1,
    // which every wave has left at the barrier that ended it.  Tile kt + 1 was
    // stored in step kt - 1 and is visible after that same barrier.
    uint4 kr[2 * NL], vr[2 * NL];
    load(0, kr, vr);
    store(0, kr, vr);
    if (kt_end > 1) {
        load(1, kr, vr);
        store(1, kr, vr);
    }
    if (kt_end > 2) load(2, kr, vr);
    __syncthreads();
    f32x4_t S[RB][NC];
    scores(0, S);
    for (int kt = 0; kt < kt_end; ++kt) {
        const int buf = kt % 3;
        if (kt < kt_w) {                                      // uniform per wave
            // the next tile's key operands up front (on the wave's last tile
            // they are read from a buffer whose scores are never used, which
            // keeps the step free of branches around the matrix-core work)
            u32x4_t kf[NC][4];
            {
                const int nb = (kt + 1) % 3;
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int bb = 0; bb < 4; ++bb) {
                        const uint4 kc = *reinterpret_cast<const uint4*>(&Ks[nb][16 * c + n16][32 * bb + 8 * kb]);
                        kf[c][bb] = u32x4_t{kc.x, kc.y, kc.z, kc.w};
                    }
            }
            // ---- softmax, part 1: masks, tile maxima, rare rescales
            float x[RB][NC][4];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int qf = qw + 16 * rb;                  // first query of the block
                // raw scores (the query carries the sign of the scale, so the
                // largest raw score is the largest scaled one); the causal mask
                // only on tiles that reach past the block's first query
                if (kPreK * kt + kPreK - 1 <= qf) {
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[rb][c][r] = S[rb][c][r];
                } else {
                    const int qpos = min(qf + n16, L - 1);    // this lane's query
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = kPreK * kt + 16 * c + 4 * kb + r;
                            x[rb][c][r] = key <= qpos ? S[rb][c][r] : -INFINITY;
                        }
                }
                float xm = fmaxf(x[rb][0][0], x[rb][0][1]);
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int r = (c == 0 ? 2 : 0); r < 4; ++r) xm = fmaxf(xm, x[rb][c][r]);
                const float mx = rows_max(xm) * sc2;           // base-2 units
                const bool grow = mx > m_r[rb] + kSlack;
                if (__builtin_amdgcn_ballot_w64(grow)) {
                    const float mn = grow ? mx : m_r[rb];
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_r[rb] - mn) : 1.0f;
                    m_r[rb] = mn;
                    l_r[rb] *= alpha;
#pragma unroll
                    for (int m = 0; m < 8; ++m) O[rb][m] *= alpha;
                }
            }
            // ---- the next tile's scores go to the matrix core while the
            // vector ALU forms this tile's probabilities
            f32x4_t Sn[RB][NC];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int c = 0; c < NC; ++c) Sn[rb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) Sn[rb][c] = mfma_bf16(kf[c][bb], bq[rb][bb], Sn[rb][c]);
            // ---- softmax, part 2: probabilities, bf16 hi + lo, row exchange
            u32x4_t phi[RB], plo[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                float p[NC][4];
                float ps = 0.f;
                const float neg_m = -m_r[rb];
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        p[c][r] = __builtin_amdgcn_exp2f(fmaf(x[rb][c][r], sc2, neg_m));
                        ps += p[c][r];
                    }
                l_r[rb] += ps;
                // pairs of keys (4 kb + 2 i, 4 kb + 2 i + 1) of each key block
                uint32_t h2[NC][2], l2[NC][2];
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int i = 0; i < 2; ++i) split_bf16(p[c][2 * i], p[c][2 * i + 1], h2[c][i], l2[c][i]);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    uint32_t a0, a1, b0, b1;
                    gather_rows(h2[0][i], h2[1][i], a0, a1);
                    gather_rows(l2[0][i], l2[1][i], b0, b1);
                    phi[rb][i] = a0;
                    phi[rb][2 + i] = a1;
                    plo[rb][i] = b0;
                    plo[rb][2 + i] = b1;
                }
            }
            // ---- PV (O^T += V^T P^T): every V operand used for the RB row blocks
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int hh = 0; hh < NL; ++hh) {
                    const uint4 av = *reinterpret_cast<const uint4*>(&VT[buf][16 * m + n16][32 * hh + 8 * kb]);
                    const u32x4_t A = {av.x, av.y, av.z, av.w};
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        O[rb][m] = mfma_bf16(A, phi[rb], O[rb][m]);
                        O[rb][m] = mfma_bf16(A, plo[rb], O[rb][m]);
                    }
                }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int c = 0; c < NC; ++c) S[rb][c] = Sn[rb][c];
        }
        if (kt + 2 < kt_end) {
            store((kt + 2) % 3, kr, vr);
            if (kt + 3 < kt_end) load(kt + 3, kr, vr);        // in flight during the next step
        }
        __syncthreads();
    }

    // ---- epilogue: lane (n16, kb) holds query qw + 16 rb + n16, channels 16 m + 4 kb + r
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int qi = qw + 16 * rb + n16;
        const float l = rows_sum(l_r[rb]);
        if (qi >= L) continue;
        const float inv = 1.0f / l;
        const int64_t o = ((int64_t)(t0 + qi) * a.Hq + j) * d + 4 * kb;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const f32x4_t v = O[rb][m] * inv;
            if (a.out_bf16) {
                const uint2 pk = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                            f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + o + 16 * m) = pk;
            } else {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + o + 16 * m) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

}  // namespace kv4
