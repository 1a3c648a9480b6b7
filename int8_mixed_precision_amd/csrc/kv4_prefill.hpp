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
//   softmax: the reference maximum of a query is raised only when one of its
//     scores exceeds it by more than kSlack (base 2), which keeps every sum
//     exact.  Each lane compares the maximum of its 8 raw scores with a raw
//     threshold; only when some lane of the wave passes it are the four lanes
//     of each column reduced (two row swaps) and the accumulators rescaled.
//     The running sum is kept per lane and reduced once at the end.
//   PV: O^T = V^T P^T on bf16 MFMA 16x16x32, with the keys of the contraction
//     in the order of the score layout: k-slots 8 kb + [0, 4) are keys 4 kb +
//     [0, 4) and k-slots 8 kb + [4, 8) are keys 16 + 4 kb + [0, 4) (the order of
//     a contraction's terms is free as long as both operands follow it).  B =
//     P^T, so the B operand of lane (n16, kb) is exactly its own 8
//     probabilities, as bf16 hi + lo (fp32-level accuracy): no lane exchange.
//     A = V^T rows (channel 16 m + n16) from LDS, where the V^T columns are
//     stored in that key order.  Lane l then holds query n16, channels 16 m +
//     4 kb + r in O[m][r]: the rescale and the final normalisation are
//     in-lane, and each lane stores 16 contiguous bytes.
constexpr int kPrefillKeys = 32;
constexpr int kPrefillRows = 2;
constexpr int kPreQ = 4 * 16 * kPrefillRows;   // queries per workgroup
constexpr int kPreGroup = 16;                  // query blocks dispatched together

// Maximum of three floats in one v_max3_f32.  fmaxf on a matrix-core result
// costs an extra canonicalising v_max per operand (the compiler cannot tell
// that the value is not a signalling NaN); the instruction itself follows the
// same IEEE maxNum rule.
__device__ __forceinline__ float max3f(float x, float y, float z)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
    return r;
}

// 16 bytes through a buffer descriptor with the default cache policy (K and V
// rows are read by every q head of the group and every query block).
__device__ __forceinline__ uint4 ld16_rows(Page r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// KT keys per tile (32), RB row blocks per wave.  LDS rows are padded to 288
// bytes (K) and 96 bytes (V^T): with those strides the operand reads of a
// wave (16 B per lane, 16 rows x 4 column chunks) measured conflict-free on
// MI355X, at the rate of a contiguous read, while the unpadded-plus-16 strides
// (272 and 80 bytes) took about 1.7 times as long.
template <int KT, int RB>
__global__ __launch_bounds__(256) void prefill_attn_kernel(PrefillArgs a)
{
    static_assert(KT == 32, "the PV key order is written for 32-key tiles");
    constexpr int kPreK = KT, NC = KT / 16;                    // key blocks of a tile
    constexpr int kKs = kHeadDim + 16, kVt = KT + 16;          // row strides (bf16 elements)
    constexpr int QB = 4 * 16 * RB;                            // queries per workgroup
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n16 = lane & 15, kb = lane >> 4;
    // grid (q head x 16 query blocks of a group, sequence, group of query
    // blocks), groups and blocks in reverse.  Workgroups are dispatched x
    // fastest, so the 16 blocks of one group of one sequence run together (at
    // Hq = 32 and two workgroups per CU, one group fills the GPU), all reading
    // the same prefix of K and V, while the heaviest groups (the most causal
    // key tiles) of every sequence start first and the cheap early ones fill
    // the tail.
    // Workgroups go to the eight XCDs in turn, so with a multiple of 8 q heads
    // every workgroup with x % 8 == c runs on XCD c.  x % Hq is taken as q head
    // c Hq/8 + (x % Hq)/8: the q heads of a kv head (consecutive), which read
    // the same K and V tiles, then share one XCD's L2 (at Hq = 32 and 8 kv
    // heads, XCD c holds exactly the four q heads of kv head c).
    const int xq = (int)blockIdx.x % a.Hq, qlow = (int)blockIdx.x / a.Hq;
    const int j = (a.Hq & 7) ? xq : (xq & 7) * (a.Hq >> 3) + (xq >> 3);
    const int b = blockIdx.y;
    const int qb = kPreGroup * ((int)gridDim.z - 1 - (int)blockIdx.z) + kPreGroup - 1 - qlow;
    const int t0 = clampi(a.cu[b], 0, a.total);
    const int L = min(clampi(a.cu[b + 1], t0, a.total) - t0, a.max_len);
    if (QB * qb >= L) return;                             // uniform over the workgroup
    const int h = j / a.gqa;
    constexpr int d = kHeadDim;
    const int qw = QB * qb + 16 * RB * w;                 // first query of this wave

    // ---- query rows of the wave's blocks (rows past the end read the last row:
    // discarded).  Scores are scaled by sc2 = |sm_scale| log2(e) > 0: a negative
    // scale negates the query instead, and a zero scale (every score 0: the
    // uniform average) zeroes it with sc2 = 1.
    const bool zero_scale = a.scale2 == 0.f;
    const float sc2 = zero_scale ? 1.0f : fabsf(a.scale2);
    const float inv_sc2 = 1.0f / sc2;
    const uint32_t qkeep = zero_scale ? 0u : 0xFFFFFFFFu;
    const uint32_t qsign = a.scale2 < 0.f ? 0x80008000u : 0u;
    u32x4_t bq[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int qi = min(qw + 16 * rb + n16, L - 1);
        const uint16_t* qr = a.q + ((int64_t)(t0 + qi) * a.Hq + j) * d;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const uint4 u = *reinterpret_cast<const uint4*>(qr + 32 * bb + 8 * kb);
            bq[rb][bb] = u32x4_t{(u.x & qkeep) ^ qsign, (u.y & qkeep) ^ qsign, (u.z & qkeep) ^ qsign,
                                 (u.w & qkeep) ^ qsign};
        }
    }

    f32x4_t O[RB][8];
    float m_r[RB], l_r[RB];        // per query n16 (base-2 units); l_r: this lane's part
    float thr[RB];                 // raw score above which m_r must be raised
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int m = 0; m < 8; ++m) O[rb][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m_r[rb] = -INFINITY;
        l_r[rb] = 0.f;
        thr[rb] = -INFINITY;
    }
    // three buffers of each tile: tiles kt and kt + 1 are read (this tile's
    // values, the next tile's scores) while tile kt + 2 is stored
    __shared__ __attribute__((aligned(16))) uint16_t Ks[3][kPreK][kKs];
    __shared__ __attribute__((aligned(16))) uint16_t VT[3][d][kVt];

    // Cooperative tile loads, two 16-byte chunks of K and two of V per thread,
    // through a buffer descriptor per tile: K key tid / 16 and 16 + tid / 16 at
    // channels 8 (tid % 16) ..; V keys 2 kp and 2 kp + 1 (kp = tid % 16) at
    // channels vch = 8 (tid / 16) .., so that each V^T store is one 32-bit word
    // holding a key pair, at column vcol: keys 4 j .. 4 j + 3 go to columns
    // 8 j .. 8 j + 3 and keys 16 + 4 j .. 16 + 4 j + 3 to columns 8 j + 4 ..
    // 8 j + 7 (the PV contraction's key order).  The descriptor's range ends with the tile's last
    // key inside the sequence: rows past it read as zero (those keys are
    // masked), and the lane offsets are the same for every tile.
    const int kp = tid & 15, vch = 8 * (tid >> 4);
    const int vcol = kp < 8 ? 8 * (kp >> 1) + 2 * (kp & 1) : 8 * ((kp - 8) >> 1) + 4 + 2 * (kp & 1);
    const int64_t rowe = (int64_t)a.Hkv * d;                  // elements per token row
    const uint32_t rowb = (uint32_t)rowe * 2u;
    const uint16_t* kseq = a.k + (int64_t)t0 * rowe + (int64_t)h * d;
    const uint16_t* vseq = a.v + (int64_t)t0 * rowe + (int64_t)h * d;
    const uint32_t ko0 = (uint32_t)(tid >> 4) * rowb + 16u * (uint32_t)(tid & 15);
    const uint32_t ko1 = ko0 + 16u * rowb;
    const uint32_t vo0 = (uint32_t)(2 * kp) * rowb + 2u * (uint32_t)vch;
    const uint32_t vo1 = vo0 + rowb;
    uint4 k0, k1, v0, v1;                                     // the tile in flight
    auto load = [&](int kt) {
        const int n = min(kPreK, L - kPreK * kt);             // keys of the tile (>= 1)
        const uint32_t range = (uint32_t)(n - 1) * rowb + 2u * d;
        const Page rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kseq + (int64_t)kPreK * kt * rowe),
                                                          0, (int)range, 0x00020000);
        const Page rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vseq + (int64_t)kPreK * kt * rowe),
                                                          0, (int)range, 0x00020000);
        k0 = ld16_rows(rk, ko0);
        k1 = ld16_rows(rk, ko1);
        v0 = ld16_rows(rv, vo0);
        v1 = ld16_rows(rv, vo1);
    };
    auto store = [&](int buf) {                               // (buf < 3)
        *reinterpret_cast<uint4*>(&Ks[buf][tid >> 4][8 * (tid & 15)]) = k0;
        *reinterpret_cast<uint4*>(&Ks[buf][16 + (tid >> 4)][8 * (tid & 15)]) = k1;
        const uint32_t w0[4] = {v0.x, v0.y, v0.z, v0.w};     // key 2 kp
        const uint32_t w1[4] = {v1.x, v1.y, v1.z, v1.w};     // key 2 kp + 1
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // channel vch + 2 e: low halves; vch + 2 e + 1: high halves
            *reinterpret_cast<uint32_t*>(&VT[buf][vch + 2 * e][vcol]) = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
            *reinterpret_cast<uint32_t*>(&VT[buf][vch + 2 * e + 1][vcol]) =
                __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
        }
    };

    const int q_last_b = min(QB * qb + QB - 1, L - 1);         // last query of the block
    const int q_last_w = min(qw + 16 * RB - 1, L - 1);         // ... and of this wave
    const int kt_end = q_last_b / kPreK + 1;                   // tiles of the workgroup
    const int kt_w = q_last_w / kPreK + 1;                     // tiles this wave computes

    // scores S^T of tile kt (in buffer buf) into S: every K operand read once
    // for the RB row blocks
    auto key_operands = [&](int buf, u32x4_t (&kf)[NC][4]) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const uint4 kc = *reinterpret_cast<const uint4*>(&Ks[buf][16 * c + n16][32 * bb + 8 * kb]);
                kf[c][bb] = u32x4_t{kc.x, kc.y, kc.z, kc.w};
            }
    };
    auto scores = [&](const u32x4_t (&kf)[NC][4], f32x4_t (&S)[RB][NC]) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int c = 0; c < NC; ++c) S[rb][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) S[rb][c] = mfma_bf16(kf[c][bb], bq[rb][bb], S[rb][c]);
    };

    // Software pipeline: in step kt the scores of tile kt + 1 go to the
    // matrix core while the vector ALU finishes the probabilities of tile kt,
    // then tile kt's values are accumulated.  Tile t lives in buffer t % 3:
    // step kt reads buffers kt % 3 (values) and (kt + 1) % 3 (keys) and
    // stores tile kt + 2 into buffer (kt + 2) % 3, last read in step kt - 1,
    // which every wave has left at the barrier that ended it.  Tile kt + 1 was
    // stored in step kt - 1 and is visible after that same barrier.
    load(0);
    store(0);
    if (kt_end > 1) {
        load(1);
        store(1);
    }
    if (kt_end > 2) load(2);
    __syncthreads();
    f32x4_t S[RB][NC];
    {
        u32x4_t kf[NC][4];
        key_operands(0, kf);
        scores(kf, S);
    }
    for (int kt = 0; kt < kt_end; ++kt) {
        const int buf = kt % 3;
        if (kt < kt_w) {                                      // uniform per wave
            // the next tile's key operands up front (on the wave's last tile
            // they are read from a buffer whose scores are never used, which
            // keeps the step free of branches around the matrix-core work)
            u32x4_t kf[NC][4];
            key_operands((kt + 1) % 3, kf);
            // ---- softmax, part 1: causal mask (tiles that reach past the
            // block's first query only), each lane's maximum of its 8 raw
            // scores (the query carries the sign of the scale, so the largest
            // raw score is the largest scaled one).  The reference maximum of a
            // query is raised only when one of its scores exceeds it by more
            // than kSlack; only then are the four lanes of its column reduced.
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int qf = qw + 16 * rb;                  // first query of the block
                if (kPreK * kt + kPreK - 1 > qf) {
                    // key kPreK kt + 4 kb + 16 c + r against this lane's query
                    const int rel = min(qf + n16, L - 1) - kPreK * kt - 4 * kb;
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (16 * c + r > rel) S[rb][c][r] = -INFINITY;
                }
                const float lmx = max3f(max3f(S[rb][0][0], S[rb][0][1], S[rb][0][2]),
                                        max3f(S[rb][0][3], S[rb][1][0], S[rb][1][1]),
                                        max3f(S[rb][1][2], S[rb][1][3], S[rb][1][3]));
                if (__builtin_amdgcn_ballot_w64(lmx > thr[rb])) {   // rare: wave-uniform branch
                    const float mx = rows_max(lmx) * sc2;           // the query's tile maximum
                    const bool grow = mx > m_r[rb] + kSlack;
                    const float mn = grow ? mx : m_r[rb];
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_r[rb] - mn) : 1.0f;
                    m_r[rb] = mn;
                    thr[rb] = (mn + kSlack) * inv_sc2;
                    l_r[rb] *= alpha;
#pragma unroll
                    for (int m = 0; m < 8; ++m) O[rb][m] *= alpha;
                }
            }
            // ---- probabilities 2^(s sc2 - m) (masked keys: 2^-inf = 0)
            float p[RB][NC][4];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float neg_m = -m_r[rb];
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[rb][c][r] = __builtin_amdgcn_exp2f(fmaf(S[rb][c][r], sc2, neg_m));
            }
            // ---- the next tile's scores go to the matrix core while the
            // vector ALU sums and splits this tile's probabilities
            scores(kf, S);
            u32x4_t phi[RB], plo[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                l_r[rb] += ((p[rb][0][0] + p[rb][0][1]) + (p[rb][0][2] + p[rb][0][3])) +
                           ((p[rb][1][0] + p[rb][1][1]) + (p[rb][1][2] + p[rb][1][3]));
                // bf16 hi + lo of the key pairs (16 c + 4 kb + 2 i, .. + 1): k-slots
                // 8 kb + 4 c + 2 i, 8 kb + 4 c + 2 i + 1 of the B operand
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        uint32_t hw, lw;
                        split_bf16(p[rb][c][2 * i], p[rb][c][2 * i + 1], hw, lw);
                        phi[rb][2 * c + i] = hw;
                        plo[rb][2 * c + i] = lw;
                    }
            }
            // ---- PV (O^T += V^T P^T): every V operand used for the RB row blocks
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint4 av = *reinterpret_cast<const uint4*>(&VT[buf][16 * m + n16][8 * kb]);
                const u32x4_t A = {av.x, av.y, av.z, av.w};
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    O[rb][m] = mfma_bf16(A, phi[rb], O[rb][m]);
                    O[rb][m] = mfma_bf16(A, plo[rb], O[rb][m]);
                }
            }
        }
        if (kt + 2 < kt_end) {
            store((kt + 2) % 3);
            if (kt + 3 < kt_end) load(kt + 3);                // in flight during the next step
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
