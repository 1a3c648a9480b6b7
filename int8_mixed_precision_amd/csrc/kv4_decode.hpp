// kv4_decode.hpp -- split-KV decode attention over the paged mixed cache and
// the log-sum-exp merge of its parts.
//
// KV4-RL (arXiv 2610.14448), Section 5.3 and Appendix A.3: the INT4 region and
// the protected (sink + recent, INT8) region are processed independently;
// each part yields a locally normalised output o_r and log-normaliser z_r and
// the parts are merged with z = log sum_r e^{z_r}, o = sum_r e^{z_r - z} o_r
// (eq. A1), with zero weight for empty parts; the same identity merges the
// pieces into which the partition below cuts a region.
//
// Work partition (balanced, persistent, with a dynamic tail): the work of a
// launch is the protected parts of every (sequence b, kv head h) and the
// 32-token tiles of their INT4 regions, in (b, h) order.  The tiles are cut
// into shares: W static shares over the first Ts tiles, balanced together with
// the protected parts so that every wave starts with the same weight, then a
// pool of chunks over the remaining tiles, of decreasing size, that waves take
// from a few atomic counters as they finish, so that waves that run faster
// (older waves on a SIMD, less loaded XCDs) take more.  The run of (b, h) in
// share s writes record b*Hkv + h + s, which is unique because along the tile
// sequence either the head index or the share index grows at every cut; which
// wave runs a share does not change its record.  The runner of the first tile
// of (b, h) stores the first and the last share of (b, h) in a header for the
// merge.
//
// Arithmetic: q stays at its bf16 value; keys and values are reconstructed in
// fp32 registers as Delta*c + m (INT4, eq. 3.3) or s*c (INT8); scores, the
// online softmax (in base 2) and the PV accumulation are fp32.  For INT4 keys
// the per-group affine identity q.k^ = Delta (q.c) + m sum(q) (eq. 5.1) is
// applied per 16-channel slice.
#pragma once

#include "kv4_common.hpp"

namespace kv4 {

constexpr int kPartPad = 4;      // floats after o[d] in a partial: z and padding
constexpr int kTile = 32;        // tokens per INT4 / BF16 unit
// Least weight (in INT4 tiles) a wave is given: fewer waves otherwise.  With
// less work per wave the launch is dominated by the slowest waves (measured
// at the Qwen3-4B batch-64 shape: 67 us at 4,096 waves, 51 us at 2,560).
constexpr int kMinUnits = 20;
constexpr int kMaxWaves = 1 << 16;
constexpr int kPoolCounters = 8;         // atomic counters of the pool
constexpr int kPoolStride = 64;          // uint32 between counters (256 bytes)
constexpr int kPoolMinChunks = 8;
constexpr int kPoolMaxChunks = 1 << 16;
constexpr uint32_t kPoolSixteenths = 3;  // share of the tiles left to the pool, in 1/16

struct DecodeArgs {
    Geo g;
    int layer;
    const uint16_t* q;            // [batch][Hq][d] bf16
    const int32_t* seq_lens;
    const int32_t* slot_ids;
    const int32_t* block_tables;
    int batch, max_ctx;
    int waves;                    // W: waves of the partition (= the grid)
    int prot_units;               // weight of a protected part in tiles: its 32-entry tiles
    int pool_chunks;              // most chunks of the pool (a power of two >= 8), 0 = no pool
    float scale2;                 // sm_scale * log2(e)
    const uint8_t* pages;
    const uint8_t* side;
    float* part;                  // records [batch*Hkv + W + pool_chunks][gqa][d + kPartPad],
                                  // then the protected records [batch*Hkv][gqa][d + kPartPad]
    int2* hdr;                    // [batch*Hkv]: first and last share of the INT4 records
    uint32_t* ctr;                // pool counters, kPoolStride apart (zero at launch)
    void* out;
    int out_dtype;
};

struct Regions {
    int n, sink_end, rec_start, n4, n8;
};

__device__ __forceinline__ Regions regions_of(int n, int S, int R)
{
    Regions r;
    r.n = n;
    r.sink_end = min(S, n);
    r.rec_start = max(S, n - R);
    r.n4 = max(r.rec_start - S, 0);
    r.n8 = r.sink_end + max(n - r.rec_start, 0);
    return r;
}

// Record `slot` (INT4 / BF16 runs) and the protected record of (b, h).
__device__ __forceinline__ float* rec_ptr(const DecodeArgs& a, int64_t slot)
{
    return a.part + slot * a.g.gqa * (int64_t)(a.g.d + kPartPad);
}

__device__ __forceinline__ float* prot_ptr(const DecodeArgs& a, int bh)
{
    return rec_ptr(a, (int64_t)a.batch * a.g.Hkv + a.waves + a.pool_chunks + bh);
}

// Tile range of the INT4 (mixed cache) or BF16 region of a sequence of n
// tokens, and whether it has a protected part.
struct Units {
    int tok_lo, tok_hi;           // token range of the tiled region
    int tile_lo, ntile;           // its tiles
    int prot;                     // 1 if the sequence has a protected part
};

__device__ __forceinline__ Units units_of(const DecodeArgs& a, int n)
{
    Units u;
    if (a.g.kind == KV4_KIND_MIXED) {
        const Regions rg = regions_of(n, a.g.S, a.g.R);
        u.tok_lo = a.g.S;
        u.tok_hi = rg.rec_start;
        u.prot = rg.n8 > 0;
    } else {
        u.tok_lo = 0;
        u.tok_hi = n;
        u.prot = 0;
    }
    u.tile_lo = u.tok_lo / kTile;
    u.ntile = u.tok_hi > u.tok_lo ? (u.tok_hi + kTile - 1) / kTile - u.tile_lo : 0;
    return u;
}

__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b)
{
    return clampi(a.seq_lens[b], 0, a.max_ctx);
}

__device__ __forceinline__ int wave_sum_i32(int x)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return __builtin_amdgcn_readfirstlane(x);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_scan_i32(int x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// floor(w X / W) for w <= W <= 2^16 without 64-bit division.
__device__ __forceinline__ uint32_t share(uint32_t w, uint32_t X, uint32_t W)
{
    const uint32_t q = X / W, r = X - q * W;
    return w * q + (w * r) / W;
}

// s_setprio takes its level as an immediate.
__device__ __forceinline__ void set_wave_prio(int p)
{
    if (p <= 0) __builtin_amdgcn_s_setprio(0);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(3);
}

// Wave priority by progress through the static share.  The instruction
// arbiter of a SIMD favours older waves, so at equal priority the waves
// dispatched first run ahead (about 20% faster with four per SIMD) and finish
// early, while the youngest set the end of the launch.  A wave therefore runs
// at a priority that falls as its share drains: 3 while more than half of it
// is left, 2 above a quarter, 1 above an eighth, then 0 (and 0 in pool
// chunks).  A wave that falls behind keeps the higher level until it catches
// up, so the waves of a SIMD finish close together.  Priority only orders
// instruction issue; results do not depend on it.
struct Pace {
    int share_len;                // tiles of the wave's static share (0: a pool chunk)
    int rem_after;                // tiles of the share after the current run
    int level;                    // current priority
    // at the start of a tile with `left` tiles of the run to go (this one included)
    __device__ __forceinline__ void tile(int left)
    {
        const int rem = rem_after + left;
        const int lv = share_len <= 0 ? 0
                     : 2 * rem > share_len ? 3 : 4 * rem > share_len ? 2 : 8 * rem > share_len ? 1 : 0;
        if (lv != level) {
            set_wave_prio(lv);
            level = lv;
        }
    }
};

// The partition of one launch.  T4 tiles in (b, h, tile) order and P
// protected parts in (b, h) order, of weight U8 tiles each; W waves.
//  - Pool: Tp = floor(3 T4 / 16) tiles in Cd chunks, Cd the largest power of
//    two <= pool_chunks with 2 Cd <= Tp (no pool when that is below 8).  With
//    A = Tp - Cd, chunk c covers pool tiles [g(c), g(c+1)), g(c) = c + A -
//    floor(A (Cd - c)^2 / Cd^2): at least one tile each, sizes falling
//    linearly from about 2 Tp / Cd to 1.
//  - Static shares over the other Ts = T4 - Tp tiles: wave w runs protected
//    parts [pbeg(w), pbeg(w+1)), pbeg(w) = floor(w P / W), and tiles [tbeg(w),
//    tbeg(w+1)), tbeg(w) = floor(w (Ts + U8 P) / W) - U8 pbeg(w), so that every
//    wave starts with the same weight and at least one tile.  When tiles are
//    too few for that, they are split evenly over the first Wt = min(W, Ts)
//    waves instead.
//  - Shares: s < S0 (S0 = W, or Wt) is static share s; s = S0 + c is chunk c,
//    tiles [Ts + g(c), Ts + g(c+1)).  Consecutive shares cover consecutive
//    tiles and none is empty, so the shares running tiles of one (b, h) are
//    consecutive and each runs some of them.
// The host bounds T4 + U8 P below 2^30.
struct Plan {
    uint32_t T4;                  // INT4 / BF16 tiles
    uint32_t P;                   // protected parts
    uint32_t U8;                  // weight of a protected part
    uint32_t W;                   // waves in use
    uint32_t Wt;                  // waves running tiles when not balanced
    bool balanced;
    uint32_t Ts;                  // tiles of the static shares
    uint32_t Cd;                  // pool chunks (0 = no pool)
    uint32_t A;                   // pool tiles - Cd
    uint32_t lg2;                 // 2 log2(Cd)
    uint32_t S0;                  // static shares
    __device__ uint32_t pbeg(uint32_t w) const { return share(w, P, W); }
    __device__ uint32_t tbeg(uint32_t w) const
    {
        return balanced ? share(w, Ts + U8 * P, W) - U8 * pbeg(w)
                        : share(min(w, Wt), Ts, Wt);
    }
    __device__ uint32_t cbeg(uint32_t c) const
    {
        const uint64_t r = Cd - c;
        return Ts + c + A - (uint32_t)(((uint64_t)A * r * r) >> lg2);
    }
    __device__ uint32_t shares() const { return S0 + Cd; }
    __device__ uint32_t sbeg(uint32_t s) const { return s <= S0 ? tbeg(s) : cbeg(s - S0); }
    // the share holding tile x (sbeg(s_lo) <= x < T4)
    __device__ uint32_t share_of_tile(uint32_t x, uint32_t s_lo) const
    {
        uint32_t lo = s_lo, hi = shares() - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (sbeg(mid) <= x) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    }
};

__device__ __forceinline__ Plan make_plan(const DecodeArgs& a)
{
    const int lane = threadIdx.x & 63;
    int t = 0, p = 0;
    // the lengths of 256 sequences per pass, their loads issued together
    for (int b0 = 0; b0 < a.batch; b0 += 4 * 64) {
        int n[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int b = b0 + 64 * k + lane;
            n[k] = b < a.batch ? seq_len(a, b) : 0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (b0 + 64 * k + lane < a.batch) {
                const Units u = units_of(a, n[k]);
                t += u.ntile;
                p += u.prot;
            }
        }
    }
    Plan pl;
    pl.T4 = (uint32_t)wave_sum_i32(t) * a.g.Hkv;
    pl.P = (uint32_t)wave_sum_i32(p) * a.g.Hkv;
    pl.U8 = (uint32_t)a.prot_units;
    const uint32_t weight = pl.T4 + pl.U8 * pl.P;
    pl.W = min((uint32_t)a.waves, max(1u, (weight + kMinUnits - 1) / kMinUnits));
    // pool: the largest power of two <= pool_chunks with two tiles per chunk
    const uint32_t tp = (pl.T4 >> 4) * kPoolSixteenths + (((pl.T4 & 15u) * kPoolSixteenths) >> 4);
    uint32_t cd = (uint32_t)a.pool_chunks;
    if (cd > 0 && 2 * cd > tp) cd = tp >= 2 ? 1u << (31 - __builtin_clz(tp / 2)) : 0u;
    if (cd < (uint32_t)kPoolMinChunks) cd = 0;
    pl.Cd = cd;
    pl.A = cd ? tp - cd : 0;
    pl.lg2 = cd ? 2 * (uint32_t)__builtin_ctz(cd) : 0;
    pl.Ts = pl.T4 - (cd ? tp : 0);
    // monotone iff every wave's share covers its protected parts
    const uint32_t pmax = (pl.P + pl.W - 1) / pl.W;
    pl.balanced = (pl.Ts + pl.U8 * pl.P) / pl.W >= pl.U8 * pmax + 1;
    pl.Wt = max(1u, min(pl.W, pl.Ts));
    pl.S0 = pl.balanced ? pl.W : pl.Wt;
    return pl;
}

// First sequence b whose cumulative count (of `field` times Hkv) exceeds x:
// returns b and the count before it in C.
template <class F>
__device__ __forceinline__ int locate_seq(const DecodeArgs& a, uint32_t x, F&& field, uint32_t& C)
{
    const int lane = threadIdx.x & 63;
    C = 0;
    // 256 sequences per pass, their lengths loaded together
    for (int b0 = 0; b0 < a.batch; b0 += 4 * 64) {
        int n[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int bb = b0 + 64 * k + lane;
            n[k] = bb < a.batch ? seq_len(a, bb) : 0;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int bb = b0 + 64 * k + lane;
            const int s = bb < a.batch ? a.g.Hkv * field(units_of(a, n[k])) : 0;
            const int incl = wave_scan_i32(s);
            const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
            if (C + tot > x) {
                const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(__ballot(C + (uint32_t)incl > x)));
                C += __builtin_amdgcn_readlane(incl - s, l);
                return b0 + 64 * k + l;
            }
            C += tot;
        }
    }
    return a.batch;
}

// Wave w's protected parts: prot(b, h) for each.
template <class Prot>
__device__ __forceinline__ void walk_prot(const DecodeArgs& a, const Plan& pl, uint32_t w, Prot&& prot)
{
    uint32_t p = pl.pbeg(w);
    const uint32_t pe = pl.pbeg(w + 1);
    if (p >= pe) return;
    uint32_t C;
    int b = locate_seq(a, p, [](const Units& u) { return u.prot; }, C);
    int h = (int)(p - C);
    for (; p < pe; ++p) {
        prot(b, h);
        if (++h == a.g.Hkv) {                   // next sequence with a protected part
            h = 0;
            do {
                if (++b >= a.batch) return;
            } while (!units_of(a, seq_len(a, b)).prot);
        }
    }
}

// The next pool chunk for this wave, as a share index (shares() when the pool
// is used up).  Chunk c belongs to counter c % 8 and is its ticket c / 8, so
// each counter hands out its chunks largest first.  A wave draws on its own
// counter j; when that one is used up it reads all eight at once and moves on
// to the next open one after j.  A counter that returned a ticket past its
// chunks is used up for good, so a wave leaves after at most eight misses, and
// a chunk is never left untaken while a wave still looks for work.
__device__ __forceinline__ uint32_t take_chunk(const DecodeArgs& a, const Plan& pl, uint32_t& j)
{
    if (pl.Cd == 0) return pl.shares();
    const int lane = threadIdx.x & 63;
    const uint32_t per = pl.Cd / kPoolCounters;
    uint32_t dead = 0;
    for (;;) {
        uint32_t n = 0;
        if (lane == 0) n = atomicAdd(a.ctr + kPoolStride * j, 1u);
        n = __builtin_amdgcn_readfirstlane(n);
        if (n < per) return pl.S0 + j + kPoolCounters * n;
        dead |= 1u << j;
        const uint32_t v = lane < kPoolCounters
            ? __hip_atomic_load(a.ctr + kPoolStride * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
            : per;
        const uint32_t open = (uint32_t)__ballot(v < per) & ~dead & 0xFFu;
        if (open == 0) return pl.shares();
        const uint32_t k = (j + 1) & 7u;
        const uint32_t rot = ((open >> k) | (open << (8u - k))) & 0xFFu;
        j = (k + (uint32_t)__builtin_ctz(rot)) & 7u;
    }
}

// Wave w's tiles: its static share, then pool chunks while there are any.
// run(b, h, tok_lo, tok_hi, rec, pace) for each maximal run of tiles of one
// (b, h) in a share s (token range clipped to the region; rec = record
// b*Hkv + h + s; pace set for the run).
// The runner of the first tile of (b, h) stores the first and the last share
// of (b, h) in the header.
template <class Run>
__device__ __forceinline__ void walk_tiles(const DecodeArgs& a, const Plan& pl, uint32_t w, Pace& pace,
                                           Run&& run)
{
    const int lane = threadIdx.x & 63;
    const int Hkv = a.g.Hkv;
    uint32_t j = w % kPoolCounters;
    uint32_t s = w < pl.S0 ? w : take_chunk(a, pl, j);
    while (s < pl.shares()) {
        uint32_t x = pl.sbeg(s);
        const uint32_t xe = pl.sbeg(s + 1);
        if (x >= xe) {                          // an empty share (no INT4 tiles at all):
            s = take_chunk(a, pl, j);           // nothing to locate, and no sequence index
            continue;                           // past the batch is ever formed
        }
        pace.share_len = s < pl.S0 ? (int)(xe - x) : 0;
        uint32_t C;
        int b = locate_seq(a, x, [](const Units& u) { return u.ntile; }, C);
        Units u = units_of(a, seq_len(a, b));
        while (x < xe) {
            const uint32_t r = x - C;
            const int h = (int)(r / (uint32_t)u.ntile);
            const int t0 = (int)(r - (uint32_t)h * u.ntile);
            const uint32_t base = C + (uint32_t)h * u.ntile;
            const int t1 = (int)min((uint32_t)u.ntile, xe - base);
            const int bh = b * Hkv + h;
            if (t0 == 0 && lane == 0) a.hdr[bh] = make_int2((int)s, (int)pl.share_of_tile(base + u.ntile - 1, s));
            pace.rem_after = (int)(xe - (base + t1));
            run(b, h, max(kTile * (u.tile_lo + t0), u.tok_lo), min(kTile * (u.tile_lo + t1), u.tok_hi),
                rec_ptr(a, (int64_t)bh + s), pace);
            x = base + t1;
            if (x < xe && x >= C + (uint32_t)Hkv * u.ntile) {  // next sequence with tiles
                C += (uint32_t)Hkv * u.ntile;
                do {
                    if (++b >= a.batch) break;
                    u = units_of(a, seq_len(a, b));
                } while (u.ntile == 0);
                if (b >= a.batch) break;
            }
        }
        s = take_chunk(a, pl, j);
    }
}

// The whole partition for wave w = blockIdx.x: its protected parts (at the
// top priority: they come first in a share), then its tiles (two separate
// loops, so that the vector-ALU and the matrix-core parts never share a loop
// body's registers).
template <class Prot, class Run>
__device__ __forceinline__ void walk_units(const DecodeArgs& a, Prot&& prot, Run&& run)
{
    const Plan pl = make_plan(a);
    const uint32_t w = blockIdx.x;
    if (w >= pl.W) return;
    Pace pace{0, 0, 3};
    set_wave_prio(3);
    walk_prot(a, pl, w, prot);
    walk_tiles(a, pl, w, pace, run);
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

// Online-softmax state of one wave for GQA query heads.
template <int GQA>
struct Online {
    float m[GQA], l[GQA], o[GQA][2];
    __device__ void init()
    {
#pragma unroll
        for (int j = 0; j < GQA; ++j) { m[j] = -INFINITY; l[j] = 0.f; o[j][0] = o[j][1] = 0.f; }
    }
};

// DPP move inside a 16-lane row (every lane active, every source in the row).
template <int CTRL>
__device__ __forceinline__ float lane_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 8 lanes 8k .. 8k+7: the quad swaps, then the half-row mirror
// (lane i reads lane 7 - i), which after the quad steps adds the other quad's
// sum -- the same additions in the same order as a butterfly over lane bits
// 0, 1, 2.
__device__ __forceinline__ float lanes8_sum(float x)
{
    x += lane_mov<0xB1>(x);                      // quad_perm [1,0,3,2]
    x += lane_mov<0x4E>(x);                      // quad_perm [2,3,0,1]
    return x + lane_mov<0x141>(x);               // row_half_mirror
}

// Maximum over the 8 lanes l, l ^ 8, ..., l ^ 56 (row rotation by 8, then the
// row swaps of v_permlane16_swap and v_permlane32_swap).
__device__ __forceinline__ float lanes_e_max(float x)
{
    x = fmaxf(x, lane_mov<0x128>(x));            // row_ror 8
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Chunk step shared by all paths: lanes (e = lane/8, sl = lane%8) hold the
// partial score of token e over their 16-channel slice.  Reduces the scores,
// updates the running max/sum and publishes the probabilities P[e][j] in LDS.
template <int GQA>
__device__ __forceinline__ void softmax_chunk(Online<GQA>& st, float (&s)[GQA], bool valid,
                                              float scale2, float (*P)[GQA], float (&alpha)[GQA])
{
    const int lane = threadIdx.x, e = lane >> 3, sl = lane & 7;
#pragma unroll
    for (int j = 0; j < GQA; ++j) {
        float x = lanes8_sum(s[j]);
        x = valid ? x * scale2 : -INFINITY;
        float mx = lanes_e_max(x);
        float mn = fmaxf(st.m[j], mx);            // finite: the chunk has a valid token
        alpha[j] = exp2f(st.m[j] - mn);
        float p = exp2f(x - mn);
        st.m[j] = mn;
        st.l[j] = st.l[j] * alpha[j] + (sl == 0 ? p : 0.f);
        if (sl == 0) P[e][j] = p;
    }
}

template <int GQA>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, Online<GQA>& st, float* rec)
{
    const int lane = threadIdx.x;
#pragma unroll
    for (int j = 0; j < GQA; ++j) {
        float l = wave_sum(st.l[j]);
        float inv = 1.0f / l;
        float* dst = rec + j * (a.g.d + kPartPad);
        *reinterpret_cast<float2*>(dst + 2 * lane) = make_float2(st.o[j][0] * inv, st.o[j][1] * inv);
        if (lane == 0) dst[a.g.d] = st.m[j] + log2f(l);
    }
}

// q slice for QK (channels 16*sl .. +15) and its sum, for GQA heads.
template <int GQA>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int b, int h, float (&qk)[GQA][16],
                                       float (&sq)[GQA])
{
    const int sl = threadIdx.x & 7;
#pragma unroll
    for (int j = 0; j < GQA; ++j) {
        const uint16_t* qr = a.q + ((int64_t)b * a.g.Hq + h * GQA + j) * a.g.d + 16 * sl;
        uint4 u0 = *reinterpret_cast<const uint4*>(qr);
        uint4 u1 = *reinterpret_cast<const uint4*>(qr + 8);
        uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qk[j][2 * i] = bf16_lo(w[i]);
            qk[j][2 * i + 1] = bf16_hi(w[i]);
        }
        if (a.g.rot) {
            // query into the keys' basis; channel bits 4-6 are lane bits 0-2
            wht_local(qk[j]);
            wht_lanes(qk[j], 1);
            wht_lanes(qk[j], 2);
            wht_lanes(qk[j], 4);
            wht_scale(qk[j]);
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += qk[j][2 * i] + qk[j][2 * i + 1];
        sq[j] = s;
    }
}

// ---------------------------------------------------------------------------
// Mixed cache, vector-ALU path: one wave runs INT4 positions [t_begin, t_end)
// of (sequence b, kv head h) (prot = false), or the protected (sink + recent)
// part read from the INT8 ring (prot = true), into record `rec`.
// ---------------------------------------------------------------------------
template <int GQA>
__device__ __forceinline__ void valu_item_kv4(const DecodeArgs& a, int b, int h, bool prot,
                                              int t_begin, int t_end, float* rec)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x, e = lane >> 3, sl = lane & 7;
    const int n = seq_len(a, b);
    const Regions rg = regions_of(n, g.S, g.R);
    if (prot) {
        t_begin = 0;
        t_end = rg.n8;
    }
    if (t_end <= t_begin) return;

    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    __shared__ float P[8][GQA];
    float qk[GQA][16], sq[GQA];
    load_q<GQA>(a, b, h, qk, sq);
    Online<GQA> st;
    st.init();
    float alpha[GQA];

    if (!prot) {
        const uint8_t* lbase = a.pages + (int64_t)a.layer * g.layer_pages;
        const int gk = (16 * sl) / g.G;          // K group of this lane's slice
        const int gv = (2 * lane) / g.G;         // V group of this lane's channels
        for (int hp = t_begin / kHalf; hp <= (t_end - 1) / kHalf; ++hp) {
            const int page = clampi(bt[hp / 2], 0, g.num_pages - 1);
            const uint8_t* pb = lbase + ((int64_t)page * g.Hkv + h) * g.pb;
            const int half = hp & 1;
            const int tok = hp * kHalf + e;
            const bool valid = tok >= t_begin && tok < t_end;
            const int tp = tok % kPage;
            // ---- scores
            const uint8_t* krow = pb + g.off_kc + tp * (g.d / 2);
            uint2 kc = make_uint2(*reinterpret_cast<const uint32_t*>(krow + 4 * kpos(2 * sl)),
                                  *reinterpret_cast<const uint32_t*>(krow + 4 * kpos(2 * sl + 1)));
            const uint16_t* kdm = reinterpret_cast<const uint16_t*>(pb + g.off_kdm) + tp * 2 * g.ng + 2 * gk;
            float D = half_bits_to_float(kdm[0]);
            float M = half_bits_to_float(kdm[1]);
            float s[GQA];
#pragma unroll
            for (int j = 0; j < GQA; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    uint32_t byte = ((i < 4 ? kc.x : kc.y) >> (8 * (i & 3))) & 0xFFu;
                    acc = fmaf(qk[j][2 * i], (float)(byte & 0xFu), acc);
                    acc = fmaf(qk[j][2 * i + 1], (float)(byte >> 4), acc);
                }
                s[j] = fmaf(D, acc, M * sq[j]);
            }
            softmax_chunk<GQA>(st, s, valid, a.scale2, P, alpha);
            __syncthreads();
            // ---- values
            const uint32_t* vw = reinterpret_cast<const uint32_t*>(pb + g.off_vc) + half * g.d;
            uint32_t w0 = vw[vpos(2 * lane)], w1 = vw[vpos(2 * lane + 1)];
            uint4 dv = *reinterpret_cast<const uint4*>(pb + g.off_vd + 2 * (gv * kPage + half * kHalf));
            uint32_t dvw[4] = {dv.x, dv.y, dv.z, dv.w};
            const uint16_t* vmt = reinterpret_cast<const uint16_t*>(pb + g.off_vm) + half * kHalf * g.ng + gv;
#pragma unroll
            for (int j = 0; j < GQA; ++j) { st.o[j][0] *= alpha[j]; st.o[j][1] *= alpha[j]; }
#pragma unroll
            for (int ee = 0; ee < kHalf; ++ee) {
                int t2 = hp * kHalf + ee;
                if (t2 < t_begin || t2 >= t_end) continue;      // uniform across the wave
                float Dv = half_bits_to_float((dvw[ee >> 1] >> (16 * (ee & 1))) & 0xFFFFu);
                float Mv = half_bits_to_float(vmt[ee * g.ng]);
                float x0 = fmaf(Dv, (float)((w0 >> (4 * ee)) & 0xFu), Mv);
                float x1 = fmaf(Dv, (float)((w1 >> (4 * ee)) & 0xFu), Mv);
#pragma unroll
                for (int j = 0; j < GQA; ++j) {
                    float p = P[ee][j];
                    st.o[j][0] = fmaf(p, x0, st.o[j][0]);
                    st.o[j][1] = fmaf(p, x1, st.o[j][1]);
                }
            }
            __syncthreads();
        }
    } else {
        // The protected positions of an n-token context occupy ring entries
        // [0, n8) (sinks, then the recent window in ring order); attention is
        // over the set, so the entries are walked in ring order.
        const uint8_t* ring = a.side + (int64_t)a.layer * g.layer_side + ((int64_t)slot * g.Hkv + h) * g.rb;
        const uint8_t* vr = ring + (int64_t)g.SR32 * g.d;
        const uint16_t* ksc = reinterpret_cast<const uint16_t*>(ring + (int64_t)2 * g.SR32 * g.d);
        const uint16_t* vsc = ksc + g.SR32;
        for (int c0 = 0; c0 < t_end; c0 += kHalf) {
            const int ent = c0 + e;                  // < SR32: the ring is padded to 32 entries
            const bool valid = ent < t_end;
            uint4 kc = *reinterpret_cast<const uint4*>(ring + (int64_t)ent * g.d + 16 * sl);
            float sk = half_bits_to_float(ksc[ent]);
            // the chunk's value codes (8 entries of this lane's two channels) and scales
            const uint2 va = *reinterpret_cast<const uint2*>(vr + ring_vbyte(c0, 2 * lane));
            const uint2 vb = *reinterpret_cast<const uint2*>(vr + ring_vbyte(c0, 2 * lane + 1));
            const uint4 svw = *reinterpret_cast<const uint4*>(vsc + c0);
            uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w};
            float s[GQA];
#pragma unroll
            for (int j = 0; j < GQA; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    int v8 = (int)(int8_t)((kw[c >> 2] >> (8 * (c & 3))) & 0xFFu);
                    acc = fmaf(qk[j][c], (float)v8, acc);
                }
                s[j] = sk * acc;
            }
            softmax_chunk<GQA>(st, s, valid, a.scale2, P, alpha);
            __syncthreads();
#pragma unroll
            for (int j = 0; j < GQA; ++j) { st.o[j][0] *= alpha[j]; st.o[j][1] *= alpha[j]; }
            const uint32_t svs[4] = {svw.x, svw.y, svw.z, svw.w};
#pragma unroll
            for (int ee = 0; ee < kHalf; ++ee) {
                // entries past the end hold garbage: select, do not multiply
                const bool ok = c0 + ee < t_end;
                const float sv = half_bits_to_float((svs[ee >> 1] >> (16 * (ee & 1))) & 0xFFFFu);
                const uint32_t wa = ee < 4 ? va.x : va.y, wb = ee < 4 ? vb.x : vb.y;
                const float x0 = ok ? sv * (float)(int)(int8_t)((wa >> (8 * (ee & 3))) & 0xFFu) : 0.f;
                const float x1 = ok ? sv * (float)(int)(int8_t)((wb >> (8 * (ee & 3))) & 0xFFu) : 0.f;
#pragma unroll
                for (int j = 0; j < GQA; ++j) {
                    float p = P[ee][j];
                    st.o[j][0] = fmaf(p, x0, st.o[j][0]);
                    st.o[j][1] = fmaf(p, x1, st.o[j][1]);
                }
            }
            __syncthreads();
        }
    }
    write_partial<GQA>(a, st, rec);
}

// One wave per workgroup; grid = W.
template <int GQA>
__global__ __launch_bounds__(64) void decode_valu_kv4_kernel(DecodeArgs a)
{
    walk_units(a, [&](int b, int h) { valu_item_kv4<GQA>(a, b, h, true, 0, 0, prot_ptr(a, b * a.g.Hkv + h)); },
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   pace.tile((hi + kTile - 1) / kTile - lo / kTile);
                   valu_item_kv4<GQA>(a, b, h, false, lo, hi, rec);
               });
}

// ---------------------------------------------------------------------------
// Integer decode path (KV4_FLAG_INT_PATH; KV4-RL Appendix A.3, "Integer
// decode path" and "Protected path and reconstruction").  The layout of
// valu_item_kv4: for the scores lanes (e = lane/8, sl = lane%8) hold token e of
// an 8-token chunk and channels 16 sl .. 16 sl + 15; for the values lane l
// holds channels 2l and 2l + 1 of every token of the chunk.
// ---------------------------------------------------------------------------

// Blocks whose largest w = p Delta_V is at most 2^-100 carry all-zero 8-bit
// codes: their weight is below 2^-100 of the block holding the maximum
// probability (p = 1, or 2^48 with the matrix-core item's scaling), and
// 255 / w would leave the binary32 range.
constexpr float kTinyW = 0x1p-100f;

__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
           ((uint32_t)(d & 0xFF) << 24);
}

// INT8 query of GQA heads in this lane's 16-channel slice: codes four per word
// in channel order (qn, against INT8 key bytes) and as the even and odd
// channels of each 8-channel half (qe, qo, against the low and high nibbles of
// the INT4 key bytes); the slice's code sum and the head's scale.
template <int GQA>
struct QInt {
    uint32_t qn[GQA][4], qe[GQA][2], qo[GQA][2];
    int qsum[GQA];
    float sq[GQA];
};

template <int GQA>
__device__ __forceinline__ void load_q_int(const DecodeArgs& a, int b, int h, QInt<GQA>& Q)
{
    float qk[GQA][16], unused[GQA];
    load_q<GQA>(a, b, h, qk, unused);            // bf16 values, rotated when keys are
#pragma unroll
    for (int j = 0; j < GQA; ++j) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(qk[j][i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));  // the head's 8 slices
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        amax = fmaxf(amax, __shfl_xor(amax, 4));
        const uint16_t sb = plus_zero16(f32_to_f16_bits(__fdiv_rn(amax, 127.0f)));
        const float S = half_bits_to_float(sb);
        int c[16], sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            c[i] = int8_code(qk[j][i], S, sb);
            sum += c[i];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) Q.qn[j][k] = pack_i8x4(c[4 * k], c[4 * k + 1], c[4 * k + 2], c[4 * k + 3]);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            Q.qe[j][k] = pack_i8x4(c[8 * k], c[8 * k + 2], c[8 * k + 4], c[8 * k + 6]);
            Q.qo[j][k] = pack_i8x4(c[8 * k + 1], c[8 * k + 3], c[8 * k + 5], c[8 * k + 7]);
        }
        Q.qsum[j] = sum;
        Q.sq[j] = S;
    }
}

// One wave runs INT4 positions [t_begin, t_end) of (sequence b, kv head h)
// (prot = false), or the protected part read from the INT8 ring (prot = true),
// into record `rec`.
template <int GQA>
__device__ __forceinline__ void int_item_kv4(const DecodeArgs& a, int b, int h, bool prot,
                                             int t_begin, int t_end, float* rec)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x, e = lane >> 3, sl = lane & 7;
    const int n = seq_len(a, b);
    const Regions rg = regions_of(n, g.S, g.R);
    if (prot) {
        t_begin = 0;
        t_end = rg.n8;
    }
    if (t_end <= t_begin) return;

    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    __shared__ float P[8][GQA];
    QInt<GQA> Q;
    load_q_int<GQA>(a, b, h, Q);
    Online<GQA> st;
    st.init();
    float alpha[GQA];

    if (!prot) {
        const uint8_t* lbase = a.pages + (int64_t)a.layer * g.layer_pages;
        const int gk = (16 * sl) / g.G;          // K group of this lane's slice
        const int gv = (2 * lane) / g.G;         // V group of this lane's channels
        // one chunk's loads (token e's K codes and (Delta, m) for the scores;
        // channels 2 lane, 2 lane + 1 of all 8 tokens for the values), issued a
        // chunk ahead of their use
        struct Ld {
            uint32_t kx, ky, kdm, w0, w1;
            uint4 dv;
            uint32_t vm[kHalf];
        };
        auto load = [&](int hp) {
            Ld L;
            const int page = clampi(bt[hp / 2], 0, g.num_pages - 1);
            const uint8_t* pb = lbase + ((int64_t)page * g.Hkv + h) * g.pb;
            const int half = hp & 1;
            const int tp = (hp * kHalf + e) % kPage;
            const uint8_t* krow = pb + g.off_kc + tp * (g.d / 2);
            L.kx = *reinterpret_cast<const uint32_t*>(krow + 4 * kpos(2 * sl));
            L.ky = *reinterpret_cast<const uint32_t*>(krow + 4 * kpos(2 * sl + 1));
            L.kdm = *reinterpret_cast<const uint32_t*>(pb + g.off_kdm + 4 * (tp * g.ng + gk));
            const uint32_t* vw = reinterpret_cast<const uint32_t*>(pb + g.off_vc) + half * g.d;
            L.w0 = vw[vpos(2 * lane)];
            L.w1 = vw[vpos(2 * lane + 1)];
            L.dv = *reinterpret_cast<const uint4*>(pb + g.off_vd + 2 * (gv * kPage + half * kHalf));
            const uint16_t* vmt = reinterpret_cast<const uint16_t*>(pb + g.off_vm) + half * kHalf * g.ng + gv;
#pragma unroll
            for (int ee = 0; ee < kHalf; ++ee) L.vm[ee] = vmt[ee * g.ng];
            return L;
        };
        const int hp_last = (t_end - 1) / kHalf;
        Ld cur = load(t_begin / kHalf);
        for (int hp = t_begin / kHalf; hp <= hp_last; ++hp) {
            const Ld nxt = load(min(hp + 1, hp_last));      // the last chunk reloads itself (cache hits)
            const int tok = hp * kHalf + e;
            const bool valid = tok >= t_begin && tok < t_end;
            // ---- scores: integer dot products of the query codes with the
            // widened nibbles, then the group's Delta and m
            const uint32_t kxl = cur.kx & 0x0F0F0F0Fu, kxh = (cur.kx >> 4) & 0x0F0F0F0Fu;
            const uint32_t kyl = cur.ky & 0x0F0F0F0Fu, kyh = (cur.ky >> 4) & 0x0F0F0F0Fu;
            const float D = half_bits_to_float(cur.kdm & 0xFFFFu);
            const float M = half_bits_to_float(cur.kdm >> 16);
            float s[GQA];
#pragma unroll
            for (int j = 0; j < GQA; ++j) {
                int I = __builtin_amdgcn_sdot4((int)Q.qe[j][0], (int)kxl, 0, false);
                I = __builtin_amdgcn_sdot4((int)Q.qo[j][0], (int)kxh, I, false);
                I = __builtin_amdgcn_sdot4((int)Q.qe[j][1], (int)kyl, I, false);
                I = __builtin_amdgcn_sdot4((int)Q.qo[j][1], (int)kyh, I, false);
                s[j] = fmaf(D, (float)I, M * (float)Q.qsum[j]) * Q.sq[j];
            }
            // one-wave workgroup: LDS operations of the wave run in order, so the
            // probability exchange needs no memory fence (which would also wait
            // for the prefetched loads)
            softmax_chunk<GQA>(st, s, valid, a.scale2, P, alpha);
            __builtin_amdgcn_wave_barrier();
            // ---- values: per head, the 8-bit operand of w = p Delta^v over the
            // chunk's tokens, an integer dot product with the value codes, and
            // the offsets' term
            const uint32_t w0l = cur.w0 & 0x0F0F0F0Fu, w0h = (cur.w0 >> 4) & 0x0F0F0F0Fu;   // tokens 0,2,4,6 / 1,3,5,7
            const uint32_t w1l = cur.w1 & 0x0F0F0F0Fu, w1h = (cur.w1 >> 4) & 0x0F0F0F0Fu;
            const uint32_t dvw[4] = {cur.dv.x, cur.dv.y, cur.dv.z, cur.dv.w};
            float Dv[kHalf], Mv[kHalf];
            bool ok[kHalf];
#pragma unroll
            for (int ee = 0; ee < kHalf; ++ee) {
                const int t2 = hp * kHalf + ee;
                ok[ee] = t2 >= t_begin && t2 < t_end;
                Dv[ee] = half_bits_to_float((dvw[ee >> 1] >> (16 * (ee & 1))) & 0xFFFFu);
                Mv[ee] = half_bits_to_float(cur.vm[ee]);
            }
#pragma unroll
            for (int j = 0; j < GQA; ++j) {
                // tokens outside the run may hold garbage metadata: select
                float w[kHalf], wmax = 0.f, off = 0.f;
#pragma unroll
                for (int ee = 0; ee < kHalf; ++ee) {
                    const float p = P[ee][j];
                    w[ee] = ok[ee] ? p * Dv[ee] : 0.f;
                    wmax = fmaxf(wmax, w[ee]);
                    off += ok[ee] ? p * Mv[ee] : 0.f;
                }
                int u[kHalf];
                const float r = wmax > kTinyW ? 255.0f * __builtin_amdgcn_rcpf(wmax) : 0.f;
#pragma unroll
                for (int ee = 0; ee < kHalf; ++ee) u[ee] = (int)fminf(rintf(w[ee] * r), 255.0f);
                const uint32_t ue = pack_i8x4(u[0], u[2], u[4], u[6]);
                const uint32_t uo = pack_i8x4(u[1], u[3], u[5], u[7]);
                const float sigma = wmax * (1.0f / 255.0f);
                const uint32_t i0 = __builtin_amdgcn_udot4(uo, w0h, __builtin_amdgcn_udot4(ue, w0l, 0u, false), false);
                const uint32_t i1 = __builtin_amdgcn_udot4(uo, w1h, __builtin_amdgcn_udot4(ue, w1l, 0u, false), false);
                st.o[j][0] = fmaf(st.o[j][0], alpha[j], fmaf(sigma, (float)i0, off));
                st.o[j][1] = fmaf(st.o[j][1], alpha[j], fmaf(sigma, (float)i1, off));
            }
            __builtin_amdgcn_wave_barrier();
            cur = nxt;
        }
    } else {
        // protected positions: ring entries [0, n8) in ring order; integer QK
        // against the INT8 keys, binary32 PV with the dequantized INT8 values
        const uint8_t* ring = a.side + (int64_t)a.layer * g.layer_side + ((int64_t)slot * g.Hkv + h) * g.rb;
        const uint8_t* vr = ring + (int64_t)g.SR32 * g.d;
        const uint16_t* ksc = reinterpret_cast<const uint16_t*>(ring + (int64_t)2 * g.SR32 * g.d);
        const uint16_t* vsc = ksc + g.SR32;
        for (int c0 = 0; c0 < t_end; c0 += kHalf) {
            const int ent = c0 + e;                  // < SR32: the ring is padded to 32 entries
            const bool valid = ent < t_end;
            const uint4 kc = *reinterpret_cast<const uint4*>(ring + (int64_t)ent * g.d + 16 * sl);
            const float sk = half_bits_to_float(ksc[ent]);
            const uint2 va = *reinterpret_cast<const uint2*>(vr + ring_vbyte(c0, 2 * lane));
            const uint2 vb = *reinterpret_cast<const uint2*>(vr + ring_vbyte(c0, 2 * lane + 1));
            const uint4 svw = *reinterpret_cast<const uint4*>(vsc + c0);
            float s[GQA];
#pragma unroll
            for (int j = 0; j < GQA; ++j) {
                int I = __builtin_amdgcn_sdot4((int)Q.qn[j][0], (int)kc.x, 0, false);
                I = __builtin_amdgcn_sdot4((int)Q.qn[j][1], (int)kc.y, I, false);
                I = __builtin_amdgcn_sdot4((int)Q.qn[j][2], (int)kc.z, I, false);
                I = __builtin_amdgcn_sdot4((int)Q.qn[j][3], (int)kc.w, I, false);
                s[j] = sk * (float)I * Q.sq[j];
            }
            softmax_chunk<GQA>(st, s, valid, a.scale2, P, alpha);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int j = 0; j < GQA; ++j) { st.o[j][0] *= alpha[j]; st.o[j][1] *= alpha[j]; }
            const uint32_t svs[4] = {svw.x, svw.y, svw.z, svw.w};
#pragma unroll
            for (int ee = 0; ee < kHalf; ++ee) {
                // entries past the end hold garbage: select, do not multiply
                const bool okk = c0 + ee < t_end;
                const float sv = half_bits_to_float((svs[ee >> 1] >> (16 * (ee & 1))) & 0xFFFFu);
                const uint32_t wa = ee < 4 ? va.x : va.y, wb = ee < 4 ? vb.x : vb.y;
                const float x0 = okk ? sv * (float)(int)(int8_t)((wa >> (8 * (ee & 3))) & 0xFFu) : 0.f;
                const float x1 = okk ? sv * (float)(int)(int8_t)((wb >> (8 * (ee & 3))) & 0xFFu) : 0.f;
#pragma unroll
                for (int j = 0; j < GQA; ++j) {
                    const float p = P[ee][j];
                    st.o[j][0] = fmaf(p, x0, st.o[j][0]);
                    st.o[j][1] = fmaf(p, x1, st.o[j][1]);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    write_partial<GQA>(a, st, rec);
}

template <int GQA>
__global__ __launch_bounds__(64) void decode_int_kv4_kernel(DecodeArgs a)
{
    walk_units(a, [&](int b, int h) { int_item_kv4<GQA>(a, b, h, true, 0, 0, prot_ptr(a, b * a.g.Hkv + h)); },
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   pace.tile((hi + kTile - 1) / kTile - lo / kTile);
                   int_item_kv4<GQA>(a, b, h, false, lo, hi, rec);
               });
}

// ---------------------------------------------------------------------------
// BF16 comparator, vector-ALU path: the same split structure over bf16 pages.
// ---------------------------------------------------------------------------
template <int GQA>
__device__ __forceinline__ void valu_item_bf16(const DecodeArgs& a, int b, int h, int t_begin,
                                               int t_end, float* rec)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x, e = lane >> 3, sl = lane & 7;
    if (t_end <= t_begin) return;
    const int slot = clampi(a.slot_ids[b], 0, g.max_slots - 1);
    const int32_t* bt = a.block_tables + (int64_t)slot * g.max_pages;
    __shared__ float P[8][GQA];
    float qk[GQA][16], sq[GQA];
    load_q<GQA>(a, b, h, qk, sq);
    Online<GQA> st;
    st.init();
    float alpha[GQA];
    const uint8_t* lbase = a.pages + (int64_t)a.layer * g.layer_pages;
    for (int hp = t_begin / kHalf; hp <= (t_end - 1) / kHalf; ++hp) {
        const int page = clampi(bt[hp / 2], 0, g.num_pages - 1);
        const uint8_t* pb = lbase + ((int64_t)page * g.Hkv + h) * g.pb;
        const int tok = hp * kHalf + e;
        const bool valid = tok >= t_begin && tok < t_end;
        const uint16_t* kr = reinterpret_cast<const uint16_t*>(pb) + (tok % kPage) * g.d + 16 * sl;
        uint4 u0 = *reinterpret_cast<const uint4*>(kr);
        uint4 u1 = *reinterpret_cast<const uint4*>(kr + 8);
        uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        float s[GQA];
#pragma unroll
        for (int j = 0; j < GQA; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                acc = fmaf(qk[j][2 * i], bf16_lo(w[i]), acc);
                acc = fmaf(qk[j][2 * i + 1], bf16_hi(w[i]), acc);
            }
            s[j] = acc;
        }
        softmax_chunk<GQA>(st, s, valid, a.scale2, P, alpha);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < GQA; ++j) { st.o[j][0] *= alpha[j]; st.o[j][1] *= alpha[j]; }
        const uint16_t* vr = reinterpret_cast<const uint16_t*>(pb + (int64_t)kPage * g.d * 2) +
                             (hp & 1) * g.d * kHalf;
        uint4 va = *reinterpret_cast<const uint4*>(vr + (2 * lane) * kHalf);
        uint4 vb = *reinterpret_cast<const uint4*>(vr + (2 * lane + 1) * kHalf);
        uint32_t vaw[4] = {va.x, va.y, va.z, va.w}, vbw[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int ee = 0; ee < kHalf; ++ee) {
            int t2 = hp * kHalf + ee;
            if (t2 < t_begin || t2 >= t_end) continue;
            float x0 = (ee & 1) ? bf16_hi(vaw[ee >> 1]) : bf16_lo(vaw[ee >> 1]);
            float x1 = (ee & 1) ? bf16_hi(vbw[ee >> 1]) : bf16_lo(vbw[ee >> 1]);
#pragma unroll
            for (int j = 0; j < GQA; ++j) {
                float p = P[ee][j];
                st.o[j][0] = fmaf(p, x0, st.o[j][0]);
                st.o[j][1] = fmaf(p, x1, st.o[j][1]);
            }
        }
        __syncthreads();
    }
    write_partial<GQA>(a, st, rec);
}

template <int GQA>
__global__ __launch_bounds__(64) void decode_valu_bf16_kernel(DecodeArgs a)
{
    walk_units(a, [&](int, int) {},
               [&](int b, int h, int lo, int hi, float* rec, Pace& pace) {
                   pace.tile((hi + kTile - 1) / kTile - lo / kTile);
                   valu_item_bf16<GQA>(a, b, h, lo, hi, rec);
               });
}

// ---------------------------------------------------------------------------
// Merge (eq. A1): one wave per (sequence, q head); 256-thread blocks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

// Zeroes the pool counters before a decode launch.
__global__ __launch_bounds__(64) void pool_reset_kernel(uint32_t* ctr)
{
    if (threadIdx.x < kPoolCounters) ctr[kPoolStride * threadIdx.x] = 0u;
}

// One wave per (sequence, q head): the stable base-2 log-sum-exp merge of the
// non-empty parts (eq. A1).  The length and the header are loaded together;
// with up to 8 parts, every part's log-normaliser (one per lane) and output
// (2 channels per lane) are then loaded at once, so a row costs two memory
// round trips.  Up to 128 parts: the log-normalisers in two loads per lane and
// the outputs 16 parts at a time; beyond that, 64 log-normalisers per pass.
__global__ __launch_bounds__(256) void merge_parts_kernel(DecodeArgs a)
{
    const Geo& g = a.g;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.batch * g.Hq) return;
    const int b = row / g.Hq, j = row % g.Hq, h = j / g.gqa, jj = j % g.gqa;
    const int bh = b * g.Hkv + h;
    const int n_b = seq_len(a, b);
    const int2 hd = a.hdr[bh];                   // read with the length; used only when bh has tiles
    const Units u = units_of(a, n_b);
    int n4p = 0, w0 = 0;
    if (u.ntile > 0) {
        const int smax = a.waves + a.pool_chunks - 1;
        w0 = clampi(hd.x, 0, smax);
        n4p = clampi(hd.y, w0, smax) - w0 + 1;
    }
    const int np = n4p + (u.prot > 0);           // the runs of (b, h), then its protected part
    const int stride = g.d + kPartPad;
    auto part_of = [&](int i) {
        return (i < n4p ? rec_ptr(a, (int64_t)bh + w0 + i) : prot_ptr(a, bh)) + jj * stride;
    };

    constexpr int kFew = 8, kBatch = 16;
    float W = 0.f, o0 = 0.f, o1 = 0.f;
    // outputs of parts [i, i + kBatch) weighted by wsel(part), loads issued together
    auto gather = [&](int i, int end, auto&& wsel) {
        float2 v[kBatch];
        float wi[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int ii = min(i + u, end - 1);
            wi[u] = i + u < end ? wsel(ii) : 0.f;
            v[u] = *reinterpret_cast<const float2*>(part_of(ii) + 2 * lane);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            o0 = fmaf(wi[u], v[u].x, o0);
            o1 = fmaf(wi[u], v[u].y, o1);
        }
    };
    if (np <= kFew) {
        const float z = lane < np ? part_of(lane)[g.d] : -INFINITY;
        float2 v[kFew];
#pragma unroll
        for (int i = 0; i < kFew; ++i)
            v[i] = i < np ? *reinterpret_cast<const float2*>(part_of(i) + 2 * lane) : make_float2(0.f, 0.f);
        const float zm = wave_max(z);
        const float w = lane < np ? exp2f(z - zm) : 0.f;
        W = wave_sum(w);
#pragma unroll
        for (int i = 0; i < kFew; ++i) {
            const float wi = __shfl(w, i);
            o0 = fmaf(wi, v[i].x, o0);
            o1 = fmaf(wi, v[i].y, o1);
        }
    } else if (np <= 128) {
        // log-normalisers of up to 128 parts in two registers; the outputs of
        // the first kFirst parts are loaded right after them (they do not
        // depend on the weights), so the wait for the log-normalisers leaves
        // those loads in flight; the rest in batches of 16 loads
        constexpr int kFirst = 16;
        const float z0 = lane < np ? part_of(lane)[g.d] : -INFINITY;
        const float z1 = 64 + lane < np ? part_of(64 + lane)[g.d] : -INFINITY;
        float2 v[kFirst];
#pragma unroll
        for (int u = 0; u < kFirst; ++u)
            v[u] = *reinterpret_cast<const float2*>(part_of(min(u, np - 1)) + 2 * lane);
        const float zm = wave_max(fmaxf(z0, z1));
        const float w0 = lane < np ? exp2f(z0 - zm) : 0.f;
        const float w1 = 64 + lane < np ? exp2f(z1 - zm) : 0.f;
        W = wave_sum(w0 + w1);
#pragma unroll
        for (int u = 0; u < kFirst; ++u) {
            const float wi = u < np ? __shfl(w0, u) : 0.f;
            o0 = fmaf(wi, v[u].x, o0);
            o1 = fmaf(wi, v[u].y, o1);
        }
        for (int i = kFirst; i < np; i += kBatch)
            gather(i, np, [&](int ii) { return ii < 64 ? __shfl(w0, ii) : __shfl(w1, ii - 64); });
    } else {
        float zmax = -INFINITY;
        for (int c = 0; c < np; c += 64)
            if (c + lane < np) zmax = fmaxf(zmax, part_of(c + lane)[g.d]);
        zmax = wave_max(zmax);
        for (int c = 0; c < np; c += 64) {
            const float w = c + lane < np ? exp2f(part_of(c + lane)[g.d] - zmax) : 0.f;
            W += wave_sum(w);
            const int m = min(64, np - c);
            for (int i = 0; i < m; i += kBatch)
                gather(c + i, c + m, [&](int ii) { return __shfl(w, ii - c); });
        }
    }
    const float inv = W > 0.f ? 1.0f / W : 0.f;  // n = 0 (clamped input) gives zeros
    o0 *= inv;
    o1 *= inv;
    int64_t off = ((int64_t)b * g.Hq + j) * g.d + 2 * lane;
    if (a.out_dtype == KV4_OUT_F32) {
        *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.out) + off) = make_float2(o0, o1);
    } else {
        reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.out) + off)[0] =
            f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16);
    }
}

}  // namespace kv4
