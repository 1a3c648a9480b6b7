// kv4_decode.hpp -- split-KV decode attention over the paged mixed cache and
// the log-sum-exp merge of its parts.
//
// KV4-RL (arXiv 2610.14448), Section 5.3 and Appendix A.3: the INT4 region and
// the protected (sink + recent, INT8) region are processed independently;
// each part yields a locally normalised output o_r and log-normaliser z_r and
// the parts are merged with z = log sum_r e^{z_r}, o = sum_r e^{z_r - z} o_r
// (eq. A1), with zero weight for empty parts; the same identity merges the
// context splits inside a region.
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
constexpr int kMaxSplit = 2048;  // longest context split (tokens) a work item covers
constexpr int kAutoSplit = 1024; // longest split the automatic choice picks

struct DecodeArgs {
    Geo g;
    int layer;
    const uint16_t* q;            // [batch][Hq][d] bf16
    const int32_t* seq_lens;
    const int32_t* slot_ids;
    const int32_t* block_tables;
    int batch, max_ctx;
    int split;                    // tokens per context split (multiple of 32)
    int nsplit;                   // INT4 splits reserved per (sequence, kv head)
    float scale2;                 // sm_scale * log2(e)
    const uint8_t* pages;
    const uint8_t* side;
    float* part;                  // [batch][Hkv][nsplit+1][gqa][d + kPartPad]
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

__device__ __forceinline__ float* part_ptr(const DecodeArgs& a, int b, int h, int item, int j)
{
    return a.part + ((((int64_t)b * a.g.Hkv + h) * (a.nsplit + 1) + item) * a.g.gqa + j) *
                        (int64_t)(a.g.d + kPartPad);
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
        float x = s[j];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x = valid ? x * scale2 : -INFINITY;
        float mx = fmaxf(x, __shfl_xor(x, 8));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        float mn = fmaxf(st.m[j], mx);            // finite: the chunk has a valid token
        alpha[j] = exp2f(st.m[j] - mn);
        float p = exp2f(x - mn);
        st.m[j] = mn;
        st.l[j] = st.l[j] * alpha[j] + (sl == 0 ? p : 0.f);
        if (sl == 0) P[e][j] = p;
    }
}

template <int GQA>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, Online<GQA>& st, int b, int h,
                                              int item)
{
    const int lane = threadIdx.x;
#pragma unroll
    for (int j = 0; j < GQA; ++j) {
        float l = wave_sum(st.l[j]);
        float inv = 1.0f / l;
        float* dst = part_ptr(a, b, h, item, j);
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
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qk[j][2 * i] = bf16_lo(w[i]);
            qk[j][2 * i + 1] = bf16_hi(w[i]);
            s += qk[j][2 * i] + qk[j][2 * i + 1];
        }
        sq[j] = s;
    }
}

// ---------------------------------------------------------------------------
// Mixed cache, vector-ALU path: one wave per work item (sequence b, kv head h,
// item); items < nsplit are INT4 context splits, item nsplit is the protected
// (sink + recent) part read from the INT8 ring.
// ---------------------------------------------------------------------------
template <int GQA>
__device__ __forceinline__ void valu_item_kv4(const DecodeArgs& a, int b, int h, int item)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x, e = lane >> 3, sl = lane & 7;
    const int n = clampi(a.seq_lens[b], 0, a.max_ctx);
    const Regions rg = regions_of(n, g.S, g.R);
    const bool prot = item == a.nsplit;
    int t_begin = 0, t_end = 0;
    if (prot) {
        t_end = rg.n8;
    } else {
        t_begin = max(item * a.split, g.S);
        t_end = min((item + 1) * a.split, rg.rec_start);
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
        const uint8_t* ring = a.side + (int64_t)a.layer * g.layer_side + ((int64_t)slot * g.Hkv + h) * g.rb;
        const uint16_t* scales = reinterpret_cast<const uint16_t*>(ring + (int64_t)2 * g.SR * g.d);
        for (int c0 = 0; c0 < t_end; c0 += kHalf) {
            const int i = c0 + e;
            const bool valid = i < t_end;
            const int pos = i < rg.sink_end ? i : rg.rec_start + (i - rg.sink_end);
            const int ent = pos < g.S ? pos : g.S + (g.R > 0 ? (pos - g.S) % g.R : 0);
            const int entc = clampi(ent, 0, g.SR - 1);
            uint4 kc = *reinterpret_cast<const uint4*>(ring + (int64_t)entc * g.d + 16 * sl);
            float sk = half_bits_to_float(scales[entc]);
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
            for (int ee = 0; ee < kHalf; ++ee) {
                int i2 = c0 + ee;
                if (i2 >= t_end) break;
                int pos2 = i2 < rg.sink_end ? i2 : rg.rec_start + (i2 - rg.sink_end);
                int ent2 = pos2 < g.S ? pos2 : g.S + (g.R > 0 ? (pos2 - g.S) % g.R : 0);
                ent2 = clampi(ent2, 0, g.SR - 1);
                uint32_t vv = reinterpret_cast<const uint16_t*>(ring + (int64_t)(g.SR + ent2) * g.d)[lane];
                float sv = half_bits_to_float(scales[g.SR + ent2]);
                float x0 = sv * (float)(int)(int8_t)(vv & 0xFFu);
                float x1 = sv * (float)(int)(int8_t)(vv >> 8);
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
    write_partial<GQA>(a, st, b, h, item);
}

// Grid (nsplit+1, Hkv, batch).
template <int GQA>
__global__ __launch_bounds__(64) void decode_split_kv4_kernel(DecodeArgs a)
{
    valu_item_kv4<GQA>(a, blockIdx.z, blockIdx.y, blockIdx.x);
}

// ---------------------------------------------------------------------------
// BF16 comparator, vector-ALU path: the same split structure over bf16 pages.
// ---------------------------------------------------------------------------
template <int GQA>
__device__ __forceinline__ void valu_item_bf16(const DecodeArgs& a, int b, int h, int item)
{
    const Geo& g = a.g;
    const int lane = threadIdx.x, e = lane >> 3, sl = lane & 7;
    const int n = clampi(a.seq_lens[b], 0, a.max_ctx);
    const int t_begin = item * a.split;
    const int t_end = min((item + 1) * a.split, n);
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
    write_partial<GQA>(a, st, b, h, item);
}

// Grid (nsplit, Hkv, batch).
template <int GQA>
__global__ __launch_bounds__(64) void decode_split_bf16_kernel(DecodeArgs a)
{
    valu_item_bf16<GQA>(a, blockIdx.z, blockIdx.y, blockIdx.x);
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

// One wave per (sequence, q head): the stable base-2 log-sum-exp merge of the
// non-empty parts (eq. A1).  The log-normalisers are read lane-parallel, 64
// parts per pass; the outputs (2 channels per lane) with four independent
// loads in flight.
__global__ __launch_bounds__(256) void merge_parts_kernel(DecodeArgs a)
{
    const Geo& g = a.g;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.batch * g.Hq) return;
    const int b = row / g.Hq, j = row % g.Hq, h = j / g.gqa, jj = j % g.gqa;
    const int n = clampi(a.seq_lens[b], 0, a.max_ctx);
    int k_lo, k_hi, has8;
    if (g.kind == KV4_KIND_MIXED) {
        Regions rg = regions_of(n, g.S, g.R);
        k_lo = g.S / a.split;
        k_hi = rg.n4 > 0 ? (rg.rec_start + a.split - 1) / a.split : k_lo;
        has8 = rg.n8 > 0;
    } else {
        k_lo = 0;
        k_hi = (n + a.split - 1) / a.split;
        has8 = 0;
    }
    k_hi = min(k_hi, a.nsplit);
    const int n4p = max(k_hi - k_lo, 0);
    const int np = n4p + has8;                   // parts to merge: splits k_lo.., then the protected part
    auto part_of = [&](int i) { return part_ptr(a, b, h, i < n4p ? k_lo + i : a.nsplit, jj); };

    float zmax = -INFINITY;
    for (int c = 0; c < np; c += 64)
        if (c + lane < np) zmax = fmaxf(zmax, part_of(c + lane)[g.d]);
    zmax = wave_max(zmax);
    float W = 0.f, o0 = 0.f, o1 = 0.f;
    for (int c = 0; c < np; c += 64) {
        const float w = c + lane < np ? exp2f(part_of(c + lane)[g.d] - zmax) : 0.f;
        W += wave_sum(w);
        const int m = min(64, np - c);
        for (int i = 0; i < m; i += 4) {
            float2 v[4];
            float wi[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ii = min(i + u, m - 1);
                wi[u] = i + u < m ? __shfl(w, ii) : 0.f;
                v[u] = *reinterpret_cast<const float2*>(part_of(c + ii) + 2 * lane);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                o0 = fmaf(wi[u], v[u].x, o0);
                o1 = fmaf(wi[u], v[u].y, o1);
            }
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
