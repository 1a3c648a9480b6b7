/*
 * kv4.h -- C ABI of the KV4 decode-step library for AMD Instinct MI355X (gfx950).
 *
 * The library implements the decode step of a rollout engine whose KV cache is
 * stored as calibration-free asymmetric INT4 with FP16 scale and offset per
 * channel group, plus symmetric INT8 side copies of the attention-sink and
 * recent positions (KV4-RL, arXiv 2610.14448: Section 3 eq. 3.3; Section 5.1;
 * Section 5.2 "Bounded selective protection"; Section 5.3; Appendix A.2
 * "Scheduling and attention" and "Phase memory management"; Appendix A.3).
 * A BF16 cache kind with the same paging and the same partition/merge structure
 * is provided as the comparator (the paper's BF16 baseline, Section 6.1).
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers unless stated otherwise; the
 *     library never allocates, frees or initialises device memory.  Pools and
 *     workspaces are owned by the caller (the one exception is the static
 *     workspace of kv4_decode_attn_noalloc, reserved with the code object).
 *   - Work is enqueued asynchronously on the given HIP stream; device-side
 *     faults surface at the caller's next synchronisation with that stream.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is launched and a KV4_ERR_* code is returned.  Device arrays
 *     (lengths, slot ids, block tables) cannot be checked on the host: the
 *     kernels clamp them into the declared ranges, so out-of-range values give
 *     wrong results but never out-of-bounds accesses.
 *   - A kv4_cache handle is not thread-safe; calls on one handle that overlap
 *     in time on different streams race on the pools.
 *
 * Layout of the pools (all little-endian; "PB" = one (page, kv-head) block):
 *   page pool, KV4 kind: [layer][page][kv_head] blocks of
 *       K codes  16 tokens x head_dim/2 bytes, token-major; a token's row is
 *                16 32-bit words, word w holding channels 8n .. 8n+7 with
 *                n = 4*(w%4) + w/4 (channel 8n+e in bits 4e..4e+3);
 *       V codes  2 halves x head_dim 32-bit words; in half h, the word at index
 *                64*(c/64) + 4*(c%16) + 2*((c/32)%2) + (c/16)%2 holds the codes of
 *                tokens 8h..8h+7 at channel c, token 8h+e in bits 4e..4e+3;
 *       K meta   [16 tokens][group] pairs (delta, offset) of binary16;
 *       V offset [16 tokens][group] binary16;
 *       V delta  [group][16 tokens] binary16;
 *     i.e. 16 * (head_dim + 8 * head_dim / group_size) bytes per PB
 *     (2,560 B at head_dim 128, group 32: 160 B per token and kv head).
 *   page pool, KV8 kind: [layer][page][kv_head] blocks of
 *       K codes  [16 tokens][head_dim] int8, token-major;
 *       V codes  2 blocks of 8 tokens x head_dim int8, channel-major: token t,
 *                channel c at (t/8)*8*head_dim + ((c%16)*8 + c/16)*8 + t%8
 *                (the side ring's V layout);
 *       K scale  [16] binary16, then V scale [16] binary16;
 *     i.e. 16 * (2*head_dim + 4) bytes per PB (4,160 B at head_dim 128).
 *   page pool, BF16 kind: [layer][page][kv_head] blocks of K [16][head_dim]
 *     bf16 (token-major) then V [2 halves][head_dim][8 tokens] bf16 -- value
 *     (t, c) at ((t/8)*head_dim + c)*8 + t%8 (8,192 B at head_dim 128).
 *   side pool (KV4 kind only): [layer][slot][kv_head] blocks of E = S + R
 *     ring entries padded to a multiple of 32:
 *       K codes [E][head_dim] int8 (entry-major);
 *       V codes [E/8] blocks of 8 entries x head_dim int8, channel-major:
 *                entry e, channel c at (e/8)*8*head_dim + ((c%16)*8 + c/16)*8 + e%8;
 *       K scale [E] binary16, then V scale [E] binary16;
 *     i.e. E * (2*head_dim + 4) bytes.  Position p of a sequence lives in ring
 *     entry p when p < S and in entry S + (p - S) mod R otherwise, so the
 *     protected positions of an n-token context are entries [0, min(n, S+R)).
 */
#ifndef KV4_H
#define KV4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define KV4_OK                0
#define KV4_ERR_INVALID_ARG   1  /* null pointer, negative size, bad enum, shape mismatch */
#define KV4_ERR_UNSUPPORTED   2  /* a valid request the library does not implement */
#define KV4_ERR_CAPACITY      3  /* batch > max_slots, layer >= num_layers, pool too small */
#define KV4_ERR_WORKSPACE     4  /* workspace pointer null or smaller than required */
#define KV4_ERR_HIP           5  /* a HIP runtime call failed (launch error) */

/* Cache kinds. */
#define KV4_KIND_MIXED 0         /* INT4 pages + INT8 sink/recent side ring */
#define KV4_KIND_BF16  1         /* BF16 pages, no protection (comparator) */
#define KV4_KIND_KV8   2         /* INT8 pages for every position, symmetric per
                                    token and kv head with a binary16 scale (the
                                    side entries' encoding, KV4-RL Appendix A.3);
                                    the paper's KV8 comparison point (Fig. 3b,
                                    Fig. 4a); sink and recent are unused; decode
                                    needs Hq/Hkv = 4 */

/* Flags (kv4_cache_desc.flags). */
/* KV4_FLAG_ROTATE_K: keys are stored in a rotated basis (KV4-RL Section 5.1,
 * Appendix A.3 "Encoding and allocation"): kv4_append replaces each new key
 * k (post-RoPE, bf16) by y = k H / sqrt(128), H the Sylvester Hadamard matrix,
 * before both the INT4 and the INT8 encoding, and the decode transforms each
 * query the same way before attention, so unquantized scores are unchanged
 * (eq. 3.4); values are not rotated.  y is computed in binary32 in one fixed
 * order: butterfly stages of span 1, 2, 4, ..., 64, each replacing every
 * channel pair (c, c + h), c & h == 0, by (y_c + y_{c+h}, y_c - y_{c+h}), then
 * every channel times the binary32 value nearest 1/sqrt(128) (0x3DB504F3).
 * Mixed kind only (KV4_ERR_UNSUPPORTED with KV4_KIND_BF16); rotated keys must
 * stay within the binary16 range. */
#define KV4_FLAG_ROTATE_K 0x1
/* KV4_FLAG_INT_PATH: the decode takes the integer path of KV4-RL Appendix A.3
 * ("Integer decode path"; "Protected path and reconstruction") instead of the
 * bf16-query, fp32-probability path.  Per (sequence, q head) the query (in the
 * keys' basis when KV4_FLAG_ROTATE_K is set) is quantized to INT8 with the side
 * entries' encoding (scale s_q = fp16(fp32(amax/127)), nearest codes, ties to
 * even).  INT4 position: score = sm_scale * s_q * sum over groups g of
 * (Delta_g * I_g + m_g * Q_g), with I_g the integer dot product of the query
 * codes and the position's 4-bit key codes over the group and Q_g the sum of
 * the query codes.  Protected position: score = sm_scale * s_q * s_k * (integer
 * dot product with the INT8 key codes).  Softmax in binary32.  INT4 values: per
 * block of the 8 positions [8k, 8k + 8) that share a V code word, value group
 * and q head, w_t = p_t * Delta^v_t is carried as an 8-bit code
 * u_t = rint(255 w_t / max w) with scale max w / 255, and the block adds
 * scale * (integer dot product of u with the value codes) + sum_t p_t m^v_t.
 * Exception: a block whose largest w is at most 2^-100 gets u = 0 for all its
 * positions (its term sum_t p_t m^v_t stays).  w is measured in each kernel's
 * own units: with p_t = 2^(score_t - m_ref) against the running maximum m_ref
 * of the scores in the vector-ALU form (KV4_FLAG_VALU_DECODE), and with
 * p_t = 2^(score_t - m_ref + 48) against a reference that trails the running
 * maximum by at most 16 in the matrix-core form (every ratio otherwise),
 * scores in base 2.
 * Either way the dropped terms sum to at most 8 * 15 * max w <= 120 * 2^-100
 * against a normaliser of at least 1 (vector ALU) or 2^32 (matrix core), so
 * every output differs from the rint rule by less than 2^-90; 255 / max w
 * would overflow binary32 there.
 * Protected values: binary32 products with the dequantized INT8 values (no
 * probability quantization).  Mixed kind only (KV4_ERR_UNSUPPORTED otherwise);
 * q/kv head ratios 1 to 8; the cache's bytes do not change. */
#define KV4_FLAG_INT_PATH 0x2
/* KV4_FLAG_VALU_DECODE: the decode runs on the vector-ALU kernels (otherwise on
 * the matrix-core kernels at every ratio), with the same partition, arithmetic
 * definitions and tolerance.  A measurement point for the choice of the matrix core (no
 * passage of the pages behind it).  Mixed and BF16 kinds at q/kv head ratios
 * 1, 2, 4 and 8 (KV4_ERR_UNSUPPORTED for KV8 and other ratios). */
#define KV4_FLAG_VALU_DECODE 0x4

/* Output dtypes of kv4_decode_attn. */
#define KV4_OUT_F32  0
#define KV4_OUT_BF16 1

/* HIP stream handle, passed through untouched (hipStream_t). */
typedef void* kv4_stream_t;

typedef struct kv4_cache_desc {
    int32_t num_layers;         /* >= 1 */
    int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads */
    int32_t num_kv_heads;       /* Hkv.  Hq / Hkv: 1 to 8 (the matrix core runs
                                   the q heads of a kv head in halves of four),
                                   or 16 for the mixed kind without
                                   KV4_FLAG_INT_PATH; KV8 1 to 8.  Others:
                                   KV4_ERR_UNSUPPORTED */
    int32_t head_dim;           /* d; the library supports 128 */
    int32_t page_size;          /* tokens per page; the library supports 16 */
    int32_t group_size;         /* G, INT4 channels per (Delta, m) pair: 32, 64 or 128 */
    int32_t sink;               /* S >= 0: first S positions kept as INT8 */
    int32_t recent;             /* R >= 0: last R positions kept as INT8 */
    int32_t num_pages;          /* pages per layer in the page pool, >= 1 */
    int32_t max_slots;          /* request slots (rows of the block table, side rings) */
    int32_t max_pages_per_seq;  /* columns of the block table */
    int32_t kind;               /* KV4_KIND_MIXED, KV4_KIND_BF16 or KV4_KIND_KV8 */
    int32_t flags;              /* KV4_FLAG_* */
    int32_t num_waves;          /* waves (one-wave workgroups) of the balanced decode
                                   partition; 0 = 16 per compute unit of the
                                   current device (when the decode runs on a
                                   kernel that keeps fewer resident -- the
                                   vector-ALU kernels, and the matrix-core
                                   kernels of q/kv ratio 8 -- as many per
                                   compute unit as that kernel keeps resident,
                                   at most 16), else 1 .. 65536 */
    int32_t pool_chunks;        /* most chunks of the decode's dynamic pool: 0 = no
                                   pool (the default), else a power of two in
                                   8 .. 65536 */
} kv4_cache_desc;

typedef struct kv4_cache kv4_cache;  /* opaque host-side handle */

/*
 * Bytes of device memory the caller must provide (KV4-RL Appendix A.2, "Phase
 * memory management": the pool is provisioned as floor(M_q / b_q) pages, where
 * b_q counts every byte of a 16-token page including metadata; side storage is
 * reserved per request slot, Appendix A.3 "Encoding and allocation").
 *   page_pool_bytes  num_layers * num_pages * num_kv_heads * PB bytes
 *   side_pool_bytes  num_layers * max_slots * num_kv_heads * ring block bytes
 *                    (0 for the BF16 kind, or when S + R = 0)
 * page_bytes_per_layer (optional, may be NULL) receives b_q for one layer, so a
 * caller can size num_pages = floor(M / (num_layers * b_q)).
 * Host-only; never touches the GPU.
 */
int kv4_cache_required_bytes(const kv4_cache_desc* desc, size_t* page_pool_bytes,
                             size_t* side_pool_bytes, size_t* page_bytes_per_layer);

/*
 * Create a handle over caller-owned pools.  page_pool / side_pool are device
 * buffers of at least the sizes kv4_cache_required_bytes returns (side_pool
 * may be NULL when that size is 0), 16-byte aligned (hipMalloc and torch
 * allocations are): the kernels move 16-byte words.  Pools need no
 * initialisation: a position is only ever read after the append that wrote
 * it.  *out receives a host object freed with kv4_cache_free.  No device work.
 * Errors: those of the description's checks (as kv4_cache_required_bytes),
 * KV4_ERR_INVALID_ARG (a needed pool or out NULL, a pool not 16-byte
 * aligned), KV4_ERR_CAPACITY (a pool smaller than required).
 */
int kv4_cache_create(const kv4_cache_desc* desc, void* page_pool, size_t page_pool_bytes,
                     void* side_pool, size_t side_pool_bytes, kv4_cache** out);

/*
 * Append new tokens' keys and values to layer `layer` (KV4-RL Section 5.3:
 * both cache representations are produced directly from the source K/V
 * vectors when each token is generated; Appendix A.3: prefill and carried-
 * prefix reconstruction populate both representations).
 *
 *   k_bf16, v_bf16  [total_new][Hkv][d] bf16, keys after RoPE, sequence-major
 *   cu_new          [batch+1] int32, prefix sums of new tokens per sequence
 *                   (cu_new[0] = 0, cu_new[batch] = total_new)
 *   ctx_before      [batch] int32, context length before this append; the new
 *                   tokens of sequence b take positions ctx_before[b] ..
 *                   ctx_before[b] + new_b - 1
 *   slot_ids        [batch] int32, request slot of each sequence (distinct)
 *   block_tables    [max_slots][max_pages_per_seq] int32, page ids per slot;
 *                   every page covering a written position must be assigned
 *
 * KV4 kind: every new position gets its INT4 codes, Delta and m written into
 * its page.  A new position also gets an INT8 entry in the slot's side ring
 * when it is protected in the context as it stands after this append, i.e.
 * p < S or p >= ctx_before + new_b - R.  A position that later leaves the
 * recent window needs no further work (demotion moves only the region
 * boundary; its INT4 entry already exists).  BF16 kind: the bf16 values are
 * copied into the pages.  KV8 kind: every new position gets its INT8 K and V
 * codes and scales (s = fp16(fp32(amax / 127)), codes the nearest integers to
 * x / s, ties to even, in [-127, 127]) written into its page.
 * batch == 0 or total_new == 0 is a no-op that returns KV4_OK once the cache,
 * the sizes and the layer are valid, before the pointers are checked (they may
 * then be NULL).
 * Errors: KV4_ERR_INVALID_ARG (cache NULL, batch < 0, total_new < 0, or a NULL
 * pointer when there is work), KV4_ERR_CAPACITY (layer out of range, batch >
 * max_slots), KV4_ERR_HIP.
 */
int kv4_append(kv4_cache* cache, int layer, const void* k_bf16, const void* v_bf16,
               const int32_t* cu_new, const int32_t* ctx_before, const int32_t* slot_ids,
               const int32_t* block_tables, int batch, int total_new, kv4_stream_t stream);

/*
 * Workspace bytes kv4_decode_attn needs for `batch` sequences (validated
 * against max_ctx, which does not change the size): the per-part outputs and
 * log-normalisers of the partition/merge, ((2*batch*Hkv + W + C) * (Hq/Hkv) *
 * (d + 4)) float32 plus batch*Hkv int32 pairs, rounded up to 256 bytes, plus
 * 2 KiB of pool counters (W, C as kv4_decode_partition gives them).  Queries
 * the current device's compute-unit count; launches nothing.
 */
int kv4_decode_workspace_bytes(const kv4_cache* cache, int batch, int max_ctx, size_t* bytes);

/*
 * GQA decode attention of one query token per sequence over its ragged, paged
 * context (KV4-RL Section 5.3 and Appendix A.3 "Regional softmax merge",
 * eq. A1): the INT4 region is cut into runs of 32-token tiles and the
 * protected region (sink + recent, read from the INT8 ring) is one more part;
 * each part yields a locally normalised output and log-normaliser, and a merge
 * kernel combines them by a stable log-sum-exp with zero weight for empty
 * parts.  The cut is a partition of the whole batch's work over W waves (see
 * kv4_decode_partials): balanced static shares, optionally followed by a
 * pool of chunks that the waves take as they finish.
 *
 *   q_bf16      [batch][Hq][d] bf16 (after RoPE)
 *   seq_lens    [batch] int32, n = context length after this step's append
 *               (1 <= n <= max_ctx); the query attends over positions [0, n)
 *   slot_ids    [batch] int32; block_tables as for kv4_append
 *   max_ctx     host bound on every n (lengths are clamped to it)
 *   sm_scale    softmax scale applied to q.k (1/sqrt(d) is the usual choice)
 *   out         [batch][Hq][d], float32 (KV4_OUT_F32) or bf16 (KV4_OUT_BF16)
 *   workspace   device buffer of >= kv4_decode_workspace_bytes(cache, batch, max_ctx)
 * q head j reads kv head j / (Hq / Hkv).  Protected positions of an n-token
 * context are [0, min(S, n)) and [max(S, n - R), n); all others read INT4.
 * Errors: KV4_ERR_INVALID_ARG, KV4_ERR_CAPACITY (also when batch * Hkv *
 * (ceil(max_ctx / 32) + 1 + U8) >= 2^30, the bound of the partition's 32-bit
 * counts), KV4_ERR_WORKSPACE, KV4_ERR_HIP.
 */
int kv4_decode_attn(kv4_cache* cache, int layer, const void* q_bf16, const int32_t* seq_lens,
                    const int32_t* slot_ids, const int32_t* block_tables, int batch,
                    int max_ctx, float sm_scale, void* out, int out_dtype, void* workspace,
                    size_t workspace_bytes, kv4_stream_t stream);

/*
 * The two phases of kv4_decode_attn, with the same arguments and results:
 * kv4_decode_attn is exactly kv4_decode_partials followed by kv4_decode_merge
 * on one stream.  They are separate entry points for callers that time the
 * attention and the merge apart, or that merge parts computed elsewhere (a
 * context split over several devices yields parts of one (sequence, head)
 * that combine by the same eq. A1 of KV4-RL Appendix A.3).
 *
 * kv4_decode_partials runs the whole step's work over W waves.  The work is,
 * for each (sequence b, kv head h), bh = b*Hkv + h in increasing order, its
 * protected part (if non-empty; indivisible, of weight U8 =
 * 3 * ceil((S + R) / 32) tiles, the measured cost of its 32-entry
 * INT8 tiles) and the 32-token tiles of its INT4 region [S, max(S, n - R))
 * (tile t covers positions [32t, 32t + 32) clipped to the region); T4 tiles
 * and P protected parts in all, W' = min(W, ceil((T4 + U8 P) / 20)) waves in
 * use.  The tile sequence is cut into shares:
 *   - a pool of the last Tp = floor(3 T4 / 16) tiles in Cd chunks, Cd the
 *     largest power of two <= the cache's pool chunk count with 2 Cd <= Tp
 *     (no pool, Tp = 0, when that is below 8); with A = Tp - Cd, chunk c is
 *     pool tiles [g(c), g(c+1)), g(c) = c + A - floor(A (Cd - c)^2 / Cd^2);
 *   - static shares over the first Ts = T4 - Tp tiles: wave w runs protected
 *     parts [floor(w P / W'), floor((w+1) P / W')) and tiles [t(w), t(w+1)),
 *     t(w) = floor(w (Ts + U8 P) / W') - U8 floor(w P / W') (every wave the same
 *     weight); when that is not increasing in w, t(w) = floor(min(w, W4) Ts /
 *     W4) with W4 = max(1, min(W', Ts)) instead;
 *   - share s < S0 (S0 = W', or W4 in the second case) is static share s,
 *     share S0 + c is chunk c.  A wave runs its static share, then takes chunks
 *     (chunk c is ticket c / 8 of atomic counter c % 8 in the workspace) until
 *     none is left.
 * Each maximal run of tiles of one bh in a share is one part.  Which wave runs
 * a share changes nothing in its results, so the output is the same from run
 * to run.  Workspace (16-byte aligned), float32 records of (Hq/Hkv) rows of
 * d + 4 floats (row j: floats [0, d) the softmax-normalised output of q head
 * h*(Hq/Hkv) + j over the part, float d its base-2 log-normaliser z = max +
 * log2(sum) of the scores scaled by sm_scale*log2(e)):
 *     run records        [batch*Hkv + W + C]  the run of bh in share s at bh + s
 *                        (C = kv4_decode_partition's pool chunk count)
 *     protected records  [batch*Hkv]      the protected part of bh at bh
 *     header             [batch*Hkv][2] int32: first and last share running
 *                        tiles of bh (written when bh has INT4 tiles)
 *     counters           8 uint32 at the next multiple of 256 bytes, 256 bytes
 *                        apart; kv4_decode_partials zeroes them before its
 *                        attention kernel, on the same stream
 * so the runs of bh are the records bh + first .. bh + last.  Parts with no
 * positions are not written.  The BF16 kind has no protected parts and tiles
 * its whole context.  Two calls in flight at once must not share a workspace.
 *
 * kv4_decode_merge combines, per (b, q head), the non-empty parts of that
 * workspace into out with weights 2^(z_k - max z) (zero for empty parts); its
 * batch, max_ctx and seq_lens must be those of the kv4_decode_partials call
 * that wrote the workspace.  The workspace must be 16-byte aligned.
 * Errors: as kv4_decode_attn.
 */
int kv4_decode_partials(kv4_cache* cache, int layer, const void* q_bf16, const int32_t* seq_lens,
                        const int32_t* slot_ids, const int32_t* block_tables, int batch,
                        int max_ctx, float sm_scale, void* workspace, size_t workspace_bytes,
                        kv4_stream_t stream);
int kv4_decode_merge(kv4_cache* cache, const int32_t* seq_lens, int batch, int max_ctx,
                     void* out, int out_dtype, const void* workspace, size_t workspace_bytes,
                     kv4_stream_t stream);

/*
 * Prefill attention (KV4-RL Appendix A.3, "Protected path and reconstruction":
 * prefill and carried-prefix reconstruction run BF16 attention over the newly
 * computed K/V, whose cache entries kv4_append then writes): causal softmax
 * attention of every packed position t of sequence b over the positions
 * [cu_seqlens[b], t] of the same sequence, on the bf16 values as given (no
 * quantization), with binary32 accumulation.  Uses the cache only for its
 * geometry (Hq, Hkv, head_dim); reads and writes no pool.
 *   q_bf16       [total][Hq][d] bf16 (after RoPE); k_bf16, v_bf16 [total][Hkv][d]
 *   cu_seqlens   [batch + 1] int32 device array, row offsets: cu[0] = 0,
 *                nondecreasing, cu[batch] = total
 *   max_seqlen   host bound on every length (longer sequences are cut to it)
 *   out          [total][Hq][d], float32 (KV4_OUT_F32) or bf16 (KV4_OUT_BF16)
 * q head j reads kv head j / (Hq / Hkv).  Offsets are clamped to [0, total].
 * Errors: KV4_ERR_INVALID_ARG (null pointers, batch < 1, total < 0,
 * max_seqlen < 1, non-finite sm_scale, bad out_dtype), KV4_ERR_CAPACITY
 * (max_seqlen above 2^23 or batch above 65,536), KV4_ERR_HIP.  total = 0
 * launches nothing.
 */
int kv4_prefill_attn(const kv4_cache* cache, const void* q_bf16, const void* k_bf16,
                     const void* v_bf16, const int32_t* cu_seqlens, int batch, int total,
                     int max_seqlen, float sm_scale, void* out, int out_dtype,
                     kv4_stream_t stream);

/*
 * kv4_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the partition's records, header and pool
 * counters live in a static device array of KV4_NOALLOC_SCRATCH_BYTES that the
 * library reserves with its code object -- each GPU the library runs on holds
 * its own copy until the process ends.  The call allocates and frees nothing;
 * it looks the array's device address up once per device (hipGetSymbolAddress,
 * on the first call with that device current).  Arguments, kernels and results
 * are those of kv4_decode_attn (the output is bit-identical); what must start
 * at zero (the pool counters) is cleared by a kernel in every call.  Every
 * call on one GPU shares that GPU's array and leaves its contents behind, so
 * calls that overlap in time on one GPU (different streams, threads or
 * handles) race: order them.
 * Errors: as kv4_decode_attn, plus KV4_ERR_CAPACITY when the batch needs more
 * workspace than the array holds (kv4_decode_workspace_bytes > the limit;
 * checked on the host, nothing launched) and KV4_ERR_HIP when the array's
 * address cannot be obtained.
 */
#define KV4_NOALLOC_SCRATCH_BYTES (32u << 20)
int kv4_decode_attn_noalloc(kv4_cache* cache, int layer, const void* q_bf16, const int32_t* seq_lens,
                            const int32_t* slot_ids, const int32_t* block_tables, int batch,
                            int max_ctx, float sm_scale, void* out, int out_dtype,
                            kv4_stream_t stream);

/* Free the host handle (the pools stay with the caller). NULL is accepted. */
int kv4_cache_free(kv4_cache* cache);

/* Static, human-readable text for a return code. */
const char* kv4_status_string(int status);

/*
 * W, the number of waves of the decode partition (desc.num_waves, or 16 per
 * compute unit of the current device), and C, the most chunks of its dynamic
 * pool (desc.pool_chunks, 0 for none); either pointer may be NULL, not both.
 * For tests and reporting; launches nothing.
 */
int kv4_decode_partition(const kv4_cache* cache, int* waves, int* pool_chunks);

/*
 * Validating build (the library compiled with KV4_VALIDATE: libkv4_validate.so;
 * a debugging aid, no passage of the pages behind it).  Before each append,
 * decode and prefill launch, a check kernel on the same stream reads the
 * device arrays as this header defines them and records every kind of
 * violation it finds; the checked launches are unchanged (they clamp as
 * described under "Conventions").  Kinds:
 *   SEQ_LEN    a decode length outside [1, max_ctx], or a prefill sequence
 *              longer than max_seqlen;
 *   SLOT       a slot id outside [0, max_slots);
 *   PAGE       a block-table entry outside [0, num_pages) for a page the call
 *              reads or writes (pages of positions [0, n) for a decode, of the
 *              new positions for an append);
 *   ROWS       row offsets (cu_new, cu_seqlens) that are negative, decreasing,
 *              past the total, or do not start at 0 and end at the total;
 *   POSITION   ctx_before[b] < 0 or ctx_before[b] + new_b beyond the block
 *              table's capacity (max_pages_per_seq * page_size);
 *   DUPLICATE_WRITE  two sequences of one append writing the same page, or the
 *              same slot's INT8 ring (pages below 2^20 and slots below 2^16
 *              are tracked).
 * kv4_validate_report stores the OR of the kinds recorded on the current
 * device since the last report into *violations and clears them (synchronous;
 * synchronise the streams that ran the checked calls first).  Errors:
 * KV4_ERR_INVALID_ARG (null pointer), KV4_ERR_UNSUPPORTED (a library built
 * without KV4_VALIDATE; *violations is set to 0), KV4_ERR_HIP.
 */
#define KV4_VIOLATION_SEQ_LEN          0x01u
#define KV4_VIOLATION_SLOT             0x02u
#define KV4_VIOLATION_PAGE             0x04u
#define KV4_VIOLATION_ROWS             0x08u
#define KV4_VIOLATION_POSITION         0x10u
#define KV4_VIOLATION_DUPLICATE_WRITE  0x20u
int kv4_validate_report(uint32_t* violations);

#ifdef __cplusplus
}
#endif

#endif /* KV4_H */
