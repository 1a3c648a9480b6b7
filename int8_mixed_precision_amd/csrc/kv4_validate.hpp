// kv4_validate.hpp -- device-side checks of the caller's device arrays, built
// into the library only when KV4_VALIDATE is defined (libkv4_validate.so).
//
// The kernels clamp lengths, slot ids, block-table entries and append offsets
// into their declared ranges (include/kv4.h, "Conventions"), so bad values
// give wrong results but no out-of-bounds access.  A validating build runs a
// check kernel on the same stream before each append, decode and prefill
// launch; it reads the arrays as the documentation defines them and ORs the
// kinds of violation it finds into a device word, which kv4_validate_report
// returns and clears.  The checked launches themselves are unchanged.
//
// An append of several sequences must not write the same bytes twice: each
// page a sequence writes, and the INT8 ring of its slot, are claimed by that
// sequence through a table of owner tags (compare-and-swap, cleared before
// every append); a second owner is a duplicate write.  Pages at or past
// kOwnPages and slots at or past kOwnSlots are not tracked.
#pragma once

#include "kv4_append.hpp"
#include "kv4_decode.hpp"
#include "kv4_prefill.hpp"

namespace kv4 {

constexpr uint32_t kVioSeqLen = 1u << 0;      // KV4_VIOLATION_SEQ_LEN
constexpr uint32_t kVioSlot = 1u << 1;        // KV4_VIOLATION_SLOT
constexpr uint32_t kVioPage = 1u << 2;        // KV4_VIOLATION_PAGE
constexpr uint32_t kVioRows = 1u << 3;        // KV4_VIOLATION_ROWS
constexpr uint32_t kVioPosition = 1u << 4;    // KV4_VIOLATION_POSITION
constexpr uint32_t kVioDuplicate = 1u << 5;   // KV4_VIOLATION_DUPLICATE_WRITE

constexpr int kOwnPages = 1 << 20;
constexpr int kOwnSlots = 1 << 16;

__device__ uint32_t g_violations;
__device__ int32_t g_page_owner[kOwnPages];
__device__ int32_t g_slot_owner[kOwnSlots];

__device__ __forceinline__ void report(uint32_t kind)
{
    atomicOr(&g_violations, kind);
}

// Claims an owner tag for sequence b; another sequence's tag is a duplicate write.
__device__ __forceinline__ void claim(int32_t* tag, int b)
{
    const int32_t prev = atomicCAS(tag, 0, b + 1);
    if (prev != 0 && prev != b + 1) report(kVioDuplicate);
}

// Block-table entries of page indices [i0, i1) of one row, one per thread.
__device__ __forceinline__ void check_pages(const Geo& g, const int32_t* bt, int i0, int i1, int b, bool own)
{
    for (int i = i0 + (int)threadIdx.x; i < i1; i += (int)blockDim.x) {
        const int id = bt[i];
        if (id < 0 || id >= g.num_pages) report(kVioPage);
        else if (own && id < kOwnPages) claim(&g_page_owner[id], b);
    }
}

__global__ __launch_bounds__(256) void validate_clear_kernel(int npages, int nslots)
{
    const int n = max(npages, nslots);
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
        if (i < npages) g_page_owner[i] = 0;
        if (i < nslots) g_slot_owner[i] = 0;
    }
}

// One workgroup per sequence: row offsets, positions, slot, the pages the
// append writes and their owners.
__global__ __launch_bounds__(256) void validate_append_kernel(AppendArgs a)
{
    const Geo& g = a.g;
    const int b = blockIdx.x;
    const int r0 = a.cu_new[b], r1 = a.cu_new[b + 1];
    const int cap = g.max_pages * kPage;
    const int c = a.ctx_before[b], slot = a.slot_ids[b];
    if (threadIdx.x == 0) {
        if (r0 < 0 || r1 < r0 || r1 > a.total_new || (b == 0 && r0 != 0) ||
            (b == a.batch - 1 && r1 != a.total_new))
            report(kVioRows);
        if (c < 0 || (int64_t)c + max(r1 - r0, 0) > cap) report(kVioPosition);
        if (slot < 0 || slot >= g.max_slots) report(kVioSlot);
    }
    // what the append kernel writes, with its own clamps
    const int row0 = clampi(r0, 0, a.total_new), row1 = clampi(r1, row0, a.total_new);
    const int p0 = clampi(c, 0, cap), p1 = min(p0 + (row1 - row0), cap);
    if (p1 <= p0) return;
    const int s = clampi(slot, 0, g.max_slots - 1);
    check_pages(g, a.block_tables + (int64_t)s * g.max_pages, p0 / kPage, (p1 - 1) / kPage + 1, b, true);
    if (threadIdx.x == 0 && g.SR > 0 && s < kOwnSlots) claim(&g_slot_owner[s], b);
}

// One workgroup per sequence: length, slot and the pages of its context.
__global__ __launch_bounds__(256) void validate_decode_kernel(DecodeArgs a)
{
    const Geo& g = a.g;
    const int b = blockIdx.x;
    const int n = a.seq_lens[b], slot = a.slot_ids[b];
    if (threadIdx.x == 0) {
        if (n < 1 || n > a.max_ctx) report(kVioSeqLen);
        if (slot < 0 || slot >= g.max_slots) report(kVioSlot);
    }
    const int nc = clampi(n, 0, a.max_ctx);
    const int s = clampi(slot, 0, g.max_slots - 1);
    check_pages(g, a.block_tables + (int64_t)s * g.max_pages, 0, (nc + kPage - 1) / kPage, b, false);
}

// One thread per sequence: row offsets and lengths of the packed prompts.
__global__ __launch_bounds__(256) void validate_prefill_kernel(PrefillArgs a)
{
    for (int b = blockIdx.x * 256 + threadIdx.x; b < a.batch; b += gridDim.x * 256) {
        const int c0 = a.cu[b], c1 = a.cu[b + 1];
        if (c0 < 0 || c1 < c0 || c1 > a.total || (b == 0 && c0 != 0) || (b == a.batch - 1 && c1 != a.total))
            report(kVioRows);
        if (c1 - c0 > a.max_len) report(kVioSeqLen);
    }
}

}  // namespace kv4
