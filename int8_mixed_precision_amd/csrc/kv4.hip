// kv4.hip -- host side of the KV4 C ABI (include/kv4.h): argument validation,
// pool sizing, work decomposition and kernel launches.  Nothing here allocates
// device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "kv4_append.hpp"
#include "kv4_common.hpp"
#include "kv4_decode.hpp"
#include "kv4_decode_mfma.hpp"
#include "kv4_prefill.hpp"
#ifdef KV4_VALIDATE
#include "kv4_validate.hpp"
#endif

// Workspace of kv4_decode_attn_noalloc: device memory reserved with the code
// object (every device that loads the library holds its own copy until the
// process ends).  Host code never passes this name to a kernel: on the host it
// is only a stand-in for the symbol, whose per-device address comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[KV4_NOALLOC_SCRATCH_BYTES];

struct kv4_cache {
    kv4_cache_desc desc;
    kv4::Geo geo;
    uint8_t* pages;
    size_t page_bytes;
    uint8_t* side;
    size_t side_bytes;
    int num_cus;                 // queried lazily at the first launch
};

namespace {

constexpr int kMaxSinkRecent = 1 << 16;

int validate_desc(const kv4_cache_desc* d)
{
    if (d == nullptr) return KV4_ERR_INVALID_ARG;
    if (d->num_layers < 1 || d->num_kv_heads < 1 || d->num_q_heads < 1 || d->head_dim < 1 ||
        d->page_size < 1 || d->group_size < 1 || d->sink < 0 || d->recent < 0 ||
        d->num_pages < 1 || d->max_slots < 1 || d->max_pages_per_seq < 1 ||
        d->num_waves < 0 || d->num_waves > kv4::kMaxWaves)
        return KV4_ERR_INVALID_ARG;
    if (d->pool_chunks < 0 || d->pool_chunks > kv4::kPoolMaxChunks ||
        (d->pool_chunks > 0 && (d->pool_chunks < kv4::kPoolMinChunks ||
                                (d->pool_chunks & (d->pool_chunks - 1)) != 0)))
        return KV4_ERR_INVALID_ARG;
    if (d->num_q_heads % d->num_kv_heads != 0) return KV4_ERR_INVALID_ARG;
    if (d->kind != KV4_KIND_MIXED && d->kind != KV4_KIND_BF16 && d->kind != KV4_KIND_KV8)
        return KV4_ERR_INVALID_ARG;
    if (d->flags & ~(KV4_FLAG_ROTATE_K | KV4_FLAG_INT_PATH | KV4_FLAG_VALU_DECODE)) return KV4_ERR_INVALID_ARG;
    if (d->head_dim % d->group_size != 0) return KV4_ERR_INVALID_ARG;
    // q/kv ratios: the matrix-core kernels take 1 .. 8 in halves of four q heads
    // (rows of heads past the ratio carry q = 0), and 16 as four halves on the
    // floating-point path of the mixed kind; the vector-ALU kernels take 1, 2,
    // 4 and 8; KV8 (below) takes 1 to 8.
    const int gqa = d->num_q_heads / d->num_kv_heads;
    const bool pow2 = gqa == 1 || gqa == 2 || gqa == 4 || gqa == 8;
    if (gqa > 8 && gqa != 16) return KV4_ERR_UNSUPPORTED;
    if (gqa == 16 && (d->kind != KV4_KIND_MIXED || (d->flags & (KV4_FLAG_INT_PATH | KV4_FLAG_VALU_DECODE))))
        return KV4_ERR_UNSUPPORTED;
    if (!pow2 && gqa != 16 && (d->flags & KV4_FLAG_VALU_DECODE)) return KV4_ERR_UNSUPPORTED;
    if (d->head_dim != kv4::kHeadDim || d->page_size != kv4::kPage) return KV4_ERR_UNSUPPORTED;
    if (d->group_size != 32 && d->group_size != 64 && d->group_size != 128) return KV4_ERR_UNSUPPORTED;
    // the rotation belongs to the quantized keys: the BF16 comparator has none
    if ((d->flags & KV4_FLAG_ROTATE_K) && d->kind != KV4_KIND_MIXED) return KV4_ERR_UNSUPPORTED;
    // the integer path reads the INT4 pages and the INT8 ring
    if ((d->flags & KV4_FLAG_INT_PATH) && d->kind != KV4_KIND_MIXED) return KV4_ERR_UNSUPPORTED;
    if (d->kind == KV4_KIND_KV8 && gqa > 8) return KV4_ERR_UNSUPPORTED;
    // KV8 pages are decoded on the matrix core only
    if (d->kind == KV4_KIND_KV8 && (d->flags & KV4_FLAG_VALU_DECODE)) return KV4_ERR_UNSUPPORTED;
    if ((int64_t)d->sink + d->recent > kMaxSinkRecent) return KV4_ERR_CAPACITY;
    if ((int64_t)d->max_pages_per_seq * kv4::kPage > INT32_MAX / 2) return KV4_ERR_CAPACITY;
    return KV4_OK;
}

void sizes(const kv4::Geo& g, size_t* page_pool, size_t* side_pool, size_t* per_layer_page)
{
    if (page_pool) *page_pool = (size_t)g.layer_pages * (size_t)g.num_layers;
    if (side_pool) *side_pool = (size_t)g.layer_side * (size_t)g.num_layers;
    if (per_layer_page) *per_layer_page = (size_t)g.pb * (size_t)g.Hkv;
}

int num_cus(kv4_cache* c)
{
    if (c->num_cus > 0) return c->num_cus;
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        c->num_cus = n;
    return c->num_cus > 0 ? c->num_cus : 256;
}

// Resident one-wave workgroups per compute unit of a vector-ALU decode kernel
// (at most 16), from the HIP occupancy query; 16 when the runtime cannot tell.
template <class K>
int resident_waves(K kernel, std::atomic<int>& known)
{
    int w = known.load(std::memory_order_relaxed);
    if (w > 0) return w;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 64, 0) != hipSuccess || nb <= 0) {
        (void)hipGetLastError();
        return 16;
    }
    w = std::min(nb, 16);
    known.store(w, std::memory_order_relaxed);
    return w;
}

int valu_waves_per_cu(const kv4_cache_desc& d, int gqa)
{
    static std::atomic<int> known[3][9];
    const int k = gqa == 1 ? 1 : gqa == 2 ? 2 : gqa == 4 ? 4 : 8;
    if (d.flags & KV4_FLAG_INT_PATH) {
        switch (k) {
            case 1: return resident_waves(kv4::decode_int_kv4_kernel<1>, known[0][1]);
            case 2: return resident_waves(kv4::decode_int_kv4_kernel<2>, known[0][2]);
            case 4: return resident_waves(kv4::decode_int_kv4_kernel<4>, known[0][4]);
            default: return resident_waves(kv4::decode_int_kv4_kernel<8>, known[0][8]);
        }
    }
    if (d.kind == KV4_KIND_MIXED) {
        switch (k) {
            case 1: return resident_waves(kv4::decode_valu_kv4_kernel<1>, known[1][1]);
            case 2: return resident_waves(kv4::decode_valu_kv4_kernel<2>, known[1][2]);
            case 4: return resident_waves(kv4::decode_valu_kv4_kernel<4>, known[1][4]);
            default: return resident_waves(kv4::decode_valu_kv4_kernel<8>, known[1][8]);
        }
    }
    switch (k) {
        case 1: return resident_waves(kv4::decode_valu_bf16_kernel<1>, known[2][1]);
        case 2: return resident_waves(kv4::decode_valu_bf16_kernel<2>, known[2][2]);
        case 4: return resident_waves(kv4::decode_valu_bf16_kernel<4>, known[2][4]);
        default: return resident_waves(kv4::decode_valu_bf16_kernel<8>, known[2][8]);
    }
}

// Resident waves per compute unit of the ratio-8 matrix-core kernel of the
// cache's path, group size and key basis.
int mfma8_waves_per_cu(const kv4_cache_desc& d)
{
    static std::atomic<int> known[3][2];
    static std::atomic<int> known_int[3][2];
    static std::atomic<int> known_bf16, known_kv8;
    if (d.kind == KV4_KIND_BF16) return resident_waves(kv4::decode_bf16_mfma8_kernel, known_bf16);
    if (d.kind == KV4_KIND_KV8) return resident_waves(kv4::decode_kv8_mfma8_kernel, known_kv8);
    const bool rot = (d.flags & KV4_FLAG_ROTATE_K) != 0;
    if (d.flags & KV4_FLAG_INT_PATH) {
        switch (d.group_size) {
            case 32:
                return rot ? resident_waves(kv4::decode_int_mfma8_kernel<32, true>, known_int[0][1])
                           : resident_waves(kv4::decode_int_mfma8_kernel<32, false>, known_int[0][0]);
            case 64:
                return rot ? resident_waves(kv4::decode_int_mfma8_kernel<64, true>, known_int[1][1])
                           : resident_waves(kv4::decode_int_mfma8_kernel<64, false>, known_int[1][0]);
            default:
                return rot ? resident_waves(kv4::decode_int_mfma8_kernel<128, true>, known_int[2][1])
                           : resident_waves(kv4::decode_int_mfma8_kernel<128, false>, known_int[2][0]);
        }
    }
    switch (d.group_size) {
        case 32:
            return rot ? resident_waves(kv4::decode_kv4_mfma8_kernel<32, true>, known[0][1])
                       : resident_waves(kv4::decode_kv4_mfma8_kernel<32, false>, known[0][0]);
        case 64:
            return rot ? resident_waves(kv4::decode_kv4_mfma8_kernel<64, true>, known[1][1])
                       : resident_waves(kv4::decode_kv4_mfma8_kernel<64, false>, known[1][0]);
        default:
            return rot ? resident_waves(kv4::decode_kv4_mfma8_kernel<128, true>, known[2][1])
                       : resident_waves(kv4::decode_kv4_mfma8_kernel<128, false>, known[2][0]);
    }
}

// Resident waves per compute unit of the ratio-16 matrix-core kernel.
int mfma16_waves_per_cu(const kv4_cache_desc& d)
{
    static std::atomic<int> known[3][2];
    const bool rot = (d.flags & KV4_FLAG_ROTATE_K) != 0;
    switch (d.group_size) {
        case 32:
            return rot ? resident_waves(kv4::decode_kv4_mfma16_kernel<32, true>, known[0][1])
                       : resident_waves(kv4::decode_kv4_mfma16_kernel<32, false>, known[0][0]);
        case 64:
            return rot ? resident_waves(kv4::decode_kv4_mfma16_kernel<64, true>, known[1][1])
                       : resident_waves(kv4::decode_kv4_mfma16_kernel<64, false>, known[1][0]);
        default:
            return rot ? resident_waves(kv4::decode_kv4_mfma16_kernel<128, true>, known[2][1])
                       : resident_waves(kv4::decode_kv4_mfma16_kernel<128, false>, known[2][0]);
    }
}

// Whether the decode of a cache runs on a matrix-core kernel of two or more
// four-head halves (q/kv ratio above 4).
bool uses_halves(const kv4_cache_desc& d)
{
    return d.num_q_heads > 4 * d.num_kv_heads && !(d.flags & KV4_FLAG_VALU_DECODE);
}

// Waves of the balanced decode partition: explicit, or 16 per compute unit
// (4 one-wave workgroups per SIMD, the occupancy the matrix-core decode
// kernels are built for), so that every wave of the grid is resident at once.
// The vector-ALU kernels hold more registers: as many waves per compute unit
// as the kernel keeps resident (at most 16), so that the partition's waves
// still run at once.
int decode_waves(const kv4_cache* c, int cus)
{
    if (c->desc.num_waves > 0) return c->desc.num_waves;
    // (the matrix-core kernels, q/kv ratios 1, 2 and 4, keep 16 resident)
    const int gqa = c->desc.num_q_heads / c->desc.num_kv_heads;
    if (uses_halves(c->desc))
        return (gqa > 8 ? mfma16_waves_per_cu(c->desc) : mfma8_waves_per_cu(c->desc)) * cus;
    if (gqa > 4 || (c->desc.flags & KV4_FLAG_VALU_DECODE)) return valu_waves_per_cu(c->desc, gqa) * cus;
    return 16 * cus;
}

// Most chunks of the dynamic pool (0: none, the default).  Measured at the
// batch-256 and 16 x 32k decode shapes, the pool is slower than the static
// shares alone: a chunk's atomic ticket takes 6-25 us under full HBM load and
// its extra records slow the merge.
int decode_pool_chunks(const kv4_cache* c, int waves)
{
    (void)waves;
    return c->desc.pool_chunks;
}

// Weight of a protected part in the partition, in INT4 tiles: an INT8 tile of
// 32 entries moves 9.7 KB against 5 KB and runs with its load latency exposed;
// measured at S + R = 132 and 260 (with the waves paced by progress), it
// costs about 3 INT4 tiles.
int prot_units(const kv4::Geo& g)
{
    if (g.kind != KV4_KIND_MIXED || g.SR == 0) return 0;
    return 3 * ((g.SR + kv4::kTile - 1) / kv4::kTile);
}

// Upper bound of the partition's total weight for a batch shape.
int64_t partition_weight(const kv4::Geo& g, int batch, int max_ctx)
{
    return (int64_t)batch * g.Hkv * ((max_ctx + kv4::kTile - 1) / kv4::kTile + 1 + prot_units(g));
}

// Records of the INT4 / BF16 runs (one per (sequence, kv head) and share),
// protected records, the (first, last) share header of every (sequence, kv
// head), then the pool counters at the next multiple of 256 bytes.
size_t records_floats(const kv4::Geo& g, int batch, int waves, int chunks)
{
    return ((size_t)2 * batch * g.Hkv + (size_t)waves + (size_t)chunks) * g.gqa * (g.d + kv4::kPartPad);
}

size_t counters_offset(const kv4::Geo& g, int batch, int waves, int chunks)
{
    const size_t end = records_floats(g, batch, waves, chunks) * sizeof(float) +
                       (size_t)batch * g.Hkv * 2 * sizeof(int32_t);
    return (end + 255) / 256 * 256;
}

size_t workspace_bytes(const kv4::Geo& g, int batch, int waves, int chunks)
{
    return counters_offset(g, batch, waves, chunks) +
           (size_t)kv4::kPoolCounters * kv4::kPoolStride * sizeof(uint32_t);
}

int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? KV4_OK : KV4_ERR_HIP;
}

// Vector-ALU kernels, used with KV4_FLAG_VALU_DECODE (ratios 1, 2, 4 and 8).
// The matrix-core kernels run the q heads of a kv head in halves of four (rows
// of heads past the ratio carry q = 0 and are not written): one half for
// ratios up to 4, two for 5 to 8 (decode_kv4_mfma8_kernel,
// decode_int_mfma8_kernel, decode_bf16_mfma8_kernel, decode_kv8_mfma8_kernel), four for 16
// (decode_kv4_mfma16_kernel).
template <int GQA>
void launch_decode_valu(const kv4::DecodeArgs& a, hipStream_t s)
{
    dim3 grid((unsigned)a.waves);
    if (a.g.kind == KV4_KIND_MIXED)
        hipLaunchKernelGGL(kv4::decode_valu_kv4_kernel<GQA>, grid, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(kv4::decode_valu_bf16_kernel<GQA>, grid, dim3(64), 0, s, a);
}

void launch_decode(const kv4::DecodeArgs& a, hipStream_t s)
{
#ifdef KV4_VALIDATE
    hipLaunchKernelGGL(kv4::validate_decode_kernel, dim3((unsigned)a.batch), dim3(256), 0, s, a);
#endif
    // the pool counters start every launch at zero (a kernel, not a memset, so
    // that the launch sequence can be captured in a graph)
    if (a.pool_chunks > 0) hipLaunchKernelGGL(kv4::pool_reset_kernel, dim3(1), dim3(64), 0, s, a.ctr);
    if (a.g.intp) {
        dim3 grid((unsigned)a.waves);
        if (a.g.gqa <= 4 && !a.g.valu) {
            switch (a.g.G) {
                case 32:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_int_mfma_kernel<32, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_int_mfma_kernel<32, false>), grid, dim3(64), 0, s, a);
                    break;
                case 64:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_int_mfma_kernel<64, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_int_mfma_kernel<64, false>), grid, dim3(64), 0, s, a);
                    break;
                default:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_int_mfma_kernel<128, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_int_mfma_kernel<128, false>), grid, dim3(64), 0, s, a);
                    break;
            }
            return;
        }
        if (a.g.gqa <= 8 && !a.g.valu) {
            switch (a.g.G) {
                case 32:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_int_mfma8_kernel<32, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_int_mfma8_kernel<32, false>), grid, dim3(64), 0, s, a);
                    break;
                case 64:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_int_mfma8_kernel<64, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_int_mfma8_kernel<64, false>), grid, dim3(64), 0, s, a);
                    break;
                default:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_int_mfma8_kernel<128, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_int_mfma8_kernel<128, false>), grid, dim3(64), 0, s, a);
                    break;
            }
            return;
        }
        switch (a.g.gqa) {
            case 1: hipLaunchKernelGGL(kv4::decode_int_kv4_kernel<1>, grid, dim3(64), 0, s, a); break;
            case 2: hipLaunchKernelGGL(kv4::decode_int_kv4_kernel<2>, grid, dim3(64), 0, s, a); break;
            case 4: hipLaunchKernelGGL(kv4::decode_int_kv4_kernel<4>, grid, dim3(64), 0, s, a); break;
            default: hipLaunchKernelGGL(kv4::decode_int_kv4_kernel<8>, grid, dim3(64), 0, s, a); break;
        }
        return;
    }
    if (a.g.gqa <= 4 && !a.g.valu) {
        dim3 grid((unsigned)a.waves);
        if (a.g.kind == KV4_KIND_MIXED) {
            switch (a.g.G) {
                case 32:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma_kernel<32, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_kv4_mfma_kernel<32, false>), grid, dim3(64), 0, s, a);
                    break;
                case 64:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma_kernel<64, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_kv4_mfma_kernel<64, false>), grid, dim3(64), 0, s, a);
                    break;
                default:
                    if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma_kernel<128, true>), grid, dim3(64), 0, s, a);
                    else hipLaunchKernelGGL((kv4::decode_kv4_mfma_kernel<128, false>), grid, dim3(64), 0, s, a);
                    break;
            }
        } else if (a.g.kind == KV4_KIND_KV8) {
            hipLaunchKernelGGL(kv4::decode_kv8_mfma_kernel, grid, dim3(64), 0, s, a);
        } else {
            hipLaunchKernelGGL(kv4::decode_bf16_mfma_kernel, grid, dim3(64), 0, s, a);
        }
        return;
    }
    if (a.g.gqa == 16 && !a.g.valu && a.g.kind == KV4_KIND_MIXED) {
        dim3 grid((unsigned)a.waves);
        switch (a.g.G) {
            case 32:
                if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma16_kernel<32, true>), grid, dim3(64), 0, s, a);
                else hipLaunchKernelGGL((kv4::decode_kv4_mfma16_kernel<32, false>), grid, dim3(64), 0, s, a);
                break;
            case 64:
                if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma16_kernel<64, true>), grid, dim3(64), 0, s, a);
                else hipLaunchKernelGGL((kv4::decode_kv4_mfma16_kernel<64, false>), grid, dim3(64), 0, s, a);
                break;
            default:
                if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma16_kernel<128, true>), grid, dim3(64), 0, s, a);
                else hipLaunchKernelGGL((kv4::decode_kv4_mfma16_kernel<128, false>), grid, dim3(64), 0, s, a);
                break;
        }
        return;
    }
    if (a.g.gqa <= 8 && !a.g.valu && a.g.kind == KV4_KIND_BF16) {
        hipLaunchKernelGGL(kv4::decode_bf16_mfma8_kernel, dim3((unsigned)a.waves), dim3(64), 0, s, a);
        return;
    }
    if (a.g.gqa <= 8 && a.g.kind == KV4_KIND_KV8) {
        hipLaunchKernelGGL(kv4::decode_kv8_mfma8_kernel, dim3((unsigned)a.waves), dim3(64), 0, s, a);
        return;
    }
    if (a.g.gqa <= 8 && !a.g.valu && a.g.kind == KV4_KIND_MIXED) {
        dim3 grid((unsigned)a.waves);
        switch (a.g.G) {
            case 32:
                if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma8_kernel<32, true>), grid, dim3(64), 0, s, a);
                else hipLaunchKernelGGL((kv4::decode_kv4_mfma8_kernel<32, false>), grid, dim3(64), 0, s, a);
                break;
            case 64:
                if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma8_kernel<64, true>), grid, dim3(64), 0, s, a);
                else hipLaunchKernelGGL((kv4::decode_kv4_mfma8_kernel<64, false>), grid, dim3(64), 0, s, a);
                break;
            default:
                if (a.g.rot) hipLaunchKernelGGL((kv4::decode_kv4_mfma8_kernel<128, true>), grid, dim3(64), 0, s, a);
                else hipLaunchKernelGGL((kv4::decode_kv4_mfma8_kernel<128, false>), grid, dim3(64), 0, s, a);
                break;
        }
        return;
    }
    switch (a.g.gqa) {
        case 1: launch_decode_valu<1>(a, s); break;
        case 2: launch_decode_valu<2>(a, s); break;
        case 4: launch_decode_valu<4>(a, s); break;
        default: launch_decode_valu<8>(a, s); break;
    }
}

// Validation and argument set-up shared by the decode phases.  `need_q` is
// false for the merge, which reads only seq_lens and the workspace.
int decode_args(kv4_cache* cache, int layer, const void* q_bf16, const int32_t* seq_lens,
                const int32_t* slot_ids, const int32_t* block_tables, int batch, int max_ctx,
                float sm_scale, const void* workspace, size_t ws_bytes, bool need_q,
                kv4::DecodeArgs& a)
{
    if (cache == nullptr || batch < 0 || max_ctx < 1) return KV4_ERR_INVALID_ARG;
    const kv4::Geo& g = cache->geo;
    if (need_q && (layer < 0 || layer >= g.num_layers)) return KV4_ERR_CAPACITY;
    if (batch > g.max_slots || max_ctx > g.max_pages * kv4::kPage) return KV4_ERR_CAPACITY;
    if (!std::isfinite(sm_scale)) return KV4_ERR_INVALID_ARG;
    if (batch > 0 && (seq_lens == nullptr ||
                      (need_q && (q_bf16 == nullptr || slot_ids == nullptr || block_tables == nullptr))))
        return KV4_ERR_INVALID_ARG;
    // the partition counts tiles and protected parts in 32-bit arithmetic
    if (partition_weight(g, batch, max_ctx) >= (int64_t)1 << 30) return KV4_ERR_CAPACITY;
    const int waves = decode_waves(cache, num_cus(cache));
    const int chunks = decode_pool_chunks(cache, waves);
    if (batch > 0 && (workspace == nullptr || ws_bytes < workspace_bytes(g, batch, waves, chunks)))
        return KV4_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return KV4_ERR_INVALID_ARG;
    a.g = g;
    a.layer = layer;
    a.q = static_cast<const uint16_t*>(q_bf16);
    a.seq_lens = seq_lens;
    a.slot_ids = slot_ids;
    a.block_tables = block_tables;
    a.batch = batch;
    a.max_ctx = max_ctx;
    a.waves = waves;
    a.prot_units = prot_units(g);
    a.pool_chunks = chunks;
    a.scale2 = sm_scale * 1.4426950408889634f;
    a.pages = cache->pages;
    a.side = cache->side;
    a.part = static_cast<float*>(const_cast<void*>(workspace));
    a.hdr = reinterpret_cast<int2*>(a.part + records_floats(g, batch, waves, chunks));
    a.ctr = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(const_cast<void*>(workspace)) +
                                        counters_offset(g, batch, waves, chunks));
    a.out = nullptr;
    a.out_dtype = KV4_OUT_F32;
    return KV4_OK;
}

void launch_merge(const kv4::DecodeArgs& a, hipStream_t s)
{
    int rows = a.batch * a.g.Hq;
    hipLaunchKernelGGL(kv4::merge_parts_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, a);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return KV4_ERR_HIP;
    }
    if (dev >= kMaxDevices) return KV4_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return KV4_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KV4_OK;
}

}  // namespace

extern "C" {

int kv4_cache_required_bytes(const kv4_cache_desc* desc, size_t* page_pool_bytes,
                             size_t* side_pool_bytes, size_t* page_bytes_per_layer)
{
    int st = validate_desc(desc);
    if (st != KV4_OK) return st;
    if (page_pool_bytes == nullptr && side_pool_bytes == nullptr && page_bytes_per_layer == nullptr)
        return KV4_ERR_INVALID_ARG;
    sizes(kv4::make_geo(*desc), page_pool_bytes, side_pool_bytes, page_bytes_per_layer);
    return KV4_OK;
}

int kv4_cache_create(const kv4_cache_desc* desc, void* page_pool, size_t page_pool_bytes,
                     void* side_pool, size_t side_pool_bytes, kv4_cache** out)
{
    if (out == nullptr) return KV4_ERR_INVALID_ARG;
    *out = nullptr;
    int st = validate_desc(desc);
    if (st != KV4_OK) return st;
    kv4::Geo g = kv4::make_geo(*desc);
    size_t need_pages = 0, need_side = 0;
    sizes(g, &need_pages, &need_side, nullptr);
    if (page_pool == nullptr) return KV4_ERR_INVALID_ARG;
    if (need_side > 0 && side_pool == nullptr) return KV4_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(page_pool) | reinterpret_cast<uintptr_t>(side_pool)) & 15u)
        return KV4_ERR_INVALID_ARG;
    if (page_pool_bytes < need_pages || side_pool_bytes < need_side) return KV4_ERR_CAPACITY;
    kv4_cache* c = new (std::nothrow) kv4_cache;
    if (c == nullptr) return KV4_ERR_CAPACITY;
    c->desc = *desc;
    c->geo = g;
    c->pages = static_cast<uint8_t*>(page_pool);
    c->page_bytes = page_pool_bytes;
    c->side = static_cast<uint8_t*>(side_pool);
    c->side_bytes = side_pool_bytes;
    c->num_cus = 0;
    *out = c;
    return KV4_OK;
}

int kv4_append(kv4_cache* cache, int layer, const void* k_bf16, const void* v_bf16,
               const int32_t* cu_new, const int32_t* ctx_before, const int32_t* slot_ids,
               const int32_t* block_tables, int batch, int total_new, kv4_stream_t stream)
{
    if (cache == nullptr || batch < 0 || total_new < 0) return KV4_ERR_INVALID_ARG;
    const kv4::Geo& g = cache->geo;
    if (layer < 0 || layer >= g.num_layers) return KV4_ERR_CAPACITY;
    if (batch > g.max_slots) return KV4_ERR_CAPACITY;
    if (batch == 0 || total_new == 0) return KV4_OK;
    if (k_bf16 == nullptr || v_bf16 == nullptr || cu_new == nullptr || ctx_before == nullptr ||
        slot_ids == nullptr || block_tables == nullptr)
        return KV4_ERR_INVALID_ARG;
    kv4::AppendArgs a;
    a.g = g;
    a.layer = layer;
    a.k = static_cast<const uint16_t*>(k_bf16);
    a.v = static_cast<const uint16_t*>(v_bf16);
    a.cu_new = cu_new;
    a.ctx_before = ctx_before;
    a.slot_ids = slot_ids;
    a.block_tables = block_tables;
    a.batch = batch;
    a.total_new = total_new;
    a.pages = cache->pages;
    a.side = cache->side;
    hipStream_t s = static_cast<hipStream_t>(stream);
#ifdef KV4_VALIDATE
    {
        const int np = std::min(g.num_pages, kv4::kOwnPages), ns = std::min(g.max_slots, kv4::kOwnSlots);
        hipLaunchKernelGGL(kv4::validate_clear_kernel, dim3((unsigned)std::min(1024, (std::max(np, ns) + 255) / 256)),
                           dim3(256), 0, s, np, ns);
        hipLaunchKernelGGL(kv4::validate_append_kernel, dim3((unsigned)batch), dim3(256), 0, s, a);
    }
#endif
    // parallelism along each sequence sized by the mean number of new tokens
    int64_t mean_new = ((int64_t)total_new + batch - 1) / batch;
    if (g.kind == KV4_KIND_MIXED) {
        // waves per (sequence, kv head): one per four half pages of the mean
        // sequence, so that a wave quantizes several half pages with the next
        // one's loads in flight, at most 128, but enough for about 6,144
        // waves in all when the batch has few (sequence, kv head) pairs.
        // Measured against one wave per half page up to 256: 190 against
        // 197 us for the populate of 32 histories (145,101 tokens), 322
        // against 408 us for 256 sequences of 1,024 tokens, and 46 against
        // 52 us for one sequence of 32,768.
        const int64_t pairs = (int64_t)batch * g.Hkv;
        const int64_t cap = std::max<int64_t>(128, (6144 + pairs - 1) / pairs);
        int gx = (int)std::min<int64_t>((mean_new + 4 * kv4::kHalf - 1) / (4 * kv4::kHalf) + 1,
                                        std::min<int64_t>(cap, 4096));
        if (mean_new <= 1) gx = 1;
        dim3 grid(gx, g.Hkv, batch);
        switch (g.G) {
            case 32: hipLaunchKernelGGL(kv4::append_kv4_kernel<32>, grid, dim3(64), 0, s, a); break;
            case 64: hipLaunchKernelGGL(kv4::append_kv4_kernel<64>, grid, dim3(64), 0, s, a); break;
            default: hipLaunchKernelGGL(kv4::append_kv4_kernel<128>, grid, dim3(64), 0, s, a); break;
        }
    } else {
        int gx = (int)std::min<int64_t>(mean_new, 256);
        dim3 grid(gx, g.Hkv, batch);
        if (g.kind == KV4_KIND_KV8)
            hipLaunchKernelGGL(kv4::append_kv8_kernel, grid, dim3(64), 0, s, a);
        else
            hipLaunchKernelGGL(kv4::append_bf16_kernel, grid, dim3(64), 0, s, a);
    }
    return launch_status();
}

int kv4_decode_partition(const kv4_cache* cache, int* waves, int* pool_chunks)
{
    if (cache == nullptr || (waves == nullptr && pool_chunks == nullptr)) return KV4_ERR_INVALID_ARG;
    const int w = decode_waves(cache, num_cus(const_cast<kv4_cache*>(cache)));
    if (waves) *waves = w;
    if (pool_chunks) *pool_chunks = decode_pool_chunks(cache, w);
    return KV4_OK;
}

int kv4_decode_workspace_bytes(const kv4_cache* cache, int batch, int max_ctx, size_t* bytes)
{
    if (cache == nullptr || bytes == nullptr || batch < 0 || max_ctx < 1) return KV4_ERR_INVALID_ARG;
    const kv4::Geo& g = cache->geo;
    if (batch > g.max_slots || max_ctx > g.max_pages * kv4::kPage) return KV4_ERR_CAPACITY;
    if (partition_weight(g, batch, max_ctx) >= (int64_t)1 << 30) return KV4_ERR_CAPACITY;
    const int waves = decode_waves(cache, num_cus(const_cast<kv4_cache*>(cache)));
    *bytes = workspace_bytes(g, batch, waves, decode_pool_chunks(cache, waves));
    return KV4_OK;
}

int kv4_decode_partials(kv4_cache* cache, int layer, const void* q_bf16, const int32_t* seq_lens,
                        const int32_t* slot_ids, const int32_t* block_tables, int batch,
                        int max_ctx, float sm_scale, void* workspace, size_t workspace_bytes_,
                        kv4_stream_t stream)
{
    kv4::DecodeArgs a;
    int st = decode_args(cache, layer, q_bf16, seq_lens, slot_ids, block_tables, batch, max_ctx,
                         sm_scale, workspace, workspace_bytes_, true, a);
    if (st != KV4_OK || batch == 0) return st;
    launch_decode(a, static_cast<hipStream_t>(stream));
    return launch_status();
}

int kv4_decode_merge(kv4_cache* cache, const int32_t* seq_lens, int batch, int max_ctx, void* out,
                     int out_dtype, const void* workspace, size_t workspace_bytes_,
                     kv4_stream_t stream)
{
    if (out_dtype != KV4_OUT_F32 && out_dtype != KV4_OUT_BF16) return KV4_ERR_INVALID_ARG;
    kv4::DecodeArgs a;
    int st = decode_args(cache, 0, nullptr, seq_lens, nullptr, nullptr, batch, max_ctx, 1.0f,
                         workspace, workspace_bytes_, false, a);
    if (st != KV4_OK || batch == 0) return st;
    if (out == nullptr) return KV4_ERR_INVALID_ARG;
    a.out = out;
    a.out_dtype = out_dtype;
    launch_merge(a, static_cast<hipStream_t>(stream));
    return launch_status();
}

int kv4_decode_attn(kv4_cache* cache, int layer, const void* q_bf16, const int32_t* seq_lens,
                    const int32_t* slot_ids, const int32_t* block_tables, int batch, int max_ctx,
                    float sm_scale, void* out, int out_dtype, void* workspace, size_t workspace_bytes_,
                    kv4_stream_t stream)
{
    if (out_dtype != KV4_OUT_F32 && out_dtype != KV4_OUT_BF16) return KV4_ERR_INVALID_ARG;
    kv4::DecodeArgs a;
    int st = decode_args(cache, layer, q_bf16, seq_lens, slot_ids, block_tables, batch, max_ctx,
                         sm_scale, workspace, workspace_bytes_, true, a);
    if (st != KV4_OK || batch == 0) return st;
    if (out == nullptr) return KV4_ERR_INVALID_ARG;
    a.out = out;
    a.out_dtype = out_dtype;
    hipStream_t s = static_cast<hipStream_t>(stream);
    launch_decode(a, s);
    st = launch_status();
    if (st != KV4_OK) return st;
    launch_merge(a, s);
    return launch_status();
}

int kv4_decode_attn_noalloc(kv4_cache* cache, int layer, const void* q_bf16, const int32_t* seq_lens,
                            const int32_t* slot_ids, const int32_t* block_tables, int batch,
                            int max_ctx, float sm_scale, void* out, int out_dtype,
                            kv4_stream_t stream)
{
    if (out_dtype != KV4_OUT_F32 && out_dtype != KV4_OUT_BF16) return KV4_ERR_INVALID_ARG;
    if (cache == nullptr || batch < 0 || max_ctx < 1) return KV4_ERR_INVALID_ARG;
    size_t need = 0;
    int st = kv4_decode_workspace_bytes(cache, batch, max_ctx, &need);
    if (st != KV4_OK) return st;
    if (need > (size_t)KV4_NOALLOC_SCRATCH_BYTES) return KV4_ERR_CAPACITY;
    if (batch == 0) return KV4_OK;
    void* ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != KV4_OK) return st;
    kv4::DecodeArgs a;
    st = decode_args(cache, layer, q_bf16, seq_lens, slot_ids, block_tables, batch, max_ctx,
                     sm_scale, ws, (size_t)KV4_NOALLOC_SCRATCH_BYTES, true, a);
    if (st != KV4_OK) return st;
    if (out == nullptr) return KV4_ERR_INVALID_ARG;
    a.out = out;
    a.out_dtype = out_dtype;
    hipStream_t s = static_cast<hipStream_t>(stream);
    launch_decode(a, s);
    st = launch_status();
    if (st != KV4_OK) return st;
    launch_merge(a, s);
    return launch_status();
}

int kv4_prefill_attn(const kv4_cache* cache, const void* q_bf16, const void* k_bf16,
                     const void* v_bf16, const int32_t* cu_seqlens, int batch, int total,
                     int max_seqlen, float sm_scale, void* out, int out_dtype, kv4_stream_t stream)
{
    if (cache == nullptr || q_bf16 == nullptr || k_bf16 == nullptr || v_bf16 == nullptr ||
        cu_seqlens == nullptr || out == nullptr)
        return KV4_ERR_INVALID_ARG;
    if (batch < 1 || total < 0 || max_seqlen < 1 || !std::isfinite(sm_scale)) return KV4_ERR_INVALID_ARG;
    if (out_dtype != KV4_OUT_F32 && out_dtype != KV4_OUT_BF16) return KV4_ERR_INVALID_ARG;
    // grid (q heads x 16 query blocks, sequences, groups of 16 query blocks): the
    // sequences are limited to 65,536, and query positions to 65,536 blocks
    if (max_seqlen > 65536 * kv4::kPreQ || batch > 65536) return KV4_ERR_CAPACITY;
    if (total == 0) return KV4_OK;
    const kv4_cache_desc& d = cache->desc;
    kv4::PrefillArgs a;
    a.q = static_cast<const uint16_t*>(q_bf16);
    a.k = static_cast<const uint16_t*>(k_bf16);
    a.v = static_cast<const uint16_t*>(v_bf16);
    a.cu = cu_seqlens;
    a.out = out;
    a.out_bf16 = out_dtype == KV4_OUT_BF16;
    a.batch = batch;
    a.total = total;
    a.max_len = max_seqlen;
    a.Hq = d.num_q_heads;
    a.Hkv = d.num_kv_heads;
    a.gqa = d.num_q_heads / d.num_kv_heads;
    a.scale2 = sm_scale * 1.4426950408889634f;
    constexpr int kGroupQ = kv4::kPreGroup * kv4::kPreQ;
    dim3 grid((unsigned)(a.Hq * kv4::kPreGroup), (unsigned)batch, (unsigned)((max_seqlen + kGroupQ - 1) / kGroupQ));
#ifdef KV4_VALIDATE
    hipLaunchKernelGGL(kv4::validate_prefill_kernel, dim3((unsigned)std::min(1024, (batch + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
#endif
    hipLaunchKernelGGL((kv4::prefill_attn_kernel<kv4::kPrefillKeys, kv4::kPrefillRows>), grid, dim3(256), 0,
                       static_cast<hipStream_t>(stream), a);
    return launch_status();
}

int kv4_validate_report(uint32_t* violations)
{
    if (violations == nullptr) return KV4_ERR_INVALID_ARG;
    *violations = 0;
#ifdef KV4_VALIDATE
    uint32_t v = 0;
    const uint32_t zero = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(kv4::g_violations), sizeof v, 0, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpyToSymbol(HIP_SYMBOL(kv4::g_violations), &zero, sizeof zero, 0, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        return KV4_ERR_HIP;
    }
    *violations = v;
    return KV4_OK;
#else
    return KV4_ERR_UNSUPPORTED;
#endif
}

int kv4_cache_free(kv4_cache* cache)
{
    delete cache;
    return KV4_OK;
}

const char* kv4_status_string(int status)
{
    switch (status) {
        case KV4_OK: return "KV4_OK: success";
        case KV4_ERR_INVALID_ARG: return "KV4_ERR_INVALID_ARG: invalid argument";
        case KV4_ERR_UNSUPPORTED: return "KV4_ERR_UNSUPPORTED: valid request not supported by the library";
        case KV4_ERR_CAPACITY: return "KV4_ERR_CAPACITY: exceeds a declared capacity";
        case KV4_ERR_WORKSPACE: return "KV4_ERR_WORKSPACE: workspace missing or too small";
        case KV4_ERR_HIP: return "KV4_ERR_HIP: HIP runtime error";
        default: return "unknown kv4 status";
    }
}

}  // extern "C"
