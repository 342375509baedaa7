// kvt_paged.hip -- the write side of the host tier: paged K/V writes and page copies.
//
// QSA-KVO, CacheLayer_qsa_offload: the K/V planes (and the indexer's raw key plane) live in
// pinned host memory as pages of page_size token rows, [n_pages][page_size][row_bytes], and
// the model appends new tokens through the block table (the paged cache update the page
// names).  Token t of sequence b lands at position p = cache_seqlens[b] + t, in row
// p % page_size of page block_table[b][p / page_size].  copy_page duplicates the first
// num_tokens rows of a page on the CPU -- the page's reasoning: a host memcpy leaves the host
// link to the attention gather -- after draining the stream, and copies the page's pooled rows
// (one per cr tokens, in HBM) on the device.  pool_rebuild_kernel is the pool kernel at the
// write head: after an append it recomputes the pooled rows of the blocks the new tokens fall
// in, from the raw key rows those blocks hold.
#include <algorithm>
#include <cstring>

#include "kvt_internal.h"

namespace {

constexpr int kMaxPlanes = 4;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWavesPerGroup * kvt::kWave;
constexpr int kMaxWaves = 1024;

struct Planes {
    const unsigned char *src[kMaxPlanes];
    unsigned char *dst[kMaxPlanes];
    int64_t row_bytes[kMaxPlanes];
};

// unit u = (plane * bsz + b) * seq + t: one wave copies that token's row of that plane
__global__ __launch_bounds__(kThreads) void paged_write_kernel(
    Planes pl, int n_planes, int bsz, int seq, const int32_t *__restrict__ cache_seqlens,
    const int32_t *__restrict__ block_table, int pages_per_seq, int page_size, int64_t n_pages)
{
    const int lane = threadIdx.x & (kvt::kWave - 1);
    const int64_t units = (int64_t)n_planes * bsz * seq;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerGroup;
    for (int64_t u = (int64_t)blockIdx.x * kWavesPerGroup +
                     __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         u < units; u += stride) {
        const int t = (int)(u % seq);
        const int64_t pb = u / seq;
        const int b = (int)(pb % bsz);
        const int plane = (int)(pb / bsz);
        const int64_t len = cache_seqlens[b];
        if (len < 0)
            continue;
        const int64_t pos = len + t;
        const int64_t slot = pos / page_size;
        if (slot >= pages_per_seq)
            continue;
        const int64_t page = block_table[(int64_t)b * pages_per_seq + slot];
        if (page < 0 || page >= n_pages)
            continue;
        const int64_t rb = pl.row_bytes[plane];
        const u32x4 *s = reinterpret_cast<const u32x4 *>(pl.src[plane] + ((int64_t)b * seq + t) * rb);
        u32x4 *d = reinterpret_cast<u32x4 *>(pl.dst[plane] +
                                             (page * page_size + pos % page_size) * rb);
        const int words = (int)(rb >> 4);
        for (int w = lane; w < words; w += kvt::kWave)
            __builtin_nontemporal_store(s[w], d + w);
    }
}

// fp64 -> fp16 bit pattern, rounding to nearest with ties to even, worked on the fp64 bits:
// keep 10 fraction bits (normal results) or count units of 2^-24 (subnormal ones) and round
// on the dropped bits.  A carry out of the fraction moves into the exponent field by the
// addition, which also turns 65504 + half an ulp and more into infinity.  NaN gives 0x7E00.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const int ex = (int)((u >> 52) & 0x7ff);
    const uint64_t frac = u & ((1ull << 52) - 1);
    if (ex == 0x7ff)
        return frac ? (uint16_t)0x7e00 : (uint16_t)(sign | 0x7c00u);
    const int e = ex - 1023;   // |x| in [2^e, 2^(e+1)) for normal fp64
    if (e > 15)
        return (uint16_t)(sign | 0x7c00u);
    if (e >= -14) {
        uint64_t q = frac >> 42;
        const uint64_t rem = frac & ((1ull << 42) - 1), half = 1ull << 41;
        q += (rem > half || (rem == half && (q & 1))) ? 1 : 0;
        return (uint16_t)(sign | (((uint32_t)(e + 15) << 10) + (uint32_t)q));
    }
    if (ex == 0)
        return (uint16_t)sign;                 // fp64 subnormal: far below 2^-25
    const int shift = 28 - e;                  // |x| / 2^-24 = significand >> shift, shift >= 43
    if (shift > 53)
        return (uint16_t)sign;                 // below half of 2^-24
    const uint64_t sig = (1ull << 52) | frac;
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
    q += (rem > half || (rem == half && (q & 1))) ? 1 : 0;
    return (uint16_t)(sign | (uint32_t)q);
}

// One wave per (sequence, k-th touched block): sequence b's append covers positions
// [len, len + seq), len = cache_seqlens[b]; block j = len / cr + k holds positions
// [j*cr, j*cr + cr), of which rows up to the write head exist.  Each lane averages one
// element over those rows (exact fp64 sum, one division, one rounding to fp16).
__global__ __launch_bounds__(256) void pool_rebuild_kernel(
    const uint16_t *__restrict__ raw, uint16_t *__restrict__ pooled, int dim, int bsz, int seq,
    const int32_t *__restrict__ cache_seqlens, const int32_t *__restrict__ block_table,
    int pages_per_seq, int page_size, int cr, int64_t n_pages, int blocks_per_seq)
{
    const int lane = threadIdx.x & (kvt::kWave - 1);
    const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t b = w / blocks_per_seq;
    if (b >= bsz)
        return;
    const int64_t len = cache_seqlens[b];
    if (len < 0)
        return;
    const int64_t end = len + seq;
    const int64_t j = len / cr + (w - b * blocks_per_seq);
    if (j > (end - 1) / cr)
        return;
    const int64_t first = j * cr;
    const int64_t slot = first / page_size;
    if (slot >= pages_per_seq)
        return;
    const int64_t page = block_table[b * pages_per_seq + slot];
    if (page < 0 || page >= n_pages)
        return;
    const int rows = (int)(end - first < cr ? end - first : cr);
    const int64_t row0 = first % page_size;
    const uint16_t *src = raw + (page * page_size + row0) * dim;
    uint16_t *dst = pooled + (page * (page_size / cr) + row0 / cr) * dim;
    for (int d = lane; d < dim; d += kvt::kWave) {
        double s = 0.0;
        for (int r = 0; r < rows; r++)
            s += (double)__builtin_bit_cast(_Float16, src[(int64_t)r * dim + d]);
        dst[d] = f64_to_f16_rne(s / (double)rows);
    }
}

int check_planes(const char *fn, const void *const *src, void *const *dst,
                 const int64_t *row_bytes, int32_t n_planes, Planes &pl)
{
    if (n_planes < 1 || n_planes > kMaxPlanes || !src || !dst || !row_bytes)
        return kvt::fail(KVT_EINVAL, "%s: n_planes=%d (1..%d) with plane arrays", fn, n_planes,
                         kMaxPlanes);
    for (int i = 0; i < n_planes; i++) {
        if (!src[i] || !dst[i])
            return kvt::fail(KVT_EINVAL, "%s: null plane %d", fn, i);
        if (row_bytes[i] < 16 || row_bytes[i] % 16 || row_bytes[i] > (1 << 24))
            return kvt::fail(KVT_EALIGN, "%s: row_bytes[%d]=%lld must be a multiple of 16 in "
                             "[16, 2^24]", fn, i, (long long)row_bytes[i]);
        if (!kvt::aligned(src[i], 16) || !kvt::aligned(dst[i], 16))
            return kvt::fail(KVT_EALIGN, "%s: plane %d not 16-byte aligned", fn, i);
        pl.src[i] = static_cast<const unsigned char *>(src[i]);
        pl.dst[i] = static_cast<unsigned char *>(dst[i]);
        pl.row_bytes[i] = row_bytes[i];
    }
    for (int i = n_planes; i < kMaxPlanes; i++) {
        pl.src[i] = nullptr;
        pl.dst[i] = nullptr;
        pl.row_bytes[i] = 0;
    }
    return KVT_OK;
}

}  // namespace

// QSA-KVO: the paged cache update writing new K/V (and raw key) rows into host-resident pages.
extern "C" int kvt_paged_write(const void *const *src, void *const *dst, const int64_t *row_bytes,
                               int32_t n_planes, int32_t bsz, int32_t seq,
                               const int32_t *cache_seqlens, const int32_t *block_table,
                               int32_t pages_per_seq, int32_t page_size, int64_t n_pages,
                               void *stream)
{
    Planes pl;
    int rc = check_planes("kvt_paged_write", src, dst, row_bytes, n_planes, pl);
    if (rc != KVT_OK)
        return rc;
    if (bsz < 0 || seq < 0 || pages_per_seq < 1 || page_size < 1 || n_pages < 0)
        return kvt::fail(KVT_EINVAL, "kvt_paged_write: bsz=%d seq=%d pages_per_seq=%d "
                         "page_size=%d n_pages=%lld", bsz, seq, pages_per_seq, page_size,
                         (long long)n_pages);
    if (!cache_seqlens || !block_table)
        return kvt::fail(KVT_EINVAL, "kvt_paged_write: null cache_seqlens or block_table");
    for (int i = 0; i < n_planes; i++)
        if (n_pages > 0 && (int64_t)page_size * row_bytes[i] > INT64_MAX / n_pages)
            return kvt::fail(KVT_ERANGE, "kvt_paged_write: plane %d too large", i);
    const int64_t units = (int64_t)n_planes * bsz * seq;
    if (units == 0)
        return KVT_OK;
    const int64_t waves = std::min<int64_t>(units, kMaxWaves);
    const unsigned groups = (unsigned)((waves + kWavesPerGroup - 1) / kWavesPerGroup);
    hipLaunchKernelGGL(paged_write_kernel, dim3(groups), dim3(kThreads), 0,
                       kvt::as_stream(stream), pl, n_planes, bsz, seq, cache_seqlens,
                       block_table, pages_per_seq, page_size, n_pages);
    KVT_LAUNCHED("paged_write_kernel");
    return KVT_OK;
}

// QSA-KVO CacheLayer_qsa_offload.copy_page: host planes by CPU memcpy, pooled rows on device.
extern "C" int kvt_copy_page(const void *const *src_host, void *const *dst_host,
                             const int64_t *row_bytes, int32_t n_planes, int64_t from_page,
                             int64_t to_page, int32_t page_size, int32_t num_tokens,
                             const void *src_pooled, void *dst_pooled, int64_t pooled_row_bytes,
                             int32_t cr, void *stream)
{
    if (n_planes < 0 || n_planes > kMaxPlanes || (n_planes > 0 && (!src_host || !dst_host ||
                                                                   !row_bytes)))
        return kvt::fail(KVT_EINVAL, "kvt_copy_page: n_planes=%d with plane arrays", n_planes);
    if (page_size < 1 || num_tokens < 0 || num_tokens > page_size || from_page < 0 ||
        to_page < 0)
        return kvt::fail(KVT_EINVAL, "kvt_copy_page: pages %lld -> %lld, %d of %d tokens",
                         (long long)from_page, (long long)to_page, num_tokens, page_size);
    for (int i = 0; i < n_planes; i++)
        if (!src_host[i] || !dst_host[i] || row_bytes[i] < 1)
            return kvt::fail(KVT_EINVAL, "kvt_copy_page: plane %d", i);
    const bool pooled = src_pooled || dst_pooled;
    if (pooled && (!src_pooled || !dst_pooled || pooled_row_bytes < 1 || cr < 1 ||
                   page_size % cr))
        return kvt::fail(KVT_EINVAL, "kvt_copy_page: pooled planes need both pointers, "
                         "row bytes and cr dividing page_size (cr=%d)", cr);
    // a page being read may still wait on a write of the stream, and one being written may
    // still be under a read: the host copy comes after everything enqueued so far
    KVT_HIP(hipStreamSynchronize(kvt::as_stream(stream)));
    for (int i = 0; i < n_planes; i++) {
        const int64_t page_bytes = (int64_t)page_size * row_bytes[i];
        const unsigned char *s = static_cast<const unsigned char *>(src_host[i]) +
                                 from_page * page_bytes;
        unsigned char *d = static_cast<unsigned char *>(dst_host[i]) + to_page * page_bytes;
        if (s != d)
            std::memmove(d, s, (size_t)num_tokens * (size_t)row_bytes[i]);
    }
    if (pooled) {
        const int64_t nb = (num_tokens + cr - 1) / cr;
        const int64_t page_bytes = (int64_t)(page_size / cr) * pooled_row_bytes;
        const unsigned char *s = static_cast<const unsigned char *>(src_pooled) +
                                 from_page * page_bytes;
        unsigned char *d = static_cast<unsigned char *>(dst_pooled) + to_page * page_bytes;
        if (nb > 0 && s != d)
            KVT_HIP(hipMemcpyAsync(d, s, (size_t)(nb * pooled_row_bytes),
                                   hipMemcpyDeviceToDevice, kvt::as_stream(stream)));
    }
    return KVT_OK;
}

// QSA-KVO, CacheLayer_qsa_offload docstring: the pool kernel at the write head.  Rebuilds the
// pooled rows of every block an append of seq tokens touched (reading the raw key plane only
// there) as the mean of the raw rows each block holds, rounded once to fp16.
extern "C" int kvt_pool_rebuild(const void *raw_k, void *pooled, int32_t dim, int32_t bsz,
                                int32_t seq, const int32_t *cache_seqlens,
                                const int32_t *block_table, int32_t pages_per_seq,
                                int32_t page_size, int32_t cr, int64_t n_pages, void *stream)
{
    if (dim < 1 || bsz < 0 || seq < 0 || pages_per_seq < 1 || page_size < 1 || cr < 1 ||
        cr > 512 || page_size % cr || n_pages < 0)
        return kvt::fail(KVT_EINVAL, "kvt_pool_rebuild: dim=%d bsz=%d seq=%d pages_per_seq=%d "
                         "page_size=%d cr=%d (1..512, dividing page_size) n_pages=%lld", dim, bsz,
                         seq, pages_per_seq, page_size, cr, (long long)n_pages);
    if (bsz == 0 || seq == 0 || n_pages == 0)
        return KVT_OK;
    if (!raw_k || !pooled || !cache_seqlens || !block_table)
        return kvt::fail(KVT_EINVAL, "kvt_pool_rebuild: null pointer");
    if (!kvt::aligned(raw_k, 2) || !kvt::aligned(pooled, 2))
        return kvt::fail(KVT_EALIGN, "kvt_pool_rebuild: planes must be 2-byte aligned");
    if ((int64_t)page_size * dim > INT64_MAX / n_pages / 2)
        return kvt::fail(KVT_ERANGE, "kvt_pool_rebuild: planes too large");
    // a sequence's append touches at most ceil(seq / cr) + 1 blocks (a partial one first)
    const int64_t blocks_per_seq = ((int64_t)seq + cr - 1) / cr + 1;
    const int64_t waves = (int64_t)bsz * blocks_per_seq;
    if (waves > 0x7fffffffll)
        return kvt::fail(KVT_ERANGE, "kvt_pool_rebuild: bsz x touched blocks too large");
    hipLaunchKernelGGL(pool_rebuild_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       kvt::as_stream(stream), static_cast<const uint16_t *>(raw_k),
                       static_cast<uint16_t *>(pooled), dim, bsz, seq, cache_seqlens,
                       block_table, pages_per_seq, page_size, cr, n_pages, (int)blocks_per_seq);
    KVT_LAUNCHED("pool_rebuild_kernel");
    return KVT_OK;
}
