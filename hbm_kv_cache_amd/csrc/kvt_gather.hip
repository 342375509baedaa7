// kvt_gather.hip -- S5 top-k gather of selected K/V blocks from host-mapped planes into HBM.
//
// QSA-KVO: the K/V planes stay in pinned host memory and only the top-k selection crosses the
// host link, so the bytes read per decode step do not grow with context.  The planes are
// reached through a base pointer plus computed offsets -- token r of block p, head h lives at
// plane + p*block_stride + h*head_stride + r*token_stride -- so any layout of the host tier
// works.  Each (plane, head, slot) unit is the block's bt rows of hd*elem_bytes, and its HBM
// side is one contiguous [bt][hd] run.
//
// Pacing, measured on MI355X for 8 MiB per step: issuing every 16-byte load of the selection
// at once (all 8 MiB requested within microseconds) moves it at 43 GB/s, whatever the launch
// shape, load flavour or host layout; the same bytes with at most ~0.25-2 MiB in flight --
// each wave moving one 1 KiB wave-load at a time -- move at 54-55 GB/s, the link's rate for a
// transfer of that size.  So a grid of at most kMaxWaves wavefronts strides over 8 KiB pieces of
// the (slot, head, plane) units and each wave copies its piece one wave-load at a time.
#include <algorithm>

#include "kvt_internal.h"

namespace {

constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWavesPerGroup * kvt::kWave;
constexpr int kMaxWaves = 1024;           // ~1 MiB in flight at one 1 KiB wave-load each
constexpr int kPieceWords = 512;          // 16-byte words per piece (8 KiB)

// One piece: words [p0, p0 + n) of a unit whose rows are wpr words long.
__device__ __forceinline__ void copy_piece(const unsigned char *__restrict__ src,
                                           unsigned char *__restrict__ dst, int64_t token_stride,
                                           int wpr, int p0, int n, int lane)
{
#pragma unroll 1
    for (int w = p0 + lane; w < p0 + n; w += kvt::kWave) {
        const int row = w / wpr, col = w - row * wpr;
        const u32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(src + row * token_stride) + col);
        reinterpret_cast<u32x4 *>(dst)[w] = v;
        __asm__ volatile("" ::: "memory");   // keep the next load behind this one
    }
}

// unit u = (plane * kvh + h) * k + i; piece c of ceil(bt*wpr / kPieceWords) per unit
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const unsigned char *__restrict__ k_plane, const unsigned char *__restrict__ v_plane,
    int64_t n_blocks, int64_t block_stride, int64_t head_stride, int64_t token_stride,
    int slice_bytes, const int32_t *__restrict__ table, int bt, const int32_t *__restrict__ ids,
    int k, int kvh, int pieces_per_unit, int64_t n_pieces, unsigned char *__restrict__ k_out,
    unsigned char *__restrict__ v_out)
{
    const int lane = threadIdx.x & (kvt::kWave - 1);
    const int wpr = slice_bytes >> 4;
    const int unit_words = bt * wpr;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerGroup;
    for (int64_t pc = (int64_t)blockIdx.x * kWavesPerGroup +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         pc < n_pieces; pc += stride) {
        const int64_t u = pc / pieces_per_unit;
        const int c = (int)(pc - u * pieces_per_unit);
        const int plane = (int)(u / ((int64_t)kvh * k));
        const int hu = (int)(u - (int64_t)plane * kvh * k);   // h * k + i
        const int h = hu / k;
        const int b = ids[hu];
        if (b < 0 || b >= n_blocks)
            continue;
        const int64_t phys = table ? table[b] : b;
        if (phys < 0 || phys >= n_blocks)
            continue;
        const unsigned char *src = (plane ? v_plane : k_plane) + phys * block_stride +
                                   (int64_t)h * head_stride;
        unsigned char *dst = (plane ? v_out : k_out) + (int64_t)hu * bt * slice_bytes;
        const int p0 = c * kPieceWords;
        const int n = min(kPieceWords, unit_words - p0);
        copy_piece(src, dst, token_stride, wpr, p0, n, lane);
    }
}

// unit u = plane * n_used + p: page table[p] of that plane -> staged page p, in pieces of
// kPieceWords words; pages whose table entry lies outside [0, n_pages) are left as they are
__global__ __launch_bounds__(kThreads) void stage_pages_kernel(
    const unsigned char *__restrict__ k_plane, const unsigned char *__restrict__ v_plane,
    int64_t page_bytes, const int32_t *__restrict__ table, int n_used, int64_t n_pages,
    int64_t pieces_per_unit, int64_t n_pieces, unsigned char *__restrict__ k_out,
    unsigned char *__restrict__ v_out)
{
    const int lane = threadIdx.x & (kvt::kWave - 1);
    const int64_t words = page_bytes >> 4;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerGroup;
    for (int64_t pc = (int64_t)blockIdx.x * kWavesPerGroup +
                      __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         pc < n_pieces; pc += stride) {
        const int64_t u = pc / pieces_per_unit;
        const int64_t c = pc - u * pieces_per_unit;
        const int plane = (int)(u / n_used);
        const int p = (int)(u - (int64_t)plane * n_used);
        const int64_t phys = table[p];
        if (phys < 0 || phys >= n_pages)
            continue;
        const int64_t w0 = c * kPieceWords;
        const int n = (int)min<int64_t>(kPieceWords, words - w0);
        const unsigned char *src = (plane ? v_plane : k_plane) + phys * page_bytes + w0 * 16;
        unsigned char *dst = (plane ? v_out : k_out) + (int64_t)p * page_bytes + w0 * 16;
        copy_piece(src, dst, 0, n, 0, n, lane);
    }
}

}  // namespace

// QSA-KVO qsa_sparse_attend_rows_staged: the used pages copied into HBM once, in logical order.
extern "C" int kvt_stage_pages(const void *k_plane, const void *v_plane, int64_t page_bytes,
                               const int32_t *block_table, int32_t n_used, int64_t n_pages,
                               void *k_out, void *v_out, void *stream)
{
    if (page_bytes < 16 || page_bytes % 16 || n_used < 0 || n_pages < 0)
        return kvt::fail(KVT_EINVAL, "kvt_stage_pages: page_bytes=%lld n_used=%d n_pages=%lld",
                         (long long)page_bytes, n_used, (long long)n_pages);
    if (!k_plane || !k_out || !block_table || (!v_plane) != (!v_out))
        return kvt::fail(KVT_EINVAL, "kvt_stage_pages: null pointer (v_plane and v_out are "
                                     "both given or both NULL)");
    if (!kvt::aligned(k_plane, 16) || !kvt::aligned(k_out, 16) || !kvt::aligned(v_plane, 16) ||
        !kvt::aligned(v_out, 16))
        return kvt::fail(KVT_EALIGN, "kvt_stage_pages: planes and outputs must be 16-byte aligned");
    if (n_used == 0)
        return KVT_OK;
    const int planes = v_plane ? 2 : 1;
    const int64_t pieces_per_unit = (page_bytes / 16 + kPieceWords - 1) / kPieceWords;
    const int64_t n_pieces = pieces_per_unit * n_used * planes;
    const int64_t waves = std::min<int64_t>(n_pieces, kMaxWaves);
    const unsigned groups = (unsigned)((waves + kWavesPerGroup - 1) / kWavesPerGroup);
    hipLaunchKernelGGL(stage_pages_kernel, dim3(groups), dim3(kThreads), 0,
                       kvt::as_stream(stream), static_cast<const unsigned char *>(k_plane),
                       static_cast<const unsigned char *>(v_plane), page_bytes, block_table,
                       (int)n_used, n_pages, pieces_per_unit, n_pieces,
                       static_cast<unsigned char *>(k_out), static_cast<unsigned char *>(v_out));
    KVT_LAUNCHED("stage_pages_kernel");
    return KVT_OK;
}

// S5: QSA-KVO top-k gather (selected blocks' rows, host -> HBM).
extern "C" int kvt_gather_blocks(const void *k_plane, const void *v_plane, int64_t n_blocks,
                                 int32_t kvh, int32_t hd, int32_t elem_bytes,
                                 int64_t block_stride, int64_t head_stride, int64_t token_stride,
                                 const int32_t *block_table, int32_t bt, const int32_t *ids,
                                 int32_t k, void *k_out, void *v_out, void *stream)
{
    if (kvh < 1 || kvh > 65535 || hd < 1 || elem_bytes < 1 || bt < 1 || k < 1 || n_blocks < 0)
        return kvt::fail(KVT_EINVAL, "kvt_gather_blocks: kvh=%d hd=%d elem_bytes=%d bt=%d k=%d",
                         kvh, hd, elem_bytes, bt, k);
    const int64_t slice = (int64_t)hd * elem_bytes;
    if (slice % 16 || block_stride % 16 || head_stride % 16 || token_stride % 16 ||
        block_stride < 0 || head_stride < 0 || token_stride < 0)
        return kvt::fail(KVT_EALIGN,
                         "kvt_gather_blocks: head slice %lld and strides (%lld, %lld, %lld) must "
                         "be non-negative multiples of 16",
                         (long long)slice, (long long)block_stride, (long long)head_stride,
                         (long long)token_stride);
    if (!k_plane || !v_plane || !ids || !k_out || !v_out)
        return kvt::fail(KVT_EINVAL, "kvt_gather_blocks: null pointer");
    if (!kvt::aligned(k_plane, 16) || !kvt::aligned(v_plane, 16) || !kvt::aligned(k_out, 16) ||
        !kvt::aligned(v_out, 16))
        return kvt::fail(KVT_EALIGN, "kvt_gather_blocks: planes and outputs must be 16-byte aligned");
    if (slice * bt > (1ll << 30) || (int64_t)kvh * k > 0x3fffffff)
        return kvt::fail(KVT_ERANGE, "kvt_gather_blocks: block of %lld bytes too large",
                         (long long)(slice * bt));
    const int64_t unit_words = slice / 16 * bt;
    const int pieces_per_unit = (int)((unit_words + kPieceWords - 1) / kPieceWords);
    const int64_t n_pieces = (int64_t)pieces_per_unit * kvh * k * 2;
    const int64_t waves = std::min<int64_t>(n_pieces, kMaxWaves);
    const unsigned groups = (unsigned)((waves + kWavesPerGroup - 1) / kWavesPerGroup);
    hipLaunchKernelGGL(gather_kernel, dim3(groups), dim3(kThreads), 0, kvt::as_stream(stream),
                       static_cast<const unsigned char *>(k_plane),
                       static_cast<const unsigned char *>(v_plane), n_blocks, block_stride,
                       head_stride, token_stride, (int)slice, block_table, bt, ids, k, kvh,
                       pieces_per_unit, n_pieces, static_cast<unsigned char *>(k_out),
                       static_cast<unsigned char *>(v_out));
    KVT_LAUNCHED("gather_kernel");
    return KVT_OK;
}
