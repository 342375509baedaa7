// kvt_gather.hip -- S5 top-k gather of selected K/V blocks from host-mapped planes into HBM.
//
// QSA-KVO: the K/V planes stay in pinned host memory and only the top-k selection crosses the
// host link, so the bytes read per decode step do not grow with context.  The planes are
// reached through a base pointer plus computed offsets -- token r of block p, head h lives at
// plane + p*block_stride + h*head_stride + r*token_stride -- so any layout of the host tier
// works.  Per (plane, head, slot) one workgroup copies the block's bt rows of hd*elem_bytes;
// every thread issues all of its 16-byte loads before its first store, so each workgroup keeps
// its whole block in flight on the link, and the HBM side is one contiguous [bt][hd] run.
//
// The host-link rate depends on how long the contiguous runs are: a token-major plane gives
// 256-byte runs (one head of one token), a block-local head-major plane [block][head][token]
// gives one run of bt*hd*elem_bytes (16 KiB) per unit.
#include "kvt_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// grid = (k, kvh, 2): x = selection slot, y = head, z = plane (0 = K, 1 = V)
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const unsigned char *__restrict__ k_plane, const unsigned char *__restrict__ v_plane,
    int64_t n_blocks, int64_t block_stride, int64_t head_stride, int64_t token_stride,
    int slice_bytes, const int32_t *__restrict__ table, int bt, const int32_t *__restrict__ ids,
    int k, unsigned char *__restrict__ k_out, unsigned char *__restrict__ v_out)
{
    const int i = blockIdx.x, h = blockIdx.y;
    const int b = ids[h * k + i];
    if (b < 0 || b >= n_blocks)
        return;
    const int64_t phys = table ? table[b] : b;
    if (phys < 0 || phys >= n_blocks)
        return;
    const unsigned char *src = (blockIdx.z ? v_plane : k_plane) + phys * block_stride +
                               (int64_t)h * head_stride;
    unsigned char *dst = (blockIdx.z ? v_out : k_out) +
                         ((int64_t)h * k + i) * (int64_t)bt * slice_bytes;
    const int wpr = slice_bytes >> 4;  // 16-byte words per row slice
    const int nw = bt * wpr;
    for (int w0 = threadIdx.x; w0 < nw; w0 += kUnroll * kThreads) {
        u32x4 r[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int w = w0 + u * kThreads;
            if (w < nw) {
                const int row = w / wpr, col = w - row * wpr;
                r[u] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(src + row * token_stride) + col);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int w = w0 + u * kThreads;
            if (w < nw)
                reinterpret_cast<u32x4 *>(dst)[w] = r[u];
        }
    }
}

}  // namespace

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
    if (slice * bt > (1ll << 30) || k > 0x7fffffff)
        return kvt::fail(KVT_ERANGE, "kvt_gather_blocks: block of %lld bytes too large",
                         (long long)(slice * bt));
    hipLaunchKernelGGL(gather_kernel, dim3(k, kvh, 2), dim3(kThreads), 0, kvt::as_stream(stream),
                       static_cast<const unsigned char *>(k_plane),
                       static_cast<const unsigned char *>(v_plane), n_blocks, block_stride,
                       head_stride, token_stride, (int)slice, block_table, bt, ids, k,
                       static_cast<unsigned char *>(k_out), static_cast<unsigned char *>(v_out));
    KVT_LAUNCHED("gather_kernel");
    return KVT_OK;
}
