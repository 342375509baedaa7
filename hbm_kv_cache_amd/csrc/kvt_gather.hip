// kvt_gather.hip -- S5 top-k gather of selected K/V blocks from host-mapped planes into HBM.
//
// QSA-KVO: the K/V planes stay in pinned host memory and only the top-k selection crosses the
// host link, so the bytes read per decode step do not grow with context.  Per (plane, head,
// slot) one workgroup copies the block's bt rows of hd*elem_bytes (256 bytes for 128 bf16
// values, at a host row stride of kvh*hd*elem_bytes).  Every thread issues all of its 16-byte
// loads before its first store, so each workgroup keeps its whole block in flight on the link;
// the HBM side is one contiguous [bt][hd] run per unit.
#include "kvt_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// grid = (k, kvh, 2): x = selection slot, y = head, z = plane (0 = K, 1 = V)
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const unsigned char *__restrict__ k_plane, const unsigned char *__restrict__ v_plane,
    int64_t n_blocks, int64_t row_stride, int slice_bytes, const int32_t *__restrict__ table,
    int bt, const int32_t *__restrict__ ids, int k, unsigned char *__restrict__ k_out,
    unsigned char *__restrict__ v_out)
{
    const int i = blockIdx.x, h = blockIdx.y;
    const int b = ids[h * k + i];
    if (b < 0 || b >= n_blocks)
        return;
    const int64_t phys = table ? table[b] : b;
    if (phys < 0 || phys >= n_blocks)
        return;
    const unsigned char *src = (blockIdx.z ? v_plane : k_plane) + phys * bt * row_stride +
                               (int64_t)h * slice_bytes;
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
                    reinterpret_cast<const u32x4 *>(src + row * row_stride) + col);
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
extern "C" int kvt_gather_blocks(const void *k_plane, const void *v_plane, int64_t n_tok,
                                 int32_t kvh, int32_t hd, int32_t elem_bytes, int64_t row_stride,
                                 const int32_t *block_table, int32_t bt, const int32_t *ids,
                                 int32_t k, void *k_out, void *v_out, void *stream)
{
    if (kvh < 1 || kvh > 65535 || hd < 1 || elem_bytes < 1 || bt < 1 || k < 1 || n_tok < 0)
        return kvt::fail(KVT_EINVAL, "kvt_gather_blocks: kvh=%d hd=%d elem_bytes=%d bt=%d k=%d",
                         kvh, hd, elem_bytes, bt, k);
    const int64_t slice = (int64_t)hd * elem_bytes;
    if (slice % 16 || row_stride % 16 || row_stride < slice * kvh)
        return kvt::fail(KVT_EALIGN,
                         "kvt_gather_blocks: head slice %lld and row stride %lld must be "
                         "multiples of 16 with stride >= kvh*slice",
                         (long long)slice, (long long)row_stride);
    if (!k_plane || !v_plane || !ids || !k_out || !v_out)
        return kvt::fail(KVT_EINVAL, "kvt_gather_blocks: null pointer");
    if (!kvt::aligned(k_plane, 16) || !kvt::aligned(v_plane, 16) || !kvt::aligned(k_out, 16) ||
        !kvt::aligned(v_out, 16))
        return kvt::fail(KVT_EALIGN, "kvt_gather_blocks: planes and outputs must be 16-byte aligned");
    if (slice * bt > (1ll << 30) || k > 0x7fffffff)
        return kvt::fail(KVT_ERANGE, "kvt_gather_blocks: block of %lld bytes too large",
                         (long long)(slice * bt));
    const int64_t n_blocks = n_tok / bt;
    hipLaunchKernelGGL(gather_kernel, dim3(k, kvh, 2), dim3(kThreads), 0, kvt::as_stream(stream),
                       static_cast<const unsigned char *>(k_plane),
                       static_cast<const unsigned char *>(v_plane), n_blocks, row_stride,
                       (int)slice, block_table, bt, ids, k, static_cast<unsigned char *>(k_out),
                       static_cast<unsigned char *>(v_out));
    KVT_LAUNCHED("gather_kernel");
    return KVT_OK;
}
