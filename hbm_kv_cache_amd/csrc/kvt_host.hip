// kvt_host.hip -- host-only entry points: version, errors, pinned host tier, pointer tables.
#include <cstring>
#include <string>

#include "kvt_internal.h"

namespace kvt {

static thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

}  // namespace kvt

using kvt::fail;

extern "C" int kvt_abi_version(void) { return KVT_ABI_VERSION; }

extern "C" const char *kvt_last_error(void) { return kvt::g_last_error; }

// Host tier: pinned, device-mapped host memory (vLLM-CPU pin_mmap_region / QSA-KVO alloc).
extern "C" int kvt_host_alloc(size_t bytes, unsigned flags, void **host_ptr, void **dev_ptr)
{
    if (!bytes || !host_ptr || !dev_ptr)
        return fail(KVT_EINVAL, "kvt_host_alloc: bytes=%zu host_ptr=%p dev_ptr=%p", bytes,
                    (void *)host_ptr, (void *)dev_ptr);
    unsigned hf = hipHostMallocMapped | hipHostMallocPortable;
    switch (flags) {
    case KVT_HOST_COHERENT: hf |= hipHostMallocCoherent; break;
    case KVT_HOST_NONCOHERENT: hf |= hipHostMallocNonCoherent; break;
    case KVT_HOST_WRITECOMBINED: hf |= hipHostMallocWriteCombined; break;
    default: return fail(KVT_EINVAL, "kvt_host_alloc: unknown flags %u", flags);
    }
    void *p = nullptr;
    hipError_t e = hipHostMalloc(&p, bytes, hf);
    if (e != hipSuccess || !p) {
        (void)hipGetLastError();  // do not leave the error for the next call to report
        return fail(KVT_ENOMEM, "kvt_host_alloc(%zu bytes): %s", bytes, hipGetErrorString(e));
    }
    void *d = nullptr;
    e = hipHostGetDevicePointer(&d, p, 0);
    if (e != hipSuccess || !d) {
        (void)hipGetLastError();
        (void)hipHostFree(p);
        return fail(KVT_EHIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
    }
    // pages come back from the OS zeroed only on first mapping; make it a guarantee
    std::memset(p, 0, bytes);
    *host_ptr = p;
    *dev_ptr = d;
    return KVT_OK;
}

extern "C" int kvt_host_free(void *host_ptr)
{
    if (!host_ptr)
        return KVT_OK;
    KVT_HIP(hipHostFree(host_ptr));
    return KVT_OK;
}

// S1: vLLM-CPU compute_sub_block_ptrs.  Sub-block j of block b: base + b*row_stride + j*page.
extern "C" int kvt_sub_block_ptrs(uint64_t base, uint64_t row_stride, uint64_t page_bytes,
                                  const int64_t *block_ids, int64_t n_ids, int32_t bpc,
                                  int32_t skip, uint64_t *out, int64_t n_out)
{
    if (bpc < 1 || skip < 0 || skip >= bpc)
        return fail(KVT_EINVAL, "kvt_sub_block_ptrs: need 0 <= skip < bpc (skip=%d bpc=%d)",
                    skip, bpc);
    if (n_ids < 0 || n_out < 0 || (n_out && (!block_ids || !out)))
        return fail(KVT_EINVAL, "kvt_sub_block_ptrs: bad counts or null tables");
    if (n_out > n_ids * (int64_t)bpc - skip)
        return fail(KVT_ERANGE, "kvt_sub_block_ptrs: %lld sub-blocks requested, %lld listed",
                    (long long)n_out, (long long)(n_ids * (int64_t)bpc - skip));
    if (bpc == 1) {
        for (int64_t i = 0; i < n_out; i++) {
            if (block_ids[i] < 0)
                return fail(KVT_ERANGE, "kvt_sub_block_ptrs: negative block id at %lld",
                            (long long)i);
            out[i] = base + (uint64_t)block_ids[i] * row_stride;
        }
        return KVT_OK;
    }
    // walk the block-major list from the skip on: block i = (o+skip)/bpc, sub-block j = rest
    int64_t i = skip / bpc;  // == 0
    int32_t j = skip;
    uint64_t row = 0;
    bool have_row = false;
    for (int64_t o = 0; o < n_out; o++) {
        if (!have_row) {
            if (block_ids[i] < 0)
                return fail(KVT_ERANGE, "kvt_sub_block_ptrs: negative block id at %lld",
                            (long long)i);
            row = base + (uint64_t)block_ids[i] * row_stride;
            have_row = true;
        }
        out[o] = row + (uint64_t)j * page_bytes;
        if (++j == bpc) {
            j = 0;
            ++i;
            have_row = false;
        }
    }
    return KVT_OK;
}

extern "C" int64_t kvt_chunks_consumed(int64_t n, int32_t skip, int32_t bpc)
{
    if (bpc < 1 || n < 0 || skip < 0)
        return -1;
    return (n + skip + bpc - 1) / bpc;
}

// Workspace sizes by operation: a dispatcher over the per-op size functions.
extern "C" size_t kvt_workspace_bytes(int32_t op, const int64_t *dims, int32_t n_dims)
{
    static const int32_t want[] = {-1, 3, 3, 4, 3};   // dims per op (NONE_NEEDED: any)
    if (op < KVT_OP_NONE_NEEDED || op > KVT_OP_PREFILL_STATE) {
        kvt::fail(KVT_EINVAL, "kvt_workspace_bytes: op=%d", op);
        return 0;
    }
    if (op == KVT_OP_NONE_NEEDED)
        return 0;
    if (!dims || n_dims != want[op]) {
        kvt::fail(KVT_EINVAL, "kvt_workspace_bytes: op %d takes %d dims, got %d", op, want[op],
                  dims ? n_dims : 0);
        return 0;
    }
    // every dimension but the 64-bit ones (n_blocks, n_kv, n_q) must fit int32
    auto i32 = [&](int i) { return dims[i] >= INT32_MIN && dims[i] <= INT32_MAX; };
    bool ok = true;
    switch (op) {
    case KVT_OP_INDEX_TOPK: ok = i32(1) && i32(2); break;
    case KVT_OP_ATTN_DECODE: ok = i32(0) && i32(1); break;
    case KVT_OP_SPARSE_ROWS: ok = i32(0) && i32(1) && i32(2) && i32(3); break;
    case KVT_OP_PREFILL_STATE: ok = i32(1) && i32(2); break;
    }
    if (!ok) {
        kvt::fail(KVT_ERANGE, "kvt_workspace_bytes: op %d: a dimension exceeds int32", op);
        return 0;
    }
    switch (op) {
    case KVT_OP_INDEX_TOPK:
        return kvt_index_topk_ws_bytes(dims[0], (int32_t)dims[1], (int32_t)dims[2]);
    case KVT_OP_ATTN_DECODE:
        return kvt_attn_decode_ws_bytes((int32_t)dims[0], (int32_t)dims[1], dims[2]);
    case KVT_OP_SPARSE_ROWS:
        return kvt_sparse_attend_rows_ws_bytes((int32_t)dims[0], (int32_t)dims[1],
                                               (int32_t)dims[2], (int32_t)dims[3]);
    default:
        return kvt_attn_prefill_state_bytes(dims[0], (int32_t)dims[1], (int32_t)dims[2]);
    }
}
