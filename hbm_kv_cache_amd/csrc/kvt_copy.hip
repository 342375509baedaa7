// kvt_copy.hip -- S2 batched block swap and S7 tail staging.
//
// vLLM-CPU transfer_async hands a swap function three u64 tables (src, dst, size) and picks
// either the copy engines or a GPU kernel that dereferences host pointers.  Here:
//   * KERNEL: each wavefront owns one 8 KiB chunk of one descriptor.  It reads the descriptor
//     and reads the chunk one 1 KiB wave-load at a time (16 bytes per lane), then stores it,
//     so thousands of waves keep ~1 MiB or more in flight without flooding the link.  Descriptors whose
//     addresses are only 8-byte aligned take an 8-byte path, anything else a byte path.  When
//     no page exceeds a chunk, a wave takes eight consecutive descriptors instead, read with
//     one load (copy_small_kernel).
//   * SDMA: one DMA-engine copy per run of adjacent descriptors, through HSA (kvt_engine.hip).
//   * RUNTIME: HIP's copy calls -- hipMemcpyBatchAsync (one submission for the batch), else one
//     hipMemcpyAsync per descriptor -- which choose the engine per copy themselves: a kernel
//     trace shows page-sized copies running as the runtime's blit kernel.
// kvt_stage_tail (llama-T tail staging) is one contiguous range: one hipMemcpyAsync (AUTO and
// RUNTIME), which the runtime runs on a copy engine at staging sizes; one engine copy driven
// through HSA (SDMA, as in kvt_swap_blocks); or the same wide-load kernel over one span.
#include <dlfcn.h>

#include <algorithm>
#include <atomic>

#include "kvt_internal.h"

namespace {

constexpr int kChunk = 8192;                      // bytes per wave unit
constexpr int kWavesPerBlock = 4;                 // 256-thread workgroups
constexpr int kCopyWaves = 1024;                  // one wave per SIMD: ~1 MiB in flight
constexpr int kSmallWaves = 2048;                 // small pages: 512 B-8 KiB per wave-load step

constexpr int kWordsPerLane16 = kChunk / 16 / kvt::kWave;  // 8
constexpr int kWordsPerLane8 = kChunk / 8 / kvt::kWave;    // 16

// One wave copies bytes [off, off+len) of a single range.  off + len <= range size.  The wave
// has one wave-load (64 lanes x 16 or 8 bytes) in flight at a time -- the empty asm that takes
// each loaded value makes the wave wait for it before the next load issues.  A whole chunk is
// stored after its last load, so no load waits behind a store; part of a chunk is copied load,
// wait, store.  How much is in flight across the chip is set by the number of waves: the
// kernels below stride a fixed grid over their work (kCopyWaves), as kvt_gather.hip does --
// host reads with every load of a transfer in flight at once ran ~20% below the link rate on
// MI355X, and a grid of one wave per SIMD keeps ~1 MiB in flight, which holds the link rate.
template <typename W, int N>
__device__ __forceinline__ void wave_copy_words(const W *sp, W *dp, uint32_t nw, int lane)
{
    if (nw == (uint32_t)N * kvt::kWave) {
        W r[N];
#pragma unroll
        for (int k = 0; k < N; k++) {
            r[k] = __builtin_nontemporal_load(sp + lane + k * kvt::kWave);
            __asm__ volatile("" : : "v"(r[k]) : "memory");
        }
#pragma unroll
        for (int k = 0; k < N; k++)
            dp[lane + k * kvt::kWave] = r[k];
    } else {
#pragma unroll 1
        for (uint32_t w = lane; w < nw; w += kvt::kWave) {
            const W v = __builtin_nontemporal_load(sp + w);
            __asm__ volatile("" : : "v"(v) : "memory");
            dp[w] = v;
        }
    }
}

__device__ __forceinline__ void wave_copy_chunk(uint64_t s, uint64_t d, uint64_t len, int lane)
{
    if (((s | d) & 15) == 0) {
        const uint32_t nw = (uint32_t)(len >> 4);
        wave_copy_words<u32x4, kWordsPerLane16>(reinterpret_cast<const u32x4 *>(s),
                                                reinterpret_cast<u32x4 *>(d), nw, lane);
        uint64_t done = (uint64_t)nw << 4;
        if (done < len && lane < (int)(len - done)) {  // < 16 trailing bytes
            reinterpret_cast<uint8_t *>(d)[done + lane] =
                reinterpret_cast<const uint8_t *>(s)[done + lane];
        }
    } else if (((s | d) & 7) == 0) {
        const uint32_t nw = (uint32_t)(len >> 3);
        wave_copy_words<u32x2, kWordsPerLane8>(reinterpret_cast<const u32x2 *>(s),
                                               reinterpret_cast<u32x2 *>(d), nw, lane);
        uint64_t done = (uint64_t)nw << 3;
        if (done < len && lane < (int)(len - done)) {
            reinterpret_cast<uint8_t *>(d)[done + lane] =
                reinterpret_cast<const uint8_t *>(s)[done + lane];
        }
    } else {
        const uint8_t *sp = reinterpret_cast<const uint8_t *>(s);
        uint8_t *dp = reinterpret_cast<uint8_t *>(d);
        for (uint64_t b = lane; b < len; b += kvt::kWave)
            dp[b] = sp[b];
    }
}

// unit u = (descriptor i, chunk c) with u = i*chunks + c; each wave strides over units
__global__ __launch_bounds__(256) void copy_desc_kernel(const uint64_t *__restrict__ src,
                                                        const uint64_t *__restrict__ dst,
                                                        const uint64_t *__restrict__ sizes,
                                                        int64_t n_units, uint32_t chunks)
{
    const int lane = threadIdx.x & (kvt::kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
    for (int64_t u = (int64_t)blockIdx.x * kWavesPerBlock + wave; u < n_units; u += stride) {
        const int64_t i = u / chunks;
        const uint64_t off = (uint64_t)(u - i * chunks) * kChunk;
        const uint64_t sz = sizes[i];
        if (off >= sz)
            continue;
        const uint64_t len = sz - off < (uint64_t)kChunk ? sz - off : (uint64_t)kChunk;
        wave_copy_chunk(src[i] + off, dst[i] + off, len, lane);
    }
}

// Pages of at most one chunk: a wave takes kGroup consecutive descriptors at a time.  Lanes
// 0..23 read the group's src, dst and size entries with one load instruction -- three 64-byte
// lines of the tables instead of a line per descriptor and table -- and the wave then copies
// the group's pages one after another, taking each descriptor from those lanes.
constexpr int kGroup = 8;

__global__ __launch_bounds__(256) void copy_small_kernel(const uint64_t *__restrict__ src,
                                                         const uint64_t *__restrict__ dst,
                                                         const uint64_t *__restrict__ sizes,
                                                         int64_t n)
{
    const int lane = threadIdx.x & (kvt::kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tab = lane / kGroup, j = lane % kGroup;
    const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock * kGroup;
    for (int64_t i0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * kGroup; i0 < n;
         i0 += stride) {
        uint64_t v = 0;
        if (tab < 3 && i0 + j < n)
            v = (tab == 0 ? src : tab == 1 ? dst : sizes)[i0 + j];
        // lane L's 64-bit value, in scalar registers (the builtin returns a signed int: each
        // half is taken as uint32_t before widening, so no half is sign-extended into the other)
        auto lane_u64 = [&](int L) -> uint64_t {
            const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, L);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), L);
            return ((uint64_t)hi << 32) | (uint64_t)lo;
        };
        const int m = n - i0 < kGroup ? (int)(n - i0) : kGroup;
        for (int k = 0; k < m; k++)
            wave_copy_chunk(lane_u64(k), lane_u64(kGroup + k), lane_u64(2 * kGroup + k), lane);
    }
}

// one contiguous range, 8 KiB chunks; each wave strides over chunks
__global__ __launch_bounds__(256) void copy_span_kernel(uint64_t src, uint64_t dst, uint64_t bytes)
{
    const int lane = threadIdx.x & (kvt::kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint64_t stride = (uint64_t)gridDim.x * kWavesPerBlock * kChunk;
    for (uint64_t off = ((uint64_t)blockIdx.x * kWavesPerBlock + wave) * kChunk; off < bytes;
         off += stride) {
        const uint64_t len = bytes - off < (uint64_t)kChunk ? bytes - off : (uint64_t)kChunk;
        wave_copy_chunk(src + off, dst + off, len, lane);
    }
}

// workgroups for `units` wave units, at most `cap` waves
unsigned copy_groups(uint64_t units, int cap)
{
    const uint64_t waves = units < (uint64_t)cap ? units : (uint64_t)cap;
    return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

// AUTO policy: vLLM-CPU _select_swap_blocks_fn keeps a kernel for small 8-byte-multiple pages
// and the copy engines otherwise.  On MI355X the kernel path measured at or above both the
// engines and the runtime's copy calls at every page size from 512 B to 64 KiB and in both
// directions (56.9 GB/s host->HBM and 55.1 GB/s HBM->host on 32 KiB pages; every per-page copy
// on the engines or through the runtime costs microseconds of submission), so AUTO takes the
// kernel whenever it is eligible and the runtime's copy calls otherwise (they take any size
// and alignment, and work under graph capture).  kvt_set_copy_threshold moves the switch point
// per direction.
std::atomic<uint64_t> g_threshold[2] = {{~0ull}, {~0ull}};

// hipMemcpyBatchAsync is resolved at run time from the HIP runtime already in the process (the
// one that owns the caller's streams); runtimes that predate it get per-copy submission.
typedef hipError_t (*batch_fn_t)(void **, void **, size_t *, size_t, hipMemcpyAttributes *,
                                 size_t *, size_t, size_t *, hipStream_t);
std::atomic<int> g_batch_state{0};  // 0 unknown, 1 usable, 2 unavailable
std::atomic<batch_fn_t> g_batch_fn{nullptr};

batch_fn_t batch_fn()
{
    int st = g_batch_state.load();
    if (st == 0) {
        void *h = dlopen("libamdhip64.so.7", RTLD_LAZY | RTLD_NOLOAD);
        void *f = h ? dlsym(h, "hipMemcpyBatchAsync") : nullptr;
        g_batch_fn.store(reinterpret_cast<batch_fn_t>(f));
        st = f ? 1 : 2;
        g_batch_state.store(st);
    }
    return st == 1 ? g_batch_fn.load() : nullptr;
}

int runtime_copies(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes, int64_t n,
                   hipStream_t s)
{
    if (batch_fn_t f = batch_fn()) {
        size_t fail_idx = 0;
        hipError_t e = f(reinterpret_cast<void **>(const_cast<uint64_t *>(dst)),
                         reinterpret_cast<void **>(const_cast<uint64_t *>(src)),
                         reinterpret_cast<size_t *>(const_cast<uint64_t *>(sizes)), (size_t)n,
                         nullptr, nullptr, 0, &fail_idx, s);
        if (e == hipSuccess)
            return KVT_OK;
        (void)hipGetLastError();
        if (e != hipErrorNotSupported && e != hipErrorInvalidValue)
            return kvt::fail(KVT_EHIP, "hipMemcpyBatchAsync failed at %zu: %s", fail_idx,
                             hipGetErrorString(e));
        g_batch_state.store(2);  // refuses this form: per-copy submission from now on
    }
    for (int64_t i = 0; i < n; i++) {
        if (!sizes[i])
            continue;
        KVT_HIP(hipMemcpyAsync(reinterpret_cast<void *>(dst[i]),
                               reinterpret_cast<const void *>(src[i]), sizes[i],
                               hipMemcpyDefault, s));
    }
    return KVT_OK;
}

}  // namespace

extern "C" uint64_t kvt_set_copy_threshold(int32_t dir, uint64_t bytes)
{
    if (dir != KVT_H2D && dir != KVT_D2H)
        return 0;
    return g_threshold[dir].exchange(bytes);
}

// S2: vLLM-CPU transfer_async -> swap_blocks_batch(src, dst, sizes).
extern "C" int kvt_swap_blocks(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes,
                               int64_t n, int32_t dir, int32_t mode, void *stream)
{
    if (n < 0 || (n && (!src || !dst || !sizes)))
        return kvt::fail(KVT_EINVAL, "kvt_swap_blocks: n=%lld with null tables", (long long)n);
    if (dir != KVT_H2D && dir != KVT_D2H)
        return kvt::fail(KVT_EINVAL, "kvt_swap_blocks: dir=%d", dir);
    if (mode < KVT_COPY_AUTO || mode > KVT_COPY_RUNTIME)
        return kvt::fail(KVT_EINVAL, "kvt_swap_blocks: mode=%d", mode);
    if (n == 0)
        return KVT_OK;
    hipStream_t s = kvt::as_stream(stream);

    uint64_t max_size = 0, or_size = 0;
    for (int64_t i = 0; i < n; i++) {
        max_size = std::max(max_size, sizes[i]);
        or_size |= sizes[i];
    }
    if (max_size == 0)
        return KVT_OK;
    const bool kernel_ok = (or_size & 7) == 0;
    if (mode == KVT_COPY_KERNEL && !kernel_ok)
        return kvt::fail(KVT_EALIGN, "kvt_swap_blocks: kernel path needs sizes %% 8 == 0");
    bool use_kernel = mode == KVT_COPY_KERNEL ||
                      (mode == KVT_COPY_AUTO && kernel_ok && max_size < g_threshold[dir].load());
    if (mode == KVT_COPY_SDMA)
        return kvt::engine_copies("kvt_swap_blocks", src, dst, sizes, n, dir, s);
    if (!use_kernel)
        return runtime_copies(src, dst, sizes, n, s);

    if (max_size <= (uint64_t)kChunk) {
        const uint64_t groups = (uint64_t)(n + kGroup - 1) / kGroup;
        hipLaunchKernelGGL(copy_small_kernel, dim3(copy_groups(groups, kSmallWaves)), dim3(256),
                           0, s, src, dst, sizes, n);
        KVT_LAUNCHED("copy_small_kernel");
        return KVT_OK;
    }
    const uint64_t chunks = (max_size + kChunk - 1) / kChunk;
    if (chunks > 0xffffffffull)
        return kvt::fail(KVT_ERANGE, "kvt_swap_blocks: page of %llu bytes too large",
                         (unsigned long long)max_size);
    const int64_t units = n * (int64_t)chunks;
    if (units / (int64_t)chunks != n)
        return kvt::fail(KVT_ERANGE, "kvt_swap_blocks: %lld descriptors of %llu chunks overflow",
                         (long long)n, (unsigned long long)chunks);
    hipLaunchKernelGGL(copy_desc_kernel, dim3(copy_groups((uint64_t)units, kCopyWaves)),
                       dim3(256), 0, s, src, dst, sizes, units, (uint32_t)chunks);
    KVT_LAUNCHED("copy_desc_kernel");
    return KVT_OK;
}

// S7: llama-T tail staging -- rows [row_begin, row_end) of a host-resident plane into HBM.
extern "C" int kvt_stage_tail(const void *plane, int64_t row_bytes, int64_t row_begin,
                              int64_t row_end, void *staging, int32_t mode, void *stream)
{
    if (row_bytes < 1 || row_begin < 0 || row_end < row_begin)
        return kvt::fail(KVT_EINVAL, "kvt_stage_tail: row_bytes=%lld rows [%lld, %lld)",
                         (long long)row_bytes, (long long)row_begin, (long long)row_end);
    if (mode < KVT_COPY_AUTO || mode > KVT_COPY_RUNTIME)
        return kvt::fail(KVT_EINVAL, "kvt_stage_tail: mode=%d", mode);
    const uint64_t bytes = (uint64_t)(row_end - row_begin) * (uint64_t)row_bytes;
    if (!bytes)
        return KVT_OK;
    if (!plane || !staging)
        return kvt::fail(KVT_EINVAL, "kvt_stage_tail: null plane or staging buffer");
    hipStream_t s = kvt::as_stream(stream);
    const uint64_t src = reinterpret_cast<uint64_t>(plane) + (uint64_t)row_begin * row_bytes;
    const uint64_t dst = reinterpret_cast<uint64_t>(staging);
    if (mode == KVT_COPY_SDMA)
        return kvt::engine_copies("kvt_stage_tail", &src, &dst, &bytes, 1, KVT_H2D, s);
    if (mode != KVT_COPY_KERNEL) {
        KVT_HIP(hipMemcpyAsync(staging, reinterpret_cast<const void *>(src), bytes,
                               hipMemcpyDefault, s));
        return KVT_OK;
    }
    hipLaunchKernelGGL(copy_span_kernel, dim3(copy_groups((bytes + kChunk - 1) / kChunk, kCopyWaves)),
                       dim3(256), 0, s, src, dst, bytes);
    KVT_LAUNCHED("copy_span_kernel");
    return KVT_OK;
}
