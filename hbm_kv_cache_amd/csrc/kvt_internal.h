// kvt_internal.h -- shared helpers of libkvt's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "kvt.h"

namespace kvt {

// Records a message for kvt_last_error() on this thread and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Checks a HIP call; on failure records its text and returns KVT_EHIP.
#define KVT_HIP(call)                                                                        \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess)                                                                \
            return ::kvt::fail(KVT_EHIP, "%s: %s (%s:%d)", #call, hipGetErrorString(e_),     \
                               __FILE__, __LINE__);                                          \
    } while (0)

// After a kernel launch: report launch-configuration errors without synchronising.
#define KVT_LAUNCHED(name)                                                                   \
    do {                                                                                     \
        hipError_t e_ = hipGetLastError();                                                   \
        if (e_ != hipSuccess)                                                                \
            return ::kvt::fail(KVT_EHIP, "launch of %s: %s", name, hipGetErrorString(e_));   \
    } while (0)

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int kWave = 64;  // CDNA wavefront width

// The SDMA copy mode: n descriptor copies on the DMA engines after the work queued on stream
// s, waited for on the calling thread (kvt_engine.hip).  dir KVT_H2D: src host, dst device;
// KVT_D2H the reverse.  fn names the entry point in error messages.
int engine_copies(const char *fn, const uint64_t *src, const uint64_t *dst,
                  const uint64_t *sizes, int64_t n, int32_t dir, hipStream_t s);
// Engines that mode spreads its copies over on device dev (0: the runtime picks per copy).
int engine_count(int dev, int32_t dir);

}  // namespace kvt

// native clang vectors (the nontemporal builtins and bit casts want these, not HIP's structs)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp16 / bf16 bit patterns -> fp32 (both exact)
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
