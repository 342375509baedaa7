// kvt_prefill.hip -- S8 tiered prefill attention (in progress).
#include "kvt_internal.h"

extern "C" int kvt_attn_prefill(const void *, int64_t, int64_t, int32_t, int32_t, int32_t,
                                const void *, const void *, int64_t, const void *, const void *,
                                int64_t, int32_t, int32_t, float, float *, void *)
{
    return kvt::fail(KVT_EUNSUPPORTED, "kvt_attn_prefill: not built yet");
}
