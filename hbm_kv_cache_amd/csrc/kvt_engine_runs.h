// kvt_engine_runs.h -- the bookkeeping of kvt_swap_blocks' engine (SDMA) mode, apart from the
// HSA calls it drives, so that host code alone can check it.
//
// The mode submits one engine copy per run of adjacent descriptors (vLLM-CPU's batched swap,
// `transfer_async` -> `swap_blocks_batch`), a long run cut into pieces of at most max_run
// bytes.  Every copy gets a completion signal of its own,
// created with value 1, which the engine counts down to 0 when the copy is done: the form the
// runtime's own copies use, and the one a memory-copy tracer that wraps each copy's signal
// expects.  A window of at most `window` signals is reused: before copy i takes the signal of
// copy i - window, that copy is waited for and the signal set back to 1.  At the end the
// outstanding copies are waited for oldest first, then every signal is destroyed.
//
// Error paths.  If a signal cannot be created, the ones created so far are destroyed and
// nothing is submitted.  If a copy cannot be submitted, no later copy is submitted; the copies
// already submitted are waited for, then every signal is destroyed.  A copy that was never
// submitted is never waited for (its signal would never reach 0).
//
// No HIP or HSA header here: a signal is an opaque 64-bit handle, and `Ops` supplies
//   int  create(uint64_t *sig)   -- a new signal of value 1; 0 on success
//   int  copy(uint64_t dst, uint64_t src, uint64_t len, uint64_t sig)   -- 0 when submitted
//   void reset(uint64_t sig)     -- set the value back to 1
//   void wait(uint64_t sig)      -- return once the value is below 1
//   void destroy(uint64_t sig)
#pragma once

#include <cstdint>
#include <vector>

namespace kvt {

struct EngineTally {
    int status = 0;            // 0, or the first failing create / copy status
    int failed_at = 0;         // 0 none, 1 signal creation, 2 copy submission
    int64_t runs = 0;          // copies the descriptors call for (runs, or their pieces)
    int64_t created = 0, submitted = 0, waited = 0, destroyed = 0;
};

// A run: descriptors i..j-1 with every next one starting where the previous ended, on both
// sides.  Zero-size descriptors are skipped and end no run.  Each run goes to f in pieces of at
// most max_run bytes (0: whole), so that one long range can be spread over several engines.
template <class F>
void for_each_engine_run(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes,
                         int64_t n, uint64_t max_run, F &&f)
{
    const uint64_t cut = max_run ? max_run : ~(uint64_t)0;
    int64_t i = 0;
    while (i < n) {
        if (!sizes[i]) {
            i++;
            continue;
        }
        const uint64_t s0 = src[i], d0 = dst[i];
        uint64_t len = sizes[i];
        int64_t k = i + 1;
        for (; k < n; k++) {
            if (!sizes[k])
                continue;
            if (src[k] != s0 + len || dst[k] != d0 + len)
                break;
            len += sizes[k];
        }
        for (uint64_t off = 0; off < len; off += cut)
            f(s0 + off, d0 + off, len - off < cut ? len - off : cut);
        i = k;
    }
}

template <class Ops>
EngineTally run_engine_copies(Ops &ops, const uint64_t *src, const uint64_t *dst,
                              const uint64_t *sizes, int64_t n, int64_t window, uint64_t max_run)
{
    EngineTally t;
    for_each_engine_run(src, dst, sizes, n, max_run,
                        [&](uint64_t, uint64_t, uint64_t) { t.runs++; });
    if (!t.runs)
        return t;
    const int64_t w = t.runs < window ? t.runs : (window > 0 ? window : 1);
    std::vector<uint64_t> sig((size_t)w, 0);
    std::vector<char> busy((size_t)w, 0);
    for (; t.created < w; t.created++) {
        const int st = ops.create(&sig[(size_t)t.created]);
        if (st) {
            t.status = st;
            t.failed_at = 1;
            break;
        }
    }
    if (!t.status) {
        for_each_engine_run(src, dst, sizes, n, max_run, [&](uint64_t s, uint64_t d,
                                                             uint64_t len) {
            if (t.status)
                return;
            const size_t slot = (size_t)(t.submitted % w);
            if (busy[slot]) {   // copy submitted - w: done before its signal is reused
                ops.wait(sig[slot]);
                t.waited++;
                busy[slot] = 0;
                ops.reset(sig[slot]);
            }
            const int st = ops.copy(d, s, len, sig[slot]);
            if (st) {
                t.status = st;
                t.failed_at = 2;
                return;
            }
            busy[slot] = 1;
            t.submitted++;
        });
        // the outstanding copies, oldest first
        const int64_t first = t.submitted > w ? t.submitted - w : 0;
        for (int64_t i = first; i < t.submitted; i++) {
            const size_t slot = (size_t)(i % w);
            if (busy[slot]) {
                ops.wait(sig[slot]);
                t.waited++;
                busy[slot] = 0;
            }
        }
    }
    for (int64_t i = 0; i < t.created; i++) {
        ops.destroy(sig[(size_t)i]);
        t.destroyed++;
    }
    return t;
}

}  // namespace kvt
