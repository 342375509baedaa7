// kvt_worker.hip -- the asynchronous transfer worker around kvt_swap_blocks (host runtime).
//
// vLLM-CPU SingleDirectionOffloadingHandler: one handler per direction keeps an ordered queue of
// transfers.  Each transfer gets a stream from a pool that waits for the compute stream (a
// store must see the KV it reads; a load must come after pending writes to its destination)
// and for the previous transfer's end, timing events from an event pool around the swap, and
// descriptor buffers from a buffer pool so the caller's tables are free as soon as submit
// returns.  get_finished polls the end events in submission order and reports each job's bytes
// and event-timed seconds, returning its stream, events and buffers to the pools; wait blocks
// on a set of jobs; shutdown drains in order and stops at the first failed synchronisation.
#include <cstring>
#include <deque>
#include <mutex>
#include <vector>

#include "kvt_internal.h"

struct kvt_worker {
    struct Buf {
        uint64_t *tab = nullptr;   // pinned, mapped: src[cap], dst[cap], sizes[cap]
        int64_t cap = 0;
    };
    struct Job {
        int64_t id;
        hipStream_t stream;
        hipEvent_t start, end;
        uint64_t bytes;
        Buf buf;
    };
    int dir = 0;
    int mode = KVT_COPY_AUTO;
    int device = 0;
    std::mutex mu;
    std::deque<Job> jobs;
    std::vector<hipStream_t> streams;
    std::vector<hipEvent_t> events;
    std::vector<Buf> bufs;
    hipEvent_t compute_point = nullptr;   // records the caller's stream at submit
};

namespace {

int new_buf(int64_t n, kvt_worker::Buf &out)
{
    const int64_t cap = n < 1024 ? 1024 : n;
    void *p = nullptr;
    const hipError_t e = hipHostMalloc(&p, (size_t)cap * 3 * sizeof(uint64_t),
                                       hipHostMallocMapped | hipHostMallocPortable |
                                           hipHostMallocCoherent);
    if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return kvt::fail(KVT_ENOMEM, "kvt_worker: descriptor buffer of %lld entries: %s",
                         (long long)cap, hipGetErrorString(e));
    }
    out.tab = static_cast<uint64_t *>(p);
    out.cap = cap;
    return KVT_OK;
}

// the smallest pooled buffer that holds n rows, else a new one
int take_buf(kvt_worker *w, int64_t n, kvt_worker::Buf &out)
{
    size_t best = w->bufs.size();
    for (size_t i = 0; i < w->bufs.size(); i++)
        if (w->bufs[i].cap >= n && (best == w->bufs.size() || w->bufs[i].cap < w->bufs[best].cap))
            best = i;
    if (best == w->bufs.size())
        return new_buf(n, out);
    out = w->bufs[best];
    w->bufs.erase(w->bufs.begin() + (long)best);
    return KVT_OK;
}

int new_event(hipEvent_t &e)
{
    KVT_HIP(hipEventCreate(&e));   // timing enabled: start -> end gives the job's duration
    return KVT_OK;
}

int new_stream(hipStream_t &s)
{
    KVT_HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));   // default priority
    return KVT_OK;
}

int take_event(kvt_worker *w, hipEvent_t &e)
{
    if (w->events.empty())
        return new_event(e);
    e = w->events.back();
    w->events.pop_back();
    return KVT_OK;
}

int take_stream(kvt_worker *w, hipStream_t &s)
{
    if (w->streams.empty())
        return new_stream(s);
    s = w->streams.back();
    w->streams.pop_back();
    return KVT_OK;
}

void give_back(kvt_worker *w, kvt_worker::Job &j)
{
    w->streams.push_back(j.stream);
    w->events.push_back(j.start);
    w->events.push_back(j.end);
    w->bufs.push_back(j.buf);
}

}  // namespace

extern "C" int kvt_worker_create(int32_t dir, int32_t mode, kvt_worker **out)
{
    if (!out || (dir != KVT_H2D && dir != KVT_D2H) ||
        mode < KVT_COPY_AUTO || mode > KVT_COPY_RUNTIME)
        return kvt::fail(KVT_EINVAL, "kvt_worker_create: dir=%d mode=%d out=%p", dir, mode,
                         (void *)out);
    if (mode == KVT_COPY_SDMA)   // it waits on the submitting thread; a worker only queues
        return kvt::fail(KVT_EUNSUPPORTED, "kvt_worker_create: the SDMA mode waits on the host; "
                                           "workers take AUTO, KERNEL or RUNTIME");
    kvt_worker *w = new (std::nothrow) kvt_worker;
    if (!w)
        return kvt::fail(KVT_ENOMEM, "kvt_worker_create: out of host memory");
    w->dir = dir;
    w->mode = mode;
    hipError_t e = hipGetDevice(&w->device);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&w->compute_point, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        delete w;
        return kvt::fail(KVT_EHIP, "kvt_worker_create: %s", hipGetErrorString(e));
    }
    *out = w;
    return KVT_OK;
}

extern "C" int kvt_worker_reserve(kvt_worker *w, int32_t jobs, int64_t entries)
{
    if (!w || jobs < 0 || jobs > 4096 || entries < 0)
        return kvt::fail(KVT_EINVAL, "kvt_worker_reserve: jobs=%d entries=%lld", jobs,
                         (long long)entries);
    std::lock_guard<std::mutex> lock(w->mu);
    int rc = KVT_OK;
    while (rc == KVT_OK && (int64_t)w->streams.size() < jobs) {
        hipStream_t s = nullptr;
        if ((rc = new_stream(s)) == KVT_OK)
            w->streams.push_back(s);
    }
    while (rc == KVT_OK && (int64_t)w->events.size() < 2ll * jobs) {
        hipEvent_t e = nullptr;
        if ((rc = new_event(e)) == KVT_OK)
            w->events.push_back(e);
    }
    // buffers: add new ones until `jobs` of the pooled ones hold `entries` rows
    int64_t big = 0;
    for (const auto &b : w->bufs)
        big += b.cap >= entries;
    while (rc == KVT_OK && big < jobs) {
        kvt_worker::Buf b;
        if ((rc = new_buf(entries, b)) == KVT_OK) {
            w->bufs.push_back(b);
            big++;
        }
    }
    return rc;
}

extern "C" int kvt_worker_submit(kvt_worker *w, int64_t job_id, const uint64_t *src,
                                 const uint64_t *dst, const uint64_t *sizes, int64_t n,
                                 void *compute_stream)
{
    if (!w)
        return kvt::fail(KVT_EINVAL, "kvt_worker_submit: null worker");
    if (n < 0 || (n > 0 && (!src || !dst || !sizes)))
        return kvt::fail(KVT_EINVAL, "kvt_worker_submit: n=%lld with null tables", (long long)n);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != w->device) {
        (void)hipGetLastError();
        return kvt::fail(KVT_EINVAL, "kvt_worker_submit: current device %d, worker's %d", dev,
                         w->device);
    }
    std::lock_guard<std::mutex> lock(w->mu);
    for (const auto &j : w->jobs)
        if (j.id == job_id)
            return kvt::fail(KVT_EINVAL, "kvt_worker_submit: job %lld is still pending",
                             (long long)job_id);
    kvt_worker::Job j{};
    j.id = job_id;
    uint64_t bytes = 0;
    for (int64_t i = 0; i < n; i++)
        bytes += sizes[i];
    j.bytes = bytes;
    int rc = take_buf(w, n, j.buf);
    if (rc != KVT_OK)
        return rc;
    uint64_t *ts = j.buf.tab, *td = j.buf.tab + j.buf.cap, *tz = j.buf.tab + 2 * j.buf.cap;
    if (n > 0) {
        std::memcpy(ts, src, (size_t)n * sizeof(uint64_t));
        std::memcpy(td, dst, (size_t)n * sizeof(uint64_t));
        std::memcpy(tz, sizes, (size_t)n * sizeof(uint64_t));
    }
    if ((rc = take_stream(w, j.stream)) != KVT_OK || (rc = take_event(w, j.start)) != KVT_OK ||
        (rc = take_event(w, j.end)) != KVT_OK) {
        w->bufs.push_back(j.buf);
        return rc;
    }
    auto undo = [&](int code) {
        give_back(w, j);
        return code;
    };
    // after the caller's work so far, and after the previous transfer of this direction
    hipError_t e = hipEventRecord(w->compute_point, kvt::as_stream(compute_stream));
    if (e == hipSuccess)
        e = hipStreamWaitEvent(j.stream, w->compute_point, 0);
    if (e == hipSuccess && !w->jobs.empty())
        e = hipStreamWaitEvent(j.stream, w->jobs.back().end, 0);
    if (e == hipSuccess)
        e = hipEventRecord(j.start, j.stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return undo(kvt::fail(KVT_EHIP, "kvt_worker_submit: %s", hipGetErrorString(e)));
    }
    if (n > 0) {
        rc = kvt_swap_blocks(ts, td, tz, n, w->dir, w->mode, j.stream);
        if (rc != KVT_OK)
            return undo(rc);
    }
    e = hipEventRecord(j.end, j.stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return undo(kvt::fail(KVT_EHIP, "kvt_worker_submit: %s", hipGetErrorString(e)));
    }
    w->jobs.push_back(j);
    return KVT_OK;
}

extern "C" int kvt_worker_get_finished(kvt_worker *w, int64_t *job_ids, uint64_t *bytes,
                                       double *seconds, int32_t max, int32_t *n_out)
{
    if (!w || !n_out || max < 0 || (max > 0 && !job_ids))
        return kvt::fail(KVT_EINVAL, "kvt_worker_get_finished: bad arguments");
    std::lock_guard<std::mutex> lock(w->mu);
    int32_t n = 0;
    while (n < max && !w->jobs.empty()) {
        kvt_worker::Job &j = w->jobs.front();
        const hipError_t q = hipEventQuery(j.end);
        if (q == hipErrorNotReady)
            break;
        if (q != hipSuccess) {
            (void)hipGetLastError();
            *n_out = n;
            return kvt::fail(KVT_EHIP, "kvt_worker_get_finished: job %lld: %s",
                             (long long)j.id, hipGetErrorString(q));
        }
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, j.start, j.end) != hipSuccess) {
            (void)hipGetLastError();
            ms = 0.f;
        }
        job_ids[n] = j.id;
        if (bytes)
            bytes[n] = j.bytes;
        if (seconds)
            seconds[n] = (double)ms * 1e-3;
        n++;
        give_back(w, j);
        w->jobs.pop_front();
    }
    *n_out = n;
    return KVT_OK;
}

extern "C" int kvt_worker_wait(kvt_worker *w, const int64_t *job_ids, int32_t n)
{
    if (!w || n < 0 || (n > 0 && !job_ids))
        return kvt::fail(KVT_EINVAL, "kvt_worker_wait: bad arguments");
    for (int32_t i = 0; i < n; i++) {
        hipEvent_t ev = nullptr;
        {
            std::lock_guard<std::mutex> lock(w->mu);
            for (const auto &j : w->jobs)
                if (j.id == job_ids[i])
                    ev = j.end;
        }
        if (ev)   // else finished and reported already, or never submitted
            KVT_HIP(hipEventSynchronize(ev));
    }
    return KVT_OK;
}

extern "C" int kvt_worker_pending(kvt_worker *w)
{
    if (!w)
        return kvt::fail(KVT_EINVAL, "kvt_worker_pending: null worker");
    std::lock_guard<std::mutex> lock(w->mu);
    return (int)w->jobs.size();
}

extern "C" int kvt_worker_destroy(kvt_worker *w)
{
    if (!w)
        return KVT_OK;
    int rc = KVT_OK;
    {
        std::lock_guard<std::mutex> lock(w->mu);
        // drain in order; after a failed synchronisation the rest are not waited for
        while (!w->jobs.empty()) {
            if (rc == KVT_OK) {
                const hipError_t e = hipEventSynchronize(w->jobs.front().end);
                if (e != hipSuccess) {
                    (void)hipGetLastError();
                    rc = kvt::fail(KVT_EHIP, "kvt_worker_destroy: job %lld: %s (%zu more skipped)",
                                   (long long)w->jobs.front().id, hipGetErrorString(e),
                                   w->jobs.size() - 1);
                }
            }
            give_back(w, w->jobs.front());
            w->jobs.pop_front();
        }
        for (hipStream_t s : w->streams)
            (void)hipStreamDestroy(s);
        for (hipEvent_t e : w->events)
            (void)hipEventDestroy(e);
        for (auto &b : w->bufs)
            (void)hipHostFree(b.tab);
        if (w->compute_point)
            (void)hipEventDestroy(w->compute_point);
    }
    delete w;
    return rc;
}
