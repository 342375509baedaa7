// kvt_engine.hip -- S2 batched swap and S7 tail staging on the DMA (SDMA) copy engines,
// driven through HSA.
//
// vLLM-CPU chooses between the copy engines and a kernel that reads host pointers.  Through
// HIP's copy calls that choice is not ours to make: the runtime picks an engine per copy, and
// on MI355X a kernel trace shows every page-sized pinned<->HBM copy of a batch
// (hipMemcpyBatchAsync or hipMemcpyAsync) running as one dispatch of the runtime's blit kernel;
// only large copies reach the DMA engines.  So the SDMA mode drives the engines itself:
// hsa_amd_memory_async_copy_on_engine between the GPU agent and a CPU agent is a DMA engine
// copy, one per run of adjacent descriptors (a run is contiguous on both sides), runs longer
// than 4 MiB cut into 4 MiB pieces.
//
// Engines.  MI355X reports 16 engines for each direction between host and device.  One engine
// takes about 10 us per copy whatever its size (2 KiB and 32 KiB copies alike), while a
// submission costs the calling thread about 0.4 us, so one engine moves 32 KiB pages at
// ~2.9 GB/s and the engines, not the thread, set the rate.  Copies therefore go round-robin
// over every engine the runtime reports available for the direction (32 KiB pages: ~29 GB/s
// from one thread over 16 engines); several submitting threads gained nothing over that.
// Descriptors write disjoint ranges, so copies may complete in any order.
//
// The mode is synchronous with respect to the calling thread: it drains the caller's stream,
// submits the copies, waits for them on this thread and returns, so work queued on the stream
// afterwards sees them.  It never waits on a runtime thread.  Ordering the copies with a stream
// host function that waited inside stalled at the first copy under a memory-copy trace, whose
// completion handler most likely needs the thread the runtime runs host functions on.
//
// Every copy has a completion signal of its own with value 1 (kvt_engine_runs.h holds that
// bookkeeping and its error paths), the form the runtime's own copies take.  One signal
// counted down once per copy is legal HSA too, but a memory-copy tracer, which completes each
// copy's signal from its own handler, rejected such a signal's value and the traced process
// then crashed.
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <mutex>
#include <new>

#include "kvt_engine_runs.h"
#include "kvt_internal.h"

namespace {

constexpr int kMaxDevices = 64;

constexpr int kMaxEngines = 16;

struct Agents {
    bool probed = false;
    int status = KVT_OK;
    hsa_agent_t gpu{}, cpu{};
    uint32_t engines[2] = {0, 0};   // available engine masks: [KVT_H2D], [KVT_D2H]
};

std::mutex g_mu;
bool g_hsa_up = false;
Agents g_agents[kMaxDevices];

struct Probe {
    uint32_t domain = 0, bus_dev = 0;   // bus_dev = bus << 5 | device (PCI BDF without function)
    bool have_gpu = false, have_cpu = false;
    hsa_agent_t gpu{}, cpu{};
};

hsa_status_t visit_agent(hsa_agent_t a, void *p)
{
    Probe *pr = static_cast<Probe *>(p);
    hsa_device_type_t type;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &type) != HSA_STATUS_SUCCESS)
        return HSA_STATUS_SUCCESS;
    if (type == HSA_DEVICE_TYPE_CPU && !pr->have_cpu) {
        pr->cpu = a;
        pr->have_cpu = true;
    } else if (type == HSA_DEVICE_TYPE_GPU && !pr->have_gpu) {
        uint32_t bdf = 0, dom = 0;
        if (hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_BDFID), &bdf) ==
                HSA_STATUS_SUCCESS &&
            hsa_agent_get_info(a, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_DOMAIN), &dom) ==
                HSA_STATUS_SUCCESS &&
            (bdf >> 3) == pr->bus_dev && dom == pr->domain) {
            pr->gpu = a;
            pr->have_gpu = true;
        }
    }
    return HSA_STATUS_SUCCESS;
}

// The HSA agents of HIP device `dev` (matched by PCI domain, bus and device) and of the CPU
// nearest to it; probed once per device.
int agents_for(int dev, Agents *out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return kvt::fail(KVT_EUNSUPPORTED, "engine copies: device %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_mu);
    Agents &a = g_agents[dev];
    if (!a.probed) {
        a.probed = true;
        a.status = KVT_EUNSUPPORTED;
        if (!g_hsa_up) {
            // the HIP runtime has HSA up already; this takes a reference of our own
            if (hsa_init() != HSA_STATUS_SUCCESS)
                return kvt::fail(KVT_EUNSUPPORTED, "engine copies: hsa_init failed");
            g_hsa_up = true;
        }
        int bus = 0, devn = 0, dom = 0;
        if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev) != hipSuccess ||
            hipDeviceGetAttribute(&devn, hipDeviceAttributePciDeviceId, dev) != hipSuccess ||
            hipDeviceGetAttribute(&dom, hipDeviceAttributePciDomainId, dev) != hipSuccess) {
            (void)hipGetLastError();
            return kvt::fail(KVT_EUNSUPPORTED, "engine copies: no PCI address for device %d", dev);
        }
        Probe pr;
        pr.domain = (uint32_t)dom;
        pr.bus_dev = ((uint32_t)bus << 5) | ((uint32_t)devn & 31);
        if (hsa_iterate_agents(visit_agent, &pr) != HSA_STATUS_SUCCESS || !pr.have_gpu ||
            !pr.have_cpu)
            return kvt::fail(KVT_EUNSUPPORTED, "engine copies: no HSA agents for device %d", dev);
        hsa_agent_t near{};
        if (hsa_agent_get_info(pr.gpu, static_cast<hsa_agent_info_t>(HSA_AMD_AGENT_INFO_NEAREST_CPU),
                               &near) == HSA_STATUS_SUCCESS && near.handle)
            pr.cpu = near;
        a.gpu = pr.gpu;
        a.cpu = pr.cpu;
        // engines the runtime reports for each direction; none reported: it picks per copy
        for (int d = 0; d < 2; d++) {
            uint32_t m = 0;
            if (hsa_amd_memory_copy_engine_status(d == KVT_H2D ? pr.gpu : pr.cpu,
                                                  d == KVT_H2D ? pr.cpu : pr.gpu,
                                                  &m) == HSA_STATUS_SUCCESS)
                a.engines[d] = m & ((1u << kMaxEngines) - 1);
        }
        a.status = KVT_OK;
    }
    if (a.status != KVT_OK)
        return kvt::fail(a.status, "engine copies: device %d has no usable HSA agents", dev);
    *out = a;
    return KVT_OK;
}

// The engine-copy operations of one call (see kvt_engine_runs.h): copies go round-robin over
// the engines in `engine` (n_engines of them; none: the runtime's own choice per copy).
struct HsaOps {
    hsa_agent_t dst_agent, src_agent;
    hsa_amd_sdma_engine_id_t engine[kMaxEngines];
    int n_engines = 0;
    int64_t next = 0;

    HsaOps(hsa_agent_t d, hsa_agent_t s, uint32_t mask) : dst_agent(d), src_agent(s)
    {
        for (int b = 0; b < kMaxEngines; b++)
            if (mask & (1u << b))
                engine[n_engines++] = static_cast<hsa_amd_sdma_engine_id_t>(1u << b);
    }
    int create(uint64_t *sig)
    {
        hsa_signal_t h;
        const hsa_status_t st = hsa_signal_create(1, 0, nullptr, &h);
        *sig = h.handle;
        return st == HSA_STATUS_SUCCESS ? 0 : (int)st;
    }
    int copy(uint64_t d, uint64_t s, uint64_t len, uint64_t sig)
    {
        void *dp = reinterpret_cast<void *>(d);
        const void *sp = reinterpret_cast<const void *>(s);
        const hsa_status_t st =
            n_engines ? hsa_amd_memory_async_copy_on_engine(dp, dst_agent, sp, src_agent, len, 0,
                                                            nullptr, hsa_signal_t{sig},
                                                            engine[next++ % n_engines], false)
                      : hsa_amd_memory_async_copy(dp, dst_agent, sp, src_agent, len, 0, nullptr,
                                                  hsa_signal_t{sig});
        return st == HSA_STATUS_SUCCESS ? 0 : (int)st;
    }
    void reset(uint64_t sig) { hsa_signal_store_screlease(hsa_signal_t{sig}, 1); }
    void wait(uint64_t sig)
    {
        while (hsa_signal_wait_scacquire(hsa_signal_t{sig}, HSA_SIGNAL_CONDITION_LT, 1, UINT64_MAX,
                                         HSA_WAIT_STATE_BLOCKED) >= 1) {
        }
    }
    void destroy(uint64_t sig) { hsa_signal_destroy(hsa_signal_t{sig}); }
};

constexpr int64_t kSignalWindow = 256;        // copies in flight at most
constexpr uint64_t kMaxRun = (uint64_t)4 << 20;   // longer runs are cut, to use more engines

}  // namespace

namespace kvt {

// The n descriptor copies on the DMA engines, after everything queued on stream s; returns
// once they are done (see the file comment).  dir KVT_H2D: src is host memory, dst device
// memory; KVT_D2H the reverse.  fn names the entry point in error messages.
int engine_copies(const char *fn, const uint64_t *src, const uint64_t *dst,
                  const uint64_t *sizes, int64_t n, int32_t dir, hipStream_t s)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    KVT_HIP(hipStreamIsCapturing(s, &cs));
    if (cs != hipStreamCaptureStatusNone)
        return fail(KVT_EUNSUPPORTED, "%s: the SDMA mode waits on the host and cannot be "
                                      "captured in a graph", fn);
    int dev = 0;
    KVT_HIP(hipStreamGetDevice(s, &dev));
    Agents a;
    const int rc = agents_for(dev, &a);
    if (rc != KVT_OK)
        return rc;
    bool any = false;
    for (int64_t i = 0; i < n && !any; i++)
        any = sizes[i] != 0;
    if (!any)
        return KVT_OK;
    KVT_HIP(hipStreamSynchronize(s));   // the copies come after the stream's earlier work
    HsaOps ops(dir == KVT_H2D ? a.gpu : a.cpu, dir == KVT_H2D ? a.cpu : a.gpu,
               a.engines[dir == KVT_H2D ? KVT_H2D : KVT_D2H]);
    const EngineTally t = run_engine_copies(ops, src, dst, sizes, n, kSignalWindow, kMaxRun);
    if (t.failed_at == 1)
        return fail(KVT_EHIP, "%s: hsa_signal_create: status %d (no copy submitted)", fn,
                    t.status);
    if (t.failed_at == 2)
        return fail(KVT_EHIP, "%s: engine copy submission: status %d after %lld of %lld copies",
                    fn, t.status, (long long)t.submitted, (long long)t.runs);
    return KVT_OK;
}

// Engines the SDMA mode spreads its copies over for direction dir on device dev (0: the
// runtime picks per copy), or a negative status.
int engine_count(int dev, int32_t dir)
{
    Agents a;
    const int rc = agents_for(dev, &a);
    if (rc != KVT_OK)
        return rc;
    return __builtin_popcount(a.engines[dir == KVT_H2D ? KVT_H2D : KVT_D2H]);
}

}  // namespace kvt

// The number of engines the SDMA mode uses on the current device for direction dir.
extern "C" int kvt_copy_engines(int32_t dir)
{
    if (dir != KVT_H2D && dir != KVT_D2H)
        return kvt::fail(KVT_EINVAL, "kvt_copy_engines: dir=%d", dir);
    int dev = 0;
    KVT_HIP(hipGetDevice(&dev));
    return kvt::engine_count(dev, dir);
}
