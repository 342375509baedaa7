// kvt_engine.hip -- S2 batched swap on the DMA (SDMA) copy engines, driven through HSA.
//
// vLLM-CPU chooses between the copy engines and a kernel that reads host pointers.  Through
// HIP's copy calls that choice is not ours to make: the runtime picks an engine per copy, and
// on MI355X a kernel trace shows every page-sized pinned<->HBM copy of a batch
// (hipMemcpyBatchAsync or hipMemcpyAsync) running as one dispatch of the runtime's blit kernel;
// only large copies reach the DMA engines.  So the SDMA mode of kvt_swap_blocks drives the
// engines itself: hsa_amd_memory_async_copy between the GPU agent and a CPU agent is a DMA
// engine copy, one per run of adjacent descriptors (a run is contiguous on both sides).
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

struct Agents {
    bool probed = false;
    int status = KVT_OK;
    hsa_agent_t gpu{}, cpu{};
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
        a.status = KVT_OK;
    }
    if (a.status != KVT_OK)
        return kvt::fail(a.status, "engine copies: device %d has no usable HSA agents", dev);
    *out = a;
    return KVT_OK;
}

// The engine-copy operations of one call (see kvt_engine_runs.h).
struct HsaOps {
    hsa_agent_t dst_agent, src_agent;
    int create(uint64_t *sig)
    {
        hsa_signal_t h;
        const hsa_status_t st = hsa_signal_create(1, 0, nullptr, &h);
        *sig = h.handle;
        return st == HSA_STATUS_SUCCESS ? 0 : (int)st;
    }
    int copy(uint64_t d, uint64_t s, uint64_t len, uint64_t sig)
    {
        const hsa_status_t st = hsa_amd_memory_async_copy(
            reinterpret_cast<void *>(d), dst_agent, reinterpret_cast<const void *>(s), src_agent,
            len, 0, nullptr, hsa_signal_t{sig});
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

constexpr int64_t kSignalWindow = 256;   // copies in flight at most

}  // namespace

namespace kvt {

// The n descriptor copies on the DMA engines, after everything queued on stream s; returns
// once they are done (see the file comment).  dir KVT_H2D: src is host memory, dst device
// memory; KVT_D2H the reverse.
int engine_copies(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes, int64_t n,
                  int32_t dir, hipStream_t s)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    KVT_HIP(hipStreamIsCapturing(s, &cs));
    if (cs != hipStreamCaptureStatusNone)
        return fail(KVT_EUNSUPPORTED, "kvt_swap_blocks: the SDMA mode waits on the host and "
                                      "cannot be captured in a graph");
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
    HsaOps ops{dir == KVT_H2D ? a.gpu : a.cpu, dir == KVT_H2D ? a.cpu : a.gpu};
    const EngineTally t = run_engine_copies(ops, src, dst, sizes, n, kSignalWindow);
    if (t.failed_at == 1)
        return fail(KVT_EHIP, "kvt_swap_blocks: hsa_signal_create: status %d (no copy submitted)",
                    t.status);
    if (t.failed_at == 2)
        return fail(KVT_EHIP, "kvt_swap_blocks: hsa_amd_memory_async_copy: status %d after %lld "
                              "of %lld copies", t.status, (long long)t.submitted,
                    (long long)t.runs);
    return KVT_OK;
}

}  // namespace kvt
