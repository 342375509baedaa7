// Host-only driver for the engine-copy bookkeeping (kvt_engine_runs.h) with fake signal and
// copy operations.  Built and run by tests/test_engine_bookkeeping.py; no HIP, no HSA, no GPU.
//
// stdin:  n window fail_create_at fail_copy_at max_run   (-1 = never fail; max_run 0 = whole)
//         n lines "src dst size"
// stdout: "T status failed_at runs created submitted waited destroyed"
//         one "C dst src len" line per submitted copy, in submission order
//         one "V message" line per rule the bookkeeping broke
// The fake engine completes a copy only when its signal is waited for, so a wait on a signal
// with no copy in flight is reported (on an engine it would never return).
#include <cstdint>
#include <cstdio>
#include <map>
#include <string>
#include <vector>

#include "kvt_engine_runs.h"

namespace {

struct Sig {
    int64_t value = 1;
    bool alive = true;
    int64_t copy = -1;   // submission index of the copy in flight on it, or -1
};

struct FakeOps {
    int64_t fail_create_at = -1, fail_copy_at = -1;
    int64_t n_create = 0, n_copy = 0, next_handle = 0x1000;
    int64_t last_completed = -1;
    std::map<uint64_t, Sig> sigs;
    std::vector<std::string> violations;
    std::vector<std::vector<uint64_t>> copies;

    void bad(const std::string &m) { violations.push_back(m); }

    int create(uint64_t *h)
    {
        if (n_create++ == fail_create_at)
            return 7;
        *h = (uint64_t)(next_handle += 0x40);
        sigs[*h] = Sig{};
        return 0;
    }
    int copy(uint64_t d, uint64_t s, uint64_t len, uint64_t h)
    {
        auto it = sigs.find(h);
        if (it == sigs.end() || !it->second.alive) {
            bad("copy on a signal that does not exist");
            return 0;
        }
        if (n_copy == fail_copy_at) {
            n_copy++;
            return 9;
        }
        if (it->second.value != 1)
            bad("copy given a signal whose value is not 1");
        if (it->second.copy >= 0)
            bad("copy given a signal another copy still holds");
        it->second.copy = (int64_t)copies.size();
        copies.push_back({d, s, len});
        n_copy++;
        return 0;
    }
    void wait(uint64_t h)
    {
        auto it = sigs.find(h);
        if (it == sigs.end() || !it->second.alive) {
            bad("wait on a signal that does not exist");
            return;
        }
        if (it->second.copy < 0) {
            bad("wait on a signal with no copy in flight (would never return)");
            return;
        }
        if (it->second.copy != last_completed + 1)
            bad("copies not waited for in submission order");
        last_completed = it->second.copy;
        it->second.copy = -1;
        it->second.value = 0;   // the engine's completion
    }
    void reset(uint64_t h)
    {
        auto it = sigs.find(h);
        if (it == sigs.end() || !it->second.alive) {
            bad("reset of a signal that does not exist");
            return;
        }
        if (it->second.copy >= 0)
            bad("reset of a signal whose copy is still in flight");
        it->second.value = 1;
    }
    void destroy(uint64_t h)
    {
        auto it = sigs.find(h);
        if (it == sigs.end() || !it->second.alive) {
            bad("destroy of a signal that does not exist");
            return;
        }
        if (it->second.copy >= 0)
            bad("destroy of a signal whose copy is still in flight");
        it->second.alive = false;
    }
};

}  // namespace

int main()
{
    long long n = 0, window = 0, fc = -1, fp = -1;
    unsigned long long max_run = 0;
    if (scanf("%lld %lld %lld %lld %llu", &n, &window, &fc, &fp, &max_run) != 5)
        return 2;
    std::vector<uint64_t> src(n), dst(n), sz(n);
    for (long long i = 0; i < n; i++) {
        unsigned long long a, b, c;
        if (scanf("%llu %llu %llu", &a, &b, &c) != 3)
            return 2;
        src[i] = a;
        dst[i] = b;
        sz[i] = c;
    }
    FakeOps ops;
    ops.fail_create_at = fc;
    ops.fail_copy_at = fp;
    const kvt::EngineTally t = kvt::run_engine_copies(ops, src.data(), dst.data(), sz.data(), n,
                                                      window, max_run);
    for (auto &kv : ops.sigs)
        if (kv.second.alive)
            ops.bad("signal left alive");
    printf("T %d %d %lld %lld %lld %lld %lld\n", t.status, t.failed_at, (long long)t.runs,
           (long long)t.created, (long long)t.submitted, (long long)t.waited,
           (long long)t.destroyed);
    for (auto &c : ops.copies)
        printf("C %llu %llu %llu\n", (unsigned long long)c[0], (unsigned long long)c[1],
               (unsigned long long)c[2]);
    for (auto &v : ops.violations)
        printf("V %s\n", v.c_str());
    return 0;
}
