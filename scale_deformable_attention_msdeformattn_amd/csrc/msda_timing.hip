// Per-kernel timing for benchmarks: event pairs recorded around each launch
// on the launch's own stream, folded into per-kernel totals on request.
#include <cstring>
#include <mutex>
#include <vector>

#include "msda_internal.h"

namespace msda {
namespace {

struct Pending {
    int entry;
    hipEvent_t start, stop;
};

struct Entry {
    const char *name;
    double total_ms;
    int64_t launches;
};

std::mutex g_mu;
bool g_enabled = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;  // recycled events
std::vector<Entry> g_entries;
thread_local int g_suppressed = 0;  // TimingOff scopes open on this thread

hipEvent_t take_event()
{
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

int entry_of(const char *name)
{
    for (size_t i = 0; i < g_entries.size(); ++i)
        if (std::strcmp(g_entries[i].name, name) == 0) return (int)i;
    g_entries.push_back({name, 0.0, 0});
    return (int)g_entries.size() - 1;
}

// Waits for every pending pair; adds it to its entry unless `discard`.
hipError_t drain(bool discard)
{
    hipError_t err = hipSuccess;
    for (const Pending &p : g_pending) {
        hipError_t e = hipEventSynchronize(p.stop);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
        if (e == hipSuccess && !discard) {
            g_entries[p.entry].total_ms += ms;
            g_entries[p.entry].launches += 1;
        }
        if (e != hipSuccess && err == hipSuccess) err = e;
        g_pool.push_back(p.start);
        g_pool.push_back(p.stop);
    }
    g_pending.clear();
    return err;
}

}  // namespace

bool timing_on(hipStream_t st)
{
    if (g_suppressed) return false;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!g_enabled) return false;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusNone;
}

TimingOff::TimingOff() { ++g_suppressed; }
TimingOff::~TimingOff() { --g_suppressed; }

KernelScope::KernelScope(const char *name, hipStream_t st) : name_(name), st_(st), start_(nullptr)
{
    if (g_suppressed) return;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_enabled) return;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    start_ = take_event();
    if (start_ && hipEventRecord(start_, st) != hipSuccess) {
        g_pool.push_back(start_);
        start_ = nullptr;
    }
}

KernelScope::~KernelScope()
{
    if (!start_) return;
    std::lock_guard<std::mutex> lock(g_mu);
    hipEvent_t stop = take_event();
    if (!stop || hipEventRecord(stop, st_) != hipSuccess) {
        g_pool.push_back(start_);
        if (stop) g_pool.push_back(stop);
        return;
    }
    g_pending.push_back({entry_of(name_), start_, stop});
}

}  // namespace msda

extern "C" {

int msda_timing_enable(int on)
{
    std::lock_guard<std::mutex> lock(msda::g_mu);
    msda::g_enabled = on != 0;
    return MSDA_OK;
}

int msda_timing_reset(void)
{
    std::lock_guard<std::mutex> lock(msda::g_mu);
    const hipError_t e = msda::drain(true);
    msda::g_entries.clear();
    return e == hipSuccess ? MSDA_OK : MSDA_E_HIP;
}

int msda_timing_read(int index, int *count, const char **name, double *total_ms, int64_t *launches)
{
    std::lock_guard<std::mutex> lock(msda::g_mu);
    const hipError_t e = msda::drain(false);
    const int n = (int)msda::g_entries.size();
    if (count) *count = n;
    if (e != hipSuccess) return MSDA_E_HIP;
    if (index == -1) return MSDA_OK;
    if (index < 0 || index >= n) return MSDA_E_DIM;
    const msda::Entry &en = msda::g_entries[index];
    if (name) *name = en.name;
    if (total_ms) *total_ms = en.total_ms;
    if (launches) *launches = en.launches;
    return MSDA_OK;
}

}  // extern "C"
