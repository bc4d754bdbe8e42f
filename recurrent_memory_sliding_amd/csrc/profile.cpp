// profile.cpp -- event pool and per-name totals behind maglev_profile_*.
#include "profile.hpp"

#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "maglev.h"

namespace maglev {
namespace prof {
namespace {

struct Pending {
    const char *name;
    int dev;
    hipEvent_t start, stop;
};
struct Total {
    int64_t launches = 0;
    double ms = 0.0;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::string g_only;   // record only this kernel name when non-empty
std::map<int, std::vector<hipEvent_t>> g_pool;   // free events per device
std::vector<Pending> g_pending;
std::map<std::string, Total> g_totals;

bool env_debug()
{
    const char *v = getenv("MAGLEV_DEBUG");
    return v && *v && strcmp(v, "0") != 0;
}
std::atomic<bool> g_debug{env_debug()};
thread_local const char *t_dbg_kernel = nullptr;
thread_local hipError_t t_dbg_err = hipSuccess;

}  // namespace

// Debug mode, after the launches of one Scope: their launch error, else what
// synchronising the stream reports (a fault in them or in earlier work).
void debug_check(const char *name, hipStream_t s)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess && t_dbg_err == hipSuccess) {
        t_dbg_err = e;
        t_dbg_kernel = name;
    }
}

void debug_after(const char *name, hipStream_t s)
{
    if (g_debug.load(std::memory_order_relaxed)) debug_check(name, s);
}

namespace {

hipEvent_t take(int dev)
{
    auto &v = g_pool[dev];
    if (!v.empty()) {
        hipEvent_t e = v.back();
        v.pop_back();
        return e;
    }
    // Timing only: no system-scope fence at record time, so recording does not
    // write back and invalidate the caches ahead of the kernel being timed
    // (a 6 µs gap on each side of it, and colder caches for what follows).
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

void give(int dev, hipEvent_t e)
{
    if (e) g_pool[dev].push_back(e);
}

// Resolve every pending pair into the totals (caller holds g_mu).
void drain()
{
    for (const Pending &p : g_pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(p.stop) == hipSuccess &&
            hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
            Total &t = g_totals[p.name];
            t.launches += 1;
            t.ms += ms;
        }
        give(p.dev, p.start);
        give(p.dev, p.stop);
    }
    g_pending.clear();
}

}  // namespace

Scope::Scope(const char *name, hipStream_t s) : name_(name), s_(s) { open(s); }

Scope::Scope(const char *name, hipStream_t s, Attach) : name_(name), s_(s), attach_(true)
{
    open(s);
}

void Scope::open(hipStream_t s)
{
    if (!g_on.load(std::memory_order_relaxed)) return;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!g_only.empty() && g_only != name_) return;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    if (hipGetDevice(&dev_) != hipSuccess) return;
    std::lock_guard<std::mutex> lk(g_mu);
    start_ = take(dev_);
    stop_ = take(dev_);
    if (!start_ || !stop_ || (!attach_ && hipEventRecord(start_, s) != hipSuccess)) {
        give(dev_, start_);
        give(dev_, stop_);
        start_ = stop_ = nullptr;
    }
}

Scope::~Scope()
{
    if (start_) {
        std::lock_guard<std::mutex> lk(g_mu);
        // Attach mode: the launch recorded both events, unless it failed (then
        // they still hold an earlier launch's times and are not read).
        const bool ok = attach_ ? hipPeekAtLastError() == hipSuccess
                                : hipEventRecord(stop_, s_) == hipSuccess;
        if (ok) {
            g_pending.push_back({name_, dev_, start_, stop_});
        } else {
            give(dev_, start_);
            give(dev_, stop_);
        }
    }
    if (g_debug.load(std::memory_order_relaxed)) debug_check(name_, s_);
}

bool debug_take(const char **kernel, hipError_t *err)
{
    if (t_dbg_err == hipSuccess) return false;
    *kernel = t_dbg_kernel;
    *err = t_dbg_err;
    t_dbg_err = hipSuccess;
    t_dbg_kernel = nullptr;
    return true;
}

}  // namespace prof
}  // namespace maglev

using namespace maglev::prof;

extern "C" {

maglev_status_t maglev_debug_enable(int on)
{
    g_debug.store(on != 0);
    return MAGLEV_OK;
}

int maglev_debug_enabled(void) { return g_debug.load() ? 1 : 0; }

maglev_status_t maglev_profile_enable(int on, const char *only)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (on) {
        drain();
        g_totals.clear();
        g_only = only ? only : "";
    }
    g_on.store(on != 0);
    return MAGLEV_OK;
}

int maglev_profile_count(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    drain();
    return (int)g_totals.size();
}

maglev_status_t maglev_profile_entry(int index, const char **name, int64_t *launches,
                                     double *total_ms)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (index < 0 || index >= (int)g_totals.size() || !name || !launches || !total_ms)
        return MAGLEV_ERR_INVALID_VALUE;
    auto it = g_totals.begin();
    std::advance(it, index);
    *name = it->first.c_str();
    *launches = it->second.launches;
    *total_ms = it->second.ms;
    return MAGLEV_OK;
}

}  // extern "C"
