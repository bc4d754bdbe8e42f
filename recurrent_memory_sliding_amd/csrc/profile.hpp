// profile.hpp -- optional per-kernel timing with HIP events.
//
// While timing is switched on (maglev_profile_enable), a Scope placed around a
// launch records one event before and one after it on the launch stream. The
// pairs are resolved and summed per kernel name by maglev_profile_count().
// A Scope made with Attach records nothing itself: the caller hands start()
// and stop() to hipExtLaunchKernelGGL, which binds both events to that one
// dispatch, so the pair reads the dispatch's own start and end times and adds
// no marker packets (each of those leaves a gap of several microseconds on the
// stream). Launches on a stream under graph capture are not recorded.
//
// Debug mode (the environment variable MAGLEV_DEBUG set to a value other than
// "0" when the library loads, or maglev_debug_enable): when a Scope ends, it
// also takes the launch error and synchronises its stream (not under graph
// capture); the first failure on this thread is kept, with the Scope's kernel
// name, for the C-ABI layer to report.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace maglev {
namespace prof {

class Scope {
public:
    struct Attach {};
    Scope(const char *name, hipStream_t s);
    Scope(const char *name, hipStream_t s, Attach);
    ~Scope();
    // Attach mode: the events for the launch (null while timing is off).
    hipEvent_t start() const { return attach_ ? start_ : nullptr; }
    hipEvent_t stop() const { return attach_ ? stop_ : nullptr; }
    Scope(const Scope &) = delete;
    Scope &operator=(const Scope &) = delete;

private:
    const char *name_;
    hipStream_t s_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
    int dev_ = -1;
    bool attach_ = false;

    void open(hipStream_t s);
};

// Debug mode only: the check a Scope makes when it ends, for launches outside one.
void debug_after(const char *name, hipStream_t s);
// Takes (and clears) the failure debug mode recorded on this thread; false if none.
bool debug_take(const char **kernel, hipError_t *err);

}  // namespace prof
}  // namespace maglev
