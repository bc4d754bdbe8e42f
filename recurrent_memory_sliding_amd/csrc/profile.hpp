// profile.hpp -- optional per-kernel timing with HIP events.
//
// While timing is switched on (maglev_profile_enable), a Scope placed around a
// launch records one event before and one after it on the launch stream. The
// pairs are resolved and summed per kernel name by maglev_profile_count().
// Launches on a stream under graph capture are not recorded.
//
// Debug mode (the environment variable MAGLEV_DEBUG set to a value other than
// "0" when the library loads, or maglev_debug_enable): when a Scope ends, it
// also takes the launch error and synchronises its stream (not under graph
// capture); the first failure on this thread is kept, with the Scope's kernel
// name, for the C-ABI layer to report.
#pragma once

#include <hip/hip_runtime.h>

namespace maglev {
namespace prof {

class Scope {
public:
    Scope(const char *name, hipStream_t s);
    ~Scope();
    Scope(const Scope &) = delete;
    Scope &operator=(const Scope &) = delete;

private:
    const char *name_;
    hipStream_t s_;
    hipEvent_t start_ = nullptr, stop_ = nullptr;
    int dev_ = -1;
};

// Debug mode only: the check a Scope makes when it ends, for launches outside one.
void debug_after(const char *name, hipStream_t s);
// Takes (and clears) the failure debug mode recorded on this thread; false if none.
bool debug_take(const char **kernel, hipError_t *err);

}  // namespace prof
}  // namespace maglev
