// profile.hpp -- optional per-kernel timing with HIP events.
//
// While timing is switched on (maglev_profile_enable), a Scope placed around a
// launch records one event before and one after it on the launch stream. The
// pairs are resolved and summed per kernel name by maglev_profile_count().
// Launches on a stream under graph capture are not recorded.
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

}  // namespace prof
}  // namespace maglev
