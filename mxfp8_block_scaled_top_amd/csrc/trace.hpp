// Optional per-launch HIP-event tracing (enabled by moe_trace_enable).
#pragma once

#include <hip/hip_runtime.h>

namespace moe {

// Records a start event on `s` when tracing is on; the destructor records the
// stop event.  Wrap exactly one kernel launch.
struct TraceScope {
    int slot;
    hipStream_t s;
    TraceScope(const char* name, hipStream_t stream);
    ~TraceScope();
};

}  // namespace moe
