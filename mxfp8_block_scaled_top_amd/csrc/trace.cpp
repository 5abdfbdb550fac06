// Per-launch HIP-event trace: the caller enables it with a capacity, runs
// library calls, synchronizes, then reads one (name, milliseconds) pair per
// kernel launch.  Events are created once, at enable time, never in the
// traced calls.  Intended for measurement; not for concurrent use from
// several host threads.
#include <hip/hip_runtime.h>

#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "moe_mi355x.h"
#include "trace.hpp"

namespace {

struct TraceState {
    std::mutex mu;
    bool on = false;
    int count = 0;
    std::vector<hipEvent_t> ev;  // 2 per slot
    std::vector<const char*> names;
    std::string prefix;          // only launches whose name starts with it
};

TraceState& st() {
    static TraceState s;
    return s;
}

}  // namespace

namespace moe {

TraceScope::TraceScope(const char* name, hipStream_t stream) : slot(-1), s(stream) {
    TraceState& t = st();
    std::lock_guard<std::mutex> g(t.mu);
    if (!t.on || t.count >= (int)t.names.size()) return;
    if (!t.prefix.empty() && strncmp(name, t.prefix.c_str(), t.prefix.size()) != 0) return;
    slot = t.count++;
    t.names[slot] = name;
    if (hipEventRecord(t.ev[2 * slot], s) != hipSuccess) slot = -1;
}

TraceScope::~TraceScope() {
    if (slot < 0) return;
    TraceState& t = st();
    std::lock_guard<std::mutex> g(t.mu);
    (void)hipEventRecord(t.ev[2 * slot + 1], s);
}

}  // namespace moe

extern "C" {

int moe_trace_enable(int capacity) {
    TraceState& t = st();
    std::lock_guard<std::mutex> g(t.mu);
    if (capacity < 1 || capacity > (1 << 20)) return MOE_ERR_ARG;
    while ((int)t.names.size() < capacity) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return MOE_ERR_HIP;
        if (hipEventCreate(&b) != hipSuccess) return MOE_ERR_HIP;
        t.ev.push_back(a);
        t.ev.push_back(b);
        t.names.push_back(nullptr);
    }
    t.count = 0;
    t.on = true;
    return MOE_OK;
}

void moe_trace_filter(const char* prefix) {
    TraceState& t = st();
    std::lock_guard<std::mutex> g(t.mu);
    t.prefix = prefix ? prefix : "";
}

void moe_trace_disable(void) {
    TraceState& t = st();
    std::lock_guard<std::mutex> g(t.mu);
    t.on = false;
}

int moe_trace_count(void) {
    TraceState& t = st();
    std::lock_guard<std::mutex> g(t.mu);
    return t.count;
}

int moe_trace_read(int i, const char** name, float* ms) {
    TraceState& t = st();
    std::lock_guard<std::mutex> g(t.mu);
    if (i < 0 || i >= t.count || !name || !ms) return MOE_ERR_ARG;
    *name = t.names[i];
    return hipEventElapsedTime(ms, t.ev[2 * i], t.ev[2 * i + 1]) == hipSuccess ? MOE_OK
                                                                                : MOE_ERR_HIP;
}

}  // extern "C"
