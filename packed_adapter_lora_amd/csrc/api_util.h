// api_util.h -- error reporting, alignment checks and kernel timing shared by
// the C ABI translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

namespace plora {

// Records the message for plora_last_error() and returns `status`.
int fail(int status, const std::string& why);
int hip_fail(hipError_t e, const char* what);

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// ---- kernel timing (process-wide switch for benchmarks) ----------------------
struct ProfRec {
    std::string cls;
    hipEvent_t a, b;
};
struct Prof {
    std::atomic<bool> on{false};
    std::vector<ProfRec> recs;
    std::vector<hipEvent_t> pool;
    std::mutex mu;
};
extern Prof g_prof;
hipEvent_t take_event();

// Runs `fn` (which enqueues kernels on `st`); with profiling on, brackets it
// with a HIP event pair recorded under kernel class `cls`.
template <class Fn>
hipError_t timed(const char* cls, hipStream_t st, Fn&& fn) {
    if (!g_prof.on.load(std::memory_order_relaxed)) return fn();
    std::lock_guard<std::mutex> lk(g_prof.mu);
    hipEvent_t a = take_event(), b = take_event();
    if (!a || !b) {  // (no events: run untimed, keep what was taken)
        if (a) g_prof.pool.push_back(a);
        if (b) g_prof.pool.push_back(b);
        return fn();
    }
    (void)hipEventRecord(a, st);
    const hipError_t e = fn();
    (void)hipEventRecord(b, st);
    g_prof.recs.push_back({cls, a, b});
    return e;
}

}  // namespace plora
