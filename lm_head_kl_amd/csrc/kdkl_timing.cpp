// Per-kernel timing with HIP events, for profiling (off by default).
//
// While enabled, every launch the library makes is bracketed by two events recorded on the
// launch's own stream. kd_timing_read synchronises the recorded pairs and adds up, per kernel
// kind, the launches and their elapsed time. Events come from a pool that grows on demand and
// is reused after kd_timing_reset. The totals and the event pool are process-wide and guarded
// by a mutex; the bracket of the launch being enqueued is per thread, so calls made from
// several threads at once each time their own launches.

#include <hip/hip_runtime_api.h>

#include <mutex>
#include <vector>

#include "kdkl.h"
#include "kdkl_internal.h"

namespace kdkl {

namespace {

const char* const kNames[kNumKinds] = {
    "plan", "teacher_prob", "validate", "fwd", "combine", "loss_final", "bwd_grad", "transpose",
    "dh", "dh_reduce", "dw", "dense_logits", "dense_rows", "sum_rows", "grad_z", "topk",
};

struct Rec {
    int kind;
    hipEvent_t a, b;
};

struct State {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> pool;  // free events
    std::vector<Rec> recs;         // recorded, not yet read
    int64_t launches[kNumKinds] = {0};
    double ms[kNumKinds] = {0};
};

// Bracket of the launch this thread is enqueueing (begin and end come from the same thread).
thread_local Rec t_open{-1, nullptr, nullptr};

State& st() {
    static State s;
    return s;
}

hipEvent_t take_event(State& s) {
    if (!s.pool.empty()) {
        hipEvent_t e = s.pool.back();
        s.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void drain(State& s) {
    for (Rec& r : s.recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
            s.launches[r.kind] += 1;
            s.ms[r.kind] += t;
        }
        s.pool.push_back(r.a);
        s.pool.push_back(r.b);
    }
    s.recs.clear();
}

}  // namespace

void timing_begin(int kind, hipStream_t stream) {
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    if (!s.on) return;
    hipEvent_t a = take_event(s), b = take_event(s);
    if (!a || !b) {
        if (a) s.pool.push_back(a);
        if (b) s.pool.push_back(b);
        return;
    }
    if (hipEventRecord(a, stream) != hipSuccess) {
        s.pool.push_back(a);
        s.pool.push_back(b);
        return;
    }
    t_open = Rec{kind, a, b};
}

void timing_end(int kind, hipStream_t stream) {
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    if (t_open.kind != kind) return;
    if (s.on && hipEventRecord(t_open.b, stream) == hipSuccess) {
        s.recs.push_back(t_open);
    } else {
        s.pool.push_back(t_open.a);
        s.pool.push_back(t_open.b);
    }
    t_open = Rec{-1, nullptr, nullptr};
}

}  // namespace kdkl

using namespace kdkl;

extern "C" {

int kd_timing_enable(int on) {
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    const int was = s.on ? 1 : 0;
    s.on = on != 0;
    return was;
}

int kd_timing_kinds(void) { return kNumKinds; }

const char* kd_timing_name(int kind) { return (kind >= 0 && kind < kNumKinds) ? kNames[kind] : "unknown"; }

kd_status kd_timing_read(int kind, int64_t* launches, double* total_ms) {
    if (kind < 0 || kind >= kNumKinds) return KD_ERR_VALUE;
    if (!launches || !total_ms) return KD_ERR_NULL;
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    drain(s);
    *launches = s.launches[kind];
    *total_ms = s.ms[kind];
    return KD_OK;
}

void kd_timing_reset(void) {
    State& s = st();
    std::lock_guard<std::mutex> g(s.mu);
    drain(s);
    for (int k = 0; k < kNumKinds; ++k) {
        s.launches[k] = 0;
        s.ms[k] = 0.0;
    }
}

}  // extern "C"
