// Per-class kernel timer: pairs of HIP events around launches, read back and summed on request.
// A measurement aid only; off unless gptq_timer_enable(1) was called.
#include "timer.hpp"

#include <mutex>
#include <vector>

namespace gptq {

namespace {

struct Record {
    hipEvent_t start, stop;
    int cls;
};

struct TimerState {
    std::mutex mu;
    bool on = false;
    std::vector<Record> records;
    std::vector<hipEvent_t> pool;   // created once, reused

    hipEvent_t take() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        return hipEventCreate(&e) == hipSuccess ? e : nullptr;
    }
    void drop_records() {
        for (const Record& r : records) {
            pool.push_back(r.start);
            pool.push_back(r.stop);
        }
        records.clear();
    }
};

TimerState& state() {
    static TimerState s;
    return s;
}

thread_local bool t_suppressed = false;

}  // namespace

TimerSuppress::TimerSuppress() : prev_(t_suppressed) { t_suppressed = true; }
TimerSuppress::~TimerSuppress() { t_suppressed = prev_; }

TimerScope::TimerScope(hipStream_t stream, int cls) : stream_(stream), cls_(cls), start_(nullptr) {
    if (t_suppressed) return;
    TimerState& s = state();
    std::lock_guard<std::mutex> g(s.mu);
    if (!s.on) return;
    start_ = s.take();
    if (start_ && hipEventRecord(start_, stream_) != hipSuccess) {
        s.pool.push_back(start_);
        start_ = nullptr;
    }
}

TimerScope::~TimerScope() {
    if (!start_) return;
    TimerState& s = state();
    std::lock_guard<std::mutex> g(s.mu);
    hipEvent_t stop = s.on ? s.take() : nullptr;
    if (stop && hipEventRecord(stop, stream_) == hipSuccess) {
        s.records.push_back({start_, stop, cls_});
        return;
    }
    s.pool.push_back(start_);
    if (stop) s.pool.push_back(stop);
}

}  // namespace gptq

extern "C" {

gptq_status_t gptq_timer_enable(int on) {
    gptq::TimerState& s = gptq::state();
    std::lock_guard<std::mutex> g(s.mu);
    for (const auto& r : s.records) {   // let pending records finish before their events are reused
        if (hipEventSynchronize(r.stop) != hipSuccess) return GPTQ_ERR_HIP;
    }
    s.drop_records();
    s.on = on != 0;
    return GPTQ_OK;
}

gptq_status_t gptq_timer_read(double* ms, int64_t* launches) {
    if (!ms) return GPTQ_ERR_ARG;
    gptq::TimerState& s = gptq::state();
    std::lock_guard<std::mutex> g(s.mu);
    for (int c = 0; c < GPTQ_TIMER_CLASSES; ++c) {
        ms[c] = 0.0;
        if (launches) launches[c] = 0;
    }
    gptq_status_t st = GPTQ_OK;
    for (const auto& r : s.records) {
        float t = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) {
            st = GPTQ_ERR_HIP;
            continue;
        }
        if (r.cls >= 0 && r.cls < GPTQ_TIMER_CLASSES) {
            ms[r.cls] += t;
            if (launches) launches[r.cls] += 1;
        }
    }
    s.drop_records();
    return st;
}

}  // extern "C"
