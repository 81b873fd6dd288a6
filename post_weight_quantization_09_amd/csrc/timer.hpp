// Optional per-class kernel timer (gptq_timer_enable / gptq_timer_read in include/gptq.h).
#pragma once

#include "gptq_common.hpp"

namespace gptq {

// Brackets the launches issued during its lifetime with two HIP events on `stream`, attributed to `cls`
// (a gptq_timer_class_t).  Does nothing while the timer is off.
class TimerScope {
public:
    TimerScope(hipStream_t stream, int cls);
    ~TimerScope();
    TimerScope(const TimerScope&) = delete;
    TimerScope& operator=(const TimerScope&) = delete;

private:
    hipStream_t stream_;
    int cls_;
    hipEvent_t start_;
};

// While one exists on a thread, TimerScope records nothing on that thread (no events are created): used by the
// entry point that must not allocate.
class TimerSuppress {
public:
    TimerSuppress();
    ~TimerSuppress();
    TimerSuppress(const TimerSuppress&) = delete;
    TimerSuppress& operator=(const TimerSuppress&) = delete;

private:
    bool prev_;
};

}  // namespace gptq
