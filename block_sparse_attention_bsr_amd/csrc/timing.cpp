// Optional per-kernel timing (bsr_attn_timing_begin/end): an event pair per
// launch, recorded on the launch stream, kept per calling thread.
//
// The events are created with hipEventDisableSystemFence: a default event
// performs a system-scope release when it completes, which writes back and
// invalidates the caches between the timed kernels and slows the kernel after
// it. These events only carry timestamps; bsr_attn_timing_end() waits for
// each stop event before reading the interval.
#include <hip/hip_runtime_api.h>

#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace bsr {
namespace {

struct TimingRec {
    std::string name;
    hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local std::vector<TimingRec> g_timing_recs;

constexpr unsigned kEventFlags = hipEventDisableSystemFence;

}  // namespace

KernelTimer::KernelTimer(const char *role, const char *dtype, int head_dim, void *stream) : stream_(stream) {
    if (!g_timing) return;
    std::string name = std::string(role) + "<" + dtype;
    if (head_dim > 0) name += "," + std::to_string(head_dim);
    TimingRec r{name + ">", nullptr, nullptr};
    if (hipEventCreateWithFlags(&r.start, kEventFlags) != hipSuccess) return;
    if (hipEventCreateWithFlags(&r.stop, kEventFlags) != hipSuccess) {
        (void)hipEventDestroy(r.start);
        return;
    }
    (void)hipEventRecord(r.start, static_cast<hipStream_t>(stream_));
    stop_ = r.stop;
    g_timing_recs.push_back(std::move(r));
}

KernelTimer::~KernelTimer() {
    if (stop_) (void)hipEventRecord(static_cast<hipEvent_t>(stop_), static_cast<hipStream_t>(stream_));
}

}  // namespace bsr

extern "C" {

bsr_attn_status bsr_attn_timing_begin(void) {
    bsr::g_timing = true;
    return BSR_ATTN_OK;
}

int bsr_attn_timing_end(bsr_attn_kernel_time *out, int max_entries) {
    using bsr::g_timing_recs;
    bsr::g_timing = false;
    std::vector<bsr_attn_kernel_time> agg;
    int status = 0;
    for (auto &r : g_timing_recs) {
        float ms = 0.f;
        if (status == 0 && (hipEventSynchronize(r.stop) != hipSuccess ||
                            hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess))
            status = -1;
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
        if (status != 0) continue;
        bsr_attn_kernel_time *slot = nullptr;
        for (auto &a : agg)
            if (r.name == a.name) slot = &a;
        if (!slot) {
            bsr_attn_kernel_time t{};
            std::strncpy(t.name, r.name.c_str(), sizeof(t.name) - 1);
            agg.push_back(t);
            slot = &agg.back();
        }
        slot->launches += 1;
        slot->total_ms += ms;
    }
    g_timing_recs.clear();
    if (status != 0) {
        bsr::set_error("HIP event query failed while collecting kernel timings");
        return -1;
    }
    const int n = static_cast<int>(agg.size());
    for (int i = 0; i < n && i < max_entries && out; ++i) out[i] = agg[i];
    return n;
}

}  // extern "C"
