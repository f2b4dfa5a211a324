// Optional per-kernel event timing.  While enabled, each bracketed launch records one HIP event
// before and one after the kernel on the stream it is launched on; a query synchronises the
// recorded events and sums the elapsed times of one kernel name.  Instrumentation only: the
// entry points behave the same with it off (the default), and it is not thread-safe.
#include <hip/hip_runtime.h>
#include <string.h>

#include <string>
#include <vector>

#include "kernels.h"

namespace jenga {

namespace {
struct Rec {
  std::string name;
  hipEvent_t start, stop;
};
bool g_on = false;
std::vector<Rec> g_recs;      // events are reused across enable/clear cycles
size_t g_used = 0;
}  // namespace

bool timing_enabled() { return g_on; }

TimedLaunch::TimedLaunch(const char* name, hipStream_t st) : st_(st), idx_(-1) {
  if (!g_on) return;
  if (g_used == g_recs.size()) {
    Rec r{std::string(), nullptr, nullptr};
    if (hipEventCreate(&r.start) != hipSuccess) return;
    if (hipEventCreate(&r.stop) != hipSuccess) { (void)hipEventDestroy(r.start); return; }
    g_recs.push_back(r);
  }
  Rec& r = g_recs[g_used];
  if (hipEventRecord(r.start, st) != hipSuccess) return;
  r.name = name;
  idx_ = (long)g_used++;
}

TimedLaunch::~TimedLaunch() {
  if (idx_ >= 0) (void)hipEventRecord(g_recs[(size_t)idx_].stop, st_);
}

void timing_set(bool on) {
  g_on = on;
  if (on) g_used = 0;
}

hipError_t timing_query(const char* name, int* launches, double* total_ms) {
  int n = 0;
  double t = 0.0;
  for (size_t i = 0; i < g_used; ++i) {
    const Rec& r = g_recs[i];
    if (r.name != name) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return e;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return e;
    ++n;
    t += ms;
  }
  *launches = n;
  *total_ms = t;
  return hipSuccess;
}

}  // namespace jenga
