// Optional per-kernel timing: when enabled, every launch of the library is
// bracketed by two HIP events recorded on the launch's own stream, so the
// elapsed time of each kernel class can be read back without a profiler.
// Disabled (the default) it costs one branch per launch.  Not for use while
// a stream is being captured into a graph.
#include <mutex>
#include <vector>

#include "kernels.hpp"

namespace csa2 {
namespace {

struct Record {
  int32_t kernel;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
thread_local bool t_suspended = false;  // this thread's launches go unrecorded
std::vector<Record> g_records;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void prof_suspend(bool on) { t_suspended = on; }

int prof_begin(int32_t kernel, hipStream_t stream) {
  if (!g_on || t_suspended) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  Record r{kernel, take_event(), take_event()};
  if (!r.start || !r.stop) return -1;
  if (hipEventRecord(r.start, stream) != hipSuccess) return -1;
  g_records.push_back(r);
  return (int)g_records.size() - 1;
}

void prof_end(int handle, hipStream_t stream) {
  if (handle < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if ((size_t)handle < g_records.size()) (void)hipEventRecord(g_records[handle].stop, stream);
}

}  // namespace csa2

using namespace csa2;

extern "C" {

int csa2_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return CSA2_OK;
}

int csa2_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_records) {
    g_free.push_back(r.start);
    g_free.push_back(r.stop);
  }
  g_records.clear();
  return CSA2_OK;
}

int csa2_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return CSA2_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  double ms = 0.0;
  int64_t n = 0;
  for (auto& r : g_records) {
    if (r.kernel != kernel) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return CSA2_ERR_HIP;
    float e = 0.0f;
    if (hipEventElapsedTime(&e, r.start, r.stop) != hipSuccess) return CSA2_ERR_HIP;
    ms += e;
    ++n;
  }
  *total_ms = ms;
  *launches = n;
  return CSA2_OK;
}

}  // extern "C"
