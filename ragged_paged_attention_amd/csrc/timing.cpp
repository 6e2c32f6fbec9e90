// Per-kernel timing for measurement (pa_bench.h): events on the launch stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "pa_bench.h"
#include "pa_internal.h"

namespace {

struct Record {
  std::string name;
  hipEvent_t start, stop;
};

bool g_on = false;
std::vector<hipEvent_t> g_pool;   // all events ever created, reused across sessions
size_t g_next = 0;                // next free event in g_pool
std::vector<Record> g_records;
std::string g_pending;            // name of the launch between mark and done
hipEvent_t g_pending_start = nullptr;

hipEvent_t next_event() {
  if (g_next == g_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_next++];
}

}  // namespace

namespace pa {

void launch_mark(const char* name, hipStream_t stream) {
  if (!g_on) return;
  g_pending = name;
  g_pending_start = next_event();
  if (g_pending_start) (void)hipEventRecord(g_pending_start, stream);
}

void launch_done(hipStream_t stream) {
  if (!g_on || !g_pending_start) return;
  hipEvent_t stop = next_event();
  if (!stop) return;
  (void)hipEventRecord(stop, stream);
  g_records.push_back({g_pending, g_pending_start, stop});
  g_pending_start = nullptr;
}

}  // namespace pa

extern "C" pa_status_t pa_bench_timing_begin(void) {
  g_on = true;
  g_next = 0;
  g_records.clear();
  return PA_OK;
}

extern "C" pa_status_t pa_bench_timing_end(pa_kernel_time_t* out, int32_t max_entries, int32_t* n_entries) {
  g_on = false;
  std::map<std::string, std::pair<int32_t, double>> agg;
  for (const Record& r : g_records) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return PA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return PA_ERR_HIP;
    auto& a = agg[r.name];
    a.first += 1;
    a.second += ms;
  }
  g_records.clear();
  std::vector<std::pair<std::string, std::pair<int32_t, double>>> v(agg.begin(), agg.end());
  std::sort(v.begin(), v.end(), [](const auto& x, const auto& y) { return x.second.second > y.second.second; });
  int32_t n = 0;
  for (const auto& e : v) {
    if (!out || n >= max_entries) break;
    std::snprintf(out[n].name, sizeof(out[n].name), "%s", e.first.c_str());
    out[n].launches = e.second.first;
    out[n].total_ms = e.second.second;
    ++n;
  }
  if (n_entries) *n_entries = n;
  return PA_OK;
}
