// Opt-in kernel timing: when enabled, every kernel the library launches is
// bracketed by a pair of HIP events on its stream; the report sums the
// elapsed times per kernel name.  Diagnostics only (off by default, one
// process-wide recorder, not thread-safe while enabled).
#include <string.h>

#include <atomic>

#include "../../include/moe_lora.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int CAP = 8192;
std::atomic<int> g_on{0};
int g_used = 0;
bool g_created = false;
hipEvent_t g_start[CAP], g_stop[CAP];
const char* g_name[CAP];
}  // namespace

void timing_pre(const char* name, hipStream_t st) {
  if (!g_on.load(std::memory_order_relaxed) || g_used >= CAP) return;
  g_name[g_used] = name;
  (void)hipEventRecord(g_start[g_used], st);
}

void timing_post(hipStream_t st) {
  if (!g_on.load(std::memory_order_relaxed) || g_used >= CAP) return;
  (void)hipEventRecord(g_stop[g_used], st);
  ++g_used;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_timing_enable(int on) {
  if (on && !g_created) {
    for (int i = 0; i < CAP; ++i) {
      if (hipEventCreate(&g_start[i]) != hipSuccess || hipEventCreate(&g_stop[i]) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    }
    g_created = true;
  }
  g_used = 0;
  g_on.store(on ? 1 : 0, std::memory_order_relaxed);
  return MOE_SUCCESS;
}

int moe_timing_report(char* names, int name_len, float* total_ms, int* launches, int max_entries) {
  int n = 0;
  for (int i = 0; i < g_used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_stop[i]) != hipSuccess) return -1;
    if (hipEventElapsedTime(&ms, g_start[i], g_stop[i]) != hipSuccess) return -1;
    int j = 0;
    while (j < n && strncmp(names + (size_t)j * name_len, g_name[i], name_len) != 0) ++j;
    if (j == n) {
      if (n >= max_entries) continue;
      strncpy(names + (size_t)n * name_len, g_name[i], name_len - 1);
      names[(size_t)n * name_len + name_len - 1] = 0;
      total_ms[n] = 0.f;
      launches[n] = 0;
      ++n;
    }
    total_ms[j] += ms;
    launches[j] += 1;
  }
  g_used = 0;
  return n;
}

}  // extern "C"
