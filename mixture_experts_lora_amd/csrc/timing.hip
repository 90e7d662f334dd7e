// Opt-in kernel timing: when enabled, every kernel the library launches is
// bracketed by a pair of HIP events on its stream; the report sums the
// elapsed times per kernel name.  Diagnostics only (off by default).  Each
// host thread has its own recorder, so the autotune of one thread and the
// calls of another do not mix their records.
#include <string.h>

#include "../../include/moe_lora.h"
#include "kernels.h"

namespace moe {

namespace {
constexpr int CAP = 8192;
struct Recorder {
  int on = 0, used = 0;
  bool created = false;
  hipEvent_t start[CAP], stop[CAP];
  const char* name[CAP];
};
// created on a thread's first enable (events and all), kept until exit
thread_local Recorder* t_rec = nullptr;
}  // namespace

void timing_pre(const char* name, hipStream_t st) {
  if (!t_rec) return;
  Recorder& r = *t_rec;
  if (!r.on || r.used >= CAP) return;
  r.name[r.used] = name;
  (void)hipEventRecord(r.start[r.used], st);
}

void timing_post(hipStream_t st) {
  if (!t_rec) return;
  Recorder& r = *t_rec;
  if (!r.on || r.used >= CAP) return;
  (void)hipEventRecord(r.stop[r.used], st);
  ++r.used;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status moe_timing_enable(int on) {
  if (!t_rec) {
    if (!on) return MOE_SUCCESS;
    t_rec = new Recorder();
  }
  Recorder& r = *t_rec;
  if (on && !r.created) {
    for (int i = 0; i < CAP; ++i) {
      if (hipEventCreate(&r.start[i]) != hipSuccess || hipEventCreate(&r.stop[i]) != hipSuccess)
        return MOE_ERROR_LAUNCH;
    }
    r.created = true;
  }
  r.used = 0;
  r.on = on ? 1 : 0;
  return MOE_SUCCESS;
}

int moe_timing_report(char* names, int name_len, float* total_ms, int* launches, int max_entries) {
  if (!t_rec) return 0;
  Recorder& r = *t_rec;
  int n = 0;
  for (int i = 0; i < r.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop[i]) != hipSuccess) return -1;
    if (hipEventElapsedTime(&ms, r.start[i], r.stop[i]) != hipSuccess) return -1;
    int j = 0;
    while (j < n && strncmp(names + (size_t)j * name_len, r.name[i], name_len) != 0) ++j;
    if (j == n) {
      if (n >= max_entries) continue;
      strncpy(names + (size_t)n * name_len, r.name[i], name_len - 1);
      names[(size_t)n * name_len + name_len - 1] = 0;
      total_ms[n] = 0.f;
      launches[n] = 0;
      ++n;
    }
    total_ms[j] += ms;
    launches[j] += 1;
  }
  r.used = 0;
  return n;
}

}  // extern "C"
