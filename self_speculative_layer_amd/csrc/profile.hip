// Kernel-timing hooks (include/ssd_profile.h).  A profiled launch goes out
// through hipExtLaunchKernel with a start and a stop event: the events take
// the dispatch's own begin and end timestamps, so no marker is queued around
// the kernel and the stream's timing is unchanged.
#include <vector>

#include "kernels.h"
#include "../../include/ssd_profile.h"

namespace ssd {

namespace {
struct ProfState {
  int cls = -1;
  int max = 0;
  bool on = false;
  std::vector<hipEvent_t> ev;   // 2 per launch
  std::vector<double> bytes;
  int used = 0;
};
ProfState g_prof;
}  // namespace

bool profile_next(int cls, hipEvent_t* start, hipEvent_t* stop) {
  if (!(g_prof.on && g_prof.cls == cls && g_prof.used < g_prof.max)) return false;
  *start = g_prof.ev[2 * g_prof.used];
  *stop = g_prof.ev[2 * g_prof.used + 1];
  return true;
}

void profile_done(double bytes) {
  g_prof.bytes[g_prof.used] = bytes;
  ++g_prof.used;
}

}  // namespace ssd

using namespace ssd;

extern "C" int ssd_profile_enable(int kernel_class, int max_launches) {
  if (kernel_class < 0 || kernel_class > 2 || max_launches < 1) return SSD_ERR_ARG;
  ssd_profile_disable();
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto& e : g_prof.ev)
    if (hipEventCreate(&e) != hipSuccess) return SSD_ERR_HIP;
  g_prof.bytes.assign(max_launches, 0.0);
  g_prof.cls = kernel_class;
  g_prof.max = max_launches;
  g_prof.used = 0;
  g_prof.on = true;
  return SSD_OK;
}

extern "C" int ssd_profile_disable(void) {
  g_prof.on = false;
  return SSD_OK;
}

extern "C" int ssd_profile_read(double* total_ms, int* n_launches, double* total_bytes) {
  if (!total_ms || !n_launches || !total_bytes) return SSD_ERR_ARG;
  double ms = 0.0, by = 0.0;
  for (int i = 0; i < g_prof.used; ++i) {
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess) return SSD_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) return SSD_ERR_HIP;
    ms += t;
    by += g_prof.bytes[i];
  }
  *total_ms = ms;
  *n_launches = g_prof.used;
  *total_bytes = by;
  return SSD_OK;
}
