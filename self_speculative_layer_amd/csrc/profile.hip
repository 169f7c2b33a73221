// Kernel-timing hooks (include/ssd_profile.h).  A profiled launch goes out
// through hipExtLaunchKernel with a start and a stop event: the events take
// the dispatch's own begin and end timestamps, so no marker is queued around
// the kernel and the stream's timing is unchanged.  Each record also has a
// device flag that says whether the launch did its work: a launch behind a
// raised device stop flag (a draft step after the confidence stop) returns at
// once and is left out of the sums.  Decode projections set the flag
// themselves; other launches with a stop flag get a one-thread marker kernel
// after them; launches without one always run.
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
  std::vector<char> host_ran;   // launch without a stop flag: ran
  int* ran_dev = nullptr;       // [max] set on the device by launches that ran
  int used = 0;
};
ProfState g_prof;
}  // namespace

__global__ void prof_mark_kernel(int* ran, const int* stop) { *ran = *stop ? 0 : 1; }

bool profile_next(int cls, hipEvent_t* start, hipEvent_t* stop, int** ran) {
  if (!(g_prof.on && g_prof.cls == cls && g_prof.used < g_prof.max)) return false;
  *start = g_prof.ev[2 * g_prof.used];
  *stop = g_prof.ev[2 * g_prof.used + 1];
  *ran = g_prof.ran_dev + g_prof.used;
  return true;
}

// stop_flag: the launch's device stop flag (nullable); self_marked: the kernel writes its ran flag.
void profile_done(double bytes, const int* stop_flag, bool self_marked, hipStream_t s) {
  const int i = g_prof.used;
  g_prof.bytes[i] = bytes;
  g_prof.host_ran[i] = stop_flag == nullptr;
  if (stop_flag && !self_marked) hipLaunchKernelGGL(prof_mark_kernel, dim3(1), dim3(1), 0, s, g_prof.ran_dev + i, stop_flag);
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
  g_prof.host_ran.assign(max_launches, 0);
  if (g_prof.ran_dev) (void)hipFree(g_prof.ran_dev);
  g_prof.ran_dev = nullptr;
  if (hipMalloc(&g_prof.ran_dev, sizeof(int) * (size_t)max_launches) != hipSuccess) return SSD_ERR_HIP;
  if (hipMemset(g_prof.ran_dev, 0, sizeof(int) * (size_t)max_launches) != hipSuccess) return SSD_ERR_HIP;
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
  int n = 0;
  std::vector<int> ran(g_prof.used, 0);
  if (g_prof.used > 0) {
    if (hipEventSynchronize(g_prof.ev[2 * g_prof.used - 1]) != hipSuccess) return SSD_ERR_HIP;
    if (hipDeviceSynchronize() != hipSuccess) return SSD_ERR_HIP;
    if (hipMemcpy(ran.data(), g_prof.ran_dev, sizeof(int) * g_prof.used, hipMemcpyDeviceToHost) != hipSuccess)
      return SSD_ERR_HIP;
  }
  for (int i = 0; i < g_prof.used; ++i) {
    if (!(g_prof.host_ran[i] || ran[i])) continue;
    if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess) return SSD_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) return SSD_ERR_HIP;
    ms += t;
    by += g_prof.bytes[i];
    ++n;
  }
  *total_ms = ms;
  *n_launches = n;
  *total_bytes = by;
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// streaming-read probe

namespace {

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, uint64_t n16,
                                                         uint32_t* __restrict__ sink) {
  // each workgroup reads one contiguous slice, eight 4 KB runs in flight per step
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t beg = min((uint64_t)blockIdx.x * per, n16), end = min(beg + per, n16);
  uint32_t acc = 0;
  uint64_t i = beg + threadIdx.x;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = src[i + k * 256];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < end; i += 256) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int k = 0; k < 256; ++k) t ^= red[k];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

extern "C" int ssd_probe_read(const void* src_dev, uint64_t bytes, uint32_t* sink_dev, void* stream) {
  if (!src_dev || !sink_dev || bytes == 0 || bytes % 64 != 0 || ((uintptr_t)src_dev & 15) != 0) return SSD_ERR_ARG;
  hipLaunchKernelGGL(probe_read_kernel, dim3(2048), dim3(256), 0, (hipStream_t)stream, (const uint4*)src_dev,
                     bytes / 16, sink_dev);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}
