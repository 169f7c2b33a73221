/*
 * ssd_profile.h — kernel-timing hooks of libssd.so, for measurement.
 *
 * While a kernel class is enabled, each launch of that class (up to
 * max_launches launches) goes out with a pair of HIP events that take the
 * dispatch's own begin and end timestamps (hipExtLaunchKernel: no marker is
 * queued around the kernel), and the library accumulates the algorithmic
 * bytes each launch must move (weights + activations read + results written,
 * each once).  ssd_profile_read waits for the events and returns the summed
 * durations.  A launch that returned at once because a device stop flag was
 * raised (a draft step after the confidence stop) moved no bytes; such
 * launches are left out of the sums and of the count.  Process-wide; not
 * thread-safe; ssd_profile_enable creates the events and a device array of
 * max_launches flags (the only device memory the hooks use).
 */
#ifndef SSD_PROFILE_H
#define SSD_PROFILE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_profile_class {
  SSD_PROF_GEMM_STORE = 0,   /* linear layers with a plain store epilogue (QKV, LM head) */
  SSD_PROF_GEMM_RESID = 1,   /* linear layers adding into the residual stream (O, down) */
  SSD_PROF_GEMM_SWIGLU = 2   /* gate/up projection with the fused SwiGLU epilogue */
} ssd_profile_class;

/* Start recording launches of `kernel_class` (discarding earlier records).
 * Returns 0, SSD_ERR_ARG (-1) or SSD_ERR_HIP (-4). */
int ssd_profile_enable(int kernel_class, int max_launches);

/* Stop recording (records are kept for ssd_profile_read). */
int ssd_profile_disable(void);

/* Synchronises the device.  *total_ms = sum of the durations of the recorded
 * launches that did their work, *n_launches = their number, *total_bytes =
 * their algorithmic bytes. */
int ssd_profile_read(double* total_ms, int* n_launches, double* total_bytes);

/* A streaming-read probe, for a measured bandwidth ceiling to set the kernels
 * against: one launch reads src_dev[0, bytes) once (2048 workgroups of 256
 * threads, each workgroup one contiguous slice, 16-byte loads, eight per thread
 * in flight)
 * and writes one word per workgroup to sink_dev[2048] (a fold of what it read,
 * so that the loads are not removed).  bytes must be a positive multiple of 64
 * and src_dev 16-byte aligned.  Enqueued on `stream` (a hipStream_t, nullable);
 * returns 0, SSD_ERR_ARG (-1) or SSD_ERR_HIP (-4). */
int ssd_probe_read(const void* src_dev, uint64_t bytes, uint32_t* sink_dev, void* stream);

#ifdef __cplusplus
}
#endif
#endif
