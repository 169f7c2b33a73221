// Allocation-free acceptance (ssd_accept_noalloc): the accept / reject rule of
// ssd_accept with its scratch — the per-row decisions and draws that pass from
// the row kernel to the emit kernel — in a file-scope device array instead of
// a sequence workspace, for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Its device address is looked up once per device (on the
// entry point's first call there, with that device current) and kept; kernels
// receive that address, never the array's host-side name.  Every call on one
// GPU shares the array: calls that overlap on one GPU (different streams) race.
// Nothing in it needs to start at zero: the row kernel writes every entry the
// emit kernel reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

using namespace ssd;

namespace {

constexpr int NA_ROWS = SSD_ACCEPT_NOALLOC_MAX_DRAFT + 1;   // verify rows of the largest chain
constexpr int NA_MAX_DEVICES = 64;

// [0, NA_ROWS): accept decisions; [NA_ROWS, 2 NA_ROWS): each row's draw
static __device__ __align__(256) int scratch[2 * NA_ROWS];

std::mutex g_mu;
int* g_scratch[NA_MAX_DEVICES] = {};   // device address of `scratch` on each device (null: not looked up yet)

int na_fail(int code, const char* msg) { return set_last_error(code, msg); }

// The array's address on the current device.
int scratch_ptr(int** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NA_MAX_DEVICES)
    return na_fail(SSD_ERR_HIP, "hipGetDevice failed or device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return na_fail(SSD_ERR_HIP, "hipGetSymbolAddress of the accept scratch array failed");
    g_scratch[dev] = (int*)p;
  }
  *out = g_scratch[dev];
  return SSD_OK;
}

}  // namespace

extern "C" int ssd_accept_noalloc(const float* p_logits_dev, const float* q_logits_dev, const int32_t* draft_tokens_dev,
                                  const int32_t* n_drafted_dev, int d_max, int vocab, float temperature, uint64_t seed,
                                  int32_t iteration, int32_t* out_tokens_dev, int32_t* n_out_dev,
                                  hipStream_t stream) {
  if (!p_logits_dev || !q_logits_dev || !draft_tokens_dev || !n_drafted_dev || !out_tokens_dev || !n_out_dev)
    return na_fail(SSD_ERR_ARG, "null argument");
  if (d_max < 1 || vocab < 1) return na_fail(SSD_ERR_ARG, "d_max and vocab must be positive");
  if (d_max > SSD_ACCEPT_NOALLOC_MAX_DRAFT)
    return na_fail(SSD_ERR_CAPACITY, "d_max exceeds SSD_ACCEPT_NOALLOC_MAX_DRAFT (the scratch array's rows)");
  if (!(temperature >= 0.f) || temperature > 3.0e38f) return na_fail(SSD_ERR_ARG, "bad temperature");
  int* sc = nullptr;
  int rc = scratch_ptr(&sc);
  if (rc != SSD_OK) return rc;
  rc = launch_accept(p_logits_dev, q_logits_dev, vocab, draft_tokens_dev, n_drafted_dev, d_max, temperature, seed,
                     nullptr, iteration, sc, sc + NA_ROWS, out_tokens_dev, n_out_dev, nullptr, stream);
  if (rc != 0) return na_fail(rc, "kernel launch failed");
  return SSD_OK;
}
