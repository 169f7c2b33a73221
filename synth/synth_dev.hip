// Device implementation of the seeded input generator (definitions in synth.h).
// Produces the same bits as synth_host.c for every element.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth.h"

namespace {

__device__ __forceinline__ void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_weight_kernel(void* out, int dtype, uint64_t e0, uint64_t n, uint64_t seed,
                                   uint32_t tid, float scale) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint64_t e = e0 + i;
    uint32_t a[4] = {(uint32_t)e, (uint32_t)(e >> 32), tid, 0u};
    uint32_t b[4] = {(uint32_t)e, (uint32_t)(e >> 32), tid, 1u};
    philox10(a, (uint32_t)seed, (uint32_t)(seed >> 32));
    philox10(b, (uint32_t)seed, (uint32_t)(seed >> 32));
    int32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += (int32_t)(a[j] & 0xFFFFu) + (int32_t)(a[j] >> 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) s += (int32_t)(b[j] & 0xFFFFu) + (int32_t)(b[j] >> 16);
    const float w = __fmul_rn((float)(s - 393210), scale);
    if (dtype == SYNTH_F32) ((float*)out)[i] = w;
    else ((uint16_t*)out)[i] = bf16_rne(w);
  }
}

__global__ void fill_tokens_kernel(int32_t* out, uint64_t n, uint64_t seed, uint32_t sid, int32_t vocab) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    uint32_t c[4] = {(uint32_t)e, (uint32_t)(e >> 32), sid, 2u};
    philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    out[e] = (int32_t)(((uint64_t)c[0] * (uint64_t)(uint32_t)vocab) >> 32);
  }
}

unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  if (g == 0) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" int synth_fill_weight_dev(void* out, int dtype, uint64_t e0, uint64_t n, uint64_t seed,
                                     uint32_t tensor_id, float std, void* stream) {
  if (!out || (dtype != SYNTH_F32 && dtype != SYNTH_BF16)) return -1;
  if (n == 0) return 0;
  const float scale = std * (1.0f / 65536.0f);
  hipLaunchKernelGGL(fill_weight_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     out, dtype, e0, n, seed, tensor_id, scale);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int synth_fill_tokens_dev(int32_t* out, uint64_t n, uint64_t seed, uint32_t stream_id,
                                     int32_t vocab, void* stream) {
  if (!out || vocab <= 0) return -1;
  if (n == 0) return 0;
  hipLaunchKernelGGL(fill_tokens_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     out, n, seed, stream_id, vocab);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
