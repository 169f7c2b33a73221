/* Host implementation of the seeded input generator (definitions in synth.h). */
#include "synth.h"
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static float weight_value(uint64_t e, uint64_t seed, uint32_t tid, float scale) {
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t ca[4] = {(uint32_t)e, (uint32_t)(e >> 32), tid, 0u};
  uint32_t cb[4] = {(uint32_t)e, (uint32_t)(e >> 32), tid, 1u};
  uint32_t a[4], b[4];
  synth_philox4x32_10(ca, key, a);
  synth_philox4x32_10(cb, key, b);
  int32_t s = 0;
  for (int i = 0; i < 4; ++i) s += (int32_t)(a[i] & 0xFFFFu) + (int32_t)(a[i] >> 16);
  for (int i = 0; i < 2; ++i) s += (int32_t)(b[i] & 0xFFFFu) + (int32_t)(b[i] >> 16);
  float z = (float)(s - 393210);            /* exact: |s - 393210| < 2^24 */
  return z * scale;                          /* one correctly rounded fp32 multiply */
}

static uint16_t bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; float f; memcpy(&f, &u, 4); return f;
}

int synth_fill_weight_host(void* out, int dtype, int round_bf16, uint64_t e0, uint64_t n,
                           uint64_t seed, uint32_t tensor_id, float std) {
  if (dtype != SYNTH_F32 && dtype != SYNTH_BF16 && dtype != SYNTH_F64) return -1;
  const float scale = std * (1.0f / 65536.0f);   /* exact: power-of-two scaling */
  long long nn = (long long)n;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < nn; ++i) {
    float w = weight_value(e0 + (uint64_t)i, seed, tensor_id, scale);
    if (dtype == SYNTH_F32) {
      ((float*)out)[i] = w;
    } else if (dtype == SYNTH_BF16) {
      ((uint16_t*)out)[i] = bf16_rne(w);
    } else {
      ((double*)out)[i] = round_bf16 ? (double)bf16_to_f32(bf16_rne(w)) : (double)w;
    }
  }
  return 0;
}

int synth_fill_tokens_host(int32_t* out, uint64_t n, uint64_t seed, uint32_t stream_id,
                           int32_t vocab) {
  if (vocab <= 0) return -1;
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (uint64_t e = 0; e < n; ++e) {
    uint32_t c[4] = {(uint32_t)e, (uint32_t)(e >> 32), stream_id, 2u}, x[4];
    synth_philox4x32_10(c, key, x);
    out[e] = (int32_t)(((uint64_t)x[0] * (uint64_t)vocab) >> 32);
  }
  return 0;
}
