/*
 * Seeded synthetic inputs shared by the CPU oracle and the GPU library's tests
 * and benchmark.  This module holds none of the decoding method's arithmetic:
 * it only turns (seed, tensor id, element index) into weights and token ids.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), counter-based, so any element can be
 * produced independently on the host or on the device with identical bits.
 *
 * Weight element e of tensor t (row-major flat index of the tensor's logical
 * [out, in] shape):
 *   a = philox(ctr = {lo32(e), hi32(e), t, 0}, key = {lo32(seed), hi32(seed)})
 *   b = philox(ctr = {lo32(e), hi32(e), t, 1}, key)
 *   S = sum of the twelve 16-bit halves a0.lo a0.hi a1.lo ... a3.hi b0.lo ... b1.hi
 *   w = fp32( (float)(S - 393210) * (std * 2^-16) )     (one IEEE fp32 multiply)
 * S - 393210 is the Irwin-Hall sum of 12 uniforms, centred: mean 0, variance
 * 65536^2 - 1, so w has mean 0 and standard deviation std (to 1e-10).  Every
 * step is integer or a single correctly rounded fp32 operation, so the host and
 * device produce the same bits.  The bf16 form is round-to-nearest-even of w.
 *
 * Token element e of stream s, vocabulary V:
 *   x = philox(ctr = {lo32(e), hi32(e), s, 2}, key).word0 ;  tok = (x * V) >> 32
 */
#ifndef SSD_SYNTH_H
#define SSD_SYNTH_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* dtype codes for synth_fill_* */
#define SYNTH_F32  0
#define SYNTH_BF16 1
#define SYNTH_F64  2

/* One Philox4x32-10 block.  ctr[4], key[2] in, out[4] out. */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Fill out[0..n) with elements [e0, e0+n) of weight tensor `tensor_id`.
 * dtype SYNTH_F32 -> float*, SYNTH_BF16 -> uint16_t* (bf16 bits),
 * SYNTH_F64 -> double* holding the fp32 value (round_bf16 != 0: the bf16 value).
 * Returns 0, or -1 on a bad dtype.  Uses OpenMP threads. */
int synth_fill_weight_host(void* out, int dtype, int round_bf16, uint64_t e0, uint64_t n,
                           uint64_t seed, uint32_t tensor_id, float std);

/* Fill out[0..n) with token ids uniform in [0, vocab) from stream `stream_id`. */
int synth_fill_tokens_host(int32_t* out, uint64_t n, uint64_t seed, uint32_t stream_id,
                           int32_t vocab);

/* Device variants (libssd_synth_dev.so): same values, written by a HIP kernel
 * into device memory `out` on `stream` (a hipStream_t, 0 = default).
 * Return 0, or a negative code (-1 bad argument, -2 HIP error). */
int synth_fill_weight_dev(void* out, int dtype, uint64_t e0, uint64_t n, uint64_t seed,
                          uint32_t tensor_id, float std, void* stream);
int synth_fill_tokens_dev(int32_t* out, uint64_t n, uint64_t seed, uint32_t stream_id,
                          int32_t vocab, void* stream);

#ifdef __cplusplus
}
#endif
#endif
