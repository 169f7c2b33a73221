// Shared device/host definitions of the self-speculative decoding library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// Flags in DevState::error_flags.
constexpr int ERRF_CAPACITY = 1;
constexpr int ERRF_NUMERIC = 2;
constexpr int ERRF_INPUT = 4;       // a device-side argument out of range (e.g. a tree leaf's depth)

// Draft trees: candidates per draft step, and leaf rows a tree verify can hold (16-row decode blocks
// with at least one chain row).
constexpr int TREE_KMAX = 8;
constexpr int TREE_SLOTS = 15;

// Per-sequence state that lives on the device, so that the host can enqueue
// a whole decode iteration without reading anything back.
struct DevState {
  int32_t kvlen;        // positions with committed K/V (= committed tokens - 1)
  int32_t last_token;   // newest committed token (input of the next step)
  int32_t iteration;    // random-draw address: 0 = prefill's token, SSD iterations from 1
  int32_t n_out;        // tokens in the output log
  int32_t error_flags;  // ERRF_* (sticky)
  int32_t n_drafted;    // d' of the last draft
  int32_t stop;         // draft early-stop flag (kernels of later draft steps exit at once)
  int32_t n_emitted;    // tokens emitted by the last commit
  int32_t verify_rows;  // d' + 1 of the current verify
  // tree verify: active rows of the full and prefix blocks, their first leaf row, and the leaf the
  // acceptance took (-1: none) with its position
  int32_t tree_rows, tree_prefix_rows, tree_side_full, tree_side_prefix, tree_leaf, tree_leaf_pos;
  int32_t pad[1];
};

// ---------------------------------------------------------------------------
// Conversions

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }

// ---------------------------------------------------------------------------
// Wave / block reductions (64-lane wavefronts)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// (value, index) maximum with the lowest index winning ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, WAVE);
    int i2 = __shfl_xor(i, o, WAVE);
    argmax_merge(v, i, v2, i2);
  }
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): the random draws of the
// accept rule.  key = (seed lo, seed hi); counter = (iteration, row, purpose,
// element / 4); word element % 4.

constexpr uint32_t PURPOSE_DRAFT = 0;
constexpr uint32_t PURPOSE_ACCEPT = 1;
constexpr uint32_t PURPOSE_SAMPLE = 2;
constexpr uint32_t PURPOSE_LEAF = 4;           // draft trees: the extra candidates of a draft step
constexpr int TREE_ROW_STRIDE = 256;           //   candidate r of draft row i: counter row i + 256 r

struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c0;
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

// Uniform in (0, 1), exact in float32: (2 * (x >> 9) + 1) * 2^-24.
__device__ __forceinline__ float word_to_uniform(uint32_t x) {
  return (float)(2u * (x >> 9) + 1u) * 5.9604644775390625e-08f;
}

// Gumbel(0, 1) noise -log(-log u), float32.
__device__ __forceinline__ float word_to_gumbel(uint32_t x) {
  return -logf(-logf(word_to_uniform(x)));
}

}  // namespace ssd

namespace ssd {

// Single-rounding float operations the compiler never fuses with a
// neighbouring operation.  The toolchain's __fmul_rn / __fadd_rn are plain
// operators that may still be contracted into a fused multiply-add, and the
// compiler chooses which product to fuse kernel by kernel; steps that several
// kernels must perform with the same bits use these instead.
__device__ __forceinline__ float fmul_nc(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float fadd_nc(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}
__device__ __forceinline__ float fsub_nc(float a, float b) {
#pragma clang fp contract(off)
  return a - b;
}

// ---------------------------------------------------------------------------
// Canonical RMS reductions.  The residual stream's sum of squares is formed
// as (1) per group of 16 consecutive features, a butterfly over 16 lanes
// (xor 8, 4, 2, 1), then (2) over the groups: lane j of one wave adds groups
// j, j + 64, j + 128, ... in order, then a butterfly over 64 lanes.  Every
// kernel that needs a row's RMS uses these functions, so the result is the
// same bits whichever kernel produced or consumes it.

// (1) with the 16 values held by 16 consecutive lanes; every lane gets the sum.
__device__ __forceinline__ float tile16_ss_lanes(float v) {
  float s = fmul_nc(v, v);
  s = fadd_nc(s, __shfl_xor(s, 8, 16));
  s = fadd_nc(s, __shfl_xor(s, 4, 16));
  s = fadd_nc(s, __shfl_xor(s, 2, 16));
  s = fadd_nc(s, __shfl_xor(s, 1, 16));
  return s;
}

// (2) by one full wave over ntiles group sums at tiles[t * stride]; every lane gets the total.
__device__ __forceinline__ float row_ss_total(const float* tiles, int stride, int ntiles) {
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int t = lane; t < ntiles; t += 64) acc += tiles[(size_t)t * stride];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, WAVE);
  return acc;
}

__device__ __forceinline__ float inv_rms(float ss_total, int D, float eps) {
  return __fdiv_rn(1.0f, __fsqrt_rn(fadd_nc(__fdiv_rn(ss_total, (float)D), eps)));
}

// Elementwise steps shared by every kernel that performs them, each written
// with the operations above so that every kernel rounds them the same way.
// Rotation of the pair (x1, x2) by the angle whose (cos, sin) is cs.  The
// table of (cos, sin)(pos * theta^(-2i/hd)) is formed in fp64 and rounded to
// fp32 when a sequence is created.
__device__ __forceinline__ void rope_apply(float x1, float x2, float2 cs, float& y1, float& y2) {
  y1 = fsub_nc(fmul_nc(x1, cs.x), fmul_nc(x2, cs.y));
  y2 = fadd_nc(fmul_nc(x2, cs.x), fmul_nc(x1, cs.y));
}

// Packed bf16 projection weights: element (n, k) of an [N, K] matrix, in
// 16-row groups of 32-column steps stored as 16 x 32 contiguous elements (one
// matrix-core A operand per 1 KB).
__device__ __forceinline__ size_t wpk_index(int n, int k, int K) {
  return ((size_t)(n >> 4) * (size_t)(K >> 5) + (size_t)(k >> 5)) * 512 + (size_t)(n & 15) * 32 + (k & 31);
}

// Activation layout of a decode block (at most 16 rows): blocks of 32
// columns, each holding the 16 rows' 32 values contiguously, so that one
// matrix-core step's activations (16 rows x 32 columns) are one 1 KB run.
__device__ __forceinline__ size_t dec_act_index(int row, int col) {
  return (size_t)(col >> 5) * 512 + (size_t)row * 32 + (col & 31);
}

// fp32 rows of a decode block (the h * gain inputs of RMSNorm consumers): the
// same 32-column blocks of 16 rows, each split into two 1 KB halves so that a
// matrix-core step's operand (lane = 16 g + row takes k = 8g .. 8g + 7) is two
// loads of 16 contiguous bytes per lane, each load one contiguous 1 KB run:
// half 0 holds k = 8g .. 8g + 3, half 1 k = 8g + 4 .. 8g + 7.
__device__ __forceinline__ size_t dec_actf_index(int row, int col) {
  const int kk = col & 31;
  return (size_t)(col >> 5) * 512 + (size_t)((kk >> 2) & 1) * 256 + (size_t)((kk >> 3) * 16 + row) * 4 + (kk & 3);
}

// Projection input of an RMSNorm: bf16 (round to nearest even, the matrix
// cores' conversion) of (h * gain) * inv_rms.  The residual's product with the
// gain is formed by whichever kernel last updated h; the consumer applies the
// row's 1 / rms before rounding, so the stored value is RMSNorm(h) * gain
// rounded once.  Every kernel that forms such an input uses these functions.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t norm_pack2(float hg0, float hg1, float inv) {
  const bf16x2_t v = {(__bf16)fmul_nc(hg0, inv), (__bf16)fmul_nc(hg1, inv)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16_t norm_bf16(float hg, float inv) {
  return (bf16_t)(norm_pack2(hg, 0.f, inv) & 0xFFFFu);
}

__device__ __forceinline__ float swiglu(float g, float u) {
  return fmul_nc(__fdiv_rn(g, fadd_nc(1.0f, expf(-g))), u);
}

}  // namespace ssd
