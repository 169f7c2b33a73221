// Attention of the mask-scoring pass (SWIFT's matchness scoring of candidate
// layer sets): every candidate's window rows attend to the shared prompt
// prefix in the paged cache and to the candidate's own window keys and values
// (the local buffer).  One workgroup takes one KV head and a block of rows of
// one candidate (all query heads of the group), and walks the keys in 64-key
// chunks in position order with a running (online) softmax, so no partial
// records and no merge launch are needed:
//   S = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16, K as A: 16 keys
//   x 32 dims, the queries as B), the chunk's maxima and probabilities in
//   fp32 registers (base 2), and O += P V on the matrix cores too, each
//   probability split into two bf16 parts (hi + lo) so that the products keep
//   ~16 bits of it.
// Each wave owns 16 queries and all 64 keys of a chunk, so the softmax needs
// no exchange between waves (the four lanes of a query exchange through
// permlane swaps).  Keys and values go straight into LDS (global_load_lds,
// double-buffered) as 1 KB tiles of 16 rows x 32 dims; the value tiles are
// read transposed (ds_read_b64_tr_b16) as the A operand of P V.
// Arithmetic differs from the split-item attention of the decode and prefill
// paths (order of the key sums, online rescaling); the scoring pass compares
// candidates with one another, never with those paths' bits.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"

namespace ssd {

namespace {

constexpr int GA_CHUNK = 64;       // keys per chunk

typedef uint32_t ga_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t ga_u32x2 __attribute__((ext_vector_type(2)));
typedef short ga_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void ga_lds_t;
typedef __attribute__((address_space(3))) ga_s16x4 ga_lds_s16x4;
typedef __attribute__((address_space(1))) const void ga_gbl_t;

// Reductions over the four lanes r, r + 16, r + 32, r + 48 (the 16-lane rows of a wave).
__device__ __forceinline__ float ga_row4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));          // rows (0, 1) and (2, 3)
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));       // halves
}
__device__ __forceinline__ float ga_row4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int HD, int NW, int PS>
__global__ __launch_bounds__(NW * 64) void attn_group_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ pool, const int* __restrict__ page_table,
    int n_lpages, int L, int layer, int H, int KVH, int M, const int* __restrict__ nrows,
    const int* __restrict__ pos, int RB, const bf16_t* __restrict__ local_kv, int local_start, int group_rows,
    bf16_t* __restrict__ out, int ldo, const int* __restrict__ stop) {
  constexpr int NDS = HD / 32;               // 32-dim slices of a row
  constexpr int NT = 4 * NDS;                // tiles (16 keys x 32 dims, 1 KB) per chunk, of K and of V each
  constexpr int NDB = HD / 16;               // 16-dim blocks of the output
  constexpr int NPG = GA_CHUNK / PS;         // pages per chunk
  static_assert(HD % 32 == 0 && NT % NW == 0, "tile split over the waves");
  // tile t = kb * NDS + ds holds keys 16 kb .. + 15, dims 32 ds .. + 31; row R (key 16 kb + R) is 64 bytes of
  // four 16-byte chunks; K tiles keep the chunks in order, V tiles put dim chunk C at position
  // C ^ (R / 4) (two-way bank conflicts for the transposed reads)
  __shared__ alignas(16) bf16_t Ks[2][NT * 512];
  __shared__ alignas(16) bf16_t Vs[2][NT * 512];

  if (stop && *stop) return;
  const int g = blockIdx.x;
  const int G = H / KVH;
  const int Ma = nrows ? min(M, *nrows) : M;
  const int r0 = blockIdx.y * RB;
  const int r1 = min(r0 + RB, Ma);
  if (r0 >= r1) return;
  const int nq = (r1 - r0) * G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;

  // the block's largest position (RB <= 64 rows)
  int maxpos = lane < r1 - r0 ? pos[r0 + lane] : -1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) maxpos = max(maxpos, __shfl_xor(maxpos, o, 64));
  maxpos = __builtin_amdgcn_readfirstlane(maxpos);    // wave-uniform: the chunk loop is scalar
  const int nch = maxpos / GA_CHUNK + 1;

  // this lane's query (column r of the wave's 16) and its row's position
  const int qi = 16 * wave + r;
  const bool qv = qi < nq;
  const int qc = min(qi, nq - 1);
  const int qrow = r0 + qc / G, qhead = g * G + qc % G;
  const int prow = qv ? pos[qrow] : -1;
  bf16x8 qf[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds)
    qf[ds] = *(const bf16x8*)(q + (size_t)qrow * ldq + (size_t)qhead * HD + 32 * ds + 8 * g4);

  const int grp_base = (local_kv && group_rows > 0) ? (r0 / group_rows) * group_rows : 0;
  // the wave's smallest query position (its valid queries): chunks at or below it need no causal mask
  int qmin = qv ? prow : 0x7fffffff;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) qmin = min(qmin, __shfl_xor(qmin, o, 64));
  qmin = __builtin_amdgcn_readfirstlane(qmin);
  // chunks [0, n_fast) lie below the candidates' own keys and at or below every row's position
  const int lstart = local_kv ? local_start : 0x7fffffff;
  const int n_fast = min(lstart, maxpos + 1) / GA_CHUNK;

  // page ids of chunk c: lane i < 64 / PS holds that of the chunk's i-th page (pages of 16, 32 or 64
  // positions, so the 16 keys of a tile share a page)
  auto pages = [&](int c) -> int {
    const int i = min(c * GA_CHUNK / PS + lane, n_lpages - 1);
    return lane * PS < GA_CHUNK ? page_table[i] : 0;
  };
  const size_t page_stride = (size_t)L * 2 * KVH * PS * HD;
  const bf16_t* pool_k = pool + (((size_t)layer * 2 + 0) * KVH + g) * PS * HD;
  const size_t vdelta = (size_t)KVH * PS * HD;         // value rows follow the key rows of a page's layer
  const size_t lrow = (size_t)2 * KVH * HD;             // local buffer: [row][K, V][KVH][HD]

  // Tile loads: lane -> row R = lane / 4 (key 16 kb + R), position lane % 4 (16 bytes, written to LDS at
  // 16 * lane).  Offsets within a page (elements) are the same for every chunk.
  const int kR = lane >> 2;
  const int kdim = 8 * (lane & 3), vdim = 8 * ((lane & 3) ^ ((lane >> 4) & 3));
  uint32_t toff[NT / NW];
#pragma unroll
  for (int j = 0; j < NT / NW; ++j) {
    const int kb = (wave + NW * j) / NDS;
    toff[j] = (uint32_t)(((16 * kb + kR) & (PS - 1)) * HD);
  }
  auto issue = [&](int c, int pgc, int b) {
    const bf16_t* pk[NPG];                              // the chunk's pages: key rows of (layer, head g)
#pragma unroll
    for (int i = 0; i < NPG; ++i) pk[i] = pool_k + (size_t)__builtin_amdgcn_readlane(pgc, i) * page_stride;
    if (c < n_fast) {
      // every key of the chunk is a prefix key of the paged cache
#pragma unroll
      for (int j = 0; j < NT / NW; ++j) {
        const int t = wave + NW * j, kb = t / NDS, ds = t % NDS;
        const bf16_t* row = pk[16 * kb / PS] + toff[j] + 32 * ds;
        __builtin_amdgcn_global_load_lds((ga_gbl_t*)(row + kdim), (ga_lds_t*)(&Ks[b][t * 512]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((ga_gbl_t*)(row + vdelta + vdim), (ga_lds_t*)(&Vs[b][t * 512]), 16, 0, 0);
      }
    } else {
      // prefix keys, the candidate's own keys (positions >= local_start: row grp_base + kp - local_start of
      // the local buffer), and positions past maxpos, which read the row of maxpos: their scores are masked
      // and their probabilities are zero
#pragma unroll
      for (int j = 0; j < NT / NW; ++j) {
        const int t = wave + NW * j, kb = t / NDS, ds = t % NDS;
        const int kp = min(c * GA_CHUNK + 16 * kb + kR, maxpos);
        const int page = __shfl(pgc, (kp - c * GA_CHUNK) / PS, 64);
        const bf16_t* pr = pool_k + (size_t)page * page_stride + (size_t)(kp & (PS - 1)) * HD;
        const bf16_t* lr = local_kv + (size_t)(grp_base + kp - local_start) * lrow + (size_t)g * HD;
        const bf16_t* kr = (kp >= lstart ? lr : pr) + 32 * ds;
        const size_t vd = kp >= lstart ? (size_t)KVH * HD : vdelta;
        __builtin_amdgcn_global_load_lds((ga_gbl_t*)(kr + kdim), (ga_lds_t*)(&Ks[b][t * 512]), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((ga_gbl_t*)(kr + vd + vdim), (ga_lds_t*)(&Vs[b][t * 512]), 16, 0, 0);
      }
    }
  };

  // transposed reads of V for the P V operand: lane (r, g4) of output block d takes dim 16 d + r of keys
  // 32 kk + 4 g4 + 0..3 (tile 2 kk) and 32 kk + 16 + 4 g4 + 0..3 (tile 2 kk + 1); as a source it reads 8 bytes
  // of row 4 g4 + r / 4, dims 16 (d % 2) + 4 (r % 4), chunk C = 2 (d % 2) + (r % 4) / 2 at position C ^ g4
  uint32_t voff2[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    voff2[h] = (uint32_t)((4 * g4 + (r >> 2)) * 32 + ((2 * h + ((r & 3) >> 1)) ^ g4) * 8 + 4 * (r & 1));

  // softmax in base 2: scores scaled by log2(e) / sqrt(HD)
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  f32x4 o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  int pg_next = pages(0);
  issue(0, pg_next, 0);
  if (nch > 1) pg_next = pages(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int b = c & 1;
    if (c + 1 < nch) {
      issue(c + 1, pg_next, b ^ 1);
      if (c + 2 < nch) pg_next = pages(c + 2);
    }
    // ---- S[key][query] for the chunk's 64 keys (kb: 16-key blocks); lane holds keys 16 kb + 4 g4 + e
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 ak = *(const bf16x8*)(&Ks[b][(kb * NDS + ds) * 512 + r * 32 + g4 * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qf[ds], s[kb], 0, 0, 0);
      }
    }
    // ---- online softmax of query r over the chunk (causal: key position <= the row's)
    float mloc = -INFINITY;
    if (c * GA_CHUNK + GA_CHUNK - 1 <= qmin) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[kb][e] *= sl2;
          mloc = fmaxf(mloc, s[kb][e]);
        }
    } else {
      const int lim = prow - (c * GA_CHUNK + 4 * g4);   // keys 16 kb + e <= lim are visible
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[kb][e] = 16 * kb + e <= lim ? s[kb][e] * sl2 : -INFINITY;
          mloc = fmaxf(mloc, s[kb][e]);
        }
    }
    mloc = ga_row4_max(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float lsum = 0.f;
    uint32_t ph[4][2], pl[4][2];                        // probability pairs as bf16: hi (truncated) and lo parts
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(s[kb][e] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(s[kb][e + 1] - m_use);
        lsum += p0;
        lsum += p1;
        const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
        ph[kb][e / 2] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
        const float q0 = p0 - __uint_as_float(u0 & 0xFFFF0000u), q1 = p1 - __uint_as_float(u1 & 0xFFFF0000u);
        pl[kb][e / 2] = __builtin_amdgcn_perm(__float_as_uint(q1), __float_as_uint(q0), 0x07060302u);
      }
    lsum = ga_row4_sum(lsum);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] *= alpha;
    // ---- O[dim][query] += V^T P^T: k slots 8 g4 + t hold keys 32 kk + 4 g4 + t (t < 4) and
    // 32 kk + 16 + 4 g4 + (t - 4), the keys this lane's probabilities belong to
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const ga_u32x4 bh = {ph[2 * kk][0], ph[2 * kk][1], ph[2 * kk + 1][0], ph[2 * kk + 1][1]};
      const ga_u32x4 bl = {pl[2 * kk][0], pl[2 * kk][1], pl[2 * kk + 1][0], pl[2 * kk + 1][1]};
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const bf16_t* t0 = &Vs[b][((2 * kk) * NDS + d / 2) * 512 + voff2[d & 1]];
        const ga_s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ga_lds_s16x4*)t0);
        const ga_s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ga_lds_s16x4*)(t0 + NDS * 512));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bh), o[d], 0, 0, 0);
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bl), o[d], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- output: lane (r, g4) holds dims 16 d + 4 g4 + e of query r
  if (qv) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    bf16_t* dst = out + (size_t)qrow * ldo + (size_t)qhead * HD + 4 * g4;
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const uint32_t lo = (uint32_t)f2bf(o[d][0] * inv) | ((uint32_t)f2bf(o[d][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f2bf(o[d][2] * inv) | ((uint32_t)f2bf(o[d][3] * inv) << 16);
      *(ga_u32x2*)(dst + 16 * d) = ga_u32x2{lo, hi};
    }
  }
}

}  // namespace

int launch_attention_groups(int head_dim, const void* q, int ldq, const KvView& kv, int L, int layer, int H, int KVH,
                            const RowBlock& rb, const void* local_kv, int local_start, int group_rows, void* out,
                            int ldo, hipStream_t s) {
  if (rb.M <= 0) return 0;
  const int G = H / KVH;
  if (G < 1 || G > 64 || group_rows <= 0 || (head_dim != 64 && head_dim != 128)) return SSD_ERR_SHAPE;
  if (kv.page_size != 16 && kv.page_size != 32 && kv.page_size != 64) return SSD_ERR_SHAPE;
  int RB = 1;                                          // rows per block: a divisor of the group, <= 64 queries
  for (int d = 1; d <= group_rows; ++d)
    if (group_rows % d == 0 && d * G <= 64) RB = d;
  const int nqb = RB * G;
  const dim3 grid(KVH, (rb.M + RB - 1) / RB);
#define GA_LAUNCH(HDV, NWV, PSV)                                                                               \
  hipLaunchKernelGGL((attn_group_kernel<HDV, NWV, PSV>), grid, dim3(NWV * 64), 0, s, (const bf16_t*)q, ldq,     \
                     (const bf16_t*)kv.pool, kv.page_table, kv.n_lpages, L, layer, H, KVH, rb.M, rb.nrows, rb.pos, \
                     RB, (const bf16_t*)local_kv, local_start, group_rows, (bf16_t*)out, ldo, rb.stop)
#define GA_PS(HDV, NWV)                                                                                         \
  do {                                                                                                          \
    if (kv.page_size == 16) GA_LAUNCH(HDV, NWV, 16);                                                            \
    else if (kv.page_size == 32) GA_LAUNCH(HDV, NWV, 32);                                                       \
    else GA_LAUNCH(HDV, NWV, 64);                                                                               \
  } while (0)
  if (head_dim == 128) {
    if (nqb <= 16) GA_PS(128, 1); else if (nqb <= 32) GA_PS(128, 2); else GA_PS(128, 4);
  } else {
    if (nqb <= 16) GA_PS(64, 1); else if (nqb <= 32) GA_PS(64, 2); else GA_PS(64, 4);
  }
#undef GA_PS
#undef GA_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : SSD_ERR_HIP;
}

}  // namespace ssd
