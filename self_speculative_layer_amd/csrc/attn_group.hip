// Attention of the mask-scoring pass (SWIFT's matchness scoring of candidate
// layer sets): every candidate's window rows attend to the shared prompt
// prefix in the paged cache and to the candidate's own window keys and values
// (the local buffer).  One workgroup takes one KV head and a block of rows of
// one candidate (all query heads of the group), and walks the keys in 64-key
// chunks in position order with a running (online) softmax, so no partial
// records and no merge launch are needed:
//   S = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16, K as A: 16 keys
//   x 32 dims, the queries as B), the chunk's maxima and probabilities in
//   fp32 registers, and O += P V on the matrix cores too, with V transposed
//   into LDS while it is staged and each probability split into two bf16
//   parts (hi + lo), so the products keep ~16 bits of the probability.
// Each wave owns 16 queries and all 64 keys of a chunk, so the softmax needs
// no exchange between waves; keys are staged double-buffered (K straight into
// LDS by global_load_lds, V through registers).
// Arithmetic differs from the split-item attention of the decode and prefill
// paths (order of the key sums, online rescaling); the scoring pass compares
// candidates with one another, never with those paths' bits.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"

namespace ssd {

namespace {

constexpr int GA_CHUNK = 64;       // keys per chunk
constexpr int GA_VTS = 72;         // row stride (elements) of the transposed V tile: conflict-light writes and reads

typedef uint32_t ga_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t ga_u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void ga_lds_t;
typedef __attribute__((address_space(1))) const void ga_gbl_t;

// Value of the lane's pair partner (lane ^ 1).
__device__ __forceinline__ uint32_t ga_swap_pair(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);   // quad_perm [1, 0, 3, 2]
}

template <int HD, int NW, int PS>
__global__ __launch_bounds__(NW * 64) void attn_group_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ pool, const int* __restrict__ page_table,
    int n_lpages, int L, int layer, int H, int KVH, int M, const int* __restrict__ nrows,
    const int* __restrict__ pos, int RB, const bf16_t* __restrict__ local_kv, int local_start, int group_rows,
    bf16_t* __restrict__ out, int ldo, const int* __restrict__ stop) {
  constexpr int NDS = HD / 32;               // 32-dim slices of a key row
  constexpr int NKT = 4 * NDS;               // K tiles (16 keys x 32 dims, 1 KB) per chunk
  constexpr int NDB = HD / 16;               // 16-dim blocks of the output
  constexpr int DG = HD / 8;                 // 16-byte groups of a row
  constexpr int KPI = 64 / DG;               // keys per V load instruction of a wave
  constexpr int NVI = GA_CHUNK / KPI;        // V load instructions per chunk
  static_assert(HD % 32 == 0 && NKT % NW == 0 && NVI % NW == 0, "tile split over the waves");
  __shared__ alignas(16) bf16_t Ks[2][NKT * 512];
  __shared__ alignas(16) bf16_t Vt[2][HD * GA_VTS];

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
  // positions, so the 4 to 16 aligned keys of one load instruction share a page)
  auto pages = [&](int c) -> int {
    const int i = min(c * GA_CHUNK / PS + lane, n_lpages - 1);
    return lane * PS < GA_CHUNK ? page_table[i] : 0;
  };
  const size_t page_stride = (size_t)L * 2 * KVH * PS * HD;
  const bf16_t* pool_k = pool + (((size_t)layer * 2 + 0) * KVH + g) * PS * HD;
  const size_t vdelta = (size_t)KVH * PS * HD;         // value rows follow the key rows of a page's layer

  // Loads.  K tile t = kb * NDS + ds (16 keys x 32 dims): lane -> key 16 kb + lane / 4, dims 32 ds + 8 (lane % 4),
  // written to LDS at 16 * lane, so a fragment read is one contiguous 1 KB.  V: lane = key parity | 16-byte
  // group << 1 | key pair << (1 + log2 DG), 16 bytes each.  Offsets within a page (elements) are the same
  // for every chunk.
  const int par = lane & 1, dg = (lane >> 1) % DG, kq = (lane >> 1) / DG;
  uint32_t koff[NKT / NW], voff[NVI / NW];
#pragma unroll
  for (int j = 0; j < NKT / NW; ++j) {
    const int t = wave + NW * j, kb = t / NDS, ds = t % NDS;
    koff[j] = (uint32_t)(((16 * kb + (lane >> 2)) & (PS - 1)) * HD + 32 * ds + 8 * (lane & 3));
  }
#pragma unroll
  for (int i = 0; i < NVI / NW; ++i) {
    const int ii = wave + NW * i;
    voff[i] = (uint32_t)(((KPI * ii + 2 * kq + par) & (PS - 1)) * HD + 8 * dg);
  }
  ga_u32x4 vreg[NVI / NW];
  constexpr int NPG = GA_CHUNK / PS;                    // pages per chunk
  auto issue = [&](int c, int pgc, int b) {
    const bf16_t* pk[NPG];                              // the chunk's pages: key rows of (layer, head g)
#pragma unroll
    for (int i = 0; i < NPG; ++i) pk[i] = pool_k + (size_t)__builtin_amdgcn_readlane(pgc, i) * page_stride;
    if (c < n_fast) {
      // every key of the chunk is a prefix key of the paged cache
#pragma unroll
      for (int j = 0; j < NKT / NW; ++j) {
        const int t = wave + NW * j, kb = t / NDS;
        __builtin_amdgcn_global_load_lds((ga_gbl_t*)(pk[16 * kb / PS] + koff[j]), (ga_lds_t*)(&Ks[b][t * 512]), 16,
                                         0, 0);
      }
#pragma unroll
      for (int i = 0; i < NVI / NW; ++i) {
        const int ii = wave + NW * i;
        vreg[i] = *(const ga_u32x4*)(pk[KPI * ii / PS] + vdelta + voff[i]);
      }
    } else {
      // prefix keys, the candidate's own keys (positions >= local_start: row grp_base + kp - local_start of
      // the local buffer), and positions past maxpos (the group's last local row, or some row of a valid
      // page): their scores are masked and their values zeroed
      const size_t lrow = (size_t)2 * KVH * HD;
#pragma unroll
      for (int j = 0; j < NKT / NW; ++j) {
        const int t = wave + NW * j, kb = t / NDS, ds = t % NDS;
        const int kp = c * GA_CHUNK + 16 * kb + (lane >> 2);
        const bf16_t* pr = pk[16 * kb / PS] + koff[j];
        const bf16_t* lr = local_kv + (size_t)(grp_base + min(kp, maxpos) - local_start) * lrow + (size_t)g * HD +
                           32 * ds + 8 * (lane & 3);
        __builtin_amdgcn_global_load_lds((ga_gbl_t*)(kp >= lstart ? lr : pr), (ga_lds_t*)(&Ks[b][t * 512]), 16, 0,
                                         0);
      }
#pragma unroll
      for (int i = 0; i < NVI / NW; ++i) {
        const int ii = wave + NW * i;
        const int kp = c * GA_CHUNK + KPI * ii + 2 * kq + par;
        const bf16_t* pr = pk[KPI * ii / PS] + vdelta + voff[i];
        const bf16_t* lr = local_kv + (size_t)(grp_base + min(kp, maxpos) - local_start) * lrow + (size_t)KVH * HD +
                           (size_t)g * HD + 8 * dg;
        vreg[i] = *(const ga_u32x4*)(kp >= lstart ? lr : pr);
        if (kp > maxpos) vreg[i] = ga_u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // V rows of a chunk into Vt[b] as [dim][key]: the two lanes of a key pair swap halves, so each writes
  // 4 dims x 2 keys as four 32-bit words, in a lane-rotated row order (fewer bank conflicts)
  const int rot = (dg >> 1) & 3;
  uint32_t vtaddr[4];                                   // byte offsets in a Vt buffer of the lane's four rows
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) vtaddr[jj] = (uint32_t)(((8 * dg + 4 * par + ((jj + rot) & 3)) * GA_VTS + 2 * kq) * 2);
  auto put_v = [&](int b) {
    char* vt = (char*)Vt[b];
#pragma unroll
    for (int i = 0; i < NVI / NW; ++i) {
      const int ii = wave + NW * i;
      const ga_u32x4 u = vreg[i];
      const uint32_t s0 = par ? u[0] : u[2], s1 = par ? u[1] : u[3];
      const uint32_t x0 = ga_swap_pair(s0), x1 = ga_swap_pair(s1);
      const uint32_t e0 = par ? x0 : u[0], e1 = par ? x1 : u[1];   // even key of the pair
      const uint32_t o0 = par ? u[2] : x0, o1 = par ? u[3] : x1;   // odd key
      uint32_t w[4];
      w[0] = __builtin_amdgcn_perm(o0, e0, 0x05040100u);          // dims 4 par + 0 .. 3: (even, odd) key
      w[1] = __builtin_amdgcn_perm(o0, e0, 0x07060302u);
      w[2] = __builtin_amdgcn_perm(o1, e1, 0x05040100u);
      w[3] = __builtin_amdgcn_perm(o1, e1, 0x07060302u);
      uint32_t y[4], z[4];                                // z[jj] = w[(jj + rot) & 3]
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) y[jj] = (rot & 1) ? w[(jj + 1) & 3] : w[jj];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) z[jj] = (rot & 2) ? y[(jj + 2) & 3] : y[jj];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) *(uint32_t*)(vt + vtaddr[jj] + 2 * KPI * ii) = z[jj];
    }
  };

  // softmax in base 2: scores scaled by log2(e) / sqrt(HD)
  const float sl2 = 1.4426950408889634f / sqrtf((float)HD);
  f32x4 o[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  int pg_next = pages(0);
  issue(0, pg_next, 0);
  if (nch > 1) pg_next = pages(1);
  put_v(0);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
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
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
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
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < NDB; ++d) o[d] *= alpha;
    // ---- O[dim][query] += V^T P^T: k slots 8 g4 + t hold keys 32 kk + 4 g4 + t (t < 4) and
    // 32 kk + 16 + 4 g4 + (t - 4), the keys this lane's probabilities belong to
    const bf16_t* vt = Vt[b];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const ga_u32x4 bh = {ph[2 * kk][0], ph[2 * kk][1], ph[2 * kk + 1][0], ph[2 * kk + 1][1]};
      const ga_u32x4 bl = {pl[2 * kk][0], pl[2 * kk][1], pl[2 * kk + 1][0], pl[2 * kk + 1][1]};
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const bf16_t* row = vt + (16 * d + r) * GA_VTS + 32 * kk + 4 * g4;
        const ga_u32x2 a0 = *(const ga_u32x2*)row, a1 = *(const ga_u32x2*)(row + 16);
        const ga_u32x4 av = {a0[0], a0[1], a1[0], a1[1]};
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bh),
                                                      o[d], 0, 0, 0);
      }
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const bf16_t* row = vt + (16 * d + r) * GA_VTS + 32 * kk + 4 * g4;
        const ga_u32x2 a0 = *(const ga_u32x2*)row, a1 = *(const ga_u32x2*)(row + 16);
        const ga_u32x4 av = {a0[0], a0[1], a1[0], a1[1]};
        o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bl),
                                                      o[d], 0, 0, 0);
      }
    }
    if (c + 1 < nch) put_v(b ^ 1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
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
