// Attention over the paged KV cache (device functions shared by the
// standalone attention kernels and the decode-mode attention kernel).
//
// Keys are split at fixed absolute positions: split s covers [64 s, 64 s + 64).
// A work item handles one KV head g, one split and a block of rows with all
// their query heads (grouped-query attention); it stages the split's 64 keys
// and values in LDS (16-byte vector loads, all in flight) in the storage type
// and writes, per query, a partial (o[HD], m, l) of the softmax restricted to
// the split.  The merge combines a row's partials in split order.  Split
// boundaries are fixed positions and every reduction runs in a fixed order,
// so a row's result does not depend on the rows batched with it.
//
// bf16 items form the scores on the matrix cores (v_mfma_f32_16x16x32_bf16:
// 16 keys x 32 dims of K as A, 32 dims x 16 queries as B), the softmax in
// fp32 registers, and P.V as fp32 FMAs over keys in order.  fp32 items use
// FMAs throughout.
#pragma once
#include "common.h"

namespace ssd {

constexpr int ATT_SPLIT = 64;
constexpr int ATT_CHUNK = 64;
constexpr int ATT_MAXQ = 64;     // queries (rows x heads of a group) per fp32 work item
constexpr int ATTB_MAXQ = 16;    // queries per bf16 work item (one matrix-core query tile)
constexpr int ATT_MAXW = 64;     // splits a block merge can hold (contexts up to 4096 positions)

// A split's partial for one query: o[HD], then m and l, then two unused floats, so that every record
// (and its (m, l) pair) starts 16-byte aligned.
__host__ __device__ constexpr int att_rec(int hd) { return hd + 4; }

// Queries (rows x heads of a KV group) one work item takes for storage type T.
template <typename T>
constexpr int att_maxq() { return sizeof(T) == 2 ? ATTB_MAXQ : ATT_MAXQ; }

__device__ __forceinline__ size_t kv_index(int page, int L, int layer, int kv, int KVH, int g, int PS, int slot,
                                           int HD) {
  return (((((size_t)page * L + layer) * 2 + kv) * KVH + g) * PS + slot) * (size_t)HD;
}

template <typename T, int HD, int NW>
struct AttnSmem {
  static constexpr int EPW = 4 / (int)sizeof(T);   // elements per 32-bit word
  static constexpr int KST = HD + EPW;              // padded row stride: lanes on different keys hit different banks
  T Ks[ATT_CHUNK * KST];
  T Vs[ATT_CHUNK * KST];
  alignas(16) T Qs[ATT_MAXQ * HD];
  float Pw[NW][ATT_CHUNK];
  int Rpos[ATT_MAXQ];
};

// bf16 items: K rows give way to the partial outputs of waves 1..3 once the
// scores are formed, and to the merge weights in a block merge.
template <int HD, int NW>
struct AttnSmem<bf16_t, HD, NW> {
  static constexpr int KST = HD + 8;                // 16-byte aligned rows
  union alignas(16) {
    bf16_t Ks[ATT_CHUNK * KST];
    float Op[NW][ATTB_MAXQ][HD];                    // each wave's P.V sums of the quads it hands over
    float Wm[2 * ATTB_MAXQ * ATT_MAXW];             // merge: [query][split] weights, then l values
  };
  alignas(16) bf16_t Vs[ATT_CHUNK * KST];
  alignas(16) bf16_t Qs[ATTB_MAXQ * KST];
  alignas(16) float P[ATT_CHUNK * ATTB_MAXQ];       // probabilities [key][query]
  float Mw[NW][ATTB_MAXQ], Sw[NW][ATTB_MAXQ];       // per-wave maximum and sum of each query
  int Rpos[ATTB_MAXQ];
  float Mx[ATTB_MAXQ], Ls[ATTB_MAXQ];
};

// bf16 items of QT > 1 query tiles (prefill, mask scoring): the keys stay in LDS for every tile, so the
// hand-over buffer of the P.V sums has its own storage.
template <int HD, int QT>
struct AttnSmemQ {
  static constexpr int KST = HD + 8;
  alignas(16) bf16_t Ks[ATT_CHUNK * KST];
  alignas(16) bf16_t Vs[ATT_CHUNK * KST];
  alignas(16) bf16_t Qs[QT * ATTB_MAXQ * KST];
  alignas(16) float P[ATT_CHUNK * ATTB_MAXQ];
  float Op[4][ATTB_MAXQ][HD];
  float Mw[4][ATTB_MAXQ], Sw[4][ATTB_MAXQ];
  int Rpos[QT * ATTB_MAXQ];
  float Mx[ATTB_MAXQ];
};

typedef uint32_t att_u32x4 __attribute__((ext_vector_type(4)));

// Partial results are stored either plainly (read by a later kernel) or with
// device-scope stores (read by another workgroup of the same kernel).
template <bool DEV>
__device__ __forceinline__ void part_store(float* p, float v) {
  if constexpr (DEV) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
// Two adjacent floats (p 8-byte aligned) in one store.
template <bool DEV>
__device__ __forceinline__ void part_store2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  if constexpr (DEV) __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *(uint64_t*)p = v;
}

// Scores, softmax partials, P.V and the partial stores of one tile of at most 16 queries: queries
// qbase .. qbase + 15 of the item's nq (rows x heads of the group), on the split's keys and values
// staged in sm.Ks / sm.Vs and the tile's queries at Qs.  Opw ([NW][16][HD] floats) takes the waves'
// P.V sums handed over; it may alias sm.Ks when no later tile needs the keys (the scores are formed
// before the barrier that precedes its first write).  Ends with a workgroup barrier.
// NQA: quad groups of P.V per lane (the tile's first 4 * (64 / (HD / 2)) * NQA queries); fewer than all
// when the tile holds only that many queries (one-row blocks); the queries it covers get the same
// arithmetic either way.
template <int HD, int NW, bool DEV, typename SM, int NQA = ATTB_MAXQ / 4 / (64 / (HD / 2))>
__device__ __forceinline__ void attn_tile_bf16(SM& sm, const bf16_t* __restrict__ Qs,
                                               float (*Opw)[ATTB_MAXQ][HD], int qbase, int nq, int G, int r0,
                                               int g, int H, int s, int nsplit, int key_beg, int key_end,
                                               float* __restrict__ part) {
  constexpr int KST = SM::KST;
  const float scale = 1.0f / sqrtf((float)HD);
  const int tid = threadIdx.x, lane = tid & 63;
  (void)tid;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- scores: wave w forms S[key][query] for its 16 keys [16 w, 16 w + 16) and the (at most 16)
  // queries; acc[i] = S[key 16 w + 4 (lane >> 4) + i][query lane & 15]
  const int ql = lane & 15, g4 = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < HD / 32; ++ds) {
    const bf16x8 bq = *(const bf16x8*)(Qs + ql * KST + 32 * ds + 8 * g4);
    const bf16x8 ak = *(const bf16x8*)(sm.Ks + (16 * wave + ql) * KST + 32 * ds + 8 * g4);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bq, acc, 0, 0, 0);
  }
  // ---- softmax of each query over the split's keys it sees (causal: key position <= its row's):
  // the maximum over the four waves' keys, then each wave's probabilities and their sum
  const bool qv = qbase + ql < nq;
  const int prow = qv ? sm.Rpos[(qbase + ql) / G] : -1;
  float sc[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kp = key_beg + 16 * wave + 4 * g4 + i;
    const bool valid = kp < key_end && kp <= prow;
    sc[i] = valid ? fmul_nc(acc[i], scale) : -INFINITY;
    mx = fmaxf(mx, sc[i]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (g4 == 0) sm.Mw[wave][ql] = mx;
  __syncthreads();                                    // also: every wave is done reading K
  mx = fmaxf(fmaxf(sm.Mw[0][ql], sm.Mw[1][ql]), fmaxf(sm.Mw[2][ql], sm.Mw[3][ql]));
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pe = sc[i] == -INFINITY ? 0.f : expf(fsub_nc(sc[i], mx));
    sm.P[(16 * wave + 4 * g4 + i) * ATTB_MAXQ + ql] = pe;
    ps += pe;
  }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  if (g4 == 0) sm.Sw[wave][ql] = ps;
  if (wave == 0 && g4 == 0) sm.Mx[ql] = mx;
  __syncthreads();

  // ---- o[query][d]: wave w sums p * v over its 16 keys in order (fp32), lane: dims 2 dp, 2 dp + 1 of
  // the query quads qh, qh + QS, ...; waves 1..3 hand their sums to wave 0, which adds them in wave order
  constexpr int DP = HD / 2;                          // dim pairs
  constexpr int QS = 64 / DP;                         // quad groups per wave (1 at hd 128, 2 at hd 64)
  constexpr int NQ4 = NQA;                            // quads per lane (all: ATTB_MAXQ / 4 / QS)
  static_assert(NQA >= 1 && NQA <= ATTB_MAXQ / 4 / QS, "quad groups");
  const int dp = lane % DP, qh = lane / DP;
  float o[NQ4][4][2];
#pragma unroll
  for (int a = 0; a < NQ4; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[a][j][0] = o[a][j][1] = 0.f;
#pragma unroll 4
  for (int kk = 0; kk < 16; ++kk) {
    const int k = 16 * wave + kk;
    const uint32_t v2 = *(const uint32_t*)(sm.Vs + k * KST + 2 * dp);
    const float vlo = __uint_as_float(v2 << 16), vhi = __uint_as_float(v2 & 0xFFFF0000u);
#pragma unroll
    for (int a = 0; a < NQ4; ++a) {
      const f32x4 p4 = *(const f32x4*)(sm.P + k * ATTB_MAXQ + 4 * (qh + QS * a));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[a][j][0] = fmaf(p4[j], vlo, o[a][j][0]);
        o[a][j][1] = fmaf(p4[j], vhi, o[a][j][1]);
      }
    }
  }
  // each wave finalises the query quads q4 with q4 % NW == wave (sum in wave order), so every wave hands
  // the other quads' sums over through LDS
#pragma unroll
  for (int a = 0; a < NQ4; ++a) {
    const int q4 = qh + QS * a;
    if ((q4 % NW) == wave) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Opw[wave][4 * q4 + j][2 * dp] = o[a][j][0];
      Opw[wave][4 * q4 + j][2 * dp + 1] = o[a][j][1];
    }
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < NQ4; ++a) {
    const int q4 = qh + QS * a;
    if ((q4 % NW) != wave) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qq = 4 * q4 + j, qi = qbase + qq;    // query in the tile, in the item
      if (qi >= nq) continue;
      if (key_beg > sm.Rpos[qi / G]) continue;        // the row sees no key of this split
      float olo = 0.f, ohi = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        olo += w == wave ? o[a][j][0] : Opw[w][qq][2 * dp];
        ohi += w == wave ? o[a][j][1] : Opw[w][qq][2 * dp + 1];
      }
      const int row = r0 + qi / G, head = g * G + qi % G;
      float* dstp = part + (((size_t)row * H + head) * nsplit + s) * att_rec(HD);
      part_store2<DEV>(dstp + 2 * dp, olo, ohi);
      if (dp == 0) {
        const float l = ((sm.Sw[0][qq] + sm.Sw[1][qq]) + sm.Sw[2][qq]) + sm.Sw[3][qq];
        part_store2<DEV>(dstp + HD, sm.Mx[qq], l);
      }
    }
  }
  __syncthreads();
}

// bf16 work item (same contract as attn_partial_item below): QT tiles of at most 16 queries each, on
// the split's keys and values staged once.
// Returns the largest position the block's rows see (-1: the item had nothing to do) and sets *r1_out
// (nullable) to the block's end row.  stop (nullable): a flag read with the first loads; set, the item
// does nothing.
template <int HD, int NW, bool DEV, int QT = 1, typename SM = AttnSmem<bf16_t, HD, NW>, bool LEAF = false>
__device__ int attn_item_bf16(SM& sm, const bf16_t* __restrict__ q, int ldq,
                              const bf16_t* __restrict__ pool, const int* __restrict__ page_table, int PS,
                              int n_lpages, int L, int layer, int H, int KVH, int M, const int* __restrict__ nrows,
                              const int* __restrict__ pos, int r0, int RB, int g, int s, int nsplit,
                              const bf16_t* __restrict__ local_kv, int local_start, int group_rows,
                              float* __restrict__ part, int side0 = 0x7fffffff, const int* __restrict__ stop = nullptr,
                              int* r1_out = nullptr) {
  static_assert(NW == 4, "four waves: 16 keys each");
  constexpr int NT = NW * 64;
  constexpr int KST = SM::KST;
  constexpr int VEC = 8;                              // bf16 per 16-byte load
  constexpr int VPR = HD / VEC;
  constexpr int NLD = ATT_CHUNK * VPR / NT;
  static_assert(NLD >= 1 && ATT_CHUNK * VPR % NT == 0 && HD % 32 == 0, "staging layout");
  const int G = H / KVH;
  const int key_beg = s * ATT_SPLIT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rmax = min(r0 + RB, M);

  // ---- round 1: the stop flag, active rows, positions, the split's page ids, the queries
  const int stopv = stop ? *stop : 0;
  const int na = nrows ? *nrows : M;
  int rp = 0;
  // rows >= side0 (tree leaves) see the cache up to the position before their own; their own key is
  // merged afterwards
  if (tid < rmax - r0) rp = pos[r0 + tid] - (LEAF && r0 + tid >= side0 ? 1 : 0);
  const int pg0 = key_beg / PS;
  const int pg = (lane * PS < ATT_CHUNK && pg0 + lane < n_lpages) ? page_table[pg0 + lane] : 0;
  constexpr int QPER = (QT * ATTB_MAXQ * VPR + NT - 1) / NT;
  const int nq_max = (rmax - r0) * G;
  att_u32x4 qreg[QPER];
#pragma unroll
  for (int j = 0; j < QPER; ++j) {
    const int e = min(tid + NT * j, nq_max * VPR - 1);
    const int qi = e / VPR, vc = e % VPR;
    const int row = r0 + qi / G, head = g * G + qi % G;
    qreg[j] = *(const att_u32x4*)(q + (size_t)row * ldq + (size_t)head * HD + vc * VEC);
  }
  if (tid < rmax - r0) sm.Rpos[tid] = rp;
  __syncthreads();
  const int Ma = min(M, na);
  const int r1 = min(r0 + RB, Ma);
  if (stopv || r1 <= r0) return -1;
  int maxpos = sm.Rpos[r1 - 1 - r0];                  // positions increase along the rows, except leaf rows
  if (LEAF && side0 < r1)
    for (int i = 0; i < r1 - r0; ++i) maxpos = max(maxpos, sm.Rpos[i]);
  if (key_beg > maxpos) return -1;
  if (r1_out) *r1_out = r1;
  const int nq = (r1 - r0) * G;
  const int key_end = min(key_beg + ATT_SPLIT, maxpos + 1);
  const int grp_base = group_rows > 0 ? (r0 / group_rows) * group_rows : 0;

  // ---- round 2: the split's keys and values (clamped addresses, zero past the end)
  att_u32x4 kreg[NLD], vreg[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int e = tid + NT * j;
    const int t = e / VPR, vc = e % VPR;
    const int kp = key_beg + t;
    const int kq = min(kp, key_end - 1);
    const int page = __shfl(pg, (kq - key_beg) / PS, 64);
    const bool local = local_kv && kq >= local_start;
    const size_t lbase = ((size_t)(grp_base + (kq - local_start)) * 2) * KVH * HD + (size_t)g * HD;
    const bf16_t* kr = local ? local_kv + lbase : pool + kv_index(page, L, layer, 0, KVH, g, PS, kq % PS, HD);
    const bf16_t* vr = local ? local_kv + lbase + (size_t)KVH * HD
                            : pool + kv_index(page, L, layer, 1, KVH, g, PS, kq % PS, HD);
    kreg[j] = *(const att_u32x4*)(kr + vc * VEC);
    vreg[j] = *(const att_u32x4*)(vr + vc * VEC);
    if (kp >= key_end) {
      kreg[j] = att_u32x4{0u, 0u, 0u, 0u};
      vreg[j] = att_u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int j = 0; j < QPER; ++j) {
    const int e = tid + NT * j;
    if (e < nq * VPR) *(att_u32x4*)(sm.Qs + (e / VPR) * KST + (e % VPR) * VEC) = qreg[j];
  }
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int e = tid + NT * j;
    const int t = e / VPR, vc = e % VPR;
    *(att_u32x4*)(sm.Ks + t * KST + vc * VEC) = kreg[j];
    *(att_u32x4*)(sm.Vs + t * KST + vc * VEC) = vreg[j];
  }
  __syncthreads();

  constexpr int QS1 = 64 / (HD / 2);                  // quads one P.V pass per lane covers
  if (nq <= 4 * QS1)
    attn_tile_bf16<HD, NW, DEV, SM, 1>(sm, sm.Qs, sm.Op, 0, nq, G, r0, g, H, s, nsplit, key_beg, key_end, part);
  else
    for (int t = 0; t * ATTB_MAXQ < nq; ++t)
      attn_tile_bf16<HD, NW, DEV>(sm, sm.Qs + t * ATTB_MAXQ * KST, sm.Op, t * ATTB_MAXQ, nq, G, r0, g, H, s, nsplit,
                                  key_beg, key_end, part);
  return maxpos;
}

// fp32 work item (FMAs throughout).
template <typename T, int HD, int NW, bool DEV>
__device__ void attn_item_scalar(AttnSmem<T, HD, NW>& sm, const T* __restrict__ q, int ldq,
                                  const T* __restrict__ pool, const int* __restrict__ page_table, int PS,
                                  int n_lpages, int L, int layer, int H, int KVH, int M,
                                  const int* __restrict__ nrows, const int* __restrict__ pos, int r0, int RB, int g,
                                  int s, int nsplit, const T* __restrict__ local_kv, int local_start, int group_rows,
                                  float* __restrict__ part) {
  constexpr int NT = NW * 64;
  constexpr int KST = AttnSmem<T, HD, NW>::KST;
  constexpr int VEC = 16 / (int)sizeof(T);            // elements per 16-byte load
  constexpr int VPR = HD / VEC;                       // 16-byte vectors per row
  constexpr int NLD = ATT_CHUNK * VPR / NT;           // vectors per thread per matrix
  static_assert(NLD >= 1 && ATT_CHUNK * VPR % NT == 0, "staging layout");
  const int G = H / KVH;
  const int key_beg = s * ATT_SPLIT;
  const float scale = 1.0f / sqrtf((float)HD);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rmax = min(r0 + RB, M);                   // rows of the block if every row is active

  // ---- round 1
  const int na = nrows ? *nrows : M;
  int rp = 0;
  if (tid < rmax - r0) rp = pos[r0 + tid];
  const int pg0 = key_beg / PS;
  const int pg = (lane * PS < ATT_CHUNK && pg0 + lane < n_lpages) ? page_table[pg0 + lane] : 0;
  constexpr int QPER = (ATT_MAXQ * VPR + NT - 1) / NT;
  const int nq_max = (rmax - r0) * G;
  att_u32x4 qreg[QPER];
#pragma unroll
  for (int j = 0; j < QPER; ++j) {
    const int e = min(tid + NT * j, nq_max * VPR - 1);      // clamped: every lane loads a valid address
    const int qi = e / VPR, vc = e % VPR;
    const int row = r0 + qi / G, head = g * G + qi % G;
    qreg[j] = *(const att_u32x4*)(q + (size_t)row * ldq + (size_t)head * HD + vc * VEC);
  }
  if (tid < rmax - r0) sm.Rpos[tid] = rp;
  __syncthreads();
  const int Ma = min(M, na);
  const int r1 = min(r0 + RB, Ma);
  if (r1 <= r0) return;                               // uniform
  const int maxpos = sm.Rpos[r1 - 1 - r0];
  if (key_beg > maxpos) return;                       // uniform: no row sees a key of this split
  const int nq = (r1 - r0) * G;
  const int key_end = min(key_beg + ATT_SPLIT, maxpos + 1);
#pragma unroll
  for (int j = 0; j < QPER; ++j) {
    const int e = tid + NT * j;
    if (e < nq * VPR) *(att_u32x4*)(sm.Qs + e * VEC) = qreg[j];
  }
  const int grp_base = group_rows > 0 ? (r0 / group_rows) * group_rows : 0;
  static_assert(ATT_SPLIT == ATT_CHUNK, "one chunk per split");
  {
    const int kc = key_beg;
    // ---- round 2: every key and value of the chunk (clamped addresses, zero past the end)
    att_u32x4 kreg[NLD], vreg[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int e = tid + NT * j;
      const int t = e / VPR, vc = e % VPR;
      const int kp = kc + t;
      const int kq = min(kp, key_end - 1);
      const int page = __shfl(pg, (kq - kc) / PS, 64);
      const bool local = local_kv && kq >= local_start;
      const size_t lbase = ((size_t)(grp_base + (kq - local_start)) * 2) * KVH * HD + (size_t)g * HD;
      const T* kr = local ? local_kv + lbase : pool + kv_index(page, L, layer, 0, KVH, g, PS, kq % PS, HD);
      const T* vr = local ? local_kv + lbase + (size_t)KVH * HD : pool + kv_index(page, L, layer, 1, KVH, g, PS, kq % PS, HD);
      kreg[j] = *(const att_u32x4*)(kr + vc * VEC);
      vreg[j] = *(const att_u32x4*)(vr + vc * VEC);
      if (kp >= key_end) {
        kreg[j] = att_u32x4{0u, 0u, 0u, 0u};
        vreg[j] = att_u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();      // the previous chunk's readers are done
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int e = tid + NT * j;
      const int t = e / VPR, vc = e % VPR;
      uint32_t* kd = (uint32_t*)(sm.Ks + t * KST + vc * VEC);
      uint32_t* vd = (uint32_t*)(sm.Vs + t * KST + vc * VEC);
#pragma unroll
      for (int w = 0; w < 4; ++w) { kd[w] = kreg[j][w]; vd[w] = vreg[j][w]; }
    }
    __syncthreads();
    // one split = one chunk: each query's partial (o, m, l) follows from an empty online-softmax
    // state (o = 0 * 0 + sum p v, m = max, l = 0 * 0 + sum p) and is written directly
    for (int qi = wave; qi < nq; qi += NW) {
      const int row = r0 + qi / G, head = g * G + qi % G;
      const int prow = sm.Rpos[row - r0];
      if (key_beg > prow) continue;             // the row sees no key of this split (wave-uniform)
      const int kp = kc + lane;
      const bool valid = kp < key_end && kp <= prow;
      float sc = -INFINITY;
      if (valid) {
        float acc = 0.f;
        const T* kr = sm.Ks + lane * KST;
        const T* qr = sm.Qs + qi * HD;
        if constexpr (sizeof(T) == 2) {
#pragma unroll 16
          for (int d = 0; d < HD; d += 2) {
            const uint32_t w2 = *(const uint32_t*)(kr + d);
            const uint32_t q2 = *(const uint32_t*)(qr + d);
            acc = fmaf(__uint_as_float(q2 << 16), __uint_as_float(w2 << 16), acc);
            acc = fmaf(__uint_as_float(q2 & 0xFFFF0000u), __uint_as_float(w2 & 0xFFFF0000u), acc);
          }
        } else {
#pragma unroll 16
          for (int d = 0; d < HD; ++d) acc = fmaf(ld(qr + d), ld(kr + d), acc);
        }
        sc = fmul_nc(acc, scale);
      }
      const float mx = wave_max(sc);
      const float pexp = valid ? expf(fsub_nc(sc, mx)) : 0.f;
      const float psum = wave_sum(pexp);
      sm.Pw[wave][lane] = pexp;
      __builtin_amdgcn_wave_barrier();
      float* dstp = part + (((size_t)row * H + head) * nsplit + s) * att_rec(HD);
      for (int d = lane; d < HD; d += 64) {
        float o = 0.f;
        // 16 keys' values are read before their 16 multiply-adds (one LDS round trip per 16 keys)
#pragma unroll 1
        for (int t0 = 0; t0 < ATT_CHUNK; t0 += 16) {
          float vv[16], pw[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            vv[u] = ld(sm.Vs + (t0 + u) * KST + d);
            pw[u] = sm.Pw[wave][t0 + u];
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) o = fmaf(pw[u], vv[u], o);
        }
        part_store<DEV>(dstp + d, o);
      }
      if (lane == 0) {
        part_store<DEV>(dstp + HD, mx);
        part_store<DEV>(dstp + HD + 1, psum);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();
}

// One work item: KV head g, split s, the rows r0 .. min(r0 + RB, Ma) - 1 with
// Ma = min(M, *nrows) (positions increasing; rows >= side0, bf16 only, are
// tree leaves: they see keys up to their position - 1).  Keys at positions >= local_start
// come from local_kv rows (scoring: the candidate's own keys/values, rows
// grouped by group_rows).  Requires all NW*64 threads of the block.
//
// Loads take two rounds: (1) the active-row count, the rows' positions, the
// chunk's page ids and the queries; (2) every key and value of the chunk.
// Items whose split starts past the block's last position return after (1).
// DEV: partials are written with device-scope stores.
template <typename T, int HD, int NW, bool DEV = false, bool LEAF = false>
__device__ void attn_partial_item(AttnSmem<T, HD, NW>& sm, const T* __restrict__ q, int ldq,
                                  const T* __restrict__ pool, const int* __restrict__ page_table, int PS,
                                  int n_lpages, int L, int layer, int H, int KVH, int M,
                                  const int* __restrict__ nrows, const int* __restrict__ pos, int r0, int RB, int g,
                                  int s, int nsplit, const T* __restrict__ local_kv, int local_start, int group_rows,
                                  float* __restrict__ part, int side0 = 0x7fffffff) {
  if constexpr (sizeof(T) == 2)
    (void)attn_item_bf16<HD, NW, DEV, 1, AttnSmem<bf16_t, HD, NW>, LEAF>(sm, q, ldq, pool, page_table, PS, n_lpages,
                                                                         L, layer, H, KVH, M, nrows, pos, r0, RB, g, s,
                                                                         nsplit, local_kv, local_start, group_rows,
                                                                         part, side0);
  else
    attn_item_scalar<T, HD, NW, DEV>(sm, q, ldq, pool, page_table, PS, n_lpages, L, layer, H, KVH, M, nrows, pos, r0,
                                     RB, g, s, nsplit, local_kv, local_start, group_rows, part);
}

// Merge the splits of (row, head) in split order; component d of the output.
template <int HD>
__device__ __forceinline__ float attn_combine_value(const float* __restrict__ part, int nsplit, int row, int head,
                                                   int H, int p, int d) {
  const int ns = p / ATT_SPLIT + 1;
  const float* pr = part + ((size_t)row * H + head) * nsplit * att_rec(HD);
  constexpr int B = 16;
  if (ns <= B) {
    // one round of loads
    float mv[B], lv[B], ov[B];
#pragma unroll
    for (int s = 0; s < B; ++s) {
      mv[s] = -INFINITY;
      lv[s] = ov[s] = 0.f;
      if (s < ns) {
        mv[s] = pr[s * att_rec(HD) + HD];
        lv[s] = pr[s * att_rec(HD) + HD + 1];
        ov[s] = pr[s * att_rec(HD) + d];
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < B; ++s) m = fmaxf(m, mv[s]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int s = 0; s < B; ++s) {
      if (s < ns) {
        const float w = expf(fsub_nc(mv[s], m));
        l = fmaf(lv[s], w, l);
        o = fmaf(ov[s], w, o);
      }
    }
    return __fdiv_rn(o, l);
  }
  float m = -INFINITY;
#pragma unroll 16
  for (int s = 0; s < ns; ++s) m = fmaxf(m, pr[s * att_rec(HD) + HD]);
  float l = 0.f, o = 0.f;
#pragma unroll 16
  for (int s = 0; s < ns; ++s) {
    const float w = expf(fsub_nc(pr[s * att_rec(HD) + HD], m));
    l = fmaf(pr[s * att_rec(HD) + HD + 1], w, l);
    o = fmaf(pr[s * att_rec(HD) + d], w, o);
  }
  return __fdiv_rn(o, l);
}

// Merge by one block of the partials of rows r0 .. r1 - 1 (all G query heads
// of KV head g), once every split has stored its partial (positions from
// sm.Rpos, at most ATT_MAXW splits).  Same arithmetic as attn_combine_value:
// per query the maximum M of its splits' m, each split's weight
// exp(m_s - M), then l and o as fma chains in split order, and o / l.
// A group of 16 lanes (inside one wave) takes one query: lane j loads the
// (m, l) of splits j, j + 16, ... and HD / 16 consecutive dimensions of o of
// every split, all in one round of loads for contexts up to 64 * MCH
// positions; the maximum is a butterfly over the group, and the weights pass
// between the group's lanes through LDS, so the merge has no workgroup
// barrier.  The output is in the decode block layout.
// Rows >= side0 (tree leaves, whose partials cover keys up to their position - 1) have their own key
// and value side_kv[(row - side0) * 2 + {0, 1}][KVH][HD] as one more split after the last: score
// (q . k) / sqrt(HD) with q the row's query (q, ldq), sum 1, output v.
template <int HD, int NW, bool LEAF = false>
__device__ __forceinline__ void attn_merge_block(AttnSmem<bf16_t, HD, NW>& sm, const float* __restrict__ part,
                                                 int nsplit, int r0, int r1, int G, int g, int H,
                                                 bf16_t* __restrict__ out, int side0 = 0x7fffffff,
                                                 const bf16_t* __restrict__ side_kv = nullptr,
                                                 const bf16_t* __restrict__ q = nullptr, int ldq = 0, int KVH = 0) {
  static_assert(NW * 64 == 16 * ATTB_MAXQ, "one 16-lane group per query");
  constexpr int REC = att_rec(HD);
  constexpr int DPT = HD / 16;                        // dimensions per lane
  constexpr int NV = DPT / 4;                         // 16-byte o loads per split
  constexpr int MCH = HD == 128 ? 12 : 16;            // splits whose o comes with the first round
  constexpr int MLR = ATT_MAXW / 16;                  // (m, l) pairs per lane
  static_assert(DPT % 4 == 0 && ATT_MAXW % 16 == 0, "merge layout");
  const int tid = threadIdx.x;
  const int nq = (r1 - r0) * G;
  float* Wt = sm.Wm;                                  // [query][term]: the weights (leaves: first the score)
  float* Lv = sm.Wm + ATTB_MAXQ * ATT_MAXW;           // [query][term]: l
  auto rec = [&](int qq, int sp) -> const float* {
    return part + (((size_t)(r0 + qq / G) * H + g * G + qq % G) * nsplit + sp) * REC;
  };
  auto nsplits = [&](int qq) { return min(sm.Rpos[qq / G] / ATT_SPLIT + 1, nsplit); };   // stored partials
  auto leaf = [&](int qq) { return LEAF && r0 + qq / G >= side0; };

  if (LEAF && side0 < r1) {
    // the leaves' own scores: one wave per query, lanes over the dimensions, then a butterfly
    const int lane = tid & 63, wave = tid >> 6;
    const float scale = 1.0f / sqrtf((float)HD);
    for (int qq = wave; qq < nq; qq += NW) {
      if (!leaf(qq)) continue;
      const int row = r0 + qq / G, head = g * G + qq % G;
      const bf16_t* qr = q + (size_t)row * ldq + (size_t)head * HD;
      const bf16_t* kr = side_kv + (size_t)(row - side0) * 2 * KVH * HD + (size_t)g * HD;
      float acc = 0.f;
      for (int d = lane; d < HD; d += 64) acc = fmaf(bf2f(qr[d]), bf2f(kr[d]), acc);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (lane == 0) Wt[qq * ATT_MAXW + nsplits(qq)] = fmul_nc(acc, scale);
    }
    __syncthreads();
  }
  const int qq = tid >> 4, j = tid & 15;
  if (qq >= nq) return;                               // whole groups; no barrier follows
  const int ns = nsplits(qq);
  const bool lf = leaf(qq);
  const int nt = ns + (lf ? 1 : 0);                   // merged terms
  const int d0 = j * DPT;
  // term c's o at dimensions d0 .. d0 + DPT - 1: a stored partial's, or the leaf's own value
  auto oload = [&](int c, f32x4 (&v)[NV]) {
    if (LEAF && c >= ns) {
      const bf16_t* vr = side_kv + ((size_t)(r0 + qq / G - side0) * 2 + 1) * KVH * HD + (size_t)g * HD + d0;
#pragma unroll
      for (int x = 0; x < NV; ++x) {
        const uint2 u = *(const uint2*)(vr + 4 * x);
        v[x] = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xFFFF0000u)};
      }
      return;
    }
#pragma unroll
    for (int x = 0; x < NV; ++x) v[x] = *(const f32x4*)(rec(qq, c) + d0 + 4 * x);
  };

  // one round of loads: (m, l) of the lane's terms, o of the first MCH terms (clamped to the last)
  float2 ml[MLR];
#pragma unroll
  for (int r = 0; r < MLR; ++r) {
    const int c = j + 16 * r;
    ml[r] = make_float2(-INFINITY, 0.f);
    if (c < ns) ml[r] = *(const float2*)(rec(qq, c) + HD);
    else if (LEAF && c < nt) ml[r] = make_float2(Wt[qq * ATT_MAXW + c], 1.f);
  }
  f32x4 ov[MCH][NV];
#pragma unroll
  for (int c = 0; c < MCH; ++c) oload(min(c, nt - 1), ov[c]);
  // the maximum over the query's terms, then each lane's terms' weights (and l) into LDS
  float m = ml[0].x;
#pragma unroll
  for (int r = 1; r < MLR; ++r) m = fmaxf(m, ml[r].x);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
#pragma unroll
  for (int r = 0; r < MLR; ++r) {
    const int c = j + 16 * r;
    if (c < nt) {
      Wt[qq * ATT_MAXW + c] = expf(fsub_nc(ml[r].x, m));
      Lv[qq * ATT_MAXW + c] = ml[r].y;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // o and l in term order, then o / l
  const float* w = Wt + qq * ATT_MAXW;
  const float* lw = Lv + qq * ATT_MAXW;
  f32x4 o[NV];
#pragma unroll
  for (int x = 0; x < NV; ++x) o[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  auto add = [&](int c, const f32x4 (&v)[NV]) {
    const float wc = w[c];
    l = fmaf(lw[c], wc, l);
#pragma unroll
    for (int x = 0; x < NV; ++x)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[x][i] = fmaf(v[x][i], wc, o[x][i]);
  };
#pragma unroll
  for (int c = 0; c < MCH; ++c)
    if (c < nt) add(c, ov[c]);
  for (int c0 = MCH; c0 < nt; c0 += MCH) {            // contexts past 64 * MCH positions
#pragma unroll
    for (int c = 0; c < MCH; ++c) oload(min(c0 + c, nt - 1), ov[c]);
#pragma unroll
    for (int c = 0; c < MCH; ++c)
      if (c0 + c < nt) add(c0 + c, ov[c]);
  }
  const int row = r0 + qq / G, head = g * G + qq % G;
  bf16_t* dst = out + dec_act_index(row, head * HD + d0);   // d0 % DPT == 0: DPT contiguous elements
  uint32_t pk[DPT / 2];
#pragma unroll
  for (int x = 0; x < NV; ++x) {
    pk[2 * x] = (uint32_t)f2bf(__fdiv_rn(o[x][0], l)) | ((uint32_t)f2bf(__fdiv_rn(o[x][1], l)) << 16);
    pk[2 * x + 1] = (uint32_t)f2bf(__fdiv_rn(o[x][2], l)) | ((uint32_t)f2bf(__fdiv_rn(o[x][3], l)) << 16);
  }
  if constexpr (DPT == 8) *(uint4*)dst = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  else *(uint2*)dst = make_uint2(pk[0], pk[1]);
}

// blocked: out in the decode block layout (ldo unused), else rows of stride ldo.
template <typename T, int HD>
__device__ __forceinline__ void attn_combine_elem(const float* __restrict__ part, int nsplit, int row, int head,
                                                  int H, int p, int d, T* __restrict__ out, int ldo, bool blocked) {
  const size_t o = blocked ? dec_act_index(row, head * HD + d) : (size_t)row * ldo + (size_t)head * HD + d;
  st(out + o, attn_combine_value<HD>(part, nsplit, row, head, H, p, d));
}

}  // namespace ssd
