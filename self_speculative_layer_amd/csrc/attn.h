// Attention over the paged KV cache (device functions shared by the
// standalone attention kernels and the persistent decode kernel).
//
// Keys are split at fixed absolute positions: split s covers [64 s, 64 s + 64).
// A work item handles one KV head g, one split and a block of rows with all
// their query heads (grouped-query attention); it stages 64 keys at a time in
// LDS (16-byte vector loads, all in flight) in the storage type, keeps an
// online softmax per query in fp32 and writes a partial (o[HD], m, l).  The
// combine merges a row's partials in split order.  Split and chunk boundaries
// are fixed positions, so a row's result does not depend on the rows batched
// with it.
#pragma once
#include "common.h"

namespace ssd {

constexpr int ATT_SPLIT = 64;
constexpr int ATT_CHUNK = 64;
constexpr int ATT_MAXQ = 64;     // queries (rows x heads of a group) per work item

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

typedef uint32_t att_u32x4 __attribute__((ext_vector_type(4)));

// Partial results are stored either plainly (read by a later kernel) or with
// device-scope stores (read by another workgroup of the same kernel).
template <bool DEV>
__device__ __forceinline__ void part_store(float* p, float v) {
  if constexpr (DEV) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}

// One work item: KV head g, split s, the rows r0 .. min(r0 + RB, Ma) - 1 with
// Ma = min(M, *nrows) (positions increasing).  Keys at positions >= local_start
// come from local_kv rows (scoring: the candidate's own keys/values, rows
// grouped by group_rows).  Requires all NW*64 threads of the block.
//
// Loads take two rounds: (1) the active-row count, the rows' positions, the
// chunk's page ids and the queries; (2) every key and value of the chunk.
// Items whose split starts past the block's last position return after (1).
// DEV: partials are written with device-scope stores.
template <typename T, int HD, int NW, bool DEV = false>
__device__ void attn_partial_item(AttnSmem<T, HD, NW>& sm, const T* __restrict__ q, int ldq,
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
        sc = __fmul_rn(acc, scale);
      }
      const float mx = wave_max(sc);
      const float pexp = valid ? expf(__fsub_rn(sc, mx)) : 0.f;
      const float psum = wave_sum(pexp);
      sm.Pw[wave][lane] = pexp;
      __builtin_amdgcn_wave_barrier();
      float* dstp = part + (((size_t)row * H + head) * nsplit + s) * (HD + 2);
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

// Merge the splits of (row, head) in split order; component d of the output.
template <int HD>
__device__ __forceinline__ float attn_combine_value(const float* __restrict__ part, int nsplit, int row, int head,
                                                   int H, int p, int d) {
  const int ns = p / ATT_SPLIT + 1;
  const float* pr = part + ((size_t)row * H + head) * nsplit * (HD + 2);
  constexpr int B = 16;
  if (ns <= B) {
    // one round of loads
    float mv[B], lv[B], ov[B];
#pragma unroll
    for (int s = 0; s < B; ++s) {
      mv[s] = -INFINITY;
      lv[s] = ov[s] = 0.f;
      if (s < ns) {
        mv[s] = pr[s * (HD + 2) + HD];
        lv[s] = pr[s * (HD + 2) + HD + 1];
        ov[s] = pr[s * (HD + 2) + d];
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int s = 0; s < B; ++s) m = fmaxf(m, mv[s]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int s = 0; s < B; ++s) {
      if (s < ns) {
        const float w = expf(__fsub_rn(mv[s], m));
        l = fmaf(lv[s], w, l);
        o = fmaf(ov[s], w, o);
      }
    }
    return __fdiv_rn(o, l);
  }
  float m = -INFINITY;
#pragma unroll 16
  for (int s = 0; s < ns; ++s) m = fmaxf(m, pr[s * (HD + 2) + HD]);
  float l = 0.f, o = 0.f;
#pragma unroll 16
  for (int s = 0; s < ns; ++s) {
    const float w = expf(__fsub_rn(pr[s * (HD + 2) + HD], m));
    l = fmaf(pr[s * (HD + 2) + HD + 1], w, l);
    o = fmaf(pr[s * (HD + 2) + d], w, o);
  }
  return __fdiv_rn(o, l);
}

template <typename T, int HD>
__device__ __forceinline__ void attn_combine_elem(const float* __restrict__ part, int nsplit, int row, int head,
                                                  int H, int p, int d, T* __restrict__ out, int ldo) {
  st(out + (size_t)row * ldo + (size_t)head * HD + d, attn_combine_value<HD>(part, nsplit, row, head, H, p, d));
}

}  // namespace ssd
