// Confidence-sized draft trees (SWIFT: "Confidence-aware inference
// acceleration", §4.2 — the draft's confidence sets how many candidates go to
// the parallel verification; §3.2.1 and Figure 2 — top-k drafts raise the
// acceptance).  Readings taken where the page gives no formula:
//   * the candidates of draft step j are the k_j most probable tokens of
//     softmax(z_j) (temperature 1 when greedy; lowest index first among equal logits),
//     k_j = the least k >= 1 whose top-k mass reaches rho, at most k_max;
//   * only the top candidate is drafted further; the others are leaves at its
//     position, attending to the prefix and themselves;
//   * leaves are kept in depth order, then rank order, up to the verify
//     pass's free rows;
//   * greedy acceptance walks the chain; where the target's choice differs
//     from the draft it may be a leaf of that depth, which is then emitted
//     with the target's choice after it;
//   * when sampling (T > 0) the leaves are further draws of softmax(z / T),
//     since the speculative-sampling rule keeps the target distribution only
//     for drawn candidates; their acceptance (the multi-candidate rule) is in
//     kernels.hip next to the chain's.
// The kernels here are control-sized (one block per draft row, or one wave);
// the verify rows themselves run through the decode-block kernels.
#include <math.h>

#include "kernels.h"
#include "attn.h"

namespace ssd {

static inline int tree_ok(hipError_t e) { return e == hipSuccess ? 0 : SSD_ERR_HIP; }

// (v, i) ranks before (tv, ti): larger value, or the same value at a lower index.
__device__ __forceinline__ bool tree_before(float v, int i, float tv, int ti) {
  return v > tv || (v == tv && i < ti);
}

// One block per draft row j < d': the row's k_max best tokens, their
// softmax(z / T) probabilities (T = 1 when T is 0) and the candidate count
// k_j.  cand[j][TREE_KMAX]: at T = 0 the ranks 0..k_max-1; at T > 0 entry r >= 1
// is the r-th extra draw of softmax(z / T) (race keys z / T + Gumbel, counter
// (iteration, j + 256 r, purpose leaf)); kcount[j].
__global__ __launch_bounds__(256) void tree_topk_kernel(const float* __restrict__ z, int V, int d,
                                                        const int32_t* __restrict__ n_drafted, float rho, int k_max,
                                                        float T, uint64_t seed, const DevState* __restrict__ st,
                                                        int* __restrict__ cand, int* __restrict__ kcount) {
  constexpr int K = TREE_KMAX;
  const int j = blockIdx.x;
  if (j >= min(*n_drafted, d)) return;
  const float* zr = z + (size_t)j * V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // each thread: its own best K in rank order (indices arrive in increasing order)
  float tv[K];
  int ti[K];
#pragma unroll
  for (int k = 0; k < K; ++k) { tv[k] = -INFINITY; ti[k] = 0x7fffffff; }
  for (int v = tid; v < V; v += 256) {
    float cv = zr[v];
    int ci = v;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const bool take = tree_before(cv, ci, tv[k], ti[k]);
      const float ov = tv[k];
      const int oi = ti[k];
      tv[k] = take ? cv : ov;
      ti[k] = take ? ci : oi;
      cv = take ? ov : cv;
      ci = take ? oi : ci;
    }
  }
  // k_max rounds of a block argmax over the threads' heads; the winner's owner drops it
  __shared__ float wv[4];
  __shared__ int wi[4];
  __shared__ float topv[K];
  __shared__ int topi[K];
  __shared__ float wsum[4];
  for (int r = 0; r < k_max; ++r) {
    float bv = tv[0];
    int bi = ti[0];
    wave_argmax(bv, bi);
    if (lane == 0) { wv[wave] = bv; wi[wave] = bi; }
    __syncthreads();
    if (tid == 0) {
      float v = wv[0];
      int i = wi[0];
      for (int w = 1; w < 4; ++w) argmax_merge(v, i, wv[w], wi[w]);
      topv[r] = v;
      topi[r] = i;
    }
    __syncthreads();
    const bool pop = ti[0] == topi[r];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
      tv[k] = pop ? tv[k + 1] : tv[k];
      ti[k] = pop ? ti[k + 1] : ti[k];
    }
    if (pop) { tv[K - 1] = -INFINITY; ti[K - 1] = 0x7fffffff; }
  }
  // softmax normaliser: sum of exp((z - max) / T), each thread's terms in index order, then wave and block
  const float m = topv[0];
  const float Tn = T > 0.f ? T : 1.f;
  float se = 0.f;
  for (int v = tid; v < V; v += 256) se += expf(__fdiv_rn(fsub_nc(zr[v], m), Tn));
  se = wave_sum(se);
  if (lane == 0) wsum[wave] = se;
  __syncthreads();
  __shared__ int s_k;
  if (tid == 0) {
    const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    float cum = 0.f;
    int k = k_max;
    for (int r = 0; r < k_max; ++r) {
      cum += __fdiv_rn(expf(__fdiv_rn(fsub_nc(topv[r], m), Tn)), tot);
      if (cum >= rho) { k = r + 1; break; }
    }
    for (int r = 0; r < K; ++r) cand[(size_t)j * K + r] = r < k_max ? topi[r] : -1;
    kcount[j] = k;
    s_k = k;
  }
  if (!(T > 0.f)) return;
  __syncthreads();
  // T > 0: the extra candidates are draws of softmax(z / T), one race per draw
  const int k = s_k;
  const int iter = st->iteration;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 1; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    const uint32_t row = (uint32_t)(j + TREE_ROW_STRIDE * r);
    for (int v4 = 4 * tid; v4 < V; v4 += 4 * 256) {
      const U4 w = philox4x32_10((uint32_t)iter, row, PURPOSE_LEAF, (uint32_t)(v4 >> 2), k0, k1);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v4 + e < V) argmax_merge(bv, bi, zr[v4 + e] / T + word_to_gumbel(ws[e]), v4 + e);
    }
    wave_argmax(bv, bi);
    if (lane == 0) { wv[wave] = bv; wi[wave] = bi; }
    __syncthreads();
    if (tid == 0) {
      float v = wv[0];
      int i = wi[0];
      for (int w = 1; w < 4; ++w) argmax_merge(v, i, wv[w], wi[w]);
      cand[(size_t)j * K + r] = i;
    }
    __syncthreads();
  }
}

// Leaves in depth order, then rank order (ranks 1 .. k_j - 1 of each step), at most max_leaves.
__global__ void tree_plan_kernel(const int* __restrict__ cand, const int* __restrict__ kcount, int d,
                                 const int32_t* __restrict__ n_drafted, int max_leaves, int32_t* __restrict__ leaf_tok,
                                 int32_t* __restrict__ leaf_depth, int32_t* __restrict__ n_leaves) {
  if (threadIdx.x != 0) return;
  const int dp = min(*n_drafted, d);
  int nl = 0;
  for (int j = 0; j < dp && nl < max_leaves; ++j)
    for (int r = 1; r < kcount[j] && nl < max_leaves; ++r) {
      leaf_tok[nl] = cand[(size_t)j * TREE_KMAX + r];
      leaf_depth[nl] = j + 1;
      ++nl;
    }
  *n_leaves = nl;
}

int launch_tree_candidates(const float* draft_logits, int V, int d, const int32_t* n_drafted, float T, uint64_t seed,
                           const DevState* st, float rho, int k_max, int max_leaves, int* cand, int* kcount,
                           int32_t* leaf_tok, int32_t* leaf_depth, int32_t* n_leaves, hipStream_t s) {
  if (k_max < 1 || k_max > TREE_KMAX || k_max > V || d < 1 || d > TREE_ROW_STRIDE) return SSD_ERR_ARG;
  hipLaunchKernelGGL(tree_topk_kernel, dim3(d), dim3(256), 0, s, draft_logits, V, d, n_drafted, rho, k_max, T, seed,
                     st, cand, kcount);
  hipLaunchKernelGGL(tree_plan_kernel, dim3(1), dim3(64), 0, s, cand, kcount, d, n_drafted, max_leaves, leaf_tok,
                     leaf_depth, n_leaves);
  return tree_ok(hipGetLastError());
}

// Rows of a tree verify.  Full block: chain rows i = 0..d' (y_i at kvlen + i), then leaf s at row
// d' + 1 + s (its token at kvlen + depth).  Prefix block (layers below the reuse boundary): y_d', then
// the leaves.  Rows past the active ones repeat the last active row.
__global__ void tree_verify_prep_kernel(DevState* st, const int32_t* __restrict__ drafts,
                                        const int32_t* __restrict__ n_drafted, int d,
                                        const int32_t* __restrict__ leaf_tok, const int32_t* __restrict__ leaf_depth,
                                        const int32_t* __restrict__ n_leaves, int max_leaves, int* __restrict__ vpos,
                                        int* __restrict__ vtok, int* __restrict__ ppos, int* __restrict__ ptok,
                                        int max_ctx) {
  if (threadIdx.x != 0) return;
  const int dp = max(min(*n_drafted, d), 0);
  const int nl = max(min(*n_leaves, max_leaves), 0);
  const int kv = st->kvlen;
  if (kv + dp >= max_ctx) st->error_flags |= ERRF_CAPACITY;
  for (int i = 0; i <= dp; ++i) {
    vpos[i] = min(kv + i, max_ctx - 1);
    vtok[i] = i == 0 ? st->last_token : drafts[i - 1];
  }
  ppos[0] = vpos[dp];
  ptok[0] = vtok[dp];
  for (int s = 0; s < nl; ++s) {
    int dep = leaf_depth[s];
    if (dep < 1 || dep > dp) {
      st->error_flags |= ERRF_INPUT;
      dep = min(max(dep, 1), max(dp, 1));
    }
    vpos[dp + 1 + s] = ppos[1 + s] = min(kv + dep, max_ctx - 1);
    vtok[dp + 1 + s] = ptok[1 + s] = leaf_tok[s];
  }
  for (int r = dp + 1 + nl; r < d + 1 + max_leaves; ++r) { vpos[r] = vpos[dp + nl]; vtok[r] = vtok[dp + nl]; }
  for (int r = 1 + nl; r < 1 + max_leaves; ++r) { ppos[r] = ppos[nl]; ptok[r] = ptok[nl]; }
  st->tree_rows = dp + 1 + nl;
  st->tree_prefix_rows = 1 + nl;
  st->tree_side_full = dp + 1;
  st->tree_side_prefix = 1;
  st->tree_leaf = -1;
}

int launch_tree_verify_prep(DevState* st, const int32_t* drafts, const int32_t* n_drafted, int d,
                            const int32_t* leaf_tok, const int32_t* leaf_depth, const int32_t* n_leaves,
                            int max_leaves, int* vpos, int* vtok, int* ppos, int* ptok, int max_ctx, hipStream_t s) {
  hipLaunchKernelGGL(tree_verify_prep_kernel, dim3(1), dim3(64), 0, s, st, drafts, n_drafted, d, leaf_tok,
                     leaf_depth, n_leaves, max_leaves, vpos, vtok, ppos, ptok, max_ctx);
  return tree_ok(hipGetLastError());
}

// Greedy tree acceptance from the verify rows' statistics (chain rows 0..d', leaf s at row d' + 1 + s).
__global__ void tree_accept_kernel(const ssd_row_stat* __restrict__ stats, const int32_t* __restrict__ drafts,
                                   const int32_t* __restrict__ n_drafted, int d,
                                   const int32_t* __restrict__ leaf_tok, const int32_t* __restrict__ leaf_depth,
                                   const int32_t* __restrict__ n_leaves, int max_leaves, DevState* st,
                                   int32_t* __restrict__ out, int32_t* __restrict__ n_out) {
  if (threadIdx.x != 0) return;
  const int dp = max(min(*n_drafted, d), 0);
  const int nl = max(min(*n_leaves, max_leaves), 0);
  st->tree_leaf = -1;
  for (int r = 0; r <= dp + nl; ++r)
    if (isnan(stats[r].max)) {          // a row with non-finite logits: nothing is emitted
      st->error_flags |= ERRF_NUMERIC;
      *n_out = 0;
      return;
    }
  for (int j = 1; j <= dp; ++j) {
    const int a = stats[j - 1].argmax;
    out[j - 1] = a;
    if (a == drafts[j - 1]) continue;
    for (int s = 0; s < nl; ++s) {
      if (leaf_depth[s] == j && leaf_tok[s] == a) {
        out[j] = stats[dp + 1 + s].argmax;
        *n_out = j + 1;
        st->tree_leaf = s;
        st->tree_leaf_pos = st->kvlen + j;
        return;
      }
    }
    *n_out = j;
    return;
  }
  out[dp] = stats[dp].argmax;
  *n_out = dp + 1;
}

// An accepted leaf's keys and values (every layer) into the cache at its position: block (layer, k/v
// and KV head).
__global__ void tree_kv_fix_kernel(const DevState* __restrict__ st, const bf16_t* __restrict__ side_kv,
                                   bf16_t* __restrict__ pool, const int* __restrict__ page_table, int PS,
                                   int n_lpages, int L, int KVH, int HD) {
  const int s = st->tree_leaf;
  if (s < 0) return;
  const int p = st->tree_leaf_pos, lp = p / PS;
  if (p < 0 || lp >= n_lpages) return;               // flagged by the verify's preparation
  const int l = blockIdx.x, kvsel = blockIdx.y / KVH, g = blockIdx.y % KVH;
  const bf16_t* src = side_kv + (((size_t)l * TREE_SLOTS + s) * 2 + kvsel) * KVH * HD + (size_t)g * HD;
  bf16_t* dst = pool + kv_index(page_table[lp], L, l, kvsel, KVH, g, PS, p % PS, HD);
  for (int i = threadIdx.x; i < HD; i += blockDim.x) dst[i] = src[i];
}

int launch_tree_accept(const ssd_row_stat* stats, const int32_t* drafts, const int32_t* n_drafted, int d,
                       const int32_t* leaf_tok, const int32_t* leaf_depth, const int32_t* n_leaves, int max_leaves,
                       DevState* st, int32_t* out, int32_t* n_out, hipStream_t s) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3(1), dim3(64), 0, s, stats, drafts, n_drafted, d, leaf_tok, leaf_depth,
                     n_leaves, max_leaves, st, out, n_out);
  return tree_ok(hipGetLastError());
}

int launch_tree_kv_fix(const DevState* st, const bf16_t* side_kv, const KvView& kv, int L, int KVH, int HD,
                       hipStream_t s) {
  hipLaunchKernelGGL(tree_kv_fix_kernel, dim3(L, 2 * KVH), dim3(64), 0, s, st, side_kv, (bf16_t*)kv.pool,
                     kv.page_table, kv.page_size, kv.n_lpages, L, KVH, HD);
  return tree_ok(hipGetLastError());
}

}  // namespace ssd
