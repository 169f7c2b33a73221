// Host-side launchers of the library's HIP kernels (kernels.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "../../include/ssd.h"

namespace ssd {

// Records msg as the calling thread's last error (ssd_last_error) and returns code.
int set_last_error(int code, const char* msg);

// GEMM epilogues: Y = X . W^T then
enum Epilogue {
  EPI_STORE = 0,    // Y[m, n] = acc                          (float)
  EPI_RESID = 1,    // Y[m, n] += acc                         (float residual stream)
  EPI_SWIGLU = 2    // A[m, f] = act(silu(acc_gate) * acc_up) (act dtype; W rows f and f + up_rows)
};

// Description of a block of rows that flows through the decoder layers.
struct RowBlock {
  int M;               // static row count (grid size)
  const int* nrows;    // device: active rows (nullable -> M)
  const int* pos;      // device: absolute position of each row [M]
  const int* ymap;     // device: residual row of each compact row (nullable -> identity)
  const int* stop;     // device: early-exit flag (nullable)
};

struct KvView {
  void* pool;          // [pages][L][2][KVH][PS][HD]
  const int* page_table;
  int n_lpages, page_size;
};

// Linear layer: X [M, K] (row stride ldx, act dtype) times W [N, K]^T.
// For EPI_SWIGLU, N = F (output features) and W holds 2F rows (gate, then up).
// rscale (nullable): per-row factor applied to the product before the
// epilogue (not for EPI_RESID).
// split_ws (nullable): at least split_floats floats of workspace, which small many-row problems use to
// split K by quarter across workgroups (4 x M x N floats).
int launch_linear(int dtype, int epi, const void* W, const void* X, int ldx, int M, int N, int K,
                  float* Y, int ldy, void* A, int lda, const float* rscale, const int* nrows, const int* ymap,
                  const int* stop, hipStream_t s, float* split_ws = nullptr, size_t split_floats = 0);

// Row-major bf16 [N, K] -> packed tile layout (K % 32 == 0).
int launch_pack_bf16(const void* src, void* dst, int N, int K, hipStream_t s);

// x[m] = act(h[hmap[m]] * gain / sqrt(mean(h^2) + eps)) (the projection input of an RMSNorm, rounded once);
// inv (nullable) receives the rows' 1 / sqrt(mean(h^2) + eps).
int launch_rowprep(int dtype, const float* h, int ldh, const float* gain, void* x, int ldx, float* inv, int M, int D,
                   float eps, const int* nrows, const int* hmap, const int* stop, hipStream_t s);

int launch_embed(int dtype, const void* emb, const int* tokens, int V, float* h, int ldh, int M, int D,
                 const int* nrows, const int* stop, hipStream_t s);

// RoPE on q and k, bf16/f32 storage of q into qout and of k, v into the cache
// (or, when local_kv != nullptr, into local_kv[row][2][KVH][HD]).
int launch_rope_kv(int dtype, int head_dim, const float* qkv, int ldqkv, void* qout, int ldq,
                   const KvView& kv, int L, int layer, int H, int KVH, const RowBlock& rb,
                   const float2* rope_cs, void* local_kv, int* err_flags, hipStream_t s);

// Attention of every row over cached keys at positions <= its own (keys at
// positions >= local_start come from local_kv rows of the row's own group of
// `group_rows` consecutive rows).  Output act dtype [M, H*HD].
// out_blocked: the output in the decode block layout (M <= 16) instead of rows of stride ldo.
int launch_attention(int dtype, int head_dim, const void* q, int ldq, const KvView& kv, int L, int layer,
                     int H, int KVH, const RowBlock& rb, int max_ctx, const void* local_kv,
                     int local_start, int group_rows, float* part, void* out, int ldo, hipStream_t s,
                     bool out_blocked = false);
// The mask-scoring pass's attention (attn_group.hip): rows in groups of group_rows consecutive rows, each
// group one candidate whose positions >= local_start come from its own keys and values in local_kv; bf16,
// head_dim 64 or 128, H / KVH <= 64.  Output rows of stride ldo.
int launch_attention_groups(int head_dim, const void* q, int ldq, const KvView& kv, int L, int layer, int H, int KVH,
                            const RowBlock& rb, const void* local_kv, int local_start, int group_rows, void* out,
                            int ldo, hipStream_t s);
// Whether launch_attention takes launch_attention_groups for candidate groups of this model shape.
inline bool attention_groups_usable(int dtype, int head_dim, int H, int KVH) {
  return dtype == SSD_DTYPE_BF16 && (head_dim == 64 || head_dim == 128) && H / KVH <= 64;
}
// Rows one launch of the split-key attention takes (the partial buffer holds this many rows); prefill
// chunks are at most this long.
constexpr int SPLIT_ATTN_MAX_ROWS = 1024;
size_t attention_partial_floats(int max_rows, int H, int head_dim, int max_ctx);
// Number of fixed key splits covering max_ctx positions (the partial buffer's split dimension).
int attention_nsplit(int max_ctx);

// Row statistics (a3).  purpose/rowid_base address the random draws.
int launch_row_stats(const float* z, int ldz, int rows, int V, float T, uint64_t seed,
                     const int* iter_ptr, int iter_const, int rowid_base, uint32_t purpose,
                     ssd_row_stat* out, const int* stop, hipStream_t s);

// Row statistics over segments of STAT_SEG logits with a merge by the last
// segment (recs: rows x stat_segments(V) records; ctr: rows counters, zero
// between launches).  With ds.st set, row 0 is draft step ds.j: the merge
// writes the draft token and applies the confidence stop instead of out.
constexpr int STAT_SEG = 2048;
constexpr int STAT_MAXSEG = 64;
struct StatRec { float v1; int i1; float v2; float s; float kv; int ki; int bad; int pad; };
struct DraftStep {
  DevState* st;            // nullptr: plain row statistics
  int j, d;
  float tau;
  int32_t* draft_tokens;
  int32_t* n_drafted_out;
};
int stat_segments(int V);
int launch_row_stats_seg(const float* z, int ldz, int rows, int V, float T, uint64_t seed, const int* iter_ptr,
                         int iter_const, int rowid_base, uint32_t purpose, ssd_row_stat* out, StatRec* recs,
                         unsigned* ctr, const int* stop, const DraftStep& ds, hipStream_t s);


// Accept / reject of a chain (d + 1 verify rows): dec, corr [d + 1] hold the per-row decisions and draws
// between the two kernels; the draws are addressed by iteration *iter_ptr (or iter_const when null).
// Rows with NaN or +inf logits emit nothing (n_out = 0) and raise ERRF_NUMERIC in *err_flags (nullable).
int launch_accept(const float* zp, const float* zq, int V, const int32_t* drafts, const int32_t* n_drafted,
                  int d, float T, uint64_t seed, const int* iter_ptr, int iter_const, int* dec, int* corr,
                  int32_t* out_tokens, int32_t* n_out, int* err_flags, hipStream_t s);

// Commits n_out tokens (at most max_n; 0 commits nothing).
int launch_commit(DevState* st, const int32_t* out_tokens, const int32_t* n_out, int32_t* log,
                  int log_cap, int max_n, hipStream_t s);

// Pick one token from a row's stats and commit it (prefill / AR step).
int launch_pick_commit(const ssd_row_stat* stat, DevState* st, int32_t* log, int log_cap, int set_kvlen,
                       int kvlen_value, hipStream_t s);

// Small control kernels.
int launch_state_init(DevState* st, hipStream_t s);
int launch_fill_positions(int* pos, int M, int start, hipStream_t s);
int launch_window_rows(const int32_t* window, int R, int gamma, int pos0, int* pos, int* tok, hipStream_t s);
// h rows dst * gamma + i = rows src * gamma + i (i < gamma) for each of the n_pairs (src, dst) pairs.
int launch_copy_candidate_rows(float* h, int D, const int* pairs, int n_pairs, int gamma, hipStream_t s);
int launch_single_row_prep(DevState* st, int* pos1, int* tok1, int max_ctx, hipStream_t s);
int launch_draft_begin(DevState* st, hipStream_t s);
int launch_draft_step_prep(DevState* st, const int32_t* drafts, int j, int* pos1, int* tok1, int max_ctx,
                           int32_t* n_drafted_out, hipStream_t s);
int launch_verify_prep(DevState* st, const int32_t* drafts, const int32_t* n_drafted, int d, int* vpos,
                       int* vtok, int* pos1, int* tok1, int max_ctx, hipStream_t s);
// Copies rows r < (count ? *count : rows) of src [.., D] to dst row r + (dst_off ? *dst_off : 0).
int launch_copy_rows(const float* src, float* dst, int rows, int D, const int* count, const int* dst_off,
                     const int* stop, hipStream_t s);
// SpecEE exit features of rows hidden states h [rows, D] for k <= 16 speculative tokens: out [rows][3k] =
// (logits, local probabilities, variation against prev [rows][k] or 0).
int launch_specee_features(int dtype, const float* h, int rows, int D, float eps, const float* gain, const void* W,
                           int V, const int32_t* tokens, int k, const float* prev, float* out, hipStream_t s);
int launch_score(const ssd_row_stat* stats, const int32_t* window, int n_masks, int gamma, float* scores,
                 int32_t* best, int32_t* row_pred, hipStream_t s);

// ---------------------------------------------------------------------------
// Draft trees (tree.hip).

// Per draft row j < d' (rows of draft_logits): the k_max best tokens into cand[j][TREE_KMAX] and the
// candidate count into kcount[j]; then the leaves (ranks 1 .. k_j - 1, depth order) into leaf_tok /
// leaf_depth, their number into n_leaves.
int launch_tree_candidates(const float* draft_logits, int V, int d, const int32_t* n_drafted, float T, uint64_t seed,
                           const DevState* st, float rho, int k_max, int max_leaves, int* cand, int* kcount,
                           int32_t* leaf_tok, int32_t* leaf_depth, int32_t* n_leaves, hipStream_t s);
// Row positions / tokens of a tree verify's full block (vpos, vtok [d + 1 + max_leaves]) and prefix block
// (ppos, ptok [1 + max_leaves]); the row counts and first leaf rows in the device state.
int launch_tree_verify_prep(DevState* st, const int32_t* drafts, const int32_t* n_drafted, int d,
                            const int32_t* leaf_tok, const int32_t* leaf_depth, const int32_t* n_leaves,
                            int max_leaves, int* vpos, int* vtok, int* ppos, int* ptok, int max_ctx, hipStream_t s);
// Greedy tree acceptance from the verify rows' statistics.
int launch_tree_accept(const ssd_row_stat* stats, const int32_t* drafts, const int32_t* n_drafted, int d,
                       const int32_t* leaf_tok, const int32_t* leaf_depth, const int32_t* n_leaves, int max_leaves,
                       DevState* st, int32_t* out, int32_t* n_out, hipStream_t s);
// Sampled (T > 0) tree acceptance (kernels.hip): the chain rule per row, then the multi-candidate rule at
// the first rejected depth when it has leaves.
int launch_tree_accept_sampled(const float* zp, const float* zq, int V, const int32_t* drafts,
                               const int32_t* n_drafted, int d, const int32_t* leaf_tok, const int32_t* leaf_depth,
                               const int32_t* n_leaves, int max_leaves, float T, uint64_t seed, DevState* st,
                               int* dec, int* corr, int32_t* out, int32_t* n_out, hipStream_t s);
// The accepted leaf's keys and values (side_kv [L][TREE_SLOTS][2][KVH * HD]) into the cache at its position.
int launch_tree_kv_fix(const DevState* st, const bf16_t* side_kv, const KvView& kv, int L, int KVH, int HD,
                       hipStream_t s);
// Whether the decode attention can merge a leaf's own term at this context length.
bool attention_dec_leaves_fit(int max_ctx);

// ---------------------------------------------------------------------------
// Decode mode (decode.hip): blocks of at most 16 rows, bf16.

enum DecEpilogue {
  DEC_STORE = 0,    // Y[m, n] = acc                                            (LM head, fp32 logits)
  DEC_RESID = 1,    // Y[m, n] += acc; then xg_next, ss_next of the new row (when gain_next)
  DEC_SWIGLU = 2,   // A[m, f] = bf16(silu(acc_gate) * acc_up)
  DEC_QKV = 3       // acc rotated (q, k), stored to q / the paged cache
};

// STORE, SWIGLU and QKV consume an RMSNorm: their input is Xf = h * gain (fp32) with the rows' 16-feature
// tile sums of h^2 in ss[m][K/16]; the product is taken with bf16(Xf[m] / sqrt(mean(h^2) + eps)).
// Activations are in the decode block layouts of common.h: X and A (bf16) by dec_act_index, Xf and
// xg_next (fp32) by dec_actf_index.
struct DecGemm {
  const bf16_t* W; int N, K;        // W [N rows (SWIGLU: 2N), K]
  const bf16_t* X;                  // RESID: activations [M <= 16, K], decode block layout
  const float* Xf;                  // STORE, SWIGLU, QKV: rows h * gain [M <= 16, K], decode block layout
  int M; const int* nrows; const int* stop;
  const float* ss; float eps;       // STORE, SWIGLU, QKV: tile sums of h^2 of the normalised rows
  float* Y; int ldy;                // STORE: output; RESID: residual stream
  bf16_t* A;                        // SWIGLU output [M, N], decode block layout
  const float* gain_next;           // RESID: gain of the next RMSNorm consumer (nullable: none)
  float* xg_next;                   //   its input h * gain [M, N] (fp32), decode block layout
  float* ss_next;                   //   tile sums of h^2 [M, N/16]
  float* y_copy;                    //   (nullable) second destination of the new residual rows (stride ldy)
  bf16_t* q; int ldq;               // QKV: rotated queries [M, H*HD]
  bf16_t* pool; const int* page_table;
  int PS, n_lpages, L, layer, H, KVH, HD;
  const int* pos; const float2* rope_cs; int* err;
  const int* side_from;             // QKV (nullable): rows >= *side_from are tree leaves; their k, v go to
  bf16_t* side_kv;                  //   side_kv[(row - *side_from) * 2 + {0, 1}][KVH * HD] instead of the cache
  int n_tiles;                      // set by the launcher
  int* prof_ran;                    // set by the launcher: timing record of a profiled launch (or null)
};
int launch_dec_gemm(int epi, const DecGemm& a, hipStream_t s);

// Attention with the split merge folded in; counters[n_row_blocks][KVH] start at zero and are left at zero.
// side_from (nullable): rows >= *side_from are tree leaves, which see the cache up to their position - 1
// and their own key / value from side_kv[(row - *side_from) * 2 + {0, 1}][KVH * HD] (needs
// attention_nsplit(max_ctx) < ATT_MAXW).
int launch_attention_dec(int head_dim, const void* q, int ldq, const KvView& kv, int L, int layer, int H, int KVH,
                         int M, const int* nrows, const int* pos, int max_ctx, float* part, void* out, int ldo,
                         unsigned* counters, const int* stop, hipStream_t s, const int* side_from = nullptr,
                         const void* side_kv = nullptr);

// Draft step j's entry row: position and token from the device state (or the end of the draft when the
// KV pages are full), then the embedding row and the first consumer's input, as launch_dec_entry.
int launch_dec_draft_entry(DevState* st, const int32_t* drafts, int j, int* pos1, int* tok1, int max_ctx,
                           int32_t* n_drafted_out, const void* emb, int V, float* h, int D, const float* gain,
                           void* xg, float* ss, hipStream_t s);

// h[dst] = embedding row of tokens[r] (tokens != nullptr) or src[r], for r < (count ? *count : rows),
// dst = r + (dst_off ? *dst_off : 0); with gain, also xg[dst] = h * gain (fp32) and ss[dst] tile sums.
// block_rows: the rows of the block the rows enter (a one-row block stores its consumer input row-major).
int launch_dec_entry(const void* emb, const int* tokens, int V, const float* src, int rows, const int* count,
                     const int* dst_off, float* h, int D, const float* gain, void* xg, float* ss, const int* stop,
                     int block_rows, hipStream_t s);

}  // namespace ssd
