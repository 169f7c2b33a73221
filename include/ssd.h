/*
 * ssd.h — C ABI of the MI355X self-speculative decoding library (libssd.so).
 *
 * One self-speculative decoding (SSD) step of a Llama-style decoder at batch 1:
 *   draft  — up to d tokens through the sub-layers a skip plan keeps (a SWIFT
 *            skip mask or a LayerSkip exit layer E), stopping early when the
 *            draft's confidence falls below a threshold;
 *   verify — one full-depth pass over the d'+1 draft positions that reuses the
 *            draft's state below the first skipped layer, then the shared LM head;
 *   accept — min(1, p/q) accept/reject with resampling from norm(max(0, p - q))
 *            and a bonus token when every draft is accepted;
 * plus SWIFT's matchness scoring of candidate skip plans against committed context
 * and its layer-set search, dynamic verification with confidence-sized draft
 * trees, lossy early-exit decoding, and SpecEE's speculative-token features.
 *
 * Sources (web pages, cited by title and section):
 *   [SWIFT]     "SWIFT: On-the-Fly Self-Speculative Decoding for LLM Inference
 *               Acceleration" (paper digest, arXiv 2410.06916v2)
 *   [LayerSkip] "ACL'24 | LayerSkip: Meta 把 Self-Speculative Decoding 从头训到尾"
 *               (blog post)
 *   [SpecEE]    "SpecEE: Accelerating Large Language Model Inference with
 *               Speculative Early Exiting" (study notes)
 *
 * Conventions
 *   - Every pointer named *_dev is device memory of the GPU current when the
 *     object was created; the caller allocates and owns it.  No entry point of
 *     this header allocates device memory; the library's own device memory is
 *     the fixed scratch array of ssd_accept_noalloc (part of its code object)
 *     and, only while profiling is enabled, the timing records of
 *     ssd_profile_enable (ssd_profile.h).  *_host pointers are host memory,
 *     read during the call only.
 *   - Weights are row-major [out_features, in_features] ("[N, K]"), in the
 *     model dtype (SSD_DTYPE_F32: float, SSD_DTYPE_BF16: bfloat16 bits).  Norm
 *     gains are float32.
 *   - Calls taking a hipStream_t enqueue work on that stream and return without
 *     waiting, except where stated.  One sequence must not be used from two
 *     streams at once; calls on one sequence are ordered by its stream.
 *   - Return value: SSD_OK (0) or a negative ssd_status.  ssd_last_error()
 *     gives a message for the calling thread's last failure.  Nothing aborts
 *     and nothing throws across this boundary.  Conditions found on the device
 *     (KV capacity exceeded, non-finite logits, a device-side argument out of
 *     range) set a sticky flag in the sequence, reported by ssd_read_state()
 *     and ssd_read_output().
 *
 * Sequence state kept on the device (so that a whole iteration can be enqueued
 * without a host round trip, and captured in a HIP graph):
 *   kvlen      number of positions whose keys/values are committed (= n - 1 for
 *              n committed tokens: the newest token is not yet in the cache);
 *   last_token the newest committed token (the next draft's input y0);
 *   iteration  SSD iteration counter (0 = the prefill's token), used to address
 *              the random draws;
 *   n_out      total tokens committed to the output log (the prefill's token
 *              counts).
 */
#ifndef SSD_H
#define SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_ARG = -1,          /* null pointer, negative size, value out of range */
  SSD_ERR_SHAPE = -2,        /* shape unsupported by the kernels (see ssd_model_create) */
  SSD_ERR_CAPACITY = -3,     /* KV pages, workspace or row limits exceeded */
  SSD_ERR_HIP = -4,          /* a HIP runtime call failed */
  SSD_ERR_UNSUPPORTED = -5,  /* option not implemented for this dtype/shape */
  SSD_ERR_NUMERIC = -6       /* non-finite logits were seen on the device */
} ssd_status;

typedef enum ssd_dtype { SSD_DTYPE_F32 = 0, SSD_DTYPE_BF16 = 1 } ssd_dtype;

typedef struct ssd_model ssd_model;
typedef struct ssd_seq ssd_seq;

/* Weight layouts.  Logical shapes below are [rows N, columns K] (y = W x).
 * fp32 models: row-major, K contiguous.
 * bf16 models: the projection weights (w_qkv, w_o, w_gate_up, w_down, lm_head)
 * are packed in matrix-core tiles: 16-row groups, each split into 32-column
 * steps of 16 x 32 elements stored contiguously (1 KB), i.e. element (n, k) at
 *   ((n / 16) * (K / 32) + k / 32) * 512 + (n % 16) * 32 + k % 32,
 * with N rounded up to a multiple of 16 (padding rows are never used for an
 * output).  ssd_pack_bf16 converts a row-major matrix; ssd_packed_bf16_bytes
 * gives the size.  The embedding stays row-major [V, D] (rows are gathered). */

/* Weights of one decoder layer. */
typedef struct ssd_layer_weights {
  const float* attn_norm;   /* [D] float32 RMSNorm gain before attention */
  const void* w_qkv;        /* [(H + 2*KVH) * hd, D]: rows 0..H*hd-1 = Wq,
                               then KVH*hd rows of Wk, then KVH*hd rows of Wv */
  const void* w_o;          /* [D, H * hd] */
  const float* mlp_norm;    /* [D] float32 RMSNorm gain before the MLP */
  const void* w_gate_up;    /* [2F, D]: rows 0..F-1 = Wgate, rows F..2F-1 = Wup */
  const void* w_down;       /* [D, F] */
} ssd_layer_weights;

/* Llama-2 style decoder ([SWIFT] §5.1 LLaMA-2 backbones; [LayerSkip] §2 one LM
 * head shared by every exit): h = Emb[t]; per layer h += Wo·Attn(RoPE(Wq x),
 * RoPE(Wk x), Wv x) with x = RMSNorm(h), then h += Wdown·(silu(Wgate x) * Wup x)
 * with x = RMSNorm(h); logits = LMhead·RMSNorm_final(h).  No biases, RoPE with
 * rotate-half pairing (i, i + hd/2), grouped-query attention (query head j uses
 * KV head j / (H / KVH)), attention scale hd^-1/2.
 * Supported: head_dim 64 or 128; D, F multiples of 64; H % KVH == 0, with at
 * most 64 (fp32) or 16 (bf16) query heads per KV head. */
typedef struct ssd_model_desc {
  int n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rms_eps;            /* e.g. 1e-5 */
  float rope_theta;         /* e.g. 10000 */
  int dtype;                /* ssd_dtype: storage of weights, activations and the KV cache */
  const void* embed;        /* [V, D] row-major */
  const float* final_norm;  /* [D] float32 */
  const void* lm_head;      /* [V, D] (bf16: packed) */
  const ssd_layer_weights* layers;  /* host array of n_layers entries (copied) */
} ssd_model_desc;

/* Per-row softmax statistics of a logits row z (row a3 of the path;
 * [LayerSkip] §3.1 softmax/argmax of the draft; [SpecEE] AdaInfer §1 "top
 * prob" and the top-2 gap). */
typedef struct ssd_row_stat {
  float max;        /* max_v z_v */
  int32_t argmax;   /* lowest index attaining max */
  float max2;       /* second largest value (z at another index); -inf if V == 1 */
  float lse;        /* log sum_v exp(z_v / T) (T = 1 when temperature is 0) */
  float conf;       /* max_v softmax(z / T)_v */
  int32_t sample;   /* argmax at T = 0, else a draw from softmax(z / T) */
} ssd_row_stat;

/* Host-visible copy of the sequence's device state (ssd_read_state). */
typedef struct ssd_state {
  int32_t kvlen, last_token, iteration, n_out, error_flags;
  int32_t last_n_drafted, last_n_emitted;
} ssd_state;

/* ---- model ---------------------------------------------------------------- */

/* Validates the shape and records the weight pointers (which must stay valid
 * until ssd_model_destroy).  Builds nothing on the device. */
int ssd_model_create(const ssd_model_desc* desc, ssd_model** out_model);

/* Bytes of a bf16 [N, K] weight in the packed tile layout (K a multiple of 32):
 * ceil(N / 16) * 16 * K * 2.  SSD_ERR_SHAPE otherwise. */
int ssd_packed_bf16_bytes(int N, int K, size_t* bytes);

/* Packs a row-major bf16 [N, K] matrix (src, device) into the tile layout
 * (dst, device, ssd_packed_bf16_bytes; caller-owned; must not overlap src);
 * padding rows are zero.  Enqueued on stream; SSD_ERR_SHAPE if K % 32 != 0. */
int ssd_pack_bf16(const void* src, void* dst, int N, int K, hipStream_t stream);
int ssd_model_destroy(ssd_model* model);

/* Bytes of the KV pool for n_pages pages of page_size positions.
 * Pool layout: [n_pages][L][2 (K, V)][KVH][page_size][hd] in the model dtype. */
int ssd_kv_pool_bytes(const ssd_model* model, int n_pages, int page_size, size_t* bytes);

/* Bytes of the per-sequence device workspace.
 *   max_rows   largest row block processed at once: d + 1 for verify, n_masks * gamma
 *              for scoring, the prefill chunk (prefill takes at most 1024 rows at a
 *              time); 1..SSD_MAX_ROWS.  Scoring more than 1024 rows needs a bf16 model
 *              with head_dim 64 or 128 and at most 64 query heads per KV head
 *              (SSD_ERR_UNSUPPORTED otherwise);
 *   max_draft  largest d passed to ssd_draft (<= 32);
 *   max_ctx    page_size * n_logical_pages of the sequence. */
#define SSD_MAX_ROWS 4096
int ssd_workspace_bytes(const ssd_model* model, int max_rows, int max_draft, int max_ctx,
                        size_t* bytes);

/* ---- sequence --------------------------------------------------------------- */

/* Creates a sequence over a caller-owned KV pool and workspace.
 *   page_table_host[n_logical_pages]: logical page i (positions
 *   i*page_size .. (i+1)*page_size-1) lives in physical pool page
 *   page_table_host[i] (each < n_pages).  Copied to the workspace (synchronous).
 *   page_size: 16, 32 or 64.  The sequence starts empty (kvlen 0). */
int ssd_seq_create(const ssd_model* model, void* kv_pool_dev, int n_pages, int page_size,
                   const int32_t* page_table_host, int n_logical_pages, void* workspace_dev,
                   size_t workspace_bytes, int max_rows, int max_draft, hipStream_t stream,
                   ssd_seq** out_seq);
int ssd_seq_destroy(ssd_seq* seq);

/* Prefill (row a7): the n prompt tokens tokens_dev[0..n-1] at positions 0..n-1
 * through the full model (in chunks of min(max_rows, 1024) rows); then the first
 * generated token is picked from the last row's logits (argmax at temperature
 * 0, else a draw with iteration 0) and committed.  After it: kvlen = n,
 * n_out = 1.  last_logits_dev[V] (nullable) receives the last row's logits. */
int ssd_prefill(ssd_seq* seq, const int32_t* tokens_dev, int n, float temperature, uint64_t seed,
                float* last_logits_dev, hipStream_t stream);

/* One plain autoregressive step with the full model (row a7; the lossless
 * reference of [SWIFT] §2): feeds last_token at position kvlen, picks the next
 * token (argmax, or a draw addressed by the current iteration) and commits it.
 * logits_dev[V] (nullable) receives the logits. */
int ssd_decode_ar(ssd_seq* seq, float temperature, uint64_t seed, float* logits_dev,
                  hipStream_t stream);

/* Lossy early-exit decoding (next row f4; [LayerSkip] §3 first mode, §4): one step as ssd_decode_ar
 * but through the plan's sub-layers only (skip_mask_host[2L], or exit_layer E when it is NULL) and the
 * shared final norm and LM head; the token is committed without verification.  Keys and values are
 * written for the kept sub-layers only (later steps of the same plan read nothing else).  The prompt is
 * prefilled by ssd_prefill with the full model. */
int ssd_decode_exit(ssd_seq* seq, const uint8_t* skip_mask_host, int exit_layer, float temperature,
                    uint64_t seed, float* logits_dev, hipStream_t stream);

/* Draft phase (row a1; [LayerSkip] §3.1, [SWIFT] §3.1 and §4.2).
 * Plan: skip_mask_host[2L] (entry 2l = skip the attention sub-layer of layer
 * l, entry 2l+1 = skip its MLP sub-layer; [SWIFT] Appendix A Fig. 10), or, when
 * skip_mask_host is NULL, exit_layer E in 0..L: run layers 0..E-1 only.
 * Step j = 1..d feeds y_{j-1} (y_0 = last_token) at position kvlen + j - 1
 * through the kept sub-layers (writing their K/V at that position), the shared
 * final norm and LM head; y_j = argmax (temperature 0) or a draw from
 * softmax(z / T) (purpose "draft"); conf_j = max softmax.  Drafting stops after
 * step j when conf_j < conf_thresh or j = d; d' = j.
 * With conf_thresh <= 0 no step can stop early: all d steps are enqueued and
 * the call returns at once.  With conf_thresh > 0 the call waits after each
 * step j < d for the stop decision (it synchronises the stream and reads 4
 * bytes) and enqueues no later step once drafting has stopped, so a stopped
 * draft costs no further launches; such a call cannot be captured into a HIP
 * graph.
 * Outputs: draft_tokens_dev[d] (first d' valid), draft_logits_dev[d * V]
 * (rows 0..d'-1 valid: the q logits), n_drafted_dev[1] = d'.
 * Also saves, for each step, the residual entering the reuse boundary b (the
 * first layer with a skipped sub-layer) for ssd_verify. */
int ssd_draft(ssd_seq* seq, const uint8_t* skip_mask_host, int exit_layer, int d, float conf_thresh,
              float temperature, uint64_t seed, int32_t* draft_tokens_dev, float* draft_logits_dev,
              int32_t* n_drafted_dev, hipStream_t stream);

/* Verify pass (row a2; [LayerSkip] §3.2).  Rows i = 0..d' carry y_0..y_d' at
 * positions kvlen + i.  With reuse != 0 only row d' runs the layers below the
 * plan's boundary b; rows < d' take the residual the draft saved there (the
 * draft's keys/values below b are the full model's).  With reuse == 0 every
 * row runs every layer.  Layers >= b run in full for all rows, overwriting the
 * draft's keys/values; attention is causal inside the block.
 * The plan must be the one of the preceding ssd_draft; d is its d.
 * Output: logits_dev[(d + 1) * V]; rows 0..d' valid; row i is the full model's
 * logits for position kvlen + i + 1. */
int ssd_verify(ssd_seq* seq, const uint8_t* skip_mask_host, int exit_layer, int d,
               const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev, int reuse,
               float* logits_dev, hipStream_t stream);

/* Accept / reject (row a4; [LayerSkip] §3.3).
 * Temperature 0: k = number of leading drafts equal to the argmax of the
 * corresponding verify row; emits y_1..y_k then argmax of verify row k.
 * Temperature T > 0: p_i = softmax(p_logits row i-1 / T), q_i = softmax(q row
 * i-1 / T); y_i is accepted when u_i * q_i(y_i) < p_i(y_i) (u_i uniform,
 * purpose "accept"), taken as log u + log q < log p in float32; at the first
 * rejection a draw from norm(max(0, p_i - q_i)) (purpose "sample", row i-1) is
 * emitted; when all d' are accepted a bonus draw from p_{d'+1} (row d').
 * Outputs: out_tokens_dev[d + 1] (first n_out valid), n_out_dev[1] = k + 1.
 * A verify row 0..d' or draft row with NaN or +inf logits decides nothing:
 * n_out = 0 and the sequence's numeric flag is raised (ssd_read_state returns
 * SSD_ERR_NUMERIC).  Does not change the sequence otherwise (see ssd_commit). */
int ssd_accept(ssd_seq* seq, const float* p_logits_dev, const float* q_logits_dev,
               const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev, int d, float temperature,
               uint64_t seed, int32_t* out_tokens_dev, int32_t* n_out_dev, hipStream_t stream);

/* Allocation-free acceptance, for callers that cannot allocate device memory
 * or hand over a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the rule and the random draws of
 * ssd_accept, without a sequence.  p_logits_dev [d + 1, vocab],
 * q_logits_dev [d, vocab] (fp32, row-major), draft_tokens_dev [d] and
 * n_drafted_dev[1] (d' in 1..d; values outside 0..d are clamped) are as in
 * ssd_accept; iteration addresses the draws (a sequence's iteration counter
 * reproduces ssd_accept's draws exactly).  Outputs: out_tokens_dev[d + 1]
 * (first n_out valid), n_out_dev[1]; n_out = 0 when a row holds NaN or +inf
 * logits.
 * Scratch: the per-row decisions and draws passed between the two kernels sit
 * in a library-owned device array of 2 x (SSD_ACCEPT_NOALLOC_MAX_DRAFT + 1)
 * int32 per GPU, created with the library's code object and held until the
 * process ends; the call itself allocates nothing.  Every call on one GPU
 * shares that array: calls that overlap on one GPU (e.g. on two streams) race
 * and must be ordered by the caller.  d > SSD_ACCEPT_NOALLOC_MAX_DRAFT returns
 * SSD_ERR_CAPACITY. */
#define SSD_ACCEPT_NOALLOC_MAX_DRAFT 32
int ssd_accept_noalloc(const float* p_logits_dev, const float* q_logits_dev, const int32_t* draft_tokens_dev,
                       const int32_t* n_drafted_dev, int d, int vocab, float temperature, uint64_t seed,
                       int32_t iteration, int32_t* out_tokens_dev, int32_t* n_out_dev, hipStream_t stream);

/* Commit (row a5): appends out_tokens_dev[0..n_out-1] to the output log,
 * kvlen += n_out, last_token = the last emitted token, iteration += 1.  Keys and
 * values at positions >= the new kvlen are dead (rejected drafts) and are
 * overwritten by later steps: roll-back is this metadata update only.
 * n_out = 0 commits nothing (iteration += 1); n_out < 0 or > max_draft + 1
 * commits nothing and raises the input flag (ssd_read_state: SSD_ERR_ARG). */
int ssd_commit(ssd_seq* seq, const int32_t* out_tokens_dev, const int32_t* n_out_dev,
               hipStream_t stream);

/* ---- draft trees: dynamic verification ([SWIFT] §4.2, §3.2.1 Figure 2) ------
 * The draft's confidence also sets how many candidates each draft step hands to
 * the verification.  Readings (the page gives no formula): the candidates of
 * step j are the k_j most probable tokens of softmax(q logits row j-1)
 * (temperature 1, lowest index first among equal logits), k_j = the least k >= 1
 * whose top-k mass reaches rho, at most k_max; only the top one (the greedy
 * draft token y_j) is drafted further, the others are leaves of depth j that sit
 * at y_j's position and attend to the prefix, y_0..y_{j-1} and themselves.
 * At temperature T > 0 the top-k tokens are not draws of q, so the leaves of step
 * j are k_j - 1 further independent draws of softmax(z_j / T) (k_j from the same
 * rule at T), and acceptance is the multi-candidate form of the speculative
 * sampling rule (SpecInfer, Miao et al.), which keeps the target distribution
 * for drawn candidates. */

/* Leaves of the last draft (draft_logits_dev / n_drafted_dev as written by
 * ssd_draft with the same temperature, or any [d, V] float rows).  Temperature 0:
 * ranks 1..k_j-1 of each step j <= d'.  T > 0: k_j - 1 draws of softmax(row / T)
 * (race keys z / T + Gumbel; Philox counter (iteration, (j - 1) + 256 r,
 * purpose 4 "leaf", v / 4) for the r-th extra draw, the iteration read from the
 * sequence's device state).  Depth order, then rank (draw) order, at most
 * max_leaves (<= 15).  k_max in 1..8, d <= 256.
 * Outputs: leaf_tokens_dev[max_leaves], leaf_depth_dev[max_leaves] (1..d'),
 * n_leaves_dev[1]. */
int ssd_tree_candidates(ssd_seq* seq, const float* draft_logits_dev, const int32_t* n_drafted_dev, int d,
                        float temperature, uint64_t seed, float rho, int k_max, int max_leaves,
                        int32_t* leaf_tokens_dev, int32_t* leaf_depth_dev, int32_t* n_leaves_dev,
                        hipStream_t stream);

/* Tree verify: ssd_verify's chain rows 0..d' plus one row per leaf s (token
 * leaf_tokens_dev[s] at position kvlen + leaf_depth_dev[s], seeing the cache up
 * to the position before its own and its own key/value).  The leaves' keys and
 * values are kept in the workspace; the cache receives only the chain's.  With
 * reuse, y_d' and the leaves run the layers below the plan's boundary, the
 * chain rows < d' take the draft's saved residual (as ssd_verify).
 * Requires a bf16 model, d + 1 + max_leaves <= 16 (and <= max_rows), and a
 * context of at most 63 * 64 positions (the attention's merge slots).
 * Output: logits_dev[(d + 1 + max_leaves) * V], rows compact: 0..d' the chain
 * (bitwise the rows ssd_verify gives), d' + 1 + s leaf s (the full model's
 * logits for the position after the leaf). */
int ssd_verify_tree(ssd_seq* seq, const uint8_t* skip_mask_host, int exit_layer, int d,
                    const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev, const int32_t* leaf_tokens_dev,
                    const int32_t* leaf_depth_dev, const int32_t* n_leaves_dev, int max_leaves, int reuse,
                    float* logits_dev, hipStream_t stream);

/* Tree acceptance over ssd_verify_tree's rows (logits_dev; q_logits_dev: the
 * draft's logits, needed at T > 0).
 * Temperature 0: for j = 1..d', y_j is accepted while it is the argmax of chain
 * row j-1; at the first mismatch, if the argmax is a leaf of depth j, that leaf
 * and the argmax of its own row are emitted, else the argmax alone; after d'
 * accepted drafts the argmax of row d' is the bonus.
 * T > 0: the chain rule of ssd_accept per depth; at the first rejected depth j
 * that has leaves, the leaves are tried in order: with p' the target after the
 * rejections so far (p' <- norm(max(0, p' - q_j)) after each, kept when that is
 * all zero), leaf c (the k-th candidate of the depth, the draft token being the
 * 0-th) is accepted when u q_j(c) < p'(c) (u: counter (iteration, (j - 1) + 256 k,
 * "accept")), and then emitted with a draw from its own row (counter
 * (iteration, (j - 1) + 256 k, "sample")); when all are rejected, a draw from the
 * last nonzero max(0, p' - q_j) (or p_j) with the chain rule's counter.  Without
 * leaves this is ssd_accept's rule draw for draw.
 * When a leaf is emitted its keys and values (every layer) are written into the
 * cache at its position, so ssd_commit's metadata update is all that remains.
 * Outputs: out_tokens_dev[d + 1] (first n_out valid), n_out_dev[1]. */
int ssd_accept_tree(ssd_seq* seq, const float* logits_dev, const float* q_logits_dev,
                    const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev, int d,
                    const int32_t* leaf_tokens_dev, const int32_t* leaf_depth_dev, const int32_t* n_leaves_dev,
                    int max_leaves, float temperature, uint64_t seed, int32_t* out_tokens_dev, int32_t* n_out_dev,
                    hipStream_t stream);

/* SWIFT matchness scoring (row a6; [SWIFT] §4.1, §4.1.2, §5.3, §D.2).
 * window_dev[gamma + 1] are committed tokens at positions pos0..pos0+gamma, and
 * the cache must hold the full model's keys/values for positions < pos0
 * (pos0 <= kvlen).  For each candidate plan c (masks_host[c * 2L .. +2L]) one
 * causal draft forward runs rows window[0..gamma-1] at positions pos0.. with
 * the candidate's own keys/values at the window positions (kept in the
 * workspace; the cache is not modified); row i predicts argmax of its logits.
 * scores_dev[c] = #(prediction i == window[i+1]) / gamma; best_dev[0] = the
 * highest-scoring candidate (lowest index on ties); row_pred_dev (nullable)
 * [n_masks * gamma] receives each row's prediction (candidate-major).
 * Candidates whose plans agree on the sub-layers before a sub-layer share its
 * computation (it runs once for them); each candidate's results are those it
 * gets when scored alone, bit for bit.
 * Requires n_masks * gamma <= max_rows. */
int ssd_score_masks(ssd_seq* seq, const uint8_t* masks_host, int n_masks, const int32_t* window_dev,
                    int pos0, int gamma, float* scores_dev, int32_t* best_dev, int32_t* row_pred_dev,
                    hipStream_t stream);

/* ---- SWIFT layer-set search (next row f1; [SWIFT] §1, §4.1.1, §4.1.2, §5.3, §B.2) ----
 * The pages' optimisation phase proposes candidate layer sets by random search
 * (with a periodic Bayesian step: bo_every below), scores them by
 * matchness on the last context window and keeps the best, stopping at a step
 * limit, after a run of steps without improvement, or above a matchness target.
 * Readings: candidates skip n_skip whole layers (both bits of a layer) or, with
 * sublayers != 0, n_skip of the 2L attention / MLP sub-layers ([SWIFT] Appendix
 * A Fig. 10); a step proposes n_cand uniformly random such sets; the incumbent is
 * replaced by the best proposal of a step (lowest index on ties) only when its
 * score is strictly higher; the uniform starting plan skips layers
 * floor((2 i + 1) L / (2 n_skip)), i = 0..n_skip-1.  Host-only helpers below
 * make no device call. */

/* mask_host[2L] = the uniform plan skipping n_skip of n_layers layers (0 <= n_skip <= n_layers). */
int ssd_uniform_mask(int n_layers, int n_skip, uint8_t* mask_host);

/* mask_host[2L] = proposal `cand` of search step `step`: a Fisher-Yates draw of n_skip of the N items
 * (sublayers == 0: the N = L layers, both bits of a drawn layer set; otherwise the N = 2L sub-layers, bit i
 * for item i), position i taking (x_i * (N - i)) >> 32 from the Philox word x_i at key seed, counter
 * (step, cand, 3, i / 4), word i % 4 (the sampling draws' generator; purpose 3 = proposal). */
int ssd_swift_propose(int n_layers, int n_skip, int sublayers, uint64_t seed, int step, int cand,
                      uint8_t* mask_host);

/* Random search on the window (same contract as ssd_score_masks: window_dev[gamma + 1] committed tokens
 * at positions pos0.., the cache holding the full model's keys/values before pos0); proposals as
 * ssd_swift_propose with the same sublayers flag.  Step t scores its
 * n_cand proposals (step 0 also the starting plan init_mask_host) in one batched scoring pass; the
 * search stops after max_steps steps, after `patience` consecutive steps without improvement, or as
 * soon as the incumbent's score exceeds `target`.  Every bo_every-th step (t > 0; 0 = never) is a
 * Bayesian-optimisation step ([SWIFT] §4.1.2 "periodic Bayesian optimization", §B.2 every 25 steps):
 * a Gaussian process over the mask vectors of the most recent 256 scored plans (scores standardised,
 * kernel exp(-|x - x'|^2 / (2 l^2)) with l^2 = the number of skipped entries, unit signal variance,
 * 1e-6 noise; double precision on the host) ranks a pool of 8 * n_cand proposals (candidates
 * 0..8 n_cand - 1 of the step's counter) by expected improvement over the incumbent, and the n_cand
 * best (lower pool index first among equal values) are scored, best first; when every score seen
 * so far is equal the step proposes at random.  Requires (n_cand + 1) * gamma <= max_rows and
 * n_cand + 1 <= 64.  Random proposals do not depend on earlier scores, so a step and the random steps
 * after it (up to the next Bayesian step, as many as max_rows / gamma window rows hold) are scored in
 * one batched pass and then applied in order; a stop drops the later steps' scores.  The results are
 * those of one pass per step, bit for bit.  Out: best_mask_host[2L] (the incumbent), *best_score,
 * *n_steps (the steps applied).  Synchronises the stream once per scoring pass. */
int ssd_swift_search(ssd_seq* seq, const int32_t* window_dev, int pos0, int gamma, const uint8_t* init_mask_host,
                     int n_skip, int sublayers, int n_cand, int max_steps, int patience, float target, uint64_t seed,
                     int bo_every, uint8_t* best_mask_host, float* best_score, int* n_steps, hipStream_t stream);

/* ---- SWIFT on the fly (next row f1; [SWIFT] §4, §4.1.1, §4.1.2, §5.3, §B.2, §D.2) ----
 * Generation alternates self-speculative iterations (ssd_draft, ssd_verify with reuse, ssd_accept,
 * ssd_commit) with the plan in use and optimisation phases (steps of ssd_swift_search) on the most recent
 * context window.  Readings (the pages name the phases and their stopping rules, not the schedule between
 * them): a phase runs once `accumulate` tokens (<= 0: gamma) have been committed since the previous phase
 * (the first: since ssd_swift_begin), optimisation is not over and at least gamma + 1 tokens have been
 * generated; its window is the last gamma + 1 committed tokens (the newest at position kvlen).  The phase
 * is ssd_swift_search with the plan in use as the starting incumbent (scored afresh on the window), at most
 * steps_per_phase steps numbered on from the earlier phases (proposal counters and the Bayesian schedule
 * bo_every count every phase's steps; the Gaussian process sees the current phase's plans), and the run of
 * unimproved steps carried over.  The plan becomes the phase's final incumbent (a different plan only when
 * a proposal scored strictly higher on the window).  Optimisation ends for good once max_steps steps have
 * run in all, once the unimproved run reaches patience, or once a phase ends with a score above target;
 * generation goes on with the last plan.  The pages' settings: gamma 32, max_steps 1000, patience 300,
 * target 0.95, bo_every 25.  With accumulate = steps_per_phase = 1 the window slides: one optimisation
 * step after every iteration. */
typedef struct ssd_swift_config {
  int32_t gamma;             /* window: tokens each candidate predicts */
  int32_t accumulate;        /* committed tokens between phases (<= 0: gamma) */
  int32_t n_skip, sublayers; /* candidate size, as ssd_swift_propose */
  int32_t n_cand;            /* proposals per step; (n_cand + 1) * gamma <= max_rows, n_cand + 1 <= 64 */
  int32_t steps_per_phase;   /* >= 1 */
  int32_t max_steps;         /* in all phases; 0 = never optimise */
  int32_t patience;          /* >= 1 */
  float target;
  int32_t bo_every;          /* 0 = no Bayesian steps */
  int32_t d;                 /* drafts per iteration, 1..max_draft */
  float conf_thresh, temperature;
  uint64_t seed;             /* the proposals' and the iterations' draws */
} ssd_swift_config;

typedef struct ssd_swift_state {
  int32_t steps;             /* optimisation steps run so far */
  int32_t unimproved;        /* the current run of steps without improvement */
  int32_t done;              /* 1: optimisation is over */
  int32_t last_phase_n_out;  /* n_out when the last phase ran (at ssd_swift_begin: the n_out then) */
  int32_t phases, switches;  /* phases run, and how many of them changed the plan */
  float score;               /* the plan's matchness on the last phase's window (NaN before the first) */
  int32_t iterations;        /* self-speculative iterations run by ssd_swift_generate */
} ssd_swift_state;

/* Starts the controller on a prefilled sequence: *state = no steps, no phases, windows counted from the
 * sequence's current n_out (the call synchronises the stream to read it); done = 1 when max_steps is 0.
 * The starting plan is the caller's plan_host[2L] (e.g. ssd_uniform_mask). */
int ssd_swift_begin(ssd_seq* seq, const ssd_swift_config* cfg, ssd_swift_state* state, hipStream_t stream);

/* Runs iterations with plan_host[2L] (in: the plan in use; out: the plan after the last phase) until at
 * least n_tokens more tokens are committed (an iteration commits 1..d + 1), with the phases above in
 * between; *state is updated.  The iterations' buffers are the caller's, as in ssd_draft / ssd_verify /
 * ssd_accept: draft_tokens_dev[d], draft_logits_dev[d * V], n_drafted_dev[1], verify_logits_dev[(d + 1) * V],
 * out_tokens_dev[d + 1], n_out_dev[1].  Synchronises the stream after every iteration (4-byte state read:
 * the committed count decides when a phase is due) and once per optimisation step.  An iteration that
 * commits nothing (non-finite logits) ends the call with SSD_ERR_NUMERIC. */
int ssd_swift_generate(ssd_seq* seq, const ssd_swift_config* cfg, ssd_swift_state* state, uint8_t* plan_host,
                       int n_tokens, int32_t* draft_tokens_dev, float* draft_logits_dev, int32_t* n_drafted_dev,
                       float* verify_logits_dev, int32_t* out_tokens_dev, int32_t* n_out_dev, hipStream_t stream);

/* SpecEE exit features (next row f4; [SpecEE] §4.3.1) of rows hidden states h_dev [rows][D] (fp32, a
 * layer's output in the residual stream) for k speculative tokens tokens_dev[k] (1 <= k <= 16):
 * features_dev[r][0..k) = speculative-token logits z_j = bf16(h * g_final) . W_lm[t_j] / rms(h) (the shared
 * final norm and LM head restricted to the k columns, with the LM head's own rounding points),
 * [k..2k) = local probabilities softmax(z) over the k tokens, [2k..3k) = their variation against the
 * previous layer's, prev_probs_dev[r][k] (0 when it is NULL).  The trained exit predictor that
 * consumes them is not part of this library. */
int ssd_specee_features(const ssd_model* model, const float* h_dev, int rows, const int32_t* tokens_dev, int k,
                        const float* prev_probs_dev, float* features_dev, hipStream_t stream);

/* Row statistics (row a3) of rows logits rows of length V, as used inside
 * draft/verify/accept; exposed for tests.  Draws use (seed, iteration, row
 * index, purpose "draft"). */
int ssd_row_stats(const float* logits_dev, int rows, int V, float temperature, uint64_t seed,
                  int32_t iteration, ssd_row_stat* stats_dev, hipStream_t stream);

/* ---- host synchronisation ------------------------------------------------------ */

/* Waits for the stream, then copies the device state.  Returns
 * SSD_ERR_CAPACITY / SSD_ERR_NUMERIC / SSD_ERR_ARG if the device flagged such a
 * condition (SSD_ERR_ARG: a device-side argument out of range, e.g. a leaf depth
 * outside 1..d'). */
int ssd_read_state(ssd_seq* seq, ssd_state* out, hipStream_t stream);

/* Waits for the stream, then copies min(n_out, max_tokens) committed tokens
 * of the output log to tokens_host; *n_tokens = that count. */
int ssd_read_output(ssd_seq* seq, int32_t* tokens_host, int max_tokens, int* n_tokens,
                    hipStream_t stream);

/* Thread-local message describing this thread's last failure ("" if none). */
const char* ssd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SSD_H */
