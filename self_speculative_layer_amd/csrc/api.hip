// C ABI of the self-speculative decoding library: model and sequence handles,
// workspace carving, and the launch sequences of draft / verify / accept /
// commit / prefill / AR decode / matchness scoring.  All per-iteration values
// (positions, tokens, draft length) are read by the kernels from the
// sequence's device state, so a whole iteration is enqueued without any
// device-to-host traffic.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <string>
#include <unordered_set>
#include <limits>
#include <vector>

#include "kernels.h"

using namespace ssd;

// ---------------------------------------------------------------------------
// errors

static thread_local std::string g_err;

static int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define CHECK_ARG(cond, msg) \
  do {                       \
    if (!(cond)) return fail(SSD_ERR_ARG, msg); \
  } while (0)

#define TRY(expr)                                                              \
  do {                                                                         \
    int _rc = (expr);                                                          \
    if (_rc != 0) return fail(_rc, std::string("launch failed: ") + #expr);    \
  } while (0)

extern "C" const char* ssd_last_error(void) { return g_err.c_str(); }

// ---------------------------------------------------------------------------
// live handles: every entry point checks that the handle it is given was created here and not destroyed

static std::mutex g_handles_mu;
static std::unordered_set<const void*> g_models, g_seqs;

static bool is_live(const std::unordered_set<const void*>& set, const void* h) {
  std::lock_guard<std::mutex> lock(g_handles_mu);
  return set.count(h) != 0;
}

#define CHECK_MODEL(m)                                                                                   \
  do {                                                                                                   \
    if (!(m)) return fail(SSD_ERR_ARG, "null model handle");                                             \
    if (!is_live(g_models, (m))) return fail(SSD_ERR_ARG, "not a live model handle (destroyed or never created)"); \
  } while (0)

#define CHECK_SEQ(q)                                                                                     \
  do {                                                                                                   \
    if (!(q)) return fail(SSD_ERR_ARG, "null sequence handle");                                          \
    if (!is_live(g_seqs, (q))) return fail(SSD_ERR_ARG, "not a live sequence handle (destroyed or never created)"); \
  } while (0)

int ssd::set_last_error(int code, const char* msg) { return fail(code, msg); }

// ---------------------------------------------------------------------------
// handles

struct ssd_model {
  ssd_model_desc d;
  std::vector<ssd_layer_weights> layers;
  int q_dim, kv_dim, qkv_dim;
  size_t elt;
};

struct Workspace {
  DevState* st;
  int* page_table;
  float2* rope_cs;
  int *pos, *tok, *pos1, *tok1, *vpos, *vtok;
  float *h, *h1, *qkv, *part, *hb, *logits1, *logits_rows, *inv;
  void *x, *x2, *qb, *local_kv;
  ssd_row_stat* stats;
  int *dec, *corr, *rowmaps;
  int32_t* log;
  // decode blocks (<= 16 rows)
  float* xg;             // next RMSNorm consumer's input h * g (fp32), decode block layout [16][max(D, q_dim)]
  float* ss;             // its 16-feature tile sums of h^2 [16][D / 16]
  unsigned* dec_ctr;     // attention merge counters [16][KVH], zero between launches
  StatRec* stat_recs;    // row statistics: segment records [rows][segments]
  unsigned* stat_ctr;    //   and per-row counters, zero between launches
  float* gemm_split;     // quarter sums of K-split projections [4][R][D]
  float* swift_scores;   // layer-set search: the scores of one scoring pass [max(64, R)]
  int32_t* swift_best;   //   and its best index
  // draft trees
  bf16_t* tree_kv;       // leaves' keys and values [L][TREE_SLOTS][2][KVH * HD] (not in the cache)
  float* hp;             // prefix-block residual rows [16][D] (y_d' and the leaves below the boundary)
  int *tvpos, *tvtok;    // full-block rows [16]
  int *ppos, *ptok;      // prefix-block rows [16]
  int *tree_cand, *tree_k;   // per draft row: best tokens [max_draft][TREE_KMAX], candidate count
};

struct ssd_seq {
  const ssd_model* m;
  KvView kv;
  int max_rows, max_draft, max_ctx, log_cap;
  Workspace w;
};

namespace {

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// Carves the workspace; with base == nullptr only computes the size.
size_t carve(const ssd_model* m, int max_rows, int max_draft, int max_ctx, char* base, Workspace* w) {
  const ssd_model_desc& d = m->d;
  const int R = max_rows, D = d.d_model, F = d.ffn_dim, V = d.vocab, L = d.n_layers;
  const int xw = std::max(D, m->q_dim);
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  };
  Workspace t{};
  t.st = (DevState*)take(sizeof(DevState));
  t.page_table = (int*)take(sizeof(int) * (size_t)((max_ctx + 15) / 16 + 1));
  t.rope_cs = (float2*)take(sizeof(float2) * (size_t)max_ctx * (d.head_dim / 2));
  t.pos = (int*)take(sizeof(int) * R);
  t.tok = (int*)take(sizeof(int) * R);
  t.pos1 = (int*)take(sizeof(int) * 4);
  t.tok1 = (int*)take(sizeof(int) * 4);
  t.vpos = (int*)take(sizeof(int) * (max_draft + 1));
  t.vtok = (int*)take(sizeof(int) * (max_draft + 1));
  t.h = (float*)take(sizeof(float) * (size_t)R * D);
  t.h1 = (float*)take(sizeof(float) * D);
  t.inv = (float*)take(sizeof(float) * R);
  t.qkv = (float*)take(sizeof(float) * (size_t)R * m->qkv_dim);
  t.part = (float*)take(sizeof(float) * attention_partial_floats(std::min(R, SPLIT_ATTN_MAX_ROWS), d.n_heads,
                                                                 d.head_dim, max_ctx));
  t.hb = (float*)take(sizeof(float) * (size_t)max_draft * D);
  t.logits1 = (float*)take(sizeof(float) * V);
  t.logits_rows = (float*)take(sizeof(float) * (size_t)R * V);
  // (decode blocks use these two in the 16-row block layout)
  t.x = take(m->elt * (size_t)std::max(R, 16) * xw);
  t.x2 = take(m->elt * (size_t)std::max(R, 16) * F);
  t.qb = take(m->elt * (size_t)R * m->q_dim);
  t.local_kv = take(m->elt * (size_t)R * 2 * m->kv_dim);
  t.stats = (ssd_row_stat*)take(sizeof(ssd_row_stat) * R);
  t.dec = (int*)take(sizeof(int) * (max_draft + 1));
  t.corr = (int*)take(sizeof(int) * (max_draft + 1));
  t.rowmaps = (int*)take(sizeof(int) * ((size_t)2 * L * R + 4 * (size_t)R));   // row lists + copy pairs
  t.log = (int32_t*)take(sizeof(int32_t) * (size_t)max_ctx);
  t.xg = (float*)take(sizeof(float) * (size_t)16 * std::max(D, m->q_dim));
  t.ss = (float*)take(sizeof(float) * (size_t)16 * (D / 16 + 1));
  t.dec_ctr = (unsigned*)take(sizeof(unsigned) * (size_t)16 * d.n_kv_heads);
  t.stat_recs = (StatRec*)take(sizeof(StatRec) * (size_t)R * stat_segments(V));
  t.stat_ctr = (unsigned*)take(sizeof(unsigned) * (size_t)R);
  t.gemm_split = (float*)take(sizeof(float) * 4 * (size_t)R * D);
  t.swift_scores = (float*)take(sizeof(float) * std::max(64, R));
  t.swift_best = (int32_t*)take(sizeof(int32_t) * 4);
  t.tree_kv = (bf16_t*)take(2 * (size_t)L * TREE_SLOTS * 2 * m->kv_dim);
  t.hp = (float*)take(sizeof(float) * 16 * (size_t)D);
  t.tvpos = (int*)take(sizeof(int) * 16);
  t.tvtok = (int*)take(sizeof(int) * 16);
  t.ppos = (int*)take(sizeof(int) * 16);
  t.ptok = (int*)take(sizeof(int) * 16);
  t.tree_cand = (int*)take(sizeof(int) * (size_t)max_draft * TREE_KMAX);
  t.tree_k = (int*)take(sizeof(int) * (size_t)max_draft);
  if (w) *w = t;
  return off;
}

// A block of rows whose residuals live in h (row i of the block at residual
// row hmap[i], or i).
struct Block {
  float* h;
  RowBlock rb;            // rb.ymap doubles as hmap for the residual stream
  void* local_kv;         // scoring: the candidates' own keys/values
  int local_start;
  int group_rows;
};

int attn_sublayer(ssd_seq* q, int l, const Block& b, hipStream_t s) {
  const ssd_model* m = q->m;
  const ssd_model_desc& d = m->d;
  const ssd_layer_weights& lw = m->layers[l];
  const Workspace& w = q->w;
  const RowBlock& rb = b.rb;
  const int D = d.d_model;
  TRY(launch_rowprep(d.dtype, b.h, D, lw.attn_norm, w.x, D, w.inv, rb.M, D, d.rms_eps, rb.nrows, rb.ymap, rb.stop,
                     s));
  TRY(launch_linear(d.dtype, EPI_STORE, lw.w_qkv, w.x, D, rb.M, m->qkv_dim, D, w.qkv, m->qkv_dim, nullptr, 0,
                    nullptr, rb.nrows, nullptr, rb.stop, s));
  TRY(launch_rope_kv(d.dtype, d.head_dim, w.qkv, m->qkv_dim, w.qb, m->q_dim, q->kv, d.n_layers, l, d.n_heads,
                     d.n_kv_heads, rb, w.rope_cs, b.local_kv, &w.st->error_flags, s));
  TRY(launch_attention(d.dtype, d.head_dim, w.qb, m->q_dim, q->kv, d.n_layers, l, d.n_heads, d.n_kv_heads, rb,
                       q->max_ctx, b.local_kv, b.local_start, b.group_rows, w.part, w.x, m->q_dim, s));
  TRY(launch_linear(d.dtype, EPI_RESID, lw.w_o, w.x, m->q_dim, rb.M, D, m->q_dim, b.h, D, nullptr, 0, nullptr,
                    rb.nrows, rb.ymap, rb.stop, s, w.gemm_split, 4 * (size_t)q->max_rows * D));
  return 0;
}

int mlp_sublayer(ssd_seq* q, int l, const Block& b, hipStream_t s) {
  const ssd_model* m = q->m;
  const ssd_model_desc& d = m->d;
  const ssd_layer_weights& lw = m->layers[l];
  const Workspace& w = q->w;
  const RowBlock& rb = b.rb;
  const int D = d.d_model, F = d.ffn_dim;
  TRY(launch_rowprep(d.dtype, b.h, D, lw.mlp_norm, w.x, D, w.inv, rb.M, D, d.rms_eps, rb.nrows, rb.ymap, rb.stop,
                     s));
  TRY(launch_linear(d.dtype, EPI_SWIGLU, lw.w_gate_up, w.x, D, rb.M, F, D, nullptr, 0, w.x2, F, nullptr, rb.nrows,
                    nullptr, rb.stop, s));
  TRY(launch_linear(d.dtype, EPI_RESID, lw.w_down, w.x2, F, rb.M, D, F, b.h, D, nullptr, 0, nullptr, rb.nrows,
                    rb.ymap, rb.stop, s, w.gemm_split, 4 * (size_t)q->max_rows * D));
  return 0;
}

bool skip_attn(const uint8_t* mask, int l) { return mask && mask[2 * l]; }
bool skip_mlp(const uint8_t* mask, int l) { return mask && mask[2 * l + 1]; }

int run_layers(ssd_seq* q, const Block& b, int l0, int l1, const uint8_t* mask, hipStream_t s) {
  for (int l = l0; l < l1; ++l) {
    if (!skip_attn(mask, l)) TRY(attn_sublayer(q, l, b, s));
    if (!skip_mlp(mask, l)) TRY(mlp_sublayer(q, l, b, s));
  }
  return 0;
}

// Final RMSNorm + LM head of M rows of h into logits [M, V].
int final_logits(ssd_seq* q, const float* h, int M, const int* nrows, float* logits, const int* stop,
                 hipStream_t s) {
  const ssd_model* m = q->m;
  const ssd_model_desc& d = m->d;
  TRY(launch_rowprep(d.dtype, h, d.d_model, d.final_norm, q->w.x, d.d_model, q->w.inv, M, d.d_model, d.rms_eps,
                     nrows, nullptr, stop, s));
  TRY(launch_linear(d.dtype, EPI_STORE, d.lm_head, q->w.x, d.d_model, M, d.vocab, d.d_model, logits, d.vocab,
                    nullptr, 0, nullptr, nrows, nullptr, stop, s));
  return 0;
}

// The plan as a mask of 2L entries (exit_layer -> suffix mask).  Returns the
// reuse boundary b, or -1 on a bad plan.
int plan_mask(const ssd_model* m, const uint8_t* mask_in, int exit_layer, std::vector<uint8_t>& mask) {
  const int L = m->d.n_layers;
  mask.assign(2 * L, 0);
  if (mask_in) {
    for (int i = 0; i < 2 * L; ++i) mask[i] = mask_in[i] ? 1 : 0;
  } else {
    if (exit_layer < 0 || exit_layer > L) return -1;
    for (int l = exit_layer; l < L; ++l) mask[2 * l] = mask[2 * l + 1] = 1;
  }
  for (int l = 0; l < L; ++l)
    if (mask[2 * l] || mask[2 * l + 1]) return l;
  return L;
}

// Sub-layer entries of layers [l0, l1) that the plan keeps (mask == nullptr: all).
void plan_entries(std::vector<int>& out, int l0, int l1, const uint8_t* mask) {
  for (int l = l0; l < l1; ++l) {
    if (!(mask && mask[2 * l])) out.push_back(2 * l);
    if (!(mask && mask[2 * l + 1])) out.push_back(2 * l + 1);
  }
}

// ---------------------------------------------------------------------------
// Decode mode: a block of at most 16 rows through a list of sub-layer entries
// (2l: attention of layer l, 2l + 1: its MLP) with the kernels of decode.hip.
// Each residual update also writes the input of the next RMSNorm consumer
// (xg, ss), so the entry list fixes every gain in advance.

bool dec_usable(const ssd_seq* q, int rows) {
  return q->m->d.dtype == SSD_DTYPE_BF16 && rows <= 16;
}

// Gain of the RMSNorm that consumes the residual entering entry e (past the
// end: the final norm when the LM head follows, else none).
const float* dec_gain(const ssd_model* m, const std::vector<int>& ent, size_t e, bool final_lm) {
  if (e < ent.size()) {
    const ssd_layer_weights& lw = m->layers[ent[e] / 2];
    return ent[e] % 2 == 0 ? lw.attn_norm : lw.mlp_norm;
  }
  return final_lm ? m->d.final_norm : nullptr;
}

DecGemm dec_base(const ssd_seq* q, int M, const int* nrows, const int* stop) {
  DecGemm a{};
  a.M = M; a.nrows = nrows; a.stop = stop;
  a.ss = q->w.ss; a.eps = q->m->d.rms_eps;
  return a;
}

// Entries [e0, e1) of ent on the residual rows h[0, M).
// copy_last (nullable): the residual rows after the last entry are also written there.
// side_from (nullable): rows >= *side_from are tree leaves (keys and values in the workspace's tree_kv).
int dec_layers(ssd_seq* q, float* h, int M, const int* nrows, const int* pos, const std::vector<int>& ent, size_t e0,
               size_t e1, bool final_lm, const int* stop, hipStream_t s, float* copy_last = nullptr,
               const int* side_from = nullptr) {
  const ssd_model* m = q->m;
  const ssd_model_desc& d = m->d;
  const Workspace& w = q->w;
  const int D = d.d_model, F = d.ffn_dim;
  for (size_t e = e0; e < e1; ++e) {
    const int l = ent[e] / 2;
    const ssd_layer_weights& lw = m->layers[l];
    DecGemm r = dec_base(q, M, nrows, stop);
    r.Y = h; r.ldy = D; r.N = D;
    r.gain_next = dec_gain(m, ent, e + 1, final_lm);
    r.xg_next = w.xg; r.ss_next = w.ss;
    r.y_copy = e + 1 == e1 ? copy_last : nullptr;
    if (ent[e] % 2 == 0) {
      DecGemm a = dec_base(q, M, nrows, stop);
      a.W = (const bf16_t*)lw.w_qkv; a.N = m->qkv_dim; a.K = D;
      a.Xf = w.xg;
      a.q = (bf16_t*)w.qb; a.ldq = m->q_dim;
      a.pool = (bf16_t*)q->kv.pool; a.page_table = q->kv.page_table; a.PS = q->kv.page_size;
      a.n_lpages = q->kv.n_lpages; a.L = d.n_layers; a.layer = l;
      a.H = d.n_heads; a.KVH = d.n_kv_heads; a.HD = d.head_dim;
      a.pos = pos; a.rope_cs = w.rope_cs; a.err = &w.st->error_flags;
      a.side_from = side_from;
      a.side_kv = side_from ? w.tree_kv + (size_t)l * TREE_SLOTS * 2 * m->kv_dim : nullptr;
      TRY(launch_dec_gemm(DEC_QKV, a, s));
      TRY(launch_attention_dec(d.head_dim, w.qb, m->q_dim, q->kv, d.n_layers, l, d.n_heads, d.n_kv_heads, M, nrows,
                               pos, q->max_ctx, w.part, w.x, m->q_dim, w.dec_ctr, stop, s, side_from, a.side_kv));
      r.W = (const bf16_t*)lw.w_o; r.K = m->q_dim; r.X = (const bf16_t*)w.x;
      TRY(launch_dec_gemm(DEC_RESID, r, s));
    } else {
      DecGemm a = dec_base(q, M, nrows, stop);
      a.W = (const bf16_t*)lw.w_gate_up; a.N = F; a.K = D;
      a.Xf = w.xg;
      a.A = (bf16_t*)w.x2;
      TRY(launch_dec_gemm(DEC_SWIGLU, a, s));
      r.W = (const bf16_t*)lw.w_down; r.K = F; r.X = (const bf16_t*)w.x2;
      TRY(launch_dec_gemm(DEC_RESID, r, s));
    }
  }
  return 0;
}

// LM head of the block's rows (their final-norm input is in xg / ss).
int dec_logits(ssd_seq* q, int M, const int* nrows, float* logits, const int* stop, hipStream_t s) {
  const ssd_model_desc& d = q->m->d;
  DecGemm a = dec_base(q, M, nrows, stop);
  a.W = (const bf16_t*)d.lm_head; a.N = d.vocab; a.K = d.d_model;
  a.Xf = q->w.xg;
  a.Y = logits; a.ldy = d.vocab;
  TRY(launch_dec_gemm(DEC_STORE, a, s));
  return 0;
}

// Rows entering a pass: h[dst] from tokens (embedding) or src rows, with the first consumer's input.
// block_rows: the rows of the block they enter (a one-row block's input is stored row-major).
int dec_entry(ssd_seq* q, const int* tokens, const float* src, int rows, const int* count, const int* dst_off,
              float* h, const float* gain, const int* stop, hipStream_t s, int block_rows) {
  const ssd_model_desc& d = q->m->d;
  TRY(launch_dec_entry(d.embed, tokens, d.vocab, src, rows, count, dst_off, h, d.d_model, gain, q->w.xg,
                       q->w.ss, stop, block_rows, s));
  return 0;
}

}  // namespace

// ---------------------------------------------------------------------------
// model

extern "C" int ssd_model_create(const ssd_model_desc* desc, ssd_model** out_model) {
  CHECK_ARG(desc && out_model, "null argument");
  const ssd_model_desc& d = *desc;
  CHECK_ARG(d.n_layers > 0 && d.d_model > 0 && d.n_heads > 0 && d.n_kv_heads > 0 && d.vocab > 0 && d.ffn_dim > 0,
            "non-positive model dimension");
  if (d.head_dim != 64 && d.head_dim != 128) return fail(SSD_ERR_SHAPE, "head_dim must be 64 or 128");
  if (d.n_heads % d.n_kv_heads != 0) return fail(SSD_ERR_SHAPE, "n_heads must be a multiple of n_kv_heads");
  if (64 / (d.n_heads / d.n_kv_heads) < 1) return fail(SSD_ERR_SHAPE, "more than 64 query heads per KV head");
  if (d.dtype == SSD_DTYPE_BF16 && d.n_heads / d.n_kv_heads > 16)
    return fail(SSD_ERR_SHAPE, "bf16 models: at most 16 query heads per KV head");
  if (d.dtype != SSD_DTYPE_F32 && d.dtype != SSD_DTYPE_BF16) return fail(SSD_ERR_ARG, "bad dtype");
  if (d.dtype == SSD_DTYPE_BF16 &&
      (d.d_model % 64 != 0 || d.ffn_dim % 64 != 0 || (d.n_heads * d.head_dim) % 64 != 0))
    return fail(SSD_ERR_SHAPE, "bf16 models need d_model, ffn_dim and n_heads*head_dim multiples of 64");
  CHECK_ARG(d.embed && d.final_norm && d.lm_head && d.layers, "null weight pointer");
  for (int l = 0; l < d.n_layers; ++l) {
    const ssd_layer_weights& lw = d.layers[l];
    CHECK_ARG(lw.attn_norm && lw.w_qkv && lw.w_o && lw.mlp_norm && lw.w_gate_up && lw.w_down,
              "null layer weight pointer");
  }
  ssd_model* m = new (std::nothrow) ssd_model;
  if (!m) return fail(SSD_ERR_CAPACITY, "out of host memory");
  m->d = d;
  m->layers.assign(d.layers, d.layers + d.n_layers);
  m->d.layers = m->layers.data();
  m->q_dim = d.n_heads * d.head_dim;
  m->kv_dim = d.n_kv_heads * d.head_dim;
  m->qkv_dim = m->q_dim + 2 * m->kv_dim;
  m->elt = d.dtype == SSD_DTYPE_BF16 ? 2 : 4;
  {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    g_models.insert(m);
  }
  *out_model = m;
  return SSD_OK;
}

extern "C" int ssd_packed_bf16_bytes(int N, int K, size_t* bytes) {
  CHECK_ARG(bytes && N > 0 && K > 0, "bad argument");
  if (K % 32 != 0) return fail(SSD_ERR_SHAPE, "K must be a multiple of 32");
  *bytes = (size_t)((N + 15) / 16) * 16 * (size_t)K * 2;
  return SSD_OK;
}

extern "C" int ssd_pack_bf16(const void* src, void* dst, int N, int K, hipStream_t stream) {
  CHECK_ARG(src && dst && N > 0 && K > 0, "bad argument");
  if (K % 32 != 0) return fail(SSD_ERR_SHAPE, "K must be a multiple of 32");
  TRY(launch_pack_bf16(src, dst, N, K, stream));
  return SSD_OK;
}

extern "C" int ssd_model_destroy(ssd_model* model) {
  CHECK_MODEL(model);
  {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    for (const void* h : g_seqs)
      if (((const ssd_seq*)h)->m == model) return fail(SSD_ERR_ARG, "a live sequence still uses this model");
    g_models.erase(model);
  }
  delete model;
  return SSD_OK;
}

extern "C" int ssd_kv_pool_bytes(const ssd_model* m, int n_pages, int page_size, size_t* bytes) {
  CHECK_MODEL(m);
  CHECK_ARG(m && bytes && n_pages > 0 && page_size > 0, "bad argument");
  *bytes = (size_t)n_pages * m->d.n_layers * 2 * m->kv_dim * page_size * m->elt;
  return SSD_OK;
}

extern "C" int ssd_workspace_bytes(const ssd_model* m, int max_rows, int max_draft, int max_ctx, size_t* bytes) {
  CHECK_MODEL(m);
  CHECK_ARG(m && bytes, "null argument");
  CHECK_ARG(max_rows >= 1 && max_rows <= SSD_MAX_ROWS, "max_rows must be in 1..4096");
  CHECK_ARG(max_draft >= 1 && max_draft <= 32, "max_draft must be in 1..32");
  CHECK_ARG(max_ctx >= 1, "max_ctx must be positive");
  *bytes = carve(m, std::max(max_rows, max_draft + 1), max_draft, max_ctx, nullptr, nullptr);
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// sequence

extern "C" int ssd_seq_create(const ssd_model* m, void* kv_pool_dev, int n_pages, int page_size,
                              const int32_t* page_table_host, int n_logical_pages, void* workspace_dev,
                              size_t workspace_bytes, int max_rows, int max_draft, hipStream_t stream,
                              ssd_seq** out_seq) {
  CHECK_MODEL(m);
  CHECK_ARG(m && kv_pool_dev && page_table_host && workspace_dev && out_seq, "null argument");
  CHECK_ARG(page_size == 16 || page_size == 32 || page_size == 64, "page_size must be 16, 32 or 64");
  CHECK_ARG(n_pages > 0 && n_logical_pages > 0, "no pages");
  CHECK_ARG(max_rows >= 1 && max_rows <= SSD_MAX_ROWS && max_draft >= 1 && max_draft <= 32, "bad row limits");
  for (int i = 0; i < n_logical_pages; ++i)
    CHECK_ARG(page_table_host[i] >= 0 && page_table_host[i] < n_pages, "page table entry out of range");
  const int R = std::max(max_rows, max_draft + 1);
  const int max_ctx = n_logical_pages * page_size;
  const size_t need = carve(m, R, max_draft, max_ctx, nullptr, nullptr);
  if (workspace_bytes < need) return fail(SSD_ERR_CAPACITY, "workspace too small");
  ssd_seq* q = new (std::nothrow) ssd_seq;
  if (!q) return fail(SSD_ERR_CAPACITY, "out of host memory");
  q->m = m;
  q->max_rows = R;
  q->max_draft = max_draft;
  q->max_ctx = max_ctx;
  q->log_cap = max_ctx;
  carve(m, R, max_draft, max_ctx, (char*)workspace_dev, &q->w);
  q->kv.pool = kv_pool_dev;
  q->kv.page_table = q->w.page_table;
  q->kv.n_lpages = n_logical_pages;
  q->kv.page_size = page_size;
  // RoPE table: (cos, sin)(pos * theta^(-2i/hd)) for every position of the sequence, in fp64, rounded to fp32
  const int half = m->d.head_dim / 2;
  std::vector<float2> cs((size_t)max_ctx * half);
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow((double)m->d.rope_theta, -2.0 * i / (double)m->d.head_dim);
    for (int pos = 0; pos < max_ctx; ++pos) {
      const double a = (double)pos * inv;
      cs[(size_t)pos * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
  }
  hipError_t e = hipMemcpy(q->w.page_table, page_table_host, sizeof(int32_t) * n_logical_pages,
                           hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(q->w.rope_cs, cs.data(), sizeof(float2) * cs.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    delete q;
    return fail(SSD_ERR_HIP, std::string("hipMemcpy: ") + hipGetErrorString(e));
  }
  int rc = launch_state_init(q->w.st, stream);
  if (rc == 0 && hipMemset(q->w.dec_ctr, 0, sizeof(unsigned) * 16 * (size_t)m->d.n_kv_heads) != hipSuccess)
    rc = SSD_ERR_HIP;
  if (rc == 0 && hipMemset(q->w.stat_ctr, 0, sizeof(unsigned) * (size_t)R) != hipSuccess) rc = SSD_ERR_HIP;
  if (rc == 0 && hipStreamSynchronize(stream) != hipSuccess) rc = SSD_ERR_HIP;
  if (rc != 0) {
    delete q;
    return fail(SSD_ERR_HIP, "state init failed");
  }
  {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    g_seqs.insert(q);
  }
  *out_seq = q;
  return SSD_OK;
}

extern "C" int ssd_seq_destroy(ssd_seq* seq) {
  CHECK_SEQ(seq);
  {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    g_seqs.erase(seq);
  }
  delete seq;
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// prefill and AR decode

extern "C" int ssd_prefill(ssd_seq* q, const int32_t* tokens_dev, int n, float temperature, uint64_t seed,
                           float* last_logits_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && tokens_dev, "null argument");
  CHECK_ARG(n >= 1, "empty prompt");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  if (n >= q->max_ctx) return fail(SSD_ERR_CAPACITY, "prompt does not fit the KV pages");
  const ssd_model_desc& d = q->m->d;
  const Workspace& w = q->w;
  TRY(launch_state_init(w.st, s));
  int last_rows = 0;
  const int chunk = std::min(q->max_rows, SPLIT_ATTN_MAX_ROWS);
  for (int c0 = 0; c0 < n; c0 += chunk) {
    const int M = std::min(chunk, n - c0);
    TRY(launch_fill_positions(w.pos, M, c0, s));
    TRY(launch_embed(d.dtype, d.embed, tokens_dev + c0, d.vocab, w.h, d.d_model, M, d.d_model, nullptr, nullptr,
                     s));
    Block b{w.h, RowBlock{M, nullptr, w.pos, nullptr, nullptr}, nullptr, 0, 0};
    TRY(run_layers(q, b, 0, d.n_layers, nullptr, s));
    last_rows = M;
  }
  float* lg = last_logits_dev ? last_logits_dev : w.logits1;
  TRY(final_logits(q, w.h + (size_t)(last_rows - 1) * d.d_model, 1, nullptr, lg, nullptr, s));
  TRY(launch_row_stats_seg(lg, d.vocab, 1, d.vocab, temperature, seed, nullptr, 0, 0, PURPOSE_SAMPLE, w.stats,
                           w.stat_recs, w.stat_ctr, nullptr, DraftStep{}, s));
  TRY(launch_pick_commit(w.stats, w.st, w.log, q->log_cap, 1, n, s));
  return SSD_OK;
}

namespace {

// One committed token through the plan's sub-layers (mask == nullptr: the full model).
int decode_one(ssd_seq* q, const uint8_t* mask, float temperature, uint64_t seed, float* logits_dev, hipStream_t s) {
  const ssd_model_desc& d = q->m->d;
  const Workspace& w = q->w;
  TRY(launch_single_row_prep(w.st, w.pos1, w.tok1, q->max_ctx, s));
  float* lg = logits_dev ? logits_dev : w.logits1;
  if (dec_usable(q, 1)) {
    std::vector<int> ent;
    plan_entries(ent, 0, d.n_layers, mask);
    TRY(dec_entry(q, w.tok1, nullptr, 1, nullptr, nullptr, w.h1, dec_gain(q->m, ent, 0, true), nullptr, s, 1));
    TRY(dec_layers(q, w.h1, 1, nullptr, w.pos1, ent, 0, ent.size(), true, nullptr, s));
    TRY(dec_logits(q, 1, nullptr, lg, nullptr, s));
  } else {
    TRY(launch_embed(d.dtype, d.embed, w.tok1, d.vocab, w.h1, d.d_model, 1, d.d_model, nullptr, nullptr, s));
    Block b{w.h1, RowBlock{1, nullptr, w.pos1, nullptr, nullptr}, nullptr, 0, 0};
    TRY(run_layers(q, b, 0, d.n_layers, mask, s));
    TRY(final_logits(q, w.h1, 1, nullptr, lg, nullptr, s));
  }
  TRY(launch_row_stats_seg(lg, d.vocab, 1, d.vocab, temperature, seed, &w.st->iteration, 0, 0, PURPOSE_SAMPLE,
                           w.stats, w.stat_recs, w.stat_ctr, nullptr, DraftStep{}, s));
  TRY(launch_pick_commit(w.stats, w.st, w.log, q->log_cap, 0, 0, s));
  return SSD_OK;
}

}  // namespace

extern "C" int ssd_decode_ar(ssd_seq* q, float temperature, uint64_t seed, float* logits_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q, "null argument");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  return decode_one(q, nullptr, temperature, seed, logits_dev, s);
}

extern "C" int ssd_decode_exit(ssd_seq* q, const uint8_t* skip_mask_host, int exit_layer, float temperature,
                               uint64_t seed, float* logits_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q, "null argument");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  std::vector<uint8_t> mask;
  CHECK_ARG(plan_mask(q->m, skip_mask_host, exit_layer, mask) >= 0, "exit_layer out of range");
  return decode_one(q, mask.data(), temperature, seed, logits_dev, s);
}

// ---------------------------------------------------------------------------
// draft / verify / accept / commit

namespace {

// Waits for the work queued on s and reads the draft's stop flag (a 4-byte copy).
int draft_stopped(ssd_seq* q, hipStream_t s, int* stopped) {
  int v = 0;
  hipError_t e = hipMemcpyAsync(&v, &q->w.st->stop, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return SSD_ERR_HIP;
  *stopped = v;
  return 0;
}

}  // namespace

extern "C" int ssd_draft(ssd_seq* q, const uint8_t* skip_mask_host, int exit_layer, int d_max, float conf_thresh,
                         float temperature, uint64_t seed, int32_t* draft_tokens_dev, float* draft_logits_dev,
                         int32_t* n_drafted_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && draft_tokens_dev && draft_logits_dev && n_drafted_dev, "null argument");
  CHECK_ARG(d_max >= 1 && d_max <= q->max_draft, "d out of range");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  const ssd_model_desc& d = q->m->d;
  const Workspace& w = q->w;
  std::vector<uint8_t> mask;
  const int b = plan_mask(q->m, skip_mask_host, exit_layer, mask);
  CHECK_ARG(b >= 0, "exit_layer out of range");
  const int* stop = &w.st->stop;
  TRY(launch_draft_begin(w.st, s));
  if (dec_usable(q, 1)) {
    std::vector<int> ent;
    plan_entries(ent, 0, b, nullptr);
    const size_t save = ent.size();
    plan_entries(ent, b, d.n_layers, mask.data());
    const float* g0 = dec_gain(q->m, ent, 0, true);
    for (int j = 1; j <= d_max; ++j) {
      TRY(launch_dec_draft_entry(w.st, draft_tokens_dev, j, w.pos1, w.tok1, q->max_ctx, n_drafted_dev, d.embed,
                                 d.vocab, w.h1, d.d_model, g0, w.xg, w.ss, s));
      // the residual at the reuse boundary is saved for the verify by the last projection below it
      float* hb = w.hb + (size_t)(j - 1) * d.d_model;
      TRY(dec_layers(q, w.h1, 1, nullptr, w.pos1, ent, 0, save, true, stop, s, hb));
      if (save == 0) TRY(launch_copy_rows(w.h1, hb, 1, d.d_model, nullptr, nullptr, stop, s));
      TRY(dec_layers(q, w.h1, 1, nullptr, w.pos1, ent, save, ent.size(), true, stop, s));
      float* lg = draft_logits_dev + (size_t)(j - 1) * d.vocab;
      TRY(dec_logits(q, 1, nullptr, lg, stop, s));
      TRY(launch_row_stats_seg(lg, d.vocab, 1, d.vocab, temperature, seed, nullptr, 0, 0, PURPOSE_DRAFT, nullptr,
                               w.stat_recs, w.stat_ctr, nullptr,
                               DraftStep{w.st, j, d_max, conf_thresh, draft_tokens_dev, n_drafted_dev}, s));
      if (conf_thresh > 0.f && j < d_max) {
        int stopped = 0;
        TRY(draft_stopped(q, s, &stopped));
        if (stopped) break;
      }
    }
    return SSD_OK;
  }
  Block blk{w.h1, RowBlock{1, nullptr, w.pos1, nullptr, stop}, nullptr, 0, 0};
  for (int j = 1; j <= d_max; ++j) {
    TRY(launch_draft_step_prep(w.st, draft_tokens_dev, j, w.pos1, w.tok1, q->max_ctx, n_drafted_dev, s));
    TRY(launch_embed(d.dtype, d.embed, w.tok1, d.vocab, w.h1, d.d_model, 1, d.d_model, nullptr, stop, s));
    TRY(run_layers(q, blk, 0, b, nullptr, s));
    TRY(launch_copy_rows(w.h1, w.hb + (size_t)(j - 1) * d.d_model, 1, d.d_model, nullptr, nullptr, stop, s));
    TRY(run_layers(q, blk, b, d.n_layers, mask.data(), s));
    float* lg = draft_logits_dev + (size_t)(j - 1) * d.vocab;
    TRY(final_logits(q, w.h1, 1, nullptr, lg, stop, s));
    TRY(launch_row_stats_seg(lg, d.vocab, 1, d.vocab, temperature, seed, nullptr, 0, 0, PURPOSE_DRAFT, nullptr,
                             w.stat_recs, w.stat_ctr, nullptr,
                             DraftStep{w.st, j, d_max, conf_thresh, draft_tokens_dev, n_drafted_dev}, s));
    if (conf_thresh > 0.f && j < d_max) {
      int stopped = 0;
      TRY(draft_stopped(q, s, &stopped));
      if (stopped) break;
    }
  }
  return SSD_OK;
}

extern "C" int ssd_verify(ssd_seq* q, const uint8_t* skip_mask_host, int exit_layer, int d_max,
                          const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev, int reuse,
                          float* logits_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && draft_tokens_dev && n_drafted_dev && logits_dev, "null argument");
  CHECK_ARG(d_max >= 1 && d_max <= q->max_draft, "d out of range");
  const ssd_model_desc& d = q->m->d;
  const Workspace& w = q->w;
  std::vector<uint8_t> mask;
  const int b = plan_mask(q->m, skip_mask_host, exit_layer, mask);
  CHECK_ARG(b >= 0, "exit_layer out of range");
  const int M = d_max + 1;
  const int* rows = &w.st->verify_rows;
  TRY(launch_verify_prep(w.st, draft_tokens_dev, n_drafted_dev, d_max, w.vpos, w.vtok, w.pos1, w.tok1, q->max_ctx,
                         s));
  if (dec_usable(q, M)) {
    std::vector<int> suffix;
    plan_entries(suffix, reuse ? b : 0, d.n_layers, nullptr);
    const float* g0 = dec_gain(q->m, suffix, 0, true);
    if (reuse) {
      // the last row (y_d') runs the layers below the boundary first (it uses row 0 of the block's
      // normalised-input buffers); then the rows < d' take the residual the draft saved there
      std::vector<int> prefix;
      plan_entries(prefix, 0, b, nullptr);
      TRY(dec_entry(q, w.tok1, nullptr, 1, nullptr, nullptr, w.h1, dec_gain(q->m, prefix, 0, false), nullptr, s, 1));
      TRY(dec_layers(q, w.h1, 1, nullptr, w.pos1, prefix, 0, prefix.size(), false, nullptr, s));
      TRY(dec_entry(q, nullptr, w.hb, d_max, n_drafted_dev, nullptr, w.h, g0, nullptr, s, M));
      TRY(dec_entry(q, nullptr, w.h1, 1, nullptr, n_drafted_dev, w.h, g0, nullptr, s, M));
    } else {
      TRY(dec_entry(q, w.vtok, nullptr, M, rows, nullptr, w.h, g0, nullptr, s, M));
    }
    TRY(dec_layers(q, w.h, M, rows, w.vpos, suffix, 0, suffix.size(), true, nullptr, s));
    TRY(dec_logits(q, M, rows, logits_dev, nullptr, s));
    return SSD_OK;
  }
  Block full{w.h, RowBlock{M, rows, w.vpos, nullptr, nullptr}, nullptr, 0, 0};
  if (reuse) {
    // rows < d' take the residual saved by the draft at the boundary
    TRY(launch_copy_rows(w.hb, w.h, d_max, d.d_model, n_drafted_dev, nullptr, nullptr, s));
    // the last row (y_d') runs the layers below the boundary
    TRY(launch_embed(d.dtype, d.embed, w.tok1, d.vocab, w.h1, d.d_model, 1, d.d_model, nullptr, nullptr, s));
    Block one{w.h1, RowBlock{1, nullptr, w.pos1, nullptr, nullptr}, nullptr, 0, 0};
    TRY(run_layers(q, one, 0, b, nullptr, s));
    TRY(launch_copy_rows(w.h1, w.h, 1, d.d_model, nullptr, n_drafted_dev, nullptr, s));
  } else {
    TRY(launch_embed(d.dtype, d.embed, w.vtok, d.vocab, w.h, d.d_model, M, d.d_model, rows, nullptr, s));
    TRY(run_layers(q, full, 0, b, nullptr, s));
  }
  TRY(run_layers(q, full, b, d.n_layers, nullptr, s));
  TRY(final_logits(q, w.h, M, rows, logits_dev, nullptr, s));
  return SSD_OK;
}

extern "C" int ssd_accept(ssd_seq* q, const float* p_logits_dev, const float* q_logits_dev,
                          const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev, int d_max, float temperature,
                          uint64_t seed, int32_t* out_tokens_dev, int32_t* n_out_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && p_logits_dev && q_logits_dev && draft_tokens_dev && n_drafted_dev && out_tokens_dev && n_out_dev,
            "null argument");
  CHECK_ARG(d_max >= 1 && d_max <= q->max_draft, "d out of range");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  TRY(launch_accept(p_logits_dev, q_logits_dev, q->m->d.vocab, draft_tokens_dev, n_drafted_dev, d_max, temperature,
                    seed, &q->w.st->iteration, 0, q->w.dec, q->w.corr, out_tokens_dev, n_out_dev,
                    &q->w.st->error_flags, s));
  return SSD_OK;
}

extern "C" int ssd_commit(ssd_seq* q, const int32_t* out_tokens_dev, const int32_t* n_out_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && out_tokens_dev && n_out_dev, "null argument");
  TRY(launch_commit(q->w.st, out_tokens_dev, n_out_dev, q->w.log, q->log_cap, q->max_draft + 1, s));
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// draft trees (dynamic verification)

extern "C" int ssd_tree_candidates(ssd_seq* q, const float* draft_logits_dev, const int32_t* n_drafted_dev, int d_max,
                                   float temperature, uint64_t seed, float rho, int k_max, int max_leaves,
                                   int32_t* leaf_tokens_dev, int32_t* leaf_depth_dev, int32_t* n_leaves_dev,
                                   hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && draft_logits_dev && n_drafted_dev && leaf_tokens_dev && leaf_depth_dev && n_leaves_dev,
            "null argument");
  CHECK_ARG(d_max >= 1 && d_max <= q->max_draft, "d out of range");
  CHECK_ARG(k_max >= 1 && k_max <= TREE_KMAX && k_max <= q->m->d.vocab, "k_max out of range");
  CHECK_ARG(max_leaves >= 0 && max_leaves <= TREE_SLOTS, "max_leaves out of range");
  CHECK_ARG(std::isfinite(rho), "bad rho");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  const Workspace& w = q->w;
  TRY(launch_tree_candidates(draft_logits_dev, q->m->d.vocab, d_max, n_drafted_dev, temperature, seed, w.st, rho,
                             k_max, max_leaves, w.tree_cand, w.tree_k, leaf_tokens_dev, leaf_depth_dev, n_leaves_dev,
                             s));
  return SSD_OK;
}

extern "C" int ssd_verify_tree(ssd_seq* q, const uint8_t* skip_mask_host, int exit_layer, int d_max,
                               const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev,
                               const int32_t* leaf_tokens_dev, const int32_t* leaf_depth_dev,
                               const int32_t* n_leaves_dev, int max_leaves, int reuse, float* logits_dev,
                               hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && draft_tokens_dev && n_drafted_dev && leaf_tokens_dev && leaf_depth_dev && n_leaves_dev && logits_dev,
            "null argument");
  CHECK_ARG(d_max >= 1 && d_max <= q->max_draft, "d out of range");
  CHECK_ARG(max_leaves >= 0 && d_max + 1 + max_leaves <= 16, "a tree verify holds at most 16 rows");
  if (!dec_usable(q, d_max + 1 + max_leaves) || q->max_rows < d_max + 1 + max_leaves)
    return fail(SSD_ERR_UNSUPPORTED, "tree verification runs bf16 models in 16-row decode blocks");
  if (!attention_dec_leaves_fit(q->max_ctx))
    return fail(SSD_ERR_UNSUPPORTED, "context too long for tree verification");
  const ssd_model_desc& d = q->m->d;
  const Workspace& w = q->w;
  std::vector<uint8_t> mask;
  const int b = plan_mask(q->m, skip_mask_host, exit_layer, mask);
  CHECK_ARG(b >= 0, "exit_layer out of range");
  const int M = d_max + 1 + max_leaves, MP = 1 + max_leaves;
  const int* rows = &w.st->tree_rows;
  TRY(launch_tree_verify_prep(w.st, draft_tokens_dev, n_drafted_dev, d_max, leaf_tokens_dev, leaf_depth_dev,
                              n_leaves_dev, max_leaves, w.tvpos, w.tvtok, w.ppos, w.ptok, q->max_ctx, s));
  std::vector<int> suffix;
  plan_entries(suffix, reuse ? b : 0, d.n_layers, nullptr);
  const float* g0 = dec_gain(q->m, suffix, 0, true);
  if (reuse) {
    // y_d' and the leaves run the layers below the boundary; the chain rows < d' take the residual
    // the draft saved there
    std::vector<int> prefix;
    plan_entries(prefix, 0, b, nullptr);
    const int* prows = &w.st->tree_prefix_rows;
    TRY(dec_entry(q, w.ptok, nullptr, MP, prows, nullptr, w.hp, dec_gain(q->m, prefix, 0, false), nullptr, s, MP));
    TRY(dec_layers(q, w.hp, MP, prows, w.ppos, prefix, 0, prefix.size(), false, nullptr, s, nullptr,
                   &w.st->tree_side_prefix));
    TRY(dec_entry(q, nullptr, w.hb, d_max, n_drafted_dev, nullptr, w.h, g0, nullptr, s, M));
    TRY(dec_entry(q, nullptr, w.hp, MP, prows, n_drafted_dev, w.h, g0, nullptr, s, M));
  } else {
    TRY(dec_entry(q, w.tvtok, nullptr, M, rows, nullptr, w.h, g0, nullptr, s, M));
  }
  TRY(dec_layers(q, w.h, M, rows, w.tvpos, suffix, 0, suffix.size(), true, nullptr, s, nullptr,
                 &w.st->tree_side_full));
  TRY(dec_logits(q, M, rows, logits_dev, nullptr, s));
  return SSD_OK;
}

extern "C" int ssd_accept_tree(ssd_seq* q, const float* logits_dev, const float* q_logits_dev,
                               const int32_t* draft_tokens_dev, const int32_t* n_drafted_dev, int d_max,
                               const int32_t* leaf_tokens_dev, const int32_t* leaf_depth_dev,
                               const int32_t* n_leaves_dev, int max_leaves, float temperature, uint64_t seed,
                               int32_t* out_tokens_dev, int32_t* n_out_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && logits_dev && draft_tokens_dev && n_drafted_dev && leaf_tokens_dev && leaf_depth_dev &&
                n_leaves_dev && out_tokens_dev && n_out_dev,
            "null argument");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  CHECK_ARG(temperature == 0.f || q_logits_dev, "sampled acceptance needs the draft's logits");
  CHECK_ARG(d_max >= 1 && d_max <= q->max_draft, "d out of range");
  CHECK_ARG(max_leaves >= 0 && d_max + 1 + max_leaves <= std::min(16, q->max_rows), "too many tree rows");
  const ssd_model_desc& d = q->m->d;
  const Workspace& w = q->w;
  const int M = d_max + 1 + max_leaves;
  if (temperature > 0.f) {
    TRY(launch_tree_accept_sampled(logits_dev, q_logits_dev, d.vocab, draft_tokens_dev, n_drafted_dev, d_max,
                                   leaf_tokens_dev, leaf_depth_dev, n_leaves_dev, max_leaves, temperature, seed,
                                   w.st, w.dec, w.corr, out_tokens_dev, n_out_dev, s));
  } else {
    TRY(launch_row_stats_seg(logits_dev, d.vocab, M, d.vocab, 0.f, 0, nullptr, 0, 0, PURPOSE_SAMPLE, w.stats,
                             w.stat_recs, w.stat_ctr, nullptr, DraftStep{}, s));
    TRY(launch_tree_accept(w.stats, draft_tokens_dev, n_drafted_dev, d_max, leaf_tokens_dev, leaf_depth_dev,
                           n_leaves_dev, max_leaves, w.st, out_tokens_dev, n_out_dev, s));
  }
  TRY(launch_tree_kv_fix(w.st, w.tree_kv, q->kv, d.n_layers, d.n_kv_heads, d.head_dim, s));
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// SWIFT matchness scoring

extern "C" int ssd_score_masks(ssd_seq* q, const uint8_t* masks_host, int n_masks, const int32_t* window_dev,
                               int pos0, int gamma, float* scores_dev, int32_t* best_dev, int32_t* row_pred_dev,
                               hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && masks_host && window_dev && scores_dev && best_dev, "null argument");
  CHECK_ARG(n_masks >= 1 && gamma >= 1, "empty scoring problem");
  CHECK_ARG(pos0 >= 0, "negative pos0");
  const ssd_model_desc& d = q->m->d;
  const int L = d.n_layers;
  const int R = n_masks * gamma;
  if (R > q->max_rows) return fail(SSD_ERR_CAPACITY, "n_masks * gamma exceeds max_rows");
  if (R > SPLIT_ATTN_MAX_ROWS && !attention_groups_usable(d.dtype, d.head_dim, d.n_heads, d.n_kv_heads))
    return fail(SSD_ERR_UNSUPPORTED, "more than 1024 scoring rows need a bf16 model with head_dim 64 or 128");
  if (pos0 + gamma > q->max_ctx) return fail(SSD_ERR_CAPACITY, "window beyond the KV pages");
  const Workspace& w = q->w;
  // Candidates whose plans agree on every sub-layer before sl carry the same residual rows into sl, so a
  // sub-layer runs once per class of such candidates, on the rows of one member (its holder).  Where a
  // class splits at sl (some members run it, the others skip it), the part without the holder becomes a
  // new class whose first member takes a copy of the holder's rows before sl runs.  Every candidate's
  // rows thus go through the same computation as when scored alone (a row's result does not depend on
  // the other rows of its launch).
  const size_t ML = 2 * (size_t)L;
  std::vector<int> cls(n_masks, 0), hold(1, 0);   // class of each candidate; holder of each class
  std::vector<int> maps, copies;                   // row lists of the sub-layers; (src, dst) holder pairs
  std::vector<size_t> map_off(2 * L), copy_off(2 * L + 2);
  std::vector<int> counts(2 * L);
  for (int sl = 0; sl < 2 * L; ++sl) {
    auto runs = [&](int c) { return masks_host[(size_t)c * ML + sl] == 0; };
    const int nc = (int)hold.size();
    std::vector<int> first_run(nc, -1), first_skip(nc, -1);
    for (int c = 0; c < n_masks; ++c) {
      int& f = runs(c) ? first_run[cls[c]] : first_skip[cls[c]];
      if (f < 0) f = c;
    }
    copy_off[sl] = copies.size();
    for (int k = 0; k < nc; ++k) {
      if (first_run[k] < 0 || first_skip[k] < 0) continue;
      const bool holder_runs = runs(hold[k]);
      const int nh = holder_runs ? first_skip[k] : first_run[k];
      for (int c = 0; c < n_masks; ++c)
        if (cls[c] == k && runs(c) != holder_runs) cls[c] = (int)hold.size();
      copies.push_back(hold[k]);
      copies.push_back(nh);
      hold.push_back(nh);
    }
    // every class now runs sl or skips it as a whole: the rows of the running classes' holders
    std::vector<int> hs;
    for (int hc : hold)
      if (runs(hc)) hs.push_back(hc);
    std::sort(hs.begin(), hs.end());
    map_off[sl] = maps.size();
    for (int hc : hs)
      for (int i = 0; i < gamma; ++i) maps.push_back(hc * gamma + i);
    counts[sl] = (int)(maps.size() - map_off[sl]);
  }
  // before the logits every candidate takes its class's rows
  copy_off[2 * L] = copies.size();
  for (int c = 0; c < n_masks; ++c)
    if (hold[cls[c]] != c) {
      copies.push_back(hold[cls[c]]);
      copies.push_back(c);
    }
  copy_off[2 * L + 1] = copies.size();
  const size_t n_maps = maps.size();
  maps.insert(maps.end(), copies.begin(), copies.end());
  hipError_t e = hipMemcpyAsync(w.rowmaps, maps.data(), sizeof(int) * maps.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "rowmap upload");
  const int* dev_copies = w.rowmaps + n_maps;
  auto copy_rows = [&](int i) {
    return launch_copy_candidate_rows(w.h, d.d_model, dev_copies + copy_off[i],
                                      (int)(copy_off[i + 1] - copy_off[i]) / 2, gamma, s);
  };
  TRY(launch_window_rows(window_dev, R, gamma, pos0, w.pos, w.tok, s));
  // the window's embedding in candidate 0's rows (the first class's holder); the others are copied
  TRY(launch_embed(d.dtype, d.embed, w.tok, d.vocab, w.h, d.d_model, gamma, d.d_model, nullptr, nullptr, s));
  for (int l = 0; l < L; ++l) {
    for (int sub = 0; sub < 2; ++sub) {
      const int sl = 2 * l + sub;
      TRY(copy_rows(sl));
      const int M = counts[sl];
      if (M == 0) continue;
      // compact row j is window row j % gamma: positions come from w.pos (filled for all R rows)
      Block b{w.h, RowBlock{M, nullptr, w.pos, w.rowmaps + map_off[sl], nullptr}, w.local_kv, pos0, gamma};
      if (sub == 0) TRY(attn_sublayer(q, l, b, s));
      else TRY(mlp_sublayer(q, l, b, s));
    }
  }
  TRY(copy_rows(2 * L));
  TRY(final_logits(q, w.h, R, nullptr, w.logits_rows, nullptr, s));
  TRY(launch_row_stats_seg(w.logits_rows, d.vocab, R, d.vocab, 0.f, 0, nullptr, 0, 0, PURPOSE_DRAFT, w.stats,
                           w.stat_recs, w.stat_ctr, nullptr, DraftStep{}, s));
  TRY(launch_score(w.stats, window_dev, n_masks, gamma, scores_dev, best_dev, row_pred_dev, s));
  // the host row lists must outlive the copy
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "stream sync");
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// SWIFT layer-set search (host driver over the batched scoring pass)

namespace {

// Philox4x32-10 (Salmon et al., SC'11), host side: the generator of the sampling draws.
void philox_host(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1, n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

constexpr uint32_t PURPOSE_PROPOSE = 3;

// n_skip of the L layers (sublayers == 0: both bits of a layer) or of the 2L sub-layers (bit i).
void propose_layers(int L, int n_skip, int sublayers, uint64_t seed, int step, int cand, uint8_t* mask) {
  const int N = sublayers ? 2 * L : L;
  std::vector<int> idx(N);
  for (int i = 0; i < N; ++i) idx[i] = i;
  uint32_t w[4] = {0, 0, 0, 0};
  for (int i = 0; i < n_skip; ++i) {
    if (i % 4 == 0) {
      w[0] = (uint32_t)step; w[1] = (uint32_t)cand; w[2] = PURPOSE_PROPOSE; w[3] = (uint32_t)(i / 4);
      philox_host(w, (uint32_t)seed, (uint32_t)(seed >> 32));
    }
    const uint64_t x = w[i % 4];
    const int r = (int)((x * (uint64_t)(N - i)) >> 32);
    std::swap(idx[i], idx[i + r]);
  }
  std::fill(mask, mask + 2 * L, (uint8_t)0);
  for (int i = 0; i < n_skip; ++i) {
    if (sublayers) mask[idx[i]] = 1;
    else mask[2 * idx[i]] = mask[2 * idx[i] + 1] = 1;
  }
}

// The search's Bayesian-optimisation step: a Gaussian process over the mask vectors of the observed
// plans (scores standardised; kernel exp(-|x - x'|^2 / (2 l^2)), l^2 = the number of skipped entries of a
// pool plan, unit signal variance, 1e-6 noise) ranks the pool's plans by expected improvement over the
// incumbent; picks = the n_cand best, lower pool index first among equal values.  Returns false when the
// observed scores are all equal (nothing to model).
bool bo_rank(const uint8_t* obs, const double* ys, int n, double inc_score, const uint8_t* pool, int P, size_t ML,
             int n_cand, std::vector<int>& picks) {
  if (n < 1) return false;
  double mean = 0.0;
  for (int i = 0; i < n; ++i) mean += ys[i];
  mean /= n;
  double var = 0.0;
  for (int i = 0; i < n; ++i) var += (ys[i] - mean) * (ys[i] - mean);
  const double sd = std::sqrt(var / n);
  if (!(sd > 0.0)) return false;
  double ell2 = 0.0;
  for (size_t e = 0; e < ML; ++e) ell2 += pool[e] ? 1.0 : 0.0;
  if (!(ell2 > 0.0)) ell2 = 1.0;
  auto kern = [&](const uint8_t* a, const uint8_t* b) {
    double d2 = 0.0;
    for (size_t e = 0; e < ML; ++e) d2 += (a[e] != 0) != (b[e] != 0) ? 1.0 : 0.0;
    return std::exp(-d2 / (2.0 * ell2));
  };
  // Cholesky factor C (lower) of K + 1e-6 I, then alpha = K^-1 y
  std::vector<double> C((size_t)n * n, 0.0), y(n), alpha(n), k(n), v(n);
  for (int i = 0; i < n; ++i) y[i] = (ys[i] - mean) / sd;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j <= i; ++j) {
      double a = kern(obs + i * ML, obs + j * ML) + (i == j ? 1e-6 : 0.0);
      for (int t = 0; t < j; ++t) a -= C[(size_t)i * n + t] * C[(size_t)j * n + t];
      C[(size_t)i * n + j] = i == j ? std::sqrt(std::max(a, 1e-300)) : a / C[(size_t)j * n + j];
    }
  auto lower_solve = [&](const std::vector<double>& b, std::vector<double>& x) {
    for (int i = 0; i < n; ++i) {
      double a = b[i];
      for (int t = 0; t < i; ++t) a -= C[(size_t)i * n + t] * x[t];
      x[i] = a / C[(size_t)i * n + i];
    }
  };
  std::vector<double> z(n);
  lower_solve(y, z);
  for (int i = n - 1; i >= 0; --i) {
    double a = z[i];
    for (int t = i + 1; t < n; ++t) a -= C[(size_t)t * n + i] * alpha[t];
    alpha[i] = a / C[(size_t)i * n + i];
  }
  const double best = (inc_score - mean) / sd;
  std::vector<double> ei(P);
  for (int p = 0; p < P; ++p) {
    double mu = 0.0;
    for (int i = 0; i < n; ++i) {
      k[i] = kern(pool + p * ML, obs + i * ML);
      mu += k[i] * alpha[i];
    }
    lower_solve(k, v);
    double vv = 0.0;
    for (int i = 0; i < n; ++i) vv += v[i] * v[i];
    const double sg = std::sqrt(std::max(1.0 - vv, 0.0));
    if (sg <= 1e-12) {
      ei[p] = std::max(mu - best, 0.0);
    } else {
      const double zz = (mu - best) / sg;
      ei[p] = (mu - best) * 0.5 * std::erfc(-zz / std::sqrt(2.0)) + sg * std::exp(-0.5 * zz * zz) / std::sqrt(2.0 * M_PI);
    }
  }
  std::vector<int> order(P);
  for (int p = 0; p < P; ++p) order[p] = p;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return ei[a] > ei[b]; });
  picks.assign(order.begin(), order.begin() + std::min(n_cand, P));
  return true;
}

constexpr int BO_POOL_FACTOR = 8;     // pool = 8 n_cand random proposals
constexpr int BO_WINDOW = 256;        // the GP sees the most recent 256 scored plans

}  // namespace

extern "C" int ssd_uniform_mask(int n_layers, int n_skip, uint8_t* mask_host) {
  CHECK_ARG(mask_host && n_layers > 0 && n_skip >= 0 && n_skip <= n_layers, "bad argument");
  std::fill(mask_host, mask_host + 2 * n_layers, (uint8_t)0);
  for (int i = 0; i < n_skip; ++i) {
    const int l = (int)(((int64_t)2 * i + 1) * n_layers / (2 * (int64_t)n_skip));
    mask_host[2 * l] = mask_host[2 * l + 1] = 1;
  }
  return SSD_OK;
}

extern "C" int ssd_swift_propose(int n_layers, int n_skip, int sublayers, uint64_t seed, int step, int cand,
                                 uint8_t* mask_host) {
  CHECK_ARG(mask_host && n_layers > 0 && n_skip >= 0 && n_skip <= (sublayers ? 2 : 1) * n_layers && step >= 0 &&
                cand >= 0,
            "bad argument");
  propose_layers(n_layers, n_skip, sublayers, seed, step, cand, mask_host);
  return SSD_OK;
}

// One run of the search on a window: steps numbered step0, step0 + 1, ... (proposal counters and the
// Bayesian schedule), the run of unimproved steps starting at unimproved0.  inc: the starting plan in, the
// final incumbent out.
// Search steps step0 .. step0 + max_steps - 1 from the incumbent `inc`.  The proposals of a random step
// depend only on (seed, step, candidate), so a step and the random steps after it (up to the next
// Bayesian step, within the sequence's row limit) are scored in one pass; the steps are then taken in
// order as if scored one by one (a row's scores do not depend on the rows batched with it), and the
// passes' extra steps after a stop are discarded.
int swift_phase(ssd_seq* q, const int32_t* window_dev, int pos0, int gamma, std::vector<uint8_t>& inc, int n_skip,
                int sublayers, int n_cand, int max_steps, int patience, float target, uint64_t seed, int bo_every,
                int step0, int unimproved0, float* score, int* n_steps, int* unimproved_out, hipStream_t s) {
  const int L = q->m->d.n_layers;
  const size_t ML = 2 * (size_t)L;
  // masks one scoring pass can hold (beyond 1024 rows only where the scoring attention takes them)
  const ssd_model_desc& d = q->m->d;
  const int row_cap = attention_groups_usable(d.dtype, d.head_dim, d.n_heads, d.n_kv_heads)
                          ? q->max_rows : std::min(q->max_rows, SPLIT_ATTN_MAX_ROWS);
  const int max_masks = std::max(n_cand + 1, row_cap / gamma);
  std::vector<uint8_t> masks;
  std::vector<float> sc;
  std::vector<int> first;               // a pass's steps: index of each one's first mask, then the end
  std::vector<uint8_t> obs_m, pool;     // every scored plan of the steps taken, in scoring order, and a BO pool
  std::vector<double> obs_s;
  std::vector<int> picks;
  float inc_score = 0.f;
  int unimproved = unimproved0, t = 0;
  bool stop = false;
  auto is_bo = [&](int st) { return bo_every > 0 && st > 0 && st % bo_every == 0; };
  while (t < max_steps && !stop) {
    // ---- the pass: step t, then random steps while they fit
    masks.clear();
    first.clear();
    for (int u = t; u < max_steps; ++u) {
      const int st = step0 + u;
      const int off = u == 0 ? 1 : 0;
      const int nm = (int)(masks.size() / ML);
      if (u > t && (is_bo(st) || nm + n_cand + off > max_masks)) break;
      first.push_back(nm);
      masks.resize((size_t)(nm + n_cand + off) * ML);
      uint8_t* m = masks.data() + (size_t)nm * ML;
      if (off) std::copy(inc.begin(), inc.end(), m);
      bool bo = false;
      if (is_bo(st)) {                  // only the pass's first step: the history is complete
        const int P = BO_POOL_FACTOR * n_cand;
        pool.resize((size_t)P * ML);
        for (int c = 0; c < P; ++c) propose_layers(L, n_skip, sublayers, seed, st, c, pool.data() + c * ML);
        const int n = std::min((int)obs_s.size(), BO_WINDOW);
        const size_t f0 = obs_s.size() - n;
        bo = bo_rank(obs_m.data() + f0 * ML, obs_s.data() + f0, n, inc_score, pool.data(), P, ML, n_cand, picks);
        if (bo)
          for (int c = 0; c < n_cand; ++c)
            std::copy(pool.begin() + picks[c] * ML, pool.begin() + (picks[c] + 1) * ML, m + (off + c) * ML);
      }
      if (!bo)
        for (int c = 0; c < n_cand; ++c) propose_layers(L, n_skip, sublayers, seed, st, c, m + (off + c) * ML);
    }
    const int total = (int)(masks.size() / ML);
    first.push_back(total);
    sc.resize(total);
    TRY(ssd_score_masks(q, masks.data(), total, window_dev, pos0, gamma, q->w.swift_scores, q->w.swift_best,
                        nullptr, s));
    if (hipMemcpy(sc.data(), q->w.swift_scores, sizeof(float) * total, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(SSD_ERR_HIP, "read scores");
    // ---- the pass's steps in order
    for (size_t i = 0; i + 1 < first.size(); ++i) {
      const int b = first[i], e = first[i + 1];
      const int off = t == 0 ? 1 : 0;
      if (t == 0) inc_score = sc[b];
      obs_m.insert(obs_m.end(), masks.begin() + (size_t)b * ML, masks.begin() + (size_t)e * ML);
      for (int c = b; c < e; ++c) obs_s.push_back((double)sc[c]);
      int k = b + off;
      for (int c = b + off + 1; c < e; ++c)
        if (sc[c] > sc[k]) k = c;
      if (sc[k] > inc_score) {
        std::copy(masks.begin() + (size_t)k * ML, masks.begin() + (size_t)(k + 1) * ML, inc.begin());
        inc_score = sc[k];
        unimproved = 0;
      } else {
        ++unimproved;
      }
      ++t;
      if (inc_score > target || unimproved >= patience) {
        stop = true;
        break;
      }
    }
  }
  *score = inc_score;
  *n_steps = t;
  *unimproved_out = unimproved;
  return SSD_OK;
}

extern "C" int ssd_swift_search(ssd_seq* q, const int32_t* window_dev, int pos0, int gamma,
                                const uint8_t* init_mask_host, int n_skip, int sublayers, int n_cand, int max_steps,
                                int patience, float target, uint64_t seed, int bo_every, uint8_t* best_mask_host,
                                float* best_score, int* n_steps, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && window_dev && init_mask_host && best_mask_host && best_score && n_steps, "null argument");
  const int L = q->m->d.n_layers;
  CHECK_ARG(n_skip >= 0 && n_skip <= (sublayers ? 2 : 1) * L && n_cand >= 1 && n_cand + 1 <= 64 && max_steps >= 1 &&
                patience >= 1 && bo_every >= 0,
            "bad search parameters");
  if ((n_cand + 1) * gamma > q->max_rows) return fail(SSD_ERR_CAPACITY, "(n_cand + 1) * gamma exceeds max_rows");
  std::vector<uint8_t> inc(init_mask_host, init_mask_host + 2 * (size_t)L);
  int unimproved = 0;
  TRY(swift_phase(q, window_dev, pos0, gamma, inc, n_skip, sublayers, n_cand, max_steps, patience, target, seed,
                  bo_every, 0, 0, best_score, n_steps, &unimproved, s));
  std::copy(inc.begin(), inc.end(), best_mask_host);
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// SWIFT on the fly: self-speculative iterations with the plan in use, and after every `accumulate`
// committed tokens (while optimisation is not over) a phase of search steps on the last gamma + 1
// committed tokens; the plan becomes the phase's incumbent.

namespace {
bool swift_config_ok(const ssd_seq* q, const ssd_swift_config* c) {
  const int L = q->m->d.n_layers;
  return c->gamma >= 1 && c->n_skip >= 0 && c->n_skip <= (c->sublayers ? 2 : 1) * L && c->n_cand >= 1 &&
         c->n_cand + 1 <= 64 && c->steps_per_phase >= 1 && c->max_steps >= 0 && c->patience >= 1 &&
         c->bo_every >= 0 && c->d >= 1 && c->d <= q->max_draft && std::isfinite(c->target) &&
         std::isfinite(c->conf_thresh) && c->temperature >= 0.f && std::isfinite(c->temperature) &&
         (c->n_cand + 1) * c->gamma <= q->max_rows;
}
}  // namespace

extern "C" int ssd_swift_begin(ssd_seq* q, const ssd_swift_config* cfg, ssd_swift_state* st, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && cfg && st, "null argument");
  if (!swift_config_ok(q, cfg)) return fail(SSD_ERR_ARG, "bad SWIFT configuration");
  ssd_state ds;
  TRY(ssd_read_state(q, &ds, s));
  *st = ssd_swift_state{};
  st->done = cfg->max_steps == 0 ? 1 : 0;
  st->last_phase_n_out = ds.n_out;
  st->score = std::numeric_limits<float>::quiet_NaN();
  return SSD_OK;
}

extern "C" int ssd_swift_generate(ssd_seq* q, const ssd_swift_config* cfg, ssd_swift_state* st, uint8_t* plan_host,
                                  int n_tokens, int32_t* draft_tokens_dev, float* draft_logits_dev,
                                  int32_t* n_drafted_dev, float* verify_logits_dev, int32_t* out_tokens_dev,
                                  int32_t* n_out_dev, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && cfg && st && plan_host && draft_tokens_dev && draft_logits_dev && n_drafted_dev &&
                verify_logits_dev && out_tokens_dev && n_out_dev && n_tokens >= 0,
            "null argument");
  if (!swift_config_ok(q, cfg)) return fail(SSD_ERR_ARG, "bad SWIFT configuration");
  const int L = q->m->d.n_layers;
  const int acc = cfg->accumulate > 0 ? cfg->accumulate : cfg->gamma;
  ssd_state ds;
  TRY(ssd_read_state(q, &ds, s));
  const int n_end = ds.n_out + n_tokens;
  std::vector<uint8_t> inc(plan_host, plan_host + 2 * (size_t)L);
  while (ds.n_out < n_end) {
    TRY(ssd_draft(q, plan_host, -1, cfg->d, cfg->conf_thresh, cfg->temperature, cfg->seed, draft_tokens_dev,
                  draft_logits_dev, n_drafted_dev, s));
    TRY(ssd_verify(q, plan_host, -1, cfg->d, draft_tokens_dev, n_drafted_dev, 1, verify_logits_dev, s));
    TRY(ssd_accept(q, verify_logits_dev, draft_logits_dev, draft_tokens_dev, n_drafted_dev, cfg->d,
                   cfg->temperature, cfg->seed, out_tokens_dev, n_out_dev, s));
    TRY(ssd_commit(q, out_tokens_dev, n_out_dev, s));
    const int before = ds.n_out;
    TRY(ssd_read_state(q, &ds, s));
    ++st->iterations;
    if (ds.n_out == before) return fail(SSD_ERR_NUMERIC, "an iteration committed no token");
    if (st->done || ds.n_out - st->last_phase_n_out < acc || ds.n_out < cfg->gamma + 1) continue;
    // the window: the last gamma + 1 committed tokens, the newest at position kvlen
    const int32_t* window = q->w.log + (ds.n_out - 1 - cfg->gamma);
    const int pos0 = ds.kvlen - cfg->gamma;
    if (ds.n_out > q->log_cap) return fail(SSD_ERR_CAPACITY, "the output log no longer holds the window");
    std::copy(plan_host, plan_host + 2 * (size_t)L, inc.begin());
    float score = 0.f;
    int ran = 0, unimproved = 0;
    TRY(swift_phase(q, window, pos0, cfg->gamma, inc, cfg->n_skip, cfg->sublayers, cfg->n_cand,
                    std::min(cfg->steps_per_phase, cfg->max_steps - st->steps), cfg->patience, cfg->target, cfg->seed,
                    cfg->bo_every, st->steps, st->unimproved, &score, &ran, &unimproved, s));
    if (!std::equal(inc.begin(), inc.end(), plan_host)) ++st->switches;
    std::copy(inc.begin(), inc.end(), plan_host);
    st->steps += ran;
    st->unimproved = unimproved;
    st->score = score;
    ++st->phases;
    st->done = (st->steps >= cfg->max_steps || unimproved >= cfg->patience || score > cfg->target) ? 1 : 0;
    st->last_phase_n_out = ds.n_out;
  }
  return SSD_OK;
}

extern "C" int ssd_specee_features(const ssd_model* m, const float* h_dev, int rows, const int32_t* tokens_dev, int k,
                                   const float* prev_probs_dev, float* features_dev, hipStream_t s) {
  CHECK_MODEL(m);
  CHECK_ARG(m && h_dev && tokens_dev && features_dev && rows >= 0, "bad argument");
  if (k < 1 || k > 16) return fail(SSD_ERR_SHAPE, "k must be 1..16");
  const ssd_model_desc& d = m->d;
  TRY(launch_specee_features(d.dtype, h_dev, rows, d.d_model, d.rms_eps, d.final_norm, d.lm_head, d.vocab,
                             tokens_dev, k, prev_probs_dev, features_dev, s));
  return SSD_OK;
}

extern "C" int ssd_row_stats(const float* logits_dev, int rows, int V, float temperature, uint64_t seed,
                             int32_t iteration, ssd_row_stat* stats_dev, hipStream_t s) {
  CHECK_ARG(logits_dev && stats_dev && rows >= 1 && V >= 1, "bad argument");
  CHECK_ARG(temperature >= 0.f && std::isfinite(temperature), "bad temperature");
  TRY(launch_row_stats(logits_dev, V, rows, V, temperature, seed, nullptr, iteration, 0, PURPOSE_DRAFT, stats_dev,
                       nullptr, s));
  return SSD_OK;
}

// ---------------------------------------------------------------------------
// host synchronisation

extern "C" int ssd_read_state(ssd_seq* q, ssd_state* out, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && out, "null argument");
  DevState st;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&st, q->w.st, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SSD_ERR_HIP, std::string("read state: ") + hipGetErrorString(e));
  out->kvlen = st.kvlen;
  out->last_token = st.last_token;
  out->iteration = st.iteration;
  out->n_out = st.n_out;
  out->error_flags = st.error_flags;
  out->last_n_drafted = st.n_drafted;
  out->last_n_emitted = st.n_emitted;
  if (st.error_flags & ERRF_CAPACITY) return fail(SSD_ERR_CAPACITY, "KV pages or output log exhausted on the device");
  if (st.error_flags & ERRF_NUMERIC) return fail(SSD_ERR_NUMERIC, "non-finite logits seen on the device");
  if (st.error_flags & ERRF_INPUT) return fail(SSD_ERR_ARG, "a device-side argument was out of range");
  return SSD_OK;
}

extern "C" int ssd_read_output(ssd_seq* q, int32_t* tokens_host, int max_tokens, int* n_tokens, hipStream_t s) {
  CHECK_SEQ(q);
  CHECK_ARG(q && tokens_host && n_tokens && max_tokens >= 0, "bad argument");
  ssd_state st;
  int rc = ssd_read_state(q, &st, s);
  if (rc != SSD_OK && rc != SSD_ERR_CAPACITY && rc != SSD_ERR_NUMERIC) return rc;
  const int n = std::min(std::min(st.n_out, max_tokens), q->log_cap);
  hipError_t e = n > 0 ? hipMemcpy(tokens_host, q->w.log, sizeof(int32_t) * n, hipMemcpyDeviceToHost) : hipSuccess;
  if (e != hipSuccess) return fail(SSD_ERR_HIP, "read output");
  *n_tokens = n;
  return rc;
}
