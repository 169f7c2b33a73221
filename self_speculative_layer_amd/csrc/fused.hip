// Persistent decode pass (bf16): one cooperative launch runs a whole forward
// pass of at most 16 rows -- an embedding or residual input, a list of
// attention / MLP sub-layers, and optionally the shared final norm + LM head.
//
// One workgroup of 4 waves per CU (one wave per SIMD, so the accumulation
// registers may use the AGPR half of the register file).  A pass is a
// sequence of phases:
//   INIT  rows -> residual h, bf16(h * gain) for the first projection, group sums of h^2
//   QKV   projection tiles; epilogue: 1/rms scale, RoPE, q -> buffer, k/v -> paged cache
//   ATTN  (KV head, key split, row block) items; the last item of a head merges its splits
//   O     projection tiles; epilogue: h += o Wo^T, bf16(h * next gain), group sums of h^2
//   GU    gate/up tiles (8 gate rows + 8 up rows); epilogue: 1/rms scale, SwiGLU
//   DOWN  like O
//   LM    LM-head tiles; epilogue: 1/rms scale, logits
// A phase's items are dealt round-robin to workgroups.  A workgroup publishes
// the number of items it finished in a phase with one device-scope release;
// a phase starts reading the previous phase's results after a device-scope
// acquire of that counter.  Weights never depend on activations, so each wave
// issues the loads of its next tile's weights before it waits: HBM keeps
// streaming across phase boundaries and across tiles (a workgroup barrier on
// gfx950 does not wait for outstanding global loads).
//
// The projection tiles split K over the 8 waves exactly as the standalone
// linear-layer kernel does (same slices, same k order, same fixed-order LDS
// reduction), and the epilogues use the same rounding steps, so a pass gives
// the same bits as the standalone kernels.
//
// Every wait is bounded: past a spin limit it sets an error flag and goes on,
// so the grid always drains.
#include "kernels.h"
#include "attn.h"

namespace ssd {

constexpr int FZ_NW = 4;
constexpr int FZ_NT = FZ_NW * 64;
constexpr int FZ_CH = 2;                        // k-blocks (of 32) per weight chunk
constexpr uint32_t FZ_SPIN_LIMIT = 1u << 22;    // x ~1 us sleeps: a few seconds at most

typedef uint32_t fz_u32x4 __attribute__((ext_vector_type(4)));

// Publishes this workgroup's results: EVERY wave waits for its own stores and
// writes back the L2 (a workgroup barrier on gfx950 does not wait for other
// waves' global stores), then thread 0 adds v to the counter.  Returns the
// counter's previous value to all threads (via *shared_old).  All threads call it.
__device__ __forceinline__ void fz_publish(unsigned* c, unsigned v, unsigned* shared_old) {
  __atomic_thread_fence(__ATOMIC_RELEASE);
  __syncthreads();
  if (threadIdx.x == 0) *shared_old = __hip_atomic_fetch_add(c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
}

// Thread 0 waits until *c >= target; then EVERY wave performs the
// device-scope acquire itself (its own cache invalidation, ordered before its
// own later loads): the activation buffers are rewritten layer after layer,
// so lines cached by earlier phases must not be read again.
__device__ __forceinline__ void fz_wait(unsigned* c, unsigned target, int* err) {
  if (threadIdx.x == 0) {
    uint32_t spins = 0;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(8);
      if (++spins > FZ_SPIN_LIMIT) {
        atomicOr(err, ERRF_TIMEOUT);
        break;
      }
    }
  }
  __syncthreads();
  __atomic_thread_fence(__ATOMIC_ACQUIRE);
}

// Weight row of MFMA row r (0..15) of a tile.
__device__ __forceinline__ int fz_wrow(int type, int tile, int r, int HD, int F) {
  if (type == PH_QKV) {
    const int tph = HD / 16;                         // tiles per head: 8 rotation pairs each
    const int head = tile / tph, pb = (tile % tph) * 8;
    return head * HD + (r < 8 ? pb + r : HD / 2 + pb + r - 8);
  }
  if (type == PH_GU) {
    const int f0 = tile * 8;
    return r < 8 ? f0 + r : F + f0 + r - 8;
  }
  return tile * 16 + r;
}

struct FzGemm {
  const bf16_t* W;
  const bf16_t* X;
  int K, nrow_w, ntiles;
};

__device__ __forceinline__ FzGemm fz_gemm(const FzParams& p, int type, int layer) {
  FzGemm g;
  const int qd = p.H * p.HD, kvd = p.KVH * p.HD;
  switch (type) {
    case PH_QKV: g.W = p.layers[layer].w_qkv; g.X = p.xg; g.K = p.D; g.nrow_w = qd + 2 * kvd; g.ntiles = (qd + 2 * kvd) / 16; break;
    case PH_O: g.W = p.layers[layer].w_o; g.X = p.ob; g.K = qd; g.nrow_w = p.D; g.ntiles = p.D / 16; break;
    case PH_GU: g.W = p.layers[layer].w_gate_up; g.X = p.xg; g.K = p.D; g.nrow_w = 2 * p.F; g.ntiles = p.F / 8; break;
    case PH_DOWN: g.W = p.layers[layer].w_down; g.X = p.ab; g.K = p.F; g.nrow_w = p.D; g.ntiles = p.D / 16; break;
    default: g.W = p.lm_head; g.X = p.xg; g.K = p.D; g.nrow_w = p.V; g.ntiles = (p.V + 15) / 16; break;
  }
  return g;
}

__device__ __forceinline__ bool fz_is_gemm(int type) {
  return type == PH_QKV || type == PH_O || type == PH_GU || type == PH_DOWN || type == PH_LM;
}

// Per-wave state of a tile: this lane's weight row pointer and the wave's k-block range.
struct FzTile {
  const bf16_t* wp;
  bool wv;
  int kb0, kb1;
};

__device__ __forceinline__ FzTile fz_tile(const FzGemm& g, int type, int tile, int HD, int F) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kg = lane >> 4;
  const int row = fz_wrow(type, tile, r, HD, F);
  FzTile t;
  t.wv = row < g.nrow_w;
  t.wp = g.W + (size_t)(t.wv ? row : 0) * g.K + kg * 8;
  const int nu = g.K >> 6;
  t.kb0 = 2 * ((nu * wave) / FZ_NW);
  t.kb1 = 2 * ((nu * (wave + 1)) / FZ_NW);
  return t;
}

// Loads of a chunk.  Only the k range is guarded (wave-uniform); a lane whose
// weight row is past the matrix reads row 0 instead and a lane whose
// activation row is inactive reads that buffer row as it is: either only
// feeds output elements that the epilogue discards (MFMA output (i, j)
// depends on A row i and B column j only).  Blocks past the range keep stale
// registers and are skipped by fz_mma.
__device__ __forceinline__ void fz_load_w(fz_u32x4 (&buf)[FZ_CH], const FzTile& t, int kb) {
#pragma unroll
  for (int u = 0; u < FZ_CH; ++u)
    if (kb + u < t.kb1) buf[u] = __builtin_nontemporal_load((const fz_u32x4*)(t.wp + (kb + u) * 32));
}

__device__ __forceinline__ void fz_load_x(fz_u32x4 (&buf)[FZ_CH], const bf16_t* xp, int kb, int kb1) {
#pragma unroll
  for (int u = 0; u < FZ_CH; ++u)
    if (kb + u < kb1) buf[u] = *(const fz_u32x4*)(xp + (kb + u) * 32);
}

__device__ __forceinline__ void fz_mma(f32x4& acc, const fz_u32x4 (&w)[FZ_CH], const fz_u32x4 (&x)[FZ_CH], int n) {
#pragma unroll
  for (int u = 0; u < FZ_CH; ++u)
    if (u < n)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[u]), __builtin_bit_cast(bf16x8, x[u]),
                                                    acc, 0, 0, 0);
}

struct FzSmemGemm {
  float red[FZ_NW][16][17];
  float inv[16];
};

template <int HD>
union FzSmem {
  AttnSmem<bf16_t, HD, FZ_NW> att;
  FzSmemGemm gm;
};

// 1/rms of rows m < Ma from the group sums (canonical reduction).
__device__ __forceinline__ void fz_row_inv(const FzParams& p, int Ma, float* inv) {
  const int wave = threadIdx.x >> 6;
  for (int m = wave; m < 16; m += FZ_NW) {
    float v = 1.f;
    if (m < Ma) v = inv_rms(row_ss_total(p.ss + m, 16, p.D / 16), p.D, p.eps);
    if ((threadIdx.x & 63) == 0) inv[m] = v;
  }
}

template <int HD>
__global__ __launch_bounds__(FZ_NT, 1) void fused_pass_kernel(FzParams p) {
  if (p.stop && *p.stop) return;
  __shared__ FzSmem<HD> sm;
  __shared__ unsigned sh_old;
  const int NWG = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63;
  const int Ma = p.nrows ? min(p.M, *p.nrows) : p.M;
  const int G = p.H / p.KVH;
  const int RB = min(16, ATT_MAXQ / G);
  const int nrb = (Ma + RB - 1) / RB;
  const int nsplit_act = p.pos[Ma - 1] / ATT_SPLIT + 1;
  unsigned* const exit_ctr = p.counters + p.n_phase;
  unsigned* const head_ctr = p.counters + p.n_phase + 1;

  int attn_idx = 0;

  for (int ph = 0; ph < p.n_phase; ++ph) {
    const int type = p.ph_type[ph];
    const int layer = p.ph_layer[ph];

    if (type == PH_INIT) {
      const float* gain = p.ph_gain[ph];
      int done = 0;
      for (int m = wg; m < p.M; m += NWG, ++done) {
        if (m >= Ma) continue;
        const int tok = p.tokens ? min(max(p.tokens[m], 0), p.V - 1) : 0;
        for (int base = 0; base < p.D; base += FZ_NT) {
          const int i = base + tid;        // D is a multiple of 64: whole 16-lane groups
          float v = 0.f;
          if (i < p.D) v = p.h_in ? p.h_in[(size_t)m * p.D + i] : bf2f(p.embed[(size_t)tok * p.D + i]);
          const float s = tile16_ss_lanes(v);
          if (i < p.D) {
            if (!p.h_in || p.h_in != p.h) p.h[(size_t)m * p.D + i] = v;
            if (gain) p.xg[(size_t)m * p.D + i] = f2bf(__fmul_rn(v, gain[i]));
            if ((i & 15) == 0) p.ss[(i >> 4) * 16 + m] = s;
          }
        }
      }
      if (done) fz_publish(p.counters + ph, done, &sh_old);
    } else if (type == PH_ATTN) {
      // all QKV tiles of this layer done
      const FzGemm prev = fz_gemm(p, PH_QKV, layer);
      fz_wait(p.counters + ph - 1, prev.ntiles, p.err);
      const int ntask = p.KVH * nsplit_act * nrb;
      const unsigned per_head = nsplit_act * nrb;
      int combined = 0;
      for (int t = wg; t < ntask; t += NWG) {
        const int g = t % p.KVH, rest = t / p.KVH;
        const int s = rest % nsplit_act, rb = rest / nsplit_act;
        const int r0 = rb * RB, r1 = min(r0 + RB, Ma);
        if (s * ATT_SPLIT <= p.pos[r1 - 1])
          attn_partial_item<bf16_t, HD, FZ_NW>(sm.att, p.qb, p.H * HD, p.pool, p.page_table, p.PS, p.L, layer, p.H,
                                               p.KVH, p.pos, r0, r1, g, s, p.nsplit_max, nullptr, 0, 0, p.part);
        // the last item of head g merges its splits
        fz_publish(head_ctr + attn_idx * p.KVH + g, 1u, &sh_old);
        if (sh_old == per_head - 1) {
          __atomic_thread_fence(__ATOMIC_ACQUIRE);
          for (int e = tid; e < Ma * G * HD; e += FZ_NT) {
            const int d = e % HD, j = (e / HD) % G, r = e / (HD * G);
            attn_combine_elem<bf16_t, HD>(p.part, p.nsplit_max, r, g * G + j, p.H, p.pos[r], d, p.ob, p.H * HD);
          }
          ++combined;
        }
        __syncthreads();
      }
      if (combined) fz_publish(p.counters + ph, combined, &sh_old);
      ++attn_idx;
    } else {
      // ---------------------------------------------------------------- projection phase
      const FzGemm gm = fz_gemm(p, type, layer);
      const int kg = lane >> 4, r = lane & 15;
      const bf16_t* xrow = gm.X + (size_t)r * gm.K + kg * 8;   // buffers hold 16 rows
      // weight chunks of the current tile; the first tile's are requested before the wait
      fz_u32x4 wA[FZ_CH], wB[FZ_CH];
      if (wg < gm.ntiles) {
        const FzTile t0 = fz_tile(gm, type, wg, HD, p.F);
        fz_load_w(wA, t0, t0.kb0);
        fz_load_w(wB, t0, t0.kb0 + FZ_CH);
      }
      // previous phase done: INIT counts its M row items, ATTN its merged KV heads, a projection its tiles
      {
        const int pt = p.ph_type[ph - 1];
        unsigned target;
        if (pt == PH_ATTN) target = p.KVH;
        else if (pt == PH_INIT) target = p.M;
        else target = fz_gemm(p, pt, p.ph_layer[ph - 1]).ntiles;
        fz_wait(p.counters + ph - 1, target, p.err);
      }
      if (ph == p.save_phase && wg == 0)
        for (int e = tid; e < Ma * p.D; e += FZ_NT) p.save_h[e] = p.h[e];
      const bool scaled = type == PH_QKV || type == PH_GU || type == PH_LM;
      if (scaled) {
        fz_row_inv(p, Ma, sm.gm.inv);
        __syncthreads();
      }
      int done = 0;
      for (int tile = wg; tile < gm.ntiles; tile += NWG, ++done) {
        const FzTile tt = fz_tile(gm, type, tile, HD, p.F);
        fz_u32x4 xA[FZ_CH], xB[FZ_CH];
        fz_load_x(xA, xrow, tt.kb0, tt.kb1);
        fz_load_x(xB, xrow, tt.kb0 + FZ_CH, tt.kb1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = tt.kb0; kb < tt.kb1; kb += 2 * FZ_CH) {
          fz_mma(acc, wA, xA, min(FZ_CH, tt.kb1 - kb));
          if (kb + 2 * FZ_CH < tt.kb1) {
            fz_load_w(wA, tt, kb + 2 * FZ_CH);
            fz_load_x(xA, xrow, kb + 2 * FZ_CH, tt.kb1);
          }
          if (kb + FZ_CH < tt.kb1) {
            fz_mma(acc, wB, xB, min(FZ_CH, tt.kb1 - kb - FZ_CH));
            if (kb + 3 * FZ_CH < tt.kb1) {
              fz_load_w(wB, tt, kb + 3 * FZ_CH);
              fz_load_x(xB, xrow, kb + 3 * FZ_CH, tt.kb1);
            }
          }
        }
        // the next tile's first weight chunks stream in during the reduction and epilogue
        if (tile + NWG < gm.ntiles) {
          const FzTile t1 = fz_tile(gm, type, tile + NWG, HD, p.F);
          fz_load_w(wA, t1, t1.kb0);
          fz_load_w(wB, t1, t1.kb0 + FZ_CH);
        }
        // reduce the 8 waves' partial tiles in a fixed order, then the epilogue
        const int wave = tid >> 6;
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.gm.red[wave][4 * kg + i][r] = acc[i];
        __syncthreads();
        if (type == PH_QKV || type == PH_GU) {
          if (tid < 128) {
            const int j = tid >> 4, m = tid & 15;
            if (m < Ma) {
              float a = 0.f, b = 0.f;
#pragma unroll
              for (int w = 0; w < FZ_NW; ++w) { a += sm.gm.red[w][j][m]; b += sm.gm.red[w][j + 8][m]; }
              a = __fmul_rn(a, sm.gm.inv[m]);
              b = __fmul_rn(b, sm.gm.inv[m]);
              if (type == PH_GU) {
                p.ab[(size_t)m * p.F + tile * 8 + j] = f2bf(swiglu(a, b));
              } else {
                const int tph = HD / 16;
                const int slot = tile / tph, i = (tile % tph) * 8 + j;   // head slot, rotation pair
                const int pm = p.pos[m];
                const int lp = pm / p.PS;
                if (lp >= p.n_lpages || pm < 0) {
                  atomicOr(p.err, ERRF_CAPACITY);
                } else {
                  if (slot < p.H + p.KVH) rope_apply(a, b, p.rope_cs[(size_t)pm * (HD / 2) + i], a, b);
                  bf16_t* dst;
                  if (slot < p.H) {
                    dst = p.qb + (size_t)m * p.H * HD + (size_t)slot * HD;
                  } else {
                    const int kvsel = slot < p.H + p.KVH ? 0 : 1;
                    const int g = slot - p.H - kvsel * p.KVH;
                    dst = p.pool + kv_index(p.page_table[lp], p.L, layer, kvsel, p.KVH, g, p.PS, pm % p.PS, HD);
                  }
                  dst[i] = f2bf(a);
                  dst[i + HD / 2] = f2bf(b);
                }
              }
            }
          }
        } else if (tid < 256) {
          const int m = tid >> 4, c = tid & 15;
          const int col = tile * 16 + c;
          float sacc = 0.f;
#pragma unroll
          for (int w = 0; w < FZ_NW; ++w) sacc += sm.gm.red[w][c][m];
          if (type == PH_LM) {
            if (m < Ma && col < p.V) p.logits[(size_t)m * p.V + col] = __fmul_rn(sacc, sm.gm.inv[m]);
          } else {
            // residual add, the next projection's bf16(h * gain), and the group sum of h^2
            float hv = 0.f;
            if (m < Ma) {
              hv = __fadd_rn(p.h[(size_t)m * p.D + col], sacc);
              p.h[(size_t)m * p.D + col] = hv;
              const float* gain = p.ph_gain[ph];
              if (gain) p.xg[(size_t)m * p.D + col] = f2bf(__fmul_rn(hv, gain[col]));
            }
            const float s = tile16_ss_lanes(hv);
            if (m < Ma && c == 0) p.ss[tile * 16 + m] = s;
          }
        }
        __syncthreads();
      }
      if (done) fz_publish(p.counters + ph, done, &sh_old);
    }
  }

  // the last workgroup out clears the counters for the next pass
  fz_publish(exit_ctr, 1u, &sh_old);
  if (sh_old == (unsigned)NWG - 1) {
    const int n = p.n_phase + 1 + attn_idx * p.KVH;
    for (int i = tid; i < n; i += FZ_NT) p.counters[i] = 0u;
  }
}

int launch_fused_pass(const FzParams& prm, int head_dim, int nwg, hipStream_t s) {
  FzParams p = prm;
  void* args[] = {(void*)&p};
  hipError_t e;
  if (head_dim == 128)
    e = hipLaunchCooperativeKernel((const void*)fused_pass_kernel<128>, dim3(nwg), dim3(FZ_NT), args, 0, s);
  else
    e = hipLaunchCooperativeKernel((const void*)fused_pass_kernel<64>, dim3(nwg), dim3(FZ_NT), args, 0, s);
  return e == hipSuccess ? 0 : SSD_ERR_HIP;
}

int fused_pass_max_blocks_per_cu(int head_dim, int* blocks) {
  hipError_t e;
  if (head_dim == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, (const void*)fused_pass_kernel<128>, FZ_NT, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, (const void*)fused_pass_kernel<64>, FZ_NT, 0);
  return e == hipSuccess ? 0 : SSD_ERR_HIP;
}

}  // namespace ssd
