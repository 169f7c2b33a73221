// Persistent decode pass (bf16): one cooperative launch runs a whole forward
// pass of at most 16 rows -- an embedding or residual input, a list of
// attention / MLP sub-layers, and optionally the shared final norm + LM head.
//
// One workgroup per CU with two kinds of waves:
//   * four streaming waves (one per SIMD) turn weight tiles into partial
//     products.  Each owns a ring of FZ_S slots in LDS; a slot receives one
//     k-block of 16 weight rows x 32 columns and the matching 16 x 32 block of
//     activations through direct global->LDS loads (global_load_lds, 16 bytes
//     per lane), so up to FZ_S k-blocks per wave are in flight without holding
//     registers.  The wave waits for a slot with an explicit vmcnt that it
//     derives from the order in which it issued its loads, then feeds the slot
//     to v_mfma_f32_16x16x32_bf16.  Streaming waves never store to global
//     memory during a projection phase and never execute a fence there, so
//     nothing drains their load queue: at the end of a projection phase they
//     already request the weights of the next projection phase, which stream
//     in while the grid synchronises (weights never depend on activations).
//   * one control wave waits for and publishes the phase counters (device-scope
//     acquire / release), forms the per-row 1/rms, and runs every projection
//     epilogue (fixed-order sum of the four partial tiles, RMS scale, RoPE,
//     SwiGLU, residual add, next sub-layer's bf16(h * gain), group sums of
//     h^2, logits).
// The embedding and attention phases use all five waves.
//
// A pass is a sequence of phases:
//   INIT  rows -> residual h, bf16(h * gain) for the first projection, group sums of h^2
//   QKV   projection tiles; epilogue: 1/rms scale, RoPE, q -> buffer, k/v -> paged cache
//   ATTN  (KV head, key split, row block) items; the last item of a head merges its splits
//   O     projection tiles; epilogue: h += o Wo^T, bf16(h * next gain), group sums of h^2
//   GU    gate/up tiles (8 gate rows + 8 up rows); epilogue: 1/rms scale, SwiGLU
//   DOWN  like O
//   LM    LM-head tiles; epilogue: 1/rms scale, logits
// A phase's items are dealt round-robin to workgroups.  A workgroup publishes
// the number of items it finished in a phase with one device-scope release;
// the next phase reads those results after a device-scope acquire of that
// counter.
//
// The projection tiles split K over the four streaming waves exactly as the
// standalone linear-layer kernel does (same slices, same k order, same
// fixed-order reduction), attention uses the standalone attention kernel's
// arithmetic for a one-chunk split, and the epilogues use the same rounding
// steps, so a pass gives the same bits as the standalone kernels.
//
// Every wait is bounded: past a spin limit it sets an error flag and goes on,
// so the grid always drains.
#include "kernels.h"
#include "attn.h"

namespace ssd {

constexpr int FZ_SW = 4;                        // streaming waves
constexpr int FZ_CW = FZ_SW;                    // wave index of the control wave
constexpr int FZ_NWV = FZ_SW + 1;
constexpr int FZ_NT = FZ_NWV * 64;
constexpr int FZ_S = 12;                        // ring slots per streaming wave
constexpr int FZ_CPOL_NT = 2;                   // cache policy of the weight stream: non-temporal
constexpr uint32_t FZ_SPIN_LIMIT = 1u << 23;    // x ~0.1-0.5 us sleeps: a few seconds at most

static_assert(ATT_SPLIT == ATT_CHUNK, "the persistent pass stages one chunk per key split");

typedef uint32_t fz_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void fz_lds_t;

// Wave index as a wave-uniform (scalar) value, so that everything derived from
// it -- k-slices, unit counters, wait counts -- stays in scalar registers and
// scalar branches.
__device__ __forceinline__ int fz_wave() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// A pointer or count that is the same in every lane (read from memory with a
// vector load), moved to scalar registers so that buffer resources built from
// it stay scalar.
template <typename T>
__device__ __forceinline__ T* fz_uniform(T* ptr) {
  const uint64_t v = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

template <int HD>
struct FzAttnSmem {
  static constexpr int VPR = HD / 8;            // 16-byte chunks per key row
  alignas(16) bf16_t Qs[ATT_MAXQ * HD];
  // chunk c of key t at chunk slot t * VPR + (c ^ (t % VPR)): rows are written by
  // direct global->LDS loads (contiguous 16-byte slots), and the XOR keeps both
  // the per-key 16-byte reads and the per-dimension reads free of bank conflicts
  alignas(16) bf16_t Ks[ATT_CHUNK * HD];
  alignas(16) bf16_t Vs[ATT_CHUNK * HD];
  float Pw[FZ_NWV][ATT_CHUNK];
};

template <int HD>
__device__ __forceinline__ int fz_kv_slot(int t, int c) {
  constexpr int VPR = HD / 8;
  return t * VPR + (c ^ (t & (VPR - 1)));
}

template <int HD>
struct FzSmem {
  alignas(16) unsigned char ring[FZ_SW][FZ_S][2][1024];   // [wave][slot][weights | activations]
  float red[2][FZ_SW][16][17];                            // partial tiles of the streaming waves
  float inv[16];
  int pos[16];
  int page[16];                                           // physical page of each row's position (-1: none)
  unsigned old;
  unsigned ready;                                         // partial tiles deposited (4 per item)
  unsigned consumed;                                      // items whose partial tiles the control wave has read
  FzAttnSmem<HD> att;
};

// ---------------------------------------------------------------------------
// Waits and publication

template <int N>
__device__ __forceinline__ void fz_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most n vector-memory operations of this wave are outstanding
// (rounded down to one of four levels: a few scalar branches per k-block).
__device__ __forceinline__ void fz_wait_vm(int n) {
  if (n >= 2 * FZ_S - 2) fz_vmcnt<2 * FZ_S - 2>();
  else if (n >= FZ_S - 1) fz_vmcnt<FZ_S - 1>();
  else if (n >= (FZ_S - 1) / 2) fz_vmcnt<(FZ_S - 1) / 2>();
  else fz_vmcnt<0>();
}

__device__ __forceinline__ void fz_vm_drain() { fz_vmcnt<0>(); }
__device__ __forceinline__ void fz_lgkm_drain() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS data only.  __syncthreads() also orders global
// memory, and the compiler implements that by waiting for every outstanding
// vector-memory operation -- including a streaming wave's queued weight loads.
// The projection phases exchange data through LDS only (partial tiles), so
// they synchronise with this barrier.
__device__ __forceinline__ void fz_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Hand-off of partial tiles from the streaming waves to the control wave
// through two LDS buffers and two LDS counters, without a workgroup barrier:
// a streaming wave that finishes its share of item ib deposits it as soon as
// the control wave has read item ib - 2 (same buffer), and the control wave
// starts the epilogue of item ib once all four shares are in.  Waves thus
// never wait for each other between tiles.
__device__ __forceinline__ unsigned fz_lds_load(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Bounded like every other wait: past the limit it flags a timeout and goes on.
__device__ __forceinline__ bool fz_spin_ok(uint32_t& spins, int* err) {
  __builtin_amdgcn_s_sleep(1);
  if (++spins <= FZ_SPIN_LIMIT) return true;
  if ((threadIdx.x & 63) == 0) atomicOr(err, ERRF_TIMEOUT);
  return false;
}

template <typename Smem>
__device__ __forceinline__ void fz_deposit(Smem& sm, unsigned ib, int wave, const f32x4& acc, int* err) {
  const int lane = threadIdx.x & 63;
  uint32_t spins = 0;
  while (fz_lds_load(&sm.consumed) + 2u <= ib && fz_spin_ok(spins, err)) {
  }
  fz_lgkm_drain();
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.red[ib & 1][wave][4 * (lane >> 4) + i][lane & 15] = acc[i];
  fz_lgkm_drain();
  if (lane == 0) __hip_atomic_fetch_add(&sm.ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <typename Smem>
__device__ __forceinline__ void fz_await_item(Smem& sm, unsigned ib, int* err) {
  uint32_t spins = 0;
  while (fz_lds_load(&sm.ready) < (unsigned)FZ_SW * (ib + 1u) && fz_spin_ok(spins, err)) {
  }
  fz_lgkm_drain();
}

template <typename Smem>
__device__ __forceinline__ void fz_release_item(Smem& sm, unsigned ib) {
  fz_lgkm_drain();
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(&sm.consumed, ib + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Data that another workgroup reads within the same pass is stored with
// device-coherent stores (sc1: written through to the device's coherence
// point), so publishing it needs no cache write-back: each wave waits for its
// own stores (vmcnt) before the barrier that precedes the control wave's
// counter update.
__device__ __forceinline__ void fz_st(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fz_st(bf16_t* p, bf16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Control wave: device-scope acquire -- invalidates the CU's vector cache and
// the non-coherent lines of its L2, which every wave of the workgroup shares,
// so the loads of all waves that follow the next barrier see published data.
__device__ __forceinline__ void fz_acquire_fence() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  fz_vm_drain();
}

// Phase counters: every workgroup arrives once per phase.  Workgroup w counts
// on group counter w % FZ_GROUPS; the last arrival of a group bumps the phase's
// top counter, so no counter sees more than 32 contending atomics.
__device__ __forceinline__ unsigned* fz_phase_ctr(const FzParams& p, int ph) { return p.counters + ph * (1 + FZ_GROUPS); }

// Control wave: arrival of this workgroup at the end of phase ph (its stores complete).
__device__ __forceinline__ void fz_arrive(const FzParams& p, int ph) {
  fz_vm_drain();
  if ((threadIdx.x & 63) == 0) {
    const int NWG = gridDim.x, grp = blockIdx.x % FZ_GROUPS;
    const unsigned gsize = (unsigned)((NWG - grp + FZ_GROUPS - 1) / FZ_GROUPS);
    unsigned* c = fz_phase_ctr(p, ph);
    const unsigned old = __hip_atomic_fetch_add(c + 1 + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1 == gsize) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Control wave: waits until every workgroup has arrived at the end of phase ph, then acquires.
__device__ __forceinline__ void fz_wait_phase(const FzParams& p, int ph) {
  if ((threadIdx.x & 63) == 0) {
    const unsigned target = (unsigned)min((int)gridDim.x, FZ_GROUPS);
    unsigned* c = fz_phase_ctr(p, ph);
    uint32_t spins = 0;
    while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > FZ_SPIN_LIMIT) {
        atomicOr(p.err, ERRF_TIMEOUT);
        break;
      }
    }
  }
  fz_acquire_fence();
}

// ---------------------------------------------------------------------------
// Projection geometry

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

__device__ __forceinline__ int fz_ntiles(const FzParams& p, int type) {
  const int qd = p.H * p.HD, kvd = p.KVH * p.HD;
  switch (type) {
    case PH_QKV: return (qd + 2 * kvd) / 16;
    case PH_O: return p.D / 16;
    case PH_GU: return p.F / 8;
    case PH_DOWN: return p.D / 16;
    default: return (p.V + 15) / 16;
  }
}

__device__ __forceinline__ bool fz_is_gemm(int type) {
  return type == PH_QKV || type == PH_O || type == PH_GU || type == PH_DOWN || type == PH_LM;
}

// The streaming waves read weights and activations with buffer loads to LDS:
// a buffer resource per matrix (base, size in bytes), a per-lane 32-bit byte
// offset and a wave-uniform offset for the k-block, so a k-block costs two
// scalar adds and one load instruction.  A lane whose activation row is >= Ma
// reads past the resource's end and receives zeros (bounds-checked buffer
// access), which keeps those MFMA columns finite without an exec mask.
constexpr int FZ_RSRC_WORD3 = 0x00020000;       // raw buffer, 32-bit data format

struct FzGeo {
  __amdgpu_buffer_rsrc_t rw, rx;
  const bf16_t* W;
  int type, K, nrow_w, ntiles;
  int kb0, nw;        // this streaming wave's k-blocks [kb0, kb0 + nw) of every tile
  int nit;            // tiles of this workgroup
  int total;          // units (k-blocks) of this wave in the phase: nit * nw
  uint32_t voff_x;    // this lane's activation offset (bytes) at the slice start
};

__device__ __forceinline__ FzGeo fz_geo(const FzParams& p, int type, int layer, int wave, int Ma) {
  FzGeo g;
  const int qd = p.H * p.HD, kvd = p.KVH * p.HD;
  const bf16_t* X;
  g.type = type;
  switch (type) {
    case PH_QKV: g.W = p.layers[layer].w_qkv; X = p.xg; g.K = p.D; g.nrow_w = qd + 2 * kvd; break;
    case PH_O: g.W = p.layers[layer].w_o; X = p.ob; g.K = qd; g.nrow_w = p.D; break;
    case PH_GU: g.W = p.layers[layer].w_gate_up; X = p.xg; g.K = p.D; g.nrow_w = 2 * p.F; break;
    case PH_DOWN: g.W = p.layers[layer].w_down; X = p.ab; g.K = p.F; g.nrow_w = p.D; break;
    default: g.W = p.lm_head; X = p.xg; g.K = p.D; g.nrow_w = p.V; break;
  }
  g.ntiles = fz_ntiles(p, type);
  const int nu = g.K >> 6;
  g.kb0 = 2 * ((nu * wave) / FZ_SW);
  g.nw = 2 * ((nu * (wave + 1)) / FZ_SW) - g.kb0;
  const int wg = blockIdx.x, NWG = gridDim.x;
  g.nit = wg < g.ntiles ? (g.ntiles - wg + NWG - 1) / NWG : 0;
  g.total = g.nit * g.nw;
  g.W = fz_uniform(g.W);
  g.rw = __builtin_amdgcn_make_buffer_rsrc((void*)g.W, (short)0, (int)min((size_t)g.nrow_w * g.K * 2, (size_t)0x7FFFFFFF),
                                           FZ_RSRC_WORD3);
  g.rx = __builtin_amdgcn_make_buffer_rsrc((void*)fz_uniform(X), (short)0,
                                           __builtin_amdgcn_readfirstlane(Ma * g.K * 2), FZ_RSRC_WORD3);
  const int lane = threadIdx.x & 63;
  g.voff_x = (uint32_t)((lane & 15) * g.K * 2 + (lane >> 4) * 16 + g.kb0 * 64);
  return g;
}

// A streaming wave's position in its unit sequence: unit u = item j (tile
// wg + j * NWG), k-block kbi of the wave's slice.
struct FzCur {
  int u, j, kbi;
  uint32_t voff;      // this lane's weight offset (bytes): its row of the current tile at the slice start
};

__device__ __forceinline__ uint32_t fz_wvoff(const FzGeo& g, int tile, int HD, int F) {
  const int lane = threadIdx.x & 63;
  const int row = fz_wrow(g.type, tile, lane & 15, HD, F);
  // a row past the matrix (last LM tile) reads past the resource: zeros, discarded outputs
  if (row >= g.nrow_w) return 0xFFFFF000u;
  return (uint32_t)row * (uint32_t)g.K * 2u + (uint32_t)((lane >> 4) * 16 + g.kb0 * 64);
}

__device__ __forceinline__ void fz_cur_init(FzCur& c, const FzGeo& g, int HD, int F) {
  c.u = 0;
  c.j = 0;
  c.kbi = 0;
  c.voff = fz_wvoff(g, blockIdx.x, HD, F);
}

__device__ __forceinline__ void fz_cur_next(FzCur& c, const FzGeo& g, int HD, int F) {
  ++c.u;
  if (++c.kbi == g.nw) {
    c.kbi = 0;
    ++c.j;
    const int tile = blockIdx.x + c.j * gridDim.x;
    if (tile < g.ntiles) c.voff = fz_wvoff(g, tile, HD, F);
  }
}

// ring: this wave's ring in LDS, FZ_S slots of (weights 1 KB, activations 1 KB)
__device__ __forceinline__ void fz_issue_w(unsigned char* ring, unsigned slot, const FzGeo& g, const FzCur& c) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rw, (fz_lds_t*)(ring + slot * 2048), 16, c.voff, c.kbi * 64, 0,
                                           FZ_CPOL_NT);
}

__device__ __forceinline__ void fz_issue_x(unsigned char* ring, unsigned slot, const FzGeo& g, const FzCur& c) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rx, (fz_lds_t*)(ring + slot * 2048 + 1024), 16, g.voff_x, c.kbi * 64, 0,
                                           0);
}

// ---------------------------------------------------------------------------
// Control-wave helpers

// 1/rms of rows m < Ma from the group sums ss[t][m] (canonical reduction:
// lane j adds groups j, j + 64, ... in order, then a butterfly over 64 lanes).
__device__ __forceinline__ void fz_row_inv(const FzParams& p, int Ma, float* inv) {
  const int lane = threadIdx.x & 63;
  const int ntiles = p.D / 16;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.f;
  for (int t = lane; t < ntiles; t += 64) {
    const fz_u32x4* src = (const fz_u32x4*)(p.ss + (size_t)t * 16);
    fz_u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[i];
#pragma unroll
    for (int m = 0; m < 16; ++m) acc[m] += __uint_as_float(v[m >> 2][m & 3]);
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    float a = acc[m];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, WAVE);
    if (lane == m) inv[m] = m < Ma ? inv_rms(a, p.D, p.eps) : 1.f;
  }
}

// Inputs of an item's epilogue that do not depend on its partial sums,
// requested ahead of the barrier that delivers those sums.
struct FzPre {
  float v[4];       // residual: h values; QKV: (cos, sin) of two elements
  float gn[4];      // residual: the next sub-layer's gain
};

template <int HD>
__device__ __forceinline__ void fz_epi_prefetch(const FzParams& p, const FzSmem<HD>& sm, int type, int tile, int Ma,
                                                const float* gain, FzPre& pre) {
  const int lane = threadIdx.x & 63;
  if (type == PH_QKV) {
    const int tph = HD / 16;
    const int slot = tile / tph;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = lane + 64 * q, j = e >> 4, m = e & 15;
      pre.v[2 * q] = 1.f;
      pre.v[2 * q + 1] = 0.f;
      if (m < Ma && slot < p.H + p.KVH && sm.page[m] >= 0) {
        const float2 cs = p.rope_cs[(size_t)sm.pos[m] * (HD / 2) + (tile % tph) * 8 + j];
        pre.v[2 * q] = cs.x;
        pre.v[2 * q + 1] = cs.y;
      }
    }
  } else if (type == PH_O || type == PH_DOWN) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 4 * q + (lane >> 4), col = tile * 16 + (lane & 15);
      pre.v[q] = m < Ma ? p.h[(size_t)m * p.D + col] : 0.f;     // after the acquire
      pre.gn[q] = gain ? gain[col] : 0.f;
    }
  }
}

template <int HD>
__device__ __forceinline__ void fz_epilogue(const FzParams& p, const FzSmem<HD>& sm, int type, int layer, int tile,
                                            int Ma, const float* gain, bool save, int buf, const FzPre& pre) {
  const int lane = threadIdx.x & 63;
  if (type == PH_QKV || type == PH_GU) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = lane + 64 * q, j = e >> 4, m = e & 15;
      if (m >= Ma) continue;
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int w = 0; w < FZ_SW; ++w) {
        a += sm.red[buf][w][j][m];
        b += sm.red[buf][w][j + 8][m];
      }
      a = __fmul_rn(a, sm.inv[m]);
      b = __fmul_rn(b, sm.inv[m]);
      if (type == PH_GU) {
        fz_st(p.ab + (size_t)m * p.F + tile * 8 + j, f2bf(swiglu(a, b)));
      } else {
        const int tph = HD / 16;
        const int slot = tile / tph, i = (tile % tph) * 8 + j;   // head slot, rotation pair
        const int page = sm.page[m];
        if (page < 0) {
          atomicOr(p.err, ERRF_CAPACITY);
          continue;
        }
        if (slot < p.H + p.KVH) rope_apply(a, b, make_float2(pre.v[2 * q], pre.v[2 * q + 1]), a, b);
        bf16_t* dst;
        if (slot < p.H) {
          dst = p.qb + (size_t)m * p.H * HD + (size_t)slot * HD;
        } else {
          const int kvsel = slot < p.H + p.KVH ? 0 : 1;
          const int g = slot - p.H - kvsel * p.KVH;
          dst = p.pool + kv_index(page, p.L, layer, kvsel, p.KVH, g, p.PS, sm.pos[m] % p.PS, HD);
        }
        fz_st(dst + i, f2bf(a));
        fz_st(dst + i + HD / 2, f2bf(b));
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 4 * q + (lane >> 4), c = lane & 15;
      const int col = tile * 16 + c;
      float sacc = 0.f;
#pragma unroll
      for (int w = 0; w < FZ_SW; ++w) sacc += sm.red[buf][w][c][m];
      if (type == PH_LM) {
        if (m < Ma && col < p.V) p.logits[(size_t)m * p.V + col] = __fmul_rn(sacc, sm.inv[m]);
      } else {
        // residual add, the next projection's bf16(h * gain), and the group sum of h^2
        float hv = 0.f;
        if (m < Ma) {
          hv = __fadd_rn(pre.v[q], sacc);
          fz_st(p.h + (size_t)m * p.D + col, hv);
          if (save) p.save_h[(size_t)m * p.D + col] = hv;
          if (gain) fz_st(p.xg + (size_t)m * p.D + col, f2bf(__fmul_rn(hv, pre.gn[q])));
        }
        const float s = tile16_ss_lanes(hv);
        if (m < Ma && c == 0) fz_st(p.ss + tile * 16 + m, s);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Attention items: KV head g, key split s (one 64-key chunk), rows r0..r1-1.
// Same arithmetic as the standalone attention kernel for a one-chunk split
// (online softmax from an empty state).

struct FzAttnItem {
  int g, s, r0, r1, key_beg, key_end;
};

__device__ __forceinline__ FzAttnItem fz_attn_geo(int t, int KVH, int nsplit_act, int RB, int Ma, const int* spos) {
  FzAttnItem it;
  it.g = t % KVH;
  const int rest = t / KVH;
  it.s = rest % nsplit_act;
  it.r0 = (rest / nsplit_act) * RB;
  it.r1 = min(it.r0 + RB, Ma);
  it.key_beg = it.s * ATT_SPLIT;
  it.key_end = min(it.key_beg + ATT_SPLIT, spos[it.r1 - 1] + 1);
  return it;
}

// Page id of the item's i-th page (PS divides 64: at most 64 / PS pages) in lane i.
__device__ __forceinline__ int fz_attn_pages(const FzParams& p, const FzAttnItem& it) {
  const int lane = threadIdx.x & 63;
  return (lane * p.PS < ATT_CHUNK && it.key_beg + lane * p.PS < it.key_end) ? p.page_table[it.key_beg / p.PS + lane]
                                                                            : 0;
}

// Requests the cached keys and values of the item (positions below cached_end,
// written by earlier launches) with direct global->LDS loads: instruction q of
// 2 * 64 * VPR / 64 fills 64 consecutive chunk slots; waves part, part + nparts, ...
template <int HD>
__device__ __forceinline__ void fz_attn_issue_cached(FzAttnSmem<HD>& sm, const FzParams& p, int layer,
                                                     const FzAttnItem& it, int pg, int cached_end, int part,
                                                     int nparts) {
  constexpr int VPR = HD / 8;
  constexpr int HALF = ATT_CHUNK * VPR / 64;          // instructions per matrix
  const int lane = threadIdx.x & 63;
  for (int q = part; q < 2 * HALF; q += nparts) {
    const int kv = q / HALF, base = (q % HALF) * 64;
    if (it.key_beg + base / VPR >= cached_end) continue;     // no key of this instruction is cached (uniform)
    const int P = base + lane;
    const int t = P / VPR, c = (P % VPR) ^ (t & (VPR - 1));
    const int kp = it.key_beg + t;
    const int page = __shfl(pg, t / p.PS, 64);
    bf16_t* dst = (kv ? sm.Vs : sm.Ks) + base * 8;
    if (kp < cached_end)
      __builtin_amdgcn_global_load_lds((const void*)(p.pool + kv_index(page, p.L, layer, kv, p.KVH, it.g, p.PS,
                                                                       kp % p.PS, HD) + c * 8),
                                       (fz_lds_t*)dst, 16, 0, 0);
  }
}

// The rest of the item with all five waves, after the QKV phase is complete and
// the cached keys are in LDS: queries and this pass's keys/values (positions
// >= pos0) into LDS, zero values past the chunk's last key, then the softmax
// partials.  Writes the partial (o[HD], m, l) of every (row, head) whose
// position reaches the split.
template <int HD>
__device__ void fz_attn_finish(FzAttnSmem<HD>& sm, const FzParams& p, const int* spos, int layer,
                               const FzAttnItem& it, int pg, int pos0) {
  constexpr int VPR = HD / 8;
  constexpr int NEWV = 16 * 2 * VPR;                  // this pass's keys: at most 16 rows
  constexpr int PER = (ATT_MAXQ * VPR + NEWV + FZ_NT - 1) / FZ_NT;
  const int G = p.H / p.KVH;
  const int nq = (it.r1 - it.r0) * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = fz_wave();
  const int nqv = nq * VPR;
  const int new_beg = max(it.key_beg, pos0);
  const int nnew = max(it.key_end - new_beg, 0);
  const int per_mat = nnew * VPR;                    // chunks of this pass's keys per matrix
  const int nnv = 2 * per_mat;
  fz_u32x4 v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid + FZ_NT * j;
    const int e2 = e - nqv;
    const bool isnew = e >= nqv && e2 < nnv;
    const int kv = isnew ? e2 / per_mat : 0, r2 = isnew ? e2 % per_mat : 0;
    const int t = new_beg - it.key_beg + r2 / VPR, c = r2 % VPR;
    const int page = __shfl(pg, t / p.PS, 64);
    v[j] = fz_u32x4{0u, 0u, 0u, 0u};
    if (e < nqv) {
      const int qi = e / VPR, cq = e % VPR;
      const int row = it.r0 + qi / G, head = it.g * G + qi % G;
      v[j] = *(const fz_u32x4*)(p.qb + (size_t)row * p.H * HD + (size_t)head * HD + cq * 8);
    } else if (isnew) {
      const int kp = it.key_beg + t;
      v[j] = *(const fz_u32x4*)(p.pool + kv_index(page, p.L, layer, kv, p.KVH, it.g, p.PS, kp % p.PS, HD) + c * 8);
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = tid + FZ_NT * j;
    const int e2 = e - nqv;
    if (e < nqv) {
      *(fz_u32x4*)(sm.Qs + e * 8) = v[j];
    } else if (e2 < nnv) {
      const int kv = e2 / per_mat, r2 = e2 % per_mat;
      const int t = new_beg - it.key_beg + r2 / VPR, c = r2 % VPR;
      *(fz_u32x4*)((kv ? sm.Vs : sm.Ks) + fz_kv_slot<HD>(t, c) * 8) = v[j];
    }
  }
  // values of keys past the chunk end are read (with weight 0) by the weighted sum: keep them finite
  const int nkeys = it.key_end - it.key_beg;
  for (int e = nkeys * VPR + tid; e < ATT_CHUNK * VPR; e += FZ_NT) *(fz_u32x4*)(sm.Vs + e * 8) = fz_u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)HD);
  for (int qi = wave; qi < nq; qi += FZ_NWV) {
    const int row = it.r0 + qi / G, head = it.g * G + qi % G;
    const int prow = spos[row];
    if (it.key_beg > prow) continue;               // the row sees no key of this split (wave-uniform)
    const int kp = it.key_beg + lane;
    const bool valid = kp < it.key_end && kp <= prow;
    float sc = -INFINITY;
    if (valid) {
      float acc = 0.f;
      const bf16_t* qr = sm.Qs + qi * HD;
#pragma unroll 4
      for (int c = 0; c < VPR; ++c) {
        const fz_u32x4 k8 = *(const fz_u32x4*)(sm.Ks + fz_kv_slot<HD>(lane, c) * 8);
        const fz_u32x4 q8 = *(const fz_u32x4*)(qr + c * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc = fmaf(__uint_as_float(q8[w] << 16), __uint_as_float(k8[w] << 16), acc);
          acc = fmaf(__uint_as_float(q8[w] & 0xFFFF0000u), __uint_as_float(k8[w] & 0xFFFF0000u), acc);
        }
      }
      sc = __fmul_rn(acc, scale);
    }
    const float mx = wave_max(sc);
    const float pexp = valid ? expf(__fsub_rn(sc, mx)) : 0.f;
    const float psum = wave_sum(pexp);
    sm.Pw[wave][lane] = pexp;
    __builtin_amdgcn_wave_barrier();
    float* dstp = p.part + (((size_t)row * p.H + head) * p.nsplit_max + it.s) * (HD + 2);
    // weighted sum of the values: lane owns HD / 64 consecutive dimensions; 16 keys' values
    // are read before their 16 multiply-adds (one LDS round trip per 16 keys, not per key)
    constexpr int DPL = HD / 64;
    const int d0 = lane * DPL;
    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = 0.f;
#pragma unroll 1
    for (int t0 = 0; t0 < ATT_CHUNK; t0 += 16) {
      uint32_t vv[16];
      float pw[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const bf16_t* src = sm.Vs + fz_kv_slot<HD>(t0 + u, d0 >> 3) * 8 + (d0 & 7);
        vv[u] = DPL == 2 ? *(const uint32_t*)src : (uint32_t)*src;
        pw[u] = sm.Pw[wave][t0 + u];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        o[0] = fmaf(pw[u], __uint_as_float(vv[u] << 16), o[0]);
        if (DPL == 2) o[DPL - 1] = fmaf(pw[u], __uint_as_float(vv[u] & 0xFFFF0000u), o[DPL - 1]);
      }
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) fz_st(dstp + d0 + i, o[i]);
    if (lane == 0) {
      fz_st(dstp + HD, mx);
      fz_st(dstp + HD + 1, psum);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------

template <int HD>
__global__ __launch_bounds__(FZ_NT, 1) void fused_pass_kernel(FzParams p) {
  // the next pass uses the other counter set: clear it (the pass that used it last has ended)
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < p.n_counters; i += FZ_NT) p.counters_next[i] = 0u;
  if (p.stop && *p.stop) return;
  __shared__ FzSmem<HD> sm;
  const int NWG = gridDim.x, wg = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = fz_wave();
  const bool ctrl = wave == FZ_CW;
  const int Ma = p.nrows ? min(p.M, *p.nrows) : p.M;
  const int G = p.H / p.KVH;
  const int RB = min(16, ATT_MAXQ / G);
  const int nrb = (Ma + RB - 1) / RB;
  unsigned* const head_ctr = p.counters + p.n_counters - p.L * p.KVH;

  if (ctrl && lane < 16) {
    int pm = 0, page = -1;
    if (lane < Ma) {
      pm = p.pos[lane];
      const int lp = pm / p.PS;
      if (pm >= 0 && lp < p.n_lpages) page = p.page_table[lp];
    }
    sm.pos[lane] = pm;
    sm.page[lane] = page;
    if (lane == 0) {
      sm.ready = 0u;
      sm.consumed = 0u;
    }
  }
  __syncthreads();
  const int nsplit_act = sm.pos[Ma - 1] / ATT_SPLIT + 1;
  const int ntask = p.KVH * nsplit_act * nrb;              // attention items of every attention phase
  // page ids of this workgroup's first attention item (the same item in every layer)
  const int pg_first = wg < ntask ? fz_attn_pages(p, fz_attn_geo(wg, p.KVH, nsplit_act, RB, Ma, sm.pos)) : 0;
  bool kv_pending = false;

  // streaming-wave state
  unsigned n_iss = 0;      // DMA operations issued by this wave
  unsigned gpos = 0;       // ring position of the current projection phase's unit 0
  int pre = 0;             // units of the coming projection phase whose weights are requested
  unsigned ib = 0;         // items (projection tiles) of this pass so far
  int attn_idx = 0;

  for (int ph = 0; ph < p.n_phase; ++ph) {
    const int type = p.ph_type[ph];
    const int layer = p.ph_layer[ph];

    if (type == PH_INIT) {
      const float* gain = p.ph_gain[ph];
      const bool save = ph == p.save_phase;
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
            if (!p.h_in || p.h_in != p.h) fz_st(p.h + (size_t)m * p.D + i, v);
            if (save) p.save_h[(size_t)m * p.D + i] = v;
            if (gain) fz_st(p.xg + (size_t)m * p.D + i, f2bf(__fmul_rn(v, gain[i])));
            if ((i & 15) == 0) fz_st(p.ss + (i >> 4) * 16 + m, s);
          }
        }
      }
      (void)done;
      fz_vm_drain();
      __syncthreads();
      if (ctrl) fz_arrive(p, ph);
    } else if (type == PH_ATTN) {
      if (ctrl) fz_wait_phase(p, ph - 1);
      // the first item's cached keys were requested at the start of the QKV phase; a streaming
      // wave that consumed no block of that phase has not waited for them yet
      if (kv_pending) fz_vm_drain();
      kv_pending = false;
      __syncthreads();
      const unsigned per_head = nsplit_act * nrb;
      int combined = 0;
      for (int t = wg; t < ntask; t += NWG) {
        const FzAttnItem it = fz_attn_geo(t, p.KVH, nsplit_act, RB, Ma, sm.pos);
        const bool first = t == wg;
        const int pg = first ? pg_first : fz_attn_pages(p, it);
        if (!first) {
          fz_attn_issue_cached(sm.att, p, layer, it, pg, min(it.key_end, sm.pos[0]), wave, FZ_NWV);
          fz_vm_drain();
          __syncthreads();
        }
        if (it.key_beg <= sm.pos[it.r1 - 1]) fz_attn_finish<HD>(sm.att, p, sm.pos, layer, it, pg, sm.pos[0]);
        // the last item of head g merges its splits
        const int g = it.g;
        fz_vm_drain();
        __syncthreads();
        if (ctrl) {
          unsigned old = 0;
          if (lane == 0)
            old = __hip_atomic_fetch_add(head_ctr + attn_idx * p.KVH + g, 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
          old = __shfl(old, 0, 64);
          if (old == per_head - 1) fz_acquire_fence();
          if (lane == 0) sm.old = old;
        }
        __syncthreads();
        if (sm.old == per_head - 1) {
          for (int e = tid; e < Ma * G * HD; e += FZ_NT) {
            const int d = e % HD, j = (e / HD) % G, r = e / (HD * G);
            const float o = attn_combine_value<HD>(p.part, p.nsplit_max, r, g * G + j, p.H, sm.pos[r], d);
            fz_st(p.ob + (size_t)r * p.H * HD + (size_t)(g * G + j) * HD + d, f2bf(o));
          }
          ++combined;
          fz_vm_drain();
        }
        __syncthreads();
      }
      (void)combined;
      if (ctrl) fz_arrive(p, ph);
      ++attn_idx;
    } else {
      // ---------------------------------------------------------------- projection phase
      const float* gain = p.ph_gain[ph];
      int nph = ph + 1;                          // the next projection phase
      while (nph < p.n_phase && !fz_is_gemm(p.ph_type[nph])) ++nph;
      const bool has_next = nph < p.n_phase;
      const int ntiles = fz_ntiles(p, type);
      const int nit = wg < ntiles ? (ntiles - wg + NWG - 1) / NWG : 0;
      if (!ctrl) {
        const FzGeo g = fz_geo(p, type, layer, wave, Ma);
        unsigned char* const ring = &sm.ring[wave][0][0][0];
        const int k = min(FZ_S, g.total);
        FzCur ci;
        fz_cur_init(ci, g, HD, p.F);
        for (int i = 0; i < pre; ++i) fz_cur_next(ci, g, HD, p.F);
        for (; ci.u < k; fz_cur_next(ci, g, HD, p.F)) {
          fz_issue_w(ring, (gpos + ci.u) % FZ_S, g, ci);
          ++n_iss;
        }
        // the cached keys/values of this workgroup's first item of the coming attention phase
        // (they do not depend on this phase); the activation loads below are issued later and
        // complete after them, so waiting for the first block also covers these
        if (type == PH_QKV && wg < ntask) {
          const FzAttnItem it0 = fz_attn_geo(wg, p.KVH, nsplit_act, RB, Ma, sm.pos);
          fz_attn_issue_cached(sm.att, p, layer, it0, pg_first, min(it0.key_end, sm.pos[0]), wave, FZ_SW);
          kv_pending = g.total == 0;
        }
        fz_lds_barrier();                                  // GO: the previous phase is complete
        const unsigned xs0 = n_iss;
        {
          FzCur cx;
          fz_cur_init(cx, g, HD, p.F);
          for (; cx.u < k; fz_cur_next(cx, g, HD, p.F)) {
            fz_issue_x(ring, (gpos + cx.u) % FZ_S, g, cx);
            ++n_iss;
          }
        }
        const unsigned rs0 = n_iss;
        // Unit u of this phase: its activation load has sequence number xs0 + u
        // (u < k) or rs0 + 2 (u - k) + 1 (its refill pair, issued after unit u - S).
        // The next phase's unit jn goes to slot (gpos + total + jn) % S once this
        // phase's unit total + jn - S, which holds that slot, has been consumed.
        FzGeo gn{};
        FzCur cn{};
        int kn = 0;
        if (has_next) {
          gn = fz_geo(p, p.ph_type[nph], p.ph_layer[nph], wave, Ma);
          kn = min(FZ_S, gn.total);
          fz_cur_init(cn, gn, HD, p.F);
          for (; cn.u < kn && g.total + cn.u - FZ_S < 0; fz_cur_next(cn, gn, HD, p.F)) {
            fz_issue_w(ring, (gpos + g.total + cn.u) % FZ_S, gn, cn);
            ++n_iss;
          }
        }
        if (g.nw == 0) {
          for (int it = 0; it < nit; ++it, ++ib) fz_deposit(sm, ib, wave, f32x4{0.f, 0.f, 0.f, 0.f}, p.err);
        } else {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          int left = g.nw;                                 // units left in the current item
          unsigned slot = gpos % FZ_S;
          // main part: every unit's slot is refilled with unit u + S of this phase.  The wait for
          // unit u: its activation load was issued in the prologue batch (u < S: at least S - 1
          // loads issued after it) or as a refill pair S units ago (exactly 2 (S - 1) after it).
          const int main_end = g.total - FZ_S;             // < 0 when the phase has fewer than S units
          int u = 0;
          for (; u < main_end; ++u, slot = slot + 1 == FZ_S ? 0 : slot + 1) {
            if (u < FZ_S) fz_vmcnt<FZ_S - 1>();
            else fz_vmcnt<2 * FZ_S - 2>();
            const fz_u32x4 a = *(const fz_u32x4*)(ring + slot * 2048 + lane * 16);
            const fz_u32x4 b = *(const fz_u32x4*)(ring + slot * 2048 + 1024 + lane * 16);
            fz_lgkm_drain();                               // the slot is read before it is refilled
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
            fz_issue_w(ring, slot, g, ci);
            fz_issue_x(ring, slot, g, ci);
            fz_cur_next(ci, g, HD, p.F);
            if (--left == 0) {
              left = g.nw;
              fz_deposit(sm, ib++, wave, acc, p.err);
              acc = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
          n_iss += 2u * (unsigned)max(main_end, 0);
          // tail: no refill of this phase; the freed slots take the next phase's weights
          for (; u < g.total; ++u, slot = slot + 1 == FZ_S ? 0 : slot + 1) {
            const unsigned seqx = u < k ? xs0 + (unsigned)u : rs0 + 2u * (unsigned)(u - k) + 1u;
            fz_wait_vm((int)(n_iss - seqx - 1u));
            const fz_u32x4 a = *(const fz_u32x4*)(ring + slot * 2048 + lane * 16);
            const fz_u32x4 b = *(const fz_u32x4*)(ring + slot * 2048 + 1024 + lane * 16);
            fz_lgkm_drain();
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
            for (; cn.u < kn && g.total + cn.u - FZ_S <= u; fz_cur_next(cn, gn, HD, p.F)) {
              fz_issue_w(ring, (gpos + g.total + cn.u) % FZ_S, gn, cn);
              ++n_iss;
            }
            if (--left == 0) {
              left = g.nw;
              fz_deposit(sm, ib++, wave, acc, p.err);
              acc = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
        for (; cn.u < kn; fz_cur_next(cn, gn, HD, p.F)) {
          fz_issue_w(ring, (gpos + g.total + cn.u) % FZ_S, gn, cn);
          ++n_iss;
        }
        gpos += g.total;
        pre = kn;
      } else {
        // control wave: every workgroup has finished the previous phase
        fz_wait_phase(p, ph - 1);
        fz_lds_barrier();                                  // GO: the streaming waves start now
        // the 1/rms of the rows and the first epilogue's inputs load while the first tile streams
        const bool scaled = type == PH_QKV || type == PH_GU || type == PH_LM;
        if (scaled) fz_row_inv(p, Ma, sm.inv);
        FzPre pf;
        if (nit > 0) fz_epi_prefetch(p, sm, type, wg, Ma, gain, pf);
        const bool save = ph == p.save_phase;
        for (int it = 0; it < nit; ++it, ++ib) {
          const int tile = wg + it * NWG;
          const FzPre cur = pf;
          if (it + 1 < nit) fz_epi_prefetch(p, sm, type, tile + NWG, Ma, gain, pf);
          fz_await_item(sm, ib, p.err);
          fz_epilogue(p, sm, type, layer, tile, Ma, gain, save, ib & 1, cur);
          fz_release_item(sm, ib);
        }
        if (ph + 1 < p.n_phase) fz_arrive(p, ph);      // nothing waits for the last phase
      }
    }
  }

  fz_vm_drain();
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
