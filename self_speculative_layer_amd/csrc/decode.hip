// Decode-mode kernels: a block of at most 16 rows (one draft token, or the
// d' + 1 rows of a verify pass) through the decoder with the small steps
// folded into the projections, so that a layer takes five launches:
//
//   QKV projection    normalised input bf16(h * gain / rms) from the RMSNorm
//                     tile sums, RoPE, q store and
//                     K/V append to the paged cache in the epilogue
//   attention         split partials; the last split of a (row block, KV head)
//                     to finish merges them
//   O projection      residual add, then the next RMSNorm consumer's input
//                     (h * gain in fp32 and the 16-feature tile sums of h^2)
//   gate/up           normalised input, SwiGLU
//   down projection   residual add, next consumer's input
//
// The arithmetic of every output element is the same as in the general
// kernels (kernels.hip), step for step: same K slices per wave, same
// reduction order, same rounding of the epilogues, same canonical RMS sums.
// A row's result never depends on the other rows of its block.
#include <hip/hip_ext.h>
#include <math.h>

#include <type_traits>

#include "kernels.h"
#include "attn.h"

namespace ssd {

typedef uint32_t dec_u32x4 __attribute__((ext_vector_type(4)));
typedef float dec_f32x8 __attribute__((ext_vector_type(8)));

// B operand (8 consecutive k of one row) of a normalised input: bf16((h * gain) * inv_rms).
__device__ __forceinline__ dec_u32x4 norm_operand(const dec_f32x8& v, float inv) {
  return dec_u32x4{norm_pack2(v[0], v[1], inv), norm_pack2(v[2], v[3], inv), norm_pack2(v[4], v[5], inv),
                   norm_pack2(v[6], v[7], inv)};
}

static inline int dec_ok(hipError_t e) { return e == hipSuccess ? 0 : SSD_ERR_HIP; }

constexpr int DEC_U = 8;      // 32-element K steps each wave keeps in flight
// Waves per workgroup.  Each wave owns a contiguous quarter of K, as in the general projection kernel
// (GEMM_NW), so the two give the same bits for a row; measured against 8 and 16 waves per tile on the
// 7B shapes, 4 was fastest for every matrix.
constexpr int DEC_NW = 4;
constexpr int DEC_SSP = 8;    // RMS tile sums per lane and row: K <= 64 * 16 * DEC_SSP
constexpr int DEC_AX = 4;     // activation steps in flight (fp32 normalised inputs)

// ===========================================================================
// Projection Y[M, N] = X[M, K] . W[N, K]^T for M <= 16, bf16 operands, fp32
// accumulation on the matrix cores (v_mfma_f32_16x16x32_bf16: weights as A,
// 16 features x 32 k; activations as B, 32 k x 16 rows).
//
// A workgroup owns one tile of 16 output features (two row sets of W for the
// SwiGLU and QKV epilogues) and all of K.  Its NW waves take contiguous
// 64-element slices of K; each wave keeps DEC_U steps (one contiguous 1 KB
// tile of each weight set per step, packed layout) in flight in registers and
// reloads a step's registers as soon as its MFMA has been issued.  The
// per-wave tiles are reduced through LDS in wave order.  Rows >= M repeat row
// M - 1's activations and rows past the active count read what their rows
// hold (no masking on the load path); neither is stored.
//
// RMSNorm consumers (QKV, gate/up, LM head) read the fp32 rows h * gain and
// the rows' tile sums of h^2: the row scale 1 / rms is formed before the
// stream starts (while the first weight steps are in flight), and each step's
// B operand is bf16(h * gain * inv), so the projection sees the normalised
// input rounded once, as the plain definition has it.
// ===========================================================================

// Per-tile output rows: f0 + i (and f1 + i for the two-set epilogues); for QKV also the head slot and
// the pair index base d0.
struct DecTile {
  int f0, f1, slot, d0;
};

template <int EPI, bool HALF>
__device__ __forceinline__ DecTile dec_tile(const DecGemm& a, int tile) {
  constexpr int SET = HALF ? 8 : 16;
  DecTile t{0, 0, 0, 0};
  if (EPI == DEC_QKV) {
    const int per = a.HD / (2 * SET);           // tiles per head slot: pairs (i, i + HD/2), i in [d0, d0 + SET)
    t.slot = tile / per;
    t.d0 = (tile % per) * SET;
    t.f0 = t.slot * a.HD + t.d0;
    t.f1 = t.f0 + a.HD / 2;
  } else {
    t.f0 = tile * SET;
    t.f1 = a.N + t.f0;                          // SwiGLU: the up rows follow the N gate rows
  }
  return t;
}

// TPW tiles per workgroup share each activation load (fewer activation reads
// per weight byte when M > 1); the arithmetic of an output element does not
// depend on TPW.
// DEVROWS: the active-row count is a device value (a.nrows); otherwise all M rows are active.
// ROW1 (a one-row block, M = 1): the fp32 normalised input is stored row-major (a step's 32 elements are
// one 128-byte line instead of four 16-byte pieces 256 bytes apart).
template <int EPI, int NW, bool HALF, int TPW, bool DEVROWS, bool ROW1>
__global__ __launch_bounds__(NW * 64) void dec_gemm_kernel(const DecGemm a) {
  // The stop flag and the active-row count travel with the first weight steps: the weight loads are
  // issued before anything waits for them.  Activation rows are clamped to the active rows (rows past
  // them would only add distinct lines to every step's loads); only rows < Ma are stored.
  const int stopv = a.stop ? *a.stop : 0;
  const int Ma = DEVROWS ? min(a.M, *a.nrows) : a.M;
  constexpr bool TWO = EPI == DEC_SWIGLU || EPI == DEC_QKV;   // outputs combine two W row sets
  constexpr bool DUAL = TWO && !HALF;                           // 16 + 16 rows: two accumulators
  static_assert(!HALF || TWO, "half tiles pair two row sets");
  constexpr bool NORM = EPI != DEC_RESID;
  constexpr int SPT = DUAL ? 2 : 1;             // accumulators (16-row W sets) per tile
  constexpr int NS = TPW * SPT;
  constexpr int U = NS <= 2 ? DEC_U : DEC_U / 2;
  constexpr int RPW = (16 + NW - 1) / NW;       // rows whose scale one wave computes
  const int K = a.K;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int ntiles = (int)gridDim.x * TPW;      // grid covers the tiles; a tile past the last one
  (void)ntiles;                                 // repeats the last (its outputs are not stored)

  // W rows: set (j, 0) = f0 + r (HALF: f0 + r for r < 8, f1 + r - 8 after), set (j, 1) = f1 + r
  const bf16_t* wp[NS];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const DecTile t = dec_tile<EPI, HALF>(a, min((int)blockIdx.x * TPW + j, a.n_tiles - 1));
    int wrow = t.f0 + r;
    if (HALF) wrow = (r < 8 ? t.f0 : t.f1) + (r & 7);
    if (EPI == DEC_STORE) wrow = min(wrow, a.N - 1);   // rows past N repeat the last W row; not stored
    wp[j * SPT] = a.W + wpk_index(wrow, g * 8, K);                  // step t: + 512 t
    if (DUAL) wp[j * SPT + 1] = a.W + wpk_index(t.f1 + r, g * 8, K);
  }
  typedef typename std::conditional<NORM, float, bf16_t>::type XT;
  typedef typename std::conditional<NORM, dec_f32x8, dec_u32x4>::type XR;
  const XT* xp = nullptr;                       // this lane's activation row (set once Ma is known)

  // Epilogue operands that do not depend on the product (the residual element and the next gain; the
  // row's position) are loaded ahead of the weight stream, so that the tail after the reduction holds
  // no dependent global loads.  Thread (erow, enn) of the epilogue; clamped rows are not stored.
  const int erow = min((int)threadIdx.x >> 4, a.M - 1), enn = threadIdx.x & 15;
  float eh[TPW], eg[TPW];
  int epos = 0;
  if constexpr (EPI == DEC_RESID) {
    const float* gsrc = a.gain_next ? a.gain_next : a.Y;     // unconditional load; unused without gain_next
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int col = dec_tile<EPI, HALF>(a, min((int)blockIdx.x * TPW + j, a.n_tiles - 1)).f0 + enn;
      eh[j] = a.Y[(size_t)erow * a.ldy + col];
      eg[j] = gsrc[col];
    }
  }
  int eside = 0x7fffffff;                     // QKV: first tree-leaf row (its keys and values go to side_kv)
  if constexpr (EPI == DEC_QKV) {
    epos = a.pos[erow];
    if (a.side_from) eside = *a.side_from;
  }

  __shared__ float sinv[16];
  const int nts = K / 16;
  float ssv[RPW][DEC_SSP];

  const int nu = K >> 6;
  const int s0 = 2 * ((nu * wave) / NW);
  const int n = 2 * ((nu * (wave + 1)) / NW) - s0;   // 32-element steps of this wave (>= 2)
  // activation steps in flight: the fp32 rows of a normalised input come from the L2 (the previous
  // kernel wrote them), so a few steps ahead cover their latency and keep the registers for the weights
  constexpr int AX = NORM && DEC_AX < U ? DEC_AX : U;
  static_assert(U % AX == 0, "activation slots divide the weight slots");
  dec_u32x4 w[NS][U];
  XR xa[AX];
  auto wload = [&](int u, int step) {
#pragma unroll
    for (int j = 0; j < NS; ++j) w[j][u] = *(const dec_u32x4*)(wp[j] + (size_t)(s0 + step) * 512);
  };
  auto xload = [&](int slot, int step) {
    if constexpr (NORM) {
      constexpr int STEP = ROW1 ? 32 : 512, HI = ROW1 ? 4 : 256;
      const f32x4 lo = *(const f32x4*)(xp + (size_t)(s0 + step) * STEP);
      const f32x4 hi = *(const f32x4*)(xp + (size_t)(s0 + step) * STEP + HI);
      xa[slot] = dec_f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      xa[slot] = *(const XR*)(xp + (size_t)(s0 + step) * 512);
    }
  };
  // Activations of row r (clamped to the active rows), k = 8g..8g+7 of each step (step t at + 512 t), and
  // the RMS tile sums of the rows this wave scales.
  auto act_setup = [&]() {
    if constexpr (NORM && ROW1) xp = a.Xf + g * 8;                            // + 4: k = 8g + 4 .. 8g + 7
    else if constexpr (NORM) xp = a.Xf + dec_actf_index(min(r, Ma - 1), g * 8);   // + 256: k = 8g + 4 .. 8g + 7
    else xp = a.X + dec_act_index(min(r, Ma - 1), g * 8);
    if constexpr (NORM) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int row = min(wave + i * NW, Ma - 1);
#pragma unroll
        for (int j = 0; j < DEC_SSP; ++j) ssv[i][j] = a.ss[(size_t)row * nts + min(lane + 64 * j, nts - 1)];
      }
    }
  };
  if constexpr (DEVROWS) {
    // the active-row count is a device value: every weight step is issued before its load is waited for
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wload(u, min(u, n - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
    act_setup();
#pragma unroll
    for (int u = 0; u < AX; ++u) {
      xload(u, min(u, n - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // all M rows are active: the steady loop's load order from the first step
    act_setup();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wload(u, min(u, n - 1));
      if (u < AX) xload(u, min(u, n - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (stopv || Ma <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no wave ends with loads in flight
    return;
  }
  if (a.prof_ran && blockIdx.x == 0 && threadIdx.x == 0) *a.prof_ran = 1;   // timing record: this launch ran

  if constexpr (NORM) {
    // canonical order: lane j adds tiles j, j + 64, ... then a butterfly over the wave
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = wave + i * NW;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < DEC_SSP; ++j)   // tiles past the row end add an exact 0 (keeps every load unconditional)
        acc += fmul_nc(ssv[i][j], lane + 64 * j < nts ? 1.f : 0.f);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, WAVE);
      if (row < Ma && lane == 0) sinv[row] = inv_rms(acc, K, a.eps);
    }
  }
  float xinv = 1.f;                             // the scale of this lane's activation row
  if constexpr (NORM) {
    __syncthreads();
    xinv = sinv[min(r, Ma - 1)];
  }
  // QKV: the row's page and rotation, issued behind the first weight steps (only the position load
  // is waited for here)
  float2 ecs[TPW];
  int epage = 0;
  if constexpr (EPI == DEC_QKV) {
    const int lp = epos / a.PS;
    const bool ok = epos >= 0 && lp < a.n_lpages;
    epage = a.page_table[ok ? lp : 0];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const DecTile t = dec_tile<EPI, HALF>(a, min((int)blockIdx.x * TPW + j, a.n_tiles - 1));
      ecs[j] = a.rope_cs[(size_t)(ok ? epos : 0) * (a.HD / 2) + t.d0 + (HALF ? (enn & 7) : enn)];
    }
  }

  f32x4 acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // steps are consumed in increasing order; the steady loop has no branches, so the compiler's
  // wait before each step's MFMAs leaves the later steps' loads in flight.  Step t sits in weight
  // slot t % U and activation slot t % AX.
  auto consume = [&](int u) {
    dec_u32x4 xb;
    if constexpr (NORM) xb = norm_operand(xa[u % AX], xinv);
    else xb = xa[u % AX];
#pragma unroll
    for (int j = 0; j < NS; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[j][u]),
                                                       __builtin_bit_cast(bf16x8, xb), acc[j], 0, 0, 0);
  };
  const int nfull = n / U, rem = n - nfull * U;
  for (int b = 1; b < nfull; ++b) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      consume(u);                                // step (b - 1) U + u
      xload(u % AX, (b - 1) * U + u + AX);       // < n: AX <= U
      wload(u, b * U + u);
      __builtin_amdgcn_sched_barrier(0);     // keep the issue order: one step's MFMAs, then its reloads
    }
  }
  if (nfull > 0) {
    if (rem > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        consume(u);
        xload(u % AX, min((nfull - 1) * U + u + AX, n - 1));
        wload(u, min(nfull * U + u, n - 1));
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        consume(u);
        if (u + AX < U) xload(u % AX, (nfull - 1) * U + u + AX);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < rem) {
      consume(u);                                // step nfull U + u
      if constexpr (AX < U) xload(u % AX, min(nfull * U + u + AX, n - 1));
    }

  // acc[j][i] holds D[feature 4g + i][row r] of set j
  __shared__ float red[NS][NW][16][17];
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[j][wave][4 * g + i][r] = acc[j][i];
  __syncthreads();
  if (threadIdx.x >= 256) return;
  const int row = threadIdx.x >> 4, nn = threadIdx.x & 15;
  if (row >= Ma) return;                        // uniform over each group of 16 lanes
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tile = (int)blockIdx.x * TPW + j;
    if (tile >= a.n_tiles) break;
    if (HALF && nn >= 8) break;
    const DecTile t = dec_tile<EPI, HALF>(a, tile);
    float s = 0.f, s2 = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      s += red[j * SPT][ww][nn][row];
      if (DUAL) s2 += red[j * SPT + 1][ww][nn][row];
      if (HALF) s2 += red[j][ww][nn + 8][row];
    }
    if constexpr (EPI == DEC_STORE) {
      if (t.f0 + nn < a.N) a.Y[(size_t)row * a.ldy + t.f0 + nn] = s;
    } else if constexpr (EPI == DEC_RESID) {
      const int col = t.f0 + nn;
      const float hn = fadd_nc(eh[j], s);
      a.Y[(size_t)row * a.ldy + col] = hn;
      if (a.y_copy) a.y_copy[(size_t)row * a.ldy + col] = hn;
      if (a.gain_next) {
        a.xg_next[a.M == 1 ? col : dec_actf_index(row, col)] = fmul_nc(hn, eg[j]);   // one-row blocks: row-major
        const float tt = tile16_ss_lanes(hn);
        if (nn == 0) a.ss_next[(size_t)row * (a.N / 16) + col / 16] = tt;
      }
    } else if constexpr (EPI == DEC_SWIGLU) {
      st(a.A + dec_act_index(row, t.f0 + nn), swiglu(s, s2));
    } else {
      const float x1 = s, x2 = s2;
      const int HD = a.HD, H = a.H, KVH = a.KVH;
      const int i = t.d0 + nn;                  // pair index
      const int p = epos;                       // row == erow here (row < Ma)
      const int lp = p / a.PS;
      if (p < 0 || lp >= a.n_lpages) {
        if (nn == 0) atomicOr(a.err, ERRF_CAPACITY);
        continue;
      }
      bf16_t* dst;
      if (t.slot < H) {
        dst = a.q + (size_t)row * a.ldq + (size_t)t.slot * HD;
      } else {
        const int kvsel = t.slot < H + KVH ? 0 : 1;
        const int gg = t.slot - H - kvsel * KVH;
        dst = row >= eside ? a.side_kv + ((size_t)(row - eside) * 2 + kvsel) * KVH * HD + (size_t)gg * HD
                           : a.pool + kv_index(epage, a.L, a.layer, kvsel, KVH, gg, a.PS, p % a.PS, HD);
      }
      if (t.slot < H + KVH) {
        float y1, y2;
        rope_apply(x1, x2, ecs[j], y1, y2);
        st(dst + i, y1);
        st(dst + i + HD / 2, y2);
      } else {
        st(dst + i, x1);
        st(dst + i + HD / 2, x2);
      }
    }
  }
}

bool profile_next(int cls, hipEvent_t* start, hipEvent_t* stop, int** ran);
void profile_done(double bytes, const int* stop_flag, bool self_marked, hipStream_t s);

// Tile shapes of the two-set projections (HALF: 8 + 8 rows per tile, twice the tiles).
constexpr bool DEC_HALF_QKV = true;
constexpr bool DEC_HALF_SWIGLU = false;

static int dec_tiles(int epi, int N) {
  if (epi == DEC_QKV) return DEC_HALF_QKV ? N / 16 : N / 32;
  if (epi == DEC_SWIGLU) return DEC_HALF_SWIGLU ? N / 8 : N / 16;
  return (N + 15) / 16;
}

// Compute units of the current device (cached per device).
static int dec_device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// Tiles per workgroup.  One-row blocks: one (most workgroups in flight; the
// row's activation loads are one line per step and cost next to nothing).
// Blocks of several rows fetch a 16-row fp32 activation step (2 KB) for every
// 1 KB weight step, so the normalised-input projections (QKV, gate/up) let each
// activation load feed 3 or 4 tiles when that still leaves at most one
// workgroup per compute unit (7B at 13 rows: QKV 768 tiles -> 256 workgroups,
// 28.2 -> 23.6 us; gate/up 688 -> 230, 37.5 -> 36.2 us); with more tiles than
// four per unit (70B gate/up) the grid stays one tile per workgroup.  The LM
// head with several rows takes two tiles per workgroup (its 2000 tiles keep
// the chip busy).
static int dec_tpw(int epi, int M, int n_tiles) {
  if (M <= 1) return 1;
  if (epi == DEC_STORE) return 2;
  if (epi == DEC_QKV || epi == DEC_SWIGLU) {
    const int ncu = dec_device_cus();
    const int t = (n_tiles + ncu - 1) / ncu;
    if (t == 3 || t == 4) return t;
  }
  return 1;
}

// e0, e1: events taking the dispatch's begin and end timestamps (profiling), or null.
template <int EPI, bool HALF, bool DEVROWS>
static void dec_launch(const DecGemm& a, int tpw, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
  const dim3 block(DEC_NW * 64);
  if (EPI != DEC_RESID && a.M == 1)
    hipExtLaunchKernelGGL((dec_gemm_kernel<EPI, DEC_NW, HALF, 1, DEVROWS, true>), dim3(a.n_tiles), block, 0, s, e0,
                          e1, 0, a);
  else if (tpw == 2)
    hipExtLaunchKernelGGL((dec_gemm_kernel<EPI, DEC_NW, HALF, 2, DEVROWS, false>), dim3((a.n_tiles + 1) / 2), block,
                          0, s, e0, e1, 0, a);
  else if (EPI != DEC_QKV && EPI != DEC_SWIGLU)
    hipExtLaunchKernelGGL((dec_gemm_kernel<EPI, DEC_NW, HALF, 1, DEVROWS, false>), dim3(a.n_tiles), block, 0, s, e0,
                          e1, 0, a);
  else if (tpw == 3)
    hipExtLaunchKernelGGL((dec_gemm_kernel<EPI, DEC_NW, HALF, (EPI == DEC_QKV || EPI == DEC_SWIGLU) ? 3 : 1, DEVROWS,
                                           false>),
                          dim3((a.n_tiles + 2) / 3), block, 0, s, e0, e1, 0, a);
  else if (tpw == 4)
    hipExtLaunchKernelGGL((dec_gemm_kernel<EPI, DEC_NW, HALF, (EPI == DEC_QKV || EPI == DEC_SWIGLU) ? 4 : 1, DEVROWS,
                                           false>),
                          dim3((a.n_tiles + 3) / 4), block, 0, s, e0, e1, 0, a);
  else
    hipExtLaunchKernelGGL((dec_gemm_kernel<EPI, DEC_NW, HALF, 1, DEVROWS, false>), dim3(a.n_tiles), block, 0, s, e0,
                          e1, 0, a);
}

template <int EPI, bool HALF>
static void dec_launch(const DecGemm& a, int tpw, hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
  if (a.nrows) dec_launch<EPI, HALF, true>(a, tpw, e0, e1, s);
  else dec_launch<EPI, HALF, false>(a, tpw, e0, e1, s);
}

int launch_dec_gemm(int epi, const DecGemm& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return 0;
  if (a.M > 16 || (epi != DEC_STORE && a.N % 16 != 0) || a.K % 64 != 0) return SSD_ERR_SHAPE;
  if (epi != DEC_RESID && a.K > 64 * 16 * DEC_SSP) return SSD_ERR_SHAPE;
  if (epi == DEC_QKV && (a.HD % 32 != 0 || a.N % a.HD != 0)) return SSD_ERR_SHAPE;
  if (a.K / 64 < DEC_NW) return SSD_ERR_SHAPE;
  if (epi == DEC_SWIGLU && a.N % (DEC_HALF_SWIGLU ? 8 : 16) != 0) return SSD_ERR_SHAPE;
  DecGemm b = a;
  b.n_tiles = dec_tiles(epi, a.N);
  const int tpw = dec_tpw(epi, a.M, b.n_tiles);
  // profile classes: 0 plain-store projections (QKV, LM head), 1 residual, 2 gate/up
  const int cls = epi == DEC_RESID ? 1 : (epi == DEC_SWIGLU ? 2 : 0);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool prof = profile_next(cls, &e0, &e1, &b.prof_ran);
  switch (epi) {
    case DEC_STORE: dec_launch<DEC_STORE, false>(b, tpw, e0, e1, s); break;
    case DEC_RESID: dec_launch<DEC_RESID, false>(b, tpw, e0, e1, s); break;
    case DEC_SWIGLU: dec_launch<DEC_SWIGLU, DEC_HALF_SWIGLU>(b, tpw, e0, e1, s); break;
    default: dec_launch<DEC_QKV, DEC_HALF_QKV>(b, tpw, e0, e1, s);
  }
  if (prof) {
    // algorithmic bytes: weights once, activations in once, results out once (residual: read + write)
    const double M = a.M, N = a.N, K = a.K;
    const double wrows = epi == DEC_SWIGLU ? 2.0 * N : N;
    double by = wrows * K * 2.0 + M * K * (epi == DEC_RESID ? 2.0 : 4.0);
    by += epi == DEC_STORE ? 4.0 * M * N : (epi == DEC_RESID ? 8.0 * M * N : 2.0 * M * N);
    profile_done(by, a.stop, true, s);
  }
  return dec_ok(hipGetLastError());
}

// ===========================================================================
// Attention of a decode block with the split merge folded in: every work item
// writes its partial with device-scope stores and counts itself on the
// (row block, KV head) counter; the item that completes the count merges the
// rows' partials (in split order) and resets the counter for the next launch.
// Rows >= *side_from (tree leaves; side_from nullable) see the cache up to
// their position - 1 and their own key / value from side_kv.
// ===========================================================================

template <typename T, int HD, bool LEAF>
__global__ __launch_bounds__(256) void attn_dec_kernel(
    const T* __restrict__ q, int ldq, const T* __restrict__ pool, const int* __restrict__ page_table, int PS,
    int n_lpages, int L, int layer, int H, int KVH, int M, const int* __restrict__ nrows,
    const int* __restrict__ pos, int RB, int nsplit, float* __restrict__ part, T* __restrict__ out, int ldo,
    unsigned* __restrict__ counters, const int* __restrict__ stop, const int* __restrict__ side_from,
    const T* __restrict__ side_kv) {
  static_assert(sizeof(T) == 2, "bf16 items");
  const int g = blockIdx.x, s = blockIdx.y, rbk = blockIdx.z;
  const int r0 = rbk * RB;
  if (r0 >= M) return;
  const int side0 = LEAF ? *side_from : 0x7fffffff;
  __shared__ AttnSmem<T, HD, 4> sm;
  __shared__ int is_last;
  // the stop flag, the active-row count, the positions, the page ids and the queries arrive in one round
  // of loads; maxp: the largest position a row of the block sees (-1: nothing to do)
  int r1 = r0;
  const int maxp = attn_item_bf16<HD, 4, true, 1, AttnSmem<bf16_t, HD, 4>, LEAF>(
      sm, q, ldq, pool, page_table, PS, n_lpages, L, layer, H, KVH, M, nrows, pos, r0, RB, g, s, nsplit, nullptr, 0,
      0, part, side0, stop, &r1);
  if (maxp < 0) return;
  const int n_act = min(maxp / ATT_SPLIT + 1, nsplit);   // splits holding a key some row of the block sees
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* c = counters + (size_t)rbk * KVH + g;
    const unsigned old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = old + 1 == (unsigned)n_act;
    if (is_last) __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  attn_merge_block<HD, 4, LEAF>(sm, part, nsplit, r0, r1, H / KVH, g, H, out, side0, side_kv, q, ldq, KVH);
}

bool attention_dec_leaves_fit(int max_ctx) { return attention_nsplit(max_ctx) < ATT_MAXW; }

int launch_attention_dec(int head_dim, const void* q, int ldq, const KvView& kv, int L, int layer, int H, int KVH,
                         int M, const int* nrows, const int* pos, int max_ctx, float* part, void* out, int ldo,
                         unsigned* counters, const int* stop, hipStream_t s, const int* side_from,
                         const void* side_kv) {
  if (M <= 0) return 0;
  const int G = H / KVH;
  const int RB = ATTB_MAXQ / G;
  if (RB < 1 || M > 16) return SSD_ERR_SHAPE;
  const int nsplit = attention_nsplit(max_ctx);
  if (side_from && nsplit >= ATT_MAXW) return SSD_ERR_UNSUPPORTED;   // a leaf's own term takes one more slot
  if (nsplit > ATT_MAXW) {
    // longer contexts: partials, then one merge block per (row, head) (the general kernels)
    const RowBlock rb{M, nrows, pos, nullptr, stop};
    return launch_attention(SSD_DTYPE_BF16, head_dim, q, ldq, kv, L, layer, H, KVH, rb, max_ctx, nullptr, 0, 0, part,
                            out, ldo, s, true);
  }
  const dim3 grid(KVH, nsplit, (M + RB - 1) / RB);
#define ATT_DEC(HD, LF)                                                                                         \
  hipLaunchKernelGGL((attn_dec_kernel<bf16_t, HD, LF>), grid, dim3(256), 0, s, (const bf16_t*)q, ldq,            \
                     (const bf16_t*)kv.pool, kv.page_table, kv.page_size, kv.n_lpages, L, layer, H, KVH, M, nrows, \
                     pos, RB, nsplit, part, (bf16_t*)out, ldo, counters, stop, side_from, (const bf16_t*)side_kv)
  // leaf rows are a separate instantiation: the chain's launches keep the plain merge
  if (side_from) {
    if (head_dim == 128) ATT_DEC(128, true); else ATT_DEC(64, true);
  } else {
    if (head_dim == 128) ATT_DEC(128, false); else ATT_DEC(64, false);
  }
#undef ATT_DEC
  return dec_ok(hipGetLastError());
}

// ===========================================================================
// Rows entering a decode pass: h from the embedding (tokens) or from saved
// residual rows, plus the first RMSNorm consumer's input.
// ===========================================================================

// Row r of the entry: h[dr] from the embedding row e (EMB) or from sr, and with NORM the first consumer's
// input xg[dr] = h * gain (fp32) and the tile sums ss[dr].
template <bool EMB, bool NORM>
// row1: the row enters a one-row block (its consumer input is stored row-major).
__device__ __forceinline__ void dec_entry_row(const bf16_t* __restrict__ e, const float* __restrict__ sr, int dr,
                                              float* __restrict__ h, int D, const float* __restrict__ gain,
                                              float* __restrict__ xg, float* __restrict__ ss, bool row1) {
  float* hr = h + (size_t)dr * D;
  // D % 16 == 0: each group of 16 lanes is entirely inside or outside the row.  Loads are issued in
  // batches of 8 per thread before their first use.
  constexpr int PER = 8;
  for (int i0 = 0; i0 < D; i0 += 256 * PER) {
    float v[PER], gv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = min(i0 + j * 256 + (int)threadIdx.x, D - 1);
      v[j] = EMB ? bf2f(e[i]) : sr[i];
      if (NORM) gv[j] = gain[i];
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = i0 + j * 256 + threadIdx.x;
      if (i0 + j * 256 >= D) break;           // uniform
      if (i < D) hr[i] = v[j];
      if (NORM) {
        const float t = tile16_ss_lanes(v[j]);
        if (i < D) {
          xg[row1 ? i : dec_actf_index(dr, i)] = fmul_nc(v[j], gv[j]);   // one-row blocks: row-major
          if ((threadIdx.x & 15) == 0) ss[(size_t)dr * (D / 16) + i / 16] = t;
        }
      }
    }
  }
}

template <bool EMB, bool NORM>
__global__ __launch_bounds__(256) void dec_entry_kernel(const bf16_t* __restrict__ emb, const int* __restrict__ tokens,
                                                        int V, const float* __restrict__ src, int rows,
                                                        const int* __restrict__ count, const int* __restrict__ dst_off,
                                                        float* __restrict__ h, int D, const float* __restrict__ gain,
                                                        float* __restrict__ xg, float* __restrict__ ss,
                                                        const int* __restrict__ stop, int block_rows) {
  if (stop && *stop) return;
  const int r = blockIdx.x;
  const int n = count ? min(rows, *count) : rows;
  if (r >= n) return;
  const int dr = r + (dst_off ? *dst_off : 0);
  const bf16_t* e = EMB ? emb + (size_t)min(max(tokens[r], 0), V - 1) * D : nullptr;   // ids are produced in range
  dec_entry_row<EMB, NORM>(e, EMB ? nullptr : src + (size_t)r * D, dr, h, D, gain, xg, ss, block_rows == 1);
}

// Draft step j (1-based): the row y_{j-1} at position kvlen + j - 1 (y_0 = the last committed token).
// Out of KV pages (the verify needs position kvlen + d' as well) it ends the draft instead.  Writes
// the row's position and token (pos1, tok1) for the step's kernels.
template <bool NORM>
__global__ __launch_bounds__(256) void dec_draft_entry_kernel(DevState* __restrict__ st,
                                                              const int32_t* __restrict__ drafts, int j,
                                                              int* __restrict__ pos1, int* __restrict__ tok1,
                                                              int max_ctx, int32_t* __restrict__ n_drafted_out,
                                                              const bf16_t* __restrict__ emb, int V,
                                                              float* __restrict__ h, int D,
                                                              const float* __restrict__ gain,
                                                              float* __restrict__ xg, float* __restrict__ ss) {
  __shared__ int s_tok, s_ok;
  if (threadIdx.x == 0) {
    int ok = !st->stop, tok = 0;
    if (ok) {
      const int p = st->kvlen + j - 1;
      if (p + 1 >= max_ctx) {
        st->error_flags |= ERRF_CAPACITY;
        st->stop = 1;
        st->n_drafted = max(j - 1, 0);
        *n_drafted_out = max(j - 1, 0);
        ok = 0;
      } else {
        tok = j == 1 ? st->last_token : drafts[j - 2];
        pos1[0] = p;
        tok1[0] = tok;
      }
    }
    s_tok = tok;
    s_ok = ok;
  }
  __syncthreads();
  if (!s_ok) return;
  dec_entry_row<true, NORM>(emb + (size_t)min(max(s_tok, 0), V - 1) * D, nullptr, 0, h, D, gain, xg, ss, true);
}

int launch_dec_draft_entry(DevState* st, const int32_t* drafts, int j, int* pos1, int* tok1, int max_ctx,
                           int32_t* n_drafted_out, const void* emb, int V, float* h, int D, const float* gain,
                           void* xg, float* ss, hipStream_t s) {
  if (D % 16 != 0) return SSD_ERR_SHAPE;
#define DENTRY(N)                                                                                                 \
  hipLaunchKernelGGL((dec_draft_entry_kernel<N>), dim3(1), dim3(256), 0, s, st, drafts, j, pos1, tok1, max_ctx,  \
                     n_drafted_out, (const bf16_t*)emb, V, h, D, gain, (float*)xg, ss)
  if (gain) DENTRY(true); else DENTRY(false);
#undef DENTRY
  return dec_ok(hipGetLastError());
}

int launch_dec_entry(const void* emb, const int* tokens, int V, const float* src, int rows, const int* count,
                     const int* dst_off, float* h, int D, const float* gain, void* xg, float* ss, const int* stop,
                     int block_rows, hipStream_t s) {
  if (rows <= 0) return 0;
  if (D % 16 != 0) return SSD_ERR_SHAPE;
#define ENTRY(E, N)                                                                                              \
  hipLaunchKernelGGL((dec_entry_kernel<E, N>), dim3(rows), dim3(256), 0, s, (const bf16_t*)emb, tokens, V, src,  \
                     rows, count, dst_off, h, D, gain, (float*)xg, ss, stop, block_rows)
  if (tokens) {
    if (gain) ENTRY(true, true); else ENTRY(true, false);
  } else {
    if (gain) ENTRY(false, true); else ENTRY(false, false);
  }
#undef ENTRY
  return dec_ok(hipGetLastError());
}

}  // namespace ssd
