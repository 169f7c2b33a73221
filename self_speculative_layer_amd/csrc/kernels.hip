// HIP kernels of the self-speculative decoding path, written for gfx950
// (CDNA4: 64-lane wavefronts, bf16 MFMA 16x16x32, 160 KB LDS per CU).
#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>

#include "kernels.h"
#include "attn.h"

namespace ssd {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

static inline int hip_ok(hipError_t e) { return e == hipSuccess ? 0 : SSD_ERR_HIP; }
static inline int last_launch() { return hip_ok(hipGetLastError()); }

__device__ __forceinline__ int active_rows(int M, const int* nrows) {
  return nrows ? min(M, *nrows) : M;
}


// ===========================================================================
// Linear layers, bf16: Y[M, N] = X[M, K] . W[N, K]^T with fp32 accumulation on
// the matrix cores (W in the packed tile layout, wpk_index).  Weight-streaming design for few rows: a workgroup owns 16
// output features for a 16-row block and all of K; its NW waves split K into
// contiguous 64-element slices (each weight row is read as whole 128-byte
// lines by one wave), accumulate with v_mfma_f32_16x16x32_bf16 (weights as
// the A operand: 16 features x 32 k; activations as B: 32 k x 16 rows), then
// reduce the per-wave tiles through LDS in a fixed order.  The reduction order
// of an output element never depends on M, so a row's result is the same
// whatever rows it is batched with.
// ===========================================================================

constexpr int GEMM_NW = 4;
constexpr int GEMM_U = 8;

template <int EPI>
__global__ __launch_bounds__(GEMM_NW * 64) void gemm_bf16_rows16(
    const bf16_t* __restrict__ W, const bf16_t* __restrict__ X, int ldx, int M, int N, int K,
    float* __restrict__ Y, int ldy, bf16_t* __restrict__ A, int lda, int n_rb, const float* __restrict__ rscale,
    const int* __restrict__ nrows, const int* __restrict__ ymap, const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int Ma = active_rows(M, nrows);
  const int rb = blockIdx.x % n_rb;
  const int tile = blockIdx.x / n_rb;
  const int m0 = rb * 16;
  if (m0 >= Ma) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = tile * 16;
  const int nrow = n0 + r;
  const bool wv = nrow < N;
  const bf16_t* wp = W + wpk_index(wv ? nrow : 0, g * 8, K);     // packed: step kb at + 512 kb
  const bf16_t* wp2 = W + wpk_index((wv ? nrow : 0) + N, g * 8, K);   // up rows (EPI_SWIGLU)
  const int m = m0 + r;
  const bool xv = m < Ma;
  const bf16_t* xp = X + (size_t)(xv ? m : 0) * ldx + g * 8;

  const int nu = K >> 6;                       // 64-element units of K
  const int kb_beg = 2 * ((nu * wave) / GEMM_NW);
  const int kb_end = 2 * ((nu * (wave + 1)) / GEMM_NW);
  const u32x4 zero = {0u, 0u, 0u, 0u};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
  int kb = kb_beg;
  for (; kb + GEMM_U <= kb_end; kb += GEMM_U) {
    u32x4 wa[GEMM_U], wb[GEMM_U], xa[GEMM_U];
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      wa[u] = wv ? *(const u32x4*)(wp + (size_t)(kb + u) * 512) : zero;
      if (EPI == EPI_SWIGLU) wb[u] = wv ? *(const u32x4*)(wp2 + (size_t)(kb + u) * 512) : zero;
      xa[u] = xv ? *(const u32x4*)(xp + (kb + u) * 32) : zero;
    }
#pragma unroll
    for (int u = 0; u < GEMM_U; ++u) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[u]),
                                                    __builtin_bit_cast(bf16x8, xa[u]), acc, 0, 0, 0);
      if (EPI == EPI_SWIGLU)
        acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wb[u]),
                                                       __builtin_bit_cast(bf16x8, xa[u]), acc2, 0, 0, 0);
    }
  }
  for (; kb < kb_end; ++kb) {
    u32x4 wa = wv ? *(const u32x4*)(wp + (size_t)kb * 512) : zero;
    u32x4 xa = xv ? *(const u32x4*)(xp + kb * 32) : zero;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa),
                                                  __builtin_bit_cast(bf16x8, xa), acc, 0, 0, 0);
    if (EPI == EPI_SWIGLU) {
      u32x4 wb = wv ? *(const u32x4*)(wp2 + (size_t)kb * 512) : zero;
      acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wb),
                                                     __builtin_bit_cast(bf16x8, xa), acc2, 0, 0, 0);
    }
  }
  // acc[i] holds D[feature 4g + i][row r].
  constexpr int NT = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ float red[NT][GEMM_NW][16][17];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[0][wave][4 * g + i][r] = acc[i];
    if (EPI == EPI_SWIGLU) red[NT - 1][wave][4 * g + i][r] = acc2[i];
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    const int mm = threadIdx.x >> 4, nn = threadIdx.x & 15;
    const int row = m0 + mm, col = n0 + nn;
    if (row < Ma && col < N) {
      float s = 0.f, s2 = 0.f;
#pragma unroll
      for (int w = 0; w < GEMM_NW; ++w) {
        s += red[0][w][nn][mm];
        if (EPI == EPI_SWIGLU) s2 += red[NT - 1][w][nn][mm];
      }
      if (rscale && EPI != EPI_RESID) { s = fmul_nc(s, rscale[row]); s2 = fmul_nc(s2, rscale[row]); }
      const int yrow = ymap ? ymap[row] : row;
      if (EPI == EPI_STORE) Y[(size_t)yrow * ldy + col] = s;
      else if (EPI == EPI_RESID) Y[(size_t)yrow * ldy + col] = fadd_nc(Y[(size_t)yrow * ldy + col], s);
      else A[(size_t)row * lda + col] = f2bf(swiglu(s, s2));
    }
  }
}

// fp32 linear layer (the fp32 workload): plain FMAs.  A workgroup owns 16
// output features (4 per wave) and a 16-row block; lanes stride K, each lane
// sums its k in order, then a fixed butterfly reduces across lanes.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_rows16(
    const float* __restrict__ W, const float* __restrict__ X, int ldx, int M, int N, int K,
    float* __restrict__ Y, int ldy, float* __restrict__ A, int lda, int n_rb, const float* __restrict__ rscale,
    const int* __restrict__ nrows, const int* __restrict__ ymap, const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int Ma = active_rows(M, nrows);
  const int rb = blockIdx.x % n_rb;
  const int tile = blockIdx.x / n_rb;
  const int m0 = rb * 16;
  if (m0 >= Ma) return;
  const int mcount = min(16, Ma - m0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int c = 0; c < 4; ++c) {
    const int col = tile * 16 + wave * 4 + c;
    if (col >= N) break;
    float acc[16], acc2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc[i] = 0.f; acc2[i] = 0.f; }
    const float* w = W + (size_t)col * K;
    const float* w2 = w + (size_t)N * K;
    for (int k = lane; k < K; k += 64) {
      const float a = w[k];
      const float a2 = (EPI == EPI_SWIGLU) ? w2[k] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < mcount) {
          const float xv = X[(size_t)(m0 + i) * ldx + k];
          acc[i] = fmaf(a, xv, acc[i]);
          if (EPI == EPI_SWIGLU) acc2[i] = fmaf(a2, xv, acc2[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < mcount) {
        float s = wave_sum(acc[i]);
        float s2 = (EPI == EPI_SWIGLU) ? wave_sum(acc2[i]) : 0.f;
        if (lane == 0) {
          const int row = m0 + i;
          if (rscale && EPI != EPI_RESID) { s = fmul_nc(s, rscale[row]); s2 = fmul_nc(s2, rscale[row]); }
          const int yrow = ymap ? ymap[row] : row;
          if (EPI == EPI_STORE) Y[(size_t)yrow * ldy + col] = s;
          else if (EPI == EPI_RESID) Y[(size_t)yrow * ldy + col] = fadd_nc(Y[(size_t)yrow * ldy + col], s);
          else A[(size_t)row * lda + col] = swiglu(s, s2);
        }
      }
    }
  }
}

// ===========================================================================
// Linear layers, bf16, for blocks of many rows (prefill, mask scoring): a
// workgroup owns 128 W rows (SwiGLU: 64 gate rows and the same 64 up rows) and
// 128 activation rows.  K goes through LDS in 64-element slabs with TG_NST
// slabs in flight: the loads write LDS directly (global_load_lds_dwordx4, one
// 1 KB tile per wave instruction), so no registers hold data in transit.  W
// slabs keep the packed 16 x 32 tiles and activation slabs are stored in the
// same tile shape, so every fragment read is one contiguous 1 KB tile.  Each
// wave forms a 64 x 64 quadrant: 4 x 4 v_mfma_f32_16x16x32_bf16 blocks.
// The arithmetic of an output element is that of gemm_bf16_rows16 and of the
// decode projections: the K quarters of the four-wave split (same boundaries)
// are each accumulated from zero by the MFMA chain in k order, and the quarter
// sums are added in quarter order.  A row's result is the same bits in all
// three kernels.
// ===========================================================================

constexpr int TG_KS = 64;            // K elements per LDS slab
constexpr int TG_NST = 2;            // slabs in flight (LDS buffers)
// Row counts from which launch_linear takes this kernel: above 16 rows gemm_bf16_rows16 would stream the
// weights once per 16-row block (at 32 rows the 64 x 64 tiles take 25-30 % less time).
constexpr int TG_MIN_ROWS = 17;

typedef __attribute__((address_space(3))) void tg_lds_t;
typedef __attribute__((address_space(1))) const void tg_gbl_t;

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (lds wave-uniform).
__device__ __forceinline__ void tg_load_lds(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((tg_gbl_t*)src, (tg_lds_t*)lds, 16, 0, 0);
}
// Workgroup barrier without a memory fence: the waits for the slab loads are explicit.
__device__ __forceinline__ void tg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// WI x WJ: MFMA blocks per wave (W row tiles x activation row tiles); the four waves form a 2 x 2 grid,
// so a workgroup covers 32 WI W rows (SwiGLU: 16 WI gate rows and the same up rows) and 32 WJ
// activation rows.  4 x 4 for large problems; 2 x 2 when the large tiles would leave CUs idle.
// SPLIT (plain epilogues only): the grid holds four copies of the tile grid, copy q forming only K
// quarter q; its quarter sum goes to part[q][row][col] (M x N per quarter), and tg_quarter_reduce_kernel
// adds the four in quarter order and applies the epilogue.
template <int EPI, int WI, int WJ, bool SPLIT = false>
__global__ __launch_bounds__(256) void gemm_bf16_tiled(
    const bf16_t* __restrict__ W, const bf16_t* __restrict__ X, int ldx, int M, int N, int K,
    float* __restrict__ Y, int ldy, bf16_t* __restrict__ A, int lda, int n_mb, const float* __restrict__ rscale,
    const int* __restrict__ nrows, const int* __restrict__ ymap, const int* __restrict__ stop,
    float* __restrict__ part = nullptr) {
  if (stop && *stop) return;
  constexpr bool SW = EPI == EPI_SWIGLU;
  static_assert(!(SPLIT && SW), "quarter split for plain epilogues");
  constexpr int WT = 2 * WI, XT = 2 * WJ;           // W / activation row tiles per workgroup
  constexpr int WSZ = WT * 2 * 512, XSZ = XT * 2 * 512;   // elements of a stage's W / activation tiles
  constexpr int H = WI / 2;
  static_assert(!SW || WI % 2 == 0, "SwiGLU pairs gate and up tiles");
  // one barrier per slab for the large tiles (measured 5-7 % faster there; 10-15 % slower for the small ones)
  constexpr bool ONE_BARRIER = WI == 4;
  static_assert(!ONE_BARRIER || TG_NST == 2, "the single-barrier order refills the other of two stages");
  const int Ma = active_rows(M, nrows);
  // workgroup i runs on XCD i % 8: consecutive logical blocks (the row blocks of one W tile) are placed
  // on one XCD, so that they share its L2 for the W slabs
  const int nblk = SPLIT ? gridDim.x / 4 : gridDim.x;
  const int qsplit = SPLIT ? blockIdx.x / nblk : 0;
  const int bx = SPLIT ? blockIdx.x % nblk : blockIdx.x;
  const int lb = (nblk % 8 == 0) ? (bx % 8) * (nblk / 8) + bx / 8 : bx;
  const int mb = lb % n_mb, nb = lb / n_mb;
  const int m0 = mb * 16 * XT;
  if (m0 >= Ma) return;
  // per stage: W tiles [row tile][k tile 0..1][16][32], then the activation tiles in the same shape
  __shared__ alignas(16) bf16_t Ls[TG_NST][WSZ + XSZ];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int r = lane & 15, g = lane >> 4;
  const int ktiles = K / 32;
  const int n_wtiles = (N + 15) / 16;                     // packed tiles per W row set

  // global packed tile (row tile index) of local W row tile t
  auto wtile = [&](int t) -> int {
    if (SW) return t < WI ? WI * nb + t : n_wtiles + WI * nb + (t - WI);   // gate f0.., then up N + f0..
    return min(WT * nb + t, n_wtiles - 1);                                 // tiles past N repeat the last
  };
  // wave w fills the LDS tiles w + 4 j of W (j < WI) and of the activations (j < WJ) per slab
  const bf16_t* wsrc[WI];
  const bf16_t* xsrc[WJ];
#pragma unroll
  for (int j = 0; j < WI; ++j) {
    const int id = wave + 4 * j;                          // local tile id = row tile * 2 + k tile
    wsrc[j] = W + ((size_t)wtile(id >> 1) * ktiles + (id & 1)) * 512 + lane * 8;
  }
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int id = wave + 4 * j;
    const int row = (id >> 1) * 16 + (lane >> 2);
    xsrc[j] = X + (size_t)min(m0 + row, Ma - 1) * ldx + (id & 1) * 32 + (lane & 3) * 8;
  }
  auto issue = [&](int sl) {                              // WI + WJ loads per thread
    bf16_t* st = Ls[sl % TG_NST];
#pragma unroll
    for (int j = 0; j < WI; ++j) tg_load_lds(wsrc[j] + (size_t)sl * 1024, st + (wave + 4 * j) * 512);
#pragma unroll
    for (int j = 0; j < WJ; ++j) tg_load_lds(xsrc[j] + (size_t)sl * TG_KS, st + WSZ + (wave + 4 * j) * 512);
  };

  // this wave's W row tiles (A fragments); activation row tiles WJ wm + j (B fragments)
  int at[WI];
#pragma unroll
  for (int i = 0; i < WI; ++i) at[i] = SW ? (i < H ? H * wn + i : WI + H * wn + (i - H)) : WI * wn + i;
  f32x4 acc[WI][WJ], sum[WI][WJ];
#pragma unroll
  for (int i = 0; i < WI; ++i)
#pragma unroll
    for (int j = 0; j < WJ; ++j) acc[i][j] = sum[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nu = K / TG_KS;                               // slabs (= 64-element units)
  const int q0 = SPLIT ? qsplit : 0, q1 = SPLIT ? qsplit + 1 : 4;
  const int sb = (nu * q0) / 4, se = (nu * q1) / 4;       // slabs of this workgroup
#pragma unroll
  for (int p = 0; p < TG_NST - 1; ++p)
    if (sb + p < se) issue(sb + p);
  int sl = sb;
  for (int q = q0; q < q1; ++q) {
    const int qe = (nu * (q + 1)) / 4;                    // quarter q: slabs [(nu q) / 4, qe)
    for (; sl < qe; ++sl) {
      if constexpr (ONE_BARRIER) {
        // wait for this wave's share of slab sl; the barrier makes the slab whole and frees the stage of
        // slab sl - 1, which the loads of slab sl + 1 then refill
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        tg_barrier();
        if (sl + 1 < se) issue(sl + 1);
      } else {
        if (sl + TG_NST - 1 < se) {
          issue(sl + TG_NST - 1);
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"((WI + WJ) * (TG_NST - 1)) : "memory");   // slab sl has landed
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        tg_barrier();                                       // ... for every wave's share of it
      }
      const bf16_t* st = Ls[sl % TG_NST];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 af[WI], bfr[WJ];
#pragma unroll
        for (int i = 0; i < WI; ++i) af[i] = *(const bf16x8*)(st + (at[i] * 2 + kt) * 512 + r * 32 + g * 8);
#pragma unroll
        for (int j = 0; j < WJ; ++j)
          bfr[j] = *(const bf16x8*)(st + WSZ + ((WJ * wm + j) * 2 + kt) * 512 + r * 32 + g * 8);
#pragma unroll
        for (int i = 0; i < WI; ++i)
#pragma unroll
          for (int j = 0; j < WJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if constexpr (!ONE_BARRIER) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's reads of the stage are done
        tg_barrier();                                         // before the stage is refilled
      }
    }
    // the quarter's sum joins the earlier quarters' (an empty quarter adds zero)
#pragma unroll
    for (int i = 0; i < WI; ++i)
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        sum[i][j] += acc[i][j];
        acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  }

  // acc layout: lane (r, g) holds D[feature 4 g + e][row r] of each 16 x 16 block
  if constexpr (SPLIT) {
    float* pq = part + (size_t)qsplit * M * N;
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int row = m0 + 16 * (WJ * wm + j) + r;
      if (row >= Ma) continue;
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = 16 * WT * nb + 16 * (WI * wn + i) + 4 * g + e;
          if (col < N) pq[(size_t)row * N + col] = sum[i][j][e];
        }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int row = m0 + 16 * (WJ * wm + j) + r;
    if (row >= Ma) continue;
    const float rs = (rscale && EPI != EPI_RESID) ? rscale[row] : 1.f;
    const int yrow = ymap ? ymap[row] : row;
    if constexpr (SW) {
#pragma unroll
      for (int i = 0; i < H; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = 16 * WI * nb + 16 * (H * wn + i) + 4 * g + e;
          float s1 = sum[i][j][e], s2 = sum[i + H][j][e];
          if (rscale) { s1 = fmul_nc(s1, rs); s2 = fmul_nc(s2, rs); }
          A[(size_t)row * lda + col] = f2bf(swiglu(s1, s2));
        }
    } else {
#pragma unroll
      for (int i = 0; i < WI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = 16 * WT * nb + 16 * (WI * wn + i) + 4 * g + e;
          if (col >= N) continue;
          float v = sum[i][j][e];
          if (EPI == EPI_STORE) {
            if (rscale) v = fmul_nc(v, rs);
            Y[(size_t)yrow * ldy + col] = v;
          } else {
            Y[(size_t)yrow * ldy + col] = fadd_nc(Y[(size_t)yrow * ldy + col], v);
          }
        }
    }
  }
}

// The four quarter sums of a split projection added in quarter order, then the plain epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void tg_quarter_reduce_kernel(const float* __restrict__ part, int M, int N,
                                                                float* __restrict__ Y, int ldy,
                                                                const float* __restrict__ rscale,
                                                                const int* __restrict__ nrows,
                                                                const int* __restrict__ ymap,
                                                                const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int Ma = active_rows(M, nrows);
  const size_t n = (size_t)Ma * N, MN = (size_t)M * N;
  for (size_t e = blockIdx.x * (size_t)256 + threadIdx.x; e < n; e += (size_t)gridDim.x * 256) {
    const int row = (int)(e / N), col = (int)(e % N);
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) v += part[q * MN + e];
    const int yrow = ymap ? ymap[row] : row;
    if (EPI == EPI_STORE) {
      if (rscale) v = fmul_nc(v, rscale[row]);
      Y[(size_t)yrow * ldy + col] = v;
    } else {
      Y[(size_t)yrow * ldy + col] = fadd_nc(Y[(size_t)yrow * ldy + col], v);
    }
  }
}

// Workgroups of the tiled projection with WI x WJ blocks per wave.
static int tg_blocks(int epi, int M, int N, int WI, int WJ) {
  const int n_mb = (M + 32 * WJ - 1) / (32 * WJ);
  const int n_nb = epi == EPI_SWIGLU ? N / (16 * WI) : (N + 32 * WI - 1) / (32 * WI);
  return n_mb * n_nb;
}

bool profile_next(int cls, hipEvent_t* start, hipEvent_t* stop, int** ran);
void profile_done(double bytes, const int* stop_flag, bool self_marked, hipStream_t s);
static int launch_linear_impl(int dtype, int epi, const void* W, const void* X, int ldx, int M, int N, int K,
                              float* Y, int ldy, void* A, int lda, int n_rb, dim3 grid, const float* rscale,
                              const int* nrows, const int* ymap, const int* stop, hipEvent_t e0, hipEvent_t e1,
                              hipStream_t s);

int launch_linear(int dtype, int epi, const void* W, const void* X, int ldx, int M, int N, int K,
                  float* Y, int ldy, void* A, int lda, const float* rscale, const int* nrows, const int* ymap,
                  const int* stop, hipStream_t s, float* split_ws, size_t split_floats) {
  if (M <= 0 || N <= 0) return 0;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int* ran = nullptr;
  const bool prof = profile_next(epi, &e0, &e1, &ran);
  int rc;
  if (dtype == SSD_DTYPE_BF16 && M >= TG_MIN_ROWS && K % TG_KS == 0 && (epi != EPI_SWIGLU || N % 64 == 0)) {
    // Tile choice (all three give the same bits), measured on the 13B shapes over M = 96 - 512:
    // - large tiles from 256 of them, or from 192 when the last 128-row block is at least three quarters
    //   full (QKV at M = 224 - 256, gate/up at M = 96 - 128: 4-20 % faster than the small tiles);
    // - otherwise plain epilogues with few small tiles take the large tiles split by K quarter (workspace
    //   permitting): below 192 small tiles, or up to 1024 of them for long K (K >= 8192), where the split
    //   wins in spite of its partial sums and reduce launch (K = 5120 at 192 - 512 small tiles: 10-20 %
    //   slower than the small tiles);
    // - otherwise the small tiles.
    const int big_blocks = tg_blocks(epi, M, N, 4, 4);
    const bool big = big_blocks >= 256 || (big_blocks >= 192 && (M % 128 == 0 || M % 128 >= 96));
    const int small_blocks = tg_blocks(epi, M, N, 2, 2);
    const bool split = !big && epi != EPI_SWIGLU && split_ws && 4 * (size_t)M * N <= split_floats &&
                       (K >= 8192 ? small_blocks <= 1024 : small_blocks < 192);
    const int WJ = big || split ? 4 : 2;
    const int n_mb = (M + 32 * WJ - 1) / (32 * WJ);
    const dim3 grid(big ? big_blocks : (split ? 4 * big_blocks : tg_blocks(epi, M, N, 2, 2)));
    const bf16_t* w = (const bf16_t*)W;
    const bf16_t* x = (const bf16_t*)X;
#define TILED(E, I, J)                                                                                            \
  hipExtLaunchKernelGGL((gemm_bf16_tiled<E, I, J>), grid, dim3(256), 0, s, e0, e1, 0, w, x, ldx, M, N, K, Y, ldy,   \
                        (bf16_t*)A, lda, n_mb, rscale, nrows, ymap, stop, nullptr)
#define TSPLIT(E)                                                                                                 \
  do {                                                                                                            \
    hipExtLaunchKernelGGL((gemm_bf16_tiled<E, 4, 4, true>), grid, dim3(256), 0, s, e0, e1, 0, w, x, ldx, M, N, K,  \
                          Y, ldy, (bf16_t*)A, lda, n_mb, rscale, nrows, ymap, stop, split_ws);                     \
    const size_t nel = (size_t)M * N;                                                                             \
    hipLaunchKernelGGL(tg_quarter_reduce_kernel<E>, dim3((unsigned)std::min<size_t>((nel + 255) / 256, 2048)),     \
                       dim3(256), 0, s, split_ws, M, N, Y, ldy, rscale, nrows, ymap, stop);                       \
  } while (0)
    if (split) {
      if (epi == EPI_STORE) TSPLIT(EPI_STORE);
      else TSPLIT(EPI_RESID);
    } else if (big) {
      if (epi == EPI_STORE) TILED(EPI_STORE, 4, 4);
      else if (epi == EPI_RESID) TILED(EPI_RESID, 4, 4);
      else TILED(EPI_SWIGLU, 4, 4);
    } else {
      if (epi == EPI_STORE) TILED(EPI_STORE, 2, 2);
      else if (epi == EPI_RESID) TILED(EPI_RESID, 2, 2);
      else TILED(EPI_SWIGLU, 2, 2);
    }
#undef TILED
#undef TSPLIT
    rc = last_launch();
  } else {
    const int n_rb = (M + 15) / 16;
    const int n_tiles = (N + 15) / 16;
    const dim3 grid(n_rb * n_tiles);
    rc = launch_linear_impl(dtype, epi, W, X, ldx, M, N, K, Y, ldy, A, lda, n_rb, grid, rscale, nrows, ymap, stop,
                            e0, e1, s);
  }
  if (prof) {
    // algorithmic bytes: weights once, activations in once, results out once (residual: read + write)
    const double elt = dtype == SSD_DTYPE_BF16 ? 2.0 : 4.0;
    const double wrows = epi == EPI_SWIGLU ? 2.0 * N : (double)N;
    double by = wrows * K * elt + (double)M * K * elt;
    by += epi == EPI_STORE ? 4.0 * M * N : (epi == EPI_RESID ? 8.0 * M * N : elt * M * N);
    profile_done(by, stop, false, s);
  }
  return rc;
}

static int launch_linear_impl(int dtype, int epi, const void* W, const void* X, int ldx, int M, int N, int K,
                              float* Y, int ldy, void* A, int lda, int n_rb, dim3 grid, const float* rscale,
                              const int* nrows, const int* ymap, const int* stop, hipEvent_t e0, hipEvent_t e1,
                              hipStream_t s) {
  if (dtype == SSD_DTYPE_BF16) {
    if (K % 64 != 0) return SSD_ERR_SHAPE;
    const bf16_t* w = (const bf16_t*)W;
    const bf16_t* x = (const bf16_t*)X;
    switch (epi) {
      case EPI_STORE:
        hipExtLaunchKernelGGL(gemm_bf16_rows16<EPI_STORE>, grid, dim3(GEMM_NW * 64), 0, s, e0, e1, 0, w, x, ldx, M, N, K, Y,
                           ldy, (bf16_t*)A, lda, n_rb, rscale, nrows, ymap, stop);
        break;
      case EPI_RESID:
        hipExtLaunchKernelGGL(gemm_bf16_rows16<EPI_RESID>, grid, dim3(GEMM_NW * 64), 0, s, e0, e1, 0, w, x, ldx, M, N, K, Y,
                           ldy, (bf16_t*)A, lda, n_rb, rscale, nrows, ymap, stop);
        break;
      default:
        hipExtLaunchKernelGGL(gemm_bf16_rows16<EPI_SWIGLU>, grid, dim3(GEMM_NW * 64), 0, s, e0, e1, 0, w, x, ldx, M, N, K, Y,
                           ldy, (bf16_t*)A, lda, n_rb, rscale, nrows, ymap, stop);
    }
  } else {
    const float* w = (const float*)W;
    const float* x = (const float*)X;
    switch (epi) {
      case EPI_STORE:
        hipExtLaunchKernelGGL(gemm_f32_rows16<EPI_STORE>, grid, dim3(256), 0, s, e0, e1, 0, w, x, ldx, M, N, K, Y, ldy,
                           (float*)A, lda, n_rb, rscale, nrows, ymap, stop);
        break;
      case EPI_RESID:
        hipExtLaunchKernelGGL(gemm_f32_rows16<EPI_RESID>, grid, dim3(256), 0, s, e0, e1, 0, w, x, ldx, M, N, K, Y, ldy,
                           (float*)A, lda, n_rb, rscale, nrows, ymap, stop);
        break;
      default:
        hipExtLaunchKernelGGL(gemm_f32_rows16<EPI_SWIGLU>, grid, dim3(256), 0, s, e0, e1, 0, w, x, ldx, M, N, K, Y, ldy,
                           (float*)A, lda, n_rb, rscale, nrows, ymap, stop);
    }
  }
  return last_launch();
}

// ===========================================================================
// RMSNorm: x[m] = act(h[hmap[m]] / sqrt(mean(h^2) + eps) * gain), fp32 sums.
// ===========================================================================

// Row preparation for a projection: x[m] = act(h[hmap[m]] * gain * inv) with
// inv = 1 / sqrt(mean(h^2) + eps), the RMSNorm's output rounded once (the same
// bits as the decode projections' operands: norm_bf16 of h * gain and inv from
// the canonical tile sums).  One workgroup per row.
template <typename T>
__global__ __launch_bounds__(1024) void rowprep_kernel(const float* __restrict__ h, int ldh,
                                                       const float* __restrict__ gain, T* __restrict__ x,
                                                       int ldx, float* __restrict__ inv, int M, int D, float eps,
                                                       const int* __restrict__ nrows,
                                                       const int* __restrict__ hmap, const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int row = blockIdx.x;
  if (row >= active_rows(M, nrows)) return;
  const float* hr = h + (size_t)(hmap ? hmap[row] : row) * ldh;
  T* xr = x + (size_t)row * ldx;
  __shared__ float tss[1024];                  // group sums, D <= 16384
  __shared__ float s_inv;
  constexpr int PER = 16;                      // D / 1024 elements per thread at most
  float v[PER], gv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {              // every load in flight before the first use
    const int i = j * 1024 + threadIdx.x;
    v[j] = i < D ? hr[i] : 0.f;
    gv[j] = i < D ? gain[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * 1024 + threadIdx.x;
    if (j * 1024 >= D) break;                  // uniform: D is a multiple of 16
    const float s = tile16_ss_lanes(v[j]);
    if (i < D && (threadIdx.x & 15) == 0) tss[i >> 4] = s;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const float tot = row_ss_total(tss, 1, D / 16);
    if (threadIdx.x == 0) {
      s_inv = inv_rms(tot, D, eps);
      if (inv) inv[row] = s_inv;
    }
  }
  __syncthreads();
  const float iv = s_inv;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * 1024 + threadIdx.x;
    if (j * 1024 >= D) break;
    if (i < D) {
      const float hg = fmul_nc(v[j], gv[j]);
      if constexpr (sizeof(T) == 2) xr[i] = norm_bf16(hg, iv);
      else xr[i] = fmul_nc(hg, iv);
    }
  }
}

int launch_rowprep(int dtype, const float* h, int ldh, const float* gain, void* x, int ldx, float* inv, int M, int D,
                   float eps, const int* nrows, const int* hmap, const int* stop, hipStream_t s) {
  if (M <= 0) return 0;
  if (D % 16 != 0 || D > 16384) return SSD_ERR_SHAPE;
  if (dtype == SSD_DTYPE_BF16)
    hipLaunchKernelGGL(rowprep_kernel<bf16_t>, dim3(M), dim3(1024), 0, s, h, ldh, gain, (bf16_t*)x, ldx, inv, M, D,
                       eps, nrows, hmap, stop);
  else
    hipLaunchKernelGGL(rowprep_kernel<float>, dim3(M), dim3(1024), 0, s, h, ldh, gain, (float*)x, ldx, inv, M, D,
                       eps, nrows, hmap, stop);
  return last_launch();
}

// ===========================================================================
// Embedding gather into the fp32 residual stream.
// ===========================================================================

template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ emb, const int* __restrict__ tokens,
                                                    int V, float* __restrict__ h, int ldh, int M, int D,
                                                    const int* __restrict__ nrows, const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int row = blockIdx.x;
  if (row >= active_rows(M, nrows)) return;
  const int t = min(max(tokens[row], 0), V - 1);   // ids are produced in range; clamp keeps reads in bounds
  const T* e = emb + (size_t)t * D;
  float* hr = h + (size_t)row * ldh;
#pragma unroll 8
  for (int i = threadIdx.x; i < D; i += 256) hr[i] = ld(e + i);
}

int launch_embed(int dtype, const void* emb, const int* tokens, int V, float* h, int ldh, int M, int D,
                 const int* nrows, const int* stop, hipStream_t s) {
  if (M <= 0) return 0;
  if (dtype == SSD_DTYPE_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(M), dim3(256), 0, s, (const bf16_t*)emb, tokens, V, h, ldh, M,
                       D, nrows, stop);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, s, (const float*)emb, tokens, V, h, ldh, M, D,
                       nrows, stop);
  return last_launch();
}

// ===========================================================================
// RoPE + KV append.  One workgroup (HD/2 threads) per (row, head slot):
// slots 0..H-1 rotate q, H..H+KVH-1 rotate k into the cache, the rest copy v.
// Angles pos * theta^(-2i/hd) are formed and reduced in fp64, cos/sin rounded
// to fp32, the rotation itself in fp32.
// ===========================================================================


template <typename T, int HD>
__global__ void rope_kv_kernel(const float* __restrict__ qkv, int ldqkv, T* __restrict__ qout, int ldq,
                               T* __restrict__ pool, const int* __restrict__ page_table, int n_lpages, int PS,
                               int L, int layer, int H, int KVH, int M, const int* __restrict__ nrows,
                               const int* __restrict__ pos, const float2* __restrict__ rope_cs,
                               T* __restrict__ local_kv, int* __restrict__ err, const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int row = blockIdx.x;
  if (row >= active_rows(M, nrows)) return;
  const int slot = blockIdx.y;
  const int i = threadIdx.x;                  // pair index 0..HD/2-1
  const int p = pos[row];
  const float* src = qkv + (size_t)row * ldqkv + (size_t)slot * HD;
  T* dst;
  if (slot < H) {
    dst = qout + (size_t)row * ldq + (size_t)slot * HD;
  } else {
    const int kvsel = slot < H + KVH ? 0 : 1;
    const int g = slot - H - kvsel * KVH;
    if (local_kv) {
      dst = local_kv + (((size_t)row * 2 + kvsel) * KVH + g) * HD;
    } else {
      const int lp = p / PS;
      if (lp >= n_lpages || p < 0) {
        if (i == 0) atomicOr(err, ERRF_CAPACITY);
        return;
      }
      dst = pool + kv_index(page_table[lp], L, layer, kvsel, KVH, g, PS, p % PS, HD);
    }
  }
  const float x1 = src[i], x2 = src[i + HD / 2];
  if (slot < H + KVH) {
    float y1, y2;
    rope_apply(x1, x2, rope_cs[(size_t)p * (HD / 2) + i], y1, y2);
    st(dst + i, y1);
    st(dst + i + HD / 2, y2);
  } else {
    st(dst + i, x1);
    st(dst + i + HD / 2, x2);
  }
}

int launch_rope_kv(int dtype, int head_dim, const float* qkv, int ldqkv, void* qout, int ldq,
                   const KvView& kv, int L, int layer, int H, int KVH, const RowBlock& rb,
                   const float2* rope_cs, void* local_kv, int* err_flags, hipStream_t s) {
  if (rb.M <= 0) return 0;
  const dim3 grid(rb.M, H + 2 * KVH);
#define ROPE_LAUNCH(T, HD)                                                                                     \
  hipLaunchKernelGGL((rope_kv_kernel<T, HD>), grid, dim3(HD / 2), 0, s, qkv, ldqkv, (T*)qout, ldq, (T*)kv.pool, \
                     kv.page_table, kv.n_lpages, kv.page_size, L, layer, H, KVH, rb.M, rb.nrows, rb.pos,        \
                     rope_cs, (T*)local_kv, err_flags, rb.stop)
  if (dtype == SSD_DTYPE_BF16) {
    if (head_dim == 128) ROPE_LAUNCH(bf16_t, 128); else ROPE_LAUNCH(bf16_t, 64);
  } else {
    if (head_dim == 128) ROPE_LAUNCH(float, 128); else ROPE_LAUNCH(float, 64);
  }
#undef ROPE_LAUNCH
  return last_launch();
}

// ===========================================================================
// Attention over the paged cache (device functions in attn.h).
// ===========================================================================

int attention_nsplit(int max_ctx) { return (max_ctx + ATT_SPLIT - 1) / ATT_SPLIT; }

size_t attention_partial_floats(int max_rows, int H, int head_dim, int max_ctx) {
  const int nsplit = attention_nsplit(max_ctx);
  return (size_t)max_rows * H * nsplit * att_rec(head_dim);
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const T* __restrict__ q, int ldq, const T* __restrict__ pool, const int* __restrict__ page_table, int PS,
    int n_lpages, int L, int layer, int H, int KVH, int M, const int* __restrict__ nrows,
    const int* __restrict__ pos, int RB, int nsplit, const T* __restrict__ local_kv, int local_start, int group_rows,
    float* __restrict__ part, const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int g = blockIdx.x, s = blockIdx.y, rbk = blockIdx.z;
  __shared__ AttnSmem<T, HD, 4> sm;
  attn_partial_item<T, HD, 4>(sm, q, ldq, pool, page_table, PS, n_lpages, L, layer, H, KVH, M, nrows, pos, rbk * RB,
                              RB, g, s, nsplit, local_kv, local_start, group_rows, part);
}

// bf16 items of QT query tiles (row blocks of QT * 16 / G rows): the split's keys and values are staged
// once for all tiles.
template <int HD, int QT>
__global__ __launch_bounds__(256) void attn_partial_multi_kernel(
    const bf16_t* __restrict__ q, int ldq, const bf16_t* __restrict__ pool, const int* __restrict__ page_table,
    int PS, int n_lpages, int L, int layer, int H, int KVH, int M, const int* __restrict__ nrows,
    const int* __restrict__ pos, int RB, int nsplit, const bf16_t* __restrict__ local_kv, int local_start,
    int group_rows, float* __restrict__ part, const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int g = blockIdx.x, s = blockIdx.y, rbk = blockIdx.z;
  __shared__ AttnSmemQ<HD, QT> sm;
  attn_item_bf16<HD, 4, false, QT>(sm, q, ldq, pool, page_table, PS, n_lpages, L, layer, H, KVH, M, nrows, pos,
                                   rbk * RB, RB, g, s, nsplit, local_kv, local_start, group_rows, part);
}

template <typename T, int HD>
__global__ void attn_combine_kernel(const float* __restrict__ part, int nsplit, int M, const int* __restrict__ nrows,
                                    const int* __restrict__ pos, int H, T* __restrict__ out, int ldo, int blocked,
                                    const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int row = blockIdx.x, head = blockIdx.y;
  if (row >= active_rows(M, nrows)) return;
  attn_combine_elem<T, HD>(part, nsplit, row, head, H, pos[row], threadIdx.x, out, ldo, blocked != 0);
}

int launch_attention(int dtype, int head_dim, const void* q, int ldq, const KvView& kv, int L, int layer,
                     int H, int KVH, const RowBlock& rb, int max_ctx, const void* local_kv,
                     int local_start, int group_rows, float* part, void* out, int ldo, hipStream_t s,
                     bool out_blocked) {
  if (rb.M <= 0) return 0;
  if (out_blocked && rb.M > 16) return SSD_ERR_SHAPE;
  const int G = H / KVH;
  // candidate groups of the scoring pass: one online-softmax walk over the keys per group and head
  if (local_kv && group_rows > 0 && !out_blocked && attention_groups_usable(dtype, head_dim, H, KVH))
    return launch_attention_groups(head_dim, q, ldq, kv, L, layer, H, KVH, rb, local_kv, local_start, group_rows,
                                   out, ldo, s);
  if (rb.M > SPLIT_ATTN_MAX_ROWS) return SSD_ERR_SHAPE;   // the partial buffer's row capacity
  int RB = (dtype == SSD_DTYPE_BF16 ? ATTB_MAXQ : ATT_MAXQ) / G;
  if (RB < 1) return SSD_ERR_SHAPE;
  // bf16 rows beyond a decode block: several 16-query tiles per item (the rows of an item share one
  // local-KV group when there is one)
  int QT = 1;
  if (dtype == SSD_DTYPE_BF16 && !out_blocked && rb.M > RB) {
    QT = 2;
    while (QT > 1 && local_kv && (group_rows % (QT * RB) != 0)) QT /= 2;
    RB *= QT;
  }
  if (group_rows > 0) {
    // a row block must not straddle two groups
    while (RB > 1 && group_rows % RB != 0) --RB;
  }
  const int nsplit = attention_nsplit(max_ctx);
  const dim3 grid(KVH, nsplit, (rb.M + RB - 1) / RB);
#define ATT_MULTI(HD, Q)                                                                                         \
  hipLaunchKernelGGL((attn_partial_multi_kernel<HD, Q>), grid, dim3(256), 0, s, (const bf16_t*)q, ldq,            \
                     (const bf16_t*)kv.pool, kv.page_table, kv.page_size, kv.n_lpages, L, layer, H, KVH, rb.M,    \
                     rb.nrows, rb.pos, RB, nsplit, (const bf16_t*)local_kv, local_start, group_rows, part, rb.stop)
#define ATT_LAUNCH(T, HD)                                                                                        \
  do {                                                                                                           \
    if (QT == 4) ATT_MULTI(HD, 4);                                                                               \
    else if (QT == 2) ATT_MULTI(HD, 2);                                                                          \
    else                                                                                                         \
      hipLaunchKernelGGL((attn_partial_kernel<T, HD>), grid, dim3(256), 0, s, (const T*)q, ldq,                  \
                         (const T*)kv.pool, kv.page_table, kv.page_size, kv.n_lpages, L, layer, H, KVH, rb.M,    \
                         rb.nrows, rb.pos, RB, nsplit, (const T*)local_kv, local_start, group_rows, part,        \
                         rb.stop);                                                                               \
    hipLaunchKernelGGL((attn_combine_kernel<T, HD>), dim3(rb.M, H), dim3(HD), 0, s, part, nsplit, rb.M, rb.nrows, \
                       rb.pos, H, (T*)out, ldo, out_blocked ? 1 : 0, rb.stop);                                  \
  } while (0)
  if (dtype == SSD_DTYPE_BF16) {
    if (head_dim == 128) ATT_LAUNCH(bf16_t, 128); else ATT_LAUNCH(bf16_t, 64);
  } else {
    if (head_dim == 128) ATT_LAUNCH(float, 128); else ATT_LAUNCH(float, 64);
  }
#undef ATT_LAUNCH
#undef ATT_MULTI
  return last_launch();
}

// ===========================================================================
// Row statistics: max, argmax (lowest index), second max, log-sum-exp of z/T,
// confidence and a draw.  One 1024-thread workgroup per row.
// ===========================================================================

// Loops over a row of logits with the loads of several iterations in flight
// before their first use.  Each thread visits its elements in the same order
// as the plain loops they replace: v = tid, tid + NT, ... (strided), or the
// quads v4 = 4 tid, 4 tid + 4 NT, ... with their elements v4 .. v4 + 3.
template <int NT, typename F>
__device__ __forceinline__ void for_strided(const float* __restrict__ z, int V, F f) {
  constexpr int B = 8;
  const int tid = threadIdx.x;
  for (int base = 0; base < V; base += NT * B) {
    float zv[B];
#pragma unroll
    for (int u = 0; u < B; ++u) zv[u] = z[min(base + u * NT + tid, V - 1)];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int v = base + u * NT + tid;
      if (v < V) f(v, zv[u]);
    }
  }
}

// f(v4, a[4], b[4]) for each quad of the thread (b: a second row, or a again); elements >= V are
// clamped copies that f must skip.
template <int NT, typename F>
__device__ __forceinline__ void for_quads(const float* __restrict__ za, const float* __restrict__ zb, int V, F f) {
  constexpr int B = 4;
  const int tid = threadIdx.x;
  for (int base = 0; base < V; base += NT * 4 * B) {
    float a[B][4], b[B][4];
#pragma unroll
    for (int u = 0; u < B; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = min(base + (u * NT + tid) * 4 + e, V - 1);
        a[u][e] = za[v];
        b[u][e] = zb[v];
      }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int v4 = base + (u * NT + tid) * 4;
      if (v4 < V) f(v4, a[u], b[u]);
    }
  }
}

// Rows up to ROWREG * 1024 elements are read once into registers (one round
// of loads), in either element order: strided r[k] = z[tid + 1024 k], or
// quads r[4 i + e] = z[4 tid + 4096 i + e].
constexpr int ROWREG = 32;

__device__ __forceinline__ void load_row_strided(const float* __restrict__ z, int V, float (&r)[ROWREG]) {
#pragma unroll
  for (int k = 0; k < ROWREG; ++k) r[k] = z[min((int)threadIdx.x + 1024 * k, V - 1)];
}

__device__ __forceinline__ void load_row_quads(const float* __restrict__ z, int V, float (&r)[ROWREG]) {
#pragma unroll
  for (int i = 0; i < ROWREG / 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * i + e] = z[min(4 * (int)threadIdx.x + 4096 * i + e, V - 1)];
}

struct Top2 { float v1; int i1; float v2; };

__device__ __forceinline__ void top2_push(Top2& t, float v, int i) {
  if (v > t.v1 || (v == t.v1 && i < t.i1)) { t.v2 = fmaxf(t.v2, t.v1); t.v1 = v; t.i1 = i; }
  else t.v2 = fmaxf(t.v2, v);
}

// The same update as selects (no branches); a push with take == false changes nothing.
__device__ __forceinline__ void top2_push_sel(Top2& t, float v, int i, bool take) {
  const bool better = take && (v > t.v1 || (v == t.v1 && i < t.i1));
  const float v2 = better ? fmaxf(t.v2, t.v1) : (take ? fmaxf(t.v2, v) : t.v2);
  t.v1 = better ? v : t.v1;
  t.i1 = better ? i : t.i1;
  t.v2 = v2;
}

__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  Top2 r;
  if (b.v1 > a.v1 || (b.v1 == a.v1 && b.i1 < a.i1)) { r.v1 = b.v1; r.i1 = b.i1; r.v2 = fmaxf(b.v2, a.v1); }
  else { r.v1 = a.v1; r.i1 = a.i1; r.v2 = fmaxf(a.v2, b.v1); }
  return r;
}

// Block-wide statistics of z[0..V).  All 1024 threads must call it.
__device__ ssd_row_stat block_row_stats(const float* __restrict__ z, int V, float T, uint64_t seed, int iter,
                                        int rowid, uint32_t purpose, bool* bad) {
  __shared__ Top2 sh_t[16];
  __shared__ float sh_f[16];
  __shared__ int sh_i[16];
  __shared__ Top2 sh_res;
  __shared__ float sh_sum;
  __shared__ int sh_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) sh_bad = 0;
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  int nonfinite = 0;
  const bool in_regs = V <= 1024 * ROWREG;          // uniform
  float rq[ROWREG];
  if (in_regs) {
    load_row_quads(z, V, rq);
#pragma unroll
    for (int i = 0; i < ROWREG / 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * tid + 4096 * i + e;
        nonfinite |= (v < V) & !isfinite(rq[4 * i + e]);
        top2_push_sel(t, rq[4 * i + e], v, v < V);
      }
  } else {
    for_strided<1024>(z, V, [&](int v, float zv) {
      if (!isfinite(zv)) nonfinite = 1;
      top2_push(t, zv, v);
    });
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Top2 u{__shfl_xor(t.v1, o, 64), __shfl_xor(t.i1, o, 64), __shfl_xor(t.v2, o, 64)};
    t = top2_merge(t, u);
  }
  __syncthreads();
  if (nonfinite) sh_bad = 1;
  if (lane == 0) sh_t[wave] = t;
  __syncthreads();
  if (tid == 0) {
    Top2 r = sh_t[0];
    for (int w = 1; w < 16; ++w) r = top2_merge(r, sh_t[w]);
    sh_res = r;
  }
  __syncthreads();
  const Top2 res = sh_res;
  const float invT = T > 0.f ? 1.0f / T : 1.0f;
  // sum exp((z - max) / T) and the race over z/T + Gumbel
  float se = 0.f;
  float kbest = -INFINITY;
  int ibest = 0x7fffffff;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  auto quad = [&](int v4, const float* zq) {
    U4 w{0, 0, 0, 0};
    if (T > 0.f) w = philox4x32_10((uint32_t)iter, (uint32_t)rowid, purpose, (uint32_t)(v4 >> 2), k0, k1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v4 + e;
      if (v < V) {
        const float zv = zq[e];
        se += expf((zv - res.v1) * invT);
        if (T > 0.f) argmax_merge(kbest, ibest, zv / T + word_to_gumbel(ws[e]), v);
      }
    }
  };
  if (in_regs) {
    // sum in quad order; elements past the row add an exact 0
#pragma unroll
    for (int i = 0; i < ROWREG / 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = expf((rq[4 * i + e] - res.v1) * invT);
        se += 4 * tid + 4096 * i + e < V ? x : 0.f;
      }
    if (T > 0.f) {
      for (int i = 0; i < ROWREG / 4; ++i) {
        const int v4 = 4 * tid + 4096 * i;
        if (v4 >= V) break;
        const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)rowid, purpose, (uint32_t)(v4 >> 2), k0, k1);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (v4 + e < V) argmax_merge(kbest, ibest, rq[4 * i + e] / T + word_to_gumbel(ws[e]), v4 + e);
      }
    }
  } else {
    for_quads<1024>(z, z, V, [&](int v4, const float* zq, const float*) { quad(v4, zq); });
  }
  se = wave_sum(se);
  wave_argmax(kbest, ibest);
  if (lane == 0) { sh_f[wave] = se; sh_i[wave] = ibest; }
  __shared__ float sh_k[16];
  if (lane == 0) sh_k[wave] = kbest;
  __syncthreads();
  ssd_row_stat out;
  if (tid == 0) {
    float tot = 0.f;
    for (int w = 0; w < 16; ++w) tot += sh_f[w];
    float kb = sh_k[0];
    int ib = sh_i[0];
    for (int w = 1; w < 16; ++w) argmax_merge(kb, ib, sh_k[w], sh_i[w]);
    sh_sum = tot;
    sh_i[0] = ib;
  }
  __syncthreads();
  out.max = res.v1;
  out.argmax = res.i1;
  out.max2 = res.v2;
  out.lse = res.v1 * invT + logf(sh_sum);
  out.conf = 1.0f / sh_sum;
  out.sample = T > 0.f ? sh_i[0] : res.i1;
  *bad = sh_bad != 0;
  __syncthreads();
  return out;
}

__global__ __launch_bounds__(1024) void row_stats_kernel(const float* __restrict__ z, int ldz, int V, float T,
                                                         uint64_t seed, const int* iter_ptr, int iter_const,
                                                         int rowid_base, uint32_t purpose,
                                                         ssd_row_stat* __restrict__ out,
                                                         const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int row = blockIdx.x;
  const int iter = iter_ptr ? *iter_ptr : iter_const;
  bool bad;
  ssd_row_stat r = block_row_stats(z + (size_t)row * ldz, V, T, seed, iter, rowid_base + row, purpose, &bad);
  if (threadIdx.x == 0) out[row] = r;
}

int launch_row_stats(const float* z, int ldz, int rows, int V, float T, uint64_t seed, const int* iter_ptr,
                     int iter_const, int rowid_base, uint32_t purpose, ssd_row_stat* out, const int* stop,
                     hipStream_t s) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(row_stats_kernel, dim3(rows), dim3(1024), 0, s, z, ldz, V, T, seed, iter_ptr, iter_const,
                     rowid_base, purpose, out, stop);
  return last_launch();
}

// ===========================================================================
// Row statistics spread over segments of STAT_SEG logits, one 256-thread
// workgroup each with all of its loads in one round (a single workgroup
// reading a whole row is bound by one CU's outstanding misses).  Each
// segment stores a record; the segment that completes the row's count
// merges the records in segment order and resets the count.
// ===========================================================================

__global__ __launch_bounds__(256) void row_stats_seg_kernel(const float* __restrict__ z, int ldz, int V, float T,
                                                            uint64_t seed, const int* iter_ptr, int iter_const,
                                                            int rowid_base, uint32_t purpose,
                                                            ssd_row_stat* __restrict__ out, StatRec* __restrict__ recs,
                                                            unsigned* __restrict__ ctr, const int* __restrict__ stop,
                                                            DraftStep ds) {
  if (stop && *stop) return;
  if (ds.st && ds.st->stop) return;
  const int seg = blockIdx.x, row = blockIdx.y, nseg = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* zr = z + (size_t)row * ldz;
  const int iter = ds.st ? ds.st->iteration : (iter_ptr ? *iter_ptr : iter_const);
  const int rowid = ds.st ? ds.j - 1 : rowid_base + row;
  const float invT = T > 0.f ? 1.0f / T : 1.0f;
  __shared__ Top2 sh_t[4];
  __shared__ float sh_s[4], sh_k[4];
  __shared__ int sh_i[4], sh_bad[4], sh_last;
  __shared__ StatRec sh_rec[STAT_MAXSEG];
  // elements 4 q + e of the quads q = seg * STAT_SEG / 4 + tid + 256 h
  float x[8];
  int vv[8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vv[4 * h + e] = 4 * (seg * (STAT_SEG / 4) + tid + 256 * h) + e;
      x[4 * h + e] = zr[min(vv[4 * h + e], V - 1)];
    }
  Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
  int bad = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    bad |= (vv[k] < V) & !isfinite(x[k]);
    top2_push_sel(t, x[k], vv[k], vv[k] < V);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Top2 u{__shfl_xor(t.v1, o, 64), __shfl_xor(t.i1, o, 64), __shfl_xor(t.v2, o, 64)};
    t = top2_merge(t, u);
  }
  bad = __any(bad) ? 1 : 0;
  if (lane == 0) { sh_t[wave] = t; sh_bad[wave] = bad; }
  __syncthreads();
  t = sh_t[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) t = top2_merge(t, sh_t[w]);
  // sum of exp((z - m) / T) over the segment (m its maximum), in a fixed order
  float se = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float ex = expf((x[k] - t.v1) * invT);
    se += vv[k] < V ? ex : 0.f;
  }
  se = wave_sum(se);
  float kbest = -INFINITY;
  int ibest = 0x7fffffff;
  if (T > 0.f) {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int v4 = vv[4 * h];
      if (v4 < V) {
        const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)rowid, purpose, (uint32_t)(v4 >> 2), k0, k1);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (v4 + e < V) argmax_merge(kbest, ibest, x[4 * h + e] / T + word_to_gumbel(ws[e]), v4 + e);
      }
    }
    wave_argmax(kbest, ibest);
  }
  if (lane == 0) { sh_s[wave] = se; sh_k[wave] = kbest; sh_i[wave] = ibest; }
  __syncthreads();
  if (tid == 0) {
    float ss = sh_s[0];
    float kb = sh_k[0];
    int ib = sh_i[0];
    int bb = sh_bad[0];
    for (int w = 1; w < 4; ++w) {
      ss += sh_s[w];
      argmax_merge(kb, ib, sh_k[w], sh_i[w]);
      bb |= sh_bad[w];
    }
    StatRec* rc = recs + (size_t)row * nseg + seg;
    __hip_atomic_store(&rc->v1, t.v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&rc->i1, t.i1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&rc->v2, t.v2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&rc->s, ss, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&rc->kv, kb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&rc->ki, ib, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&rc->bad, bb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the record is stored before the count
    const unsigned old = __hip_atomic_fetch_add(ctr + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh_last = old + 1 == (unsigned)nseg;
    if (sh_last) __hip_atomic_store(ctr + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!sh_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (tid < nseg) sh_rec[tid] = recs[(size_t)row * nseg + tid];
  __syncthreads();
  if (tid != 0) return;
  Top2 r{sh_rec[0].v1, sh_rec[0].i1, sh_rec[0].v2};
  for (int k = 1; k < nseg; ++k) r = top2_merge(r, Top2{sh_rec[k].v1, sh_rec[k].i1, sh_rec[k].v2});
  float S = 0.f;
  float kb = -INFINITY;
  int ib = 0x7fffffff;
  int bb = 0;
  for (int k = 0; k < nseg; ++k) {
    S = fmaf(sh_rec[k].s, expf((sh_rec[k].v1 - r.v1) * invT), S);
    argmax_merge(kb, ib, sh_rec[k].kv, sh_rec[k].ki);
    bb |= sh_rec[k].bad;
  }
  ssd_row_stat o;
  o.max = r.v1;
  o.argmax = r.i1;
  o.max2 = r.v2;
  o.lse = r.v1 * invT + logf(S);
  o.conf = 1.0f / S;
  o.sample = T > 0.f ? ib : r.i1;
  if (ds.st) {
    ds.draft_tokens[ds.j - 1] = o.sample;
    if (bb) atomicOr(&ds.st->error_flags, ERRF_NUMERIC);
    if (o.conf < ds.tau || ds.j == ds.d) {
      ds.st->stop = 1;
      ds.st->n_drafted = ds.j;
      *ds.n_drafted_out = ds.j;
    }
  } else {
    if (bb) o.max = __int_as_float(0x7fc00000);          // non-finite logits: the row's max reads NaN
    out[row] = o;
  }
}

int stat_segments(int V) { return (V + STAT_SEG - 1) / STAT_SEG; }

int launch_row_stats_seg(const float* z, int ldz, int rows, int V, float T, uint64_t seed, const int* iter_ptr,
                         int iter_const, int rowid_base, uint32_t purpose, ssd_row_stat* out, StatRec* recs,
                         unsigned* ctr, const int* stop, const DraftStep& ds, hipStream_t s) {
  if (rows <= 0) return 0;
  const int nseg = stat_segments(V);
  if (nseg > STAT_MAXSEG) return SSD_ERR_SHAPE;
  hipLaunchKernelGGL(row_stats_seg_kernel, dim3(nseg, rows), dim3(256), 0, s, z, ldz, V, T, seed, iter_ptr,
                     iter_const, rowid_base, purpose, out, recs, ctr, stop, ds);
  return last_launch();
}


// ===========================================================================
// Accept / reject.  One workgroup per verify row i = 0..d' computes its
// decision and its correction (or, for i = d', the bonus); a one-wave kernel
// then scans the decisions in order.
// ===========================================================================

__device__ float block_sum_1024(float v) {
  __shared__ float sh[16];
  __shared__ float tot;
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < 16; ++w) t += sh[w];
    tot = t;
  }
  __syncthreads();
  const float r = tot;
  __syncthreads();
  return r;
}

__device__ int block_argmax_1024(float v, int i) {
  __shared__ float shv[16];
  __shared__ int shi[16];
  __shared__ int res;
  wave_argmax(v, i);
  if ((threadIdx.x & 63) == 0) { shv[threadIdx.x >> 6] = v; shi[threadIdx.x >> 6] = i; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = shv[0];
    int bi = shi[0];
    for (int w = 1; w < 16; ++w) argmax_merge(bv, bi, shv[w], shi[w]);
    res = bi;
  }
  __syncthreads();
  const int r = res;
  __syncthreads();
  return r;
}

__device__ float block_max_1024(float v) {
  __shared__ float sh[16];
  __shared__ float tot;
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = sh[0];
    for (int w = 1; w < 16; ++w) t = fmaxf(t, sh[w]);
    tot = t;
  }
  __syncthreads();
  const float r = tot;
  __syncthreads();
  return r;
}

// log-sum-exp of z/T over the row (T > 0)
__device__ float block_lse(const float* z, int V, float T) {
  float m = -INFINITY;
  float se = 0.f;
  if (V <= 1024 * ROWREG) {
    float r[ROWREG];
    load_row_strided(z, V, r);
#pragma unroll
    for (int k = 0; k < ROWREG; ++k)
      if ((int)threadIdx.x + 1024 * k < V) m = fmaxf(m, r[k]);
    m = block_max_1024(m);
#pragma unroll
    for (int k = 0; k < ROWREG; ++k)
      if ((int)threadIdx.x + 1024 * k < V) se += expf((r[k] - m) / T);
  } else {
    for_strided<1024>(z, V, [&](int, float zv) { m = fmaxf(m, zv); });
    m = block_max_1024(m);
    for_strided<1024>(z, V, [&](int, float zv) { se += expf((zv - m) / T); });
  }
  se = block_sum_1024(se);
  return m / T + logf(se);
}

__global__ __launch_bounds__(1024) void accept_rows_kernel(const float* __restrict__ zp, const float* __restrict__ zq,
                                                           int V, const int32_t* __restrict__ drafts,
                                                           const int32_t* __restrict__ n_drafted, float T,
                                                           uint64_t seed, const int* __restrict__ iter_ptr,
                                                           int iter_const, int* __restrict__ dec,
                                                           int* __restrict__ corr) {
  const int i = blockIdx.x;
  const int dp = min(max(*n_drafted, 0), (int)gridDim.x - 1);   // d' (the grid has d + 1 rows)
  if (i > dp) return;
  const float* p = zp + (size_t)i * V;
  const int tid = threadIdx.x;
  // a row holding NaN or +inf decides nothing: corr[i] = -1 marks it for the emit step
  if (T == 0.f) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    int bad = 0;
    if (V <= 1024 * ROWREG) {
      float r[ROWREG];
      load_row_strided(p, V, r);
#pragma unroll
      for (int k = 0; k < ROWREG; ++k)
        if (tid + 1024 * k < V) {
          argmax_merge(bv, bi, r[k], tid + 1024 * k);
          bad |= isnan(r[k]) || r[k] == INFINITY;
        }
    } else {
      for_strided<1024>(p, V, [&](int v, float pv) {
        argmax_merge(bv, bi, pv, v);
        bad |= isnan(pv) || pv == INFINITY;
      });
    }
    const int am = block_argmax_1024(bv, bi);
    const int anybad = __syncthreads_or(bad);
    if (tid == 0) {
      corr[i] = anybad ? -1 : am;
      dec[i] = !anybad && (i < dp) && (am == drafts[i]);
    }
    return;
  }
  const int iter = iter_ptr ? *iter_ptr : iter_const;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const float lse_p = block_lse(p, V, T);
  if (!isfinite(lse_p) || (i < dp && !isfinite(block_lse(zq + (size_t)i * V, V, T)))) {
    if (tid == 0) { corr[i] = -1; dec[i] = 0; }
    return;
  }
  float kbest = -INFINITY;
  int ibest = 0x7fffffff;
  if (i == dp) {
    // bonus: a draw from p_{d'+1}
    for_quads<1024>(p, p, V, [&](int v4, const float* pq, const float*) {
      const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)i, PURPOSE_SAMPLE, (uint32_t)(v4 >> 2), k0, k1);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v4 + e < V) argmax_merge(kbest, ibest, pq[e] / T + word_to_gumbel(ws[e]), v4 + e);
    });
    const int b = block_argmax_1024(kbest, ibest);
    if (tid == 0) { corr[i] = b; dec[i] = 0; }
    return;
  }
  const float* q = zq + (size_t)i * V;
  const float lse_q = block_lse(q, V, T);
  // residual norm(max(0, p - q)) as a race over log(r) + Gumbel
  int any_pos = 0;
  for_quads<1024>(p, q, V, [&](int v4, const float* pq, const float* qq) {
    const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)i, PURPOSE_SAMPLE, (uint32_t)(v4 >> 2), k0, k1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v4 + e;
      if (v < V) {
        const float r = expf(pq[e] / T - lse_p) - expf(qq[e] / T - lse_q);
        if (r > 0.f) { any_pos = 1; argmax_merge(kbest, ibest, logf(r) + word_to_gumbel(ws[e]), v); }
      }
    }
  });
  const int anyp = block_sum_1024((float)any_pos) > 0.f;
  int c;
  if (anyp) {
    c = block_argmax_1024(kbest, ibest);
  } else {
    kbest = -INFINITY; ibest = 0x7fffffff;
    for_quads<1024>(p, p, V, [&](int v4, const float* pq, const float*) {
      const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)i, PURPOSE_SAMPLE, (uint32_t)(v4 >> 2), k0, k1);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v4 + e < V) argmax_merge(kbest, ibest, (pq[e] / T - lse_p) + word_to_gumbel(ws[e]), v4 + e);
    });
    c = block_argmax_1024(kbest, ibest);
  }
  if (tid == 0) {
    const int y = drafts[i];
    const float lp = p[y] / T - lse_p;
    const float lq = q[y] / T - lse_q;
    const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)i, PURPOSE_ACCEPT, 0u, k0, k1);
    const float u = word_to_uniform(w.x);
    dec[i] = (logf(u) + lq) < lp;
    corr[i] = c;
  }
}

// Rows marked non-finite (corr = -1) emit nothing: n_out = 0 and ERRF_NUMERIC in *err (nullable).
__global__ void accept_emit_kernel(const int32_t* __restrict__ drafts, const int32_t* __restrict__ n_drafted, int d,
                                   const int* __restrict__ dec, const int* __restrict__ corr,
                                   int32_t* __restrict__ out, int32_t* __restrict__ n_out, int* __restrict__ err) {
  if (threadIdx.x != 0) return;
  const int dp = min(max(*n_drafted, 0), d);
  for (int r = 0; r <= dp; ++r)
    if (corr[r] < 0) {
      *n_out = 0;
      if (err) atomicOr(err, ERRF_NUMERIC);
      return;
    }
  int k = 0;
  while (k < dp && dec[k]) { out[k] = drafts[k]; ++k; }
  out[k] = corr[k];
  *n_out = k + 1;
}

// Sampled tree acceptance (T > 0), after accept_rows_kernel on the chain rows (dec[i]: the chain's
// candidate of depth i + 1 accepted, corr[i]: the chain rule's draw at row i).  At the first rejected
// depth, if it has leaves, its candidates are taken in order (the chain's token, then the leaves in
// leaf order): with p' = p_j, candidate c_k (k >= 1) is accepted when u_k q(c_k) < p'(c_k) (u_k:
// counter (iteration, i + 256 k, accept)); after each rejection p' becomes norm(max(0, p' - q)) (kept
// when that is all zero).  A leaf accepted: it and a draw from its own row (counter (iteration, i + 256 k,
// sample)) are emitted.  All rejected: a draw from the last nonzero residual, unnormalised, or from p
// when there was none (counter (iteration, i, sample)).  Tree rows: chain rows 0..d', leaf s at d' + 1 + s.
__global__ __launch_bounds__(1024) void tree_accept_sampled_kernel(
    const float* __restrict__ zp, const float* __restrict__ zq, int V, const int32_t* __restrict__ drafts,
    const int32_t* __restrict__ n_drafted, int d, const int32_t* __restrict__ leaf_tok,
    const int32_t* __restrict__ leaf_depth, const int32_t* __restrict__ n_leaves, int max_leaves, float T,
    uint64_t seed, DevState* st, const int* __restrict__ dec, const int* __restrict__ corr, int32_t* __restrict__ out,
    int32_t* __restrict__ n_out) {
  __shared__ int s_i, s_nd, s_acc;
  __shared__ float tots[TREE_KMAX + TREE_SLOTS + 1];
  const int tid = threadIdx.x;
  const int dp = max(min(*n_drafted, d), 0);
  const int nl = max(min(*n_leaves, max_leaves), 0);
  if (tid == 0) {
    st->tree_leaf = -1;
    int bad = 0;
    for (int r = 0; r <= dp; ++r) bad |= corr[r] < 0;
    if (bad) st->error_flags |= ERRF_NUMERIC;
    int i = bad ? -1 : 0;
    while (i >= 0 && i < dp && dec[i]) { out[i] = drafts[i]; ++i; }
    int nd = 0;
    if (i < dp)
      for (int s = 0; s < nl; ++s) nd += leaf_depth[s] == i + 1;
    s_i = i;
    s_nd = nd;
    if (i < 0) *n_out = 0;                                 // non-finite logits: nothing is emitted
    else if (i == dp || nd == 0) { out[i] = corr[i]; *n_out = i + 1; }
  }
  __syncthreads();
  const int i = s_i;
  if (i < 0 || i == dp || s_nd == 0) return;
  const float* p = zp + (size_t)i * V;
  const float* q = zq + (size_t)i * V;
  const float lse_p = block_lse(p, V, T);
  const float lse_q = block_lse(q, V, T);
  const int iter = st->iteration;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  int nu = 0;                                     // residual updates with a nonzero sum so far
  // p'(v) after the first u updates
  auto cur = [&](float pv, float qv, int u) {
    float x = expf(pv / T - lse_p);
    const float qq = expf(qv / T - lse_q);
    for (int t = 0; t < u; ++t) x = fmaxf(0.f, x - qq) / tots[t];
    return x;
  };
  auto update = [&]() {                           // after a rejection: the sum of max(0, p' - q)
    float acc = 0.f;
    for_quads<1024>(p, q, V, [&](int v4, const float* pq, const float* qq4) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v4 + e < V) acc += fmaxf(0.f, cur(pq[e], qq4[e], nu) - expf(qq4[e] / T - lse_q));
    });
    const float tot = block_sum_1024(acc);
    if (tot > 0.f) {
      if (tid == 0) tots[nu] = tot;
      __syncthreads();
      ++nu;
    }
  };
  update();                                       // the chain's candidate was rejected
  int k = 0;
  for (int s = 0; s < nl; ++s) {
    if (leaf_depth[s] != i + 1) continue;
    ++k;
    const int c = min(max(leaf_tok[s], 0), V - 1);
    if (tid == 0) {
      const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)(i + TREE_ROW_STRIDE * k), PURPOSE_ACCEPT, 0u, k0, k1);
      const float u = word_to_uniform(w.x);
      const float lqc = q[c] / T - lse_q;
      float lpc = p[c] / T - lse_p;
      if (nu > 0) {
        const float x = cur(p[c], q[c], nu);
        lpc = x > 0.f ? logf(x) : -INFINITY;
      }
      s_acc = (logf(u) + lqc) < lpc;
    }
    __syncthreads();
    if (s_acc) {
      // the leaf and a draw from its own row
      const float* zl = zp + (size_t)(dp + 1 + s) * V;
      float kb = -INFINITY;
      int ib = 0x7fffffff;
      const uint32_t row = (uint32_t)(i + TREE_ROW_STRIDE * k);
      for_quads<1024>(zl, zl, V, [&](int v4, const float* a, const float*) {
        const U4 w = philox4x32_10((uint32_t)iter, row, PURPOSE_SAMPLE, (uint32_t)(v4 >> 2), k0, k1);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (v4 + e < V) argmax_merge(kb, ib, a[e] / T + word_to_gumbel(ws[e]), v4 + e);
      });
      const int b = block_argmax_1024(kb, ib);
      if (tid == 0) {
        out[i] = c;
        out[i + 1] = b;
        *n_out = i + 2;
        st->tree_leaf = s;
        st->tree_leaf_pos = st->kvlen + i + 1;
      }
      return;
    }
    update();
  }
  // every candidate rejected: a draw from the last nonzero residual (or from p)
  float kb = -INFINITY;
  int ib = 0x7fffffff;
  for_quads<1024>(p, q, V, [&](int v4, const float* pq, const float* qq4) {
    const U4 w = philox4x32_10((uint32_t)iter, (uint32_t)i, PURPOSE_SAMPLE, (uint32_t)(v4 >> 2), k0, k1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (v4 + e >= V) continue;
      float key;
      if (nu == 0) {
        key = (pq[e] / T - lse_p) + word_to_gumbel(ws[e]);
      } else {
        const float r = fmaxf(0.f, cur(pq[e], qq4[e], nu - 1) - expf(qq4[e] / T - lse_q));
        if (!(r > 0.f)) continue;
        key = logf(r) + word_to_gumbel(ws[e]);
      }
      argmax_merge(kb, ib, key, v4 + e);
    }
  });
  const int b = block_argmax_1024(kb, ib);
  if (tid == 0) {
    out[i] = b;
    *n_out = i + 1;
  }
}

int launch_tree_accept_sampled(const float* zp, const float* zq, int V, const int32_t* drafts,
                               const int32_t* n_drafted, int d, const int32_t* leaf_tok, const int32_t* leaf_depth,
                               const int32_t* n_leaves, int max_leaves, float T, uint64_t seed, DevState* st,
                               int* dec, int* corr, int32_t* out, int32_t* n_out, hipStream_t s) {
  hipLaunchKernelGGL(accept_rows_kernel, dim3(d + 1), dim3(1024), 0, s, zp, zq, V, drafts, n_drafted, T, seed,
                     &st->iteration, 0, dec, corr);
  hipLaunchKernelGGL(tree_accept_sampled_kernel, dim3(1), dim3(1024), 0, s, zp, zq, V, drafts, n_drafted, d, leaf_tok,
                     leaf_depth, n_leaves, max_leaves, T, seed, st, dec, corr, out, n_out);
  return last_launch();
}

int launch_accept(const float* zp, const float* zq, int V, const int32_t* drafts, const int32_t* n_drafted, int d,
                  float T, uint64_t seed, const int* iter_ptr, int iter_const, int* dec, int* corr,
                  int32_t* out_tokens, int32_t* n_out, int* err_flags, hipStream_t s) {
  hipLaunchKernelGGL(accept_rows_kernel, dim3(d + 1), dim3(1024), 0, s, zp, zq, V, drafts, n_drafted, T, seed,
                     iter_ptr, iter_const, dec, corr);
  hipLaunchKernelGGL(accept_emit_kernel, dim3(1), dim3(64), 0, s, drafts, n_drafted, d, dec, corr, out_tokens,
                     n_out, err_flags);
  return last_launch();
}

// ===========================================================================
// Commit and control kernels (single wave).
// ===========================================================================

// n_out outside 0..max_n: ERRF_INPUT, nothing committed; n_out = 0 (an acceptance that saw non-finite
// logits): nothing committed, the iteration counter still moves on.
__global__ void commit_kernel(DevState* st, const int32_t* __restrict__ out_tokens, const int32_t* __restrict__ n_out,
                              int32_t* __restrict__ log, int log_cap, int max_n) {
  if (threadIdx.x != 0) return;
  const int n = *n_out;
  if (n < 0 || n > max_n) {
    st->error_flags |= ERRF_INPUT;
    st->n_emitted = 0;
    return;
  }
  if (n == 0) {
    st->iteration += 1;
    st->n_emitted = 0;
    return;
  }
  for (int t = 0; t < n; ++t) {
    const int idx = st->n_out + t;
    if (idx < log_cap) log[idx] = out_tokens[t];
    else st->error_flags |= ERRF_CAPACITY;
  }
  st->n_out += n;
  st->kvlen += n;
  st->last_token = out_tokens[n - 1];
  st->iteration += 1;
  st->n_emitted = n;
}

int launch_commit(DevState* st, const int32_t* out_tokens, const int32_t* n_out, int32_t* log, int log_cap, int max_n,
                  hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, s, st, out_tokens, n_out, log, log_cap, max_n);
  return last_launch();
}

__global__ void pick_commit_kernel(const ssd_row_stat* __restrict__ stat, DevState* st, int32_t* __restrict__ log,
                                   int log_cap, int set_kvlen, int kvlen_value) {
  if (threadIdx.x != 0) return;
  const int tok = stat->sample;
  if (!isfinite(stat->max) || !isfinite(stat->lse)) st->error_flags |= ERRF_NUMERIC;
  if (st->n_out < log_cap) log[st->n_out] = tok;
  else st->error_flags |= ERRF_CAPACITY;
  st->n_out += 1;
  st->kvlen = set_kvlen ? kvlen_value : st->kvlen + 1;
  st->last_token = tok;
  st->iteration += 1;
  st->n_emitted = 1;
}

int launch_pick_commit(const ssd_row_stat* stat, DevState* st, int32_t* log, int log_cap, int set_kvlen,
                       int kvlen_value, hipStream_t s) {
  hipLaunchKernelGGL(pick_commit_kernel, dim3(1), dim3(64), 0, s, stat, st, log, log_cap, set_kvlen, kvlen_value);
  return last_launch();
}

__global__ void state_init_kernel(DevState* st) {
  if (threadIdx.x == 0) {
    st->kvlen = 0; st->last_token = 0; st->iteration = 0; st->n_out = 0; st->error_flags = 0;
    st->n_drafted = 0; st->stop = 0; st->n_emitted = 0; st->verify_rows = 0;
    st->tree_rows = st->tree_prefix_rows = st->tree_side_full = st->tree_side_prefix = 0;
    st->tree_leaf = -1; st->tree_leaf_pos = 0;
  }
}

int launch_state_init(DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(64), 0, s, st);
  return last_launch();
}

__global__ void fill_positions_kernel(int* pos, int M, int start) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < M) pos[i] = start + i;
}

int launch_fill_positions(int* pos, int M, int start, hipStream_t s) {
  hipLaunchKernelGGL(fill_positions_kernel, dim3((M + 255) / 256), dim3(256), 0, s, pos, M, start);
  return last_launch();
}

// Scoring rows j = c * gamma + i: token window[i] at position pos0 + i.
__global__ void window_rows_kernel(const int32_t* __restrict__ window, int R, int gamma, int pos0, int* pos,
                                   int* tok) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < R) { pos[j] = pos0 + j % gamma; tok[j] = window[j % gamma]; }
}

int launch_window_rows(const int32_t* window, int R, int gamma, int pos0, int* pos, int* tok, hipStream_t s) {
  hipLaunchKernelGGL(window_rows_kernel, dim3((R + 255) / 256), dim3(256), 0, s, window, R, gamma, pos0, pos, tok);
  return last_launch();
}

// Residual rows of candidate pairs (src, dst): rows dst * gamma + i take rows src * gamma + i, i < gamma.
// One block per copied row.
__global__ __launch_bounds__(256) void copy_candidate_rows_kernel(float* __restrict__ h, int D,
                                                                  const int* __restrict__ pairs, int gamma) {
  const int p = blockIdx.x / gamma, i = blockIdx.x % gamma;
  const float* src = h + ((size_t)pairs[2 * p] * gamma + i) * D;
  float* dst = h + ((size_t)pairs[2 * p + 1] * gamma + i) * D;
  for (int k = threadIdx.x; k < D; k += 256) dst[k] = src[k];
}

int launch_copy_candidate_rows(float* h, int D, const int* pairs, int n_pairs, int gamma, hipStream_t s) {
  if (n_pairs <= 0) return 0;
  hipLaunchKernelGGL(copy_candidate_rows_kernel, dim3(n_pairs * gamma), dim3(256), 0, s, h, D, pairs, gamma);
  return last_launch();
}

// AR step: the newest token at position kvlen.
__global__ void single_row_prep_kernel(DevState* st, int* pos1, int* tok1, int max_ctx) {
  if (threadIdx.x != 0) return;
  const int p = st->kvlen;
  if (p >= max_ctx) st->error_flags |= ERRF_CAPACITY;
  pos1[0] = min(p, max_ctx - 1);
  tok1[0] = st->last_token;
}

int launch_single_row_prep(DevState* st, int* pos1, int* tok1, int max_ctx, hipStream_t s) {
  hipLaunchKernelGGL(single_row_prep_kernel, dim3(1), dim3(64), 0, s, st, pos1, tok1, max_ctx);
  return last_launch();
}

__global__ void draft_begin_kernel(DevState* st) {
  if (threadIdx.x == 0) { st->stop = 0; st->n_drafted = 0; }
}

int launch_draft_begin(DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(draft_begin_kernel, dim3(1), dim3(64), 0, s, st);
  return last_launch();
}

// Draft step j feeds y_{j-1} at position kvlen + j - 1.
__global__ void draft_step_prep_kernel(DevState* st, const int32_t* __restrict__ drafts, int j, int* pos1,
                                       int* tok1, int max_ctx, int32_t* __restrict__ n_drafted_out) {
  if (threadIdx.x != 0 || st->stop) return;
  const int p = st->kvlen + j - 1;
  if (p + 1 >= max_ctx) {
    // out of KV pages: end the draft (verify needs position kvlen + d' too)
    st->error_flags |= ERRF_CAPACITY;
    st->stop = 1;
    st->n_drafted = max(j - 1, 0);
    *n_drafted_out = max(j - 1, 0);
    return;
  }
  pos1[0] = p;
  tok1[0] = j == 1 ? st->last_token : drafts[j - 2];
}

int launch_draft_step_prep(DevState* st, const int32_t* drafts, int j, int* pos1, int* tok1, int max_ctx,
                           int32_t* n_drafted_out, hipStream_t s) {
  hipLaunchKernelGGL(draft_step_prep_kernel, dim3(1), dim3(64), 0, s, st, drafts, j, pos1, tok1, max_ctx,
                     n_drafted_out);
  return last_launch();
}

// Verify rows i = 0..d': tokens y_0..y_d' at positions kvlen + i; pos1/tok1 = the last row.
__global__ void verify_prep_kernel(DevState* st, const int32_t* __restrict__ drafts,
                                   const int32_t* __restrict__ n_drafted, int d, int* vpos, int* vtok, int* pos1,
                                   int* tok1, int max_ctx) {
  const int i = threadIdx.x;
  const int dp = min(*n_drafted, d);
  const int kv = st->kvlen;
  if (i <= d) {
    const int p = min(kv + i, max_ctx - 1);
    vpos[i] = p;
    vtok[i] = i == 0 ? st->last_token : drafts[i - 1];
  }
  __syncthreads();
  if (i == 0) {
    if (kv + dp >= max_ctx) st->error_flags |= ERRF_CAPACITY;
    st->verify_rows = dp + 1;
    pos1[0] = vpos[dp];
    tok1[0] = vtok[dp];
  }
}

int launch_verify_prep(DevState* st, const int32_t* drafts, const int32_t* n_drafted, int d, int* vpos, int* vtok,
                       int* pos1, int* tok1, int max_ctx, hipStream_t s) {
  hipLaunchKernelGGL(verify_prep_kernel, dim3(1), dim3(64), 0, s, st, drafts, n_drafted, d, vpos, vtok, pos1, tok1,
                     max_ctx);
  return last_launch();
}

__global__ void copy_rows_kernel(const float* __restrict__ src, float* __restrict__ dst, int rows, int D,
                                 const int* __restrict__ count, const int* __restrict__ dst_off,
                                 const int* __restrict__ stop) {
  if (stop && *stop) return;
  const int r = blockIdx.x;
  const int n = count ? min(rows, *count) : rows;
  if (r >= n) return;
  const int off = dst_off ? *dst_off : 0;
  for (int i = threadIdx.x; i < D; i += 256) dst[(size_t)(r + off) * D + i] = src[(size_t)r * D + i];
}

int launch_copy_rows(const float* src, float* dst, int rows, int D, const int* count, const int* dst_off,
                     const int* stop, hipStream_t s) {
  if (rows <= 0) return 0;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(rows), dim3(256), 0, s, src, dst, rows, D, count, dst_off, stop);
  return last_launch();
}

// Row-major bf16 [N, K] -> packed tile layout (wpk_index); one thread per 16
// bytes of the output, padding rows zero.
__global__ __launch_bounds__(256) void pack_bf16_kernel(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst,
                                                        int N, int K) {
  const size_t total = (size_t)((N + 15) / 16) * 16 * K / 8;
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= total) return;
  const size_t e = c * 8;
  const size_t blk = e / 512;
  const int within = (int)(e % 512);
  const int ksteps = K / 32;
  const int n = (int)(blk / ksteps) * 16 + within / 32;
  const int k = (int)(blk % ksteps) * 32 + within % 32;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (n < N) v = *(const u32x4*)(src + (size_t)n * K + k);
  *(u32x4*)(dst + e) = v;
}

int launch_pack_bf16(const void* src, void* dst, int N, int K, hipStream_t s) {
  if (N <= 0 || K <= 0 || K % 32 != 0) return SSD_ERR_SHAPE;
  const size_t total = (size_t)((N + 15) / 16) * 16 * K / 8;
  hipLaunchKernelGGL(pack_bf16_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, (const bf16_t*)src,
                     (bf16_t*)dst, N, K);
  return last_launch();
}

// Matchness: per candidate the fraction of rows whose argmax equals the next
// window token; best = highest score, lowest index on ties.
__global__ void score_kernel(const ssd_row_stat* __restrict__ stats, const int32_t* __restrict__ window,
                             int n_masks, int gamma, float* __restrict__ scores, int32_t* __restrict__ best,
                             int32_t* __restrict__ row_pred) {
  __shared__ int hits[1024];
  const int c = threadIdx.x;
  if (c < n_masks) {
    int h = 0;
    for (int i = 0; i < gamma; ++i) {
      const int pr = stats[c * gamma + i].argmax;
      h += pr == window[i + 1];
      if (row_pred) row_pred[c * gamma + i] = pr;
    }
    hits[c] = h;
    scores[c] = (float)h / (float)gamma;
  }
  __syncthreads();
  if (c == 0) {
    int b = 0;
    for (int k = 1; k < n_masks; ++k)
      if (hits[k] > hits[b]) b = k;
    *best = b;
  }
}

// ===========================================================================
// SpecEE exit features of hidden states (SpecEE notes §4.3.1): for k
// speculative tokens t_j, z_j = the shared final norm and LM head restricted to
// the k columns (bf16(h / rms(h) * g) . W[t_j], the LM head's own rounding
// point), the local probabilities p = softmax(z) over the k, and the variation
// p - p_prev against the previous layer's (0 without one).  One workgroup per row.
// ===========================================================================

// Two passes over the row: the sum of squares (canonical tile order) gives the row's 1 / rms; then each
// thread keeps the k dot products of its 8-element chunks of x = rnd(h * gain * inv), and the wave sums
// (butterfly) are added in wave order.
template <typename T>
__global__ __launch_bounds__(256) void specee_features_kernel(const float* __restrict__ h, int D, float eps,
                                                              const float* __restrict__ gain, const T* __restrict__ W,
                                                              int V, const int32_t* __restrict__ tokens, int k,
                                                              const float* __restrict__ prev, float* __restrict__ out) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int KM = 16;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* hr = h + (size_t)row * D;
  __shared__ float red[4][KM];
  __shared__ float tss[1024];                  // 16-feature tile sums, D <= 16384
  __shared__ float s_inv;
  int tk[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) tk[j] = j < k ? min(max(tokens[j], 0), V - 1) : 0;
  for (int i0 = 0; i0 < D; i0 += 256) {        // D % 16 == 0: each 16-lane group is inside or outside the row
    const int i = i0 + tid;
    const float t = tile16_ss_lanes(i < D ? hr[i] : 0.f);
    if (i < D && (tid & 15) == 0) tss[i >> 4] = t;
  }
  __syncthreads();
  if (tid < 64) {
    const float tot = row_ss_total(tss, 1, D / 16);
    if (tid == 0) s_inv = inv_rms(tot, D, eps);
  }
  __syncthreads();
  const float inv = s_inv;
  float part[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) part[j] = 0.f;
  for (int c = tid; c < D / 8; c += 256) {
    const int i = 8 * c;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float hg = fmul_nc(hr[i + e], gain[i + e]);
      x[e] = BF ? bf2f(norm_bf16(hg, inv)) : fmul_nc(hg, inv);
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= k) break;
      const T* wp = BF ? W + wpk_index(tk[j], i, D) : W + (size_t)tk[j] * D + i;   // 8 consecutive elements
#pragma unroll
      for (int e = 0; e < 8; ++e) part[j] = fmaf(x[e], ld(wp + e), part[j]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
    for (int j = 0; j < KM; ++j) part[j] += __shfl_xor(part[j], o, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) red[wave][j] = part[j];
  }
  __syncthreads();
  if (tid == 0) {
    float z[KM];
    float m = -INFINITY;
    for (int j = 0; j < k; ++j) {
      z[j] = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
      m = fmaxf(m, z[j]);
    }
    float sum = 0.f;
    for (int j = 0; j < k; ++j) sum += expf(z[j] - m);
    float* o = out + (size_t)row * 3 * k;
    for (int j = 0; j < k; ++j) {
      const float p = expf(z[j] - m) / sum;
      o[j] = z[j];
      o[k + j] = p;
      o[2 * k + j] = prev ? p - prev[(size_t)row * k + j] : 0.f;
    }
  }
}

int launch_specee_features(int dtype, const float* h, int rows, int D, float eps, const float* gain, const void* W,
                           int V, const int32_t* tokens, int k, const float* prev, float* out, hipStream_t s) {
  if (rows <= 0) return 0;
  if (k < 1 || k > 16 || D % 16 != 0 || D > 16384) return SSD_ERR_SHAPE;
  if (dtype == SSD_DTYPE_BF16)
    hipLaunchKernelGGL(specee_features_kernel<bf16_t>, dim3(rows), dim3(256), 0, s, h, D, eps, gain,
                       (const bf16_t*)W, V, tokens, k, prev, out);
  else
    hipLaunchKernelGGL(specee_features_kernel<float>, dim3(rows), dim3(256), 0, s, h, D, eps, gain,
                       (const float*)W, V, tokens, k, prev, out);
  return last_launch();
}

int launch_score(const ssd_row_stat* stats, const int32_t* window, int n_masks, int gamma, float* scores,
                 int32_t* best, int32_t* row_pred, hipStream_t s) {
  if (n_masks > 1024) return SSD_ERR_CAPACITY;
  hipLaunchKernelGGL(score_kernel, dim3(1), dim3(1024), 0, s, stats, window, n_masks, gamma, scores, best,
                     row_pred);
  return last_launch();
}

}  // namespace ssd
