// BF16 / FP8 MFMA GEMM for many rows (the batched forward's layer GEMMs, its lm_head with
// the argmax epilogue, and the batched context append): 64 x 128 output tiles, activations
// (hi + lo bf16 terms) through an LDS ring by the global->LDS load, weights straight into
// registers from the T16 tiled copy.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dfl {

// Wide form for many rows (the batched forward): one workgroup computes WD_M rows x WD_N
// columns; wave w owns columns [32w, 32w + 32) as two T16 tiles. Per output element the MFMA
// sequence is the skinny kernels': 256-deep chains from zero, each 32-deep step one MFMA on
// the hi term, then one on the lo term.
//  * partial mode (layer GEMMs): the workgroup takes one group of gsz consecutive 256-deep
//    splits and adds their chains in split order from zero (each times the row's RMSNorm
//    scale under NORM). That is the group sum the consumers form from the skinny kernel's
//    per-split partials (sum_splits), so one partial per group is handed over.
//  * argmax mode (lm_head): one chain over the full K, then per row the best (value, lowest
//    index) over the workgroup's columns, and optionally the drafted rows' fp32 logits.
// Data movement: the k range streams in WD_KC-deep chunks. A chunk's activation rows (hi and
// lo) go through a ring of WD_NS LDS stages by the gfx950 global->LDS 16-byte load (no
// registers; each lane picks its source so that unit u of row r lands at unit u ^ ((r >> 1)
// & 7), which keeps the 16 rows one LDS cycle serves on distinct banks); its weight operands
// go straight into registers (every load one contiguous 1 KB run), as many chunks ahead.
// Chunk j + WD_NS - 1 is requested right after the barrier that ends chunk j - 1, and a wave
// waits only for its own loads of chunk j, so WD_NS - 1 chunks are in flight while one is
// multiplied.
constexpr int WD_M = 64;    // rows per workgroup (four 16-row tiles)
constexpr int WD_N = 128;   // columns per workgroup: 4 waves x 2 tiles
constexpr int WD_KC = 64;   // depth of one chunk
constexpr int WD_NS = 3;    // chunks in the ring (activation stages in LDS, weight sets in registers)
static_assert(WD_NS == 3, "the wide kernel's waits and stage rotation are written for three chunks");

struct WideOut {
  float* P;            // partial mode: P[group][M][N]
  long long ps;        //   group stride (elements)
  int gsz;             //   splits per group
  NormIn nrm;          //   NORM: the rows' slice sums of squares
  float* best_v;       // argmax mode: [M][n_groups]
  int* best_i;
  int n_groups, gamma;
  float* logits;       //   drafted rows' logits [rows][N] or null
  const float* wsc;    // FP8 weights: the per-row scales (padded to whole tiles)
};

// one ring stage: the activation chunk of WD_M rows, hi and (SPLIT) lo, each row WD_KC deep
// (8 units of 16 bytes, swizzled)
template <bool SPLIT>
struct WideStage {
  bf16 a[SPLIT ? 2 : 1][WD_M * WD_KC];
};

// s_waitcnt with vmcnt <= N (vmcnt[3:0] | vmcnt[5:4] << 14; expcnt and lgkmcnt left at maximum)
#define DFL_WIDE_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))

// SPLIT: the activation carries a lo term (A_lo); without it A is exact bf16 (the context
// append's target hidden states) and each step is one MFMA. FP8: W in the T16-FP8 layout
// (one 16-byte piece per tile and chunk), codes converted to exact bf16 operands in
// registers, each column scaled by its row scale as the skinny kernel scales it.
template <bool ARGMAX, bool NORM>
struct WideLds {
  float srs[NORM ? WD_M : 1];
  float sv[ARGMAX ? 4 : 1][ARGMAX ? WD_M : 1];
  int si[ARGMAX ? 4 : 1][ARGMAX ? WD_M : 1];
};

template <bool ARGMAX, bool NORM, bool SPLIT, bool FP8>
__device__ __forceinline__ void gemm_wide_wg(WideStage<SPLIT>& st0, WideStage<SPLIT>& st1, WideStage<SPLIT>& st2,
                                             WideLds<ARGMAX, NORM>& sm,
                                             const bf16* __restrict__ A, const bf16* __restrict__ A_lo, int lda,
                                             int M, const bf16* __restrict__ W, int N, int K, int gx, int gy,
                                             const WideOut& o) {
  constexpr int WM = WD_M / 16;
  constexpr int NT = SPLIT ? 2 : 1;          // activation terms
  constexpr int NWL = FP8 ? 1 : 2;           // weight loads per tile and chunk
  constexpr int OPS = NT * 2 + 2 * NWL;      // memory instructions a wave issues per chunk
  auto& srs = sm.srs;
  auto& sv = sm.sv;
  auto& si = sm.si;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  // workgroup id -> (column group x, row group y, split group z). Workgroups go to the eight
  // XCDs round robin, so the row groups of one column group get ids 8 apart: one XCD, one
  // L2, and their weight tiles leave HBM once.
  const int id = blockIdx.x;
  int q = id >> 3;
  const int y = q % gy;
  q /= gy;
  const int gx8 = (gx + 7) / 8;
  const int x = (q % gx8) * 8 + (id & 7), z = q / gx8;
  if (x >= gx) return;
  const int m0 = y * WD_M;
  const int S = K / 256;
  const int s_lo = ARGMAX ? 0 : z * o.gsz;
  const int s_hi = ARGMAX ? S : min(S, s_lo + o.gsz);
  const int kb = s_lo * 256;
  const int nck = (s_hi - s_lo) * (256 / WD_KC);
  const int ntiles = (N + 15) / 16;
  const int tile0 = x * 8 + wave * 2;
  // tiles past the last one re-read the last tile; their columns are never used
  const bf16* wp0 = W + (size_t)min(tile0, ntiles - 1) * 16 * K + lane * 8;
  const bf16* wp1 = W + (size_t)min(tile0 + 1, ntiles - 1) * 16 * K + lane * 8;
  const uint8_t* qp0 = reinterpret_cast<const uint8_t*>(W) + (size_t)min(tile0, ntiles - 1) * 16 * K + lane * 16;
  const uint8_t* qp1 = reinterpret_cast<const uint8_t*>(W) + (size_t)min(tile0 + 1, ntiles - 1) * 16 * K + lane * 16;
  float wsc[FP8 ? 2 : 1];
  if (FP8) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) wsc[FP8 ? nt : 0] = o.wsc[min(tile0 + nt, ntiles - 1) * 16 + c];
  }
  // this wave's two 1 KB pieces of each activation term of a stage: LDS units
  // P = (2 wave + h) * 64 + lane, row P / 8 (rows past M repeat the last row; their results
  // are never stored), source unit (P % 8) ^ ((row >> 1) & 7)
  // (the lane's part of the address is a loop-invariant element offset: the chunk is chosen by
  // a uniform base, so no address register is rewritten while a load that read it may be in
  // flight, which made the compiler wait for every load before reusing it)
  uint32_t voff[2];   // bytes
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int P = (2 * wave + h) * 64 + lane;
    const int r = P >> 3, u = (P & 7) ^ ((r >> 1) & 7);
    voff[h] = (uint32_t)(min(m0 + r, M - 1) * lda + u * 8) * 2u;
  }
  const bf16* srcA[NT] = {A + kb};
  if (SPLIT) srcA[NT - 1] = A_lo + kb;

  if (NORM) {
    // the rows' RMSNorm scales, each row's slice sums added as the skinny kernel adds them
    for (int r = threadIdx.x; r < WD_M; r += 256) {
      const float* qv = o.nrm.ssq + (size_t)min(m0 + r, M - 1) * SSQ_STRIDE;
      float s4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < SSQ_STRIDE / 4; ++t) s += qv[j + 4 * t];
        s4[j] = s;
      }
      srs[NORM ? r : 0] = rsqrtf(((s4[0] + s4[1]) + (s4[2] + s4[3])) / (float)o.nrm.h + o.nrm.eps);
    }
    __syncthreads();   // the scales, before any wave folds a split (and before any DMA is in flight)
  }

  // chunk j's loads: the activation stage (DMA into LDS), then the weight operands as raw
  // 16-byte pieces (bf16: one per tile and 32-deep step; FP8: one per tile). Every step issues
  // the same loads: past the last chunk it re-reads the last one (from L2) into a stage and a
  // weight set nothing reads again, so that the compiler sees one fixed count of loads in
  // flight (with a conditional issue it waited for every load before each chunk's MFMAs)
  auto issue = [&](WideStage<SPLIT>& st, u32x4 (&w)[2][NWL], int j) {
    // (a scalar: kept out of the per-lane address arithmetic)
    const int k = __builtin_amdgcn_readfirstlane(min(j, nck - 1) * WD_KC);   // relative to kb
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // (the empty asm keeps the 32-bit offset a value of this block, so the load takes the
        // scalar-base + 32-bit vector-offset form instead of a 64-bit address register)
        uint32_t vo = voff[h];
        asm volatile("" : "+v"(vo));
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(srcA[t] + k) + vo,
                                         st.a[t] + (2 * wave + h) * 512, 16, 0, 0);
      }
    const int kk = kb + k;
    if (FP8) {
      const size_t off = (size_t)(kk >> 8) * T16Q_BLOCK + ((kk & 255) >> 6) * 1024;
      w[0][0] = *reinterpret_cast<const u32x4*>(qp0 + off);
      w[1][0] = *reinterpret_cast<const u32x4*>(qp1 + off);
    } else {
      const size_t off = (size_t)(kk >> 8) * T16_BLOCK + ((kk & 255) >> 5) * 512;
#pragma unroll
      for (int s = 0; s < NWL; ++s) {
        w[0][s] = *reinterpret_cast<const u32x4*>(wp0 + off + s * 512);
        w[1][s] = *reinterpret_cast<const u32x4*>(wp1 + off + s * 512);
      }
    }
  };
  f32x4 acc[WM][2];
  f32x4 gs[ARGMAX ? 1 : WM][2];
#pragma unroll
  for (int mt = 0; mt < WM; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!ARGMAX) gs[ARGMAX ? 0 : mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // one chunk: per 32-deep step, the hi MFMAs of every (row tile, column tile), then the lo
  // ones (per element: hi, then lo, step after step)
  auto mma = [&](const WideStage<SPLIT>& st, const u32x4 (&w)[2][NWL]) {
#pragma unroll
    for (int s = 0; s < WD_KC / 32; ++s) {
      bf16x8 wv[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        wv[nt] = FP8 ? fp8x8_bf16(w[nt][0][2 * s], w[nt][0][2 * s + 1]) : __builtin_bit_cast(bf16x8, w[nt][FP8 ? 0 : s]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x8 av[WM];
        const bf16* base = st.a[t];
#pragma unroll
        for (int mt = 0; mt < WM; ++mt) {
          const int r = mt * 16 + c, u = s * 4 + g;
          av[mt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + r * WD_KC + ((u ^ ((r >> 1) & 7)) * 8)));
        }
#pragma unroll
        for (int mt = 0; mt < WM; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma16(av[mt], wv[nt], acc[mt][nt]);
      }
    }
  };
  // after chunk j: a 256-deep split ends every 256/WD_KC chunks; add its chain to the group
  // sum (times the row scale: a separate rounding, as when the skinny kernel stores it)
  auto fold = [&](int j) {
    if (ARGMAX || (j + 1) % (256 / WD_KC) != 0) return;
    {
#pragma clang fp contract(off)
#pragma unroll
    for (int mt = 0; mt < WM; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = acc[mt][nt][e];
          if (FP8) v = v * wsc[FP8 ? nt : 0];
          if (NORM) v = v * srs[NORM ? mt * 16 + 4 * g + e : 0];
          gs[ARGMAX ? 0 : mt][nt][e] += v;
        }
        acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // chunk j sits in ring stage j % WD_NS and weight set j % WD_NS; on entry to its step the
  // chunks j .. j + WD_NS - 2 are requested. The wave waits for its own loads of chunk j; the
  // barrier makes every wave's share of the stage visible and ends every wave's reads of stage
  // (j - 1) % WD_NS, which chunk j + WD_NS - 1 refills once chunk j's MFMAs are issued (its
  // weight set was last read by chunk j - 1's MFMAs)
  u32x4 wr[WD_NS][2][NWL];
  auto step = [&](int j, WideStage<SPLIT>& cur, const u32x4 (&wc)[2][NWL], WideStage<SPLIT>& nxt,
                  u32x4 (&wn)[2][NWL]) {
    DFL_WIDE_WAIT_VM(OPS);   // chunk j + 1's loads may still be in flight
    __builtin_amdgcn_s_barrier();
    mma(cur, wc);
    issue(nxt, wn, j + WD_NS - 1);
    fold(j);
  };
  issue(st0, wr[0], 0);
  issue(st1, wr[1], 1);
  for (int j = 0; j < nck; j += WD_NS) {
    step(j, st0, wr[0], st2, wr[2]);
    if (j + 1 < nck) step(j + 1, st1, wr[1], st0, wr[0]);
    if (j + 2 < nck) step(j + 2, st2, wr[2], st1, wr[1]);
  }

  if (!ARGMAX) {
    float* pp = o.P + (long long)z * o.ps;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int n = (tile0 + nt) * 16 + c;
      if (n >= N) continue;
#pragma unroll
      for (int mt = 0; mt < WM; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + mt * 16 + 4 * g + e;
          if (m < M) pp[(size_t)m * N + n] = gs[ARGMAX ? 0 : mt][nt][e];
        }
    }
    return;
  }
  // argmax: per row, the best over this lane's two columns, the 16 lanes of its row group,
  // then the four waves
#pragma unroll
  for (int mt = 0; mt < WM; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = m0 + mt * 16 + 4 * g + e;
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int n = (tile0 + nt) * 16 + c;
        if (n < N) {
          const float v = FP8 ? acc[mt][nt][e] * wsc[FP8 ? nt : 0] : acc[mt][nt][e];
          better(bv, bi, v, n);
          if (o.logits != nullptr && m < M) {
            const int b = m / o.gamma, i = m % o.gamma;
            if (i != 0) o.logits[(size_t)(b * (o.gamma - 1) + i - 1) * N + n] = v;
          }
        }
      }
#pragma unroll
      for (int of = 1; of < 16; of <<= 1) {
        const float ov = __shfl_xor(bv, of, 64);
        const int oi = __shfl_xor(bi, of, 64);
        better(bv, bi, ov, oi);
      }
      if (c == 0) {
        sv[ARGMAX ? wave : 0][ARGMAX ? mt * 16 + 4 * g + e : 0] = bv;
        si[ARGMAX ? wave : 0][ARGMAX ? mt * 16 + 4 * g + e : 0] = bi;
      }
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < WD_M; r += 256) {
    float bv = sv[0][ARGMAX ? r : 0];
    int bi = si[0][ARGMAX ? r : 0];
#pragma unroll
    for (int w = 1; w < 4; ++w) better(bv, bi, sv[ARGMAX ? w : 0][ARGMAX ? r : 0], si[ARGMAX ? w : 0][ARGMAX ? r : 0]);
    if (m0 + r < M) {
      o.best_v[(size_t)(m0 + r) * o.n_groups + x] = bv;
      o.best_i[(size_t)(m0 + r) * o.n_groups + x] = bi;
    }
  }
}

template <bool ARGMAX, bool NORM, bool SPLIT, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_wide(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, int lda, int M,
    const bf16* __restrict__ W, int N, int K, int gx, int gy, WideOut o) {
  // the ring's stages are separate LDS objects: the compiler then knows that a stage's reads
  // do not alias the loads in flight into the others (one array made it wait for every load
  // before the first read of each chunk)
  __shared__ __attribute__((aligned(16))) WideStage<SPLIT> st0, st1, st2;
  __shared__ WideLds<ARGMAX, NORM> sm;
  gemm_wide_wg<ARGMAX, NORM, SPLIT, FP8>(st0, st1, st2, sm, A, A_lo, lda, M, W, N, K, gx, gy, o);
}

static unsigned wide_grid(int gx, int gy, int gz) { return (unsigned)((gx + 7) / 8 * 8) * gy * gz; }

int gemm_wide_groups(int K, int gsz) { return (K / 256 + gsz - 1) / gsz; }

hipError_t launch_gemm_wide(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W, int N, int K,
                            int gsz, float* P, long long part_stride, hipStream_t st, const NormIn* norm,
                            const float* wsc) {
  if (M < 1 || N < 16 || N % 16 || K < 256 || K % 256 || gsz < 1) return hipErrorInvalidValue;
  if (norm && (!A_lo || norm->h != K || K > SSQ_STRIDE * SSQ_COLS)) return hipErrorInvalidValue;
  if (wsc && !A_lo) return hipErrorInvalidValue;
  const int gx = (N + WD_N - 1) / WD_N, gy = (M + WD_M - 1) / WD_M, gz = gemm_wide_groups(K, gsz);
  WideOut o{};
  o.P = P; o.ps = part_stride; o.gsz = gsz; o.wsc = wsc;
  const unsigned grid = wide_grid(gx, gy, gz);
  if (norm) o.nrm = *norm;
  if (wsc) {
    if (norm) (void)launch(k_gemm_wide<false, true, true, true>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, gx, gy, o);
    else (void)launch(k_gemm_wide<false, false, true, true>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, gx, gy, o);
  } else if (norm) {
    (void)launch(k_gemm_wide<false, true, true, false>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, gx, gy, o);
  } else if (A_lo) {
    (void)launch(k_gemm_wide<false, false, true, false>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, gx, gy, o);
  } else {
    (void)launch(k_gemm_wide<false, false, false, false>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, gx, gy, o);
  }
  return hipGetLastError();
}

int lmhead_wide_groups(int V) { return (V + WD_N - 1) / WD_N; }

hipError_t launch_lmhead_wide(const bf16* Y, const bf16* Y_lo, int ldy, int M, const bf16* W, int V, int K,
                              float* best_v, int* best_i, int n_groups, int gamma, float* logits, hipStream_t st,
                              const float* wsc) {
  if (M < 1 || !Y_lo || V < 1 || K < 256 || K % 256 || n_groups != lmhead_wide_groups(V) || gamma < 2)
    return hipErrorInvalidValue;
  WideOut o{};
  o.best_v = best_v; o.best_i = best_i; o.n_groups = n_groups; o.gamma = gamma; o.logits = logits; o.wsc = wsc;
  const int gy = (M + WD_M - 1) / WD_M;
  if (wsc)
    (void)launch(k_gemm_wide<true, false, true, true>, wide_grid(n_groups, gy, 1), 256, 0, st, Y, Y_lo, ldy, M, W, V,
                 K, n_groups, gy, o);
  else
    (void)launch(k_gemm_wide<true, false, true, false>, wide_grid(n_groups, gy, 1), 256, 0, st, Y, Y_lo, ldy, M, W, V,
                 K, n_groups, gy, o);
  return hipGetLastError();
}

}  // namespace dfl
