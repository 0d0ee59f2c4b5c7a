// LDS-tiled 256 x 256 BF16 MFMA GEMM for the context append (thousands of rows), fed by a
// ring of global->LDS stages.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dfl {

constexpr int TB_M = 256, TB_N = 256;  // output tile of a workgroup
constexpr int TK = 32;                 // depth of one stage (one MFMA step)
constexpr int T_WAVES = 8;             // 2 row halves x 4 column quarters: a wave owns 128 x 64
constexpr int T_KS_MAX = 4;            // k splits at most

// one stage: the A rows (hi and, with SPLIT, lo) and the W rows of a 32-deep k step, 64 bytes
// a row; row r's 16-byte unit u sits at unit u ^ ((r >> 1) & 3), so the 8 lanes an LDS cycle
// serves (rows 0-7 of a 16-row fragment, one unit) hit distinct 16-byte bank groups
template <bool SPLIT>
struct TiledStage {
  bf16 a[TB_M * TK];
  bf16 al[SPLIT ? TB_M * TK : 8];
  bf16 w[TB_N * TK];
};

// s_waitcnt with vmcnt <= N (vmcnt[3:0] | vmcnt[5:4] << 14; expcnt and lgkmcnt left at maximum)
#define DFL_GEMM_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))

// k splits: from (N, K) alone, never from the row count, so that a row's result does not
// depend on how rows are grouped into launches. A narrow output (few 256-column tiles) splits
// its K in two or four so that a 2048-row launch still has about a chip's worth of workgroups.
int gemm_tiled_splits(int N, int K) {
  const int tiles = (APPEND_ROWS / TB_M) * ((N + TB_N - 1) / TB_N);
  int ks = 1;
  while (ks < T_KS_MAX && tiles * ks * 2 <= 256 && K % (TK * ks * 2) == 0) ks *= 2;
  return ks;
}

// C[z] = A W^T over k split z (plain fp32 results; within a split the sum over k runs in
// order, step by step, the hi then the lo term at every 32-deep step). One 8-wave workgroup
// per 256 x 256 tile and split, each wave 128 x 64 (eight 16-row by four 16-column MFMA
// tiles): per step a wave reads 16 (hi, lo) activation fragments and 4 weight fragments for
// 64 MFMAs, and the workgroup brings 48 KB into LDS for 256 x 256 x 32 products (a 128 x 128
// tile brings 24 KB for a quarter of them). The steps stream through a ring of three LDS
// stages with the gfx950 global->LDS 16-byte load: wave v brings an eighth of every operand
// of a stage, 1 KB an instruction, each lane choosing its source so that the LDS copy is
// swizzled. Step j+2 is requested right after the barrier that ends step j-1; a wave waits
// only for its own loads of step j (one barrier per step). Every step issues the same loads
// (past the last step it re-reads the last one into a stage nobody reads again), so the
// compiler sees one fixed count in flight, and the three stages are separate LDS objects.
template <bool SPLIT>
__device__ __forceinline__ void gemm_tiled_wg(TiledStage<SPLIT>& st0, TiledStage<SPLIT>& st1, TiledStage<SPLIT>& st2,
                                              const bf16* __restrict__ A, const bf16* __restrict__ A_lo, int lda,
                                              int M, const bf16* __restrict__ W, int N, int K, int kps,
                                              float* __restrict__ C, int ldc) {
  constexpr int NI = SPLIT ? 6 : 4;   // DMA instructions per wave and stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = blockIdx.y * TB_M, n0 = blockIdx.x * TB_N;
  const int kb = blockIdx.z * kps;
  const int nk = kps / TK;
  const int c = lane & 15, g = lane >> 4;
  // this wave's two 1 KB pieces of each operand of a stage: LDS units P = (2 wave + h) * 64 +
  // lane, row P / 4, source unit (P % 4) ^ ((row >> 1) & 3); byte offsets (rows past M or N
  // repeat the last one; their results are never stored), loop-invariant
  uint32_t offA[2], offW[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int P = (2 * wave + h) * 64 + lane;
    const int r = P >> 2, u = (P & 3) ^ ((r >> 1) & 3);
    offA[h] = (uint32_t)((size_t)min(m0 + r, M - 1) * lda + u * 8) * 2u;
    offW[h] = (uint32_t)((size_t)min(n0 + r, N - 1) * K + u * 8) * 2u;
  }
  const bf16* srcA = A + kb;
  const bf16* srcAl = SPLIT ? A_lo + kb : A;
  const bf16* srcW = W + kb;
  auto issue = [&](TiledStage<SPLIT>& st, int j) {
    const int k = __builtin_amdgcn_readfirstlane(min(j, nk - 1) * TK);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = (2 * wave + h) * 512;
      uint32_t va = offA[h], vw = offW[h];
      asm volatile("" : "+v"(va), "+v"(vw));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(srcA + k) + va, &st.a[o], 16, 0, 0);
      if (SPLIT) __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(srcAl + k) + va, &st.al[o], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(srcW + k) + vw, &st.w[o], 16, 0, 0);
    }
  };
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const bf16* base, int r) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + r * TK + ((g ^ ((r >> 1) & 3)) * 8)));
  };
  auto mma = [&](const TiledStage<SPLIT>& st) {
    bf16x8 b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag(st.w, wn * 64 + j * 16 + c);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x8 a = frag(st.a, wm * 128 + i * 16 + c);
      const bf16x8 al = SPLIT ? frag(st.al, wm * 128 + i * 16 + c) : a;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma16(a, b[j], acc[i][j]);
        if (SPLIT) acc[i][j] = mfma16(al, b[j], acc[i][j]);
      }
    }
  };
  auto step = [&](int j, const TiledStage<SPLIT>& cur, TiledStage<SPLIT>& nxt) {
    DFL_GEMM_WAIT_VM(NI);   // step j + 1's loads may still be in flight
    __builtin_amdgcn_s_barrier();
    issue(nxt, j + 2);
    if (j < nk) mma(cur);
  };
  issue(st0, 0);
  issue(st1, 1);
  for (int j = 0; j < nk; j += 3) {
    step(j, st0, st2);
    step(j + 1, st1, st0);
    step(j + 2, st2, st1);
  }
  DFL_GEMM_WAIT_VM(0);   // the loads past the last step land before the workgroup ends
  float* Cz = C + (size_t)blockIdx.z * M * ldc;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + c;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 128 + i * 16 + 4 * g + e;
        if (m < M) Cz[(size_t)m * ldc + n] = acc[i][j][e];
      }
    }
  }
}

template <bool SPLIT>
__global__ __launch_bounds__(T_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void k_gemm_tiled(
    const bf16* __restrict__ A, const bf16* __restrict__ A_lo, int lda, int M, const bf16* __restrict__ W, int N,
    int K, int kps, float* __restrict__ C, int ldc) {
  __shared__ __attribute__((aligned(16))) TiledStage<SPLIT> st0, st1, st2;
  gemm_tiled_wg<SPLIT>(st0, st1, st2, A, A_lo, lda, M, W, N, K, kps, C, ldc);
}

hipError_t launch_gemm_tiled(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W, int N, int K, int ks,
                             float* C, int ldc, hipStream_t st) {
  if (M <= 0 || N <= 0 || ks < 1 || ks > T_KS_MAX || K % (TK * ks) != 0 || (lda % 8) != 0 || ldc < N)
    return hipErrorInvalidValue;
  // the DMA offsets are 32-bit byte offsets from the operands' bases
  if ((size_t)M * lda * 2 >= (1ull << 32) || (size_t)N * K * 2 >= (1ull << 32)) return hipErrorInvalidValue;
  dim3 grid((N + TB_N - 1) / TB_N, (M + TB_M - 1) / TB_M, ks);
  const int kps = K / ks;
  if (A_lo)
    (void)launch(k_gemm_tiled<true>, grid, T_WAVES * 64, 0, st, A, A_lo, lda, M, W, N, K, kps, C, ldc);
  else
    (void)launch(k_gemm_tiled<false>, grid, T_WAVES * 64, 0, st, A, A_lo, lda, M, W, N, K, kps, C, ldc);
  return hipGetLastError();
}

}  // namespace dfl
