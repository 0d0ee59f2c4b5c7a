// LDS-tiled 128 x 128 x 64 BF16 MFMA GEMM for the context append (thousands of rows), fed
// by a ring of global->LDS stages.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dfl {

constexpr int TB = 128, TK = 64;
constexpr int T_ST = 3;   // stages of the LDS ring

// one stage: the A rows (hi and, with SPLIT, lo) and the W rows of a 64-deep k tile; row r's
// 16-byte unit u sits at unit u ^ ((r >> 1) & 7), so the 8 or 16 lanes an LDS cycle serves
// (16 consecutive rows, one unit) hit distinct banks
template <bool SPLIT>
struct TiledStage {
  bf16 a[TB * TK];
  bf16 al[SPLIT ? TB * TK : 8];
  bf16 w[TB * TK];
};

// s_waitcnt with vmcnt <= N (vmcnt[3:0] | vmcnt[5:4] << 14; expcnt and lgkmcnt left at maximum)
#define DFL_GEMM_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))

// C = A W^T over the full K (plain fp32 results; the sum over k runs in order, k tile by k
// tile, the hi then the lo term at every 32-deep step). One 4-wave workgroup per 128x128
// tile, each wave 64x64. The k tiles stream through a ring of three LDS stages with the
// gfx950 global->LDS 16-byte load: wave v brings a quarter of every operand of a stage, 1 KB
// an instruction, each lane choosing its source so that the LDS copy is swizzled. Tile j+2 is
// requested right after the barrier that ends tile j-1; a wave waits only for its own loads
// of tile j (one barrier per tile).
template <bool SPLIT>
__device__ __forceinline__ void gemm_tiled_wg(TiledStage<SPLIT> (&ring)[T_ST], const bf16* __restrict__ A,
                                              const bf16* __restrict__ A_lo, int lda, int M,
                                              const bf16* __restrict__ W, int N, int K,
                                              float* __restrict__ C, int ldc) {
  constexpr int NI = SPLIT ? 12 : 8;   // DMA instructions per wave and stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  const int c = lane & 15, g = lane >> 4;
  const int nk = K / TK;
  // this wave's four 1 KB pieces of an operand: LDS units P = wave*256 + q*64 + lane
  const bf16* srcA[4];
  const bf16* srcAl[4];
  const bf16* srcW[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int P = wave * 256 + q * 64 + lane;
    const int r = P >> 3, u = (P & 7) ^ ((r >> 1) & 7);
    const int gm = min(m0 + r, M - 1), gn = min(n0 + r, N - 1);
    srcA[q] = A + (size_t)gm * lda + u * 8;
    srcAl[q] = SPLIT ? A_lo + (size_t)gm * lda + u * 8 : nullptr;
    srcW[q] = W + (size_t)gn * K + u * 8;
  }
  auto issue = [&](TiledStage<SPLIT>& st, int kt) {
    const int k0 = kt * TK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = (wave * 4 + q) * 512;
      __builtin_amdgcn_global_load_lds(srcA[q] + k0, &st.a[o], 16, 0, 0);
      if (SPLIT) __builtin_amdgcn_global_load_lds(srcAl[q] + k0, &st.al[o], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(srcW[q] + k0, &st.w[o], 16, 0, 0);
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const bf16* base, int r, int u) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + r * TK + ((u ^ ((r >> 1) & 7)) * 8)));
  };
  auto step = [&](int kt, const TiledStage<SPLIT>& cur, TiledStage<SPLIT>& nxt) {
    if (kt + 1 < nk) DFL_GEMM_WAIT_VM(NI); else DFL_GEMM_WAIT_VM(0);
    __builtin_amdgcn_s_barrier();
    if (kt + 2 < nk) issue(nxt, kt + 2);
#pragma unroll
    for (int kk = 0; kk < TK; kk += 32) {
      bf16x8 a[4], al[4], b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = frag(cur.a, wm * 64 + t * 16 + c, kk / 8 + g);
        if (SPLIT) al[t] = frag(cur.al, wm * 64 + t * 16 + c, kk / 8 + g);
        b[t] = frag(cur.w, wn * 64 + t * 16 + c, kk / 8 + g);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
          if (SPLIT) acc[i][j] = mfma16(al[i], b[j], acc[i][j]);
        }
    }
  };
  issue(ring[0], 0);
  if (nk > 1) issue(ring[1], 1);
  for (int k0 = 0; k0 < nk; k0 += T_ST) {
    step(k0, ring[0], ring[2]);
    if (k0 + 1 < nk) step(k0 + 1, ring[1], ring[0]);
    if (k0 + 2 < nk) step(k0 + 2, ring[2], ring[1]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + j * 16 + c;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + i * 16 + 4 * g + e;
        if (m < M) C[(size_t)m * ldc + n] = acc[i][j][e];
      }
    }
  }
}

template <bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_tiled(const bf16* __restrict__ A,
                                                    const bf16* __restrict__ A_lo, int lda, int M,
                                                    const bf16* __restrict__ W, int N, int K,
                                                    float* __restrict__ C, int ldc) {
  __shared__ __attribute__((aligned(16))) TiledStage<SPLIT> ring[T_ST];
  gemm_tiled_wg<SPLIT>(ring, A, A_lo, lda, M, W, N, K, C, ldc);
}

hipError_t launch_gemm_tiled(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W,
                             int N, int K, float* C, int ldc, hipStream_t st) {
  if (M <= 0 || N <= 0 || K < TK || (K % TK) != 0 || (lda % 8) != 0) return hipErrorInvalidValue;
  dim3 grid((N + TB - 1) / TB, (M + TB - 1) / TB);
  if (A_lo)
    (void)launch(k_gemm_tiled<true>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, C, ldc);
  else
    (void)launch(k_gemm_tiled<false>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, C, ldc);
  return hipGetLastError();
}

}  // namespace dfl
