// BF16 MFMA GEMMs of the drafter: Y = A W^T with W row-major [N, K] (weights stored
// [out_features, in_features]).
//
//  * k_gemm_skinny: the weight-streaming form for the block forward (M = bands * gamma
//    rows, at most 64 per launch). One wavefront owns 16 output columns over one K split
//    and streams those 16 weight rows exactly once; the activation rows come from L2.
//    Partial sums of every split go to P[s][M][N] and are added in split order by the
//    consumer, so a row's result never depends on how many other rows share the launch.
//  * k_gemm_tiled: an LDS-tiled 128x128x64 form for the context append (thousands of rows).
//  * k_lmhead_argmax: the skinny form over the vocabulary with a running (max, index) per
//    row in the epilogue instead of a logits store; k_argmax_reduce finishes the argmax.
#include "common.hpp"
#include "kernels.hpp"

namespace dfl {

template <int MT>
__global__ __launch_bounds__(256) void k_gemm_skinny(const bf16* __restrict__ A, int lda, int M,
                                                     const bf16* __restrict__ W, int N, int K,
                                                     int k_len, float* __restrict__ P,
                                                     long long part_stride) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  if (n0 >= N) return;
  const int s = blockIdx.y;
  const int kb = s * k_len;
  const int ke = min(K, kb + k_len);
  const int c = lane & 15, g = lane >> 4;
  const int n = n0 + c;
  const bool nv = n < N;
  // out-of-range columns / rows read a valid row; their results are never stored
  const bf16* wp = W + (size_t)(nv ? n : n0) * K + g * 8;
  const bf16* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + c;
    ap[mt] = A + (size_t)(m < M ? m : 0) * lda + g * 8;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k = kb; k < ke; k += 128) {
    bf16x8 b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) b[u] = ld8(wp + k + u * 32);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      bf16x8 a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = ld8(ap[mt] + k + u * 32);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[mt] = mfma16(a[u], b[u], acc[mt]);
    }
  }
  if (!nv) return;
  float* pp = P + (long long)s * part_stride;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * g + i;
      if (m < M) pp[(size_t)m * N + n] = acc[mt][i];
    }
  }
}

hipError_t launch_gemm_skinny(const bf16* A, int lda, int M, const bf16* W, int N, int K,
                              int k_len, float* P, long long part_stride, hipStream_t st) {
  const int S = (K + k_len - 1) / k_len;
  dim3 grid((N + 63) / 64, S);
  const int mt = (M + 15) / 16;
  switch (mt) {
    case 1: k_gemm_skinny<1><<<grid, 256, 0, st>>>(A, lda, M, W, N, K, k_len, P, part_stride); break;
    case 2: k_gemm_skinny<2><<<grid, 256, 0, st>>>(A, lda, M, W, N, K, k_len, P, part_stride); break;
    case 3: k_gemm_skinny<3><<<grid, 256, 0, st>>>(A, lda, M, W, N, K, k_len, P, part_stride); break;
    case 4: k_gemm_skinny<4><<<grid, 256, 0, st>>>(A, lda, M, W, N, K, k_len, P, part_stride); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------

constexpr int TB = 128, TK = 64, TPAD = 8;

__global__ __launch_bounds__(256) void k_gemm_tiled(const bf16* __restrict__ A, int lda, int M,
                                                    const bf16* __restrict__ W, int N, int K,
                                                    float* __restrict__ C, int ldc) {
  __shared__ __attribute__((aligned(16))) bf16 sA[TB][TK + TPAD];
  __shared__ __attribute__((aligned(16))) bf16 sW[TB][TK + TPAD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  const int c = lane & 15, g = lane >> 4;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + i * 256;
      const int r = ch >> 3, cc = (ch & 7) * 8;
      const int gm = min(m0 + r, M - 1), gn = min(n0 + r, N - 1);
      *reinterpret_cast<u32x4*>(&sA[r][cc]) =
          *reinterpret_cast<const u32x4*>(A + (size_t)gm * lda + k0 + cc);
      *reinterpret_cast<u32x4*>(&sW[r][cc]) =
          *reinterpret_cast<const u32x4*>(W + (size_t)gn * K + k0 + cc);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; kk += 32) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sA[wm * 64 + t * 16 + c][kk + g * 8]));
        b[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sW[wn * 64 + t * 16 + c][kk + g * 8]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
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

hipError_t launch_gemm_tiled(const bf16* A, int lda, int M, const bf16* W, int N, int K,
                             float* C, int ldc, hipStream_t st) {
  if (M <= 0 || N <= 0 || (K % TK) != 0) return hipErrorInvalidValue;
  dim3 grid((N + TB - 1) / TB, (M + TB - 1) / TB);
  k_gemm_tiled<<<grid, 256, 0, st>>>(A, lda, M, W, N, K, C, ldc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// lm_head + argmax. Each wave walks LM_TILES consecutive 16-column vocabulary tiles over
// the full K, keeping per row the best (value, lowest index); the workgroup's four waves
// then merge into one partial per (row, workgroup).

constexpr int LM_TILES = 2;
constexpr int LM_COLS = 4 * 16 * LM_TILES;  // vocabulary columns per workgroup

int lmhead_groups(int V) { return (V + LM_COLS - 1) / LM_COLS; }

__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

template <int MT>
__global__ __launch_bounds__(256) void k_lmhead_argmax(const bf16* __restrict__ Y, int ldy, int M,
                                                       int r0, const bf16* __restrict__ W, int V,
                                                       int K, float* __restrict__ best_v,
                                                       int* __restrict__ best_i, int n_groups,
                                                       int gamma, float* __restrict__ logits) {
  __shared__ float sv[4][64];
  __shared__ int si[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const bf16* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + c;
    ap[mt] = Y + (size_t)(m < M ? m : 0) * ldy + g * 8;
  }
  float bv[MT][4];
  int bi[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) { bv[mt][e] = -INFINITY; bi[mt][e] = 0x7fffffff; }

  for (int t = 0; t < LM_TILES; ++t) {
    const int n0 = (blockIdx.x * 4 * LM_TILES + wave * LM_TILES + t) * 16;
    if (n0 >= V) break;
    const int n = n0 + c;
    const bool nv = n < V;
    const bf16* wp = W + (size_t)(nv ? n : n0) * K + g * 8;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; k += 128) {
      bf16x8 b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) b[u] = ld8(wp + k + u * 32);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = ld8(ap[mt] + k + u * 32);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[mt] = mfma16(a[u], b[u], acc[mt]);
      }
    }
    if (nv) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[mt][e];
          better(bv[mt][e], bi[mt][e], v, n);
          const int m = mt * 16 + 4 * g + e;
          if (logits != nullptr && m < M) {
            const int r = r0 + m, b = r / gamma, i = r % gamma;
            if (i != 0) logits[(size_t)(b * (gamma - 1) + i - 1) * V + n] = v;
          }
        }
      }
    }
  }
  // merge across the 16 lanes that share a row group g (they hold different columns)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = bv[mt][e];
      int i = bi[mt][e];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(v, o, 64);
        const int oi = __shfl_xor(i, o, 64);
        better(v, i, ov, oi);
      }
      bv[mt][e] = v;
      bi[mt][e] = i;
    }
  }
  // then across the four waves, one row tile at a time
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (c == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[wave][4 * g + e] = bv[mt][e];
        si[wave][4 * g + e] = bi[mt][e];
      }
    }
    __syncthreads();
    if (wave == 0 && lane < 16) {
      float v = sv[0][lane];
      int i = si[0][lane];
      for (int w = 1; w < 4; ++w) better(v, i, sv[w][lane], si[w][lane]);
      const int m = mt * 16 + lane;
      if (m < M) {
        best_v[(size_t)(r0 + m) * n_groups + blockIdx.x] = v;
        best_i[(size_t)(r0 + m) * n_groups + blockIdx.x] = i;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_lmhead_argmax(const bf16* Y, int ldy, int M, int r0, const bf16* W, int V,
                                int K, float* best_v, int* best_i, int n_groups, int gamma,
                                float* logits, hipStream_t st) {
  dim3 grid(n_groups);
  switch ((M + 15) / 16) {
    case 1: k_lmhead_argmax<1><<<grid, 256, 0, st>>>(Y, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    case 2: k_lmhead_argmax<2><<<grid, 256, 0, st>>>(Y, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    case 3: k_lmhead_argmax<3><<<grid, 256, 0, st>>>(Y, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    case 4: k_lmhead_argmax<4><<<grid, 256, 0, st>>>(Y, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// one workgroup per drafted row (band b, row i in 1..gamma-1)
__global__ __launch_bounds__(256) void k_argmax_reduce(const float* __restrict__ best_v,
                                                       const int* __restrict__ best_i,
                                                       int n_groups, int gamma,
                                                       int* __restrict__ tokens) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int d = blockIdx.x;                 // drafted row index b*(gamma-1) + i-1
  const int b = d / (gamma - 1), i = d % (gamma - 1) + 1;
  const size_t r = (size_t)b * gamma + i;
  float v = -INFINITY;
  int ix = 0x7fffffff;
  for (int j = threadIdx.x; j < n_groups; j += 256) better(v, ix, best_v[r * n_groups + j], best_i[r * n_groups + j]);
  sv[threadIdx.x] = v;
  si[threadIdx.x] = ix;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      float ov = sv[threadIdx.x + o];
      int oi = si[threadIdx.x + o];
      float mv = sv[threadIdx.x];
      int mi = si[threadIdx.x];
      better(mv, mi, ov, oi);
      sv[threadIdx.x] = mv;
      si[threadIdx.x] = mi;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) tokens[d] = si[0];
}

hipError_t launch_argmax_reduce(const float* best_v, const int* best_i, int n_groups,
                                int n_bands, int gamma, int* tokens, hipStream_t st) {
  k_argmax_reduce<<<n_bands * (gamma - 1), 256, 0, st>>>(best_v, best_i, n_groups, gamma, tokens);
  return hipGetLastError();
}

}  // namespace dfl
