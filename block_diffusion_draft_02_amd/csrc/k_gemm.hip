// BF16 MFMA GEMMs of the drafter for few rows: Y = A W^T with W row-major [N, K] (weights
// stored [out_features, in_features]). The wide form for many rows is in k_gemm_wide.hip,
// the LDS-tiled form for the context append in k_gemm_tiled.hip.
//
// Activations enter as two bf16 terms (hi + lo, about 16 significant bits): every k-step
// issues one MFMA per term against the same exact bf16 weight operand. The weight stream,
// not the MFMA rate, bounds these GEMMs at the forward's row counts.
//
//  * k_gemm_split / k_gemm_skinny: the weight-streaming form for the block forward
//    (M = bands * gamma rows, at most 64 per launch). One wavefront owns 16 output columns
//    over one K split and streams those 16 weight rows exactly once; the activation rows
//    come from L2. Partial sums of every split go to P[s][M][N] and are added by the
//    consumer in the canonical order (sum_splits), so a row's result never depends on how
//    many other rows share the launch.
//  * k_lmhead_argmax / k_lmhead_persist: the skinny form over the vocabulary with a running
//    (max, index) per row in the epilogue instead of a logits store; k_argmax_reduce
//    finishes the argmax.
//  * k_tile_weight, k_row_scale_fp8, k_quant_fp8_t16: the create-time weight copies (T16
//    tiled bf16, and FP8 E4M3 codes with per-row scales).
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dfl {

// Depth of one activation chunk staged in LDS and of one weight chunk a wavefront has in
// flight: 512 k = sixteen 16-byte loads per lane.
constexpr int KS = 512;
constexpr int APAD = 8;  // LDS row padding (bf16): rows 1040 B apart keep 8-lane groups conflict-free

// The workgroup's shared activation chunk: the hi (and with SPLIT the lo) term of MT*16
// rows x KS columns.
template <int MT, bool SPLIT>
struct AChunk {
  bf16 v[SPLIT ? 2 : 1][MT * 16][KS + APAD];
};

// Stage activation columns [k0, k0 + kn) of rows 0..MT*16-1 (rows >= M repeat row 0; their
// results are never stored) into LDS. kn is 256 or 512.
template <int MT, bool SPLIT>
__device__ __forceinline__ void stage_a(AChunk<MT, SPLIT>& sa, const bf16* __restrict__ A,
                                        const bf16* __restrict__ A_lo, int lda, int M, int k0,
                                        int kn) {
  const int per_row = kn / 8;  // 16-byte pieces per row
  for (int ch = threadIdx.x; ch < MT * 16 * per_row; ch += 256) {
    const int r = ch / per_row, cc = (ch % per_row) * 8;
    const size_t src = (size_t)(r < M ? r : 0) * lda + k0 + cc;
    *reinterpret_cast<u32x4*>(&sa.v[0][r][cc]) = *reinterpret_cast<const u32x4*>(A + src);
    if (SPLIT) *reinterpret_cast<u32x4*>(&sa.v[SPLIT ? 1 : 0][r][cc]) = *reinterpret_cast<const u32x4*>(A_lo + src);
  }
}

__global__ __launch_bounds__(256) void k_tile_weight(const bf16* __restrict__ src, int N, int K,
                                                     int n_pad, bf16* __restrict__ dst) {
  const size_t p = (size_t)blockIdx.x * 256 + threadIdx.x;   // destination piece
  if (p >= (size_t)n_pad * K / 8) return;
  const int lane = (int)(p & 63);
  const size_t q = p >> 6;
  const int u = (int)(q & 7);
  const size_t blk = q >> 3;
  const int S = K / 256;
  const int s = (int)(blk % S);
  const size_t n = (blk / S) * 16 + (lane & 15);
  const int k = s * 256 + u * 32 + (lane >> 4) * 8;
  u32x4 v = u32x4{0u, 0u, 0u, 0u};   // rows past N (padding to a whole tile) are zero
  if (n < (size_t)N) v = *reinterpret_cast<const u32x4*>(src + n * K + k);
  *reinterpret_cast<u32x4*>(dst + p * 8) = v;
}

hipError_t launch_tile_weight(const bf16* src, int N, int K, bf16* dst, hipStream_t st) {
  if (N < 1 || K < 256 || K % 256) return hipErrorInvalidValue;
  const int n_pad = (N + 15) / 16 * 16;
  const size_t pieces = (size_t)n_pad * K / 8;
  k_tile_weight<<<(unsigned)((pieces + 255) / 256), 256, 0, st>>>(src, N, K, n_pad, dst);
  return hipGetLastError();
}

// row scale = max |w| / 448 (the largest finite E4M3 value); an all-zero row has scale 1
__global__ __launch_bounds__(256) void k_row_scale_fp8(const bf16* __restrict__ src, int N, int K, int n_pad,
                                                       float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= n_pad) return;
  float amax = 0.f;
  if (n < N)
    for (int k = lane * 8; k < K; k += 64 * 8) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)n * K + k);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf(__uint_as_float(v[j] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(v[j] & 0xffff0000u)));
      }
    }
  amax = wave_max(amax);
  if (lane == 0) scale[n] = amax > 0.f ? amax / 448.f : 1.f;
}

// x (finite) to the nearest E4M3 code, ties to even, saturating at +-448
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = __float_as_uint(x) >> 31;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 448.f) {
    code = 0x7e;
  } else if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.f);   // 8 is the smallest normal, 2^-6
  } else {
    const uint32_t b = __float_as_uint(a);
    code = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
    code = code > 0x7eu ? 0x7eu : code;
  }
  return code | (sign << 7);
}

// one thread per 16-byte destination piece; rows past N (padding to whole tiles) are zero
__global__ __launch_bounds__(256) void k_quant_fp8_t16(const bf16* __restrict__ src, int N, int K, int n_pad,
                                                       const float* __restrict__ scale,
                                                       uint8_t* __restrict__ dst) {
  const size_t p = (size_t)blockIdx.x * 256 + threadIdx.x;   // destination piece
  if (p >= (size_t)n_pad * K / 16) return;
  const int lane = (int)(p & 63);
  const size_t q = p >> 6;
  const int qq = (int)(q & 3);
  const size_t blk = q >> 2;
  const int S = K / 256;
  const size_t n = (blk / S) * 16 + (lane & 15);
  const int k0 = (int)(blk % S) * 256 + qq * 64 + (lane >> 4) * 8;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (n < (size_t)N) {
    const float sc = scale[n];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + n * K + k0 + half * 32);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t bits = (j & 1) ? (v[j >> 1] & 0xffff0000u) : (v[j >> 1] << 16);
        w[half * 2 + (j >> 2)] |= e4m3_code(__uint_as_float(bits) / sc) << (8 * (j & 3));
      }
    }
  }
  *reinterpret_cast<u32x4*>(dst + p * 16) = u32x4{w[0], w[1], w[2], w[3]};
}

hipError_t launch_quant_fp8(const bf16* src, int N, int K, uint8_t* dst, float* scale, hipStream_t st) {
  if (N < 1 || K < 256 || K % 256) return hipErrorInvalidValue;
  const int n_pad = (N + 15) / 16 * 16;
  k_row_scale_fp8<<<(unsigned)((n_pad + 3) / 4), 256, 0, st>>>(src, N, K, n_pad, scale);
  const size_t pieces = (size_t)n_pad * K / 16;
  k_quant_fp8_t16<<<(unsigned)((pieces + 255) / 256), 256, 0, st>>>(src, N, K, n_pad, scale, dst);
  return hipGetLastError();
}

// One KS-deep (or 256-deep, full = false) weight chunk at depth k for the lane: row-major
// (wp = row + (lane/16)*8) or T16 (wp = tile + lane*8).
template <bool TILED>
__device__ __forceinline__ void load_w(bf16x8 (&w)[16], const bf16* __restrict__ wp, int k, bool full) {
  const bf16* b = TILED ? wp + (size_t)(k >> 8) * T16_BLOCK : wp + k;
  constexpr int step = TILED ? 512 : 32;
#pragma unroll
  for (int u = 0; u < 8; ++u) w[u] = ld8(b + u * step);
  if (full) {
#pragma unroll
    for (int u = 8; u < 16; ++u) w[u] = ld8(b + u * step);
  }
}

template <int MT, bool SPLIT>
__device__ __forceinline__ void mfma_chunk(const AChunk<MT, SPLIT>& sa, const bf16x8 (&w)[16], bool full,
                                           int c, int g, f32x4 (&acc)[MT]) {
  const int nu = full ? 16 : 8;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    if (u < nu) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sa.v[0][mt * 16 + c][u * 32 + g * 8]));
        acc[mt] = mfma16(a, w[u], acc[mt]);
        if (SPLIT) {
          const bf16x8 al = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sa.v[SPLIT ? 1 : 0][mt * 16 + c][u * 32 + g * 8]));
          acc[mt] = mfma16(al, w[u], acc[mt]);
        }
      }
    }
  }
}

// The workgroup's weight stream over k in [kb, ke) (ke - kb a multiple of 256): each
// wavefront owns 16 weight rows (lane l reads row wp's n0 + l%16); the rows arrive in KS-deep
// chunks, double-buffered in registers so the next chunk is in flight while the current one
// meets its activation chunk in LDS. The activation chunk is staged before the next weight
// chunk is requested: loads complete in issue order, so waiting for the activations then
// never waits for the prefetch. Every k-step is one MFMA per activation term, in ascending
// k, starting from zero.
template <int MT, bool SPLIT, bool TILED>
__device__ __forceinline__ void stream_tile(AChunk<MT, SPLIT>& sa, const bf16* __restrict__ wp,
                                            const bf16* __restrict__ A, const bf16* __restrict__ A_lo,
                                            int lda, int M, int kb, int ke, f32x4 (&acc)[MT]) {
  const int c = (threadIdx.x & 63) & 15, g = (threadIdx.x & 63) >> 4;
  bf16x8 w0[16], w1[16];
  bool f0 = ke - kb >= KS;
  load_w<TILED>(w0, wp, kb, f0);
  for (int k = kb; k < ke;) {
    // chunk at k sits in w0 (full = f0); prefetch the next one into w1
    const int k1 = k + (f0 ? KS : 256);
    const bool has1 = k1 < ke;
    const bool f1 = ke - k1 >= KS;
    stage_a<MT, SPLIT>(sa, A, A_lo, lda, M, k, f0 ? KS : 256);
    if (has1) load_w<TILED>(w1, wp, k1, f1);
    __syncthreads();
    mfma_chunk<MT, SPLIT>(sa, w0, f0, c, g, acc);
    __syncthreads();
    if (!has1) break;
    const int k2 = k1 + (f1 ? KS : 256);
    const bool has2 = k2 < ke;
    const bool f2 = ke - k2 >= KS;
    stage_a<MT, SPLIT>(sa, A, A_lo, lda, M, k1, f1 ? KS : 256);
    if (has2) load_w<TILED>(w0, wp, k2, f2);
    __syncthreads();
    mfma_chunk<MT, SPLIT>(sa, w1, f1, c, g, acc);
    __syncthreads();
    k = k2;
    f0 = f2;
  }
}

// One 256-deep split per workgroup (the forward's GEMMs): four wavefronts x 16 weight rows.
// The activation pieces are requested first (they come from L2), then the eight weight
// loads per lane; the activations go to LDS while the weights are still in flight. Small
// LDS and register footprints keep every workgroup of a launch resident at once.
constexpr int KT = 256;

// NORM: the activation (A, A_lo) is x * w of an RMSNorm (NormIn); the result rows are
// multiplied by the rows' scales 1/sqrt(mean(x^2) + eps). FP8: W is in the T16-FP8 layout,
// its codes become exact bf16 operands in registers, and each result column is multiplied
// by its row scale wsc[n] (before the RMSNorm scale, each a rounding of its own).
template <int MT, bool SPLIT, bool TILED, bool NORM, bool FP8>
__global__ __launch_bounds__(256) void k_gemm_split(const bf16* __restrict__ A,
                                                    const bf16* __restrict__ A_lo, int lda, int M,
                                                    const bf16* __restrict__ W, int N, int K,
                                                    float* __restrict__ P, long long part_stride,
                                                    NormIn nrm, const float* __restrict__ wsc) {
  __shared__ __attribute__((aligned(16))) bf16 sa[SPLIT ? 2 : 1][MT * 16][KT + APAD];
  __shared__ float srs[NORM ? MT * 16 : 1];
  constexpr int PT = MT * 16 * KT / 8 / 256;   // 16-byte activation pieces per thread and term
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  const int kb = blockIdx.y * KT;
  const int c = lane & 15, g = lane >> 4;
  const int n = n0 + c;
  const bool nv = n < N;
  // RMSNorm scales (requested first: the shuffles that combine them need nothing else):
  // wave w < MT takes rows 16w..16w+15, four lanes a row; lane q of a row adds slices q,
  // q + 4, ... (the rows are SSQ_STRIDE long with a zero tail, so every load is unconditional),
  // then the four lanes combine in a fixed order
  constexpr int SQ_PER_LANE = SSQ_STRIDE / 4;
  float sqv[NORM ? SQ_PER_LANE : 1];
  if (NORM) {
    const int row = wave * 16 + (lane >> 2);
    const float* q = nrm.ssq + (size_t)(wave < MT && row < M ? row : 0) * SSQ_STRIDE + (lane & 3);
#pragma unroll
    for (int t = 0; t < SQ_PER_LANE; ++t) sqv[NORM ? t : 0] = q[4 * t];
  }
  u32x4 ah[PT], al[SPLIT ? PT : 1];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int ch = u * 256 + threadIdx.x;
    const int r = ch / (KT / 8), cc = (ch % (KT / 8)) * 8;
    const size_t src = (size_t)(r < M ? r : 0) * lda + kb + cc;   // rows >= M repeat row 0
    ah[u] = *reinterpret_cast<const u32x4*>(A + src);
    if (SPLIT) al[SPLIT ? u : 0] = *reinterpret_cast<const u32x4*>(A_lo + src);
  }
  // out-of-range columns read a valid row (every wave stays for the barrier); their results
  // are never stored
  bf16x8 w[KT / 32];
  u32x4 wq[FP8 ? KT / 64 : 1];
  float sc = 1.f;
  if (FP8) {
    const uint8_t* q8 = reinterpret_cast<const uint8_t*>(W) +
                        ((size_t)min(n0, N - 16) / 16 * (K / KT) + blockIdx.y) * T16Q_BLOCK + lane * 16;
#pragma unroll
    for (int u = 0; u < KT / 64; ++u) wq[FP8 ? u : 0] = *reinterpret_cast<const u32x4*>(q8 + u * 1024);
    sc = wsc[nv ? n : min(n0, N - 1)];
  } else {
    const bf16* wp = TILED ? W + ((size_t)min(n0, N - 16) / 16 * (K / KT) + blockIdx.y) * T16_BLOCK + lane * 8
                           : W + (size_t)(nv ? n : min(n0, N - 1)) * K + kb + g * 8;
#pragma unroll
    for (int u = 0; u < KT / 32; ++u) w[u] = ld8(wp + u * (TILED ? 512 : 32));
  }
  if (NORM) {
    // after the weight loads are issued: waiting on the sums does not wait on the weights
    float ssum = 0.f;
#pragma unroll
    for (int t = 0; t < SQ_PER_LANE; ++t) ssum += sqv[NORM ? t : 0];
    ssum += __shfl_xor(ssum, 1, 64);
    ssum += __shfl_xor(ssum, 2, 64);
    if (wave < MT && (lane & 3) == 0) srs[wave * 16 + (lane >> 2)] = rsqrtf(ssum / (float)nrm.h + nrm.eps);
  }
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int ch = u * 256 + threadIdx.x;
    const int r = ch / (KT / 8), cc = (ch % (KT / 8)) * 8;
    *reinterpret_cast<u32x4*>(&sa[0][r][cc]) = ah[u];
    if (SPLIT) *reinterpret_cast<u32x4*>(&sa[SPLIT ? 1 : 0][r][cc]) = al[SPLIT ? u : 0];
  }
  __syncthreads();
  if (FP8) {
#pragma unroll
    for (int u = 0; u < KT / 64; ++u) {
      w[2 * u] = fp8x8_bf16(wq[FP8 ? u : 0][0], wq[FP8 ? u : 0][1]);
      w[2 * u + 1] = fp8x8_bf16(wq[FP8 ? u : 0][2], wq[FP8 ? u : 0][3]);
    }
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < KT / 32; ++u) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sa[0][mt * 16 + c][u * 32 + g * 8]));
      acc[mt] = mfma16(a, w[u], acc[mt]);
      if (SPLIT) {
        const bf16x8 a2 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sa[SPLIT ? 1 : 0][mt * 16 + c][u * 32 + g * 8]));
        acc[mt] = mfma16(a2, w[u], acc[mt]);
      }
    }
  }
  if (!nv) return;
  float* pp = P + (long long)blockIdx.y * part_stride;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * g + i;
      float v = acc[mt][i];
      if (FP8) v = v * sc;
      if (NORM) v = v * srs[NORM ? m : 0];
      if (m < M) pp[(size_t)m * N + n] = v;
    }
  }
}

template <int MT, bool SPLIT>
__global__ __launch_bounds__(256) void k_gemm_skinny(const bf16* __restrict__ A,
                                                     const bf16* __restrict__ A_lo, int lda, int M,
                                                     const bf16* __restrict__ W, int N, int K,
                                                     int k_len, float* __restrict__ P,
                                                     long long part_stride) {
  __shared__ __attribute__((aligned(16))) AChunk<MT, SPLIT> sa;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wave) * 16;
  const int s = blockIdx.y;
  const int kb = s * k_len;
  const int ke = min(K, kb + k_len);
  const int c = lane & 15, g = lane >> 4;
  const int n = n0 + c;
  const bool nv = n < N;
  // out-of-range columns read a valid row (every wave stays for the workgroup's barriers);
  // their results are never stored
  const bf16* wp = W + (size_t)(nv ? n : min(n0, N - 1)) * K + g * 8;
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  stream_tile<MT, SPLIT, false>(sa, wp, A, A_lo, lda, M, kb, ke, acc);
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

hipError_t launch_gemm_skinny(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W,
                              int N, int K, int k_len, float* P, long long part_stride, bool w_tiled,
                              hipStream_t st, const NormIn* norm, const float* wsc) {
  const int S = (K + k_len - 1) / k_len;
  dim3 grid((N + 63) / 64, S);
  const int mt = (M + 15) / 16;
  if (mt < 1 || mt > 4) return hipErrorInvalidValue;
  if (w_tiled && (k_len != KT || K % KT || N % 16)) return hipErrorInvalidValue;
  const NormIn nn = norm ? *norm : NormIn{};
  if (norm && (!w_tiled || !A_lo || nn.h != K || K % SSQ_COLS || K > SSQ_STRIDE * SSQ_COLS)) return hipErrorInvalidValue;
  if (wsc && (!w_tiled || !A_lo)) return hipErrorInvalidValue;
  if (k_len == KT && K % KT == 0) {
#define DFL_SPLIT(MTV, SP, TL, NM, F8) (void)launch(k_gemm_split<MTV, SP, TL, NM, F8>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, P, part_stride, nn, wsc)
#define DFL_SPLIT_MT(SP, TL, NM, F8) switch (mt) { case 1: DFL_SPLIT(1, SP, TL, NM, F8); break; case 2: DFL_SPLIT(2, SP, TL, NM, F8); break; \
                                                   case 3: DFL_SPLIT(3, SP, TL, NM, F8); break; default: DFL_SPLIT(4, SP, TL, NM, F8); break; }
    if (wsc) {
      if (norm) { DFL_SPLIT_MT(true, true, true, true) } else { DFL_SPLIT_MT(true, true, false, true) }
    } else if (norm) {
      DFL_SPLIT_MT(true, true, true, false)
    } else if (A_lo) {
      if (w_tiled) { DFL_SPLIT_MT(true, true, false, false) } else { DFL_SPLIT_MT(true, false, false, false) }
    } else {
      if (w_tiled) { DFL_SPLIT_MT(false, true, false, false) } else { DFL_SPLIT_MT(false, false, false, false) }
    }
#undef DFL_SPLIT_MT
#undef DFL_SPLIT
    return hipGetLastError();
  }
  if (norm || w_tiled || wsc) return hipErrorInvalidValue;
#define DFL_SKINNY(MTV, SP) (void)launch(k_gemm_skinny<MTV, SP>, grid, 256, 0, st, A, A_lo, lda, M, W, N, K, k_len, P, part_stride)
  if (A_lo) {
    switch (mt) { case 1: DFL_SKINNY(1, true); break; case 2: DFL_SKINNY(2, true); break;
                  case 3: DFL_SKINNY(3, true); break; default: DFL_SKINNY(4, true); break; }
  } else {
    switch (mt) { case 1: DFL_SKINNY(1, false); break; case 2: DFL_SKINNY(2, false); break;
                  case 3: DFL_SKINNY(3, false); break; default: DFL_SKINNY(4, false); break; }
  }
#undef DFL_SKINNY
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// lm_head + argmax. Each wave streams one 16-column vocabulary tile over the full K and
// keeps per row the best (value, lowest index); the workgroup's four waves then merge into
// one partial per (row, workgroup).

constexpr int LM_COLS = 4 * 16;  // vocabulary columns per workgroup (one 16-column tile per wave)

int lmhead_groups(int V) { return (V + LM_COLS - 1) / LM_COLS; }

template <int MT>
__global__ __launch_bounds__(256) void k_lmhead_argmax(const bf16* __restrict__ Y,
                                                       const bf16* __restrict__ Y_lo, int ldy, int M,
                                                       int r0, const bf16* __restrict__ W, int V,
                                                       int K, float* __restrict__ best_v,
                                                       int* __restrict__ best_i, int n_groups,
                                                       int gamma, float* __restrict__ logits) {
  __shared__ __attribute__((aligned(16))) AChunk<MT, true> sa;
  __shared__ float sv[4][64];
  __shared__ int si[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  float bv[MT][4];
  int bi[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) { bv[mt][e] = -INFINITY; bi[mt][e] = 0x7fffffff; }

  const int n0 = (blockIdx.x * 4 + wave) * 16;
  {
    const int n = n0 + c;
    const bool nv = n < V;
    // W is in the T16 layout with V padded to whole tiles; every wave takes part in the
    // workgroup's barriers, waves past the last tile re-read the last tile
    const int n_tiles = (V + 15) / 16;
    const bf16* wp = W + (size_t)min(n0 / 16, n_tiles - 1) * 16 * K + lane * 8;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    stream_tile<MT, true, true>(sa, wp, Y, Y_lo, ldy, M, 0, K, acc);
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

hipError_t launch_lmhead_argmax(const bf16* Y, const bf16* Y_lo, int ldy, int M, int r0, const bf16* W, int V,
                                int K, float* best_v, int* best_i, int n_groups, int gamma,
                                float* logits, hipStream_t st) {
  dim3 grid(n_groups);
  switch ((M + 15) / 16) {
    case 1: (void)launch(k_lmhead_argmax<1>, grid, 256, 0, st, Y, Y_lo, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    case 2: (void)launch(k_lmhead_argmax<2>, grid, 256, 0, st, Y, Y_lo, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    case 3: (void)launch(k_lmhead_argmax<3>, grid, 256, 0, st, Y, Y_lo, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    case 4: (void)launch(k_lmhead_argmax<4>, grid, 256, 0, st, Y, Y_lo, ldy, M, r0, W, V, K, best_v, best_i, n_groups, gamma, logits); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// lm_head + argmax for one group of at most 16 rows whose normed rows fit in LDS whole
// (K <= LMP_KMAX): persistent workgroups of eight wavefronts, one per CU. The rows (hi, lo)
// are staged once; every wavefront then streams its T16 vocabulary tiles (tiles w, w + W,
// ... over all waves W of the grid) as one continuous sequence of 512-deep chunks,
// double-buffered in registers, with no barrier or restaging in the loop, and keeps a
// running (max, lowest index) per row. The waves merge in LDS and write one partial per
// (row, workgroup).
constexpr int LMP_WAVES = 8;
constexpr int LMP_KMAX = 2048;

int lmhead_persistent_groups(int V, int K, int M, int n_cu) {
  // (K a multiple of the 512-deep chunk: the bf16 and the FP8 weight streams both need it)
  if (M > 16 || K > LMP_KMAX || K % KS) return 0;
  const int tiles = (V + 15) / 16;
  return std::max(1, std::min(n_cu, (tiles + LMP_WAVES - 1) / LMP_WAVES));
}

// FP8: W in the T16-FP8 layout (a 512-deep chunk is 8 pieces per lane), codes converted to
// exact bf16 operands, each logit multiplied by its vocabulary row's scale (loaded with the
// chunk that starts the tile, so it is there when the tile ends).
template <bool FP8>
__global__ __launch_bounds__(LMP_WAVES * 64) void k_lmhead_persist(const bf16* __restrict__ Y,
                                                                 const bf16* __restrict__ Y_lo, int ldy,
                                                                 int M, int r0, const bf16* __restrict__ W,
                                                                 int V, int K, float* __restrict__ best_v,
                                                                 int* __restrict__ best_i, int gamma,
                                                                 float* __restrict__ logits,
                                                                 const float* __restrict__ wsc) {
  __shared__ __attribute__((aligned(16))) bf16 sy[2][16][LMP_KMAX + APAD];
  __shared__ float sv[LMP_WAVES][16];
  __shared__ int si[LMP_WAVES][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  // the rows, hi and lo (rows >= M are zero; their results are never used)
  for (int pc = threadIdx.x; pc < 16 * K / 8; pc += LMP_WAVES * 64) {
    const int r = pc / (K / 8), k8 = (pc % (K / 8)) * 8;
    u32x4 h = u32x4{0u, 0u, 0u, 0u}, l = h;
    if (r < M) {
      h = *reinterpret_cast<const u32x4*>(Y + (size_t)r * ldy + k8);
      l = *reinterpret_cast<const u32x4*>(Y_lo + (size_t)r * ldy + k8);
    }
    *reinterpret_cast<u32x4*>(&sy[0][r][k8]) = h;
    *reinterpret_cast<u32x4*>(&sy[1][r][k8]) = l;
  }
  __syncthreads();
  float bv[4];
  int bi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { bv[e] = -INFINITY; bi[e] = 0x7fffffff; }
  const int n_tiles = (V + 15) / 16;
  const int nch = K / KS;
  const int stride = gridDim.x * LMP_WAVES;
  const int t0 = blockIdx.x * LMP_WAVES + wave;
  const int my_tiles = t0 < n_tiles ? (n_tiles - 1 - t0) / stride + 1 : 0;
  const int items = my_tiles * nch;   // (tile, chunk) pairs this wave streams, in order
  auto tile_of = [&](int q) { return t0 + (q / nch) * stride; };
  // one chunk (item q) of the wave's stream: bf16, 16 pieces of 16 bytes; FP8, 8 pieces
  constexpr int NP = FP8 ? KS / 64 : KS / 32;
  auto load_chunk = [&](u32x4 (&w)[NP], float& sc, int q) {
    const int j = q % nch;
    if (FP8) {
      const uint8_t* b = reinterpret_cast<const uint8_t*>(W) + (size_t)tile_of(q) * 16 * K + (size_t)j * (KS / 256) * T16Q_BLOCK + lane * 16;
#pragma unroll
      for (int v = 0; v < NP; ++v) w[v] = *reinterpret_cast<const u32x4*>(b + (v >> 2) * T16Q_BLOCK + (v & 3) * 1024);
      if (j == 0) sc = wsc[tile_of(q) * 16 + c];
    } else {
      const bf16* b = W + (size_t)tile_of(q) * 16 * K + (size_t)j * (KS / 256) * T16_BLOCK + lane * 8;
#pragma unroll
      for (int v = 0; v < NP; ++v) w[v] = *reinterpret_cast<const u32x4*>(b + v * 512);
    }
  };
  u32x4 w0[NP], w1[NP];
  float sc0 = 1.f, sc1 = 1.f, sc = 1.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const u32x4 (&w)[NP], float scq, int q) {
    const int j = q % nch;
    if (FP8 && j == 0) sc = scq;
#pragma unroll
    for (int u = 0; u < KS / 32; ++u) {
      const bf16x8 wv = FP8 ? fp8x8_bf16(w[u >> 1][(u & 1) * 2], w[u >> 1][(u & 1) * 2 + 1])
                            : __builtin_bit_cast(bf16x8, w[FP8 ? 0 : u]);
      const int k = j * KS + u * 32 + g * 8;
      acc = mfma16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sy[0][c][k])), wv, acc);
      acc = mfma16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&sy[1][c][k])), wv, acc);
    }
    if (j == nch - 1) {
      // tile done: lane (c, g) holds rows 4g..4g+3 of column t*16 + c
      const int n = tile_of(q) * 16 + c;
      if (n < V) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = FP8 ? acc[e] * sc : acc[e];
          better(bv[e], bi[e], v, n);
          const int m = 4 * g + e;
          if (logits != nullptr && m < M) {
            const int r = r0 + m, b = r / gamma, i = r % gamma;
            if (i != 0) logits[(size_t)(b * (gamma - 1) + i - 1) * V + n] = v;
          }
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  if (items > 0) load_chunk(w0, sc0, 0);
  for (int q = 0; q < items; q += 2) {
    if (q + 1 < items) load_chunk(w1, sc1, q + 1);
    consume(w0, sc0, q);
    if (q + 1 >= items) break;
    if (q + 2 < items) load_chunk(w0, sc0, q + 2);
    consume(w1, sc1, q + 1);
  }
  // merge across the 16 lanes of a row group, then across the waves
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = bv[e];
    int i = bi[e];
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oi = __shfl_xor(i, o, 64);
      better(v, i, ov, oi);
    }
    if (c == 0) {
      sv[wave][4 * g + e] = v;
      si[wave][4 * g + e] = i;
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float v = sv[0][threadIdx.x];
    int i = si[0][threadIdx.x];
    for (int w = 1; w < LMP_WAVES; ++w) better(v, i, sv[w][threadIdx.x], si[w][threadIdx.x]);
    if ((int)threadIdx.x < M) {
      best_v[(size_t)(r0 + threadIdx.x) * gridDim.x + blockIdx.x] = v;
      best_i[(size_t)(r0 + threadIdx.x) * gridDim.x + blockIdx.x] = i;
    }
  }
}

hipError_t launch_lmhead_persistent(const bf16* Y, const bf16* Y_lo, int ldy, int M, int r0, const bf16* W,
                                    int V, int K, float* best_v, int* best_i, int n_groups, int gamma,
                                    float* logits, hipStream_t st, const float* wsc) {
  if (M < 1 || M > 16 || K > LMP_KMAX || K % KS || n_groups < 1) return hipErrorInvalidValue;
  if (wsc)
    (void)launch(k_lmhead_persist<true>, n_groups, LMP_WAVES * 64, 0, st, Y, Y_lo, ldy, M, r0, W, V, K, best_v,
                 best_i, gamma, logits, wsc);
  else
    (void)launch(k_lmhead_persist<false>, n_groups, LMP_WAVES * 64, 0, st, Y, Y_lo, ldy, M, r0, W, V, K, best_v,
                 best_i, gamma, logits, wsc);
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
  (void)launch(k_argmax_reduce, n_bands * (gamma - 1), 256, 0, st, best_v, best_i, n_groups, gamma, tokens);
  return hipGetLastError();
}

}  // namespace dfl
