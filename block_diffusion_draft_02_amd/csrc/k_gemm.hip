// BF16 MFMA GEMMs of the drafter: Y = A W^T with W row-major [N, K] (weights stored
// [out_features, in_features]).
//
// Activations enter as two bf16 terms (hi + lo, about 16 significant bits): every k-step
// issues one MFMA per term against the same exact bf16 weight operand. The weight stream,
// not the MFMA rate, bounds these GEMMs at the forward's row counts.
//
//  * k_gemm_skinny: the weight-streaming form for the block forward (M = bands * gamma
//    rows, at most 64 per launch). One wavefront owns 16 output columns over one K split
//    and streams those 16 weight rows exactly once; the activation rows come from L2.
//    Partial sums of every split go to P[s][M][N] and are added by the consumer in the
//    canonical order (sum_splits), so a row's result never depends on how many other rows
//    share the launch.
//  * k_gemm_wide: the batched forward's form (more than 64 rows): 128 x 128 output tiles
//    with the same per-element MFMA chains, adding each group of splits itself; and the
//    batched lm_head with the argmax epilogue.
//  * k_gemm_tiled: an LDS-tiled 128x128x64 form for the context append (thousands of rows).
//  * k_lmhead_argmax: the skinny form over the vocabulary with a running (max, index) per
//    row in the epilogue instead of a logits store; k_argmax_reduce finishes the argmax.
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

// T16 weight layout (the forward's GEMMs and the lm_head): the rows of a [N, K] weight go
// in tiles of 16; a tile's K is a run of 256-deep blocks, and a block holds its 16 x 256
// values as 8 x 64 16-byte pieces in exactly the order the 64 lanes of a wavefront load them
// (piece (u, lane) = row lane%16, k = u*32 + (lane/16)*8 .. +7). A tile is then 16*K
// contiguous values, and every load instruction of a wavefront reads 1 KB in one run.
constexpr int T16_BLOCK = 16 * 256;

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

// FP8 weights: OCP E4M3 codes with one fp32 scale per row (weight = code value x scale), in
// the T16-FP8 layout: the rows go in tiles of 16, a tile's K in 256-deep blocks of 4 KB, and a
// block holds 4 x 64 16-byte pieces in the order the lanes load them: piece (q, lane) is row
// lane % 16, the 8 codes of k = 64q + 8g .. (the lane's operand of 32-deep step 2q, g = lane/16)
// followed by the 8 codes of k = 64q + 32 + 8g .. (step 2q + 1).
constexpr int T16Q_BLOCK = 16 * 256;   // bytes of one 256-deep block of a tile

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

// running argmax: a larger value, or an equal one at a lower index, wins (NaN never does)
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

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

// ---------------------------------------------------------------------------------------

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
