// Device-side helpers shared by the gfx950 kernels: bf16 storage, 16-byte vector loads,
// the 16x16x32 bf16 MFMA and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef uint16_t bf16;  // storage type: raw IEEE bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ bf16 f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

// v = bf2f(hi) + bf2f(lo) to about 16 significant bits: a float carried through bf16
// MFMA operands as two terms
__device__ __forceinline__ void split_bf16(float v, bf16& hi, bf16& lo) {
  hi = f2bf(v);
  lo = f2bf(v - bf2f(hi));
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Eight OCP FP8 E4M3 codes (two 32-bit words, lowest byte first) as eight bf16 values: every
// E4M3 value (subnormals included) is exact in bf16; gfx950 converts two a cycle.
__device__ __forceinline__ bf16x8 fp8x8_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// eight bf16 bit patterns as one 16-byte word (element 0 lowest)
__device__ __forceinline__ u32x4 pack_bits8(const bf16 (&b)[8]) {
  return u32x4{(uint32_t)b[0] | ((uint32_t)b[1] << 16), (uint32_t)b[2] | ((uint32_t)b[3] << 16),
               (uint32_t)b[4] | ((uint32_t)b[5] << 16), (uint32_t)b[6] | ((uint32_t)b[7] << 16)};
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  u32x4 u;
  u[0] = pack2(v[0], v[1]);
  u[1] = pack2(v[2], v[3]);
  u[2] = pack2(v[4], v[5]);
  u[3] = pack2(v[6], v[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// D(16x16) += A(16x32) * B(32x16). Lane l holds A row (l%16) and B column (l%16), each
// 8 consecutive k-values of group (l/16); it receives D rows 4*(l/16)+i, column l%16.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// running argmax: a larger value, or an equal one at a lower index, wins (NaN never does)
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// block-wide sum for blockDim.x == 256 (4 waves); `red` is 4 floats of shared memory
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// The canonical sum of S split-K partials p[s * ps], s = 0..S-1: consecutive groups of gsz
// splits are each added in split order starting from zero, then the group sums in group
// order starting from zero. Every consumer of the forward's GEMM partials adds them this
// way, so a GEMM that forms the group sums itself (handing over one partial per group, then
// gsz = 1) gives the same bits. Loads go out up to B at a time before their adds, so none
// waits for another.
template <typename T>
__device__ __forceinline__ T ld_part(const float* p) { return *reinterpret_cast<const T*>(p); }

template <int B, typename T>
__device__ __forceinline__ T sum_splits(const float* __restrict__ p, int S, long long ps, int gsz) {
  // one split (a plain result): one load, and the same 0 + v the general path forms
  if (S == 1) return T{} + ld_part<T>(p);
  T t = T{}, grp = T{};
  int in_grp = 0;
  for (int s0 = 0; s0 < S; s0 += B) {
    // every load of the pass issued before the first add; none past the last split (S is
    // uniform, so the skips are scalar branches; re-reading the last split instead cost the
    // consumers up to four times their loads)
    T v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) v[u] = s0 + u < S ? ld_part<T>(p + (long long)(s0 + u) * ps) : T{};
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (s0 + u < S) {
        grp += v[u];
        if (++in_grp == gsz || s0 + u + 1 == S) {
          t += grp;
          grp = T{};
          in_grp = 0;
        }
      }
    }
  }
  return t;
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// NeoX rotation of the pair (x1, x2) = (x[j], x[j + d/2]) by pos * inv_freq[j]. The angle
// and its sine/cosine are taken in double precision: positions reach tens of thousands,
// where a float angle would be off by ~1e-3 rad.
__device__ __forceinline__ void rope_pair(float& x1, float& x2, int pos, double inv_freq) {
  double s, c;
  sincos((double)pos * inv_freq, &s, &c);
  const float cf = (float)c, sf = (float)s;
  const float y1 = x1 * cf - x2 * sf;
  const float y2 = x2 * cf + x1 * sf;
  x1 = y1;
  x2 = y2;
}

}  // namespace dfl
