// DSpark Markov head (docs.rs memra-engine, dflash.rs: the `markov` head of DflashDraft and the
// semi-autoregressive chain of generate_spec_dflash; spark_model/layers/dflash_head.rs: the
// head's markov_w1 / markov_w2 tables): after the lm_head has written the drafted rows'
// logits, row k of every band gets the bias W2 @ W1[t_k] (t_0 = the band's bonus token, t_k =
// the token drafted at row k-1) and its draft is the argmax of the biased row. One launch per
// row k; the rows are sequential because t_k is the previous launch's argmax.
//
// A launch streams the T16 copy of W2 once for all bands (the bands are the rows of one or two
// 16-row MFMA tiles, the W1 rows of their previous tokens staged in LDS), adds the fp32 sum to
// the row's logits and keeps a running argmax per band. Every workgroup folds its argmax per
// band into one 64-bit key with a device-scope atomic max (the value's order-preserving bits
// above the complemented index, so a tie goes to the lower index); the next launch reads the
// keys after the kernel boundary, and a last one-workgroup launch writes the drafts and
// clears the keys. Nothing waits on another workgroup and no cache-wide fence is needed.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dfl {

namespace {

constexpr int MK_T16_BLOCK = 16 * 256;   // one 256-deep block of a T16 tile (elements)
constexpr int MK_PAD = 8;                // LDS row padding: rows 16 B off the bank period
constexpr int MK_DEPTH = 2;              // W2 tiles in flight per wavefront (2 or 3)

// wavefronts a workgroup: 8, except for two band tiles of a rank-512 head, whose registers
// fit 256 per lane only with 4
constexpr int mk_waves(int mt, int rb) { return mt == 2 && rb == 2 ? 4 : 8; }

__device__ __forceinline__ void mk_better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

// argmax key: larger value first, then lower index; -0 counts as +0 (the comparisons of the
// running argmax do not tell them apart). Zero is below every key a finite value makes.
__device__ __forceinline__ unsigned long long mk_key(float v, int i) {
  uint32_t u = v == 0.f ? 0u : __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)i);
}
__device__ __forceinline__ int mk_key_index(unsigned long long key) {
  return (int)(0xffffffffu - (uint32_t)(key & 0xffffffffu));
}

// max over the 16 lanes that share lane / 16 (lower index on a tie)
__device__ __forceinline__ void mk_reduce16(float& bv, int& bi) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    mk_better(bv, bi, ov, oi);
  }
}

// MT: 16-band row tiles (bands <= 16 * MT); RB: 256-deep blocks of the rank
template <int MT, int RB>
__global__ __launch_bounds__(mk_waves(MT, RB) * 64) void k_markov_step(const MarkovStep a) {
  constexpr int MK_WAVES = mk_waves(MT, RB);
  constexpr int R = RB * 256;
  constexpr int NP = RB * 8;   // 16-byte W2 pieces a lane loads per tile
  __shared__ __attribute__((aligned(16))) bf16 se[MT * 16][R + MK_PAD];
  __shared__ float rv[MK_WAVES][MT * 16];
  __shared__ int ri[MK_WAVES][MT * 16];
  const bf16* __restrict__ w2t = a.w2t;
  float* __restrict__ logits = a.logits;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int g1 = a.gamma - 1, V = a.V, n = a.n;

  // W1 rows of the bands' previous tokens; rows past the last band are zero
  for (int p = threadIdx.x; p < MT * 16 * (R / 8); p += MK_WAVES * 64) {
    const int b = p / (R / 8), cc = (p % (R / 8)) * 8;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (b < n) {
      // (a previous row with no finite logit leaves no valid token: clamped, never out of range)
      const int prev = a.k == 0 ? a.bonus[b]
                                : mk_key_index(__hip_atomic_load(a.best + (a.k - 1) * MAX_BANDS + b, __ATOMIC_RELAXED,
                                                                 __HIP_MEMORY_SCOPE_AGENT));
      const int t = min(max(prev, 0), V - 1);
      v = *reinterpret_cast<const u32x4*>(a.w1 + (size_t)t * R + cc);
    }
    *reinterpret_cast<u32x4*>(&se[b][cc]) = v;
  }

  float bv[MT][4];
  int bi[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) { bv[mt][e] = -INFINITY; bi[mt][e] = 0x7fffffff; }

  // A wave streams tiles t0, t0 + stride, ... with the next tile's W2 pieces and logits in
  // flight while the current one is computed. Lane (c, g) holds bands 16 mt + 4 g + e of
  // vocabulary column t * 16 + c.
  const int n_tiles = (V + 15) / 16;
  const int stride = gridDim.x * MK_WAVES;
  auto load = [&](u32x4 (&w)[NP], float (&l)[MT][4], int t) {
    const bf16* wp = w2t + (size_t)t * 16 * R + lane * 8;
#pragma unroll
    for (int u = 0; u < NP; ++u) w[u] = *reinterpret_cast<const u32x4*>(wp + (u >> 3) * MK_T16_BLOCK + (u & 7) * 512);
    const int col = min(t * 16 + c, V - 1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = mt * 16 + 4 * g + e;
        l[mt][e] = b < n ? logits[(size_t)(b * g1 + a.k) * V + col] : 0.f;
      }
  };
  auto consume = [&](const u32x4 (&w)[NP], const float (&l)[MT][4], int t) {
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NP; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = mfma16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&se[mt * 16 + c][u * 32 + g * 8])),
                         __builtin_bit_cast(bf16x8, w[u]), acc[mt]);
    const int col = t * 16 + c;
    if (col < V) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b = mt * 16 + 4 * g + e;
          if (b < n) {
            const float v = l[mt][e] + acc[mt][e];
            if (a.store) logits[(size_t)(b * g1 + a.k) * V + col] = v;
            mk_better(bv[mt][e], bi[mt][e], v, col);
          }
        }
    }
  };
  // a ring of MK_DEPTH tiles in flight per wave
  u32x4 w0[NP], w1[NP], w2[NP];
  float l0[MT][4], l1[MT][4], l2[MT][4];
  int t = blockIdx.x * MK_WAVES + wave;
  if (t < n_tiles) load(w0, l0, t);
  if (MK_DEPTH == 3 && t + stride < n_tiles) load(w1, l1, t + stride);
  __syncthreads();   // the staged W1 rows (the first tiles' loads are already in flight)
  const int ahead = (MK_DEPTH - 1) * stride;
  while (t < n_tiles) {
    if (t + ahead < n_tiles) load(MK_DEPTH == 3 ? w2 : w1, MK_DEPTH == 3 ? l2 : l1, t + ahead);
    consume(w0, l0, t);
    if ((t += stride) >= n_tiles) break;
    if (t + ahead < n_tiles) load(w0, l0, t + ahead);
    consume(w1, l1, t);
    if ((t += stride) >= n_tiles) break;
    if (MK_DEPTH == 3) {
      if (t + ahead < n_tiles) load(w1, l1, t + ahead);
      consume(w2, l2, t);
      t += stride;
    }
  }

  // the workgroup's argmax per band, folded into the band's key
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mk_reduce16(bv[mt][e], bi[mt][e]);
      if (c == 0) { rv[wave][mt * 16 + 4 * g + e] = bv[mt][e]; ri[wave][mt * 16 + 4 * g + e] = bi[mt][e]; }
    }
  __syncthreads();
  if (threadIdx.x < n) {
    const int b = threadIdx.x;
    float v = rv[0][b];
    int i = ri[0][b];
#pragma unroll
    for (int w = 1; w < MK_WAVES; ++w) mk_better(v, i, rv[w][b], ri[w][b]);
    __hip_atomic_fetch_max(a.best + a.k * MAX_BANDS + b, mk_key(v, i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// the drafts of every row from the keys, which are then cleared for the next forward
__global__ __launch_bounds__(256) void k_markov_finish(unsigned long long* __restrict__ best, int n, int gamma,
                                                       int* __restrict__ tokens) {
  const int g1 = gamma - 1;
  for (int q = threadIdx.x; q < g1 * MAX_BANDS; q += 256) {
    const int k = q / MAX_BANDS, b = q % MAX_BANDS;
    if (b < n) tokens[b * g1 + k] = mk_key_index(__hip_atomic_load(best + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    __hip_atomic_store(best + q, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

int markov_step_groups(int V, int n_cu) {
  const int n_tiles = (V + 15) / 16;
  return std::max(1, std::min((n_tiles + 7) / 8, n_cu));
}

hipError_t launch_markov_step(const MarkovStep& a, int groups, hipStream_t st) {
  if (a.n < 1 || a.n > MAX_BANDS || a.k < 0 || a.k >= a.gamma - 1 || a.gamma - 1 > MARKOV_MAX_ROWS || groups < 1 ||
      groups > MARKOV_MAX_GROUPS || (a.R != 256 && a.R != 512))
    return hipErrorInvalidValue;
  const dim3 grid(groups);
  if (a.n <= 16)
    return a.R == 256 ? launch(k_markov_step<1, 1>, grid, dim3(mk_waves(1, 1) * 64), 0, st, a)
                      : launch(k_markov_step<1, 2>, grid, dim3(mk_waves(1, 2) * 64), 0, st, a);
  return a.R == 256 ? launch(k_markov_step<2, 1>, grid, dim3(mk_waves(2, 1) * 64), 0, st, a)
                    : launch(k_markov_step<2, 2>, grid, dim3(mk_waves(2, 2) * 64), 0, st, a);
}

hipError_t launch_markov_finish(unsigned long long* best, int n, int gamma, int* tokens, hipStream_t st) {
  if (n < 1 || n > MAX_BANDS || gamma < 2 || gamma - 1 > MARKOV_MAX_ROWS) return hipErrorInvalidValue;
  return launch(k_markov_finish, dim3(1), dim3(256), 0, st, best, n, gamma, tokens);
}

}  // namespace dfl
