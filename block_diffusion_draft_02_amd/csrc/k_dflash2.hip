// DFlash2 (spark_model/layers/dflash_head.rs: the DFlash2 fields of BlockDiffusionDraftHead --
// attention_conv / mlp_conv base kernels [2 applications, kernel, hidden] and kernel
// projections [2 * kernel * groups, hidden]; the scratch conv_dyn, conv_tmp, sel_vals, sel_idx,
// sel_hproj; the dflash2_conv2, dflash2_topk16 and dflash2_selector_walk kernels). The pages
// give shapes and kernel names; the composition is this library's reading:
//
// * a conv site (the attention input and the MLP input of every layer) turns the site's normed
//   input h_n into the per-row dynamic taps D_t = proj @ h_n,t, viewed [application][tap]
//   [group]; channel c's tap is base[a][j][c] + D_t[a][j][c / 16];
// * prepare: u_t = sum_j tap[0][j] * h_n,t-j (two taps looking back along the band's rows,
//   zero before its first row); the sublayer runs on u;
// * finish: the sublayer's output s is convolved the same way with application 1's taps
//   before the residual add;
// * candidates: each drafted row's 16 largest logits (ties to the lower index);
// * walk: H_t = hidden_projection @ y_t; candidate c scores logit(c) + sum_r pred[p][r] *
//   H_t[r] * succ[c][r] after previous pick p (the bonus token before the first row); the
//   best candidate (the earlier one on a tie) is the row's draft.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace dfl {

namespace {

constexpr int DC_GS = 16;   // channels per conv group
constexpr int TOPK = 16;

__device__ __forceinline__ float row_scale(const float* __restrict__ ssq, int row, int h, float eps) {
  float s = 0.f;
  for (int q = 0; q < h / SSQ_COLS; ++q) s += ssq[(size_t)row * SSQ_STRIDE + q];
  return rsqrtf(s / (float)h + eps);
}

__device__ __forceinline__ void load4(const bf16* __restrict__ p, float (&v)[4]) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  v[0] = bf2f((bf16)(w.x & 0xffff)); v[1] = bf2f((bf16)(w.x >> 16));
  v[2] = bf2f((bf16)(w.y & 0xffff)); v[3] = bf2f((bf16)(w.y >> 16));
}

__device__ __forceinline__ void store_hilo4(const float (&v)[4], bf16* __restrict__ hi_p, bf16* __restrict__ lo_p) {
  bf16 hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16(v[e], hi[e], lo[e]);
  *reinterpret_cast<u32x2*>(hi_p) = u32x2{(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
  *reinterpret_cast<u32x2*>(lo_p) = u32x2{(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
}

// One 64-thread workgroup per (row, 256-column slice = 16 groups). Xw = x * w (hi + lo) and the
// rows' slice sums of squares give h_n = Xw * rs; P holds the projection's split partials.
__global__ __launch_bounds__(64) void k_dconv_prepare(const bf16* __restrict__ Xw, const bf16* __restrict__ Xw_lo,
                                                      const float* __restrict__ ssq, float eps, int h, int gamma,
                                                      const float* __restrict__ P, int S, long long ps, int gsz,
                                                      const bf16* __restrict__ base, float* __restrict__ dyn,
                                                      bf16* __restrict__ U, bf16* __restrict__ U_lo) {
  __shared__ float sD[4 * 16];
  const int r = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
  const int G = h / DC_GS, Np = 4 * G;
  {
    // this slice's dynamic taps: thread (a*2 + tap, group) sums the projection's splits
    const int aj = tid >> 4, g = j * 16 + (tid & 15);
    const float v = sum_splits<8, float>(P + (size_t)r * Np + aj * G + g, S, ps, gsz);
    sD[tid] = v;
    dyn[(size_t)r * Np + aj * G + g] = v;
  }
  const bool has_prev = (r % gamma) != 0;
  const float rs0 = row_scale(ssq, r, h, eps);
  const float rs1 = has_prev ? row_scale(ssq, r - 1, h, eps) : 0.f;
  const int col = j * SSQ_COLS + tid * 4;
  float a0[4], l0[4], a1[4], l1[4], b0[4], b1[4];
  load4(Xw + (size_t)r * h + col, a0);
  load4(Xw_lo + (size_t)r * h + col, l0);
  load4(base + col, b0);            // application 0, tap 0
  load4(base + h + col, b1);        // application 0, tap 1
  if (has_prev) {
    load4(Xw + (size_t)(r - 1) * h + col, a1);
    load4(Xw_lo + (size_t)(r - 1) * h + col, l1);
  }
  __syncthreads();
  const float d0 = sD[0 * 16 + tid / 4], d1 = sD[1 * 16 + tid / 4];   // 4 columns of one group
  float u[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    u[e] = (b0[e] + d0) * ((a0[e] + l0[e]) * rs0);
    if (has_prev) u[e] += (b1[e] + d1) * ((a1[e] + l1[e]) * rs1);
  }
  store_hilo4(u, U + (size_t)r * h + col, U_lo + (size_t)r * h + col);
}

// The finish application and the residual add: X[t] += tap[1][0] * s_t + tap[1][1] * s_t-1, s =
// the canonical sum of the sublayer's split partials; then the slice's sum of squares and X * w
// (the next norm's activation, hi + lo), as the plain residual kernel does.
__global__ __launch_bounds__(64) void k_resid_dconv(float* __restrict__ X, const float* __restrict__ P, int S,
                                                    long long ps, int gsz, int h, int gamma,
                                                    const float* __restrict__ dyn, const bf16* __restrict__ base,
                                                    const bf16* __restrict__ w, float* __restrict__ ssq,
                                                    bf16* __restrict__ Xw, bf16* __restrict__ Xw_lo) {
  const int r = blockIdx.x, j = blockIdx.y;
  const int G = h / DC_GS, Np = 4 * G;
  const int col = j * SSQ_COLS + threadIdx.x * 4;
  const size_t o = (size_t)r * h + col;
  const bool has_prev = (r % gamma) != 0;
  const f32x4 s0 = sum_splits<32, f32x4>(P + o, S, ps, gsz);
  const f32x4 s1 = has_prev ? sum_splits<32, f32x4>(P + o - h, S, ps, gsz) : f32x4{0.f, 0.f, 0.f, 0.f};
  const int g = col / DC_GS;
  const float d0 = dyn[(size_t)r * Np + 2 * G + g], d1 = dyn[(size_t)r * Np + 3 * G + g];
  float b0[4], b1[4], wf[4];
  load4(base + 2 * h + col, b0);    // application 1, tap 0
  load4(base + 3 * h + col, b1);    // application 1, tap 1
  load4(w + col, wf);
  const f32x4 x = *reinterpret_cast<const f32x4*>(X + o);
  float y[4], yw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = (b0[e] + d0) * s0[e];
    if (has_prev) v += (b1[e] + d1) * s1[e];
    y[e] = x[e] + v;
    yw[e] = y[e] * wf[e];
  }
  *reinterpret_cast<f32x4*>(X + o) = f32x4{y[0], y[1], y[2], y[3]};
  store_hilo4(yw, Xw + o, Xw_lo + o);
  const float ss = wave_sum(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
  if (threadIdx.x == 0) ssq[(size_t)r * SSQ_STRIDE + j] = ss;
}

// ---- top-16 --------------------------------------------------------------------------------
// a larger value, or an equal one at a lower index, ranks first (NaN never enters). Written
// without short-circuit evaluation: with the operands in LDS, `||` / `&&` made the compiler
// branch around (and wait on) each load.
__device__ __forceinline__ bool tk_before(float v, int i, float bv, int bi) {
  return (v > bv) | ((v == bv) & (i < bi));
}

// how many of the N candidates in LDS rank before (v, i); unique indices make the ranks
// unique. N is fixed (unused slots hold (-inf, distinct indices past the vocabulary), which
// rank after every real candidate); the loop is unrolled with four counters so the LDS
// reads are issued back to back.
template <int N>
__device__ __forceinline__ int tk_rank(float v, int i, const float* sv, const int* si) {
  int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
#pragma unroll
  for (int j = 0; j < N; j += 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(sv + j);
    const i32x4 b = *reinterpret_cast<const i32x4*>(si + j);
    r0 += (int)tk_before(a[0], b[0], v, i);
    r1 += (int)tk_before(a[1], b[1], v, i);
    r2 += (int)tk_before(a[2], b[2], v, i);
    r3 += (int)tk_before(a[3], b[3], v, i);
  }
  return (r0 + r1) + (r2 + r3);
}

// insert (v, i) into a thread's sorted list (best first) if it ranks above its last entry
__device__ __forceinline__ void tk_insert(float (&lv)[TOPK], int (&li)[TOPK], float v, int i) {
  if (!tk_before(v, i, lv[TOPK - 1], li[TOPK - 1])) return;
  lv[TOPK - 1] = v;
  li[TOPK - 1] = i;
#pragma unroll
  for (int q = TOPK - 1; q > 0; --q) {
    if (tk_before(lv[q], li[q], lv[q - 1], li[q - 1])) {
      const float tv = lv[q]; lv[q] = lv[q - 1]; lv[q - 1] = tv;
      const int ti = li[q]; li[q] = li[q - 1]; li[q - 1] = ti;
    }
  }
}

// The wavefront's 16 best over its lanes' sorted lists: 16 rounds, each taking the best list
// head across the lanes (no barrier) and popping it from its owner's list. Lane q gets entry q
// in (wv, wi) for q < 16.
__device__ __forceinline__ void tk_wave(float (&lv)[TOPK], int (&li)[TOPK], float& wv, int& wi) {
  const int lane = threadIdx.x & 63;
  wv = -INFINITY;
  wi = 0x7fffffff;
  for (int q = 0; q < TOPK; ++q) {
    float v = lv[0];
    int i = li[0], t = lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oi = __shfl_xor(i, o, 64), ot = __shfl_xor(t, o, 64);
      if (tk_before(ov, oi, v, i)) { v = ov; i = oi; t = ot; }
    }
    if (lane == q) { wv = v; wi = i; }
    if (lane == t) {
#pragma unroll
      for (int p = 0; p < TOPK - 1; ++p) { lv[p] = lv[p + 1]; li[p] = li[p + 1]; }
      lv[TOPK - 1] = -INFINITY;
      li[TOPK - 1] = 0x7fffffff;
    }
  }
}

// The 16 best of up to 64 candidates, one a lane (-inf where there is none): lane q gets entry q.
__device__ __forceinline__ void tk_wave64(float v0, int i0, float& wv, int& wi) {
  float lv[TOPK];
  int li[TOPK];
  lv[0] = v0;
  li[0] = i0;
#pragma unroll
  for (int q = 1; q < TOPK; ++q) { lv[q] = -INFINITY; li[q] = 0x7fffffff; }
  tk_wave(lv, li, wv, wi);
}

// Visit the elements [lo, hi) of a logits row, thread by thread: f(x, index). With a 16-byte
// aligned row and 4-aligned bounds the loads are float4, four per lane in flight per round;
// otherwise one float at a time.
template <class F>
__device__ __forceinline__ void tk_scan(const float* __restrict__ lr, int lo, int hi, bool vec, F&& f) {
  if (vec) {
    constexpr int U = 4;
    const f32x4* l4 = reinterpret_cast<const f32x4*>(lr);
    const int lo4 = lo / 4, hi4 = hi / 4;
    for (int q = lo4 + (int)threadIdx.x; q < hi4; q += 256 * U) {
      f32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = q + u * 256;
        x[u] = k < hi4 ? l4[k] : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) f(x[u][e], (q + u * 256) * 4 + e);
    }
  } else {
    for (int v = lo + (int)threadIdx.x; v < hi; v += 256) f(lr[v], v);
  }
}

// One 256-thread workgroup per (drafted row, vocabulary slice): the slice's 16 best logits.
// Pass 1: every thread's maximum; the 16th largest of those (by rank: each wave's 16 best, then
// the best 16 of those 64) is a lower bound T of the slice's 16th largest value, since the 16
// largest maxima are 16 distinct elements. Pass 2: the elements >= T are gathered in LDS (an
// LDS counter) and ranked. More than 64 of them (mass ties) fall back to every thread's
// sorted list, so the result is exact either way.
__global__ __launch_bounds__(256) void k_topk_partial(const float* __restrict__ logits, int V, int slice,
                                                      float* __restrict__ cv, int* __restrict__ ci) {
  constexpr int CAP = 64;
  __shared__ __attribute__((aligned(16))) float mv[256];
  __shared__ __attribute__((aligned(16))) int mix[256];
  __shared__ __attribute__((aligned(16))) float tv[4 * TOPK];
  __shared__ __attribute__((aligned(16))) int ti[4 * TOPK];
  __shared__ __attribute__((aligned(16))) float gv[CAP];
  __shared__ __attribute__((aligned(16))) int gi[CAP];
  __shared__ int cnt;
  __shared__ float thr;
  const int row = blockIdx.x, sl = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lo = sl * slice, hi = min(V, lo + slice);
  const float* lr = logits + (size_t)row * V;
  const bool vec = (V & 3) == 0 && (slice & 3) == 0 && ((uintptr_t)logits & 15) == 0;
  float mx = -INFINITY;
  int mi = 0x7fffffff - (int)threadIdx.x;   // empty threads stay distinct (and last)
  tk_scan(lr, lo, hi, vec, [&](float x, int v) {
    if (tk_before(x, v, mx, mi)) { mx = x; mi = v; }
  });
  mv[threadIdx.x] = mx;
  mix[threadIdx.x] = mi;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  {
    const int r = tk_rank<64>(mx, mi, mv + wave * 64, mix + wave * 64);
    if (r < TOPK) { tv[wave * TOPK + r] = mx; ti[wave * TOPK + r] = mi; }
  }
  __syncthreads();
  if (wave == 0 && tk_rank<4 * TOPK>(tv[lane], ti[lane], tv, ti) == TOPK - 1) thr = tv[lane];
  if (wave == 1) { gv[lane] = -INFINITY; gi[lane] = 0x7fffffff - lane; }   // unused gather slots
  __syncthreads();
  const float t = thr;
  tk_scan(lr, lo, hi, vec, [&](float x, int v) {
    if (x >= t) {
      const int q = atomicAdd(&cnt, 1);
      if (q < CAP) { gv[q] = x; gi[q] = v; }
    }
  });
  __syncthreads();
  const int n = cnt;
  const size_t o = ((size_t)row * gridDim.y + sl) * TOPK;
  if (n <= CAP) {
    // n >= 16: the 16 largest maxima are all >= T
    if (wave == 0 && lane < n) {
      const int r = tk_rank<CAP>(gv[lane], gi[lane], gv, gi);
      if (r < TOPK) { cv[o + r] = gv[lane]; ci[o + r] = gi[lane]; }
    }
    return;
  }
  // mass ties at the threshold: every thread's sorted list, then the waves' 16 best, then wave 0
  float lv[TOPK];
  int li[TOPK];
#pragma unroll
  for (int q = 0; q < TOPK; ++q) { lv[q] = -INFINITY; li[q] = 0x7fffffff; }
  tk_scan(lr, lo, hi, vec, [&](float x, int v) { tk_insert(lv, li, x, v); });
  float wv;
  int wi;
  tk_wave(lv, li, wv, wi);
  if (lane < TOPK) { tv[wave * TOPK + lane] = wv; ti[wave * TOPK + lane] = wi; }
  __syncthreads();
  if (wave == 0) {
    tk_wave64(tv[lane], ti[lane], wv, wi);
    if (lane < TOPK) { cv[o + lane] = wv; ci[o + lane] = wi; }
  }
}

// ---- selector ------------------------------------------------------------------------------
// One 256-thread workgroup per drafted row d (band b, block row i = d % (gamma-1) + 1): the pair
// scores T[p][c] = logit(c) + sum_r pred[prev_p][r] * H[r] * succ[c][r] for the row's candidates
// c and the previous row's candidates p (the band's bonus token alone for its first drafted
// row). H = the canonical sum of the hidden projection's split partials for block row b*gamma+i.
// The 16 predecessor rows (times H) and the 16 successor rows are staged in LDS with all their
// loads issued at once; each thread then forms one (p, c) dot product from LDS.
template <int R>
__global__ __launch_bounds__(256) void k_selector_pairs(const float* __restrict__ cv, const int* __restrict__ ci,
                                                        int n_slices, const float* __restrict__ Hp, int S, long long ps,
                                                        int gsz, int gamma, int V, SelectorBonus bonus,
                                                        const bf16* __restrict__ pred, const bf16* __restrict__ succ,
                                                        float* __restrict__ sel_v, int* __restrict__ sel_i,
                                                        float* __restrict__ pair) {
  __shared__ float sH[R];
  // pred[prev_p] * H and succ[cand_c]; rows 4 floats apart mod 64 banks: 16 lanes reading one
  // float4 each from 16 rows touch 64 distinct banks
  __shared__ __attribute__((aligned(16))) float sG[TOPK][R + 4];
  __shared__ __attribute__((aligned(16))) float sS[TOPK][R + 4];
  __shared__ float scv[TOPK];
  __shared__ int sprev[TOPK], scand[TOPK];
  __shared__ __attribute__((aligned(16))) float mv2[2][TOPK_MAX_SLICES * TOPK];
  __shared__ __attribute__((aligned(16))) int mi2[2][TOPK_MAX_SLICES * TOPK];
  const int d = blockIdx.x, g1 = gamma - 1, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = d / g1, i = d % g1 + 1;
  const int row = b * gamma + i;
  const int np = i == 1 ? 1 : TOPK;
  // the row's candidates (wave 0) and the previous row's (wave 1), each the 16 best of the
  // row's slice lists (at most 64 entries, one a lane); the first drafted row's predecessor is
  // the band's bonus token
  // the slices' lists of this row (k = 0) and of the previous drafted row (k = 1): at most
  // 256 entries each, every one ranked by one thread
  const int nc = n_slices * TOPK;
  const int nrows = i > 1 ? 2 : 1;
  for (int k = 0; k < nrows; ++k) {
    const size_t base = (size_t)(d - k) * nc;
    const bool in = (int)threadIdx.x < nc;
    mv2[k][threadIdx.x] = in ? cv[base + threadIdx.x] : -INFINITY;
    mi2[k][threadIdx.x] = in ? ci[base + threadIdx.x] : 0x7fffffff - (int)threadIdx.x;
  }
  for (int q = threadIdx.x; q < R; q += 256) sH[q] = sum_splits<8, float>(Hp + (size_t)row * R + q, S, ps, gsz);
  __syncthreads();
  for (int k = 0; k < nrows; ++k)
    if ((int)threadIdx.x < nc) {
      const float v = mv2[k][threadIdx.x];
      const int id = mi2[k][threadIdx.x];
      const int r = tk_rank<TOPK_MAX_SLICES * TOPK>(v, id, mv2[k], mi2[k]);
      if (r < TOPK) {
        // (ids are clamped: a row with fewer than 16 finite logits leaves placeholder entries)
        const int cid = min(max(id, 0), V - 1);
        if (k == 0) {
          scand[r] = cid;
          scv[r] = v;
          sel_v[(size_t)d * TOPK + r] = v;
          sel_i[(size_t)d * TOPK + r] = id;
        } else {
          sprev[r] = cid;
        }
      }
    }
  if (i == 1 && threadIdx.x < TOPK) sprev[threadIdx.x] = min(max(bonus.t[b], 0), V - 1);
  __syncthreads();
  // 8 bf16 per 16-byte piece: R / 8 pieces a row, 2 * TOPK rows
  constexpr int PPR = R / 8;
  constexpr int NPIECE = 2 * TOPK * PPR;
  u32x4 v[(NPIECE + 255) / 256];
#pragma unroll
  for (int u = 0; u < (NPIECE + 255) / 256; ++u) {
    const int q = threadIdx.x + u * 256;
    const int r2 = q / PPR, k = (q % PPR) * 8;
    const bool is_pred = r2 < TOPK;
    const int id = is_pred ? sprev[r2] : scand[r2 - TOPK];
    v[u] = u32x4{0u, 0u, 0u, 0u};
    if (q < NPIECE && (!is_pred || r2 < np))
      v[u] = *reinterpret_cast<const u32x4*>((is_pred ? pred : succ) + (size_t)id * R + k);
  }
#pragma unroll
  for (int u = 0; u < (NPIECE + 255) / 256; ++u) {
    const int q = threadIdx.x + u * 256;
    if (q >= NPIECE) continue;
    const int r2 = q / PPR, k = (q % PPR) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = bf2f((bf16)((v[u][e >> 1] >> (16 * (e & 1))) & 0xffff));
      if (r2 < TOPK) sG[r2][k + e] = f * sH[k + e];
      else sS[r2 - TOPK][k + e] = f;
    }
  }
  __syncthreads();
  const int p = threadIdx.x >> 4, c = threadIdx.x & 15;
  if (p >= np) return;
  float acc = 0.f;
#pragma unroll 8
  for (int k = 0; k < R; k += 4) {
    const f32x4 g4 = *reinterpret_cast<const f32x4*>(&sG[p][k]);
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(&sS[c][k]);
    acc += g4[0] * s4[0];
    acc += g4[1] * s4[1];
    acc += g4[2] * s4[2];
    acc += g4[3] * s4[3];
  }
  pair[((size_t)d * TOPK + p) * TOPK + c] = scv[c] + acc;
}

// One wavefront per band: the greedy walk over the pair tables, staged in LDS first (all
// loads issued at once, so no step waits on memory), the drafts written per row.
__global__ __launch_bounds__(256) void k_selector_walk(const int* __restrict__ sel_i, const float* __restrict__ pair,
                                                       int gamma, int* __restrict__ tokens) {
  constexpr int NP4 = (MAX_GAMMA - 1) * TOPK * TOPK / 4;   // float4 pieces of the largest band
  __shared__ f32x4 sp4[NP4];
  __shared__ int sc[MAX_GAMMA - 1][TOPK];
  const int b = blockIdx.x, lane = threadIdx.x & 63, g1 = gamma - 1;
  const size_t d0 = (size_t)b * g1;
  // every load of the staging issued before the first store (a fixed, unrolled count)
  const f32x4* src = reinterpret_cast<const f32x4*>(pair + d0 * TOPK * TOPK);
  const int n4 = g1 * TOPK * TOPK / 4;
  f32x4 v[(NP4 + 255) / 256];
#pragma unroll
  for (int u = 0; u < (NP4 + 255) / 256; ++u) {
    const int q = threadIdx.x + u * 256;
    v[u] = q < n4 ? src[q] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int ci_ = threadIdx.x < g1 * TOPK ? sel_i[d0 * TOPK + threadIdx.x] : 0;
#pragma unroll
  for (int u = 0; u < (NP4 + 255) / 256; ++u) {
    const int q = threadIdx.x + u * 256;
    if (q < n4) sp4[q] = v[u];
  }
  if (threadIdx.x < g1 * TOPK) (&sc[0][0])[threadIdx.x] = ci_;
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const float* sp = reinterpret_cast<const float*>(sp4);
  int p = 0;   // position of the previous pick in the previous row's candidates (0 = the bonus row)
  for (int k = 0; k < g1; ++k) {
    // the row's best candidate: the lane whose score no other candidate beats
    const float* rowp = sp + (k * TOPK + p) * TOPK;
    bool best = false;
    if (lane < TOPK) {
      const float v = rowp[lane];
      int r = 0;
#pragma unroll
      for (int j = 0; j < TOPK; ++j) r += tk_before(rowp[j], j, v, lane) ? 1 : 0;
      best = r == 0 && v == v;
    }
    const unsigned long long m = __ballot(best);
    // (no finite score at all: the first candidate is taken)
    p = m ? __ffsll((long long)m) - 1 : 0;
    if (lane == 0) tokens[d0 + k] = sc[k][p];
  }
}

}  // namespace

hipError_t launch_dconv_prepare(const bf16* Xw, const bf16* Xw_lo, const float* ssq, float eps, int M, int h,
                                int gamma, const float* P, int S, long long part_stride, int gsz, const bf16* base,
                                float* dyn, bf16* U, bf16* U_lo, hipStream_t st) {
  if (M < 1 || h % SSQ_COLS || h > SSQ_STRIDE * SSQ_COLS || gamma < 1 || gsz < 1) return hipErrorInvalidValue;
  return launch(k_dconv_prepare, dim3(M, h / SSQ_COLS), dim3(64), 0, st, Xw, Xw_lo, ssq, eps, h, gamma, P, S,
                part_stride, gsz, base, dyn, U, U_lo);
}

hipError_t launch_resid_dconv(float* X, const float* P, int S, long long part_stride, int gsz, int M, int h, int gamma,
                              const float* dyn, const bf16* base, const bf16* w, float* ssq, bf16* Xw, bf16* Xw_lo,
                              hipStream_t st) {
  if (M < 1 || h % SSQ_COLS || h > SSQ_STRIDE * SSQ_COLS || gamma < 1 || gsz < 1) return hipErrorInvalidValue;
  return launch(k_resid_dconv, dim3(M, h / SSQ_COLS), dim3(64), 0, st, X, P, S, part_stride, gsz, h, gamma, dyn,
                base, w, ssq, Xw, Xw_lo);
}

int topk_slices(int V) { return std::max(1, std::min(TOPK_MAX_SLICES, (V + 8191) / 8192)); }

hipError_t launch_topk_partial(const float* logits, int rows, int V, float* cv, int* ci, hipStream_t st) {
  if (rows < 1 || V < TOPK) return hipErrorInvalidValue;
  const int ns = topk_slices(V);
  const int slice = ((V + ns - 1) / ns + 3) / 4 * 4;   // 4-aligned slice bounds
  return launch(k_topk_partial, dim3(rows, ns), dim3(256), 0, st, logits, V, slice, cv, ci);
}

hipError_t launch_selector_pairs(const float* cv, const int* ci, const float* Hp, int S, long long part_stride, int gsz,
                                 int rank, int n_bands, int gamma, const SelectorBonus& bonus, const bf16* pred,
                                 const bf16* succ, int vocab, float* sel_v, int* sel_i, float* pair, hipStream_t st) {
  if (n_bands < 1 || n_bands > MAX_BANDS || gamma < 2 || gamma > MAX_GAMMA || vocab < TOPK || gsz < 1)
    return hipErrorInvalidValue;
  const dim3 grid(n_bands * (gamma - 1)), block(256);
  const int ns = topk_slices(vocab);
  if (rank == 256)
    return launch(k_selector_pairs<256>, grid, block, 0, st, cv, ci, ns, Hp, S, part_stride, gsz, gamma, vocab, bonus,
                  pred, succ, sel_v, sel_i, pair);
  if (rank == 512)
    return launch(k_selector_pairs<512>, grid, block, 0, st, cv, ci, ns, Hp, S, part_stride, gsz, gamma, vocab, bonus,
                  pred, succ, sel_v, sel_i, pair);
  return hipErrorInvalidValue;
}

hipError_t launch_selector_walk(const int* sel_i, const float* pair, int n_bands, int gamma, int* tokens,
                                hipStream_t st) {
  if (n_bands < 1 || n_bands > MAX_BANDS || gamma < 2 || gamma > MAX_GAMMA) return hipErrorInvalidValue;
  return launch(k_selector_walk, dim3(n_bands), dim3(256), 0, st, sel_i, pair, gamma, tokens);
}

}  // namespace dfl
