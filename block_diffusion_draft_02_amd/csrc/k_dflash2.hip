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
// a larger value, or an equal one at a lower index, ranks first (NaN never enters)
__device__ __forceinline__ bool tk_before(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

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

// The workgroup's 16 best over every thread's sorted list: 16 rounds, each taking the best
// list head (a wave reduction, then the 4 waves) and popping it from its owner's list.
__device__ void tk_workgroup(float (&lv)[TOPK], int (&li)[TOPK], float* __restrict__ out_v,
                             int* __restrict__ out_i) {
  __shared__ float wv[4];
  __shared__ int wi[4], wt[4];
  __shared__ int win_t;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int q = 0; q < TOPK; ++q) {
    float v = lv[0];
    int i = li[0], t = threadIdx.x;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oi = __shfl_xor(i, o, 64), ot = __shfl_xor(t, o, 64);
      if (tk_before(ov, oi, v, i)) { v = ov; i = oi; t = ot; }
    }
    if (lane == 0) { wv[wave] = v; wi[wave] = i; wt[wave] = t; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = wv[0];
      int bi = wi[0], bt = wt[0];
      for (int w = 1; w < 4; ++w)
        if (tk_before(wv[w], wi[w], bv, bi)) { bv = wv[w]; bi = wi[w]; bt = wt[w]; }
      out_v[q] = bv;
      out_i[q] = bi;
      win_t = bt;
    }
    __syncthreads();
    if ((int)threadIdx.x == win_t) {
#pragma unroll
      for (int p = 0; p < TOPK - 1; ++p) { lv[p] = lv[p + 1]; li[p] = li[p + 1]; }
      lv[TOPK - 1] = -INFINITY;
      li[TOPK - 1] = 0x7fffffff;
    }
  }
}

// One 256-thread workgroup per (drafted row, vocabulary slice): the slice's 16 best logits.
__global__ __launch_bounds__(256) void k_topk_partial(const float* __restrict__ logits, int V, int slice,
                                                      float* __restrict__ cv, int* __restrict__ ci) {
  const int row = blockIdx.x, sl = blockIdx.y;
  float lv[TOPK];
  int li[TOPK];
#pragma unroll
  for (int q = 0; q < TOPK; ++q) { lv[q] = -INFINITY; li[q] = 0x7fffffff; }
  const int lo = sl * slice, hi = min(V, lo + slice);
  const float* lr = logits + (size_t)row * V;
  for (int v = lo + threadIdx.x; v < hi; v += 256) tk_insert(lv, li, lr[v], v);
  const size_t o = ((size_t)row * gridDim.y + sl) * TOPK;
  tk_workgroup(lv, li, cv + o, ci + o);
}

// One workgroup per drafted row: the row's 16 best over its slices' lists.
__global__ __launch_bounds__(256) void k_topk_merge(const float* __restrict__ cv, const int* __restrict__ ci,
                                                    int n_slices, float* __restrict__ sel_v, int* __restrict__ sel_i) {
  const int row = blockIdx.x;
  float lv[TOPK];
  int li[TOPK];
#pragma unroll
  for (int q = 0; q < TOPK; ++q) { lv[q] = -INFINITY; li[q] = 0x7fffffff; }
  const size_t base = (size_t)row * n_slices * TOPK;
  for (int q = threadIdx.x; q < n_slices * TOPK; q += 256) tk_insert(lv, li, cv[base + q], ci[base + q]);
  tk_workgroup(lv, li, sel_v + (size_t)row * TOPK, sel_i + (size_t)row * TOPK);
}

// ---- selector ------------------------------------------------------------------------------
// One 256-thread workgroup per drafted row d (band b, block row i = d % (gamma-1) + 1): the pair
// scores T[p][c] = logit(c) + sum_r pred[prev_p][r] * H[r] * succ[c][r] for the row's candidates
// c and the previous row's candidates p (the band's bonus token alone for its first drafted
// row). H = the canonical sum of the hidden projection's split partials for block row b*gamma+i.
__global__ __launch_bounds__(256) void k_selector_pairs(const int* __restrict__ sel_i, const float* __restrict__ sel_v,
                                                        const float* __restrict__ Hp, int S, long long ps, int gsz,
                                                        int rank, int gamma, int V, SelectorBonus bonus,
                                                        const bf16* __restrict__ pred, const bf16* __restrict__ succ,
                                                        float* __restrict__ pair) {
  __shared__ float sH[SELECTOR_MAX_RANK];
  __shared__ int sprev[TOPK], scand[TOPK];
  const int d = blockIdx.x, g1 = gamma - 1;
  const int b = d / g1, i = d % g1 + 1;
  const int row = b * gamma + i;
  for (int q = threadIdx.x; q < rank; q += 256) sH[q] = sum_splits<8, float>(Hp + (size_t)row * rank + q, S, ps, gsz);
  if (threadIdx.x < TOPK) {
    scand[threadIdx.x] = sel_i[(size_t)d * TOPK + threadIdx.x];
    sprev[threadIdx.x] = i == 1 ? bonus.t[b] : sel_i[(size_t)(d - 1) * TOPK + threadIdx.x];
  }
  __syncthreads();
  // thread (p, c): one dot product over the rank (p = 0 only for the band's first row)
  const int p = threadIdx.x >> 4, c = threadIdx.x & 15;
  if (i == 1 && p > 0) return;
  // (ids are clamped: a row with fewer than 16 finite logits leaves placeholder entries)
  const int tp = min(max(sprev[p], 0), V - 1), tc = min(max(scand[c], 0), V - 1);
  const bf16* pr = pred + (size_t)tp * rank;
  const bf16* sr = succ + (size_t)tc * rank;
  float acc = 0.f;
  for (int q = 0; q < rank; q += 4) {
    float pv[4], sv[4];
    load4(pr + q, pv);
    load4(sr + q, sv);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += pv[e] * sH[q + e] * sv[e];
  }
  pair[((size_t)d * TOPK + p) * TOPK + c] = sel_v[(size_t)d * TOPK + c] + acc;
}

// One wavefront per band: the greedy walk over the pair tables, the drafts written per row.
__global__ __launch_bounds__(64) void k_selector_walk(const int* __restrict__ sel_i, const float* __restrict__ pair,
                                                      int gamma, int* __restrict__ tokens) {
  const int b = blockIdx.x, lane = threadIdx.x, g1 = gamma - 1;
  int p = 0;   // position of the previous pick in the previous row's candidates (0 = the bonus row)
  for (int k = 0; k < g1; ++k) {
    const size_t d = (size_t)b * g1 + k;
    float v = lane < TOPK ? pair[(d * TOPK + p) * TOPK + lane] : -INFINITY;
    int c = lane < TOPK ? lane : 0x7fffffff;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oc = __shfl_xor(c, o, 64);
      if (tk_before(ov, oc, v, c)) { v = ov; c = oc; }
    }
    // (no finite score leaves c past the list: the first candidate is taken)
    p = c < TOPK ? c : 0;
    if (lane == 0) tokens[d] = sel_i[d * TOPK + p];
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

int topk_slices(int V) { return std::max(1, std::min(TOPK_MAX_SLICES, (V + 2047) / 2048)); }

hipError_t launch_topk_partial(const float* logits, int rows, int V, float* cv, int* ci, hipStream_t st) {
  if (rows < 1 || V < TOPK) return hipErrorInvalidValue;
  const int ns = topk_slices(V);
  return launch(k_topk_partial, dim3(rows, ns), dim3(256), 0, st, logits, V, (V + ns - 1) / ns, cv, ci);
}

hipError_t launch_topk_merge(const float* cv, const int* ci, int rows, int V, float* sel_v, int* sel_i,
                             hipStream_t st) {
  if (rows < 1 || V < TOPK) return hipErrorInvalidValue;
  return launch(k_topk_merge, dim3(rows), dim3(256), 0, st, cv, ci, topk_slices(V), sel_v, sel_i);
}

hipError_t launch_selector_pairs(const int* sel_i, const float* sel_v, const float* Hp, int S, long long part_stride,
                                 int gsz, int rank, int n_bands, int gamma, const SelectorBonus& bonus,
                                 const bf16* pred, const bf16* succ, int vocab, float* pair, hipStream_t st) {
  if (n_bands < 1 || n_bands > MAX_BANDS || gamma < 2 || rank < 4 || rank % 4 || rank > SELECTOR_MAX_RANK ||
      vocab < TOPK || gsz < 1)
    return hipErrorInvalidValue;
  return launch(k_selector_pairs, dim3(n_bands * (gamma - 1)), dim3(256), 0, st, sel_i, sel_v, Hp, S, part_stride,
                gsz, rank, gamma, vocab, bonus, pred, succ, pair);
}

hipError_t launch_selector_walk(const int* sel_i, const float* pair, int n_bands, int gamma, int* tokens,
                                hipStream_t st) {
  if (n_bands < 1 || n_bands > MAX_BANDS || gamma < 2) return hipErrorInvalidValue;
  return launch(k_selector_walk, dim3(n_bands), dim3(64), 0, st, sel_i, pair, gamma, tokens);
}

}  // namespace dfl
