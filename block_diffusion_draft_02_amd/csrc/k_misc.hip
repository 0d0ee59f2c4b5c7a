// Row-wise kernels of the drafter: the forward prologue (block-table updates, block-row
// slots, embedding gather + first input RMSNorm), the Q/K/V epilogue (per-head RMSNorm,
// RoPE, YaRN mscale, K/V writeback into the paged pool), residual add + RMSNorm, SwiGLU,
// and the context-append kernels (slots, hidden_norm, context K/V writeback).
//
// Arithmetic follows memra_engine/dflash.rs (DflashDraft::forward_round, ::ingest_ctx,
// ::ctx_features, ::rope_rows): vanilla RMSNorm x * w / sqrt(mean(x^2) + eps) (the form
// spark_model/layers/dflash_head/from_weights.rs picks for the drafter), NeoX RoPE over
// the whole head, mscale multiplied into q and k after the rotation under YaRN.
#include "common.hpp"
#include "kernels.hpp"

#include <type_traits>

namespace dfl {

// ---- forward prologue ------------------------------------------------------------------
// workgroup 0: block-table updates, slots and stamped positions of the block rows, band
// table; workgroup 1 + r: embedding row of block row r into the residual stream, the sums
// of squares of its 256-column slices (wave w takes slices w, w + 4, ...) and the row times
// layer 0's input-norm weight as hi + lo bf16.
__global__ __launch_bounds__(256) void k_fwd_prologue(FwdArgs a, Band* __restrict__ bands_dev,
                                                      int* __restrict__ bt,
                                                      long long* __restrict__ slots,
                                                      int* __restrict__ kpos,
                                                      const bf16* __restrict__ embed,
                                                      const bf16* __restrict__ w_in0, int h,
                                                      float* __restrict__ X, float* __restrict__ ssq,
                                                      bf16* __restrict__ Xw, bf16* __restrict__ Xw_lo) {
  if (blockIdx.x == 0) {
    for (int j = threadIdx.x; j < a.n_upd; j += 256) bt[a.upd_off[j]] = a.upd_page[j];
    const int M = a.n_bands * a.gamma;
    for (int r = threadIdx.x; r < M; r += 256) {
      const int b = r / a.gamma, i = r % a.gamma;
      const int C = a.bands[b].kv_len;
      const int p = C + i;
      const int lp = (p >> 4) - (C >> 4);
      const long long slot = (long long)a.bands[b].pg[lp] * PAGE + (p & (PAGE - 1));
      slots[r] = slot;
      kpos[slot] = a.bands[b].q_pos + i;
    }
    for (int b = threadIdx.x; b < a.n_bands; b += 256) bands_dev[b] = a.bands[b];
    return;
  }
  const int r = blockIdx.x - 1;
  const int b = r / a.gamma, i = r % a.gamma;
  const int tok = (i == 0) ? a.bands[b].bonus : a.mask_token;
  const bf16* e = embed + (size_t)tok * h;
  float* x = X + (size_t)r * h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nsl = h / SSQ_COLS;
  for (int j = wave; j < nsl; j += 4) {
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < SSQ_COLS / 64; ++q) {
      const int col = j * SSQ_COLS + q * 64 + lane;
      const float v = bf2f(e[col]);
      x[col] = v;
      ss += v * v;
      split_bf16(v * bf2f(w_in0[col]), Xw[(size_t)r * h + col], Xw_lo[(size_t)r * h + col]);
    }
    ss = wave_sum(ss);
    if (lane == 0) ssq[(size_t)r * SSQ_STRIDE + j] = ss;
  }
}

hipError_t launch_fwd_prologue(const FwdArgs& a, Band* bands_dev, int* bt, long long* slots,
                               int* kpos, const bf16* embed, const bf16* w_in0, int h, float* X,
                               float* ssq, bf16* Xw, bf16* Xw_lo, hipStream_t st) {
  if (h % SSQ_COLS || h > SSQ_STRIDE * SSQ_COLS) return hipErrorInvalidValue;
  const int M = a.n_bands * a.gamma;
  (void)launch(k_fwd_prologue, 1 + M, 256, 0, st, a, bands_dev, bt, slots, kpos, embed, w_in0, h, X, ssq, Xw, Xw_lo);
  return hipGetLastError();
}

// ---- Q/K/V epilogue ---------------------------------------------------------------------
// one wavefront per (row, head) of the fused [q | k | v] projection; lane l < hd/2 owns the
// RoPE pair (l, l + hd/2)
template <int HD>
__global__ __launch_bounds__(64) void k_qkv_post(const float* __restrict__ P, int S,
                                                 long long ps, int gsz, int N, int gamma,
                                                 const Band* __restrict__ bands, int nh, int nkv,
                                                 const bf16* __restrict__ qn,
                                                 const bf16* __restrict__ kn, float eps,
                                                 const double* __restrict__ inv_freq,
                                                 float mscale, const long long* __restrict__ slots,
                                                 KvGeom g, int layer, bf16* __restrict__ Q,
                                                 bf16* __restrict__ Q_lo) {
  constexpr int H2 = HD / 2;
  const int r = blockIdx.x, hh = blockIdx.y, l = threadIdx.x;
  const bool act = l < H2;
  const int col = hh * HD + (act ? l : 0);
  float x1 = 0.f, x2 = 0.f;
  if (act) {
    const float* p = P + (size_t)r * N + col;
    x1 = sum_splits<8, float>(p, S, ps, gsz);
    x2 = sum_splits<8, float>(p + H2, S, ps, gsz);
  }
  const int kind = hh < nh ? 0 : (hh < nh + nkv ? 1 : 2);
  if (kind != 2) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float rs = rsqrtf(ss / (float)HD + eps);
    if (act) {
      const bf16* w = kind == 0 ? qn : kn;
      x1 *= rs * bf2f(w[l]);
      x2 *= rs * bf2f(w[l + H2]);
      const int b = r / gamma, i = r % gamma;
      rope_pair(x1, x2, bands[b].q_pos + i, inv_freq[l]);
      x1 *= mscale;
      x2 *= mscale;
    }
  }
  if (!act) return;
  if (kind == 0) {
    const size_t o = ((size_t)r * nh + hh) * HD;
    split_bf16(x1, Q[o + l], Q_lo[o + l]);
    split_bf16(x2, Q[o + l + H2], Q_lo[o + l + H2]);
    return;
  }
  const long long slot = slots[r];
  const long long page = slot >> 4;
  const int off = (int)(slot & (PAGE - 1));
  bf16* pg = g.pool + ((size_t)layer * g.num_pages + page) * page_layer_elems(g.nkv, HD);
  if (kind == 1) {
    bf16* k = pg + ((size_t)(hh - nh) * PAGE + off) * HD;
    k[l] = f2bf(x1);
    k[l + H2] = f2bf(x2);
  } else {
    bf16* v = pg + (size_t)(g.nkv + hh - nh - nkv) * HD * PAGE + off;
    v[(size_t)l * PAGE] = f2bf(x1);
    v[(size_t)(l + H2) * PAGE] = f2bf(x2);
  }
}

hipError_t launch_qkv_post(const float* P, int S, long long part_stride, int gsz, int M, int gamma,
                           const Band* bands_dev, int nh, int nkv, int hd, const bf16* q_norm,
                           const bf16* k_norm, float eps, const double* inv_freq, float mscale,
                           const long long* slots, KvGeom g, int layer, bf16* Q, bf16* Q_lo,
                           hipStream_t st) {
  const int N = (nh + 2 * nkv) * hd;
  dim3 grid(M, nh + 2 * nkv);
  switch (hd) {
    case 32: (void)launch(k_qkv_post<32>, grid, 64, 0, st, P, S, part_stride, gsz, N, gamma, bands_dev, nh, nkv, q_norm, k_norm, eps, inv_freq, mscale, slots, g, layer, Q, Q_lo); break;
    case 64: (void)launch(k_qkv_post<64>, grid, 64, 0, st, P, S, part_stride, gsz, N, gamma, bands_dev, nh, nkv, q_norm, k_norm, eps, inv_freq, mscale, slots, g, layer, Q, Q_lo); break;
    case 128: (void)launch(k_qkv_post<128>, grid, 64, 0, st, P, S, part_stride, gsz, N, gamma, bands_dev, nh, nkv, q_norm, k_norm, eps, inv_freq, mscale, slots, g, layer, Q, Q_lo); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---- residual add + RMSNorm ---------------------------------------------------------------
// The row-wise consumers of split-K partials: one workgroup per row (rn_threads(h) threads),
// thread t owns the 4-float slices t, t + T, ... of the row and adds their partials in the
// canonical order.
constexpr int RN_HMAX = 8192;      // row length the LDS row buffer holds

// x (LDS row of h floats, complete) -> out = x * rs * w as hi + lo bf16
__device__ __forceinline__ void norm_out(const float* xs, int h, float rs, const bf16* __restrict__ w,
                                         bf16* __restrict__ o, bf16* __restrict__ ol) {
  for (int j = threadIdx.x * 4; j < h; j += blockDim.x * 4) {
    // the norm weight is a caller's pointer with only bf16 alignment guaranteed
    const float wf[4] = {bf2f(w[j]), bf2f(w[j + 1]), bf2f(w[j + 2]), bf2f(w[j + 3])};
    bf16 hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_bf16(xs[j + e] * rs * wf[e], hi[e], lo[e]);
    *reinterpret_cast<u32x2*>(o + j) = u32x2{(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
    *reinterpret_cast<u32x2*>(ol + j) = u32x2{(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
  }
}

// threads of a row workgroup: one per 4-float slice up to 1024 (whole waves; a row of 2048 took
// 1024 threads with half of them idle, and twice the rounds of workgroups)
static unsigned rn_threads(int h) { return (unsigned)std::min(1024, std::max(64, (h / 4 + 63) / 64 * 64)); }

// Sum of the split partials of row r (plus the residual X when given), kept in the LDS row
// xs and written back to X; returns the row's sum of squares (valid in every thread).
__device__ __forceinline__ float rows_gather(float* __restrict__ X, const float* __restrict__ p, int S,
                                             long long ps, int gsz, int h, float* xs, float* red_ss) {
  float ss = 0.f;
  for (int j = threadIdx.x * 4; j < h; j += blockDim.x * 4) {
    f32x4 y = sum_splits<16, f32x4>(p + j, S, ps, gsz);
    if (X != nullptr) y = *reinterpret_cast<const f32x4*>(X + j) + y;
    *reinterpret_cast<f32x4*>(xs + j) = y;
    if (X != nullptr) *reinterpret_cast<f32x4*>(X + j) = y;
    ss += y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red_ss[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += red_ss[i];
  return tot;
}

// X[r] += sum_s P[s][r]; Xn[r] = RMSNorm_w(X[r]) as hi + lo bf16; one workgroup per row
__global__ __launch_bounds__(1024) void k_resid_norm(float* __restrict__ X, const float* __restrict__ P,
                                                     int S, long long ps, int gsz, int h,
                                                     const bf16* __restrict__ w, float eps,
                                                     bf16* __restrict__ Xn, bf16* __restrict__ Xn_lo) {
  __shared__ __attribute__((aligned(16))) float xs[RN_HMAX];
  __shared__ float red_ss[16];
  const int r = blockIdx.x;
  const float tot = rows_gather(X + (size_t)r * h, P + (size_t)r * h, S, ps, gsz, h, xs, red_ss);
  const float rs = rsqrtf(tot / (float)h + eps);
  norm_out(xs, h, rs, w, Xn + (size_t)r * h, Xn_lo + (size_t)r * h);
}

hipError_t launch_resid_norm(float* X, const float* P, int S, long long part_stride, int gsz, int M,
                             int h, const bf16* w, float eps, bf16* Xn, bf16* Xn_lo,
                             hipStream_t st) {
  if (h > RN_HMAX || h % 4 || gsz < 1) return hipErrorInvalidValue;
  (void)launch(k_resid_norm, M, rn_threads(h), 0, st, X, P, S, part_stride, gsz, h, w, eps, Xn, Xn_lo);
  return hipGetLastError();
}

// ---- residual add, parallel form ----------------------------------------------------------
// One 64-thread workgroup per (row, 256-column slice): X[r] += the canonical sum of the split
// partials (every load of a pass issued before the first add); then the slice's sum of
// squares (the next GEMM turns the row's sums into its RMSNorm scale) and X * w as the next
// GEMM's hi + lo activation.
__global__ __launch_bounds__(64) void k_resid_sum(float* __restrict__ X, const float* __restrict__ P,
                                                  int S, long long ps, int gsz, int h, const bf16* __restrict__ w,
                                                  float* __restrict__ ssq, bf16* __restrict__ Xw,
                                                  bf16* __restrict__ Xw_lo) {
  const int r = blockIdx.x, j = blockIdx.y;
  const int col = j * SSQ_COLS + threadIdx.x * 4;
  const size_t o = (size_t)r * h + col;
  const f32x4 x = *reinterpret_cast<const f32x4*>(X + o);
  const u32x2 wb = *reinterpret_cast<const u32x2*>(w + col);   // the context's aligned copy
  const f32x4 acc = sum_splits<32, f32x4>(P + o, S, ps, gsz);   // up to 32 splits in one load pass
  const f32x4 y = x + acc;
  *reinterpret_cast<f32x4*>(X + o) = y;
  const float wf[4] = {bf2f((bf16)(wb.x & 0xffff)), bf2f((bf16)(wb.x >> 16)), bf2f((bf16)(wb.y & 0xffff)), bf2f((bf16)(wb.y >> 16))};
  bf16 hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16(y[e] * wf[e], hi[e], lo[e]);
  *reinterpret_cast<u32x2*>(Xw + o) = u32x2{(uint32_t)hi[0] | ((uint32_t)hi[1] << 16), (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
  *reinterpret_cast<u32x2*>(Xw_lo + o) = u32x2{(uint32_t)lo[0] | ((uint32_t)lo[1] << 16), (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
  const float ss = wave_sum(y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3]);
  if (threadIdx.x == 0) ssq[(size_t)r * SSQ_STRIDE + j] = ss;
}

hipError_t launch_resid_sum(float* X, const float* P, int S, long long part_stride, int gsz, int M, int h,
                            const bf16* w, float* ssq, bf16* Xw, bf16* Xw_lo, hipStream_t st) {
  if (h % SSQ_COLS || h > SSQ_STRIDE * SSQ_COLS || gsz < 1) return hipErrorInvalidValue;
  (void)launch(k_resid_sum, dim3(M, h / SSQ_COLS), 64, 0, st, X, P, S, part_stride, gsz, h, w, ssq, Xw, Xw_lo);
  return hipGetLastError();
}

// ---- SwiGLU -----------------------------------------------------------------------------
// the fused gate/up projection's columns are [gate (ff) | up (ff)]; one thread per four
// consecutive columns of a row (16-byte partial loads), each column's arithmetic on its own
__global__ __launch_bounds__(256) void k_silu_mul(const float* __restrict__ P, int S, long long ps,
                                                  int gsz, int M, int ff, bf16* __restrict__ A,
                                                  bf16* __restrict__ A_lo) {
  const int fq = ff / 4;
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (size_t)M * fq) return;
  const size_t r = q / fq, j = (q % fq) * 4;
  const float* p = P + r * 2 * ff + j;
  const f32x4 gs = sum_splits<8, f32x4>(p, S, ps, gsz), us = sum_splits<8, f32x4>(p + ff, S, ps, gsz);
  bf16 hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) split_bf16(silu(gs[e]) * us[e], hi[e], lo[e]);
  *reinterpret_cast<uint2*>(A + r * ff + j) = uint2{hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16)};
  *reinterpret_cast<uint2*>(A_lo + r * ff + j) = uint2{lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16)};
}

hipError_t launch_silu_mul(const float* P, int S, long long part_stride, int gsz, int M, int ff,
                           bf16* A, bf16* A_lo, hipStream_t st) {
  // 16-byte partial loads: ff and the split stride in whole quads
  if (gsz < 1 || ff % 4 != 0 || part_stride % 4 != 0) return hipErrorInvalidValue;
  const size_t n = (size_t)M * (ff / 4);
  (void)launch(k_silu_mul, (unsigned)((n + 255) / 256), 256, 0, st, P, S, part_stride, gsz, M, ff, A, A_lo);
  return hipGetLastError();
}

// ---- context append ------------------------------------------------------------------------
// the batched append's setup: thread r finds its sequence by the row offsets (at most
// MAX_BANDS); the single-sequence append's setup is done by its row kernel (below)
__global__ __launch_bounds__(256) void k_append_batch_setup(AppendBatchArgs a, int* __restrict__ bt,
                                                            long long* __restrict__ slots,
                                                            int* __restrict__ rowpos,
                                                            int* __restrict__ kpos) {
  for (int j = threadIdx.x; j < a.n_upd; j += 256) bt[a.upd_off[j]] = a.upd_page[j];
  for (int r = threadIdx.x; r < a.n_rows; r += 256) {
    int b = 0;
    while (b + 1 < a.n_seqs && r >= a.row0[b + 1]) ++b;
    const int p = a.kv_len[b] + r - a.row0[b];
    const long long slot = (long long)a.pages[a.pg0[b] + (p >> 4) - a.lp0[b]] * PAGE + (p & (PAGE - 1));
    const int pos = a.positions ? a.positions[r] : p;
    slots[r] = slot;
    rowpos[r] = pos;
    kpos[slot] = pos;
  }
}

hipError_t launch_append_batch_setup(const AppendBatchArgs& a, int* bt, long long* slots, int* rowpos,
                                     int* kpos, hipStream_t st) {
  if (a.n_seqs < 1 || a.n_seqs > MAX_BANDS || a.n_rows < 1 || a.n_rows > APPEND_BATCH_ROWS) return hipErrorInvalidValue;
  (void)launch(k_append_batch_setup, 1, 256, 0, st, a, bt, slots, rowpos, kpos);
  return hipGetLastError();
}

// The single-sequence append's setup, done by the row kernel (SETUP): row r's slot
// (pages[logical page] * 16 + position % 16, positions kv_len + r onwards in the cache) and
// stamped position (the caller's, else kv_len + r), written into slots, rowpos and the pool's
// kpos; workgroup 0 also writes the new block-table entries.
struct RowsSetup {
  AppendArgs a;
  int* bt;
  long long* slots;
  int* rowpos;
  int* kpos;
};

// one workgroup per row: the sum of the row's S split-K partials, RMSNorm'd; optionally the
// row's RoPE (cos, sin) pairs for the fused K/V epilogue (one thread per pair), and (SETUP)
// the append's slots, positions and block tables
template <bool SETUP>
__global__ __launch_bounds__(1024) void k_rows_rmsnorm(const float* __restrict__ X, int S, long long ps,
                                                       int gsz, int h, const bf16* __restrict__ w, float eps,
                                                       bf16* __restrict__ out,
                                                       bf16* __restrict__ out_lo,
                                                       const int* __restrict__ rowpos,
                                                       const double* __restrict__ inv_freq, int half,
                                                       float2* __restrict__ cs,
                                                       std::conditional_t<SETUP, RowsSetup, int> su) {
  __shared__ __attribute__((aligned(16))) float xs[RN_HMAX];
  __shared__ float red_ss[16];
  const int r = blockIdx.x;
  int pos = 0;
  if constexpr (SETUP) {
    const AppendArgs& a = su.a;
    if (r == 0)
      for (int j = threadIdx.x; j < a.n_upd; j += blockDim.x) su.bt[a.upd_off[j]] = a.upd_page[j];
    const int p = a.kv_len + r;
    const long long slot = (long long)a.pages[(p >> 4) - a.first_lpage] * PAGE + (p & (PAGE - 1));
    pos = a.positions ? a.positions[r] : p;
    if (threadIdx.x == 0) {
      su.slots[r] = slot;
      su.rowpos[r] = pos;
      su.kpos[slot] = pos;
    }
  } else {
    if (cs) pos = rowpos[r];
  }
  const float tot = rows_gather(nullptr, X + (size_t)r * h, S, ps, gsz, h, xs, red_ss);
  const float rs = rsqrtf(tot / (float)h + eps);
  norm_out(xs, h, rs, w, out + (size_t)r * h, out_lo + (size_t)r * h);
  // the angles last: their double-precision sincos would otherwise hold the row's loads
  // (and every other wave, at the gather's barrier) behind it
  if (cs && (int)threadIdx.x < half) {
    double sn, cn;
    sincos((double)pos * inv_freq[threadIdx.x], &sn, &cn);
    cs[(size_t)r * half + threadIdx.x] = make_float2((float)cn, (float)sn);
  }
}

hipError_t launch_rows_rmsnorm(const float* X, int S, long long part_stride, int gsz, int M, int h,
                               const bf16* w, float eps, bf16* out, bf16* out_lo, hipStream_t st,
                               const int* rowpos, const double* inv_freq, int half, float2* cs,
                               const AppendArgs* setup, int* bt, long long* slots, int* rowpos_out, int* kpos) {
  if (h > RN_HMAX || h % 4 || gsz < 1) return hipErrorInvalidValue;
  if (cs && (!inv_freq || half < 1 || half > (int)rn_threads(h) || (!setup && !rowpos))) return hipErrorInvalidValue;
  if (setup) {
    if (setup->n != M || !bt || !slots || !rowpos_out || !kpos) return hipErrorInvalidValue;
    const RowsSetup su{*setup, bt, slots, rowpos_out, kpos};
    (void)launch(k_rows_rmsnorm<true>, M, rn_threads(h), 0, st, X, S, part_stride, gsz, h, w, eps, out, out_lo,
                 rowpos, inv_freq, half, cs, su);
  } else {
    (void)launch(k_rows_rmsnorm<false>, M, rn_threads(h), 0, st, X, S, part_stride, gsz, h, w, eps, out, out_lo,
                 rowpos, inv_freq, half, cs, 0);
  }
  return hipGetLastError();
}

// one workgroup per (16 rows, layer, K|V, KH kv heads) of the fused [K0 | V0 | K1 | V1 | ...]
// output (16 waves), every load of the workgroup issued before any is used (KH = 4 for long
// appends; 1 for short ones, which need the workgroups more). K: a wave per row (sum of the
// split partials, k-norm over the head, RoPE with the row's angles taken once for its KH
// heads), written along the page's [key][d] rows. V: the rows staged in LDS, then written
// along the page's [d][key] rows, consecutive threads on consecutive keys of one dim.
template <int HD, int KH>
__global__ __launch_bounds__(1024) void k_kv_append_post(const float* __restrict__ KV, int S,
                                                         long long ps, int gsz, int n, int L,
                                                         const bf16* __restrict__ kn_all, float eps,
                                                         const double* __restrict__ inv_freq, float mscale,
                                                         const long long* __restrict__ slots,
                                                         const int* __restrict__ rowpos, KvGeom g) {
  constexpr int H2 = HD / 2;
  __shared__ float vt[KH][16][HD + 1];
  const int r0 = blockIdx.x * 16;
  const int nkv = g.nkv, nq = (nkv + KH - 1) / KH;
  const int layer = blockIdx.y / (2 * nq), rem = blockIdx.y % (2 * nq);
  const int kv = rem / nq, h0 = (rem % nq) * KH;
  const int nhh = min(KH, nkv - h0);
  const int nr = min(16, n - r0);
  const size_t ld = (size_t)L * 2 * nkv * HD;
  const size_t col0 = ((size_t)(layer * 2 + kv) * nkv + h0) * HD;   // head h0's first column
  const size_t pl = page_layer_elems(nkv, HD);
  if (kv == 0) {
    const int i = threadIdx.x >> 6, l = threadIdx.x & 63;
    const bool act = l < H2;
    if (i >= nr) return;
    const int r = r0 + i;
    const float* src = KV + (size_t)r * ld + col0;
    float x1[KH], x2[KH];
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      const bool on = act && h < nhh;
      x1[h] = on ? sum_splits<8, float>(src + h * HD + l, S, ps, gsz) : 0.f;
      x2[h] = on ? sum_splits<8, float>(src + h * HD + l + H2, S, ps, gsz) : 0.f;
    }
    // the pair's angle in double precision (positions reach tens of thousands)
    float cf = 0.f, sf = 0.f;
    if (act) {
      double sn, cn;
      sincos((double)rowpos[r] * inv_freq[l], &sn, &cn);
      cf = (float)cn;
      sf = (float)sn;
    }
    const long long slot = slots[r];
    bf16* kpg = g.pool + ((size_t)layer * g.num_pages + (slot >> 4)) * pl + (int)(slot & (PAGE - 1)) * HD;
    const bf16* wn = kn_all + (size_t)layer * HD;
    const float w1 = act ? bf2f(wn[l]) : 0.f, w2 = act ? bf2f(wn[l + H2]) : 0.f;
#pragma unroll
    for (int h = 0; h < KH; ++h) {
      if (h >= nhh) break;
      const float ss = wave_sum(x1[h] * x1[h] + x2[h] * x2[h]);
      const float rs = rsqrtf(ss / (float)HD + eps);
      if (!act) continue;
      const float a = x1[h] * (rs * w1), b = x2[h] * (rs * w2);
      const float y1 = a * cf - b * sf;
      const float y2 = b * cf + a * sf;
      bf16* k = kpg + (size_t)(h0 + h) * PAGE * HD;
      k[l] = f2bf(y1 * mscale);
      k[l + H2] = f2bf(y2 * mscale);
    }
    return;
  }
  constexpr int NE = KH * 16 * HD;
  constexpr int NU = (NE + 1023) / 1024;   // elements per thread
  // every load first (one round trip), then the LDS stores
  float tv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int e = threadIdx.x + u * 1024;
    const int h = e / (16 * HD), i = (e / HD) % 16, d = e % HD;
    tv[u] = e < NE && h < nhh && i < nr
                ? sum_splits<8, float>(KV + (size_t)(r0 + i) * ld + col0 + (size_t)h * HD + d, S, ps, gsz)
                : 0.f;
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int e = threadIdx.x + u * 1024;
    if (e < NE) vt[e / (16 * HD)][(e / HD) % 16][e % HD] = tv[u];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NE; e += 1024) {
    const int h = e / (16 * HD), d = (e / 16) % HD, i = e % 16;
    if (h >= nhh || i >= nr) continue;
    const long long slot = slots[r0 + i];
    bf16* v = g.pool + ((size_t)layer * g.num_pages + (slot >> 4)) * pl + (size_t)(nkv + h0 + h) * HD * PAGE +
              (size_t)d * PAGE + (int)(slot & (PAGE - 1));
    *v = f2bf(vt[h][i][d]);
  }
}

hipError_t launch_kv_append_post(const float* KV, int S, long long part_stride, int gsz, int n, int L,
                                 const bf16* k_norm_all, float eps, const double* inv_freq, float mscale,
                                 const long long* slots, const int* rowpos, KvGeom g, hipStream_t st) {
  if (gsz < 1) return hipErrorInvalidValue;
  if (n < 1) return hipErrorInvalidValue;
  // four kv heads a workgroup once a launch has enough rows to fill the chip without them
  const bool wide = n >= 256;
  const int kh = wide ? 4 : 1;
  dim3 grid((n + 15) / 16, L * 2 * ((g.nkv + kh - 1) / kh));
#define DFL_POST(HDV, KHV) (void)launch(k_kv_append_post<HDV, KHV>, grid, 1024, 0, st, KV, S, part_stride, gsz, n, L, k_norm_all, eps, inv_freq, mscale, slots, rowpos, g)
  switch (g.hd) {
    case 32: if (wide) DFL_POST(32, 4); else DFL_POST(32, 1); break;
    case 64: if (wide) DFL_POST(64, 4); else DFL_POST(64, 1); break;
    case 128: if (wide) DFL_POST(128, 4); else DFL_POST(128, 1); break;
    default: return hipErrorInvalidValue;
  }
#undef DFL_POST
  return hipGetLastError();
}

}  // namespace dfl
