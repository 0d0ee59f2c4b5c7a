// Launch interface between the host runtime and the gfx950 kernels. Every launcher
// enqueues on `st` and returns hipGetLastError().
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

// Start/stop events the next launches attach to their own dispatch packets (so they time the
// kernel alone, as a profiler's kernel trace does); both null when timing is off.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

template <typename... KA, typename... A>
inline hipError_t launch(void (*k)(KA...), dim3 grid, dim3 block, size_t shmem, hipStream_t st,
                         A... args) {
  const LaunchEvents& e = launch_events();
  hipExtLaunchKernelGGL(k, grid, block, (uint32_t)shmem, st, e.start, e.stop, 0u, args...);
  return hipGetLastError();
}

typedef uint16_t bf16;

constexpr int PAGE = 16;          // tokens per KV page
constexpr int MAX_BANDS = 32;     // sequences in one forward call
constexpr int APPEND_ROWS = 2048; // context rows per append launch sequence
constexpr int APPEND_PAGES = APPEND_ROWS / PAGE + 1;

// T16 weight layout (the forward's GEMMs and the lm_head): the rows of a [N, K] weight go
// in tiles of 16; a tile's K is a run of 256-deep blocks, and a block holds its 16 x 256
// values as 8 x 64 16-byte pieces in exactly the order the 64 lanes of a wavefront load them
// (piece (u, lane) = row lane%16, k = u*32 + (lane/16)*8 .. +7). A tile is then 16*K
// contiguous values, and every load instruction of a wavefront reads 1 KB in one run.
constexpr int T16_BLOCK = 16 * 256;

// FP8 weights: OCP E4M3 codes with one fp32 scale per row (weight = code value x scale), in
// the T16-FP8 layout: the rows go in tiles of 16, a tile's K in 256-deep blocks of 4 KB, and a
// block holds 4 x 64 16-byte pieces in the order the lanes load them: piece (q, lane) is row
// lane % 16, the 8 codes of k = 64q + 8g .. (the lane's operand of 32-deep step 2q, g = lane/16)
// followed by the 8 codes of k = 64q + 32 + 8g .. (step 2q + 1).
constexpr int T16Q_BLOCK = 16 * 256;   // bytes of one 256-deep block of a tile

// One band (sequence) of a forward call, as the kernels see it.
struct Band {
  int seq;       // sequence slot
  int kv_len;    // context rows already cached (C)
  int q_pos;     // RoPE position of block row 0 (P)
  int bonus;     // token of block row 0
  int pg[2];     // physical pages of logical pages C/16 and C/16 + 1
  // split-KV work of full-attention and of sliding-window layers: keys from kstart
  // (page aligned) to C + gamma, `nch` chunks of `ck` keys, partial slots from `base`
  int kstart[2], ck[2], nch[2], base[2];
};

// A GEMM activation under an RMSNorm whose per-row scale is applied to the result: the
// activation operand (A, A_lo) holds x * w, and row r of the result is multiplied by
// rs[r] = 1/sqrt(sum_j ssq[r][j] / h + eps), where ssq[r][j] is the sum of squares of
// columns [256j, 256j + 256) of the residual row x (written by the producer with x * w).
// ssq rows are SSQ_STRIDE floats; entries past h/256 stay zero (h <= 8192).
constexpr int SSQ_COLS = 256;
constexpr int SSQ_STRIDE = 32;
struct NormIn {
  const float* ssq;
  float eps;
  int h;
};

// the band table of one forward, passed by value to the kernels that need it at their start
// The bands of an attention launch (the call's bands, in call order) and the path each takes.
struct AttnBands {
  int n;
  unsigned lds_mask;      // bit b: band b stages its K/V through LDS
  int dbase[MAX_BANDS];   // the band's first chunk among its path's chunks
  // the LDS path's chunks in dispatch order, longest first, as runs of equal-length chunks
  // (a band's full chunks, then its last one): run g holds dispatch positions
  // lg_start[g] .. lg_start[g + 1] - 1, chunks lg_chunk[g], lg_chunk[g] + 1, ... of band lg_band[g]
  int n_lg;
  unsigned short lg_start[2 * MAX_BANDS + 1];
  unsigned char lg_band[2 * MAX_BANDS], lg_chunk[2 * MAX_BANDS];
  Band b[MAX_BANDS];
};

struct FwdArgs {
  int n_bands, gamma, mask_token, per_seq;
  int n_upd;                   // block-table entries to write: bt[upd_off] = upd_page
  int upd_off[2 * MAX_BANDS];
  int upd_page[2 * MAX_BANDS];
  Band bands[MAX_BANDS];
};

struct AppendArgs {
  int seq, kv_len, n, per_seq;
  int first_lpage, n_lpages;   // logical pages touched by rows kv_len..kv_len+n-1
  int pages[APPEND_PAGES];     // their physical pages
  int n_upd;
  int upd_off[APPEND_PAGES];
  int upd_page[APPEND_PAGES];
  const int* positions;        // device int32 [n] or nullptr (kv_len + r)
};

// A batched append: new rows of up to MAX_BANDS sequences in one pass, seq-major (rows
// row0[b] .. row0[b+1]-1 belong to sequence seq[b] and go to its positions kv_len[b] ...).
constexpr int APPEND_BATCH_ROWS = 256;
constexpr int APPEND_BATCH_PAGES = APPEND_BATCH_ROWS / PAGE + 2 * MAX_BANDS;
struct AppendBatchArgs {
  int n_seqs, n_rows, per_seq;
  int seq[MAX_BANDS], kv_len[MAX_BANDS], row0[MAX_BANDS + 1];
  int lp0[MAX_BANDS];            // first logical page the sequence's rows touch
  int pg0[MAX_BANDS];            // where that page's physical id sits in pages[]
  int pages[APPEND_BATCH_PAGES];
  int n_upd;                     // block-table entries to write: bt[upd_off] = upd_page
  int upd_off[APPEND_BATCH_PAGES];
  int upd_page[APPEND_BATCH_PAGES];
  const int* positions;          // device int32 [n_rows] or nullptr (kv_len[b] + i)
};

// Geometry the attention / writeback kernels need.
struct KvGeom {
  bf16* pool;        // [L][num_pages][2][nkv] x (K [16][hd] | V [hd][16])
  int* kpos;         // [num_pages * 16]
  int* bt;           // [max_batch][per_seq]
  long long num_pages;
  int nkv, hd, per_seq;
};

__host__ __device__ inline size_t page_layer_elems(int nkv, int hd) { return (size_t)2 * nkv * PAGE * hd; }

// ---- GEMMs (k_gemm.hip, k_gemm_wide.hip, k_gemm_tiled.hip) ----------------------------
// Y[M,N] = A[M,K] W[N,K]^T where the activation A = A_hi + A_lo is carried as two bf16
// terms (each k-step issues two MFMAs). Skinny form: partials P[s][M][N] over K splits of
// k_len (k_len, K multiples of 256); M <= 64 per launch. W is row-major, or (w_tiled) in the
// T16 layout, which needs k_len 256 and N a multiple of 16.
// wsc: W holds FP8 codes in the T16-FP8 layout with these per-row scales (w_tiled, A_lo required)
hipError_t launch_gemm_skinny(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W,
                              int N, int K, int k_len, float* P, long long part_stride, bool w_tiled,
                              hipStream_t st, const NormIn* norm = nullptr, const float* wsc = nullptr);
// Wide form for more than 64 rows (A_lo optional: without it A is exact bf16; W in the T16
// layout, K a multiple of 256, N of 16): partials P[z][M][N] (z < gemm_wide_groups(K, gsz), stride part_stride),
// each the sum of the 256-deep split chains of group z (splits z*gsz .. z*gsz + gsz - 1)
// as the consumers' canonical order forms it from the skinny kernel's per-split partials.
int gemm_wide_groups(int K, int gsz);
hipError_t launch_gemm_wide(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W, int N, int K,
                            int gsz, float* P, long long part_stride, hipStream_t st,
                            const NormIn* norm = nullptr, const float* wsc = nullptr);
// Quantize a row-major [N, K] bf16 weight to OCP FP8 E4M3 codes in the T16-FP8 layout
// (ceil(N/16)*16 rows of K bytes, padding rows zero) with per-row scales max|w| / 448
// (1 for an all-zero row; padding rows 1): codes = nearest E4M3 of w / scale, ties to even,
// saturating at +-448. K a multiple of 256.
hipError_t launch_quant_fp8(const bf16* src, int N, int K, uint8_t* dst, float* scale, hipStream_t st);
// Copy a row-major [N, K] bf16 weight into the T16 layout (ceil(N/16)*16 rows, the padding
// rows zero); K a multiple of 256.
hipError_t launch_tile_weight(const bf16* src, int N, int K, bf16* dst, hipStream_t st);
// Tiled form for large M: ks k splits (gemm_tiled_splits(N, K)), split z's fp32 result in
// C + z*M*ldc ([M, N], row stride ldc); K a multiple of 32*ks; A_lo may be null (A exact).
int gemm_tiled_splits(int N, int K);
hipError_t launch_gemm_tiled(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W,
                             int N, int K, int ks, float* C, int ldc, hipStream_t st);
// The append's fused K/V GEMM with k_norm, RoPE and the page writes in its epilogue (one k
// split, whatever gemm_tiled_splits says): N = L * 2 * nkv * hd ([K0 | V0 | K1 | V1 | ...]),
// nkv * hd a multiple of 256, hd 32, 64 or 128. Row r of A goes to pool slot slots[r]; cs holds
// the rows' RoPE (cos, sin) pairs, float2 [M][hd / 2]. Per element the arithmetic of
// launch_kv_append_post on a one-split launch_gemm_tiled result, except the order in which a
// head's squares are summed for the k_norm.
bool gemm_tiled_kv_fusable(int N, int nkv, int hd);
hipError_t launch_gemm_tiled_kv(const bf16* A, const bf16* A_lo, int lda, int M, const bf16* W, int N, int K,
                                const bf16* k_norm_all, float eps, float mscale, const long long* slots,
                                const float2* cs, KvGeom g, hipStream_t st);
// lm_head (W in the T16 layout) + argmax partials: for rows r0..r0+M-1 of the forward (M <= 64), best (value,
// index) per row over each workgroup's vocabulary range; optionally the fp32 logits of
// drafted rows (row % gamma != 0) into logits[(r/gamma)*(gamma-1) + r%gamma - 1][V].
int lmhead_groups(int V);
// The persistent lm_head (<= 16 rows, K <= 2048, W in the T16 layout): its number of
// workgroups = argmax partials per row (0 when the shape does not qualify).
int lmhead_persistent_groups(int V, int K, int M, int n_cu);
hipError_t launch_lmhead_persistent(const bf16* Y, const bf16* Y_lo, int ldy, int M, int r0, const bf16* W,
                                    int V, int K, float* best_v, int* best_i, int n_groups, int gamma,
                                    float* logits, hipStream_t st, const float* wsc = nullptr);
// The wide lm_head (any row count, rows 0..M-1 of the forward; W in the T16 layout): one
// argmax partial per (row, 128-column group); n_groups = lmhead_wide_groups(V).
int lmhead_wide_groups(int V);
hipError_t launch_lmhead_wide(const bf16* Y, const bf16* Y_lo, int ldy, int M, const bf16* W, int V, int K,
                              float* best_v, int* best_i, int n_groups, int gamma, float* logits,
                              hipStream_t st, const float* wsc = nullptr);
hipError_t launch_lmhead_argmax(const bf16* Y, const bf16* Y_lo, int ldy, int M, int r0, const bf16* W, int V,
                                int K, float* best_v, int* best_i, int n_groups, int gamma,
                                float* logits, hipStream_t st);
hipError_t launch_argmax_reduce(const float* best_v, const int* best_i, int n_groups,
                                int n_bands, int gamma, int* tokens, hipStream_t st);

// ---- forward elementwise (k_misc.hip) ------------------------------------------------
// The consumers of the forward's GEMM partials take (P, S, part_stride, gsz) and add the S
// partials in the canonical order of sum_splits: groups of gsz splits, each in split order
// from zero, then the group sums in group order from zero.
// block tables, slots, band table; X = the block rows' embeddings, their slice sums of
// squares ssq [rows][h/256], and X * w_in0 as hi + lo bf16 (Xw, Xw_lo)
hipError_t launch_fwd_prologue(const FwdArgs& a, Band* bands_dev, int* bt, long long* slots,
                               int* kpos, const bf16* embed, const bf16* w_in0, int h, float* X,
                               float* ssq, bf16* Xw, bf16* Xw_lo, hipStream_t st);
hipError_t launch_qkv_post(const float* P, int S, long long part_stride, int gsz, int M, int gamma,
                           const Band* bands_dev, int nh, int nkv, int hd, const bf16* q_norm,
                           const bf16* k_norm, float eps, const double* inv_freq, float mscale,
                           const long long* slots, KvGeom g, int layer, bf16* Q, bf16* Q_lo,
                           hipStream_t st);
hipError_t launch_resid_norm(float* X, const float* P, int S, long long part_stride, int gsz, int M,
                             int h, const bf16* w, float eps, bf16* Xn, bf16* Xn_lo,
                             hipStream_t st);
// X[r] += sum_s P[s][r] (canonical order); the slice sums of squares of the new rows and
// X * w as hi + lo bf16 (w: the norm weight of the GEMM that consumes them)
hipError_t launch_resid_sum(float* X, const float* P, int S, long long part_stride, int gsz, int M, int h,
                            const bf16* w, float* ssq, bf16* Xw, bf16* Xw_lo, hipStream_t st);
hipError_t launch_silu_mul(const float* P, int S, long long part_stride, int gsz, int M, int ff,
                           bf16* A, bf16* A_lo, hipStream_t st);

// ---- attention (k_attn.hip) ----------------------------------------------------------
// A chunk (one workgroup's keys) spans at most this many pages; the runtime's chunk plan
// keeps to it (sequences of at most 16 * 16384 keys).
constexpr int ATTN_CHUNK_PAGES_MAX = 512;
// The attention of one layer is one launch whose bands take one of two paths, chosen by a
// property of each band alone (so a band's arithmetic never depends on the other bands of
// the call): with the LDS path enabled (a property of the drafter, fixed at create), bands
// of more than ATTN_LDS_MIN_PAGES pages (2048 keys) on a head_dim-128 layer without a window
// stream K/V through LDS, planned in at most 12 chunks; the rest load K/V straight into
// registers. plan_attn fills the table and counts each path's chunks; partials stay indexed
// by the call-wide chunk numbering (Band::base), sized [sum of nch * nkv][128][hd].
constexpr int ATTN_LDS_MIN_PAGES = 128;
// query-row slots of one (chunk, kv head) partial: part_o [items][ATTN_PART_ROWS][hd] and
// part_ml [items][ATTN_PART_ROWS][2] for items = (chunks of the call) * nkv
constexpr int ATTN_PART_ROWS = 128;
void plan_attn(const Band* bands, int n, int sw, int hd, int window, bool lds_path, int gamma, AttnBands& out,
               int& reg_chunks, int& lds_chunks);
hipError_t launch_block_attn(const bf16* Q, const bf16* Q_lo, const AttnBands& bands, int reg_chunks, int lds_chunks,
                             int gamma, int nh, KvGeom g, int layer, int sw, int window,
                             float scale_log2, float* part_o, float* part_ml, hipStream_t st);
hipError_t launch_attn_combine(const float* part_o, const float* part_ml, const Band* bands_dev,
                               int n_bands, int max_nch, int gamma, int nh, int nkv, int hd, int sw,
                               bf16* out, bf16* out_lo, hipStream_t st);

// ---- context append (k_misc.hip) -----------------------------------------------------
hipError_t launch_append_batch_setup(const AppendBatchArgs& a, int* bt, long long* slots, int* rowpos,
                                     int* kpos, hipStream_t st);
// inputs are split-K partials X[s][M][...] added in the canonical order (S = 1, gsz = 1 for a
// plain result). With cs non-null, row r also writes its RoPE (cos, sin) pairs at position
// rowpos[r] into cs[r][0..half) (angles in double precision, then rounded to float). With
// setup non-null (M = setup->n), the launch also does the single-sequence append's setup for
// those rows (their slots, stamped positions and the new block-table entries into slots,
// rowpos_out, kpos and bt), and the angles use the positions it stamps.
hipError_t launch_rows_rmsnorm(const float* X, int S, long long part_stride, int gsz, int M, int h,
                               const bf16* w, float eps, bf16* out, bf16* out_lo, hipStream_t st,
                               const int* rowpos = nullptr, const double* inv_freq = nullptr, int half = 0,
                               float2* cs = nullptr, const AppendArgs* setup = nullptr, int* bt = nullptr,
                               long long* slots = nullptr, int* rowpos_out = nullptr, int* kpos = nullptr);
hipError_t launch_kv_append_post(const float* KV, int S, long long part_stride, int gsz, int n, int L,
                                 const bf16* k_norm_all, float eps, const double* inv_freq, float mscale,
                                 const long long* slots, const int* rowpos, KvGeom g, hipStream_t st);

// ---- DSpark Markov chain (k_markov.hip) -----------------------------------------------
// One drafted row k of every band: logits[b*(gamma-1)+k][:] += W2 @ W1[t], t = bonus[b] for
// k = 0 and row k-1's draft otherwise; the row's argmax goes into key best[k][b] (a 64-bit
// atomic max). k_markov_finish then writes tokens[b*(gamma-1)+k] for every row and clears
// the keys (they are zero before the first step of a forward).
constexpr int MARKOV_MAX_GROUPS = 1024;
constexpr int MARKOV_MAX_ROWS = 15;   // gamma_max - 1
struct MarkovStep {
  const bf16* w1;              // [V, R] previous-token table (the caller's, row-major)
  const bf16* w2t;             // W2 [V, R] in the T16 layout (rows padded to whole tiles)
  float* logits;               // [n*(gamma-1), V] the lm_head's logits, biased in place when store
  unsigned long long* best;    // [MARKOV_MAX_ROWS][MAX_BANDS] argmax keys
  int V, R, n, gamma, k, store;
  int bonus[MAX_BANDS];
};
int markov_step_groups(int V, int n_cu);
hipError_t launch_markov_step(const MarkovStep& a, int groups, hipStream_t st);
hipError_t launch_markov_finish(unsigned long long* best, int n, int gamma, int* tokens, hipStream_t st);


// ---- DFlash2 (k_dflash2.hip) -------------------------------------------------------------
// grouped dynamic causal convs: two taps, 16-channel groups; the projection's columns are
// [application 2][tap 2][group h/16]. Rows of a band are consecutive (band b = rows
// b*gamma .. b*gamma+gamma-1); tap 1 reads the band's previous row.
hipError_t launch_dconv_prepare(const bf16* Xw, const bf16* Xw_lo, const float* ssq, float eps, int M, int h,
                                int gamma, const float* P, int S, long long part_stride, int gsz, const bf16* base,
                                float* dyn, bf16* U, bf16* U_lo, hipStream_t st);
hipError_t launch_resid_dconv(float* X, const float* P, int S, long long part_stride, int gsz, int M, int h, int gamma,
                              const float* dyn, const bf16* base, const bf16* w, float* ssq, bf16* Xw, bf16* Xw_lo,
                              hipStream_t st);
// top-16 candidates per drafted row: sliced partial lists (cv, ci: [rows][slices][16], at most
// 16 slices), merged (best first, ties to the lower index) by the selector's pair kernel
constexpr int TOPK_MAX_SLICES = 16;
constexpr int MAX_GAMMA = 16;
int topk_slices(int V);
hipError_t launch_topk_partial(const float* logits, int rows, int V, float* cv, int* ci, hipStream_t st);
// the candidate selector: each drafted row's 16 candidates into sel_v, sel_i [rows][16], pair
// scores [rows][16 prev][16 cand], then the greedy walk per band
constexpr int SELECTOR_MAX_RANK = 512;
struct SelectorBonus {
  int t[MAX_BANDS];
};
hipError_t launch_selector_pairs(const float* cv, const int* ci, const float* Hp, int S, long long part_stride, int gsz,
                                 int rank, int n_bands, int gamma, const SelectorBonus& bonus, const bf16* pred,
                                 const bf16* succ, int vocab, float* sel_v, int* sel_i, float* pair, hipStream_t st);
hipError_t launch_selector_walk(const int* sel_i, const float* pair, int n_bands, int gamma, int* tokens,
                                hipStream_t st);

}  // namespace dfl
