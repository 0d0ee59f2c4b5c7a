// Host runtime behind include/dflash.h: configuration checks, the paged KV pool and its
// free list, block tables, scratch, the fused weight copies, and the launch sequences of
// the context append and of the gamma-block forward. One stream per call, no host sync
// inside a call, no environment reads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.hpp"

using namespace dfl;

// Scratch of dflash_block_forward_noalloc: the forward's partials when the caller cannot
// allocate. In host code `scratch` is only a stand-in for the symbol: its device address on
// each device comes from hipGetSymbolAddress (scratch_setup), and only that address is used.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)DFLASH_NOALLOC_SCRATCH_MB << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int RING = 8;          // staging slots for caller-stamped append positions
constexpr int ROW_GROUP = 64;    // rows per skinny-GEMM launch
constexpr int APPEND_SKINNY = 64; // appends of up to this many rows stream their weights once

struct LayerDev {
  const bf16 *q_norm, *k_norm;
  bf16 *in_norm, *post_norm;   // owned copies (16-byte aligned: the GEMM staging reads them whole)
  // owned T16 copies of the forward's weights: fused [q;k;v], fused [gate;up], o, down
  bf16 *w_qkv, *w_gu, *o_proj, *down_proj;
  // FP8 weights instead (weight_format 1): T16-FP8 codes and per-row scales of the same four
  uint8_t *q_qkv, *q_gu, *q_o, *q_down;
  float *s_qkv, *s_gu, *s_o, *s_down;
  // DFlash2: the two conv sites' base kernels (the caller's) and T16 copies of their projections
  const bf16 *cba = nullptr, *cbm = nullptr;
  bf16 *w_cpa = nullptr, *w_cpm = nullptr;
};

// The pool's free list: a ring of page ids sized once at create, so that taking and returning
// pages never allocates
struct FreeList {
  std::vector<int> ring;
  size_t head = 0, count = 0;
  void init(size_t cap) { ring.assign(std::max<size_t>(cap, 1), 0); head = count = 0; }
  size_t size() const { return count; }
  int front() const { return ring[head]; }
  void pop_front() { head = (head + 1) % ring.size(); --count; }
  void push_back(int p) { ring[(head + count) % ring.size()] = p; ++count; }
};

struct SeqState {
  std::vector<int> bt;   // physical page of each logical page
  std::vector<int> pos;  // stamped position of every cached context row
  int kv_len = 0;
};

// A forward GEMM: K splits of klen, added by the consumers in groups of gsz splits
struct GemmPlan { int N, K, klen, S, gsz; };

}  // namespace

struct dflash_ctx {
  // configuration
  int L, h, nh, nkv, hd, qd, kvd, ff, V, T, Ht, gmax, mask, max_seq, max_batch;
  float eps;
  int rope_type, window;
  std::vector<uint8_t> sliding;
  double mscale = 1.0;
  long long num_pages;
  int per_seq;
  int m_max;
  // weights
  const bf16 *fc, *hidden_norm, *norm, *embed;
  bf16* lm_head = nullptr;   // owned T16 copy, vocab padded to whole tiles
  bool fp8 = false;          // weight_format 1: FP8 E4M3 forward weights and lm_head
  uint8_t* lm_q = nullptr;   // FP8: T16-FP8 lm_head codes and per-row scales
  float* lm_s = nullptr;
  // DSpark Markov head (markov_rank R > 0)
  int R = 0;
  const bf16* mk_w1 = nullptr;   // [V, R] previous-token table (the caller's)
  bf16* mk_w2t = nullptr;        // owned T16 copy of W2 [V, R]
  float* mk_logits = nullptr;    // [max_batch*(gamma_max-1), V] logits when the caller wants none
  unsigned long long* mk_best = nullptr;   // [MARKOV_MAX_ROWS][MAX_BANDS] argmax keys, zero between forwards
  int mk_groups = 1;
  // DFlash2 (selector_rank > 0): convs, top-16 candidates and the selector
  // bands past 2048 keys stream attention K/V through LDS (drafters made for 8 or more
  // sequences: one band alone fills the chip better with the register path, a crowd of them
  // reads less from L2 with this one; fixed at create, so no call's bands change another's
  // bits)
  bool attn_lds = false;
  bool d2 = false;
  int sel_rank = 0;
  const bf16 *sel_pred = nullptr, *sel_succ = nullptr;
  bf16* sel_h = nullptr;            // T16 copy of the hidden projection [rank, h]
  float *dyn_a = nullptr, *dyn_m = nullptr;   // [rows][h/4] dynamic taps of the two sites
  bf16 *U = nullptr, *U_lo = nullptr;         // convolved sublayer input, hi + lo
  float* tk_v = nullptr;            // [drafted rows][TOPK_MAX_SLICES][16] per-slice candidates
  int* tk_i = nullptr;
  float* sel_v = nullptr;           // [drafted rows][16] candidates and their logits
  int* sel_i = nullptr;
  float* sel_pair = nullptr;        // [drafted rows][16][16] pair scores
  GemmPlan g_cp{}, g_sh{};
  std::vector<LayerDev> layers;
  bf16* w_kv = nullptr;        // [L*2*kvd, h]: K0;V0;K1;V1;... (row-major, for the tiled GEMM)
  bf16* w_kv_t = nullptr;      // the same in the T16 layout (short appends)
  bf16* fc_t = nullptr;        // fc in the T16 layout (short appends)
  bf16* knorm_all = nullptr;   // [L, hd]
  double* inv_freq = nullptr;  // [hd/2]
  // pool and tables
  bf16* pool = nullptr;
  int* kpos = nullptr;
  int* bt_dev = nullptr;
  long long* slots = nullptr;
  int* rowpos = nullptr;
  Band* bands_dev = nullptr;
  // forward scratch
  float* X = nullptr;          // residual stream, fp32
  float* ssq = nullptr;        // [rows][SSQ_STRIDE] slice sums of squares of X (zero tail)
  bf16 *Xn = nullptr, *Xn_lo = nullptr;    // activations as hi + lo bf16 terms
  bf16 *Qb = nullptr, *Qb_lo = nullptr;
  bf16 *attn = nullptr, *attn_lo = nullptr;
  bf16 *act = nullptr, *act_lo = nullptr;
  float* part = nullptr;
  size_t part_elems = 0;
  float* aparts_o = nullptr;
  float* aparts_ml = nullptr;
  float* best_v = nullptr;
  int* best_i = nullptr;
  int lm_groups = 0;
  int n_cu = 1;               // compute units of the device the context was created on
  int dev = 0;                // that device
  GemmPlan g_qkv, g_o, g_gu, g_down, g_fc, g_kvapp;
  // append scratch
  float* F32 = nullptr;
  bf16 *Fb = nullptr, *Fb_lo = nullptr;
  float* KV32 = nullptr;       // the K/V GEMM's fp32 result where its epilogue cannot be fused
  float2* rope_cs = nullptr;   // [APPEND_ROWS][hd / 2] the appended rows' RoPE (cos, sin)
  bool kv_fused = false;       // long appends: the K/V GEMM writes the pages itself
  int* ring_host = nullptr;
  int* ring_dev = nullptr;
  hipEvent_t ring_ev[RING] = {};
  int ring_next = 0;
  // per-layer intermediates of the last forward (dflash_debug_capture): [L][m_max][width]
  bool cap_on = false;
  bf16 *cap_q = nullptr, *cap_q_lo = nullptr, *cap_a = nullptr, *cap_a_lo = nullptr;
  float *cap_x1 = nullptr, *cap_x = nullptr;
  // launch timing (opt-in per class)
  uint32_t tmask = 0;
  std::vector<hipEvent_t> tev;   // pairs (start, end)
  std::vector<int> tcls;         // class of each recorded pair
  double tms[DFLASH_K_NUM_CLASSES] = {};
  long long tcnt[DFLASH_K_NUM_CLASSES] = {};
  // host state
  std::vector<SeqState> seqs;
  FreeList free_pages;
  std::vector<void*> owned;
  char err[512] = {0};
  bool poisoned = false;
};

namespace {

int fail(dflash_ctx* c, int code, const char* fmt, ...) {
  if (c) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(c->err, sizeof c->err, fmt, ap);
    va_end(ap);
    if (code == DFLASH_EHIP) c->poisoned = true;
  }
  return code;
}

#define HIPCHK(c, expr)                                                                     \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail((c), DFLASH_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));        \
  } while (0)

template <class T>
int dalloc(dflash_ctx* c, T** p, size_t elems) {
  void* q = nullptr;
  const size_t bytes = std::max<size_t>(elems * sizeof(T), 256);
  hipError_t e = hipMalloc(&q, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(c, DFLASH_ENOMEM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  }
  c->owned.push_back(q);
  *p = static_cast<T*>(q);
  return DFLASH_OK;
}

GemmPlan plan_gemm(int N, int K) {
  // K splits of 256: each workgroup streams one 64-column x 256-deep weight tile, so even the
  // narrow projections launch several hundred workgroups and the whole matrix is in flight at
  // once. Depends on (N, K) only, never on the number of rows.
  const int klen = 256;
  const int S = (K + klen - 1) / klen;
  // splits per group of the consumers' canonical order: from (N, K) alone, so that the wide
  // kernel of a 256-row forward (2 row groups x ceil(N/128) column groups per split group)
  // has at least about a chip's worth (256) of workgroups; a divisor of S, so the groups match
  const int per_group = 2 * ((N + 127) / 128);
  const int want = std::max(1, (256 + per_group - 1) / per_group);
  int gsz = std::max(1, S / want);
  while (S % gsz) --gsz;
  return GemmPlan{N, K, klen, S, gsz};
}

int chunk_pages(int pages, bool lds) {
  // (pages <= 16384 by the config check, so a chunk never exceeds ATTN_CHUNK_PAGES_MAX)
  // 16 pages (256 keys: two passes of the attention workgroup's four 32-key wave slices) per
  // chunk, widened in steps of 16 pages so that a band never has more than 32 chunks: a
  // 4K-key band keeps every workgroup of a layer resident at once, long bands keep the
  // partial traffic and the merge bounded. Bands on the attention's LDS path (one workgroup
  // per chunk and kv head, not four) take at most 12 chunks, as long as a chunk's page ids
  // fit the workgroup's table: fewer partials and less merge work (12 ran the 16-band and the
  // long-context forwards faster than 16, 10 or 8)
  if (lds && pages > ATTN_LDS_MIN_PAGES) return std::min(ATTN_CHUNK_PAGES_MAX, 16 * ((pages + 191) / 192));
  return 16 * std::max(1, (pages + 511) / 512);
}

void plan_chunks(int kstart, int kend, bool lds, int& ck, int& nch) {
  const int pages = (kend - kstart + PAGE - 1) / PAGE;
  const int ckp = chunk_pages(pages, lds);
  nch = (pages + ckp - 1) / ckp;
  ck = ckp * PAGE;
}

int max_chunks(int pages_max) {
  int m = 1;
  // (the LDS path's plan never has more chunks than the register path's)
  for (int p = 1; p <= pages_max; ++p) m = std::max(m, (p + chunk_pages(p, false) - 1) / chunk_pages(p, false));
  return m;
}

bool sliding_layer(const dflash_ctx* c, int l) { return c->window > 0 && c->sliding[l]; }

constexpr size_t TIMING_PAIRS = 4096;

}  // namespace

namespace dfl {
LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}
}  // namespace dfl

namespace {

hipError_t timing_harvest(dflash_ctx* c) {
  const size_t n = c->tcls.size();
  if (n == 0) return hipSuccess;
  hipError_t e = hipEventSynchronize(c->tev[2 * n - 1]);
  if (e != hipSuccess) return e;
  for (size_t i = 0; i < n; ++i) {
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, c->tev[2 * i], c->tev[2 * i + 1]);
    if (e != hipSuccess) return e;
    c->tms[c->tcls[i]] += ms;
    c->tcnt[c->tcls[i]] += 1;
  }
  c->tcls.clear();
  return hipSuccess;
}

// run `launch` (one kernel launch on st); time it if its class is timed
template <class F>
hipError_t timed(dflash_ctx* c, int cls, hipStream_t st, F&& launch) {
  if (!((c->tmask >> cls) & 1u)) return launch();
  if (c->tcls.size() == TIMING_PAIRS) {
    hipError_t e = timing_harvest(c);
    if (e != hipSuccess) return e;
  }
  const size_t i = c->tcls.size();
  while (c->tev.size() < 2 * (i + 1)) {
    hipEvent_t ev;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return e;
    c->tev.push_back(ev);
  }
  // the events ride on the kernel's own dispatch: they time the kernel alone
  launch_events() = LaunchEvents{c->tev[2 * i], c->tev[2 * i + 1]};
  hipError_t e = launch();
  launch_events() = LaunchEvents{};
  if (e != hipSuccess) return e;
  c->tcls.push_back(cls);
  return hipSuccess;
}

KvGeom geom(dflash_ctx* c) {
  return KvGeom{c->pool, c->kpos, c->bt_dev, c->num_pages, c->nkv, c->hd, c->per_seq};
}

int check_config(const dflash_config* cfg, const dflash_weights* w, std::string& why) {
  auto bad = [&](const char* m) { why = m; return DFLASH_EINVAL; };
  if (!cfg || !w || !w->layers) return bad("NULL config or weights");
  if (cfg->num_layers <= 0 || cfg->hidden <= 0 || cfg->vocab <= 0 || cfg->num_taps <= 0 ||
      cfg->target_hidden <= 0 || cfg->intermediate <= 0)
    return bad("sizes must be positive");
  if (cfg->head_dim != 32 && cfg->head_dim != 64 && cfg->head_dim != 128)
    return bad("head_dim must be 32, 64 or 128");
  if (cfg->num_kv_heads <= 0 || cfg->num_q_heads % cfg->num_kv_heads != 0)
    return bad("num_q_heads must be a multiple of num_kv_heads");
  if (cfg->num_q_heads / cfg->num_kv_heads > 8) return bad("at most 8 query heads per kv head");
  if (cfg->gamma_max < 2 || cfg->gamma_max > 16) return bad("gamma_max must be in [2, 16]");
  if (cfg->hidden > 8192) return bad("hidden must be at most 8192");
  if (cfg->hidden % 256 || cfg->intermediate % 256 || (cfg->num_q_heads * cfg->head_dim) % 256 ||
      (cfg->num_taps * cfg->target_hidden) % 256)
    return bad("hidden, intermediate, q_dim and num_taps*target_hidden must be multiples of 256");
  if (cfg->mask_token_id < 0 || cfg->mask_token_id >= cfg->vocab) return bad("mask_token_id out of range");
  if (cfg->max_batch < 1 || cfg->max_batch > MAX_BANDS) return bad("max_batch must be in [1, 32]");
  // an attention chunk of the longest sequence must fit the kernel's page-id table
  if (cfg->max_seq_len < 1 || (long long)cfg->max_seq_len + cfg->gamma_max + 1 > 16LL * 16384)
    return bad("max_seq_len + gamma_max must be below 262144");
  if (!(cfg->rms_eps >= 0.f)) return bad("rms_eps must be >= 0");
  if (!(cfg->rope_theta > 1.0)) return bad("rope_theta must be > 1");
  if (cfg->rope_type != 0 && cfg->rope_type != 1) return bad("rope_type must be 0 or 1");
  if (cfg->weight_format != DFLASH_WEIGHTS_BF16 && cfg->weight_format != DFLASH_WEIGHTS_FP8_E4M3)
    return bad("weight_format must be DFLASH_WEIGHTS_BF16 or DFLASH_WEIGHTS_FP8_E4M3");
  if (cfg->markov_rank != 0 && cfg->markov_rank != 256 && cfg->markov_rank != 512)
    return bad("markov_rank must be 0, 256 or 512");
  if (cfg->markov_rank && (!w->markov_w1 || !w->markov_w2)) return bad("a Markov head needs markov_w1 and markov_w2");
  if (cfg->conv_kernel_size || cfg->conv_group_size || cfg->selector_rank || cfg->selector_top_k) {
    if (cfg->conv_kernel_size != 2 || cfg->conv_group_size != 16 || cfg->selector_top_k != 16 ||
        (cfg->selector_rank != 256 && cfg->selector_rank != 512))
      return bad("DFlash2 needs conv_kernel_size 2, conv_group_size 16, selector_top_k 16, selector_rank 256 or 512");
    if (cfg->markov_rank) return bad("a DFlash2 drafter has no Markov head");
    if (cfg->vocab < 16) return bad("DFlash2 needs a vocabulary of at least 16");
    if (!w->selector_pred || !w->selector_succ || !w->selector_hidden_proj) return bad("NULL selector weight");
    auto a16 = [](const void* p) { return p && ((uintptr_t)p & 15) == 0; };
    if (!a16(w->selector_pred) || !a16(w->selector_succ) || !a16(w->selector_hidden_proj))
      return bad("selector weights must be non-NULL and 16-byte aligned");
    for (int l = 0; l < cfg->num_layers; ++l) {
      const dflash_layer_weights& lw = w->layers[l];
      if (!a16(lw.attention_conv_base) || !a16(lw.attention_conv_proj) || !a16(lw.mlp_conv_base) ||
          !a16(lw.mlp_conv_proj))
        return bad("DFlash2 conv weights must be non-NULL and 16-byte aligned");
    }
  }
  if (cfg->rope_type == 1 && !(cfg->yarn_factor > 0 && cfg->yarn_orig_max_pos > 0 &&
                               cfg->yarn_beta_fast > 0 && cfg->yarn_beta_slow > 0))
    return bad("YaRN parameters must be positive");
  if (cfg->sliding_window < 0) return bad("sliding_window must be >= 0");
  if (cfg->num_pages != 0 && cfg->num_pages < 2) return bad("num_pages must be 0 or >= 2");
  if (!w->fc || !w->hidden_norm || !w->norm || !w->embed_tokens || !w->lm_head)
    return bad("NULL head weight");
  for (int l = 0; l < cfg->num_layers; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    if (!lw.q_proj || !lw.k_proj || !lw.v_proj || !lw.o_proj || !lw.q_norm || !lw.k_norm ||
        !lw.input_layernorm || !lw.post_attention_layernorm || !lw.gate_proj || !lw.up_proj ||
        !lw.down_proj)
      return bad("NULL layer weight");
  }
  // matrices are streamed with 16-byte loads
  auto a16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  if (!a16(w->fc) || !a16(w->embed_tokens) || !a16(w->lm_head)) return bad("head weight matrices must be 16-byte aligned");
  if (cfg->markov_rank && (!a16(w->markov_w1) || !a16(w->markov_w2))) return bad("Markov head tables must be 16-byte aligned");
  for (int l = 0; l < cfg->num_layers; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    if (!a16(lw.q_proj) || !a16(lw.k_proj) || !a16(lw.v_proj) || !a16(lw.o_proj) || !a16(lw.gate_proj) ||
        !a16(lw.up_proj) || !a16(lw.down_proj))
      return bad("layer weight matrices must be 16-byte aligned");
  }
  return DFLASH_OK;
}

// inverse frequencies, double precision: plain theta^(-2j/d), or the YaRN blend
// (memra_engine/dflash.rs, DflashDraft::load; spark_model/layers/dflash_head/
// from_weights.rs, from_weights: ramp from low to high pair index, plain frequency below,
// frequency / factor above; a zero-width ramp gets +0.001)
std::vector<double> inv_freq_table(const dflash_config* cfg, double* mscale) {
  const int hd = cfg->head_dim, half = hd / 2;
  const double base = cfg->rope_theta, d = hd;
  std::vector<double> f(half);
  for (int j = 0; j < half; ++j) f[j] = std::pow(base, -2.0 * j / d);
  *mscale = 1.0;
  if (cfg->rope_type == 1) {
    const double fac = cfg->yarn_factor, orig = cfg->yarn_orig_max_pos;
    auto corr = [&](double r) { return d * std::log(orig / (r * 2.0 * M_PI)) / (2.0 * std::log(base)); };
    const double low = std::max(std::floor(corr(cfg->yarn_beta_fast)), 0.0);
    const double high = std::min(std::ceil(corr(cfg->yarn_beta_slow)), d - 1.0);
    const double den = std::fabs(high - low) < 1e-6 ? high - low + 0.001 : high - low;
    for (int j = 0; j < half; ++j) {
      const double ramp = std::min(1.0, std::max(0.0, (j - low) / den));
      f[j] = (f[j] / fac) * ramp + f[j] * (1.0 - ramp);
    }
    *mscale = 0.1 * std::log(fac) + 1.0;
  }
  return f;
}

// The no-allocation forward's scratch on each device: every device the library runs on holds
// its own copy of `scratch` until the process ends; dflash_create looks its address up once
// per device, with that device current, and kernels get that address (g_scratch_ptr).
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

int scratch_setup(dflash_ctx* c) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (c->dev < 0 || c->dev >= MAX_DEVICES) return fail(c, DFLASH_EINVAL, "device %d beyond the library's %d", c->dev, MAX_DEVICES);
  if (g_scratch_ptr[c->dev]) return DFLASH_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p)
    return fail(c, DFLASH_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
  g_scratch_ptr[c->dev] = p;
  return DFLASH_OK;
}

void release(dflash_ctx* c) {
  if (!c) return;
  for (int i = 0; i < RING; ++i)
    if (c->ring_ev[i]) (void)hipEventDestroy(c->ring_ev[i]);
  if (c->ring_host) (void)hipHostFree(c->ring_host);
  for (hipEvent_t e : c->tev) (void)hipEventDestroy(e);
  for (void* p : c->owned) (void)hipFree(p);
  delete c;
}

}  // namespace

// fc + hidden_norm + the fused K/V GEMM + k_norm/RoPE/writeback for nc context rows. With
// setup, the row kernel after the fc GEMM first writes the rows' slots, positions and block
// tables (the fc GEMM needs none of them); otherwise they are already on the device
// (c->slots, c->rowpos)
int append_chain(dflash_ctx* c, const bf16* Hc, int ld, int nc, hipStream_t st, const AppendArgs* setup) {
  const KvGeom g = geom(c);
  const int nkv2 = c->L * 2 * c->kvd;
  if (nc <= APPEND_BATCH_ROWS) {
    // up to 64 rows: the weight-streaming skinny GEMMs, one partial per 256-deep split;
    // up to 256: the wide GEMMs, one partial per split group. Both weights in the T16 layout,
    // the partials added by the consumers.
    const bool wide = nc > APPEND_SKINNY;
    const long long ps_fc = (long long)nc * c->h, ps_kv = (long long)nc * nkv2;
    const int S_fc = wide ? gemm_wide_groups(c->g_fc.K, c->g_fc.gsz) : c->g_fc.S;
    const int G_fc = wide ? 1 : c->g_fc.gsz;
    const int S_kv = wide ? gemm_wide_groups(c->g_kvapp.K, c->g_kvapp.gsz) : c->g_kvapp.S;
    const int G_kv = wide ? 1 : c->g_kvapp.gsz;
    HIPCHK(c, timed(c, DFLASH_K_APPEND_GEMM, st, [&] {
      return wide ? launch_gemm_wide(Hc, nullptr, ld, nc, c->fc_t, c->h, ld, c->g_fc.gsz, c->part, ps_fc, st)
                  : launch_gemm_skinny(Hc, nullptr, ld, nc, c->fc_t, c->h, ld, c->g_fc.klen, c->part, ps_fc, true, st);
    }));
    HIPCHK(c, timed(c, DFLASH_K_APPEND_MISC, st, [&] {
      return launch_rows_rmsnorm(c->part, S_fc, ps_fc, G_fc, nc, c->h, c->hidden_norm, c->eps, c->Fb, c->Fb_lo, st,
                                 nullptr, nullptr, 0, nullptr, setup, c->bt_dev, c->slots, c->rowpos, c->kpos);
    }));
    HIPCHK(c, timed(c, DFLASH_K_APPEND_GEMM, st, [&] {
      return wide ? launch_gemm_wide(c->Fb, c->Fb_lo, c->h, nc, c->w_kv_t, nkv2, c->h, c->g_kvapp.gsz, c->part, ps_kv,
                                     st)
                  : launch_gemm_skinny(c->Fb, c->Fb_lo, c->h, nc, c->w_kv_t, nkv2, c->h, c->g_kvapp.klen, c->part,
                                       ps_kv, true, st);
    }));
    HIPCHK(c, timed(c, DFLASH_K_APPEND_MISC, st, [&] {
      return launch_kv_append_post(c->part, S_kv, ps_kv, G_kv, nc, c->L, c->knorm_all, c->eps, c->inv_freq,
                                   (float)c->mscale, c->slots, c->rowpos, g, st);
    }));
    return DFLASH_OK;
  }
  // many rows: the LDS-tiled GEMMs (MFMA-bound), plain fp32 results of each k split, added
  // in split order by the consumers; the K/V GEMM writes the pages from its epilogue where the
  // shape allows (the row kernel then also takes the rows' RoPE angles)
  const int ks_fc = gemm_tiled_splits(c->h, ld), ks_kv = gemm_tiled_splits(nkv2, c->h);
  HIPCHK(c, timed(c, DFLASH_K_APPEND_GEMM, st, [&] {
    return launch_gemm_tiled(Hc, nullptr, ld, nc, c->fc, c->h, ld, ks_fc, c->F32, c->h, st);
  }));
  HIPCHK(c, timed(c, DFLASH_K_APPEND_MISC, st, [&] {
    return launch_rows_rmsnorm(c->F32, ks_fc, (long long)nc * c->h, ks_fc, nc, c->h, c->hidden_norm, c->eps, c->Fb,
                               c->Fb_lo, st, c->rowpos, c->inv_freq, c->hd / 2, c->kv_fused ? c->rope_cs : nullptr,
                               setup, c->bt_dev, c->slots, c->rowpos, c->kpos);
  }));
  if (c->kv_fused) {
    HIPCHK(c, timed(c, DFLASH_K_APPEND_GEMM, st, [&] {
      return launch_gemm_tiled_kv(c->Fb, c->Fb_lo, c->h, nc, c->w_kv, nkv2, c->h, c->knorm_all, c->eps,
                                  (float)c->mscale, c->slots, c->rope_cs, g, st);
    }));
    return DFLASH_OK;
  }
  HIPCHK(c, timed(c, DFLASH_K_APPEND_GEMM, st, [&] {
    return launch_gemm_tiled(c->Fb, c->Fb_lo, c->h, nc, c->w_kv, nkv2, c->h, ks_kv, c->KV32, nkv2, st);
  }));
  HIPCHK(c, timed(c, DFLASH_K_APPEND_MISC, st, [&] {
    return launch_kv_append_post(c->KV32, ks_kv, (long long)nc * nkv2, ks_kv, nc, c->L, c->knorm_all, c->eps,
                                 c->inv_freq, (float)c->mscale, c->slots, c->rowpos, g, st);
  }));
  return DFLASH_OK;
}

extern "C" {

const char* dflash_strerror(int code) {
  switch (code) {
    case DFLASH_OK: return "ok";
    case DFLASH_EINVAL: return "invalid argument";
    case DFLASH_ENOMEM: return "out of memory";
    case DFLASH_EPOOL: return "KV pool exhausted";
    case DFLASH_ERANGE: return "out of range";
    case DFLASH_EHIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char* dflash_last_error(const dflash_ctx* c) { return c ? c->err : ""; }

int dflash_create(const dflash_config* cfg, const dflash_weights* w, void* stream, dflash_ctx** out) {
  if (!out) return DFLASH_EINVAL;
  *out = nullptr;
  std::string why;
  int rc = check_config(cfg, w, why);
  if (rc != DFLASH_OK) return rc;
  dflash_ctx* c = new dflash_ctx();
  hipStream_t st = (hipStream_t)stream;
  c->L = cfg->num_layers; c->h = cfg->hidden; c->nh = cfg->num_q_heads; c->nkv = cfg->num_kv_heads;
  c->hd = cfg->head_dim; c->qd = c->nh * c->hd; c->kvd = c->nkv * c->hd; c->ff = cfg->intermediate;
  c->V = cfg->vocab; c->T = cfg->num_taps; c->Ht = cfg->target_hidden; c->gmax = cfg->gamma_max;
  c->mask = cfg->mask_token_id; c->max_seq = cfg->max_seq_len; c->max_batch = cfg->max_batch;
  c->attn_lds = cfg->max_batch >= 8;
  c->fp8 = cfg->weight_format == DFLASH_WEIGHTS_FP8_E4M3;
  c->R = cfg->markov_rank;
  c->mk_w1 = (const bf16*)w->markov_w1;
  c->d2 = cfg->selector_rank > 0;
  c->sel_rank = cfg->selector_rank;
  c->sel_pred = (const bf16*)w->selector_pred;
  c->sel_succ = (const bf16*)w->selector_succ;
  c->eps = cfg->rms_eps; c->rope_type = cfg->rope_type; c->window = cfg->sliding_window;
  c->sliding.assign(c->L, 0);
  if (cfg->layer_sliding)
    for (int l = 0; l < c->L; ++l) c->sliding[l] = cfg->layer_sliding[l] ? 1 : 0;
  // pool: ceil((max_seq_len + gamma + 1) / 16) pages per sequence, times max_batch, + 1
  // (spark_model/layers/dflash_head/from_weights.rs, from_weights); page 0 is the spare,
  // a zeroed sentinel that is never handed out
  c->per_seq = (c->max_seq + c->gmax + 1 + PAGE - 1) / PAGE;
  c->num_pages = cfg->num_pages ? cfg->num_pages : (long long)c->per_seq * c->max_batch + 1;
  c->free_pages.init((size_t)c->num_pages);
  if (cfg->page_order) {
    std::vector<char> seen(c->num_pages, 0);
    for (long long i = 0; i + 1 < c->num_pages; ++i) {
      const int p = cfg->page_order[i];
      if (p < 1 || p >= c->num_pages || seen[p]) {
        release(c);
        return DFLASH_EINVAL;
      }
      seen[p] = 1;
      c->free_pages.push_back(p);
    }
  } else {
    for (long long p = 1; p < c->num_pages; ++p) c->free_pages.push_back((int)p);
  }
  c->seqs.resize(c->max_batch);
  // a sequence's tables never outgrow these, so appends and forwards never reallocate them
  for (SeqState& q : c->seqs) {
    q.bt.reserve(c->per_seq);
    q.pos.reserve(c->max_seq);
  }
  c->m_max = c->max_batch * c->gmax;
  c->kv_fused = gemm_tiled_kv_fusable(c->L * 2 * c->kvd, c->nkv, c->hd);
  c->fc = (const bf16*)w->fc; c->hidden_norm = (const bf16*)w->hidden_norm; c->norm = (const bf16*)w->norm;
  c->embed = (const bf16*)w->embed_tokens;

  auto fin = [&](int r) { if (r != DFLASH_OK) release(c); return r; };
  const size_t hsz = (size_t)c->h;
  const size_t pl = page_layer_elems(c->nkv, c->hd);
  c->g_qkv = plan_gemm(c->qd + 2 * c->kvd, c->h);
  c->g_o = plan_gemm(c->h, c->qd);
  c->g_gu = plan_gemm(2 * c->ff, c->h);
  c->g_down = plan_gemm(c->h, c->ff);
  c->g_fc = plan_gemm(c->h, c->T * c->Ht);
  c->g_kvapp = plan_gemm(c->L * 2 * c->kvd, c->h);
  size_t part = 0;
  if (c->d2) {
    c->g_cp = plan_gemm(c->h / 4, c->h);
    c->g_sh = plan_gemm(c->sel_rank, c->h);
  }
  for (const GemmPlan* g : {&c->g_qkv, &c->g_o, &c->g_gu, &c->g_down, &c->g_cp, &c->g_sh})
    part = std::max(part, (size_t)g->S * c->m_max * g->N);
  for (const GemmPlan* g : {&c->g_fc, &c->g_kvapp}) {
    part = std::max(part, (size_t)g->S * APPEND_SKINNY * g->N);
    part = std::max(part, (size_t)gemm_wide_groups(g->K, g->gsz) * APPEND_BATCH_ROWS * g->N);
  }
  c->part_elems = part;
  c->lm_groups = lmhead_groups(c->V);
  {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fin(fail(c, DFLASH_EHIP, "hipGetDevice failed"));
    c->dev = dev;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
      c->n_cu = ncu;
  }
  // the no-allocation forward's scratch: its device address, looked up once per device
  if ((rc = scratch_setup(c)) != DFLASH_OK) return fin(rc);
  // split-KV partial slots: chunks per band are bounded by the chunk plan
  const size_t items = (size_t)c->max_batch * max_chunks(c->per_seq) * c->nkv;
  if ((rc = dalloc(c, &c->pool, (size_t)c->L * c->num_pages * pl)) ||
      (rc = dalloc(c, &c->kpos, (size_t)c->num_pages * PAGE)) ||
      (rc = dalloc(c, &c->bt_dev, (size_t)c->max_batch * c->per_seq)) ||
      (rc = dalloc(c, &c->slots, (size_t)std::max(c->m_max, APPEND_ROWS))) ||
      (rc = dalloc(c, &c->rowpos, (size_t)APPEND_ROWS)) ||
      (rc = dalloc(c, &c->bands_dev, (size_t)MAX_BANDS)) ||
      (rc = dalloc(c, &c->X, (size_t)c->m_max * hsz)) ||
      (rc = dalloc(c, &c->ssq, (size_t)c->m_max * SSQ_STRIDE)) ||
      (rc = dalloc(c, &c->Xn, (size_t)c->m_max * hsz)) ||
      (rc = dalloc(c, &c->Xn_lo, (size_t)c->m_max * hsz)) ||
      (rc = dalloc(c, &c->Qb, (size_t)c->m_max * c->qd)) ||
      (rc = dalloc(c, &c->Qb_lo, (size_t)c->m_max * c->qd)) ||
      (rc = dalloc(c, &c->attn, (size_t)c->m_max * c->qd)) ||
      (rc = dalloc(c, &c->attn_lo, (size_t)c->m_max * c->qd)) ||
      (rc = dalloc(c, &c->act, (size_t)c->m_max * c->ff)) ||
      (rc = dalloc(c, &c->act_lo, (size_t)c->m_max * c->ff)) ||
      (rc = dalloc(c, &c->part, part)) ||
      (rc = dalloc(c, &c->aparts_o, items * 128 * c->hd)) ||
      (rc = dalloc(c, &c->aparts_ml, items * 128 * 2)) ||
      (rc = dalloc(c, &c->best_v, (size_t)c->m_max * c->lm_groups)) ||
      (rc = dalloc(c, &c->best_i, (size_t)c->m_max * c->lm_groups)) ||
      (rc = dalloc(c, &c->F32, (size_t)gemm_tiled_splits(c->h, c->T * c->Ht) * APPEND_ROWS * hsz)) ||
      (rc = dalloc(c, &c->Fb, (size_t)APPEND_ROWS * hsz)) ||
      (rc = dalloc(c, &c->Fb_lo, (size_t)APPEND_ROWS * hsz)) ||
      (rc = dalloc(c, &c->KV32, c->kv_fused ? 0 : (size_t)gemm_tiled_splits(c->L * 2 * c->kvd, c->h) * APPEND_ROWS * c->L * 2 * c->kvd)) ||
      (rc = dalloc(c, &c->rope_cs, (size_t)APPEND_ROWS * (c->hd / 2))) ||
      (rc = dalloc(c, &c->ring_dev, (size_t)RING * APPEND_ROWS)) ||
      (rc = dalloc(c, &c->w_kv, (size_t)c->L * 2 * c->kvd * hsz)) ||
      (rc = dalloc(c, &c->w_kv_t, (size_t)c->L * 2 * c->kvd * hsz)) ||
      (rc = dalloc(c, &c->fc_t, (size_t)hsz * c->T * c->Ht)) ||
      (rc = dalloc(c, &c->knorm_all, (size_t)c->L * c->hd)) ||
      (rc = dalloc(c, &c->inv_freq, (size_t)c->hd / 2)) ||
      (c->fp8 ? (rc = dalloc(c, &c->lm_q, (size_t)(c->V + 15) / 16 * 16 * hsz)) ||
                    (rc = dalloc(c, &c->lm_s, (size_t)(c->V + 15) / 16 * 16))
              : (rc = dalloc(c, &c->lm_head, (size_t)(c->V + 15) / 16 * 16 * hsz))))
    return fin(rc);
  if (c->R) {
    c->mk_groups = markov_step_groups(c->V, c->n_cu);
    if ((rc = dalloc(c, &c->mk_w2t, (size_t)(c->V + 15) / 16 * 16 * c->R)) ||
        (rc = dalloc(c, &c->mk_best, (size_t)MARKOV_MAX_ROWS * MAX_BANDS)))
      return fin(rc);
  }
  const size_t drafted = (size_t)c->max_batch * (c->gmax - 1);
  if ((c->R || c->d2) && (rc = dalloc(c, &c->mk_logits, drafted * c->V))) return fin(rc);
  if (c->d2 &&
      ((rc = dalloc(c, &c->sel_h, (size_t)c->sel_rank * hsz)) ||
       (rc = dalloc(c, &c->dyn_a, (size_t)c->m_max * (hsz / 4))) ||
       (rc = dalloc(c, &c->dyn_m, (size_t)c->m_max * (hsz / 4))) ||
       (rc = dalloc(c, &c->U, (size_t)c->m_max * hsz)) || (rc = dalloc(c, &c->U_lo, (size_t)c->m_max * hsz)) ||
       (rc = dalloc(c, &c->tk_v, drafted * TOPK_MAX_SLICES * 16)) ||
       (rc = dalloc(c, &c->tk_i, drafted * TOPK_MAX_SLICES * 16)) ||
       (rc = dalloc(c, &c->sel_v, drafted * 16)) || (rc = dalloc(c, &c->sel_i, drafted * 16)) ||
       (rc = dalloc(c, &c->sel_pair, drafted * 16 * 16))))
    return fin(rc);
  c->layers.resize(c->L);
  for (int l = 0; l < c->L; ++l) {
    LayerDev& d = c->layers[l];
    const dflash_layer_weights& lw = w->layers[l];
    d.q_norm = (const bf16*)lw.q_norm; d.k_norm = (const bf16*)lw.k_norm;
    if ((rc = dalloc(c, &d.in_norm, hsz)) || (rc = dalloc(c, &d.post_norm, hsz)))
      return fin(rc);
    if (c->d2) {
      d.cba = (const bf16*)lw.attention_conv_base;
      d.cbm = (const bf16*)lw.mlp_conv_base;
      if ((rc = dalloc(c, &d.w_cpa, (hsz / 4) * hsz)) || (rc = dalloc(c, &d.w_cpm, (hsz / 4) * hsz)))
        return fin(rc);
    }
    if (c->fp8) {
      if ((rc = dalloc(c, &d.q_qkv, (size_t)(c->qd + 2 * c->kvd) * hsz)) ||
          (rc = dalloc(c, &d.s_qkv, (size_t)(c->qd + 2 * c->kvd))) ||
          (rc = dalloc(c, &d.q_gu, (size_t)2 * c->ff * hsz)) || (rc = dalloc(c, &d.s_gu, (size_t)2 * c->ff)) ||
          (rc = dalloc(c, &d.q_o, (size_t)hsz * c->qd)) || (rc = dalloc(c, &d.s_o, hsz)) ||
          (rc = dalloc(c, &d.q_down, (size_t)hsz * c->ff)) || (rc = dalloc(c, &d.s_down, hsz)))
        return fin(rc);
    } else if ((rc = dalloc(c, &d.w_qkv, (size_t)(c->qd + 2 * c->kvd) * hsz)) ||
               (rc = dalloc(c, &d.w_gu, (size_t)2 * c->ff * hsz)) ||
               (rc = dalloc(c, &d.o_proj, (size_t)hsz * c->qd)) ||
               (rc = dalloc(c, &d.down_proj, (size_t)hsz * c->ff))) {
      return fin(rc);
    }
  }
  if (hipHostMalloc((void**)&c->ring_host, (size_t)RING * APPEND_ROWS * sizeof(int), hipHostMallocDefault) != hipSuccess) {
    c->ring_host = nullptr;
    return fin(fail(c, DFLASH_ENOMEM, "hipHostMalloc failed"));
  }
  for (int i = 0; i < RING; ++i)
    if (hipEventCreateWithFlags(&c->ring_ev[i], hipEventDisableTiming) != hipSuccess)
      return fin(fail(c, DFLASH_EHIP, "hipEventCreate failed"));

  auto cp = [&](void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
  };
  const size_t kb = (size_t)c->kvd * hsz * 2;
  hipError_t e = hipSuccess;
  // the forward's weights in the T16 layout: a tiled [A;B] is tiled A followed by tiled B
  // when A's rows are a whole number of 16-row tiles (q_dim, kv_dim and ff all are)
  auto tile = [&](const void* src, int N, int K, bf16* dst) {
    return launch_tile_weight((const bf16*)src, N, K, dst, st);
  };
  // FP8 weights ([metrale-fw] from_weights, the FP8 weights phase): the same seven per-layer
  // matrices and the lm_head quantized once, here, with per-row scales; a fused [A;B] is A's
  // codes and scales followed by B's
  auto quant = [&](const void* src, int N, int K, uint8_t* dst, float* sc) {
    return launch_quant_fp8((const bf16*)src, N, K, dst, sc, st);
  };
  for (int l = 0; l < c->L && e == hipSuccess; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    LayerDev& d = c->layers[l];
    if (c->fp8) {
      if ((e = quant(lw.q_proj, c->qd, c->h, d.q_qkv, d.s_qkv)) ||
          (e = quant(lw.k_proj, c->kvd, c->h, d.q_qkv + (size_t)c->qd * hsz, d.s_qkv + c->qd)) ||
          (e = quant(lw.v_proj, c->kvd, c->h, d.q_qkv + (size_t)(c->qd + c->kvd) * hsz, d.s_qkv + c->qd + c->kvd)) ||
          (e = quant(lw.gate_proj, c->ff, c->h, d.q_gu, d.s_gu)) ||
          (e = quant(lw.up_proj, c->ff, c->h, d.q_gu + (size_t)c->ff * hsz, d.s_gu + c->ff)) ||
          (e = quant(lw.o_proj, c->h, c->qd, d.q_o, d.s_o)) ||
          (e = quant(lw.down_proj, c->h, c->ff, d.q_down, d.s_down)))
        break;
    } else if ((e = tile(lw.q_proj, c->qd, c->h, d.w_qkv)) ||
               (e = tile(lw.k_proj, c->kvd, c->h, d.w_qkv + (size_t)c->qd * hsz)) ||
               (e = tile(lw.v_proj, c->kvd, c->h, d.w_qkv + (size_t)(c->qd + c->kvd) * hsz)) ||
               (e = tile(lw.gate_proj, c->ff, c->h, d.w_gu)) ||
               (e = tile(lw.up_proj, c->ff, c->h, d.w_gu + (size_t)c->ff * hsz)) ||
               (e = tile(lw.o_proj, c->h, c->qd, d.o_proj)) ||
               (e = tile(lw.down_proj, c->h, c->ff, d.down_proj))) {
      break;
    }
    if ((e = cp(d.in_norm, lw.input_layernorm, hsz * 2)) ||
        (e = cp(d.post_norm, lw.post_attention_layernorm, hsz * 2)) ||
        (e = cp((char*)c->w_kv + (size_t)l * 2 * kb, lw.k_proj, kb)) ||
        (e = cp((char*)c->w_kv + (size_t)l * 2 * kb + kb, lw.v_proj, kb)) ||
        (e = cp(c->knorm_all + (size_t)l * c->hd, lw.k_norm, (size_t)c->hd * 2)))
      break;
  }
  if (e == hipSuccess) e = c->fp8 ? quant(w->lm_head, c->V, c->h, c->lm_q, c->lm_s) : tile(w->lm_head, c->V, c->h, c->lm_head);
  if (e == hipSuccess) e = tile(w->fc, c->h, c->T * c->Ht, c->fc_t);
  if (e == hipSuccess && c->R) e = tile(w->markov_w2, c->V, c->R, c->mk_w2t);
  if (e == hipSuccess && c->d2) {
    e = tile(w->selector_hidden_proj, c->sel_rank, c->h, c->sel_h);
    for (int l = 0; l < c->L && e == hipSuccess; ++l) {
      if ((e = tile(w->layers[l].attention_conv_proj, c->h / 4, c->h, c->layers[l].w_cpa)) == hipSuccess)
        e = tile(w->layers[l].mlp_conv_proj, c->h / 4, c->h, c->layers[l].w_cpm);
    }
  }
  if (e == hipSuccess && c->R) e = hipMemsetAsync(c->mk_best, 0, (size_t)MARKOV_MAX_ROWS * MAX_BANDS * 8, st);
  if (e == hipSuccess) e = tile(c->w_kv, c->L * 2 * c->kvd, c->h, c->w_kv_t);   // after the copies above, same stream
  std::vector<double> f = inv_freq_table(cfg, &c->mscale);
  if (e == hipSuccess) e = hipMemcpyAsync(c->inv_freq, f.data(), f.size() * sizeof(double), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemsetAsync(c->pool, 0, (size_t)c->L * c->num_pages * pl * 2, st);
  if (e == hipSuccess) e = hipMemsetAsync(c->kpos, 0, (size_t)c->num_pages * PAGE * 4, st);
  if (e == hipSuccess) e = hipMemsetAsync(c->ssq, 0, (size_t)c->m_max * SSQ_STRIDE * 4, st);
  if (e == hipSuccess) e = hipMemsetAsync(c->bt_dev, 0, (size_t)c->max_batch * c->per_seq * 4, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fin(fail(c, DFLASH_EHIP, "create: %s", hipGetErrorString(e)));
  *out = c;
  return DFLASH_OK;
}

void dflash_destroy(dflash_ctx* c) {
  if (!c) return;
  (void)hipDeviceSynchronize();
  release(c);
}

int dflash_seq_reset(dflash_ctx* c, int32_t seq) {
  if (!c) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  if (seq < 0 || seq >= c->max_batch) return fail(c, DFLASH_ERANGE, "seq %d out of range", seq);
  SeqState& s = c->seqs[seq];
  for (int p : s.bt) c->free_pages.push_back(p);
  // device block-table rows of freed pages go back to the sentinel lazily: every reader
  // bounds its page lookups by the sequence's length, and new pages overwrite the entries
  s.bt.clear();
  s.pos.clear();
  s.kv_len = 0;
  return DFLASH_OK;
}

int dflash_seq_info(const dflash_ctx* c, int32_t seq, int32_t* kv_len, int32_t* n_pages,
                    int32_t* block_table, int32_t cap) {
  if (!c || seq < 0 || seq >= c->max_batch) return DFLASH_ERANGE;
  const SeqState& s = c->seqs[seq];
  if (kv_len) *kv_len = s.kv_len;
  if (n_pages) *n_pages = (int32_t)s.bt.size();
  if (block_table)
    for (int i = 0; i < cap && i < (int)s.bt.size(); ++i) block_table[i] = s.bt[i];
  return DFLASH_OK;
}

int dflash_pool_geometry(const dflash_ctx* c, int64_t* num_pages, int64_t* pages_per_seq,
                         int64_t* page_layer_bytes, int64_t* pool_bytes, int64_t* fused_kv_weight_bytes) {
  if (!c) return DFLASH_EINVAL;
  const int64_t plb = (int64_t)page_layer_elems(c->nkv, c->hd) * 2;
  if (num_pages) *num_pages = c->num_pages;
  if (pages_per_seq) *pages_per_seq = c->per_seq;
  if (page_layer_bytes) *page_layer_bytes = plb;
  if (pool_bytes) *pool_bytes = plb * c->L * c->num_pages;
  if (fused_kv_weight_bytes) *fused_kv_weight_bytes = (int64_t)c->L * 2 * c->kvd * c->h * 2;
  return DFLASH_OK;
}

int dflash_debug_copy(dflash_ctx* c, int32_t buffer, void* dst, size_t offset, size_t bytes, void* stream) {
  if (!c || !dst) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  const char* base = nullptr;
  size_t size = 0;
  switch (buffer) {
    case DFLASH_BUF_POOL: base = (const char*)c->pool; size = (size_t)c->L * c->num_pages * page_layer_elems(c->nkv, c->hd) * 2; break;
    case DFLASH_BUF_KPOS: base = (const char*)c->kpos; size = (size_t)c->num_pages * PAGE * 4; break;
    case DFLASH_BUF_SLOTS: base = (const char*)c->slots; size = (size_t)std::max(c->m_max, APPEND_ROWS) * 8; break;
    case DFLASH_BUF_BLOCKTAB: base = (const char*)c->bt_dev; size = (size_t)c->max_batch * c->per_seq * 4; break;
    case DFLASH_BUF_HIDDEN: base = (const char*)c->Xn; size = (size_t)c->m_max * c->h * 2; break;
    case DFLASH_BUF_HIDDEN_LO: base = (const char*)c->Xn_lo; size = (size_t)c->m_max * c->h * 2; break;
    case DFLASH_BUF_FP8_LMHEAD:
      if (!c->fp8) return fail(c, DFLASH_EINVAL, "not an FP8 context");
      base = (const char*)c->lm_q; size = (size_t)(c->V + 15) / 16 * 16 * c->h; break;
    case DFLASH_BUF_FP8_LMHEAD_SCALE:
      if (!c->fp8) return fail(c, DFLASH_EINVAL, "not an FP8 context");
      base = (const char*)c->lm_s; size = (size_t)(c->V + 15) / 16 * 16 * 4; break;
    case DFLASH_BUF_SEL_IDX:
      if (!c->d2) return fail(c, DFLASH_EINVAL, "not a DFlash2 context");
      base = (const char*)c->sel_i; size = (size_t)c->max_batch * (c->gmax - 1) * 16 * 4; break;
    case DFLASH_BUF_SEL_VALS:
      if (!c->d2) return fail(c, DFLASH_EINVAL, "not a DFlash2 context");
      base = (const char*)c->sel_v; size = (size_t)c->max_batch * (c->gmax - 1) * 16 * 4; break;
    case DFLASH_BUF_CTX_FEAT: base = (const char*)c->Fb; size = (size_t)APPEND_ROWS * c->h * 2; break;
    case DFLASH_BUF_CTX_FEAT_LO: base = (const char*)c->Fb_lo; size = (size_t)APPEND_ROWS * c->h * 2; break;
    case DFLASH_BUF_LAYER_Q:
    case DFLASH_BUF_LAYER_Q_LO:
    case DFLASH_BUF_LAYER_ATTN:
    case DFLASH_BUF_LAYER_ATTN_LO:
    case DFLASH_BUF_LAYER_X1:
    case DFLASH_BUF_LAYER_X: {
      if (!c->cap_q) return fail(c, DFLASH_EINVAL, "no capture: call dflash_debug_capture first");
      const size_t rows = (size_t)c->L * c->m_max;
      const void* bufs[] = {c->cap_q, c->cap_q_lo, c->cap_a, c->cap_a_lo, c->cap_x1, c->cap_x};
      base = (const char*)bufs[buffer - DFLASH_BUF_LAYER_Q];
      size = buffer >= DFLASH_BUF_LAYER_X1 ? rows * c->h * 4 : rows * c->qd * 2;
      break;
    }
    default: return fail(c, DFLASH_EINVAL, "unknown buffer %d", buffer);
  }
  if (offset > size || bytes > size - offset) return fail(c, DFLASH_ERANGE, "copy past the end of buffer %d", buffer);
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(c, hipMemcpyAsync(dst, base + offset, bytes, hipMemcpyDefault, st));
  HIPCHK(c, hipStreamSynchronize(st));
  return DFLASH_OK;
}

int dflash_ctx_kv_append(dflash_ctx* c, int32_t seq, const void* target_hidden,
                         const int32_t* positions, int32_t n, void* stream) {
  if (!c) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  if (seq < 0 || seq >= c->max_batch) return fail(c, DFLASH_ERANGE, "seq %d out of range", seq);
  if (n <= 0) return fail(c, DFLASH_EINVAL, "n must be positive");
  if (!target_hidden) return fail(c, DFLASH_EINVAL, "NULL target_hidden");
  SeqState& s = c->seqs[seq];
  const int C = s.kv_len;
  if ((long long)C + n > c->max_seq) return fail(c, DFLASH_ERANGE, "kv_len %d + n %d exceeds max_seq_len %d", C, n, c->max_seq);
  long long last = s.pos.empty() ? -1 : s.pos.back();
  for (int i = 0; i < n; ++i) {
    const long long p = positions ? positions[i] : (long long)C + i;
    if (p <= last || p >= (1LL << 30))
      return fail(c, DFLASH_EINVAL, "positions must be strictly increasing, in [0, 2^30)");
    last = p;
  }
  const int need = (C + n + PAGE - 1) / PAGE - (int)s.bt.size();
  if (need > (int)c->free_pages.size()) return fail(c, DFLASH_EPOOL, "KV pool exhausted (%d pages needed, %zu free)", need, c->free_pages.size());
  // --- committed from here on
  const int old_pages = (int)s.bt.size();
  for (int i = 0; i < need; ++i) {
    s.bt.push_back(c->free_pages.front());
    c->free_pages.pop_front();
  }
  hipStream_t st = (hipStream_t)stream;
  const int ld = c->T * c->Ht;
  for (int r0 = 0; r0 < n; r0 += APPEND_ROWS) {
    const int nc = std::min(APPEND_ROWS, n - r0);
    AppendArgs a{};
    a.seq = seq; a.kv_len = C + r0; a.n = nc; a.per_seq = c->per_seq;
    a.first_lpage = (C + r0) / PAGE;
    a.n_lpages = (C + r0 + nc - 1) / PAGE - a.first_lpage + 1;
    a.n_upd = 0;
    for (int i = 0; i < a.n_lpages; ++i) {
      const int lp = a.first_lpage + i;
      a.pages[i] = s.bt[lp];
      if (lp >= old_pages) {
        a.upd_off[a.n_upd] = seq * c->per_seq + lp;
        a.upd_page[a.n_upd] = s.bt[lp];
        ++a.n_upd;
      }
    }
    a.positions = nullptr;
    int slot = -1;
    if (positions) {
      slot = c->ring_next;
      c->ring_next = (c->ring_next + 1) % RING;
      HIPCHK(c, hipEventSynchronize(c->ring_ev[slot]));
      int* hp = c->ring_host + (size_t)slot * APPEND_ROWS;
      int* dp = c->ring_dev + (size_t)slot * APPEND_ROWS;
      memcpy(hp, positions + r0, (size_t)nc * sizeof(int));
      HIPCHK(c, hipMemcpyAsync(dp, hp, (size_t)nc * sizeof(int), hipMemcpyHostToDevice, st));
      a.positions = dp;
    }
    // (the row kernel of the chain does this chunk's setup, reading the positions the ring
    // slot holds; the slot is free again once the chain has run)
    const int rc = append_chain(c, (const bf16*)target_hidden + (size_t)r0 * ld, ld, nc, st, &a);
    if (rc != DFLASH_OK) return rc;
    if (slot >= 0) HIPCHK(c, hipEventRecord(c->ring_ev[slot], st));
  }
  for (int i = 0; i < n; ++i) s.pos.push_back(positions ? positions[i] : C + i);
  s.kv_len = C + n;
  return DFLASH_OK;
}

int dflash_ctx_kv_append_batch(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int32_t* counts,
                               const void* target_hidden, const int32_t* positions, void* stream) {
  if (!c) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  if (n_seqs < 1 || n_seqs > c->max_batch) return fail(c, DFLASH_EINVAL, "n_seqs %d not in [1, %d]", n_seqs, c->max_batch);
  if (!seqs || !counts || !target_hidden) return fail(c, DFLASH_EINVAL, "NULL seqs, counts or target_hidden");
  bool seen[MAX_BANDS] = {};   // max_batch <= MAX_BANDS
  long long total = 0;
  int need = 0;
  for (int b = 0; b < n_seqs; ++b) {
    const int q = seqs[b];
    if (q < 0 || q >= c->max_batch || seen[q]) return fail(c, DFLASH_ERANGE, "seq %d out of range or repeated", q);
    seen[q] = 1;
    if (counts[b] < 0) return fail(c, DFLASH_EINVAL, "counts must be >= 0");
    const SeqState& s = c->seqs[q];
    if ((long long)s.kv_len + counts[b] > c->max_seq)
      return fail(c, DFLASH_ERANGE, "seq %d: kv_len %d + %d exceeds max_seq_len %d", q, s.kv_len, counts[b], c->max_seq);
    total += counts[b];
    need += std::max(0, (s.kv_len + counts[b] + PAGE - 1) / PAGE - (int)s.bt.size());
  }
  if (total < 1 || total > APPEND_BATCH_ROWS)
    return fail(c, DFLASH_EINVAL, "total rows %lld not in [1, %d]", total, APPEND_BATCH_ROWS);
  if (positions) {
    long long r = 0;
    for (int b = 0; b < n_seqs; ++b) {
      const SeqState& s = c->seqs[seqs[b]];
      long long last = s.pos.empty() ? -1 : s.pos.back();
      for (int i = 0; i < counts[b]; ++i, ++r) {
        if (positions[r] <= last || positions[r] >= (1LL << 30))
          return fail(c, DFLASH_EINVAL, "positions must be strictly increasing per sequence, in [0, 2^30)");
        last = positions[r];
      }
    }
  }
  if (need > (int)c->free_pages.size()) return fail(c, DFLASH_EPOOL, "KV pool exhausted (%d pages needed, %zu free)", need, c->free_pages.size());
  // --- committed from here on: pages are taken in call order, each sequence's in logical order
  AppendBatchArgs a{};
  a.per_seq = c->per_seq;
  a.n_rows = (int)total;
  int np = 0;
  for (int b = 0; b < n_seqs; ++b) {
    if (counts[b] == 0) continue;
    const int q = seqs[b];
    SeqState& s = c->seqs[q];
    const int old_pages = (int)s.bt.size();
    const int want = (s.kv_len + counts[b] + PAGE - 1) / PAGE;
    while ((int)s.bt.size() < want) {
      s.bt.push_back(c->free_pages.front());
      c->free_pages.pop_front();
    }
    const int k = a.n_seqs++;
    a.seq[k] = q;
    a.kv_len[k] = s.kv_len;
    a.row0[k + 1] = a.row0[k] + counts[b];
    a.lp0[k] = s.kv_len / PAGE;
    a.pg0[k] = np;
    for (int lp = a.lp0[k]; lp < want; ++lp) {
      a.pages[np++] = s.bt[lp];
      if (lp >= old_pages) {
        a.upd_off[a.n_upd] = q * c->per_seq + lp;
        a.upd_page[a.n_upd] = s.bt[lp];
        ++a.n_upd;
      }
    }
  }
  hipStream_t st = (hipStream_t)stream;
  a.positions = nullptr;
  int slot = -1;
  if (positions) {
    slot = c->ring_next;
    c->ring_next = (c->ring_next + 1) % RING;
    HIPCHK(c, hipEventSynchronize(c->ring_ev[slot]));
    int* hp = c->ring_host + (size_t)slot * APPEND_ROWS;
    int* dp = c->ring_dev + (size_t)slot * APPEND_ROWS;
    memcpy(hp, positions, (size_t)total * sizeof(int));
    HIPCHK(c, hipMemcpyAsync(dp, hp, (size_t)total * sizeof(int), hipMemcpyHostToDevice, st));
    a.positions = dp;
  }
  HIPCHK(c, timed(c, DFLASH_K_APPEND_MISC, st, [&] {
    return launch_append_batch_setup(a, c->bt_dev, c->slots, c->rowpos, c->kpos, st);
  }));
  if (slot >= 0) HIPCHK(c, hipEventRecord(c->ring_ev[slot], st));
  const int rc = append_chain(c, (const bf16*)target_hidden, c->T * c->Ht, (int)total, st, nullptr);
  if (rc != DFLASH_OK) return rc;
  long long r = 0;
  for (int b = 0; b < n_seqs; ++b) {
    SeqState& s = c->seqs[seqs[b]];
    for (int i = 0; i < counts[b]; ++i, ++r) s.pos.push_back(positions ? positions[r] : s.kv_len + i);
    s.kv_len += counts[b];
  }
  return DFLASH_OK;
}

}  // extern "C"

namespace {

// The device scratch one forward writes and reads back: split-K partials, attention
// partials and lm_head argmax partials (all fully written before they are read)
struct FwdScratch {
  float* part;
  float* aparts_o;
  float* aparts_ml;
  float* best_v;
  int* best_i;
};

// what a forward of n_seqs bands of `gamma` rows needs of each scratch buffer (elements),
// given the call's total attention chunks of full-attention layers
struct FwdNeed {
  size_t part, aparts_o, aparts_ml, best;
};

FwdNeed fwd_need(const dflash_ctx* c, int n_seqs, int gamma, int chunks_full) {
  const int M = n_seqs * gamma;
  const bool wide = M > ROW_GROUP;
  FwdNeed n{};
  for (const GemmPlan* g : {&c->g_qkv, &c->g_o, &c->g_gu, &c->g_down, &c->g_cp, &c->g_sh}) {
    if (g->N == 0) continue;   // (the DFlash2 plans of a plain drafter)
    const int cnt = wide ? gemm_wide_groups(g->K, g->gsz) : g->S;
    n.part = std::max(n.part, (size_t)cnt * M * g->N);
  }
  // a sliding layer's keys start at or after a full layer's, so its chunks are never more
  const size_t items = (size_t)chunks_full * c->nkv;
  n.aparts_o = items * ATTN_PART_ROWS * c->hd;
  n.aparts_ml = items * ATTN_PART_ROWS * 2;
  n.best = (size_t)M * std::max(c->lm_groups, lmhead_wide_groups(c->V));
  return n;
}

size_t align256(size_t bytes) { return (bytes + 255) & ~(size_t)255; }

// the forward's scratch carved out of the device's static array; false if it does not fit
bool carve_static(const dflash_ctx* c, const FwdNeed& n, FwdScratch& sc, size_t& total) {
  const size_t b_part = align256(n.part * 4), b_o = align256(n.aparts_o * 4), b_ml = align256(n.aparts_ml * 4),
               b_bv = align256(n.best * 4), b_bi = align256(n.best * 4);
  total = b_part + b_o + b_ml + b_bv + b_bi;
  if (total > NOALLOC_SCRATCH_BYTES) return false;
  char* base = (char*)g_scratch_ptr[c->dev];
  sc.part = (float*)base;
  sc.aparts_o = (float*)(base + b_part);
  sc.aparts_ml = (float*)(base + b_part + b_o);
  sc.best_v = (float*)(base + b_part + b_o + b_ml);
  sc.best_i = (int*)(base + b_part + b_o + b_ml + b_bv);
  return true;
}

// a band's split-KV plan for full (sw 0) and sliding (sw 1) layers: keys from kstart (page
// aligned) to kv_len + gamma in nch chunks of ck keys
void band_plan(const dflash_ctx* c, const SeqState& s, int q_pos, int gamma, Band& B) {
  const int C = s.kv_len;
  const int kend = C + gamma;
  // full layers: every key; sliding layers: from the first context row whose stamped
  // position is within the window of block row 0 (rows further down see a subset)
  int klo = 0;
  if (c->window > 0) {
    const long long lim = (long long)q_pos - c->window;  // visible iff pos > lim
    klo = (int)(std::upper_bound(s.pos.begin(), s.pos.end(), lim) - s.pos.begin());
  }
  for (int sw = 0; sw < 2; ++sw) {
    B.kstart[sw] = sw == 0 ? 0 : (klo / PAGE) * PAGE;
    // full layers of a drafter with the LDS path plan its bands for it (the same page rule
    // picks the path)
    plan_chunks(B.kstart[sw], kend, c->attn_lds && c->hd == 128 && sw == 0, B.ck[sw], B.nch[sw]);
  }
}

int block_forward(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int32_t* bonus,
                  const int32_t* q_rope_pos, int32_t gamma, int32_t* draft_tokens, float* logits, void* stream,
                  bool noalloc) {
  if (!c) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  if (n_seqs < 1 || n_seqs > c->max_batch) return fail(c, DFLASH_EINVAL, "n_seqs %d not in [1, %d]", n_seqs, c->max_batch);
  if (!seqs || !bonus || !draft_tokens) return fail(c, DFLASH_EINVAL, "NULL seqs, bonus_tokens or draft_tokens");
  if (gamma < 2 || gamma > c->gmax) return fail(c, DFLASH_ERANGE, "gamma %d not in [2, %d]", gamma, c->gmax);
  bool seen[MAX_BANDS] = {};   // max_batch <= MAX_BANDS
  FwdArgs a{};
  int need = 0, chunks_full = 0;
  for (int b = 0; b < n_seqs; ++b) {
    const int q = seqs[b];
    if (q < 0 || q >= c->max_batch || seen[q]) return fail(c, DFLASH_ERANGE, "seq %d out of range or repeated", q);
    seen[q] = 1;
    if (bonus[b] < 0 || bonus[b] >= c->V) return fail(c, DFLASH_EINVAL, "bonus token %d out of range", bonus[b]);
    if (q_rope_pos && (q_rope_pos[b] < 0 || q_rope_pos[b] >= (1 << 30)))
      return fail(c, DFLASH_EINVAL, "q_rope_pos must be in [0, 2^30)");
    const SeqState& s = c->seqs[q];
    need += std::max(0, (s.kv_len + gamma + PAGE - 1) / PAGE - (int)s.bt.size());
    Band& B = a.bands[b];
    B.seq = q; B.kv_len = s.kv_len; B.q_pos = q_rope_pos ? q_rope_pos[b] : s.kv_len; B.bonus = bonus[b];
    band_plan(c, s, B.q_pos, gamma, B);
    chunks_full += B.nch[0];
  }
  if (need > (int)c->free_pages.size()) return fail(c, DFLASH_EPOOL, "KV pool exhausted (%d pages needed, %zu free)", need, c->free_pages.size());
  FwdScratch sc{c->part, c->aparts_o, c->aparts_ml, c->best_v, c->best_i};
  if (noalloc) {
    size_t total = 0;
    if (!carve_static(c, fwd_need(c, n_seqs, gamma, chunks_full), sc, total))
      return fail(c, DFLASH_ERANGE, "this forward needs %zu bytes of scratch, above the no-allocation limit of %zu",
                  total, NOALLOC_SCRATCH_BYTES);
  }
  // --- committed from here on
  a.n_bands = n_seqs; a.gamma = gamma; a.mask_token = c->mask; a.per_seq = c->per_seq; a.n_upd = 0;
  int base[2] = {0, 0};
  for (int b = 0; b < n_seqs; ++b) {
    const int q = seqs[b];
    SeqState& s = c->seqs[q];
    const int C = s.kv_len;
    const int want = (C + gamma + PAGE - 1) / PAGE;
    while ((int)s.bt.size() < want) {
      const int p = c->free_pages.front();
      c->free_pages.pop_front();
      a.upd_off[a.n_upd] = q * c->per_seq + (int)s.bt.size();
      a.upd_page[a.n_upd] = p;
      ++a.n_upd;
      s.bt.push_back(p);
    }
    Band& B = a.bands[b];
    const int lp0 = C / PAGE;
    B.pg[0] = s.bt[lp0];
    B.pg[1] = lp0 + 1 < (int)s.bt.size() ? s.bt[lp0 + 1] : 0;
    for (int sw = 0; sw < 2; ++sw) {
      B.base[sw] = base[sw];
      base[sw] += B.nch[sw];
    }
  }
  hipStream_t st = (hipStream_t)stream;
  const KvGeom g = geom(c);
  const int M = n_seqs * gamma;
  // the attention launches of full and of sliding-window layers
  AttnBands ab[2];
  int ab_reg[2], ab_lds[2];
  for (int sw = 0; sw < 2; ++sw)
    plan_attn(a.bands, n_seqs, sw, c->hd, sw ? c->window : 0, c->attn_lds, gamma, ab[sw], ab_reg[sw], ab_lds[sw]);
  const float scale_log2 = (float)(1.0 / std::sqrt((double)c->hd) * 1.4426950408889634);
  HIPCHK(c, timed(c, DFLASH_K_PROLOGUE, st, [&] {
    return launch_fwd_prologue(a, c->bands_dev, c->bt_dev, c->slots, c->kpos, c->embed, c->layers[0].in_norm, c->h,
                               c->X, c->ssq, c->Xn, c->Xn_lo, st);
  }));
  // normed: (A, A_lo) is the residual stream times a norm weight, and the result rows take
  // the rows' RMSNorm scales from the slice sums of squares
  // More than one row group: the wide kernel, one launch, one partial per split group;
  // otherwise the skinny kernel, one partial per split. parts(p) = what the consumer adds:
  // (partials, splits per group).
  const bool wide = M > ROW_GROUP;
  auto parts = [&](const GemmPlan& p) {
    return wide ? std::make_pair(gemm_wide_groups(p.K, p.gsz), 1) : std::make_pair(p.S, p.gsz);
  };
  // wsc: W holds FP8 codes with these row scales
  auto gemm = [&](const bf16* A, const bf16* A_lo, int lda, const bf16* W, const float* wsc, const GemmPlan& p,
                  bool normed) -> hipError_t {
    const long long ps = (long long)M * p.N;
    if (wide) {
      const NormIn nn{c->ssq, c->eps, c->h};
      return timed(c, DFLASH_K_GEMM, st, [&] {
        return launch_gemm_wide(A, A_lo, lda, M, W, p.N, p.K, p.gsz, sc.part, ps, st, normed ? &nn : nullptr, wsc);
      });
    }
    for (int r0 = 0; r0 < M; r0 += ROW_GROUP) {
      const int mg = std::min(ROW_GROUP, M - r0);
      const NormIn nn{c->ssq + (size_t)r0 * SSQ_STRIDE, c->eps, c->h};
      hipError_t e = timed(c, DFLASH_K_GEMM, st, [&] {
        return launch_gemm_skinny(A + (size_t)r0 * lda, A_lo + (size_t)r0 * lda, lda, mg, W, p.N, p.K, p.klen,
                                  sc.part + (size_t)r0 * p.N, ps, true, st, normed ? &nn : nullptr, wsc);
      });
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  };
  // DFlash2 conv site: the projection of the normed rows (x * w with the rows' RMSNorm
  // scales, as the QKV and gate/up GEMMs take them), then the taps and the prepare application
  auto dconv_site = [&](const bf16* w_proj, const bf16* base, float* dyn) -> hipError_t {
    hipError_t e = gemm(c->Xn, c->Xn_lo, c->h, w_proj, nullptr, c->g_cp, true);
    if (e != hipSuccess) return e;
    return timed(c, DFLASH_K_DCONV, st, [&] {
      return launch_dconv_prepare(c->Xn, c->Xn_lo, c->ssq, c->eps, M, c->h, gamma, sc.part, parts(c->g_cp).first,
                                  (long long)M * c->g_cp.N, parts(c->g_cp).second, base, dyn, c->U, c->U_lo, st);
    });
  };
  for (int l = 0; l < c->L; ++l) {
    const LayerDev& d = c->layers[l];
    const int sw = sliding_layer(c, l) ? 1 : 0;
    const bool q8 = c->fp8;
    // DFlash2: the attention input through its dynamic conv (projection of the normed input,
    // then taps + convolution); the QKV GEMM then reads the convolved rows as they are
    if (c->d2) HIPCHK(c, dconv_site(d.w_cpa, d.cba, c->dyn_a));
    HIPCHK(c, gemm(c->d2 ? c->U : c->Xn, c->d2 ? c->U_lo : c->Xn_lo, c->h, q8 ? (const bf16*)d.q_qkv : d.w_qkv,
                   q8 ? d.s_qkv : nullptr, c->g_qkv, !c->d2));
    HIPCHK(c, timed(c, DFLASH_K_QKV_POST, st, [&] {
      return launch_qkv_post(sc.part, parts(c->g_qkv).first, (long long)M * c->g_qkv.N, parts(c->g_qkv).second,
                             M, gamma, c->bands_dev,
                             c->nh, c->nkv, c->hd, d.q_norm, d.k_norm, c->eps, c->inv_freq,
                             (float)c->mscale, c->slots, g, l, c->Qb, c->Qb_lo, st);
    }));
    // the debug seam's copies (dflash_debug_capture): device-to-device, stream-ordered
    auto capture = [&](void* dst, const void* src, size_t row_bytes) -> hipError_t {
      if (!c->cap_on || noalloc) return hipSuccess;
      return hipMemcpyAsync((char*)dst + (size_t)l * c->m_max * row_bytes, src, (size_t)M * row_bytes,
                            hipMemcpyDeviceToDevice, st);
    };
    HIPCHK(c, capture(c->cap_q, c->Qb, (size_t)c->qd * 2));
    HIPCHK(c, capture(c->cap_q_lo, c->Qb_lo, (size_t)c->qd * 2));
    HIPCHK(c, timed(c, DFLASH_K_ATTN, st, [&] {
      return launch_block_attn(c->Qb, c->Qb_lo, ab[sw], ab_reg[sw], ab_lds[sw], gamma, c->nh, g, l, sw,
                               sw ? c->window : 0, scale_log2, sc.aparts_o, sc.aparts_ml, st);
    }));
    HIPCHK(c, timed(c, DFLASH_K_ATTN_COMBINE, st, [&] {
      int max_nch = 1;
      for (int b = 0; b < n_seqs; ++b) max_nch = std::max(max_nch, a.bands[b].nch[sw]);
      return launch_attn_combine(sc.aparts_o, sc.aparts_ml, c->bands_dev, n_seqs, max_nch, gamma, c->nh,
                                 c->nkv, c->hd, sw, c->attn, c->attn_lo, st);
    }));
    HIPCHK(c, capture(c->cap_a, c->attn, (size_t)c->qd * 2));
    HIPCHK(c, capture(c->cap_a_lo, c->attn_lo, (size_t)c->qd * 2));
    HIPCHK(c, gemm(c->attn, c->attn_lo, c->qd, q8 ? (const bf16*)d.q_o : d.o_proj, q8 ? d.s_o : nullptr, c->g_o, false));
    HIPCHK(c, timed(c, DFLASH_K_RESID_NORM, st, [&] {
      if (c->d2)
        return launch_resid_dconv(c->X, sc.part, parts(c->g_o).first, (long long)M * c->g_o.N, parts(c->g_o).second,
                                  M, c->h, gamma, c->dyn_a, d.cba, d.post_norm, c->ssq, c->Xn, c->Xn_lo, st);
      return launch_resid_sum(c->X, sc.part, parts(c->g_o).first, (long long)M * c->g_o.N, parts(c->g_o).second,
                              M, c->h, d.post_norm, c->ssq, c->Xn, c->Xn_lo, st);
    }));
    HIPCHK(c, capture(c->cap_x1, c->X, (size_t)c->h * 4));
    if (c->d2) HIPCHK(c, dconv_site(d.w_cpm, d.cbm, c->dyn_m));
    HIPCHK(c, gemm(c->d2 ? c->U : c->Xn, c->d2 ? c->U_lo : c->Xn_lo, c->h, q8 ? (const bf16*)d.q_gu : d.w_gu,
                   q8 ? d.s_gu : nullptr, c->g_gu, !c->d2));
    HIPCHK(c, timed(c, DFLASH_K_SILU, st, [&] {
      return launch_silu_mul(sc.part, parts(c->g_gu).first, (long long)M * c->g_gu.N, parts(c->g_gu).second, M,
                             c->ff, c->act, c->act_lo, st);
    }));
    HIPCHK(c, gemm(c->act, c->act_lo, c->ff, q8 ? (const bf16*)d.q_down : d.down_proj, q8 ? d.s_down : nullptr,
                   c->g_down, false));
    if (c->d2) {
      // the MLP output through the finish application, then (after the last layer) the
      // final norm of the residual rows
      const bf16* nw = l + 1 < c->L ? c->layers[l + 1].in_norm : c->norm;
      HIPCHK(c, timed(c, DFLASH_K_RESID_NORM, st, [&] {
        return launch_resid_dconv(c->X, sc.part, parts(c->g_down).first, (long long)M * c->g_down.N,
                                  parts(c->g_down).second, M, c->h, gamma, c->dyn_m, d.cbm, nw, c->ssq, c->Xn,
                                  c->Xn_lo, st);
      }));
      if (l + 1 == c->L)
        HIPCHK(c, timed(c, DFLASH_K_RESID_NORM, st, [&] {
          return launch_rows_rmsnorm(c->X, 1, 0, 1, M, c->h, c->norm, c->eps, c->Xn, c->Xn_lo, st);
        }));
    } else if (l + 1 < c->L) {
      HIPCHK(c, timed(c, DFLASH_K_RESID_NORM, st, [&] {
        return launch_resid_sum(c->X, sc.part, parts(c->g_down).first, (long long)M * c->g_down.N,
                                parts(c->g_down).second, M, c->h, c->layers[l + 1].in_norm, c->ssq, c->Xn,
                                c->Xn_lo, st);
      }));
    } else {
      // the last residual add also applies the final norm: the lm_head's rows (hi + lo)
      HIPCHK(c, timed(c, DFLASH_K_RESID_NORM, st, [&] {
        return launch_resid_norm(c->X, sc.part, parts(c->g_down).first, (long long)M * c->g_down.N,
                                 parts(c->g_down).second, M, c->h, c->norm, c->eps, c->Xn, c->Xn_lo, st);
      }));
    }
    HIPCHK(c, capture(c->cap_x, c->X, (size_t)c->h * 4));
  }
  // one row group of at most 16 rows with the rows in LDS whole: the persistent lm_head;
  // more than one row group (or FP8 weights beyond the persistent form): the wide lm_head;
  // otherwise one launch per row group
  const int ng_p = lmhead_persistent_groups(c->V, c->h, M, c->n_cu);
  const bool lm_wide = wide || (c->fp8 && ng_p == 0);
  const int ng = lm_wide ? lmhead_wide_groups(c->V) : ng_p > 0 ? std::min(ng_p, c->lm_groups) : c->lm_groups;
  const bf16* lmw = c->fp8 ? (const bf16*)c->lm_q : c->lm_head;
  const float* lms = c->fp8 ? c->lm_s : nullptr;
  // a Markov head and DFlash2's candidates need every drafted row's logits: the caller's
  // buffer, else the context's
  float* const user_logits = logits;
  if ((c->R || c->d2) && !logits) logits = c->mk_logits;
  if (lm_wide) {
    HIPCHK(c, timed(c, DFLASH_K_LMHEAD, st, [&] {
      return launch_lmhead_wide(c->Xn, c->Xn_lo, c->h, M, lmw, c->V, c->h, sc.best_v, sc.best_i, ng, gamma,
                                logits, st, lms);
    }));
  } else if (ng_p > 0) {
    HIPCHK(c, timed(c, DFLASH_K_LMHEAD, st, [&] {
      return launch_lmhead_persistent(c->Xn, c->Xn_lo, c->h, M, 0, lmw, c->V, c->h, sc.best_v, sc.best_i,
                                      ng, gamma, logits, st, lms);
    }));
  } else {
    for (int r0 = 0; r0 < M; r0 += ROW_GROUP) {
      const int mg = std::min(ROW_GROUP, M - r0);
      HIPCHK(c, timed(c, DFLASH_K_LMHEAD, st, [&] {
        return launch_lmhead_argmax(c->Xn + (size_t)r0 * c->h, c->Xn_lo + (size_t)r0 * c->h, c->h, mg, r0,
                                    c->lm_head, c->V, c->h,
                                    sc.best_v, sc.best_i, ng, gamma, logits, st);
      }));
    }
  }
  if (c->d2) {
    // the selector's hidden projection of the final-normed rows, the top-16 candidates of
    // every drafted row, their pair scores and the walk
    HIPCHK(c, gemm(c->Xn, c->Xn_lo, c->h, c->sel_h, nullptr, c->g_sh, false));
    SelectorBonus sb{};
    for (int b = 0; b < n_seqs; ++b) sb.t[b] = bonus[b];
    const int drafted = n_seqs * (gamma - 1);
    HIPCHK(c, timed(c, DFLASH_K_SELECTOR, st, [&] {
      return launch_topk_partial(logits, drafted, c->V, c->tk_v, c->tk_i, st);
    }));
    HIPCHK(c, timed(c, DFLASH_K_SELECTOR, st, [&] {
      return launch_selector_pairs(c->tk_v, c->tk_i, sc.part, parts(c->g_sh).first, (long long)M * c->g_sh.N,
                                   parts(c->g_sh).second, c->sel_rank, n_seqs, gamma, sb, c->sel_pred, c->sel_succ,
                                   c->V, c->sel_v, c->sel_i, c->sel_pair, st);
    }));
    HIPCHK(c, timed(c, DFLASH_K_SELECTOR, st, [&] {
      return launch_selector_walk(c->sel_i, c->sel_pair, n_seqs, gamma, draft_tokens, st);
    }));
    return DFLASH_OK;
  }
  if (!c->R) {
    HIPCHK(c, timed(c, DFLASH_K_ARGMAX, st, [&] {
      return launch_argmax_reduce(sc.best_v, sc.best_i, ng, n_seqs, gamma, draft_tokens, st);
    }));
    return DFLASH_OK;
  }
  // DSpark: the drafted rows one after another, each biased by the previous draft's row of
  // the Markov head and reduced to its draft (the lm_head's own argmax is not used)
  MarkovStep ms{};
  ms.w1 = c->mk_w1; ms.w2t = c->mk_w2t; ms.logits = logits; ms.best = c->mk_best;
  ms.V = c->V; ms.R = c->R; ms.n = n_seqs; ms.gamma = gamma; ms.store = user_logits != nullptr;
  for (int b = 0; b < n_seqs; ++b) ms.bonus[b] = bonus[b];
  for (int k = 0; k < gamma - 1; ++k) {
    ms.k = k;
    HIPCHK(c, timed(c, DFLASH_K_MARKOV, st, [&] { return launch_markov_step(ms, c->mk_groups, st); }));
  }
  HIPCHK(c, timed(c, DFLASH_K_ARGMAX, st, [&] { return launch_markov_finish(c->mk_best, n_seqs, gamma, draft_tokens, st); }));
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int dflash_block_forward(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int32_t* bonus,
                         const int32_t* q_rope_pos, int32_t gamma, int32_t* draft_tokens,
                         float* logits, void* stream) {
  return block_forward(c, n_seqs, seqs, bonus, q_rope_pos, gamma, draft_tokens, logits, stream, false);
}

int dflash_block_forward_noalloc(dflash_ctx* c, int32_t n_seqs, const int32_t* seqs, const int32_t* bonus,
                                 const int32_t* q_rope_pos, int32_t gamma, int32_t* draft_tokens,
                                 float* logits, void* stream) {
  if (!c) return DFLASH_EINVAL;
  // launch timing would create events: it is off for this call
  const uint32_t tmask = c->tmask;
  c->tmask = 0;
  const int rc = block_forward(c, n_seqs, seqs, bonus, q_rope_pos, gamma, draft_tokens, logits, stream, true);
  c->tmask = tmask;
  return rc;
}

int dflash_debug_capture(dflash_ctx* c, int32_t on) {
  if (!c) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  if (on && !c->cap_q) {
    const size_t rows = (size_t)c->L * c->m_max;
    int rc;
    if ((rc = dalloc(c, &c->cap_q, rows * c->qd)) || (rc = dalloc(c, &c->cap_q_lo, rows * c->qd)) ||
        (rc = dalloc(c, &c->cap_a, rows * c->qd)) || (rc = dalloc(c, &c->cap_a_lo, rows * c->qd)) ||
        (rc = dalloc(c, &c->cap_x1, rows * c->h)) || (rc = dalloc(c, &c->cap_x, rows * c->h)))
      return rc;
  }
  c->cap_on = on != 0;
  return DFLASH_OK;
}

int dflash_timing(dflash_ctx* c, uint32_t class_mask) {
  if (!c) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  c->tmask = class_mask & ((1u << DFLASH_K_NUM_CLASSES) - 1u);
  return DFLASH_OK;
}

int dflash_timing_read(dflash_ctx* c, double* ms, int64_t* launches, int32_t n_classes) {
  if (!c) return DFLASH_EINVAL;
  if (c->poisoned) return fail(c, DFLASH_EHIP, "context unusable after an earlier HIP error");
  HIPCHK(c, timing_harvest(c));
  for (int i = 0; i < n_classes && i < DFLASH_K_NUM_CLASSES; ++i) {
    if (ms) ms[i] = c->tms[i];
    if (launches) launches[i] = c->tcnt[i];
  }
  for (int i = 0; i < DFLASH_K_NUM_CLASSES; ++i) { c->tms[i] = 0.0; c->tcnt[i] = 0; }
  return DFLASH_OK;
}

}  // extern "C"
