// Host-side memory and undefined-behaviour check of the drafter library's runtime.
//
// Built with AddressSanitizer and UndefinedBehaviorSanitizer on the runtime's host code
// (runtime.hip compiled with those sanitizers for the host pass only; the kernels and their
// device code are the library's own), this program drives every entry point of dflash.h
// through its success and refusal paths, so that an out-of-bounds host access, a use after
// free, a leak of the runtime's own allocations or an undefined operation in the allocator,
// the chunk planner, the configuration checks or the argument checks ends the run with a
// sanitizer report.
//
//   abi_check cpu   no device needed: the attention planner's band tables over random band
//                   sets, error names, every configuration refusal, the NULL handle paths,
//                   and (only where no device is present) create's unwind when the device
//                   cannot be used; nothing is enqueued
//   abi_check gpu   on a GPU: bf16, FP8, Markov-head and DFlash2 drafters; single and
//                   batched appends; forwards of several widths and band sets (results
//                   bit for bit equal band by band and between the two forward entry
//                   points); the capture seam, timing, resets, pool exhaustion and every
//                   argument refusal, each leaving the sequence state unchanged
//
// Prints "abi_check <mode> ok" and exits 0; a failed check prints what failed and exits 1.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <algorithm>
#include <string>
#include <vector>

#include "dflash.h"
#include "kernels.hpp"   // the attention planner's band table (dfl::plan_attn)

namespace {

int g_fail = 0;

#define CHECK(cond, ...)                                       \
  do {                                                         \
    if (!(cond)) {                                             \
      std::fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                       \
      std::fprintf(stderr, "\n");                              \
      ++g_fail;                                                \
    }                                                          \
  } while (0)

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(1);                                                        \
    }                                                                      \
  } while (0)

// deterministic bf16 bit patterns: uniform in [-a, a] (a > 0) or 1 + [-0.1, 0.1] (a == 0)
struct Lcg {
  uint64_t s;
  explicit Lcg(uint64_t seed) : s(seed * 6364136223846793005ULL + 1442695040888963407ULL) {}
  float next() {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((s >> 40) & 0xffffff) / 16777216.0f * 2.0f - 1.0f;
  }
};

uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fff + ((u >> 16) & 1);
  return (uint16_t)(u >> 16);
}

struct Model {
  int L, h, nh, nkv, hd, ff, V, taps, th, gmax;
};
// the shapes of the parity tests' small drafters: a 16:2-head, head_dim-128 one (both
// attention paths) and a 8:2-head, head_dim-32 one
const Model kWide128 = {2, 512, 16, 2, 128, 1024, 2048, 2, 512, 16};
const Model kTiny = {2, 256, 8, 2, 32, 512, 1024, 3, 256, 16};

// every device buffer of one drafter's weights, freed at the end
struct Weights {
  std::vector<void*> bufs;
  std::vector<dflash_layer_weights> layers;
  dflash_weights w{};
  uint64_t seed = 1;

  void* bf16_buf(size_t n, float a) {
    std::vector<uint16_t> h(n);
    Lcg g(seed++);
    for (size_t i = 0; i < n; ++i) h[i] = to_bf16(a > 0 ? a * g.next() : 1.0f + 0.1f * g.next());
    void* d = nullptr;
    HIP_OK(hipMalloc(&d, n * 2));
    HIP_OK(hipMemcpy(d, h.data(), n * 2, hipMemcpyHostToDevice));
    bufs.push_back(d);
    return d;
  }
  void build(const Model& m, int markov_rank, int selector_rank) {
    const size_t qd = (size_t)m.nh * m.hd, kvd = (size_t)m.nkv * m.hd;
    w.fc = bf16_buf((size_t)m.h * m.taps * m.th, 0.05f);
    w.hidden_norm = bf16_buf(m.h, 0);
    w.norm = bf16_buf(m.h, 0);
    w.embed_tokens = bf16_buf((size_t)m.V * m.h, 0.5f);
    w.lm_head = bf16_buf((size_t)m.V * m.h, 0.06f);
    layers.resize(m.L);
    for (auto& l : layers) {
      l = dflash_layer_weights{};
      l.q_proj = bf16_buf(qd * m.h, 0.06f);
      l.k_proj = bf16_buf(kvd * m.h, 0.06f);
      l.v_proj = bf16_buf(kvd * m.h, 0.06f);
      l.o_proj = bf16_buf(m.h * qd, 0.04f);
      l.q_norm = bf16_buf(m.hd, 0);
      l.k_norm = bf16_buf(m.hd, 0);
      l.input_layernorm = bf16_buf(m.h, 0);
      l.post_attention_layernorm = bf16_buf(m.h, 0);
      l.gate_proj = bf16_buf((size_t)m.ff * m.h, 0.06f);
      l.up_proj = bf16_buf((size_t)m.ff * m.h, 0.06f);
      l.down_proj = bf16_buf((size_t)m.h * m.ff, 0.04f);
      if (selector_rank) {
        l.attention_conv_base = bf16_buf((size_t)2 * 2 * m.h, 0.3f);
        l.attention_conv_proj = bf16_buf((size_t)2 * 2 * m.h / 16 * m.h, 0.02f);
        l.mlp_conv_base = bf16_buf((size_t)2 * 2 * m.h, 0.3f);
        l.mlp_conv_proj = bf16_buf((size_t)2 * 2 * m.h / 16 * m.h, 0.02f);
      }
    }
    w.layers = layers.data();
    if (markov_rank) {
      w.markov_w1 = bf16_buf((size_t)m.V * markov_rank, 0.1f);
      w.markov_w2 = bf16_buf((size_t)m.V * markov_rank, 0.1f);
    }
    if (selector_rank) {
      w.selector_pred = bf16_buf((size_t)m.V * selector_rank, 0.1f);
      w.selector_succ = bf16_buf((size_t)m.V * selector_rank, 0.1f);
      w.selector_hidden_proj = bf16_buf((size_t)selector_rank * m.h, 0.05f);
    }
  }
  ~Weights() {
    for (void* p : bufs) (void)hipFree(p);
  }
};

dflash_config base_config(const Model& m, int max_seq, int max_batch) {
  dflash_config c{};
  c.num_layers = m.L; c.hidden = m.h; c.num_q_heads = m.nh; c.num_kv_heads = m.nkv; c.head_dim = m.hd;
  c.intermediate = m.ff; c.vocab = m.V; c.num_taps = m.taps; c.target_hidden = m.th; c.gamma_max = m.gmax;
  c.mask_token_id = m.V - 1; c.rms_eps = 1e-6f; c.rope_theta = 1e6; c.rope_type = 0;
  c.max_seq_len = max_seq; c.max_batch = max_batch;
  return c;
}

// ---- no device ------------------------------------------------------------------------------

// dfl::plan_attn, the attention launch's band table: over seeded random band sets, the register
// path's chunk bases must tile its chunks, and the LDS path's dispatch runs must hold each of
// its chunks exactly once, in order of non-increasing length (any order computes the same
// bits; a chunk missed or taken twice would not)
void check_attn_plan() {
  uint64_t s = 12345;
  auto rnd = [&](int n) {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (int)((s >> 33) % (uint64_t)n);
  };
  int bad = 0;
  for (int it = 0; it < 4000; ++it) {
    const int n = 1 + rnd(dfl::MAX_BANDS), gamma = 1 + rnd(16);
    dfl::Band bands[dfl::MAX_BANDS] = {};
    for (int b = 0; b < n; ++b) {
      dfl::Band& B = bands[b];
      B.seq = b;
      B.kv_len = rnd(it % 3 == 0 ? 40000 : 9000);
      const int pages = (B.kv_len + gamma + dfl::PAGE - 1) / dfl::PAGE;
      const int ckp = 16 * std::max(1 + rnd(12), (pages + 16 * 32 - 1) / (16 * 32));   // at most 32 chunks
      B.ck[0] = ckp * dfl::PAGE;
      B.nch[0] = (pages + ckp - 1) / ckp;
    }
    dfl::AttnBands ab;
    int reg = 0, lds = 0;
    dfl::plan_attn(bands, n, 0, 128, 0, true, gamma, ab, reg, lds);
    std::vector<int> seen_reg, seen_lds;
    int want_reg = 0, want_lds = 0;
    for (int b = 0; b < n; ++b) {
      const bool on_lds = (ab.lds_mask >> b) & 1u;
      const int pages = (bands[b].kv_len + gamma + dfl::PAGE - 1) / dfl::PAGE;
      bool ok = on_lds == (pages > dfl::ATTN_LDS_MIN_PAGES);
      if (on_lds) want_lds += bands[b].nch[0];
      else {
        want_reg += bands[b].nch[0];
        for (int c = 0; c < bands[b].nch[0]; ++c) seen_reg.push_back(ab.dbase[b] + c);
      }
      if (!ok) ++bad;
    }
    int prev = 1 << 30;
    bool ok = ab.n_lg <= 2 * dfl::MAX_BANDS && (lds == 0 || (ab.n_lg > 0 && ab.lg_start[0] == 0 && ab.lg_start[ab.n_lg] == lds));
    for (int g = 0; ok && g < ab.n_lg; ++g) {
      const int b = ab.lg_band[g];
      ok = b < n && ((ab.lds_mask >> b) & 1u) && ab.lg_start[g + 1] > ab.lg_start[g];
      for (int d = ab.lg_start[g]; ok && d < ab.lg_start[g + 1]; ++d) {
        const int c = ab.lg_chunk[g] + (d - ab.lg_start[g]);
        const dfl::Band& B = bands[b];
        const int len = std::min(B.ck[0], B.kv_len + gamma - B.kstart[0] - c * B.ck[0]);
        ok = c < B.nch[0] && len > 0 && len <= prev;
        prev = len;
        seen_lds.push_back(b * 256 + c);
      }
    }
    std::sort(seen_reg.begin(), seen_reg.end());
    std::sort(seen_lds.begin(), seen_lds.end());
    for (int i = 0; ok && i < (int)seen_reg.size(); ++i) ok = seen_reg[i] == i;
    ok = ok && reg == want_reg && lds == want_lds && (int)seen_lds.size() == want_lds &&
         std::adjacent_find(seen_lds.begin(), seen_lds.end()) == seen_lds.end();
    if (!ok) ++bad;
  }
  CHECK(bad == 0, "attention planner: %d of 4000 random band sets planned wrongly", bad);
}

int run_cpu() {
  check_attn_plan();
  for (int code : {(int)DFLASH_OK, (int)DFLASH_EINVAL, (int)DFLASH_ENOMEM, (int)DFLASH_EPOOL, (int)DFLASH_ERANGE,
                   (int)DFLASH_EHIP, 7, -99})
    CHECK(dflash_strerror(code) != nullptr && std::strlen(dflash_strerror(code)) > 0, "strerror %d", code);
  CHECK(std::string(dflash_last_error(nullptr)).empty(), "last_error(NULL)");

  // host stand-ins for the weights (aligned, non-NULL): every call below that gets them is
  // refused before anything reads them
  alignas(16) static uint8_t fake[256];
  const Model m = kTiny;
  std::vector<dflash_layer_weights> lw(m.L);
  for (auto& l : lw) {
    l = dflash_layer_weights{};
    l.q_proj = l.k_proj = l.v_proj = l.o_proj = l.q_norm = l.k_norm = fake;
    l.input_layernorm = l.post_attention_layernorm = l.gate_proj = l.up_proj = l.down_proj = fake;
  }
  dflash_weights w{};
  w.fc = w.hidden_norm = w.norm = w.embed_tokens = w.lm_head = fake;
  w.layers = lw.data();
  dflash_ctx* ctx = reinterpret_cast<dflash_ctx*>(0x1);
  CHECK(dflash_create(nullptr, &w, nullptr, &ctx) == DFLASH_EINVAL && ctx == nullptr, "NULL config");
  const dflash_config good = base_config(m, 512, 2);
  CHECK(dflash_create(&good, nullptr, nullptr, &ctx) == DFLASH_EINVAL, "NULL weights");
  CHECK(dflash_create(&good, &w, nullptr, nullptr) == DFLASH_EINVAL, "NULL out");

  struct Bad { const char* what; void (*edit)(dflash_config&); };
  const Bad bad[] = {
      {"layers 0", [](dflash_config& c) { c.num_layers = 0; }},
      {"head_dim 96", [](dflash_config& c) { c.head_dim = 96; }},
      {"heads not a multiple", [](dflash_config& c) { c.num_q_heads = 3; }},
      {"group of 16", [](dflash_config& c) { c.num_q_heads = 32; c.num_kv_heads = 2; }},
      {"gamma 1", [](dflash_config& c) { c.gamma_max = 1; }},
      {"gamma 17", [](dflash_config& c) { c.gamma_max = 17; }},
      {"hidden 8448", [](dflash_config& c) { c.hidden = 8448; }},
      {"hidden 200", [](dflash_config& c) { c.hidden = 200; }},
      {"mask id", [](dflash_config& c) { c.mask_token_id = c.vocab; }},
      {"max_batch 0", [](dflash_config& c) { c.max_batch = 0; }},
      {"max_batch 33", [](dflash_config& c) { c.max_batch = 33; }},
      {"max_seq 0", [](dflash_config& c) { c.max_seq_len = 0; }},
      {"max_seq huge", [](dflash_config& c) { c.max_seq_len = 262144; }},
      {"eps NaN", [](dflash_config& c) { c.rms_eps = std::numeric_limits<float>::quiet_NaN(); }},
      {"theta 1", [](dflash_config& c) { c.rope_theta = 1.0; }},
      {"rope type", [](dflash_config& c) { c.rope_type = 2; }},
      {"yarn params", [](dflash_config& c) { c.rope_type = 1; c.yarn_factor = 0; }},
      {"weight format", [](dflash_config& c) { c.weight_format = 5; }},
      {"markov rank", [](dflash_config& c) { c.markov_rank = 128; }},
      {"markov tables", [](dflash_config& c) { c.markov_rank = 256; }},
      {"dflash2 sizes", [](dflash_config& c) { c.conv_kernel_size = 3; c.conv_group_size = 16; c.selector_rank = 256; c.selector_top_k = 16; }},
      {"dflash2 weights", [](dflash_config& c) { c.conv_kernel_size = 2; c.conv_group_size = 16; c.selector_rank = 256; c.selector_top_k = 16; }},
      {"window", [](dflash_config& c) { c.sliding_window = -1; }},
      {"num_pages 1", [](dflash_config& c) { c.num_pages = 1; }},
  };
  for (const Bad& b : bad) {
    dflash_config c = good;
    b.edit(c);
    ctx = reinterpret_cast<dflash_ctx*>(0x1);
    CHECK(dflash_create(&c, &w, nullptr, &ctx) == DFLASH_EINVAL && ctx == nullptr, "config '%s' accepted", b.what);
  }
  {  // a misaligned matrix and a NULL layer weight
    dflash_weights w2 = w;
    w2.lm_head = fake + 2;
    CHECK(dflash_create(&good, &w2, nullptr, &ctx) == DFLASH_EINVAL, "misaligned lm_head accepted");
    std::vector<dflash_layer_weights> lw2 = lw;
    lw2[1].down_proj = nullptr;
    w2 = w;
    w2.layers = lw2.data();
    CHECK(dflash_create(&good, &w2, nullptr, &ctx) == DFLASH_EINVAL, "NULL layer weight accepted");
  }
  {  // a page order that is not a permutation: refused after the free list is built
    dflash_config c = good;
    c.num_pages = 6;
    const int32_t order[5] = {1, 2, 2, 4, 5};
    c.page_order = order;
    ctx = reinterpret_cast<dflash_ctx*>(0x1);
    CHECK(dflash_create(&c, &w, nullptr, &ctx) == DFLASH_EINVAL && ctx == nullptr, "page order with a repeat");
    const int32_t order2[5] = {1, 2, 3, 4, 6};
    c.page_order = order2;
    CHECK(dflash_create(&c, &w, nullptr, &ctx) == DFLASH_EINVAL, "page order out of range");
  }
  // a valid configuration without a usable device: create unwinds what it built. Only where
  // no device is present: with one, create would run its weight copies on these host
  // stand-ins, which no device code may read
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
    ctx = reinterpret_cast<dflash_ctx*>(0x1);
    const int rc = dflash_create(&good, &w, nullptr, &ctx);
    CHECK(rc != DFLASH_OK && ctx == nullptr, "create without a device returned %d", rc);
  }
  // NULL handles
  int32_t seq = 0, bonus = 1, toks[15];
  CHECK(dflash_ctx_kv_append(nullptr, 0, fake, nullptr, 1, nullptr) == DFLASH_EINVAL, "append(NULL)");
  CHECK(dflash_ctx_kv_append_batch(nullptr, 1, &seq, &seq, fake, nullptr, nullptr) == DFLASH_EINVAL, "append_batch(NULL)");
  CHECK(dflash_block_forward(nullptr, 1, &seq, &bonus, nullptr, 16, toks, nullptr, nullptr) == DFLASH_EINVAL, "forward(NULL)");
  CHECK(dflash_block_forward_noalloc(nullptr, 1, &seq, &bonus, nullptr, 16, toks, nullptr, nullptr) == DFLASH_EINVAL, "noalloc(NULL)");
  CHECK(dflash_seq_reset(nullptr, 0) == DFLASH_EINVAL, "reset(NULL)");
  CHECK(dflash_seq_info(nullptr, 0, nullptr, nullptr, nullptr, 0) != DFLASH_OK, "info(NULL)");
  CHECK(dflash_pool_geometry(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == DFLASH_EINVAL, "geometry(NULL)");
  CHECK(dflash_debug_copy(nullptr, 0, fake, 0, 1, nullptr) == DFLASH_EINVAL, "debug_copy(NULL)");
  CHECK(dflash_debug_capture(nullptr, 1) == DFLASH_EINVAL, "capture(NULL)");
  CHECK(dflash_timing(nullptr, 1) == DFLASH_EINVAL, "timing(NULL)");
  CHECK(dflash_timing_read(nullptr, nullptr, nullptr, 0) == DFLASH_EINVAL, "timing_read(NULL)");
  dflash_destroy(nullptr);
  return g_fail;
}

// ---- on a GPU -------------------------------------------------------------------------------

struct SeqSnap {
  int32_t kv_len = -1, n_pages = -1;
  std::vector<int32_t> bt;
  bool operator==(const SeqSnap& o) const { return kv_len == o.kv_len && n_pages == o.n_pages && bt == o.bt; }
};

SeqSnap snap(dflash_ctx* c, int seq) {
  SeqSnap s;
  s.bt.assign(4096, -1);
  (void)dflash_seq_info(c, seq, &s.kv_len, &s.n_pages, s.bt.data(), (int32_t)s.bt.size());
  s.bt.resize(s.n_pages > 0 ? s.n_pages : 0);
  return s;
}

struct Dev {
  void* p = nullptr;
  explicit Dev(size_t bytes) { HIP_OK(hipMalloc(&p, bytes)); }
  ~Dev() { (void)hipFree(p); }
};

void* hidden_rows(const Model& m, int n, uint64_t seed, std::vector<void*>& keep) {
  std::vector<uint16_t> h((size_t)n * m.taps * m.th);
  Lcg g(seed);
  for (auto& x : h) x = to_bf16(g.next());
  void* d = nullptr;
  HIP_OK(hipMalloc(&d, h.size() * 2));
  HIP_OK(hipMemcpy(d, h.data(), h.size() * 2, hipMemcpyHostToDevice));
  keep.push_back(d);
  return d;
}

struct Out {
  std::vector<int32_t> toks;
  std::vector<float> logits;
  bool operator==(const Out& o) const {
    return toks == o.toks && logits.size() == o.logits.size() &&
           std::memcmp(logits.data(), o.logits.data(), logits.size() * 4) == 0;
  }
};

int forward(dflash_ctx* c, const Model& m, const std::vector<int32_t>& seqs, const std::vector<int32_t>& bonus,
            int gamma, bool noalloc, Out* out, const int32_t* qpos = nullptr) {
  const int n = (int)seqs.size();
  Dev t((size_t)n * (gamma - 1) * 4), l((size_t)n * (gamma - 1) * m.V * 4);
  const int rc = (noalloc ? dflash_block_forward_noalloc : dflash_block_forward)(
      c, n, seqs.data(), bonus.data(), qpos, gamma, (int32_t*)t.p, (float*)l.p, nullptr);
  if (rc == DFLASH_OK && out) {
    out->toks.resize((size_t)n * (gamma - 1));
    out->logits.resize((size_t)n * (gamma - 1) * m.V);
    HIP_OK(hipMemcpy(out->toks.data(), t.p, out->toks.size() * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out->logits.data(), l.p, out->logits.size() * 4, hipMemcpyDeviceToHost));
  }
  HIP_OK(hipDeviceSynchronize());
  return rc;
}

// one drafter through appends, forwards and refusals
void exercise(const char* name, const Model& m, dflash_config cfg, int markov_rank, int selector_rank) {
  std::fprintf(stderr, "-- %s\n", name);
  Weights W;
  W.build(m, markov_rank, selector_rank);
  cfg.markov_rank = markov_rank;
  if (selector_rank) {
    cfg.conv_kernel_size = 2; cfg.conv_group_size = 16; cfg.selector_rank = selector_rank; cfg.selector_top_k = 16;
  }
  dflash_ctx* c = nullptr;
  int rc = dflash_create(&cfg, &W.w, nullptr, &c);
  CHECK(rc == DFLASH_OK && c, "%s: create %d", name, rc);
  if (!c) return;
  std::vector<void*> keep;
  const int nb = cfg.max_batch < 4 ? cfg.max_batch : 4;
  // appends: one long sequence in pieces, with explicit (spread) positions, the rest batched
  const int long_rows = cfg.max_seq_len - 64;
  int done = 0;
  while (done < long_rows) {
    const int n = std::min(1500, long_rows - done);
    std::vector<int32_t> pos(n);
    for (int i = 0; i < n; ++i) pos[i] = 3 * (done + i);
    rc = dflash_ctx_kv_append(c, 0, hidden_rows(m, n, 100 + done, keep), pos.data(), n, nullptr);
    CHECK(rc == DFLASH_OK, "%s: append %d rows at %d: %d (%s)", name, n, done, rc, dflash_last_error(c));
    if (rc != DFLASH_OK) break;
    done += n;
  }
  if (nb > 1) {
    std::vector<int32_t> seqs, counts;
    int tot = 0;
    for (int s = 1; s < nb; ++s) { seqs.push_back(s); counts.push_back(17 + 20 * s); tot += 17 + 20 * s; }
    rc = dflash_ctx_kv_append_batch(c, (int32_t)seqs.size(), seqs.data(), counts.data(), hidden_rows(m, tot, 7, keep),
                                    nullptr, nullptr);
    CHECK(rc == DFLASH_OK, "%s: batched append %d (%s)", name, rc, dflash_last_error(c));
  }
  HIP_OK(hipDeviceSynchronize());
  // forwards: all bands, each band alone (bit for bit), and the no-allocation entry point
  std::vector<int32_t> seqs, bonus;
  for (int s = 0; s < nb; ++s) { seqs.push_back(s); bonus.push_back(11 + 97 * s); }
  for (int gamma : {16, 5, 2}) {
    Out all, na;
    rc = forward(c, m, seqs, bonus, gamma, false, &all);
    CHECK(rc == DFLASH_OK, "%s: forward gamma %d: %d (%s)", name, gamma, rc, dflash_last_error(c));
    rc = forward(c, m, seqs, bonus, gamma, true, &na);
    CHECK(rc == DFLASH_OK && na == all, "%s: no-allocation forward gamma %d differs (rc %d)", name, gamma, rc);
    for (int b = 0; b < nb && rc == DFLASH_OK; ++b) {
      Out one;
      rc = forward(c, m, {seqs[b]}, {bonus[b]}, gamma, false, &one);
      const size_t t0 = (size_t)b * (gamma - 1), tn = gamma - 1;
      bool same = rc == DFLASH_OK &&
                  std::equal(one.toks.begin(), one.toks.end(), all.toks.begin() + t0) &&
                  std::memcmp(one.logits.data(), all.logits.data() + t0 * m.V, tn * m.V * 4) == 0;
      CHECK(same, "%s: band %d alone differs at gamma %d", name, b, gamma);
    }
    for (int32_t t : all.toks) CHECK(t >= 0 && t < m.V, "%s: token %d out of range", name, t);
  }
  {  // RoPE positions past kv_len
    std::vector<int32_t> qp;
    for (int s = 0; s < nb; ++s) qp.push_back(snap(c, s).kv_len + 40 * s);
    rc = forward(c, m, seqs, bonus, 16, false, nullptr, qp.data());
    CHECK(rc == DFLASH_OK, "%s: forward with positions: %d", name, rc);
  }
  // capture seam and debug copies
  CHECK(dflash_debug_capture(c, 1) == DFLASH_OK, "%s: capture on", name);
  rc = forward(c, m, {0}, {5}, 16, false, nullptr);
  CHECK(rc == DFLASH_OK, "%s: captured forward", name);
  std::vector<uint8_t> host(1 << 20);
  for (int buf : {DFLASH_BUF_POOL, DFLASH_BUF_KPOS, DFLASH_BUF_SLOTS, DFLASH_BUF_BLOCKTAB, DFLASH_BUF_HIDDEN,
                  DFLASH_BUF_HIDDEN_LO, DFLASH_BUF_CTX_FEAT, DFLASH_BUF_CTX_FEAT_LO, DFLASH_BUF_LAYER_Q,
                  DFLASH_BUF_LAYER_Q_LO, DFLASH_BUF_LAYER_ATTN, DFLASH_BUF_LAYER_ATTN_LO, DFLASH_BUF_LAYER_X1,
                  DFLASH_BUF_LAYER_X}) {
    rc = dflash_debug_copy(c, buf, host.data(), 0, 256, nullptr);
    CHECK(rc == DFLASH_OK, "%s: debug_copy %d: %d (%s)", name, buf, rc, dflash_last_error(c));
    CHECK(dflash_debug_copy(c, buf, host.data(), (size_t)1 << 40, 16, nullptr) != DFLASH_OK, "%s: copy past the end", name);
  }
  CHECK(dflash_debug_copy(c, 99, host.data(), 0, 16, nullptr) != DFLASH_OK, "%s: unknown buffer", name);
  CHECK(dflash_debug_capture(c, 0) == DFLASH_OK, "%s: capture off", name);
  // timing
  CHECK(dflash_timing(c, 0xffffffffu) == DFLASH_OK, "%s: timing on", name);
  rc = forward(c, m, seqs, bonus, 16, false, nullptr);
  double ms[DFLASH_K_NUM_CLASSES];
  int64_t launches[DFLASH_K_NUM_CLASSES];
  CHECK(dflash_timing_read(c, ms, launches, DFLASH_K_NUM_CLASSES) == DFLASH_OK, "%s: timing read", name);
  CHECK(launches[DFLASH_K_GEMM] > 0, "%s: no GEMM launches timed", name);
  CHECK(dflash_timing(c, 0) == DFLASH_OK, "%s: timing off", name);
  // refusals leave every sequence as it was
  std::vector<SeqSnap> before;
  for (int s = 0; s < cfg.max_batch; ++s) before.push_back(snap(c, s));
  // device buffers throughout, large enough for any of these calls, so that a refusal that
  // did not happen would still only write where it may
  Dev tk((size_t)64 * 4);
  int32_t* toks = (int32_t*)tk.p;
  void* h1 = hidden_rows(m, 300, 3, keep);
  const int32_t dup[2] = {0, 0}, one = 0, bad_seq = cfg.max_batch, b2[2] = {1, 2};
  CHECK(dflash_block_forward(c, 2, dup, b2, nullptr, 16, toks, nullptr, nullptr) == DFLASH_ERANGE, "%s: duplicate bands", name);
  CHECK(dflash_block_forward(c, 1, &bad_seq, b2, nullptr, 16, toks, nullptr, nullptr) == DFLASH_ERANGE, "%s: seq out of range", name);
  CHECK(dflash_block_forward(c, 1, &one, b2, nullptr, 1, toks, nullptr, nullptr) != DFLASH_OK, "%s: gamma 1", name);
  CHECK(dflash_block_forward(c, 1, &one, b2, nullptr, 17, toks, nullptr, nullptr) != DFLASH_OK, "%s: gamma 17", name);
  CHECK(dflash_block_forward(c, 0, &one, b2, nullptr, 16, toks, nullptr, nullptr) != DFLASH_OK, "%s: no bands", name);
  CHECK(dflash_block_forward(c, 1, &one, b2, nullptr, 16, nullptr, nullptr, nullptr) != DFLASH_OK, "%s: NULL drafts", name);
  const int32_t bad_tok = m.V;
  CHECK(dflash_block_forward(c, 1, &one, &bad_tok, nullptr, 16, toks, nullptr, nullptr) != DFLASH_OK, "%s: bonus out of vocab", name);
  const int32_t neg_pos = -5;
  CHECK(dflash_block_forward(c, 1, &one, b2, &neg_pos, 16, toks, nullptr, nullptr) != DFLASH_OK, "%s: negative position", name);
  CHECK(dflash_ctx_kv_append(c, 0, h1, nullptr, 100, nullptr) == DFLASH_ERANGE, "%s: append past max_seq_len", name);
  CHECK(dflash_ctx_kv_append(c, bad_seq, h1, nullptr, 1, nullptr) == DFLASH_ERANGE, "%s: append seq out of range", name);
  CHECK(dflash_ctx_kv_append(c, 1, h1, nullptr, 0, nullptr) == DFLASH_EINVAL, "%s: append of 0 rows", name);
  CHECK(dflash_ctx_kv_append(c, 1, nullptr, nullptr, 1, nullptr) == DFLASH_EINVAL, "%s: append of NULL", name);
  const int32_t back[2] = {0, 0};
  CHECK(dflash_ctx_kv_append(c, cfg.max_batch - 1, h1, back, 2, nullptr) == DFLASH_EINVAL, "%s: positions not increasing", name);
  const int32_t cnt_bad[2] = {1, -1};
  const int32_t two[2] = {0, 1};
  CHECK(dflash_ctx_kv_append_batch(c, 2, two, cnt_bad, h1, nullptr, nullptr) == DFLASH_EINVAL, "%s: batched negative count", name);
  CHECK(dflash_ctx_kv_append_batch(c, 2, dup, b2, h1, nullptr, nullptr) != DFLASH_OK, "%s: batched duplicate", name);
  const int32_t big[1] = {257};
  CHECK(dflash_ctx_kv_append_batch(c, 1, &one, big, h1, nullptr, nullptr) != DFLASH_OK, "%s: batched over 256 rows", name);
  for (int s = 0; s < cfg.max_batch; ++s) CHECK(snap(c, s) == before[s], "%s: seq %d changed by a refusal", name, s);
  // resets return pages; the freed pages serve a new sequence
  CHECK(dflash_seq_reset(c, 0) == DFLASH_OK && snap(c, 0).kv_len == 0 && snap(c, 0).n_pages == 0, "%s: reset", name);
  CHECK(dflash_seq_reset(c, bad_seq) == DFLASH_ERANGE, "%s: reset out of range", name);
  rc = dflash_ctx_kv_append(c, 0, h1, nullptr, 100, nullptr);
  CHECK(rc == DFLASH_OK && snap(c, 0).kv_len == 100, "%s: append after reset", name);
  rc = forward(c, m, seqs, bonus, 16, false, nullptr);
  CHECK(rc == DFLASH_OK, "%s: forward after reset", name);
  int64_t np = 0, pps = 0, plb = 0, pb = 0, fkv = 0;
  CHECK(dflash_pool_geometry(c, &np, &pps, &plb, &pb, &fkv) == DFLASH_OK && np > 1 && pb == plb * m.L * np, "%s: geometry", name);
  HIP_OK(hipDeviceSynchronize());
  dflash_destroy(c);
  for (void* p : keep) (void)hipFree(p);
}

int run_gpu() {
  {  // bf16, YaRN, a window on layer 0, 8 sequences (the LDS attention path for a band past 2048 keys)
    const Model m = kWide128;
    dflash_config c = base_config(m, 2600, 8);
    c.rope_type = 1; c.yarn_factor = 4; c.yarn_orig_max_pos = 1024; c.yarn_beta_fast = 32; c.yarn_beta_slow = 1;
    const uint8_t sliding[2] = {1, 0};
    c.sliding_window = 700;
    c.layer_sliding = sliding;
    exercise("bf16", m, c, 0, 0);
  }
  const Model m = kTiny;
  {
    dflash_config c = base_config(m, 600, 2);
    c.weight_format = DFLASH_WEIGHTS_FP8_E4M3;
    exercise("fp8", m, c, 0, 0);
  }
  exercise("markov", m, base_config(m, 600, 3), 256, 0);
  exercise("dflash2", m, base_config(m, 600, 3), 0, 256);
  {  // a pool of 12 pages: an append or a forward that needs more is refused and changes nothing
    Weights W;
    W.build(m, 0, 0);
    dflash_config c = base_config(m, 600, 2);
    c.num_pages = 12;
    dflash_ctx* ctx = nullptr;
    CHECK(dflash_create(&c, &W.w, nullptr, &ctx) == DFLASH_OK, "small pool create");
    std::vector<void*> keep;
    if (ctx) {
      // 176 rows fill the 11 pages the pool hands out (page 0 is the sentinel)
      CHECK(dflash_ctx_kv_append(ctx, 0, hidden_rows(m, 176, 9, keep), nullptr, 176, nullptr) == DFLASH_OK, "pool: first append");
      const SeqSnap a = snap(ctx, 0), b = snap(ctx, 1);
      CHECK(dflash_ctx_kv_append(ctx, 1, hidden_rows(m, 40, 10, keep), nullptr, 40, nullptr) == DFLASH_EPOOL, "pool: exhaustion");
      CHECK(snap(ctx, 0) == a && snap(ctx, 1) == b, "pool: a refused append changed state");
      int32_t s = 0, bo = 3;
      Dev t((size_t)15 * 4);
      CHECK(dflash_block_forward(ctx, 1, &s, &bo, nullptr, 16, (int32_t*)t.p, nullptr, nullptr) == DFLASH_EPOOL,
            "pool: forward needs a page");
      CHECK(dflash_seq_reset(ctx, 0) == DFLASH_OK, "pool: reset");
      CHECK(dflash_ctx_kv_append(ctx, 1, hidden_rows(m, 40, 10, keep), nullptr, 40, nullptr) == DFLASH_OK, "pool: reuse");
      HIP_OK(hipDeviceSynchronize());
      dflash_destroy(ctx);
    }
    for (void* p : keep) (void)hipFree(p);
  }
  return g_fail;
}

}  // namespace

int main(int argc, char** argv) {
  const std::string mode = argc > 1 ? argv[1] : "";
  if (mode != "cpu" && mode != "gpu") {
    std::fprintf(stderr, "usage: abi_check cpu|gpu\n");
    return 2;
  }
  const int fails = mode == "cpu" ? run_cpu() : run_gpu();
  if (fails) {
    std::fprintf(stderr, "abi_check %s: %d checks failed\n", mode.c_str(), fails);
    return 1;
  }
  std::printf("abi_check %s ok\n", mode.c_str());
  return 0;
}
