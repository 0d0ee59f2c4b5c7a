/*
 * dflash.h -- C ABI of the DFlash block-diffusion drafter's gamma-block forward on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (page titles and sections of the describing pages):
 *  - memra_engine/dflash.rs, DflashDraft::ctx_features and ::ingest_ctx: tapped target
 *    hidden states are concatenated, projected through `fc`, normalised by
 *    `hidden_norm`, and every layer's context K (k_norm + RoPE) and V are written to the
 *    drafter's KV cache.
 *  - memra_engine/dflash.rs, DflashDraft::forward_round and
 *    HybridModel::generate_spec_dflash: the block [bonus, mask x (gamma-1)] is embedded
 *    with the shared target embedding and runs through every layer (RMSNorm, Q/K/V,
 *    per-head q/k RMSNorm, RoPE, block K/V written after the context, non-causal GQA
 *    attention over context + block, o_proj + residual, SwiGLU MLP + residual); the
 *    final norm, the shared lm_head and a per-row argmax over rows 1..gamma-1 give
 *    gamma-1 draft tokens.
 *  - spark_model/layers/dflash_head/from_weights.rs, from_weights: a paged BF16 KV pool
 *    of 16-token pages sized ceil((max_seq_len + gamma + 1) / 16) * max_batch + 1.
 *  - spark_model/layers/dflash_head.rs, DflashBatch and DraftProposer::propose_batch:
 *    several sequences in one call, sequence i owning rows [i*gamma, (i+1)*gamma).
 *
 * Conventions for every entry point:
 *  - Weights, hidden states and outputs are caller-owned DEVICE memory (bf16 = raw
 *    IEEE bfloat16 bit patterns, row-major, matrices [out_features, in_features]).
 *    Weight pointers are borrowed: they must stay valid until dflash_destroy.
 *  - Everything named "host" is host memory read during the call only.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on it and
 *    the call returns; outputs are valid once the stream has reached that point. A
 *    context is used by one host thread at a time, and the work of its calls must be
 *    ordered: every call reuses the context's scratch and writes its KV pool, so calls
 *    enqueued on different streams must be ordered by the caller (events or syncs), or they
 *    race.
 *  - Every condition the host can check is checked before anything is enqueued, and a
 *    failing call changes no state (no pages taken, kv_len unchanged). A HIP runtime
 *    failure returns DFLASH_EHIP and leaves the context unusable (every later call
 *    returns DFLASH_EHIP). dflash_last_error() gives a message for the last failure.
 *  - No environment variables are read.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dflash_ctx dflash_ctx;

enum {
  DFLASH_OK = 0,
  DFLASH_EINVAL = -1, /* bad argument / unsupported shape */
  DFLASH_ENOMEM = -2, /* device or host allocation failed */
  DFLASH_EPOOL = -3,  /* the KV pool cannot supply the pages this call needs */
  DFLASH_ERANGE = -4, /* seq id, gamma, or kv_len + n beyond max_seq_len */
  DFLASH_EHIP = -5    /* HIP runtime error; the context is unusable */
};

/* Model and pool configuration (all host memory, copied by dflash_create).
 * Supported shapes: head_dim in {32, 64, 128}; num_q_heads % num_kv_heads == 0 with a
 * group of at most 8 query heads; gamma_max in [2, 16]; hidden, intermediate,
 * num_q_heads*head_dim and num_taps*target_hidden multiples of 256; hidden <= 8192;
 * max_batch in [1, 32];
 * max_seq_len >= 1 with max_seq_len + gamma_max + 1 <= 262144. Positions (stamped and RoPE)
 * lie in [0, 2^30). */
typedef struct {
  int32_t num_layers, hidden, num_q_heads, num_kv_heads, head_dim, intermediate, vocab;
  int32_t num_taps, target_hidden; /* fc in_features = num_taps * target_hidden */
  int32_t gamma_max;               /* widest block a forward call may ask for */
  int32_t mask_token_id;           /* id of the mask rows 1..gamma-1 */
  float rms_eps;                   /* RMSNorm eps (vanilla form x * w / sqrt(mean(x^2)+eps)) */
  double rope_theta;
  int32_t rope_type;               /* 0 = plain NeoX RoPE, 1 = YaRN */
  double yarn_factor, yarn_orig_max_pos, yarn_beta_fast, yarn_beta_slow;
  int32_t sliding_window;          /* window W of sliding layers, 0 = none */
  const uint8_t *layer_sliding;    /* host [num_layers], 1 = sliding layer; NULL = none */
  int32_t max_seq_len;             /* context rows a sequence may hold */
  int32_t max_batch;               /* sequence slots 0..max_batch-1; with 8 or more, bands of
                                      more than 2048 keys on head_dim-128 layers without a
                                      window take the attention path that stages K/V in LDS
                                      (faster in a crowd of bands, slower for one alone);
                                      fixed at create, so it never ties one band's results to
                                      the others of a call */
  int32_t num_pages;               /* 0 = the formula above; >= 2 = explicit pool size */
  const int32_t *page_order;       /* host [num_pages-1]: free-list order, a permutation of
                                      1..num_pages-1; NULL = ascending. Page 0 is a zeroed
                                      sentinel and is never handed out. */
  int32_t weight_format;           /* DFLASH_WEIGHTS_BF16 or DFLASH_WEIGHTS_FP8_E4M3 */
  int32_t markov_rank;             /* DSpark Markov head: 0 = none, else its rank R, 256 or 512
                                      (see dflash_weights and dflash_block_forward) */
  int32_t conv_kernel_size, conv_group_size, selector_rank, selector_top_k;
                                   /* DFlash2: all 0 = none; else 2, 16, 256 or 512, 16 (see
                                      dflash_layer_weights, dflash_weights, dflash_block_forward).
                                      Not together with a Markov head. */
} dflash_config;

/* Weight formats (metrale_model_arch/dflash_head/from_weights.rs, the FP8 weights phase of
 * from_weights; spark_model/layers/dflash_head.rs, DflashQuantization::Fp8Weights): with
 * DFLASH_WEIGHTS_FP8_E4M3 the seven per-layer GEMM weights (q, k, v, o, gate, up, down) and
 * the lm_head are quantized once at create to OCP
 * FP8 E4M3 codes with one fp32 scale per row: scale = max|row| / 448 (1 for an all-zero row),
 * code = the nearest E4M3 value of w / scale (fp32 division), ties to even, saturating at
 * +-448; the GEMMs use code value x scale. Activations, the KV cache, the context-append
 * weights (fc, the fused K/V weight) and the norms stay bf16. The caller's weights are
 * still bf16. */
enum { DFLASH_WEIGHTS_BF16 = 0, DFLASH_WEIGHTS_FP8_E4M3 = 1 };

/* Per-layer weights, device bf16. q/k/v/o/gate/up/down are [out, in]; norms [hidden]
 * or [head_dim] (q_norm, k_norm). Matrices (here and fc, embed_tokens, lm_head below)
 * must be 16-byte aligned: create fails with EINVAL otherwise. */
typedef struct {
  const void *q_proj, *k_proj, *v_proj, *o_proj, *q_norm, *k_norm;
  const void *input_layernorm, *post_attention_layernorm;
  const void *gate_proj, *up_proj, *down_proj;
  /* DFlash2 only (NULL otherwise; spark_model/layers/dflash_head.rs, the DFlash2 fields):
   * the grouped dynamic conv of the attention input and of the MLP input, each a base kernel
   * [2 applications][conv_kernel_size][hidden] and a kernel projection
   * [2 * conv_kernel_size * hidden / conv_group_size, hidden] (rows [application][tap][group]);
   * device bf16, 16-byte aligned; the base kernels are read in place, the projections copied */
  const void *attention_conv_base, *attention_conv_proj, *mlp_conv_base, *mlp_conv_proj;
} dflash_layer_weights;

/* fc [hidden, num_taps*target_hidden]; hidden_norm, norm [hidden]; embed_tokens and
 * lm_head [vocab, hidden] are the target's, shared (they may alias). `layers` is a host
 * array [num_layers]. With markov_rank R > 0, the DSpark Markov head (docs.rs
 * memra-engine, dflash.rs: DflashDraft's `markov` head; spark_model/layers/dflash_head.rs:
 * markov_w1, markov_w2): markov_w1 [vocab, R], the table indexed by the previous token, and
 * markov_w2 [vocab, R], the rank-R latent to vocabulary projection, both device bf16,
 * borrowed (markov_w1 is read in place; markov_w2 is copied at create); NULL otherwise.
 * They stay bf16 under DFLASH_WEIGHTS_FP8_E4M3. */
typedef struct {
  const void *fc, *hidden_norm, *norm, *embed_tokens, *lm_head;
  const dflash_layer_weights *layers;
  const void *markov_w1, *markov_w2;
  /* DFlash2 only (NULL otherwise): the candidate selector's predecessor and successor
   * codebooks [vocab, selector_rank] (read in place) and hidden projection
   * [selector_rank, hidden] (copied); device bf16, 16-byte aligned */
  const void *selector_pred, *selector_succ, *selector_hidden_proj;
} dflash_weights;

/* Create a drafter: validates the configuration, allocates the KV pool, block tables and
 * scratch, builds the inverse-frequency table (plain or YaRN, in double precision) and
 * copies the weights: the all-layer [K0;V0;K1;V1;...] weight of the context append
 * (spark_model/layers/dflash_head/from_weights.rs, fused K/V weight), and, in a tiled order
 * the weight-streaming GEMMs read in whole runs, that weight, fc and the forward's
 * matrices ([Wq;Wk;Wv] and [Wgate;Wup] fused per layer, Wo, Wdown, lm_head). The copies
 * are enqueued on `stream`.
 * On success *out owns everything it allocated; on failure *out is NULL. */
int dflash_create(const dflash_config *cfg, const dflash_weights *w, void *stream,
                  dflash_ctx **out);

/* Append n context rows to sequence `seq` (memra_engine/dflash.rs, ctx_features +
 * ingest_ctx): F = hidden_norm(H fc^T); per layer K = RoPE(k_norm(F Wk^T)), V = F Wv^T,
 * written at logical positions kv_len..kv_len+n-1; then kv_len += n. Pages are taken from
 * the pool as positions first touch them (in ascending page order).
 *   target_hidden: device bf16 [n, num_taps*target_hidden], taps concatenated in the
 *                  drafter's target_layer_ids order;
 *   positions:     host int32 [n], the RoPE position stamped on each row, strictly
 *                  increasing and above the sequence's last stamped position; NULL means
 *                  kv_len + i.
 * Errors: ERANGE (seq, kv_len + n > max_seq_len), EINVAL (n <= 0, NULL hidden, positions
 * not increasing), EPOOL. */
int dflash_ctx_kv_append(dflash_ctx *ctx, int32_t seq, const void *target_hidden,
                         const int32_t *positions, int32_t n, void *stream);

/* Batched incremental append (metrale_model_arch/dflash_head/from_weights.rs,
 * DraftProposer::propose_batch with its one batched context precompute, the staging size
 * PRECOMPUTE_BATCH_ROWS, and the per-sequence watermark DflashProposerState::ctx_committed):
 * the new rows of several sequences in one pass of fc + hidden_norm and one fused K/V GEMM,
 * so the append weights are streamed once per call instead of once per sequence. Sequence
 * seqs[b] receives counts[b] rows (0 allowed) at its watermark kv_len; the result is the
 * same as dflash_ctx_kv_append called for each sequence in turn (up to the rounding of the
 * GEMM form chosen by the total row count), and pages are taken in call order, each
 * sequence's in ascending logical order.
 *   seqs, counts:  host int32 [n_seqs], seqs distinct;
 *   target_hidden: device bf16 [sum(counts), num_taps*target_hidden], the sequences' rows
 *                  one after another in call order;
 *   positions:     host int32 [sum(counts)] in the same order, strictly increasing within
 *                  each sequence and above its last stamped position; NULL means kv_len + i.
 * At most 256 rows per call (sum(counts) in [1, 256]). Errors: ERANGE (seq out of range or
 * repeated, kv_len + count > max_seq_len), EINVAL (n_seqs, NULL pointers, negative counts,
 * total rows, positions), EPOOL; all checked before anything is enqueued. */
int dflash_ctx_kv_append_batch(dflash_ctx *ctx, int32_t n_seqs, const int32_t *seqs,
                               const int32_t *counts, const void *target_hidden,
                               const int32_t *positions, void *stream);

/* One gamma-block forward for n_seqs sequences at once (band b = seqs[b] owns rows
 * [b*gamma, (b+1)*gamma)). Row i of band b is token bonus_tokens[b] (i = 0) or
 * mask_token_id, at RoPE position q_rope_pos[b] + i (q_rope_pos NULL: the sequence's
 * kv_len). The block's K/V are written to slots kv_len..kv_len+gamma-1 (pages taken as
 * needed) but kv_len does NOT advance: the next append overwrites them.
 *   draft_tokens: device int32 [n_seqs, gamma-1]: argmax of rows 1..gamma-1 (lowest
 *                 index on an exact tie);
 *   logits:       device fp32 [n_seqs*(gamma-1), vocab] or NULL.
 * With a Markov head (markov_rank > 0; docs.rs memra-engine, dflash.rs,
 * generate_spec_dflash, the semi-autoregressive chain, greedy) the drafted rows are taken
 * left to right: row k (k = 0..gamma-2, block row k+1) gets the fp32 bias
 * markov_w2 @ markov_w1[t_k] added to its logits, with t_0 = bonus_tokens[b] and t_k =
 * draft_tokens[b][k-1], and draft_tokens[b][k] is the argmax of the biased row; `logits`
 * then holds the biased rows.
 * DFlash2 (conv_kernel_size > 0; spark_model/layers/dflash_head.rs: the dflash2_conv2,
 * dflash2_topk16 and dflash2_selector_walk kernels and their scratch; the pages give shapes
 * and names, the composition here is this library's reading):
 *   - every layer's attention and MLP inputs pass through a grouped dynamic causal conv:
 *     with h_n the sublayer's normed input, row t's taps are base[a][j][c] +
 *     (proj @ h_n[t])[(a * conv_kernel_size + j) * (hidden / 16) + c / 16]; the sublayer reads
 *     u[t] = sum_j tap[0][j] * h_n[t-j] and its output s is added to the residual as
 *     sum_j tap[1][j] * s[t-j] (rows before the band's first contribute zero);
 *   - each drafted row's 16 largest logits are its candidates (ties to the lower index);
 *     H = selector_hidden_proj @ y (y: the row's final-normed hidden state); candidate c
 *     scores logit(c) + sum_r pred[p][r] * H[r] * succ[c][r], p the previous row's draft
 *     (bonus_tokens[b] for the first); the best-scoring candidate (the earlier one on a tie)
 *     is the row's draft. `logits` holds the plain lm_head logits.
 * Errors: EINVAL (n_seqs not in 1..max_batch, NULL pointers, bonus token out of range),
 * ERANGE (seq out of range or repeated, gamma not in [2, gamma_max]), EPOOL. */
int dflash_block_forward(dflash_ctx *ctx, int32_t n_seqs, const int32_t *seqs,
                         const int32_t *bonus_tokens, const int32_t *q_rope_pos,
                         int32_t gamma, int32_t *draft_tokens, float *logits, void *stream);

/* dflash_block_forward without any allocation, for callers that cannot allocate device
 * memory during the call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it): the same arguments, checks, kernels and results (bit for bit), but the
 * forward's split-K, attention and argmax partials live in one static device array of
 * DFLASH_NOALLOC_SCRATCH_MB MiB per device instead of the context's scratch. The call makes
 * no hipMalloc / hipFree or host heap allocation and never times its launches (dflash_timing
 * is ignored for it).
 *   - A forward whose partials do not fit the array is refused with DFLASH_ERANGE before
 *     anything is enqueued (batch 1 of a 2048-hidden, 8-layer drafter at a 4096-row context
 *     needs about 11 MiB; many long bands can need more than the limit).
 *   - Every call on one device shares that device's array, whatever the context: calls that
 *     overlap on the GPU (on different streams, or from different contexts without ordering)
 *     race on it. The array keeps the last call's contents; every partial is written before
 *     it is read, so nothing needs clearing. */
#define DFLASH_NOALLOC_SCRATCH_MB 64
int dflash_block_forward_noalloc(dflash_ctx *ctx, int32_t n_seqs, const int32_t *seqs,
                                 const int32_t *bonus_tokens, const int32_t *q_rope_pos,
                                 int32_t gamma, int32_t *draft_tokens, float *logits, void *stream);

/* Release everything the context owns (waits for its outstanding work). NULL is a no-op. */
void dflash_destroy(dflash_ctx *ctx);

/* ---- sequence management and introspection ------------------------------------- */

/* Return a sequence's pages to the tail of the free list (block-table order) and set its
 * kv_len to 0 (spark_model/layers/dflash_head.rs, DraftProposer::free_state). */
int dflash_seq_reset(dflash_ctx *ctx, int32_t seq);

/* Host view of a sequence: kv_len, number of pages and up to `cap` block-table entries. */
int dflash_seq_info(const dflash_ctx *ctx, int32_t seq, int32_t *kv_len, int32_t *n_pages,
                    int32_t *block_table, int32_t cap);

/* Pool geometry: pages in the pool, pages per sequence, bytes of one page of one layer
 * (K and V of every kv head), total pool bytes, and bytes of the fused append weight. */
int dflash_pool_geometry(const dflash_ctx *ctx, int64_t *num_pages, int64_t *pages_per_seq,
                         int64_t *page_layer_bytes, int64_t *pool_bytes,
                         int64_t *fused_kv_weight_bytes);

/* Copy `bytes` bytes at byte `offset` of a device-side buffer into `dst` (host or device)
 * and wait for it. Buffers:
 *   DFLASH_BUF_POOL      the KV pool: bf16 [num_layers][num_pages][2][num_kv_heads]x
 *                        {K: [16][head_dim], V: [head_dim][16]} (V pages are stored
 *                        transposed);
 *   DFLASH_BUF_KPOS      int32 [num_pages*16]: the position stamped on every slot;
 *   DFLASH_BUF_SLOTS     int64 slots written by the last append / forward call;
 *   DFLASH_BUF_BLOCKTAB  int32 [max_batch][pages_per_seq]: the device block tables;
 *   DFLASH_BUF_HIDDEN    bf16 [rows][hidden]: the final-normed hidden rows of the last
 *                        forward (debug seam), high bf16 term;
 *   DFLASH_BUF_HIDDEN_LO the same rows' low bf16 term (hidden = high + low);
 *   DFLASH_BUF_FP8_LMHEAD (FP8 contexts) the lm_head's E4M3 codes, uint8 in the T16-FP8
 *                        layout: vocab rows in tiles of 16, a tile's hidden dimension in
 *                        256-deep blocks of 4096 bytes, byte (q*64 + lane)*16 + b of a block
 *                        holding row lane%16 at k = 64q + 32*(b/8) + 8*(lane/16) + b%8;
 *   DFLASH_BUF_FP8_LMHEAD_SCALE (FP8 contexts) float [vocab rounded up to 16]: the row scales;
 *   DFLASH_BUF_SEL_IDX   (DFlash2) int32 [n_seqs*(gamma-1)][16]: the last forward's candidates
 *                        per drafted row, best first;
 *   DFLASH_BUF_SEL_VALS  (DFlash2) float [n_seqs*(gamma-1)][16]: their logits;
 *   DFLASH_BUF_CTX_FEAT, DFLASH_BUF_CTX_FEAT_LO  bf16 [2048][hidden]: the context features
 *                        F = hidden_norm(H fc^T) of the last append's last (at most
 *                        2048-row) launch chunk, rows in order, as high + low bf16 terms;
 * and, once dflash_debug_capture has turned capture on, the per-layer intermediates of the
 * last forward, each [num_layers][max_batch * gamma_max][width], rows of layer l at
 * l * max_batch * gamma_max, the call's rows first (band b's row i at b * gamma + i):
 *   DFLASH_BUF_LAYER_Q, _Q_LO       bf16, width num_q_heads*head_dim: Q after q_norm and RoPE
 *                                   (times the YaRN mscale), high and low terms;
 *   DFLASH_BUF_LAYER_ATTN, _ATTN_LO bf16, width num_q_heads*head_dim: the attention output
 *                                   (before o_proj), high and low terms;
 *   DFLASH_BUF_LAYER_X1  float, width hidden: the residual after the attention block;
 *   DFLASH_BUF_LAYER_X   float, width hidden: the layer's output (residual after the MLP). */
enum { DFLASH_BUF_POOL = 0, DFLASH_BUF_KPOS = 1, DFLASH_BUF_SLOTS = 2,
       DFLASH_BUF_BLOCKTAB = 3, DFLASH_BUF_HIDDEN = 4, DFLASH_BUF_HIDDEN_LO = 5,
       DFLASH_BUF_FP8_LMHEAD = 6, DFLASH_BUF_FP8_LMHEAD_SCALE = 7, DFLASH_BUF_SEL_IDX = 8,
       DFLASH_BUF_SEL_VALS = 9, DFLASH_BUF_CTX_FEAT = 10, DFLASH_BUF_CTX_FEAT_LO = 11,
       DFLASH_BUF_LAYER_Q = 12, DFLASH_BUF_LAYER_Q_LO = 13, DFLASH_BUF_LAYER_ATTN = 14,
       DFLASH_BUF_LAYER_ATTN_LO = 15, DFLASH_BUF_LAYER_X1 = 16, DFLASH_BUF_LAYER_X = 17 };
int dflash_debug_copy(dflash_ctx *ctx, int32_t buffer, void *dst, size_t offset, size_t bytes,
                      void *stream);

/* Test seam (memra_engine/dflash.rs, DflashDraft::forward_block: its per-layer dumps of q,
 * attn, x1 and every layer's output for parity against a reference): on != 0 makes every
 * later dflash_block_forward also copy each layer's Q, attention output and residuals into
 * capture buffers (allocated here on first use, ENOMEM if that fails) that dflash_debug_copy
 * reads; 0 stops the copies. The copies are stream-ordered device-to-device copies and change
 * no result. dflash_block_forward_noalloc never captures. */
int dflash_debug_capture(dflash_ctx *ctx, int32_t on);

/* ---- kernel timing ------------------------------------------------------------------
 * Launch classes of the append and forward sequences. With timing on, every launch of a
 * class whose bit (1 << class) is set in `class_mask` carries a start and a stop HIP event
 * in its own dispatch (hipExtLaunchKernel), so the pair times that kernel alone;
 * dflash_timing_read waits for them and returns, per class, the summed milliseconds and
 * the number of launches since the last read (arrays of n_classes entries), then clears
 * the tallies. class_mask 0 turns timing off. */
enum {
  DFLASH_K_PROLOGUE = 0,      /* block-table updates, block-row slots, embedding + first norm */
  DFLASH_K_GEMM = 1,          /* weight-streaming Q/K/V, O, gate/up, down GEMMs of the forward */
  DFLASH_K_QKV_POST = 2,      /* q/k RMSNorm, RoPE, K/V writeback */
  DFLASH_K_ATTN = 3,          /* split-KV block attention */
  DFLASH_K_ATTN_COMBINE = 4,  /* merge of the attention chunks */
  DFLASH_K_RESID_NORM = 5,    /* residual add + RMSNorm */
  DFLASH_K_SILU = 6,          /* SwiGLU */
  DFLASH_K_LMHEAD = 7,        /* lm_head + argmax partials */
  DFLASH_K_ARGMAX = 8,        /* argmax reduction */
  DFLASH_K_APPEND_GEMM = 9,   /* fc and fused K/V GEMMs of the context append */
  DFLASH_K_APPEND_MISC = 10,  /* append slots, hidden_norm, K/V epilogue + writeback */
  DFLASH_K_MARKOV = 11,       /* the Markov head's chain steps (one per drafted row) */
  DFLASH_K_DCONV = 12,        /* DFlash2 conv prepare (taps + convolved sublayer input) */
  DFLASH_K_SELECTOR = 13,     /* DFlash2 top-16 candidates, pair scores and walk */
  DFLASH_K_NUM_CLASSES = 14
};
int dflash_timing(dflash_ctx *ctx, uint32_t class_mask);
int dflash_timing_read(dflash_ctx *ctx, double *ms, int64_t *launches, int32_t n_classes);

/* Message of the last failure on this context ("" if none); valid until the next call. */
const char *dflash_last_error(const dflash_ctx *ctx);
/* Static name of an error code. */
const char *dflash_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
