"""DFlash gamma-block drafter -- plain, slow CPU oracle.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this module. The HIP library and its Python binding never
call it, and the two share no code: no kernels, headers, helpers or tables.

Sources (page title -- section). Every function below names the one it follows.
  [memra]   memra_engine/dflash.rs (docs.rs source page) -- the drafter written as a
            readable forward: DflashDraft::ctx_features, ::forward_block, ::ingest_ctx,
            ::forward_round, ::rope_rows, DflashDraft::load (YaRN table),
            HybridModel::generate_spec_dflash (block construction, lm_head rows, argmax).
  [atlas-fw]  spark_model/layers/dflash_head/from_weights.rs -- from_weights: vanilla
            RMSNorm choice, paged KV pool sizing, inv_freq table (plain and YaRN), fused
            K/V weight layout.
  [atlas-head] spark_model/layers/dflash_head.rs -- DflashBatch (bands of gamma rows per
            sequence) and DraftProposer::propose_batch (drop row 0 of each band).
  [metrale-fw] metrale_model_arch/dflash_head/from_weights.rs -- DraftProposer::propose_batch
            (one batched context precompute), PRECOMPUTE_BATCH_ROWS,
            DflashProposerState::ctx_committed (the per-sequence watermark), the FP8
            weights phase of from_weights.
  [atlas-head] also: DflashQuantization (weight-only FP8 with per-row f32 scales) and the
            DSpark head fields markov_rank / markov_w1 / markov_w2.
  [memra] also: DflashDraft's `markov` head and the semi-autoregressive chain of
            generate_spec_dflash (DSpark, greedy).

Arithmetic: numpy float64 by default (float32 on request, for timing only). Inputs
arrive as bf16 bit patterns (uint16) and are widened exactly; no intermediate value is
rounded. Where the pages leave a step open, the reading taken is marked READING.

Parity unpinned (no worked example on the pages fixes them): the sliding-window rule
inside a non-causal block (READING c1 below), the placement of the YaRN mscale when
a trained checkpoint is used (READING c2), and DFlash2's composition of its dynamic
convolutions and selector walk (READINGS c21, c23; the pages give shapes and kernel
names only). They are pinned only by invariants and by their own definitions.
"""
from __future__ import annotations

import math
import os

import numpy as np

# ----------------------------------------------------------------------------------
# bf16 inputs
# ----------------------------------------------------------------------------------


_WIDEN_CHUNK = 1 << 20
_WIDEN_POOL = None


def _widen_chunk(src: np.ndarray, dst: np.ndarray, s: int, e: int):
    u = src[s:e].astype(np.uint32)
    u <<= np.uint32(16)
    dst[s:e] = u.view(np.float32)


def widen(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Exact bf16 -> float widening of uint16 bit patterns (a bf16 is the top half of
    an IEEE binary32). Large arrays are converted in cache-sized chunks on a few threads;
    the result is the same element by element."""
    global _WIDEN_POOL
    src = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(src.shape, dtype=dtype)
    fs, fd = src.reshape(-1), out.reshape(-1)
    n = fs.size
    if n <= _WIDEN_CHUNK:
        _widen_chunk(fs, fd, 0, n)
        return out
    if _WIDEN_POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _WIDEN_POOL = ThreadPoolExecutor(max_workers=max(1, min(16, len(os.sched_getaffinity(0)))))
    futs = [_WIDEN_POOL.submit(_widen_chunk, fs, fd, i, min(n, i + _WIDEN_CHUNK)) for i in range(0, n, _WIDEN_CHUNK)]
    for f in futs:
        f.result()
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits, ties to even), in one step
    from x's own precision: x = f * 2^e with 0.5 <= |f| < 1, and f * 256 is rounded to an
    integer half-to-even (exact arithmetic in binary64). Values stay in x's float type.
    (bf16 subnormals, below 2^-126, do not occur in the drafter's K/V.)"""
    x = np.asarray(x)
    f, e = np.frexp(x.astype(np.float64))
    return np.ldexp(np.round(f * 256.0) / 256.0, e).astype(x.dtype)


# ----------------------------------------------------------------------------------
# FP8 weights ([metrale-fw] from_weights, the FP8 weights phase; [atlas-head]
# DflashQuantization::Fp8Weights). READING c19: the scale and rounding rules below.
# ----------------------------------------------------------------------------------
# OCP FP8 E4M3 ("E4M3FN"): sign, 4 exponent bits with bias 7, 3 mantissa bits; no
# infinities; codes 0x7F and 0xFF are NaN; the largest finite value is 448 (0x7E);
# exponent field 0 holds the subnormals m * 2^-9.
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code, from the format's definition, in float64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


_E4M3_POS = e4m3_decode(np.arange(0x7F))   # the 127 non-negative finite values, ascending


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each (finite) value, ties to the even code, saturating at +-448;
    the sign of x (also of zero) is kept."""
    x = np.asarray(x)
    a = np.minimum(np.abs(x).astype(np.float64), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dl, dh = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    code = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e4m3_encode_f32(x: np.ndarray) -> np.ndarray:
    """e4m3_encode for float32 input, by rounding the binary32 bits (the test suite checks it
    against e4m3_encode on dense samples and at every rounding boundary): below 2^-6 the
    E4M3 values are the multiples of 2^-9 (round-half-even of x * 512); from 2^-6 on, the
    3 leading mantissa bits rounded half to even, the exponent rebiased from 127 to 7; at
    448 and above, 448."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x)
    b = a.view(np.uint32)
    normal = ((b + np.uint32(0x7FFFF) + ((b >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)).astype(np.int32) - 960
    code = np.where(a < np.float32(2.0 ** -6), np.rint(a * np.float32(512.0)).astype(np.int32), np.minimum(normal, 0x7E))
    code = np.where(a >= np.float32(E4M3_MAX), 0x7E, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_rows_fp8(bits: np.ndarray):
    """Per-row FP8 quantization of a bf16 [N, K] weight, in float32 (the precision the
    pages keep the row scales in): scale = max|row| / 448 (1 for an all-zero row), codes =
    nearest E4M3 of w / scale. Returns (codes uint8 [N, K], scale float32 [N])."""
    w = widen(bits, np.float32)
    amax = np.abs(w).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return e4m3_encode_f32(w / scale[:, None]), scale


def dequant_fp8(codes: np.ndarray, scale: np.ndarray, dtype=np.float64) -> np.ndarray:
    """The weight an FP8 GEMM uses: code value x row scale (exact in float64)."""
    return (e4m3_decode(codes) * scale.astype(np.float64)[:, None]).astype(dtype)


# ----------------------------------------------------------------------------------
# elementary steps
# ----------------------------------------------------------------------------------


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis in the vanilla (HF) form out = x * w / RMS(x).

    [atlas-fw] from_weights, kernel table: the drafter uses the vanilla form, not the
    offset form x*(1+w). READING c6: RMS(x) = sqrt(mean(x^2) + eps).
    """
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def inv_freq_plain(theta: float, head_dim: int) -> np.ndarray:
    """inv_freq[j] = theta^(-2j/d), j < d/2, rotary dim = head_dim.
    [atlas-fw] from_weights, inv_freq table (default arm)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / head_dim)


def yarn_bounds(head_dim: int, theta: float, factor: float, orig: float,
                beta_fast: float, beta_slow: float):
    """The YaRN correction range (low, high) in pair-index units.

    [memra] DflashDraft::load, YaRN arm; [atlas-fw] from_weights, YaRN arm:
    corr(r) = d * ln(orig / (2 pi r)) / (2 ln base); low = max(floor(corr(beta_fast)), 0);
    high = min(ceil(corr(beta_slow)), d - 1).
    """
    d = float(head_dim)

    def corr(r):
        return d * math.log(orig / (r * 2.0 * math.pi)) / (2.0 * math.log(theta))

    low = max(math.floor(corr(beta_fast)), 0.0)
    high = min(math.ceil(corr(beta_slow)), d - 1.0)
    return float(low), float(high)


def inv_freq_yarn(head_dim: int, theta: float, factor: float, orig: float,
                  beta_fast: float, beta_slow: float) -> np.ndarray:
    """YaRN-blended inverse frequencies.

    [memra] DflashDraft::load and [atlas-fw] from_weights (YaRN arm): a linear ramp over
    pair index j from `low` to `high` moves each frequency from the plain value
    (extrapolation, ramp 0) to the plain value divided by `factor` (interpolation,
    ramp 1). READING c3: when high == low the ramp denominator gets +0.001 (the Atlas
    page's guard; the memra page has none -- never hit by the shapes used here).
    """
    low, high = yarn_bounds(head_dim, theta, factor, orig, beta_fast, beta_slow)
    base = inv_freq_plain(theta, head_dim)
    denom = (high - low) if abs(high - low) >= 1e-6 else (high - low + 0.001)
    j = np.arange(head_dim // 2, dtype=np.float64)
    ramp = np.clip((j - low) / denom, 0.0, 1.0)
    return (base / factor) * ramp + base * (1.0 - ramp)


def yarn_mscale(factor: float) -> float:
    """[memra] DflashDraft::load: attention scaling 0.1 * ln(factor) + 1."""
    return 0.1 * math.log(factor) + 1.0


def rope_neox(x: np.ndarray, pos: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """NeoX (rotate-half) rotary embedding over the whole head.

    x: [..., head_dim]; pos: integer positions broadcastable to x.shape[:-1].
    For j < d/2 with angle a = pos * inv_freq[j]:
      out[j]       = x[j] cos a - x[j + d/2] sin a
      out[j + d/2] = x[j + d/2] cos a + x[j] sin a
    [memra] DflashDraft::rope_rows (rope_neox, rotary dim = head_dim); [atlas-fw]
    from_weights ("applies rope to full head_dim"). READING c4: pairs (j, j + d/2).
    """
    half = x.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq.astype(np.float64)
    c = np.cos(ang).astype(x.dtype)
    s = np.sin(ang).astype(x.dtype)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gqa_attention(q: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
                  k_pos: np.ndarray, scale: float, window: int) -> np.ndarray:
    """Non-causal grouped-query softmax attention.

    q: [T, nh, d]; k, v: [Tk, nkv, d]; q_pos [T], k_pos [Tk] integer positions.
    Query head h reads kv head h // (nh / nkv) (READING c5: contiguous groups).
    Every query sees every key (non-causal) unless `window` > 0, in which case key j
    is visible to query i iff q_pos[i] - k_pos[j] < window (READING c1: the usual
    decoder window that includes the query's own position, no upper bound).
    [memra] DflashDraft::forward_round (sdpa_naive, causal = false, scale 1/sqrt(d)).
    """
    T, nh, d = q.shape
    nkv = k.shape[1]
    G = nh // nkv
    out = np.empty((T, nh, d), dtype=q.dtype)
    if window > 0:
        vis = (q_pos[:, None].astype(np.int64) - k_pos[None, :].astype(np.int64)) < window
    else:
        vis = np.ones((T, k.shape[0]), dtype=bool)
    for h in range(nh):
        kh = h // G
        s = (q[:, h, :] @ k[:, kh, :].T) * scale          # [T, Tk]
        s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kh, :]
    return out


def argmax_lowest(x: np.ndarray) -> np.ndarray:
    """Row-wise argmax; READING c7: the lowest index wins an exact tie."""
    return np.argmax(x, axis=-1).astype(np.int32)


# ----------------------------------------------------------------------------------
# paged KV pool: the integer model
# ----------------------------------------------------------------------------------

PAGE = 16  # tokens per page ([atlas-fw] from_weights: block size 16)


def pool_pages(max_seq_len: int, gamma_max: int, max_batch: int) -> tuple[int, int]:
    """(pages per sequence, pages in the pool).

    [atlas-fw] from_weights, pool sizing: per sequence ceil((max_seq_len + gamma + 1) / 16)
    pages, times max_batch, plus one spare. The spare is page 0 here: a zeroed sentinel
    that is never handed out (READING: the spare page doubles as the dummy block).
    """
    per_seq = -(-(max_seq_len + gamma_max + 1) // PAGE)
    return per_seq, per_seq * max(1, max_batch) + 1


class PoolError(Exception):
    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


class PagePool:
    """Free list + per-sequence block tables.

    The free list starts as `page_order` (a permutation of 1..P-1) or ascending 1..P-1.
    Allocation pops from the head, in sequence-then-page order; a page is taken the first
    time a sequence writes a position inside it (context rows and transient block rows
    alike). Resetting a sequence appends its pages to the tail of the free list in
    block-table order. slot(p) = block_table[p // 16] * 16 + p % 16 (int64).
    [atlas-fw] from_weights (lazy per-sequence allocation, pool exhaustion is an error);
    [atlas-head] slot mapping from the block table.
    """

    def __init__(self, max_seq_len, gamma_max, max_batch, page_order=None, num_pages=0):
        self.per_seq, self.num_pages = pool_pages(max_seq_len, gamma_max, max_batch)
        if num_pages:            # an explicit (smaller) pool, to exercise exhaustion
            self.num_pages = int(num_pages)
        if page_order is None:
            self.free = list(range(1, self.num_pages))
        else:
            po = [int(p) for p in page_order]
            if sorted(po) != list(range(1, self.num_pages)):
                raise PoolError("EINVAL", "page_order is not a permutation of 1..P-1")
            self.free = po
        self.bt = {s: [] for s in range(max(1, max_batch))}

    def pages_needed(self, seq: int, end_pos: int) -> int:
        """New pages sequence `seq` needs so that logical positions [0, end_pos) are backed."""
        need = -(-end_pos // PAGE)
        return max(0, need - len(self.bt[seq]))

    def ensure(self, seq: int, end_pos: int) -> list[int]:
        n = self.pages_needed(seq, end_pos)
        if n > len(self.free):
            raise PoolError("EPOOL", "KV pool exhausted")
        if len(self.bt[seq]) + n > self.per_seq:
            raise PoolError("ERANGE", "sequence exceeds its page budget")
        new, self.free = self.free[:n], self.free[n:]
        self.bt[seq].extend(new)
        return new

    def slots(self, seq: int, positions) -> np.ndarray:
        bt = self.bt[seq]
        return np.array([bt[p // PAGE] * PAGE + (p % PAGE) for p in positions], dtype=np.int64)

    def reset(self, seq: int):
        self.free.extend(self.bt[seq])
        self.bt[seq] = []


# ----------------------------------------------------------------------------------
# the drafter
# ----------------------------------------------------------------------------------


class Drafter:
    """The drafter's arithmetic on one sequence at a time.

    m: model dict (hidden, heads, taps, rope, window ...); weights: name -> bf16 bits.
    """

    def __init__(self, m: dict, weights: dict, dtype=np.float64, cache_weights: bool = True,
                 kv_bf16: bool = True):
        self.m = m
        self.bits = weights
        self.dtype = dtype
        # The drafter's KV cache holds bf16 values (spark_model/layers/dflash_head/
        # from_weights.rs, from_weights: the paged drafter pool is KvCacheDtype::Bf16;
        # spark_model/layers/dflash_head.rs: the gamma-block attention reads BF16 K/V from
        # the layer pool). Every K/V row written to the cache -- context rows and the
        # block's own rows -- is therefore rounded to bf16; kv_bf16=False keeps them exact.
        self.kv_bf16 = kv_bf16
        self.cache_weights = cache_weights
        self._cache = {}
        hd = m["head_dim"]
        if m.get("rope_type", "plain") == "yarn":
            self.inv_freq = inv_freq_yarn(hd, m["rope_theta"], m["yarn_factor"], m["yarn_orig_max_pos"],
                                          m["yarn_beta_fast"], m["yarn_beta_slow"])
            self.mscale = yarn_mscale(m["yarn_factor"])
        else:
            self.inv_freq = inv_freq_plain(m["rope_theta"], hd)
            self.mscale = None

    def w(self, name: str) -> np.ndarray:
        if name in self._cache:
            return self._cache[name]
        a = widen(self.bits[name], self.dtype)
        if self.cache_weights:
            self._cache[name] = a
        return a

    def lw(self, l: int, name: str) -> np.ndarray:
        return self.w(f"layers.{l}.{name}")

    # the matrices the FP8 weight format quantizes: the block forward's seven per-layer
    # GEMMs and the lm_head ([metrale-fw] from_weights); the context append keeps bf16
    FP8_NAMES = ("q_proj", "k_proj", "v_proj", "o_proj", "gate_proj", "up_proj", "down_proj")

    def fw(self, name: str) -> np.ndarray:
        """A weight of the block forward's GEMMs: bf16, or dequantized FP8 under
        weight_format "fp8"."""
        if self.m.get("weight_format") != "fp8" or not (name == "lm_head" or name.split(".")[-1] in self.FP8_NAMES):
            return self.w(name)
        key = "fp8:" + name
        if key in self._cache:
            return self._cache[key]
        a = dequant_fp8(*quantize_rows_fp8(self.bits[name]), dtype=self.dtype)
        if self.cache_weights:
            self._cache[key] = a
        return a

    def flw(self, l: int, name: str) -> np.ndarray:
        return self.fw(f"layers.{l}.{name}")

    def cache_store(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.kv_bf16 else x

    def sliding(self, l: int) -> bool:
        ls = self.m.get("layer_sliding")
        return bool(ls[l]) if ls else False

    def rope_rows(self, x: np.ndarray, pos: np.ndarray) -> np.ndarray:
        """[memra] DflashDraft::rope_rows: NeoX RoPE, then (YaRN only) multiply by mscale.
        READING c2: mscale multiplies both q and k after the rotation."""
        y = rope_neox(x, pos, self.inv_freq)
        if self.mscale is not None:
            y = y * self.mscale
        return y

    # -- context append -----------------------------------------------------------

    def ctx_features(self, taps_bits: np.ndarray) -> np.ndarray:
        """F = hidden_norm(taps @ fc^T). taps: [n, num_taps * target_hidden], taps in
        target_layer_ids order (READING c13). [memra] DflashDraft::ctx_features."""
        m = self.m
        x = widen(taps_bits, self.dtype)
        f = x @ self.w("fc").T
        return rms_norm(f, self.w("hidden_norm"), m["rms_eps"])

    def ctx_kv(self, F: np.ndarray, positions: np.ndarray):
        """Per layer: K = rope(k_norm(F Wk^T per head), pos), V = F Wv^T, as stored in the
        cache (bf16 unless kv_bf16 is off). Context features are not passed through
        input_layernorm.
        [memra] DflashDraft::ingest_ctx; DflashDraft::forward_block (ctx features are
        norm-free per layer)."""
        m = self.m
        n = F.shape[0]
        nkv, hd = m["num_kv_heads"], m["head_dim"]
        out = []
        for l in range(m["num_layers"]):
            k = (F @ self.lw(l, "k_proj").T).reshape(n, nkv, hd)
            v = (F @ self.lw(l, "v_proj").T).reshape(n, nkv, hd)
            k = rms_norm(k, self.lw(l, "k_norm"), m["rms_eps"])
            k = self.rope_rows(k, np.asarray(positions)[:, None])
            out.append((self.cache_store(k), self.cache_store(v)))
        return out

    # -- one gamma block ------------------------------------------------------------

    def block_forward(self, ctx_k, ctx_v, ctx_pos, bonus: int, q_rope_pos: int, gamma: int,
                      want_hidden: bool = False, markov_prev=None, capture=None):
        """One band: block [bonus, mask x (gamma-1)] through every layer, final norm,
        lm_head on rows 1..gamma-1, argmax.

        ctx_k[l], ctx_v[l]: [C, nkv, hd] cached context K (normed, roped) and V; ctx_pos [C].
        Row i of the block sits at position q_rope_pos + i (READING c9).
        [memra] HybridModel::generate_spec_dflash (block = [last, MASK x b-1]; drafts =
        argmax(lm_head(rows 1..b))) and DflashDraft::forward_round (per-layer math, block
        K/V appended after the context keys, never committed).
        """
        toks = np.full(gamma, self.m["mask_token_id"], dtype=np.int64)
        toks[0] = bonus
        bpos = q_rope_pos + np.arange(gamma, dtype=np.int64)
        y = self.block_hidden(ctx_k, ctx_v, ctx_pos, toks, bpos, capture=capture)
        logits = self.lm_head(y[1:])
        extra = {}
        if self.m.get("markov_rank", 0):
            logits, drafts = self.markov_chain(logits, bonus, markov_prev)
        elif self.dflash2():
            drafts, extra = self.selector_walk(y[1:], logits, bonus, markov_prev)
        else:
            drafts = argmax_lowest(logits)
        res = dict(logits=logits, tokens=drafts, **extra)
        if want_hidden:
            res["hidden"] = y
        return res

    def markov_chain(self, logits: np.ndarray, bonus: int, prev=None):
        """DSpark semi-autoregressive Markov head, greedy ([memra] DflashDraft's `markov` head
        and the chain in generate_spec_dflash; [atlas-head] the head's markov_w1 / markov_w2
        fields). W1 [V, R] is a table indexed by the previous token, W2 [V, R] maps the
        rank-R latent to the vocabulary. Left to right over the drafted rows k = 0..g-1:
        row k's logits get W2 @ W1[t_k], where t_0 is the bonus token and t_k the token
        drafted at row k-1, and the draft at row k is the argmax of the biased row. The
        bias stays in the logits' precision (READING c20).

        prev: optional [g] tokens that replace t_k (teacher forcing, for comparing against
        a run whose chain took another branch at a near-tie); drafts are still each
        biased row's argmax. Returns (biased logits [g, V], drafts [g])."""
        out = np.array(logits, dtype=self.dtype, copy=True)
        drafts = np.empty(out.shape[0], dtype=np.int32)
        w2 = self.w("markov_w2")
        t = int(bonus)
        for k in range(out.shape[0]):
            tk = t if prev is None else int(prev[k])
            out[k] += w2 @ widen(self.bits["markov_w1"][tk], self.dtype)
            drafts[k] = argmax_lowest(out[k])
            t = int(drafts[k])
        return out, drafts

    # ---- DFlash2 ([atlas-head] BlockDiffusionDraftHead's DFlash2 fields and scratch:
    # attention_conv / mlp_conv base kernels [2 applications, kernel, hidden] and kernel
    # projections [2*kernel*groups, hidden]; conv_dyn, conv_tmp; the candidate selector's
    # predecessor / successor codebooks [V, rank] and hidden projection [rank, hidden];
    # sel_vals / sel_idx top-16 and sel_hproj; the dflash2_conv2, dflash2_topk16 and
    # dflash2_selector_walk kernels). The pages give shapes and kernel names only: the
    # composition below is READING c21-c23 and its parity is unpinned.

    def dflash2(self) -> bool:
        return bool(self.m.get("selector_rank", 0))

    def dconv_prepare(self, l: int, site: str, hn: np.ndarray):
        """The prepare application of a grouped dynamic causal conv site (READING c21).
        hn [T, h]: the site's normed input (the block rows of one band, in order). Per row t
        the dynamic taps D_t = hn_t @ proj^T, viewed as [application 2][tap k][group G]
        (G = h / group_size), and the kernel of channel c is base[a][j][c] + D_t[a][j][c //
        group_size]. The prepare output is u_t = sum_j kern_t[0][j] * hn_{t-j} (rows before
        the band's first contribute zero). Returns (u, kern [T, 2, k, h])."""
        m = self.m
        T, h = hn.shape
        k, gs = m["conv_kernel_size"], m["conv_group_size"]
        base = self.lw(l, site + "_conv_base").reshape(2, k, h)
        D = (hn @ self.lw(l, site + "_conv_proj").T).reshape(T, 2, k, h // gs)
        kern = base[None] + np.repeat(D, gs, axis=3)
        u = np.zeros_like(hn)
        for j in range(min(k, T)):
            u[j:] += kern[j:, 0, j] * hn[:T - j]
        return u, kern

    @staticmethod
    def dconv_finish(sub: np.ndarray, kern: np.ndarray) -> np.ndarray:
        """The finish application (READING c21): v_t = sum_j kern_t[1][j] * sub_{t-j}, on the
        sublayer's output before the residual add, with the taps computed at prepare."""
        T = sub.shape[0]
        v = np.zeros_like(sub)
        for j in range(min(kern.shape[2], T)):
            v[j:] += kern[j:, 1, j] * sub[:T - j]
        return v

    @staticmethod
    def top_k_candidates(logits: np.ndarray, k: int):
        """READING c22: each row's k largest logits in descending order, a tie to the lower
        index (what taking the argmax k times, removing it each time, yields)."""
        idx = np.argsort(-logits, axis=-1, kind="stable")[..., :k]
        return idx.astype(np.int32), np.take_along_axis(logits, idx, axis=-1)

    def selector_walk(self, y: np.ndarray, logits: np.ndarray, bonus: int, prev=None):
        """The candidate selector's chain walk, greedy (READING c23). y [g, h]: the drafted
        rows' final-normed hidden states (the lm_head's input); logits [g, V]. Per row the
        top-k candidates with their logits; H_t = hidden_projection @ y_t [rank]; a
        candidate c scores logit_t(c) + sum_r pred[t_prev][r] * H_t[r] * succ[c][r], with
        t_prev the bonus token for the first row and the previous row's pick after; the
        row's draft is the best-scoring candidate (the earlier candidate on a tie).
        prev: optional [g] previous tokens (teacher forcing). Returns (drafts, extras)."""
        k = self.m["selector_top_k"]
        cand, vals = self.top_k_candidates(logits, k)
        H = y @ self.w("selector_hidden_proj").T
        drafts = np.empty(logits.shape[0], dtype=np.int32)
        scores = np.empty((logits.shape[0], k), dtype=self.dtype)
        t = int(bonus)
        for r in range(logits.shape[0]):
            tp = t if prev is None else int(prev[r])
            gate = widen(self.bits["selector_pred"][tp], self.dtype) * H[r]
            scores[r] = vals[r] + widen(self.bits["selector_succ"][cand[r]], self.dtype) @ gate
            drafts[r] = cand[r][int(np.argmax(scores[r]))]
            t = int(drafts[r])
        return drafts, dict(cand=cand, cand_logits=vals, sel_h=H, scores=scores)

    def block_hidden(self, ctx_k, ctx_v, ctx_pos, toks, bpos, capture=None):
        """Final-normed hidden rows [T, h] of a block with explicit token ids `toks` [T]
        at explicit positions `bpos` [T]; the gamma-block forward calls it with
        [bonus, mask x (gamma-1)] at q_rope_pos + i. Keys are the context keys followed by
        the block's own keys; every query sees every key (non-causal).
        [memra] DflashDraft::forward_round: per layer input_layernorm on block rows,
        q/k/v projections, per-head q_norm / k_norm, RoPE, attention over context + block,
        o_proj + residual, post_attention_layernorm, SwiGLU MLP + residual; final norm.

        capture: an optional list that receives, per layer, the intermediates [memra]
        DflashDraft::forward_block dumps for parity runs: q (after q_norm, RoPE and mscale,
        [T, nh, hd]), the block's k and v as cached, the attention output [T, nh*hd], x1 (the
        residual after attention) and x (the layer output). Recording them changes nothing.
        """
        m = self.m
        h, nh, nkv, hd = m["hidden"], m["num_q_heads"], m["num_kv_heads"], m["head_dim"]
        eps = m["rms_eps"]
        gamma = len(toks)
        bpos = np.asarray(bpos, dtype=np.int64)
        x = widen(self.bits["embed_tokens"][np.asarray(toks)], self.dtype)       # [T, h]
        scale = 1.0 / math.sqrt(hd)
        d2 = self.dflash2()
        for l in range(m["num_layers"]):
            xn = rms_norm(x, self.lw(l, "input_layernorm"), eps)
            if d2:
                xn, kern_a = self.dconv_prepare(l, "attention", xn)
            q = (xn @ self.flw(l, "q_proj").T).reshape(gamma, nh, hd)
            kb = (xn @ self.flw(l, "k_proj").T).reshape(gamma, nkv, hd)
            vb = (xn @ self.flw(l, "v_proj").T).reshape(gamma, nkv, hd)
            q = self.rope_rows(rms_norm(q, self.lw(l, "q_norm"), eps), bpos[:, None])
            kb = self.rope_rows(rms_norm(kb, self.lw(l, "k_norm"), eps), bpos[:, None])
            k_all = np.concatenate([ctx_k[l], self.cache_store(kb)], axis=0)
            v_all = np.concatenate([ctx_v[l], self.cache_store(vb)], axis=0)
            k_pos = np.concatenate([np.asarray(ctx_pos, dtype=np.int64), bpos])
            win = int(m.get("sliding_window", 0) or 0) if self.sliding(l) else 0
            attn = gqa_attention(q, bpos, k_all, v_all, k_pos, scale, win).reshape(gamma, nh * hd)
            o = attn @ self.flw(l, "o_proj").T
            x1 = x + (self.dconv_finish(o, kern_a) if d2 else o)
            x1n = rms_norm(x1, self.lw(l, "post_attention_layernorm"), eps)
            if d2:
                x1n, kern_m = self.dconv_prepare(l, "mlp", x1n)
            g = x1n @ self.flw(l, "gate_proj").T
            u = x1n @ self.flw(l, "up_proj").T
            mo = (silu(g) * u) @ self.flw(l, "down_proj").T
            x = x1 + (self.dconv_finish(mo, kern_m) if d2 else mo)
            if capture is not None:
                capture.append(dict(q=q, k=k_all[-gamma:], v=v_all[-gamma:], attn=attn, x1=x1, x=x))
        return rms_norm(x, self.w("norm"), eps)

    def lm_head(self, y: np.ndarray, chunk: int = 16384) -> np.ndarray:
        """logits = y @ lm_head^T, the vocabulary taken in chunks (memory only)."""
        if self.cache_weights:
            return y @ self.fw("lm_head").T
        V = self.m["vocab"]
        out = np.empty((y.shape[0], V), dtype=self.dtype)
        fp8 = self.m.get("weight_format") == "fp8"
        for s in range(0, V, chunk):
            e = min(V, s + chunk)
            rows = self.bits["lm_head"][s:e]
            wt = dequant_fp8(*quantize_rows_fp8(rows), dtype=self.dtype) if fp8 else widen(rows, self.dtype)
            out[:, s:e] = y @ wt.T
        return out


# ----------------------------------------------------------------------------------
# the whole boundary, as the C ABI exposes it
# ----------------------------------------------------------------------------------


class Engine:
    """Host-side model of the four calls: create / ctx_kv_append / block_forward /
    seq_reset, with the pool's integer state (block tables, slots) and each sequence's
    cached context K/V kept contiguous (the memra page's DflashKv layout).

    Every check happens before any state changes; a failing call raises PoolError and
    leaves the engine as it was ([atlas-head] propose_batch: a sequence that cannot be
    served aborts the whole batch).
    """

    def __init__(self, m: dict, weights: dict, max_seq_len: int, max_batch: int,
                 page_order=None, dtype=np.float64, cache_weights: bool = True, num_pages: int = 0,
                 kv_bf16: bool = True):
        self.m = m
        self.d = Drafter(m, weights, dtype, cache_weights, kv_bf16)
        self.max_seq_len = max_seq_len
        self.max_batch = max_batch
        self.pool = PagePool(max_seq_len, m["gamma_max"], max_batch, page_order, num_pages)
        self.seqs = {s: self._empty() for s in range(max_batch)}
        self.last_slots = np.zeros(0, dtype=np.int64)

    def _empty(self):
        L = self.m["num_layers"]
        nkv, hd = self.m["num_kv_heads"], self.m["head_dim"]
        z = np.zeros((0, nkv, hd), dtype=self.d.dtype)
        return dict(k=[z] * L, v=[z] * L, pos=np.zeros(0, dtype=np.int64))

    def kv_len(self, seq: int) -> int:
        return int(self.seqs[seq]["pos"].shape[0])

    def block_table(self, seq: int) -> list[int]:
        return list(self.pool.bt[seq])

    def seq_reset(self, seq: int):
        if not (0 <= seq < self.max_batch):
            raise PoolError("ERANGE", "seq out of range")
        self.pool.reset(seq)
        self.seqs[seq] = self._empty()

    def ctx_kv_append(self, seq: int, taps_bits: np.ndarray, positions=None):
        if not (0 <= seq < self.max_batch):
            raise PoolError("ERANGE", "seq out of range")
        n = int(taps_bits.shape[0])
        if n <= 0:
            raise PoolError("EINVAL", "n must be positive")
        s = self.seqs[seq]
        C = self.kv_len(seq)
        if C + n > self.max_seq_len:
            raise PoolError("ERANGE", "kv_len + n exceeds max_seq_len")
        if positions is None:
            positions = np.arange(C, C + n, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        last = s["pos"][-1] if C else -1
        if positions.shape[0] != n or positions[0] <= last or np.any(np.diff(positions) <= 0) \
                or positions[-1] > np.iinfo(np.int32).max:
            raise PoolError("EINVAL", "positions must be strictly increasing")
        self.pool.ensure(seq, C + n)
        self.last_slots = self.pool.slots(seq, range(C, C + n))
        F = self.d.ctx_features(taps_bits)
        kv = self.d.ctx_kv(F, positions)
        for l, (k, v) in enumerate(kv):
            s["k"][l] = np.concatenate([s["k"][l], k], axis=0)
            s["v"][l] = np.concatenate([s["v"][l], v], axis=0)
        s["pos"] = np.concatenate([s["pos"], positions])

    # rows one batched context precompute holds ([metrale-fw] PRECOMPUTE_BATCH_ROWS)
    APPEND_BATCH_ROWS = 256

    def ctx_kv_append_batch(self, seqs, counts, taps_bits: np.ndarray, positions=None):
        """The batched incremental append ([metrale-fw] DraftProposer::propose_batch, its one
        context precompute over every sequence's rows past the watermark
        DflashProposerState::ctx_committed): by definition the per-sequence appends in call
        order, after every check of the whole call has passed (pages are then taken in call
        order). taps_bits holds sum(counts) rows, the sequences' rows one after another;
        positions likewise (None: each sequence's kv_len + i)."""
        seqs = [int(x) for x in seqs]
        counts = [int(x) for x in counts]
        if len(seqs) == 0 or len(seqs) > self.max_batch or len(counts) != len(seqs):
            raise PoolError("EINVAL", "bad number of sequences")
        if len(set(seqs)) != len(seqs) or any(not (0 <= x < self.max_batch) for x in seqs):
            raise PoolError("ERANGE", "seq out of range or repeated")
        if any(c < 0 for c in counts):
            raise PoolError("EINVAL", "negative count")
        for q, c in zip(seqs, counts):
            if self.kv_len(q) + c > self.max_seq_len:
                raise PoolError("ERANGE", "kv_len + count exceeds max_seq_len")
        total = sum(counts)
        if not (1 <= total <= self.APPEND_BATCH_ROWS) or int(taps_bits.shape[0]) != total:
            raise PoolError("EINVAL", "total rows out of range")
        if positions is not None:
            positions = np.asarray(positions, dtype=np.int64)
            r = 0
            for q, c in zip(seqs, counts):
                p = positions[r:r + c]
                last = self.seqs[q]["pos"][-1] if self.kv_len(q) else -1
                if c and (p[0] <= last or np.any(np.diff(p) <= 0) or p[-1] > np.iinfo(np.int32).max):
                    raise PoolError("EINVAL", "positions must be strictly increasing")
                r += c
        need = sum(self.pool.pages_needed(q, self.kv_len(q) + c) for q, c in zip(seqs, counts))
        if need > len(self.pool.free):
            raise PoolError("EPOOL", "KV pool exhausted")
        slots, r = [], 0
        for q, c in zip(seqs, counts):
            if c:
                self.ctx_kv_append(q, taps_bits[r:r + c], None if positions is None else positions[r:r + c])
                slots.append(self.last_slots)
            r += c
        self.last_slots = np.concatenate(slots)

    def block_forward(self, seqs, bonus, q_rope_pos=None, gamma=None, want_hidden=False, markov_prev=None,
                      capture=False):
        """The C ABI's block forward over bands `seqs`. markov_prev (DSpark and DFlash2
        heads): optional [n, gamma-1] previous tokens per band for the Markov chain or the
        selector walk (teacher forcing; see Drafter.markov_chain, Drafter.selector_walk)."""
        m = self.m
        gamma = m["gamma_max"] if gamma is None else gamma
        seqs = [int(x) for x in seqs]
        if len(seqs) == 0 or len(seqs) > self.max_batch:
            raise PoolError("EINVAL", "bad number of sequences")
        if len(set(seqs)) != len(seqs) or any(not (0 <= x < self.max_batch) for x in seqs):
            raise PoolError("ERANGE", "seq out of range or repeated")
        if not (2 <= gamma <= m["gamma_max"]):
            raise PoolError("ERANGE", "gamma out of range")
        if any(not (0 <= int(b) < m["vocab"]) for b in bonus):
            raise PoolError("EINVAL", "bonus token out of range")
        # page budget for every band, checked before anything is taken
        need = sum(self.pool.pages_needed(x, self.kv_len(x) + gamma) for x in seqs)
        if need > len(self.pool.free):
            raise PoolError("EPOOL", "KV pool exhausted")
        slots = []
        for x in seqs:
            C = self.kv_len(x)
            self.pool.ensure(x, C + gamma)
            slots.append(self.pool.slots(x, range(C, C + gamma)))
        self.last_slots = np.concatenate(slots)
        outs, caps = [], []
        for i, x in enumerate(seqs):
            s = self.seqs[x]
            C = self.kv_len(x)
            P = C if q_rope_pos is None else int(q_rope_pos[i])
            cap = [] if capture else None
            outs.append(self.d.block_forward(s["k"], s["v"], s["pos"], int(bonus[i]), P, gamma,
                                             want_hidden=want_hidden,
                                             markov_prev=None if markov_prev is None else markov_prev[i],
                                             capture=cap))
            caps.append(cap)
        res = dict(tokens=np.stack([o["tokens"] for o in outs]),
                   logits=np.stack([o["logits"] for o in outs]))
        for key in ("cand", "cand_logits", "sel_h", "scores"):
            if key in outs[0]:
                res[key] = np.stack([o[key] for o in outs])
        if want_hidden:
            res["hidden"] = np.stack([o["hidden"] for o in outs])
        if capture:
            res["layers"] = caps   # [band][layer] dicts of Drafter.block_hidden's capture
        return res
