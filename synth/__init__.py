"""Seeded synthetic inputs for the DFlash gamma-block drafter.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds workload shapes and seeded random draws only: no step of the
drafter's arithmetic lives here. Every tensor is returned as bf16 bit patterns
(numpy uint16) so that both sides start from the same exact values.

Recipe:
  * generator: numpy PCG64 seeded with SeedSequence([seed, stream, index]);
    float32 draws rounded to bf16 with round-to-nearest-even;
  * weight matrices ~ N(0, 0.02); norm weights ~ 1 + N(0, 0.02); a DSpark Markov head's
    token table ~ N(0, 1) and its projection ~ N(0, 0.03); DFlash2 conv base kernels
    ~ 0.5 + N(0, 0.02), kernel projections ~ N(0, 0.002), selector codebooks ~ N(0, 0.1);
  * tapped target hidden states ~ N(0, 1);
  * bonus tokens uniform over the vocabulary; context lengths uniform over the
    workload's range; the pool's page order is a seeded permutation.

No public dataset or benchmark is involved: these draws stand in for the pages'
drafters (trained checkpoints) and for hidden states captured from a target model.
"""
from __future__ import annotations

import copy
import os

import numpy as np

# --------------------------------------------------------------------------------------
# model shapes (the drafter families the pages describe) and workloads
# --------------------------------------------------------------------------------------

_TINY = dict(
    num_layers=2, hidden=256, num_q_heads=8, num_kv_heads=2, head_dim=32,
    intermediate=512, vocab=1024, num_taps=3, target_hidden=256, gamma_max=16,
    mask_token_id=4, rms_eps=1e-6, rope_theta=1e6, rope_type="plain",
    sliding_window=0, layer_sliding=None,
)

_QWEN3_8L_2048 = dict(
    num_layers=8, hidden=2048, num_q_heads=32, num_kv_heads=4, head_dim=128,
    intermediate=6144, vocab=151936, num_taps=5, target_hidden=2048, gamma_max=16,
    mask_token_id=4, rms_eps=1e-6, rope_theta=1e6, rope_type="plain",
    sliding_window=0, layer_sliding=None,
)

_WIDE_5L_5376 = dict(
    num_layers=5, hidden=5376, num_q_heads=64, num_kv_heads=8, head_dim=128,
    intermediate=10752, vocab=262144, num_taps=6, target_hidden=5376, gamma_max=16,
    mask_token_id=4, rms_eps=1e-6, rope_theta=1e6, rope_type="yarn",
    yarn_factor=32.0, yarn_orig_max_pos=8192.0, yarn_beta_fast=32.0,
    yarn_beta_slow=1.0, sliding_window=2048,
    layer_sliding=[True, True, True, True, False],
)

MODELS = {
    "tiny-L2-h256": _TINY,
    "qwen3-L8-h2048": _QWEN3_8L_2048,
    "wide-L5-h5376-yarn-swa2048": _WIDE_5L_5376,
    # the same drafters with a DSpark Markov head of rank 256 (the rank the pages quote);
    # their other weights are the same draws as the plain models' under the same seed
    "tiny-L2-h256-dspark": dict(_TINY, markov_rank=256),
    "qwen3-L8-h2048-dspark": dict(_QWEN3_8L_2048, markov_rank=256),
    # DFlash2: two-tap grouped dynamic convs with 16-channel groups and a rank-256, top-16
    # candidate selector (the sizes the pages name)
    "tiny-L2-h256-dflash2": dict(_TINY, conv_kernel_size=2, conv_group_size=16, selector_rank=256, selector_top_k=16),
    "qwen3-L8-h2048-dflash2": dict(_QWEN3_8L_2048, conv_kernel_size=2, conv_group_size=16, selector_rank=256,
                                   selector_top_k=16),
}

# A workload = a model, how many sequences one forward call carries, how their
# contexts are filled, and the pool geometry.
#   ctx: (lo, hi) inclusive range of existing context lengths per sequence
#   append: rows appended (timed) right before the block forward, 0 = none
WORKLOADS = {
    "tiny-L2-h256-ctx64-b1": dict(
        model="tiny-L2-h256", batch=1, ctx=(64, 64), append=0,
        max_seq_len=128, max_batch=1, permute_pages=False, seed=1001),
    "qwen3-L8-h2048-ctx4096-b1": dict(
        model="qwen3-L8-h2048", batch=1, ctx=(4096, 4096), append=0,
        max_seq_len=8192, max_batch=1, permute_pages=False, seed=1002),
    "qwen3-L8-h2048-b16-ctx512to8192": dict(
        model="qwen3-L8-h2048", batch=16, ctx=(512, 8192), append=0,
        max_seq_len=8192, max_batch=16, permute_pages=True, seed=1003),
    "wide-L5-h5376-yarn-swa2048-ctx16384-b1": dict(
        model="wide-L5-h5376-yarn-swa2048", batch=1, ctx=(16384, 16384), append=0,
        max_seq_len=20480, max_batch=1, permute_pages=False, seed=1004),
    "qwen3-L8-h2048-b32-ctx8192to32768-append2048": dict(
        model="qwen3-L8-h2048", batch=32, ctx=(8192, 32768), append=2048,
        max_seq_len=34816, max_batch=32, permute_pages=True, seed=1005),
}


def model(name: str) -> dict:
    return copy.deepcopy(MODELS[name])


def workload(name: str) -> dict:
    w = copy.deepcopy(WORKLOADS[name])
    w["name"] = name
    w["model_cfg"] = model(w["model"])
    return w


# --------------------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------------------

# stream ids (second word of every SeedSequence)
S_WEIGHTS, S_HIDDEN, S_BONUS, S_CTXLEN, S_PAGES, S_POS = 1, 2, 3, 4, 5, 6


def rng(seed: int, stream: int, index: int = 0, block=None) -> np.random.Generator:
    words = [seed, stream, index] + ([] if block is None else [block])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(words)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BLOCK = 1 << 22   # elements per independently seeded block of a normal draw
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(16, len(os.sched_getaffinity(0)))))
    return _POOL


def _normal_block(out: np.ndarray, seed: int, stream: int, index: int, j: int, mean: float, std: float):
    s, e = j * BLOCK, min(out.size, (j + 1) * BLOCK)
    x = rng(seed, stream, index, j).standard_normal(e - s, dtype=np.float32)
    x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    out[s:e] = f32_to_bf16_bits(x)


def _normal_bf16(seed: int, stream: int, index: int, shape, mean: float, std: float, wait=True):
    """N(mean, std) in float32, rounded to bf16 bits; the row-major elements are drawn in
    blocks of BLOCK, block j from PCG64(SeedSequence([seed, stream, index, j]))."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    futs = [_pool().submit(_normal_block, out, seed, stream, index, j, mean, std)
            for j in range((n + BLOCK - 1) // BLOCK)]
    if not wait:
        return out.reshape(shape), futs
    for f in futs:
        f.result()
    return out.reshape(shape)


def weight_specs(m: dict):
    """(name, shape, kind) in the fixed generation order; kind is 'mat' or 'norm'."""
    h, hd = m["hidden"], m["head_dim"]
    qd, kvd, ff = m["num_q_heads"] * hd, m["num_kv_heads"] * hd, m["intermediate"]
    specs = [
        ("fc", (h, m["num_taps"] * m["target_hidden"]), "mat"),
        ("hidden_norm", (h,), "norm"),
        ("norm", (h,), "norm"),
        ("embed_tokens", (m["vocab"], h), "mat"),
        ("lm_head", (m["vocab"], h), "mat"),
    ]
    for l in range(m["num_layers"]):
        p = f"layers.{l}."
        specs += [
            (p + "q_proj", (qd, h), "mat"),
            (p + "k_proj", (kvd, h), "mat"),
            (p + "v_proj", (kvd, h), "mat"),
            (p + "o_proj", (h, qd), "mat"),
            (p + "q_norm", (hd,), "norm"),
            (p + "k_norm", (hd,), "norm"),
            (p + "input_layernorm", (h,), "norm"),
            (p + "post_attention_layernorm", (h,), "norm"),
            (p + "gate_proj", (ff, h), "mat"),
            (p + "up_proj", (ff, h), "mat"),
            (p + "down_proj", (h, ff), "mat"),
        ]
    if m.get("markov_rank", 0):
        # DSpark Markov head: a previous-token embedding table and a latent-to-vocabulary
        # projection, both [vocab, rank]
        specs += [("markov_w1", (m["vocab"], m["markov_rank"]), "embed"),
                  ("markov_w2", (m["vocab"], m["markov_rank"]), "proj")]
    if m.get("selector_rank", 0):
        # DFlash2: per layer two grouped dynamic convs (base kernel [2, kernel, hidden],
        # kernel projection [2 * kernel * hidden / group, hidden]); the candidate selector's
        # codebooks [vocab, rank] and hidden projection [rank, hidden]
        k, ng, r = m["conv_kernel_size"], 2 * m["conv_kernel_size"] * h // m["conv_group_size"], m["selector_rank"]
        for l in range(m["num_layers"]):
            for site in ("attention", "mlp"):
                specs += [(f"layers.{l}.{site}_conv_base", (2, k, h), "convbase"),
                          (f"layers.{l}.{site}_conv_proj", (ng, h), "dynproj")]
        specs += [("selector_pred", (m["vocab"], r), "codebook"),
                  ("selector_succ", (m["vocab"], r), "codebook"),
                  ("selector_hidden_proj", (r, h), "mat")]
    return specs


# (mean, standard deviation) of each kind of tensor
_KIND_DIST = {"mat": (0.0, 0.02), "norm": (1.0, 0.02), "embed": (0.0, 1.0), "proj": (0.0, 0.03),
              "convbase": (0.5, 0.02), "dynproj": (0.0, 0.002), "codebook": (0.0, 0.1)}


def _weight_args(m: dict, name: str):
    for i, (n, shape, kind) in enumerate(weight_specs(m)):
        if n == name:
            return (i, shape) + _KIND_DIST[kind]
    raise KeyError(name)


def gen_weight(m: dict, seed: int, name: str) -> np.ndarray:
    """Weight `name`: matrices N(0, 0.02), norm weights 1 + N(0, 0.02), the Markov head's
    token table N(0, 1) and its projection N(0, 0.03) (a bias of about the logits' spread),
    DFlash2's conv base kernels 0.5 + N(0, 0.02) (a two-tap smoothing), kernel projections
    N(0, 0.002) (dynamic taps a fifth of the base at hidden 2048) and selector codebooks
    N(0, 0.1) (pair scores of about the top-16 logits' spacing); tensor i of the fixed
    order draws from stream S_WEIGHTS, index i."""
    i, shape, mean, std = _weight_args(m, name)
    return _normal_bf16(seed, S_WEIGHTS, i, shape, mean, std)


def gen_weights(m: dict, seed: int) -> dict:
    """All weights, every block of every tensor drawn in parallel."""
    pending = {}
    for n, _, _ in weight_specs(m):
        i, shape, mean, std = _weight_args(m, n)
        pending[n] = _normal_bf16(seed, S_WEIGHTS, i, shape, mean, std, wait=False)
    out = {}
    for n, (arr, futs) in pending.items():
        for f in futs:
            f.result()
        out[n] = arr
    return out


def gen_hidden(m: dict, seed: int, n_rows: int, index: int = 0) -> np.ndarray:
    """Tapped target hidden states, [n_rows, num_taps * target_hidden] bf16 bits."""
    return _normal_bf16(seed, S_HIDDEN, index, (n_rows, m["num_taps"] * m["target_hidden"]), 0.0, 1.0)


def gen_bonus(m: dict, seed: int, n: int, index: int = 0) -> np.ndarray:
    return rng(seed, S_BONUS, index).integers(0, m["vocab"], size=n, dtype=np.int64).astype(np.int32)


def gen_ctx_lengths(lo: int, hi: int, n: int, seed: int) -> np.ndarray:
    return rng(seed, S_CTXLEN).integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)


def gen_page_order(n_allocatable: int, seed: int) -> np.ndarray:
    """A seeded permutation of page ids 1..n_allocatable (page 0 is never handed out)."""
    return (rng(seed, S_PAGES).permutation(n_allocatable) + 1).astype(np.int32)


def gen_positions_gapped(start: int, n: int, seed: int, index: int = 0, max_gap: int = 3) -> np.ndarray:
    """Strictly increasing stamped positions with random gaps in 1..max_gap."""
    gaps = rng(seed, S_POS, index).integers(1, max_gap + 1, size=n, dtype=np.int64)
    return (start + np.cumsum(gaps) - gaps[0]).astype(np.int32)
