"""Planted mistakes for the oracle (a pytest plugin, loaded only by tests/test_oracle_mutants.py
into a child pytest run of the oracle's pins: `-p _oracle_mutants` with DFLASH_ORACLE_MUTANT
naming one entry of MUTANTS).

Each mistake is one textual change to one function or method of oracle/dflash_oracle.py: its
source is read, the change applied (the original text must occur exactly once), and the
changed definition is compiled in the module's namespace and put in place of the original,
for the child process only. The oracle's file is never modified. The changes are the kinds
of mistake the pins are meant to catch: a dropped term or normalisation, a wrong sign, index,
offset or constant, swapped operands, a wrong tie rule."""
import inspect
import os
import sys
import textwrap

# name: (function or Class.method, original text, planted text)
MUTANTS = {
    # elementary steps
    "rms_offset_form": ("rms_norm", "np.sqrt(ms + eps) * w", "np.sqrt(ms + eps) * (1.0 + w)"),
    "rms_eps_outside": ("rms_norm", "np.sqrt(ms + eps)", "(np.sqrt(ms) + eps)"),
    "silu_is_sigmoid": ("silu", "x / (1.0 + np.exp(-x))", "1.0 / (1.0 + np.exp(-x))"),
    "inv_freq_exponent": ("inv_freq_plain", "-2.0 * j / head_dim", "-1.0 * j / head_dim"),
    "yarn_ramp_reversed": ("inv_freq_yarn", "(base / factor) * ramp + base * (1.0 - ramp)",
                           "base * ramp + (base / factor) * (1.0 - ramp)"),
    "yarn_low_from_slow": ("yarn_bounds", "math.floor(corr(beta_fast))", "math.floor(corr(beta_slow))"),
    "yarn_mscale_coef": ("yarn_mscale", "0.1 * math.log(factor)", "0.07 * math.log(factor)"),
    "rope_sign": ("rope_neox", "x1 * c - x2 * s", "x1 * c + x2 * s"),
    "rope_interleaved_pairs": ("rope_neox", "x1, x2 = x[..., :half], x[..., half:]",
                               "x1, x2 = x[..., 0::2], x[..., 1::2]"),
    "gqa_head_map": ("gqa_attention", "kh = h // G", "kh = h % nkv"),
    "window_inclusive": ("gqa_attention", "k_pos[None, :].astype(np.int64)) < window",
                         "k_pos[None, :].astype(np.int64)) <= window"),
    "attn_unscaled": ("gqa_attention", ".T) * scale", ".T) * 1.0"),
    "attn_causal": ("gqa_attention", "vis = np.ones((T, k.shape[0]), dtype=bool)",
                    "vis = q_pos[:, None].astype(np.int64) >= k_pos[None, :].astype(np.int64)"),
    "argmax_highest_tie": ("argmax_lowest", "np.argmax(x, axis=-1)",
                           "(x.shape[-1] - 1 - np.argmax(x[..., ::-1], axis=-1))"),
    "bf16_truncates": ("round_bf16", "np.round(f * 256.0)", "np.trunc(f * 256.0)"),
    "pool_no_spare": ("pool_pages", "per_seq * max(1, max_batch) + 1", "per_seq * max(1, max_batch)"),
    "pool_no_gamma": ("pool_pages", "(max_seq_len + gamma_max + 1)", "(max_seq_len + 1)"),
    # FP8
    "e4m3_bias_8": ("e4m3_decode", "np.exp2((e - 7)", "np.exp2((e - 8)"),
    "e4m3_ties_up": ("e4m3_encode", "np.where(lo % 2 == 0, lo, hi)", "hi"),
    "fp8_scale_over_240": ("quantize_rows_fp8", "amax / np.float32(E4M3_MAX)", "amax / np.float32(240.0)"),
    # context append
    "fc_no_hidden_norm": ("Drafter.ctx_features", 'return rms_norm(f, self.w("hidden_norm"), m["rms_eps"])',
                          "return f"),
    "ctx_k_no_norm": ("Drafter.ctx_kv", 'k = rms_norm(k, self.lw(l, "k_norm"), m["rms_eps"])', "k = k"),
    "ctx_pos_shift": ("Drafter.ctx_kv", "np.asarray(positions)[:, None]", "(np.asarray(positions) + 1)[:, None]"),
    "ctx_k_v_swapped": ("Drafter.ctx_kv", "out.append((self.cache_store(k), self.cache_store(v)))",
                        "out.append((self.cache_store(v), self.cache_store(k)))"),
    "mscale_squared": ("Drafter.rope_rows", "y = y * self.mscale", "y = y * self.mscale * self.mscale"),
    # block forward
    "q_norm_dropped": ("Drafter.block_hidden", 'q = self.rope_rows(rms_norm(q, self.lw(l, "q_norm"), eps), bpos[:, None])',
                       "q = self.rope_rows(q, bpos[:, None])"),
    "block_k_no_norm": ("Drafter.block_hidden", 'kb = self.rope_rows(rms_norm(kb, self.lw(l, "k_norm"), eps), bpos[:, None])',
                        "kb = self.rope_rows(kb, bpos[:, None])"),
    "attn_residual_dropped": ("Drafter.block_hidden", "x1 = x + (self.dconv_finish(o, kern_a) if d2 else o)",
                              "x1 = (self.dconv_finish(o, kern_a) if d2 else o)"),
    "mlp_residual_dropped": ("Drafter.block_hidden", "x = x1 + (self.dconv_finish(mo, kern_m) if d2 else mo)",
                             "x = (self.dconv_finish(mo, kern_m) if d2 else mo)"),
    "gate_up_swapped": ("Drafter.block_hidden", "(silu(g) * u)", "(silu(u) * g)"),
    "post_norm_weight": ("Drafter.block_hidden", 'rms_norm(x1, self.lw(l, "post_attention_layernorm"), eps)',
                         'rms_norm(x1, self.lw(l, "input_layernorm"), eps)'),
    "final_norm_dropped": ("Drafter.block_hidden", 'return rms_norm(x, self.w("norm"), eps)', "return x"),
    "block_keys_zeroed": ("Drafter.block_hidden", "k_all = np.concatenate([ctx_k[l], self.cache_store(kb)], axis=0)",
                          "k_all = np.concatenate([ctx_k[l], 0.0 * self.cache_store(kb)], axis=0)"),
    "block_k_unrounded": ("Drafter.block_hidden", "k_all = np.concatenate([ctx_k[l], self.cache_store(kb)], axis=0)",
                          "k_all = np.concatenate([ctx_k[l], kb], axis=0)"),
    "drafts_from_row_0": ("Drafter.block_forward", "logits = self.lm_head(y[1:])", "logits = self.lm_head(y[:-1])"),
    "block_pos_shift": ("Drafter.block_forward", "bpos = q_rope_pos + np.arange(gamma, dtype=np.int64)",
                        "bpos = q_rope_pos + 1 + np.arange(gamma, dtype=np.int64)"),
    "lm_head_chunk_gap": ("Drafter.lm_head", "e = min(V, s + chunk)", "e = min(V, s + chunk - 1)"),
    # the page model
    "slot_page_offset": ("PagePool.slots", "bt[p // PAGE] * PAGE + (p % PAGE)", "bt[p // PAGE] * PAGE + (p % (PAGE - 1))"),
    "pool_lifo_free": ("PagePool.ensure", "new, self.free = self.free[:n], self.free[n:]",
                       "new, self.free = self.free[len(self.free) - n:], self.free[:len(self.free) - n]"),
    # DSpark
    "markov_no_feedback": ("Drafter.markov_chain", "t = int(drafts[k])", "t = int(bonus)"),
    "markov_w1_w2_order": ("Drafter.markov_chain", 'out[k] += w2 @ widen(self.bits["markov_w1"][tk], self.dtype)',
                           'out[k] += w2 @ widen(self.bits["markov_w1"][t], self.dtype) * 0.5'),
    # DFlash2
    "dconv_tap_shift": ("Drafter.dconv_prepare", "u[j:] += kern[j:, 0, j] * hn[:T - j]",
                        "u[j:] += kern[j:, 0, j] * hn[j:]"),
    "dconv_no_dynamic": ("Drafter.dconv_prepare", "kern = base[None] + np.repeat(D, gs, axis=3)",
                         "kern = base[None] + 0.0 * np.repeat(D, gs, axis=3)"),
    "dconv_finish_app0": ("Drafter.dconv_finish", "v[j:] += kern[j:, 1, j] * sub[:T - j]",
                          "v[j:] += kern[j:, 0, j] * sub[:T - j]"),
    "topk_ties_high": ("Drafter.top_k_candidates", 'np.argsort(-logits, axis=-1, kind="stable")',
                       'np.argsort(-logits[..., ::-1], axis=-1, kind="stable")'),
    "selector_no_chain": ("Drafter.selector_walk", "t = int(drafts[r])", "t = int(bonus)"),
}


def _plant(mod, target, old, new):
    owner, name = (mod, target) if "." not in target else (getattr(mod, target.split(".")[0]), target.split(".")[1])
    raw = owner.__dict__[name]
    fn = raw.__func__ if isinstance(raw, staticmethod) else raw
    src = textwrap.dedent(inspect.getsource(fn))
    if src.count(old) != 1:
        raise RuntimeError(f"mutant text for {target} occurs {src.count(old)} times")
    src = src.replace(old, new)
    if src.startswith("@staticmethod"):
        src = src[len("@staticmethod"):].lstrip()
    ns = {}
    exec(compile(src, f"<mutant of {target}>", "exec"), mod.__dict__, ns)
    planted = ns[name]
    setattr(owner, name, staticmethod(planted) if isinstance(raw, staticmethod) else planted)


def pytest_configure(config):
    name = os.environ.get("DFLASH_ORACLE_MUTANT", "")
    if not name:
        return
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    from oracle import dflash_oracle as O
    target, old, new = MUTANTS[name]
    _plant(O, target, old, new)
