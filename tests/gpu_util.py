"""Helpers shared by the GPU parity tests: device copies of the seeded inputs, the
GPU-side drafter next to the CPU oracle, and the parity criteria.

Parity bar (floating point): max |logit_gpu - logit_oracle| <= 3e-2 * max |logit_oracle|
over the drafted rows, and >= 99.5 % argmax agreement over positions whose oracle top-2
gap is at least 1e-2. Integer state (block tables, slots, stamped positions) is compared
bit for bit."""
from __future__ import annotations

import numpy as np
import torch

import synth
from block_diffusion_draft_02_amd import binding as B
from oracle import dflash_oracle as O

DEV = torch.device("cuda:0")
LOGIT_REL_TOL = 3e-2
NEAR_TIE = 1e-2
AGREE_MIN = 0.995


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_weights(W: dict) -> dict:
    return {k: dev_bf16(v) for k, v in W.items()}


class Pair:
    """The HIP drafter and the oracle engine on the same seeded weights and pool."""

    def __init__(self, m, W, max_seq_len, max_batch, page_order=None, num_pages=0, oracle_cache=True):
        self.m, self.W = m, W
        self.Wd = dev_weights(W)
        self.gpu = B.Drafter(m, self.Wd, max_seq_len, max_batch, num_pages=num_pages, page_order=page_order)
        self.ora = O.Engine(m, W, max_seq_len, max_batch, page_order=page_order, num_pages=num_pages,
                            cache_weights=oracle_cache)

    def append(self, seq, H, positions=None):
        self.gpu.dflash_ctx_kv_append(seq, dev_bf16(H), positions=positions)
        self.ora.ctx_kv_append(seq, H, positions=positions)

    def append_batch(self, seqs, counts, H, positions=None):
        self.gpu.dflash_ctx_kv_append_batch(seqs, counts, dev_bf16(H), positions=positions)
        self.ora.ctx_kv_append_batch(seqs, counts, H, positions=positions)

    def forward(self, seqs, bonus, q_rope_pos=None, gamma=None, with_logits=True):
        """One forward on both sides. With a Markov head (or a DFlash2 selector) the oracle's
        chain is teacher-forced onto the GPU's drafts (row k's bias, or pair score, uses the
        GPU's draft of row k-1), so a branch the GPU took at a near-tie is compared on its own
        terms; the criteria then check each row's draft against the oracle's choice for the
        same previous token.
        with_logits=False passes no logits buffer (the drafts alone; logits are None)."""
        gamma = self.m["gamma_max"] if gamma is None else gamma
        n = len(seqs)
        toks = torch.full((n, gamma - 1), -1, dtype=torch.int32, device=DEV)
        logits = torch.empty((n * (gamma - 1), self.m["vocab"]), dtype=torch.float32, device=DEV) if with_logits else None
        self.gpu.dflash_block_forward(seqs, bonus, toks, logits, q_rope_pos=q_rope_pos, gamma=gamma)
        torch.cuda.synchronize()
        t = toks.cpu().numpy()
        prev = None
        if self.m.get("markov_rank", 0) or self.m.get("selector_rank", 0):
            prev = np.concatenate([np.asarray(bonus, dtype=np.int64).reshape(n, 1), t[:, :-1]], axis=1)
        ref = self.ora.block_forward(seqs, bonus, q_rope_pos=q_rope_pos, gamma=gamma, markov_prev=prev)
        lg = logits.cpu().numpy().astype(np.float64).reshape(n, gamma - 1, -1) if with_logits else None
        return (t, lg, ref)

    def close(self):
        self.gpu.close()


class Agreement:
    """Pools argmax agreement over many blocks."""

    def __init__(self):
        self.n = 0
        self.ok = 0
        self.max_rel = 0.0

    def add(self, toks, logits, ref):
        rl = ref["logits"]
        err = np.abs(logits - rl).max()
        scale = np.abs(rl).max()
        self.max_rel = max(self.max_rel, err / scale)
        assert err <= LOGIT_REL_TOL * scale, f"max|dlogit| {err:.4g} > {LOGIT_REL_TOL} * {scale:.4g}"
        s = np.sort(rl, axis=-1)
        keep = (s[..., -1] - s[..., -2]) >= NEAR_TIE
        self.n += int(keep.sum())
        self.ok += int(((toks == ref["tokens"]) & keep).sum())

    def check(self, min_positions=1):
        assert self.n >= min_positions, f"only {self.n} positions outside near-ties"
        rate = self.ok / self.n
        assert rate >= AGREE_MIN, f"argmax agreement {rate:.4f} over {self.n} positions"
        return rate


def pool_view(gpu: B.Drafter):
    """The whole KV pool as a host numpy uint16 array [L, P, 2, nkv, 16*hd]."""
    geo = gpu.dflash_pool_geometry()
    m = gpu.m
    buf = torch.empty(geo["pool_bytes"] // 2, dtype=torch.int16)
    gpu.dflash_debug_copy(B.DFLASH_BUF_POOL, buf)
    return buf.numpy().view(np.uint16).reshape(m["num_layers"], geo["num_pages"], 2, m["num_kv_heads"], -1)


def read_i32(gpu, which, n):
    buf = torch.empty(n, dtype=torch.int32)
    gpu.dflash_debug_copy(which, buf)
    return buf.numpy()


def read_i64(gpu, which, n):
    buf = torch.empty(n, dtype=torch.int64)
    gpu.dflash_debug_copy(which, buf)
    return buf.numpy()


def read_slot_kv(gpu, layer: int, slots: np.ndarray):
    """K and V rows stored at the given int64 slots of one layer, each [len(slots), nkv, hd]
    bf16 bits, read page by page (the pool of a large workload is not copied whole)."""
    geo = gpu.dflash_pool_geometry()
    m = gpu.m
    nkv, hd = m["num_kv_heads"], m["head_dim"]
    plb = geo["page_layer_bytes"]
    K = np.empty((len(slots), nkv, hd), dtype=np.uint16)
    V = np.empty((len(slots), nkv, hd), dtype=np.uint16)
    buf = torch.empty(plb // 2, dtype=torch.int16)
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        page, off = int(s) // 16, int(s) % 16
        gpu.dflash_debug_copy(B.DFLASH_BUF_POOL, buf, offset=(layer * geo["num_pages"] + page) * plb, nbytes=plb)
        pg = buf.numpy().view(np.uint16).reshape(2, nkv, -1)
        K[i] = pg[0].reshape(nkv, 16, hd)[:, off, :]
        V[i] = pg[1].reshape(nkv, hd, 16)[:, :, off]
    return K, V


# The pool holds bf16 K/V and the oracle rounds every cached row to bf16 once, from float64.
# The GPU rounds its fp32 result once too, so an element either matches the oracle's or sits
# one bf16 step away (when the two unrounded values straddle a rounding boundary). Elements
# near zero get an absolute floor: there the GPU's fp32 sums may differ from the exact ones by
# more than the element's own (tiny) step.
KV_FLOOR = 2.0 ** -16


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """The bf16 step at each value's magnitude: 2^(e-8) for |x| in [2^(e-1), 2^e); 0 at 0."""
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.where(x != 0, np.ldexp(1.0, e - 8), 0.0)


def assert_kv_close(got_bits: np.ndarray, want: np.ndarray, what: str, slots=None):
    """Cached K or V rows [n, nkv, hd] (bf16 bits) against the oracle's, element by element:
    |got - want| <= ulp(want) + KV_FLOOR * max|want|. The message names the layer / tensor
    (`what`), the slot, the kv head and the element of the worst miss."""
    g = O.widen(got_bits)
    w = np.asarray(want, dtype=np.float64)
    tol = bf16_ulp(w) + KV_FLOOR * np.abs(w).max()
    excess = np.abs(g - w) - tol
    if (excess > 0).any():
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        row = i[0] if slots is None else f"slot {int(np.asarray(slots)[i[0]])}"
        n_bad = int((excess > 0).sum())
        raise AssertionError(f"{what}: {n_bad} elements beyond one bf16 step; worst at row {row}, kv head {i[1]}, "
                             f"element {i[2]}: got {g[i]!r}, want {w[i]!r} (tolerance {tol[i]:.3g})")

