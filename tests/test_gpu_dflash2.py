"""GPU parity of DFlash2 (spark_model/layers/dflash_head.rs: the DFlash2 fields, scratch and
kernel names; the composition is the library's reading, so parity is against the oracle's
reading of it, which the pages do not pin): logits to the bf16 parity bar; each drafted row's
16 candidates against the oracle's, where its 16th and 17th logits are not a near-tie (and
within the near-tie where they are); the walk's drafts against the oracle teacher-forced onto
the GPU's previous drafts, wherever both sides hold the same candidates and the oracle's best
two scores are not a near-tie; bitwise batch invariance on the skinny and the wide trunk."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_02_amd import binding as B
from oracle import dflash_oracle as O
from gpu_util import LOGIT_REL_TOL, NEAR_TIE, AGREE_MIN, Pair, dev_bf16, DEV

pytestmark = pytest.mark.gpu

SEED = 1401


@pytest.fixture(scope="module")
def tiny():
    m = synth.model("tiny-L2-h256-dflash2")
    return m, synth.gen_weights(m, SEED)


class D2Check:
    """Pools the DFlash2 criteria over many calls."""

    def __init__(self):
        self.rows = self.cand_ok = self.cand_n = self.pick_ok = self.pick_n = 0
        self.max_rel = 0.0

    def add(self, pair, toks, logits, ref):
        rl = ref["logits"]
        err, scale = np.abs(logits - rl).max(), np.abs(rl).max()
        self.max_rel = max(self.max_rel, err / scale)
        assert err <= LOGIT_REL_TOL * scale, f"max|dlogit| {err:.4g} > {LOGIT_REL_TOL} * {scale:.4g}"
        n, g1 = toks.shape
        sel = torch.empty(n * g1 * 16, dtype=torch.int32)
        pair.gpu.dflash_debug_copy(B.DFLASH_BUF_SEL_IDX, sel, nbytes=n * g1 * 16 * 4)
        sel = sel.numpy().reshape(n, g1, 16)
        srt = -np.sort(-rl, axis=-1)
        for b in range(n):
            for r in range(g1):
                self.rows += 1
                assert toks[b, r] in sel[b, r], "a draft outside the row's candidates"
                boundary = srt[b, r, 15] - srt[b, r, 16]
                if boundary >= NEAR_TIE:
                    self.cand_n += 1
                    self.cand_ok += int(set(sel[b, r]) == set(ref["cand"][b, r]))
                else:
                    # a near-tie at the boundary: every GPU candidate still ranks within it
                    assert (rl[b, r, sel[b, r]] >= srt[b, r, 15] - NEAR_TIE).all()
                # the draft is comparable wherever both sides hold the same candidates
                sc = np.sort(ref["scores"][b, r])
                if set(sel[b, r]) == set(ref["cand"][b, r]) and sc[-1] - sc[-2] >= NEAR_TIE:
                    self.pick_n += 1
                    self.pick_ok += int(toks[b, r] == ref["tokens"][b, r])

    def check(self, min_rows):
        assert self.cand_n >= min_rows // 2 and self.pick_n >= min_rows, (self.rows, self.cand_n, self.pick_n)
        cr, pr = self.cand_ok / self.cand_n, self.pick_ok / self.pick_n
        assert cr >= AGREE_MIN, f"candidate sets agree on {cr:.4f} of {self.cand_n} rows"
        assert pr >= AGREE_MIN, f"walk drafts agree on {pr:.4f} of {self.pick_n} rows"
        return cr, pr


def test_parity_many_blocks(tiny):
    m, W = tiny
    nb = 6
    pair = Pair(m, W, 256, nb, page_order=synth.gen_page_order(O.pool_pages(256, 16, nb)[1] - 1, SEED))
    lens = synth.gen_ctx_lengths(1, 180, nb, SEED)
    for s in range(nb):
        pair.append(s, synth.gen_hidden(m, SEED, int(lens[s]), 10 + s))
    chk = D2Check()
    rng = np.random.default_rng(12)
    for call in range(16):
        n = [1, 3, 6, 2][call % 4]
        seqs = [int(s) for s in rng.permutation(nb)[:n]]
        gamma = [16, 9, 16, 2][call % 4]
        qpos = [int(pair.ora.seqs[s]["pos"][-1]) + 1 + call for s in seqs] if call % 3 == 2 else None
        bonus = synth.gen_bonus(m, SEED, n, index=call)
        toks, logits, ref = pair.forward(seqs, bonus, q_rope_pos=qpos, gamma=gamma)
        chk.add(pair, toks, logits, ref)
        # without a logits buffer the drafts are the same
        t2 = torch.full((n, gamma - 1), -1, dtype=torch.int32, device=DEV)
        pair.gpu.dflash_block_forward(seqs, bonus, t2, None, q_rope_pos=qpos, gamma=gamma)
        torch.cuda.synchronize()
        assert np.array_equal(t2.cpu().numpy(), toks)
    cr, pr = chk.check(min_rows=200)
    print(f"tiny dflash2: {chk.rows} rows, candidates {cr:.4f}, drafts {pr:.4f}, max rel dlogit {chk.max_rel:.3e}")
    pair.close()


@pytest.mark.parametrize("nb", [7, 20])
def test_batch_invariance_bitwise(tiny, nb):
    """7 and 20 bands (the wide trunk, the convs' row pairs never crossing a band) against
    each band alone (the skinny trunk): drafts and logits bit for bit."""
    m, W = tiny
    d = B.Drafter(m, {k: dev_bf16(v) for k, v in W.items()}, 128, nb)
    lens = synth.gen_ctx_lengths(1, 100, nb, SEED + nb)
    for s in range(nb):
        d.dflash_ctx_kv_append(s, dev_bf16(synth.gen_hidden(m, SEED, int(lens[s]), 60 + s)))
    bonus = synth.gen_bonus(m, SEED, nb, index=90 + nb)
    V = m["vocab"]
    tb = torch.empty((nb, 15), dtype=torch.int32, device=DEV)
    lb = torch.empty((nb * 15, V), dtype=torch.float32, device=DEV)
    d.dflash_block_forward(list(range(nb)), bonus, tb, lb)
    for s in range(0, nb, 3):
        t1 = torch.empty((1, 15), dtype=torch.int32, device=DEV)
        l1 = torch.empty((15, V), dtype=torch.float32, device=DEV)
        d.dflash_block_forward([s], [bonus[s]], t1, l1)
        torch.cuda.synchronize()
        assert torch.equal(t1[0], tb[s]) and torch.equal(l1, lb[s * 15:(s + 1) * 15])
    d.close()


def test_fp8_trunk(tiny):
    """FP8 E4M3 trunk weights (the convs' projections and the selector stay bf16)."""
    m0, _ = tiny
    m = dict(m0, weight_format="fp8")
    W = synth.gen_weights(m, SEED + 1)
    pair = Pair(m, W, 128, 4)
    for s, n in enumerate([9, 70, 33, 101]):
        pair.append(s, synth.gen_hidden(m, SEED + 1, n, 20 + s))
    chk = D2Check()
    for call in range(6):
        seqs = [[0], [1, 2], [3, 0, 1, 2], [2], [1], [3, 2]][call]
        toks, logits, ref = pair.forward(seqs, synth.gen_bonus(m, SEED, len(seqs), index=40 + call))
        chk.add(pair, toks, logits, ref)
    chk.check(min_rows=60)
    pair.close()


def test_fullsize_batch1_and_batch16():
    """The 2048-hidden drafter with DFlash2 convs (128 groups a site) and a rank-256 selector
    over vocab 151936: one band on a 2048-row context, then 16 bands."""
    m = synth.model("qwen3-L8-h2048-dflash2")
    seed = 1402
    W = synth.gen_weights(m, seed)
    pair = Pair(m, W, 2304, 16, page_order=synth.gen_page_order(O.pool_pages(2304, 16, 16)[1] - 1, seed))
    pair.append(0, synth.gen_hidden(m, seed, 2048, 0))
    lens = synth.gen_ctx_lengths(1, 200, 15, seed)
    for s in range(1, 16):
        pair.append(s, synth.gen_hidden(m, seed, int(lens[s - 1]), s))
    chk = D2Check()
    for call in range(6):
        toks, logits, ref = pair.forward([0], synth.gen_bonus(m, seed, 1, index=call))
        chk.add(pair, toks, logits, ref)
    toks, logits, ref = pair.forward(list(range(16))[::-1], synth.gen_bonus(m, seed, 16, index=50))
    chk.add(pair, toks, logits, ref)
    cr, pr = chk.check(min_rows=150)
    print(f"full-size dflash2: {chk.rows} rows, candidates {cr:.4f}, drafts {pr:.4f}, max rel dlogit {chk.max_rel:.3e}")
    pair.close()
