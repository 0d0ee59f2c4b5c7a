"""GPU parity of the FP8 E4M3 weight-only drafter (the FP8 weights phase of
metrale_model_arch/dflash_head/from_weights.rs): the quantized lm_head's codes and row
scales bit for bit against the oracle's quantizer, the forward against the oracle run on the
same dequantized weights (the bf16 parity bar), and bitwise batch invariance. Also a
vocabulary that is not a multiple of 16, in both weight formats."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_02_amd import binding as B
from oracle import dflash_oracle as O
from gpu_util import Agreement, Pair, dev_bf16, DEV

pytestmark = pytest.mark.gpu

SEED = 1101


def fp8(m):
    return dict(m, weight_format="fp8")


@pytest.fixture(scope="module")
def tiny():
    m = synth.model("tiny-L2-h256")
    return m, synth.gen_weights(m, SEED)


@pytest.fixture(scope="module")
def qwen3():
    w = synth.workload("qwen3-L8-h2048-ctx4096-b1")
    m = w["model_cfg"]
    return m, synth.gen_weights(m, w["seed"]), w["seed"]


def t16fp8_rows(raw: np.ndarray, K: int) -> np.ndarray:
    """Undo the T16-FP8 layout: tiles of 16 rows, 256-deep blocks of 4096 bytes whose byte
    (q*64 + lane)*16 + b holds row lane%16 at k = 64q + 32*(b/8) + 8*(lane/16) + b%8."""
    t = raw.size // (16 * K)
    a = raw.reshape(t, K // 256, 4, 4, 16, 2, 8)          # tile, block, q, lane/16, lane%16, b/8, b%8
    return a.transpose(0, 4, 1, 2, 5, 3, 6).reshape(t * 16, K)


def read_lmhead_tiles(gpu, tiles, K):
    """Codes [len(tiles)*16, K] and scales of the given 16-row tiles of the device lm_head."""
    tb = 16 * K
    buf = torch.empty(tb, dtype=torch.uint8)
    codes = []
    for t in tiles:
        gpu.dflash_debug_copy(B.DFLASH_BUF_FP8_LMHEAD, buf, offset=int(t) * tb, nbytes=tb)
        codes.append(t16fp8_rows(buf.numpy().copy(), K))
    sc = torch.empty(16, dtype=torch.float32)
    scales = []
    for t in tiles:
        gpu.dflash_debug_copy(B.DFLASH_BUF_FP8_LMHEAD_SCALE, sc, offset=int(t) * 64, nbytes=64)
        scales.append(sc.numpy().copy())
    return np.concatenate(codes), np.concatenate(scales)


@pytest.mark.parametrize("vocab", [1024, 1000])
def test_lmhead_codes_and_scales_bit_exact(tiny, vocab):
    m, W = tiny
    m = fp8(dict(m, vocab=vocab))
    W = dict(W, lm_head=W["lm_head"][:vocab], embed_tokens=W["embed_tokens"][:vocab])
    W["lm_head"] = W["lm_head"].copy()
    W["lm_head"][5] = 0                                    # an all-zero row: scale 1, codes 0
    W["lm_head"][9, 3] = synth.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]   # negative maximum
    d = B.Drafter(m, {k: dev_bf16(v) for k, v in W.items()}, 64, 1)
    tiles = range((vocab + 15) // 16)
    codes, scales = read_lmhead_tiles(d, tiles, m["hidden"])
    want_c, want_s = O.quantize_rows_fp8(W["lm_head"])
    assert np.array_equal(codes[:vocab], want_c) and np.array_equal(scales[:vocab], want_s)
    assert not codes[vocab:].any()                           # padding rows of the last tile
    assert scales[5] == 1.0 and codes[9, 3] == 0xFE
    d.close()


def test_forward_parity_many_blocks(tiny):
    """Skinny FP8 GEMMs and the persistent FP8 lm_head: 8 sequences, ragged contexts, non-
    contiguous pages, gaps in the positions, bands with a later query position."""
    m, W = tiny
    m = fp8(m)
    nb = 8
    P = O.pool_pages(256, 16, nb)[1]
    pair = Pair(m, W, 256, nb, page_order=synth.gen_page_order(P - 1, SEED + 1))
    lens = synth.gen_ctx_lengths(1, 200, nb, SEED)
    for s in range(nb):
        pos = synth.gen_positions_gapped(0, int(lens[s]), SEED, index=s) if s % 3 == 1 else None
        pair.append(s, synth.gen_hidden(m, SEED, int(lens[s]), 10 + s), positions=pos)
    agree = Agreement()
    rng = np.random.default_rng(7)
    for call in range(12):
        n = [1, 2, 4, 3][call % 4]
        seqs = [int(s) for s in rng.permutation(nb)[:n]]
        qpos = None
        if call % 2:
            qpos = [int(pair.ora.seqs[s]["pos"][-1]) + 1 + int(rng.integers(0, 5)) for s in seqs]
        toks, logits, ref = pair.forward(seqs, synth.gen_bonus(m, SEED, n, index=call), q_rope_pos=qpos,
                                         gamma=[16, 7, 16, 2][call % 4])
        agree.add(toks, logits, ref)
    rate = agree.check(min_positions=150)
    print(f"tiny fp8 parity: {agree.n} positions, agreement {rate:.4f}, max rel dlogit {agree.max_rel:.3e}")
    pair.close()


def test_wide_rows_parity_and_batch_invariance(tiny):
    """Seven bands (112 rows: the wide FP8 GEMMs and the wide FP8 lm_head) against the oracle,
    and each band equal bit for bit to the same band run alone (the skinny kernels)."""
    m, W = tiny
    m = fp8(m)
    nb = 7
    pair = Pair(m, W, 256, nb)
    lens = [7, 100, 33, 160, 64, 1, 17]
    for s in range(nb):
        pair.append(s, synth.gen_hidden(m, SEED, lens[s], 20 + s))
    agree = Agreement()
    bonus = synth.gen_bonus(m, SEED, nb, index=7)
    toks, logits, ref = pair.forward(list(range(nb)), bonus)
    agree.add(toks, logits, ref)
    agree.check(min_positions=80)
    V = m["vocab"]
    for s in range(nb):
        t1 = torch.empty((1, 15), dtype=torch.int32, device=DEV)
        l1 = torch.empty((15, V), dtype=torch.float32, device=DEV)
        pair.gpu.dflash_block_forward([s], [bonus[s]], t1, l1)
        torch.cuda.synchronize()
        assert np.array_equal(t1.cpu().numpy()[0], toks[s])
        assert np.array_equal(l1.cpu().numpy().astype(np.float64), logits[s])
    pair.close()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_ragged_vocab_forward(tiny, fmt):
    """vocab 1000: the lm_head's last 16-row tile holds 8 rows; no draft lands past the
    vocabulary, on the skinny and on the wide lm_head."""
    m, W = tiny
    m = dict(m, vocab=1000, weight_format=fmt)
    W = dict(W, lm_head=W["lm_head"][:1000], embed_tokens=W["embed_tokens"][:1000])
    pair = Pair(m, W, 128, 6)
    for s in range(6):
        pair.append(s, synth.gen_hidden(m, SEED, 30 + 9 * s, 40 + s))
    agree = Agreement()
    for call, seqs in enumerate(([0], [3, 1], list(range(6)))):
        toks, logits, ref = pair.forward(seqs, synth.gen_bonus(m, SEED, len(seqs), index=60 + call))
        agree.add(toks, logits, ref)
        assert toks.min() >= 0 and toks.max() < 1000
    agree.check(min_positions=100)
    pair.close()


def test_fullsize_lmhead_codes_sampled(qwen3):
    """vocab 151936 x 2048: the first, the last and 62 random 16-row tiles, bit for bit."""
    m, W, seed = qwen3
    m = fp8(m)
    d = B.Drafter(m, {k: dev_bf16(v) for k, v in W.items()}, 64, 1)
    nt = m["vocab"] // 16
    tiles = np.concatenate([[0, nt - 1], np.random.default_rng(seed).choice(np.arange(1, nt - 1), 62, replace=False)])
    codes, scales = read_lmhead_tiles(d, tiles, m["hidden"])
    rows = (tiles[:, None] * 16 + np.arange(16)).ravel()
    want_c, want_s = O.quantize_rows_fp8(W["lm_head"][rows])
    assert np.array_equal(scales, want_s) and np.array_equal(codes, want_c)
    d.close()


def test_fullsize_ctx4096_batch1_parity(qwen3):
    m, W, seed = qwen3
    m = fp8(m)
    pair = Pair(m, W, 8192, 1)
    pair.append(0, synth.gen_hidden(m, seed, 4096, 0))
    agree = Agreement()
    for call in range(24):
        qpos = None if call % 3 else [4096 + 7 * call]
        toks, logits, ref = pair.forward([0], synth.gen_bonus(m, seed, 1, index=call), q_rope_pos=qpos)
        agree.add(toks, logits, ref)
    rate = agree.check(min_positions=300)
    print(f"ctx4096 fp8 parity: {agree.n} positions, agreement {rate:.4f}, max rel dlogit {agree.max_rel:.3e}")
    pair.close()


def test_fullsize_batch16_parity_and_band_invariance(qwen3):
    """16 bands (240 rows: the wide FP8 GEMMs and lm_head) on non-contiguous pages against
    the oracle; four bands again alone, bit for bit."""
    m, W, seed = qwen3
    m = fp8(m)
    nb, max_seq = 16, 512
    P = O.pool_pages(max_seq, 16, nb)[1]
    pair = Pair(m, W, max_seq, nb, page_order=synth.gen_page_order(P - 1, seed))
    lens = synth.gen_ctx_lengths(1, 300, nb, seed)
    for s in range(nb):
        pair.append(s, synth.gen_hidden(m, seed, int(lens[s]), 50 + s))
    bonus = synth.gen_bonus(m, seed, nb, index=77)
    agree = Agreement()
    toks, logits, ref = pair.forward(list(range(nb)), bonus)
    agree.add(toks, logits, ref)
    rate = agree.check(min_positions=200)
    print(f"batch16 fp8 parity: {agree.n} positions, agreement {rate:.4f}, max rel dlogit {agree.max_rel:.3e}")
    V = m["vocab"]
    for s in (0, 5, 11, 15):
        t1 = torch.empty((1, 15), dtype=torch.int32, device=DEV)
        l1 = torch.empty((15, V), dtype=torch.float32, device=DEV)
        pair.gpu.dflash_block_forward([s], [bonus[s]], t1, l1)
        torch.cuda.synchronize()
        assert np.array_equal(t1.cpu().numpy()[0], toks[s])
        assert np.array_equal(l1.cpu().numpy().astype(np.float64), logits[s])
    pair.close()
