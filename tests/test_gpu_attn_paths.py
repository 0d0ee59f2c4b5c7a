"""GPU parity of the two attention paths in one call: in a drafter made for 8 or more
sequences, on a head_dim-128 layer without a window, a band of more than 2048 keys (planned
in at most 12 chunks) streams its K/V through
LDS, every other band loads K/V straight into registers; windowed layers always take the
register path. A small head_dim-128 drafter (2 layers, hidden 512, 16:2 heads) with bands on
both sides of 2048 keys, three LDS chunk widths, last chunks of 1 and of 30 keys, a windowed
layer next to a full one, and block widths
that leave query-row waves idle (gamma 2, 9, 16): logits against the oracle to the bf16
parity bar, and every band of the mixed call bit for bit equal to the same band alone."""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from gpu_util import Agreement, Pair, DEV

pytestmark = pytest.mark.gpu

SEED = 1501
# C + 16 keys: 2049 (LDS path, 9 chunks of 256 keys, the last holding 1 key), 2048 (the
# register path's largest band: 8 chunks of 256), 9246 (LDS path, 10 chunks of 1024, the last
# 30 keys), 316 (register path), 14016 (LDS path, 11 chunks of 1280: the longest chunks,
# dispatched first)
LENS = [2033, 2032, 9230, 300, 14000]


def _model(window):
    m = synth.model("qwen3-L8-h2048")
    m.update(num_layers=2, hidden=512, num_q_heads=16, num_kv_heads=2, head_dim=128, intermediate=1024,
             vocab=2048, num_taps=2, target_hidden=512)
    if window:
        m.update(sliding_window=window, layer_sliding=[True, False])
    return m


@pytest.mark.parametrize("window", [0, 3000])
def test_mixed_paths_parity_and_band_invariance(window):
    m = _model(window)
    W = synth.gen_weights(m, SEED)
    nb = len(LENS)
    # made for 8 sequences: the LDS path is on
    pair = Pair(m, W, max(LENS) + 64, 8,
                page_order=synth.gen_page_order(O.pool_pages(max(LENS) + 64, 16, 8)[1] - 1, SEED))
    for s, n in enumerate(LENS):
        pair.append(s, synth.gen_hidden(m, SEED, n, 70 + s))
    agree = Agreement()
    for call, gamma in enumerate([16, 9, 2]):
        bonus = synth.gen_bonus(m, SEED, nb, index=10 * call + (window > 0))
        seqs = list(range(nb))[::-1] if call == 1 else list(range(nb))
        toks, logits, ref = pair.forward(seqs, bonus, gamma=gamma)
        agree.add(toks, logits, ref)
        V = m["vocab"]
        for i, s in enumerate(seqs):
            t1 = torch.empty((1, gamma - 1), dtype=torch.int32, device=DEV)
            l1 = torch.empty((gamma - 1, V), dtype=torch.float32, device=DEV)
            pair.gpu.dflash_block_forward([s], [bonus[i]], t1, l1, gamma=gamma)
            torch.cuda.synchronize()
            assert np.array_equal(t1[0].cpu().numpy(), toks[i]), f"band {s} (C={LENS[s]}) drafts"
            assert np.array_equal(l1.cpu().numpy().astype(np.float64), logits[i]), f"band {s} (C={LENS[s]}) logits"
    rate = agree.check(min_positions=100)
    print(f"attention paths (window {window}): {agree.n} positions, agreement {rate:.4f}, "
          f"max rel dlogit {agree.max_rel:.3e}")
    pair.close()


# A drafter made for fewer than 8 sequences keeps every band on the register path, whose chunk
# plan widens chunks in 16-page steps so a band never has more than 32: 9000 keys take 32-page
# chunks (18 of them), 16400 keys (the wide drafter's full-attention layer) 48-page chunks (22),
# 24000 keys 48-page chunks (32, the cap; the last one partial).
WIDE_LENS = [8984, 16384, 23984]


@pytest.mark.parametrize("window", [0, 5000])
def test_widened_register_chunks_parity_and_band_invariance(window):
    m = _model(window)
    W = synth.gen_weights(m, SEED + 1)
    nb = len(WIDE_LENS)
    max_seq = max(WIDE_LENS) + 64
    pair = Pair(m, W, max_seq, 4,
                page_order=synth.gen_page_order(O.pool_pages(max_seq, 16, 4)[1] - 1, SEED + 1))
    for s, n in enumerate(WIDE_LENS):
        pair.append(s, synth.gen_hidden(m, SEED + 1, n, 90 + s))
    agree = Agreement()
    V = m["vocab"]
    for call, gamma in enumerate([16, 9, 16]):
        bonus = synth.gen_bonus(m, SEED + 1, nb, index=20 * call + (window > 0))
        seqs = list(range(nb))[::-1] if call == 1 else list(range(nb))
        qpos = [WIDE_LENS[s] + 40 * call for s in seqs] if call == 2 else None
        toks, logits, ref = pair.forward(seqs, bonus, q_rope_pos=qpos, gamma=gamma)
        agree.add(toks, logits, ref)
        for i, s in enumerate(seqs):
            t1 = torch.empty((1, gamma - 1), dtype=torch.int32, device=DEV)
            l1 = torch.empty((gamma - 1, V), dtype=torch.float32, device=DEV)
            pair.gpu.dflash_block_forward([s], [bonus[i]], t1, l1, q_rope_pos=None if qpos is None else [qpos[i]],
                                          gamma=gamma)
            torch.cuda.synchronize()
            assert np.array_equal(t1[0].cpu().numpy(), toks[i]), f"band {s} (C={WIDE_LENS[s]}) drafts"
            assert np.array_equal(l1.cpu().numpy().astype(np.float64), logits[i]), f"band {s} logits"
    rate = agree.check(min_positions=80)
    print(f"widened register chunks (window {window}): {agree.n} positions, agreement {rate:.4f}, "
          f"max rel dlogit {agree.max_rel:.3e}")
    pair.close()
