"""GPU parity at the wide drafter's full shape (5 layers, hidden 5376, GQA 64:8,
head_dim 128, ff 10752, vocab 262144, 6 taps of hidden 5376, YaRN factor 32 with mscale on
q and k, window 2048 on layers 0-3).

  * a 2200-row context: every block row of the sliding layers loses its oldest keys to the
    window, so the sliding layers start their key range mid-context; 64 blocks, some at
    RoPE positions past kv_len, against the oracle;
  * the workload's own 16384-row context (the full-attention layer's 16400 keys run the
    register path's widened 48-page chunks, the sliding layers start 14000+ keys in): the
    cached K/V of sampled rows of every layer against the oracle, then 64 blocks against the
    oracle computing the whole context in fp64, a third of them at RoPE positions past
    kv_len; and the forward is deterministic."""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from gpu_util import Agreement, Pair, assert_kv_close, dev_bf16, read_slot_kv, DEV
from block_diffusion_draft_02_amd import binding as B

pytestmark = pytest.mark.gpu
WORKLOAD = "wide-L5-h5376-yarn-swa2048-ctx16384-b1"


@pytest.fixture(scope="module")
def wide():
    w = synth.workload(WORKLOAD)
    m = w["model_cfg"]
    return m, synth.gen_weights(m, w["seed"]), w["seed"], w


def test_wide_window_crossing_parity(wide):
    m, W, seed, _ = wide
    C = 2200
    pair = Pair(m, W, C + 200, 1)
    pair.append(0, synth.gen_hidden(m, seed, C, 0))
    agree = Agreement()
    for call in range(64):
        qpos = None if call % 3 else [C + 5 * call]
        toks, logits, ref = pair.forward([0], synth.gen_bonus(m, seed, 1, index=call), q_rope_pos=qpos)
        agree.add(toks, logits, ref)
    rate = agree.check(min_positions=900)
    print(f"wide ctx{C} parity: {agree.n} positions, agreement {rate:.4f}, max rel dlogit {agree.max_rel:.3e}")
    pair.close()


def test_wide_full_context_parity_64_blocks(wide):
    m, W, seed, w = wide
    C = w["ctx"][0]
    H = synth.gen_hidden(m, seed, C, 1)
    pair = Pair(m, W, w["max_seq_len"], 1)
    for r0 in range(0, C, 2048):
        pair.append(0, H[r0:r0 + 2048])
        print(f"appended {r0 + 2048} of {C} rows on both sides", flush=True)
    assert pair.gpu.dflash_seq_info(0)[0] == C == pair.ora.kv_len(0)
    rows = np.array([0, 1, 2047, 2048, 8191, 12345, C - 17, C - 1])
    slots = pair.ora.pool.slots(0, rows)
    st = pair.ora.seqs[0]
    for l in range(m["num_layers"]):
        K, V = read_slot_kv(pair.gpu, l, slots)
        for got, want, name in ((K, st["k"][l][rows], "K"), (V, st["v"][l][rows], "V")):
            assert_kv_close(got, want, f"layer {l} {name}", slots)
    agree = Agreement()
    for call in range(64):
        qpos = None if call % 3 else [C + 11 * call]
        toks, logits, ref = pair.forward([0], synth.gen_bonus(m, seed, 1, index=500 + call), q_rope_pos=qpos)
        agree.add(toks, logits, ref)
        if call % 16 == 15:
            print(f"{call + 1} blocks: {agree.n} positions, agreement {agree.ok / max(1, agree.n):.4f}, "
                  f"max rel dlogit {agree.max_rel:.3e}", flush=True)
    rate = agree.check(min_positions=900)
    print(f"wide ctx{C} parity: {agree.n} positions, agreement {rate:.4f}, max rel dlogit {agree.max_rel:.3e}")
    V_ = m["vocab"]
    outs = []
    for _ in range(2):
        t = torch.empty((1, 15), dtype=torch.int32, device=DEV)
        lg = torch.empty((15, V_), dtype=torch.float32, device=DEV)
        pair.gpu.dflash_block_forward([0], [7], t, lg)
        torch.cuda.synchronize()
        outs.append((t.clone(), lg.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    pair.close()
