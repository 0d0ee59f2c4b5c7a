"""GPU parity at the wide drafter's full shape (5 layers, hidden 5376, GQA 64:8,
head_dim 128, ff 10752, vocab 262144, 6 taps of hidden 5376, YaRN factor 32 with mscale on
q and k, window 2048 on layers 0-3).

  * a 2200-row context: every block row of the sliding layers loses its oldest keys to the
    window, so the sliding layers start their key range mid-context; 64 blocks, some at
    RoPE positions past kv_len, against the oracle;
  * the workload's own 16384-row context: the K/V the append caches for sampled rows of
    every layer against the oracle computed row by row (the append is row-independent),
    and two forwards of that context, deterministic and in range."""
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


def test_wide_full_context_sampled_kv_and_forward(wide):
    m, W, seed, w = wide
    C = w["ctx"][0]
    H = synth.gen_hidden(m, seed, C, 1)
    d = B.Drafter(m, {k: dev_bf16(v) for k, v in W.items()}, w["max_seq_len"], 1)
    for r0 in range(0, C, 2048):
        d.dflash_ctx_kv_append(0, dev_bf16(H[r0:r0 + 2048]))
    assert d.dflash_seq_info(0)[0] == C
    print(f"appended {C} rows", flush=True)
    rows = np.array([0, 1, 2047, 2048, 8191, 12345, C - 17, C - 1])
    ref = O.Drafter(m, W)
    F = ref.ctx_features(H[rows])
    kv = ref.ctx_kv(F, rows)
    bt = d.dflash_seq_info(0)[1]
    slots = np.asarray(bt, dtype=np.int64)[rows // 16] * 16 + rows % 16
    for l in range(m["num_layers"]):
        K, V = read_slot_kv(d, l, slots)
        for got, want, name in ((K, kv[l][0], "K"), (V, kv[l][1], "V")):
            assert_kv_close(got, want, f"layer {l} {name}", slots)
    V_ = m["vocab"]
    outs = []
    for _ in range(2):
        t = torch.empty((1, 15), dtype=torch.int32, device=DEV)
        lg = torch.empty((15, V_), dtype=torch.float32, device=DEV)
        d.dflash_block_forward([0], [7], t, lg)
        torch.cuda.synchronize()
        outs.append((t.clone(), lg.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert bool(torch.isfinite(outs[0][1]).all()) and int(outs[0][0].min()) >= 0 and int(outs[0][0].max()) < V_
    d.close()
