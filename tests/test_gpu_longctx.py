"""The long-context batched workload: 32 sequences with contexts U{8192..32768} on a pool
of permuted pages, 2048 more rows appended to each, then one 32-band block forward.

  * sampled rows of every sequence's 2048-row append: the cached K/V of every layer
    against the oracle computed row by row (the append is row-independent);
  * the band with the shortest context against the oracle, which computes that whole
    sequence (prefix, append and block) in fp64;
  * sampled bands of the 32-band call bit for bit equal to the same band run alone."""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from gpu_util import Agreement, assert_kv_close, dev_bf16, read_slot_kv, DEV
from block_diffusion_draft_02_amd import binding as B

pytestmark = pytest.mark.gpu
WORKLOAD = "qwen3-L8-h2048-b32-ctx8192to32768-append2048"
CHUNK = 2048


def test_longctx_32_bands_append_and_forward():
    w = synth.workload(WORKLOAD)
    m, seed, nb = w["model_cfg"], w["seed"], w["batch"]
    W = synth.gen_weights(m, seed)
    lens = synth.gen_ctx_lengths(w["ctx"][0], w["ctx"][1], nb, seed)
    gamma, V = m["gamma_max"], m["vocab"]
    per_seq = -(-(w["max_seq_len"] + gamma + 1) // 16)
    d = B.Drafter(m, {k: dev_bf16(v) for k, v in W.items()}, w["max_seq_len"], nb,
                  page_order=synth.gen_page_order(per_seq * nb, seed))

    def hidden(s, c, n):   # chunk c of sequence s; the appended rows are chunk 999
        return synth.gen_hidden(m, seed, n, 1000 * s + c)

    for s in range(nb):
        for c, r0 in enumerate(range(0, int(lens[s]), CHUNK)):
            d.dflash_ctx_kv_append(s, dev_bf16(hidden(s, c, min(CHUNK, int(lens[s]) - r0))))
    print(f"prefilled {int(lens.sum())} rows over {nb} sequences", flush=True)
    app = {}
    for s in range(nb):
        app[s] = hidden(s, 999, w["append"])
        d.dflash_ctx_kv_append(s, dev_bf16(app[s]))
        assert d.dflash_seq_info(s)[0] == int(lens[s]) + w["append"]

    ref = O.Drafter(m, W)
    rows = np.array([0, 777, w["append"] - 1])
    for s in (0, 13, nb - 1):
        F = ref.ctx_features(app[s][rows])
        pos = int(lens[s]) + rows
        kv = ref.ctx_kv(F, pos)
        bt = np.asarray(d.dflash_seq_info(s)[1], dtype=np.int64)
        slots = bt[pos // 16] * 16 + pos % 16
        for l in range(m["num_layers"]):
            K, Vv = read_slot_kv(d, l, slots)
            for got, want, name in ((K, kv[l][0], "K"), (Vv, kv[l][1], "V")):
                assert_kv_close(got, want, f"seq {s} layer {l} {name}", slots)

    bonus = synth.gen_bonus(m, seed, nb)
    tb = torch.empty((nb, gamma - 1), dtype=torch.int32, device=DEV)
    lb = torch.empty((nb * (gamma - 1), V), dtype=torch.float32, device=DEV)
    d.dflash_block_forward(list(range(nb)), bonus, tb, lb)
    torch.cuda.synchronize()
    assert int(tb.min()) >= 0 and int(tb.max()) < V
    s_min = int(np.argmin(lens))
    for s in sorted({0, s_min, nb - 1}):
        t1 = torch.empty((1, gamma - 1), dtype=torch.int32, device=DEV)
        l1 = torch.empty((gamma - 1, V), dtype=torch.float32, device=DEV)
        d.dflash_block_forward([s], [bonus[s]], t1, l1)
        torch.cuda.synchronize()
        assert torch.equal(t1[0], tb[s]) and torch.equal(l1, lb[s * (gamma - 1):(s + 1) * (gamma - 1)])
    got_t = tb[s_min].cpu().numpy()[None]
    got_l = lb[s_min * (gamma - 1):(s_min + 1) * (gamma - 1)].cpu().numpy().astype(np.float64)[None]
    d.close()

    # the oracle on the shortest band, the same rows in the same chunks
    eng = O.Engine(m, W, int(lens[s_min]) + w["append"] + gamma + 16, 1)
    for c, r0 in enumerate(range(0, int(lens[s_min]), CHUNK)):
        eng.ctx_kv_append(0, hidden(s_min, c, min(CHUNK, int(lens[s_min]) - r0)))
    eng.ctx_kv_append(0, app[s_min])
    r = eng.block_forward([0], [int(bonus[s_min])])
    agree = Agreement()
    agree.add(got_t, got_l, r)
    rate = agree.check(min_positions=10)
    print(f"longctx band {s_min} (C={int(lens[s_min]) + w['append']}): agreement {rate:.4f}, "
          f"max rel dlogit {agree.max_rel:.3e}")
