"""Context appends of more than 256 rows on drafters whose K/V block (num_kv_heads * head_dim
columns) is a multiple of 256 wide: there the K/V GEMM applies k_norm and RoPE and writes K and
V into the pages from its own epilogue. Head dims 32, 64 and 128 (plain RoPE and YaRN), appends
that start mid-page and end in a ragged row tile, pages handed out in a permuted order, caller
positions with gaps:
  * every cached row of every layer against the oracle, pages nobody owns still zero;
  * the same rows appended in one call and in two (both long) equal bit for bit;
  * forwards over the result against the oracle."""
import numpy as np
import pytest

import synth
from oracle import dflash_oracle as O
from gpu_util import Agreement, Pair, assert_kv_close, dev_bf16, dev_weights, pool_view, read_i32
from block_diffusion_draft_02_amd import binding as B

pytestmark = pytest.mark.gpu
SEED = 2027

SHAPES = {
    "hd32": dict(num_q_heads=8, num_kv_heads=8, head_dim=32),
    "hd64": dict(num_q_heads=8, num_kv_heads=4, head_dim=64),
    "hd128-yarn": dict(num_q_heads=4, num_kv_heads=2, head_dim=128, rope_type="yarn", yarn_factor=4.0,
                       yarn_orig_max_pos=256.0, yarn_beta_fast=32.0, yarn_beta_slow=1.0),
}


def _model(name):
    return dict(synth.model("tiny-L2-h256"), **SHAPES[name])


def _check_pool(pair, seqs):
    m = pair.m
    hd, nkv = m["head_dim"], m["num_kv_heads"]
    geo = pair.gpu.dflash_pool_geometry()
    pool = pool_view(pair.gpu)
    kpos = read_i32(pair.gpu, B.DFLASH_BUF_KPOS, geo["num_pages"] * 16)
    owned = set()
    for seq in seqs:
        s = pair.ora.seqs[seq]
        n = s["pos"].shape[0]
        slots = pair.ora.pool.slots(seq, range(n))
        pages, offs = slots // 16, slots % 16
        owned |= set(pair.ora.block_table(seq))
        assert np.array_equal(kpos[slots], s["pos"]), "stamped positions"
        for l in range(m["num_layers"]):
            K = pool[l, pages, 0].reshape(n, nkv, 16, hd)[np.arange(n), :, offs, :]
            V = pool[l, pages, 1].reshape(n, nkv, hd, 16)[np.arange(n), :, :, offs]
            for got, want, name in ((K, s["k"][l], "K"), (V, s["v"][l], "V")):
                assert_kv_close(got, want, f"seq {seq} layer {l} {name}", slots)
    free = [p for p in range(geo["num_pages"]) if p not in owned]
    assert 0 in free and not pool[:, free].any(), "a write outside the owned pages"


@pytest.mark.parametrize("shape", list(SHAPES))
def test_fused_append_rows_match_oracle(shape):
    """Sequence 0: 21 rows (the skinny form), then 1000 (four row tiles, the last ragged,
    starting at page offset 5), then 300 (page offset 13). Sequence 1: 777 rows at gapped
    caller positions. Then forwards over both."""
    m = _model(shape)
    W = synth.gen_weights(m, SEED)
    P = O.pool_pages(1400, m["gamma_max"], 2)[1]
    pair = Pair(m, W, 1400, 2, page_order=synth.gen_page_order(P - 1, SEED))
    pair.append(0, synth.gen_hidden(m, SEED, 21, 0))
    pair.append(0, synth.gen_hidden(m, SEED, 1000, 1))
    pair.append(1, synth.gen_hidden(m, SEED, 777, 2), positions=synth.gen_positions_gapped(9, 777, SEED, 3))
    pair.append(0, synth.gen_hidden(m, SEED, 300, 4))
    _check_pool(pair, (0, 1))
    agree = Agreement()
    for call in range(3):
        toks, logits, ref = pair.forward([0, 1], synth.gen_bonus(m, SEED, 2, index=50 + call))
        agree.add(toks, logits, ref)
    agree.check()
    pair.close()


@pytest.mark.parametrize("shape", ["hd64", "hd128-yarn"])
def test_fused_append_split_calls_equal_one_call(shape):
    """2600 rows in one call (launches of 2048 and 552 rows) against 700 + 1900 rows in two
    calls, after a 37-row start: the pools are equal bit for bit."""
    m = _model(shape)
    Wd = dev_weights(synth.gen_weights(m, SEED))
    H0 = synth.gen_hidden(m, SEED, 37, 10)
    H = synth.gen_hidden(m, SEED, 2600, 11)
    a = B.Drafter(m, Wd, 2700, 1)
    a.dflash_ctx_kv_append(0, dev_bf16(H0))
    a.dflash_ctx_kv_append(0, dev_bf16(H))
    b = B.Drafter(m, Wd, 2700, 1)
    b.dflash_ctx_kv_append(0, dev_bf16(H0))
    b.dflash_ctx_kv_append(0, dev_bf16(H[:700]))
    b.dflash_ctx_kv_append(0, dev_bf16(H[700:]))
    assert np.array_equal(pool_view(a), pool_view(b))
    b.close()
    a.close()
