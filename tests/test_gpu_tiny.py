"""GPU parity on the tiny drafter (2 layers, hidden 256, 8:2 heads, head_dim 32, vocab 1024):
every step of the HIP path against the CPU oracle, element by element, plus the integer
state of the paged pool bit for bit."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_02_amd import binding as B
from oracle import dflash_oracle as O
from gpu_util import Agreement, Pair, assert_kv_close, dev_bf16, pool_view, read_i32, read_i64, DEV

pytestmark = pytest.mark.gpu

SEED = 1001


@pytest.fixture(scope="module")
def tiny():
    m = synth.model("tiny-L2-h256")
    return m, synth.gen_weights(m, SEED)


def _check_seq_pool(pair, seq, pool, kpos):
    """K/V of every cached row of `seq` sit at the oracle's slots, with the oracle's values."""
    m = pair.m
    hd, nkv = m["head_dim"], m["num_kv_heads"]
    s = pair.ora.seqs[seq]
    n = s["pos"].shape[0]
    slots = pair.ora.pool.slots(seq, range(n))
    pages, offs = slots // 16, slots % 16
    assert np.array_equal(kpos[slots], s["pos"]), "stamped positions"
    for l in range(m["num_layers"]):
        K = pool[l, pages, 0].reshape(n, nkv, 16, hd)[np.arange(n), :, offs, :]      # [n, nkv, hd]
        V = pool[l, pages, 1].reshape(n, nkv, hd, 16)[np.arange(n), :, :, offs]      # [n, nkv, hd]
        for got, want, name in ((K, s["k"][l], "K"), (V, s["v"][l], "V")):
            assert_kv_close(got, want, f"seq {seq} layer {l} {name}", slots)


def test_append_tables_slots_and_writeback(tiny):
    m, W = tiny
    P = O.pool_pages(128, 16, 3)[1]
    order = synth.gen_page_order(P - 1, SEED)
    pair = Pair(m, W, 128, 3, page_order=order)
    pair.append(0, synth.gen_hidden(m, SEED, 20, 0))
    pair.append(1, synth.gen_hidden(m, SEED, 40, 1), positions=synth.gen_positions_gapped(3, 40, SEED))
    pair.append(0, synth.gen_hidden(m, SEED, 37, 2))
    # slots of the last call, bit for bit
    slots = read_i64(pair.gpu, B.DFLASH_BUF_SLOTS, 37)
    assert np.array_equal(slots, pair.ora.last_slots)
    # host and device block tables
    geo = pair.gpu.dflash_pool_geometry()
    dev_bt = read_i32(pair.gpu, B.DFLASH_BUF_BLOCKTAB, 3 * geo["pages_per_seq"]).reshape(3, -1)
    for s in range(3):
        kv, bt = pair.gpu.dflash_seq_info(s)
        assert kv == pair.ora.kv_len(s) and bt == pair.ora.block_table(s)
        assert list(dev_bt[s, :len(bt)]) == bt
    pool = pool_view(pair.gpu)
    kpos = read_i32(pair.gpu, B.DFLASH_BUF_KPOS, geo["num_pages"] * 16)
    for s in (0, 1):
        _check_seq_pool(pair, s, pool, kpos)
    # no stray writes: pages nobody owns (and the sentinel page 0) are still zero
    owned = set(pair.ora.block_table(0)) | set(pair.ora.block_table(1))
    free = [p for p in range(geo["num_pages"]) if p not in owned]
    assert 0 in free and not pool[:, free].any()
    pair.close()


def test_block_forward_parity_many_blocks(tiny):
    """>= 200 blocks over 8 sequences of ragged context, non-contiguous pages."""
    m, W = tiny
    nb = 8
    P = O.pool_pages(256, 16, nb)[1]
    pair = Pair(m, W, 256, nb, page_order=synth.gen_page_order(P - 1, SEED + 1))
    lens = synth.gen_ctx_lengths(1, 200, nb, SEED)
    for s in range(nb):
        pos = synth.gen_positions_gapped(0, int(lens[s]), SEED, index=s) if s % 3 == 1 else None
        pair.append(s, synth.gen_hidden(m, SEED, int(lens[s]), 10 + s), positions=pos)
    agree = Agreement()
    rng = np.random.default_rng(5)
    for call in range(26):
        seqs = list(rng.permutation(nb))
        bonus = synth.gen_bonus(m, SEED, nb, index=call)
        qpos = None
        if call % 2:
            qpos = [int(pair.ora.seqs[s]["pos"][-1]) + 1 + int(rng.integers(0, 5)) for s in seqs]
        toks, logits, ref = pair.forward(seqs, bonus, q_rope_pos=qpos)
        agree.add(toks, logits, ref)
    rate = agree.check(min_positions=2500)
    print(f"tiny parity: {agree.n} positions, agreement {rate:.4f}, max rel dlogit {agree.max_rel:.3e}")
    pair.close()


@pytest.mark.parametrize("gamma", [2, 5, 16])
def test_gamma_widths(tiny, gamma):
    m, W = tiny
    pair = Pair(m, W, 128, 2)
    pair.append(0, synth.gen_hidden(m, SEED, 45, 3))
    pair.append(1, synth.gen_hidden(m, SEED, 16, 4))
    agree = Agreement()
    for call in range(8):
        toks, logits, ref = pair.forward([1, 0], synth.gen_bonus(m, SEED, 2, index=100 + call), gamma=gamma)
        agree.add(toks, logits, ref)
    agree.check()
    pair.close()


def test_batch_invariance_bitwise(tiny):
    """A band's drafts and logits do not depend on the other bands in the call."""
    m, W = tiny
    nb = 6
    d = B.Drafter(m, {k: dev_bf16(v) for k, v in W.items()}, 256, nb)
    lens = [7, 100, 33, 160, 64, 1]
    for s in range(nb):
        d.dflash_ctx_kv_append(s, dev_bf16(synth.gen_hidden(m, SEED, lens[s], 20 + s)))
    bonus = synth.gen_bonus(m, SEED, nb, index=7)
    V = m["vocab"]
    tb = torch.empty((nb, 15), dtype=torch.int32, device=DEV)
    lb = torch.empty((nb * 15, V), dtype=torch.float32, device=DEV)
    d.dflash_block_forward(list(range(nb)), bonus, tb, lb)
    for s in range(nb):
        t1 = torch.empty((1, 15), dtype=torch.int32, device=DEV)
        l1 = torch.empty((15, V), dtype=torch.float32, device=DEV)
        d.dflash_block_forward([s], [bonus[s]], t1, l1)
        torch.cuda.synchronize()
        assert torch.equal(t1[0], tb[s])
        assert torch.equal(l1, lb[s * 15:(s + 1) * 15])
    d.close()


def test_wide_rows_parity_yarn_window(tiny):
    """Seven bands (112 rows: more than one 64-row group, so the wide GEMMs and the wide
    lm_head run, with a partial 128-row tile) under YaRN and a sliding window, against the
    oracle."""
    m, W = tiny
    my = dict(m, rope_type="yarn", yarn_factor=4.0, yarn_orig_max_pos=64.0, yarn_beta_fast=32.0,
              yarn_beta_slow=1.0, sliding_window=40, layer_sliding=[True, False])
    nb = 7
    pair = Pair(my, W, 200, nb)
    lens = [3, 150, 47, 16, 90, 1, 121]
    for s in range(nb):
        pair.append(s, synth.gen_hidden(m, SEED, lens[s], 60 + s))
    agree = Agreement()
    for call in range(4):
        order = list(range(nb)) if call % 2 == 0 else list(range(nb))[::-1]
        toks, logits, ref = pair.forward(order, synth.gen_bonus(m, SEED, nb, index=300 + call))
        agree.add(toks, logits, ref)
    agree.check(min_positions=300)
    pair.close()


def test_many_bands_many_chunks_window(tiny):
    """32 bands of 4900-5000 keys (17-20 attention chunks each; the sliding-window layer,
    window 4200, starts its chunks past the hidden keys and masks inside the first one) under
    YaRN: checked against the oracle, and bit for bit against single-band calls."""
    m, W = tiny
    my = dict(m, rope_type="yarn", yarn_factor=4.0, yarn_orig_max_pos=64.0, yarn_beta_fast=32.0,
              yarn_beta_slow=1.0, sliding_window=4200, layer_sliding=[True, False])
    nb = 32
    pair = Pair(my, W, 5200, nb)
    lens = [4900 + (37 * s) % 101 for s in range(nb)]
    for s in range(nb):
        pair.append(s, synth.gen_hidden(m, SEED, lens[s], 400 + s))
    agree = Agreement()
    bonus = synth.gen_bonus(m, SEED, nb, index=500)
    toks, logits, ref = pair.forward(list(range(nb)), bonus)
    agree.add(toks, logits, ref)
    agree.check(min_positions=400)
    V = m["vocab"]
    for s in (0, 13, 31):
        t1 = torch.empty((1, 15), dtype=torch.int32, device=DEV)
        l1 = torch.empty((15, V), dtype=torch.float32, device=DEV)
        pair.gpu.dflash_block_forward([s], [bonus[s]], t1, l1)
        torch.cuda.synchronize()
        assert np.array_equal(t1[0].cpu().numpy(), toks[s])
        assert np.array_equal(l1.cpu().numpy().astype(np.float64), logits[s])
    pair.close()


def test_yarn_and_sliding_window(tiny):
    m, W = tiny
    my = dict(m, rope_type="yarn", yarn_factor=4.0, yarn_orig_max_pos=64.0, yarn_beta_fast=32.0,
              yarn_beta_slow=1.0, sliding_window=40, layer_sliding=[True, False])
    pair = Pair(my, W, 300, 3)
    pair.append(0, synth.gen_hidden(m, SEED, 250, 30))
    pair.append(1, synth.gen_hidden(m, SEED, 90, 31), positions=synth.gen_positions_gapped(5, 90, SEED, 1))
    pair.append(2, synth.gen_hidden(m, SEED, 12, 32))
    agree = Agreement()
    for call in range(12):
        qpos = None if call % 2 == 0 else [260 + call, int(pair.ora.seqs[1]["pos"][-1]) + 3, 12 + call]
        toks, logits, ref = pair.forward([0, 1, 2], synth.gen_bonus(m, SEED, 3, index=200 + call), q_rope_pos=qpos)
        agree.add(toks, logits, ref)
    agree.check()
    pair.close()


def test_long_append_crosses_launch_chunks(tiny):
    """3000 rows in one call (the runtime splits appends into 2048-row launches) equal the same
    rows appended in two calls, bit for bit, and match the oracle."""
    m, W = tiny
    H = synth.gen_hidden(m, SEED, 3000, 40)
    pair = Pair(m, W, 3100, 1)
    pair.append(0, H)
    d2 = B.Drafter(m, pair.Wd, 3100, 1)
    d2.dflash_ctx_kv_append(0, dev_bf16(H[:1234]))
    d2.dflash_ctx_kv_append(0, dev_bf16(H[1234:]))
    p1, p2 = pool_view(pair.gpu), pool_view(d2)
    assert np.array_equal(p1, p2)
    geo = pair.gpu.dflash_pool_geometry()
    _check_seq_pool(pair, 0, p1, read_i32(pair.gpu, B.DFLASH_BUF_KPOS, geo["num_pages"] * 16))
    agree = Agreement()
    for call in range(4):
        toks, logits, ref = pair.forward([0], synth.gen_bonus(m, SEED, 1, index=300 + call))
        agree.add(toks, logits, ref)
    agree.check()
    d2.close()
    pair.close()


@pytest.mark.parametrize("counts", [[3, 0, 16, 1, 37], [16, 16, 16, 16, 16, 16, 16, 16], [60, 1, 100, 95]])
def test_batched_append_matches_oracle(tiny, counts):
    """One batched append over several sequences (totals of 57, 128 and 256 rows: the skinny
    and the wide GEMM forms), with caller positions on one sequence and a sequence given no
    rows: slots, block tables and stamped positions bit for bit, every cached K/V row against
    the oracle, then forwards over all of them."""
    m, W = tiny
    nb = len(counts)
    P = O.pool_pages(400, 16, nb)[1]
    pair = Pair(m, W, 400, nb, page_order=synth.gen_page_order(P - 1, SEED + 7))
    for s in range(nb):
        if s % 2 == 0:
            pair.append(s, synth.gen_hidden(m, SEED, 5 + 11 * s, 70 + s))
    H = synth.gen_hidden(m, SEED, sum(counts), 90)
    pos = None
    if nb > 4:
        # caller positions, gapped, on sequence 1 only (the others continue from kv_len)
        pos = []
        for s, c in enumerate(counts):
            base = pair.ora.kv_len(s)
            last = int(pair.ora.seqs[s]["pos"][-1]) if base else -1
            pos += [last + 3 + 2 * i for i in range(c)] if s == 1 else list(range(base, base + c))
    seqs = list(range(nb))[::-1]
    order_counts = [counts[s] for s in seqs]
    Hs = np.concatenate([H[sum(counts[:s]):sum(counts[:s + 1])] for s in seqs]) if nb else H
    ps = None
    if pos is not None:
        ps = np.concatenate([np.asarray(pos[sum(counts[:s]):sum(counts[:s + 1])], dtype=np.int64) for s in seqs])
    pair.append_batch(seqs, order_counts, Hs, positions=ps)
    total = sum(counts)
    assert np.array_equal(read_i64(pair.gpu, B.DFLASH_BUF_SLOTS, total), pair.ora.last_slots)
    geo = pair.gpu.dflash_pool_geometry()
    dev_bt = read_i32(pair.gpu, B.DFLASH_BUF_BLOCKTAB, nb * geo["pages_per_seq"]).reshape(nb, -1)
    for s in range(nb):
        kv, bt = pair.gpu.dflash_seq_info(s)
        assert kv == pair.ora.kv_len(s) and bt == pair.ora.block_table(s)
        assert list(dev_bt[s, :len(bt)]) == bt
    pool = pool_view(pair.gpu)
    kpos = read_i32(pair.gpu, B.DFLASH_BUF_KPOS, geo["num_pages"] * 16)
    for s in range(nb):
        if pair.ora.kv_len(s):
            _check_seq_pool(pair, s, pool, kpos)
    agree = Agreement()
    live = [s for s in range(nb) if pair.ora.kv_len(s)]
    for call in range(3):
        toks, logits, ref = pair.forward(live, synth.gen_bonus(m, SEED, len(live), index=600 + call))
        agree.add(toks, logits, ref)
    agree.check()
    pair.close()


def test_batched_append_errors_change_nothing(tiny):
    """Every refused batched append leaves block tables, kv_len and the pool as they were."""
    m, W = tiny
    pair = Pair(m, W, 300, 3, num_pages=9)             # 8 allocatable pages
    pair.append(0, synth.gen_hidden(m, SEED, 30, 80))   # 2 pages
    pair.append(1, synth.gen_hidden(m, SEED, 10, 81))   # 1 page: 5 left
    before = [pair.gpu.dflash_seq_info(s) for s in range(3)]
    H = dev_bf16(synth.gen_hidden(m, SEED, 257, 82))
    cases = [
        (dict(seqs=[0, 0], counts=[1, 1]), "ERANGE"),          # repeated sequence
        (dict(seqs=[3], counts=[1]), "ERANGE"),                 # out of range
        (dict(seqs=[1, 0], counts=[1, 271]), "ERANGE"),         # 30 + 271 > max_seq_len 300
        (dict(seqs=[1, 2], counts=[-1, 2]), "EINVAL"),          # negative count
        (dict(seqs=[1, 2], counts=[0, 0]), "EINVAL"),           # no rows
        (dict(seqs=[1, 2], counts=[200, 57]), "EINVAL"),        # 257 rows > 256 per call
        (dict(seqs=[1, 2], counts=[40, 40]), "EPOOL"),          # 3 + 3 pages, 5 free
    ]
    for kw, name in cases:
        # the C entry directly (the binding would refuse a row-count mismatch itself)
        rc = pair.gpu.L.dflash_ctx_kv_append_batch(pair.gpu.ctx, len(kw["seqs"]), B._i32_array(kw["seqs"]),
                                                   B._i32_array(kw["counts"]), B._ptr(H), None, None)
        assert rc == getattr(B, "DFLASH_" + name), (kw, rc)
    with pytest.raises(B.DflashError) as ei:           # positions not increasing within sequence 1
        pair.gpu.dflash_ctx_kv_append_batch([1, 2], [2, 1], H[:3], positions=[40, 39, 0])
    assert ei.value.name == "EINVAL"
    with pytest.raises(B.DflashError) as ei:           # at or below sequence 1's last position
        pair.gpu.dflash_ctx_kv_append_batch([1], [1], H[:1], positions=[9])
    assert ei.value.name == "EINVAL"
    assert [pair.gpu.dflash_seq_info(s) for s in range(3)] == before
    # still exact afterwards
    pair.append_batch([2, 1], [5, 7], synth.gen_hidden(m, SEED, 12, 84))
    agree = Agreement()
    toks, logits, ref = pair.forward([0, 1, 2], synth.gen_bonus(m, SEED, 3, index=700))
    agree.add(toks, logits, ref)
    agree.check()
    pair.close()


def test_errors_change_nothing_and_reset_reuses_pages(tiny):
    m, W = tiny
    pair = Pair(m, W, 64, 2, num_pages=6)
    pair.append(0, synth.gen_hidden(m, SEED, 32, 50))
    pair.append(1, synth.gen_hidden(m, SEED, 20, 51))
    before = [pair.gpu.dflash_seq_info(s) for s in (0, 1)]
    V = m["vocab"]
    toks = torch.empty((2, 15), dtype=torch.int32, device=DEV)
    with pytest.raises(B.DflashError) as ei:          # 2 pages needed, 1 free
        pair.gpu.dflash_block_forward([0, 1], [1, 2], toks)
    assert ei.value.name == "EPOOL"
    with pytest.raises(B.DflashError) as ei:
        pair.gpu.dflash_ctx_kv_append(1, dev_bf16(synth.gen_hidden(m, SEED, 45, 52)))
    assert ei.value.name == "ERANGE"
    with pytest.raises(B.DflashError) as ei:
        pair.gpu.dflash_ctx_kv_append(1, dev_bf16(synth.gen_hidden(m, SEED, 29, 52)))
    assert ei.value.name == "EPOOL"
    with pytest.raises(B.DflashError) as ei:
        pair.gpu.dflash_ctx_kv_append(1, dev_bf16(synth.gen_hidden(m, SEED, 2, 52)), positions=[3, 4])
    assert ei.value.name == "EINVAL"
    for bad in (dict(seqs=[0, 0], bonus=[1, 2]), dict(seqs=[2], bonus=[1]), dict(seqs=[0], bonus=[V])):
        with pytest.raises(B.DflashError):
            pair.gpu.dflash_block_forward(bad["seqs"], bad["bonus"], toks)
    with pytest.raises(B.DflashError) as ei:
        pair.gpu.dflash_block_forward([0], [1], toks, gamma=17)
    assert ei.value.name == "ERANGE"
    assert [pair.gpu.dflash_seq_info(s) for s in (0, 1)] == before
    # the engine is still exact after the refused calls
    agree = Agreement()
    toks, logits, ref = pair.forward([0], [9])
    agree.add(toks, logits, ref)
    pair.gpu.dflash_seq_reset(1)
    pair.ora.seq_reset(1)
    toks, logits, ref = pair.forward([1], [10])           # reuses a freed page
    agree.add(toks, logits, ref)
    pair.append(1, synth.gen_hidden(m, SEED, 10, 53))
    toks, logits, ref = pair.forward([1, 0], [11, 12])
    agree.add(toks, logits, ref)
    agree.check()
    for s in (0, 1):
        assert pair.gpu.dflash_seq_info(s) == (pair.ora.kv_len(s), pair.ora.block_table(s))
    pair.close()
